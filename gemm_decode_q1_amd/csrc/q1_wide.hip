// Wide-M packed Q1 matmul on the matrix cores (gfx950): y[M, N] = x[M, K] *
// W^T for M > 8 activation rows, straight from the packed weights (Higgs PR
// #212, "What": wider batches fall back to a dense path; here the dense path
// is replaced by the same fp8 x fp4 products as the narrow matrix-core
// kernel, so the weights are read as bits, not as a bf16 copy).
//
// Two launches:
//  * q1_act_image_kernel converts x once into a ready-to-load A operand image
//    (see q1_fp8.h): per row block rb (16 activation rows) and group g one
//    2 KB tile per piece in MFMA lane order, [lane][32 B] (bytes 0..15 =
//    k-half 0, 16..31 = k-half 1) -- symmetric tensors two fp8 pieces (hi,
//    lo), affine ones three bf8 pieces; per (rb, span of 4 groups) one E8M0
//    scale dword per piece and lane (byte g % 4); per (rb, g) 16 floats for
//    the accumulator input (-X/2), or the group sums X for affine tensors.
//  * q1_wide_kernel: a workgroup of 8 waves owns 8 row blocks (128 rows) and
//    TNB * 16 weight rows; wave w owns row block w and all TNB column blocks,
//    so its A operands come straight from the image, while the weights of
//    each span (4 groups) are staged once per workgroup in LDS as [row][word
//    q][group] (80-byte rows: the staging writes and the reads of lane
//    (row, q) spread over the banks), with their scales (and biases) as fp32.
//    Per half span (2 groups) and column block a lane reads its 2 words and
//    scales, expands each word with one AND per bit class and chains two
//    MFMAs per group through the accumulator input (hi, then lo with its own
//    block scale), so the expansion and the group-scale multiply-add are paid
//    once per 16 activation rows.  Affine tensors chain the three pieces and
//    take, per weight row and group, the product over the code d whose weight
//    is larger in magnitude (the word complemented when d = 0), adding
//    (w_d - w_o) S_d + w_o X (as the narrow matrix-core kernel does, for the
//    same reason: the error stays relative to sum |w x|).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "q1_device.h"
#include "q1_fp8.h"
#include "q1_internal.h"

namespace q1 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float v2f_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowB = 80;  // LDS bytes per staged weight row: [4 words][4 groups] + pad

template <bool MBF16>
__device__ __forceinline__ float meta_val(uint32_t bits) {
  return MBF16 ? __uint_as_float(bits << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// ---- activation image: one thread per (row m, group g, word b) ----
template <bool AFFINE>
__global__ __launch_bounds__(256) void q1_act_image_kernel(const uint16_t* __restrict__ x, int64_t x_ld, int64_t M,
                                                           int G, int nspan, unsigned char* __restrict__ img,
                                                           unsigned char* __restrict__ sc_img,
                                                           float* __restrict__ xs_img) {
  const int tid = threadIdx.x;
  const int b = tid & 3;
  const int g = (int)blockIdx.x * 64 + (tid >> 2);
  const int64_t m = blockIdx.y;  // 0 .. 16*MB-1
  const int Gp = 4 * nspan;  // groups padded to whole spans (zero operands)
  uint32_t wd[16];
  if (g < G && m < M) {
    const u32x4* src = reinterpret_cast<const u32x4*>(x + m * x_ld + (int64_t)g * 128 + b * 32);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 v = src[c];
#pragma unroll
      for (int e = 0; e < 4; ++e) wd[4 * c + e] = v[e];
    }
  } else {
#pragma unroll
    for (int d = 0; d < 16; ++d) wd[d] = 0u;  // rows past M: zero operands, zero sums
  }
  constexpr int NP = AFFINE ? 3 : 2;  // pieces
  uint32_t pc[NP][4][2];
  int sc[NP];
  float X;
  if constexpr (AFFINE) {
    q1_convert_word_bf8(wd, pc, sc, X);
  } else {
    int s0;
    q1_convert_word(wd, pc[0], pc[1], s0, X);
    sc[0] = s0;
    sc[1] = s0 - 4;  // lo = residual * 16
  }
  X += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, X), 0xB1, 0xf, 0xf, false));
  X += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, X), 0x4E, 0xf, 0xf, false));
  if (g >= Gp) return;
  const int64_t rb = m >> 4;
  const int ml = (int)(m & 15);
  // chunk (quarter qa = 2*(b & 1) + c, k-half b >> 1) of lane qa*16 + ml holds
  // in dword 2*(j & 1) + hh the class-j bytes of half word hh, j >> 1 == c
  unsigned char* tile = img + (rb * Gp + g) * (NP * 2048) + (b >> 1) * 16;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int qa = 2 * (b & 1) + c;
      *reinterpret_cast<u32x4*>(tile + p * 2048 + (qa * 16 + ml) * 32) =
          u32x4{pc[p][2 * c][0], pc[p][2 * c][1], pc[p][2 * c + 1][0], pc[p][2 * c + 1][1]};
    }
  }
  // scale of A row r, 32-weight block j (= word b) sits in lane r + 16 j
  unsigned char* sp = sc_img + (rb * nspan + (g >> 2)) * (NP * 256) + (ml + 16 * b) * 4 + (g & 3);
#pragma unroll
  for (int p = 0; p < NP; ++p) sp[256 * p] = (unsigned char)(sc[p] + 127);
  if (b == 0) xs_img[(rb * Gp + g) * 16 + ml] = AFFINE ? X : -0.5f * X;
}

struct WideArgs {
  const uint32_t* packed;
  const uint16_t* scales;
  const uint16_t* biases;
  const unsigned char* img;
  const uint32_t* sc_img;
  const float* xs_img;
  int64_t M, N;
  int32_t K, G, nspan, MB, mtiles, ntn;
  uint32_t packed_bytes, meta_bytes;
  int32_t out_dtype;
  void* out;
  int64_t out_ld;
};

// Workgroup barrier for LDS traffic only: waits for this wave's LDS accesses
// (lgkmcnt 0), not for its global loads (__syncthreads would also wait for
// vmcnt 0 and drain the next span's loads).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
}

constexpr uint32_t kBufWord3 = 0x00020000u;
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, (int)kBufWord3);
}

// One group's NP chained products for this lane: piece 0 (accumulator input
// C), then each further piece with the previous result as accumulator input,
// block scale byte BYTE of piece p's scale dword.  CBSZ: A format (0 fp8
// E4M3, 1 bf8 E5M2); B fp4 with unit scales.
template <int BYTE, int CBSZ, int NP>
__device__ __forceinline__ v4f mfma_chain(const v8i (&A)[NP], const v8i& B, const v4f& C, const uint32_t (&sc)[NP]) {
  v4f d = C;
#pragma unroll
  for (int p = 0; p < NP; ++p)
    d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[p], B, d, CBSZ, 4, BYTE, (int)sc[p], 0, 0x7f7f7f7f);
  return d;
}

template <bool AFFINE, bool MBF16, int TNB>
__global__ __launch_bounds__(kThreads) void q1_wide_kernel(WideArgs a) {
  constexpr int ROWS = TNB * 16;                   // weight rows of the workgroup
  constexpr int LOADS = (ROWS * 4 + kThreads - 1) / kThreads;  // 16-byte staging loads per thread
  static_assert(ROWS <= kThreads, "one thread per staged row for the scales");
  constexpr int NP = AFFINE ? 3 : 2;       // activation pieces (see q1_fp8.h)
  __shared__ __align__(16) unsigned char wsm[2][ROWS * kRowB];
  // per row and group, fp32: the scale (symmetric), or w_d - w_o (affine)
  __shared__ __align__(16) float ssm[2][ROWS * 4];
  // affine: w_o per row and group, and the code polarity (byte g = 0xff: the
  // product runs over the clear bits, the word is complemented)
  __shared__ __align__(16) float bsm[AFFINE ? 2 : 1][AFFINE ? ROWS * 4 : 4];
  __shared__ uint32_t pol[AFFINE ? 2 : 1][AFFINE ? ROWS : 1];
  __shared__ __align__(16) float xsm[2][kWaves * 4 * 16];  // group sums of a span: [row block][group][row]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // XCD-aware order: the row-block tiles sharing one weight tile run on the
  // same XCD (workgroups are dealt round-robin over 8 XCDs)
  const int nwg = a.mtiles * a.ntn;
  int logical = (int)blockIdx.x;
  if ((nwg & 7) == 0) logical = (logical & 7) * (nwg >> 3) + (logical >> 3);
  const int tm = logical % a.mtiles, tn = logical / a.mtiles;
  const int rb = tm * kWaves + wave;
  const bool live = rb < a.MB;  // (uniform) the wave has activation rows
  const int64_t n0 = (int64_t)tn * ROWS;
  const int nl = lane & 15, q = lane >> 4;

  const __amdgpu_buffer_rsrc_t rp = rsrc(a.packed, a.packed_bytes);
  const __amdgpu_buffer_rsrc_t rs = rsrc(a.scales, a.meta_bytes);
  const __amdgpu_buffer_rsrc_t rbias = rsrc(AFFINE ? a.biases : a.scales, a.meta_bytes);
  const uint32_t row_bytes = (uint32_t)a.K >> 3;

  // ---- staging of span sp's weights: thread -> (row, group chunk) ----
  u32x4 wreg[LOADS];
  uint32_t sreg[2], breg[2];
  float xreg;
  auto stage_load = [&](int sp) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int t = tid + i * kThreads;
      const int row = t >> 2, c = t & 3;
      const int64_t n = n0 + row;
      const int g = 4 * sp + c;
      const bool ok = row < ROWS && n < a.N && g < a.G;
      const uint32_t off = ((uint32_t)n * row_bytes + (uint32_t)g * 16u) | (ok ? 0u : kOOB);
      wreg[i] = __builtin_amdgcn_raw_buffer_load_b128(rp, off, 0, 2);
    }
    {  // group sums: thread -> (row block, group, row); a row block past
       // MB (its wave computes nothing) reads the last one's
      const int rbl = tid >> 6, g = 4 * sp + ((tid >> 4) & 3);
      const int rbg = min(tm * kWaves + rbl, a.MB - 1);
      xreg = a.xs_img[((int64_t)rbg * (4 * a.nspan) + g) * 16 + (tid & 15)];
    }
    // scales (and biases) of groups 4sp..4sp+3, one row per thread
    const int row = tid;
    const int64_t n = n0 + row;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t v = 0, bv = 0;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int g = 4 * sp + 2 * h + e;
        const bool ok = row < ROWS && n < a.N && g < a.G;
        const uint32_t mo = ((uint32_t)n * (uint32_t)a.G + (uint32_t)g) * 2u | (ok ? 0u : kOOB);
        v |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, mo, 0, 0) << (16 * e);
        if (AFFINE) bv |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rbias, mo, 0, 0) << (16 * e);
      }
      sreg[h] = v;
      breg[h] = bv;
    }
  };
  auto stage_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int t = tid + i * kThreads;
      const int row = t >> 2, c = t & 3;
      if (row < ROWS) {
        uint32_t* dst = reinterpret_cast<uint32_t*>(wsm[buf] + row * kRowB) + c;
#pragma unroll
        for (int k = 0; k < 4; ++k) dst[4 * k] = wreg[i][k];  // word k of group c -> [k][c]
      }
    }
    xsm[buf][tid] = xreg;
    if (tid < ROWS) {
      const v4f sv = v4f{meta_val<MBF16>(sreg[0]), meta_val<MBF16>(sreg[0] >> 16), meta_val<MBF16>(sreg[1]),
                         meta_val<MBF16>(sreg[1] >> 16)};
      if constexpr (AFFINE) {
        const v4f bv = v4f{meta_val<MBF16>(breg[0]), meta_val<MBF16>(breg[0] >> 16), meta_val<MBF16>(breg[1]),
                           meta_val<MBF16>(breg[1] >> 16)};
        v4f sd, wo;
        uint32_t pm = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {  // codes' weights w1 = s + b, w0 = b; d: the larger
          const float w1 = sv[c] + bv[c];
          const bool d1 = fabsf(w1) >= fabsf(bv[c]);
          const float dw = w1 - bv[c];
          sd[c] = d1 ? dw : -dw;
          wo[c] = d1 ? bv[c] : w1;
          pm |= d1 ? 0u : (0xffu << (8 * c));
        }
        *reinterpret_cast<v4f*>(&ssm[buf][4 * tid]) = sd;
        *reinterpret_cast<v4f*>(&bsm[buf][4 * tid]) = wo;
        pol[buf][tid] = pm;
      } else {
        *reinterpret_cast<v4f*>(&ssm[buf][4 * tid]) = sv;
      }
    }
  };

  // ---- this wave's A operands: half span h (groups 4sp+2h, 4sp+2h+1) ----
  // A[e][p] = piece p of group 4sp+2h+e
  auto a_load = [&](int sp, int h, v8i (&Ao)[2][NP]) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int g = 4 * sp + 2 * h + e;  // (groups past G are zero in the image)
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) {
        const u32x4* t = reinterpret_cast<const u32x4*>(a.img + ((int64_t)rb * (4 * a.nspan) + g) * (NP * 2048) +
                                                        pp * 2048 + lane * 32);
        const u32x4 h0 = t[0], h1 = t[1];
        Ao[e][pp] = v8i{(int)h0[0], (int)h0[1], (int)h0[2], (int)h0[3], (int)h1[0], (int)h1[1], (int)h1[2], (int)h1[3]};
      }
    }
  };
  auto sc_load = [&](int sp, uint32_t (&sc)[NP]) {
    const uint32_t* t = a.sc_img + ((int64_t)rb * a.nspan + sp) * (NP * 64) + lane;
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) sc[pp] = t[64 * pp];
  };

  v4f acc[TNB];
#pragma unroll
  for (int j = 0; j < TNB; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};

  // ---- products of half span h from LDS buffer buf ----
  auto compute = [&](int buf, int h, const v8i (&A)[2][NP], const uint32_t (&sc)[NP]) {
    // groups past G (last span) have zero A operands, zero weights and zero
    // scales, so every span runs all its groups without branches
    v4f XS[2];  // this wave's group sums, rows 4q..4q+3
#pragma unroll
    for (int e = 0; e < 2; ++e)
      XS[e] = reinterpret_cast<const v4f*>(&xsm[buf][(wave * 4 + 2 * h + e) * 16])[q];
    // the LDS reads of column block j+1 are issued before block j's work
    auto rd_w = [&](int j) { return *reinterpret_cast<const u32x2*>(wsm[buf] + (j * 16 + nl) * kRowB + q * 16 + 8 * h); };
    auto rd_s = [&](int j) { return *reinterpret_cast<const v2f_t*>(&ssm[buf][4 * (j * 16 + nl) + 2 * h]); };
    auto rd_b = [&](int j) {
      return AFFINE ? *reinterpret_cast<const v2f_t*>(&bsm[buf][4 * (j * 16 + nl) + 2 * h]) : v2f_t{0.f, 0.f};
    };
    auto rd_pol = [&](int j) -> uint32_t { return AFFINE ? pol[buf][j * 16 + nl] : 0u; };
    auto fma_block = [&](int j, const v4f (&Dv)[2], v2f_t sv, v2f_t bv) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] = fmaf(sv[e], Dv[e][i], acc[j][i]);
        if (AFFINE) {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[j][i] = fmaf(bv[e], XS[e][i], acc[j][i]);
        }
      }
    };
    u32x2 w2n = rd_w(0);
    v2f_t s2n = rd_s(0), b2n = rd_b(0);
    uint32_t pn = rd_pol(0);
    v4f Dp[2];
    v2f_t s2p = {0.f, 0.f}, b2p = {0.f, 0.f};
#pragma unroll
    for (int j = 0; j < TNB; ++j) {
      const u32x2 w2 = w2n;
      const v2f_t s2 = s2n, b2 = b2n;
      const uint32_t pj = pn;
      if (j + 1 < TNB) {
        w2n = rd_w(j + 1);
        s2n = rd_s(j + 1);
        b2n = rd_b(j + 1);
        pn = rd_pol(j + 1);
      }
      v4f D[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        int Bv[8];
        // affine: complement the word when the product runs over the clear bits
        const uint32_t wv = AFFINE ? w2[e] ^ (uint32_t)__builtin_amdgcn_sbfe((int)pj, 8 * (2 * h + e), 8) : w2[e];
        q1_expand_b(wv, Bv);
        const v8i B = {Bv[0], Bv[1], Bv[2], Bv[3], 0, 0, 0, 0};
        const v4f C = AFFINE ? v4f{0.f, 0.f, 0.f, 0.f} : XS[e];
        constexpr int CB = AFFINE ? 1 : 0;
        if (h == 0 && e == 0) D[e] = mfma_chain<0, CB, NP>(A[e], B, C, sc);
        else if (h == 0) D[e] = mfma_chain<1, CB, NP>(A[e], B, C, sc);
        else if (e == 0) D[e] = mfma_chain<2, CB, NP>(A[e], B, C, sc);
        else D[e] = mfma_chain<3, CB, NP>(A[e], B, C, sc);
      }
      // the scale multiply-adds of block j-1 go after block j's products,
      // so they never wait for a product just issued
      if (j > 0) fma_block(j - 1, Dp, s2p, b2p);
      Dp[0] = D[0];
      Dp[1] = D[1];
      s2p = s2;
      b2p = b2;
      // keep later blocks' LDS reads from being hoisted (their results would
      // all be live at once)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
    fma_block(TNB - 1, Dp, s2p, b2p);
  };

  // A0 holds the first half span's operands, A1 the second's; each loads
  // while the other half computes (no register copies between spans)
  v8i A0[2][NP], A1[2][NP];
  uint32_t scc[NP], scn[NP];
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) scc[pp] = scn[pp] = 0u;
  stage_load(0);
  if (live) {
    a_load(0, 0, A0);
    sc_load(0, scc);
  }
  stage_store(0);
  lds_barrier();

  for (int sp = 0; sp < a.nspan; ++sp) {
    const int buf = sp & 1;
    const bool more = sp + 1 < a.nspan;
    if (more) stage_load(sp + 1);
    if (live) {
      a_load(sp, 1, A1);
      compute(buf, 0, A0, scc);
      // (the next loads must not move above the products that read A0)
      __builtin_amdgcn_sched_barrier(0);
      {
        const int spn = more ? sp + 1 : 0;
        a_load(spn, 0, A0);
        sc_load(spn, scn);
      }
      compute(buf, 1, A1, scc);
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) scc[pp] = scn[pp];
    }
    if (more) stage_store(buf ^ 1);  // that buffer was last read before the previous barrier
    lds_barrier();
  }

  if (!live) return;
  // lane l: activation rows 16 rb + 4 (l >> 4) + i, weight row l & 15 of each
  // column block
  const int64_t m0 = (int64_t)rb * 16 + 4 * q;
#pragma unroll
  for (int j = 0; j < TNB; ++j) {
    const int64_t n = n0 + j * 16 + nl;
    if (n < a.N) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (m0 + i < a.M) store_out(a.out, a.out_dtype, (m0 + i) * a.out_ld + n, acc[j][i]);
    }
  }
}

template <int TNB>
hipError_t launch_wide_t(const WidePlan& p, const WideArgs& g, bool affine, bool mbf16, hipStream_t s) {
  const dim3 grid((unsigned)p.wgs), block(kThreads);
  if (affine) {
    if (mbf16) hipLaunchKernelGGL((q1_wide_kernel<true, true, TNB>), grid, block, 0, s, g);
    else hipLaunchKernelGGL((q1_wide_kernel<true, false, TNB>), grid, block, 0, s, g);
  } else {
    if (mbf16) hipLaunchKernelGGL((q1_wide_kernel<false, true, TNB>), grid, block, 0, s, g);
    else hipLaunchKernelGGL((q1_wide_kernel<false, false, TNB>), grid, block, 0, s, g);
  }
  return hipGetLastError();
}

}  // namespace

bool plan_wide(int64_t M, int64_t N, int64_t K, bool affine, WidePlan* p, const char** why) {
  if (M < 1 || N < 1 || K < 128 || K % 128 != 0) {
    *why = "bad shape";
    return false;
  }
  if (N * (K / 8) >= ((int64_t)1 << 31) || N * (K / 128) * 2 >= ((int64_t)1 << 31)) {
    *why = "matrix too large for 32-bit buffer offsets";
    return false;
  }
  p->M = M;
  p->N = N;
  p->K = (int)K;
  p->G = (int)(K / 128);
  p->nspan = (p->G + 3) / 4;
  p->MB = (int)((M + 15) / 16);
  p->mtiles = (p->MB + kWaves - 1) / kWaves;
  // column blocks per workgroup: the choice that keeps the most CUs busy in
  // the last round of workgroups (ties: the wider tile)
  const int cus = device_cus();
  const int64_t nbk = (N + 15) / 16;
  const int cand[3] = {17, 16, 10};
  double best = -1.0;
  for (int tnb : cand) {
    const int64_t ntn = (nbk + tnb - 1) / tnb;
    const int64_t wgs = ntn * p->mtiles;
    const double eff = (double)wgs / (double)(((wgs + cus - 1) / cus) * cus);
    if (eff > best + 1e-9) {
      best = eff;
      p->tnb = tnb;
      p->ntn = (int)ntn;
      p->wgs = wgs;
    }
  }
  const size_t np = affine ? 3 : 2;  // activation pieces per value
  const size_t img = (size_t)p->MB * p->nspan * 4 * 2048 * np;
  const size_t sc = (size_t)p->MB * p->nspan * 256 * np;
  const size_t xs = (size_t)p->MB * p->nspan * 4 * 64;
  p->sc_off = (img + 255) / 256 * 256;
  p->xs_off = p->sc_off + (sc + 255) / 256 * 256;
  p->ws_bytes = p->xs_off + (xs + 255) / 256 * 256;
  return true;
}

hipError_t launch_wide(const WidePlan& p, const uint16_t* x, int64_t x_ld, const QMat& w, void* out, int32_t out_dtype,
                       int64_t out_ld, unsigned char* ws, hipStream_t s, bool make_image) {
  unsigned char* img = ws;
  unsigned char* sc = ws + p.sc_off;
  float* xs = reinterpret_cast<float*>(ws + p.xs_off);
  if (make_image) {
    const dim3 ig((unsigned)((4 * p.nspan + 63) / 64), (unsigned)(p.MB * 16));
    if (w.symmetric)
      hipLaunchKernelGGL((q1_act_image_kernel<false>), ig, dim3(256), 0, s, x, x_ld, p.M, p.G, p.nspan, img, sc, xs);
    else
      hipLaunchKernelGGL((q1_act_image_kernel<true>), ig, dim3(256), 0, s, x, x_ld, p.M, p.G, p.nspan, img, sc, xs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  WideArgs g;
  g.packed = w.packed;
  g.scales = w.scales;
  g.biases = w.biases;
  g.img = img;
  g.sc_img = reinterpret_cast<const uint32_t*>(sc);
  g.xs_img = xs;
  g.M = p.M;
  g.N = p.N;
  g.K = p.K;
  g.G = p.G;
  g.nspan = p.nspan;
  g.MB = p.MB;
  g.mtiles = p.mtiles;
  g.ntn = p.ntn;
  g.packed_bytes = (uint32_t)(p.N * (p.K / 8));
  g.meta_bytes = (uint32_t)(p.N * p.G * 2);
  g.out_dtype = out_dtype;
  g.out = out;
  g.out_ld = out_ld;
  const bool affine = !w.symmetric, mbf16 = w.meta_bf16 != 0;
  if (p.tnb == 17) return launch_wide_t<17>(p, g, affine, mbf16, s);
  if (p.tnb == 16) return launch_wide_t<16>(p, g, affine, mbf16, s);
  return launch_wide_t<10>(p, g, affine, mbf16, s);
}

}  // namespace q1
