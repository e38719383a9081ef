// Wide-M packed Q1 matmul on the matrix cores (gfx950): y[M, N] = x[M, K] *
// W^T for M > 8 activation rows, straight from the packed weights (Higgs PR
// #212, "What": wider batches fall back to a dense path; here the dense path
// is replaced by the same fp8 x fp4 products as the narrow matrix-core
// kernel, so the weights are read as bits, not as a bf16 copy).
//
// Two launches:
//  * q1_act_image_kernel converts x once into a ready-to-load A operand image
//    (see q1_fp8.h for the split): per row block rb (8 activation rows) and
//    group g a 2 KB tile in MFMA lane order, [lane][32 B] (bytes 0..15 =
//    k-half 0, 16..31 = k-half 1); per (rb, span of 4 groups) one E8M0 scale
//    dword per lane (byte g % 4); per (rb, g) 16 floats for the accumulator
//    input (-X/2 or X on the hi rows, 0 on the lo rows).
//  * q1_wide_kernel: a workgroup of 8 waves owns 8 row blocks (64 rows) and
//    TNB * 16 weight rows; wave w owns row block w and all TNB column blocks,
//    so its A operand comes straight from the image (no sharing needed),
//    while the weights of each span (4 groups) are staged once per
//    workgroup in LDS as [row][word q][group] (80-byte rows: the staging
//    writes and the 16-byte reads of lane (row, q) spread over the banks).
//    Per span and column block a lane reads its words of the 4 groups and
//    their 4 scales, expands each word with one AND per bit class and issues
//    one MFMA per group; the group scale multiplies the result into the
//    accumulator (and b * X for affine tensors).
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

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowB = 80;  // LDS bytes per staged weight row: [4 words][4 groups] + pad

int wide_device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      cus = v;
    else
      cus = 256;
  }
  return cus;
}

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
  const int64_t m = blockIdx.y;  // 0 .. 8*MB-1
  const bool valid = g < G;
  uint32_t wd[16];
  if (valid && m < M) {
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
  uint32_t hi[4][2], lo[4][2];
  int sc;
  float X;
  q1_convert_word(wd, hi, lo, sc, X);
  X += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, X), 0xB1, 0xf, 0xf, false));
  X += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, X), 0x4E, 0xf, 0xf, false));
  if (!valid) return;
  const int64_t rb = m >> 3;
  const int ml = (int)(m & 7);
  // chunk (quarter qa = 2*(b & 1) + c, k-half b >> 1) holds in dword
  // 2*(j & 1) + hh the class-j bytes of half word hh, j >> 1 == c
  unsigned char* tile = img + ((rb * G + g) * 64) * 32 + (b >> 1) * 16;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int qa = 2 * (b & 1) + c;
    *reinterpret_cast<u32x4*>(tile + (qa * 16 + ml) * 32) =
        u32x4{hi[2 * c][0], hi[2 * c][1], hi[2 * c + 1][0], hi[2 * c + 1][1]};
    *reinterpret_cast<u32x4*>(tile + (qa * 16 + 8 + ml) * 32) =
        u32x4{lo[2 * c][0], lo[2 * c][1], lo[2 * c + 1][0], lo[2 * c + 1][1]};
  }
  // scale of A row r, 32-weight block j (= word b) sits in lane r + 16 j
  unsigned char* sp = sc_img + ((rb * nspan + (g >> 2)) * 64) * 4 + (g & 3);
  sp[(ml + 16 * b) * 4] = (unsigned char)(sc + 127);
  sp[(8 + ml + 16 * b) * 4] = (unsigned char)(sc + 123);
  float* xs = xs_img + (rb * G + g) * 16;
  if (b == 0) xs[ml] = AFFINE ? X : -0.5f * X;
  if (b == 1) xs[8 + ml] = 0.0f;
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

template <bool AFFINE, bool MBF16, int TNB>
__global__ __launch_bounds__(kThreads) void q1_wide_kernel(WideArgs a) {
  constexpr int ROWS = TNB * 16;                   // weight rows of the workgroup
  constexpr int LOADS = (ROWS * 4 + kThreads - 1) / kThreads;  // 16-byte staging loads per thread
  __shared__ __align__(16) unsigned char wsm[2][ROWS * kRowB];
  __shared__ __align__(16) uint32_t ssm[2][ROWS * 2];  // 4 fp16/bf16 scales per row
  __shared__ __align__(16) uint32_t bsm[AFFINE ? 2 : 1][AFFINE ? ROWS * 2 : 2];
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
    {  // group sums: thread -> (row block, group, row)
      const int rbl = tid >> 6, g = 4 * sp + ((tid >> 4) & 3);
      const int rbg = tm * kWaves + rbl;
      xreg = (rbg < a.MB && g < a.G) ? a.xs_img[((int64_t)rbg * a.G + g) * 16 + (tid & 15)] : 0.0f;
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
      ssm[buf][2 * tid] = sreg[0];
      ssm[buf][2 * tid + 1] = sreg[1];
      if (AFFINE) {
        bsm[buf][2 * tid] = breg[0];
        bsm[buf][2 * tid + 1] = breg[1];
      }
    }
  };

  // ---- this wave's A operands for span sp (4 groups) ----
  v8i A[4];
  uint32_t scale_a = 0;
  auto a_load = [&](int sp, v8i (&Ao)[4], uint32_t& so) {
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int g = 4 * sp + gi;
      if (g < a.G) {  // (uniform)
        const u32x4* t = reinterpret_cast<const u32x4*>(a.img + (((int64_t)rb * a.G + g) * 64 + lane) * 32);
        const u32x4 h0 = t[0], h1 = t[1];
        Ao[gi] = v8i{(int)h0[0], (int)h0[1], (int)h0[2], (int)h0[3], (int)h1[0], (int)h1[1], (int)h1[2], (int)h1[3]};
      } else {
        Ao[gi] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
    so = a.sc_img[((int64_t)rb * a.nspan + sp) * 64 + lane];
  };

  v4f acc[TNB];
#pragma unroll
  for (int j = 0; j < TNB; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};

  stage_load(0);
  if (live) a_load(0, A, scale_a);
  stage_store(0);
  lds_barrier();

  for (int sp = 0; sp < a.nspan; ++sp) {
    const int buf = sp & 1;
    v8i An[4];
    uint32_t sn = 0;
    if (sp + 1 < a.nspan) {
      stage_load(sp + 1);
      if (live) a_load(sp + 1, An, sn);
    }
    if (live) {
      // groups past G (last span) have zero A operands, zero weights and zero
      // scales, so every span runs all 4 groups without branches
      // the LDS reads of column block j+1 are issued before block j's work
      auto rd_w = [&](int j) { return *reinterpret_cast<const u32x4*>(wsm[buf] + (j * 16 + nl) * kRowB + q * 16); };
      auto rd_s = [&](int j) { return *reinterpret_cast<const u32x2*>(&ssm[buf][2 * (j * 16 + nl)]); };
      auto rd_b = [&](int j) {
        return AFFINE ? *reinterpret_cast<const u32x2*>(&bsm[buf][2 * (j * 16 + nl)]) : u32x2{0u, 0u};
      };
      v4f XS[4];  // this wave's group sums of the span, rows 4q..4q+3
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) XS[gi] = reinterpret_cast<const v4f*>(&xsm[buf][(wave * 4 + gi) * 16])[q];
      v4f Dp[4];
      u32x2 s4p = {0u, 0u}, b4p = {0u, 0u};
      auto fma_block = [&](int j, const v4f (&Dv)[4], u32x2 sv4, u32x2 bv4) {
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          const float sv = meta_val<MBF16>(sv4[gi >> 1] >> (16 * (gi & 1)));
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[j][i] = fmaf(sv, Dv[gi][i], acc[j][i]);
          if (AFFINE) {
            const float bv = meta_val<MBF16>(bv4[gi >> 1] >> (16 * (gi & 1)));
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[j][i] = fmaf(bv, XS[gi][i], acc[j][i]);
          }
        }
      };
      u32x4 w4n = rd_w(0);  // word q of groups 0..3
      u32x2 s4n = rd_s(0), b4n = rd_b(0);
#pragma unroll
      for (int j = 0; j < TNB; ++j) {
        const u32x4 w4 = w4n;
        const u32x2 s4 = s4n, b4 = b4n;
        if (j + 1 < TNB) {
          w4n = rd_w(j + 1);
          s4n = rd_s(j + 1);
          b4n = rd_b(j + 1);
        }
        v4f D[4];
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          int Bv[8];
          q1_expand_b(w4[gi], Bv);
          const v8i B = {Bv[0], Bv[1], Bv[2], Bv[3], 0, 0, 0, 0};
          const v4f C = AFFINE ? v4f{0.f, 0.f, 0.f, 0.f} : XS[gi];
          if (gi == 0)
            D[0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[0], B, C, 0, 4, 0, (int)scale_a, 0, 0x7f7f7f7f);
          else if (gi == 1)
            D[1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[1], B, C, 0, 4, 1, (int)scale_a, 0, 0x7f7f7f7f);
          else if (gi == 2)
            D[2] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[2], B, C, 0, 4, 2, (int)scale_a, 0, 0x7f7f7f7f);
          else
            D[3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[3], B, C, 0, 4, 3, (int)scale_a, 0, 0x7f7f7f7f);
        }
        // the scale multiply-adds of block j-1 go after block j's products,
        // so they never wait for a product just issued
        if (j > 0) fma_block(j - 1, Dp, s4p, b4p);
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) Dp[gi] = D[gi];
        s4p = s4;
        b4p = b4;
      }
      fma_block(TNB - 1, Dp, s4p, b4p);
    }
    if (sp + 1 < a.nspan) stage_store(buf ^ 1);  // that buffer was last read before the previous barrier
    lds_barrier();
    if (sp + 1 < a.nspan && live) {
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        A[gi] = An[gi];
      }
      scale_a = sn;
    }
  }

  if (!live) return;
  // lane l of half ab: activation row 4*((l>>4)&1) + 2*ab + (l>>5) of the row
  // block (hi + lo added), weight row l & 15 of the column block
#pragma unroll
  for (int j = 0; j < TNB; ++j) {
    auto p01 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[j][0]), __float_as_uint(acc[j][1]), false, false);
    auto p23 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[j][2]), __float_as_uint(acc[j][3]), false, false);
    const float v0 = __uint_as_float(p01[0]) + __uint_as_float(p01[1]);
    const float v1 = __uint_as_float(p23[0]) + __uint_as_float(p23[1]);
    const int64_t n = n0 + j * 16 + nl;
    const int64_t mA = (int64_t)rb * 8 + 4 * ((lane >> 4) & 1) + (lane >> 5);
    if (n < a.N) {
      if (mA < a.M) store_out(a.out, a.out_dtype, mA * a.out_ld + n, v0);
      if (mA + 2 < a.M) store_out(a.out, a.out_dtype, (mA + 2) * a.out_ld + n, v1);
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
  p->MB = (int)((M + 7) / 8);
  p->mtiles = (p->MB + kWaves - 1) / kWaves;
  // column blocks per workgroup: the choice that keeps the most CUs busy in
  // the last round of workgroups (ties: the wider tile)
  const int cus = wide_device_cus();
  const int64_t nbk = (N + 15) / 16;
  const int cand[3] = {17, 16, 10};
  double best = -1.0;
  for (int tnb : cand) {
    if (affine && tnb == 17) continue;  // (its bias registers would spill)
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
  const size_t img = (size_t)p->MB * p->G * 2048;
  const size_t sc = (size_t)p->MB * p->nspan * 256;
  const size_t xs = (size_t)p->MB * p->G * 64;
  p->sc_off = (img + 255) / 256 * 256;
  p->xs_off = p->sc_off + (sc + 255) / 256 * 256;
  p->ws_bytes = p->xs_off + (xs + 255) / 256 * 256;
  return true;
}

hipError_t launch_wide(const WidePlan& p, const uint16_t* x, int64_t x_ld, const QMat& w, void* out, int32_t out_dtype,
                       int64_t out_ld, unsigned char* ws, hipStream_t s) {
  unsigned char* img = ws;
  unsigned char* sc = ws + p.sc_off;
  float* xs = reinterpret_cast<float*>(ws + p.xs_off);
  const dim3 ig((unsigned)((p.G + 63) / 64), (unsigned)(p.MB * 8));
  if (w.symmetric)
    hipLaunchKernelGGL((q1_act_image_kernel<false>), ig, dim3(256), 0, s, x, x_ld, p.M, p.G, p.nspan, img, sc, xs);
  else
    hipLaunchKernelGGL((q1_act_image_kernel<true>), ig, dim3(256), 0, s, x, x_ld, p.M, p.G, p.nspan, img, sc, xs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
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
