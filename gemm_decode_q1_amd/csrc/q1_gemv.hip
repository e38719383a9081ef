// Packed narrow-M Q1 matmul: the nibble-table kernel (the default for one
// activation row; 2..8 rows when the matrix-core plan rejects a shape or
// Q1_PACKED_KERNEL=table), instantiated for M = 1..8 at the end.
//
// y[m][n] = sum_k x[m][k] * w[n][k],  w = scale*bit + bias (symmetric:
// bias = -scale/2), for M <= 8 activation rows (Higgs PR #212, "What": narrow
// Q1 matmuls stay packed; rMLX issue #207: 32 weights per uint32, LSB first,
// one scale/bias per 128 weights).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "q1_device.h"
#include "q1_internal.h"

namespace q1 {

// ---------------------------------------------------------------------------
// Work decomposition.  A chunk is 32 consecutive words of a row (1024
// weights).  A wave processes one *pair* of output units at a time: lanes
// 0..31 handle unit 2j and lanes 32..63 unit 2j+1, lane s of a half owning
// word s of every chunk, so each half-wave load is 128 contiguous bytes of
// one row.  In single mode the units are rows 2j, 2j+1 of one matrix; in pair
// mode (FFN gate/up) they are row j of gate and row j of up.
//
// Lookup tables.  For a word holding weights k..k+31 and nibble i (weights
// k+4i..k+4i+3), the table entry for nibble value p is
//   symmetric: 1/2 * sum_b (p_b ? +x : -x)[k+4i+b]   (bias -scale/2 folded in)
//   affine:    sum_b p_b * x[k+4i+b]                  (bias term added per word)
// so a symmetric word contributes scale * sum_i T[i][nibble_i].  An affine
// word's codes have weights w1 = fl(scale + bias) and w0 = bias, of any
// relative size; the lookups run over the code d whose weight is larger in
// magnitude (the word is complemented when d = 0, so the table gives
// S_d = sum of x over the codes equal to d) and the word contributes
// (w_d - w_o) S_d + w_o X with X the word's activation sum: the rounding of X
// and of the fp32 table sums is then multiplied by the smaller weight.
// Tables live in LDS as [i/2][p][i&1][slot] floats: entry address
//   (i>>1)*4096 + p*256 + (i&1)*128 + slot*4,
// so a half-wave (32 distinct slots) always hits 32 distinct banks, whatever
// the nibble values.  The per-lane part p*256 + slot*4 is assembled by one
// v_perm_b32 from a nibble-per-byte copy of the word; (i, chunk, row of x) go
// into the instruction's immediate offset.  Per word: 3 ops to split the
// nibbles, 8 perms, 8 LDS reads, 7 adds, 1 convert, 1 FMA per row of x.
//
// Loads.  Packed words and metadata are read with raw buffer loads: one
// 32-bit offset per pair, chunk offsets as immediates.  A unit past the end of
// the range gets an offset beyond the buffer, which the hardware range check
// turns into zeros (scale 0: no contribution), so the hot loop has no masking.
//
// Split K.  A workgroup owns a range of units and a range of chunks
// (grid.y).  With more than one K range each range writes fp32 partial sums;
// a separate reduction launch adds them in a fixed order, so results do not
// depend on timing.
// ---------------------------------------------------------------------------

template <int M>
struct GemvCfg {
  static constexpr int KRMAX = gemv_krmax(M);                                   // chunks per K range
  static constexpr int CLB = gemv_chunk_block(M);                               // bytes per chunk block
  static constexpr int TAB_BYTES = (KRMAX - 1) * CLB + M * kTabBytes;
  static constexpr int NT = gemv_threads(M);
  static constexpr int WPE = (M == 1) ? 8 : 4;  // waves per SIMD the register budget targets
  // prefetch ring slots (pairs in flight + 1); one pair ahead is enough for
  // one activation row too (measured: 2 slots 5.6 us at K=5120, N=17408 and
  // 22.1 us on the tied head; 3 slots 6.0 and 23.0; 4 slots 7.6 and 26.5)
  static constexpr int R = 2;
};

constexpr uint32_t kBufWord3 = 0x00020000u;  // raw buffer descriptor, gfx9 family
constexpr uint32_t kOOB = 0x80000000u;       // offset that always fails the range check
constexpr int kNT = 2;                       // cache policy: non-temporal (words and metadata are streamed once)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, (int)kBufWord3);
}

// The compiler's writelane intrinsic (no clang builtin spells it for gfx9);
// the backend places the lane index in m0 itself.
extern "C" __device__ int q1_llvm_writelane(int src, int lane, int old) __asm("llvm.amdgcn.writelane.i32");

// Write the wave-uniform value v into lane `lane` of r (v_writelane_b32).
__device__ __forceinline__ float write_lane(float r, float v, int lane) {
  const int vi = __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v));
  const int li = __builtin_amdgcn_readfirstlane(lane);
  return __builtin_bit_cast(float, q1_llvm_writelane(vi, li, __builtin_bit_cast(int, r)));
}

// Sum over the 32 lanes of each half-wave; the total ends up in lanes 16..31
// (first half) and 48..63 (second half).
__device__ __forceinline__ float half_wave_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xf, 0xf, true));  // row_ror:8
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x124, 0xf, 0xf, true));  // row_ror:4
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x122, 0xf, 0xf, true));  // row_ror:2
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x121, 0xf, 0xf, true));  // row_ror:1
  // row_bcast:15 into rows 1 and 3: lanes 16..31 add lane 15, lanes 48..63 add lane 47
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xa, 0xf, false));
  return v;
}

// EXACT: every K range of this launch has exactly KRMAX chunks of 32 words
// (no ragged K, no short last range), so no chunk needs masking.
template <int M, bool AFFINE, bool MBF16, bool EXACT, bool PAIR>
__global__ __launch_bounds__(gemv_threads(M)) __attribute__((amdgpu_waves_per_eu(AFFINE ? 4 : GemvCfg<M>::WPE)))
void q1_gemv_kernel(GemvArgs a) {
  using C = GemvCfg<M>;
  constexpr int KRMAX = C::KRMAX;
  constexpr int NT = C::NT;
  constexpr int NW = NT / 64;
  __shared__ __align__(16) unsigned char smem[C::TAB_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int half = lane >> 5;
  const int slot = lane & 31;
  const int ks = blockIdx.y;
  const int c0 = (int)(((int64_t)ks * a.chunks) / a.KS);
  const int c1 = (int)(((int64_t)(ks + 1) * a.chunks) / a.KS);
  const int nc = c1 - c0;

  // unit indices fit in 31 bits (the plan refuses more than 2^29 rows)
  const int u0 = (int)blockIdx.x * (int)a.units_per_wg;
  const int u1 = (u0 + (int)a.units_per_wg < (int)a.units) ? u0 + (int)a.units_per_wg : (int)a.units;
  const int npairs = (u1 - u0 + 1) >> 1;

  // buffer resources (uniform); the plan keeps every buffer below 2^31 bytes
  const __amdgpu_buffer_rsrc_t rp0 = make_rsrc(a.p0, a.packed_bytes);
  const __amdgpu_buffer_rsrc_t rs0 = make_rsrc(a.s0, a.meta_bytes);
  const __amdgpu_buffer_rsrc_t rb0 = make_rsrc(AFFINE ? a.b0 : a.s0, a.meta_bytes);
  const __amdgpu_buffer_rsrc_t rp1 = make_rsrc(a.p1, a.packed_bytes);
  const __amdgpu_buffer_rsrc_t rs1 = make_rsrc(a.s1, a.meta_bytes);
  const __amdgpu_buffer_rsrc_t rb1 = make_rsrc(AFFINE ? a.b1 : a.s1, a.meta_bytes);

  struct Slot {
    uint32_t w[KRMAX];
    uint32_t s[KRMAX];
    uint32_t b[KRMAX];
  };

  // Byte offsets of this lane's first word / metadata element of pair j, or
  // kOOB (reads return 0) when the unit does not exist.  Pair j covers rows
  // row0 + s*j (s = 2 single, 1 pair mode), so the offsets are this lane's
  // offsets for pair 0 plus a wave-uniform step: one scalar multiply per pair
  // (the word step is 16 s gpr bytes, the metadata step an eighth of it).
  const uint32_t wi = (uint32_t)(c0 * kChunkWords + slot);
  const uint32_t row0 = (uint32_t)(PAIR ? (u0 >> 1) : u0 + half);
  const uint32_t ow0 = (row0 * (uint32_t)a.wpr + wi) * 4u;
  const uint32_t om0 = (row0 * (uint32_t)a.gpr + (wi >> 2)) * 2u;
  const uint32_t ostep = (uint32_t)(PAIR ? 1 : 2) * (uint32_t)a.wpr * 4u;
  auto offsets = [&](int j, uint32_t& ow, uint32_t& om) {
    const bool valid = (j < npairs) && (u0 + 2 * j + half < u1);
    const uint32_t d = (uint32_t)j * ostep;  // j is uniform across the wave
    ow = valid ? ow0 + d : kOOB;
    om = valid ? om0 + (d >> 3) : kOOB;
  };

  auto load = [&](Slot& sl, int j) {
    uint32_t ow, om;
    offsets(j, ow, om);
    if (!PAIR) {
#pragma unroll
      for (int cl = 0; cl < KRMAX; ++cl) {
        sl.w[cl] = __builtin_amdgcn_raw_buffer_load_b32(rp0, ow + cl * 128, 0, kNT);
        sl.s[cl] = __builtin_amdgcn_raw_buffer_load_b16(rs0, om + cl * 16, 0, kNT);
        if (AFFINE) sl.b[cl] = __builtin_amdgcn_raw_buffer_load_b16(rb0, om + cl * 16, 0, kNT);
      }
    } else {
      // gate rows in the first half-wave, up rows in the second: each load is
      // issued once per matrix with the other half's offsets out of range
      const uint32_t ow0 = half ? kOOB : ow, ow1 = half ? ow : kOOB;
      const uint32_t om0 = half ? kOOB : om, om1 = half ? om : kOOB;
#pragma unroll
      for (int cl = 0; cl < KRMAX; ++cl) {
        sl.w[cl] = __builtin_amdgcn_raw_buffer_load_b32(rp0, ow0 + cl * 128, 0, kNT) |
                   __builtin_amdgcn_raw_buffer_load_b32(rp1, ow1 + cl * 128, 0, kNT);
        sl.s[cl] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs0, om0 + cl * 16, 0, kNT) |
                   (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs1, om1 + cl * 16, 0, kNT);
        if (AFFINE)
          sl.b[cl] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rb0, om0 + cl * 16, 0, kNT) |
                     (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rb1, om1 + cl * 16, 0, kNT);
      }
    }
  };

  // ---- activation loads, then the first pair of weights; the tables; then
  // any other prefetched pairs (none with a 2-slot ring).  Loads retire from
  // the vector-memory counter in issue order, so the activations, issued
  // first, can be waited for (and the tables built) while the weights are
  // still in flight; and a wave stalls while issuing loads into a full memory
  // pipeline, so issuing more prefetched pairs before the tables delays them.
  constexpr int COMBOS = KRMAX * M;  // (chunk, row of x) tables
  constexpr int PASSES = (COMBOS * 256 + NT - 1) / NT;
  uint2 xv[PASSES];
  {
    const int i = (tid >> 5) & 7;
    const int ss = tid & 31;
#pragma unroll
    for (int q = 0; q < PASSES; ++q) {
      const int cm = (tid >> 8) + q * (NT / 256);
      const int cl = cm / M, m = cm - (cm / M) * M;
      const int k0 = (c0 + cl) * kChunkK + ss * 32 + i * 4;
      xv[q] = make_uint2(0u, 0u);
      if (cm < nc * M && k0 < a.K) xv[q] = *reinterpret_cast<const uint2*>(a.x + m * a.x_ld + k0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  constexpr int R = C::R;
  Slot buf[R];
  load(buf[0], wave);
  __builtin_amdgcn_sched_barrier(0);

  // ---- lookup tables for chunks [c0, c1) and every activation row
  {
    const int i = (tid >> 5) & 7;
    const int ss = tid & 31;
#pragma unroll
    for (int q = 0; q < PASSES; ++q) {
      const int cm = (tid >> 8) + q * (NT / 256);
      if (cm < COMBOS) {
        const int cl = cm / M, m = cm - (cm / M) * M;
        const float x0 = __uint_as_float(xv[q].x << 16), x1 = __uint_as_float(xv[q].x & 0xffff0000u);
        const float x2 = __uint_as_float(xv[q].y << 16), x3 = __uint_as_float(xv[q].y & 0xffff0000u);
        float L[4], H[4];
        if (AFFINE) {
          L[0] = 0.f; L[1] = x0; L[2] = x1; L[3] = x0 + x1;
          H[0] = 0.f; H[1] = x2; H[2] = x3; H[3] = x2 + x3;
        } else {
          const float ha = 0.5f * x0, hb = 0.5f * x1, hc = 0.5f * x2, hd = 0.5f * x3;
          L[0] = -ha - hb; L[1] = ha - hb; L[2] = hb - ha; L[3] = ha + hb;
          H[0] = -hc - hd; H[1] = hc - hd; H[2] = hd - hc; H[3] = hc + hd;
        }
        unsigned char* base = smem + cl * C::CLB + m * kTabBytes + (i >> 1) * 4096 + (i & 1) * 128 + ss * 4;
#pragma unroll
        for (int p = 0; p < 16; ++p) *reinterpret_cast<float*>(base + p * 256) = L[p & 3] + H[p >> 2];
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 1; r < R - 1; ++r) load(buf[r], wave + NW * r);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();

  // affine: sum of x over this lane's word of each chunk (entry p = 15 summed
  // over the 8 nibbles), kept in registers
  float xs[KRMAX][M];
#pragma unroll
  for (int cl = 0; cl < KRMAX; ++cl)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      xs[cl][m] = 0.f;
      if (AFFINE) {
        const unsigned char* base = smem + cl * C::CLB + m * kTabBytes + 15 * 256 + slot * 4;
#pragma unroll
        for (int i = 0; i < 8; ++i) xs[cl][m] += *reinterpret_cast<const float*>(base + (i >> 1) * 4096 + (i & 1) * 128);
      }
    }

  const uint32_t lanebase = (uint32_t)slot * 4u;

  auto compute = [&](const Slot& sl, int j, float (&res)[M], int b) {
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.f;
#pragma unroll
    for (int cl = 0; cl < KRMAX; ++cl) {
      uint32_t word = sl.w[cl];
      float sf = meta_to_f32<MBF16>(sl.s[cl]);
      float bf = 0.f;
      if (AFFINE) bf = meta_to_f32<MBF16>(sl.b[cl]);
      if (!EXACT) {
        // short last K range or ragged K: drop chunks/words outside the range
        const bool okc = (cl < nc) && ((c0 + cl) * kChunkWords + slot < a.wpr);
        sf = okc ? sf : 0.f;
        bf = okc ? bf : 0.f;
      }
      if (AFFINE) {  // sf <- w_d - w_o, bf <- w_o, word <- the codes equal to d
        const float w1 = sf + bf;
        const bool d1 = fabsf(w1) >= fabsf(bf);
        const float dw = w1 - bf;
        sf = d1 ? dw : -dw;
        bf = d1 ? bf : w1;
        word ^= d1 ? 0u : 0xffffffffu;
      }
      const uint32_t lo = word & 0x0f0f0f0fu;
      const uint32_t hi = (word >> 4) & 0x0f0f0f0fu;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const int off = cl * C::CLB + m * kTabBytes;  // compile-time
        const uint32_t lb = lanebase | ((uint32_t)(off >> 16) << 16);
        const unsigned char* tb = smem + (off & 0xffff);
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          // byte (i>>1) of lo/hi -> address byte 1; bytes 0 and 2 from lb
          const uint32_t sel = 0x03020400u | ((uint32_t)(4 + (i >> 1)) << 8);
          const uint32_t addr = __builtin_amdgcn_perm((i & 1) ? hi : lo, lb, sel);
          const float v = *reinterpret_cast<const float*>(tb + addr + (i >> 1) * 4096 + (i & 1) * 128);
          part = (i == 0) ? v : part + v;
        }
        acc[m] = __builtin_fmaf(sf, part, acc[m]);
        if (AFFINE) acc[m] = __builtin_fmaf(bf, xs[cl][m], acc[m]);
      }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = half_wave_sum(acc[m]);
    // Park the pair's results in lane 2b (+1) of res[m] (b = position in the
    // current batch of 32 pairs); stores happen once per batch, outside the
    // hot path.  Pair mode parks h = SiLU(gate) * up in lane b.
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float v0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, acc[m]), 31));
      const float v1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, acc[m]), 63));
      if (PAIR && a.KS == 1) {
        res[m] = write_lane(res[m], silu_f32(v0) * v1, b);
      } else {
        res[m] = write_lane(res[m], v0, 2 * b);
        res[m] = write_lane(res[m], v1, 2 * b + 1);
      }
    }
  };

  // Store the parked results of pairs j = wave + NW*(t0 + b), b < nb.
  auto flush = [&](const float (&res)[M], int t0, int nb) {
    if (PAIR && a.KS == 1) {
      const int j = wave + NW * (t0 + lane);
      if (lane < nb) {
        const int64_t n = (int64_t)(u0 >> 1) + j;
#pragma unroll
        for (int m = 0; m < M; ++m) static_cast<uint16_t*>(a.out)[m * a.out_ld + n] = (uint16_t)f32_to_bf16_bits(res[m]);
      }
    } else {
      const int j = wave + NW * (t0 + (lane >> 1));
      const int u = u0 + 2 * j + (lane & 1);
      if (lane < 2 * nb && u < u1) {
        if (a.KS == 1) {
#pragma unroll
          for (int m = 0; m < M; ++m) store_out(a.out, a.out_dtype, m * a.out_ld + (int64_t)u, res[m]);
        } else {
#pragma unroll
          for (int m = 0; m < M; ++m) a.partial[((int64_t)ks * M + m) * a.units + (int64_t)u] = res[m];
        }
      }
    }
  };

  // ---- stream the pairs of this wave, R-1 pairs of prefetch ahead
  float res[M];
#pragma unroll
  for (int m = 0; m < M; ++m) res[m] = 0.f;
  int tb = 0;  // first pair index (in units of this wave's pairs) of the open batch
  for (int t = 0; wave + NW * t < npairs; t += R) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int j = wave + NW * (t + r);
      if (j >= npairs) break;  // uniform across the wave
      load(buf[(r + R - 1) % R], j + NW * (R - 1));
      compute(buf[r], j, res, t + r - tb);
      if (t + r - tb == 31) {  // batch full (uniform)
        flush(res, tb, 32);
        tb = t + r + 1;
      }
    }
  }
  {
    int nb = 0;  // pairs in the open batch
    while (wave + NW * (tb + nb) < npairs) ++nb;
    if (nb > 0) flush(res, tb, nb);
  }
}

template <int M, bool AFFINE, bool MBF16, bool EXACT, bool PAIR>
static hipError_t launch_gemv_t(const GemvPlan& plan, const GemvArgs& args, hipStream_t stream) {
  hipLaunchKernelGGL((q1_gemv_kernel<M, AFFINE, MBF16, EXACT, PAIR>), dim3(plan.wgs_x, plan.KS),
                     dim3(gemv_threads(M)), 0, stream, args);
  return hipGetLastError();
}

template <int M, bool AFFINE, bool MBF16>
static hipError_t launch_gemv_e(const GemvPlan& plan, const GemvArgs& args, hipStream_t stream) {
  const bool exact = plan.exact != 0;
  if (args.pair)
    return exact ? launch_gemv_t<M, AFFINE, MBF16, true, true>(plan, args, stream)
                 : launch_gemv_t<M, AFFINE, MBF16, false, true>(plan, args, stream);
  return exact ? launch_gemv_t<M, AFFINE, MBF16, true, false>(plan, args, stream)
               : launch_gemv_t<M, AFFINE, MBF16, false, false>(plan, args, stream);
}

template <int M>
hipError_t launch_gemv_m(const GemvPlan& plan, const GemvArgs& args, bool affine, bool mbf16, hipStream_t stream) {
  if (affine) return mbf16 ? launch_gemv_e<M, true, true>(plan, args, stream) : launch_gemv_e<M, true, false>(plan, args, stream);
  return mbf16 ? launch_gemv_e<M, false, true>(plan, args, stream) : launch_gemv_e<M, false, false>(plan, args, stream);
}

template hipError_t launch_gemv_m<1>(const GemvPlan&, const GemvArgs&, bool, bool, hipStream_t);
template hipError_t launch_gemv_m<2>(const GemvPlan&, const GemvArgs&, bool, bool, hipStream_t);
template hipError_t launch_gemv_m<3>(const GemvPlan&, const GemvArgs&, bool, bool, hipStream_t);
template hipError_t launch_gemv_m<4>(const GemvPlan&, const GemvArgs&, bool, bool, hipStream_t);
template hipError_t launch_gemv_m<5>(const GemvPlan&, const GemvArgs&, bool, bool, hipStream_t);
template hipError_t launch_gemv_m<6>(const GemvPlan&, const GemvArgs&, bool, bool, hipStream_t);
template hipError_t launch_gemv_m<7>(const GemvPlan&, const GemvArgs&, bool, bool, hipStream_t);
template hipError_t launch_gemv_m<8>(const GemvPlan&, const GemvArgs&, bool, bool, hipStream_t);

}  // namespace q1
