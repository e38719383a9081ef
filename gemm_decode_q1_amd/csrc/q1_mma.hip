// Packed narrow-M Q1 matmul on the CDNA4 matrix cores: one launch of the
// stage in q1_mma_stage.h (which describes the scheme), its plan and its
// launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "q1_mma_stage.h"

namespace q1 {
namespace {

template <bool AFFINE, bool MBF16, bool PAIR, bool SC128, int MR, int RT>
__global__ __launch_bounds__(kThreads) void q1_mma_kernel(MmaArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  __shared__ int last_flag;
  __shared__ int wave_k0[kNW];
  mma_stage<AFFINE, MBF16, PAIR, SC128, MR, RT>(a, (int)(blockIdx.x % (unsigned)a.S), (int)(blockIdx.x / (unsigned)a.S),
                                                lds, &last_flag, wave_k0, NoWait{});
}

// Split K: the S segments' partial sums [S][M][NMAT][N], added in segment
// order (the stream runs this after the matmul launch); pair mode writes
// h = bf16(SiLU(g) * u).  The loads go out four at a time.
template <bool PAIR>
__global__ __launch_bounds__(256) void q1_mma_reduce(const float* __restrict__ partial, int S, int M, int64_t N,
                                                     void* out, int32_t out_dtype, int64_t out_ld) {
  constexpr int NMAT = PAIR ? 2 : 1;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)M * N) return;
  const int m = (int)(i / N);
  const int64_t n = i - (int64_t)m * N;
  const int64_t sstep = (int64_t)M * NMAT * N;
  float v[NMAT];
#pragma unroll
  for (int mt = 0; mt < NMAT; ++mt) {
    const float* pp = partial + ((int64_t)m * NMAT + mt) * N + n;
    float sum = 0.0f;
    for (int s2 = 0; s2 < S; s2 += 4) {  // a short last batch re-reads segment S-1 and drops it
      const int sl = S - 1;
      const float p0 = pp[s2 * sstep], p1 = pp[min(s2 + 1, sl) * sstep], p2 = pp[min(s2 + 2, sl) * sstep],
                  p3 = pp[min(s2 + 3, sl) * sstep];
      sum += p0;
      if (s2 + 1 < S) sum += p1;
      if (s2 + 2 < S) sum += p2;
      if (s2 + 3 < S) sum += p3;
    }
    v[mt] = sum;
  }
  if (PAIR)
    static_cast<uint16_t*>(out)[m * out_ld + n] = (uint16_t)f32_to_bf16_bits(silu_f32(v[0]) * v[1]);
  else
    store_out(out, out_dtype, m * out_ld + n, v[0]);
}

template <bool AFFINE, bool MBF16, bool PAIR, bool SC128, int MR, int RT>
hipError_t launch_k(const MmaPlan& p, const MmaArgs& a, hipStream_t s) {
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&q1_mma_kernel<AFFINE, MBF16, PAIR, SC128, MR, RT>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 64);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((q1_mma_kernel<AFFINE, MBF16, PAIR, SC128, MR, RT>), dim3((unsigned)p.wgs), dim3(kThreads),
                     p.lds_bytes, s, a);
  if (a.S > 1) {
    const int64_t n = (int64_t)a.M * a.N;
    hipLaunchKernelGGL((q1_mma_reduce<PAIR>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.partial, a.S, a.M,
                       a.N, a.out, a.out_dtype, a.out_ld);
  }
  return hipGetLastError();
}

// Live accumulator rows per lane quarter (MR) and affine row tiles (RT).
template <bool AFFINE, bool MBF16, bool PAIR, bool SC128>
hipError_t launch_r(const MmaPlan& p, const MmaArgs& a, hipStream_t s) {
  if constexpr (AFFINE) {
    if (a.M > 4) return launch_k<AFFINE, MBF16, PAIR, SC128, 4, 2>(p, a, s);
    if constexpr (PAIR) {
      return launch_k<AFFINE, MBF16, PAIR, SC128, 4, 1>(p, a, s);
    } else {
      if (a.M > 2) return launch_k<AFFINE, MBF16, PAIR, SC128, 4, 1>(p, a, s);
      return a.M == 1 ? launch_k<AFFINE, MBF16, PAIR, SC128, 1, 1>(p, a, s)
                      : launch_k<AFFINE, MBF16, PAIR, SC128, 2, 1>(p, a, s);
    }
  } else if constexpr (PAIR) {
    return launch_k<AFFINE, MBF16, PAIR, SC128, 4, 1>(p, a, s);
  } else {
    // (the full image is the four-row layout: its extra rows are never read)
    if (a.M > 2 || p.rb == 8) return launch_k<AFFINE, MBF16, PAIR, SC128, 4, 1>(p, a, s);
    return a.M == 1 ? launch_k<AFFINE, MBF16, PAIR, SC128, 1, 1>(p, a, s)
                    : launch_k<AFFINE, MBF16, PAIR, SC128, 2, 1>(p, a, s);
  }
}

template <bool AFFINE, bool MBF16, bool PAIR>
hipError_t launch_t(const MmaPlan& p, const MmaArgs& a, hipStream_t s) {
  return (a.G % 8 == 0) ? launch_r<AFFINE, MBF16, PAIR, true>(p, a, s) : launch_r<AFFINE, MBF16, PAIR, false>(p, a, s);
}

}  // namespace

bool plan_mma_split(int M, int64_t N, int64_t K, bool pair, bool affine, int S, int64_t P, MmaPlan* c,
                    bool full_image) {
  const int nmat = pair ? 2 : 1;
  c->M = M;
  c->pair = pair ? 1 : 0;
  c->G = (int)(K / 128);
  c->nspan = (c->G + 3) / 4;
  c->ntiles = (N + 15) / 16;
  const int ndsp = (c->nspan + 1) / 2;  // double spans
  if (S < 1 || S > ndsp || P < 1) return false;
  const int kds = (ndsp + S - 1) / S;
  c->S = (ndsp + kds - 1) / kds;
  if (c->S != S) return false;  // same split as a smaller S
  c->KSP = 2 * kds;
  c->P = (int)std::min<int64_t>(P, c->ntiles);
  c->nb = (int)((c->ntiles + c->P - 1) / c->P);  // tiles per workgroup (at most)
  c->wgs = (int64_t)c->S * c->P;
  // Tiles one wave's item range [i0, i1) touches: floor((i1-1)/nds) -
  // floor(i0/nds) + 1 < (i1-1-i0)/nds + 2 < nbp/8 + 2 for every workgroup
  // size nbp <= nb and segment length nds, so at most ceil(nb/8) + 1.
  c->TW = (int)std::min<int64_t>(c->nb, (c->nb + kNW - 1) / kNW + 1);
  const int rb = (pair || M > 2 || full_image) ? 8 : M;
  c->rb = affine ? 8 : rb;
  const size_t span = affine ? (size_t)aff_span_bytes(M > 4 ? 2 : 1) : (size_t)span_bytes(rb);
  const size_t scratch = (size_t)kNW * nmat * kScrDwords * 4;
  c->red_bytes = (size_t)kNW * c->TW * nmat * 512;
  c->lds_bytes = (size_t)c->KSP * span + c->red_bytes + scratch;
  if (c->lds_bytes > 160 * 1024 - 64 || (int64_t)M * c->KSP * 16 > (int64_t)kPrepRounds * kThreads) return false;
  if ((int64_t)c->nb * 128 >= ((int64_t)1 << 22)) return false;  // result-slot index arithmetic
  c->partial_floats = c->S > 1 ? (size_t)c->S * M * N * nmat : 0;
  return true;
}

bool plan_mma(int M, int64_t N, int64_t K, bool pair, bool affine, MmaPlan* p, const char** why) {
  if (M < 1 || M > 8) {
    *why = "matrix-core packed path handles 1..8 activation rows";
    return false;
  }
  if (N < 1 || K < 128 || K % 128 != 0) {
    *why = "bad shape";
    return false;
  }
  if (N * (K / 8) >= ((int64_t)1 << 31) || N * (K / 128) * 2 >= ((int64_t)1 << 31) ||
      (int64_t)M * K * 2 >= ((int64_t)1 << 31)) {
    *why = "matrix too large for 32-bit buffer offsets (split it along N)";
    return false;
  }
  const int cus = device_cus();
  const int ndsp = ((int)(K / 128) + 7) / 8;
  // Number of K segments S: among the splits whose LDS image, result slots
  // and scratch fit, the one with the fewest items in the busiest workgroup
  // (tiles are whole per workgroup, so S also balances the work), where a
  // split (the partial sums' round trips at the end, S partials per result)
  // counts as 6 + S/2 items (measured on the shapes with 17408-weight rows).
  // With two activation rows the compact image (live A rows only) holds
  // longer K segments, the full one is faster per item (K=5120, N=17408:
  // 7.8 -> 7.4 us): the full image wins ties.
  MmaPlan best;
  int64_t best_cost = -1;
  const int layouts = (M == 2 && !pair && !affine) ? 2 : 1;
  for (int full = layouts - 1; full >= 0; --full) {
    for (int S = 1; S <= ndsp; ++S) {
      MmaPlan c;
      if (!plan_mma_split(M, N, K, pair, affine, S, cus / S > 0 ? cus / S : 1, &c, full != 0)) continue;
      const int64_t cost = (int64_t)c.nb * (c.KSP / 2) + (c.S > 1 ? 6 + c.S / 2 : 0);
      if (best_cost < 0 || cost < best_cost) {
        best = c;
        best_cost = cost;
      }
    }
  }
  if (best_cost < 0) {
    *why = "LDS budget exceeded";
    return false;
  }
  *p = best;
  return true;
}

MmaArgs mma_args(const MmaPlan& p, const uint16_t* x, int64_t x_ld, const QMat& a, const QMat* b, void* out,
                 int32_t out_dtype, int64_t out_ld, float* partial, uint32_t* counters) {
  MmaArgs g;
  g.x = x;
  g.x_ld = x_ld;
  g.p0 = a.packed;
  g.s0 = a.scales;
  g.b0 = a.biases;
  g.p1 = b ? b->packed : a.packed;
  g.s1 = b ? b->scales : a.scales;
  g.b1 = b ? b->biases : a.biases;
  g.N = a.N;
  g.M = p.M;
  g.K = (int32_t)a.K;
  g.G = p.G;
  g.nspan = p.nspan;
  g.S = p.S;
  g.KSP = p.KSP;
  g.P = p.P;
  g.nb = p.nb;
  g.TW = p.TW;
  g.red_bytes = (uint32_t)p.red_bytes;
  g.x_bytes = (uint32_t)(((p.M - 1) * x_ld + a.K) * 2);
  g.packed_bytes = (uint32_t)(a.N * (a.K / 8));
  g.meta_bytes = (uint32_t)(a.N * (a.K / 128) * 2);
  g.out_dtype = out_dtype;
  g.out = out;
  g.out_ld = out_ld;
  g.partial = partial;
  g.counters = counters;
  return g;
}

hipError_t launch_mma(const MmaPlan& p, const uint16_t* x, int64_t x_ld, const QMat& a, const QMat* b, void* out,
                      int32_t out_dtype, int64_t out_ld, float* partial, hipStream_t s) {
  const MmaArgs g = mma_args(p, x, x_ld, a, b, out, out_dtype, out_ld, partial, nullptr);
  const bool affine = !a.symmetric, mbf16 = a.meta_bf16 != 0, pair = b != nullptr;
  if (pair) {
    if (affine) return mbf16 ? launch_t<true, true, true>(p, g, s) : launch_t<true, false, true>(p, g, s);
    return mbf16 ? launch_t<false, true, true>(p, g, s) : launch_t<false, false, true>(p, g, s);
  }
  if (affine) return mbf16 ? launch_t<true, true, false>(p, g, s) : launch_t<true, false, false>(p, g, s);
  return mbf16 ? launch_t<false, true, false>(p, g, s) : launch_t<false, false, false>(p, g, s);
}

}  // namespace q1
