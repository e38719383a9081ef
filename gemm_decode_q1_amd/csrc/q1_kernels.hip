// HIP kernels of the packed Q1 decode path for gfx950 (MI355X, CDNA4).
//
// Format and operations: rMLX issue #207 ("The good news -- packing is
// standard": 32 weights per uint32, one scale/bias per 128 weights), Cactus
// PR #775 (commit notes: linear LSB layout), Higgs PR #212 ("What", "Why",
// "Limitations": w = scale*bit + bias, symmetric bias = -scale/2, packed
// narrow-M matmul, dense fallback for wide M, fused dense FFN).
//
// Kernels
//   q1_dequant_kernel  bit-exact dequantisation of whole matrices or of
//                      gathered rows (embedding lookup).
//   q1_gemv_kernel     packed narrow-M (M <= 8) matmul: nibble lookup tables
//                      of the activations in LDS, one table read per 4
//                      weights, fp32 accumulation.
//   q1_gemm_bf16       wide-M fallback: bf16 MFMA GEMM on the dequantised
//                      matrix, fp32 accumulation.
//   q1_silu_mul        h = bf16(SiLU(g) * u) for the unfused FFN paths.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>

#include "q1_internal.h"
#include "q1_device.h"

namespace q1 {

// ---------------------------------------------------------------------------
// Dequantisation / row gather.  A piece is 8 consecutive outputs of a row (16
// bytes for 16-bit outputs), so a wave stores 1 KB contiguous.  Per group only
// two values exist: v0 = fl(fl(s*0) + b) and v1 = fl(s + b); they are rounded
// once and selected by the bits.  A thread takes kDqU pieces, stride apart,
// and issues all their loads (ids first, then words and metadata) before any
// store, so the id -> word -> store chain of one piece overlaps the others'.
// The row of piece t is t / per_row by a multiply-high and shift (DivMagic,
// exact for every 32-bit t; the launch keeps T * per_row below 2^32).
// ---------------------------------------------------------------------------

constexpr int kDqU = 4;

// q = floor(t / d) = (umulhi(t, m) + t) >> l for 0 <= t < 2^32, with
// l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1 (round-up method).
struct DivMagic {
  uint32_t m, l;
};

static DivMagic div_magic(uint32_t d) {
  uint32_t l = 0;
  while (((uint64_t)1 << l) < d) ++l;
  const uint64_t m = ((((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d) + 1;
  return DivMagic{(uint32_t)m, l};
}

__device__ __forceinline__ uint32_t div_by(uint32_t t, DivMagic dm) {
  return (uint32_t)(((uint64_t)__umulhi(t, dm.m) + t) >> dm.l);
}

typedef float f32x4_st __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_st __attribute__((ext_vector_type(4)));

// 16-byte output store.  Gathered rows are written with the non-temporal
// hint (measured 22 % faster for 4096 rows of K = 5120); a whole dequantised
// matrix keeps normal stores, since it usually feeds a product right away and
// (at 178 MB for the FFN shapes) can stay in the last-level cache for it.
template <bool NT, typename V>
__device__ __forceinline__ void store16(V* p, V v) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

// GATHER: rows are selected by `ids` (embedding lookup), else rows 0..T-1.
template <int OUT, bool MBF16, bool GATHER>
__global__ __launch_bounds__(256) void q1_dequant_kernel(const uint32_t* __restrict__ packed,
                                                         const uint16_t* __restrict__ scales,
                                                         const uint16_t* __restrict__ biases, int symmetric,
                                                         int64_t nrows, int64_t K, const void* __restrict__ ids,
                                                         int ids64, uint32_t total, DivMagic per_row_div,
                                                         void* __restrict__ out) {
  const uint32_t per_row = (uint32_t)(K >> 3);
  const int64_t wpr = K >> 5, gpr = K >> 7;
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t t0 = blockIdx.x * blockDim.x + threadIdx.x; t0 < total; t0 += kDqU * stride) {
    uint32_t r[kDqU], piece[kDqU];
    int64_t row[kDqU];
    bool ok[kDqU];
#pragma unroll
    for (int u = 0; u < kDqU; ++u) {
      const uint32_t t = t0 + (uint32_t)u * stride;  // < 2^32: total + kDqU * stride fits (launch)
      r[u] = div_by(t, per_row_div);
      piece[u] = t - r[u] * per_row;
      row[u] = r[u];
      if (GATHER && t < total)
        row[u] = ids64 ? static_cast<const int64_t*>(ids)[r[u]] : (int64_t) static_cast<const int32_t*>(ids)[r[u]];
    }
    uint32_t word[kDqU], sb[kDqU], bb[kDqU];
#pragma unroll
    for (int u = 0; u < kDqU; ++u) {
      const uint32_t t = t0 + (uint32_t)u * stride;
      ok[u] = t < total && row[u] >= 0 && row[u] < nrows;
      word[u] = 0u;
      sb[u] = 0u;
      bb[u] = 0u;
      if (ok[u]) {
        const int64_t g = row[u] * gpr + (piece[u] >> 4);
        word[u] = packed[row[u] * wpr + (piece[u] >> 2)];
        sb[u] = scales[g];
        if (!symmetric) bb[u] = biases[g];
      }
    }
#pragma unroll
    for (int u = 0; u < kDqU; ++u) {
      const uint32_t t = t0 + (uint32_t)u * stride;
      if (t >= total) continue;
      const uint32_t bits = ok[u] ? (word[u] >> (8 * (piece[u] & 3u))) & 0xffu : 0u;
      float v0 = 0.0f, v1 = 0.0f;
      if (ok[u]) {
        const float s = meta_to_f32<MBF16>(sb[u]);
        const float b = symmetric ? -0.5f * s : meta_to_f32<MBF16>(bb[u]);
        v0 = __builtin_fmaf(s, 0.0f, b);
        v1 = __builtin_fmaf(s, 1.0f, b);
      }
      const int64_t o = (int64_t)r[u] * K + (int64_t)piece[u] * 8;
      if (OUT == F32) {
        float vals[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) vals[j] = ((bits >> j) & 1u) ? v1 : v0;
        f32x4_st* dst = reinterpret_cast<f32x4_st*>(static_cast<float*>(out) + o);
        store16<GATHER>(dst, f32x4_st{vals[0], vals[1], vals[2], vals[3]});
        store16<GATHER>(dst + 1, f32x4_st{vals[4], vals[5], vals[6], vals[7]});
      } else {
        const uint32_t o0 = (OUT == BF16) ? f32_to_bf16_bits(v0) : f32_to_f16_bits(v0);
        const uint32_t o1 = (OUT == BF16) ? f32_to_bf16_bits(v1) : f32_to_f16_bits(v1);
        uint32_t d[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t lo = ((bits >> (2 * j)) & 1u) ? o1 : o0;
          const uint32_t hi = ((bits >> (2 * j + 1)) & 1u) ? o1 : o0;
          d[j] = lo | (hi << 16);
        }
        store16<GATHER>(reinterpret_cast<u32x4_st*>(static_cast<uint16_t*>(out) + o), u32x4_st{d[0], d[1], d[2], d[3]});
      }
    }
  }
}

// ---------------------------------------------------------------------------
// h = bf16(SiLU(g) * u)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void q1_silu_mul(const float* __restrict__ g, const float* __restrict__ u,
                                                   uint16_t* __restrict__ h, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    h[i] = (uint16_t)f32_to_bf16_bits(silu_f32(g[i]) * u[i]);
}

// ---------------------------------------------------------------------------
// Wide-M fallback: C[M, N] = A[M, K] * B[N, K]^T, bf16 in, fp32 accumulate,
// with v_mfma_f32_16x16x32_bf16.  Workgroup tile 128 x 128, K step 64, four
// waves in a 2 x 2 arrangement of 64 x 64 wave tiles (4 x 4 MFMA tiles each).
// LDS rows are padded to 72 bf16 so that 16-byte fragment reads of
// consecutive rows fall in different banks.  Tiles are visited so that the
// M-tiles sharing one N-tile run on the same XCD at the same time.
// ---------------------------------------------------------------------------

typedef short bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int GBM = 128, GBN = 128, GBK = 64, GLD = GBK + 8;

__global__ __launch_bounds__(256) void q1_gemm_bf16(const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bm,
                                                    int64_t M, int64_t N, int64_t K, void* __restrict__ Cout,
                                                    int32_t c_dtype, int tiles_m, int tiles_n) {
  __shared__ __align__(16) uint16_t As[GBM * GLD];
  __shared__ __align__(16) uint16_t Bs[GBN * GLD];

  // XCD-aware tile order: workgroups are dealt round-robin to 8 XCDs, so map
  // consecutive logical tiles to the same XCD.
  const int nwg = tiles_m * tiles_n;
  const int bid = blockIdx.x;
  int logical = bid;
  if ((nwg & 7) == 0) logical = (bid & 7) * (nwg >> 3) + (bid >> 3);
  const int tm = logical % tiles_m;
  const int tn = logical / tiles_m;
  const int64_t m0 = (int64_t)tm * GBM, n0 = (int64_t)tn * GBN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = (wave & 1) * 64, wn = (wave >> 1) * 64;

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // global -> register staging: each thread moves 4 x 16 B of A and of B
  uint4 ra[4], rb[4];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = (tid >> 3) + 32 * r;
      const int col = (tid & 7) * 8;
      const int64_t gm = m0 + row, gn = n0 + row;
      ra[r] = (gm < M) ? *reinterpret_cast<const uint4*>(A + gm * K + k0 + col) : make_uint4(0, 0, 0, 0);
      rb[r] = (gn < N) ? *reinterpret_cast<const uint4*>(Bm + gn * K + k0 + col) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = (tid >> 3) + 32 * r;
      const int col = (tid & 7) * 8;
      *reinterpret_cast<uint4*>(As + row * GLD + col) = ra[r];
      *reinterpret_cast<uint4*>(Bs + row * GLD + col) = rb[r];
    }
  };

  gload(0);
  for (int64_t k0 = 0; k0 < K; k0 += GBK) {
    __syncthreads();  // previous tile fully consumed
    sstore();
    __syncthreads();
    if (k0 + GBK < K) gload(k0 + GBK);
#pragma unroll
    for (int kk = 0; kk < GBK; kk += 32) {
      bf16x8_t af[4], bfr[4];
      const int r16 = lane & 15;
      const int kq = (lane >> 4) * 8;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(As + (wm + i * 16 + r16) * GLD + kk + kq);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(Bs + (wn + j * 16 + r16) * GLD + kk + kq);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // D layout: lane holds rows (lane>>4)*4 + e, column lane & 15 of each 16 x 16 tile
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn + j * 16 + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = m0 + wm + i * 16 + (lane >> 4) * 4 + e;
        if (row < M && col < N) store_out(Cout, c_dtype, row * N + col, acc[i][j][e]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Split-K reduction: partial sums [KS][M][units] -> y (single) or h (pair),
// adding the K ranges in a fixed order.  Runs as its own launch after the
// packed kernel, so the kernel boundary orders the partial stores.
// ---------------------------------------------------------------------------
template <int M>
__global__ __launch_bounds__(256) void q1_splitk_reduce(const float* __restrict__ partial, int KS, int64_t units,
                                                        int pair, void* __restrict__ out, int32_t out_dtype,
                                                        int64_t out_ld, int64_t units_per_block) {
  const int64_t u0 = (int64_t)blockIdx.x * units_per_block;
  const int64_t u1 = (u0 + units_per_block < units) ? u0 + units_per_block : units;
  splitk_finish<M>(partial, KS, units, pair, out, out_dtype, out_ld, u0, u1, threadIdx.x, 256);
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------

int device_cus() {
  // cached per device id; the plans of every kernel size their grids by it
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev < 0 || dev >= 64) {
    int v = 0;
    return hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0 ? v : 256;
  }
  int cus = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
  if (cus == 0) {
    int v = 0;
    cus = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0 ? v : 256;
    __atomic_store_n(&cache[dev], cus, __ATOMIC_RELAXED);
  }
  return cus;
}

bool plan_gemv(int M, int64_t N, int64_t K, bool pair, bool affine, GemvPlan* p, const char** why) {
  (void)affine;
  if (M < 1 || M > 8) {
    *why = "packed kernel serves 1..8 rows";
    return false;
  }
  if (N * (K / 8) >= ((int64_t)1 << 31) || N * (K / 64) >= ((int64_t)1 << 31)) {
    *why = "packed matrix too large for one packed launch (2 GiB of packed words)";
    return false;
  }
  p->M = M;
  p->chunks = (int)((K + kChunkK - 1) / kChunkK);
  const int krmax = gemv_krmax(M);
  p->KS = (p->chunks + krmax - 1) / krmax;
  p->KR = (p->chunks + p->KS - 1) / p->KS;
  p->exact = (K % kChunkK == 0 && p->chunks % krmax == 0) ? 1 : 0;
  p->units = pair ? 2 * N : N;
  if (p->units >= ((int64_t)1 << 30)) {
    *why = "too many rows for the packed kernel (limit 2^29)";
    return false;
  }
  p->lds_bytes = (size_t)gemv_lds_bytes(M);
  p->threads = gemv_threads(M);
  // Workgroups: as many as are resident at once, the units split evenly over
  // them (an even count each, so gate/up pairs never straddle two
  // workgroups).  A second round of workgroups on a few CUs would double
  // those CUs' work, so the count never exceeds the resident slots.  A
  // second workgroup per CU (when the tables leave room for it) builds the
  // same tables again and launches twice the waves: it pays only when each CU
  // has many rows to stream (measured: one per CU at 68 rows per CU, FFN
  // up/gate; two at 594, the tied head).
  const int cus = device_cus();
  const bool two = (int)((160 * 1024) / p->lds_bytes) >= 2 && p->units >= (int64_t)256 * cus;
  const int64_t slots = (int64_t)cus * (two ? 2 : 1);
  const int64_t wx = slots / p->KS > 0 ? slots / p->KS : 1;
  int64_t upw = (p->units + wx - 1) / wx;
  upw += upw & 1;
  if (upw < 2) upw = 2;
  p->units_per_wg = upw;
  p->wgs_x = (int)((p->units + upw - 1) / upw);
  p->partial_floats = (p->KS > 1) ? (size_t)p->KS * M * p->units : 0;
  return true;
}

template <int M>
static hipError_t launch_reduce_m(const GemvPlan& plan, const GemvArgs& g, hipStream_t stream) {
  const int64_t upb = 512;  // even, so gate/up pairs never straddle blocks
  const int64_t blocks = (plan.units + upb - 1) / upb;
  hipLaunchKernelGGL(q1_splitk_reduce<M>, dim3((unsigned)blocks), dim3(256), 0, stream, g.partial, g.KS, g.units,
                     g.pair, g.out, g.out_dtype, g.out_ld, upb);
  return hipGetLastError();
}

hipError_t launch_gemv(const GemvPlan& plan, const uint16_t* x, int64_t x_ld, const QMat& a, const QMat* b, void* out,
                       int32_t out_dtype, int64_t out_ld, float* partial, hipStream_t stream) {
  GemvArgs g{};
  g.x = x;
  g.x_ld = x_ld;
  g.p0 = a.packed;
  g.s0 = a.scales;
  g.b0 = a.biases;
  g.p1 = b ? b->packed : a.packed;
  g.s1 = b ? b->scales : a.scales;
  g.b1 = b ? b->biases : a.biases;
  g.N = a.N;
  g.K = (int32_t)a.K;
  g.wpr = (int32_t)(a.K / 32);
  g.gpr = (int32_t)(a.K / 128);
  g.chunks = plan.chunks;
  g.KS = plan.KS;
  g.pair = b ? 1 : 0;
  g.full_chunks = (int32_t)(a.K / kChunkK);
  g.units = plan.units;
  g.units_per_wg = plan.units_per_wg;
  g.packed_bytes = (uint32_t)(a.N * (a.K / 8));
  g.meta_bytes = (uint32_t)(a.N * (a.K / 128) * 2);
  g.out_dtype = out_dtype;
  g.out = out;
  g.out_ld = out_ld;
  g.partial = partial;
  const bool affine = !a.symmetric;
  const bool mbf16 = a.meta_bf16 != 0;
  hipError_t e;
  switch (plan.M) {
    case 1: e = launch_gemv_m<1>(plan, g, affine, mbf16, stream); break;
    case 2: e = launch_gemv_m<2>(plan, g, affine, mbf16, stream); break;
    case 3: e = launch_gemv_m<3>(plan, g, affine, mbf16, stream); break;
    case 4: e = launch_gemv_m<4>(plan, g, affine, mbf16, stream); break;
    case 5: e = launch_gemv_m<5>(plan, g, affine, mbf16, stream); break;
    case 6: e = launch_gemv_m<6>(plan, g, affine, mbf16, stream); break;
    case 7: e = launch_gemv_m<7>(plan, g, affine, mbf16, stream); break;
    case 8: e = launch_gemv_m<8>(plan, g, affine, mbf16, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || plan.KS == 1) return e;
  switch (plan.M) {
    case 1: return launch_reduce_m<1>(plan, g, stream);
    case 2: return launch_reduce_m<2>(plan, g, stream);
    case 3: return launch_reduce_m<3>(plan, g, stream);
    case 4: return launch_reduce_m<4>(plan, g, stream);
    case 5: return launch_reduce_m<5>(plan, g, stream);
    case 6: return launch_reduce_m<6>(plan, g, stream);
    case 7: return launch_reduce_m<7>(plan, g, stream);
    default: return launch_reduce_m<8>(plan, g, stream);
  }
}

hipError_t launch_dequant(const QMat& w, const void* ids, int ids_int64, int64_t T, void* out, int32_t out_dtype,
                          hipStream_t stream) {
  const int64_t per_row = w.K >> 3;
  if (T == 0 || per_row == 0) return hipSuccess;
  const DivMagic dm = div_magic((uint32_t)per_row);
  const int sym = w.symmetric ? 1 : 0;
  const size_t osz = out_dtype == F32 ? 4 : 2;
  // Rows in launches of at most 2^31 pieces, so piece indices (and the
  // strided indices of a thread's last round) stay below 2^32.
  const int64_t rows_per_launch = ((int64_t)1 << 31) / per_row;
  for (int64_t r0 = 0; r0 < T; r0 += rows_per_launch) {
    const int64_t tr = (T - r0 < rows_per_launch) ? T - r0 : rows_per_launch;
    const uint32_t total = (uint32_t)(tr * per_row);
    int64_t blocks = ((int64_t)total + 256 * kDqU - 1) / (256 * kDqU);
    const int64_t cap = (int64_t)device_cus() * 16;
    if (blocks > cap) blocks = cap;
    const void* ids_c = ids == nullptr ? nullptr
                                       : static_cast<const char*>(ids) + r0 * (ids_int64 ? 8 : 4);
    const uint32_t* pk = ids == nullptr ? w.packed + r0 * (w.K >> 5) : w.packed;
    const uint16_t* sc = ids == nullptr ? w.scales + r0 * (w.K >> 7) : w.scales;
    const uint16_t* bi = (ids == nullptr && w.biases != nullptr) ? w.biases + r0 * (w.K >> 7) : w.biases;
    const int64_t nrows = ids == nullptr ? tr : w.N;
    void* o = static_cast<char*>(out) + (size_t)r0 * (size_t)w.K * osz;
#define Q1_DQ(OUT, MB)                                                                                      \
  do {                                                                                                       \
    if (ids != nullptr)                                                                                      \
      hipLaunchKernelGGL((q1_dequant_kernel<OUT, MB, true>), dim3((unsigned)blocks), dim3(256), 0, stream, pk, \
                         sc, bi, sym, nrows, w.K, ids_c, ids_int64, total, dm, o);                            \
    else                                                                                                     \
      hipLaunchKernelGGL((q1_dequant_kernel<OUT, MB, false>), dim3((unsigned)blocks), dim3(256), 0, stream,   \
                         pk, sc, bi, sym, nrows, w.K, ids_c, ids_int64, total, dm, o);                        \
  } while (0)
    if (w.meta_bf16) {
      if (out_dtype == F32) Q1_DQ(F32, true);
      else if (out_dtype == F16) Q1_DQ(F16, true);
      else Q1_DQ(BF16, true);
    } else {
      if (out_dtype == F32) Q1_DQ(F32, false);
      else if (out_dtype == F16) Q1_DQ(F16, false);
      else Q1_DQ(BF16, false);
    }
#undef Q1_DQ
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemm_bf16(const uint16_t* x, const uint16_t* B, int64_t M, int64_t N, int64_t K, void* y,
                            int32_t y_dtype, hipStream_t stream) {
  const int tm = (int)((M + GBM - 1) / GBM);
  const int tn = (int)((N + GBN - 1) / GBN);
  if (tm == 0 || tn == 0) return hipSuccess;
  hipLaunchKernelGGL(q1_gemm_bf16, dim3(tm * tn), dim3(256), 0, stream, x, B, M, N, K, y, y_dtype, tm, tn);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const float* g, const float* u, uint16_t* h, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(q1_silu_mul, dim3((unsigned)blocks), dim3(256), 0, stream, g, u, h, n);
  return hipGetLastError();
}

}  // namespace q1
