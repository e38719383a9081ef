// Internal interface between the C ABI (q1_api.cpp) and the HIP kernels
// (q1_kernels.hip).  Not installed; not part of the public boundary.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace q1 {

enum Dtype : int32_t { F32 = 0, F16 = 1, BF16 = 2 };

// Weight rows per packed-kernel chunk: 32 words = 1024 weights along K.
constexpr int kChunkWords = 32;
constexpr int kChunkK = 1024;
// Bytes of lookup table per (chunk, activation row).
constexpr int kTabBytes = 16384;
// Threads per packed-kernel workgroup: 16 waves for one activation row
// (small register footprint, two workgroups per CU share the LDS), 8 waves
// otherwise.
constexpr int gemv_threads(int M) { return M == 1 ? 1024 : 512; }
// Chunks of K one workgroup covers (its lookup tables must fit in LDS).
constexpr int gemv_krmax(int M) { return M == 1 ? 5 : M == 2 ? 2 : 1; }
// LDS bytes between the tables of consecutive chunks (a chunk's M tables never
// straddle a 64 KB window).
constexpr int gemv_chunk_block(int M) { return M == 1 ? 16384 : M == 2 ? 32768 : M <= 4 ? 65536 : 131072; }
constexpr int gemv_lds_bytes(int M) { return (gemv_krmax(M) - 1) * gemv_chunk_block(M) + M * 16384; }
// Bytes at the start of every workspace reserved for arrival counters
// (Q1_WS_RESERVED_BYTES in the public header).
constexpr int kCounterBytes = 16384;

// Compute units of the current device (cached per device id).
int device_cus();

// Size of the library-owned device scratch that q1_qmm_noalloc uses instead
// of a caller workspace (Q1_STATIC_SCRATCH_BYTES in the public header).
constexpr size_t kStaticScratchBytes = (size_t)8 << 20;

// Device address of the current device's static scratch (set up on the
// first call on a device: symbol address, counters cleared on `stream`).
hipError_t static_scratch(hipStream_t stream, void** ptr);

struct QMat {
  const uint32_t* packed;
  const uint16_t* scales;
  const uint16_t* biases;  // null when symmetric
  int32_t meta_bf16;       // 1: bf16 metadata, 0: fp16
  int32_t symmetric;
  int64_t N, K;
};

// Plan of one packed launch (chosen on the host, see plan_gemv).
struct GemvPlan {
  int M;
  int chunks;   // ceil(K / 1024)
  int KS;       // K splits (grid.y)
  int KR;       // chunks per split (the last split may have fewer)
  int64_t units;         // N (single) or 2N (gate/up pair)
  int64_t units_per_wg;  // even
  int wgs_x;             // grid.x
  int threads;           // workgroup size
  int exact;             // every K range has exactly gemv_krmax(M) full chunks
  size_t lds_bytes;
  size_t partial_floats;  // KS > 1: KS*M*units
};

// Kernel arguments of one packed launch.
struct GemvArgs {
  const uint16_t* x;
  int64_t x_ld;
  const uint32_t* p0;
  const uint32_t* p1;
  const uint16_t* s0;
  const uint16_t* s1;
  const uint16_t* b0;
  const uint16_t* b1;
  int64_t N;
  int32_t K, wpr, gpr, chunks;
  int32_t KS, pair;
  int32_t full_chunks;   // chunks with all 32 words inside the row (K / 1024)
  int64_t units, units_per_wg;
  uint32_t packed_bytes;  // N * K / 8      (< 2^31)
  uint32_t meta_bytes;    // N * K / 128 * 2 (< 2^31)
  int32_t out_dtype;
  void* out;
  int64_t out_ld;
  float* partial;
};

// Launch the packed kernel for M activation rows (q1_gemv.hip).
template <int M>
hipError_t launch_gemv_m(const GemvPlan& plan, const GemvArgs& args, bool affine, bool mbf16, hipStream_t stream);

// ---- matrix-core packed path ------------------------------------------------

// Plan of one matrix-core packed launch (see q1_mma.hip for the scheme).
struct MmaPlan {
  int M;
  int pair;        // 1: FFN gate/up (two matrices, SiLU(g)*u epilogue)
  int G;           // groups of 128 along K
  int nspan;       // spans of 4 groups (512 weights)
  int64_t ntiles;  // tiles of 16 rows
  int S;           // K segments (grid split); S > 1: a reduce launch adds them
  int KSP;         // spans per K segment (the last may have fewer)
  int P;           // workgroups per K segment
  int nb;          // tiles per workgroup (at most)
  int TW;          // result slots per wave: tiles one wave's items touch (at most)
  size_t red_bytes;  // LDS for the per-wave tile results
  int64_t wgs;     // S * P
  size_t lds_bytes;
  size_t partial_floats;  // S > 1: S*M*N*(pair ? 2 : 1)
  int rb;                 // A rows per half in the LDS image: 8, or M (1, 2) for the compact image
};

struct MmaArgs {
  const uint16_t* x;
  int64_t x_ld;
  const uint32_t* p0;
  const uint32_t* p1;
  const uint16_t* s0;
  const uint16_t* s1;
  const uint16_t* b0;
  const uint16_t* b1;
  int64_t N;
  int32_t M, K, G, nspan;
  int32_t S, KSP, P, nb, TW;
  uint32_t red_bytes;
  uint32_t x_bytes, packed_bytes, meta_bytes;
  int32_t out_dtype;
  void* out;
  int64_t out_ld;
  float* partial;
  uint32_t* counters;
};

bool plan_mma(int M, int64_t N, int64_t K, bool pair, bool affine, MmaPlan* plan, const char** why);
// The plan for a given split: S K segments of P workgroups each (P is
// capped at the tile count).  False when S is not a distinct split of K or
// the segment's LDS image, result slots and scratch do not fit.
// full_image: keep all 8 A rows per half in the LDS image even for M <= 2.
bool plan_mma_split(int M, int64_t N, int64_t K, bool pair, bool affine, int S, int64_t P, MmaPlan* plan,
                    bool full_image = false);

// Kernel arguments of one matrix-core stage (plan + operands).
MmaArgs mma_args(const MmaPlan& plan, const uint16_t* x, int64_t x_ld, const QMat& a, const QMat* b, void* out,
                 int32_t out_dtype, int64_t out_ld, float* partial, uint32_t* counters);

hipError_t launch_mma(const MmaPlan& plan, const uint16_t* x, int64_t x_ld, const QMat& a, const QMat* b, void* out,
                      int32_t out_dtype, int64_t out_ld, float* partial, hipStream_t stream);

// ---- single-launch FFN (q1_ffn.hip) ----------------------------------------

// One persistent launch of one workgroup per compute unit: phase 1 is the
// gate/up pair (whole K per workgroup, h written as bf16), phase 2 the down
// projection split into K segments, each waiting for the phase-1 tiles that
// produce its part of h.
struct FfnPlan {
  MmaPlan gu;   // phase 1 (S = 1, P = its workgroups)
  MmaPlan d;    // phase 2 (S segments x P workgroups)
  int64_t wgs;  // grid
  size_t lds_bytes;
  int sync_words;  // uint32 words of the counter block in use (split-K, segment and exit counters)
};

// Status word of the single-launch FFN: the last uint32 of the counter block
// at the start of the workspace.
constexpr int kFfnStatusWord = kCounterBytes / 4 - 1;

bool plan_ffn(int M, int64_t I, int64_t H, int64_t Ho, bool affine, FfnPlan* plan, const char** why);

// gate, up and down share symmetry and metadata dtype.  h: bf16 [M, I];
// y: bf16 [M, Ho]; partial: plan.d.partial_floats floats; sync: the
// workspace's counter block (zero on entry, zero again on exit).
hipError_t launch_ffn(const FfnPlan& plan, const uint16_t* x, const QMat& gate, const QMat& up, const QMat& down,
                      uint16_t* h, void* y, float* partial, uint32_t* sync, hipStream_t stream);

// Returns false (with a message) when the request cannot be planned.
bool plan_gemv(int M, int64_t N, int64_t K, bool pair, bool affine, GemvPlan* plan, const char** why);

// y (single) or h (pair) from packed weights.  `a` is the matrix for single
// mode and gate for pair mode; `b` is up (pair mode) or ignored.
// out_dtype: F32/BF16/F16 for single mode; pair mode always writes bf16 h.
// partial: workspace region sized by the plan (may be null if KS==1).
hipError_t launch_gemv(const GemvPlan& plan, const uint16_t* x, int64_t x_ld, const QMat& a, const QMat* b,
                       void* out, int32_t out_dtype, int64_t out_ld, float* partial, hipStream_t stream);

// Dequantise rows of `w` into out[T, K] (row r of the output is weight row
// rows[r], or r when rows is null).  ids may be int32 or int64.
hipError_t launch_dequant(const QMat& w, const void* ids, int ids_int64, int64_t T, void* out, int32_t out_dtype,
                          hipStream_t stream);

// y[M, N] (bf16 or fp32) = x[M, K] (bf16) * B[N, K]^T (bf16), fp32 accumulate.
// Plan of one wide (M > 8) matrix-core launch pair (activation image, then
// the product straight from the packed weights; see q1_wide.hip).
struct WidePlan {
  int64_t M, N;
  int K, G, nspan;
  int MB;      // row blocks of 8 activation rows
  int mtiles;  // workgroups along M (8 row blocks each)
  int tnb;     // 16-row column blocks per workgroup
  int ntn;     // workgroups along N
  int64_t wgs;
  size_t sc_off, xs_off, ws_bytes;  // workspace: A image, scale image, group sums
};

bool plan_wide(int64_t M, int64_t N, int64_t K, bool affine, WidePlan* plan, const char** why);
// make_image = false reuses the image already in ws (same x, same K, same
// symmetric/affine kind: the group-sum terms differ between the two kinds).
hipError_t launch_wide(const WidePlan& plan, const uint16_t* x, int64_t x_ld, const QMat& w, void* out,
                       int32_t out_dtype, int64_t out_ld, unsigned char* ws, hipStream_t stream,
                       bool make_image = true);

hipError_t launch_gemm_bf16(const uint16_t* x, const uint16_t* B, int64_t M, int64_t N, int64_t K, void* y,
                            int32_t y_dtype, hipStream_t stream);

// Symmetric-bias check of one affine tensor's metadata (ngroups = N*K/128):
// *count = groups whose stored bias cannot be replaced by -scale/2 (the
// counter is cleared by the launch sequence itself).
hipError_t launch_symcheck(const uint16_t* scales, const uint16_t* biases, int64_t ngroups, bool meta_bf16,
                           uint32_t* count, hipStream_t stream);

// Sign packer: dense [N, K] (bf16 or fp16) -> packed [N, K/32], scales
// [N, K/128] (symmetric); *count = groups that do not round-trip exactly.
hipError_t launch_pack(const uint16_t* dense, bool dense_bf16, int64_t N, int64_t K, uint32_t* packed,
                       uint16_t* scales, bool meta_bf16, uint32_t* count, hipStream_t stream);

// One read pass over `bytes` bytes (16-byte loads), for the read ceiling.
hipError_t launch_read(const void* data, size_t bytes, uint32_t* sink, hipStream_t stream);

// h[i] = bf16(SiLU(g[i]) * u[i]) for fp32 g, u (n elements).
hipError_t launch_silu_mul(const float* g, const float* u, uint16_t* h, int64_t n, hipStream_t stream);

}  // namespace q1
