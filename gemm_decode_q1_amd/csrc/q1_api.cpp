// C ABI of the packed Q1 library: argument validation, dispatch between the
// packed narrow-M kernels and the wide path, workspace layout.
//
// Dispatch rule (Higgs PR #212, "What" and "Limitations"): Q1 matmuls of up
// to 8 flattened rows stay packed; wider ones take the wide path -- here the
// matrix cores straight from the packed words, or (Q1_WIDE_KERNEL=dequant) the
// pages' dense fallback, dequantisation to bf16 and a dense GEMM.  The row
// threshold is an override.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/q1.h"
#include "../../include/q1_measure.h"
#include "q1_internal.h"

namespace {

thread_local char g_err[512] = "";

q1_status fail(q1_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

q1_status ok() {
  g_err[0] = '\0';
  return Q1_OK;
}

int initial_max_rows() {
  const char* e = getenv("Q1_QMM_MAX_ROWS");
  if (e) {
    const int v = atoi(e);
    if (v >= 1 && v <= 8) return v;
  }
  return 8;
}

int g_max_rows = initial_max_rows();

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool valid_out_dtype(int32_t d) { return d == Q1_F32 || d == Q1_F16 || d == Q1_BF16; }

size_t dtype_size(int32_t d) { return d == Q1_F32 ? 4 : 2; }

q1_status check_weight(const q1_weight* w, const char* name) {
  if (w == nullptr) return fail(Q1_ERR_INVALID_ARG, "%s: weight descriptor is NULL", name);
  if (w->packed == nullptr) return fail(Q1_ERR_INVALID_ARG, "%s: packed pointer is NULL", name);
  if (w->scales == nullptr) return fail(Q1_ERR_INVALID_ARG, "%s: scales pointer is NULL", name);
  if (w->group_size != 128)
    return fail(Q1_ERR_UNSUPPORTED, "%s: group_size %d not supported (only 128)", name, (int)w->group_size);
  if (w->reserved != 0) return fail(Q1_ERR_INVALID_ARG, "%s: reserved field must be 0", name);
  if (w->meta_dtype != Q1_F16 && w->meta_dtype != Q1_BF16)
    return fail(Q1_ERR_INVALID_ARG, "%s: metadata dtype must be Q1_F16 or Q1_BF16", name);
  if (w->symmetric != 0 && w->symmetric != 1) return fail(Q1_ERR_INVALID_ARG, "%s: symmetric must be 0 or 1", name);
  if (w->symmetric && w->biases != nullptr)
    return fail(Q1_ERR_INVALID_ARG, "%s: symmetric tensor must not carry biases (bias is derived as -scale/2)", name);
  if (!w->symmetric && w->biases == nullptr)
    return fail(Q1_ERR_INVALID_ARG, "%s: affine tensor needs a biases pointer (or set symmetric=1)", name);
  if (w->N <= 0) return fail(Q1_ERR_INVALID_ARG, "%s: N must be positive (got %lld)", name, (long long)w->N);
  if (w->K <= 0 || w->K % 128 != 0)
    return fail(Q1_ERR_INVALID_ARG, "%s: K must be a positive multiple of 128 (got %lld)", name, (long long)w->K);
  if (w->K > (int64_t)1 << 30) return fail(Q1_ERR_UNSUPPORTED, "%s: K too large", name);
  if (w->N > ((int64_t)1 << 40) / w->K) return fail(Q1_ERR_UNSUPPORTED, "%s: matrix too large", name);
  if (!aligned(w->packed, 4)) return fail(Q1_ERR_INVALID_ARG, "%s: packed must be 4-byte aligned", name);
  if (!aligned(w->scales, 2) || (w->biases && !aligned(w->biases, 2)))
    return fail(Q1_ERR_INVALID_ARG, "%s: scales/biases must be 2-byte aligned", name);
  return Q1_OK;
}

q1::QMat to_mat(const q1_weight* w) {
  q1::QMat m;
  m.packed = w->packed;
  m.scales = static_cast<const uint16_t*>(w->scales);
  m.biases = static_cast<const uint16_t*>(w->biases);
  m.meta_bf16 = w->meta_dtype == Q1_BF16 ? 1 : 0;
  m.symmetric = w->symmetric;
  m.N = w->N;
  m.K = w->K;
  return m;
}

// Device check, cached per device id.
std::mutex g_dev_mu;
signed char g_dev_ok[256];  // 0 unknown, 1 ok, -1 unsupported

q1_status check_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(Q1_ERR_HIP, "hipGetDevice failed");
  if (dev >= 0 && dev < 256) {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_ok[dev] == 1) return Q1_OK;
  }
  return q1_device_supported(dev);
}

q1_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(Q1_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// ---- workspace layouts --------------------------------------------------

// Every workspace starts with Q1_WS_RESERVED_BYTES reserved for the
// single-launch FFN's counters and status word (the other launches leave it
// untouched); a packed launch's fp32 partial sums go at `base`.
constexpr size_t kReserved = Q1_WS_RESERVED_BYTES;

// Packed narrow-M launches: the nibble-table kernel (q1_gemv.hip) for one
// activation row, the matrix-core kernel (q1_mma.hip) for 2..8 rows, where
// table lookups grow with the row count.  Q1_PACKED_KERNEL=table|mma forces
// one of them for every row count (read on every call, like
// Q1_WIDE_KERNEL; the workspace query must see the same setting as the call).
// 0: default routing, 1: table kernel forced, 2: matrix-core kernel forced
int packed_kernel_env() {
  const char* e = getenv("Q1_PACKED_KERNEL");
  if (e && strcmp(e, "table") == 0) return 1;
  if (e && strcmp(e, "mma") == 0) return 2;
  return 0;
}

// More than 8 rows: the wide matrix-core kernel straight from the packed
// weights.  Q1_WIDE_KERNEL=dequant selects the dense fallback (dequantise to bf16, then
// the bf16 GEMM) for M > max rows; read on every call, so a caller can switch
// between the two wide paths (the workspace query must see the same setting
// as the call it sizes).
bool use_wide_kernel() {
  const char* e = getenv("Q1_WIDE_KERNEL");
  return !(e && strcmp(e, "dequant") == 0);
}

// Packed FFN: Q1_FFN_KERNEL=single runs gate/up, SiLU*mul and down in one
// persistent launch when the three matrices are of one kind (q1_ffn.hip);
// otherwise the pair launch, then the down launch, which is faster on MI355X
// (the single launch's agent-scope release of h is an L2 writeback that waits
// behind the weight stream).  Read on every call and by the workspace query.
bool ffn_single_enabled() {
  const char* e = getenv("Q1_FFN_KERNEL");
  return e && strcmp(e, "single") == 0;
}

struct PackedPlan {
  bool table;
  q1::GemvPlan g;
  q1::MmaPlan m;
  size_t partial_floats() const { return table ? (g.KS > 1 ? g.partial_floats : 0) : m.partial_floats; }
};

// Default routing: one activation row goes to the table kernel unless its
// plan needs a K split, where the matrix-core kernel is faster (K=17408,
// N=5120: 10.4 against 11.6-12.0 us, both with a reduce launch); 2..8 rows go
// to the matrix-core kernel, with the table kernel as the fallback for shapes
// its plan rejects.
bool plan_packed(int M, int64_t N, int64_t K, bool pair, bool affine, PackedPlan* p, const char** why) {
  const int env = packed_kernel_env();
  if (env == 1) {
    p->table = true;
    return q1::plan_gemv(M, N, K, pair, affine, &p->g, why);
  }
  if (env == 2) {
    p->table = false;
    return q1::plan_mma(M, N, K, pair, affine, &p->m, why);
  }
  const char* why_t = nullptr;
  const char* why_m = nullptr;
  const bool ok_t = q1::plan_gemv(M, N, K, pair, affine, &p->g, &why_t);
  const bool ok_m = q1::plan_mma(M, N, K, pair, affine, &p->m, &why_m);
  if (M == 1)
    p->table = ok_t && (p->g.KS == 1 || !ok_m);
  else
    p->table = !ok_m && ok_t;
  if (!ok_t && !ok_m) {
    *why = M == 1 ? why_t : why_m;
    return false;
  }
  return true;
}

struct PackedWs {
  size_t partial_off, bytes;  // bytes used from `base` on
};

PackedWs packed_ws(const PackedPlan& p, size_t base) {
  PackedWs w;
  w.partial_off = base;
  w.bytes = align_up(p.partial_floats() * sizeof(float), 256);
  return w;
}

struct FfnWs {
  bool packed, fused;
  bool single;                     // one persistent launch (q1_ffn.hip)
  q1::FfnPlan fp;
  size_t part_off;                 // single: down split-K partials
  PackedPlan pgu, pg, pu, pd;
  size_t h_off, gu_off, d_off;     // packed: partial-sum blocks
  size_t g_off, u_off;             // unfused / wide: fp32 g and u
  size_t deq_off;                  // wide: operand image (matrix-core path) or dequantised matrix
  bool wide_mma;                   // wide: matrix-core path
  q1::WidePlan wg, wu, wd;
  size_t bytes;
};

bool same_format(const q1_weight* a, const q1_weight* b) {
  return a->meta_dtype == b->meta_dtype && a->symmetric == b->symmetric && a->N == b->N && a->K == b->K;
}

q1_status ffn_layout(int64_t M, const q1_weight* gate, const q1_weight* up, const q1_weight* down, FfnWs* L) {
  const int64_t I = gate->N, H = gate->K, Ho = down->N;
  L->packed = M <= g_max_rows;
  L->wide_mma = false;
  L->fused = L->packed && same_format(gate, up);
  L->h_off = kReserved;
  size_t off = align_up(kReserved + (size_t)M * I * 2, 256);
  const char* why = "";
  L->single = L->fused && ffn_single_enabled() && down->symmetric == gate->symmetric &&
              down->meta_dtype == gate->meta_dtype && q1::plan_ffn((int)M, I, H, Ho, !gate->symmetric, &L->fp, &why);
  if (L->single) {
    L->part_off = off;
    L->bytes = align_up(off + L->fp.d.partial_floats * sizeof(float), 256);
    return Q1_OK;
  }
  if (L->packed) {
    if (L->fused) {
      if (!plan_packed((int)M, I, H, true, !gate->symmetric, &L->pgu, &why)) return fail(Q1_ERR_UNSUPPORTED, "%s", why);
      PackedWs w = packed_ws(L->pgu, off);
      L->gu_off = off;
      off += w.bytes;
    } else {
      if (!plan_packed((int)M, I, H, false, !gate->symmetric, &L->pg, &why) ||
          !plan_packed((int)M, up->N, up->K, false, !up->symmetric, &L->pu, &why))
        return fail(Q1_ERR_UNSUPPORTED, "%s", why);
      L->g_off = off;
      off = align_up(off + (size_t)M * I * 4, 256);
      L->u_off = off;
      off = align_up(off + (size_t)M * I * 4, 256);
      L->gu_off = off;  // shared by the two sequential launches
      PackedWs wg = packed_ws(L->pg, off), wu = packed_ws(L->pu, off);
      off += wg.bytes > wu.bytes ? wg.bytes : wu.bytes;
    }
    if (!plan_packed((int)M, Ho, I, false, !down->symmetric, &L->pd, &why)) return fail(Q1_ERR_UNSUPPORTED, "%s", why);
    L->d_off = off;
    off += packed_ws(L->pd, off).bytes;
  } else {
    L->g_off = off;
    off = align_up(off + (size_t)M * I * 4, 256);
    L->u_off = off;
    off = align_up(off + (size_t)M * I * 4, 256);
    L->deq_off = off;
    L->wide_mma = use_wide_kernel() && q1::plan_wide(M, I, H, !gate->symmetric, &L->wg, &why) &&
                  q1::plan_wide(M, up->N, up->K, !up->symmetric, &L->wu, &why) &&
                  q1::plan_wide(M, Ho, I, !down->symmetric, &L->wd, &why);
    if (L->wide_mma) {
      size_t big = L->wg.ws_bytes;
      if (L->wu.ws_bytes > big) big = L->wu.ws_bytes;
      if (L->wd.ws_bytes > big) big = L->wd.ws_bytes;
      off = align_up(off + big, 256);
    } else {
      size_t big = (size_t)I * H;
      if ((size_t)Ho * I > big) big = (size_t)Ho * I;
      off = align_up(off + big * 2, 256);
    }
  }
  L->bytes = off;
  return Q1_OK;
}

q1_status run_packed(const PackedPlan& p, const uint16_t* x, int64_t x_ld, const q1::QMat& a, const q1::QMat* b,
                     void* out, int32_t out_dtype, int64_t out_ld, unsigned char* ws, size_t base, hipStream_t s) {
  PackedWs w = packed_ws(p, base);
  const bool split = p.partial_floats() > 0;
  float* partial = split ? reinterpret_cast<float*>(ws + w.partial_off) : nullptr;
  if (p.table)
    return hip_status(q1::launch_gemv(p.g, x, x_ld, a, b, out, out_dtype, out_ld, partial, s),
                      "packed kernel launch");
  return hip_status(q1::launch_mma(p.m, x, x_ld, a, b, out, out_dtype, out_ld, partial, s),
                    "packed kernel launch");
}

// Argument checks of q1_qmm and q1_qmm_noalloc (no HIP call).  *done: M == 0
// (nothing to do).
q1_status qmm_args(const void* x, int32_t x_dtype, int64_t M, const q1_weight* w, const void* y, int32_t y_dtype,
                   bool* done) {
  *done = false;
  q1_status st = check_weight(w, "w");
  if (st != Q1_OK) return st;
  if (M < 0) return fail(Q1_ERR_INVALID_ARG, "M must be >= 0 (got %lld)", (long long)M);
  if (x_dtype != Q1_BF16) return fail(Q1_ERR_UNSUPPORTED, "x must be bf16");
  if (!valid_out_dtype(y_dtype)) return fail(Q1_ERR_INVALID_ARG, "y dtype must be Q1_F32, Q1_F16 or Q1_BF16");
  if (M == 0) {
    *done = true;
    return ok();
  }
  if (x == nullptr || y == nullptr) return fail(Q1_ERR_INVALID_ARG, "x and y must not be NULL");
  if (!aligned(x, 16)) return fail(Q1_ERR_INVALID_ARG, "x must be 16-byte aligned");
  if (!aligned(y, dtype_size(y_dtype))) return fail(Q1_ERR_INVALID_ARG, "y is misaligned");
  return Q1_OK;
}

q1_status qmm_run(const void* x, int64_t M, const q1_weight* w, void* y, int32_t y_dtype, void* workspace,
                  hipStream_t s) {
  const q1::QMat a = to_mat(w);
  auto* ws = static_cast<unsigned char*>(workspace);
  if (M <= g_max_rows) {
    PackedPlan p;
    const char* why = "";
    if (!plan_packed((int)M, w->N, w->K, false, !w->symmetric, &p, &why)) return fail(Q1_ERR_UNSUPPORTED, "%s", why);
    return run_packed(p, static_cast<const uint16_t*>(x), w->K, a, nullptr, y, y_dtype, w->N, ws, kReserved, s);
  }
  q1::WidePlan wp;
  const char* why = "";
  if (use_wide_kernel() && q1::plan_wide(M, w->N, w->K, !w->symmetric, &wp, &why))
    return hip_status(q1::launch_wide(wp, static_cast<const uint16_t*>(x), w->K, a, y, y_dtype, w->N, ws + kReserved, s),
                      "wide launch");
  uint16_t* deq = reinterpret_cast<uint16_t*>(ws + kReserved);
  hipError_t e = q1::launch_dequant(a, nullptr, 0, w->N, deq, q1::BF16, s);
  if (e != hipSuccess) return hip_status(e, "dequant launch");
  return hip_status(q1::launch_gemm_bf16(static_cast<const uint16_t*>(x), deq, M, w->N, w->K, y, y_dtype, s),
                    "gemm launch");
}

}  // namespace

extern "C" {

const char* q1_last_error(void) { return g_err; }

const char* q1_version(void) { return "q1-gfx950 0.1"; }

int q1_set_max_packed_rows(int rows) {
  if (rows < 1 || rows > 8) return -1;
  const int prev = g_max_rows;
  g_max_rows = rows;
  return prev;
}

q1_status q1_device_supported(int device) {
  hipDeviceProp_t prop;
  hipError_t e = hipGetDeviceProperties(&prop, device);
  if (e != hipSuccess) return fail(Q1_ERR_HIP, "hipGetDeviceProperties(%d): %s", device, hipGetErrorString(e));
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(Q1_ERR_UNSUPPORTED, "device %d is %s; the Q1 kernels are built for gfx950 (MI355X) only", device,
                prop.gcnArchName);
  if (device >= 0 && device < 256) {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    g_dev_ok[device] = 1;
  }
  return ok();
}

size_t q1_qmm_workspace_bytes(int64_t M, const q1_weight* w) {
  if (check_weight(w, "w") != Q1_OK) return 0;
  if (M < 0) {
    fail(Q1_ERR_INVALID_ARG, "M must be >= 0");
    return 0;
  }
  if (M == 0) return 0;
  if (M <= g_max_rows) {
    PackedPlan p;
    const char* why = "";
    if (!plan_packed((int)M, w->N, w->K, false, !w->symmetric, &p, &why)) {
      fail(Q1_ERR_UNSUPPORTED, "%s", why);
      return 0;
    }
    const size_t part = packed_ws(p, kReserved).bytes;
    return part ? kReserved + part : 0;
  }
  q1::WidePlan wp;
  const char* why = "";
  if (use_wide_kernel() && q1::plan_wide(M, w->N, w->K, !w->symmetric, &wp, &why)) return kReserved + wp.ws_bytes;
  return kReserved + align_up((size_t)w->N * w->K * 2, 256);
}

q1_status q1_qmm(const void* x, int32_t x_dtype, int64_t M, const q1_weight* w, void* y, int32_t y_dtype,
                 void* workspace, size_t workspace_bytes, void* stream) {
  bool done = false;
  q1_status st = qmm_args(x, x_dtype, M, w, y, y_dtype, &done);
  if (st != Q1_OK || done) return st;
  const size_t need = q1_qmm_workspace_bytes(M, w);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(Q1_ERR_WORKSPACE, "workspace too small: need %zu bytes, got %zu", need, workspace ? workspace_bytes : 0);
  if (need > 0 && !aligned(workspace, 256)) return fail(Q1_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  st = check_current_device();
  if (st != Q1_OK) return st;
  return qmm_run(x, M, w, y, y_dtype, workspace, static_cast<hipStream_t>(stream));
}

q1_status q1_qmm_noalloc(const void* x, int32_t x_dtype, int64_t M, const q1_weight* w, void* y,
                         int32_t y_dtype, void* stream) {
  bool done = false;
  q1_status st = qmm_args(x, x_dtype, M, w, y, y_dtype, &done);
  if (st != Q1_OK || done) return st;
  const size_t need = q1_qmm_workspace_bytes(M, w);
  if (need > q1::kStaticScratchBytes)
    return fail(Q1_ERR_WORKSPACE,
                "this call needs %zu bytes of scratch; the static scratch holds %zu (use q1_qmm with a workspace)",
                need, q1::kStaticScratchBytes);
  st = check_current_device();
  if (st != Q1_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = q1::static_scratch(s, &ws);
    if (e != hipSuccess) return hip_status(e, "static scratch set-up");
  }
  return qmm_run(x, M, w, y, y_dtype, ws, s);
}

q1_status q1_dequantize(const q1_weight* w, void* out, int32_t out_dtype, void* stream) {
  q1_status st = check_weight(w, "w");
  if (st != Q1_OK) return st;
  if (!valid_out_dtype(out_dtype)) return fail(Q1_ERR_INVALID_ARG, "out dtype must be Q1_F32, Q1_F16 or Q1_BF16");
  if (out == nullptr) return fail(Q1_ERR_INVALID_ARG, "out must not be NULL");
  if (!aligned(out, 16)) return fail(Q1_ERR_INVALID_ARG, "out must be 16-byte aligned");
  st = check_current_device();
  if (st != Q1_OK) return st;
  return hip_status(q1::launch_dequant(to_mat(w), nullptr, 0, w->N, out, out_dtype, static_cast<hipStream_t>(stream)),
                    "dequant launch");
}

q1_status q1_embed_rows(const void* ids, int32_t ids_are_int64, int64_t T, const q1_weight* table, void* out,
                        int32_t out_dtype, void* stream) {
  q1_status st = check_weight(table, "table");
  if (st != Q1_OK) return st;
  if (!valid_out_dtype(out_dtype)) return fail(Q1_ERR_INVALID_ARG, "out dtype must be Q1_F32, Q1_F16 or Q1_BF16");
  if (ids_are_int64 != 0 && ids_are_int64 != 1) return fail(Q1_ERR_INVALID_ARG, "ids_are_int64 must be 0 or 1");
  if (T < 0) return fail(Q1_ERR_INVALID_ARG, "T must be >= 0");
  if (T == 0) return ok();
  if (ids == nullptr || out == nullptr) return fail(Q1_ERR_INVALID_ARG, "ids and out must not be NULL");
  if (!aligned(ids, ids_are_int64 ? 8 : 4)) return fail(Q1_ERR_INVALID_ARG, "ids misaligned");
  if (!aligned(out, 16)) return fail(Q1_ERR_INVALID_ARG, "out must be 16-byte aligned");
  st = check_current_device();
  if (st != Q1_OK) return st;
  return hip_status(
      q1::launch_dequant(to_mat(table), ids, ids_are_int64, T, out, out_dtype, static_cast<hipStream_t>(stream)),
      "gather launch");
}

q1_status q1_check_symmetric(const q1_weight* w, uint32_t* count, void* stream) {
  q1_status st = check_weight(w, "w");
  if (st != Q1_OK) return st;
  if (w->symmetric) return fail(Q1_ERR_INVALID_ARG, "w: already symmetric (no biases to check)");
  if (count == nullptr || !aligned(count, 4)) return fail(Q1_ERR_INVALID_ARG, "count must be a 4-byte aligned device pointer");
  st = check_current_device();
  if (st != Q1_OK) return st;
  return hip_status(q1::launch_symcheck(static_cast<const uint16_t*>(w->scales), static_cast<const uint16_t*>(w->biases),
                                        w->N * (w->K / 128), w->meta_dtype == Q1_BF16, count,
                                        static_cast<hipStream_t>(stream)),
                    "symmetric check launch");
}

q1_status q1_pack_signs(const void* dense, int32_t dense_dtype, int64_t N, int64_t K, uint32_t* packed, void* scales,
                        int32_t meta_dtype, uint32_t* inexact, void* stream) {
  if (dense_dtype != Q1_BF16 && dense_dtype != Q1_F16)
    return fail(Q1_ERR_INVALID_ARG, "dense dtype must be Q1_BF16 or Q1_F16");
  if (meta_dtype != Q1_BF16 && meta_dtype != Q1_F16)
    return fail(Q1_ERR_INVALID_ARG, "metadata dtype must be Q1_BF16 or Q1_F16");
  if (N <= 0) return fail(Q1_ERR_INVALID_ARG, "N must be positive (got %lld)", (long long)N);
  if (K <= 0 || K % 128 != 0) return fail(Q1_ERR_INVALID_ARG, "K must be a positive multiple of 128 (got %lld)", (long long)K);
  if (K > (int64_t)1 << 30 || N > ((int64_t)1 << 40) / K) return fail(Q1_ERR_UNSUPPORTED, "matrix too large");
  if (dense == nullptr || packed == nullptr || scales == nullptr || inexact == nullptr)
    return fail(Q1_ERR_INVALID_ARG, "dense, packed, scales and inexact must not be NULL");
  if (!aligned(dense, 16)) return fail(Q1_ERR_INVALID_ARG, "dense must be 16-byte aligned");
  if (!aligned(packed, 4) || !aligned(scales, 2) || !aligned(inexact, 4))
    return fail(Q1_ERR_INVALID_ARG, "packed/inexact must be 4-byte and scales 2-byte aligned");
  const q1_status st = check_current_device();
  if (st != Q1_OK) return st;
  return hip_status(q1::launch_pack(static_cast<const uint16_t*>(dense), dense_dtype == Q1_BF16, N, K, packed,
                                    static_cast<uint16_t*>(scales), meta_dtype == Q1_BF16, inexact,
                                    static_cast<hipStream_t>(stream)),
                    "pack launch");
}

q1_status q1_stream_read(const void* data, size_t bytes, uint32_t* sink, void* stream) {
  if (data == nullptr || sink == nullptr) return fail(Q1_ERR_INVALID_ARG, "data and sink must not be NULL");
  if (!aligned(data, 16) || bytes % 16 != 0) return fail(Q1_ERR_INVALID_ARG, "data must be 16-byte aligned, bytes a multiple of 16");
  if (bytes >= ((size_t)1 << 31)) return fail(Q1_ERR_UNSUPPORTED, "bytes must be below 2^31");
  const q1_status st = check_current_device();
  if (st != Q1_OK) return st;
  if (bytes == 0) return ok();
  return hip_status(q1::launch_read(data, bytes, sink, static_cast<hipStream_t>(stream)), "read launch");
}

size_t q1_ffn_workspace_bytes(int64_t M, const q1_weight* gate, const q1_weight* up, const q1_weight* down) {
  if (check_weight(gate, "gate") != Q1_OK || check_weight(up, "up") != Q1_OK || check_weight(down, "down") != Q1_OK)
    return 0;
  if (up->N != gate->N || up->K != gate->K || down->K != gate->N) {
    fail(Q1_ERR_INVALID_ARG, "FFN shapes: need gate [I,H], up [I,H], down [H_out,I]");
    return 0;
  }
  if (M <= 0) return 0;
  FfnWs L;
  if (ffn_layout(M, gate, up, down, &L) != Q1_OK) return 0;
  return L.bytes;
}

q1_status q1_ffn(const void* x, int64_t M, const q1_weight* gate, const q1_weight* up, const q1_weight* down, void* y,
                 void* workspace, size_t workspace_bytes, void* stream) {
  q1_status st = check_weight(gate, "gate");
  if (st == Q1_OK) st = check_weight(up, "up");
  if (st == Q1_OK) st = check_weight(down, "down");
  if (st != Q1_OK) return st;
  if (up->N != gate->N || up->K != gate->K || down->K != gate->N)
    return fail(Q1_ERR_INVALID_ARG, "FFN shapes: need gate [I,H], up [I,H], down [H_out,I] (got gate %lldx%lld, up %lldx%lld, down %lldx%lld)",
                (long long)gate->N, (long long)gate->K, (long long)up->N, (long long)up->K, (long long)down->N,
                (long long)down->K);
  if (M < 0) return fail(Q1_ERR_INVALID_ARG, "M must be >= 0");
  if (M == 0) return ok();
  if (x == nullptr || y == nullptr) return fail(Q1_ERR_INVALID_ARG, "x and y must not be NULL");
  if (!aligned(x, 16) || !aligned(y, 2)) return fail(Q1_ERR_INVALID_ARG, "x must be 16-byte aligned, y 2-byte aligned");
  FfnWs L;
  st = ffn_layout(M, gate, up, down, &L);
  if (st != Q1_OK) return st;
  if (workspace == nullptr || workspace_bytes < L.bytes)
    return fail(Q1_ERR_WORKSPACE, "workspace too small: need %zu bytes, got %zu", L.bytes, workspace ? workspace_bytes : 0);
  if (!aligned(workspace, 256)) return fail(Q1_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  st = check_current_device();
  if (st != Q1_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  auto* ws = static_cast<unsigned char*>(workspace);
  const int64_t I = gate->N, H = gate->K, Ho = down->N;
  const auto* xb = static_cast<const uint16_t*>(x);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + L.h_off);
  const q1::QMat g = to_mat(gate), u = to_mat(up), d = to_mat(down);
  if (L.single)
    return hip_status(q1::launch_ffn(L.fp, xb, g, u, d, h, y, reinterpret_cast<float*>(ws + L.part_off),
                                     reinterpret_cast<uint32_t*>(ws), s),
                      "FFN launch");
  if (L.packed) {
    if (L.fused) {
      st = run_packed(L.pgu, xb, H, g, &u, h, Q1_BF16, I, ws, L.gu_off, s);
    } else {
      float* gf = reinterpret_cast<float*>(ws + L.g_off);
      float* uf = reinterpret_cast<float*>(ws + L.u_off);
      st = run_packed(L.pg, xb, H, g, nullptr, gf, Q1_F32, I, ws, L.gu_off, s);
      if (st == Q1_OK) st = run_packed(L.pu, xb, H, u, nullptr, uf, Q1_F32, I, ws, L.gu_off, s);
      if (st == Q1_OK) st = hip_status(q1::launch_silu_mul(gf, uf, h, M * I, s), "silu-mul launch");
    }
    if (st != Q1_OK) return st;
    return run_packed(L.pd, h, I, d, nullptr, y, Q1_BF16, Ho, ws, L.d_off, s);
  }
  float* gf = reinterpret_cast<float*>(ws + L.g_off);
  float* uf = reinterpret_cast<float*>(ws + L.u_off);
  if (L.wide_mma) {  // the operand image region is reused by the three products in turn
    unsigned char* img = ws + L.deq_off;
    hipError_t e = q1::launch_wide(L.wg, xb, H, g, gf, q1::F32, I, img, s);
    // gate and up read the same x: one image serves both when their
    // accumulator terms agree (both symmetric or both affine)
    if (e == hipSuccess)
      e = q1::launch_wide(L.wu, xb, H, u, uf, q1::F32, I, img, s, g.symmetric != u.symmetric);
    if (e == hipSuccess) e = q1::launch_silu_mul(gf, uf, h, M * I, s);
    if (e == hipSuccess) e = q1::launch_wide(L.wd, h, I, d, y, q1::BF16, Ho, img, s);
    return hip_status(e, "wide FFN launch");
  }
  uint16_t* deq = reinterpret_cast<uint16_t*>(ws + L.deq_off);
  hipError_t e = q1::launch_dequant(g, nullptr, 0, I, deq, q1::BF16, s);
  if (e == hipSuccess) e = q1::launch_gemm_bf16(xb, deq, M, I, H, gf, q1::F32, s);
  if (e == hipSuccess) e = q1::launch_dequant(u, nullptr, 0, I, deq, q1::BF16, s);
  if (e == hipSuccess) e = q1::launch_gemm_bf16(xb, deq, M, I, H, uf, q1::F32, s);
  if (e == hipSuccess) e = q1::launch_silu_mul(gf, uf, h, M * I, s);
  if (e == hipSuccess) e = q1::launch_dequant(d, nullptr, 0, Ho, deq, q1::BF16, s);
  if (e == hipSuccess) e = q1::launch_gemm_bf16(h, deq, M, Ho, I, y, q1::BF16, s);
  return hip_status(e, "wide FFN launch");
}

}  // extern "C"
