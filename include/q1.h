/*
 * q1.h -- C ABI of the packed Q1 (1-bit affine, group 128) decode library for
 * AMD MI355X (gfx950).
 *
 * Format (rMLX issue #207, "The good news -- packing is standard"; Cactus PR
 * #775, commit notes, "linear LSB layout"; mlx-gen backlog 0004, "Context"):
 *   packed  uint32 [N, K/32], row-major; weight k of row n is bit (k & 31) of
 *           word (k >> 5) (least significant bit first);
 *   scales  fp16 or bf16 [N, K/128], row-major, one per 128 weights along K;
 *   biases  same shape and dtype, or NULL for a symmetric tensor.
 * Dequantisation (Higgs PR #212, "What", "Why"): w = scale * bit + bias; a
 * symmetric tensor derives bias = -scale/2 (computed in fp32, exact), so its
 * codes map to -scale/2 and +scale/2.  The dequantised value is
 * fl32(fl32(scale * bit) + bias) -- a single rounding.
 *
 * Conventions shared by every call:
 *   - All tensor pointers are caller-owned device memory, contiguous and
 *     row-major.  The library keeps no reference after a call returns and never
 *     allocates device memory; temporaries live in a caller workspace.
 *   - Every call checks shapes, dtypes, flags, pointers and alignment before
 *     any HIP call.  The workspace check comes next: the size a call needs
 *     depends on the device's compute-unit count, one attribute query cached
 *     per device.  Then the current device is checked (gfx950).  Failures
 *     return Q1_ERR_INVALID_ARG / Q1_ERR_UNSUPPORTED / Q1_ERR_WORKSPACE with a
 *     short message in q1_last_error() (thread-local); Q1_ERR_HIP reports a
 *     failed HIP call or launch.  Kernel faults surface at the caller's next
 *     synchronisation.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *     work on it and return.
 *   - Rounding of every stored result is round-to-nearest-even; subnormals are
 *     kept.
 */
#ifndef Q1_H
#define Q1_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum q1_status {
  Q1_OK = 0,
  Q1_ERR_INVALID_ARG = -1, /* a shape, pointer, dtype or flag is wrong */
  Q1_ERR_UNSUPPORTED = -2, /* valid request this build does not serve (e.g. not gfx950) */
  Q1_ERR_WORKSPACE = -3,   /* workspace NULL or smaller than the *_workspace_bytes query */
  Q1_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
} q1_status;

typedef enum q1_dtype { Q1_F32 = 0, Q1_F16 = 1, Q1_BF16 = 2 } q1_dtype;

/* The first Q1_WS_RESERVED_BYTES bytes of every workspace are reserved for
 * the arrival counters of the single-launch q1_ffn.  They must be zero before
 * a workspace is first used; every call leaves them zero again once the stream
 * has executed it, and no call writes anything else there, with one
 * exception: the single-launch q1_ffn sets the last uint32 of the block
 * (Q1_WS_STATUS_WORD, an index in uint32 units) to 1 if one of its waits gives
 * up (see q1_ffn); nothing clears it but the caller.  All other temporaries
 * start after the block. */
#define Q1_WS_RESERVED_BYTES 16384
#define Q1_WS_STATUS_WORD (Q1_WS_RESERVED_BYTES / 4 - 1)

/* One packed Q1 matrix (caller-owned device memory). */
typedef struct q1_weight {
  const uint32_t* packed; /* [N, K/32]; 4-byte aligned */
  const void* scales;     /* [N, K/128], meta_dtype */
  const void* biases;     /* [N, K/128], meta_dtype; NULL iff symmetric */
  int32_t meta_dtype;     /* Q1_F16 or Q1_BF16 */
  int32_t symmetric;      /* 1: bias = -scale/2 derived in-kernel (biases must be NULL) */
  int64_t N;              /* rows (output features) */
  int64_t K;              /* weights per row; K % 128 == 0 */
  int32_t group_size;     /* must be 128 */
  int32_t reserved;       /* must be 0 */
} q1_weight;

/*
 * q1_qmm -- y[M, N] = x[M, K] . W^T  (Higgs PR #212, "What": packed Q1 linear
 * and tied head; "Limitations": wider forwards use the dense fallback).
 *   x        bf16 [M, K] (M = product of the caller's leading dims)
 *   x_dtype  must be Q1_BF16
 *   w        the packed matrix (N, K)
 *   y        [M, N] in y_dtype (Q1_F32, Q1_BF16 or Q1_F16)
 *   M <= max packed rows (default 8): packed narrow-M kernel, fp32
 *     accumulation, one rounding to y_dtype.
 *   M  > max packed rows: the wide matrix-core path -- the activations are
 *     converted once into an fp8 operand image in the workspace, then the
 *     product runs on the matrix cores straight from the packed weights
 *     (fp32 accumulation).  With the environment variable
 *     Q1_WIDE_KERNEL=dequant (read on every call, and by the workspace query)
 *     the matrix is instead dequantised to bf16 in the workspace and a bf16
 *     MFMA GEMM runs (Higgs PR #212, "Limitations": the dense fallback).
 *   workspace  device memory of at least q1_qmm_workspace_bytes(M, w) bytes,
 *     256-byte aligned (may be NULL when that query returns 0).  Its first
 *     Q1_WS_RESERVED_BYTES must be zero (see above).  Calls that share one
 *     workspace must be ordered (same stream); concurrent calls need separate
 *     workspaces.
 */
q1_status q1_qmm(const void* x, int32_t x_dtype, int64_t M, const q1_weight* w, void* y, int32_t y_dtype,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes q1_qmm needs for these shapes (0 is a valid answer only if
 * the call needs none).  Returns 0 and sets q1_last_error() on invalid input. */
size_t q1_qmm_workspace_bytes(int64_t M, const q1_weight* w);

/* Bytes of the library-owned device scratch used by q1_qmm_noalloc. */
#define Q1_STATIC_SCRATCH_BYTES (8u << 20)

/*
 * q1_qmm_noalloc -- q1_qmm for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, kernels and results as q1_qmm, without the
 * workspace: temporaries live in a device array the library owns, one copy
 * per GPU it runs on, Q1_STATIC_SCRATCH_BYTES large, held until the process
 * ends.  Calls needing more (q1_qmm_workspace_bytes(M, w) above that size)
 * fail with Q1_ERR_WORKSPACE.  The call allocates nothing.  The first call on
 * a device sets the array up (its address, and a clearing kernel enqueued on
 * `stream`).  All calls on one GPU share its array: calls that overlap on one
 * GPU (different streams, no ordering) race; calls ordered on one stream do
 * not.
 */
q1_status q1_qmm_noalloc(const void* x, int32_t x_dtype, int64_t M, const q1_weight* w, void* y, int32_t y_dtype,
                         void* stream);

/*
 * q1_dequantize -- out[N, K] = round(fl32(fl32(scale*bit) + bias)), bit-exact
 * (Higgs PR #212, "Walkthrough": Q1 dequantization kernel; rMLX #207,
 * "Current behavior": the affine_dequantize_bfloat16 kernel upstream lacks).
 *   out_dtype  Q1_BF16, Q1_F16 or Q1_F32.
 */
q1_status q1_dequantize(const q1_weight* w, void* out, int32_t out_dtype, void* stream);

/*
 * q1_embed_rows -- out[t, :] = dequantised row ids[t] of the table, rounded to
 * out_dtype, bit-exact; an id outside [0, N) writes a row of zeros (Higgs PR
 * #212, "What": embedding routed through the Q1 kernels).
 *   ids            device int32 [T] (ids_are_int64 = 0) or int64 [T] (= 1)
 *   out            [T, K] in out_dtype (Q1_BF16, Q1_F16 or Q1_F32)
 */
q1_status q1_embed_rows(const void* ids, int32_t ids_are_int64, int64_t T, const q1_weight* table, void* out,
                        int32_t out_dtype, void* stream);

/*
 * q1_ffn -- fused dense FFN, y = (SiLU(x Wg^T) * (x Wu^T)) Wd^T (Higgs PR #212,
 * "What": fused dense-FFN operations; the SiLU-times-up form is the standard
 * gated FFN of the Qwen3.5 family).
 *   x      bf16 [M, H], H = gate.K = up.K
 *   gate, up   [I, H];  down [H_out, I]  (down.K == gate.N == up.N)
 *   y      bf16 [M, H_out]
 *   Gate and up accumulate in fp32; h = SiLU(g)*u is rounded once to bf16 and
 *   is left in the workspace at byte offset Q1_WS_RESERVED_BYTES (bf16 [M, I]).
 *   With Q1_FFN_KERNEL=single (read on every call and by the workspace
 *   query), M <= max packed rows, all three matrices of one kind (symmetry
 *   and metadata dtype) and H, I multiples of 1024: ONE launch, one
 *   workgroup per compute unit.  Its workgroups first compute gate/up tiles and their h
 *   rows, then each takes a K segment of the down projection and waits until
 *   every h row of that segment is written.  The waits end because the whole
 *   grid is resident; should one still spin past its bound (about a second;
 *   only another kernel holding compute units that long can cause it), the
 *   launch sets workspace uint32 Q1_WS_STATUS_WORD to 1, finishes with y
 *   undefined, and still leaves the other counters zero.  (On MI355X it is
 *   slower than the default below.)  Otherwise, for M <= max packed
 *   rows: gate+up in one packed launch with the SiLU*mul
 *   epilogue (when gate and up share metadata dtype and symmetry; otherwise
 *   two packed launches and an element-wise kernel), then the packed down
 *   projection.  M > max packed rows: the wide path of q1_qmm per projection
 *   (gate and up share one activation image when they are the same kind),
 *   then SiLU*mul, then the down projection.
 *   workspace  q1_ffn_workspace_bytes(...) bytes; same rules as for q1_qmm.
 */
q1_status q1_ffn(const void* x, int64_t M, const q1_weight* gate, const q1_weight* up, const q1_weight* down,
                 void* y, void* workspace, size_t workspace_bytes, void* stream);

size_t q1_ffn_workspace_bytes(int64_t M, const q1_weight* gate, const q1_weight* up, const q1_weight* down);

/*
 * q1_check_symmetric -- validation of symmetric metadata stored with an
 * explicit bias (Higgs PR #212, "What": validate symmetric Q1 metadata and
 * derive bias = -scale/2; "Walkthrough": loaders compact exact symmetric
 * biases).
 *   w      an affine tensor (symmetric = 0, biases non-NULL); only its scales
 *          and biases are read.
 *   count  device uint32, written (not accumulated) by the call: the number
 *          of groups where scale or bias is not finite, or where either code
 *          dequantises to different fp32 bits with the stored bias than with
 *          the derived -scale/2 (for a nonzero scale: bias != -scale/2; a zero
 *          scale accepts either zero bias).
 *   When *count == 0 the same scales with biases = NULL, symmetric = 1 give
 *   bit-identical results in every call, without the bias bytes.
 */
q1_status q1_check_symmetric(const q1_weight* w, uint32_t* count, void* stream);

/*
 * q1_pack_signs -- dense weights to a symmetric packed Q1 tensor (Cactus PR
 * #775, commit notes: groups that hold exactly {-s, +s} repack to sign bits
 * with zero error and round-trip bit-exactly, linear LSB layout; rMLX issue
 * #207, "The good news -- packing is standard": bit0 -> -s_g, bit1 -> +s_g).
 *   dense      [N, K] in dense_dtype (Q1_BF16 or Q1_F16), 16-byte aligned
 *   packed     out: uint32 [N, K/32]
 *   scales     out: [N, K/128] in meta_dtype (Q1_BF16 or Q1_F16)
 *   inexact    device uint32, written by the call: groups that do not
 *              round-trip (see below)
 *   Per group of 128 weights: scale = round(2 * max|w|) in meta_dtype, bit =
 *   (w > 0).  A group is exact when q1_dequantize of the result (to
 *   dense_dtype) gives back every weight bit for bit -- true for any group
 *   whose weights are all +v or -v with 2v representable in meta_dtype (and
 *   v = scale/2 representable in dense_dtype); a group holding a NaN is
 *   inexact.  Inexact groups are still written (signs and max-magnitude
 *   scale: a lossy 1-bit code); the count tells the caller whether the
 *   packing lost anything.
 */
q1_status q1_pack_signs(const void* dense, int32_t dense_dtype, int64_t N, int64_t K, uint32_t* packed, void* scales,
                        int32_t meta_dtype, uint32_t* inexact, void* stream);

/* Largest M served by the packed kernel (1..8, default 8, initial value from
 * the environment variable Q1_QMM_MAX_ROWS).  Returns the previous value, or
 * -1 (value unchanged) when rows is outside 1..8.  (Higgs PR #212,
 * "Limitations": the packed-rows threshold is a tuning override.) */
int q1_set_max_packed_rows(int rows);

/* Q1_OK if `device` is a gfx950 GPU; Q1_ERR_UNSUPPORTED with a message
 * otherwise (mlx-gen backlog 0004: fail early with an explicit message when
 * the runtime cannot execute 1-bit kernels). */
q1_status q1_device_supported(int device);

/* Text of the last error on this thread ("" if none).  Static storage. */
const char* q1_last_error(void);

/* Library version string. */
const char* q1_version(void);

#ifdef __cplusplus
}
#endif

#endif /* Q1_H */
