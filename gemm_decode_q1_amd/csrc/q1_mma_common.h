// Shared pieces of the matrix-core packed kernels (q1_mma.hip, q1_ffn.hip):
// the LDS image of the fp8/bf8 activation operand and its conversion, the
// buffer-load helpers, the lane-quarter transpose and the scaled MFMA for one
// group.  Internal to the library.
#pragma once

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

// LDS image of one span (4 groups): A operand [g4][half][64 lanes][16 B],
// block scales [64 lanes][4 groups] bytes, and the group sums of the
// activations [g4][16 D rows] floats (-X/2 for symmetric tensors, X for
// affine; zero for the lo rows 8..15 and rows of activation index >= M).
// With RB = 8 (any M) each 1 KB block (g4, half) stores the 16-byte chunk of
// lane 16*qa + row at position 16*qa + (row ^ a_swz(qa, block)), and the
// blocks of group g4 start 16*g4 bytes late: reads of 8 (or 16) consecutive
// lanes still cover distinct banks, and the conversion's chunk writes (one
// activation row per 16 lanes) spread over the banks too.  With RB = 1 or 2
// (M = 1 or 2) only the live rows are stored: hi rows 0..RB-1 and lo rows
// 8..8+RB-1, 2*RB chunks per quarter; the lanes of the other rows read the
// chunk of row (row & (RB-1)) of their half (an LDS broadcast), which only
// reaches MFMA result rows that are never read.  The smaller image lets one
// workgroup hold a longer K segment.
__device__ __forceinline__ int a_blk_off(int blk) { return blk * 1024 + (blk >> 1) * 16; }
__device__ __forceinline__ int a_swz(int qa, int blk) { return qa | ((blk & 3) << 2); }

template <int RB>
struct ALay {
  static constexpr int kA = RB == 8 ? 4 * 2064 : 1024 * RB;  // A operand bytes
  static constexpr int kSc = kA;                              // block scales
  static constexpr int kXs = kA + 256;                        // group sums
  static constexpr int kSpan = kA + 512;                      // one span
  // byte offset of the chunk of (block, quarter qa, tile row r); r is a live
  // row for the writer, any row for a reader
  static __device__ __forceinline__ int chunk(int blk, int qa, int r) {
    if (RB == 8) return a_blk_off(blk) + (qa * 16 + (r ^ a_swz(qa, blk))) * 16;
    return blk * (128 * RB) + (qa * 2 * RB + (r & (RB - 1)) + RB * (r >> 3)) * 16;
  }
};
constexpr int span_bytes(int rb) { return rb == 8 ? 4 * 2064 + 512 : 1024 * rb + 512; }

// LDS image of one span for affine tensors (RT row tiles of 4 activation
// rows): per row tile an A operand image laid out as ALay<8> (rows 4p + i:
// piece p of activation row 4 rt + i; rows 12..15 zero), the block scales
// [rt][64 lanes][4 groups] bytes, and the group sums [g4][rt][16] floats (X of
// activation row 4 rt + i in entry i for the piece-0 lanes, zero in entries
// 4..15, so only one quarter of the result adds w_o X).
template <int RT>
struct AffLay {
  static constexpr int kTileA = 4 * 2064;
  static constexpr int kA = RT * kTileA;
  static constexpr int kSc = kA;
  static constexpr int kXs = kA + RT * 256;
  static constexpr int kSpan = kA + RT * 512;
};
constexpr int aff_span_bytes(int rt) { return rt * (4 * 2064 + 512); }

// per-wave LDS scratch of the word transpose: 16 rows x 34 dwords (32 used)
constexpr int kScrStride = 34;
constexpr int kScrDwords = 16 * kScrStride;

constexpr uint32_t kBufWord3 = 0x00020000u;
constexpr uint32_t kOOB = 0x80000000u;
// cache policy of loads read once per launch (packed words, scales, biases):
// non-temporal (scales with it measured 1-3 % faster at K=5120, N=17408)
constexpr int kNTLoad = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, (int)kBufWord3);
}

__device__ __forceinline__ float dpp_xor1(float v) {  // quad_perm [1,0,3,2]
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xf, 0xf, false));
}
__device__ __forceinline__ float dpp_xor2(float v) {  // quad_perm [2,3,0,1]
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xf, 0xf, false));
}


// Conversion of the activations of spans [span0, span0 + nsp) into the LDS
// image.  Item = (row m, span, word): the 32 activations of one packed word's
// weights, giving for the hi and the lo piece the two 16-byte A chunks of the
// word (bit classes 0,1 and 2,3).  The loads of all of a thread's items (at
// most kPrepRounds) are issued first (prep_load), so they can be in flight
// together with the weight loads issued right after them.
constexpr int kPrepRounds = 4;

struct PrepLoads {
  u32x4 q[kPrepRounds][4];
};

// NT: threads of the workgroup (a multiple of 64).
template <class Args>
__device__ __forceinline__ void prep_load(const Args& a, int span0, int nsp, int tid, int NT, PrepLoads& L) {
  const __amdgpu_buffer_rsrc_t rx = rsrc(a.x, a.x_bytes);
  const int items = a.M * nsp * 16;
  const float inv_nsp = 1.0f / (float)nsp;
#pragma unroll
  for (int r = 0; r < kPrepRounds; ++r) {
    const int it = tid + r * NT;
    const bool valid = it < items;
    const int wi = it & 15, ms = it >> 4;
    const int m = (int)(((float)ms + 0.5f) * inv_nsp);  // ms / nsp (exact: ms < 2^20)
    const int sp = ms - m * nsp;
    const int k0 = (span0 + sp) * 512 + wi * 32;
    const uint32_t off = (uint32_t)(((int64_t)m * a.x_ld + k0) * 2) | ((valid && k0 < a.K) ? 0u : kOOB);
    if (r * NT < items) {  // uniform: skip rounds nobody needs
#pragma unroll
      for (int c = 0; c < 4; ++c) L.q[r][c] = __builtin_amdgcn_raw_buffer_load_b128(rx, off + 16 * c, 0, 0);
    }
  }
}

template <bool AFFINE, int RB, class Args>
__device__ void prep_compute(const Args& a, int nsp, unsigned char* lds, int tid, int NT, const PrepLoads& L) {
  using Lay = ALay<RB>;
  // A rows of activation index >= M and their scales are never written: the
  // MFMA keeps rows apart, so whatever they hold only reaches result rows that
  // are never read.  The group sums enter as the accumulator input of every
  // row and must be zero for the lo rows 8..15 (and are for rows >= M).
  for (int idx = tid; idx < nsp * 64; idx += NT) {  // [g4][16] sums
    if ((idx & 15) >= a.M) reinterpret_cast<float*>(lds + (idx >> 6) * Lay::kSpan + Lay::kXs)[idx & 63] = 0.0f;
  }
  const int items = a.M * nsp * 16;
  // item = tid + 512 r: the word wi does not depend on the round; the (row,
  // span) index ms = tid/16 + 32 r is split by a rounded reciprocal
  const int wi = tid & 15;
  const int g4 = wi >> 2, b = wi & 3;
  const int blk = 2 * g4 + (b >> 1);
  const float inv_nsp = 1.0f / (float)nsp;
#pragma unroll
  for (int r = 0; r < kPrepRounds; ++r) {
    if (r * NT >= items) break;  // uniform; rounds with items keep whole waves (items % 64 == 0)
    const int it = tid + r * NT;
    const bool valid = it < items;
    const int ms = it >> 4;
    const int m = (int)(((float)ms + 0.5f) * inv_nsp);
    const int sp = ms - m * nsp;
    uint32_t wd[16];
#pragma unroll
    for (int d = 0; d < 16; ++d) wd[d] = L.q[r][d >> 2][d & 3];
    uint32_t hi[4][2], lo[4][2];
    int sc;
    float X;
    q1_convert_word(wd, hi, lo, sc, X);
    // sum over the group's 4 words (neighbouring lanes)
    X += dpp_xor1(X);
    X += dpp_xor2(X);
    if (valid) {
      // A chunk (row, quarter qa = 2*(b & 1) + c, block (g4, b >> 1)) holds in
      // dword 2*(j & 1) + hh the class-j bytes of half word hh, j >> 1 == c
      unsigned char* base = lds + sp * Lay::kSpan;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int qa = 2 * (b & 1) + c;
        *reinterpret_cast<u32x4*>(base + Lay::chunk(blk, qa, m)) =
            u32x4{hi[2 * c][0], hi[2 * c][1], hi[2 * c + 1][0], hi[2 * c + 1][1]};
        *reinterpret_cast<u32x4*>(base + Lay::chunk(blk, qa, 8 + m)) =
            u32x4{lo[2 * c][0], lo[2 * c][1], lo[2 * c + 1][0], lo[2 * c + 1][1]};
      }
      base[Lay::kSc + (m + 16 * b) * 4 + g4] = (unsigned char)(sc + 127);
      base[Lay::kSc + (8 + m + 16 * b) * 4 + g4] = (unsigned char)(sc + 123);
      if (b == 0) reinterpret_cast<float*>(base + Lay::kXs)[g4 * 16 + m] = AFFINE ? X : -0.5f * X;
    }
  }
}

// Affine conversion (AffLay<RT>): three E5M2 pieces per activation.  Zeroes
// A rows 12..15 and their scale bytes (1.0), and the group-sum entries no
// live piece-0 lane owns; the rows of activation index >= M inside a row
// tile are left unwritten (the MFMA keeps rows apart, and those results are
// never read).
template <int RT, class Args>
__device__ void prep_compute_aff(const Args& a, int nsp, unsigned char* lds, int tid, int NT, const PrepLoads& L) {
  using Lay = AffLay<RT>;
  using AL = ALay<8>;
  // zero rows 12..15: per span and row tile, 8 blocks x 4 quarters x 4 rows
  for (int idx = tid; idx < nsp * RT * 128; idx += NT) {
    const int c = idx & 127, srt = idx >> 7;
    const int sp = srt / RT, rt = srt - sp * RT;
    const int blk = c >> 4, qa = (c >> 2) & 3, r = 12 + (c & 3);
    *reinterpret_cast<u32x4*>(lds + sp * Lay::kSpan + rt * Lay::kTileA + AL::chunk(blk, qa, r)) = u32x4{0u, 0u, 0u, 0u};
  }
  // their scale dwords (lanes 12..15 + 16 j) and the group-sum entries
  // [g4][rt][16] that no conversion writes
  for (int idx = tid; idx < nsp * RT * 16; idx += NT) {
    const int j = idx & 3, r = 12 + ((idx >> 2) & 3), srt = idx >> 4;
    const int sp = srt / RT, rt = srt - sp * RT;
    reinterpret_cast<uint32_t*>(lds + sp * Lay::kSpan + Lay::kSc + rt * 256)[r + 16 * j] = 0x7f7f7f7fu;
  }
  for (int idx = tid; idx < nsp * 4 * RT * 16; idx += NT) {
    const int e = idx & 15, rest = idx >> 4;  // rest = (sp * 4 + g4) * RT + rt
    const int rt = rest % RT;
    if (e >= 4 || 4 * rt + e >= a.M)
      reinterpret_cast<float*>(lds + (rest / (4 * RT)) * Lay::kSpan + Lay::kXs)[(rest % (4 * RT)) * 16 + e] = 0.0f;
  }
  const int items = a.M * nsp * 16;
  const int wi = tid & 15;
  const int g4 = wi >> 2, b = wi & 3;
  const int blk = 2 * g4 + (b >> 1);
  const float inv_nsp = 1.0f / (float)nsp;
#pragma unroll
  for (int r = 0; r < kPrepRounds; ++r) {
    if (r * NT >= items) break;  // uniform
    const int it = tid + r * NT;
    const bool valid = it < items;
    const int ms = it >> 4;
    const int m = (int)(((float)ms + 0.5f) * inv_nsp);
    const int sp = ms - m * nsp;
    uint32_t wd[16];
#pragma unroll
    for (int d = 0; d < 16; ++d) wd[d] = L.q[r][d >> 2][d & 3];
    uint32_t pc[3][4][2];
    int sc[3];
    float X;
    q1_convert_word_bf8(wd, pc, sc, X);
    X += dpp_xor1(X);
    X += dpp_xor2(X);
    if (valid) {
      const int rt = m >> 2, i = m & 3;
      unsigned char* base = lds + sp * Lay::kSpan;
#pragma unroll
      for (int p = 0; p < 3; ++p) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int qa = 2 * (b & 1) + c;
          *reinterpret_cast<u32x4*>(base + rt * Lay::kTileA + AL::chunk(blk, qa, 4 * p + i)) =
              u32x4{pc[p][2 * c][0], pc[p][2 * c][1], pc[p][2 * c + 1][0], pc[p][2 * c + 1][1]};
        }
        base[Lay::kSc + rt * 256 + (4 * p + i + 16 * b) * 4 + g4] = (unsigned char)(sc[p] + 127);
      }
      if (b == 0) reinterpret_cast<float*>(base + Lay::kXs)[(g4 * RT + rt) * 16 + i] = X;
    }
  }
}

template <bool MBF16>
__device__ __forceinline__ float meta_f32(uint32_t bits) {
  return MBF16 ? __uint_as_float(bits << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS accesses
// (lgkmcnt 0), not for its global loads, so the load ring stays in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
}

// 4x4 transpose of (lane quarter, component): afterwards quarter q holds, in
// component c, what quarter c held in component q.
__device__ __forceinline__ void transpose_quarters(u32x4& w) {
  auto r02 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
  auto r13 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
  auto r01 = __builtin_amdgcn_permlane16_swap(r02[0], r13[0], false, false);
  auto r23 = __builtin_amdgcn_permlane16_swap(r02[1], r13[1], false, false);
  w[0] = r01[0];
  w[1] = r01[1];
  w[2] = r23[0];
  w[3] = r23[1];
}

// Scales (or biases) of one row for the 8 groups of a double span, packed as
// 16-bit values two per register.  With G % 8 == 0 they are one aligned
// 16-byte load; otherwise 8 loads of 16 bits (groups past the end read 0).
// (The 16-bit loads are combined only at use: combining them right after
// issue would make the wave wait for them.)
template <bool SC128>
__device__ __forceinline__ void load_meta8(__amdgpu_buffer_rsrc_t r, bool rowok, uint32_t row_off, int G, int g0,
                                           uint32_t* v) {
  if (SC128) {
    const u32x4 d = __builtin_amdgcn_raw_buffer_load_b128(r, (row_off + (uint32_t)g0 * 2) | (rowok ? 0u : kOOB), 0, kNTLoad);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = d[i];
  } else {
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const uint32_t o = (row_off + (uint32_t)(g0 + g) * 2) | ((rowok && g0 + g < G) ? 0u : kOOB);
      v[g] = __builtin_amdgcn_raw_buffer_load_b16(r, o, 0, kNTLoad);
    }
  }
}

template <bool MBF16, bool SC128>
__device__ __forceinline__ float meta_at(const uint32_t* v, int g) {
  if (SC128) return meta_f32<MBF16>((g & 1) ? (v[g >> 1] >> 16) : (v[g >> 1] & 0xffffu));
  return meta_f32<MBF16>(v[g]);
}

// One scaled MFMA for group g4 of a span (op_sel g4 picks the scale byte);
// g4 is a constant after unrolling.  CBSZ: A format (0 fp8 E4M3, 1 bf8 E5M2);
// B is fp4 (E2M1) with unit scales.
template <int CBSZ>
__device__ __forceinline__ v4f mfma_group(int g4, const v8i& A, const v8i& B, const v4f& C, uint32_t sa) {
  switch (g4) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, C, CBSZ, 4, 0, (int)sa, 0, 0x7f7f7f7f);
    case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, C, CBSZ, 4, 1, (int)sa, 0, 0x7f7f7f7f);
    case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, C, CBSZ, 4, 2, (int)sa, 0, 0x7f7f7f7f);
    default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, C, CBSZ, 4, 3, (int)sa, 0, 0x7f7f7f7f);
  }
}

}  // namespace
}  // namespace q1
