// The narrow-M matrix-core stage: one workgroup's share of a packed Q1
// matmul (or of the FFN's gate/up pair) for M <= 8 activation rows.
// Internal to the library.
//
//
//   y[m][n] = sum_k x[m][k] * w[n][k],   w = s*bit + b   (symmetric: b = -s/2)
//
// for M <= 8 activation rows, straight from the packed weights (Higgs PR #212,
// "What": narrow Q1 matmuls stay packed; rMLX issue #207 for the format: 32
// weights per uint32, LSB first, one scale and bias per 128 weights).
//
// Per weight row n and group g of 128 weights
//   sum_k w x = s*S + b*X,   S = sum_k bit_k x_k,   X = sum_k x_k
// (symmetric: s*(S - X/2)).  S is the product of a 0/1 matrix with the
// activations, and that product runs on v_mfma_scale_f32_16x16x128_f8f6f4:
//
// * B operand: the bits of one packed word per lane, expanded to fp4 (E2M1)
//   codes by bit class j (bits 4i+j of the word, nibble i): classes 0, 1, 2
//   keep their bit in place (codes 0.5, 1 and 2 for a set bit, 0 for a clear
//   one: one AND each) and class 3 moves its bit to position 2 (code 2).  The
//   activations of class j are pre-multiplied by 1/code (2, 1, 1/2, 1/2, all
//   powers of two, so exact), which makes each MFMA compute
//   D = S = sum of x over the set bits of the group.  Then
//     symmetric: sum w x = s (S - X/2),  affine: sum w x = s S + b X,
//   with X the group sum of x: for symmetric tensors -X/2 enters as the
//   MFMA's accumulator input, for affine ones b X is added after it.
// * A operand, symmetric tensors: each activation as two fp8 (E4M3) pieces,
//   x = hi + lo/16, with one power-of-two block scale per 32 weights chosen
//   from the block's largest |x|.  A bf16 value has 8 significant bits, hi
//   carries the top 4 (rounded) and lo the rest, so the pair is exact for
//   every element within 2^11 of its block's largest magnitude; below that
//   the error is at most 2^-19 of the block maximum, and since every weight
//   of a symmetric group has the same magnitude s/2, the product's error
//   stays below 2^-14 s sum|x| -- an eighth of the tolerance.  Rows 0..7 of
//   the 16-row A tile hold hi for the M activation rows and rows 8..15 hold
//   lo; the two halves of the result are added at the end.
// * Affine tensors: the weights of a group are w1 = fl(s + b) (set bits) and
//   w0 = b (clear bits), of any relative size, so an error relative to the
//   block's largest |x| is not relative to sum |w x|.  Two changes make it so:
//   (1) each activation is split into three E5M2 (bf8) pieces with their own
//   block scales, exact for every element within 2^25 of its block maximum
//   (q1_fp8.h); piece p of activation row m is A row 4p + m % 4 of row tile
//   m / 4 (rows 12..15 hold zeros); (2) per weight row and group the product
//   runs over the code class d whose weight is larger in magnitude (the B
//   word is complemented when d = 0), and the group's contribution is
//     (w_d - w_o) S_d + w_o X,   S_d = sum of x over the codes equal to d,
//   so the rounding of X and of the fp32 sums is multiplied by the smaller
//   weight w_o, and S_d's error by 2 |w_d|, both within the tolerance.
// * One instruction covers 16 weight rows x one group (128 weights): its fp32
//   result is multiplied by the group scale (and the bias term added) on the
//   vector ALU.
//
// Operand layouts of the instruction (gfx950, fp8 A / fp4 B):
//   A lane l: row l%16; byte e holds k-index 16*(l/16) + e (e < 16) or
//             64 + 16*(l/16) + e - 16 (e >= 16); the scale of (row r, 32-k
//             block j) is in lane r + 16*j, byte op_sel.
//   B lane l: column l%16; code e (dword e/8, nibble e%8) holds k-index
//             32*(l/16) + e, so lane l/16 = q carries word q of the group.
//   D lane l: column l%16, rows 4*(l/16) .. +3.
//
// Work decomposition.  A workgroup (8 waves) owns tiles of 16 weight rows and
// a segment of K (spans of 4 groups).  First its threads convert the segment's
// activations into the A operand image in LDS; then its items (tile, double
// span) are split evenly over the waves, each lane loading 16 bytes (one
// group's 4 words of one row) and a per-wave LDS transpose giving lane (n, q)
// word q of each group of row n.  The waves' partial sums meet in LDS and are
// added in a fixed order.  With more than one K segment (grid split), each
// segment writes fp32 partials and a second launch adds them in segment order
// (in the single-launch FFN, the last workgroup of a column does), so results
// never depend on timing.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "q1_mma_common.h"

namespace q1 {
namespace {

constexpr int kNW = 8;  // waves per workgroup
constexpr int kThreads = kNW * 64;

// Work.  Workgroup p of K segment `seg` owns tiles p, p + P, p + 2P, .. (16
// rows each; consecutive tiles go to different workgroups) and the segment's
// double spans (8 groups, 128 bytes of every row).  Its items (local tile k,
// double span d), tiles outer, are split evenly over its 8 waves: wave w takes
// items [w*I/8, (w+1)*I/8).  Each wave leaves its sum for every tile its range
// touches in LDS (slot = tile - its first tile); after the loop the slots of a
// tile are added in wave order and stored.  The ring loop itself stores
// nothing to memory: stores there would count in the same counter as the ring's
// loads and make the waits for each slot's data also wait for newer loads.
// Item i of a wave sits in ring slot i % D; its loads are issued D items
// ahead.
//
// Loads: instruction h of an item reads rows 8h..8h+7 of the tile, lane l the
// 16 bytes (group l%8, 4 words) of row l/8, so each row's 128 bytes come from
// 8 neighbouring lanes.  The MFMA B operand wants lane (n, q) = word q of every
// group of row n: the words go through a per-wave LDS scratch (row stride 34
// dwords: the 8-byte writes and 4-byte reads are bank-conflict free).
// MR: accumulator rows per lane quarter that can hold a live activation row
// (1 for M = 1, 2 for M = 2, else 4); the others are never read, so their
// scale multiply-adds are skipped.  RT (affine tensors): row tiles of 4
// activation rows (1 for M <= 4, 2 for M = 5..8); symmetric tensors use one.
//
// The stage runs as the whole of q1_mma_kernel (q1_mma.hip) and as either
// phase of the single-launch FFN (q1_ffn.hip).  WFIRST: issue the ring's first
// weight loads, then call wait() (which returns once the activations are
// readable), then load and convert the activations; otherwise the activation
// loads go first (they gate the first MFMA).  HANDOFF: with a split K, the
// last of a column's S workgroups adds the segments' partial sums itself
// (the single launch, which cannot launch again); otherwise the stage ends
// with its partials stored and a second launch adds them (q1_mma_reduce:
// the kernel boundary orders them, and measured 0.7-1.4 us faster than the
// in-kernel handoff at K=17408, N=5120).  A workgroup-uniform return ends the
// stage; lds, last_flag and wave_k0 are the caller's LDS.
struct NoWait {
  __device__ __forceinline__ void operator()() const {}
};

template <bool AFFINE, bool MBF16, bool PAIR, bool SC128, int MR, int RT, bool WFIRST = false, bool HANDOFF = false,
          class Wait = NoWait>
__device__ __forceinline__ void mma_stage(const MmaArgs& a, int seg, int p, unsigned char* lds, int* last_flag_p,
                                          int* wave_k0, const Wait& wait) {
  constexpr int RB = (AFFINE || MR == 4) ? 8 : MR;  // symmetric: A rows kept in LDS per half
  using Lay = ALay<RB>;
  constexpr int kSpanB = AFFINE ? AffLay<RT>::kSpan : Lay::kSpan;
  constexpr int NMAT = PAIR ? 2 : 1;
  // Ring slots (items in flight + those being computed).  Two: more items in
  // flight per wave congest the memory pipeline the waves issue into
  // (measured at K=5120, N=17408: 2 slots 2-5 % faster than 4 at M=2..8;
  // at K=17408, N=5120 9 % at M=1, 2; 3, 5, 6 slots slower than 4 at M=4).
  constexpr int D = 2;
  constexpr int NSC = SC128 ? 4 : 8;  // registers of metadata per row and item
  int& last_flag = *last_flag_p;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int span0 = seg * a.KSP;                                    // even
  const int nsp = (span0 + a.KSP <= a.nspan) ? a.KSP : a.nspan - span0;
  const int nds = (nsp + 1) >> 1;                                   // double spans of the segment
  const int ntiles = (int)((a.N + 15) >> 4);
  const int nbp = (ntiles - p + a.P - 1) / a.P;                     // tiles of this workgroup
  const int I = nbp * nds;                                          // items of this workgroup
  const int i0 = (wave * I) / kNW, i1 = ((wave + 1) * I) / kNW;
  const int nitems = i1 - i0;
  // [w][slot][mt][ab][64] (affine: [w][slot][mt][rt][64])
  float* red = reinterpret_cast<float*>(lds + (size_t)a.KSP * kSpanB);
  uint32_t* scr = reinterpret_cast<uint32_t*>(lds + (size_t)a.KSP * kSpanB + (size_t)a.red_bytes) +
                  wave * (NMAT * kScrDwords);

  const __amdgpu_buffer_rsrc_t rp[2] = {rsrc(a.p0, a.packed_bytes), rsrc(PAIR ? a.p1 : a.p0, a.packed_bytes)};
  const __amdgpu_buffer_rsrc_t rs[2] = {rsrc(a.s0, a.meta_bytes), rsrc(PAIR ? a.s1 : a.s0, a.meta_bytes)};
  const __amdgpu_buffer_rsrc_t rbias[2] = {rsrc(AFFINE ? a.b0 : a.s0, a.meta_bytes),
                                           rsrc(AFFINE && PAIR ? a.b1 : a.s0, a.meta_bytes)};

  const int nl = lane & 15;   // weight row within a tile (B and D column)
  const int q = lane >> 4;    // lane quarter
  const int lr = lane >> 3;   // row within a load instruction
  const int lc = lane & 7;    // 16-byte chunk (group) within a row's 128 bytes
  const int a_lane0 = Lay::chunk(0, q, nl);  // (RB < 8) this lane's A chunk within a block
  const uint32_t row_bytes = (uint32_t)a.K >> 3;
  // row indices fit in 31 bits (the plan keeps N*K/8 below 2^31)
  const int Nrows = (int)a.N;
  auto tile_of = [&](int k) -> int { return k * a.P + p; };

  u32x4 words[D][NMAT][2];
  uint32_t sreg[D][NMAT][NSC];
  uint32_t breg[D][NMAT][NSC];
  float acc[NMAT][4 * RT];  // [mt][rt * 4 + i]
#pragma unroll
  for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
    for (int i = 0; i < 4 * RT; ++i) acc[mt][i] = 0.0f;

  // issue the loads of item (local tile k, double span d) into slot u
  auto issue = [&](int u, int k, int d, bool ok) {
    const int sp = span0 + 2 * d;  // first span of the double span
    const int r0 = tile_of(k) * 16 + lr;
    const int g = 4 * sp + lc;     // this lane's group
    const uint32_t col = (uint32_t)(sp * 64) + (uint32_t)lc * 16u;
    const bool gok = ok && g < a.G;
    const uint32_t o0 = ((uint32_t)r0 * row_bytes + col) | ((gok && r0 < Nrows) ? 0u : kOOB);
    const uint32_t o1 = ((uint32_t)(r0 + 8) * row_bytes + col) | ((gok && r0 + 8 < Nrows) ? 0u : kOOB);
    const int n = tile_of(k) * 16 + nl;
    const bool nok = ok && n < Nrows;
    const uint32_t mo = (uint32_t)n * (uint32_t)a.G * 2u;
#pragma unroll
    for (int mt = 0; mt < NMAT; ++mt) {
      words[u][mt][0] = __builtin_amdgcn_raw_buffer_load_b128(rp[mt], o0, 0, kNTLoad);
      words[u][mt][1] = __builtin_amdgcn_raw_buffer_load_b128(rp[mt], o1, 0, kNTLoad);
      load_meta8<SC128>(rs[mt], nok, mo, a.G, 4 * sp, sreg[u][mt]);
      if (AFFINE) load_meta8<SC128>(rbias[mt], nok, mo, a.G, 4 * sp, breg[u][mt]);
    }
  };

  // activation loads first, then the first item of weights, the conversion
  // (which waits for the activations only), then the other D - 1 items.  A
  // wave issues its loads in order and stalls while the memory pipeline is
  // full, so issuing all D items before the conversion delays it (measured:
  // 5-7 % slower at config 2).  Slots are still issued in the loop's order,
  // so the loop-head waits stay exact.
  PrepLoads pl;
  if constexpr (!WFIRST) prep_load(a, span0, 2 * nds, tid, kThreads, pl);
  int pk = i0 / (nds > 0 ? nds : 1), pd = i0 - pk * nds;
  auto issue_next = [&](int u) {
    issue(u, pk, pd, u < nitems);
    __builtin_amdgcn_sched_barrier(0);
    if (++pd == nds) {
      pd = 0;
      ++pk;
    }
  };
  issue_next(0);
  if constexpr (WFIRST) {
#pragma unroll
    for (int u = 1; u < D; ++u) issue_next(u);
    wait();
    prep_load(a, span0, 2 * nds, tid, kThreads, pl);
  }
  if constexpr (AFFINE)
    prep_compute_aff<RT>(a, 2 * nds, lds, tid, kThreads, pl);
  else
    prep_compute<false, RB>(a, 2 * nds, lds, tid, kThreads, pl);
  if constexpr (!WFIRST) {
#pragma unroll
    for (int u = 1; u < D; ++u) issue_next(u);
  }
  lds_barrier();

  auto compute = [&](int u, int d) {
    // B words of all groups: lane (n, q) gets word q of groups 0..7 of row n
    uint32_t bw[NMAT][8];
#pragma unroll
    for (int mt = 0; mt < NMAT; ++mt) {
      uint32_t* t = scr + mt * kScrDwords;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint2* dst = reinterpret_cast<uint2*>(t + (8 * h + lr) * kScrStride + 4 * lc);
        dst[0] = uint2{words[u][mt][h][0], words[u][mt][h][1]};
        dst[1] = uint2{words[u][mt][h][2], words[u][mt][h][3]};
      }
#pragma unroll
      for (int g = 0; g < 8; ++g) bw[mt][g] = t[nl * kScrStride + 4 * g + q];
    }
    if constexpr (AFFINE) {
      using AL = AffLay<RT>;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const unsigned char* base = lds + (2 * d + half) * kSpanB;
        uint32_t scale_a[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          scale_a[rt] = reinterpret_cast<const uint32_t*>(base + AL::kSc + rt * 256)[lane];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          v8i A[RT];
          v4f XS[RT];
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const unsigned char* tb = base + rt * AL::kTileA;
            const int lane_sw = lane ^ q;
            const u32x4 h0 = reinterpret_cast<const u32x4*>(tb + a_blk_off(2 * g4))[lane_sw ^ ((g4 & 1) << 3)];
            const u32x4 h1 = reinterpret_cast<const u32x4*>(tb + a_blk_off(2 * g4 + 1))[lane_sw ^ (4 | ((g4 & 1) << 3))];
            A[rt] = v8i{(int)h0[0], (int)h0[1], (int)h0[2], (int)h0[3], (int)h1[0], (int)h1[1], (int)h1[2], (int)h1[3]};
            XS[rt] = reinterpret_cast<const v4f*>(base + AL::kXs)[(g4 * RT + rt) * 4 + q];
          }
#pragma unroll
          for (int mt = 0; mt < NMAT; ++mt) {
            // weights of the two codes; the product runs over the code whose
            // weight is larger in magnitude (d), the other enters through X
            const float sv = meta_at<MBF16, SC128>(sreg[u][mt], 4 * half + g4);
            const float bv = meta_at<MBF16, SC128>(breg[u][mt], 4 * half + g4);
            const float w1 = sv + bv;
            const bool d1 = fabsf(w1) >= fabsf(bv);
            const float dw = w1 - bv;
            const float sd = d1 ? dw : -dw;  // w_d - w_o
            const float wo = d1 ? bv : w1;
            const uint32_t wd = bw[mt][4 * half + g4] ^ (d1 ? 0u : 0xffffffffu);
            const v8i B = {(int)(wd & 0x11111111u), (int)(wd & 0x22222222u), (int)(wd & 0x44444444u),
                           (int)((wd >> 1) & 0x44444444u), 0, 0, 0, 0};
            const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
              const v4f Dv = mfma_group<1>(g4, A[rt], B, zero, scale_a[rt]);
#pragma unroll
              for (int i = 0; i < MR; ++i) {
                acc[mt][4 * rt + i] = fmaf(sd, Dv[i], acc[mt][4 * rt + i]);
                acc[mt][4 * rt + i] = fmaf(wo, XS[rt][i], acc[mt][4 * rt + i]);
              }
            }
          }
        }
      }
    } else {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const unsigned char* base = lds + (2 * d + half) * Lay::kSpan;
        const uint32_t scale_a = reinterpret_cast<const uint32_t*>(base + Lay::kSc)[lane];
        v8i A[4];
        v4f XS[4];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          u32x4 h0, h1;
          if (RB == 8) {
            const int lane_sw = lane ^ q;  // position before the block's part of the swizzle
            h0 = reinterpret_cast<const u32x4*>(base + a_blk_off(2 * g4))[lane_sw ^ ((g4 & 1) << 3)];
            h1 = reinterpret_cast<const u32x4*>(base + a_blk_off(2 * g4 + 1))[lane_sw ^ (4 | ((g4 & 1) << 3))];
          } else {
            h0 = *reinterpret_cast<const u32x4*>(base + 2 * g4 * (128 * RB) + a_lane0);
            h1 = *reinterpret_cast<const u32x4*>(base + (2 * g4 + 1) * (128 * RB) + a_lane0);
          }
          A[g4] = v8i{(int)h0[0], (int)h0[1], (int)h0[2], (int)h0[3], (int)h1[0], (int)h1[1], (int)h1[2], (int)h1[3]};
          XS[g4] = reinterpret_cast<const v4f*>(base + Lay::kXs)[g4 * 4 + q];
        }
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt) {
          v4f Dg[4];
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const uint32_t wd = bw[mt][4 * half + g4];
            const v8i B = {(int)(wd & 0x11111111u), (int)(wd & 0x22222222u), (int)(wd & 0x44444444u),
                           (int)((wd >> 1) & 0x44444444u), 0, 0, 0, 0};
            Dg[g4] = mfma_group<0>(g4, A[g4], B, XS[g4], scale_a);  // C = -X/2
          }
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const float sv = meta_at<MBF16, SC128>(sreg[u][mt], 4 * half + g4);
#pragma unroll
            for (int i = 0; i < MR; ++i) acc[mt][i] = fmaf(sv, Dg[g4][i], acc[mt][i]);
          }
        }
      }
    }
  };

  // one result (activation row m, weight row `row`): the output, or with a
  // split K the segment's partial sum
  auto emit = [&](int m, int row, const float* v) {
    if (a.S == 1) {
      if (PAIR)
        static_cast<uint16_t*>(a.out)[m * a.out_ld + row] = (uint16_t)f32_to_bf16_bits(silu_f32(v[0]) * v[1]);
      else
        store_out(a.out, a.out_dtype, m * a.out_ld + row, v[0]);
    } else {
#pragma unroll
      for (int mt = 0; mt < NMAT; ++mt) {
        float* dst = &a.partial[(((int64_t)seg * a.M + m) * NMAT + mt) * a.N + row];
        if (HANDOFF)
          __hip_atomic_store(dst, v[mt], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          *dst = v[mt];
      }
    }
  };

  // End of this wave's part of local tile k: lane l of half ab holds
  // activation row 4*((l>>4)&1) + 2*ab + (l>>5) of weight row l & 15 (hi + lo
  // combined); it goes to LDS slot (wave, k - first tile of the wave).
  const int kfirst = i0 / (nds > 0 ? nds : 1);
  // Affine: quarter q of row tile rt holds piece q of activation rows
  // 4 rt + i (element i); the four quarters are added (quarter 3 is zero),
  // leaving activation row 4 rt + i in 16-lane row ((i & 1) << 1) | (i >> 1)
  // of slot rt.
  auto tile_done = [&](int k) {
#pragma unroll
    for (int mt = 0; mt < NMAT; ++mt) {
      float* slot = red + (((wave * a.TW + (k - kfirst)) * NMAT + mt) * 2) * 64 + lane;
      if constexpr (AFFINE) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const float* v = &acc[mt][4 * rt];
          auto p01 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0]), __float_as_uint(v[1]), false, false);
          auto p23 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[2]), __float_as_uint(v[3]), false, false);
          const float s01 = __uint_as_float(p01[0]) + __uint_as_float(p01[1]);
          const float s23 = __uint_as_float(p23[0]) + __uint_as_float(p23[1]);
          auto pp = __builtin_amdgcn_permlane16_swap(__float_as_uint(s01), __float_as_uint(s23), false, false);
          slot[64 * rt] = __uint_as_float(pp[0]) + __uint_as_float(pp[1]);
        }
      } else {
        auto p01 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[mt][0]), __float_as_uint(acc[mt][1]), false,
                                                    false);
        auto p23 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[mt][2]), __float_as_uint(acc[mt][3]), false,
                                                    false);
        slot[0] = __uint_as_float(p01[0]) + __uint_as_float(p01[1]);
        slot[64] = __uint_as_float(p23[0]) + __uint_as_float(p23[1]);
      }
#pragma unroll
      for (int i = 0; i < 4 * RT; ++i) acc[mt][i] = 0.0f;
    }
  };

  // Whole turns of the ring (slots past the end load nothing, compute
  // nothing and end no tile): a loop body without early exits keeps the ring
  // in place across iterations.
  const int nitems_pad = (nitems + D - 1) / D * D;
  int k = kfirst, d = i0 - kfirst * nds;  // current item
  int ik = k, id = d + D;                 // item + D (next loads)
  while (nds > 0 && id >= nds) {
    id -= nds;
    ++ik;
  }
  for (int base = 0; base < nitems_pad; base += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      if (base + u < nitems) compute(u, d);  // (uniform) the last turn's empty slots do no work
      issue(u, ik, id, base + u + D < nitems);
      __builtin_amdgcn_sched_barrier(0);  // keep items apart: bounded register use
      if (base + u < nitems && (d == nds - 1 || base + u == nitems - 1)) tile_done(k);
      if (++d == nds) {
        d = 0;
        ++k;
      }
      if (++id == nds) {
        id = 0;
        ++ik;
      }
    }
  }

  // ---- tile results: the slots of the waves that touched each tile, in
  // wave order.  Thread o takes (tile kk, activation row m, weight row r),
  // rows fastest; the waves' first tiles come through LDS, so the loop does
  // no integer division. ----
  if (lane == 0) wave_k0[wave] = kfirst;
  lds_barrier();
  {
    const int per_t = 16 * a.M;
    const float inv_per_t = 1.0f / (float)per_t;
    const float inv_I = I > 0 ? 1.0f / (float)I : 0.0f;
    for (int o = tid; o < nbp * per_t; o += kThreads) {
      const int kk = (int)(((float)o + 0.5f) * inv_per_t);  // o / per_t (exact: o < 2^22)
      const int rem = o - kk * per_t;
      const int m = rem >> 4, r = rem & 15;
      const int row = tile_of(kk) * 16 + r;
      if (row >= Nrows) continue;
      const int t0 = kk * nds, t1 = t0 + nds;  // the tile's items
      // wave holding item t0: the last w with w*I/8 <= t0 (estimate, then exact)
      int wa = (int)((float)(8 * t0 + 7) * inv_I);
      wa = wa > kNW - 1 ? kNW - 1 : wa;
      while (wa > 0 && ((wa * I) >> 3) > t0) --wa;
      while (wa < kNW - 1 && (((wa + 1) * I) >> 3) <= t0) ++wa;
      // position of (m, r) in the slots (see tile_done)
      const int l = AFFINE ? r + 16 * (((m & 1) << 1) | ((m >> 1) & 1)) : r + 16 * ((m >> 2) & 1) + 32 * (m & 1);
      const int ab = AFFINE ? (m >> 2) : (m >> 1) & 1;
      float v[NMAT];
#pragma unroll
      for (int mt = 0; mt < NMAT; ++mt) v[mt] = 0.0f;
      for (int w2 = wa; w2 < kNW && ((w2 * I) >> 3) < t1; ++w2) {
        if ((((w2 + 1) * I) >> 3) == ((w2 * I) >> 3)) continue;  // wave without items
        const int sl = kk - wave_k0[w2];
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt) v[mt] += red[(((w2 * a.TW + sl) * NMAT + mt) * 2 + ab) * 64 + l];
      }
      emit(m, row, v);
    }
  }
  if (a.S == 1 || !HANDOFF) return;

  // ---- split K: the last of the S workgroups with this p adds the
  // partials of p's tiles in segment order.  The workgroup's partial stores
  // happen before its arrival: a workgroup barrier, then an agent-scope
  // release on the counter.  The last arrival's read of the counter is
  // followed by one agent-scope acquire fence (thread 0), and the barrier
  // that hands out the flag orders the other waves' reads after it.  (An
  // acquire in every wave costs an L2 invalidation each: measured +8 us at
  // K=17408, N=5120, against +1 us for the single one; acq_rel on every
  // arrival +2 us.) ----
  __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores have completed
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&a.counters[p], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    last_flag = old == (uint32_t)(a.S - 1);
    if (last_flag) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  if (!last_flag) return;
  const int per_m = nbp * 16;
  const float inv_per_m = 1.0f / (float)per_m;
  for (int o = tid; o < per_m * a.M; o += kThreads) {
    const int m = (int)(((float)o + 0.5f) * inv_per_m);  // o / per_m (exact: o < 2^22)
    const int rem = o - m * per_m;
    const int row = tile_of(rem >> 4) * 16 + (rem & 15);
    if (row >= Nrows) continue;
    float v[NMAT];
#pragma unroll
    for (int mt = 0; mt < NMAT; ++mt) {
      // segment order; the loads go out four at a time (one after the other,
      // each waited for before the next, they cost S memory latencies)
      const float* pp = a.partial + ((int64_t)m * NMAT + mt) * a.N + row;
      const int64_t sstep = (int64_t)a.M * NMAT * a.N;
      auto ld = [&](int s2) { return __hip_atomic_load(pp + s2 * sstep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
      float sum = 0.0f;
      for (int s2 = 0; s2 < a.S; s2 += 4) {  // a short last batch re-reads segment S-1 and drops it
        const int sl = a.S - 1;
        const float p0 = ld(s2), p1 = ld(min(s2 + 1, sl)), p2 = ld(min(s2 + 2, sl)), p3 = ld(min(s2 + 3, sl));
        sum += p0;
        if (s2 + 1 < a.S) sum += p1;
        if (s2 + 2 < a.S) sum += p2;
        if (s2 + 3 < a.S) sum += p3;
      }
      v[mt] = sum;
    }
    if (PAIR)
      static_cast<uint16_t*>(a.out)[m * a.out_ld + row] = (uint16_t)f32_to_bf16_bits(silu_f32(v[0]) * v[1]);
    else
      store_out(a.out, a.out_dtype, m * a.out_ld + row, v[0]);
  }
  if (tid == 0) __hip_atomic_store(&a.counters[p], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace
}  // namespace q1
