// Single-launch dense FFN for M <= 8 activation rows:
//
//   h = bf16(SiLU(x Wg^T) * (x Wu^T)),   y = h Wd^T
//
// (Higgs PR #212, "What": the fused dense-FFN operations of the Bonsai models;
// the same page's "Validation" fuses tensor pairs the same way).  Gate, up and
// down are packed Q1 matrices of one kind (all symmetric or all affine, one
// metadata dtype).
//
// One persistent workgroup per compute unit runs two phases of the
// matrix-core stage (q1_mma_stage.h):
//
// * Phase 1, the gate/up pair: workgroup w < P1 owns row tiles w, w + P1, ..
//   of both matrices over the whole of K and writes their h rows (bf16).
//   When its stores have completed it publishes them with one agent-scope
//   release, then adds, per K segment of the down projection, the number of
//   its tiles that fall in that segment (h row 16t..16t+15 of tile t is
//   column 16t.. of down's K).
// * Phase 2, the down projection split into S K segments (plan_ffn picks
//   the split whose busiest workgroup, phase-1 items plus its phase-2 unit,
//   has the fewest items).  A unit (segment, column p) issues its first weight loads,
//   then waits until its segment's counter shows every phase-1 tile of the
//   segment, takes one agent-scope acquire, and converts its part of h; the
//   segments' partial sums meet in the stage's in-kernel handoff (HANDOFF in
//   q1_mma_stage.h: the last arrival per column adds them in segment order).
//
// Every phase-1 tile is owned by a workgroup of the same grid, and the grid
// is one workgroup per compute unit, so all producers are resident and the
// waits end.  They are bounded anyway: a wait that spins past its limit (which
// takes another kernel holding compute units for the whole time) sets the
// status word at the end of the workspace's counter block to 1 and goes on
// with whatever h holds, so every workgroup exits; y is then undefined.  The
// last workgroup to finish clears the segment counters and its own exit
// counter, so a call leaves the counter block as it found it.
//
// Measured at hidden 5120, intermediate 17408 (fp16 symmetric, M = 1..8):
// 32-39 us against 18-24 us for the pair launch followed by the down launch,
// which therefore stays the default (this launch is selected by
// Q1_FFN_KERNEL=single).  Per-workgroup timestamps show why: the agent-scope
// release that publishes h is an L2 write-back, which under the weight stream
// takes about 5 us; and since every phase-1 workgroup owns tiles in every
// segment, phase 2 starts only once phase 1 has ended everywhere, so the two
// phases do not overlap beyond the first two weight items of each wave.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "q1_mma_stage.h"

namespace q1 {
namespace {

struct FfnArgs {
  MmaArgs gu;          // phase 1
  MmaArgs d;           // phase 2 (x = h)
  uint32_t* seg_done;  // [kSegStride * s]: phase-1 tiles finished in down K segment s
  uint32_t* exit_cnt;  // workgroups finished
  uint32_t* status;    // 1: a wait gave up
  int32_t units2;      // phase-2 units (d.S * d.P), on workgroups wgs-1, wgs-2, ..
  int32_t seg_tiles;   // phase-1 tiles per down K segment
  uint32_t spin_limit;
};

// A wait polls about once a microsecond (s_sleep 24 = 1536 clocks, plus the
// load): 2^20 polls bound it near a second.  Each segment counter sits on a
// 256-byte line of its own, away from the split-K counters, so the waiting
// workgroups of one segment poll one line and the producers' adds land on
// lines nobody else polls (one shared line measured 3-6 us of extra delay).
constexpr uint32_t kSpinLimit = 1u << 20;
constexpr int kSegBase = 1024, kSegStride = 64, kExitWord = 2048;  // uint32 indices in the counter block

// RT: affine row tiles (1 for M <= 4, 2 for M = 5..8); MR2: live accumulator
// rows of the down phase (1 for M = 1, 2 for M = 2, else 4; the pair phase
// always keeps 8-row activation images, as in q1_mma.hip).
template <bool AFFINE, bool MBF16, int RT, int MR2>
__global__ __launch_bounds__(kThreads) void q1_ffn_kernel(FfnArgs f) {
  extern __shared__ __align__(16) unsigned char lds[];
  __shared__ int last_flag;
  __shared__ int wave_k0[kNW];
  const int w = (int)blockIdx.x;
  const int tid = threadIdx.x;
  const int ntiles1 = (int)((f.gu.N + 15) >> 4);

  if (w < f.gu.P) {
    mma_stage<AFFINE, MBF16, true, true, 4, RT>(f.gu, 0, w, lds, &last_flag, wave_k0, NoWait{});
    __builtin_amdgcn_s_waitcnt(0);  // this wave's h stores have completed
    __syncthreads();
    if (tid == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      // tiles w + k P1 in increasing k: their segments do not decrease
      int t = w;
      while (t < ntiles1) {
        const int s = t / f.seg_tiles;
        uint32_t n = 0;
        while (t < ntiles1 && t / f.seg_tiles == s) {
          ++n;
          t += f.gu.P;
        }
        __hip_atomic_fetch_add(&f.seg_done[kSegStride * s], n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }

  const int u = (int)gridDim.x - 1 - w;
  if (u < f.units2) {
    const int seg = u % f.d.S, p2 = u / f.d.S;
    const int t0 = seg * f.seg_tiles;
    const uint32_t need = (uint32_t)(std::min(t0 + f.seg_tiles, ntiles1) - t0);
    auto wait_h = [&]() {
      if (tid == 0) {
        uint32_t spins = 0;
        while (__hip_atomic_load(&f.seg_done[kSegStride * seg], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
          if (++spins > f.spin_limit) {
            __hip_atomic_store(f.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(24);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      }
      __syncthreads();
    };
    mma_stage<AFFINE, MBF16, false, true, MR2, RT, true, true>(f.d, seg, p2, lds, &last_flag, wave_k0, wait_h);
  }

  __syncthreads();
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(f.exit_cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == gridDim.x - 1) {
      for (int s = 0; s < f.d.S; ++s) __hip_atomic_store(&f.seg_done[kSegStride * s], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(f.exit_cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <bool AFFINE, bool MBF16, int RT, int MR2>
hipError_t launch_f(const FfnPlan& p, const FfnArgs& a, hipStream_t s) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&q1_ffn_kernel<AFFINE, MBF16, RT, MR2>), hipFuncAttributeMaxDynamicSharedMemorySize,
      160 * 1024 - 64);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((q1_ffn_kernel<AFFINE, MBF16, RT, MR2>), dim3((unsigned)p.wgs), dim3(kThreads), p.lds_bytes, s, a);
  return hipGetLastError();
}

template <bool AFFINE, bool MBF16>
hipError_t launch_m(const FfnPlan& p, const FfnArgs& a, hipStream_t s) {
  const int M = p.gu.M;
  if constexpr (AFFINE) {
    if (M > 4) return launch_f<AFFINE, MBF16, 2, 4>(p, a, s);
  }
  if (M > 2) return launch_f<AFFINE, MBF16, 1, 4>(p, a, s);
  return M == 1 ? launch_f<AFFINE, MBF16, 1, 1>(p, a, s) : launch_f<AFFINE, MBF16, 1, 2>(p, a, s);
}

}  // namespace

bool plan_ffn(int M, int64_t I, int64_t H, int64_t Ho, bool affine, FfnPlan* p, const char** why) {
  if (M < 1 || M > 8) {
    *why = "single-launch FFN handles 1..8 activation rows";
    return false;
  }
  if (H % 1024 != 0 || I % 1024 != 0 || Ho < 1) {
    *why = "single-launch FFN needs hidden and intermediate sizes that are multiples of 1024";
    return false;
  }
  if (I * (H / 8) >= ((int64_t)1 << 31) || Ho * (I / 8) >= ((int64_t)1 << 31) || (int64_t)M * I * 2 >= ((int64_t)1 << 31)) {
    *why = "FFN matrices too large for 32-bit buffer offsets";
    return false;
  }
  const int cus = device_cus();
  p->wgs = cus;
  if (!plan_mma_split(M, I, H, true, affine, 1, cus, &p->gu)) {
    *why = "gate/up rows too long for one workgroup's activation image";
    return false;
  }
  const int P1 = p->gu.P;
  const int nds1 = p->gu.KSP / 2;
  const int64_t nt1 = p->gu.ntiles;
  auto load1 = [&](int w) -> int64_t { return w < P1 ? 2 * nds1 * ((nt1 - w + P1 - 1) / P1) : 0; };
  int64_t max1 = 0;
  for (int w = 0; w < cus; ++w) max1 = std::max(max1, load1(w));
  // Phase-2 split: the one whose busiest workgroup (phase-1 items plus its
  // phase-2 unit, a split counting as in plan_mma) has the fewest items.
  const int ndsp2 = ((int)(I / 128) + 7) / 8;
  int64_t best_cost = -1;
  for (int S = 1; S <= ndsp2; ++S) {
    MmaPlan c;
    if (!plan_mma_split(M, Ho, I, false, affine, S, cus / S > 0 ? cus / S : 1, &c)) continue;
    const int units = c.S * c.P;
    if (units > cus || c.P > kSegBase || kSegBase + kSegStride * c.S > kExitWord) continue;
    int64_t cost = max1;
    for (int u = 0; u < units; ++u) {
      const int seg = u % c.S, p2 = u / c.S;
      const int nsp = std::min(c.KSP, c.nspan - seg * c.KSP);
      const int64_t items = ((c.ntiles - p2 + c.P - 1) / c.P) * ((nsp + 1) / 2) + (c.S > 1 ? 6 + c.S / 2 : 0);
      cost = std::max(cost, load1(cus - 1 - u) + items);
    }
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      p->d = c;
    }
  }
  if (best_cost < 0) {
    *why = "no split of the down projection fits";
    return false;
  }
  p->lds_bytes = std::max(p->gu.lds_bytes, p->d.lds_bytes);
  p->sync_words = kExitWord + 1;
  return true;
}

hipError_t launch_ffn(const FfnPlan& p, const uint16_t* x, const QMat& gate, const QMat& up, const QMat& down,
                      uint16_t* h, void* y, float* partial, uint32_t* sync, hipStream_t s) {
  FfnArgs a;
  const int64_t I = gate.N, H = gate.K, Ho = down.N;
  a.gu = mma_args(p.gu, x, H, gate, &up, h, BF16, I, nullptr, nullptr);
  a.d = mma_args(p.d, h, I, down, nullptr, y, BF16, Ho, partial, sync);
  a.seg_done = sync + kSegBase;
  a.exit_cnt = sync + kExitWord;
  a.status = sync + kFfnStatusWord;
  a.units2 = p.d.S * p.d.P;
  a.seg_tiles = p.d.KSP * 32;
  a.spin_limit = kSpinLimit;
  const bool mbf16 = gate.meta_bf16 != 0;
  if (gate.symmetric) return mbf16 ? launch_m<false, true>(p, a, s) : launch_m<false, false>(p, a, s);
  return mbf16 ? launch_m<true, true>(p, a, s) : launch_m<true, false>(p, a, s);
}

}  // namespace q1
