// Metadata kernels of the Q1 library: the symmetric-bias check and the exact
// sign packer.
//
// q1_symcheck_kernel  Higgs PR #212 ("What": validate symmetric Q1 metadata;
//                     "Walkthrough": loaders compact exact symmetric biases).
//                     A group can drop its bias when the derived bias -s/2
//                     gives the same dequantised values as the stored one.
// q1_pack_kernel      Cactus PR #775 (commit notes: groups that hold exactly
//                     {-s, +s} repack to one sign bit per weight with zero
//                     error, round trip bit-exact; linear LSB layout) in the
//                     format of rMLX issue #207 (bit0 -> -s_g, bit1 -> +s_g,
//                     stored scale 2 s_g, symmetric).
//
// Both are HBM-bound streams; both count through one device counter (one
// atomic per workgroup) that a one-thread kernel clears first (a kernel, not a memset, so the calls can be
// captured in a graph).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "q1_device.h"
#include "q1_internal.h"

namespace q1 {
namespace {

__global__ void q1_clear_u32(uint32_t* p) { *p = 0u; }

__device__ __forceinline__ bool finite_f32(float v) { return (__float_as_uint(v) & 0x7f800000u) != 0x7f800000u; }

constexpr int kMetaThreads = 1024;

// Add the workgroup's per-thread counts to *count: a wave sum, a sum of the
// waves in LDS, then one atomic per workgroup (only when nonzero).  Every
// thread of the workgroup must call it.  Atomics on the one counter serialise,
// so the launches keep to two workgroups per CU.
__device__ __forceinline__ void block_count(uint32_t v, uint32_t* count) {
  __shared__ uint32_t part[kMetaThreads / 64];
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t sum = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) sum += part[w];
    if (sum != 0) atomicAdd(count, sum);
  }
}

// ---------------------------------------------------------------------------
// Symmetric check.  Group g matches when scale and bias are finite and both
// codes dequantise to the same fp32 bits with the stored bias b and with the
// derived bias -s/2:  fl(s*c + b) == fl(s*c - s/2) for c = 0, 1.  (For a
// nonzero scale that is b == -s/2; a zero scale accepts either zero.)
// ---------------------------------------------------------------------------
template <bool MBF16>
__global__ __launch_bounds__(kMetaThreads) void q1_symcheck_kernel(const uint16_t* __restrict__ scales,
                                                          const uint16_t* __restrict__ biases, int64_t ngroups,
                                                          uint32_t* __restrict__ count) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t bad = 0;
  for (int64_t g = t0; g < ngroups; g += stride) {
    const float s = meta_to_f32<MBF16>(scales[g]);
    const float b = meta_to_f32<MBF16>(biases[g]);
    const float d = -0.5f * s;
    const bool same = finite_f32(s) && finite_f32(b) &&
                      __float_as_uint(__builtin_fmaf(s, 0.0f, b)) == __float_as_uint(__builtin_fmaf(s, 0.0f, d)) &&
                      __float_as_uint(__builtin_fmaf(s, 1.0f, b)) == __float_as_uint(__builtin_fmaf(s, 1.0f, d));
    bad += same ? 0u : 1u;
  }
  block_count(bad, count);
}

// ---------------------------------------------------------------------------
// Sign packer.  One thread per packed word (32 consecutive weights of a row);
// the 4 words of a group are 4 neighbouring lanes (a DPP quad), since words
// are row-major [N, K/32] with K/32 a multiple of 4.  Per group:
//   a = max |w| (fp32), scale = round_meta(2a), bit = (w > 0),
//   exact  iff every weight equals its dequantised value
//          round_dense(fl(scale*bit - scale/2)) bit for bit,
// so exact groups survive q1_dequantize unchanged.  A NaN makes its group
// inexact.  The count of inexact groups is added to *count.
// ---------------------------------------------------------------------------
template <bool DBF16>
__device__ __forceinline__ float dense_to_f32(uint32_t b) {
  return DBF16 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
}

template <bool DBF16>
__device__ __forceinline__ uint32_t f32_to_dense(float v) {
  return DBF16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v);
}

__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xf, 0xf, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xf, 0xf, false)));
  return v;
}

__device__ __forceinline__ uint32_t quad_and(uint32_t v) {
  v &= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xf, 0xf, false);
  v &= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xf, 0xf, false);
  return v;
}

template <bool DBF16, bool MBF16>
__global__ __launch_bounds__(kMetaThreads) void q1_pack_kernel(const uint16_t* __restrict__ dense, int64_t nwords,
                                                      uint32_t* __restrict__ packed, uint16_t* __restrict__ scales,
                                                      uint32_t* __restrict__ count) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;  // a multiple of 64
  // Every lane runs the same number of iterations (indices past the end are
  // clamped and their results dropped), so the quad exchanges always see
  // whole, active quads.
  const int64_t base0 = (int64_t)blockIdx.x * blockDim.x;
  const int64_t iters = nwords > base0 ? (nwords - base0 + stride - 1) / stride : 0;
  uint32_t bad = 0;
  for (int64_t it = 0; it < iters; ++it) {
    const int64_t t = base0 + it * stride + threadIdx.x;
    const bool live = t < nwords;  // nwords % 4 == 0: quads are live or dead together
    const int64_t tc = live ? t : nwords - 1;
    const uint4* src = reinterpret_cast<const uint4*>(dense + tc * 32);
    uint32_t h[16];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 v = src[c];
      h[4 * c + 0] = v.x;
      h[4 * c + 1] = v.y;
      h[4 * c + 2] = v.z;
      h[4 * c + 3] = v.w;
    }
    float a = 0.0f;
    bool nan = false;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float w = dense_to_f32<DBF16>((h[i >> 1] >> (16 * (i & 1))) & 0xffffu);
      nan |= (w != w);
      a = fmaxf(a, fabsf(w));
    }
    a = quad_max(a);
    const uint32_t sbits = MBF16 ? f32_to_bf16_bits(2.0f * a) : f32_to_f16_bits(2.0f * a);
    const float s = meta_to_f32<MBF16>(sbits);
    const float b = -0.5f * s;
    const uint32_t d0 = f32_to_dense<DBF16>(__builtin_fmaf(s, 0.0f, b));
    const uint32_t d1 = f32_to_dense<DBF16>(__builtin_fmaf(s, 1.0f, b));
    uint32_t word = 0u, exact = nan ? 0u : 1u;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t hb = (h[i >> 1] >> (16 * (i & 1))) & 0xffffu;
      const bool bit = dense_to_f32<DBF16>(hb) > 0.0f;
      word |= (bit ? 1u : 0u) << i;
      exact &= (hb == (bit ? d1 : d0)) ? 1u : 0u;
    }
    exact = quad_and(exact);
    if (live) {
      packed[t] = word;
      if ((t & 3) == 0) scales[t >> 2] = (uint16_t)sbits;
    }
    bad += (live && (t & 3) == 0 && exact == 0u) ? 1u : 0u;
  }
  block_count(bad, count);
}

// ---------------------------------------------------------------------------
// Read ceiling (measurement aid): one pass over `bytes` bytes with 16-byte
// non-temporal buffer loads, the access the packed kernels make, and nothing
// else.  The XOR of the data is stored only if it equals a sentinel, which
// keeps the loads alive without a store per workgroup.
// ---------------------------------------------------------------------------
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(1024) void q1_read_kernel(const void* data, uint32_t bytes, uint32_t* sink) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(data), (short)0, (int)bytes, (int)0x00020000);
  const uint32_t nvec = bytes >> 4;
  uint32_t acc = 0u;
  for (uint32_t i = blockIdx.x * 1024u + threadIdx.x; i < nvec; i += gridDim.x * 1024u) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, i * 16u, 0, 2);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9E3779B9u) *sink = acc;
}

}  // namespace

hipError_t launch_read(const void* data, size_t bytes, uint32_t* sink, hipStream_t stream) {
  const int64_t blocks = (int64_t)device_cus() * 2;  // two 1024-thread workgroups per CU
  hipLaunchKernelGGL(q1_read_kernel, dim3((unsigned)blocks), dim3(1024), 0, stream, data, (uint32_t)bytes, sink);
  return hipGetLastError();
}

hipError_t launch_symcheck(const uint16_t* scales, const uint16_t* biases, int64_t ngroups, bool meta_bf16,
                           uint32_t* count, hipStream_t stream) {
  hipLaunchKernelGGL(q1_clear_u32, dim3(1), dim3(1), 0, stream, count);
  int64_t blocks = (ngroups + kMetaThreads - 1) / kMetaThreads;
  const int64_t cap = (int64_t)device_cus() / 2;  // metadata is small: few workgroups, few atomics
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  if (meta_bf16)
    hipLaunchKernelGGL((q1_symcheck_kernel<true>), dim3((unsigned)blocks), dim3(kMetaThreads), 0, stream, scales, biases,
                       ngroups, count);
  else
    hipLaunchKernelGGL((q1_symcheck_kernel<false>), dim3((unsigned)blocks), dim3(kMetaThreads), 0, stream, scales, biases,
                       ngroups, count);
  return hipGetLastError();
}

hipError_t launch_pack(const uint16_t* dense, bool dense_bf16, int64_t N, int64_t K, uint32_t* packed,
                       uint16_t* scales, bool meta_bf16, uint32_t* count, hipStream_t stream) {
  hipLaunchKernelGGL(q1_clear_u32, dim3(1), dim3(1), 0, stream, count);
  const int64_t nwords = N * (K / 32);
  int64_t blocks = (nwords + kMetaThreads - 1) / kMetaThreads;
  const int64_t cap = (int64_t)device_cus() * 2;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
#define Q1_PK(D, MB)                                                                                       \
  hipLaunchKernelGGL((q1_pack_kernel<D, MB>), dim3((unsigned)blocks), dim3(kMetaThreads), 0, stream, dense, nwords, \
                     packed, scales, count)
  if (dense_bf16) {
    if (meta_bf16) Q1_PK(true, true);
    else Q1_PK(true, false);
  } else {
    if (meta_bf16) Q1_PK(false, true);
    else Q1_PK(false, false);
  }
#undef Q1_PK
  return hipGetLastError();
}

}  // namespace q1
