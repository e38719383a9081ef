// Activation split for the fp8 x fp4 matrix-core kernels (gfx950).
//
// One packed word carries 32 weights (bit t = weight t, least significant
// bit first; rMLX issue #207 "Q1 layout"), and its 32 activations become the
// A operand bytes that meet those bits in v_mfma_scale_f32_16x16x128_f8f6f4.
// The B side expands bit class j (bits 4i+j) with one AND to fp4 codes
// 0.5, 1, 2, 2 (class 3 moved to bit position 2), so the activations of class
// j are multiplied by 1/code(j) = 2, 1, 1/2, 1/2 (powers of two: exact) and
// every product is bit * x.  Each value is split into fp8 (E4M3) pieces,
// x = hi + lo/16, with one power-of-two scale for the word's 32 values:
// sc = frexp(max |x|) - 7, so |x| * 2^-sc < 2^7 and at most 2^8 after the
// class factor, below fp8's largest value (448).  hi carries the top 4 of a
// bf16's 8 significant bits (rounded), lo the rest, so the pair is exact for
// every value within a factor 2^11 of the word's largest magnitude (lo then
// stays on fp8's grid); below that the error is at most 2^-19 of it.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace q1 {

typedef short q1_v2s __attribute__((ext_vector_type(2)));
typedef float q1_v2f __attribute__((ext_vector_type(2)));
typedef __bf16 q1_v2bf __attribute__((ext_vector_type(2)));

// A register whose contents do not matter (the scaled conversions overwrite
// half of their destination and keep the other half; the first conversion
// of each dword needs no old value).  The empty asm statement hands over
// whatever the register holds instead of materialising a zero.
__device__ __forceinline__ q1_v2s q1_undef_v2s() {
  q1_v2s r;
  asm volatile("" : "=v"(r));
  return r;
}

// wd: the word's 32 bf16 activations as 16 dwords (dword d = values 2d, 2d+1).
// Out: hi[j][hh], lo[j][hh] = the 4 bytes of class j, half word hh (value
// 16*hh + 4*i + j in byte i), the scale exponent sc (E8M0 bytes sc + 127 for
// hi, sc + 123 for lo), and the plain sum of the 32 values.
__device__ __forceinline__ void q1_convert_word(const uint32_t (&wd)[16], uint32_t (&hi)[4][2], uint32_t (&lo)[4][2],
                                                int& sc, float& xsum) {
  const q1_v2bf ones = __builtin_bit_cast(q1_v2bf, 0x3F803F80u);
  float xv[32];
  float X = 0.0f;
#pragma unroll
  for (int d = 0; d < 16; ++d) {
    // (the sum is taken on the dword already in hand: extracting it again
    // from a vector for the bf16 dot has compiled to the wrong element)
    xv[2 * d] = __uint_as_float(wd[d] << 16);
    xv[2 * d + 1] = __uint_as_float(wd[d] & 0xffff0000u);
    X = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(q1_v2bf, wd[d]), ones, X, false);
  }
  float amax = 0.0f;
#pragma unroll
  for (int t = 0; t < 32; ++t) amax = fmaxf(amax, fabsf(xv[t]));
  // the clamp keeps every divisor a normal fp32 power of two (bf16 data never
  // reaches it at the top)
  int s = amax > 0.0f ? __builtin_amdgcn_frexp_expf(amax) - 7 : 0;
  s = s < -118 ? -118 : (s > 125 ? 125 : s);
  // The scaled conversions divide by (and the decode multiplies by) a power
  // of two: 2^sc / factor(j) for hi, 16 times less for lo.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = s - (j == 0 ? 1 : (j == 1 ? 0 : -1));  // 2^e = 2^sc / factor(j)
    const float dh = __uint_as_float((uint32_t)(e + 127) << 23);
    const float dl = __uint_as_float((uint32_t)(e + 123) << 23);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const float* v = xv + 16 * hh + j;  // v[0], v[4], v[8], v[12]
      q1_v2s h = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(q1_undef_v2s(), v[0], v[4], dh, false);
      h = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(h, v[8], v[12], dh, true);
      const uint32_t hb = __builtin_bit_cast(uint32_t, h);
      const q1_v2f d01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hb, dh, false);
      const q1_v2f d23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hb, dh, true);
      q1_v2s l = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(q1_undef_v2s(), v[0] - d01[0], v[4] - d01[1], dl, false);
      l = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(l, v[8] - d23[0], v[12] - d23[1], dl, true);
      hi[j][hh] = hb;
      lo[j][hh] = __builtin_bit_cast(uint32_t, l);
    }
  }
  sc = s;
  xsum = X;
}

// Exponent e of a block scale 2^e for E5M2 pieces: the block's largest
// class-scaled magnitude a lands in [2^14, 2^15) after division by 2^e (the
// top binade of E5M2, largest finite value 57344), so rounding never
// overflows.  Clamped so that 2^e / factor stays a normal fp32 number.
__device__ __forceinline__ int q1_bf8_block_exp(float a) {
  int e = a > 0.0f ? __builtin_amdgcn_frexp_expf(a) - 15 : -125;
  return e < -125 ? -125 : (e > 125 ? 125 : e);
}

// Three-piece split of a word's 32 activations into E5M2 (bf8) bytes for
// affine tensors: x = P0 + P1 + P2, each piece with its own power-of-two
// block scale 2^sc[p] chosen from the largest magnitude of what the earlier
// pieces left.  E5M2 spans 30 binades, so each piece keeps 3 significant bits
// of every value within ~2^28 of its block maximum; together the pieces give
// back all 8 bits of every bf16 value within 2^25 of the word's largest
// (class-scaled) magnitude, and smaller values to within 2^-35 of that
// magnitude (measured on a CPU model of the conversion: exact through
// 2^-26, 2^-38 absolute below).  Layout of p[piece][j][hh] as hi[j][hh] of
// q1_convert_word; class factors as there.  xsum: the plain sum of the 32
// values.
__device__ __forceinline__ void q1_convert_word_bf8(const uint32_t (&wd)[16], uint32_t (&pc)[3][4][2], int (&sc)[3],
                                                    float& xsum) {
  const q1_v2bf ones = __builtin_bit_cast(q1_v2bf, 0x3F803F80u);
  float r[32];
  float X = 0.0f;
#pragma unroll
  for (int d = 0; d < 16; ++d) {
    r[2 * d] = __uint_as_float(wd[d] << 16);
    r[2 * d + 1] = __uint_as_float(wd[d] & 0xffff0000u);
    X = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(q1_v2bf, wd[d]), ones, X, false);
  }
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    // largest class-scaled magnitude: value t is in class t % 4, factor 2, 1, 1/2, 1/2
    float cm[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < 32; ++t) cm[t & 3] = fmaxf(cm[t & 3], fabsf(r[t]));
    const float a = fmaxf(fmaxf(2.0f * cm[0], cm[1]), 0.5f * fmaxf(cm[2], cm[3]));
    const int s = q1_bf8_block_exp(a);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = s - (j == 0 ? 1 : (j == 1 ? 0 : -1));  // 2^e = 2^s / factor(j)
      const float dv = __uint_as_float((uint32_t)(e + 127) << 23);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float* v = r + 16 * hh + j;  // v[0], v[4], v[8], v[12]
        q1_v2s b = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(q1_undef_v2s(), v[0], v[4], dv, false);
        b = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(b, v[8], v[12], dv, true);
        const uint32_t bb = __builtin_bit_cast(uint32_t, b);
        pc[p][j][hh] = bb;
        if (p < 2) {  // what this piece leaves for the next (exact in fp32)
          const q1_v2f d01 = __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(bb, dv, false);
          const q1_v2f d23 = __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(bb, dv, true);
          v[0] -= d01[0];
          v[4] -= d01[1];
          v[8] -= d23[0];
          v[12] -= d23[1];
        }
      }
    }
    sc[p] = s;
  }
  xsum = X;
}

// fp4 (E2M1) B operand of one group for one lane: the lane's packed word,
// one AND per bit class (class 3 moved to bit position 2).
__device__ __forceinline__ void q1_expand_b(uint32_t wd, int (&B)[8]) {
  B[0] = (int)(wd & 0x11111111u);
  B[1] = (int)(wd & 0x22222222u);
  B[2] = (int)(wd & 0x44444444u);
  B[3] = (int)((wd >> 1) & 0x44444444u);
  B[4] = B[5] = B[6] = B[7] = 0;
}

}  // namespace q1
