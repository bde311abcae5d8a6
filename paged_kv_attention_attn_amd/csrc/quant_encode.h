// Device-side encoding of one bf16 vector (one token of one KV head) into the
// quantized cache formats, by one wave. Used by the encoder kernels and by
// the quantized cache append.
//
// Q8: scale = max|x| / 127, code = x / scale rounded to nearest even, codes in
// [-127, 127], all IEEE binary32; a zero vector has scale 0, a vector holding
// a non-finite value scale NaN, both with codes 0.
// Q4: the same at 4 bits (max|x| / 7, codes in [-7, 7]) stored as the nibble
// code + 8, two per byte, dim 2i in the low nibble of byte i.
// Source: the ExLlamaV2 "Dynamic Generator" page, "Usage", names the Q4 and
// Q8 cache modes without giving a format; the formats are this library's.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

__device__ __forceinline__ float enc_bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// The wave's largest finite magnitude and whether every value is finite.
__device__ __forceinline__ void enc_wave_stats(float amax, bool finite, float& wave_amax, bool& all_finite) {
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  wave_amax = amax;
  all_finite = __builtin_amdgcn_ballot_w64(!finite) == 0;
}

// Q8: lane l holds values l * D/64 .. + D/64 - 1 and writes their codes.
template <int D>
__device__ __forceinline__ void q8_encode_wave(const uint16_t* __restrict__ x, int8_t* __restrict__ codes,
                                               float* __restrict__ scale_out) {
  constexpr int EPL = D / 64;
  const int lane = threadIdx.x & 63;
  float v[EPL];
  float amax = 0.f;
  bool finite = true;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    v[e] = enc_bf16_to_f32(x[lane * EPL + e]);
    finite &= __builtin_isfinite(v[e]);
    amax = fmaxf(amax, __builtin_isfinite(v[e]) ? fabsf(v[e]) : 0.f);
  }
  bool all_finite;
  enc_wave_stats(amax, finite, amax, all_finite);
  const float scale = amax / 127.f;  // IEEE division, rounded to nearest
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    int q = 0;
    if (all_finite && scale > 0.f) q = (int)fminf(fmaxf(__builtin_rintf(v[e] / scale), -127.f), 127.f);
    codes[lane * EPL + e] = (int8_t)q;
  }
  if (lane == 0) *scale_out = all_finite ? scale : __builtin_nanf("");
}

// Q4: lane l holds dims 2l and 2l + 1 (lanes past D / 2 hold nothing) and
// writes byte l of the codes.
template <int D>
__device__ __forceinline__ void q4_encode_wave(const uint16_t* __restrict__ x, uint8_t* __restrict__ codes,
                                               float* __restrict__ scale_out) {
  const int lane = threadIdx.x & 63;
  const bool active = lane < D / 2;
  float v[2] = {0.f, 0.f};
  if (active) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(x + 2 * lane);
    v[0] = enc_bf16_to_f32((uint16_t)(w & 0xFFFFu));
    v[1] = enc_bf16_to_f32((uint16_t)(w >> 16));
  }
  bool finite = true;
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    finite &= __builtin_isfinite(v[e]);
    amax = fmaxf(amax, __builtin_isfinite(v[e]) ? fabsf(v[e]) : 0.f);
  }
  bool all_finite;
  enc_wave_stats(amax, finite, amax, all_finite);
  const float scale = amax / 7.f;  // IEEE division, rounded to nearest
  uint32_t nib[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    int q = 0;
    if (all_finite && scale > 0.f) q = (int)fminf(fmaxf(__builtin_rintf(v[e] / scale), -7.f), 7.f);
    nib[e] = (uint32_t)(q + 8);
  }
  if (active) codes[lane] = (uint8_t)(nib[0] | (nib[1] << 4));
  if (lane == 0) *scale_out = all_finite ? scale : __builtin_nanf("");
}

}  // namespace pkv
