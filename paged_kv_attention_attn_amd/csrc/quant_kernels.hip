// Quantized cache encoding for gfx950: bf16 token vectors -> 8-bit (Q8) or
// 4-bit (Q4) codes with one fp32 scale per vector.
//
// Source: ExLlamaV2 "Dynamic Generator" page, section "Usage" (preparing the
// model and the generator): a quantized cache mode replaces the plain one; an
// 8-bit mode is announced as about as compact as an FP8 cache but more
// accurate. The page gives no format; this library's: per vector of D values
// (one token, one KV head), scale = max|x| / 127 and code = x / scale rounded
// to nearest, ties to even, in IEEE binary32; a zero vector has scale 0, a
// vector with a non-finite value scale NaN, both with codes 0. Decoding (in the
// attention kernels) is bf16(code * scale).
//
// Q4 is the same scheme at 4 bits: scale = max|x| / 7, codes in [-7, 7],
// stored as the nibble code + 8, two per byte (dim 2i in the low nibble of
// byte i).
//
// One wave per vector: each lane holds D / 64 values (Q4: a pair of adjacent
// values, one output byte), the largest magnitude and the all-finite test are
// wave reductions.

#include "internal.h"

#include "pkv.h"

namespace pkv {
namespace {

constexpr int kEncThreads = 256;
constexpr int kEncWaves = kEncThreads / 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <int D>
__global__ __launch_bounds__(kEncThreads) void q8_encode_kernel(const uint16_t* __restrict__ src,
                                                                int8_t* __restrict__ codes,
                                                                float* __restrict__ scales, long rows) {
  constexpr int EPL = D / 64;  // values per lane
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * kEncWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint16_t* x = src + row * D + lane * EPL;
  float v[EPL];
  float amax = 0.f;
  bool finite = true;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    v[e] = bf16_to_f32(x[e]);
    finite &= __builtin_isfinite(v[e]);
    amax = fmaxf(amax, __builtin_isfinite(v[e]) ? fabsf(v[e]) : 0.f);
  }
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  const bool all_finite = __builtin_amdgcn_ballot_w64(!finite) == 0;
  const float scale = amax / 127.f;  // IEEE division, rounded to nearest
  int8_t* c = codes + row * D + lane * EPL;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    int q = 0;
    if (all_finite && scale > 0.f) {
      const float t = __builtin_rintf(v[e] / scale);
      q = (int)fminf(fmaxf(t, -127.f), 127.f);
    }
    c[e] = (int8_t)q;
  }
  if (lane == 0) scales[row] = all_finite ? scale : __builtin_nanf("");
}

// Q4: lane l holds dims 2l and 2l + 1 (lanes past D / 2 hold nothing) and
// writes byte l of the vector's codes.
template <int D>
__global__ __launch_bounds__(kEncThreads) void q4_encode_kernel(const uint16_t* __restrict__ src,
                                                                uint8_t* __restrict__ codes,
                                                                float* __restrict__ scales, long rows) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * kEncWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  const bool active = lane < D / 2;
  float v[2] = {0.f, 0.f};
  if (active) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(src + row * D + 2 * lane);
    v[0] = bf16_to_f32((uint16_t)(w & 0xFFFFu));
    v[1] = bf16_to_f32((uint16_t)(w >> 16));
  }
  bool finite = true;
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    finite &= __builtin_isfinite(v[e]);
    amax = fmaxf(amax, __builtin_isfinite(v[e]) ? fabsf(v[e]) : 0.f);
  }
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  const bool all_finite = __builtin_amdgcn_ballot_w64(!finite) == 0;
  const float scale = amax / 7.f;  // IEEE division, rounded to nearest
  uint32_t nib[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    int q = 0;
    if (all_finite && scale > 0.f) q = (int)fminf(fmaxf(__builtin_rintf(v[e] / scale), -7.f), 7.f);
    nib[e] = (uint32_t)(q + 8);
  }
  if (active) codes[row * (D / 2) + lane] = (uint8_t)(nib[0] | (nib[1] << 4));
  if (lane == 0) scales[row] = all_finite ? scale : __builtin_nanf("");
}

}  // namespace

hipError_t launch_q4_encode(const uint16_t* src, uint8_t* codes, float* scales, long rows, int D,
                            hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const long blocks = (rows + kEncWaves - 1) / kEncWaves;
  if (D == 64)
    hipLaunchKernelGGL(q4_encode_kernel<64>, dim3((unsigned)blocks), dim3(kEncThreads), 0, stream, src, codes,
                       scales, rows);
  else
    hipLaunchKernelGGL(q4_encode_kernel<128>, dim3((unsigned)blocks), dim3(kEncThreads), 0, stream, src, codes,
                       scales, rows);
  return hipGetLastError();
}

hipError_t launch_q8_encode(const uint16_t* src, int8_t* codes, float* scales, long rows, int D,
                            hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const long blocks = (rows + kEncWaves - 1) / kEncWaves;
  if (D == 64)
    hipLaunchKernelGGL(q8_encode_kernel<64>, dim3((unsigned)blocks), dim3(kEncThreads), 0, stream, src, codes,
                       scales, rows);
  else
    hipLaunchKernelGGL(q8_encode_kernel<128>, dim3((unsigned)blocks), dim3(kEncThreads), 0, stream, src, codes,
                       scales, rows);
  return hipGetLastError();
}

}  // namespace pkv
