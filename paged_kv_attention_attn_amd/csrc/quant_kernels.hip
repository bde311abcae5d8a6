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
// wave reductions. The grid is capped at kEncMaxBlocks workgroups, each
// striding over the rows, so any row count the ABI accepts fits one launch.

#include "internal.h"

#include <algorithm>

#include "pkv.h"
#include "quant_encode.h"

namespace pkv {
namespace {

constexpr int kEncThreads = 256;
constexpr int kEncWaves = kEncThreads / 64;
constexpr long kEncMaxBlocks = 1L << 16;  // 64 Ki workgroups: 256 per CU, far past what fills the chip

template <int D>
__global__ __launch_bounds__(kEncThreads) void q8_encode_kernel(const uint16_t* __restrict__ src,
                                                                int8_t* __restrict__ codes,
                                                                float* __restrict__ scales, long rows) {
  for (long row = (long)blockIdx.x * kEncWaves + (threadIdx.x >> 6); row < rows; row += (long)gridDim.x * kEncWaves)
    q8_encode_wave<D>(src + row * D, codes + row * D, scales + row);
}

template <int D>
__global__ __launch_bounds__(kEncThreads) void q4_encode_kernel(const uint16_t* __restrict__ src,
                                                                uint8_t* __restrict__ codes,
                                                                float* __restrict__ scales, long rows) {
  for (long row = (long)blockIdx.x * kEncWaves + (threadIdx.x >> 6); row < rows; row += (long)gridDim.x * kEncWaves)
    q4_encode_wave<D>(src + row * D, codes + row * (D / 2), scales + row);
}

}  // namespace

hipError_t launch_q4_encode(const uint16_t* src, uint8_t* codes, float* scales, long rows, int D,
                            hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const long blocks = std::min((rows + kEncWaves - 1) / kEncWaves, kEncMaxBlocks);
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
  const long blocks = std::min((rows + kEncWaves - 1) / kEncWaves, kEncMaxBlocks);
  if (D == 64)
    hipLaunchKernelGGL(q8_encode_kernel<64>, dim3((unsigned)blocks), dim3(kEncThreads), 0, stream, src, codes,
                       scales, rows);
  else
    hipLaunchKernelGGL(q8_encode_kernel<128>, dim3((unsigned)blocks), dim3(kEncThreads), 0, stream, src, codes,
                       scales, rows);
  return hipGetLastError();
}

}  // namespace pkv
