// MX-FP8 quantisation of row-major matrices: each thread takes one block of 32 consecutive
// values of a row, finds its largest magnitude, writes the block's E8M0 scale byte and the
// 32 E4M3 codes of value / 2^X. Used for the expert weights (once, by the caller) and for
// the layer's input x (every call, before the FP8 grouped GEMM).
#include "mxfp8.h"

namespace moe {
namespace {

template <bool BF16>
__global__ __launch_bounds__(256) void mx_quant_rows(const void* __restrict__ src,
                                                     uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales,
                                                     int64_t n_blocks) {
  for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < n_blocks;
       b += (int64_t)gridDim.x * 256) {
    float v[32];
    if (BF16) {
      const uint4* p = static_cast<const uint4*>(src) + b * 4;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 q = p[c];
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[c * 8 + 2 * i] = __uint_as_float(w[i] << 16);
          v[c * 8 + 2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
      }
    } else {
      const float4* p = static_cast<const float4*>(src) + b * 8;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float4 q = p[c];
        v[4 * c] = q.x; v[4 * c + 1] = q.y; v[4 * c + 2] = q.z; v[4 * c + 3] = q.w;
      }
    }
    uint32_t amax = 0;   // magnitudes compared as integers: same order as the values
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = max(amax, mag_bits(v[i]));
    const int x = mx_exponent(amax);
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = mx_pack4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3], x);
    uint4* out = reinterpret_cast<uint4*>(codes + b * 32);
    out[0] = uint4{w[0], w[1], w[2], w[3]};
    out[1] = uint4{w[4], w[5], w[6], w[7]};
    scales[b] = (uint8_t)(x + 127);
  }
}

}  // namespace

int launch_mx_quant(const void* src, bool bf16, int64_t rows, int cols, uint8_t* codes,
                    uint8_t* scales, hipStream_t st) {
  const int64_t n = rows * (cols / 32);
  if (n == 0) return MOE_OK;
  const int64_t want = (n + 255) / 256;
  const unsigned grid = (unsigned)(want < 8192 ? want : 8192);
  if (bf16)
    hipLaunchKernelGGL(mx_quant_rows<true>, dim3(grid), dim3(256), 0, st, src, codes, scales, n);
  else
    hipLaunchKernelGGL(mx_quant_rows<false>, dim3(grid), dim3(256), 0, st, src, codes, scales, n);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // namespace moe
