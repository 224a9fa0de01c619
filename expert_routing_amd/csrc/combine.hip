// Combine: y[t] = sum_k w[t,k] * yp[dest_row[t,k]] (+ y_sh[t - t0]) with fp32
// accumulation in k order, one rounding to the activation dtype at the end.
// One wave per (token, row segment of 64*CB_CH 16-byte chunks); each lane owns chunks
// of the segment, so small batches still spread over the chip.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int CB_CH = 4;   // 16-byte chunks per lane per pass

__device__ __forceinline__ void unpack(const uint4& v, float* f, bool bf16) {
  if (bf16) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(u[i] << 16);
      f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  } else {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
}

// The token's rows are read in batches of CB_KB: every load of a batch is issued before
// the batch's accumulations, so a wave keeps CB_KB * CB_CH 16-byte loads in flight per lane.
// Dropped pairs (dest_row < 0) load nothing; the sum runs in k order either way.
constexpr int CB_KB = 4;   // rows per batch

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ yp,
                                                      const int32_t* __restrict__ dest_row,
                                                      const float* __restrict__ w,
                                                      const uint4* __restrict__ ysh,
                                                      uint4* __restrict__ y, int T, int K,
                                                      int row_chunks, int64_t t0, int64_t t1) {
  constexpr int EPC = BF16 ? 8 : 4;   // elements per 16-byte chunk
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const bool has_sh = ysh && t >= t0 && t < t1;
  const int base = blockIdx.y * 64 * CB_CH;
  float acc[CB_CH][EPC];
#pragma unroll
  for (int u = 0; u < CB_CH; ++u)
#pragma unroll
    for (int i = 0; i < EPC; ++i) acc[u][i] = 0.f;
  for (int k0 = 0; k0 < K; k0 += CB_KB) {
    int d[CB_KB];
    float wk[CB_KB];
    uint4 v[CB_KB][CB_CH];
#pragma unroll
    for (int j = 0; j < CB_KB; ++j) {
      d[j] = k0 + j < K ? dest_row[t * K + k0 + j] : -1;
      wk[j] = k0 + j < K ? w[t * K + k0 + j] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < CB_KB; ++j) {
      if (d[j] >= 0) {
        const uint4* src = yp + (int64_t)d[j] * row_chunks;
#pragma unroll
        for (int u = 0; u < CB_CH; ++u) {
          const int i = base + u * 64 + lane;
          v[j][u] = i < row_chunks ? src[i] : uint4{0, 0, 0, 0};
        }
      }
    }
#pragma unroll
    for (int j = 0; j < CB_KB; ++j) {
      if (d[j] >= 0) {
#pragma unroll
        for (int u = 0; u < CB_CH; ++u) {
          float f[EPC];
          unpack(v[j][u], f, BF16);
#pragma unroll
          for (int i = 0; i < EPC; ++i) acc[u][i] = fmaf(wk[j], f[i], acc[u][i]);
        }
      }
    }
  }
  if (has_sh) {
    const uint4* src = ysh + (t - t0) * row_chunks;
#pragma unroll
    for (int u = 0; u < CB_CH; ++u) {
      const int i = base + u * 64 + lane;
      if (i < row_chunks) {
        float f[EPC];
        unpack(src[i], f, BF16);
#pragma unroll
        for (int q = 0; q < EPC; ++q) acc[u][q] += f[q];
      }
    }
  }
#pragma unroll
  for (int u = 0; u < CB_CH; ++u) {
    const int i = base + u * 64 + lane;
    if (i >= row_chunks) continue;
    uint4 o;
    if (BF16) {
      uint32_t p[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        p[q] = (uint32_t)f32_to_bf16(acc[u][2 * q]) |
               ((uint32_t)f32_to_bf16(acc[u][2 * q + 1]) << 16);
      o = uint4{p[0], p[1], p[2], p[3]};
    } else {
      o = uint4{__float_as_uint(acc[u][0]), __float_as_uint(acc[u][1]),
                __float_as_uint(acc[u][2]), __float_as_uint(acc[u][3])};
    }
    y[t * row_chunks + i] = o;
  }
}

}  // namespace

int launch_combine(const moe_problem* p, const Dims& d, const void* yp, const int32_t* dest_row,
                   const float* w, const void* y_sh, void* y, hipStream_t st) {
  const int row_chunks = d.h * d.s / 16;
  const int64_t t0 = p->n_shared ? (int64_t)d.rank * d.tpr : 0;
  const int64_t t1 = p->n_shared ? t0 + d.tpr : 0;
  const dim3 grid((unsigned)((d.T + 3) / 4), (unsigned)((row_chunks + 64 * CB_CH - 1) / (64 * CB_CH)));
  if (d.bf16)
    hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, st,
                       static_cast<const uint4*>(yp), dest_row, w,
                       static_cast<const uint4*>(y_sh), static_cast<uint4*>(y), (int)d.T, d.K,
                       row_chunks, t0, t1);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, st,
                       static_cast<const uint4*>(yp), dest_row, w,
                       static_cast<const uint4*>(y_sh), static_cast<uint4*>(y), (int)d.T, d.K,
                       row_chunks, t0, t1);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // namespace moe
