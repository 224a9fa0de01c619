// Router: logits = x . W_r^T in fp32, then per-token scoring, group limit, top-K and
// weights.
//
// bf16 activations: the GEMM runs on bf16 MFMA. Each fp32 router weight w is split
// exactly into three bf16 parts, w = hi + mid + lo (truncation leaves 16, then 8
// significant bits, so every remainder is representable), and x*hi + x*mid + x*lo are
// summed into fp32 accumulators. Every product of bf16 operands is exact in fp32, so
// this is an fp32 GEMM with exact operands and fp32 accumulation, at bf16 MFMA rate.
// fp32 activations take a plain VALU GEMM. The reduction is split along h into k-slices
// (enough blocks for the chip) whose partial logits are added in slice order before, or
// while, selecting.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int RT_BM = 64;   // tokens per block
constexpr int RT_BK = 64;   // k per stage

// LDS index (in 16-byte chunks) of chunk c of row r for a [rows][64 bf16] tile with an
// XOR swizzle that keeps 8 consecutive rows on distinct bank groups.
__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ (r & 7)); }

__device__ __forceinline__ void split3(float w, bf16_t& hi, bf16_t& mid, bf16_t& lo) {
  uint32_t u = __float_as_uint(w);
  uint32_t uh = u & 0xffff0000u;
  float r1 = w - __uint_as_float(uh);
  uint32_t u1 = __float_as_uint(r1) & 0xffff0000u;
  float r2 = r1 - __uint_as_float(u1);
  uint32_t u2 = __float_as_uint(r2);
  hi = static_cast<bf16_t>(uh >> 16);
  mid = static_cast<bf16_t>(u1 >> 16);
  lo = static_cast<bf16_t>(u2 >> 16);
}

// One block: 64 tokens x BE experts (BE in {16, 32, 64}); 4 waves; MFMA 16x16x32.
template <int BE>
__global__ __launch_bounds__(256) void router_gemm_bf16(const bf16_t* __restrict__ x,
                                                        const float* __restrict__ w,
                                                        float* __restrict__ logits,
                                                        int T, int h, int E, int kslice) {
  __shared__ uint4 xs[RT_BM * 8];           // [64 rows][8 chunks]
  __shared__ uint4 wsm[3][BE * 8];          // hi / mid / lo planes, [BE rows][8 chunks]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * RT_BM, ebase = blockIdx.y * BE;
  constexpr int NEG = BE / 16;              // expert groups of 16 in the tile
  const int eg = wave % NEG;
  const int tg0 = (wave / NEG) * NEG;       // this wave's NEG token groups
  floatx4 acc[NEG];
#pragma unroll
  for (int i = 0; i < NEG; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  // K-slice blockIdx.z of the reduction; its partial logits go to slab z
  const int kb = blockIdx.z * kslice, ke = kb + kslice < h ? kb + kslice : h;
  logits += (size_t)blockIdx.z * T * E;

  // Global loads of the next k-step go to registers while the MFMAs run on the current
  // one, so a block always has one stage in flight.
  constexpr int WPT = BE * 16 / 256;         // float4 of W per thread per k-step
  uint4 xr[2];
  float4 wr[WPT];
  auto load = [&](int k0) __attribute__((always_inline)) {
    // x tile: 64 rows x 8 chunks = 512 chunks, 2 per thread
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int id = tid + i * 256, r = id >> 3, c = id & 7;
      const int t = t0 + r < T ? t0 + r : T - 1;
      xr[i] = *reinterpret_cast<const uint4*>(x + (size_t)t * h + k0 + c * 8);
    }
    // w tile: BE rows x 64 fp32 = BE*16 float4
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int id = tid + i * 256, r = id >> 4, q = id & 15;
      const int e = ebase + r;
      wr[i] = e < E ? *reinterpret_cast<const float4*>(w + (size_t)e * h + k0 + q * 4)
                    : float4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto store = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int id = tid + i * 256, r = id >> 3, c = id & 7;
      xs[swz(r, c)] = xr[i];
    }
    // W split into 3 bf16 planes; 4 bf16 = half a 16-byte chunk
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int id = tid + i * 256, r = id >> 4, q = id & 15;
      const float4 v = wr[i];
      bf16_t h0, m0, l0, h1, m1, l1, h2, m2, l2, h3, m3, l3;
      split3(v.x, h0, m0, l0); split3(v.y, h1, m1, l1);
      split3(v.z, h2, m2, l2); split3(v.w, h3, m3, l3);
      const int chunk = swz(r, q >> 1), half = q & 1;
      uint2* p0 = reinterpret_cast<uint2*>(&wsm[0][chunk]) + half;
      uint2* p1 = reinterpret_cast<uint2*>(&wsm[1][chunk]) + half;
      uint2* p2 = reinterpret_cast<uint2*>(&wsm[2][chunk]) + half;
      *p0 = uint2{(uint32_t)h0 | ((uint32_t)h1 << 16), (uint32_t)h2 | ((uint32_t)h3 << 16)};
      *p1 = uint2{(uint32_t)m0 | ((uint32_t)m1 << 16), (uint32_t)m2 | ((uint32_t)m3 << 16)};
      *p2 = uint2{(uint32_t)l0 | ((uint32_t)l1 << 16), (uint32_t)l2 | ((uint32_t)l3 << 16)};
    }
  };

  if (kb < ke) load(kb);
  for (int k0 = kb; k0 < ke; k0 += RT_BK) {
    store();
    __syncthreads();
    if (k0 + RT_BK < ke) load(k0 + RT_BK);
#pragma unroll
    for (int s = 0; s < 2; ++s) {            // two k32 steps
      const int c = s * 4 + (lane >> 4);
      const int er = eg * 16 + (lane & 15);
      bf16x8_t b0 = __builtin_bit_cast(bf16x8_t, wsm[0][swz(er, c)]);
      bf16x8_t b1 = __builtin_bit_cast(bf16x8_t, wsm[1][swz(er, c)]);
      bf16x8_t b2 = __builtin_bit_cast(bf16x8_t, wsm[2][swz(er, c)]);
#pragma unroll
      for (int i = 0; i < NEG; ++i) {
        const int tr = (tg0 + i) * 16 + (lane & 15);
        bf16x8_t a = __builtin_bit_cast(bf16x8_t, xs[swz(tr, c)]);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b2, acc[i], 0, 0, 0);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b1, acc[i], 0, 0, 0);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b0, acc[i], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // acc[i][j]: token row (lane>>4)*4 + j of token group tg0+i, expert column lane&15
  const int e = ebase + eg * 16 + (lane & 15);
#pragma unroll
  for (int i = 0; i < NEG; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int t = t0 + (tg0 + i) * 16 + (lane >> 4) * 4 + j;
      if (t < T && e < E) logits[(size_t)t * E + e] = acc[i][j];
    }
  }
}

// fp32 activations: 64 tokens x 64 experts per block, 4x4 outputs per thread.
__global__ __launch_bounds__(256) void router_gemm_f32(const float* __restrict__ x,
                                                       const float* __restrict__ w,
                                                       float* __restrict__ logits,
                                                       int T, int h, int E, int kslice) {
  constexpr int BK = 16;
  __shared__ float xs[BK][64 + 4];
  __shared__ float wsm[BK][64 + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  float acc[4][4] = {};
  const int kb = blockIdx.z * kslice, ke = kb + kslice < h ? kb + kslice : h;
  logits += (size_t)blockIdx.z * T * E;
  for (int k0 = kb; k0 < ke; k0 += BK) {
    for (int id = tid; id < 64 * BK; id += 256) {
      int r = id / BK, k = id % BK;
      int t = t0 + r, e = e0 + r, kk = k0 + k;
      xs[k][r] = (t < T && kk < ke) ? x[(size_t)t * h + kk] : 0.f;
      wsm[k][r] = (e < E && kk < ke) ? w[(size_t)e * h + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = xs[k][ty * 4 + i]; b[i] = wsm[k][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int t = t0 + ty * 4 + i, e = e0 + tx * 4 + j;
      if (t < T && e < E) logits[(size_t)t * E + e] = acc[i][j];
    }
}

// (key, index) order: larger key first, lower index on ties.
__device__ __forceinline__ bool better(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

constexpr int SEL_KPL = 8;     // keys per lane: E <= 512
constexpr int SEL_TOK = 4;     // tokens (waves) per block

// One wave per token. Lane l holds experts l, l+64, ...
__global__ __launch_bounds__(256) void select_topk(const float* __restrict__ logits,
                                                   const float* __restrict__ bias,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ wout, int T, int E,
                                                   int K, int score, int renorm, int n_groups,
                                                   int topk_groups, int nsplit) {
  __shared__ float keys_s[SEL_TOK][512];
  __shared__ float gscore_s[SEL_TOK][512];
  __shared__ int gallow_s[SEL_TOK][512];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * SEL_TOK + wave;
  const bool active = t < T;
  const int kpl = (E + 63) >> 6;
  float L[SEL_KPL], key[SEL_KPL], raw[SEL_KPL];
#pragma unroll
  for (int j = 0; j < SEL_KPL; ++j) {
    const int e = j * 64 + lane;
    float l = -INFINITY, k = -INFINITY, r = 0.f;
    if (active && j < kpl && e < E) {
      l = logits[t * E + e];
      // partial logits added in slice order; loads in groups of 8 so they overlap
      for (int z0 = 1; z0 < nsplit; z0 += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          v[u] = z0 + u < nsplit ? logits[(size_t)(z0 + u) * T * E + t * E + e] : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (z0 + u < nsplit) l += v[u];
      }
      const float b = bias ? bias[e] : 0.f;
      if (score == MOE_SCORE_SOFTMAX) {
        l += b;
        k = l;
      } else {
        r = 1.f / (1.f + __expf(-l));
        k = r + b;
      }
    }
    L[j] = l; key[j] = k; raw[j] = r;
  }
  const bool glimit = n_groups > 1 && topk_groups < n_groups;
  if (glimit) {   // uniform across the block: every wave takes the same barriers
    const int gsz = E / n_groups;
#pragma unroll
    for (int j = 0; j < SEL_KPL; ++j) {
      const int e = j * 64 + lane;
      if (j < kpl && e < E) keys_s[wave][e] = key[j];
    }
    __syncthreads();
    for (int g = lane; g < n_groups; g += 64) {
      float b1 = -INFINITY, b2 = -INFINITY;
      for (int i = 0; i < gsz; ++i) {
        const float v = keys_s[wave][g * gsz + i];
        if (v > b1) { b2 = b1; b1 = v; } else if (v > b2) { b2 = v; }
      }
      gscore_s[wave][g] = gsz > 1 ? b1 + b2 : b1;
    }
    __syncthreads();
    for (int g = lane; g < n_groups; g += 64) {
      const float sg = gscore_s[wave][g];
      int rank = 0;
      for (int q = 0; q < n_groups; ++q) {
        const float sq = gscore_s[wave][q];
        rank += (sq > sg || (sq == sg && q < g)) ? 1 : 0;
      }
      gallow_s[wave][g] = rank < topk_groups;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < SEL_KPL; ++j) {
      const int e = j * 64 + lane;
      if (j < kpl && e < E && !gallow_s[wave][e / gsz]) key[j] = -INFINITY;
    }
  }
  if (!active) return;

  // K rounds of a wave-wide arg-max over the remaining allowed experts.
  uint32_t taken = 0;
  int win_e = -1;        // lane k < K keeps the k-th winner
  float win_L = 0.f, win_r = 0.f;
  for (int k = 0; k < K; ++k) {
    float bk = -INFINITY; int bi = 0x7fffffff; float bl = 0.f, br = 0.f;
#pragma unroll
    for (int j = 0; j < SEL_KPL; ++j) {
      const int e = j * 64 + lane;
      if (j < kpl && e < E && !(taken >> j & 1u) && key[j] != -INFINITY &&
          better(key[j], e, bk, bi)) {
        bk = key[j]; bi = e; bl = L[j]; br = raw[j];
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ok = __shfl_xor(bk, off);
      const int oi = __shfl_xor(bi, off);
      const float ol = __shfl_xor(bl, off);
      const float orr = __shfl_xor(br, off);
      if (better(ok, oi, bk, bi)) { bk = ok; bi = oi; bl = ol; br = orr; }
    }
    if (bi < E && (bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == k) { win_e = bi; win_L = bl; win_r = br; }
  }
  // Weights of the K winners (lanes 0..K-1).
  float wv = 0.f;
  if (score == MOE_SCORE_SOFTMAX) {
    if (renorm) {
      const float m = __shfl(win_L, 0);      // first winner has the largest logit
      const float ex = lane < K ? __expf(win_L - m) : 0.f;
      float z = ex;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off);
      wv = ex / z;
    } else {
      float m = -INFINITY;
#pragma unroll
      for (int j = 0; j < SEL_KPL; ++j) m = fmaxf(m, L[j]);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
      float z = 0.f;
#pragma unroll
      for (int j = 0; j < SEL_KPL; ++j) {
        const int e = j * 64 + lane;
        if (j < kpl && e < E) z += __expf(L[j] - m);
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off);
      wv = __expf(win_L - m) / z;
    }
  } else {
    if (renorm) {
      float z = lane < K ? win_r : 0.f;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off);
      wv = win_r / z;
    } else {
      wv = win_r;
    }
  }
  // Ascending-id order: position = number of winners with a smaller id.
  int pos = 0;
  for (int q = 0; q < K; ++q) {
    const int oe = __shfl(win_e, q);
    pos += (oe < win_e) ? 1 : 0;
  }
  if (lane < K) {
    ids[t * K + pos] = win_e;
    wout[t * K + pos] = wv;
  }
}

// Partial logits of the k-slices added in slice order into slab 0, one thread per
// logit (the same additions, in the same order, as select_topk's own summation).
__global__ __launch_bounds__(256) void logits_reduce(float* __restrict__ logits, int64_t n,
                                                     int nsplit) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * 256) {
    float v[32];
    const int m = nsplit < 32 ? nsplit : 32;
#pragma unroll
    for (int z = 0; z < 32; ++z)
      if (z < m) v[z] = logits[(size_t)z * n + i];
    float l = v[0];
#pragma unroll
    for (int z = 1; z < 32; ++z)
      if (z < m) l += v[z];
    for (int z = 32; z < nsplit; ++z) l += logits[(size_t)z * n + i];
    logits[i] = l;
  }
}

}  // namespace

// K-slices of the router GEMM: enough blocks for about four per CU (each keeps one
// k-step of loads in flight, so four hide most of the memory latency), slices of at
// least 256 along h (a multiple of the 64-wide k-step).
int route_split(const Dims& d) {
  const int64_t tiles = ((d.T + RT_BM - 1) / RT_BM) *
                        ((d.E + 63) / 64 > 0 ? (d.E + 63) / 64 : 1);
  int s = tiles > 0 ? (int)((1024 + tiles - 1) / tiles) : 1;
  const int smax = d.h / 256 > 1 ? d.h / 256 : 1;
  s = s < 1 ? 1 : (s > smax ? smax : s);
  return s;
}

static int select_with(const moe_problem* p, const Dims& d, const float* logits, int nsplit,
                       const float* bias, int32_t* ids, float* w, hipStream_t st) {
  const unsigned grid = (unsigned)((d.T + SEL_TOK - 1) / SEL_TOK);
  hipLaunchKernelGGL(select_topk, dim3(grid), dim3(256), 0, st, logits, bias, ids, w,
                     (int)d.T, d.E, d.K, p->score, p->renorm, p->n_groups, p->topk_groups,
                     nsplit);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

int launch_select(const moe_problem* p, const Dims& d, const float* logits, const float* bias,
                  int32_t* ids, float* w, hipStream_t st) {
  return select_with(p, d, logits, 1, bias, ids, w, st);
}

int launch_route(const moe_problem* p, const Dims& d, const void* x, const float* w_router,
                 const float* bias, int32_t* ids, float* w, float* logits, hipStream_t st) {
  const unsigned gt = (unsigned)((d.T + RT_BM - 1) / RT_BM);
  const int S = d.route_split;
  // k-slice length: a multiple of 64 covering h in S slices
  const int kslice = ((d.h + S - 1) / S + 63) / 64 * 64;
  const unsigned gz = (unsigned)((d.h + kslice - 1) / kslice);
  if (d.bf16) {
    const int be = d.E <= 16 ? 16 : (d.E <= 32 ? 32 : 64);
    const dim3 grid(gt, (unsigned)((d.E + be - 1) / be), gz);
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    if (be == 16)
      hipLaunchKernelGGL(router_gemm_bf16<16>, grid, dim3(256), 0, st, xb, w_router, logits,
                         (int)d.T, d.h, d.E, kslice);
    else if (be == 32)
      hipLaunchKernelGGL(router_gemm_bf16<32>, grid, dim3(256), 0, st, xb, w_router, logits,
                         (int)d.T, d.h, d.E, kslice);
    else
      hipLaunchKernelGGL(router_gemm_bf16<64>, grid, dim3(256), 0, st, xb, w_router, logits,
                         (int)d.T, d.h, d.E, kslice);
  } else {
    const dim3 grid(gt, (unsigned)((d.E + 63) / 64), gz);
    hipLaunchKernelGGL(router_gemm_f32, grid, dim3(256), 0, st, static_cast<const float*>(x),
                       w_router, logits, (int)d.T, d.h, d.E, kslice);
  }
  if (hipGetLastError() != hipSuccess) return MOE_ERR_LAUNCH;
  if (gz >= 8 && d.T <= 1024) {
    // small batch, many slabs: select would run too few waves to add them quickly; add
    // them with one thread per logit, then select reads one
    const int64_t n = d.T * d.E;
    const unsigned blocks = (unsigned)((n + 255) / 256 < 2048 ? (n + 255) / 256 : 2048);
    hipLaunchKernelGGL(logits_reduce, dim3(blocks), dim3(256), 0, st, logits, n, (int)gz);
    if (hipGetLastError() != hipSuccess) return MOE_ERR_LAUNCH;
    return select_with(p, d, logits, 1, bias, ids, w, st);
  }
  return select_with(p, d, logits, (int)gz, bias, ids, w, st);
}

}  // namespace moe
