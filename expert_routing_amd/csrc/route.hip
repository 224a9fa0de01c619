// Router: logits = x . W_r^T in fp32, then per-token scoring, group limit, top-K and
// weights.
//
// bf16 activations: the GEMM runs on bf16 MFMA. Each fp32 router weight w is split
// exactly into three bf16 parts, w = hi + mid + lo (truncation leaves 16, then 8
// significant bits, so every remainder is representable), and x*hi + x*mid + x*lo are
// summed into fp32 accumulators. Every product of bf16 operands is exact in fp32, so
// this is an fp32 GEMM with exact operands and fp32 accumulation, at bf16 MFMA rate.
// fp32 activations take a plain VALU GEMM.
//
// Three shapes of router: up to 16 experts (bf16), one fused kernel computes a group of
// tokens' logits and selects in its epilogue, so the logits never reach HBM; batches of at
// most 64 tokens stream the router weight once (it outweighs x) into k-slabs of partial
// logits; everything else runs a tiled GEMM whose k-slices write slabs of partial logits.
// Slabs are added in slab order by the selection kernel (deterministic).
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
// zero / n_zero: ints the first block clears for the selection that follows (its chunk
// histogram), or nullptr.
template <int BE>
__global__ __launch_bounds__(256) void router_gemm_bf16(const bf16_t* __restrict__ x,
                                                        const float* __restrict__ w,
                                                        float* __restrict__ logits,
                                                        int T, int h, int E, int kslice,
                                                        int32_t* __restrict__ zero, int n_zero) {
  if (zero && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
    for (int i = threadIdx.x; i < n_zero; i += 256) zero[i] = 0;
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
  uint4 xr0, xr1;       // (two named registers: an array here was kept in scratch)
  float4 wr[WPT];
  // x tile: 64 rows x 8 chunks = 512 chunks, 2 per thread (rows r and r + 32)
  const int xr_r = tid >> 3, xr_c = tid & 7;
  const int xt0 = t0 + xr_r < T ? t0 + xr_r : T - 1;
  const int xt1 = t0 + xr_r + 32 < T ? t0 + xr_r + 32 : T - 1;
  auto load = [&](int k0) __attribute__((always_inline)) {
    xr0 = *reinterpret_cast<const uint4*>(x + (size_t)xt0 * h + k0 + xr_c * 8);
    xr1 = *reinterpret_cast<const uint4*>(x + (size_t)xt1 * h + k0 + xr_c * 8);
    // w tile: BE rows x 64 fp32 = BE*16 float4
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int id = tid + i * 256, r = id >> 4, q = id & 15;
      const int e = ebase + r;
      // rows past E load row E - 1 and are zeroed after the load (a lane-divergent load
      // would keep wr out of registers)
      const float4 v =
          *reinterpret_cast<const float4*>(w + (size_t)(e < E ? e : E - 1) * h + k0 + q * 4);
      wr[i] = e < E ? v : float4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto store = [&]() __attribute__((always_inline)) {
    xs[swz(xr_r, xr_c)] = xr0;
    xs[swz(xr_r + 32, xr_c)] = xr1;
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
                                                       int T, int h, int E, int kslice,
                                                       int32_t* __restrict__ zero, int n_zero) {
  if (zero && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
    for (int i = threadIdx.x; i < n_zero; i += 256) zero[i] = 0;
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

// ---- selection of one token by a segment of SEG lanes --------------------------------
// Order-preserving code of a key (a larger float gives a larger code; +0 and -0 share one);
// code 0 is below every real key (the code of -inf is 0x007fffff) and marks non-candidates.
__device__ __forceinline__ uint32_t ord_key(float f) {
  uint32_t u = __float_as_uint(f);
  u = (u == 0x80000000u) ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Sum / max over the SEG lanes of a segment (xor butterfly: every lane gets the result).
template <int SEG>
__device__ __forceinline__ float seg_sum(float v) {
#pragma unroll
  for (int off = SEG / 2; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
template <int SEG>
__device__ __forceinline__ float seg_max(float v) {
#pragma unroll
  for (int off = SEG / 2; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// Lane j of the segment holds experts j, j + SEG, ... (KPL keys per lane; KPL * SEG >= E).
// Scoring, group limit, top-K, weights, and the ids written in ascending order with
// weights aligned. Top-K is a radix select on the key codes: the K-th largest code is
// built bit by bit from ballot counts, the codes above it are taken, and ties at it go to
// the lowest expert ids, so a key of -inf is an ordinary candidate (after every finite key,
// by index). The group limit scores each group by the sum of its two largest keys: with
// groups that are aligned power-of-two runs of at most SEG lanes it runs on shuffles,
// otherwise through LDS rows ks / gs / ga of this token (keys [E], group scores and flags
// [n_groups]; then every thread of the block must call this, as it synchronises the
// block). `active`: the segment has a token. hist (LDS or global, may be nullptr): each
// winner adds 1 at its expert id (integer atomics: the counts do not depend on order).
template <int SEG, int KPL>
__device__ __forceinline__ void select_token(
    const float (&Lin)[KPL], bool active, const float* __restrict__ bias, int E, int K,
    int score, int renorm, int n_groups, int topk_groups, float* ks, float* gs, int* ga,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out, int* hist) {
  const int lane = threadIdx.x & 63;
  const int sl = lane & (SEG - 1), base = lane & ~(SEG - 1);
  const uint64_t segmask = SEG == 64 ? ~0ull : (((1ull << SEG) - 1ull) << base);
  const uint64_t below = (1ull << lane) - 1ull;     // lanes under this one
  float L[KPL], key[KPL], raw[KPL];
  uint32_t allow = 0;   // bit j: expert j*SEG + sl is a candidate
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int e = j * SEG + sl;
    float l = -INFINITY, k = -INFINITY, r = 0.f;
    if (active && e < E) {
      allow |= 1u << j;
      l = Lin[j];
      const float b = bias ? bias[e] : 0.f;
      if (score == MOE_SCORE_SOFTMAX) {
        l += b;
        k = l;
      } else {
        r = 1.f / (1.f + expf(-l));
        k = r + b;
      }
    }
    L[j] = l; key[j] = k; raw[j] = r;
  }
  if (n_groups > 1 && topk_groups < n_groups) {
    const int gsz = E / n_groups;
    const bool shuffled = (gsz & (gsz - 1)) == 0 && gsz <= SEG && n_groups <= SEG;
    if (shuffled) {   // uniform: E and n_groups are kernel arguments
      // top-2 of each aligned run of gsz lanes (per j), then the group's score
      float gsc[KPL];
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        float v1 = key[j], v2 = -INFINITY;
        for (int off = 1; off < gsz; off <<= 1) {
          const float o1 = __shfl_xor(v1, off), o2 = __shfl_xor(v2, off);
          const float hi = fmaxf(v1, o1), lo = fminf(v1, o1);
          v2 = fmaxf(lo, fmaxf(v2, o2));
          v1 = hi;
        }
        gsc[j] = gsz > 1 ? v1 + v2 : v1;
      }
      // segment lane q < n_groups takes group q's score, ranks it among the groups
      const int q = sl;
      const int qj = (q * gsz) / SEG, qlane = base + (q * gsz) % SEG;
      float mine = -INFINITY;
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const float v = __shfl(gsc[j], qlane);
        if (j == qj) mine = v;
      }
      int rank = 0;
      for (int g = 0; g < n_groups; ++g) {
        const float sg = __shfl(mine, base + g);
        rank += better(sg, g, mine, q) ? 1 : 0;
      }
      const int gallow = (q < n_groups && rank < topk_groups) ? 1 : 0;
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const int e = j * SEG + sl;
        const int ok = __shfl(gallow, base + (e < E ? e / gsz : 0));
        if (e < E && !ok) allow &= ~(1u << j);
      }
    } else {
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const int e = j * SEG + sl;
        if (e < E) ks[e] = key[j];
      }
      __syncthreads();
      for (int g = sl; g < n_groups; g += SEG) {
        float b1 = -INFINITY, b2 = -INFINITY;
        for (int i = 0; i < gsz; ++i) {
          const float v = ks[g * gsz + i];
          if (v > b1) { b2 = b1; b1 = v; } else if (v > b2) { b2 = v; }
        }
        gs[g] = gsz > 1 ? b1 + b2 : b1;
      }
      __syncthreads();
      for (int g = sl; g < n_groups; g += SEG) {
        const float sg = gs[g];
        int rank = 0;
        for (int q = 0; q < n_groups; ++q) rank += better(gs[q], q, sg, g) ? 1 : 0;
        ga[g] = rank < topk_groups;
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const int e = j * SEG + sl;
        if (e < E && !ga[e / gsz]) allow &= ~(1u << j);
      }
    }
  }
  if (!active) return;

  // radix select: thr = the largest code with at least K candidate codes >= thr
  uint32_t code[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) code[j] = (allow >> j & 1u) ? ord_key(key[j]) : 0u;
  uint32_t thr = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) cnt += __popcll(__ballot(code[j] >= cand) & segmask);
    if (cnt >= K) thr = cand;
  }
  int gt = 0;
#pragma unroll
  for (int j = 0; j < KPL; ++j) gt += __popcll(__ballot(code[j] > thr) & segmask);
  const int need = K - gt;   // ties at thr taken, lowest expert ids first
  uint32_t sel = 0;
  int eq_before = 0;
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const uint64_t eqm = __ballot(code[j] == thr) & segmask;
    const bool take =
        code[j] > thr || (code[j] == thr && eq_before + __popcll(eqm & below) < need);
    if (take) sel |= 1u << j;
    eq_before += __popcll(eqm);
  }
  // weights over the selected set
  float m = -INFINITY, z = 0.f;
  if (score == MOE_SCORE_SOFTMAX) {
#pragma unroll
    for (int j = 0; j < KPL; ++j)
      if (renorm ? (sel >> j & 1u) : j * SEG + sl < E) m = fmaxf(m, L[j]);
    m = seg_max<SEG>(m);
#pragma unroll
    for (int j = 0; j < KPL; ++j)
      if (renorm ? (sel >> j & 1u) : j * SEG + sl < E) z += expf(L[j] - m);
    z = seg_sum<SEG>(z);
  } else if (renorm) {
#pragma unroll
    for (int j = 0; j < KPL; ++j)
      if (sel >> j & 1u) z += raw[j];
    z = seg_sum<SEG>(z);
  }
  // positions in ascending expert-id order: selected experts of lower j, then lower lanes
  int sel_before = 0;
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const uint64_t sm = __ballot(sel >> j & 1u) & segmask;
    if (sel >> j & 1u) {
      const int pos = sel_before + __popcll(sm & below);
      const int e = j * SEG + sl;
      float wv;
      if (score == MOE_SCORE_SOFTMAX) wv = expf(L[j] - m) / z;
      else wv = renorm ? raw[j] / z : raw[j];
      ids_out[pos] = e;
      w_out[pos] = wv;
      if (hist) atomicAdd(&hist[e], 1);
    }
    sel_before += __popcll(sm);
  }
}

// ---- fused router for E <= 16 (bf16 activations) -------------------------------------
// One block of 16 waves per group of 16 tokens (grid-stride over groups). The waves split
// h into k32 steps (wave w takes steps w, w + 16, ...): per step a lane loads 16 bytes of
// one token's row of x and 8 fp32 of one expert's router row, splits the latter into bf16
// hi / mid / lo parts, and runs bf16 MFMA 16x16x32 with the tokens as rows. With E <= 8
// the 16 MFMA columns hold hi (experts 0..7) and mid (the same experts), the lo part
// rides in a second MFMA, so each step takes two MFMAs. Columns past E compute values
// nobody reads. With E <= 8 the two lanes of an expert (columns n and n + 8) each load and
// split half of the step's 8 values and swap parts through DPP. The waves' partial logits
// meet in LDS and are added in wave order; then
// each wave selects for 4 tokens, 16 lanes per token. The logits never leave the chip.
// The next batch of loads is issued before the current batch's MFMAs.
constexpr int RS_NW = 16;     // waves per block

// Steps per load batch: the paired layout holds 16 bytes of x and 16 of W per step and lane,
// the other one 16 + 32 (within the 128 VGPRs of 16 waves per CU).
template <bool PAIRED>
constexpr int rs_u() { return PAIRED ? 8 : 4; }

// W: with PAIRED, lane n < 8 loads k-values 0..3 of the lane's 8-value chunk and lane n + 8
// loads 4..7 (a float4 each); otherwise a lane loads all 8 (two float4).
template <bool PAIRED, int U>
__device__ __forceinline__ void rs_load(uint4 (&xv)[U], float4 (&wv)[U][PAIRED ? 1 : 2],
                                        const bf16_t* __restrict__ xrow,
                                        const float* __restrict__ wrow, int s0, int S) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    int s = s0 + u * RS_NW;
    s = s < S ? s : S - 1;      // past the end: a valid address, never used
    xv[u] = *reinterpret_cast<const uint4*>(xrow + s * 32);
    wv[u][0] = *reinterpret_cast<const float4*>(wrow + s * 32);
    if (!PAIRED) wv[u][PAIRED ? 0 : 1] = *reinterpret_cast<const float4*>(wrow + s * 32 + 4);
  }
}

// Packs the bf16 hi / mid / lo parts of two fp32 values into one dword per part.
__device__ __forceinline__ void split3_pair(float a, float b, uint32_t& ph, uint32_t& pm,
                                            uint32_t& pl) {
  bf16_t h0, m0, l0, h1, m1, l1;
  split3(a, h0, m0, l0);
  split3(b, h1, m1, l1);
  ph = (uint32_t)h0 | ((uint32_t)h1 << 16);
  pm = (uint32_t)m0 | ((uint32_t)m1 << 16);
  pl = (uint32_t)l0 | ((uint32_t)l1 << 16);
}

// Value of the lane 8 positions away within the lane's row of 16 (DPP row rotate by 8).
__device__ __forceinline__ uint32_t row_swap8(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xf, 0xf, false);
}

template <bool PAIRED, int U>
__device__ __forceinline__ void rs_compute(floatx4& acc, const uint4 (&xv)[U],
                                           const float4 (&wv)[U][PAIRED ? 1 : 2], int s0,
                                           int S, bool hi_col) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (s0 + u * RS_NW < S) {
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, xv[u]);
      if (PAIRED) {
        // this lane splits its 4 values; the partner lane (n xor 8) split the other 4 of
        // the same expert's chunk. Column n < 8 takes hi (+ lo in the second MFMA) of all 8
        // values, column n + 8 takes mid.
        uint32_t h[2], m[2], l[2];
        split3_pair(wv[u][0].x, wv[u][0].y, h[0], m[0], l[0]);
        split3_pair(wv[u][0].z, wv[u][0].w, h[1], m[1], l[1]);
        uint32_t hp[2], mp[2], lp[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          hp[q] = row_swap8(h[q]);
          mp[q] = row_swap8(m[q]);
          lp[q] = row_swap8(l[q]);
        }
        // hi lanes own k 0..3 (partner 4..7); mid lanes own k 4..7 (partner 0..3)
        uint4 b1, b2;
        b1.x = hi_col ? h[0] : mp[0]; b1.y = hi_col ? h[1] : mp[1];
        b1.z = hi_col ? hp[0] : m[0]; b1.w = hi_col ? hp[1] : m[1];
        b2.x = hi_col ? l[0] : 0u;    b2.y = hi_col ? l[1] : 0u;
        b2.z = hi_col ? lp[0] : 0u;   b2.w = hi_col ? lp[1] : 0u;
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, b2), acc,
                                                      0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, b1), acc,
                                                      0, 0, 0);
      } else {
        const float f[8] = {wv[u][0].x, wv[u][0].y, wv[u][0].z, wv[u][0].w,
                            wv[u][PAIRED ? 0 : 1].x, wv[u][PAIRED ? 0 : 1].y,
                            wv[u][PAIRED ? 0 : 1].z, wv[u][PAIRED ? 0 : 1].w};
        uint32_t ph[4], pm[4], pl[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) split3_pair(f[2 * q], f[2 * q + 1], ph[q], pm[q], pl[q]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            a, __builtin_bit_cast(bf16x8_t, uint4{pl[0], pl[1], pl[2], pl[3]}), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            a, __builtin_bit_cast(bf16x8_t, uint4{pm[0], pm[1], pm[2], pm[3]}), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            a, __builtin_bit_cast(bf16x8_t, uint4{ph[0], ph[1], ph[2], ph[3]}), acc, 0, 0, 0);
      }
    }
  }
}

template <bool PAIRED>
__global__ __launch_bounds__(64 * RS_NW) void router_small_e(
    const bf16_t* __restrict__ x, const float* __restrict__ w, const float* __restrict__ bias,
    int32_t* __restrict__ ids, float* __restrict__ wout, int T, int h, int E, int K,
    int score, int renorm, int n_groups, int topk_groups, int32_t* __restrict__ group_counts) {
  __shared__ float red[RS_NW][16][17];
  __shared__ int hist_s[16];
  __shared__ float lg[16][17];
  __shared__ float sel_k[4 * RS_NW][16];
  __shared__ float sel_g[4 * RS_NW][16];
  __shared__ int sel_a[4 * RS_NW][16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, kq = lane >> 4;
  int e_row = PAIRED ? (n & 7) : n;
  e_row = e_row < E ? e_row : E - 1;                  // columns past E: ignored results
  const bool hi_col = n < 8;
  const int S = h / 32;                               // k32 steps
  const int ngroups = (T + 15) / 16;
  const float* wrow = w + (size_t)e_row * h + kq * 8 + ((PAIRED && !hi_col) ? 4 : 0);
  constexpr int RS_U = rs_u<PAIRED>();
  constexpr int STRIDE = RS_NW * RS_U;
  for (int grp = blockIdx.x; grp < ngroups; grp += gridDim.x) {
    const int t0 = grp * 16;
    const int tok = t0 + n < T ? t0 + n : T - 1;      // MFMA row = token
    const bf16_t* xrow = x + (size_t)tok * h + kq * 8;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    uint4 xa[RS_U];
    float4 wa[RS_U][PAIRED ? 1 : 2];
    // one batch of RS_U steps in flight per wave: with 16 waves that is all of h <= 4096
    for (int s0 = wave; s0 < S; s0 += STRIDE) {
      rs_load<PAIRED>(xa, wa, xrow, wrow, s0, S);
      rs_compute<PAIRED>(acc, xa, wa, s0, S, hi_col);
    }
    // acc[j]: token 4*kq + j, column n (PAIRED: columns n and n + 8 hold one expert)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v = acc[j];
      if (PAIRED) v += __shfl_xor(v, 8);
      red[wave][4 * kq + j][n] = v;
    }
    __syncthreads();
    if (tid < 256) {
      const int tk = tid >> 4, e = tid & 15;
      float s = red[0][tk][e];
#pragma unroll
      for (int q = 1; q < RS_NW; ++q) s += red[q][tk][e];
      lg[tk][e] = s;
    }
    if (tid < 16) hist_s[tid] = 0;
    __syncthreads();
    // selection: wave w takes tokens 4w .. 4w + 3 of the group (waves 4.. have none but
    // still pass the group limit's barriers), 16 lanes per token
    const int slot = wave * 4 + kq;
    const bool active = slot < 16 && t0 + slot < T;
    const float L[1] = {active ? lg[slot][n] : 0.f};
    const size_t t = (size_t)(t0 + (active ? slot : 0));
    select_token<16, 1>(L, active, bias, E, K, score, renorm, n_groups, topk_groups,
                        sel_k[slot], sel_g[slot], sel_a[slot], ids + t * K, wout + t * K,
                        group_counts ? hist_s : nullptr);
    __syncthreads();
    // the group's per-expert pair counts: dispatch's histogram, 16 tokens per row
    if (group_counts && tid < E) group_counts[(size_t)grp * E + tid] = hist_s[tid];
  }
}

// ---- router for small batches (T <= 64, bf16 activations) ----------------------------
// The router weight (E x h fp32) is the bulk of the bytes: every block streams a slab of
// 16 experts x kslice of it once, with the batch's x columns for that k range staged in
// LDS. 16 threads per expert split the k range in float4 steps, each holding TB token
// accumulators (fp32 FMA on exact bf16 -> fp32 activations); a butterfly over those 16
// lanes adds them, and the block's partial logits go to slab blockIdx.y, which select adds
// in slab order.
constexpr int GV_EB = 16;
constexpr int GV_MAXI = 16;   // float4 steps per thread: kslice <= 16 * 64 = 1024
constexpr int GV_XB = 8;      // x chunks per thread loaded together when staging

template <int TB>
__global__ __launch_bounds__(256) void router_gemv(const bf16_t* __restrict__ x,
                                                   const float* __restrict__ w,
                                                   float* __restrict__ logits, int T, int h,
                                                   int E, int kslice,
                                                   int32_t* __restrict__ zero, int n_zero) {
  if (zero && blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i < n_zero; i += 256) zero[i] = 0;
  extern __shared__ uint4 xs_raw[];                   // [TB][kslice] bf16
  bf16_t* xs = reinterpret_cast<bf16_t*>(xs_raw);
  const int tid = threadIdx.x, kl = tid & 15;
  const int e = blockIdx.x * GV_EB + (tid >> 4);
  const int kb = blockIdx.y * kslice;
  const int klen = kb + kslice <= h ? kslice : h - kb;   // a multiple of 64
  // the thread's float4 steps of its expert's row (k = 4*kl + 64*i), all issued before x
  // is staged, so one memory round trip covers both; steps past klen load a valid
  // address and are never used
  const float* wr = w + (size_t)(e < E ? e : E - 1) * h + kb;
  float4 wv[GV_MAXI];
#pragma unroll
  for (int i = 0; i < GV_MAXI; ++i) {
    const int k0 = 4 * kl + 64 * i;
    wv[i] = *reinterpret_cast<const float4*>(wr + (k0 < klen ? k0 : 4 * kl));
  }
  // stage x[0..T)[kb, kb + klen) as 16-byte chunks; rows past T are zero. A thread's
  // chunks are loaded in batches of GV_XB, every load of a batch issued before its LDS
  // stores (one memory round trip per batch rather than per chunk)
  const int cpr = klen / 8, nchunk = TB * cpr;
  for (int base = tid; base < nchunk; base += 256 * GV_XB) {
    uint4 v[GV_XB];
#pragma unroll
    for (int j = 0; j < GV_XB; ++j) {
      const int i = base + 256 * j;
      v[j] = uint4{0, 0, 0, 0};
      if (i < nchunk && i / cpr < T)
        v[j] = *reinterpret_cast<const uint4*>(x + (size_t)(i / cpr) * h + kb + (i % cpr) * 8);
    }
#pragma unroll
    for (int j = 0; j < GV_XB; ++j) {
      const int i = base + 256 * j;
      if (i < nchunk)
        *reinterpret_cast<uint4*>(xs + (size_t)(i / cpr) * kslice + (i % cpr) * 8) = v[j];
    }
  }
  __syncthreads();
  float acc[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) acc[t] = 0.f;
#pragma unroll
  for (int i = 0; i < GV_MAXI; ++i) {
    const int k0 = 4 * kl + 64 * i;
    if (k0 >= klen) break;
    const float4 v4 = wv[i];
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const uint2 xv = *reinterpret_cast<const uint2*>(xs + (size_t)t * kslice + k0);
      float a = acc[t];
      a = fmaf(v4.x, __uint_as_float(xv.x << 16), a);
      a = fmaf(v4.y, __uint_as_float(xv.x & 0xffff0000u), a);
      a = fmaf(v4.z, __uint_as_float(xv.y << 16), a);
      a = fmaf(v4.w, __uint_as_float(xv.y & 0xffff0000u), a);
      acc[t] = a;
    }
  }
#pragma unroll
  for (int t = 0; t < TB; ++t) {
    float v = acc[t];
    v += __shfl_xor(v, 8);
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 1);
    acc[t] = v;
  }
  if (e < E) {
    float* out = logits + (size_t)blockIdx.y * T * E;
#pragma unroll
    for (int t = 0; t < TB; ++t)
      if ((t & 15) == kl && t < T) out[(size_t)t * E + e] = acc[t];
  }
}

constexpr int SEL_TOK = 4;     // tokens (waves) per block

// One wave per token. Lane l holds experts l, l+64, ... (KPL keys per lane, 64 * KPL >= E).
// Partial logits of nsplit slabs are added in slab order, then select_token scores and
// selects. chunk_counts (or nullptr): [T / 256 chunks][E] pair counts for dispatch, zeroed
// by the router GEMM.
template <int KPL>
__global__ __launch_bounds__(256) void select_topk(const float* __restrict__ logits,
                                                   const float* __restrict__ bias,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ wout, int T, int E,
                                                   int K, int score, int renorm, int n_groups,
                                                   int topk_groups, int nsplit,
                                                   int32_t* __restrict__ chunk_counts) {
  __shared__ float keys_s[SEL_TOK][64 * KPL];
  __shared__ float gscore_s[SEL_TOK][64 * KPL];
  __shared__ int gallow_s[SEL_TOK][64 * KPL];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * SEL_TOK + wave;
  const bool active = t < T;
  // partial logits of the nsplit slabs added in slab order; every load of a chunk of 8
  // slabs is issued before the additions (lanes past E read a valid address)
  constexpr int SB = 8;
  const int64_t tr = active ? t : 0;
  float L[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) L[j] = 0.f;
  for (int z0 = 0; z0 < nsplit; z0 += SB) {
    float v[SB][KPL];
#pragma unroll
    for (int u = 0; u < SB; ++u)
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const int e = j * 64 + lane;
        v[u][j] = z0 + u < nsplit
                      ? logits[(size_t)(z0 + u) * T * E + tr * E + (e < E ? e : E - 1)]
                      : 0.f;
      }
#pragma unroll
    for (int u = 0; u < SB; ++u)
#pragma unroll
      for (int j = 0; j < KPL; ++j)
        if (z0 + u < nsplit) L[j] = (z0 + u == 0) ? v[u][j] : L[j] + v[u][j];
  }
  select_token<64, KPL>(L, active, bias, E, K, score, renorm, n_groups, topk_groups,
                        keys_s[wave], gscore_s[wave], gallow_s[wave], ids + tr * K,
                        wout + tr * K,
                        chunk_counts ? chunk_counts + (tr / kDispatchChunk) * E : nullptr);
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

// Which router a problem takes: the fused small-expert-count router, the weight-streaming
// router for small batches, or the tiled GEMM with k-slices plus a selection kernel.
enum class RouterPath { Fused, Gemv, Gemm };

static RouterPath router_path(const Dims& d) {
  if (d.bf16 && d.E <= 16) return RouterPath::Fused;
  if (d.bf16 && d.T <= 64) return RouterPath::Gemv;
  return RouterPath::Gemm;
}

static int gemv_tb(const Dims& d) { return d.T <= 32 ? 32 : 64; }

// k-slice length of the small-batch router: about 256 blocks, slices a multiple of 64
// along h whose staged x (tb rows) fits 64 KB of LDS.
static int gemv_kslice(const Dims& d) {
  const int eb = (d.E + GV_EB - 1) / GV_EB;
  int z = (256 + eb - 1) / eb;
  const int zmax = d.h / 64;
  z = z < 1 ? 1 : (z > zmax ? zmax : z);
  int ks = ((d.h + z - 1) / z + 63) / 64 * 64;
  const int ks_max = (64 * 1024) / (2 * gemv_tb(d));
  return ks > ks_max ? ks_max : ks;
}

// K-slices of the router GEMM: enough blocks for about four per CU (each keeps one
// k-step of loads in flight, so four hide most of the memory latency), slices of at
// least 256 along h (a multiple of the 64-wide k-step).
static int gemm_split(const Dims& d) {
  const int64_t tiles = ((d.T + RT_BM - 1) / RT_BM) *
                        ((d.E + 63) / 64 > 0 ? (d.E + 63) / 64 : 1);
  int s = tiles > 0 ? (int)((1024 + tiles - 1) / tiles) : 1;
  const int smax = d.h / 256 > 1 ? d.h / 256 : 1;
  s = s < 1 ? 1 : (s > smax ? smax : s);
  return s;
}

// Slabs of partial logits [T][E] fp32 the router leaves in the workspace.
int route_split(const Dims& d) {
  switch (router_path(d)) {
    case RouterPath::Fused: return 0;
    case RouterPath::Gemv: {
      const int ks = gemv_kslice(d);
      return (d.h + ks - 1) / ks;
    }
    default: return gemm_split(d);
  }
}

static int select_with(const moe_problem* p, const Dims& d, const float* logits, int nsplit,
                       const float* bias, int32_t* ids, float* w, int32_t* chunk_counts,
                       hipStream_t st) {
  const unsigned grid = (unsigned)((d.T + SEL_TOK - 1) / SEL_TOK);
  const int kpl = (d.E + 63) / 64;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, st, logits, bias, ids, w, (int)d.T, d.E,
                       d.K, p->score, p->renorm, p->n_groups, p->topk_groups, nsplit,
                       chunk_counts);
  };
  if (kpl <= 1) go(select_topk<1>);
  else if (kpl <= 2) go(select_topk<2>);
  else if (kpl <= 4) go(select_topk<4>);
  else go(select_topk<8>);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

int route_count_tokens(const Dims& d) {
  return router_path(d) == RouterPath::Fused ? 16 : kDispatchChunk;
}

int launch_select(const moe_problem* p, const Dims& d, const float* logits, const float* bias,
                  int32_t* ids, float* w, hipStream_t st) {
  return select_with(p, d, logits, 1, bias, ids, w, nullptr, st);
}

int launch_route(const moe_problem* p, const Dims& d, const void* x, const float* w_router,
                 const float* bias, int32_t* ids, float* w, float* logits,
                 int32_t* chunk_counts, hipStream_t st) {
  const bf16_t* xb = static_cast<const bf16_t*>(x);
  const RouterPath path = router_path(d);
  // the selection's chunk histogram: the GEMM before it clears it
  const int n_zero = (int)((d.T + kDispatchChunk - 1) / kDispatchChunk) * d.E;
  if (path == RouterPath::Fused) {
    const int64_t groups = (d.T + 15) / 16;
    const unsigned grid = (unsigned)(groups < 2048 ? groups : 2048);
    if (d.E <= 8)
      hipLaunchKernelGGL(router_small_e<true>, dim3(grid), dim3(64 * RS_NW), 0, st, xb,
                         w_router, bias, ids, w, (int)d.T, d.h, d.E, d.K, p->score, p->renorm,
                         p->n_groups, p->topk_groups, chunk_counts);
    else
      hipLaunchKernelGGL(router_small_e<false>, dim3(grid), dim3(64 * RS_NW), 0, st, xb,
                         w_router, bias, ids, w, (int)d.T, d.h, d.E, d.K, p->score, p->renorm,
                         p->n_groups, p->topk_groups, chunk_counts);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
  }
  if (path == RouterPath::Gemv) {
    const int ks = gemv_kslice(d);
    const int z = (d.h + ks - 1) / ks;
    const int tb = gemv_tb(d);
    const dim3 grid((unsigned)((d.E + GV_EB - 1) / GV_EB), (unsigned)z);
    const size_t lds = (size_t)tb * ks * 2;
    if (tb == 32)
      hipLaunchKernelGGL(router_gemv<32>, grid, dim3(256), lds, st, xb, w_router, logits,
                         (int)d.T, d.h, d.E, ks, chunk_counts, n_zero);
    else
      hipLaunchKernelGGL(router_gemv<64>, grid, dim3(256), lds, st, xb, w_router, logits,
                         (int)d.T, d.h, d.E, ks, chunk_counts, n_zero);
    if (hipGetLastError() != hipSuccess) return MOE_ERR_LAUNCH;
    return select_with(p, d, logits, z, bias, ids, w, chunk_counts, st);
  }
  const unsigned gt = (unsigned)((d.T + RT_BM - 1) / RT_BM);
  const int S = d.route_split;
  // k-slice length: a multiple of 64 covering h in S slices
  const int kslice = ((d.h + S - 1) / S + 63) / 64 * 64;
  const unsigned gz = (unsigned)((d.h + kslice - 1) / kslice);
  if (d.bf16) {
    const int be = d.E <= 32 ? 32 : 64;
    const dim3 grid(gt, (unsigned)((d.E + be - 1) / be), gz);
    if (be == 32)
      hipLaunchKernelGGL(router_gemm_bf16<32>, grid, dim3(256), 0, st, xb, w_router, logits,
                         (int)d.T, d.h, d.E, kslice, chunk_counts, n_zero);
    else
      hipLaunchKernelGGL(router_gemm_bf16<64>, grid, dim3(256), 0, st, xb, w_router, logits,
                         (int)d.T, d.h, d.E, kslice, chunk_counts, n_zero);
  } else {
    const dim3 grid(gt, (unsigned)((d.E + 63) / 64), gz);
    hipLaunchKernelGGL(router_gemm_f32, grid, dim3(256), 0, st, static_cast<const float*>(x),
                       w_router, logits, (int)d.T, d.h, d.E, kslice, chunk_counts, n_zero);
  }
  if (hipGetLastError() != hipSuccess) return MOE_ERR_LAUNCH;
  if (gz >= 8 && d.T <= 1024) {
    // small batch, many slabs: select would run too few waves to add them quickly; add
    // them with one thread per logit, then select reads one
    const int64_t n = d.T * d.E;
    const unsigned blocks = (unsigned)((n + 255) / 256 < 2048 ? (n + 255) / 256 : 2048);
    hipLaunchKernelGGL(logits_reduce, dim3(blocks), dim3(256), 0, st, logits, n, (int)gz);
    if (hipGetLastError() != hipSuccess) return MOE_ERR_LAUNCH;
    return select_with(p, d, logits, 1, bias, ids, w, chunk_counts, st);
  }
  return select_with(p, d, logits, (int)gz, bias, ids, w, chunk_counts, st);
}

}  // namespace moe
