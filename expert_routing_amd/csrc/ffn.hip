// Expert FFN as two grouped GEMMs over the ragged per-expert row blocks:
//   GEMM1 (gated):  H[r] = silu(A[r] W_g^T) * (A[r] W_u^T)      -> hbuf (act dtype)
//   GEMM2 (down):   Y[r] = H[r] W_d^T                             -> yp / y_sh
// Groups are the local experts (rows from `offsets`, read on the device) plus the
// optional shared expert over this rank's token block. A one-block prep kernel turns
// the offsets into a tile table; every GEMM block finds its (group, n-tile, m-tile) by
// binary search, so the host never waits for the routing result.
//
// bf16 path: 256 threads (4 waves), MFMA 32x32x16 bf16 with fp32 accumulators; operand
// tiles stream by buffer->LDS DMA into two 64-deep stages of XOR-swizzled 128-byte rows,
// one k-step ahead of the MFMAs; an LDS-staged epilogue writes 16-byte coalesced rows;
// an XCD-aware block order keeps consecutive tiles of one expert on one XCD's L2. Tile
// shapes (256, 128 or 32 rows by 256 weight rows) are chosen per GEMM from the rows per
// expert; with 128- and 32-row tiles a short remainder rides on an expert's last tile
// (tall tiles); an XCD's last, partial round of tiles is split along K (fp32 partials,
// summed in slice order by the last slice to arrive). Without xp the gate/up GEMM reads
// its A rows straight from x through the row -> token map.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int G_MAX = 513;       // local experts (<= 512) + shared expert
constexpr int G_PAD = 520;
constexpr int kMaxSplit = 4;     // k-slices of a tile in an XCD's last, partial round
constexpr int kCuPerXcdMax = 32; // MI355X: 256 CUs in 8 XCDs
constexpr int kArriveSlots = kNumXcd * kCuPerXcdMax;   // split tiles per GEMM

struct FfnGroup {
  const void* A1;  // [rows][h], or with gidx the token rows x [T][h]
  const int32_t* gidx;  // gathered A rows: row r is token gidx[r] / gK (< 0: zero row)
  const void* B1;  // [2*inter][h]
  void* C1;        // [rows][inter]  (hbuf)
  const void* B2;  // [h][inter]
  void* C2;        // [rows][h]
  int rows;
  int inter;
  int mt[2];    // m-tiles of the gate/up [0] and down [1] GEMMs (their tile heights differ)
  int tall[2];  // 1: the last m-tile also takes the (short) remainder: BM + tall_extra rows,
                // split into tall_split narrower tiles per n-tile
  int arows;  // rows addressable through A1 (rows, or T when gathering)
  int gK;     // pairs per token (row index -> token) when gathering
};

struct FfnSched {
  int n_groups;
  int total1;
  int total2;
  int tall_split[2];
  int cu_per_xcd;   // CUs of one XCD (one round of blocks there)
  int split_max;    // 1: no split-K; else the most k-slices a tile may take
  int pad2_;
  int start1[G_PAD];
  int start2[G_PAD];
  FfnGroup g[G_MAX];
};

// One block of 1024 threads.
__global__ __launch_bounds__(1024) void ffn_prep(FfnSched* __restrict__ sc,
                                                 const int32_t* __restrict__ offsets,
                                                 const char* xp, const char* w13, const char* w2,
                                                 const char* x, const char* w13_sh,
                                                 const char* w2_sh, char* hbuf, char* yp,
                                                 char* y_sh, int El, int has_shared,
                                                 int64_t sh_rows, int64_t sh_t0, int h, int inter,
                                                 int sh_inter, int64_t R_max, int s, int BM1,
                                                 int BM2, int tall_extra1, int tall_extra2,
                                                 int tall_split1, int tall_split2, int BN1,
                                                 int BN2, int cu_per_xcd, int split_max,
                                                 int* __restrict__ arrive,
                                                 const int32_t* __restrict__ row_src, int K,
                                                 int64_t T) {
  __shared__ int s1[1024], s2[1024];
  const int g = threadIdx.x;
  const int G = El + has_shared;
  int t1 = 0, t2 = 0;
  if (g < G) {
    FfnGroup fg;
    int rows, I;
    if (g < El) {
      const int r0 = offsets[g];
      rows = offsets[g + 1] - r0;
      I = inter;
      fg.A1 = row_src ? x : xp + (size_t)r0 * h * s;
      fg.gidx = row_src ? row_src + r0 : nullptr;
      fg.B1 = w13 + (size_t)g * 2 * inter * h * s;
      fg.C1 = hbuf + (size_t)r0 * inter * s;
      fg.B2 = w2 + (size_t)g * h * inter * s;
      fg.C2 = yp + (size_t)r0 * h * s;
    } else {
      rows = (int)sh_rows;
      I = sh_inter;
      fg.A1 = x + (size_t)sh_t0 * h * s;
      fg.gidx = nullptr;
      fg.B1 = w13_sh;
      fg.C1 = hbuf + (size_t)R_max * inter * s;
      fg.B2 = w2_sh;
      fg.C2 = y_sh;
    }
    // A remainder of at most tall_extra rows rides on the expert's last full tile (it
    // reads the same weights) instead of costing a tile of its own. Per n-tile: mt tiles,
    // or mt - 1 full ones and tall_split tall ones.
    int per_n[2];
    const int BMg[2] = {BM1, BM2}, TEg[2] = {tall_extra1, tall_extra2};
    const int TSg[2] = {tall_split1, tall_split2};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int q = rows / BMg[k], r = rows % BMg[k];
      const int tall = q >= 1 && r > 0 && r <= TEg[k];
      fg.mt[k] = tall ? q : (rows + BMg[k] - 1) / BMg[k];
      fg.tall[k] = tall;
      per_n[k] = tall ? fg.mt[k] - 1 + TSg[k] : fg.mt[k];
    }
    fg.rows = rows;
    fg.inter = I;
    fg.arows = fg.gidx ? (int)T : rows;
    fg.gK = K;
    sc->g[g] = fg;
    t1 = per_n[0] * ((I + BN1 - 1) / BN1);
    t2 = per_n[1] * ((h + BN2 - 1) / BN2);
  }
  s1[g] = t1;
  s2[g] = t2;
  __syncthreads();
  for (int st = 1; st < 1024; st <<= 1) {
    const int a1 = g >= st ? s1[g - st] : 0;
    const int a2 = g >= st ? s2[g - st] : 0;
    __syncthreads();
    s1[g] += a1;
    s2[g] += a2;
    __syncthreads();
  }
  if (g <= G) {
    sc->start1[g] = g == 0 ? 0 : s1[g - 1];
    sc->start2[g] = g == 0 ? 0 : s2[g - 1];
  }
  for (int i = g; i < 2 * kArriveSlots; i += 1024) arrive[i] = 0;
  if (g == 0) {
    sc->n_groups = G;
    sc->tall_split[0] = tall_split1;
    sc->tall_split[1] = tall_split2;
    sc->cu_per_xcd = cu_per_xcd;
    sc->split_max = split_max;
    sc->total1 = s1[G - 1];
    sc->total2 = s2[G - 1];
  }
}

// Tile lookup shared by the GEMM kernels. The tile list is dealt to the XCDs in
// contiguous ranges (consecutive tiles of an expert share its weights in one L2); an
// XCD runs its range in rounds of cu_per_xcd blocks. When the last round would leave
// at least half of the XCD idle, each of its tiles is cut into S k-slices (split-K):
// the slices store fp32 partial sums that a second kernel adds in slice order.
struct TileRef {
  int g, m_tile, n_tile;
  int tall;     // 0: full tile; 1 + s: part s of the expert's tall last tile
  int slice;    // k-slice of a split tile, else 0
  int nslice;   // k-slices of the tile (1: not split)
  int piece;    // partial-sum slot of slice 0 of a split tile, else -1
  int pstride;  // slots between consecutive slices of the tile
  int tid_x;    // the tile's split index on its XCD (arrival counter)
};

struct XcdPlan {
  int base, cnt;     // the XCD's tiles: [base, base + cnt)
  int full, rem, S;  // whole rounds, tiles left for the last round, k-slices each
};

__device__ __forceinline__ XcdPlan xcd_plan(const FfnSched* sc, bool first, int xcd) {
  const int total = first ? sc->total1 : sc->total2;
  const int per = (total + kNumXcd - 1) / kNumXcd;
  XcdPlan q;
  q.base = xcd * per;
  q.cnt = max(0, min(per, total - q.base));
  const int cpx = sc->cu_per_xcd;
  q.full = q.cnt / cpx * cpx;
  q.rem = q.cnt - q.full;
  q.S = 1;
  if (sc->split_max > 1 && q.rem > 0 && 2 * q.rem <= cpx) q.S = min(sc->split_max, cpx / q.rem);
  return q;
}

// Expert, m-tile, n-tile and tall part of tile L.
__device__ __forceinline__ void locate(const FfnSched* sc, bool first, int L, TileRef& t) {
  const int* start = first ? sc->start1 : sc->start2;
  int lo = 0, hi = sc->n_groups;          // start[lo] <= L < start[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (start[mid] <= L) lo = mid; else hi = mid;
  }
  t.g = lo;
  const int gi = first ? 0 : 1;
  const int mt = sc->g[lo].mt[gi];
  const int local = L - start[lo];
  if (sc->g[lo].tall[gi]) {
    const int per_n = mt - 1 + sc->tall_split[gi];
    const int w = local % per_n;
    t.n_tile = local / per_n;
    t.m_tile = w < mt - 1 ? w : mt - 1;
    t.tall = w < mt - 1 ? 0 : 1 + w - (mt - 1);
  } else {
    t.m_tile = local % mt;
    t.n_tile = local / mt;
    t.tall = 0;
  }
}

__device__ __forceinline__ bool find_tile(const FfnSched* sc, bool first, TileRef& t) {
  const int xcd = blockIdx.x % kNumXcd, slot = blockIdx.x / kNumXcd;
  const XcdPlan q = xcd_plan(sc, first, xcd);
  int L;
  t.slice = 0;
  t.nslice = 1;
  t.piece = -1;
  t.pstride = 0;
  t.tid_x = -1;
  if (slot < q.full || q.S == 1) {
    if (slot >= q.cnt) return false;
    L = q.base + slot;
  } else {
    const int p = slot - q.full;
    if (p >= q.rem * q.S) return false;
    L = q.base + q.full + p % q.rem;
    t.slice = p / q.rem;
    t.nslice = q.S;
    t.piece = xcd * sc->cu_per_xcd + p % q.rem;
    t.pstride = q.rem;
    t.tid_x = xcd * sc->cu_per_xcd + p % q.rem;
  }
  locate(sc, first, L, t);
  if (t.tall && t.nslice > 1) {   // tall parts are not split: slice 0 takes all of K
    if (t.slice > 0) return false;
    t.nslice = 1;
    t.piece = -1;
  }
  return true;
}

__device__ __forceinline__ float silu(float v) { return v / (1.f + __expf(-v)); }

// silu for the bf16 epilogues: the hardware reciprocal (about 1 ulp) instead of an IEEE
// divide; the result is rounded to bf16 right after.
__device__ __forceinline__ float silu_fast(float v) {
  return v * __builtin_amdgcn_rcpf(1.f + __expf(-v));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw buffer: stride 0, num_records = bytes; reads past the end return zero
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}


#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// Slot of a 16-byte chunk in a 128-byte LDS row: chunk c of row r sits at
// c ^ row_swz(r). Any 8 aligned consecutive rows (one 128-byte bank sweep) and any 16
// aligned consecutive rows (one 256-byte sweep) then hold a given chunk in distinct
// slots, so ds_read_b128 fragment reads (lanes = consecutive rows, same chunk) are free
// of bank conflicts whether the LDS serves 8 or 16 lanes per cycle.
__device__ __forceinline__ int row_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

constexpr int kDmaStride = 2;   // MFMAs per interleaved DMA instruction

constexpr int kLdsBytes = 160 * 1024;   // LDS per workgroup on gfx950

// s_waitcnt immediate for vmcnt(n) with the other counters left open (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier without the memory fence __syncthreads() carries (the fence would
// also wait for LDS DMA still in flight); callers wait for the DMA they need first.
__device__ __forceinline__ void lds_barrier() { __builtin_amdgcn_s_barrier(); }

// Epilogue of a bf16 tile. acc[i][j][q]: token row wm*WTM + i*32 + (lane&31); output
// column (col-tile base) + 8*(q>>2) + 4*(lane>>5) + (q&3). Stages bf16 in LDS (the
// caller has finished with the operand stages and synchronised), then stores 16-byte
// row-contiguous chunks. GATED: out = silu(gate) * up, gate col-tiles first.
template <int BM, int BN, int WM, int WN, bool GATED>
__device__ __forceinline__ void store_tile(const floatx16 (&acc)[BM / WM / 32][BN / WN / 32],
                                           const FfnGroup& fg, int m0, int n0, int h,
                                           uint4* __restrict__ smem) {
  constexpr int NT = 64 * WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int BNO = GATED ? BN / 2 : BN;
  constexpr int PITCH = BNO * 2 + 16;                  // bytes per staged row
  static_assert((size_t)BM * PITCH <= (size_t)kLdsBytes, "staged tile fits the LDS");
  const int rows = fg.rows;
  const int Nout = GATED ? fg.inter : h;
  bf16_t* C = static_cast<bf16_t*>(GATED ? fg.C1 : fg.C2);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  char* stage = reinterpret_cast<char*>(smem);
  constexpr int TNO = GATED ? TN / 2 : TN;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int row = wm * WTM + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < TNO; ++j) {
      const int cbase = (GATED ? wn * (WTN / 2) : wn * WTN) + j * 32 + 4 * (lane >> 5);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int q = q4 * 4 + u;
          v[u] = GATED ? silu_fast(acc[i][j][q]) * acc[i][j + TN / 2][q] : acc[i][j][q];
        }
        bf16x4_t pk = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
        *reinterpret_cast<bf16x4_t*>(stage + row * PITCH + (cbase + 8 * q4) * 2) = pk;
      }
    }
  }
  __syncthreads();
  constexpr int RCH = BNO / 8;                         // 16-byte chunks per row
  for (int id = tid; id < BM * RCH; id += NT) {
    const int r = id / RCH, cc = id % RCH;
    const int gr = m0 + r, gc = n0 + cc * 8;
    if (gr < rows && gc < Nout)
      *reinterpret_cast<uint4*>(C + (size_t)gr * Nout + gc) =
          *reinterpret_cast<const uint4*>(stage + r * PITCH + cc * 16);
  }
}

// Epilogue of a split tile, run by its last k-slice: element values are the fp32
// partial sums of the slices (fragment order, one slot every pstride floats) added in
// slice order, then staged and stored as in store_tile.
template <int BM, int BN, int WM, int WN, bool GATED>
__device__ __forceinline__ void store_tile_parts(const float* __restrict__ part, size_t pstride,
                                                 int nslice, const FfnGroup& fg, int m0, int n0,
                                                 int h, uint4* __restrict__ smem) {
  constexpr int NT = 64 * WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int BNO = GATED ? BN / 2 : BN;
  constexpr int PITCH = BNO * 2 + 16;
  const int rows = fg.rows;
  const int Nout = GATED ? fg.inter : h;
  bf16_t* C = static_cast<bf16_t*>(GATED ? fg.C1 : fg.C2);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  char* stage = reinterpret_cast<char*>(smem);
  constexpr int TNO = GATED ? TN / 2 : TN;
  // Buffer loads: a slot past the last slice lies past the descriptor's end and reads
  // zero without touching memory, so every 32x32 block issues all its loads at once
  // (slices x 4 float4, twice when gated) before adding them in slice order.
  const __amdgpu_buffer_rsrc_t prs =
      make_rsrc(part, (uint32_t)((size_t)nslice * pstride * sizeof(float)));
  const uint32_t lane_off =
      (uint32_t)(((size_t)wave * TM * TN * 4 * 64 + lane) * sizeof(float4));
  const uint32_t slice_bytes = (uint32_t)(pstride * sizeof(float));
  auto ld = [&](int i, int j, int q4, int sl) __attribute__((always_inline)) {
    return __builtin_bit_cast(
        float4, __builtin_amdgcn_raw_buffer_load_b128(
                    prs, lane_off + (uint32_t)(((i * TN + j) * 4 + q4) * 64 * sizeof(float4)),
                    (uint32_t)sl * slice_bytes, 0));
  };
  auto add_slices = [&](const float4 (&v)[kMaxSplit]) __attribute__((always_inline)) {
    float4 a = v[0];
#pragma unroll
    for (int sl = 1; sl < kMaxSplit; ++sl) {
      a.x += v[sl].x; a.y += v[sl].y; a.z += v[sl].z; a.w += v[sl].w;
    }
    return a;
  };
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int row = wm * WTM + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < TNO; ++j) {
      const int cbase = (GATED ? wn * (WTN / 2) : wn * WTN) + j * 32 + 4 * (lane >> 5);
      float4 g[4][kMaxSplit], u[GATED ? 4 : 1][kMaxSplit];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
        for (int sl = 0; sl < kMaxSplit; ++sl) {
          g[q4][sl] = ld(i, j, q4, sl);
          if (GATED) u[q4][sl] = ld(i, j + TN / 2, q4, sl);
        }
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 gs = add_slices(g[q4]);
        float v[4] = {gs.x, gs.y, gs.z, gs.w};
        if (GATED) {
          const float4 us = add_slices(u[q4]);
          v[0] = silu_fast(v[0]) * us.x;
          v[1] = silu_fast(v[1]) * us.y;
          v[2] = silu_fast(v[2]) * us.z;
          v[3] = silu_fast(v[3]) * us.w;
        }
        bf16x4_t pk = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
        *reinterpret_cast<bf16x4_t*>(stage + row * PITCH + (cbase + 8 * q4) * 2) = pk;
      }
      __builtin_amdgcn_sched_barrier(0);   // one block's loads in flight at a time
    }
  }
  __syncthreads();
  constexpr int RCH = BNO / 8;
  for (int id = tid; id < BM * RCH; id += NT) {
    const int r = id / RCH, cc = id % RCH;
    const int gr = m0 + r, gc = n0 + cc * 8;
    if (gr < rows && gc < Nout)
      *reinterpret_cast<uint4*>(C + (size_t)gr * Nout + gc) =
          *reinterpret_cast<const uint4*>(stage + r * PITCH + cc * 16);
  }
}

// bf16 grouped GEMM. Block tile BM x BN (BN counts weight rows: for GATED half gate,
// half up), k-step 64, WM x WN waves (4 or 8), each wave (BM/WM) x (BN/WN) as 32x32
// MFMA tiles. With 8 waves two share each SIMD, so one wave's MFMAs keep the matrix
// core busy while the other waits to issue its memory instructions. Operand tiles stream into two LDS stages by buffer->LDS DMA (no register
// staging) one k-step ahead of the MFMAs. Every DMA request covers whole 128-byte row
// segments (half-line requests roughly halve what L2 can deliver per CU). The MFMA takes
// the weight fragment first, so a lane's accumulators hold 4 consecutive output columns.
template <int BM, int BN, int WM, int WN, bool GATED, bool GATHER = false, int NS = 2>
__device__ __forceinline__ void gemm_bf16_body(const FfnGroup& fg, int m0, int n0, int h,
                                               uint4* __restrict__ smem, int slice,
                                               int nslice, float* __restrict__ part,
                                               size_t pstride, int* __restrict__ arrive) {
  constexpr int NW = WM * WN, NT = 64 * NW;
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  static_assert(TM >= 1 && TN >= 1, "tile");
  static_assert(!GATED || TN % 2 == 0, "gated needs gate/up pairs");
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "DMA rows split evenly over waves");
  constexpr int BNO = GATED ? BN / 2 : BN;          // output columns per tile
  constexpr int AI = BM / (8 * NW), BI = BN / (8 * NW);  // DMA instructions per wave per stage
  constexpr int LPS = AI + BI;
  constexpr int A_ST = BM * 8, B_ST = BN * 8;       // uint4 per stage
  constexpr int NMF = TM * TN;                      // MFMAs per k16 phase
  static_assert(NS >= 2 && NS <= 4 && LPS * (NS - 2) < 64, "LDS stages");
  uint4* As = smem;                                 // [NS][BM rows][8 chunks]
  uint4* Bs = smem + NS * A_ST;                     // [NS][BN rows][8 chunks]

  const int rows = fg.rows, I = fg.inter;
  const bf16_t* A = static_cast<const bf16_t*>(GATED ? fg.A1 : fg.C1);
  const bf16_t* B = static_cast<const bf16_t*>(GATED ? fg.B1 : fg.B2);
  bf16_t* C = static_cast<bf16_t*>(GATED ? fg.C1 : fg.C2);
  const int Kd = GATED ? h : I;         // reduction length = lda = ldb
  const int Nout = GATED ? I : h;       // output columns = ldc
  const uint32_t b_rows = GATED ? 2 * I : h;
  const uint32_t a_bytes = (uint32_t)(GATHER ? fg.arows : rows) * Kd * 2;
  const __amdgpu_buffer_rsrc_t ra_rs = make_rsrc(A, a_bytes);
  const __amdgpu_buffer_rsrc_t rb_rs = make_rsrc(B, b_rows * (uint32_t)Kd * 2);

  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a scalar, so LDS DMA destinations (M0) are computed in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // DMA: instruction j of this wave fills tile rows 8*(NW*j+wave) .. +8; lane L lands on
  // row +L/8, slot L&7, so it fetches logical chunk (L&7) ^ row_swz(row) (NW is even, so
  // bit 3 of the row is wave&1). The lane part of the source offset sits in one VGPR per
  // operand (two for the gated B: gate rows and up rows); the rest is uniform (soffset).
  // Rows past an operand's end read as zero; for the gated B, gate rows past I read up
  // rows, which only feed output columns past I that are never stored.
  const int dr = lane >> 3;
  const int dc = (lane & 7) ^ dr ^ (wave & 1);
  const uint32_t a_lane = ((uint32_t)(m0 + 8 * wave + dr) * Kd + dc * 8) * 2;
  const uint32_t b_lane = ((uint32_t)(n0 + 8 * wave + dr) * Kd + dc * 8) * 2;
  const uint32_t b_lane_up = GATED ? b_lane + (uint32_t)I * Kd * 2 : b_lane;
  const uint32_t x_stride = (uint32_t)(8 * NW) * Kd * 2;   // bytes between instructions
  constexpr int BH = GATED ? BI / 2 : BI;                   // instructions per B half
  // Gathered A (the gate/up GEMM reading x through the row -> token map): one offset per
  // instruction and lane; rows past the group or unclaimed read zero (offset past the end).
  uint32_t a_off[GATHER ? AI : 1];
  if constexpr (GATHER) {
    // all AI indices in flight at once (clamped, then masked), as global-memory loads
    const __attribute__((address_space(1))) int32_t* gidx =
        (const __attribute__((address_space(1))) int32_t*)fg.gidx;
    int src[AI];
#pragma unroll
    for (int x = 0; x < AI; ++x) {
      const int r = m0 + 8 * (NW * x + wave) + dr;
      src[x] = gidx[r < rows ? r : rows - 1];
    }
#pragma unroll
    for (int x = 0; x < AI; ++x) {
      const int r = m0 + 8 * (NW * x + wave) + dr;
      a_off[x] = (r < rows && src[x] >= 0) ? ((uint32_t)(src[x] / fg.gK) * Kd + dc * 8) * 2
                                           : a_bytes;
    }
  }
  // DMA instruction `x` (0 <= x < LPS) of k-step `step` into stage `stage`.
  // k-steps [kb, kb + nk) of the Kd / 64: all of them, or this tile's k-slice (wave-
  // uniform values, kept in SGPRs: the DMA takes the k offset as soffset)
  const int kb = __builtin_amdgcn_readfirstlane(slice * (Kd / 64) / nslice);
  const int nk = __builtin_amdgcn_readfirstlane((slice + 1) * (Kd / 64) / nslice) - kb;
  auto issue_one = [&](int step, int stage, int x) __attribute__((always_inline)) {
    const uint32_t soff = (uint32_t)(kb + step) * 128;
    if (x < AI) {
      if constexpr (GATHER)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra_rs, LDS_PTR(As + stage * A_ST + 64 * (NW * x + wave)), 16, a_off[x], soff, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra_rs, LDS_PTR(As + stage * A_ST + 64 * (NW * x + wave)), 16, a_lane,
            soff + x * x_stride, 0, 0);
    } else {
      const int y = x - AI;
      const int yh = y % BH;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb_rs, LDS_PTR(Bs + stage * B_ST + 64 * (NW * y + wave)), 16,
          y < BH ? b_lane : b_lane_up, soff + yh * x_stride, 0, 0);
    }
  };

  floatx16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // Fragment rows (within the tile) and the B row of each col-tile.
  int arow[TM], brow[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) arow[i] = wm * WTM + i * 32 + (lane & 31);
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    int br;
    if (GATED)
      br = j < TN / 2 ? wn * (WTN / 2) + j * 32 : BN / 2 + wn * (WTN / 2) + (j - TN / 2) * 32;
    else
      br = wn * WTN + j * 32;
    brow[j] = br + (lane & 31);
  }
  bf16x8_t fa[2][TM], fb[2][TN];
  auto read_frags = [&](int set, int stage, int kk) __attribute__((always_inline)) {
    const uint4* as = As + stage * A_ST;
    const uint4* bs = Bs + stage * B_ST;
    const int c = kk * 2 + (lane >> 5);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      fb[set][j] = __builtin_bit_cast(bf16x8_t, bs[brow[j] * 8 + (c ^ row_swz(brow[j]))]);
#pragma unroll
    for (int i = 0; i < TM; ++i)
      fa[set][i] = __builtin_bit_cast(bf16x8_t, as[arow[i] * 8 + (c ^ row_swz(arow[i]))]);
  };

  // One k-step: four k16 phases. A phase runs one MFMA (its fragments were read a phase
  // earlier, so the compiler's full LDS wait there is free), reads the next phase's
  // fragments, then its other MFMAs. With `dma`, the next k-step's DMA rides along one
  // instruction every kDmaStride MFMAs: a burst of VMEM issues would block the wave, and
  // one per MFMA (measured) outruns what the address units accept from four waves.
  auto kstep = [&](int stage, bool dma, int next_step, int dma_stage)
                   __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int cur = kk & 1;
#pragma unroll
      for (int t = 0; t < NMF; ++t) {
        acc[t / TN][t % TN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            fb[cur][t % TN], fa[cur][t / TN], acc[t / TN][t % TN], 0, 0, 0);
        const int slot = kk * NMF + t;            // MFMA index within the k-step
        if (dma && slot >= 1 && (slot - 1) % kDmaStride == 0 && (slot - 1) / kDmaStride < LPS)
          issue_one(next_step, dma_stage, (slot - 1) / kDmaStride);
        if (t == 0 && kk < 3) {
          __builtin_amdgcn_sched_barrier(0);
          read_frags(cur ^ 1, stage, kk + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (dma) {   // instructions left over when the k-step has too few MFMAs
#pragma unroll
      for (int x = (4 * NMF - 2) / kDmaStride + 1; x < LPS; ++x)
        issue_one(next_step, dma_stage, x);
    }
  };

  // NS stages: k-step kt lives in stage kt % NS; up to NS - 1 k-steps are in flight.
  if (nk > 0) {
#pragma unroll
  for (int s0 = 0; s0 < NS - 1; ++s0)
    if (s0 < nk)
#pragma unroll
      for (int x = 0; x < LPS; ++x) issue_one(s0, s0, x);
  if (nk >= NS - 1) wait_vmcnt<LPS * (NS - 2)>();   // k-step 0 has landed
  else wait_vmcnt<0>();
  lds_barrier();
  read_frags(0, 0, 0);
  int kt = 0;
  for (; kt + NS - 1 < nk; ++kt) {
    // the DMA of k-step kt + NS - 1 refills the stage k-step kt - 1 used: every wave
    // passed the barrier after its last reads there
    kstep(kt % NS, true, kt + NS - 1, (kt + NS - 1) % NS);
    // k-step kt+1 has landed (this wave's DMA; the NS - 2 after it may still be in
    // flight) and every wave is past its reads of stage kt % NS; the barrier publishes
    // the DMA of all waves
    wait_vmcnt<LPS * (NS - 2)>();
    lds_barrier();
    read_frags(0, (kt + 1) % NS, 0);
  }
  for (; kt + 1 < nk; ++kt) {   // the last NS - 2 k-steps: nothing left to fetch
    kstep(kt % NS, false, 0, 0);
    const int after = nk - kt - 2;   // k-steps still in flight behind k-step kt+1
    if (NS > 3 && after >= 2) wait_vmcnt<LPS * (NS > 3 ? 2 : 0)>();
    else if (NS > 2 && after >= 1) wait_vmcnt<LPS * (NS > 2 ? 1 : 0)>();
    else wait_vmcnt<0>();
    lds_barrier();
    read_frags(0, (kt + 1) % NS, 0);
  }
  kstep((nk - 1) % NS, false, 0, 0);
  }
  __syncthreads();

  if (part) {
    // Split tile: store this slice's fp32 partial sums (fragment order, so each store is
    // 1 KB contiguous), then count the slice in. The last slice to arrive adds all of
    // them in slice order (the same order whichever arrives last) and stores the tile.
    const size_t frag = (size_t)wave * TM * TN * 4 * 64 + lane;
    float4* dst = reinterpret_cast<float4*>(part + (size_t)slice * pstride) + frag;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          dst[((i * TN + j) * 4 + q4) * 64] =
              make_float4(acc[i][j][4 * q4], acc[i][j][4 * q4 + 1], acc[i][j][4 * q4 + 2],
                          acc[i][j][4 * q4 + 3]);
    __threadfence();
    __syncthreads();
    // the flag lives in the (now idle) operand LDS: a second LDS object would make the
    // compiler wait for all LDS DMA before every fragment read of the main loop
    int* last = reinterpret_cast<int*>(smem);
    if (tid == 0) *last = atomicAdd(arrive, 1) == nslice - 1;
    __syncthreads();
    if (!*last) return;
    __threadfence();
    store_tile_parts<BM, BN, WM, WN, GATED>(part, pstride, nslice, fg, m0, n0, h, smem);
    return;
  }
  store_tile<BM, BN, WM, WN, GATED>(acc, fg, m0, n0, h, smem);
}

template <int BM, int BN, bool GATED, int NS = 2>
constexpr size_t bf16_lds_bytes() {
  constexpr size_t ops = NS * (size_t)(BM + BN) * 8 * 16;
  constexpr size_t stg = (size_t)BM * ((GATED ? BN / 2 : BN) * 2 + 16);
  return ops > stg ? ops : stg;
}

template <size_t A, size_t B>
constexpr size_t cmax() { return A > B ? A : B; }

// Two kernel names, so profiles tell the gate/up GEMM from the down projection. A block
// takes a BM x BN tile, or one of the parts of an expert's tall last tile: (BM + 32*WM)
// rows (one more MFMA row per wave) by BN / TSPLIT, which keeps the accumulators within
// the register file.
template <int WM, int WN>
constexpr int tall_split() { return WM > 1 ? 2 : 1; }

// LDS stages per tile shape: the 256-row tile fits two; the smaller ones take more, so
// more k-steps of operands are in flight (they stream more bytes per MFMA).
template <int BM>
constexpr int kernel_stages() { return BM >= 256 ? 2 : (BM >= 128 ? 3 : 4); }

template <int BM, int BN, int WM, int WN, bool GATED, bool TALL>
__device__ __forceinline__ void gemm_bf16_tile(const FfnSched* __restrict__ sc, int h,
                                               float* __restrict__ part,
                                               int* __restrict__ arrive,
                                               uint4* __restrict__ smem) {
  constexpr int BMT = BM + 32 * WM, TS = tall_split<WM, WN>(), BNT = BN / TS;
  constexpr int BNO = GATED ? BN / 2 : BN;
  constexpr int NS = kernel_stages<BM>();
  TileRef t;
  if (!find_tile(sc, GATED, t)) return;
  // the tile is the same for the whole block: keep it (and the operand pointers and
  // buffer descriptors derived from it) in SGPRs
  t.g = __builtin_amdgcn_readfirstlane(t.g);
  t.m_tile = __builtin_amdgcn_readfirstlane(t.m_tile);
  t.n_tile = __builtin_amdgcn_readfirstlane(t.n_tile);
  t.tall = __builtin_amdgcn_readfirstlane(t.tall);
  t.slice = __builtin_amdgcn_readfirstlane(t.slice);
  t.nslice = __builtin_amdgcn_readfirstlane(t.nslice);
  t.piece = __builtin_amdgcn_readfirstlane(t.piece);
  t.pstride = __builtin_amdgcn_readfirstlane(t.pstride);
  t.tid_x = __builtin_amdgcn_readfirstlane(t.tid_x);
  const FfnGroup& fg = sc->g[t.g];
  const int m0 = t.m_tile * BM, n0 = t.n_tile * BNO;
  float* pt = t.piece >= 0 ? part + (size_t)t.piece * BM * BN : nullptr;
  int* ar = arrive + (GATED ? 0 : kArriveSlots) + (t.tid_x >= 0 ? t.tid_x : 0);
  const size_t ps = (size_t)t.pstride * BM * BN;
  const int n0t = n0 + (t.tall - 1) * (BNO / TS);
  if (GATED && fg.gidx) {   // gate/up reading x through the row -> token map
    if (TALL && t.tall)
      gemm_bf16_body<TALL ? BMT : BM, TALL ? BNT : BN, WM, WN, GATED, GATED, NS>(
          fg, m0, n0t, h, smem, 0, 1, nullptr, 0, nullptr);
    else
      gemm_bf16_body<BM, BN, WM, WN, GATED, GATED, NS>(fg, m0, n0, h, smem, t.slice, t.nslice, pt,
                                                   ps, ar);
  } else {
    if (TALL && t.tall)
      gemm_bf16_body<TALL ? BMT : BM, TALL ? BNT : BN, WM, WN, GATED, false, NS>(
          fg, m0, n0t, h, smem, 0, 1, nullptr, 0, nullptr);
    else
      gemm_bf16_body<BM, BN, WM, WN, GATED, false, NS>(fg, m0, n0, h, smem, t.slice, t.nslice, pt,
                                                       ps, ar);
  }
}

template <int BM, int BN, int WM, int WN, bool GATED, bool TALL>
constexpr size_t tile_lds_bytes() {
  constexpr int NS = kernel_stages<BM>();
  return TALL ? cmax<bf16_lds_bytes<BM, BN, GATED, NS>(),
                     bf16_lds_bytes<BM + 32 * WM, BN / tall_split<WM, WN>(), GATED, NS>()>()
              : bf16_lds_bytes<BM, BN, GATED, NS>();
}

template <int BM, int BN, int WM, int WN, bool TALL>
__global__ __launch_bounds__(64 * WM * WN) void ffn_gate_up_bf16(const FfnSched* __restrict__ sc,
                                                                 int h, float* part,
                                                                 int* arrive) {
  __shared__ uint4 smem[tile_lds_bytes<BM, BN, WM, WN, true, TALL>() / 16];
  gemm_bf16_tile<BM, BN, WM, WN, true, TALL>(sc, h, part, arrive, smem);
}
template <int BM, int BN, int WM, int WN, bool TALL>
__global__ __launch_bounds__(64 * WM * WN) void ffn_down_bf16(const FfnSched* __restrict__ sc,
                                                              int h, float* part,
                                                              int* arrive) {
  __shared__ uint4 smem[tile_lds_bytes<BM, BN, WM, WN, false, TALL>() / 16];
  gemm_bf16_tile<BM, BN, WM, WN, false, TALL>(sc, h, part, arrive, smem);
}

// fp32 grouped GEMM: 64 x 64 tiles (gated: 32 gate + 32 up columns), 4x4 per thread.
constexpr int F_BM = 64, F_BN = 64, F_BK = 16;
template <bool GATED>
__global__ __launch_bounds__(256) void ffn_gemm_f32(const FfnSched* __restrict__ sc, int h) {
  __shared__ float As[F_BK][F_BM + 4];
  __shared__ float Bs[F_BK][F_BN + 4];
  TileRef t;
  if (!find_tile(sc, GATED, t)) return;
  const FfnGroup fg = sc->g[t.g];
  const int rows = fg.rows, I = fg.inter;
  const float* A = static_cast<const float*>(GATED ? fg.A1 : fg.C1);
  const float* B = static_cast<const float*>(GATED ? fg.B1 : fg.B2);
  float* C = static_cast<float*>(GATED ? fg.C1 : fg.C2);
  const int Kd = GATED ? h : I;
  const int Nout = GATED ? I : h;
  const bool gather = GATED && fg.gidx;   // A rows are tokens of x
  constexpr int BNO = GATED ? F_BN / 2 : F_BN;
  const int m0 = t.m_tile * F_BM, n0 = t.n_tile * BNO;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < Kd; k0 += F_BK) {
    for (int id = tid; id < F_BM * F_BK; id += 256) {
      const int r = id / F_BK, k = id % F_BK, kk = k0 + k;
      const int gr = m0 + r;
      const int src = gr < rows ? (gather ? fg.gidx[gr] : gr) : -1;
      const int64_t arow = gather ? (src >= 0 ? src / fg.gK : -1) : src;
      As[k][r] = (arow >= 0 && kk < Kd) ? A[(size_t)arow * Kd + kk] : 0.f;
      int wrow = -1;
      if (GATED) {
        const int half = r >= F_BN / 2;
        const int col = n0 + (half ? r - F_BN / 2 : r);
        if (col < I) wrow = col + (half ? I : 0);
      } else {
        const int col = n0 + r;
        if (col < Nout) wrow = col;
      }
      Bs[k][r] = (wrow >= 0 && kk < Kd) ? B[(size_t)wrow * Kd + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < F_BK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[k][ty * 4 + i];
      if (GATED) {
        b[0] = Bs[k][tx * 2]; b[1] = Bs[k][tx * 2 + 1];
        b[2] = Bs[k][F_BN / 2 + tx * 2]; b[3] = Bs[k][F_BN / 2 + tx * 2 + 1];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = Bs[k][tx * 4 + j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gr = m0 + ty * 4 + i;
    if (gr >= rows) continue;
    if (GATED) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int gc = n0 + tx * 2 + j;
        if (gc < Nout) C[(size_t)gr * Nout + gc] = silu(acc[i][j]) * acc[i][j + 2];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int gc = n0 + tx * 4 + j;
        if (gc < Nout) C[(size_t)gr * Nout + gc] = acc[i][j];
      }
    }
  }
}

// Tile shapes chosen from the expected rows per local expert, T*K/E, for each GEMM. The
// gate/up GEMM reduces over h (long) and takes 256-row tiles from ~100 rows per expert on;
// the down GEMM reduces over I (often short), where per-tile overhead and the rows a
// 256-row tile wastes on small experts weigh more, so it switches later (measured on the
// DeepSeek-V3 share: gate/up 519 -> 424 us with 256-row tiles, down 249 -> 315 us).
enum class Tiles { Large, Medium, Small };

Tiles tile_kind(const Dims& d, bool gate_up) {
  const double per_expert = d.E > 0 ? (double)d.T * d.K / d.E : 0.0;
  const double large = gate_up ? 96 : 384;
  return per_expert >= large ? Tiles::Large : (per_expert >= 48 ? Tiles::Medium : Tiles::Small);
}

struct Tiling {
  int BM, tall_extra, tall_split;   // tall: 32 rows per wave row; halves when WM = 2
};
Tiling tiling(Tiles k) {
  switch (k) {
    case Tiles::Large: return {256, 0, 1};   // its tall parts would cost as much as tiles
    case Tiles::Medium: return {128, 64, 2};
    default: return {32, 32, 1};
  }
}

template <int BM, int BN, int WM, int WN, bool TALL>
bool launch_bf16_gemm(bool gated, const FfnSched* sc, int h, int64_t ub, int cpx, float* part,
                      int* arrive, hipStream_t st) {
  constexpr int NT = 64 * WM * WN;
  if (ub <= 0) return true;
  // per XCD: its share of the tiles plus room for one round of k-slices
  const int64_t g = ((ub + kNumXcd - 1) / kNumXcd + cpx) * kNumXcd;
  if (gated)
    hipLaunchKernelGGL((ffn_gate_up_bf16<BM, BN, WM, WN, TALL>), dim3((unsigned)g), dim3(NT), 0,
                       st, sc, h, part, arrive);
  else
    hipLaunchKernelGGL((ffn_down_bf16<BM, BN, WM, WN, TALL>), dim3((unsigned)g), dim3(NT), 0,
                       st, sc, h, part, arrive);
  return hipGetLastError() == hipSuccess;
}

bool launch_bf16(Tiles k, bool gated, const FfnSched* sc, int h, int64_t ub, int cpx,
                 float* part, int* arrive, hipStream_t st) {
  switch (k) {
    case Tiles::Large:
      return launch_bf16_gemm<256, 256, 2, 2, false>(gated, sc, h, ub, cpx, part, arrive, st);
    case Tiles::Medium:
      return launch_bf16_gemm<128, 256, 2, 2, true>(gated, sc, h, ub, cpx, part, arrive, st);
    default:
      return launch_bf16_gemm<32, 256, 1, 4, true>(gated, sc, h, ub, cpx, part, arrive, st);
  }
}

}  // namespace

size_t ffn_sched_bytes(const Dims&) { return sizeof(FfnSched); }

size_t ffn_arrive_bytes(const Dims&) { return 2 * kArriveSlots * sizeof(int); }

size_t ffn_splitk_bytes(const Dims& d) {
  if (!d.bf16) return 0;
  size_t tile = 0;
  for (int gu = 0; gu < 2; ++gu) {
    const Tiles k = tile_kind(d, gu == 1);
    const size_t t = k == Tiles::Large ? 256 * 256 : (k == Tiles::Medium ? 128 * 256 : 32 * 256);
    tile = t > tile ? t : tile;
  }
  return (size_t)kNumXcd * kCuPerXcdMax * tile * 4;
}

int launch_ffn(const moe_problem* p, const Dims& d, const void* xp, const int32_t* offsets,
               const void* w13, const void* w2, const void* x, const void* w13_sh,
               const void* w2_sh, void* yp, void* y_sh, char* ws, const WsLayout& L,
               hipStream_t st, hipEvent_t const* ev, const int32_t* gather_rows) {
  FfnSched* sc = reinterpret_cast<FfnSched*>(ws + L.sched);
  float* part = reinterpret_cast<float*>(ws + L.splitk);
  int* arrive = reinterpret_cast<int*>(ws + L.arrive);
  const int has_sh = (p->n_shared && d.sh_rows > 0) ? 1 : 0;
  const int64_t sh_t0 = (int64_t)d.rank * d.tpr;
  Tiles k1 = Tiles::Large, k2 = Tiles::Large;
  Tiling t1{F_BM, 0, 1}, t2{F_BM, 0, 1};
  int BN1 = F_BN / 2, BN2 = F_BN, split_max = 1;
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return MOE_ERR_LAUNCH;
  const int cpx = n_cu / kNumXcd < 1 ? 1 : (n_cu / kNumXcd > kCuPerXcdMax ? kCuPerXcdMax
                                                                         : n_cu / kNumXcd);
  if (d.bf16) {
    k1 = tile_kind(d, true);
    k2 = tile_kind(d, false);
    t1 = tiling(k1);
    t2 = tiling(k2);
    int min_k = d.h < p->inter ? d.h : p->inter;
    if (has_sh && p->shared_inter < min_k) min_k = p->shared_inter;
    split_max = min_k / 64 < kMaxSplit ? min_k / 64 : kMaxSplit;
    BN1 = 128;   // output columns of the gated tile (256 B rows: 128 gate + 128 up)
    BN2 = 256;
  }
  hipLaunchKernelGGL(ffn_prep, dim3(1), dim3(1024), 0, st, sc, offsets,
                     static_cast<const char*>(xp), static_cast<const char*>(w13),
                     static_cast<const char*>(w2), static_cast<const char*>(x),
                     static_cast<const char*>(w13_sh), static_cast<const char*>(w2_sh),
                     ws + L.hbuf, static_cast<char*>(yp), static_cast<char*>(y_sh), d.El, has_sh,
                     d.sh_rows, sh_t0, d.h, p->inter, p->shared_inter, d.R_max, d.s, t1.BM,
                     t2.BM, t1.tall_extra, t2.tall_extra, t1.tall_split, t2.tall_split, BN1, BN2,
                     cpx, split_max, arrive, gather_rows, d.K, d.T);
  if (hipGetLastError() != hipSuccess) return MOE_ERR_LAUNCH;
  if (ev && hipEventRecord(ev[0], st) != hipSuccess) return MOE_ERR_LAUNCH;
  // Upper bound on m-tiles: sum_e ceil(rows_e / BM) <= R_max / BM + E_l (an expert with a
  // tall last tile has mt - 1 + tall_split <= ceil(rows_e / BM) tiles per n-tile).
  auto m_ub = [&](int BM) { return d.R_max / BM + d.El; };
  auto m_sh = [&](int BM) { return has_sh ? (d.sh_rows + BM - 1) / BM : (int64_t)0; };
  const int64_t nt1 = (p->inter + BN1 - 1) / BN1;
  const int64_t nt1s = has_sh ? (p->shared_inter + BN1 - 1) / BN1 : 0;
  const int64_t nt2 = (d.h + BN2 - 1) / BN2;
  const int64_t ub1 = m_ub(t1.BM) * nt1 + m_sh(t1.BM) * nt1s;
  const int64_t ub2 = (m_ub(t2.BM) + m_sh(t2.BM)) * nt2;
  bool ok = true;
  if (d.bf16) {
    ok = launch_bf16(k1, true, sc, d.h, ub1, cpx, part, arrive, st);
    if (ok && ev) ok = hipEventRecord(ev[1], st) == hipSuccess;
    if (ok) ok = launch_bf16(k2, false, sc, d.h, ub2, cpx, part, arrive, st);
  } else {
    const int64_t g1 = (ub1 + kNumXcd - 1) / kNumXcd * kNumXcd;
    const int64_t g2 = (ub2 + kNumXcd - 1) / kNumXcd * kNumXcd;
    if (g1 > 0)
      hipLaunchKernelGGL(ffn_gemm_f32<true>, dim3((unsigned)g1), dim3(256), 0, st, sc, d.h);
    if (ev && hipEventRecord(ev[1], st) != hipSuccess) return MOE_ERR_LAUNCH;
    if (g2 > 0)
      hipLaunchKernelGGL(ffn_gemm_f32<false>, dim3((unsigned)g2), dim3(256), 0, st, sc, d.h);
    ok = hipGetLastError() == hipSuccess;
  }
  if (ok && ev) ok = hipEventRecord(ev[2], st) == hipSuccess;
  return ok ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // namespace moe
