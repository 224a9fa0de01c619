// Expert FFN as two grouped GEMMs over the ragged per-expert row blocks:
//   GEMM1 (gated):  H[r] = silu(A[r] W_g^T) * (A[r] W_u^T)      -> hbuf (act dtype)
//   GEMM2 (down):   Y[r] = H[r] W_d^T                             -> yp / y_sh
// Groups are the local experts (rows from `offsets`, read on the device) plus the
// optional shared expert over this rank's token block. The offsets become a tile table
// (built by dispatch, or by a one-block prep kernel); every GEMM block finds its (group,
// n-tile, m-tile) by binary search, so the host never waits for the routing result.
//
// bf16 path: 256 threads (4 waves), MFMA 32x32x16 bf16 with fp32 accumulators; operand
// tiles stream by buffer->LDS DMA into 64-deep stages of XOR-swizzled 128-byte rows
// (two activation and three weight stages for 256-row tiles, three for 128-row and four
// for 32-row tiles); an LDS-staged epilogue writes 16-byte coalesced rows; an
// XCD-aware block order keeps consecutive tiles of one expert on one XCD's L2. Tile shapes
// (256, 128 or 32 rows by 256 weight rows) are chosen per GEMM from the rows per expert;
// with 128- and 32-row tiles a short remainder rides on an expert's last tile (tall
// tiles), with 256-row tiles a 65..192-row remainder gets a short last tile; an XCD's
// last, partial round of tiles is split along K (fp32 partials, summed in slice order by
// the last slice to arrive). Without xp the gate/up GEMM reads its A rows straight from x
// through the row -> token map.
//
// Packed bf16 weights (MOE_DTYPE_BF16_PACKED): the same tiles with the weights stored in
// MFMA-fragment order, loaded straight into registers; only the token rows go through LDS
// (see its section below).
//
// MX-FP8 path: the same tiles and pipeline on scaled FP8 MFMAs (see its section below).
#include "ffn_sched.h"
#include "mxfp8.h"

namespace moe {
namespace {

// One block of 1024 threads: the tile table from the offsets in device memory.
__global__ __launch_bounds__(1024) void ffn_prep(FfnPrepArgs a,
                                                 const int32_t* __restrict__ offsets) {
  __shared__ int wsum[16];
  ffn_build_sched<1024>(a, offsets, wsum);
}

// One block of 1024 threads: the XCD split by work of the table built before.
__global__ __launch_bounds__(1024) void ffn_split(FfnPrepArgs a) {
  __shared__ int wsum[16];
  ffn_split_by_work<1024>(a, wsum);
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
  const int* xb = sc->xb[first ? 0 : 1];
  XcdPlan q;
  q.base = xb[xcd];
  q.cnt = xb[xcd + 1] - xb[xcd];
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
    if (sc->tall_split[gi] == 0 && t.m_tile == mt - 1) {
      // short last m-tile: a remainder of up to 192 rows rounded up to 64, 128 or 192 rows
      // (64 only on packed weights: with both operands in LDS a 64-row tile writes as many
      // weight bytes to LDS per k-step as a full one and was measured no faster)
      const int rem = sc->g[lo].rows - t.m_tile * sc->bm[gi];
      const int q64 = (rem + 63) >> 6;
      t.tall = q64 >= sc->short_min[gi] && q64 <= 3 && rem < sc->bm[gi] ? q64 : 0;
    }
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
  // tall parts are not split (slice 0 takes all of K); short last tiles are
  if (t.tall && t.nslice > 1 && sc->tall_split[first ? 0 : 1] != 0) {
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

// The row -> token map read as global memory (global_load rather than flat loads, which
// would also count against the LDS wait counter).
typedef const __attribute__((address_space(1))) int32_t global_i32;
__device__ __forceinline__ global_i32* as_global(const int32_t* p) { return (global_i32*)p; }

// Slot of a 16-byte chunk in a 128-byte LDS row: chunk c of row r sits at
// c ^ row_swz(r). Any 8 aligned consecutive rows (one 128-byte bank sweep) and any 16
// aligned consecutive rows (one 256-byte sweep) then hold a given chunk in distinct
// slots, so ds_read_b128 fragment reads (lanes = consecutive rows, same chunk) are free
// of bank conflicts whether the LDS serves 8 or 16 lanes per cycle.
__device__ __forceinline__ int row_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

constexpr int kDmaStride = 2;   // MFMAs per interleaved DMA instruction (MX-FP8, bf16 gate/up)
// The bf16 down GEMM spreads its DMA wider: its weights stream from HBM once per four
// m-tiles, and every third MFMA measured 6% faster than every second at the Mixtral shape.
constexpr int kDmaStrideDown = 3;

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

// The end of a tile, once every wave is past its last operand read: the whole tile goes
// through store_tile; a k-slice of a split tile stores its fp32 partial sums (fragment
// order, so each store is 1 KB contiguous) and counts itself in, and the last slice to
// arrive adds all of them in slice order (the same order whichever arrives last) and
// stores the tile.
template <int BM, int BN, int WM, int WN, bool GATED>
__device__ __forceinline__ void finish_tile(const floatx16 (&acc)[BM / WM / 32][BN / WN / 32],
                                            const FfnGroup& fg, int m0, int n0, int h,
                                            uint4* __restrict__ smem, int slice, int nslice,
                                            float* __restrict__ part, size_t pstride,
                                            int* __restrict__ arrive) {
  constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (part) {
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

// bf16 grouped GEMM. Block tile BM x BN (BN counts weight rows: for GATED half gate,
// half up), k-step 64, WM x WN waves (4 or 8), each wave (BM/WM) x (BN/WN) as 32x32
// MFMA tiles. With 8 waves two share each SIMD, so one wave's MFMAs keep the matrix
// core busy while the other waits to issue its memory instructions. Operand tiles stream
// into NS LDS stages by buffer->LDS DMA (no register staging), up to NS - 1 k-steps ahead
// of the MFMAs; with NB = 3 the weights take three stages and the activations two, so the
// weights are fetched two k-steps ahead and the activations one. Every DMA request covers
// whole 128-byte row segments (half-line requests roughly halve what L2 can deliver per
// CU). The MFMA takes
// the weight fragment first, so a lane's accumulators hold 4 consecutive output columns.
// VARIANT only tells apart instantiations that are otherwise identical but reached from
// different tile kinds (an expert's short last tile in the 256-row kernels and the 128-row
// kernels' full tile): the host compilation pass rejects a second use of the same
// specialisation of this body from another kernel.
template <int BM, int BN, int WM, int WN, bool GATED, bool GATHER = false, int NS = 2,
          int VARIANT = 0, int NB = NS>
__device__ __forceinline__ void gemm_bf16_body(const FfnGroup& fg, int m0, int n0, int h,
                                               uint4* __restrict__ smem, int slice,
                                               int nslice, float* __restrict__ part,
                                               size_t pstride, int* __restrict__ arrive) {
  constexpr int NW = WM * WN;
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  static_assert(TM >= 1 && TN >= 1, "tile");
  static_assert(!GATED || TN % 2 == 0, "gated needs gate/up pairs");
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "DMA rows split evenly over waves");
  constexpr int AI = BM / (8 * NW), BI = BN / (8 * NW);  // DMA instructions per wave per stage
  constexpr int LPS = AI + BI;
  constexpr int A_ST = BM * 8, B_ST = BN * 8;       // uint4 per stage
  constexpr int NMF = TM * TN;                      // MFMAs per k16 phase
  static_assert(NS >= 2 && NS <= 4 && LPS * (NS - 2) < 64, "LDS stages");
  static_assert(NB == NS || (NS == 2 && NB == 3), "B stages: as A, or 3 with 2 A stages");
  uint4* As = smem;                                 // [NS][BM rows][8 chunks]
  uint4* Bs = smem + NS * A_ST;                     // [NS][BN rows][8 chunks]

  const int rows = fg.rows, I = fg.inter;
  const bf16_t* A = static_cast<const bf16_t*>(GATED ? fg.A1 : fg.C1);
  const bf16_t* B = static_cast<const bf16_t*>(GATED ? fg.B1 : fg.B2);
  const int Kd = GATED ? h : I;         // reduction length = lda = ldb
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
    const global_i32* gidx = as_global(fg.gidx);
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
    if (NB != NS && x >= AI) stage = step % NB;
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
  auto read_frags = [&](int set, int stage, int kk, int bstage) __attribute__((always_inline)) {
    const uint4* as = As + stage * A_ST;
    const uint4* bs = Bs + bstage * B_ST;
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
  // dma: A of next_step (and, with NB == NS, its B); dmab: B of bnext (NB != NS only)
  // Early barrier (the gate/up GEMM with three weight stages): every A instruction of a
  // k-step is issued before its last phase, so the wait for the next k-step's operands and
  // the workgroup barrier sit after that phase's first MFMA, and the next k-step's first
  // fragments are read under the phase's other MFMAs rather than after the k-step. The
  // barrier also orders every wave's reads of the current stages before the DMA that
  // refills them (issued from the next k-step on), so the k-steps need no other barrier.
  // The weight instructions of kt + 2 issued before the barrier (NBB) may stay in flight.
  constexpr int DS = GATED ? kDmaStride : kDmaStrideDown;
  constexpr bool EB = GATED && NS == 2 && NB == 3 && (AI - 1) * DS + 1 <= 3 * NMF;
  constexpr int NBB_RAW = (3 * NMF - 1) / DS + 1 - AI;
  constexpr int NBB = NBB_RAW < 0 ? 0 : (NBB_RAW > BI ? BI : NBB_RAW);
  auto kstep = [&](int stage, bool dma, int next_step, int dma_stage, int bstage, bool dmab,
                   int bnext, bool eb = false, int nstage = 0, int nbstage = 0)
                   __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int cur = kk & 1;
#pragma unroll
      for (int t = 0; t < NMF; ++t) {
        acc[t / TN][t % TN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            fb[cur][t % TN], fa[cur][t / TN], acc[t / TN][t % TN], 0, 0, 0);
        const int slot = kk * NMF + t;            // MFMA index within the k-step
        if (slot >= 1 && (slot - 1) % DS == 0 && (slot - 1) / DS < LPS) {
          const int xx = (slot - 1) / DS;
          if (NB == NS || xx < AI) {
            if (dma) issue_one(next_step, dma_stage, xx);
          } else if (dmab) {
            issue_one(bnext, 0, xx);
          }
        }
        if (t == 0 && kk < 3) {
          __builtin_amdgcn_sched_barrier(0);
          read_frags(cur ^ 1, stage, kk + 1, bstage);
        }
        if constexpr (EB) {
          if (t == 0 && kk == 3 && eb) {
            __builtin_amdgcn_sched_barrier(0);
            // this wave's reads of the current stages have returned (lgkmcnt(0)), and its
            // DMA of the next k-step's operands has landed
            __builtin_amdgcn_s_waitcnt(0xC07F);
            if (dmab) wait_vmcnt<NBB>();
            else wait_vmcnt<0>();
            lds_barrier();
            read_frags(0, nstage, 0, nbstage);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // instructions left over when the k-step has too few MFMAs
#pragma unroll
    for (int x = (4 * NMF - 2) / DS + 1; x < LPS; ++x) {
      if (NB == NS || x < AI) {
        if (dma) issue_one(next_step, dma_stage, x);
      } else if (dmab) {
        issue_one(bnext, 0, x);
      }
    }
  };

  if constexpr (NB != NS) {
    // two A stages, three B stages: during k-step kt the DMA fetches A of kt + 1 and B of
    // kt + 2 (A instructions first), so the weights have two k-steps of lead time
    if (nk > 0) {
#pragma unroll
      for (int x = 0; x < LPS; ++x) issue_one(0, 0, x);             // A0, B0
      if (nk > 1) {
#pragma unroll
        for (int x = AI; x < LPS; ++x) issue_one(1, 0, x);          // B1
        wait_vmcnt<BI>();
      } else {
        wait_vmcnt<0>();
      }
      lds_barrier();
      read_frags(0, 0, 0, 0);
      int kt = 0;
      for (; kt + 2 < nk; ++kt) {   // A of kt + 1, B of kt + 2
        if constexpr (EB) {
          kstep(kt % NS, true, kt + 1, (kt + 1) % NS, kt % NB, true, kt + 2, true,
                (kt + 1) % NS, (kt + 1) % NB);
        } else {
          kstep(kt % NS, true, kt + 1, (kt + 1) % NS, kt % NB, true, kt + 2);
          wait_vmcnt<BI>();
          lds_barrier();
          read_frags(0, (kt + 1) % NS, 0, (kt + 1) % NB);
        }
      }
      if (kt + 1 < nk) {            // A of the last k-step
        if constexpr (EB) {
          kstep(kt % NS, true, kt + 1, (kt + 1) % NS, kt % NB, false, 0, true, (kt + 1) % NS,
                (kt + 1) % NB);
        } else {
          kstep(kt % NS, true, kt + 1, (kt + 1) % NS, kt % NB, false, 0);
          wait_vmcnt<0>();
          lds_barrier();
          read_frags(0, (kt + 1) % NS, 0, (kt + 1) % NB);
        }
        ++kt;
      }
      kstep(kt % NS, false, 0, 0, kt % NB, false, 0);
    }
  } else {
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
  read_frags(0, 0, 0, 0);
  int kt = 0;
  for (; kt + NS - 1 < nk; ++kt) {
    // the DMA of k-step kt + NS - 1 refills the stage k-step kt - 1 used: every wave
    // passed the barrier after its last reads there
    kstep(kt % NS, true, kt + NS - 1, (kt + NS - 1) % NS, kt % NS, true, kt + NS - 1);
    // k-step kt+1 has landed (this wave's DMA; the NS - 2 after it may still be in
    // flight) and every wave is past its reads of stage kt % NS; the barrier publishes
    // the DMA of all waves
    wait_vmcnt<LPS * (NS - 2)>();
    lds_barrier();
    read_frags(0, (kt + 1) % NS, 0, (kt + 1) % NS);
  }
  for (; kt + 1 < nk; ++kt) {   // the last NS - 2 k-steps: nothing left to fetch
    kstep(kt % NS, false, 0, 0, kt % NS, false, 0);
    const int after = nk - kt - 2;   // k-steps still in flight behind k-step kt+1
    if (NS > 3 && after >= 2) wait_vmcnt<LPS * (NS > 3 ? 2 : 0)>();
    else if (NS > 2 && after >= 1) wait_vmcnt<LPS * (NS > 2 ? 1 : 0)>();
    else wait_vmcnt<0>();
    lds_barrier();
    read_frags(0, (kt + 1) % NS, 0, (kt + 1) % NS);
  }
  kstep((nk - 1) % NS, false, 0, 0, (nk - 1) % NS, false, 0);
  }
  }
  __syncthreads();
  finish_tile<BM, BN, WM, WN, GATED>(acc, fg, m0, n0, h, smem, slice, nslice, part, pstride,
                                     arrive);
}

// ---- bf16 grouped GEMM on packed weights ---------------------------------------------
// Weights in MFMA-fragment order (moe_pack_weights): 32 weight rows by 16 k values form one
// 1 KB block in which lane l's 16 bytes are row l % 32, k 8*(l/32) .. +7, exactly the
// weight operand of one 32x32x16 MFMA. A wave loads its weight fragments straight into
// registers, one coalesced 1 KB load each, NS - 1 k-steps ahead into a ring of NS
// k-steps; only the activation tile goes through LDS (buffer->LDS DMA into NS stages,
// NS - 1 k-steps ahead). Measured on gfx950: a k-step's LDS writes cost more than its
// reads, and writing the weight tile to LDS (by DMA or by ds_write) was a quarter of the
// 256-row GEMM's time. The waves sit side by side (WM = 1): each streams its own weight
// columns, none twice. The workgroup barrier of a k-step follows the first MFMA of its
// last phase (the wait there is for the next k-step's activations), and the next
// k-step's first fragments are read under the rest of that phase.
template <int V>
struct IC {
  static constexpr int value = V;
};

template <int BM, int BN, int WM, int WN, bool GATED, bool GATHER, int NS, int VARIANT = 0>
__device__ __forceinline__ void gemm_pk_body(const FfnGroup& fg, int m0, int n0, int h,
                                             uint4* __restrict__ smem, int slice, int nslice,
                                             float* __restrict__ part, size_t pstride,
                                             int* __restrict__ arrive) {
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  static_assert(TM >= 1 && TN >= 1, "tile");
  static_assert(!GATED || TN % 2 == 0, "gated needs gate/up pairs");
  static_assert(BM % (8 * NW) == 0, "DMA rows split evenly over waves");
  constexpr int AI = BM / (8 * NW);     // activation DMA instructions per wave per k-step
  constexpr int LB = 4 * TN;            // weight loads per wave per k-step
  constexpr int LPS = AI + LB;          // a k-step's group of instructions
  constexpr int A_ST = BM * 8;          // uint4 per stage
  constexpr int NMF = TM * TN;          // MFMAs per k16 phase
  constexpr int DS = kDmaStride;
  constexpr int EBS = 3 * NMF;          // the barrier follows MFMA EBS (first of phase 3)
  static_assert(NS >= 3 && NS <= 4, "stages");
  // Issue order of the group of k-step kt + NS - 1 during k-step kt: weight loads from
  // the first MFMA on, one every DS MFMAs; the activation DMA only after the barrier
  // (into the stage k-step kt - 1 used, whose reads every wave has consumed by then);
  // weight loads that did not fit before the barrier after the DMA. At the barrier of
  // k-step kt the activations of kt + 1 (issued during k-step kt + 2 - NS, after its
  // barrier) have landed once all but the instructions issued after them are done:
  // that group's remaining weights, the NS - 3 whole groups after it and this k-step's
  // weights so far, LB + (NS - 3) * LPS in all.
  constexpr int WB_RAW = (EBS - 1) / DS + 1;        // weight loads up to the barrier
  constexpr int WB = WB_RAW > LB ? LB : WB_RAW;
  constexpr int A_SLOTS = (4 * NMF - 1 - EBS - 1) / DS + 1;   // DMA slots after it
  constexpr int AB = A_SLOTS > AI ? AI : (A_SLOTS < 0 ? 0 : A_SLOTS);
  constexpr int N_EB = LB + (NS - 3) * LPS;
  static_assert(N_EB < 64, "vmcnt range");
  uint4* As = smem;                     // [NS][BM rows][8 chunks]

  const int rows = fg.rows, I = fg.inter;
  const bf16_t* A = static_cast<const bf16_t*>(GATED ? fg.A1 : fg.C1);
  const bf16_t* B = static_cast<const bf16_t*>(GATED ? fg.B1 : fg.B2);
  const int Kd = GATED ? h : I;
  const uint32_t b_rows = GATED ? 2 * I : h;
  const uint32_t a_bytes = (uint32_t)(GATHER ? fg.arows : rows) * Kd * 2;
  const __amdgpu_buffer_rsrc_t ra_rs = make_rsrc(A, a_bytes);
  const __amdgpu_buffer_rsrc_t rb_rs = make_rsrc(B, b_rows * (uint32_t)Kd * 2);
  const __amdgpu_buffer_rsrc_t rz_rs = make_rsrc(A, 0);   // every load reads zero

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // activation DMA: as in gemm_bf16_body
  const int dr = lane >> 3;
  const int dc = (lane & 7) ^ dr ^ (wave & 1);
  const uint32_t a_lane = ((uint32_t)(m0 + 8 * wave + dr) * Kd + dc * 8) * 2;
  const uint32_t x_stride = (uint32_t)(8 * NW) * Kd * 2;
  uint32_t a_off[GATHER ? AI : 1];
  if constexpr (GATHER) {
    const global_i32* gidx = as_global(fg.gidx);
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
  // Weight col-tile j of this wave: 32 weight rows from wr (a multiple of 32), so its
  // fragment for k16 chunk c sits at byte wr*Kd*2 + c*1024 + lane*16 of the packed
  // matrix. Gated: gate col-tiles first, then the up rows of the same output columns.
  // Rows past the matrix read as zero; gate rows past I read up rows, which only feed
  // output columns past I that are never stored.
  uint32_t b_off[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    int wr;
    if (GATED)
      wr = j < TN / 2 ? n0 + wn * (WTN / 2) + j * 32 : I + n0 + wn * (WTN / 2) + (j - TN / 2) * 32;
    else
      wr = n0 + wn * WTN + j * 32;
    b_off[j] = ((uint32_t)wr * Kd + lane * 8) * 2;
  }

  const int kb = __builtin_amdgcn_readfirstlane(slice * (Kd / 64) / nslice);
  const int nk = __builtin_amdgcn_readfirstlane((slice + 1) * (Kd / 64) / nslice) - kb;
  // k-steps rounded up to whole rounds of NS: the ones past nk load zeros (activations
  // and weights alike) and add exactly nothing, so the k-loop has no exit inside a round
  const int nkp = (nk + NS - 1) / NS * NS;

  floatx16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  int arow[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) arow[i] = wm * WTM + i * 32 + (lane & 31);
  // Activation fragments: one per row-tile, each replaced by the next phase's as soon as
  // the phase's last MFMA on it is issued (a phase of MFMAs ahead of its use).
  bf16x8_t fa[TM];
  bf16x8_t fw[NS][4][TN];   // weight fragments of NS k-steps: [ring slot][k16 phase][col-tile]
  auto read_a = [&](int i, int stage, int kk) __attribute__((always_inline)) {
    const uint4* as = As + stage * A_ST;
    const int c = kk * 2 + (lane >> 5);
    fa[i] = __builtin_bit_cast(bf16x8_t, as[arow[i] * 8 + (c ^ row_swz(arow[i]))]);
  };
  // The group of k-step `step` (stage and ring slot `slot` = step % NS): activation DMA
  // instruction x, weight load y. k-steps past nk read zeros.
  auto issue_a = [&](int step, int slot, int x) __attribute__((always_inline)) {
    const uint32_t soff = (uint32_t)(kb + step) * 128;
    const __amdgpu_buffer_rsrc_t rs = step < nk ? ra_rs : rz_rs;
    if constexpr (GATHER)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, LDS_PTR(As + slot * A_ST + 64 * (NW * x + wave)), 16, a_off[x], soff, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, LDS_PTR(As + slot * A_ST + 64 * (NW * x + wave)), 16, a_lane, soff + x * x_stride,
          0, 0);
  };
  auto issue_w = [&](int step, int slot, int y) __attribute__((always_inline)) {
    const int kk = y / TN, j = y % TN;
    const uint32_t soff = (uint32_t)(4 * (kb + step) + kk) * 1024;
    fw[slot][kk][j] = __builtin_bit_cast(
        bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(step < nk ? rb_rs : rz_rs, b_off[j],
                                                        soff, 0));
  };

  // k-step kt (kt % NS == P): four k16 phases of NMF MFMAs, and the group of k-step
  // kt + NS - 1. Every k-step issues a whole group, so the issue points and the counts
  // the waits use are fixed and the MFMAs stay one straight run of code.
  auto step = [&](auto PC, int kt) __attribute__((always_inline)) {
    constexpr int P = decltype(PC)::value;
    constexpr int NX = (P + 1) % NS;          // stage of kt + 1
    constexpr int FS = (P + NS - 1) % NS;     // stage and ring slot of kt + NS - 1
    const int ft = kt + NS - 1;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int t = 0; t < NMF; ++t) {
        const int i = t / TN, j = t % TN;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[P][kk][j], fa[i], acc[i][j], 0,
                                                            0, 0);
        const int slot = kk * NMF + t;
        if (slot >= 1 && slot <= EBS && (slot - 1) % DS == 0 && (slot - 1) / DS < WB)
          issue_w(ft, FS, (slot - 1) / DS);
        if (slot == EBS) {
          __builtin_amdgcn_sched_barrier(0);
          // the next k-step's activations have landed, here and (barrier) in every wave
          // (after the last k-step this reads a stage nothing uses, which is harmless)
          wait_vmcnt<N_EB>();
          lds_barrier();
        }
        if (slot > EBS && (slot - EBS - 1) % DS == 0 && (slot - EBS - 1) / DS < AB)
          issue_a(ft, FS, (slot - EBS - 1) / DS);
        if (j == TN - 1) {   // last MFMA on fa[i] in this phase
          __builtin_amdgcn_sched_barrier(0);
          if (kk < 3) read_a(i, P, kk + 1);
          else read_a(i, NX, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int x = AB; x < AI; ++x) issue_a(ft, FS, x);
#pragma unroll
    for (int y = WB; y < LB; ++y) issue_w(ft, FS, y);
  };

  if (nk > 0) {
    // groups of k-steps 0 .. NS - 2, then wait for k-step 0's activations
    // the groups of k-steps 0 .. NS - 2, each in the order a k-step issues one (weights
    // up to the barrier, activations, the other weights), so the counts above hold
#pragma unroll
    for (int s0 = 0; s0 < NS - 1; ++s0) {
#pragma unroll
      for (int y = 0; y < WB; ++y) issue_w(s0, s0, y);
#pragma unroll
      for (int x = 0; x < AI; ++x) issue_a(s0, s0, x);
#pragma unroll
      for (int y = WB; y < LB; ++y) issue_w(s0, s0, y);
    }
    wait_vmcnt<(LB - WB) + (NS - 2) * LPS>();   // k-step 0's activations
    lds_barrier();
#pragma unroll
    for (int i = 0; i < TM; ++i) read_a(i, 0, 0);
    for (int kt = 0; kt < nkp; kt += NS) {
      step(IC<0>{}, kt);
      step(IC<1>{}, kt + 1);
      if constexpr (NS > 2) step(IC<2>{}, kt + 2);
      if constexpr (NS > 3) step(IC<3>{}, kt + 3);
    }
    wait_vmcnt<0>();   // the zero groups past the end land before the LDS is reused
  }
  __syncthreads();
  finish_tile<BM, BN, WM, WN, GATED>(acc, fg, m0, n0, h, smem, slice, nslice, part, pstride,
                                     arrive);
}

template <int BM, int BN, bool GATED, int NS = 2, int NB = NS>
constexpr size_t bf16_lds_bytes() {
  constexpr size_t ops = (NS * (size_t)BM + NB * (size_t)BN) * 8 * 16;
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

// An expert's short last m-tile in a 256-row-tile GEMM: 64 * q rows (q = 2, 3) by BN, or
// one k-slice of it (the partial sums use a prefix of the tile's slot). The 128-row body
// gets a third stage (it streams more bytes per MFMA).
template <int BN, int WM, int WN, bool GATED, bool GATHER>
__device__ __forceinline__ void bf16_short(int q, const FfnGroup& fg, int m0, int n0, int h,
                                           uint4* __restrict__ smem, int slice, int nslice,
                                           float* part, size_t pstride, int* arrive) {
  if (q == 2)
    gemm_bf16_body<128, BN, WM, WN, GATED, GATHER, 3, 1>(fg, m0, n0, h, smem, slice, nslice,
                                                         part, pstride, arrive);
  else
    gemm_bf16_body<192, BN, WM, WN, GATED, GATHER, 2>(fg, m0, n0, h, smem, slice, nslice, part,
                                                      pstride, arrive);
}

template <int BM, int BN, int WM, int WN, bool GATED, bool TALL, bool DEEP = false>
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
  if constexpr (!TALL) {
    if (t.tall) {   // an expert's short last m-tile (128 or 192 rows)
      if (GATED && fg.gidx)
        bf16_short<BN, WM, WN, GATED, GATED>(t.tall, fg, m0, n0, h, smem, t.slice, t.nslice, pt,
                                             ps, ar);
      else
        bf16_short<BN, WM, WN, GATED, false>(t.tall, fg, m0, n0, h, smem, t.slice, t.nslice, pt,
                                             ps, ar);
      return;
    }
  }
  if constexpr (TALL) {
    if (t.tall) {   // part of an expert's tall last tile: all of K
      if (GATED && fg.gidx)   // gate/up reading x through the row -> token map
        gemm_bf16_body<BMT, BNT, WM, WN, GATED, GATED, NS>(fg, m0, n0t, h, smem, 0, 1, nullptr,
                                                           0, nullptr);
      else
        gemm_bf16_body<BMT, BNT, WM, WN, GATED, false, NS>(fg, m0, n0t, h, smem, 0, 1, nullptr,
                                                           0, nullptr);
      return;
    }
  }
  constexpr int NB = DEEP ? 3 : NS;   // three weight stages (two-ahead weight prefetch)
  if (GATED && fg.gidx)
    gemm_bf16_body<BM, BN, WM, WN, GATED, GATED, NS, 0, NB>(fg, m0, n0, h, smem, t.slice,
                                                            t.nslice, pt, ps, ar);
  else
    gemm_bf16_body<BM, BN, WM, WN, GATED, false, NS, 0, NB>(fg, m0, n0, h, smem, t.slice,
                                                            t.nslice, pt, ps, ar);
}

template <int BM, int BN, int WM, int WN, bool GATED, bool TALL, bool DEEP = false>
constexpr size_t tile_lds_bytes() {
  constexpr int NS = kernel_stages<BM>();
  return TALL ? cmax<bf16_lds_bytes<BM, BN, GATED, NS>(),
                     bf16_lds_bytes<BM + 32 * WM, BN / tall_split<WM, WN>(), GATED, NS>()>()
              : cmax<bf16_lds_bytes<BM, BN, GATED, NS, DEEP ? 3 : NS>(),
                     cmax<bf16_lds_bytes<128, BN, GATED, 3>(),
                          bf16_lds_bytes<192, BN, GATED, 2>()>()>();
}

template <int BM, int BN, int WM, int WN, bool TALL, bool DEEP = false>
__global__ __launch_bounds__(64 * WM * WN) void ffn_gate_up_bf16(const FfnSched* __restrict__ sc,
                                                                 int h, float* part,
                                                                 int* arrive) {
  __shared__ uint4 smem[tile_lds_bytes<BM, BN, WM, WN, true, TALL, DEEP>() / 16];
  gemm_bf16_tile<BM, BN, WM, WN, true, TALL, DEEP>(sc, h, part, arrive, smem);
}
template <int BM, int BN, int WM, int WN, bool TALL, bool DEEP = false>
__global__ __launch_bounds__(64 * WM * WN) void ffn_down_bf16(const FfnSched* __restrict__ sc,
                                                              int h, float* part,
                                                              int* arrive) {
  __shared__ uint4 smem[tile_lds_bytes<BM, BN, WM, WN, false, TALL, DEEP>() / 16];
  gemm_bf16_tile<BM, BN, WM, WN, false, TALL, DEEP>(sc, h, part, arrive, smem);
}

template <int BM, int BN, bool GATED, int NS>
constexpr size_t pk_lds_bytes() {
  constexpr size_t ops = (size_t)NS * BM * 8 * 16;
  constexpr size_t stg = (size_t)BM * ((GATED ? BN / 2 : BN) * 2 + 16);
  return ops > stg ? ops : stg;
}

// Activation stages on packed weights: the LDS holds nothing else, and smaller tiles
// stream more bytes per MFMA.
template <int BM>
constexpr int pk_stages() { return BM >= 128 ? 3 : 4; }

template <int BN, int WM, int WN, bool GATED, bool GATHER>
__device__ __forceinline__ void pk_short(int q, const FfnGroup& fg, int m0, int n0, int h,
                                         uint4* __restrict__ smem, int slice, int nslice,
                                         float* part, size_t pstride, int* arrive) {
  if (q == 1)
    gemm_pk_body<64, BN, WM, WN, GATED, GATHER, 3, 2>(fg, m0, n0, h, smem, slice, nslice, part,
                                                      pstride, arrive);
  else if (q == 2)
    gemm_pk_body<128, BN, WM, WN, GATED, GATHER, 3, 1>(fg, m0, n0, h, smem, slice, nslice, part,
                                                       pstride, arrive);
  else
    gemm_pk_body<192, BN, WM, WN, GATED, GATHER, 3>(fg, m0, n0, h, smem, slice, nslice, part,
                                                    pstride, arrive);
}

// The tile of a block on packed weights: as gemm_bf16_tile.
template <int BM, int BN, int WM, int WN, bool GATED, bool TALL>
__device__ __forceinline__ void gemm_pk_tile(const FfnSched* __restrict__ sc, int h,
                                             float* __restrict__ part, int* __restrict__ arrive,
                                             uint4* __restrict__ smem) {
  constexpr int BMT = BM + 32 * WM, TS = tall_split<WM, WN>(), BNT = BN / TS;
  constexpr int BNO = GATED ? BN / 2 : BN;
  constexpr int NS = pk_stages<BM>();
  TileRef t;
  if (!find_tile(sc, GATED, t)) return;
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
  if constexpr (!TALL) {
    if (t.tall) {   // an expert's short last m-tile (128 or 192 rows)
      if (GATED && fg.gidx)
        pk_short<BN, WM, WN, GATED, GATED>(t.tall, fg, m0, n0, h, smem, t.slice, t.nslice, pt, ps,
                                           ar);
      else
        pk_short<BN, WM, WN, GATED, false>(t.tall, fg, m0, n0, h, smem, t.slice, t.nslice, pt, ps,
                                           ar);
      return;
    }
  }
  if constexpr (TALL) {
    if (t.tall) {   // part of an expert's tall last tile: all of K
      if (GATED && fg.gidx)
        gemm_pk_body<BMT, BNT, WM, WN, GATED, GATED, NS>(fg, m0, n0t, h, smem, 0, 1, nullptr, 0,
                                                         nullptr);
      else
        gemm_pk_body<BMT, BNT, WM, WN, GATED, false, NS>(fg, m0, n0t, h, smem, 0, 1, nullptr, 0,
                                                         nullptr);
      return;
    }
  }
  if (GATED && fg.gidx)
    gemm_pk_body<BM, BN, WM, WN, GATED, GATED, NS>(fg, m0, n0, h, smem, t.slice, t.nslice, pt, ps,
                                                   ar);
  else
    gemm_pk_body<BM, BN, WM, WN, GATED, false, NS>(fg, m0, n0, h, smem, t.slice, t.nslice, pt, ps,
                                                   ar);
}

template <int BM, int BN, int WM, int WN, bool GATED, bool TALL>
constexpr size_t pk_tile_lds_bytes() {
  constexpr int NS = pk_stages<BM>();
  return TALL ? cmax<pk_lds_bytes<BM, BN, GATED, NS>(),
                     pk_lds_bytes<BM + 32 * WM, BN / tall_split<WM, WN>(), GATED, NS>()>()
              : cmax<pk_lds_bytes<BM, BN, GATED, NS>(),
                     cmax<pk_lds_bytes<128, BN, GATED, 3>(), pk_lds_bytes<192, BN, GATED, 3>()>()>();
}

template <int BM, int BN, int WM, int WN, bool TALL>
__global__ __launch_bounds__(64 * WM * WN) void ffn_gate_up_pk(const FfnSched* __restrict__ sc,
                                                               int h, float* part, int* arrive) {
  __shared__ uint4 smem[pk_tile_lds_bytes<BM, BN, WM, WN, true, TALL>() / 16];
  gemm_pk_tile<BM, BN, WM, WN, true, TALL>(sc, h, part, arrive, smem);
}
template <int BM, int BN, int WM, int WN, bool TALL>
__global__ __launch_bounds__(64 * WM * WN) void ffn_down_pk(const FfnSched* __restrict__ sc,
                                                            int h, float* part, int* arrive) {
  __shared__ uint4 smem[pk_tile_lds_bytes<BM, BN, WM, WN, false, TALL>() / 16];
  gemm_pk_tile<BM, BN, WM, WN, false, TALL>(sc, h, part, arrive, smem);
}

// Weights in the packed order the GEMMs above read: one thread per 16-byte output chunk o
// = ((m * rows/32 + b) * cols/16 + k) * 64 + l, holding row 32b + l%32, columns
// 16k + 8(l/32) .. +7 of matrix m.
__global__ __launch_bounds__(256) void pack_weights(const uint4* __restrict__ src,
                                                    uint4* __restrict__ dst, int64_t chunks,
                                                    int rows, int cols) {
  const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (o >= chunks) return;
  const int l = (int)(o & 63);
  int64_t rest = o >> 6;
  const int kblocks = cols / 16, rblocks = rows / 32;
  const int k = (int)(rest % kblocks);
  rest /= kblocks;
  const int b = (int)(rest % rblocks);
  const int64_t m = rest / rblocks;
  const int64_t row = (int64_t)b * 32 + (l & 31);
  const int64_t col = (int64_t)k * 16 + 8 * (l >> 5);
  dst[o] = src[((m * rows + row) * cols + col) / 8];
}

// fp32 grouped GEMM: 64 x 64 tiles (gated: 32 gate + 32 up columns), 4x4 per thread.
// ---- MX-FP8 grouped GEMM --------------------------------------------------------------
// Same tiles, DMA layout and pipeline as the bf16 body. A k-step is still 128 bytes of each
// operand row, now 128 E4M3 values, and takes two scaled MFMAs 32x32x64 per fragment pair.
// In a lane of that MFMA's operand, bytes 0-15 hold k 16h..16h+15 of the first 32-value
// scale block and bytes 16-31 k 32+16h..32+16h+15 of the second (h = lane / 32): exactly the
// two 16-byte chunks the bf16 body reads in its phases 2c and 2c+1, so the swizzled LDS rows
// carry over unchanged and MFMA c takes chunks 4c+h and 4c+2+h. Each stage also holds the
// scale dword (the 4 blocks of the k-step) of every A and B row, fetched by 4-byte DMA.
// The hardware takes a row's first block scale from lane r and its second from lane r+32,
// so MFMA c needs block 2c+h in the lanes of half h: byte 0 (c = 0) or byte 2 (c = 1) of the
// row's dword shifted right by 8h. Those bytes of a wave's (at most four) A fragments are
// packed into one word per half, likewise for B, and op_sel picks the fragment's byte:
// four scale registers instead of one per fragment, which keeps the 256-row tile's
// register file from spilling.
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef int intx4 __attribute__((ext_vector_type(4)));

// Scaled MFMA 32x32x64 whose scale bytes op_sel picks out of packed words (oa, ob in 0..3:
// constants after unrolling, so the switch folds to one instruction).
__device__ __forceinline__ floatx16 mfma_mx(intx8 a, intx8 b, floatx16 c, int sa, int oa, int sb,
                                            int ob) {
#define MX_CASE(X, Y) \
  case X * 4 + Y: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, X, sa, Y, sb);
  switch (oa * 4 + ob) {
    MX_CASE(0, 0) MX_CASE(0, 1) MX_CASE(0, 2) MX_CASE(0, 3)
    MX_CASE(1, 0) MX_CASE(1, 1) MX_CASE(1, 2) MX_CASE(1, 3)
    MX_CASE(2, 0) MX_CASE(2, 1) MX_CASE(2, 2) MX_CASE(2, 3)
    MX_CASE(3, 0) MX_CASE(3, 1) MX_CASE(3, 2) MX_CASE(3, 3)
    default: return c;
  }
#undef MX_CASE
}

template <int BM, int BN, int NW>
struct Fp8Shape {
  static constexpr int BMS = (BM + 63) / 64 * 64;   // A scale dwords per stage
  static constexpr int ZA = BMS / 64, ZB = BN / 64; // 64-row scale DMA instructions
  static constexpr int SPW = (ZA + ZB + NW - 1) / NW;   // ... per wave (some repeat one)
  static constexpr int S_ST = BMS + BN;              // scale dwords per stage
};

template <int BM>
constexpr int fp8_stages() { return BM >= 256 ? 2 : 3; }

// Epilogue of the gated MX-FP8 tile: H = silu(gate) * up in fp32, then per token row and
// 32 output columns (one lane pair holds them: lane r and r+32, 16 values each) the block
// exponent from the largest magnitude, E4M3 codes staged in LDS and stored as 16-byte row
// chunks, and the scale byte stored by the first lane of the pair.
template <int BM, int BN, int WM, int WN>
__device__ __forceinline__ void store_tile_mx(const floatx16 (&acc)[BM / WM / 32][BN / WN / 32],
                                              const FfnGroup& fg, int m0, int n0,
                                              uint4* __restrict__ smem) {
  constexpr int NT = 64 * WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int BNO = BN / 2;
  constexpr int PITCH = BNO + 16;
  const int rows = fg.rows, Nout = fg.inter, KSo = fg.inter / 32;
  uint8_t* C = static_cast<uint8_t*>(fg.C1);
  uint8_t* Cs = fg.C1s;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  char* stage = reinterpret_cast<char*>(smem);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int row = wm * WTM + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < TN / 2; ++j) {
      float v[16];
      uint32_t am = 0;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        v[q] = silu_fast(acc[i][j][q]) * acc[i][j + TN / 2][q];
        am = max(am, mag_bits(v[q]));
      }
      am = max(am, (uint32_t)__shfl_xor((int)am, 32));
      const int x = mx_exponent(am);
      const int cblk = wn * (WTN / 2) + j * 32;          // the block's first column
      const int cbase = cblk + 4 * (lane >> 5);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<uint32_t*>(stage + row * PITCH + cbase + 8 * q4) =
            mx_pack4(v[4 * q4], v[4 * q4 + 1], v[4 * q4 + 2], v[4 * q4 + 3], x);
      const int gr = m0 + row, gb = (n0 + cblk) / 32;
      if (lane < 32 && gr < rows && gb < KSo) Cs[(size_t)gr * KSo + gb] = (uint8_t)(x + 127);
    }
  }
  __syncthreads();
  constexpr int RCH = BNO / 16;
  for (int id = tid; id < BM * RCH; id += NT) {
    const int r = id / RCH, cc = id % RCH;
    const int gr = m0 + r, gc = n0 + cc * 16;
    if (gr < rows && gc < Nout)
      *reinterpret_cast<uint4*>(C + (size_t)gr * Nout + gc) =
          *reinterpret_cast<const uint4*>(stage + r * PITCH + cc * 16);
  }
}

template <int BM, int BN, int WM, int WN, bool GATED, bool GATHER, int NS>
__device__ __forceinline__ void gemm_mx_body(const FfnGroup& fg, int m0, int n0, int h,
                                             uint4* __restrict__ smem) {
  constexpr int NW = WM * WN;
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  static_assert(TM >= 1 && TN >= 1, "tile");
  static_assert(!GATED || TN % 2 == 0, "gated needs gate/up pairs");
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "DMA rows split evenly over waves");
  using SH = Fp8Shape<BM, BN, NW>;
  constexpr int AI = BM / (8 * NW), BI = BN / (8 * NW);
  constexpr int SPW = SH::SPW;
  constexpr int LPS = AI + BI + SPW;                // DMA instructions per wave per stage
  constexpr int A_ST = BM * 8, B_ST = BN * 8;       // uint4 per stage
  constexpr int NMF = TM * TN;                      // MFMAs per 64-k half step
  static_assert(NS >= 2 && NS <= 4 && LPS * (NS - 2) < 64, "LDS stages");
  uint4* As = smem;                                 // [NS][BM rows][8 chunks]
  uint4* Bs = smem + NS * A_ST;                     // [NS][BN rows][8 chunks]
  uint32_t* Ss = reinterpret_cast<uint32_t*>(smem + NS * (A_ST + B_ST));   // [NS][S_ST]

  const int rows = fg.rows, I = fg.inter;
  const uint8_t* A = static_cast<const uint8_t*>(GATED ? fg.A1 : fg.C1);
  const uint8_t* Asc = GATED ? fg.A1s : fg.C1s;
  const uint8_t* B = static_cast<const uint8_t*>(GATED ? fg.B1 : fg.B2);
  const uint8_t* Bsc = GATED ? fg.B1s : fg.B2s;
  const int Kd = GATED ? h : I;          // reduction length = row bytes
  const int KS = Kd / 32;                // scale bytes per row
  const uint32_t b_rows = GATED ? 2 * I : h;
  const uint32_t a_rows = (uint32_t)(GATHER ? fg.arows : rows);
  const uint32_t a_bytes = a_rows * (uint32_t)Kd;
  const uint32_t as_bytes = a_rows * (uint32_t)KS;
  const __amdgpu_buffer_rsrc_t ra_rs = make_rsrc(A, a_bytes);
  const __amdgpu_buffer_rsrc_t rb_rs = make_rsrc(B, b_rows * (uint32_t)Kd);
  const __amdgpu_buffer_rsrc_t rsa_rs = make_rsrc(Asc, as_bytes);
  const __amdgpu_buffer_rsrc_t rsb_rs = make_rsrc(Bsc, b_rows * (uint32_t)KS);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // operand DMA as in the bf16 body, one byte per element
  const int dr = lane >> 3;
  const int dc = (lane & 7) ^ dr ^ (wave & 1);
  const uint32_t a_lane = (uint32_t)(m0 + 8 * wave + dr) * Kd + dc * 16;
  const uint32_t b_lane = (uint32_t)(n0 + 8 * wave + dr) * Kd + dc * 16;
  const uint32_t b_lane_up = GATED ? b_lane + (uint32_t)I * Kd : b_lane;
  const uint32_t x_stride = (uint32_t)(8 * NW) * Kd;
  constexpr int BH = GATED ? BI / 2 : BI;
  const global_i32* gidx = as_global(fg.gidx);
  uint32_t a_off[GATHER ? AI : 1];
  if constexpr (GATHER) {
    int src[AI];
#pragma unroll
    for (int x = 0; x < AI; ++x) {
      const int r = m0 + 8 * (NW * x + wave) + dr;
      src[x] = gidx[r < rows ? r : rows - 1];
    }
#pragma unroll
    for (int x = 0; x < AI; ++x) {
      const int r = m0 + 8 * (NW * x + wave) + dr;
      a_off[x] = (r < rows && src[x] >= 0) ? (uint32_t)(src[x] / fg.gK) * Kd + dc * 16 : a_bytes;
    }
  }
  // scale DMA: instruction z covers 64 rows (A rows first, then B rows); lane L fetches the
  // k-step's scale dword of row 64z + L (past an operand's end: zero)
  int s_z[SPW];
  uint32_t s_off[SPW];
#pragma unroll
  for (int y = 0; y < SPW; ++y) {
    // wave-uniform: the descriptor and the LDS destination (M0) stay scalar
    const int z = __builtin_amdgcn_readfirstlane(min(NW * y + wave, SH::ZA + SH::ZB - 1));
    s_z[y] = z;
    if (z < SH::ZA) {
      const int r = 64 * z + lane, gr = m0 + r;
      bool ok = r < BM && gr < rows;
      int srow = gr;
      if constexpr (GATHER) {
        const int sv = gidx[ok ? gr : 0];
        ok = ok && sv >= 0;
        srow = sv / fg.gK;
      }
      s_off[y] = ok ? (uint32_t)srow * KS : as_bytes;
    } else {
      const int r = 64 * (z - SH::ZA) + lane;
      const int gr = GATED ? (r < BN / 2 ? n0 + r : I + n0 + r - BN / 2) : n0 + r;
      s_off[y] = (uint32_t)gr * KS;
    }
  }
  const int nk = __builtin_amdgcn_readfirstlane(Kd / 128);   // k-steps, in an SGPR
  auto issue_one = [&](int step, int stage, int x) __attribute__((always_inline)) {
    const uint32_t soff = (uint32_t)step * 128;
    if (x < AI) {
      if constexpr (GATHER)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra_rs, LDS_PTR(As + stage * A_ST + 64 * (NW * x + wave)), 16, a_off[x], soff, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra_rs, LDS_PTR(As + stage * A_ST + 64 * (NW * x + wave)), 16, a_lane,
            soff + x * x_stride, 0, 0);
    } else if (x < AI + BI) {
      const int y = x - AI;
      const int yh = y % BH;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb_rs, LDS_PTR(Bs + stage * B_ST + 64 * (NW * y + wave)), 16,
          y < BH ? b_lane : b_lane_up, soff + yh * x_stride, 0, 0);
    } else {
      const int y = x - AI - BI;
      const int z = s_z[y];
      const uint32_t ks = __builtin_amdgcn_readfirstlane(step * 4);
      if (z < SH::ZA)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsa_rs, LDS_PTR(Ss + stage * SH::S_ST + 64 * z), 4, s_off[y], ks, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsb_rs, LDS_PTR(Ss + stage * SH::S_ST + SH::BMS + 64 * (z - SH::ZA)), 4, s_off[y],
            ks, 0, 0);
    }
  };

  floatx16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

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
  // B fragments of both halves are live together (the second half's are read after the
  // first MFMA); an A fragment is re-read for the second half right after its last use in
  // the first, so only one set of A fragments is live (the register file also holds the
  // accumulators).
  intx8 fa[TM], fb[2][TN];
  uint32_t pa[2], pb[2];   // per half: byte i = the scale of fragment i's rows
  static_assert(TM <= 4 && TN <= 4, "op_sel addresses four fragments");
  auto frag = [&](const uint4* base, int r, int c) __attribute__((always_inline)) {
    const int sw = row_swz(r);
    const intx4 lo = __builtin_bit_cast(intx4, base[r * 8 + (c ^ sw)]);
    const intx4 hi = __builtin_bit_cast(intx4, base[r * 8 + ((c + 2) ^ sw)]);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // fragments of MFMA `half` (0 or 1) of the k-step in `stage`
  auto read_b = [&](int set, int stage, int half) __attribute__((always_inline)) {
    const int c = 4 * half + (lane >> 5);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[set][j] = frag(Bs + stage * B_ST, brow[j], c);
  };
  auto read_a = [&](int i, int stage, int half) __attribute__((always_inline)) {
    fa[i] = frag(As + stage * A_ST, arow[i], 4 * half + (lane >> 5));
  };
  auto read_frags = [&](int stage) __attribute__((always_inline)) {
    read_b(0, stage, 0);
#pragma unroll
    for (int i = 0; i < TM; ++i) read_a(i, stage, 0);
  };
  auto read_scales = [&](int stage) __attribute__((always_inline)) {
    const uint32_t* ss = Ss + stage * SH::S_ST;
    const int sh = 8 * (lane >> 5);
    pa[0] = pa[1] = pb[0] = pb[1] = 0;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const uint32_t d = ss[arow[i]] >> sh;
      pa[0] |= (d & 0xffu) << (8 * i);
      pa[1] |= ((d >> 16) & 0xffu) << (8 * i);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const uint32_t d = ss[SH::BMS + brow[j]] >> sh;
      pb[0] |= (d & 0xffu) << (8 * j);
      pb[1] |= ((d >> 16) & 0xffu) << (8 * j);
    }
  };

  // One k-step: two halves of NMF scaled MFMAs; the second half's fragments are read
  // after the first MFMA; the next k-step's DMA rides along one instruction per MFMA.
  auto kstep = [&](int stage, bool dma, int next_step, int dma_stage)
                   __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int t = 0; t < NMF; ++t) {
        const int i = t / TN, j = t % TN;
        acc[i][j] = mfma_mx(fb[c][j], fa[i], acc[i][j], (int)pb[c], j, (int)pa[c], i);
        const int slot = c * NMF + t;
        if (dma && slot >= 1 && slot - 1 < LPS) issue_one(next_step, dma_stage, slot - 1);
        if (c == 0 && t == 0) {
          __builtin_amdgcn_sched_barrier(0);
          read_b(1, stage, 1);
        }
        if (c == 0 && j == TN - 1) {   // last use of fa[i] in this half
          __builtin_amdgcn_sched_barrier(0);
          read_a(i, stage, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (dma) {
#pragma unroll
      for (int x = 2 * NMF - 1; x < LPS; ++x) issue_one(next_step, dma_stage, x);
    }
  };

  if (nk > 0) {
#pragma unroll
    for (int s0 = 0; s0 < NS - 1; ++s0)
      if (s0 < nk)
#pragma unroll
        for (int x = 0; x < LPS; ++x) issue_one(s0, s0, x);
    if (nk >= NS - 1) wait_vmcnt<LPS * (NS - 2)>();
    else wait_vmcnt<0>();
    lds_barrier();
    read_frags(0);
    read_scales(0);
    int kt = 0;
    for (; kt + NS - 1 < nk; ++kt) {
      kstep(kt % NS, true, kt + NS - 1, (kt + NS - 1) % NS);
      wait_vmcnt<LPS * (NS - 2)>();
      lds_barrier();
      read_frags((kt + 1) % NS);
      read_scales((kt + 1) % NS);
    }
    for (; kt + 1 < nk; ++kt) {
      kstep(kt % NS, false, 0, 0);
      const int after = nk - kt - 2;
      if (NS > 3 && after >= 2) wait_vmcnt<LPS * (NS > 3 ? 2 : 0)>();
      else if (NS > 2 && after >= 1) wait_vmcnt<LPS * (NS > 2 ? 1 : 0)>();
      else wait_vmcnt<0>();
      lds_barrier();
      read_frags((kt + 1) % NS);
      read_scales((kt + 1) % NS);
    }
    kstep((nk - 1) % NS, false, 0, 0);
  }
  __syncthreads();
  if constexpr (GATED)
    store_tile_mx<BM, BN, WM, WN>(acc, fg, m0, n0, smem);
  else
    store_tile<BM, BN, WM, WN, false>(acc, fg, m0, n0, h, smem);
}

template <int BM, int BN, int WM, int WN, bool GATED, int NS>
constexpr size_t mx_lds_bytes() {
  using SH = Fp8Shape<BM, BN, WM * WN>;
  constexpr size_t ops = NS * ((size_t)(BM + BN) * 8 * 16 + (size_t)SH::S_ST * 4);
  constexpr size_t stg = GATED ? (size_t)BM * (BN / 2 + 16) : (size_t)BM * (BN * 2 + 16);
  return ops > stg ? ops : stg;
}

template <int BM, int BN, int WM, int WN, bool GATED, bool TALL>
constexpr size_t mx_tile_lds_bytes() {
  constexpr int NS = fp8_stages<BM>();
  return TALL ? cmax<mx_lds_bytes<BM, BN, WM, WN, GATED, NS>(),
                     mx_lds_bytes<BM + 32 * WM, BN / tall_split<WM, WN>(), WM, WN, GATED, NS>()>()
              : cmax<mx_lds_bytes<BM, BN, WM, WN, GATED, NS>(),
                     mx_lds_bytes<192, BN, WM, WN, GATED, 2>()>();
}

template <int BN, int WM, int WN, bool GATED, bool GATHER>
__device__ __forceinline__ void mx_short(int q, const FfnGroup& fg, int m0, int n0, int h,
                                         uint4* __restrict__ smem) {
  if (q == 2) gemm_mx_body<128, BN, WM, WN, GATED, GATHER, 2>(fg, m0, n0, h, smem);
  else gemm_mx_body<192, BN, WM, WN, GATED, GATHER, 2>(fg, m0, n0, h, smem);
}

template <int BM, int BN, int WM, int WN, bool GATED, bool TALL>
__device__ __forceinline__ void gemm_mx_tile(const FfnSched* __restrict__ sc, int h,
                                             uint4* __restrict__ smem) {
  constexpr int BMT = BM + 32 * WM, TS = tall_split<WM, WN>(), BNT = BN / TS;
  constexpr int BNO = GATED ? BN / 2 : BN;
  constexpr int NS = fp8_stages<BM>();
  TileRef t;
  if (!find_tile(sc, GATED, t)) return;   // no split-K here: every tile takes all of K
  t.g = __builtin_amdgcn_readfirstlane(t.g);
  t.m_tile = __builtin_amdgcn_readfirstlane(t.m_tile);
  t.n_tile = __builtin_amdgcn_readfirstlane(t.n_tile);
  t.tall = __builtin_amdgcn_readfirstlane(t.tall);
  const FfnGroup& fg = sc->g[t.g];
  const int m0 = t.m_tile * BM, n0 = t.n_tile * BNO;
  const int n0t = n0 + (t.tall - 1) * (BNO / TS);
  if constexpr (!TALL) {
    if (t.tall) {   // an expert's short last m-tile (128 or 192 rows)
      if (GATED && fg.gidx) mx_short<BN, WM, WN, GATED, true>(t.tall, fg, m0, n0, h, smem);
      else mx_short<BN, WM, WN, GATED, false>(t.tall, fg, m0, n0, h, smem);
      return;
    }
  }
  if (GATED && fg.gidx) {
    if (TALL && t.tall)
      gemm_mx_body<TALL ? BMT : BM, TALL ? BNT : BN, WM, WN, GATED, GATED, NS>(fg, m0, n0t, h,
                                                                               smem);
    else
      gemm_mx_body<BM, BN, WM, WN, GATED, GATED, NS>(fg, m0, n0, h, smem);
  } else {
    if (TALL && t.tall)
      gemm_mx_body<TALL ? BMT : BM, TALL ? BNT : BN, WM, WN, GATED, false, NS>(fg, m0, n0t, h,
                                                                               smem);
    else
      gemm_mx_body<BM, BN, WM, WN, GATED, false, NS>(fg, m0, n0, h, smem);
  }
}

template <int BM, int BN, int WM, int WN, bool TALL>
__global__ __launch_bounds__(64 * WM * WN) void ffn_gate_up_mxfp8(const FfnSched* __restrict__ sc,
                                                                  int h) {
  __shared__ uint4 smem[mx_tile_lds_bytes<BM, BN, WM, WN, true, TALL>() / 16];
  gemm_mx_tile<BM, BN, WM, WN, true, TALL>(sc, h, smem);
}
template <int BM, int BN, int WM, int WN, bool TALL>
__global__ __launch_bounds__(64 * WM * WN) void ffn_down_mxfp8(const FfnSched* __restrict__ sc,
                                                               int h) {
  __shared__ uint4 smem[mx_tile_lds_bytes<BM, BN, WM, WN, false, TALL>() / 16];
  gemm_mx_tile<BM, BN, WM, WN, false, TALL>(sc, h, smem);
}

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
Tiling tiling(Tiles k, bool waves_side_by_side) {
  switch (k) {
    // 256-row tiles: tall parts would cost as much as tiles; an expert's last m-tile is a
    // short one instead when its remainder is 65..192 rows (tall_split 0)
    case Tiles::Large: return {256, 0, 0};
    case Tiles::Medium: return waves_side_by_side ? Tiling{128, 32, 1} : Tiling{128, 64, 2};
    default: return {32, 32, 1};
  }
}

template <int BM, int BN, int WM, int WN, bool TALL, bool DEEP = false>
bool launch_bf16_gemm(bool gated, const FfnSched* sc, int h, int64_t ub, int cpx, float* part,
                      int* arrive, hipStream_t st) {
  constexpr int NT = 64 * WM * WN;
  if (ub <= 0) return true;
  // per XCD: its share of the tiles plus room for one round of k-slices
  const int64_t g = ((ub + kNumXcd - 1) / kNumXcd + cpx) * kNumXcd;
  if (gated)
    hipLaunchKernelGGL((ffn_gate_up_bf16<BM, BN, WM, WN, TALL, DEEP>), dim3((unsigned)g),
                       dim3(NT), 0, st, sc, h, part, arrive);
  else
    hipLaunchKernelGGL((ffn_down_bf16<BM, BN, WM, WN, TALL, DEEP>), dim3((unsigned)g), dim3(NT),
                       0, st, sc, h, part, arrive);
  return hipGetLastError() == hipSuccess;
}

// 256-row tiles stream each weight tile once per 4+ m-tiles; with three weight stages in
// LDS (two A stages: 160 KB in all) the weights are fetched two k-steps ahead.
bool launch_bf16(Tiles k, bool gated, const FfnSched* sc, int h, int64_t ub, int cpx,
                 float* part, int* arrive, hipStream_t st) {
  switch (k) {
    case Tiles::Large:
      return launch_bf16_gemm<256, 256, 2, 2, false, true>(gated, sc, h, ub, cpx, part, arrive,
                                                           st);
    case Tiles::Medium:
      return launch_bf16_gemm<128, 256, 2, 2, true>(gated, sc, h, ub, cpx, part, arrive, st);
    default:
      return launch_bf16_gemm<32, 256, 1, 4, true>(gated, sc, h, ub, cpx, part, arrive, st);
  }
}

template <int BM, int BN, int WM, int WN, bool TALL>
bool launch_pk_gemm(bool gated, const FfnSched* sc, int h, int64_t ub, int cpx, float* part,
                    int* arrive, hipStream_t st) {
  constexpr int NT = 64 * WM * WN;
  if (ub <= 0) return true;
  const int64_t g = ((ub + kNumXcd - 1) / kNumXcd + cpx) * kNumXcd;
  if (gated)
    hipLaunchKernelGGL((ffn_gate_up_pk<BM, BN, WM, WN, TALL>), dim3((unsigned)g), dim3(NT), 0,
                       st, sc, h, part, arrive);
  else
    hipLaunchKernelGGL((ffn_down_pk<BM, BN, WM, WN, TALL>), dim3((unsigned)g), dim3(NT), 0, st,
                       sc, h, part, arrive);
  return hipGetLastError() == hipSuccess;
}

// Packed weights: every tile kind with its four waves side by side.
bool launch_pk(Tiles k, bool gated, const FfnSched* sc, int h, int64_t ub, int cpx,
               float* part, int* arrive, hipStream_t st) {
  switch (k) {
    case Tiles::Large:
      return launch_pk_gemm<256, 256, 1, 4, false>(gated, sc, h, ub, cpx, part, arrive, st);
    case Tiles::Medium:
      return launch_pk_gemm<128, 256, 1, 4, true>(gated, sc, h, ub, cpx, part, arrive, st);
    default:
      return launch_pk_gemm<32, 256, 1, 4, true>(gated, sc, h, ub, cpx, part, arrive, st);
  }
}

template <int BM, int BN, int WM, int WN, bool TALL>
bool launch_mx_gemm(bool gated, const FfnSched* sc, int h, int64_t ub, hipStream_t st) {
  constexpr int NT = 64 * WM * WN;
  if (ub <= 0) return true;
  const int64_t g = (ub + kNumXcd - 1) / kNumXcd * kNumXcd;
  if (gated)
    hipLaunchKernelGGL((ffn_gate_up_mxfp8<BM, BN, WM, WN, TALL>), dim3((unsigned)g), dim3(NT), 0,
                       st, sc, h);
  else
    hipLaunchKernelGGL((ffn_down_mxfp8<BM, BN, WM, WN, TALL>), dim3((unsigned)g), dim3(NT), 0, st,
                       sc, h);
  return hipGetLastError() == hipSuccess;
}

// MX-FP8 tiles: the same shapes as bf16.
Tiles mx_tiles(Tiles k) { return k; }

bool launch_mx(Tiles k, bool gated, const FfnSched* sc, int h, int64_t ub, hipStream_t st) {
  switch (mx_tiles(k)) {
    case Tiles::Large: return launch_mx_gemm<256, 256, 2, 2, false>(gated, sc, h, ub, st);
    case Tiles::Medium: return launch_mx_gemm<128, 256, 2, 2, true>(gated, sc, h, ub, st);
    default: return launch_mx_gemm<32, 256, 1, 4, true>(gated, sc, h, ub, st);
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

// Upper bounds on each GEMM's tiles, which the launches size their grids by:
// sum_e ceil(rows_e / BM) <= R_max / BM + E_l m-tiles (an expert with a tall last tile has
// mt - 1 + tall_split <= ceil(rows_e / BM) tiles per n-tile), plus the shared expert's.
void ffn_tile_bounds(const moe_problem* p, const Dims& d, const FfnPrepArgs& a, int64_t* ub1,
                     int64_t* ub2) {
  const int has_sh = a.has_shared;
  auto m_ub = [&](int BM) { return d.R_max / BM + d.El; };
  auto m_sh = [&](int BM) { return has_sh ? (d.sh_rows + BM - 1) / BM : (int64_t)0; };
  const int64_t nt1 = (p->inter + a.BN1 - 1) / a.BN1;
  const int64_t nt1s = has_sh ? (p->shared_inter + a.BN1 - 1) / a.BN1 : 0;
  const int64_t nt2 = (d.h + a.BN2 - 1) / a.BN2;
  *ub1 = m_ub(a.BM1) * nt1 + m_sh(a.BM1) * nt1s;
  *ub2 = (m_ub(a.BM2) + m_sh(a.BM2)) * nt2;
}

int ffn_prep_args(const moe_problem* p, const Dims& d, const void* xp, const void* w13,
                  const void* w2, const void* x, const void* w13_sh, const void* w2_sh, void* yp,
                  void* y_sh, char* ws, const WsLayout& L, const int32_t* gather_rows,
                  FfnPrepArgs* a) {
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return MOE_ERR_LAUNCH;
  const int cpx = n_cu / kNumXcd < 1 ? 1 : (n_cu / kNumXcd > kCuPerXcdMax ? kCuPerXcdMax
                                                                         : n_cu / kNumXcd);
  Tiling t1{F_BM, 0, 1}, t2{F_BM, 0, 1};
  int BN1 = F_BN / 2, BN2 = F_BN, split_max = 1;
  const int has_sh = (p->n_shared && d.sh_rows > 0) ? 1 : 0;
  if (d.bf16) {
    t1 = tiling(d.mx ? mx_tiles(tile_kind(d, true)) : tile_kind(d, true), d.pk);
    t2 = tiling(d.mx ? mx_tiles(tile_kind(d, false)) : tile_kind(d, false), d.pk);
    int min_k = d.h < p->inter ? d.h : p->inter;
    if (has_sh && p->shared_inter < min_k) min_k = p->shared_inter;
    split_max = min_k / 64 < kMaxSplit ? min_k / 64 : kMaxSplit;
    if (d.mx) split_max = 1;   // the MX-FP8 GEMMs take whole tiles
    BN1 = 128;   // output columns of the gated tile (256 B rows: 128 gate + 128 up)
    BN2 = 256;
  }
  a->sc = reinterpret_cast<FfnSched*>(ws + L.sched);
  a->xp = static_cast<const char*>(xp);
  a->w13 = static_cast<const char*>(w13);
  a->w2 = static_cast<const char*>(w2);
  a->x = static_cast<const char*>(x);
  a->w13_sh = static_cast<const char*>(w13_sh);
  a->w2_sh = static_cast<const char*>(w2_sh);
  a->hbuf = ws + L.hbuf;
  a->yp = static_cast<char*>(yp);
  a->y_sh = static_cast<char*>(y_sh);
  a->arrive = reinterpret_cast<int*>(ws + L.arrive);
  a->row_src = gather_rows;
  a->phys_expert = nullptr;
  // MX-FP8: the GEMM operands are E4M3 (x's copy and the gated product in the workspace);
  // the weight scales are filled in by the caller
  a->x_s = a->w13_s = a->w2_s = a->w13_sh_s = a->w2_sh_s = nullptr;
  a->hbuf_s = nullptr;
  if (d.mx) {
    a->x = ws + L.xq;
    a->x_s = ws + L.xs;
    a->hbuf_s = ws + L.hbuf_s;
  }
  a->p0 = d.e0;
  a->sh_rows = d.sh_rows;
  a->sh_t0 = (int64_t)d.rank * d.tpr;
  a->R_max = d.R_max;
  a->T = d.T;
  a->El = d.El;
  a->has_shared = has_sh;
  a->h = d.h;
  a->inter = p->inter;
  a->sh_inter = p->shared_inter;
  a->s = d.mx ? 1 : d.s;
  a->sy = d.s;
  a->K = d.K;
  a->BM1 = t1.BM; a->BM2 = t2.BM;
  a->tall_extra1 = t1.tall_extra; a->tall_extra2 = t2.tall_extra;
  a->tall_split1 = t1.tall_split; a->tall_split2 = t2.tall_split;
  a->BN1 = BN1; a->BN2 = BN2;
  a->cu_per_xcd = cpx;
  a->split_max = split_max;
  a->short_min = d.pk ? 1 : 2;
  int64_t ub1 = 0, ub2 = 0;
  ffn_tile_bounds(p, d, *a, &ub1, &ub2);
  a->ub1 = (int)(ub1 < INT32_MAX ? ub1 : INT32_MAX);
  a->ub2 = (int)(ub2 < INT32_MAX ? ub2 : INT32_MAX);
  // (the split differs from one by count only with 256-row tiles: others all weigh one)
  const int64_t rounds8 = 8 * kNumXcd * cpx;
  a->by_work = (t1.tall_split == 0 && ub1 >= rounds8) || (t2.tall_split == 0 && ub2 >= rounds8);
  return MOE_OK;
}

int launch_ffn_prep(const FfnPrepArgs& a, const int32_t* offsets, hipStream_t st) {
  hipLaunchKernelGGL(ffn_prep, dim3(1), dim3(1024), 0, st, a, offsets);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

int launch_ffn(const moe_problem* p, const Dims& d, const void* xp, const int32_t* offsets,
               const void* w13, const void* w2, const void* x, const void* w13_sh,
               const void* w2_sh, void* yp, void* y_sh, char* ws, const WsLayout& L,
               hipStream_t st, hipEvent_t const* ev, const int32_t* gather_rows,
               const FfnPrepArgs* prepped) {
  FfnPrepArgs a;
  int rc = MOE_OK;
  if (prepped) {
    a = *prepped;     // the table was built by dispatch
  } else {
    if ((rc = ffn_prep_args(p, d, xp, w13, w2, x, w13_sh, w2_sh, yp, y_sh, ws, L, gather_rows,
                            &a)) != MOE_OK)
      return rc;
    if ((rc = launch_ffn_prep(a, offsets, st)) != MOE_OK) return rc;
  }
  if (a.by_work) {   // a GEMM may be large enough to split its tiles by work
    hipLaunchKernelGGL(ffn_split, dim3(1), dim3(1024), 0, st, a);
    if (hipGetLastError() != hipSuccess) return MOE_ERR_LAUNCH;
  }
  if (ev && hipEventRecord(ev[0], st) != hipSuccess) return MOE_ERR_LAUNCH;
  const FfnSched* sc = a.sc;
  float* part = reinterpret_cast<float*>(ws + L.splitk);
  const int cpx = a.cu_per_xcd;
  int64_t ub1 = 0, ub2 = 0;
  ffn_tile_bounds(p, d, a, &ub1, &ub2);
  bool ok = true;
  if (d.mx) {
    ok = launch_mx(tile_kind(d, true), true, sc, d.h, ub1, st);
    if (ok && ev) ok = hipEventRecord(ev[1], st) == hipSuccess;
    if (ok) ok = launch_mx(tile_kind(d, false), false, sc, d.h, ub2, st);
  } else if (d.bf16) {
    auto run = d.pk ? launch_pk : launch_bf16;
    ok = run(tile_kind(d, true), true, sc, d.h, ub1, cpx, part, a.arrive, st);
    if (ok && ev) ok = hipEventRecord(ev[1], st) == hipSuccess;
    if (ok) ok = run(tile_kind(d, false), false, sc, d.h, ub2, cpx, part, a.arrive, st);
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

int launch_pack_weights(int64_t mats, int rows, int cols, const void* src, void* dst,
                        hipStream_t st) {
  const int64_t chunks = mats * rows * (int64_t)cols / 8;
  if (chunks <= 0) return MOE_OK;
  hipLaunchKernelGGL(pack_weights, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st,
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), chunks, rows, cols);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // namespace moe
