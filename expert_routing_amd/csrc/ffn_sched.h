// The expert FFN's tile table: which (group, m-tile, n-tile) each GEMM block takes. Built on
// the device from the local experts' row offsets, either by its own one-block kernel before
// the GEMMs or by the dispatch kernel that produces the offsets (one launch fewer). Shared by
// ffn.hip and dispatch.hip; not part of the ABI.
#pragma once

#include "moe_internal.h"

namespace moe {

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
  // MX-FP8 only: E8M0 scale bytes, one per 32 values along each row's reduction dimension
  const uint8_t* A1s;  // of A1's rows: [arows][h/32]
  const uint8_t* B1s;  // [2*inter][h/32]
  uint8_t* C1s;        // of the gated product's rows: [rows][inter/32]
  const uint8_t* B2s;  // [h][inter/32]
};

struct FfnSched {
  int n_groups;
  int total1;
  int total2;
  int tall_split[2];  // 0: no tall tiles; an expert's last m-tile is a short one instead
                      // (64, 128 or 192 rows when its remainder fits)
  int short_min[2];   // smallest short tile of each GEMM, in 64-row units (1 or 2)
  int bm[2];          // rows of a full m-tile of each GEMM
  int xb[2][kNumXcd + 1];   // XCD x takes tiles [xb[k][x], xb[k][x + 1]) of GEMM k
  int cu_per_xcd;   // CUs of one XCD (one round of blocks there)
  int split_max;    // 1: no split-K; else the most k-slices a tile may take
  int start1[G_PAD];
  int start2[G_PAD];
  FfnGroup g[G_MAX];
};

// Everything the table is built from besides the offsets (filled on the host).
struct FfnPrepArgs {
  FfnSched* sc;
  const char* xp;
  const char* w13;
  const char* w2;
  const char* x;
  const char* w13_sh;
  const char* w2_sh;
  char* hbuf;
  char* yp;
  char* y_sh;
  int* arrive;              // split-K arrival counters, zeroed here
  const int32_t* row_src;   // gathered gate/up A rows, or nullptr
  const int32_t* phys_expert;  // replica map: group g runs with the weights of logical
                               // expert phys_expert[p0 + g] (w13 / w2 hold every logical
                               // expert); nullptr: group g uses weight block g
  int p0;
  // MX-FP8 (else nullptr): scale bytes of x (token rows, [T][h/32]), of the weights and of
  // the gated product's rows (beside hbuf)
  const char* x_s;
  const char* w13_s;
  const char* w2_s;
  const char* w13_sh_s;
  const char* w2_sh_s;
  char* hbuf_s;
  int64_t sh_rows, sh_t0, R_max, T;
  int El, has_shared, h, inter, sh_inter, K;
  int s;    // bytes per element of x, the weights and hbuf (the GEMM operands)
  int sy;   // bytes per element of yp / y_sh
  int BM1, BM2, tall_extra1, tall_extra2, tall_split1, tall_split2, BN1, BN2;
  int cu_per_xcd, split_max;
  int short_min;
  int ub1, ub2;   // tiles the launches have blocks for (per XCD: (ub + 7) / 8)
  int by_work;    // 0: no GEMM can reach the size where its tiles are split by work
};

// Inclusive scan of one int per thread over a block of NT threads: wave scans by shuffles,
// then each thread adds the totals of the waves before its own (read from wsum, NT/64 ints
// of LDS). Every thread of the block must call it; *total receives the block's sum.
template <int NT>
__device__ inline int block_inclusive_scan(int v, int* wsum, int* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int s = wsum[w];
    before += w < wave ? s : 0;
    tot += s;
  }
  __syncthreads();   // wsum is free for the next scan
  *total = tot;
  return v + before;
}

// Work of one n-column of a group's tiles, for splitting the tiles among the XCDs: one unit
// a tile, except with 256-row tiles (tall_split 0), where a full tile counts BM/64 + 1 and
// an expert's short last tile of q 64-row units q + 1. wf: a full tile's work.
__device__ inline int column_work(int rows, int mt, int per_n, int BM, int TS, int short_min,
                                  int* wf) {
  *wf = 1;
  if (TS != 0 || mt <= 0) return per_n;
  *wf = BM / 64 + 1;
  const int rem = rows - (mt - 1) * BM;
  const int q64 = (rem + 63) >> 6;
  const int wl = (q64 >= short_min && q64 <= 3 && rem < BM) ? q64 + 1 : *wf;
  return (per_n - 1) * *wf + wl;
}

// Builds a.sc from offsets[0..El] (any address space) with the calling block's NT threads;
// every thread of the block must call it. Thread i takes groups [i*PER, (i+1)*PER): per
// group the m-tiles of each GEMM (a short remainder of at most tall_extra rows rides on the
// last full tile) and its tiles; the groups' starting tile indices are an exclusive scan.
// wsum: NT/64 ints of LDS.
template <int NT>
__device__ inline void ffn_build_sched(const FfnPrepArgs& a, const int32_t* offsets, int* wsum) {
  constexpr int PER = (G_MAX + 1 + NT - 1) / NT;   // covers index G (the end of the table)
  const int tid = threadIdx.x;
  const int G = a.El + a.has_shared;
  int c1[PER], c2[PER];
  int s1 = 0, s2 = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int g = tid * PER + i;
    c1[i] = c2[i] = 0;
    if (g < G) {
      FfnGroup fg;
      fg.A1s = fg.B1s = fg.B2s = nullptr;
      fg.C1s = nullptr;
      int rows, I;
      if (g < a.El) {
        const int r0 = offsets[g];
        rows = offsets[g + 1] - r0;
        I = a.inter;
        fg.A1 = a.row_src ? a.x : a.xp + (size_t)r0 * a.h * a.s;
        fg.gidx = a.row_src ? a.row_src + r0 : nullptr;
        const int wg = a.phys_expert ? a.phys_expert[a.p0 + g] : g;   // weight block
        fg.B1 = a.w13 + (size_t)wg * 2 * a.inter * a.h * a.s;
        fg.C1 = a.hbuf + (size_t)r0 * a.inter * a.s;
        fg.B2 = a.w2 + (size_t)wg * a.h * a.inter * a.s;
        fg.C2 = a.yp + (size_t)r0 * a.h * a.sy;
        if (a.w13_s) {
          fg.A1s = reinterpret_cast<const uint8_t*>(a.x_s);
          fg.B1s = reinterpret_cast<const uint8_t*>(a.w13_s) + (size_t)wg * 2 * a.inter * (a.h / 32);
          fg.C1s = reinterpret_cast<uint8_t*>(a.hbuf_s) + (size_t)r0 * (a.inter / 32);
          fg.B2s = reinterpret_cast<const uint8_t*>(a.w2_s) + (size_t)wg * a.h * (a.inter / 32);
        }
      } else {
        rows = (int)a.sh_rows;
        I = a.sh_inter;
        fg.A1 = a.x + (size_t)a.sh_t0 * a.h * a.s;
        fg.gidx = nullptr;
        fg.B1 = a.w13_sh;
        fg.C1 = a.hbuf + (size_t)a.R_max * a.inter * a.s;
        fg.B2 = a.w2_sh;
        fg.C2 = a.y_sh;
        if (a.w13_s) {
          fg.A1s = reinterpret_cast<const uint8_t*>(a.x_s) + (size_t)a.sh_t0 * (a.h / 32);
          fg.B1s = reinterpret_cast<const uint8_t*>(a.w13_sh_s);
          fg.C1s = reinterpret_cast<uint8_t*>(a.hbuf_s) + (size_t)a.R_max * (a.inter / 32);
          fg.B2s = reinterpret_cast<const uint8_t*>(a.w2_sh_s);
        }
      }
      int per_n[2];
      const int BMg[2] = {a.BM1, a.BM2}, TEg[2] = {a.tall_extra1, a.tall_extra2};
      const int TSg[2] = {a.tall_split1, a.tall_split2};
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
      fg.arows = fg.gidx ? (int)a.T : rows;
      fg.gK = a.K;
      a.sc->g[g] = fg;
      const int ncol1 = (I + a.BN1 - 1) / a.BN1, ncol2 = (a.h + a.BN2 - 1) / a.BN2;
      c1[i] = per_n[0] * ncol1;
      c2[i] = per_n[1] * ncol2;
    }
    s1 += c1[i];
    s2 += c2[i];
  }
  int tot1 = 0, tot2 = 0;
  int e1 = block_inclusive_scan<NT>(s1, wsum, &tot1) - s1;
  int e2 = block_inclusive_scan<NT>(s2, wsum, &tot2) - s2;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int g = tid * PER + i;
    if (g <= G) {          // start[G] = the total: the binary search's upper end
      a.sc->start1[g] = e1;
      a.sc->start2[g] = e2;
    }
    e1 += c1[i];
    e2 += c2[i];
  }
  // XCD split by count; ffn_split_by_work may replace it (a launch of its own)
  if (tid < 2) {
    const int k = tid, tot = k == 0 ? tot1 : tot2;
    const int per = (tot + kNumXcd - 1) / kNumXcd;
    for (int x = 0; x <= kNumXcd; ++x) a.sc->xb[k][x] = x * per < tot ? x * per : tot;
    a.sc->short_min[k] = 2;
  }
  for (int i = tid; i < 2 * kArriveSlots; i += NT) a.arrive[i] = 0;
  if (tid == 0) {
    a.sc->n_groups = G;
    a.sc->tall_split[0] = a.tall_split1;
    a.sc->tall_split[1] = a.tall_split2;
    a.sc->bm[0] = a.BM1;
    a.sc->bm[1] = a.BM2;
    a.sc->cu_per_xcd = a.cu_per_xcd;
    a.sc->split_max = a.split_max;
    a.sc->total1 = tot1;
    a.sc->total2 = tot2;
  }
}

// Splits the tiles of each GEMM with 8 or more rounds of blocks among the XCDs by work
// instead of by count (the last round's imbalance is then small against the work moved),
// where the launches have blocks for it, and lets those GEMMs take 64-row short tiles
// (under a split by count the XCDs without them set the time: measured slower). Reads
// the table ffn_build_sched wrote; one block of NT threads.
template <int NT>
__device__ inline void ffn_split_by_work(const FfnPrepArgs& a, int* wsum) {
  constexpr int PER = (G_MAX + 1 + NT - 1) / NT;
  __shared__ int xbs[2][kNumXcd + 1];
  __shared__ int cst[2][G_PAD];                          // work before each group
  __shared__ int colw_s[2][G_PAD], pern_s[2][G_PAD];   // work and tiles of one n-column
  const int tid = threadIdx.x;
  const int G = a.El + a.has_shared;
  const FfnSched* sc = a.sc;
  const int tot[2] = {sc->total1, sc->total2};
  const int rounds8 = 8 * kNumXcd * a.cu_per_xcd;
  const bool bw[2] = {tot[0] >= rounds8, tot[1] >= rounds8};
  const int BM[2] = {a.BM1, a.BM2}, TS[2] = {a.tall_split1, a.tall_split2};
  int cl[2][PER], pn[2][PER], cw[2][PER], w[2] = {0, 0};
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int g = tid * PER + i;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      cl[k][i] = pn[k][i] = cw[k][i] = 0;
      if (g < G) {
        const FfnGroup& fg = sc->g[g];
        pn[k][i] = fg.tall[k] ? fg.mt[k] - 1 + TS[k] : fg.mt[k];
        int wf;
        cl[k][i] = column_work(fg.rows, fg.mt[k], pn[k][i], BM[k], TS[k], a.short_min, &wf);
        const int ncol = k == 0 ? (fg.inter + a.BN1 - 1) / a.BN1 : (a.h + a.BN2 - 1) / a.BN2;
        cw[k][i] = pn[k][i] > 0 ? cl[k][i] * ncol : 0;
      }
      w[k] += cw[k][i];
    }
  }
  int wt[2], f[2];
  f[0] = block_inclusive_scan<NT>(w[0], wsum, &wt[0]) - w[0];
  f[1] = block_inclusive_scan<NT>(w[1], wsum, &wt[1]) - w[1];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int g = tid * PER + i;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (g <= G) {
        cst[k][g] = f[k];
        colw_s[k][g] = cl[k][i];
        pern_s[k][g] = pn[k][i];
      }
      f[k] += cw[k][i];
    }
  }
  __syncthreads();
  // XCD x of GEMM k starts at the tile that holds work offset x*W/8 (one thread each)
  if (tid < 2 * (kNumXcd + 1)) {
    const int k = tid / (kNumXcd + 1), x = tid % (kNumXcd + 1);
    int b = x == 0 ? 0 : tot[k];
    if (x > 0 && x < kNumXcd && wt[k] > 0) {
      const int target = (int)((int64_t)x * wt[k] / kNumXcd);
      int lo = 0, hi = G;          // cst[k][lo] <= target < cst[k][hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cst[k][mid] <= target) lo = mid; else hi = mid;
      }
      const int colw = colw_s[k][lo], per_n = pern_s[k][lo];
      const int wf = TS[k] == 0 ? BM[k] / 64 + 1 : 1;
      const int off = target - cst[k][lo];
      const int m = min((off % colw) / wf, per_n - 1);
      b = (k == 0 ? sc->start1[lo] : sc->start2[lo]) + off / colw * per_n + m;
    }
    xbs[k][x] = b;
  }
  __syncthreads();
  if (tid < 2) {
    const int k = tid;
    const int budget = ((k == 0 ? a.ub1 : a.ub2) + kNumXcd - 1) / kNumXcd;
    bool by_work = bw[k];
    for (int x = 0; x < kNumXcd; ++x) by_work = by_work && xbs[k][x + 1] - xbs[k][x] <= budget;
    if (by_work) {
      for (int x = 0; x <= kNumXcd; ++x) a.sc->xb[k][x] = xbs[k][x];
      a.sc->short_min[k] = a.short_min;
    }
  }
}

}  // namespace moe
