// Dispatch: per-expert histogram, capacity, expert-contiguous layout of this rank's
// pairs, the virtual-rank send matrix, and the row copy x -> xp.
//
// A pair (t, e) has rank = the number of earlier tokens that chose e (a token names an
// expert at most once). It is kept iff rank < cap, and its row in the local buffer is
// offsets[e - e0] + rank: rows are ordered by (expert, token) with no sort. The rank is
// built without float atomics or ordering races:
//   hist    per 256-token chunk, LDS-atomic counts per expert;
//   scan    one block: per-expert exclusive scan over chunks, capacity, local offsets,
//           dropped pairs;
//   layout  per chunk: each wave ORs 64-bit lane masks per expert in LDS, so a pair's
//           rank inside the chunk is a popcount of earlier lanes and earlier waves;
//   fill    rows nobody claims get row_src = -1 (pad rows also zero xp);
//   copy    one wave per (token, row segment) reads the segment of x[t] once and writes
//           it to each of the token's rows (skipped when the caller passes no xp);
//   stats   (moe_layout_stats) the same ranks and kept flags, reduced to per-token
//           target ranks instead of rows.
#include "ffn_sched.h"

namespace moe {
namespace {

constexpr int CH = kDispatchChunk;   // tokens per chunk (= threads per block)

// The K expert ids of token t (K <= 16; -1 past T, past K and for ids outside [0, E)), every
// load issued before any is used, so they share one memory round trip.
__device__ __forceinline__ void load_pair_ids(const int32_t* __restrict__ ids, int64_t t,
                                              int64_t T, int K, int E, int (&ev)[16]) {
#pragma unroll
  for (int k = 0; k < 16; ++k) ev[k] = (k < K && t < T) ? ids[t * K + k] : -1;
#pragma unroll
  for (int k = 0; k < 16; ++k)
    if (ev[k] < 0 || ev[k] >= E) ev[k] = -1;
}

__global__ __launch_bounds__(CH) void disp_hist(const int32_t* __restrict__ ids,
                                                int32_t* __restrict__ chunk_counts, int T,
                                                int K, int E) {
  __shared__ int cnt[512];
  const int c = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += CH) cnt[e] = 0;
  __syncthreads();
  const int64_t t = (int64_t)c * CH + threadIdx.x;
  int ev[16];
  load_pair_ids(ids, t, T, K, E, ev);
#pragma unroll
  for (int k = 0; k < 16; ++k)
    if (ev[k] >= 0) atomicAdd(&cnt[ev[k]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += CH) chunk_counts[(size_t)c * E + e] = cnt[e];
}

// One block of 1024 threads.
__global__ __launch_bounds__(1024) void disp_scan(const int32_t* __restrict__ chunk_counts,
                                                  int32_t* __restrict__ chunk_base,
                                                  int32_t* __restrict__ counts,
                                                  int32_t* __restrict__ kept_out,
                                                  int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ n_dropped,
                                                  int64_t* __restrict__ send_bytes,
                                                  int n_chunks, int E, int El, int e0,
                                                  int64_t cap, int pad, int N) {
  __shared__ int kept_s[512];
  __shared__ int scan_s[1024];
  __shared__ int drop_s[1024];
  const int tid = threadIdx.x;
  int drop = 0;
  for (int e = tid; e < E; e += 1024) {
    int run = 0;
    for (int c = 0; c < n_chunks; ++c) {
      chunk_base[(size_t)c * E + e] = run;
      run += chunk_counts[(size_t)c * E + e];
    }
    counts[e] = run;
    const int kept = (cap < 0 || run < cap) ? run : (int)cap;
    kept_out[e] = kept;
    kept_s[e] = kept;
    drop += run - kept;
  }
  drop_s[tid] = drop;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if (tid < s) drop_s[tid] += drop_s[tid + s];
    __syncthreads();
  }
  if (tid == 0) *n_dropped = drop_s[0];
  // exclusive scan of the local experts' row counts (El <= 512)
  int v = 0;
  if (tid < El) v = pad ? (int)cap : kept_s[e0 + tid];
  scan_s[tid] = v;
  __syncthreads();
  for (int s = 1; s < 1024; s <<= 1) {
    int add = tid >= s ? scan_s[tid - s] : 0;
    __syncthreads();
    scan_s[tid] += add;
    __syncthreads();
  }
  if (tid < El) offsets[tid + 1] = scan_s[tid];
  if (tid == 0) offsets[0] = 0;
  if (send_bytes) {
    for (int i = tid; i < N * N; i += 1024) send_bytes[i] = 0;
  }
}

// Per chunk of 256 tokens: ranks, kept flags, dest_row / row_src, send counts.
__global__ __launch_bounds__(CH) void disp_layout(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ chunk_base,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ dest_row,
    int32_t* __restrict__ row_src, int64_t* __restrict__ send_bytes, int T, int K, int E,
    int El, int e0, int64_t cap, int64_t tpr, int N, int64_t row_bytes, int lds_span) {
  __shared__ unsigned long long masks[CH / 64][512];
  extern __shared__ int ncount[];   // [lds_span][N] when lds_span > 0
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x;
  const int64_t tfirst = (int64_t)c * CH;
  const int64_t t = tfirst + tid;
  for (int i = tid; i < (CH / 64) * E; i += CH) masks[i / E][i % E] = 0ull;
  if (send_bytes && lds_span > 0)
    for (int i = tid; i < lds_span * N; i += CH) ncount[i] = 0;
  __syncthreads();
  int ev[16];
  load_pair_ids(ids, t, T, K, E, ev);
#pragma unroll
  for (int k = 0; k < 16; ++k)
    if (k < K && ev[k] >= 0) atomicOr(&masks[wave][ev[k]], 1ull << lane);
  __syncthreads();
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t src_rank = (send_bytes && tpr > 0) ? t / tpr : 0;
  const int64_t src_first = (send_bytes && tpr > 0) ? tfirst / tpr : 0;
  for (int k = 0; k < K; ++k) {
    const int e = ev[k];
    if (t >= T) break;
    int dr = -1;
    if (e >= 0) {
      int rank = chunk_base[(size_t)c * E + e] + __popcll(masks[wave][e] & below);
      for (int w = 0; w < wave; ++w) rank += __popcll(masks[w][e]);
      const bool kept = cap < 0 || rank < cap;
      if (kept) {
        if (e >= e0 && e < e0 + El) {
          dr = offsets[e - e0] + rank;
          row_src[dr] = (int32_t)(t * K + k);
        }
        if (send_bytes) {
          const int dst = e / El;
          if (lds_span > 0)
            atomicAdd(&ncount[(src_rank - src_first) * N + dst], 1);
          else
            atomicAdd(reinterpret_cast<unsigned long long*>(&send_bytes[src_rank * N + dst]),
                      (unsigned long long)row_bytes);
        }
      }
    }
    dest_row[t * K + k] = dr;
  }
  if (send_bytes && lds_span > 0) {
    __syncthreads();
    for (int i = tid; i < lds_span * N; i += CH) {
      const int n = ncount[i];
      const int64_t src = src_first + i / N;
      if (n > 0 && src < N)
        atomicAdd(reinterpret_cast<unsigned long long*>(&send_bytes[src * N + (i % N)]),
                  (unsigned long long)((int64_t)n * row_bytes));
    }
  }
}

// ---- two-launch dispatch -------------------------------------------------------------
// count: per chunk of 256 tokens an LDS-atomic histogram (chunk_counts[c][E]); block 0 also
// zeroes the send matrix the placement adds into. At least one block runs (T = 0 included).
__global__ __launch_bounds__(CH) void disp_count(const int32_t* __restrict__ ids,
                                                 int32_t* __restrict__ chunk_counts, int T,
                                                 int K, int E, int n_chunks,
                                                 int64_t* __restrict__ send_bytes, int n_send) {
  __shared__ int cnt[512];
  const int c = blockIdx.x;
  if (c == 0 && send_bytes)
    for (int i = threadIdx.x; i < n_send; i += CH) send_bytes[i] = 0;
  if (c >= n_chunks) return;
  for (int e = threadIdx.x; e < E; e += CH) cnt[e] = 0;
  __syncthreads();
  const int64_t t = (int64_t)c * CH + threadIdx.x;
  int ev[16];
  load_pair_ids(ids, t, T, K, E, ev);
#pragma unroll
  for (int k = 0; k < 16; ++k)
    if (ev[k] >= 0) atomicAdd(&cnt[ev[k]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += CH) chunk_counts[(size_t)c * E + e] = cnt[e];
}

// How the placement fills the send matrix.
enum SendMode { kSendNone = 0, kSendAtomic = 1, kSendFromCounts = 2 };

// place: every block derives what it needs of the global scan from the pair counts itself
// (the per-expert totals and the sums over earlier tokens), so no scan kernel runs between
// the histogram and the placement: capacity and kept counts, the local experts' row offsets
// (exclusive scan), then its chunk's ranks, dest_row / row_src and send counts as
// disp_layout computes them, and row_src = -1 for its share of the unclaimed rows. Block 0
// writes counts, offsets, kept and n_dropped; two other blocks (extra ones when there are
// fewer chunks) derive the send matrix and build the expert FFN's tile table, in parallel.
// The counts come in n_rows rows of gtok tokens (gtok divides 256: the histogram kernel's
// 256-token chunks, or the fused router's 16-token groups). Send matrix: kSendAtomic adds
// into a send_bytes zeroed by disp_count; kSendFromCounts (every row inside one source
// rank) lets block 0 derive it from the counts: a row's kept pairs on expert e are those
// ranked below cap, i.e. clamp(cap - earlier pairs on e, 0, pairs).
//
// With a replica map (rm.rep_start != nullptr) the buffers are laid out over physical
// experts: a pair ranked rho among its logical expert e's pairs goes to replica rho mod r_e
// (physical id rep_list[rep_start[e] + rho mod r_e]) where it ranks rho / r_e; a physical
// expert's pair count follows from e's total (floor(n_e / r_e) plus one for the first
// n_e mod r_e replicas), and the capacity applies per physical expert. El / e0 are then the
// local physical experts.
__global__ __launch_bounds__(CH) void disp_place(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ chunk_counts, int n_rows,
    int gtok, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ kept_out, int32_t* __restrict__ n_dropped,
    int32_t* __restrict__ dest_row, int32_t* __restrict__ row_src,
    int64_t* __restrict__ send_bytes, int send_mode, int T, int K, int E, int El, int e0,
    int64_t cap, int pad, int64_t R_max, int64_t tpr, int N, int64_t row_bytes, int lds_span,
    int send_block, int do_ffn, int ffn_block, FfnPrepArgs ffn, ReplicaArgs rm) {
  __shared__ unsigned long long masks[CH / 64][512];
  __shared__ int base_s[512];
  __shared__ int tot_s[512];
  __shared__ int kept_s[512];   // local (physical) experts
  __shared__ int off_s[513];
  __shared__ int wsum[CH / 64];
  __shared__ int drop_s[CH / 64];
  extern __shared__ int ncount[];   // kSendAtomic: [lds_span][N]; kSendFromCounts: [N][N]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x;
  const int g0 = c * (CH / gtok);   // first count row of this block's tokens
  const bool lds_send = send_mode == kSendAtomic && lds_span > 0;
  // Row walks per expert are split over LPE consecutive lanes (a power of two, LPE * E <=
  // 256 when E < 256), each taking a contiguous range of rows; lane sums meet by shuffles.
  int LPE = 1;
  while (LPE < 64 && LPE * 2 * E <= CH) LPE *= 2;
  const int P = rm.rep_start ? rm.P : E;   // physical experts
  // (a) per logical expert: total over all rows, and the sum over rows before this chunk
  for (int eb = 0; eb < E; eb += CH / LPE) {
    const int e = eb + tid / LPE, p = tid % LPE;
    const bool ok = e < E;
    const int r0 = (int)((int64_t)p * n_rows / LPE);
    const int r1 = (int)((int64_t)(p + 1) * n_rows / LPE);
    int tot = 0, bs = 0;
    if (ok) {
      int r = r0;
      for (; r + 8 <= r1; r += 8) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = chunk_counts[(size_t)(r + u) * E + e];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          tot += v[u];
          bs += r + u < g0 ? v[u] : 0;
        }
      }
      for (; r < r1; ++r) {
        const int v = chunk_counts[(size_t)r * E + e];
        tot += v;
        bs += r < g0 ? v : 0;
      }
    }
    for (int off = LPE / 2; off > 0; off >>= 1) {
      tot += __shfl_xor(tot, off);
      bs += __shfl_xor(bs, off);
    }
    if (ok && p == 0) {
      base_s[e] = bs;
      tot_s[e] = tot;
      if (c == 0) {
        counts[e] = tot;
        kept_out[e] = (cap < 0 || tot < cap) ? tot : (int)cap;
      }
    }
  }
  __syncthreads();
  // (a') pairs per physical expert (= per logical one without a map), kept ones, dropped
  auto phys_pairs = [&](int p) {
    if (!rm.rep_start) return tot_s[p];
    const int e = rm.phys_expert[p], q = rm.phys_replica[p];
    const int r = rm.rep_start[e + 1] - rm.rep_start[e];
    return tot_s[e] / r + (q < tot_s[e] % r ? 1 : 0);
  };
  for (int el = tid; el < El; el += CH) {
    const int n = phys_pairs(e0 + el);
    kept_s[el] = (cap < 0 || n < cap) ? n : (int)cap;
  }
  int drop = 0;
  if (c == 0) {
    for (int p = tid; p < P; p += CH) {
      const int n = phys_pairs(p);
      drop += n - ((cap < 0 || n < cap) ? n : (int)cap);
      if (rm.phys_counts) rm.phys_counts[p] = n;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) drop += __shfl_xor(drop, off);
  if (lane == 0) drop_s[wave] = drop;
  __syncthreads();
  // (b) exclusive scan of the local experts' rows (El <= 2 * CH: two per thread)
  const int el0 = 2 * tid;
  const int v0 = el0 < El ? (pad ? (int)cap : kept_s[el0]) : 0;
  const int v1 = el0 + 1 < El ? (pad ? (int)cap : kept_s[el0 + 1]) : 0;
  int rows_total = 0;
  const int excl = block_inclusive_scan<CH>(v0 + v1, wsum, &rows_total) - v0 - v1;
  if (el0 < El) off_s[el0] = excl;
  if (el0 + 1 < El) off_s[el0 + 1] = excl + v0;
  if (tid == 0) off_s[El] = rows_total;
  // (c) clear the rank masks and the send counters
  for (int i = tid; i < (CH / 64) * E; i += CH) masks[i / E][i % E] = 0ull;
  if (lds_send)
    for (int i = tid; i < lds_span * N; i += CH) ncount[i] = 0;
  if (send_mode == kSendFromCounts && c == send_block)
    for (int i = tid; i < N * N; i += CH) ncount[i] = 0;
  __syncthreads();
  if (c == 0) {
    for (int i = tid; i <= El; i += CH) offsets[i] = off_s[i];
    if (tid == 0) {
      int dsum = 0;
      for (int w = 0; w < CH / 64; ++w) dsum += drop_s[w];
      *n_dropped = dsum;
    }
  }
  // (d) ranks of this chunk's pairs: earlier chunks (base_s), earlier waves, earlier lanes
  const int64_t tfirst = (int64_t)c * CH;
  const int64_t t = tfirst + tid;
  int ev[16];
  load_pair_ids(ids, t, T, K, E, ev);
#pragma unroll
  for (int k = 0; k < 16; ++k)
    if (k < K && ev[k] >= 0) atomicOr(&masks[wave][ev[k]], 1ull << lane);
  __syncthreads();
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t src_rank = (send_mode == kSendAtomic && tpr > 0) ? t / tpr : 0;
  const int64_t src_first = (send_mode == kSendAtomic && tpr > 0) ? tfirst / tpr : 0;
  for (int k = 0; k < K && t < T; ++k) {
    const int e = ev[k];
    int dr = -1;
    if (e >= 0) {
      int rank = base_s[e] + __popcll(masks[wave][e] & below);
      for (int w = 0; w < wave; ++w) rank += __popcll(masks[w][e]);
      int pe = e;   // physical expert of the pair and its rank there
      if (rm.rep_start) {
        const int r = rm.rep_start[e + 1] - rm.rep_start[e];
        pe = rm.rep_list[rm.rep_start[e] + rank % r];
        rank = rank / r;
      }
      const bool kept = cap < 0 || rank < cap;
      if (kept) {
        if (pe >= e0 && pe < e0 + El) {
          dr = off_s[pe - e0] + rank;
          row_src[dr] = (int32_t)(t * K + k);
        }
        if (send_mode == kSendAtomic) {
          const int dst = pe / El;
          if (lds_span > 0)
            atomicAdd(&ncount[(src_rank - src_first) * N + dst], 1);
          else
            atomicAdd(reinterpret_cast<unsigned long long*>(&send_bytes[src_rank * N + dst]),
                      (unsigned long long)row_bytes);
        }
      }
    }
    dest_row[t * K + k] = dr;
  }
  // (e) unclaimed rows: past the last local expert's rows, or (padded) past an expert's
  // kept rows within its cap-row block; the blocks share them in a grid stride
  const int64_t stride = (int64_t)gridDim.x * CH;
  if (pad) {
    for (int64_t r = tfirst + tid; r < R_max; r += stride) {
      const int64_t el = r / cap;
      if (r - el * cap >= kept_s[el]) row_src[r] = -1;
    }
  } else {
    for (int64_t r = off_s[El] + tfirst + tid; r < R_max; r += stride) row_src[r] = -1;
  }
  if (lds_send) {
    __syncthreads();
    for (int i = tid; i < lds_span * N; i += CH) {
      const int n = ncount[i];
      const int64_t src = src_first + i / N;
      if (n > 0 && src < N)
        atomicAdd(reinterpret_cast<unsigned long long*>(&send_bytes[src * N + (i % N)]),
                  (unsigned long long)((int64_t)n * row_bytes));
    }
  }
  if (send_mode == kSendFromCounts && c == send_block) {
    // n_ij from the counts: each expert's rows in token order, split over its P lanes; a
    // lane starts from the pairs on e before its range (an exclusive scan of the lane sums)
    for (int eb = 0; eb < E; eb += CH / LPE) {
      const int e = eb + tid / LPE, p = tid % LPE;
      const bool ok = e < E;
      const int r0 = (int)((int64_t)p * n_rows / LPE);
      const int r1 = (int)((int64_t)(p + 1) * n_rows / LPE);
      int sum = 0;
      if (ok) {
        int r = r0;
        for (; r + 8 <= r1; r += 8) {   // eight loads in flight
          int v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = chunk_counts[(size_t)(r + u) * E + e];
#pragma unroll
          for (int u = 0; u < 8; ++u) sum += v[u];
        }
        for (; r < r1; ++r) sum += chunk_counts[(size_t)r * E + e];
      }
      int incl = sum;
      for (int off = 1; off < LPE; off <<= 1) {
        const int v = __shfl_up(incl, off, LPE);
        if (p >= off) incl += v;
      }
      if (ok) {
        int before = incl - sum, cur = -1, acc = 0;
        const int dst = e / El;
        for (int rb = r0; rb < r1; rb += 8) {   // rows in chunks of eight loads in flight
          int vb[8];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            vb[u] = rb + u < r1 ? chunk_counts[(size_t)(rb + u) * E + e] : 0;
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int r = rb + u;
            if (r >= r1) break;
            const int v = vb[u];
            int kept = v;
            if (cap >= 0) {
              const int64_t room = cap - before;
              kept = room <= 0 ? 0 : (room < v ? (int)room : v);
            }
            before += v;
            const int src = (int)(((int64_t)r * gtok) / tpr);
            if (src != cur) {
              if (acc > 0) atomicAdd(&ncount[cur * N + dst], acc);
              cur = src;
              acc = 0;
            }
            acc += kept;
          }
        }
        if (acc > 0) atomicAdd(&ncount[cur * N + dst], acc);
      }
    }
    __syncthreads();
    for (int i = tid; i < N * N; i += CH) send_bytes[i] = (int64_t)ncount[i] * row_bytes;
  }
  // (f) the expert FFN's tile table from the offsets (block-uniform branch)
  if (do_ffn && c == ffn_block) {
    __syncthreads();
    ffn_build_sched<CH>(ffn, off_s, wsum);
  }
}

// One wave per row r < R_max: unclaimed rows get row_src = -1; pad rows zero xp.
__global__ __launch_bounds__(256) void disp_fill(const int32_t* __restrict__ offsets,
                                                 const int32_t* __restrict__ kept,
                                                 int32_t* __restrict__ row_src,
                                                 uint4* __restrict__ xp, int64_t R_max,
                                                 int El, int e0, int64_t cap, int pad,
                                                 int row_chunks) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R_max) return;
  bool filled, is_pad = false;
  if (pad) {
    const int64_t el = r / cap;
    filled = (r - el * cap) < kept[e0 + el];
    is_pad = !filled;
  } else {
    filled = r < offsets[El];
  }
  if (filled) return;
  if (lane == 0) row_src[r] = -1;
  if (is_pad && xp) {
    for (int i = lane; i < row_chunks; i += 64) xp[r * row_chunks + i] = uint4{0, 0, 0, 0};
  }
}

// One wave per (token, row segment of 64*CP_UNROLL 16-byte chunks): the segment of x[t]
// is read once and stored to every row the token owns here.
constexpr int CP_UNROLL = 8;
__global__ __launch_bounds__(256) void disp_copy(const uint4* __restrict__ x,
                                                 const int32_t* __restrict__ dest_row,
                                                 uint4* __restrict__ xp, int T, int K,
                                                 int row_chunks) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  // the token's rows here (a compacted list would live in scratch memory: dynamic index)
  bool any = false;
  for (int k = 0; k < K; ++k) any = any || dest_row[t * K + k] >= 0;
  if (!any) return;
  const uint4* src = x + t * row_chunks;
  {
    const int base = blockIdx.y * 64 * CP_UNROLL;   // this wave's row segment
    uint4 v[CP_UNROLL];
#pragma unroll
    for (int u = 0; u < CP_UNROLL; ++u) {   // unconditional (clamped) loads keep v in VGPRs
      const int i = base + u * 64 + lane;
      v[u] = src[i < row_chunks ? i : row_chunks - 1];
    }
    for (int k = 0; k < K; ++k) {
      const int d = dest_row[t * K + k];
      if (d < 0) continue;
      uint4* out = xp + (int64_t)d * row_chunks;
#pragma unroll
      for (int u = 0; u < CP_UNROLL; ++u) {
        const int i = base + u * 64 + lane;
        if (i < row_chunks) out[i] = v[u];
      }
    }
  }
}

// Layout statistics (no rows written): per chunk the same ranks and kept flags as
// disp_layout, then per token its distinct target chips among kept pairs.
//   tokens_to[i][j] += 1 per distinct target chip j of a token of chip i,
//   recv[j] += 1 per kept pair on chip j, hist[f] += 1 for a token reaching f chips.
__global__ __launch_bounds__(CH) void disp_stats(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ chunk_base, int T, int K,
    int E, int El, int64_t cap, int64_t tpr, int N, unsigned long long* __restrict__ tokens_to,
    unsigned long long* __restrict__ recv, unsigned long long* __restrict__ hist) {
  __shared__ unsigned long long masks[CH / 64][512];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x;
  const int64_t t = (int64_t)c * CH + tid;
  for (int i = tid; i < (CH / 64) * E; i += CH) masks[i / E][i % E] = 0ull;
  __syncthreads();
  int ev[16];
  load_pair_ids(ids, t, T, K, E, ev);
#pragma unroll
  for (int k = 0; k < 16; ++k)
    if (k < K && ev[k] >= 0) atomicOr(&masks[wave][ev[k]], 1ull << lane);
  __syncthreads();
  if (t >= T) return;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int dst[16];
  for (int k = 0; k < K; ++k) {
    const int e = ev[k];
    dst[k] = -1;
    if (e < 0) continue;
    int rank = chunk_base[(size_t)c * E + e] + __popcll(masks[wave][e] & below);
    for (int w = 0; w < wave; ++w) rank += __popcll(masks[w][e]);
    if (cap < 0 || rank < cap) {
      dst[k] = e / El;
      if (recv) atomicAdd(&recv[dst[k]], 1ull);
    }
  }
  int fan = 0;
  for (int k = 0; k < K; ++k) {
    if (dst[k] < 0) continue;
    bool seen = false;
    for (int q = 0; q < k; ++q) seen = seen || dst[q] == dst[k];
    if (seen) continue;
    ++fan;
    if (tokens_to) atomicAdd(&tokens_to[(t / tpr) * N + dst[k]], 1ull);
  }
  if (hist) atomicAdd(&hist[fan], 1ull);
}

__global__ __launch_bounds__(256) void fill_zero_u64(unsigned long long* __restrict__ p,
                                                     int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0ull;
}

// One block: the largest of n values.
__global__ __launch_bounds__(256) void max_u64(const unsigned long long* __restrict__ v, int n,
                                               unsigned long long* __restrict__ out) {
  __shared__ unsigned long long m[256];
  unsigned long long x = 0ull;
  for (int i = threadIdx.x; i < n; i += 256) x = v[i] > x ? v[i] : x;
  m[threadIdx.x] = x;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s && m[threadIdx.x + s] > m[threadIdx.x]) m[threadIdx.x] = m[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = m[0];
}

}  // namespace

// The placement re-reads chunk_counts in every block: n_chunks * E values each, so the
// one-pass path is taken up to this product (for example 128 chunks of 256 tokens x 256
// experts); larger problems run histogram, one-block scan and layout as three kernels.
constexpr int64_t kPlaceMaxScan = 32768;

// Bytes one pair puts on the wire: its activation row, or with MX-FP8 expert weights the
// row's E4M3 codes and scale bytes (x is quantised before dispatch).
static int64_t send_row_bytes(const Dims& d) {
  return d.mx ? (int64_t)d.h + d.h / 32 : (int64_t)d.h * d.s;
}

int launch_dispatch(const moe_problem* p, const Dims& d, const void* x, const int32_t* ids,
                    int32_t* counts, int32_t* offsets, int32_t* dest_row, int32_t* row_src,
                    int64_t* send_bytes, int32_t* n_dropped, void* xp, char* ws,
                    const WsLayout& L, hipStream_t st, const FfnPrepArgs* ffn,
                    int counted_rows, const ReplicaArgs* rm) {
  const ReplicaArgs rmap = rm ? *rm : ReplicaArgs{};
  const int n_chunks = (int)((d.T + CH - 1) / CH);
  int32_t* chunk_counts = reinterpret_cast<int32_t*>(ws + L.chunk_counts);
  int32_t* chunk_base = reinterpret_cast<int32_t*>(ws + L.chunk_base);
  int32_t* kept = reinterpret_cast<int32_t*>(ws + L.kept);
  const int pad = p->pad_to_capacity;
  // LDS counters for the send matrix: the source ranks one chunk spans times N.
  int lds_span = 0;
  if (send_bytes && d.tpr > 0) {
    const int64_t span = (CH + d.tpr - 1) / d.tpr + 1;
    const int64_t s = span < d.N ? span : d.N;
    if (s * d.N <= 8192) lds_span = (int)s;
  }
  const size_t lds = (size_t)lds_span * d.N * sizeof(int);
  const int row_chunks = d.h * d.s / 16;
  // count rows: the router's (counted_rows tokens each) or disp_count's 256-token chunks
  int gtok = counted_rows > 0 ? counted_rows : CH;
  int64_t n_rows = (d.T + gtok - 1) / gtok;
  if (n_rows * d.E <= kPlaceMaxScan && n_chunks * (int64_t)d.E <= kPlaceMaxScan) {
    // the send matrix from the counts needs every row inside one source rank
    auto rows_in_one_rank = [&](int gt) { return d.tpr > 0 && (d.N == 1 || d.tpr % gt == 0); };
    // (with replicas a row's pairs spread over replicas on several ranks: atomics instead)
    const bool from_counts = send_bytes && !rmap.rep_start && rows_in_one_rank(gtok) &&
                             d.N * d.N <= 4096;
    if (counted_rows == 0 || (send_bytes && !from_counts)) {
      gtok = CH;
      n_rows = n_chunks;
      hipLaunchKernelGGL(disp_count, dim3((unsigned)(n_chunks > 0 ? n_chunks : 1)), dim3(CH),
                         0, st, ids, chunk_counts, (int)d.T, d.K, d.E, n_chunks, send_bytes,
                         d.N * d.N);
    }
    const bool counts_mode = send_bytes && !rmap.rep_start && rows_in_one_rank(gtok) &&
                             d.N * d.N <= 4096;
    const int send_mode = !send_bytes ? kSendNone : (counts_mode ? kSendFromCounts : kSendAtomic);
    const size_t plds = send_mode == kSendFromCounts ? (size_t)d.N * d.N * sizeof(int)
                        : (send_mode == kSendAtomic ? lds : 0);
    // blocks: one per chunk, and at least three so the send matrix (last block) and the
    // tile table (the one before) are derived beside block 0's outputs
    const int grid = n_chunks > 3 ? n_chunks : 3;
    hipLaunchKernelGGL(disp_place, dim3((unsigned)grid), dim3(CH), plds, st, ids, chunk_counts,
                       (int)n_rows, gtok, counts, offsets, kept, n_dropped, dest_row, row_src,
                       send_bytes, send_mode, (int)d.T, d.K, d.E, d.El, d.e0, d.cap, pad,
                       d.R_max, d.tpr, d.N, send_row_bytes(d), lds_span, grid - 1, ffn ? 1 : 0,
                       grid - 2, ffn ? *ffn : FfnPrepArgs{}, rmap);
    if (pad && xp && d.R_max > 0)   // zero the pad rows of xp
      hipLaunchKernelGGL(disp_fill, dim3((unsigned)((d.R_max + 3) / 4)), dim3(256), 0, st,
                         offsets, kept, row_src, static_cast<uint4*>(xp), d.R_max, d.El, d.e0,
                         d.cap, pad, row_chunks);
  } else {
    if (rmap.rep_start) return MOE_ERR_UNSUPPORTED;   // the map needs the one-pass placement
    if (n_chunks > 0)
      hipLaunchKernelGGL(disp_hist, dim3(n_chunks), dim3(CH), 0, st, ids, chunk_counts,
                         (int)d.T, d.K, d.E);
    hipLaunchKernelGGL(disp_scan, dim3(1), dim3(1024), 0, st, chunk_counts, chunk_base, counts,
                       kept, offsets, n_dropped, send_bytes, n_chunks, d.E, d.El, d.e0, d.cap,
                       pad, d.N);
    if (n_chunks > 0)
      hipLaunchKernelGGL(disp_layout, dim3(n_chunks), dim3(CH), lds, st, ids, chunk_base,
                         offsets, dest_row, row_src, send_bytes, (int)d.T, d.K, d.E, d.El, d.e0,
                         d.cap, d.tpr, d.N, send_row_bytes(d), lds_span);
    if (d.R_max > 0)
      hipLaunchKernelGGL(disp_fill, dim3((unsigned)((d.R_max + 3) / 4)), dim3(256), 0, st,
                         offsets, kept, row_src, static_cast<uint4*>(xp), d.R_max, d.El, d.e0,
                         d.cap, pad, row_chunks);
    if (hipGetLastError() != hipSuccess) return MOE_ERR_LAUNCH;
    if (ffn && launch_ffn_prep(*ffn, offsets, st) != MOE_OK) return MOE_ERR_LAUNCH;
  }
  if (x && xp && d.T > 0)
    hipLaunchKernelGGL(disp_copy,
                       dim3((unsigned)((d.T + 3) / 4),
                            (unsigned)((row_chunks + 64 * CP_UNROLL - 1) / (64 * CP_UNROLL))),
                       dim3(256), 0, st,
                       static_cast<const uint4*>(x), dest_row, static_cast<uint4*>(xp), (int)d.T,
                       d.K, row_chunks);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

int launch_layout_stats(const moe_problem* p, const Dims& d, const int32_t* ids,
                        int64_t* tokens_to, int64_t* recv_pairs, int64_t* fanout_hist,
                        int64_t* busiest, char* ws, const WsLayout& L, hipStream_t st) {
  const int n_chunks = (int)((d.T + CH - 1) / CH);
  int32_t* chunk_counts = reinterpret_cast<int32_t*>(ws + L.chunk_counts);
  int32_t* chunk_base = reinterpret_cast<int32_t*>(ws + L.chunk_base);
  int32_t* kept = reinterpret_cast<int32_t*>(ws + L.kept);
  // counts, offsets and dropped of the scan go to scratch: only the ranks are needed
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.stats);
  int32_t* offsets = counts + d.E;
  int32_t* dropped = offsets + d.El + 1;
  unsigned long long* recv = reinterpret_cast<unsigned long long*>(recv_pairs);
  if (busiest && !recv)   // the maximum needs the per-chip loads: keep them in scratch
    recv = reinterpret_cast<unsigned long long*>(ws + L.stats + L.stats_recv);
  auto zero = [&](void* q, int64_t n) {
    if (q && n > 0)
      hipLaunchKernelGGL(fill_zero_u64, dim3((unsigned)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024)),
                         dim3(256), 0, st, static_cast<unsigned long long*>(q), n);
  };
  zero(tokens_to, (int64_t)d.N * d.N);
  zero(recv, d.N);
  zero(fanout_hist, d.K + 1);
  if (n_chunks > 0) {
    hipLaunchKernelGGL(disp_hist, dim3(n_chunks), dim3(CH), 0, st, ids, chunk_counts, (int)d.T,
                       d.K, d.E);
    hipLaunchKernelGGL(disp_scan, dim3(1), dim3(1024), 0, st, chunk_counts, chunk_base, counts,
                       kept, offsets, dropped, static_cast<int64_t*>(nullptr), n_chunks, d.E,
                       d.El, d.e0, d.cap, 0, d.N);
    hipLaunchKernelGGL(disp_stats, dim3(n_chunks), dim3(CH), 0, st, ids, chunk_base, (int)d.T,
                       d.K, d.E, d.El, d.cap, d.tpr, d.N,
                       reinterpret_cast<unsigned long long*>(tokens_to), recv,
                       reinterpret_cast<unsigned long long*>(fanout_hist));
  }
  if (busiest)
    hipLaunchKernelGGL(max_u64, dim3(1), dim3(256), 0, st, recv, d.N,
                       reinterpret_cast<unsigned long long*>(busiest));
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // namespace moe
