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
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int CH = kDispatchChunk;   // tokens per chunk (= threads per block)

__global__ __launch_bounds__(CH) void disp_hist(const int32_t* __restrict__ ids,
                                                int32_t* __restrict__ chunk_counts, int T,
                                                int K, int E) {
  __shared__ int cnt[512];
  const int c = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += CH) cnt[e] = 0;
  __syncthreads();
  const int64_t t = (int64_t)c * CH + threadIdx.x;
  if (t < T) {
    for (int k = 0; k < K; ++k) {
      const int e = ids[t * K + k];
      if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
  }
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
  for (int k = 0; k < K; ++k) {
    int e = t < T ? ids[t * K + k] : -1;
    if (e < 0 || e >= E) e = -1;
    ev[k] = e;
    if (e >= 0) atomicOr(&masks[wave][e], 1ull << lane);
  }
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
  int dst[16];
  int nd = 0;
  for (int k = 0; k < K; ++k) {
    const int d = dest_row[t * K + k];
    if (d >= 0) dst[nd++] = d;
  }
  if (nd == 0) return;
  const uint4* src = x + t * row_chunks;
  {
    const int base = blockIdx.y * 64 * CP_UNROLL;   // this wave's row segment
    uint4 v[CP_UNROLL];
#pragma unroll
    for (int u = 0; u < CP_UNROLL; ++u) {
      const int i = base + u * 64 + lane;
      if (i < row_chunks) v[u] = src[i];
    }
    for (int j = 0; j < nd; ++j) {
      uint4* out = xp + (int64_t)dst[j] * row_chunks;
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
  for (int k = 0; k < K; ++k) {
    int e = t < T ? ids[t * K + k] : -1;
    if (e < 0 || e >= E) e = -1;
    ev[k] = e;
    if (e >= 0) atomicOr(&masks[wave][e], 1ull << lane);
  }
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

int launch_dispatch(const moe_problem* p, const Dims& d, const void* x, const int32_t* ids,
                    int32_t* counts, int32_t* offsets, int32_t* dest_row, int32_t* row_src,
                    int64_t* send_bytes, int32_t* n_dropped, void* xp, char* ws,
                    const WsLayout& L, hipStream_t st) {
  const int n_chunks = (int)((d.T + CH - 1) / CH);
  int32_t* chunk_counts = reinterpret_cast<int32_t*>(ws + L.chunk_counts);
  int32_t* chunk_base = reinterpret_cast<int32_t*>(ws + L.chunk_base);
  int32_t* kept = reinterpret_cast<int32_t*>(ws + L.kept);
  const int pad = p->pad_to_capacity;
  if (n_chunks > 0)
    hipLaunchKernelGGL(disp_hist, dim3(n_chunks), dim3(CH), 0, st, ids, chunk_counts, (int)d.T,
                       d.K, d.E);
  hipLaunchKernelGGL(disp_scan, dim3(1), dim3(1024), 0, st, chunk_counts, chunk_base, counts,
                     kept, offsets, n_dropped, send_bytes, n_chunks, d.E, d.El, d.e0, d.cap, pad,
                     d.N);
  if (n_chunks > 0) {
    // LDS counters for the send matrix: the source ranks one chunk spans times N.
    int lds_span = 0;
    if (send_bytes && d.tpr > 0) {
      const int64_t span = (CH + d.tpr - 1) / d.tpr + 1;
      const int64_t s = span < d.N ? span : d.N;
      if (s * d.N <= 8192) lds_span = (int)s;
    }
    const size_t lds = (size_t)lds_span * d.N * sizeof(int);
    hipLaunchKernelGGL(disp_layout, dim3(n_chunks), dim3(CH), lds, st, ids, chunk_base, offsets,
                       dest_row, row_src, send_bytes, (int)d.T, d.K, d.E, d.El, d.e0, d.cap,
                       d.tpr, d.N, (int64_t)d.h * d.s, lds_span);
  }
  const int row_chunks = d.h * d.s / 16;
  if (d.R_max > 0)
    hipLaunchKernelGGL(disp_fill, dim3((unsigned)((d.R_max + 3) / 4)), dim3(256), 0, st, offsets,
                       kept, row_src, static_cast<uint4*>(xp), d.R_max, d.El, d.e0, d.cap, pad,
                       row_chunks);
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
