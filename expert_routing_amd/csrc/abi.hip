// C ABI: validation, sizing, the stage entry points, the whole-layer forward (optionally
// traced) and the layout statistics. Host code only; the kernels live in route.hip,
// dispatch.hip, ffn.hip and combine.hip.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "ffn_sched.h"

namespace moe {

static bool cap_exact(double cf, int64_t T, int K, int E, int64_t* cap) {
  // cap = ceil(cf * T * K / E) on the exact binary value of cf.
  if (!(cf > 0.0)) { *cap = -1; return true; }
  if (!isfinite(cf)) return false;
  int e2 = 0;
  double f = frexp(cf, &e2);                       // cf = f * 2^e2, f in [0.5, 1)
  int64_t m = (int64_t)ldexp(f, 53);               // exact 53-bit integer
  int sh = e2 - 53;                                 // cf = m * 2^sh
  unsigned __int128 num = (unsigned __int128)m * (unsigned __int128)T * (unsigned __int128)K;
  unsigned __int128 den = (unsigned __int128)E;
  if (sh >= 0) {
    if (sh > 20) return false;                     // cf >= 2^73: no meaningful cap
    num <<= sh;                                    // num < 2^108
  } else {
    const int r = -sh;
    // num < 2^88 (m < 2^53, T*K < 2^31, + 2^4 slack); E*2^r < 2^120 for r <= 110
    if (r > 110) { *cap = (num == 0) ? 0 : 1; return true; }
    den <<= r;
  }
  unsigned __int128 c = (num + den - 1) / den;
  if (c > (unsigned __int128)INT64_MAX) return false;
  *cap = (int64_t)c;
  return true;
}

int make_dims(const moe_problem* p, Dims* d) {
  if (!p) return MOE_ERR_INVALID;
  if (p->T < 0 || p->h <= 0 || p->E < 1 || p->E > 512) return MOE_ERR_INVALID;
  if (p->K < 1 || p->K > p->E || p->K > 16) return MOE_ERR_INVALID;
  if (p->score != MOE_SCORE_SOFTMAX && p->score != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID;
  if (p->renorm != 0 && p->renorm != 1) return MOE_ERR_INVALID;
  if (p->n_ep < 1 || p->E % p->n_ep != 0) return MOE_ERR_INVALID;
  if (p->ep_rank < 0 || p->ep_rank >= p->n_ep) return MOE_ERR_INVALID;
  if (p->n_groups < 1 || p->E % p->n_groups != 0) return MOE_ERR_INVALID;
  if (p->topk_groups < 1 || p->topk_groups > p->n_groups) return MOE_ERR_INVALID;
  if ((int64_t)p->topk_groups * (p->E / p->n_groups) < p->K) return MOE_ERR_INVALID;
  if (p->act_dtype != MOE_DTYPE_F32 && p->act_dtype != MOE_DTYPE_BF16 &&
      p->act_dtype != MOE_DTYPE_MXFP8 && p->act_dtype != MOE_DTYPE_BF16_PACKED)
    return MOE_ERR_INVALID;
  if (p->n_shared != 0 && p->n_shared != 1) return MOE_ERR_INVALID;
  if (p->inter < 0 || p->shared_inter < 0) return MOE_ERR_INVALID;
  if (p->n_shared == 1 && (p->shared_inter <= 0 || p->T % p->n_ep != 0)) return MOE_ERR_INVALID;
  if (p->pad_to_capacity != 0 && p->pad_to_capacity != 1) return MOE_ERR_INVALID;
  int64_t cap = -1;
  if (!cap_exact(p->capacity_factor, p->T, p->K, p->E, &cap)) return MOE_ERR_UNSUPPORTED;
  if (p->pad_to_capacity && cap < 0) return MOE_ERR_INVALID;
  const bool mx = p->act_dtype == MOE_DTYPE_MXFP8;
  const bool pk = p->act_dtype == MOE_DTYPE_BF16_PACKED;
  const bool bf16 = p->act_dtype == MOE_DTYPE_BF16 || mx || pk;
  if (mx && (p->h % 128 != 0 || p->inter % 128 != 0 || p->shared_inter % 128 != 0))
    return MOE_ERR_UNSUPPORTED;   // 128-value k-steps: four scale blocks per row and step
  if (bf16) {
    if (p->h % 64 != 0 || p->inter % 64 != 0 || p->shared_inter % 64 != 0)
      return MOE_ERR_UNSUPPORTED;
  } else {
    if (p->h % 4 != 0) return MOE_ERR_UNSUPPORTED;
  }
  if (p->T * (int64_t)p->K >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  if (p->n_ep > 1024) return MOE_ERR_UNSUPPORTED;
  d->T = p->T; d->h = p->h; d->E = p->E; d->K = p->K;
  d->N = p->n_ep; d->rank = p->ep_rank;
  d->El = p->E / p->n_ep; d->e0 = p->ep_rank * d->El;
  d->cap = cap;
  const int64_t per_tok = p->K < d->El ? p->K : d->El;
  int64_t rmax = p->T * per_tok;
  if (cap >= 0) {
    const int64_t capped = (int64_t)d->El * cap;
    rmax = p->pad_to_capacity ? capped : (capped < rmax ? capped : rmax);
  }
  if (rmax >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  if (bf16) {
    // the bf16 GEMMs address each operand with 32-bit byte offsets (buffer descriptors):
    // x and one expert's row block (at most T rows, a token names an expert once; cap
    // rows when padding), weight blocks of 2*inter rows
    int64_t lead = p->h > p->inter ? p->h : p->inter;
    lead = lead > p->shared_inter ? lead : p->shared_inter;
    const int64_t rows = (p->pad_to_capacity && cap > p->T) ? cap : p->T;
    const int64_t wrows = 2 * (int64_t)(p->inter > p->shared_inter ? p->inter : p->shared_inter);
    if ((rows + 1) * lead * 2 >= (int64_t)1 << 32 || wrows * p->h * 2 >= (int64_t)1 << 32)
      return MOE_ERR_UNSUPPORTED;
  }
  d->R_max = rmax;
  d->tpr = (p->T % p->n_ep == 0) ? p->T / p->n_ep : 0;
  d->sh_rows = p->n_shared ? d->tpr : 0;
  d->s = bf16 ? 2 : 4;
  d->bf16 = bf16;
  d->mx = mx;
  d->pk = pk;
  d->route_split = route_split(*d);
  return MOE_OK;
}

int make_dims_replicated(const moe_problem* p, int P, Dims* d) {
  int st = make_dims(p, d);
  if (st != MOE_OK) return st;
  if (P < p->E || P % p->n_ep != 0) return MOE_ERR_INVALID;
  if (p->pad_to_capacity) return MOE_ERR_UNSUPPORTED;
  const int Pl = P / p->n_ep;
  if (Pl > 512 || P > 8192) return MOE_ERR_UNSUPPORTED;
  // the placement derives the scan in every block: the one-pass bound on count rows
  const int64_t rows256 = (p->T + kDispatchChunk - 1) / kDispatchChunk;
  const int rt = route_count_tokens(*d);
  const int64_t rows_rt = (p->T + rt - 1) / rt;
  if ((rows256 > rows_rt ? rows256 : rows_rt) * p->E > 32768) return MOE_ERR_UNSUPPORTED;
  int64_t cap = -1;
  if (!cap_exact(p->capacity_factor, p->T, p->K, P, &cap)) return MOE_ERR_UNSUPPORTED;
  d->El = Pl;
  d->e0 = p->ep_rank * Pl;
  d->cap = cap;
  const int64_t per_tok = p->K < Pl ? p->K : Pl;
  int64_t rmax = p->T * per_tok;
  if (cap >= 0 && (int64_t)Pl * cap < rmax) rmax = (int64_t)Pl * cap;
  if (rmax >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  d->R_max = rmax;
  return MOE_OK;
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

WsLayout ws_layout(const moe_problem* p, const Dims& d) {
  WsLayout L;
  size_t off = 0;
  const size_t n_chunks = (size_t)((d.T + kDispatchChunk - 1) / kDispatchChunk);
  // pair-count rows: dispatch's 256-token chunks, or the router's smaller token groups
  const int rt = route_count_tokens(d);
  const size_t n_count_rows = std::max(n_chunks, (size_t)((d.T + rt - 1) / rt));
  L.logits = off;       off = align256(off + (size_t)d.route_split * d.T * d.E * 4);
  L.chunk_counts = off; off = align256(off + n_count_rows * d.E * 4);
  L.chunk_base = off;   off = align256(off + n_chunks * d.E * 4);
  L.kept = off;         off = align256(off + (size_t)d.E * 4);
  L.sched = off;        off = align256(off + ffn_sched_bytes(d));
  const int imax = p->inter > p->shared_inter ? p->inter : p->shared_inter;
  if (d.mx) {
    L.hbuf = off;       off = align256(off + (size_t)(d.R_max + d.sh_rows) * imax);
    L.hbuf_s = off;     off = align256(off + (size_t)(d.R_max + d.sh_rows) * (imax / 32));
    L.xq = off;         off = align256(off + (size_t)d.T * d.h);
    L.xs = off;         off = align256(off + (size_t)d.T * (d.h / 32));
  } else {
    L.hbuf = off;       off = align256(off + (size_t)(d.R_max + d.sh_rows) * imax * d.s);
    L.hbuf_s = L.xq = L.xs = 0;
  }
  L.splitk = off;       off = align256(off + ffn_splitk_bytes(d));
  L.arrive = off;       off = align256(off + ffn_arrive_bytes(d));
  L.stats_recv = align256((size_t)(d.E + d.El + 2) * 4);
  L.stats = off;        off = align256(off + L.stats_recv + (size_t)d.N * 8);
  L.total = off;
  return L;
}

static int check_ws(const moe_problem* p, const Dims& d, void* ws, size_t ws_bytes) {
  if (!ws || ((uintptr_t)ws & 255)) return MOE_ERR_WORKSPACE;
  if (ws_bytes < ws_layout(p, d).total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

int moe_check_problem(const moe_problem* p) {
  Dims d;
  return make_dims(p, &d);
}

int moe_capacity(const moe_problem* p, int64_t* cap) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (!cap) return MOE_ERR_INVALID;
  *cap = d.cap;
  return MOE_OK;
}

int moe_max_rows(const moe_problem* p, int64_t* rows) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (!rows) return MOE_ERR_INVALID;
  *rows = d.R_max;
  return MOE_OK;
}

int moe_workspace_bytes(const moe_problem* p, size_t* bytes) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID;
  *bytes = ws_layout(p, d).total;
  return MOE_OK;
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape";
    case MOE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"

// Argument checks of each stage (host only, nothing enqueued).
namespace moe {
static int v_route(const moe_problem* p, const Dims& d, const void* x, const float* w_router,
                   const int32_t* ids, const float* w, void* ws, size_t ws_bytes) {
  if (d.T == 0) return MOE_OK;
  if (!x || !w_router || !ids || !w) return MOE_ERR_INVALID;
  return check_ws(p, d, ws, ws_bytes);
}
static int v_dispatch(const moe_problem* p, const Dims& d, const void* x, const int32_t* ids,
                      const int32_t* counts, const int32_t* offsets, const int32_t* dest_row,
                      const int32_t* row_src, const int64_t* send_bytes, const int32_t* n_dropped,
                      const void* xp, void* ws, size_t ws_bytes) {
  if (!counts || !offsets || !n_dropped) return MOE_ERR_INVALID;
  if (d.T > 0 && (!ids || !dest_row)) return MOE_ERR_INVALID;
  if (d.R_max > 0 && !row_src) return MOE_ERR_INVALID;
  if ((x == nullptr) != (xp == nullptr)) return MOE_ERR_INVALID;
  if (send_bytes && d.tpr == 0 && d.T > 0) return MOE_ERR_INVALID;
  return check_ws(p, d, ws, ws_bytes);
}
static int v_ffn(const moe_problem* p, const Dims& d, const void* xp, const int32_t* offsets,
                 const void* w13, const void* w2, const void* x, const void* w13_sh,
                 const void* w2_sh, const void* yp, const void* y_sh, void* ws, size_t ws_bytes,
                 bool gather = false) {
  if (p->inter <= 0) return MOE_ERR_INVALID;
  if (!offsets || !w13 || !w2) return MOE_ERR_INVALID;
  if (d.R_max > 0 && ((!xp && !gather) || !yp)) return MOE_ERR_INVALID;
  if (p->n_shared) {
    if (d.sh_rows > 0 && (!x || !w13_sh || !w2_sh || !y_sh)) return MOE_ERR_INVALID;
  } else if (w13_sh || w2_sh || y_sh) {
    return MOE_ERR_INVALID;
  }
  return check_ws(p, d, ws, ws_bytes);
}
static int v_combine(const moe_problem* p, const Dims& d, const void* yp, const int32_t* dest_row,
                     const float* w, const void* y_sh, const void* y) {
  if (d.T == 0) return MOE_OK;
  if (!dest_row || !w || !y) return MOE_ERR_INVALID;
  if (d.R_max > 0 && !yp) return MOE_ERR_INVALID;
  if (y_sh && !p->n_shared) return MOE_ERR_INVALID;
  if (p->n_shared && d.sh_rows > 0 && !y_sh) return MOE_ERR_INVALID;
  return MOE_OK;
}
}  // namespace moe

extern "C" {

int moe_route(const moe_problem* p, const void* x, const float* w_router, const float* bias,
              int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if ((st = v_route(p, d, x, w_router, topk_ids, topk_w, ws, ws_bytes)) != MOE_OK) return st;
  if (d.T == 0) return MOE_OK;
  WsLayout L = ws_layout(p, d);
  return launch_route(p, d, x, w_router, bias, topk_ids, topk_w,
                      (float*)((char*)ws + L.logits), nullptr, (hipStream_t)stream);
}

int moe_select(const moe_problem* p, const float* logits, const float* bias,
               int32_t* topk_ids, float* topk_w, void* stream) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (d.T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_w) return MOE_ERR_INVALID;
  return launch_select(p, d, logits, bias, topk_ids, topk_w, (hipStream_t)stream);
}

int moe_dispatch(const moe_problem* p, const void* x, const int32_t* topk_ids,
                 int32_t* counts, int32_t* offsets, int32_t* dest_row, int32_t* row_src,
                 int64_t* send_bytes, int32_t* n_dropped, void* xp,
                 void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if ((st = v_dispatch(p, d, x, topk_ids, counts, offsets, dest_row, row_src, send_bytes,
                       n_dropped, xp, ws, ws_bytes)) != MOE_OK)
    return st;
  WsLayout L = ws_layout(p, d);
  return launch_dispatch(p, d, x, topk_ids, counts, offsets, dest_row, row_src, send_bytes,
                         n_dropped, xp, (char*)ws, L, (hipStream_t)stream);
}

int moe_expert_ffn(const moe_problem* p, const void* xp, const int32_t* row_src,
                   const int32_t* offsets, const void* w13, const void* w2, const void* x,
                   const void* w13_sh, const void* w2_sh, void* yp, void* y_sh,
                   void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (d.mx) return MOE_ERR_UNSUPPORTED;   // the weight scales travel in moe_tensors
  // no xp: the gate/up GEMM gathers its rows from x through row_src
  const bool gather = xp == nullptr;
  if (gather && d.R_max > 0 && (!row_src || !x)) return MOE_ERR_INVALID;
  if ((st = v_ffn(p, d, xp, offsets, w13, w2, x, w13_sh, w2_sh, yp, y_sh, ws, ws_bytes,
                  gather)) != MOE_OK)
    return st;
  WsLayout L = ws_layout(p, d);
  return launch_ffn(p, d, xp, offsets, w13, w2, x, w13_sh, w2_sh, yp, y_sh, (char*)ws, L,
                    (hipStream_t)stream, nullptr, gather ? row_src : nullptr);
}

int moe_combine(const moe_problem* p, const void* yp, const int32_t* dest_row,
                const float* topk_w, const void* y_sh, void* y, void* stream) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if ((st = v_combine(p, d, yp, dest_row, topk_w, y_sh, y)) != MOE_OK) return st;
  if (d.T == 0) return MOE_OK;
  return launch_combine(p, d, yp, dest_row, topk_w, y_sh, y, (hipStream_t)stream);
}

int moe_layout_stats(const moe_problem* p, const int32_t* topk_ids, int64_t* tokens_to,
                     int64_t* recv_pairs, int64_t* fanout_hist, int64_t* busiest, void* ws,
                     size_t ws_bytes, void* stream) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (d.T > 0 && !topk_ids) return MOE_ERR_INVALID;
  if (tokens_to && d.T > 0 && d.tpr == 0) return MOE_ERR_INVALID;   // T % n_ep != 0
  if ((st = check_ws(p, d, ws, ws_bytes)) != MOE_OK) return st;
  const WsLayout L = ws_layout(p, d);
  return launch_layout_stats(p, d, topk_ids, tokens_to, recv_pairs, fanout_hist, busiest,
                             (char*)ws, L, (hipStream_t)stream);
}

static int forward_impl(const moe_problem* p, const moe_tensors* t, void* ws, size_t ws_bytes,
                        void* stream, void* const* events,
                        const moe_replica_map* map = nullptr) {
  if (!t) return MOE_ERR_INVALID;
  Dims d;
  int st = map ? make_dims_replicated(p, map->P, &d) : make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (map && (!map->rep_start || !map->rep_list || !map->phys_expert || !map->phys_replica))
    return MOE_ERR_INVALID;
  if (p->inter <= 0 || (d.T > 0 && !t->x)) return MOE_ERR_INVALID;
  // No xp: the row copy is skipped and the gate/up GEMM reads x through row_src.
  const bool gather = t->xp == nullptr;
  if (events) {
    for (int i = 0; i < MOE_TRACE_POINTS; ++i)
      if (!events[i]) return MOE_ERR_INVALID;
  }
  // Check every stage before the first launch, so an error enqueues nothing.
  if ((st = v_route(p, d, t->x, t->w_router, t->topk_ids, t->topk_w, ws, ws_bytes)) != MOE_OK ||
      (st = v_dispatch(p, d, gather ? nullptr : t->x, t->topk_ids, t->counts, t->offsets,
                       t->dest_row, t->row_src, t->send_bytes, t->n_dropped, t->xp, ws,
                       ws_bytes)) != MOE_OK ||
      (st = v_ffn(p, d, t->xp, t->offsets, t->w13, t->w2, t->x, t->w13_sh, t->w2_sh, t->yp,
                  t->y_sh, ws, ws_bytes, gather)) != MOE_OK ||
      (st = v_combine(p, d, t->yp, t->dest_row, t->topk_w, t->y_sh, t->y)) != MOE_OK)
    return st;
  if (d.mx) {
    if (!t->w13_scale || !t->w2_scale) return MOE_ERR_INVALID;
    if (p->n_shared && d.sh_rows > 0 && (!t->w13_sh_scale || !t->w2_sh_scale))
      return MOE_ERR_INVALID;
  } else if (t->w13_scale || t->w2_scale || t->w13_sh_scale || t->w2_sh_scale) {
    return MOE_ERR_INVALID;
  }
  const hipStream_t s = (hipStream_t)stream;
  hipEvent_t const* ev = reinterpret_cast<hipEvent_t const*>(events);
  auto mark = [&](int i) {
    return !ev || hipEventRecord(ev[i], s) == hipSuccess;
  };
  const WsLayout L = ws_layout(p, d);
  char* w = (char*)ws;
  if (!mark(MOE_TRACE_BEGIN)) return MOE_ERR_LAUNCH;
  // the router also leaves dispatch's pair counts in the workspace
  int32_t* chunk_counts = reinterpret_cast<int32_t*>(w + L.chunk_counts);
  if (d.T > 0 && (st = launch_route(p, d, t->x, t->w_router, t->bias, t->topk_ids, t->topk_w,
                                    (float*)(w + L.logits), chunk_counts, s)) != MOE_OK)
    return st;
  if (!mark(MOE_TRACE_ROUTE)) return MOE_ERR_LAUNCH;
  // dispatch also builds the expert FFN's tile table from the offsets it produces
  // MX-FP8: the gate/up GEMM always reads the token rows of x's E4M3 copy through row_src
  const bool gather_a = gather || d.mx;
  FfnPrepArgs fa;
  if ((st = ffn_prep_args(p, d, t->xp, t->w13, t->w2, t->x, t->w13_sh, t->w2_sh, t->yp,
                          t->y_sh, w, L, gather_a ? t->row_src : nullptr, &fa)) != MOE_OK)
    return st;
  if (d.mx) {
    fa.w13_s = reinterpret_cast<const char*>(t->w13_scale);
    fa.w2_s = reinterpret_cast<const char*>(t->w2_scale);
    fa.w13_sh_s = reinterpret_cast<const char*>(t->w13_sh_scale);
    fa.w2_sh_s = reinterpret_cast<const char*>(t->w2_sh_scale);
    // x quantised once per token (before dispatch: the rows a rank would send)
    if (d.T > 0 && (st = launch_mx_quant(t->x, true, d.T, d.h, (uint8_t*)(w + L.xq),
                                         (uint8_t*)(w + L.xs), s)) != MOE_OK)
      return st;
  }
  ReplicaArgs rm{};
  if (map) {
    rm = ReplicaArgs{map->rep_start, map->rep_list, map->phys_expert, map->phys_replica,
                     map->P, nullptr};
    fa.phys_expert = map->phys_expert;   // each physical expert runs its logical weights
  }
  if ((st = launch_dispatch(p, d, gather ? nullptr : t->x, t->topk_ids, t->counts, t->offsets,
                            t->dest_row, t->row_src, t->send_bytes, t->n_dropped, t->xp, w, L,
                            s, &fa, route_count_tokens(d), map ? &rm : nullptr)) != MOE_OK)
    return st;
  if (!mark(MOE_TRACE_DISPATCH)) return MOE_ERR_LAUNCH;
  if ((st = launch_ffn(p, d, t->xp, t->offsets, t->w13, t->w2, t->x, t->w13_sh, t->w2_sh, t->yp,
                       t->y_sh, w, L, s, ev ? ev + MOE_TRACE_FFN_PREP : nullptr,
                       gather_a ? t->row_src : nullptr, &fa)) != MOE_OK)
    return st;
  if (d.T > 0 && (st = launch_combine(p, d, t->yp, t->dest_row, t->topk_w, t->y_sh, t->y, s)) !=
                     MOE_OK)
    return st;
  if (!mark(MOE_TRACE_COMBINE)) return MOE_ERR_LAUNCH;
  return MOE_OK;
}

int moe_forward(const moe_problem* p, const moe_tensors* t, void* ws, size_t ws_bytes,
                void* stream) {
  return forward_impl(p, t, ws, ws_bytes, stream, nullptr);
}

int moe_forward_traced(const moe_problem* p, const moe_tensors* t, void* ws, size_t ws_bytes,
                       void* stream, void* const* events) {
  if (!events) return MOE_ERR_INVALID;
  return forward_impl(p, t, ws, ws_bytes, stream, events);
}

int moe_quantize_mx(int64_t rows, int32_t cols, int32_t src_dtype, const void* src,
                    uint8_t* codes, uint8_t* scales, void* stream) {
  if (rows < 0 || cols <= 0 || cols % 32 != 0) return MOE_ERR_INVALID;
  if (src_dtype != MOE_DTYPE_F32 && src_dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID;
  if (rows > 0 && (!src || !codes || !scales)) return MOE_ERR_INVALID;
  if (rows * (int64_t)cols / 32 >= ((int64_t)1 << 40)) return MOE_ERR_UNSUPPORTED;
  return launch_mx_quant(src, src_dtype == MOE_DTYPE_BF16, rows, cols, codes, scales,
                         (hipStream_t)stream);
}

int moe_pack_weights(int64_t mats, int32_t rows, int32_t cols, const void* src, void* dst,
                     void* stream) {
  if (mats < 0 || rows <= 0 || cols <= 0) return MOE_ERR_INVALID;
  if (rows % 32 != 0 || cols % 16 != 0) return MOE_ERR_INVALID;
  if (mats == 0) return MOE_OK;
  if (!src || !dst) return MOE_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 != 0)
    return MOE_ERR_INVALID;
  if ((int64_t)rows * cols >= ((int64_t)1 << 40) / mats) return MOE_ERR_UNSUPPORTED;
  const uintptr_t bytes = (uintptr_t)(mats * rows * (int64_t)cols * 2);
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a < b + bytes && b < a + bytes) return MOE_ERR_INVALID;   // overlapping
  return launch_pack_weights(mats, rows, cols, src, dst, (hipStream_t)stream);
}

int moe_replicated_sizes(const moe_problem* p, int32_t P, int64_t* max_rows, size_t* ws_bytes) {
  Dims d;
  int st = make_dims_replicated(p, P, &d);
  if (st != MOE_OK) return st;
  if (!max_rows || !ws_bytes) return MOE_ERR_INVALID;
  *max_rows = d.R_max;
  *ws_bytes = ws_layout(p, d).total;
  return MOE_OK;
}

int moe_dispatch_replicated(const moe_problem* p, const moe_replica_map* map,
                            const int32_t* topk_ids, int32_t* counts, int32_t* phys_counts,
                            int32_t* offsets, int32_t* dest_row, int32_t* row_src,
                            int64_t* send_bytes, int32_t* n_dropped, void* ws, size_t ws_bytes,
                            void* stream) {
  if (!map) return MOE_ERR_INVALID;
  Dims d;
  int st = make_dims_replicated(p, map->P, &d);
  if (st != MOE_OK) return st;
  if (!map->rep_start || !map->rep_list || !map->phys_expert || !map->phys_replica)
    return MOE_ERR_INVALID;
  if ((st = v_dispatch(p, d, nullptr, topk_ids, counts, offsets, dest_row, row_src, send_bytes,
                       n_dropped, nullptr, ws, ws_bytes)) != MOE_OK)
    return st;
  const WsLayout L = ws_layout(p, d);
  const ReplicaArgs rm{map->rep_start, map->rep_list, map->phys_expert, map->phys_replica,
                       map->P, phys_counts};
  return launch_dispatch(p, d, nullptr, topk_ids, counts, offsets, dest_row, row_src,
                         send_bytes, n_dropped, nullptr, (char*)ws, L, (hipStream_t)stream,
                         nullptr, 0, &rm);
}

int moe_forward_replicated(const moe_problem* p, const moe_replica_map* map,
                           const moe_tensors* t, void* ws, size_t ws_bytes, void* stream) {
  if (!map) return MOE_ERR_INVALID;
  return forward_impl(p, t, ws, ws_bytes, stream, nullptr, map);
}

int moe_replica_plan(int32_t E, int32_t R, int32_t n_ep, const int64_t* load, int32_t* counts,
                     int32_t* rep_start, int32_t* rep_list, int32_t* phys_expert,
                     int32_t* phys_replica) {
  if (E < 1 || E > 512 || R < 0 || n_ep < 1 || (E + R) % n_ep != 0 || E + R > 8192)
    return MOE_ERR_INVALID;
  if (!load || !counts || !rep_start || !rep_list || !phys_expert || !phys_replica)
    return MOE_ERR_INVALID;
  for (int e = 0; e < E; ++e)
    if (load[e] < 0 || load[e] > INT32_MAX) return MOE_ERR_INVALID;
  const int P = E + R, per = P / n_ep;
  // replica counts: each redundant slot to the largest load per replica, ties to lower id
  for (int e = 0; e < E; ++e) counts[e] = 1;
  for (int slot = 0; slot < R; ++slot) {
    int best = 0;
    for (int e = 1; e < E; ++e)
      if (load[e] * counts[best] > load[best] * counts[e]) best = e;
    ++counts[best];
  }
  rep_start[0] = 0;
  for (int e = 0; e < E; ++e) rep_start[e + 1] = rep_start[e] + counts[e];
  // packing: replicas by their pair share (descending; ties lower id, then lower replica)
  // onto the least loaded rank with a free slot (ties to the lower rank)
  struct Rep { int64_t w; int e, q; };
  Rep* reps = new Rep[P];
  int n = 0;
  for (int e = 0; e < E; ++e)
    for (int q = 0; q < counts[e]; ++q)
      reps[n++] = Rep{load[e] / counts[e] + (q < load[e] % counts[e] ? 1 : 0), e, q};
  std::sort(reps, reps + n, [](const Rep& a, const Rep& b) {
    if (a.w != b.w) return a.w > b.w;
    if (a.e != b.e) return a.e < b.e;
    return a.q < b.q;
  });
  int64_t* rank_load = new int64_t[n_ep]();
  int* fill = new int[n_ep]();
  for (int i = 0; i < n; ++i) {
    int best = -1;
    for (int j = 0; j < n_ep; ++j)
      if (fill[j] < per && (best < 0 || rank_load[j] < rank_load[best])) best = j;
    const int pid = best * per + fill[best]++;
    rank_load[best] += reps[i].w;
    phys_expert[pid] = reps[i].e;
    phys_replica[pid] = reps[i].q;
    rep_list[rep_start[reps[i].e] + reps[i].q] = pid;
  }
  delete[] reps;
  delete[] rank_load;
  delete[] fill;
  return MOE_OK;
}

}  // extern "C"

// ---- allocation-free forward --------------------------------------------------------
// The workspace of moe_forward_noalloc is this file-scope device array: every GPU the
// library runs on holds one copy (at its own address) until the process ends. In host
// code `scratch` names a host-side stand-in, so kernels get the device address found by
// hipGetSymbolAddress, once per device, with that device current.
namespace moe {
namespace {
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's scratch array (nullptr if the runtime refuses).
void* scratch_ptr(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!ptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}
}  // namespace
}  // namespace moe

extern "C" {

int moe_forward_noalloc(const moe_problem* p, const moe_tensors* t, void* stream) {
  Dims d;
  int st = make_dims(p, &d);
  if (st != MOE_OK) return st;
  if (ws_layout(p, d).total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_LAUNCH;
  void* ws = scratch_ptr(dev);
  if (!ws) return MOE_ERR_LAUNCH;
  return forward_impl(p, t, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

}  // extern "C"
