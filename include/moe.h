/*
 * moe.h - C ABI of an MI355X (gfx950) MoE-layer forward pass on one GPU's share of an
 * expert-parallel (EP) deployment: route -> dispatch -> expert FFN -> combine.
 *
 * The four stages are the ones the EP pages list for one MoE layer: the router scores
 * every expert for every token and keeps the top-K; dispatch regroups the tokens by
 * destination expert; each expert runs its FFN on the tokens it received; combine
 * returns the results to token order and sums them with the routing weights
 * ("总览" (EP chapter overview), section "MoE 路由机制是什么？top-K 怎么用？" and
 * glossary; "專家並行（Expert Parallelism, EP）", section "技術原理", steps 1-4).
 * Remote EP ranks appear only as virtual rank ids in the layout: nothing here talks
 * to another GPU.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller. The library
 *     allocates nothing, keeps no state between calls and never synchronises with the
 *     host: work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     outputs are valid once that stream has reached the call.
 *   - Row-major, densely packed arrays; shapes are given in brackets.
 *     "act" is the activation/expert-weight dtype selected by moe_problem.act_dtype
 *     (fp32, or bf16 stored as raw 16-bit words). Routing weights are always fp32.
 *   - Return value: MOE_OK, or a negative status. Arguments are validated on the host
 *     before anything is enqueued, so an error status means nothing was launched
 *     (MOE_ERR_LAUNCH excepted: the HIP runtime refused a launch).
 *   - Workspace: `ws` is device scratch of at least moe_workspace_bytes() bytes,
 *     256-byte aligned. Calls that run concurrently need distinct workspaces.
 *   - Values the library leaves undefined are said so per argument; everything else
 *     is written completely.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID = -1,     /* an argument breaks the problem's definition        */
  MOE_ERR_UNSUPPORTED = -2, /* a valid shape this build does not handle           */
  MOE_ERR_WORKSPACE = -3,   /* workspace missing, misaligned or too small         */
  MOE_ERR_LAUNCH = -4       /* the HIP runtime refused a kernel launch            */
};

enum moe_score { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 };
enum moe_dtype {
  MOE_DTYPE_F32 = 0,
  MOE_DTYPE_BF16 = 1,
  MOE_DTYPE_MXFP8 = 2,
  MOE_DTYPE_BF16_PACKED = 3
};

/*
 * The problem statement of one MoE layer call, in the pages' own quantities: T tokens
 * of hidden size h, E experts, top-K, a capacity factor, and E/N_EP local experts
 * ("总览" glossary: top-K, EP 度; "专家并行与 MoE", sections "MoE 结构回顾" and
 * "Expert Parallelism（EP）": each card holds E/N experts).
 *
 *  T            tokens routed in this call (>= 0)
 *  h            hidden size (> 0)
 *  E            routed experts in the layer (1..512)
 *  K            experts per token (1..min(E, 16))
 *  score        MOE_SCORE_SOFTMAX: key = logit = x.W_r + bias; weights = softmax of
 *                 the selected logits (= full softmax renormalised over the selection)
 *               MOE_SCORE_SIGMOID: s = sigmoid(x.W_r); key = s + bias (the bias only
 *                 steers selection, as aux-loss-free balancing does: "专家并行与 MoE",
 *                 section "负载均衡"); weights = s over the selection
 *  renorm       1: selected weights divided by their sum; 0: raw softmax / sigmoid
 *  n_groups     expert groups for group-limited routing ("总览" glossary "Expert
 *               group"); groups are contiguous blocks of E/n_groups experts; 1 = off
 *  topk_groups  groups a token may use (1..n_groups); a group's score is the sum of its
 *               two largest keys (its only key when a group has one expert)
 *  capacity_factor  <= 0: no limit. Otherwise cap = ceil(cf * T * K / E), computed
 *               exactly on the double's value ("專家並行", key parameters: capacity
 *               factor). Pairs beyond cap are dropped in token order, and a dropped
 *               pair adds nothing ("专家并行与 MoE": over-capacity tokens skip the
 *               expert).
 *  pad_to_capacity  1: every local expert owns exactly cap rows, unused rows zero
 *               ("专家并行与 MoE", section "负载均衡": drop or pad). Needs a capacity.
 *  n_ep, ep_rank  virtual EP ranks and the one this GPU plays. Local experts are
 *               [ep_rank*E/n_ep, (ep_rank+1)*E/n_ep) ("总览", "Dispatch 通信矩阵":
 *               chip = expert_id / experts-per-chip); token t sits on rank
 *               t / (T/n_ep) ("总览": 512 tokens over 64 chips, 8 per chip).
 *  inter        SwiGLU intermediate size of a routed expert (> 0 for the FFN)
 *  n_shared     0 or 1 shared expert, run on this rank's token block
 *               [ep_rank*T/n_ep, (ep_rank+1)*T/n_ep) ("总览" glossary "Expert":
 *               256 routed + 1 shared expert)
 *  shared_inter SwiGLU intermediate size of the shared expert
 *  act_dtype    MOE_DTYPE_F32 or MOE_DTYPE_BF16 (activations and expert weights;
 *               accumulation is fp32 either way), or MOE_DTYPE_MXFP8: activations
 *               (x, xp, yp, y_sh, y) bf16 and the expert weights MX-FP8 (E4M3 codes
 *               with E8M0 scales, see moe_quantize_mx). The expert FFN then runs on the
 *               FP8 matrix cores: x is quantised once per token before dispatch, the
 *               GEMMs apply the block scales inside the MFMA, and the gated product is
 *               quantised in the gate/up GEMM's epilogue ("Expert-Parallelism",
 *               关键观察 observation 3: quantise / dequantise passes cost as much as the
 *               GEMMs unless fused). Only moe_forward and its variants take it; the
 *               stage call moe_expert_ffn returns MOE_ERR_UNSUPPORTED.
 *               MOE_DTYPE_BF16_PACKED: bf16 throughout, as MOE_DTYPE_BF16, with the
 *               routed and shared expert weights (w13, w2, w13_sh, w2_sh) in the order
 *               moe_pack_weights writes. The GEMMs then load weight fragments straight
 *               into registers and keep the LDS for the token rows; results are the same
 *               as with MOE_DTYPE_BF16 on the unpacked weights up to fp32 summation order.
 */
typedef struct moe_problem {
  int64_t T;
  int32_t h, E, K;
  int32_t score;
  int32_t renorm;
  int32_t n_groups, topk_groups;
  double capacity_factor;
  int32_t pad_to_capacity;
  int32_t n_ep, ep_rank;
  int32_t inter, n_shared, shared_inter;
  int32_t act_dtype;
} moe_problem;

/* ---- host-only queries (no device work) ---------------------------------------- */

/* MOE_OK if the problem is valid and supported, else the status the calls return.
 * Invalid: T < 0, h <= 0, E not in 1..512, K not in 1..min(E,16), E % n_ep != 0,
 * ep_rank outside [0, n_ep), E % n_groups != 0, topk_groups outside 1..n_groups,
 * topk_groups*E/n_groups < K, padding without a capacity, n_shared not 0/1,
 * n_shared = 1 with T % n_ep != 0. Unsupported (MX-FP8): h, inter or shared_inter not a
 * multiple of 128, and the bf16 limits below; (bf16): h % 64 != 0, inter % 64 != 0,
 * shared_inter % 64 != 0, or operands beyond the GEMMs' 32-bit byte offsets:
 * (rows + 1) * max(h, inter, shared_inter) * 2 >= 2^32 with rows = T (the capacity when
 * padding to a larger one), or 2 * max(inter, shared_inter) * h * 2 >= 2^32;
 * (fp32): h % 4 != 0; both: T*K >= 2^31. */
int moe_check_problem(const moe_problem* p);

/* Capacity per expert in *cap (-1 when there is no limit). */
int moe_capacity(const moe_problem* p, int64_t* cap);

/* Rows of this rank's expert buffer the caller must allocate for xp / yp / row_src:
 * T*min(K, E_l) without capacity, E_l*cap padded, min(T*min(K,E_l), E_l*cap) else. */
int moe_max_rows(const moe_problem* p, int64_t* rows);

/* Workspace bytes that any entry point below needs for this problem. */
int moe_workspace_bytes(const moe_problem* p, size_t* bytes);

/* Static text for a status code. */
const char* moe_status_string(int status);

/* ---- stage 1: route --------------------------------------------------------------
 * Router scores, optional group limit, top-K, weights ("总览" glossary "Router";
 * "專家並行", "技術原理" step 1). Logits are computed in fp32 (bf16 activations are
 * exact in fp32; the fp32 router weight enters exactly, as three bf16 parts summed
 * into fp32 accumulators).
 *   x         [T][h] act
 *   w_router  [E][h] fp32 (one row per expert, as a Linear(h, E) weight)
 *   bias      [E] fp32 or NULL (meaning set by `score`)
 *   topk_ids  [T][K] int32 out: selected experts, ascending ids; ties between equal
 *             keys go to the lower expert id (and the lower group id)
 *   topk_w    [T][K] fp32 out: weights aligned with topk_ids                        */
int moe_route(const moe_problem* p, const void* x, const float* w_router, const float* bias,
              int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes, void* stream);

/* Selection only, from given fp32 logits [T][E] (for example uniform random keys):
 * the same scoring, group limit, top-K and weights as moe_route after its GEMM.      */
int moe_select(const moe_problem* p, const float* logits, const float* bias,
               int32_t* topk_ids, float* topk_w, void* stream);

/* ---- stage 2: dispatch -----------------------------------------------------------
 * Per-expert histogram, capacity, expert-contiguous permutation of this rank's pairs
 * and the send-count matrix C[i][j] = n_ij*h*dtype_size of the pairs virtual rank i
 * routes to rank j ("总览", eq. par-ep-dispatch-matrix). Rows are ordered by (local
 * expert, token); a pair's rank among its expert's pairs is its token order.
 *   x          [T][h] act, or NULL for a layout-only call (then xp must be NULL)
 *   topk_ids   [T][K] int32, each row K distinct ids in [0, E)
 *   counts     [E] int32 out: pairs per expert before capacity (all experts)
 *   offsets    [E_l+1] int32 out: first row of each local expert; offsets[E_l] = rows
 *   dest_row   [T][K] int32 out: row of the pair in this rank's buffer, -1 if the pair
 *              was dropped or its expert is remote
 *   row_src    [R_max] int32 out: t*K+k of the row's pair, -1 for pad / unused rows
 *   send_bytes [n_ep][n_ep] int64 out or NULL; kept pairs only, diagonal included;
 *              needs T % n_ep == 0. With MOE_DTYPE_MXFP8 a pair counts h + h/32 bytes
 *              (the row's E4M3 codes and scale bytes: x is quantised before dispatch)
 *   n_dropped  [1] int32 out: pairs dropped by capacity, over all E experts
 *   xp         [R_max][h] act out or NULL: xp[r] = x[row_src[r]/K]; pad rows zero;
 *              rows at or past offsets[E_l] (compact layout) are left undefined      */
int moe_dispatch(const moe_problem* p, const void* x, const int32_t* topk_ids,
                 int32_t* counts, int32_t* offsets, int32_t* dest_row, int32_t* row_src,
                 int64_t* send_bytes, int32_t* n_dropped, void* xp,
                 void* ws, size_t ws_bytes, void* stream);

/* ---- stage 3: expert FFN ---------------------------------------------------------
 * Every local expert's SwiGLU FFN on its rows as one grouped GEMM pair ("專家並行",
 * "技術原理" step 3; "MoE 服務的專家並行性": grouped GEMM batching many experts):
 *   yp = (silu(xp W_g^T) * (xp W_u^T)) W_d^T, fp32 accumulation; the gated product is
 *   rounded to act once before the down projection.
 *   xp        [R_max][h] act (rows below offsets[E_l] are read), or NULL: then the
 *             gate/up GEMM reads row r straight from x[row_src[r] / K] (a row whose
 *             row_src is negative reads zeros), the permutation folded into its operand
 *             loads, and xp need not exist
 *   row_src   [R_max] int32 (device) as written by moe_dispatch; needed when xp is NULL,
 *             ignored otherwise
 *   offsets   [E_l+1] int32 (device) as written by moe_dispatch
 *   w13       [E_l][2*inter][h] act: per expert W_g rows then W_u rows
 *   w2        [E_l][h][inter] act: per expert W_d
 *   x         [T][h] act: the shared expert's input, and the gate/up GEMM's rows when
 *             xp is NULL; may be NULL otherwise
 *   w13_sh, w2_sh   shared expert weights [2*shared_inter][h] and [h][shared_inter];
 *             NULL when n_shared = 0
 *   yp        [R_max][h] act out: rows below offsets[E_l] written, others undefined
 *   y_sh      [T/n_ep][h] act out (NULL when n_shared = 0)                           */
int moe_expert_ffn(const moe_problem* p, const void* xp, const int32_t* row_src,
                   const int32_t* offsets, const void* w13, const void* w2, const void* x,
                   const void* w13_sh, const void* w2_sh, void* yp, void* y_sh,
                   void* ws, size_t ws_bytes, void* stream);

/* ---- stage 4: combine ------------------------------------------------------------
 * y[t] = sum_{k=0..K-1, dest_row[t][k] >= 0} topk_w[t][k] * yp[dest_row[t][k]]
 *        (+ y_sh[t - t0] for t in this rank's token block when y_sh is not NULL),
 * accumulated in fp32 in k order, rounded to act once ("專家並行", "技術原理" step 4).
 * A token with no kept local pair and no shared output gets exact zeros.
 *   yp [R_max][h] act;  dest_row [T][K];  topk_w [T][K] fp32;
 *   y_sh [T/n_ep][h] act or NULL;  y [T][h] act out                                */
int moe_combine(const moe_problem* p, const void* yp, const int32_t* dest_row,
                const float* topk_w, const void* y_sh, void* y, void* stream);

/* ---- layout statistics -----------------------------------------------------------
 * What the routing in topk_ids sends where, after capacity exactly as moe_dispatch
 * keeps pairs, over n_ep virtual ranks (experts in contiguous blocks of E/n_ep, tokens
 * in contiguous blocks of T/n_ep). A token reaches at most K ranks while one rank's
 * tokens together reach many ("总览" section "Dispatch 通信矩阵": per-token versus
 * per-chip fan-out; node-limited routing is the group limit with one group per node);
 * the busiest rank's load over random top-K selections is the Monte Carlo estimate of
 * "如何在不跑模型时估算 EP 负载？". Every output may be NULL; all are int64, overwritten.
 *   tokens_to   [n_ep][n_ep]: distinct tokens of rank i with at least one kept pair on
 *               rank j (one row copy per target rank; send_bytes counts every pair).
 *               Needs T % n_ep == 0, else MOE_ERR_INVALID
 *   recv_pairs  [n_ep]: kept pairs whose expert lives on rank j
 *   fanout_hist [K+1]: tokens by their number of distinct target ranks
 *   busiest     [1]: the largest recv_pairs entry                                     */
int moe_layout_stats(const moe_problem* p, const int32_t* topk_ids, int64_t* tokens_to,
                     int64_t* recv_pairs, int64_t* fanout_hist, int64_t* busiest, void* ws,
                     size_t ws_bytes, void* stream);

/* ---- the whole layer -------------------------------------------------------------
 * route -> dispatch -> expert FFN -> combine on one stream, with every intermediate
 * kept in caller memory (so each stage's output can be inspected). xp may be NULL: the
 * row copy is then skipped and the gate/up GEMM reads each row's token straight from x
 * through row_src (the permutation folded into the GEMM's operand loads); every other
 * output is bit-identical to a call with xp.                                          */
typedef struct moe_tensors {
  const void* x;            /* [T][h] act                                  */
  const float* w_router;    /* [E][h] fp32                                 */
  const float* bias;        /* [E] fp32 or NULL                            */
  const void* w13;          /* [E_l][2*inter][h] act                       */
  const void* w2;           /* [E_l][h][inter] act                         */
  const void* w13_sh;       /* [2*shared_inter][h] act or NULL             */
  const void* w2_sh;        /* [h][shared_inter] act or NULL               */
  int32_t* topk_ids;        /* [T][K]                                      */
  float* topk_w;            /* [T][K]                                      */
  int32_t* counts;          /* [E]                                         */
  int32_t* offsets;         /* [E_l+1]                                     */
  int32_t* dest_row;        /* [T][K]                                      */
  int32_t* row_src;         /* [R_max]                                     */
  int64_t* send_bytes;      /* [n_ep][n_ep] or NULL                        */
  int32_t* n_dropped;       /* [1]                                         */
  void* xp;                 /* [R_max][h] act, or NULL (see above)         */
  void* yp;                 /* [R_max][h] act                              */
  void* y_sh;               /* [T/n_ep][h] act or NULL                     */
  void* y;                  /* [T][h] act out                              */
  /* MX-FP8 only (NULL otherwise): E8M0 scale bytes of the weights, one per 32 values
   * along h for w13 / w13_sh and along the intermediate dimension for w2 / w2_sh; the
   * weights themselves are then E4M3 codes in the layouts above.                      */
  const uint8_t* w13_scale;     /* [E_l][2*inter][h/32]                      */
  const uint8_t* w2_scale;      /* [E_l][h][inter/32]                        */
  const uint8_t* w13_sh_scale;  /* [2*shared_inter][h/32] or NULL            */
  const uint8_t* w2_sh_scale;   /* [h][shared_inter/32] or NULL              */
} moe_tensors;

int moe_forward(const moe_problem* p, const moe_tensors* t, void* ws, size_t ws_bytes,
                void* stream);

/* ---- tracing -----------------------------------------------------------------------
 * moe_forward with timing marks: events[i] (caller-created hipEvent_t handles, all
 * non-NULL) is recorded on `stream` at trace point i, so the caller can time each
 * kernel group with hipEventElapsedTime. The work enqueued is identical to
 * moe_forward's.                                                                     */
enum moe_trace_point {
  MOE_TRACE_BEGIN = 0,        /* before the router GEMM                        */
  MOE_TRACE_ROUTE = 1,        /* after router GEMM + top-K selection           */
  MOE_TRACE_DISPATCH = 2,     /* after histogram, placement (and row copy)     */
  MOE_TRACE_FFN_PREP = 3,     /* after the FFN tile table (built by dispatch)  */
  MOE_TRACE_FFN_GATE_UP = 4,  /* after the gate/up grouped GEMM (silu * mul)   */
  MOE_TRACE_FFN_DOWN = 5,     /* after the down-projection grouped GEMM        */
  MOE_TRACE_COMBINE = 6,      /* after combine                                 */
  MOE_TRACE_POINTS = 7
};
int moe_forward_traced(const moe_problem* p, const moe_tensors* t, void* ws, size_t ws_bytes,
                       void* stream, void* const* events);

/* ---- MX-FP8 quantisation ------------------------------------------------------------
 * OCP E4M3 codes with one power-of-two scale per 32 consecutive values of a row (OCP
 * Microscaling): a block's scale is 2^X, X = floor(log2(max |v|)) - 8 (the largest E4M3
 * exponent), -127 for an all-zero block, clamped to [-127, 127], stored as the byte X + 127;
 * each value becomes the E4M3 code of v / 2^X, rounded to nearest with ties to the even
 * code and saturated at +-448 (no NaN codes are produced; the sign bit is v's). FP8 data
 * paths of MoE layers spend much of their time in such quantise / dequantise passes next to
 * the GEMMs ("Expert-Parallelism", 关键观察, observation 3).
 *   src     [rows][cols] device, src_dtype MOE_DTYPE_F32 or MOE_DTYPE_BF16; cols % 32 == 0
 *   codes   [rows][cols] uint8 out;  scales [rows][cols/32] uint8 out                   */
int moe_quantize_mx(int64_t rows, int32_t cols, int32_t src_dtype, const void* src,
                    uint8_t* codes, uint8_t* scales, void* stream);

/* Weight packing for MOE_DTYPE_BF16_PACKED (a one-time transform, like loading a
 * checkpoint into the kernels' layout). src holds `mats` row-major bf16 matrices
 * [mats][rows][cols]; dst (same size, caller-owned, not overlapping src) receives them
 * as [mats][rows/32][cols/16][64][8]: the 1 KB block (b, k) of a matrix holds, for lane
 * l = 0..63, row 32*b + l%32, columns 16*k + 8*(l/32) .. +7. That is the operand
 * fragment of one 32x32x16 bf16 MFMA, so a GEMM reads each fragment as one coalesced
 * 1 KB load. Pack w13 with (E_l, 2*inter, h), w2 with (E_l, h, inter) and the shared
 * expert's with mats = 1. Requires rows % 32 == 0, cols % 16 == 0, 16-byte aligned
 * pointers (else MOE_ERR_INVALID); enqueued on `stream`. */
int moe_pack_weights(int64_t mats, int32_t rows, int32_t cols, const void* src, void* dst,
                     void* stream);

/* ---- redundant experts ---------------------------------------------------------------
 * A logical -> physical replica map: P = E + R physical experts (replicas), P a multiple of
 * n_ep, rank j holding physical ids [j*P/n_ep, (j+1)*P/n_ep) ("总览" glossary: logical
 * expert, physical expert / replica, redundant expert: 256 logical + 32 redundant = 288
 * physical; "Expert-Parallelism", 设计空间与取舍, route 3: replicate hot experts). The pairs
 * of logical expert e are dealt to its r_e replicas round robin in token order: the pair
 * ranked rho among e's pairs goes to replica rho mod r_e, where it ranks rho / r_e. With a
 * capacity factor the capacity is per physical expert, ceil(cf * T * K / P). No padding.
 *   P             physical experts
 *   rep_start     [E+1] device: replicas of e are rep_list[rep_start[e] .. rep_start[e+1])
 *   rep_list      [P] device: physical id of replica q of e, in replica order
 *   phys_expert   [P] device: the logical expert a physical id holds
 *   phys_replica  [P] device: its replica index q                                       */
typedef struct moe_replica_map {
  int32_t P;
  const int32_t* rep_start;
  const int32_t* rep_list;
  const int32_t* phys_expert;
  const int32_t* phys_replica;
} moe_replica_map;

/* Host only (all pointers host memory): the map for per-expert loads load[E] (for example
 * a routing's pair counts) with R redundant replicas over n_ep ranks. Replica counts: one
 * each, then every redundant slot to the expert with the largest load per replica (ties to
 * the lower id). Packing: replicas by the pairs they will receive (descending; ties: lower
 * expert id, then lower replica index) onto the rank with the least load so far among ranks
 * with a free slot (ties to the lower rank); a rank's slots fill in placement order. Writes
 * counts[E] (r_e), rep_start[E+1], rep_list[P], phys_expert[P], phys_replica[P].
 * MOE_ERR_INVALID for E outside 1..512, R < 0, (E+R) % n_ep != 0, E + R > 8192, loads
 * outside 0..2^31-1 or NULL pointers.                                                  */
int moe_replica_plan(int32_t E, int32_t R, int32_t n_ep, const int64_t* load, int32_t* counts,
                     int32_t* rep_start, int32_t* rep_list, int32_t* phys_expert,
                     int32_t* phys_replica);

/* Rows of this rank's buffer and workspace bytes for the problem over P physical experts.
 * MOE_ERR_INVALID when P < E or P % n_ep != 0; MOE_ERR_UNSUPPORTED with padding, more than
 * 512 physical experts per rank, or more than 32768 (pair-count rows x E).            */
int moe_replicated_sizes(const moe_problem* p, int32_t P, int64_t* max_rows, size_t* ws_bytes);

/* moe_dispatch (layout only: no x / xp) over the map. counts [E]: pairs per logical expert;
 * phys_counts [P] (or NULL): pairs per physical expert before capacity; offsets [P/n_ep+1]:
 * first row of each local physical expert; rows ordered by (physical expert, token);
 * dest_row / row_src / send_bytes / n_dropped as moe_dispatch with the destination rank of a
 * pair the one holding its replica; workspace of moe_replicated_sizes.               */
int moe_dispatch_replicated(const moe_problem* p, const moe_replica_map* map,
                            const int32_t* topk_ids, int32_t* counts, int32_t* phys_counts,
                            int32_t* offsets, int32_t* dest_row, int32_t* row_src,
                            int64_t* send_bytes, int32_t* n_dropped, void* ws, size_t ws_bytes,
                            void* stream);

/* moe_forward over the map: w13 [E][2*inter][h] and w2 [E][h][inter] hold every LOGICAL
 * expert and each local physical expert runs with its logical expert's weights (no copy);
 * offsets has P/n_ep + 1 entries; row buffers and workspace from moe_replicated_sizes.  */
int moe_forward_replicated(const moe_problem* p, const moe_replica_map* map,
                           const moe_tensors* t, void* ws, size_t ws_bytes, void* stream);

/* ---- allocation-free forward ------------------------------------------------------
 * For callers that cannot allocate device memory or pass a workspace (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): moe_forward with its
 * workspace taken from a device array of MOE_NOALLOC_SCRATCH_BYTES that the library holds
 * on every GPU it runs on, until the process ends. The caller still passes every input and
 * output in `t`, exactly as for moe_forward, and gets bit-identical results.
 *   - Problems whose moe_workspace_bytes() exceeds MOE_NOALLOC_SCRATCH_BYTES are refused
 *     with MOE_ERR_WORKSPACE before anything is enqueued (64 MiB fits, for example, a
 *     decode batch of up to ~1000 tokens with 256 experts of DeepSeek-V3 shape resident).
 *   - The call allocates nothing. Its first call on a device looks up that device's copy
 *     of the array (MOE_ERR_LAUNCH if the runtime refuses).
 *   - Every call on one GPU uses that GPU's one array: calls that overlap in time on one
 *     GPU (other streams, other host threads) race and must be serialised by the caller.
 *     A call needs nothing in the array to start at zero.                               */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_forward_noalloc(const moe_problem* p, const moe_tensors* t, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
