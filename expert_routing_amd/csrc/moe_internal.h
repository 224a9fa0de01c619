// Internal declarations shared by the library's HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef uint16_t bf16_t;  // raw bf16 storage
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;          // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int kDispatchChunk = 256; // tokens per dispatch block

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// Derived sizes of a validated problem (host side).
struct Dims {
  int64_t T;
  int h, E, K, El, e0, N, rank;
  int64_t cap;      // -1: no limit
  int64_t R_max;    // rows of the local buffer
  int64_t tpr;      // tokens per virtual rank (T / N), 0 when T % N != 0
  int64_t sh_rows;  // shared-expert rows (T/N or 0)
  int s;            // activation bytes
  bool bf16;        // bf16 activations (also with MX-FP8 expert weights)
  bool mx;          // MX-FP8 expert weights and GEMM operands
  bool pk;          // bf16 expert weights in the packed fragment order
  int route_split;  // K-slices of the router GEMM (partial logits summed in order)
};

// Workspace carve-up (byte offsets from ws, each 256-aligned).
struct WsLayout {
  size_t logits;        // [T][E] f32
  size_t chunk_counts;  // [n_chunks][E] i32
  size_t chunk_base;    // [n_chunks][E] i32
  size_t kept;          // [E_l] i32
  size_t sched;         // ffn tile schedule
  size_t hbuf;          // [R_max + sh_rows][I_max] act (MX-FP8: E4M3 codes)
  size_t hbuf_s;        // MX-FP8: the gated product's scale bytes [..][I_max/32]
  size_t xq, xs;        // MX-FP8: x as E4M3 codes [T][h] and scale bytes [T][h/32]
  size_t splitk;        // split-K partial sums (fp32), bf16 problems only
  size_t arrive;        // split-K arrival counters
  size_t stats;         // layout statistics scratch: scan outputs [E + E_l + 2] i32, then
  size_t stats_recv;    //   (at this offset from stats) per-chip loads [N] u64
  size_t total;
};

struct FfnPrepArgs;   // ffn_sched.h: what the expert FFN's tile table is built from

// The replica map as the placement reads it (rep_start == nullptr: physical = logical).
struct ReplicaArgs {
  const int32_t* rep_start;    // [E + 1]
  const int32_t* rep_list;     // [P]
  const int32_t* phys_expert;  // [P]
  const int32_t* phys_replica; // [P]
  int P;                       // physical experts
  int32_t* phys_counts;        // [P] out: pairs per physical expert before capacity, or nullptr
};


int make_dims(const moe_problem* p, Dims* d);
// Dims over P physical experts (a replica map): El / e0 count this rank's physical experts,
// cap is per physical expert, R_max the rows of its buffer.
int make_dims_replicated(const moe_problem* p, int P, Dims* d);
int route_split(const Dims& d);   // defined with the router kernels
WsLayout ws_layout(const moe_problem* p, const Dims& d);

// Stage launchers (arguments already validated; return MOE_OK or MOE_ERR_LAUNCH).
// chunk_counts (or nullptr): the router also leaves dispatch's per-expert pair counts of
// every route_count_tokens(d) tokens there ([rows][E]).
int launch_route(const moe_problem* p, const Dims& d, const void* x, const float* w_router,
                 const float* bias, int32_t* ids, float* w, float* logits,
                 int32_t* chunk_counts, hipStream_t st);
int route_count_tokens(const Dims& d);
int launch_select(const moe_problem* p, const Dims& d, const float* logits, const float* bias,
                  int32_t* ids, float* w, hipStream_t st);
// `ffn`: also build the expert FFN's tile table from the offsets (nullptr: do not).
// `counted_rows` > 0: the router already left the pair counts of every `counted_rows`
// tokens in the workspace's chunk counts (launch_route with chunk_counts).
// `rm`: a replica map (Dims then counts physical experts: make_dims_replicated).
int launch_dispatch(const moe_problem* p, const Dims& d, const void* x, const int32_t* ids,
                    int32_t* counts, int32_t* offsets, int32_t* dest_row, int32_t* row_src,
                    int64_t* send_bytes, int32_t* n_dropped, void* xp, char* ws,
                    const WsLayout& L, hipStream_t st, const FfnPrepArgs* ffn = nullptr,
                    int counted_rows = 0, const ReplicaArgs* rm = nullptr);
// Host: the tile table's parameters (tile shapes, operand pointers) for this problem.
int ffn_prep_args(const moe_problem* p, const Dims& d, const void* xp, const void* w13,
                  const void* w2, const void* x, const void* w13_sh, const void* w2_sh, void* yp,
                  void* y_sh, char* ws, const WsLayout& L, const int32_t* gather_rows,
                  FfnPrepArgs* a);
// The one-block kernel that builds the table from offsets in device memory.
int launch_ffn_prep(const FfnPrepArgs& a, const int32_t* offsets, hipStream_t st);
// The two grouped GEMMs; `prepped`: the table was already built (by dispatch) from these
// arguments, else the prep kernel runs first.
int launch_ffn(const moe_problem* p, const Dims& d, const void* xp, const int32_t* offsets,
               const void* w13, const void* w2, const void* x, const void* w13_sh,
               const void* w2_sh, void* yp, void* y_sh, char* ws, const WsLayout& L,
               hipStream_t st, hipEvent_t const* ev = nullptr,
               const int32_t* gather_rows = nullptr, const FfnPrepArgs* prepped = nullptr);
int launch_layout_stats(const moe_problem* p, const Dims& d, const int32_t* ids,
                        int64_t* tokens_to, int64_t* recv_pairs, int64_t* fanout_hist,
                        int64_t* busiest, char* ws, const WsLayout& L, hipStream_t st);
int launch_combine(const moe_problem* p, const Dims& d, const void* yp, const int32_t* dest_row,
                   const float* w, const void* y_sh, void* y, hipStream_t st);

// MX-FP8 quantisation of a rows x cols matrix (cols % 32 == 0): codes [rows][cols],
// scale bytes [rows][cols / 32].
int launch_pack_weights(int64_t mats, int rows, int cols, const void* src, void* dst,
                        hipStream_t st);
int launch_mx_quant(const void* src, bool bf16, int64_t rows, int cols, uint8_t* codes,
                    uint8_t* scales, hipStream_t st);

size_t ffn_sched_bytes(const Dims& d);
size_t ffn_splitk_bytes(const Dims& d);
size_t ffn_arrive_bytes(const Dims& d);

}  // namespace moe
