// host_checks.hpp -- host-only rules of libmoe: the limits the kernels are
// built for, buffer sizes and launch geometry, and the argument checks of
// every entry point.  Plain C++17 with no HIP dependency, so that it can be
// compiled and exercised on its own (for instance under address and
// undefined-behaviour sanitizers); the kernels' launchers include it for the
// same sizes.  Return codes and the meaning of each argument: include/moe.h.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ---- limits the kernels are written for ------------------------------------
constexpr int kMaxExperts = 1024;     // expert scans hold 4 (LDS plan) or 2 experts a thread
constexpr int kMaxTopK = 64;          // one slot per lane of a wave64
constexpr int kPlanThreads = 512;     // plan kernels: 8 waves per block
constexpr int kPlanTilePairs = 2048;  // count tile of the plan kernels (whole tokens)
constexpr int kPlanSubPairs = kPlanThreads;  // assign block: one 64-pair chunk per wave
constexpr int kSmallPairs = 2048;     // plan-and-dispatch in one launch: pairs it plans
constexpr int kTileHist = 2048;       // tiled plan-and-dispatch: histogram entries it reads
constexpr int kMapThreads = 256;      // routing-map conversion block
constexpr int kMapLaneExperts = 16;   // map bytes per lane

// ---- sizes -------------------------------------------------------------------

// Rows of the packed buffer: N*k + E*(A-1), or E*cap with a fixed capacity.
inline int64_t max_rows(const moe_problem &p) {
  if (p.expert_capacity > 0) return static_cast<int64_t>(p.n_experts) * p.expert_capacity;
  return p.n_tokens * p.top_k + static_cast<int64_t>(p.n_experts) * (p.pad_multiple - 1);
}

int64_t payload_row_bytes(const moe_problem &p);  // of a valid problem
int64_t scale_row_bytes(const moe_problem &p);

// How the (token, k) pairs are split into tiles for the plan kernels.
struct PlanGeom {
  int64_t npairs;      // N * k
  int tile_tokens;     // whole tokens per tile (at most kPlanTilePairs pairs)
  int64_t tile_pairs;  // tile_tokens * k
  int ntiles;          // ceil(N / tile_tokens), >= 1
  int subs;            // sub-tiles of kPlanSubPairs pairs per count tile (assign blocks)
  bool single;         // one count tile: no separate counting kernel
  int key_bits;        // bits needed for an expert id (ceil(log2 E))
};
PlanGeom plan_geometry(const moe_problem &p);
// ntiles * (E + 1) int32 (tile histograms, then each tile's fault bits),
// rounded up to 256 bytes; 0 for a single-tile plan
size_t plan_workspace_bytes(const moe_problem &p);

// How moe_plan_and_dispatch runs a problem: one launch (at most kSmallPairs
// pairs), tiled (the counting kernel, then one launch that finishes the plan
// and dispatches; at most kTileHist histogram entries), or the plan's
// kernels then the dispatch.  A fixed expert capacity takes the same modes
// (each expert's first cap pairs kept, the rest dropped by the launch that
// places them).
enum class PlanDispatchMode { kOneLaunch, kTiled, kSeparate };
PlanDispatchMode plan_dispatch_mode(const moe_problem &p);
// In one-launch mode without padding (A = 1) or capacity, a pair's packed row is the
// count of valid pairs ahead of it in (expert, pair index) order, which a
// workgroup can count for its own pairs with ballots and one barrier, while
// workgroup 0 writes the plan arrays (the dispatch launcher also bounds the
// ballots a wave makes); otherwise every workgroup builds the plan in LDS.
bool one_launch_direct(const moe_problem &p);

// Workspace of the exchange plan: [EP][E+1] offsets and [EP][N*k] packed_src
// of the per-rank plans, then EP copies of the single-rank plan workspace.
struct ExchangeLayout {
  size_t offsets, packed_src, plan_ws, total;
  size_t plan_ws_bytes;  // per rank
};
moe_problem exchange_rank_problem(const moe_problem &p);  // one rank's own plan
ExchangeLayout exchange_layout(const moe_problem &p);

// Routing-map conversion: lanes per token (ceil(E/16) rounded up to a power
// of two), blocks, and workspace (one flag word per block, 256-byte rounded).
int map_lanes_per_token(int n_experts);
int map_blocks(const moe_problem &p);
size_t map_workspace_bytes(const moe_problem &p);

// ceil(cf * N * k / E) in double precision, or a negative error code
int64_t expert_capacity(int64_t n_tokens, int32_t top_k, int32_t n_experts, double cf);

// ---- argument checks: MOE_OK or the code the entry point returns -----------
namespace host {

int check_problem(const moe_problem *p);
int check_exchange(const moe_problem *p);

int check_plan_args(const moe_problem *p, const int32_t *topk_ids, const moe_plan *plan,
                    const void *workspace);
// moe_plan_and_dispatch and its halves: the plan's arguments and the dispatch's
int check_plan_and_dispatch_args(const moe_problem *p, const int32_t *topk_ids, const moe_plan *plan,
                                 const uint16_t *hidden, const float *topk_weights,
                                 const float *input_scale, const void *payload, const void *scales,
                                 const void *workspace);
int check_dispatch_args(const moe_problem *p, const moe_plan *plan, const uint16_t *hidden,
                        const void *payload, const void *scales);
int check_dispatch_scaled_args(const moe_problem *p, const moe_plan *plan, const uint16_t *hidden,
                               const float *input_scale, const void *payload, const void *scales);
int check_dispatch_gated_args(const moe_problem *p, const moe_plan *plan, const uint16_t *hidden,
                              const float *topk_weights, const void *payload, const void *scales);
int check_combine_args(const moe_problem *p, const moe_plan *plan, const uint16_t *expert_out,
                       const float *topk_weights, const uint16_t *out);

int check_exchange_plan_args(const moe_problem *p, const int32_t *topk_ids, const moe_exchange *x,
                             const void *workspace);
int check_exchange_dispatch_args(const moe_problem *p, const moe_exchange *x, const uint16_t *hidden,
                                 const void *payload, const void *scales);
int check_exchange_dispatch_scaled_args(const moe_problem *p, const moe_exchange *x,
                                        const uint16_t *hidden, const float *input_scale,
                                        const void *payload, const void *scales);
int check_exchange_dispatch_gated_args(const moe_problem *p, const moe_exchange *x,
                                       const uint16_t *hidden, const float *topk_weights,
                                       const void *payload, const void *scales);
int check_exchange_combine_args(const moe_problem *p, const moe_exchange *x, const uint16_t *expert_out,
                                const float *topk_weights, const uint16_t *out);

int check_map_args(const moe_problem *p, const uint8_t *routing_map, const float *probs,
                   const int32_t *topk_ids, const float *topk_weights, const uint32_t *status,
                   const void *workspace);

const char *error_text(int code);

}  // namespace host
}  // namespace moe
