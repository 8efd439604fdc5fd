// moe_kernels.hpp -- launchers behind the C ABI (internal to libmoe).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "host_checks.hpp"
#include "moe.h"

namespace moe {

constexpr int kPlanWaves = kPlanThreads / 64;

hipError_t launch_plan(const moe_problem &p, const int32_t *ids, const moe_plan &plan,
                       void *workspace, hipStream_t stream);

// Distance, in elements, between consecutive ranks' arrays of a batch of
// plans made in one launch (one rank per blockIdx.y).
struct PlanStrides {
  int64_t pairs = 0;      // topk_ids and slot
  int64_t rows = 0;       // packed_src
  int64_t workspace = 0;  // plan workspace, in int32 elements
  int counts = 0, offsets = 0, dest = 0, table = 0;
};

// `ranks` independent plans of problem p (each over its own N tokens).
hipError_t launch_plan_ranks(const moe_problem &p, int ranks, const int32_t *ids,
                             const moe_plan &plan, const PlanStrides &st, void *workspace,
                             hipStream_t stream);

// Exchange across p.ep simulated ranks (rank s owns tokens s*N .. s*N+N-1).
hipError_t launch_exchange_plan(const moe_problem &p, const int32_t *ids, const moe_exchange &x,
                                void *workspace, hipStream_t stream);
hipError_t launch_exchange_dispatch(const moe_problem &p, const moe_exchange &x, const uint16_t *hidden,
                                    const float *gates, const float *gscale, void *payload, void *scales,
                                    hipStream_t stream);

// Multihot routing map [N][E] (+ optional dense probabilities) -> compact
// top-k IDs and weights; status gets MOE_STATUS_MAP_OVERFLOW.
hipError_t launch_routing_map_to_topk(const moe_problem &p, const uint8_t *map, const float *probs,
                                      int32_t *ids, float *weights, uint32_t *status, void *workspace,
                                      hipStream_t stream);
hipError_t launch_exchange_combine(const moe_problem &p, const moe_exchange &x, const uint16_t *expert_out,
                                   const float *weights, uint16_t *out, hipStream_t stream);

// gates: NULL, or [N][k] weights applied to each copy at dispatch;
// gscale: the NVFP4 global encode scale (device, one float) or NULL
hipError_t launch_dispatch(const moe_problem &p, const moe_plan &plan, const uint16_t *hidden,
                           const float *gates, const float *gscale, void *payload, void *scales,
                           hipStream_t stream);

// The plan's counting kernel alone: tile histograms and fault bits into
// the plan workspace (problems of more than one count tile); it also clears
// *status, into which the launch that finishes the plan ORs its bits.
hipError_t launch_plan_count(const moe_problem &p, const int32_t *ids, uint32_t *status,
                             void *workspace, hipStream_t stream);

// The launch that plans (or, tiled, finishes the plan after
// launch_plan_count) and dispatches; only where plan_dispatch_mode(p) is
// kOneLaunch or kTiled.
hipError_t launch_plan_dispatch(const moe_problem &p, const int32_t *ids, const moe_plan &plan,
                                const uint16_t *hidden, const float *gates, const float *gscale,
                                void *payload, void *scales, void *workspace, hipStream_t stream);

// rows: rows of expert_out; a slot outside [0, rows) is skipped like a
// masked one, and no row that no slot names is read
hipError_t launch_combine(const moe_problem &p, const moe_plan &plan, const uint16_t *expert_out,
                          int64_t rows, const float *weights, uint16_t *out, hipStream_t stream);

}  // namespace moe
