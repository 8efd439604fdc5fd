// host_checks.cpp -- host-only rules of libmoe (see host_checks.hpp): sizes,
// launch geometry and the argument checks of every entry point.  No HIP
// calls; nothing here touches device memory.
#include "host_checks.hpp"

#include <math.h>

namespace moe {
namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

}  // namespace

int64_t payload_row_bytes(const moe_problem &p) {
  if (p.fmt == MOE_FMT_BF16) return 2 * static_cast<int64_t>(p.hidden);
  if (p.fmt == MOE_FMT_FP8_E4M3_B128) return p.hidden;
  return p.hidden / 2;  // MX-FP4 and NVFP4: two E2M1 codes a byte
}

int64_t scale_row_bytes(const moe_problem &p) {
  if (p.fmt == MOE_FMT_BF16) return 0;
  if (p.fmt == MOE_FMT_FP8_E4M3_B128) return 4 * static_cast<int64_t>(p.hidden / 128);
  if (p.fmt == MOE_FMT_NVFP4_B16) return p.hidden / 16;
  return p.hidden / 32;
}

PlanGeom plan_geometry(const moe_problem &p) {
  PlanGeom geo;
  geo.npairs = p.n_tokens * p.top_k;
  geo.tile_tokens = kPlanTilePairs / p.top_k > 1 ? kPlanTilePairs / p.top_k : 1;
  geo.tile_pairs = static_cast<int64_t>(geo.tile_tokens) * p.top_k;
  geo.ntiles = p.n_tokens == 0 ? 1
                               : static_cast<int>((p.n_tokens + geo.tile_tokens - 1) / geo.tile_tokens);
  geo.single = geo.ntiles == 1;
  // sub-tiles per count tile: every tile but the last holds tile_pairs pairs
  const int64_t span = geo.single ? geo.npairs : geo.tile_pairs;
  geo.subs = span > kPlanSubPairs ? static_cast<int>((span + kPlanSubPairs - 1) / kPlanSubPairs) : 1;
  int bits = 0;
  while ((1 << bits) < p.n_experts) ++bits;
  geo.key_bits = bits;
  return geo;
}

size_t plan_workspace_bytes(const moe_problem &p) {
  const PlanGeom geo = plan_geometry(p);
  if (geo.single) return 0;
  return align256(static_cast<size_t>(geo.ntiles) * (p.n_experts + 1) * sizeof(int32_t));
}

PlanDispatchMode plan_dispatch_mode(const moe_problem &p) {
  const int64_t npairs = p.n_tokens * p.top_k;
  if (npairs <= kSmallPairs) return PlanDispatchMode::kOneLaunch;
  const PlanGeom geo = plan_geometry(p);
  if (static_cast<int64_t>(geo.ntiles) * p.n_experts <= kTileHist && max_rows(p) <= INT32_MAX)
    return PlanDispatchMode::kTiled;
  return PlanDispatchMode::kSeparate;
}

bool one_launch_direct(const moe_problem &p) {
  return plan_dispatch_mode(p) == PlanDispatchMode::kOneLaunch && p.pad_multiple == 1 &&
         p.expert_capacity == 0;
}

moe_problem exchange_rank_problem(const moe_problem &p) {
  moe_problem q = p;
  q.pad_multiple = 1;
  q.recv_capacity = INT64_MAX;  // capacity applies to receive buffers only
  q.flags = 0;
  q.expert_capacity = 0;
  return q;
}

ExchangeLayout exchange_layout(const moe_problem &p) {
  const size_t R = static_cast<size_t>(p.ep);
  ExchangeLayout L;
  size_t at = 0;
  L.offsets = at;
  at += align256(R * (p.n_experts + 1) * sizeof(int32_t));
  L.packed_src = at;
  at += align256(R * static_cast<size_t>(p.n_tokens) * p.top_k * sizeof(int32_t));
  L.plan_ws_bytes = plan_workspace_bytes(exchange_rank_problem(p));
  L.plan_ws = at;
  at += R * L.plan_ws_bytes;
  L.total = at;
  return L;
}

int map_lanes_per_token(int n_experts) {
  const int need = (n_experts + kMapLaneExperts - 1) / kMapLaneExperts;
  int lpt = 1;
  while (lpt < need) lpt <<= 1;
  return lpt;
}

int map_blocks(const moe_problem &p) {
  const int64_t per = kMapThreads / map_lanes_per_token(p.n_experts);
  return static_cast<int>((p.n_tokens + per - 1) / per);
}

size_t map_workspace_bytes(const moe_problem &p) {
  return align256(static_cast<size_t>(map_blocks(p)) * sizeof(uint32_t));
}

int64_t expert_capacity(int64_t n_tokens, int32_t top_k, int32_t n_experts, double cf) {
  if (n_tokens < 0 || top_k < 1 || n_experts < 1 || !(cf >= 0.0)) return MOE_EINVAL;
  const double cap = ceil(cf * static_cast<double>(n_tokens) * static_cast<double>(top_k) /
                          static_cast<double>(n_experts));
  if (!(cap <= static_cast<double>(INT32_MAX))) return MOE_EOVERFLOW;
  return static_cast<int64_t>(cap);
}

namespace host {

int check_problem(const moe_problem *p) {
  if (!p) return MOE_EINVAL;
  if (p->n_tokens < 0 || p->hidden <= 0 || p->hidden % 8 != 0) return MOE_EINVAL;
  if (p->n_experts < 1 || p->n_experts > kMaxExperts) return MOE_EINVAL;
  if (p->top_k < 1 || p->top_k > p->n_experts || p->top_k > kMaxTopK) return MOE_EINVAL;
  if (p->ep < 1 || p->n_experts % p->ep != 0) return MOE_EINVAL;
  if (p->pad_multiple < 1 || p->recv_capacity < 0) return MOE_EINVAL;
  if (p->expert_capacity < 0 || (p->expert_capacity > 0 && p->pad_multiple != 1)) return MOE_EINVAL;
  if (p->expert_capacity > INT32_MAX) return MOE_EOVERFLOW;
  if (p->flags & ~MOE_FLAG_ZERO_TAIL) return MOE_EINVAL;
  switch (p->fmt) {
    case MOE_FMT_BF16: break;
    case MOE_FMT_FP8_E4M3_B128: if (p->hidden % 128 != 0) return MOE_EINVAL; break;
    case MOE_FMT_MXFP4_B32: if (p->hidden % 32 != 0) return MOE_EINVAL; break;
    case MOE_FMT_NVFP4_B16: if (p->hidden % 32 != 0) return MOE_EINVAL; break;
    default: return MOE_EINVAL;
  }
  // pair indices, rows and token*H offsets are int32 / uint32 on the device
  if (p->n_tokens > INT32_MAX / p->top_k) return MOE_EOVERFLOW;
  // E*(A-1) must not overflow before it is compared: A < 2^31, E <= 1024
  const int64_t r_max = max_rows(*p);
  if (r_max > INT32_MAX) return MOE_EOVERFLOW;
  // with a fixed capacity the plan forms e*cap + (rank in expert) and
  // e*cap + 2*cap in int32
  if (p->expert_capacity > 0 && r_max + p->expert_capacity + p->n_tokens * p->top_k > INT32_MAX)
    return MOE_EOVERFLOW;
  if (r_max * static_cast<int64_t>(p->hidden) >= (int64_t{1} << 32)) return MOE_EOVERFLOW;
  if (p->n_tokens * static_cast<int64_t>(p->hidden) >= (int64_t{1} << 40)) return MOE_EOVERFLOW;
  // one wave per (token, column slab of >= 512 values) must index within int
  if (p->n_tokens * ((static_cast<int64_t>(p->hidden) + 511) / 512) > INT32_MAX / 4) return MOE_EOVERFLOW;
  return MOE_OK;
}

// The exchange: EP ranks of N tokens in one launch, receive buffers of C rows.
int check_exchange(const moe_problem *p) {
  const int rc = check_problem(p);
  if (rc != MOE_OK) return rc;
  if (p->pad_multiple != 1 || p->expert_capacity != 0) return MOE_EINVAL;
  const int64_t ranks = p->ep;
  const int64_t tokens = p->n_tokens * ranks;  // < 2^31 * 1024: no overflow
  // global pair and token indices, receive rows: int32; table: uint32 elements
  if (tokens > INT32_MAX / p->top_k) return MOE_EOVERFLOW;
  if (p->recv_capacity > INT32_MAX / ranks) return MOE_EOVERFLOW;
  if (tokens * p->top_k * static_cast<int64_t>(p->hidden) >= (int64_t{1} << 32)) return MOE_EOVERFLOW;
  if (tokens * static_cast<int64_t>(p->hidden) >= (int64_t{1} << 40)) return MOE_EOVERFLOW;
  if (tokens * ((static_cast<int64_t>(p->hidden) + 511) / 512) > INT32_MAX / 4) return MOE_EOVERFLOW;
  return MOE_OK;
}

int check_plan_args(const moe_problem *p, const int32_t *topk_ids, const moe_plan *plan,
                    const void *workspace) {
  const int rc = check_problem(p);
  if (rc != MOE_OK) return rc;
  if (!plan || !plan->expert_counts || !plan->expert_offsets || !plan->dest_counts ||
      !plan->rank_table || !plan->status)
    return MOE_EINVAL;
  const int64_t npairs = p->n_tokens * p->top_k;
  if (npairs > 0 && (!topk_ids || !plan->slot)) return MOE_EINVAL;
  if (max_rows(*p) > 0 && !plan->packed_src) return MOE_EINVAL;
  if (plan_workspace_bytes(*p) > 0 && !workspace) return MOE_EINVAL;
  if (!aligned(topk_ids, 4) || !aligned(plan->expert_counts, 4) || !aligned(plan->expert_offsets, 4) ||
      !aligned(plan->dest_counts, 4) || !aligned(plan->rank_table, 4) || !aligned(plan->slot, 4) ||
      !aligned(plan->packed_src, 4) || !aligned(plan->status, 4) || !aligned(workspace, 256))
    return MOE_EALIGN;
  return MOE_OK;
}

int check_plan_and_dispatch_args(const moe_problem *p, const int32_t *topk_ids, const moe_plan *plan,
                                 const uint16_t *hidden, const float *topk_weights,
                                 const float *input_scale, const void *payload, const void *scales,
                                 const void *workspace) {
  const int rc = check_plan_args(p, topk_ids, plan, workspace);
  if (rc != MOE_OK) return rc;
  // a global scale only for NVFP4, which takes no gates
  const bool nvfp4 = p->fmt == MOE_FMT_NVFP4_B16;
  if (nvfp4 != (input_scale != nullptr) || (nvfp4 && topk_weights)) return MOE_EINVAL;
  if (p->n_tokens > 0 && !hidden) return MOE_EINVAL;
  const bool quant = p->fmt != MOE_FMT_BF16;
  if (max_rows(*p) > 0 && (!payload || (quant && !scales))) return MOE_EINVAL;
  if (!quant && scales) return MOE_EINVAL;
  if (!aligned(hidden, 16) || !aligned(payload, 16) || !aligned(topk_weights, 4) ||
      !aligned(input_scale, 4) || (p->fmt == MOE_FMT_FP8_E4M3_B128 && !aligned(scales, 4)))
    return MOE_EALIGN;
  return MOE_OK;
}

int check_dispatch_args(const moe_problem *p, const moe_plan *plan, const uint16_t *hidden,
                        const void *payload, const void *scales) {
  const int rc = check_problem(p);
  if (rc != MOE_OK) return rc;
  if (!plan || !plan->expert_counts || !plan->expert_offsets) return MOE_EINVAL;
  if (p->n_tokens > 0 && (!hidden || !plan->slot)) return MOE_EINVAL;
  const bool quant = p->fmt != MOE_FMT_BF16;
  if (max_rows(*p) > 0 && (!payload || (quant && !scales))) return MOE_EINVAL;
  if (!quant && scales) return MOE_EINVAL;
  if (!aligned(hidden, 16) || !aligned(payload, 16) || !aligned(plan->slot, 4) ||
      !aligned(plan->expert_counts, 4) || !aligned(plan->expert_offsets, 4) ||
      (p->fmt == MOE_FMT_FP8_E4M3_B128 && !aligned(scales, 4)))
    return MOE_EALIGN;
  if (p->fmt == MOE_FMT_NVFP4_B16) return MOE_EINVAL;  // needs its global scale: moe_dispatch_scaled
  return MOE_OK;
}

int check_dispatch_scaled_args(const moe_problem *p, const moe_plan *plan, const uint16_t *hidden,
                               const float *input_scale, const void *payload, const void *scales) {
  const int rc = check_problem(p);
  if (rc != MOE_OK) return rc;
  if (p->fmt != MOE_FMT_NVFP4_B16 || !input_scale) return MOE_EINVAL;
  if (!plan || !plan->expert_counts || !plan->expert_offsets) return MOE_EINVAL;
  if (p->n_tokens > 0 && (!hidden || !plan->slot)) return MOE_EINVAL;
  if (max_rows(*p) > 0 && (!payload || !scales)) return MOE_EINVAL;
  if (!aligned(hidden, 16) || !aligned(payload, 16) || !aligned(plan->slot, 4) || !aligned(input_scale, 4) ||
      !aligned(plan->expert_counts, 4) || !aligned(plan->expert_offsets, 4))
    return MOE_EALIGN;
  return MOE_OK;
}

int check_dispatch_gated_args(const moe_problem *p, const moe_plan *plan, const uint16_t *hidden,
                              const float *topk_weights, const void *payload, const void *scales) {
  const int rc = check_problem(p);
  if (rc != MOE_OK) return rc;
  if (!plan || !plan->expert_counts || !plan->expert_offsets) return MOE_EINVAL;
  if (p->n_tokens > 0 && (!hidden || !plan->slot || !topk_weights)) return MOE_EINVAL;
  const bool quant = p->fmt != MOE_FMT_BF16;
  if (max_rows(*p) > 0 && (!payload || (quant && !scales))) return MOE_EINVAL;
  if (!quant && scales) return MOE_EINVAL;
  if (!aligned(hidden, 16) || !aligned(payload, 16) || !aligned(plan->slot, 4) || !aligned(topk_weights, 4) ||
      !aligned(plan->expert_counts, 4) || !aligned(plan->expert_offsets, 4) ||
      (p->fmt == MOE_FMT_FP8_E4M3_B128 && !aligned(scales, 4)))
    return MOE_EALIGN;
  if (p->fmt == MOE_FMT_NVFP4_B16) return MOE_EINVAL;
  return MOE_OK;
}

int check_combine_args(const moe_problem *p, const moe_plan *plan, const uint16_t *expert_out,
                       const float *topk_weights, const uint16_t *out) {
  const int rc = check_problem(p);
  if (rc != MOE_OK) return rc;
  if (!plan) return MOE_EINVAL;
  // expert_out may be NULL only when no slot can name a row (R_max = 0)
  if (p->n_tokens > 0 && (!out || !plan->slot || (max_rows(*p) > 0 && !expert_out))) return MOE_EINVAL;
  if (!aligned(expert_out, 16) || !aligned(out, 16) || !aligned(topk_weights, 4) || !aligned(plan->slot, 4))
    return MOE_EALIGN;
  return MOE_OK;
}

int check_exchange_plan_args(const moe_problem *p, const int32_t *topk_ids, const moe_exchange *x,
                             const void *workspace) {
  const int rc = check_exchange(p);
  if (rc != MOE_OK) return rc;
  if (!x || !x->expert_counts || !x->send_counts || !x->recv_expert_counts || !x->recv_rows ||
      !x->rank_table || !x->status || !workspace)
    return MOE_EINVAL;
  const int64_t pairs = p->n_tokens * p->ep * p->top_k;
  if (pairs > 0 && (!topk_ids || !x->recv_slot)) return MOE_EINVAL;
  if (p->recv_capacity > 0 && !x->recv_src) return MOE_EINVAL;
  if (!aligned(topk_ids, 4) || !aligned(x->expert_counts, 4) || !aligned(x->send_counts, 4) ||
      !aligned(x->recv_expert_counts, 4) || !aligned(x->recv_rows, 4) || !aligned(x->rank_table, 4) ||
      !aligned(x->recv_slot, 4) || !aligned(x->recv_src, 4) || !aligned(x->status, 4) ||
      !aligned(workspace, 256))
    return MOE_EALIGN;
  return MOE_OK;
}

int check_exchange_dispatch_args(const moe_problem *p, const moe_exchange *x, const uint16_t *hidden,
                                 const void *payload, const void *scales) {
  const int rc = check_exchange(p);
  if (rc != MOE_OK) return rc;
  if (!x || !x->recv_rows) return MOE_EINVAL;
  if (p->n_tokens > 0 && (!hidden || !x->recv_slot)) return MOE_EINVAL;
  const bool quant = p->fmt != MOE_FMT_BF16;
  if (p->recv_capacity > 0 && (!payload || (quant && !scales))) return MOE_EINVAL;
  if (!quant && scales) return MOE_EINVAL;
  if (!aligned(hidden, 16) || !aligned(payload, 16) || !aligned(x->recv_slot, 4) ||
      !aligned(x->recv_rows, 4) || (p->fmt == MOE_FMT_FP8_E4M3_B128 && !aligned(scales, 4)))
    return MOE_EALIGN;
  if (p->fmt == MOE_FMT_NVFP4_B16) return MOE_EINVAL;  // moe_exchange_dispatch_scaled
  return MOE_OK;
}

int check_exchange_dispatch_scaled_args(const moe_problem *p, const moe_exchange *x,
                                        const uint16_t *hidden, const float *input_scale,
                                        const void *payload, const void *scales) {
  const int rc = check_exchange(p);
  if (rc != MOE_OK) return rc;
  if (p->fmt != MOE_FMT_NVFP4_B16 || !input_scale) return MOE_EINVAL;
  if (!x || !x->recv_rows) return MOE_EINVAL;
  if (p->n_tokens > 0 && (!hidden || !x->recv_slot)) return MOE_EINVAL;
  if (p->recv_capacity > 0 && (!payload || !scales)) return MOE_EINVAL;
  if (!aligned(hidden, 16) || !aligned(payload, 16) || !aligned(x->recv_slot, 4) ||
      !aligned(x->recv_rows, 4) || !aligned(input_scale, 4))
    return MOE_EALIGN;
  return MOE_OK;
}

int check_exchange_dispatch_gated_args(const moe_problem *p, const moe_exchange *x,
                                       const uint16_t *hidden, const float *topk_weights,
                                       const void *payload, const void *scales) {
  const int rc = check_exchange(p);
  if (rc != MOE_OK) return rc;
  if (!x || !x->recv_rows) return MOE_EINVAL;
  if (p->n_tokens > 0 && (!hidden || !x->recv_slot || !topk_weights)) return MOE_EINVAL;
  const bool quant = p->fmt != MOE_FMT_BF16;
  if (p->recv_capacity > 0 && (!payload || (quant && !scales))) return MOE_EINVAL;
  if (!quant && scales) return MOE_EINVAL;
  if (!aligned(hidden, 16) || !aligned(payload, 16) || !aligned(x->recv_slot, 4) ||
      !aligned(x->recv_rows, 4) || !aligned(topk_weights, 4) ||
      (p->fmt == MOE_FMT_FP8_E4M3_B128 && !aligned(scales, 4)))
    return MOE_EALIGN;
  if (p->fmt == MOE_FMT_NVFP4_B16) return MOE_EINVAL;
  return MOE_OK;
}

int check_exchange_combine_args(const moe_problem *p, const moe_exchange *x, const uint16_t *expert_out,
                                const float *topk_weights, const uint16_t *out) {
  const int rc = check_exchange(p);
  if (rc != MOE_OK) return rc;
  if (!x) return MOE_EINVAL;
  // expert_out may be NULL only when no receive row exists (EP * C = 0)
  const bool no_rows = p->recv_capacity == 0;
  if (p->n_tokens > 0 && (!out || !x->recv_slot || (!no_rows && !expert_out))) return MOE_EINVAL;
  if (!aligned(expert_out, 16) || !aligned(out, 16) || !aligned(topk_weights, 4) || !aligned(x->recv_slot, 4))
    return MOE_EALIGN;
  return MOE_OK;
}

int check_map_args(const moe_problem *p, const uint8_t *routing_map, const float *probs,
                   const int32_t *topk_ids, const float *topk_weights, const uint32_t *status,
                   const void *workspace) {
  const int rc = check_problem(p);
  if (rc != MOE_OK) return rc;
  if (!status) return MOE_EINVAL;
  if (p->n_tokens > 0 && (!routing_map || !topk_ids || !workspace)) return MOE_EINVAL;
  if (!aligned(probs, 4) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4) || !aligned(status, 4) ||
      !aligned(workspace, 256))
    return MOE_EALIGN;
  return MOE_OK;
}

const char *error_text(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (null pointer, shape or divisibility)";
    case MOE_EALIGN: return "misaligned pointer (rows need 16 bytes, index arrays 4)";
    case MOE_EOVERFLOW: return "problem too large for 32-bit row indices or element counts";
    case MOE_EHIP: return "HIP launch error";
    case MOE_ESCRATCH:
      return "the problem's workspace exceeds the static scratch of moe_plan_and_dispatch_noalloc "
             "(MOE_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown error code";
  }
}

}  // namespace host
}  // namespace moe
