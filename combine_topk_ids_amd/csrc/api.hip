// api.hip -- the C ABI of libmoe: argument checks, sizes, and launches.
// Declarations, argument meaning, layouts and error behaviour: include/moe.h.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "moe.h"
#include "moe_kernels.hpp"

// Workspace of moe_plan_and_dispatch_noalloc: one per GPU, for the life of
// the process.  In host code `scratch` names a host-side stand-in, not the
// device array: host code uses only the address that hipGetSymbolAddress
// returns for the current device (noalloc_scratch below).
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int64_t max_rows_unchecked(const moe_problem &p) { return moe::max_rows(p); }

int check(const moe_problem *p) {
  if (!p) return MOE_EINVAL;
  if (p->n_tokens < 0 || p->hidden <= 0 || p->hidden % 8 != 0) return MOE_EINVAL;
  if (p->n_experts < 1 || p->n_experts > moe::kMaxExperts) return MOE_EINVAL;
  if (p->top_k < 1 || p->top_k > p->n_experts || p->top_k > moe::kMaxTopK) return MOE_EINVAL;
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
  const int64_t r_max = max_rows_unchecked(*p);
  if (r_max > INT32_MAX) return MOE_EOVERFLOW;
  // with a fixed capacity the plan forms e*cap + (rank in expert) and
  // e*cap + 2*cap in int32
  if (p->expert_capacity > 0 &&
      r_max + p->expert_capacity + p->n_tokens * p->top_k > INT32_MAX)
    return MOE_EOVERFLOW;
  if (r_max * static_cast<int64_t>(p->hidden) >= (int64_t{1} << 32)) return MOE_EOVERFLOW;
  if (p->n_tokens * static_cast<int64_t>(p->hidden) >= (int64_t{1} << 40)) return MOE_EOVERFLOW;
  // one wave per (token, column slab of >= 512 values) must index within int
  if (p->n_tokens * ((static_cast<int64_t>(p->hidden) + 511) / 512) > INT32_MAX / 4) return MOE_EOVERFLOW;
  return MOE_OK;
}

// The exchange: EP ranks of N tokens in one launch, receive buffers of C rows.
int check_exchange(const moe_problem *p) {
  const int rc = check(p);
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

int launched(hipError_t err) { return err == hipSuccess ? MOE_OK : MOE_EHIP; }

// Arguments of a plan: moe_dispatch_plan and both halves of
// moe_plan_and_dispatch.
int check_plan_args(const moe_problem *p, const int32_t *topk_ids, const moe_plan *plan,
                    const void *workspace) {
  const int rc = check(p);
  if (rc != MOE_OK) return rc;
  if (!plan || !plan->expert_counts || !plan->expert_offsets || !plan->dest_counts ||
      !plan->rank_table || !plan->status)
    return MOE_EINVAL;
  const int64_t npairs = p->n_tokens * p->top_k;
  if (npairs > 0 && (!topk_ids || !plan->slot)) return MOE_EINVAL;
  if (max_rows_unchecked(*p) > 0 && !plan->packed_src) return MOE_EINVAL;
  if (moe::plan_workspace_bytes(*p) > 0 && !workspace) return MOE_EINVAL;
  if (!aligned(topk_ids, 4) || !aligned(plan->expert_counts, 4) || !aligned(plan->expert_offsets, 4) ||
      !aligned(plan->dest_counts, 4) || !aligned(plan->rank_table, 4) || !aligned(plan->slot, 4) ||
      !aligned(plan->packed_src, 4) || !aligned(plan->status, 4) || !aligned(workspace, 256))
    return MOE_EALIGN;
  return MOE_OK;
}

// The dispatch arguments of moe_plan_and_dispatch (after check_plan_args):
// a global scale only for NVFP4, which takes no gates.
int check_pd_dispatch_args(const moe_problem *p, const uint16_t *hidden, const float *topk_weights,
                           const float *input_scale, const void *payload, const void *scales) {
  const bool nvfp4 = p->fmt == MOE_FMT_NVFP4_B16;
  if (nvfp4 != (input_scale != nullptr) || (nvfp4 && topk_weights)) return MOE_EINVAL;
  if (p->n_tokens > 0 && !hidden) return MOE_EINVAL;
  const bool quant = p->fmt != MOE_FMT_BF16;
  if (max_rows_unchecked(*p) > 0 && (!payload || (quant && !scales))) return MOE_EINVAL;
  if (!quant && scales) return MOE_EINVAL;
  if (!aligned(hidden, 16) || !aligned(payload, 16) || !aligned(topk_weights, 4) ||
      !aligned(input_scale, 4) || (p->fmt == MOE_FMT_FP8_E4M3_B128 && !aligned(scales, 4)))
    return MOE_EALIGN;
  return MOE_OK;
}

int pd_mode(const moe_problem &p) {
  switch (moe::plan_dispatch_mode(p)) {
    case moe::PlanDispatchMode::kOneLaunch: return MOE_PD_ONE_LAUNCH;
    case moe::PlanDispatchMode::kTiled: return MOE_PD_TILED;
    default: return MOE_PD_SEPARATE;
  }
}

// The launches of moe_plan_and_dispatch that need only topk_ids.
int pd_begin(const moe_problem &p, const int32_t *ids, const moe_plan &plan, void *workspace,
             hipStream_t s) {
  switch (moe::plan_dispatch_mode(p)) {
    case moe::PlanDispatchMode::kOneLaunch: return MOE_OK;
    case moe::PlanDispatchMode::kTiled:
      return launched(moe::launch_plan_count(p, ids, plan.status, workspace, s));
    default: return launched(moe::launch_plan(p, ids, plan, workspace, s));
  }
}

// The launch of moe_plan_and_dispatch that writes the payload.
int pd_end(const moe_problem &p, const int32_t *ids, const moe_plan &plan, const uint16_t *hidden,
           const float *topk_weights, const float *input_scale, void *payload, void *scales,
           void *workspace, hipStream_t s) {
  // a null weight pointer selects the ungated kernels
  const float *w = p.n_tokens > 0 ? topk_weights : nullptr;
  if (moe::plan_dispatch_mode(p) == moe::PlanDispatchMode::kSeparate)
    return launched(moe::launch_dispatch(p, plan, hidden, w, input_scale, payload, scales, s));
  return launched(moe::launch_plan_dispatch(p, ids, plan, hidden, w, input_scale, payload, scales,
                                            workspace, s));
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices] = {};

int noalloc_scratch(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOE_EHIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

MOE_API int moe_check_problem(const moe_problem *p) { return check(p); }

MOE_API int64_t moe_max_rows(const moe_problem *p) {
  const int rc = check(p);
  return rc != MOE_OK ? rc : max_rows_unchecked(*p);
}

MOE_API int64_t moe_expert_capacity(int64_t n_tokens, int32_t top_k, int32_t n_experts,
                                    double capacity_factor) {
  if (n_tokens < 0 || top_k < 1 || n_experts < 1 || !(capacity_factor >= 0.0)) return MOE_EINVAL;
  const double cap = ceil(capacity_factor * static_cast<double>(n_tokens) * static_cast<double>(top_k) /
                          static_cast<double>(n_experts));
  if (cap > static_cast<double>(INT32_MAX)) return MOE_EOVERFLOW;
  return static_cast<int64_t>(cap);
}

MOE_API int64_t moe_payload_row_bytes(const moe_problem *p) {
  const int rc = check(p);
  if (rc != MOE_OK) return rc;
  if (p->fmt == MOE_FMT_BF16) return 2 * static_cast<int64_t>(p->hidden);
  if (p->fmt == MOE_FMT_FP8_E4M3_B128) return p->hidden;
  if (p->fmt == MOE_FMT_NVFP4_B16) return p->hidden / 2;
  return p->hidden / 2;
}

MOE_API int64_t moe_scale_row_bytes(const moe_problem *p) {
  const int rc = check(p);
  if (rc != MOE_OK) return rc;
  if (p->fmt == MOE_FMT_BF16) return 0;
  if (p->fmt == MOE_FMT_FP8_E4M3_B128) return 4 * static_cast<int64_t>(p->hidden / 128);
  if (p->fmt == MOE_FMT_NVFP4_B16) return p->hidden / 16;
  return p->hidden / 32;
}

MOE_API size_t moe_workspace_bytes(const moe_problem *p) {
  if (check(p) != MOE_OK) return 0;
  return moe::plan_workspace_bytes(*p);
}

MOE_API int moe_dispatch_plan(const moe_problem *p, const int32_t *topk_ids, const moe_plan *plan,
                              void *workspace, void *stream) {
  const int rc = check_plan_args(p, topk_ids, plan, workspace);
  if (rc != MOE_OK) return rc;
  return launched(moe::launch_plan(*p, topk_ids, *plan, workspace, static_cast<hipStream_t>(stream)));
}

MOE_API int moe_dispatch(const moe_problem *p, const moe_plan *plan, const uint16_t *hidden,
                         void *payload, void *scales, void *stream) {
  const int rc = check(p);
  if (rc != MOE_OK) return rc;
  if (!plan || !plan->expert_counts || !plan->expert_offsets) return MOE_EINVAL;
  if (p->n_tokens > 0 && (!hidden || !plan->slot)) return MOE_EINVAL;
  const bool quant = p->fmt != MOE_FMT_BF16;
  if (max_rows_unchecked(*p) > 0 && (!payload || (quant && !scales))) return MOE_EINVAL;
  if (!quant && scales) return MOE_EINVAL;
  if (!aligned(hidden, 16) || !aligned(payload, 16) || !aligned(plan->slot, 4) ||
      !aligned(plan->expert_counts, 4) || !aligned(plan->expert_offsets, 4) ||
      (p->fmt == MOE_FMT_FP8_E4M3_B128 && !aligned(scales, 4)))
    return MOE_EALIGN;
  if (p->fmt == MOE_FMT_NVFP4_B16) return MOE_EINVAL;  // needs its global scale: moe_dispatch_scaled
  return launched(moe::launch_dispatch(*p, *plan, hidden, nullptr, nullptr, payload, scales,
                                       static_cast<hipStream_t>(stream)));
}

MOE_API int moe_dispatch_scaled(const moe_problem *p, const moe_plan *plan, const uint16_t *hidden,
                                const float *input_scale, void *payload, void *scales, void *stream) {
  const int rc = check(p);
  if (rc != MOE_OK) return rc;
  if (p->fmt != MOE_FMT_NVFP4_B16 || !input_scale) return MOE_EINVAL;
  if (!plan || !plan->expert_counts || !plan->expert_offsets) return MOE_EINVAL;
  if (p->n_tokens > 0 && (!hidden || !plan->slot)) return MOE_EINVAL;
  if (max_rows_unchecked(*p) > 0 && (!payload || !scales)) return MOE_EINVAL;
  if (!aligned(hidden, 16) || !aligned(payload, 16) || !aligned(plan->slot, 4) || !aligned(input_scale, 4) ||
      !aligned(plan->expert_counts, 4) || !aligned(plan->expert_offsets, 4))
    return MOE_EALIGN;
  return launched(moe::launch_dispatch(*p, *plan, hidden, nullptr, input_scale, payload, scales,
                                       static_cast<hipStream_t>(stream)));
}

MOE_API int moe_dispatch_gated(const moe_problem *p, const moe_plan *plan, const uint16_t *hidden,
                               const float *topk_weights, void *payload, void *scales, void *stream) {
  const int rc = check(p);
  if (rc != MOE_OK) return rc;
  if (!plan || !plan->expert_counts || !plan->expert_offsets) return MOE_EINVAL;
  if (p->n_tokens > 0 && (!hidden || !plan->slot || !topk_weights)) return MOE_EINVAL;
  const bool quant = p->fmt != MOE_FMT_BF16;
  if (max_rows_unchecked(*p) > 0 && (!payload || (quant && !scales))) return MOE_EINVAL;
  if (!quant && scales) return MOE_EINVAL;
  if (!aligned(hidden, 16) || !aligned(payload, 16) || !aligned(plan->slot, 4) || !aligned(topk_weights, 4) ||
      !aligned(plan->expert_counts, 4) || !aligned(plan->expert_offsets, 4) ||
      (p->fmt == MOE_FMT_FP8_E4M3_B128 && !aligned(scales, 4)))
    return MOE_EALIGN;
  // a null weight pointer selects the ungated kernels: keep the gated call gated
  if (p->fmt == MOE_FMT_NVFP4_B16) return MOE_EINVAL;
  const float *w = p->n_tokens > 0 ? topk_weights : nullptr;
  return launched(moe::launch_dispatch(*p, *plan, hidden, w, nullptr, payload, scales,
                                       static_cast<hipStream_t>(stream)));
}

MOE_API int moe_plan_and_dispatch_mode(const moe_problem *p) {
  const int rc = check(p);
  if (rc != MOE_OK) return rc;
  return pd_mode(*p);
}

MOE_API int moe_plan_and_dispatch_begin(const moe_problem *p, const int32_t *topk_ids, const moe_plan *plan,
                                        void *workspace, void *stream) {
  const int rc = check_plan_args(p, topk_ids, plan, workspace);
  if (rc != MOE_OK) return rc;
  return pd_begin(*p, topk_ids, *plan, workspace, static_cast<hipStream_t>(stream));
}

MOE_API int moe_plan_and_dispatch_end(const moe_problem *p, const int32_t *topk_ids, const moe_plan *plan,
                                      const uint16_t *hidden, const float *topk_weights,
                                      const float *input_scale, void *payload, void *scales, void *workspace,
                                      void *stream) {
  int rc = check_plan_args(p, topk_ids, plan, workspace);
  if (rc == MOE_OK) rc = check_pd_dispatch_args(p, hidden, topk_weights, input_scale, payload, scales);
  if (rc != MOE_OK) return rc;
  return pd_end(*p, topk_ids, *plan, hidden, topk_weights, input_scale, payload, scales, workspace,
                static_cast<hipStream_t>(stream));
}

MOE_API int moe_plan_and_dispatch(const moe_problem *p, const int32_t *topk_ids, const moe_plan *plan,
                                  const uint16_t *hidden, const float *topk_weights,
                                  const float *input_scale, void *payload, void *scales, void *workspace,
                                  void *stream) {
  int rc = check_plan_args(p, topk_ids, plan, workspace);
  if (rc == MOE_OK) rc = check_pd_dispatch_args(p, hidden, topk_weights, input_scale, payload, scales);
  if (rc != MOE_OK) return rc;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  rc = pd_begin(*p, topk_ids, *plan, workspace, s);
  if (rc != MOE_OK) return rc;
  return pd_end(*p, topk_ids, *plan, hidden, topk_weights, input_scale, payload, scales, workspace, s);
}

MOE_API int moe_plan_and_dispatch_noalloc(const moe_problem *p, const int32_t *topk_ids,
                                          const moe_plan *plan, const uint16_t *hidden,
                                          const float *topk_weights, const float *input_scale,
                                          void *payload, void *scales, void *stream) {
  const int rc = check(p);
  if (rc != MOE_OK) return rc;
  const size_t need = moe::plan_workspace_bytes(*p);
  if (need > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ESCRATCH;
  void *ws = nullptr;
  if (need > 0) {
    const int src = noalloc_scratch(&ws);
    if (src != MOE_OK) return src;
  }
  return moe_plan_and_dispatch(p, topk_ids, plan, hidden, topk_weights, input_scale, payload, scales,
                               ws, stream);
}

MOE_API int moe_combine(const moe_problem *p, const moe_plan *plan, const uint16_t *expert_out,
                        const float *topk_weights, uint16_t *out, void *stream) {
  const int rc = check(p);
  if (rc != MOE_OK) return rc;
  if (!plan) return MOE_EINVAL;
  // expert_out may be NULL only when no slot can name a row (R_max = 0)
  const int64_t rows = max_rows_unchecked(*p);
  if (p->n_tokens > 0 && (!out || !plan->slot || (rows > 0 && !expert_out))) return MOE_EINVAL;
  if (!aligned(expert_out, 16) || !aligned(out, 16) || !aligned(topk_weights, 4) || !aligned(plan->slot, 4))
    return MOE_EALIGN;
  return launched(moe::launch_combine(*p, *plan, expert_out, rows, topk_weights, out,
                                      static_cast<hipStream_t>(stream)));
}

MOE_API int moe_check_exchange(const moe_problem *p) { return check_exchange(p); }

MOE_API size_t moe_exchange_workspace_bytes(const moe_problem *p) {
  if (check_exchange(p) != MOE_OK) return 0;
  return moe::exchange_workspace_bytes(*p);
}

MOE_API int moe_exchange_plan(const moe_problem *p, const int32_t *topk_ids, const moe_exchange *x,
                              void *workspace, void *stream) {
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
  return launched(moe::launch_exchange_plan(*p, topk_ids, *x, workspace, static_cast<hipStream_t>(stream)));
}

MOE_API int moe_exchange_dispatch(const moe_problem *p, const moe_exchange *x, const uint16_t *hidden,
                                  void *recv_payload, void *recv_scales, void *stream) {
  const int rc = check_exchange(p);
  if (rc != MOE_OK) return rc;
  if (!x || !x->recv_rows) return MOE_EINVAL;
  if (p->n_tokens > 0 && (!hidden || !x->recv_slot)) return MOE_EINVAL;
  const bool quant = p->fmt != MOE_FMT_BF16;
  if (p->recv_capacity > 0 && (!recv_payload || (quant && !recv_scales))) return MOE_EINVAL;
  if (!quant && recv_scales) return MOE_EINVAL;
  if (!aligned(hidden, 16) || !aligned(recv_payload, 16) || !aligned(x->recv_slot, 4) ||
      !aligned(x->recv_rows, 4) || (p->fmt == MOE_FMT_FP8_E4M3_B128 && !aligned(recv_scales, 4)))
    return MOE_EALIGN;
  if (p->fmt == MOE_FMT_NVFP4_B16) return MOE_EINVAL;  // moe_exchange_dispatch_scaled
  return launched(moe::launch_exchange_dispatch(*p, *x, hidden, nullptr, nullptr, recv_payload, recv_scales,
                                                static_cast<hipStream_t>(stream)));
}

MOE_API int moe_exchange_dispatch_scaled(const moe_problem *p, const moe_exchange *x, const uint16_t *hidden,
                                         const float *input_scale, void *recv_payload, void *recv_scales,
                                         void *stream) {
  const int rc = check_exchange(p);
  if (rc != MOE_OK) return rc;
  if (p->fmt != MOE_FMT_NVFP4_B16 || !input_scale) return MOE_EINVAL;
  if (!x || !x->recv_rows) return MOE_EINVAL;
  if (p->n_tokens > 0 && (!hidden || !x->recv_slot)) return MOE_EINVAL;
  if (p->recv_capacity > 0 && (!recv_payload || !recv_scales)) return MOE_EINVAL;
  if (!aligned(hidden, 16) || !aligned(recv_payload, 16) || !aligned(x->recv_slot, 4) ||
      !aligned(x->recv_rows, 4) || !aligned(input_scale, 4))
    return MOE_EALIGN;
  return launched(moe::launch_exchange_dispatch(*p, *x, hidden, nullptr, input_scale, recv_payload,
                                                recv_scales, static_cast<hipStream_t>(stream)));
}

MOE_API int moe_exchange_dispatch_gated(const moe_problem *p, const moe_exchange *x, const uint16_t *hidden,
                                        const float *topk_weights, void *recv_payload, void *recv_scales,
                                        void *stream) {
  const int rc = check_exchange(p);
  if (rc != MOE_OK) return rc;
  if (!x || !x->recv_rows) return MOE_EINVAL;
  if (p->n_tokens > 0 && (!hidden || !x->recv_slot || !topk_weights)) return MOE_EINVAL;
  const bool quant = p->fmt != MOE_FMT_BF16;
  if (p->recv_capacity > 0 && (!recv_payload || (quant && !recv_scales))) return MOE_EINVAL;
  if (!quant && recv_scales) return MOE_EINVAL;
  if (!aligned(hidden, 16) || !aligned(recv_payload, 16) || !aligned(x->recv_slot, 4) ||
      !aligned(x->recv_rows, 4) || !aligned(topk_weights, 4) ||
      (p->fmt == MOE_FMT_FP8_E4M3_B128 && !aligned(recv_scales, 4)))
    return MOE_EALIGN;
  if (p->fmt == MOE_FMT_NVFP4_B16) return MOE_EINVAL;
  const float *w = p->n_tokens > 0 ? topk_weights : nullptr;
  return launched(moe::launch_exchange_dispatch(*p, *x, hidden, w, nullptr, recv_payload, recv_scales,
                                                static_cast<hipStream_t>(stream)));
}

MOE_API int moe_exchange_combine(const moe_problem *p, const moe_exchange *x, const uint16_t *expert_out,
                                 const float *topk_weights, uint16_t *out, void *stream) {
  const int rc = check_exchange(p);
  if (rc != MOE_OK) return rc;
  if (!x) return MOE_EINVAL;
  // expert_out may be NULL only when no receive row exists (EP * C = 0)
  const bool no_rows = p->recv_capacity == 0;
  if (p->n_tokens > 0 && (!out || !x->recv_slot || (!no_rows && !expert_out))) return MOE_EINVAL;
  if (!aligned(expert_out, 16) || !aligned(out, 16) || !aligned(topk_weights, 4) || !aligned(x->recv_slot, 4))
    return MOE_EALIGN;
  return launched(moe::launch_exchange_combine(*p, *x, expert_out, topk_weights, out,
                                               static_cast<hipStream_t>(stream)));
}

MOE_API size_t moe_map_workspace_bytes(const moe_problem *p) {
  if (check(p) != MOE_OK) return 0;
  return moe::map_workspace_bytes(*p);
}

MOE_API int moe_routing_map_to_topk(const moe_problem *p, const uint8_t *routing_map, const float *probs,
                                    int32_t *topk_ids, float *topk_weights, uint32_t *status,
                                    void *workspace, void *stream) {
  const int rc = check(p);
  if (rc != MOE_OK) return rc;
  if (!status) return MOE_EINVAL;
  if (p->n_tokens > 0 && (!routing_map || !topk_ids || !workspace)) return MOE_EINVAL;
  if (!aligned(probs, 4) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4) || !aligned(status, 4) ||
      !aligned(workspace, 256))
    return MOE_EALIGN;
  return launched(moe::launch_routing_map_to_topk(*p, routing_map, probs, topk_ids, topk_weights, status,
                                                  workspace, static_cast<hipStream_t>(stream)));
}

MOE_API const char *moe_strerror(int code) {
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

}  // extern "C"
