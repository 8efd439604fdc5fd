// api.hip -- the C ABI of libmoe: each entry point runs its host-side
// argument check (host_checks.cpp) and then its launches.  Declarations,
// argument meaning, layouts and error behaviour: include/moe.h.
#include <stdint.h>

#include <mutex>

#include "host_checks.hpp"
#include "moe.h"
#include "moe_kernels.hpp"

// Workspace of moe_plan_and_dispatch_noalloc: one per GPU, for the life of
// the process.  In host code `scratch` names a host-side stand-in, not the
// device array: host code uses only the address that hipGetSymbolAddress
// returns for the current device (noalloc_scratch below).
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

int launched(hipError_t err) { return err == hipSuccess ? MOE_OK : MOE_EHIP; }

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

using namespace moe::host;

MOE_API int moe_check_problem(const moe_problem *p) { return check_problem(p); }

MOE_API int64_t moe_max_rows(const moe_problem *p) {
  const int rc = check_problem(p);
  return rc != MOE_OK ? rc : moe::max_rows(*p);
}

MOE_API int64_t moe_expert_capacity(int64_t n_tokens, int32_t top_k, int32_t n_experts,
                                    double capacity_factor) {
  return moe::expert_capacity(n_tokens, top_k, n_experts, capacity_factor);
}

MOE_API int64_t moe_payload_row_bytes(const moe_problem *p) {
  const int rc = check_problem(p);
  return rc != MOE_OK ? rc : moe::payload_row_bytes(*p);
}

MOE_API int64_t moe_scale_row_bytes(const moe_problem *p) {
  const int rc = check_problem(p);
  return rc != MOE_OK ? rc : moe::scale_row_bytes(*p);
}

MOE_API size_t moe_workspace_bytes(const moe_problem *p) {
  if (check_problem(p) != MOE_OK) return 0;
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
  const int rc = check_dispatch_args(p, plan, hidden, payload, scales);
  if (rc != MOE_OK) return rc;
  return launched(moe::launch_dispatch(*p, *plan, hidden, nullptr, nullptr, payload, scales,
                                       static_cast<hipStream_t>(stream)));
}

MOE_API int moe_dispatch_scaled(const moe_problem *p, const moe_plan *plan, const uint16_t *hidden,
                                const float *input_scale, void *payload, void *scales, void *stream) {
  const int rc = check_dispatch_scaled_args(p, plan, hidden, input_scale, payload, scales);
  if (rc != MOE_OK) return rc;
  return launched(moe::launch_dispatch(*p, *plan, hidden, nullptr, input_scale, payload, scales,
                                       static_cast<hipStream_t>(stream)));
}

MOE_API int moe_dispatch_gated(const moe_problem *p, const moe_plan *plan, const uint16_t *hidden,
                               const float *topk_weights, void *payload, void *scales, void *stream) {
  const int rc = check_dispatch_gated_args(p, plan, hidden, topk_weights, payload, scales);
  if (rc != MOE_OK) return rc;
  // a null weight pointer selects the ungated kernels: keep the gated call gated
  const float *w = p->n_tokens > 0 ? topk_weights : nullptr;
  return launched(moe::launch_dispatch(*p, *plan, hidden, w, nullptr, payload, scales,
                                       static_cast<hipStream_t>(stream)));
}

MOE_API int moe_plan_and_dispatch_mode(const moe_problem *p) {
  const int rc = check_problem(p);
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
  const int rc = check_plan_and_dispatch_args(p, topk_ids, plan, hidden, topk_weights, input_scale, payload,
                                              scales, workspace);
  if (rc != MOE_OK) return rc;
  return pd_end(*p, topk_ids, *plan, hidden, topk_weights, input_scale, payload, scales, workspace,
                static_cast<hipStream_t>(stream));
}

MOE_API int moe_plan_and_dispatch(const moe_problem *p, const int32_t *topk_ids, const moe_plan *plan,
                                  const uint16_t *hidden, const float *topk_weights,
                                  const float *input_scale, void *payload, void *scales, void *workspace,
                                  void *stream) {
  int rc = check_plan_and_dispatch_args(p, topk_ids, plan, hidden, topk_weights, input_scale, payload, scales,
                                        workspace);
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
  const int rc = check_problem(p);
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
  const int rc = check_combine_args(p, plan, expert_out, topk_weights, out);
  if (rc != MOE_OK) return rc;
  return launched(moe::launch_combine(*p, *plan, expert_out, moe::max_rows(*p), topk_weights, out,
                                      static_cast<hipStream_t>(stream)));
}

MOE_API int moe_check_exchange(const moe_problem *p) { return check_exchange(p); }

MOE_API size_t moe_exchange_workspace_bytes(const moe_problem *p) {
  if (check_exchange(p) != MOE_OK) return 0;
  return moe::exchange_layout(*p).total;
}

MOE_API int moe_exchange_plan(const moe_problem *p, const int32_t *topk_ids, const moe_exchange *x,
                              void *workspace, void *stream) {
  const int rc = check_exchange_plan_args(p, topk_ids, x, workspace);
  if (rc != MOE_OK) return rc;
  return launched(moe::launch_exchange_plan(*p, topk_ids, *x, workspace, static_cast<hipStream_t>(stream)));
}

MOE_API int moe_exchange_dispatch(const moe_problem *p, const moe_exchange *x, const uint16_t *hidden,
                                  void *recv_payload, void *recv_scales, void *stream) {
  const int rc = check_exchange_dispatch_args(p, x, hidden, recv_payload, recv_scales);
  if (rc != MOE_OK) return rc;
  return launched(moe::launch_exchange_dispatch(*p, *x, hidden, nullptr, nullptr, recv_payload, recv_scales,
                                                static_cast<hipStream_t>(stream)));
}

MOE_API int moe_exchange_dispatch_scaled(const moe_problem *p, const moe_exchange *x, const uint16_t *hidden,
                                         const float *input_scale, void *recv_payload, void *recv_scales,
                                         void *stream) {
  const int rc = check_exchange_dispatch_scaled_args(p, x, hidden, input_scale, recv_payload, recv_scales);
  if (rc != MOE_OK) return rc;
  return launched(moe::launch_exchange_dispatch(*p, *x, hidden, nullptr, input_scale, recv_payload,
                                                recv_scales, static_cast<hipStream_t>(stream)));
}

MOE_API int moe_exchange_dispatch_gated(const moe_problem *p, const moe_exchange *x, const uint16_t *hidden,
                                        const float *topk_weights, void *recv_payload, void *recv_scales,
                                        void *stream) {
  const int rc = check_exchange_dispatch_gated_args(p, x, hidden, topk_weights, recv_payload, recv_scales);
  if (rc != MOE_OK) return rc;
  const float *w = p->n_tokens > 0 ? topk_weights : nullptr;
  return launched(moe::launch_exchange_dispatch(*p, *x, hidden, w, nullptr, recv_payload, recv_scales,
                                                static_cast<hipStream_t>(stream)));
}

MOE_API int moe_exchange_combine(const moe_problem *p, const moe_exchange *x, const uint16_t *expert_out,
                                 const float *topk_weights, uint16_t *out, void *stream) {
  const int rc = check_exchange_combine_args(p, x, expert_out, topk_weights, out);
  if (rc != MOE_OK) return rc;
  return launched(moe::launch_exchange_combine(*p, *x, expert_out, topk_weights, out,
                                               static_cast<hipStream_t>(stream)));
}

MOE_API size_t moe_map_workspace_bytes(const moe_problem *p) {
  if (check_problem(p) != MOE_OK) return 0;
  return moe::map_workspace_bytes(*p);
}

MOE_API int moe_routing_map_to_topk(const moe_problem *p, const uint8_t *routing_map, const float *probs,
                                    int32_t *topk_ids, float *topk_weights, uint32_t *status,
                                    void *workspace, void *stream) {
  const int rc = check_map_args(p, routing_map, probs, topk_ids, topk_weights, status, workspace);
  if (rc != MOE_OK) return rc;
  return launched(moe::launch_routing_map_to_topk(*p, routing_map, probs, topk_ids, topk_weights, status,
                                                  workspace, static_cast<hipStream_t>(stream)));
}

MOE_API const char *moe_strerror(int code) { return error_text(code); }

}  // extern "C"
