// routing_map.hip -- dense multihot routing map to the compact top-k form.
//
// What is computed (pages cited by title and section):
//   NeMo Automodel token_dispatcher API -- _DeepepManager._indices_to_multihot
//     (top-k indices with -1 masks and their probabilities correspond to a
//     multihot routing map and multihot probabilities), the conversion from
//     top-k indices to the multihot routing_map format, and
//     TokenDispatcherConfig.moe_hybridep_compact_routing (routing handed over
//     either as compact top-k indices or as a dense Boolean map).
//
// For every token: the experts whose map byte is nonzero, in ascending
// order, fill ids[t][0..); their probabilities (1 without a probability
// array) fill weights[t][0..); the remaining slots get -1 and 0.  A token
// with more than k routed experts keeps its first k, and the call's status
// word gets MOE_STATUS_MAP_OVERFLOW.
//
// Design for gfx950.  The work is tiny, so latency decides.  A token's row
// is read by a group of lanes in one round of loads: each lane takes 16
// experts (one 16-byte load when rows are 16-byte aligned, else byte
// loads), so a group is ceil(E/16) lanes rounded up to a power of two, at
// most a wave (E <= 1024).  A segmented prefix sum of the lanes' counts of
// routed experts gives every lane the first output slot of its experts;
// the probabilities of those experts are loaded together, then stored.
// Each block ORs its overflow flags into one workspace word, and a
// one-block kernel ORs those into the status word, so the status needs no
// clearing before the call.
#include "moe_device.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

constexpr int kThreads = kMapThreads;
constexpr int kLaneExperts = kMapLaneExperts;  // map bytes per lane

struct MapArgs {
  const uint8_t *map;
  const float *probs;
  int32_t *ids;
  float *w;
  uint32_t *partial;  // [nblocks] overflow flags per block
  uint32_t *status;
  int64_t n;
  int e, k;
  int lpt;            // lanes per token: a power of two, at most a wave
  int nblocks;
  bool vec;           // rows are 16-byte aligned
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void map_to_topk_kernel(MapArgs g) {
  const int lpt = g.lpt;
  const int sl = threadIdx.x & (lpt - 1);  // lane within the token's group
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (kThreads / lpt) + threadIdx.x / lpt;
  const bool live = t < g.n;
  const int e0 = sl * kLaneExperts;  // this lane's experts e0 .. e0+15
  uint32_t nz = 0;                   // bit i: expert e0 + i is routed
  if (live && e0 < g.e) {
    const uint8_t *row = g.map + t * g.e;
    if (g.vec) {  // E % 16 == 0, so e0 + 16 <= E
      const u32x4 v = *reinterpret_cast<const u32x4 *>(row + e0);
      const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < kLaneExperts; ++i)
        nz |= ((wd[i / 4] >> (8 * (i % 4))) & 0xFFu) != 0 ? 1u << i : 0u;
    } else {
      uint8_t b[kLaneExperts];
#pragma unroll
      for (int i = 0; i < kLaneExperts; ++i) b[i] = e0 + i < g.e ? row[e0 + i] : 0;
#pragma unroll
      for (int i = 0; i < kLaneExperts; ++i) nz |= b[i] != 0 ? 1u << i : 0u;
    }
  }
  // routed experts before this lane's, and in the whole row
  const int cnt = __popc(nz);
  int inc = cnt;
  for (int d = 1; d < lpt; d <<= 1) {
    const int v = __shfl_up(inc, d, lpt);
    if (sl >= d) inc += v;
  }
  const int total = __shfl(inc, lpt - 1, lpt);
  const uint32_t fl = live && total > g.k ? MOE_STATUS_MAP_OVERFLOW : 0u;
  if (live) {
    int32_t *ids = g.ids + t * g.k;
    float *w = g.w ? g.w + t * g.k : nullptr;
    const float *pr = g.probs ? g.probs + t * g.e : nullptr;
    int pos = inc - cnt;
    // the ascending experts of this lane that still fit: probabilities
    // loaded together first, then every store
    uint32_t keep = 0;
    {
      uint32_t m = nz;
      for (int p = pos; m != 0 && p < g.k; ++p) {
        keep |= m & (~m + 1u);
        m &= m - 1u;
      }
    }
    float pv[kLaneExperts];
#pragma unroll
    for (int i = 0; i < kLaneExperts; ++i) pv[i] = (w && pr && ((keep >> i) & 1u)) ? pr[e0 + i] : 1.0f;
#pragma unroll
    for (int i = 0; i < kLaneExperts; ++i) {
      if ((keep >> i) & 1u) {
        ids[pos] = e0 + i;
        if (w) w[pos] = pv[i];
        ++pos;
      }
    }
    for (int j = total + sl; j < g.k; j += lpt) {
      ids[j] = -1;
      if (w) w[j] = 0.0f;
    }
  }
  const uint64_t any = ballot(fl != 0);
  __shared__ uint32_t s_fl;
  if (threadIdx.x == 0) s_fl = 0;
  __syncthreads();
  if (lane_id() == 0 && any) atomicOr(&s_fl, MOE_STATUS_MAP_OVERFLOW);
  __syncthreads();
  if (threadIdx.x == 0) g.partial[blockIdx.x] = s_fl;
}

__global__ __launch_bounds__(kThreads) void map_status_kernel(MapArgs g) {
  uint32_t fl = 0;
  for (int b = threadIdx.x; b < g.nblocks; b += kThreads) fl |= g.partial[b];
  const uint64_t any = ballot(fl != 0);
  __shared__ uint32_t s_fl;
  if (threadIdx.x == 0) s_fl = 0;
  __syncthreads();
  if (lane_id() == 0 && any) atomicOr(&s_fl, MOE_STATUS_MAP_OVERFLOW);
  __syncthreads();
  if (threadIdx.x == 0) *g.status = s_fl;
}

}  // namespace

hipError_t launch_routing_map_to_topk(const moe_problem &p, const uint8_t *map, const float *probs,
                                      int32_t *ids, float *weights, uint32_t *status, void *workspace,
                                      hipStream_t stream) {
  MapArgs g;
  g.map = map;
  g.probs = probs;
  g.ids = ids;
  g.w = weights;
  g.partial = static_cast<uint32_t *>(workspace);
  g.status = status;
  g.n = p.n_tokens;
  g.e = p.n_experts;
  g.k = p.top_k;
  g.lpt = map_lanes_per_token(p.n_experts);
  g.nblocks = map_blocks(p);
  g.vec = p.n_experts % 16 == 0 && (reinterpret_cast<uintptr_t>(map) & 15) == 0;
  if (g.nblocks > 0) map_to_topk_kernel<<<g.nblocks, kThreads, 0, stream>>>(g);
  map_status_kernel<<<1, kThreads, 0, stream>>>(g);
  return hipGetLastError();
}

}  // namespace moe
