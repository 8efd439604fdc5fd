// plan.hip -- routing-plan kernels: per-expert counts, padded cumsum offsets,
// the (4, EP) counts/displacements table, fault bits, and a stable slot for
// every (token, k) pair.
//
// What is computed (pages cited by title and section):
//   NKI permute_a2av API reference -- description: rows of each destination
//     rank are packed at cumsum(send_counts) offsets and described by a
//     (4, EP) uint32 table of counts and displacements in elements;
//     :param packed_source_indices: source rows in [0, N), destination-major;
//     :param recv_capacity: the dropless per-rank bound N * min(top_k, L).
//   NeMo Automodel token_dispatcher API -- dispatch_postprocess (tokens per
//     expert), TokenDispatcherConfig.moe_router_expert_pad_multiple (each
//     expert padded to a multiple), _indices_to_multihot (-1 masks a slot),
//     _HybridEPMetadataProcessor.forward (metadata built on the device with
//     no host round trip, so it can live inside a captured graph).
//   DeepSpeed v0.19.4 function index, page 15 -- SplitPlan entry: the
//     per-expert histogram read as an [ep_size, E_local] count matrix.
//   Mojo shmem ep_comm module -- block_prefix_sum (block-wide scan).
//
// Design for gfx950.  The pairs t*k+j are cut into tiles of 2048.  Slots
// must follow flat pair order inside each expert whatever order atomics land
// in, so every position comes from counts and scans, never from an atomic's
// return value:
//   plan_count   (one block per tile) histogram of the tile in LDS -> HBM
//                [ntiles][E] plus the tile's fault bits.
//   plan_assign  (one block per tile) every block re-reduces the small
//                histogram matrix (totals and the prefix over earlier
//                tiles), scans the padded counts over experts, then each wave
//                walks its 64-pair chunks in order, ranking equal expert IDs
//                inside the chunk with a ballot-based match (one ballot per ID
//                bit) and advancing a per-wave cursor per expert in LDS;
//                block 0 also writes counts, offsets, table and status.
// A plan of at most 2048 pairs (decode shapes) runs as one block of
// plan_assign that also does the counting: one launch.
//
// Latency matters more than bandwidth here (the whole plan moves < 2 MB):
// each kernel issues all of its global loads first, keeps every
// intermediate in LDS, and issues its global stores last, so no barrier has
// to wait for stores to drain.
#include "moe_device.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

constexpr int kTilePairs = 2048;                       // multiple of kPlanThreads
constexpr int kPairsPerThread = kTilePairs / kPlanThreads;
constexpr int kHistBatch = 32;                         // histogram loads in flight per thread

struct PlanArgs {
  const int32_t *ids;
  int64_t npairs;
  int64_t r_max;
  int64_t cap;
  uint32_t h;
  int k, e, ep, a;
  int ntiles;
  int key_bits;
  int32_t *counts, *offsets, *dest_counts;
  uint32_t *table;
  int32_t *slot, *packed_src;
  uint32_t *status;
  int32_t *hist;     // workspace [ntiles][E]
  uint32_t *tflags;  // workspace [ntiles]
};

__device__ __forceinline__ int padded(int c, int a) { return ((c + a - 1) / a) * a; }

__device__ __forceinline__ uint32_t wave_or_bits(uint32_t v) {
  return (ballot(v & 1u) ? 1u : 0u) | (ballot(v & 2u) ? 2u : 0u) | (ballot(v & 4u) ? 4u : 0u);
}

// Load the tile's IDs into LDS, starting at the first pair of the token that
// owns pair `begin` (so each token's earlier slots are at hand for the
// repeated-ID check).  All loads are issued before any is used.  Returns the
// lead-in length (< k).  The caller places a barrier before reading s_ids.
__device__ int stage_ids(const PlanArgs &g, int64_t begin, int64_t end, int *s_ids) {
  const int tid = threadIdx.x;
  // pair indices fit in 31 bits (checked on the host)
  const int pre = static_cast<int>(static_cast<uint32_t>(begin) % static_cast<uint32_t>(g.k));
  const int len = static_cast<int>(end - begin);
  int v[kPairsPerThread];
#pragma unroll
  for (int u = 0; u < kPairsPerThread; ++u) {
    const int i = u * kPlanThreads + tid;
    v[u] = i < len ? g.ids[begin + i] : -1;
  }
  const int lead = tid < pre ? g.ids[begin - pre + tid] : 0;
#pragma unroll
  for (int u = 0; u < kPairsPerThread; ++u) {
    const int i = u * kPlanThreads + tid;
    if (i < len) s_ids[pre + i] = v[u];
  }
  if (tid < pre) s_ids[tid] = lead;
  return pre;
}

// Histogram of the valid pairs of [begin, end) into s_cnt (zeroed); returns
// this thread's BAD_ID / DUP_ID bits.
__device__ uint32_t count_tile(const PlanArgs &g, int64_t begin, int64_t end, const int *s_ids,
                               int pre, int *s_cnt) {
  uint32_t fl = 0;
  const int len = static_cast<int>(end - begin);
  const uint32_t k = static_cast<uint32_t>(g.k);
  const uint32_t j0 = static_cast<uint32_t>(pre);  // position in its token of pair `begin`
#pragma unroll
  for (int u = 0; u < kPairsPerThread; ++u) {
    const int i = u * kPlanThreads + threadIdx.x;
    if (i >= len) break;
    const int e = s_ids[pre + i];
    if (e == -1) continue;
    if (e < -1 || e >= g.e) {
      fl |= MOE_STATUS_BAD_ID;
      continue;
    }
    const int j = static_cast<int>((j0 + static_cast<uint32_t>(i)) % k);
    for (int q = pre + i - j; q < pre + i; ++q)
      if (s_ids[q] == e) fl |= MOE_STATUS_DUP_ID;
    atomicAdd(&s_cnt[e], 1);
  }
  return fl;
}

__global__ __launch_bounds__(kPlanThreads) void plan_count_kernel(PlanArgs g) {
  extern __shared__ int smem[];
  int *s_cnt = smem;        // [E]
  int *s_ids = smem + g.e;  // [kTilePairs + kMaxTopK]
  __shared__ uint32_t s_fl;
  const int b = blockIdx.x;
  const int64_t begin = static_cast<int64_t>(b) * kTilePairs;
  const int64_t end = min(begin + kTilePairs, g.npairs);
  const int pre = stage_ids(g, begin, end, s_ids);
  for (int e = threadIdx.x; e < g.e; e += kPlanThreads) s_cnt[e] = 0;
  if (threadIdx.x == 0) s_fl = 0;
  __syncthreads();
  const uint32_t fl = wave_or_bits(count_tile(g, begin, end, s_ids, pre, s_cnt));
  if (lane_id() == 0 && fl) atomicOr(&s_fl, fl);
  __syncthreads();
  int32_t *hrow = g.hist + static_cast<int64_t>(b) * g.e;
  for (int e = threadIdx.x; e < g.e; e += kPlanThreads) hrow[e] = s_cnt[e];
  if (threadIdx.x == 0) g.tflags[b] = s_fl;
}

template <bool kSingle>
__global__ __launch_bounds__(kPlanThreads) void plan_assign_kernel(PlanArgs g) {
  extern __shared__ int smem[];
  const int E = g.e;
  int *s_tot = smem;                    // [E]   c_e
  int *s_pre = s_tot + E;               // [E]   pairs of e in tiles before this one
  int *s_off = s_pre + E;               // [E+1] padded exclusive cumsum
  int *s_cpre = s_off + E + 1;          // [E+1] unpadded exclusive cumsum
  int *s_cur = s_cpre + E + 1;          // [kPlanWaves][E] per-wave cursors
  int *s_ids = s_cur + kPlanWaves * E;  // [kTilePairs + kMaxTopK]
  __shared__ uint32_t s_fl;
  __shared__ int s_scan[2][kPlanWaves];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int b = blockIdx.x;
  const int64_t begin = static_cast<int64_t>(b) * kTilePairs;
  const int64_t end = min(begin + kTilePairs, g.npairs);
  const int len = static_cast<int>(end - begin);

  // ---- global loads first: the first batch of the histogram matrix, then
  // the tile's IDs ---------------------------------------------------------
  const int total = kSingle ? 0 : g.ntiles * E;
  int hv[kHistBatch];
#pragma unroll
  for (int u = 0; u < kHistBatch; ++u) {
    const int i = u * kPlanThreads + tid;
    hv[u] = i < total ? g.hist[i] : 0;
  }
  const int pre = stage_ids(g, begin, end, s_ids);
  for (int e = tid; e < E; e += kPlanThreads) {
    s_tot[e] = 0;
    s_pre[e] = 0;
  }
  for (int i = tid; i < kPlanWaves * E; i += kPlanThreads) s_cur[i] = 0;
  if (tid == 0) s_fl = 0;
  __syncthreads();

  uint32_t fl = 0;
  if (kSingle) {
    fl = count_tile(g, begin, end, s_ids, pre, s_tot);
  } else {
    for (int base = 0; base < total; base += kHistBatch * kPlanThreads) {
      if (base > 0) {
#pragma unroll
        for (int u = 0; u < kHistBatch; ++u) {
          const int i = base + u * kPlanThreads + tid;
          hv[u] = i < total ? g.hist[i] : 0;
        }
      }
#pragma unroll
      for (int u = 0; u < kHistBatch; ++u) {
        if (hv[u]) {
          const int i = base + u * kPlanThreads + tid;
          const int tile = i / E;
          const int e = i - tile * E;
          atomicAdd(&s_tot[e], hv[u]);
          if (tile < b) atomicAdd(&s_pre[e], hv[u]);
        }
      }
    }
    for (int i = tid; i < g.ntiles; i += kPlanThreads) fl |= g.tflags[i];
  }
  // per-wave counts of this tile's pairs (cursor bases come later)
  // pairs per wave: the tile split evenly over the waves in 64-pair chunks
  const int wp = ((len + kPlanWaves * kWave - 1) / (kPlanWaves * kWave)) * kWave;
  const int wb = wave * wp, we = min(wb + wp, len);
  int *cur = s_cur + wave * E;
  for (int i = wb + lane; i < we; i += kWave) {
    const int e = s_ids[pre + i];
    if (e >= 0 && e < E) atomicAdd(&cur[e], 1);
  }
  fl = wave_or_bits(fl);
  if (lane == 0 && fl) atomicOr(&s_fl, fl);
  __syncthreads();

  // ---- padded and unpadded exclusive scans over experts -----------------
  {
    const int per = (E + kPlanThreads - 1) / kPlanThreads;
    const int e0 = min(tid * per, E), e1 = min(e0 + per, E);
    int sp = 0, sc = 0;
    for (int e = e0; e < e1; ++e) {
      const int c = s_tot[e];
      sc += c;
      sp += padded(c, g.a);
    }
    const int ip = wave_incl_scan(sp), ic = wave_incl_scan(sc);
    if (lane == kWave - 1) {
      s_scan[0][wave] = ip;
      s_scan[1][wave] = ic;
    }
    __syncthreads();
    int xp = ip - sp, xc = ic - sc;
    for (int w = 0; w < wave; ++w) {
      xp += s_scan[0][w];
      xc += s_scan[1][w];
    }
    for (int e = e0; e < e1; ++e) {
      const int c = s_tot[e];
      s_off[e] = xp;
      s_cpre[e] = xc;
      xp += padded(c, g.a);
      xc += c;
    }
    if (tid == 0) {
      int tp = 0, tc = 0;
      for (int w = 0; w < kPlanWaves; ++w) {
        tp += s_scan[0][w];
        tc += s_scan[1][w];
      }
      s_off[E] = tp;
      s_cpre[E] = tc;
    }
  }
  __syncthreads();

  // ---- cursor bases: offset + earlier tiles + earlier waves of this tile --
  for (int e = tid; e < E; e += kPlanThreads) {
    int run = s_off[e] + s_pre[e];
#pragma unroll
    for (int w = 0; w < kPlanWaves; ++w) {
      const int c = s_cur[w * E + e];
      s_cur[w * E + e] = run;
      run += c;
    }
  }
  // capacity check (block 0 only needs it; cheap everywhere)
  const int L = E / g.ep;
  uint32_t cap = 0;
  for (int r = tid; r < g.ep; r += kPlanThreads)
    if (s_cpre[(r + 1) * L] - s_cpre[r * L] > g.cap) cap = MOE_STATUS_CAPACITY;
  cap = wave_or_bits(cap);
  if (lane == 0 && cap) atomicOr(&s_fl, cap);
  __syncthreads();

  // ---- stores only from here on -------------------------------------------
  // stable slots: walk this wave's pairs in 64-pair chunks, in order
  const uint32_t k = static_cast<uint32_t>(g.k);
  for (int i0 = wb; i0 < we; i0 += kWave) {
    const int i = i0 + lane;
    const bool in = i < we;
    const int e = in ? s_ids[pre + i] : -1;
    const bool valid = in && e >= 0 && e < E;
    int sl = -1;
    const uint64_t act = ballot(valid);
    if (valid) {
      const uint64_t m = match_any(static_cast<uint32_t>(e), g.key_bits, act);
      const int r = lanes_below(m);
      const int base = cur[e];
      sl = base + r;
      if (r == 0) cur[e] = base + __popcll(m);
      const uint32_t p = static_cast<uint32_t>(begin + i);
      g.packed_src[sl] = static_cast<int32_t>(p / k);
    }
    if (in) g.slot[begin + i] = sl;
  }

  // block 0: counts, offsets, per-rank table, status
  if (b == 0) {
    for (int e = tid; e < E; e += kPlanThreads) {
      g.counts[e] = s_tot[e];
      g.offsets[e] = s_off[e];
    }
    if (tid == 0) {
      g.offsets[E] = s_off[E];
      *g.status = s_fl;
    }
    for (int r = tid; r < g.ep; r += kPlanThreads) {
      const int lo = r * L, hi = lo + L;
      const int S = s_cpre[hi] - s_cpre[lo];
      const int P = s_off[hi] - s_off[lo];
      g.dest_counts[r] = S;
      g.table[r] = static_cast<uint32_t>(S) * g.h;
      g.table[g.ep + r] = static_cast<uint32_t>(s_cpre[lo]) * g.h;
      g.table[2 * g.ep + r] = static_cast<uint32_t>(P) * g.h;
      g.table[3 * g.ep + r] = static_cast<uint32_t>(s_off[lo]) * g.h;
    }
  }

  // packed_src = -1 on pad rows (an expert has at most A-1 of them: the grid
  // strides over all E*(A-1) candidates) and on the tail rows
  if (g.a > 1) {
    const int per = g.a - 1;
    const int cand = E * per;
    for (int q = b * kPlanThreads + tid; q < cand; q += g.ntiles * kPlanThreads) {
      const int e = q / per;
      const int r = s_off[e] + s_tot[e] + (q - e * per);
      if (r < s_off[e + 1]) g.packed_src[r] = -1;
    }
  }
  for (int64_t r = s_off[E] + static_cast<int64_t>(b) * kPlanThreads + tid; r < g.r_max;
       r += static_cast<int64_t>(g.ntiles) * kPlanThreads)
    g.packed_src[r] = -1;
}

}  // namespace

PlanGeom plan_geometry(const moe_problem &p) {
  PlanGeom geo;
  geo.npairs = p.n_tokens * p.top_k;
  geo.tile_pairs = kTilePairs;
  geo.ntiles = geo.npairs == 0 ? 1 : static_cast<int>((geo.npairs + kTilePairs - 1) / kTilePairs);
  geo.single = geo.ntiles == 1;
  int bits = 0;
  while ((1 << bits) < p.n_experts) ++bits;
  geo.key_bits = bits;
  return geo;
}

size_t plan_workspace_bytes(const moe_problem &p) {
  const PlanGeom geo = plan_geometry(p);
  if (geo.single) return 0;
  const size_t bytes = static_cast<size_t>(geo.ntiles) * (p.n_experts + 1) * sizeof(int32_t);
  return (bytes + 255) & ~static_cast<size_t>(255);
}

hipError_t launch_plan(const moe_problem &p, const int32_t *ids, const moe_plan &plan,
                       void *workspace, hipStream_t stream) {
  const PlanGeom geo = plan_geometry(p);
  PlanArgs g;
  g.ids = ids;
  g.npairs = geo.npairs;
  g.r_max = p.n_tokens * p.top_k + static_cast<int64_t>(p.n_experts) * (p.pad_multiple - 1);
  g.cap = p.recv_capacity;
  g.h = static_cast<uint32_t>(p.hidden);
  g.k = p.top_k;
  g.e = p.n_experts;
  g.ep = p.ep;
  g.a = p.pad_multiple;
  g.ntiles = geo.ntiles;
  g.key_bits = geo.key_bits;
  g.counts = plan.expert_counts;
  g.offsets = plan.expert_offsets;
  g.dest_counts = plan.dest_counts;
  g.table = plan.rank_table;
  g.slot = plan.slot;
  g.packed_src = plan.packed_src;
  g.status = plan.status;
  g.hist = static_cast<int32_t *>(workspace);
  g.tflags = geo.single ? nullptr
                        : reinterpret_cast<uint32_t *>(g.hist + static_cast<int64_t>(geo.ntiles) * p.n_experts);
  const size_t ids_lds = (kTilePairs + kMaxTopK) * sizeof(int);
  const size_t assign_lds = (8 * static_cast<size_t>(p.n_experts) + 2) * sizeof(int) + ids_lds;
  if (geo.single) {
    plan_assign_kernel<true><<<1, kPlanThreads, assign_lds, stream>>>(g);
  } else {
    const size_t count_lds = static_cast<size_t>(p.n_experts) * sizeof(int) + ids_lds;
    plan_count_kernel<<<geo.ntiles, kPlanThreads, count_lds, stream>>>(g);
    plan_assign_kernel<false><<<geo.ntiles, kPlanThreads, assign_lds, stream>>>(g);
  }
  return hipGetLastError();
}

}  // namespace moe
