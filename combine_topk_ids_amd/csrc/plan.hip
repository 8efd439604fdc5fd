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
// Design for gfx950.  Slots must follow flat pair order (t*k + j) inside
// each expert whatever order atomics land in, so every position comes from
// counts and scans, never from an atomic's return value.  Pairs are cut
// into count tiles of at most 2048 pairs (whole tokens) and each count tile
// into sub-tiles of 512 pairs, one 64-pair chunk per wave of a 512-thread
// block:
//   plan_count   (one block per count tile) histogram of the tile -> HBM
//                [ntiles][E], plus the tile's fault bits.
//   plan_assign  (one block per sub-tile) sums the histogram columns (each
//                expert's total and its count in earlier count tiles),
//                counts the pairs of its own count tile that precede the
//                sub-tile, scans the padded counts over experts, gives every
//                wave a base row per expert, and ranks each pair among the
//                equal IDs of its chunk with ballots (one ballot per ID bit);
//                block 0 also writes counts, offsets, table and status.
// Plans of at most 2048 pairs (decode shapes) skip plan_count: the whole
// problem is one count tile that every plan_assign block counts itself.
// plan_count alone (launch_plan_count) also serves the tiled mode of the
// plan-and-dispatch call, whose dispatch workgroups then finish the plan
// from its histograms (small_plan.hpp) instead of plan_assign.
//
// Latency matters more than bandwidth here (the whole plan moves < 2 MB):
// each kernel issues its global loads first, keeps every intermediate in LDS
// or registers, and issues its global stores last, so no barrier waits for
// stores to drain; no slot depends on another slot, so there is no serial
// chain.
#include "moe_device.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

constexpr int kThreads = kPlanThreads;                  // 8 waves
constexpr int kWaves = kPlanWaves;
constexpr int kTilePairs = kPlanTilePairs;             // count tile, whole tokens
constexpr int kSubPairs = kPlanSubPairs;                // sub-tile: one chunk per wave
static_assert(kSubPairs == kThreads, "an assign block takes one 64-pair chunk per wave");
constexpr int kPairsPerThread = kTilePairs / kThreads;  // staging loads per thread
constexpr int kHistBatch = 16;                          // column loads in flight
static_assert(kMaxExperts <= 2 * kThreads, "the expert scan gives each thread two experts");

struct PlanArgs {
  const int32_t *ids;
  int64_t n;          // tokens
  int64_t npairs;
  int64_t r_max;
  int64_t cap;
  uint32_t h;
  int k, e, ep, a;
  int ecap;           // fixed capacity per expert (0: dropless, padded to A)
  int tile_tokens;    // tokens per count tile
  int ntiles;         // count tiles
  int subs;           // sub-tiles per count tile
  int nblocks;        // plan_assign blocks = ntiles * subs
  int key_bits;
  int32_t *counts, *offsets, *dest_counts;
  uint32_t *table;
  int32_t *slot, *packed_src;
  uint32_t *status;
  int32_t *hist;      // workspace [ntiles][E]
  uint32_t *tflags;   // workspace [ntiles]
  // Batched plans (one per simulated rank, blockIdx.y = rank): distance
  // between consecutive ranks' arrays, in elements.  Unused with one rank.
  int64_t st_pairs;   // ids, slot
  int64_t st_rows;    // packed_src
  int64_t st_ws;      // hist and tflags
  int st_counts, st_offsets, st_dest, st_table;
};

// Point every per-rank array at this block's rank.
__device__ __forceinline__ void select_rank(PlanArgs &g) {
  const int r = blockIdx.y;
  if (r == 0) return;
  g.ids += r * g.st_pairs;
  g.slot += r * g.st_pairs;
  g.packed_src += r * g.st_rows;
  g.counts += static_cast<int64_t>(r) * g.st_counts;
  g.offsets += static_cast<int64_t>(r) * g.st_offsets;
  g.dest_counts += static_cast<int64_t>(r) * g.st_dest;
  g.table += static_cast<int64_t>(r) * g.st_table;
  g.status += r;
  if (g.hist) {
    g.hist += r * g.st_ws;
    g.tflags += r * g.st_ws;
  }
}

__device__ __forceinline__ int padded(int c, int a) { return ((c + a - 1) / a) * a; }

__device__ __forceinline__ uint32_t wave_or_bits(uint32_t v) {
  return (ballot(v & 1u) ? 1u : 0u) | (ballot(v & 2u) ? 2u : 0u) | (ballot(v & 4u) ? 4u : 0u) |
         (ballot(v & MOE_STATUS_DROPPED) ? MOE_STATUS_DROPPED : 0u) |
         (ballot(v & MOE_STATUS_BAD_PLAN) ? MOE_STATUS_BAD_PLAN : 0u);
}

struct Tile {
  int64_t tok0;   // first token
  int ntok;       // tokens in the tile
  int64_t pair0;  // first pair = tok0 * k
  int len;        // pairs = ntok * k
};

__device__ __forceinline__ Tile tile_of(const PlanArgs &g, int c, int k) {
  Tile t;
  t.tok0 = static_cast<int64_t>(c) * g.tile_tokens;
  t.ntok = static_cast<int>(min(static_cast<int64_t>(g.tile_tokens), g.n - t.tok0));
  if (t.ntok < 0) t.ntok = 0;
  t.pair0 = t.tok0 * k;
  t.len = t.ntok * k;
  return t;
}

// Coalesced load of the first `len` IDs of a tile into LDS (all loads issued
// first).  The caller places a barrier before s_ids is read.
__device__ __forceinline__ void stage_ids(const PlanArgs &g, int64_t pair0, int len, int *s_ids) {
  int v[kPairsPerThread];
#pragma unroll
  for (int u = 0; u < kPairsPerThread; ++u) {
    const int i = u * kThreads + threadIdx.x;
    v[u] = i < len ? g.ids[pair0 + i] : -1;
  }
#pragma unroll
  for (int u = 0; u < kPairsPerThread; ++u) {
    const int i = u * kThreads + threadIdx.x;
    if (i < len) s_ids[i] = v[u];
  }
}

// Histogram of a tile's valid pairs into s_cnt, one thread per token, and
// (if s_before) of those with tile-relative index < before into s_before;
// returns this thread's BAD_ID / DUP_ID bits.  With a compile-time k the
// token's IDs sit in registers for the repeated-ID check.
template <int KC>
__device__ uint32_t count_tokens(const PlanArgs &g, const Tile &t, const int *s_ids, int *s_cnt,
                                 int *s_before, int before) {
  uint32_t fl = 0;
  const int E = g.e;
  const int k = KC > 0 ? KC : g.k;
  for (int tl = threadIdx.x; tl < t.ntok; tl += kThreads) {
    if (KC > 0) {
      int e[KC > 0 ? KC : 1];
#pragma unroll
      for (int j = 0; j < KC; ++j) e[j] = s_ids[tl * KC + j];
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        if (e[j] == -1) continue;
        if (e[j] < -1 || e[j] >= E) {
          fl |= MOE_STATUS_BAD_ID;
          continue;
        }
#pragma unroll
        for (int jj = 0; jj < j; ++jj)
          if (e[jj] == e[j]) fl |= MOE_STATUS_DUP_ID;
        atomicAdd(&s_cnt[e[j]], 1);
        if (s_before && tl * KC + j < before) atomicAdd(&s_before[e[j]], 1);
      }
    } else {
      const int *row = s_ids + tl * k;
      for (int j = 0; j < k; ++j) {
        const int e = row[j];
        if (e == -1) continue;
        if (e < -1 || e >= E) {
          fl |= MOE_STATUS_BAD_ID;
          continue;
        }
        for (int jj = 0; jj < j; ++jj)
          if (row[jj] == e) fl |= MOE_STATUS_DUP_ID;
        atomicAdd(&s_cnt[e], 1);
        if (s_before && tl * k + j < before) atomicAdd(&s_before[e], 1);
      }
    }
  }
  return fl;
}

template <int KC>
__global__ __launch_bounds__(kThreads) void plan_count_kernel(PlanArgs g) {
  select_rank(g);
  extern __shared__ int smem[];
  int *s_cnt = smem;        // [E]
  int *s_ids = smem + g.e;  // [kTilePairs]
  __shared__ uint32_t s_fl;
  const int k = KC > 0 ? KC : g.k;
  const int c = blockIdx.x;
  const Tile t = tile_of(g, c, k);
  stage_ids(g, t.pair0, t.len, s_ids);
  for (int e = threadIdx.x; e < g.e; e += kThreads) s_cnt[e] = 0;
  if (threadIdx.x == 0) s_fl = 0;
  __syncthreads();
  const uint32_t fl = wave_or_bits(count_tokens<KC>(g, t, s_ids, s_cnt, nullptr, 0));
  if (lane_id() == 0 && fl) atomicOr(&s_fl, fl);
  __syncthreads();
  int32_t *hrow = g.hist + static_cast<int64_t>(c) * g.e;
  for (int e = threadIdx.x; e < g.e; e += kThreads) hrow[e] = s_cnt[e];
  if (threadIdx.x == 0) g.tflags[c] = s_fl;
  // the launch after this one ORs its bits into the status word
  if (c == 0 && threadIdx.x == 0 && g.status) *g.status = 0u;
}

// kFused: the whole problem is one count tile, counted here by every block.
template <int KC, bool kFused>
__global__ __launch_bounds__(kThreads) void plan_assign_kernel(PlanArgs g) {
  select_rank(g);
  extern __shared__ int smem[];
  const int E = g.e;
  int *s_tot = smem;                 // [E]   c_e
  int *s_pre = s_tot + E;            // [E]   pairs of e before this sub-tile
  int *s_off = s_pre + E;            // [E+1] padded exclusive cumsum
  int *s_cpre = s_off + E + 1;       // [E+1] unpadded exclusive cumsum
  int *s_cur = s_cpre + E + 1;       // [kWaves][E] per-wave counts, then bases
  int *s_ids = s_cur + kWaves * E;   // [kTilePairs]
  int *s_red = s_ids + kTilePairs;   // [2][kThreads] partial column sums
  __shared__ uint32_t s_fl;
  __shared__ int s_scan[2][kWaves];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int k = KC > 0 ? KC : g.k;
  const int b = blockIdx.x;
  const int c = b / g.subs;                       // count tile
  const int sub0 = (b - c * g.subs) * kSubPairs;  // sub-tile start inside it
  const Tile t = tile_of(g, c, k);
  const int sub_len = max(0, min(kSubPairs, t.len - sub0));

  // ---- global loads: histogram columns first, then the tile's IDs -------
  // Experts are taken in passes of up to kThreads; inside a pass, `tpe`
  // threads share an expert and each sums every tpe-th count tile.
  const int e_pass = min(E, kThreads);
  const int tpe = kThreads / e_pass;
  const int grp = tid / e_pass, e_loc = tid - grp * e_pass;
  int col_tot = 0, col_pre = 0;
  if (!kFused && grp < tpe) {
    for (int t0 = grp; t0 < g.ntiles; t0 += kHistBatch * tpe) {
      int v[kHistBatch];
#pragma unroll
      for (int u = 0; u < kHistBatch; ++u) {
        const int tt = t0 + u * tpe;
        v[u] = tt < g.ntiles ? g.hist[static_cast<int64_t>(tt) * E + e_loc] : 0;
      }
#pragma unroll
      for (int u = 0; u < kHistBatch; ++u) {
        col_tot += v[u];
        col_pre += (t0 + u * tpe < c) ? v[u] : 0;
      }
    }
  }
  uint32_t fl = 0;
  if (!kFused)
    for (int i = tid; i < g.ntiles; i += kThreads) fl |= g.tflags[i];
  // fused: the whole tile (for totals); otherwise up to the sub-tile's end
  stage_ids(g, t.pair0, kFused ? t.len : sub0 + sub_len, s_ids);
  for (int e = tid; e < E; e += kThreads) {
    s_tot[e] = 0;
    s_pre[e] = 0;
  }
  for (int i = tid; i < kWaves * E; i += kThreads) s_cur[i] = 0;
  if (tid == 0) s_fl = 0;
  if (!kFused) {
    s_red[tid] = grp < tpe ? col_tot : 0;
    s_red[kThreads + tid] = grp < tpe ? col_pre : 0;
  }
  __syncthreads();

  // ---- c_e totals and counts of the pairs before this sub-tile -----------
  if (kFused) {
    fl = count_tokens<KC>(g, t, s_ids, s_tot, s_pre, sub0);
  } else {
    // pairs of this count tile ahead of the sub-tile
#pragma unroll
    for (int u = 0; u < kPairsPerThread; ++u) {
      const int i = u * kThreads + tid;
      if (i < sub0) {
        const int e = s_ids[i];
        if (e >= 0 && e < E) atomicAdd(&s_pre[e], 1);
      }
    }
    for (int pass = 0; pass * e_pass < E; ++pass) {
      if (pass > 0) {  // E > kThreads: sum the columns of the next experts
        __syncthreads();
        const int e = pass * e_pass + e_loc;
        int ct = 0, cp = 0;
        if (grp < tpe && e < E)
          for (int tt = grp; tt < g.ntiles; tt += tpe) {
            const int v = g.hist[static_cast<int64_t>(tt) * E + e];
            ct += v;
            cp += tt < c ? v : 0;
          }
        s_red[tid] = ct;
        s_red[kThreads + tid] = cp;
        __syncthreads();
      }
      if (tid < e_pass && pass * e_pass + tid < E) {
        int ct = 0, cp = 0;
        for (int q = 0; q < tpe; ++q) {
          ct += s_red[q * e_pass + tid];
          cp += s_red[kThreads + q * e_pass + tid];
        }
        s_tot[pass * e_pass + tid] = ct;
        atomicAdd(&s_pre[pass * e_pass + tid], cp);
      }
    }
  }
  // this wave's chunk: IDs into registers, per-wave counts into LDS
  const int i_loc = sub0 + wave * kWave + lane;  // tile-relative pair index
  const bool in = wave * kWave + lane < sub_len;
  const int ev = in ? s_ids[i_loc] : -1;
  const bool valid = ev >= 0 && ev < E;
  int *cur = s_cur + wave * E;
  if (valid) atomicAdd(&cur[ev], 1);
  fl = wave_or_bits(fl);
  if (lane == 0 && fl) atomicOr(&s_fl, fl);
  __syncthreads();

  // ---- padded and unpadded exclusive scans over experts -----------------
  // thread tid owns experts 2*tid and 2*tid+1 (E <= 1024 = 2 * kThreads)
  {
    const int e0 = 2 * tid;
    // segment sizes: c padded to A, or the fixed capacity; with a fixed
    // capacity the unpadded sums count kept pairs, min(c, cap)
    int c0 = e0 < E ? s_tot[e0] : 0;
    int c1 = e0 + 1 < E ? s_tot[e0 + 1] : 0;
    int p0 = padded(c0, g.a), p1 = padded(c1, g.a);
    if (g.ecap > 0) {
      c0 = min(c0, g.ecap);
      c1 = min(c1, g.ecap);
      p0 = e0 < E ? g.ecap : 0;
      p1 = e0 + 1 < E ? g.ecap : 0;
    }
    const int ip = wave_incl_scan(p0 + p1), ic = wave_incl_scan(c0 + c1);
    if (lane == kWave - 1) {
      s_scan[0][wave] = ip;
      s_scan[1][wave] = ic;
    }
    __syncthreads();
    int xp = ip - (p0 + p1), xc = ic - (c0 + c1);
    int tp = 0, tc = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int sp = s_scan[0][w], sc = s_scan[1][w];
      xp += w < wave ? sp : 0;
      xc += w < wave ? sc : 0;
      tp += sp;
      tc += sc;
    }
    if (e0 < E) {
      s_off[e0] = xp;
      s_cpre[e0] = xc;
    }
    if (e0 + 1 < E) {
      s_off[e0 + 1] = xp + p0;
      s_cpre[e0 + 1] = xc + c0;
    }
    if (tid == 0) {
      s_off[E] = tp;
      s_cpre[E] = tc;
    }
  }
  __syncthreads();

  // ---- per-wave base rows: offset + earlier pairs + earlier waves --------
  // one thread per expert column: read the wave counts, write the bases
  for (int e = tid; e < E; e += kThreads) {
    int cw[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) cw[w] = s_cur[w * E + e];
    int run = s_off[e] + s_pre[e];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      s_cur[w * E + e] = run;
      run += cw[w];
    }
  }
  const int L = E / g.ep;
  uint32_t cap = 0;
  for (int r = tid; r < g.ep; r += kThreads)
    if (s_cpre[(r + 1) * L] - s_cpre[r * L] > g.cap) cap = MOE_STATUS_CAPACITY;
  if (g.ecap > 0)
    for (int e = tid; e < E; e += kThreads)
      if (s_tot[e] > g.ecap) cap |= MOE_STATUS_DROPPED;
  cap = wave_or_bits(cap);
  if (lane == 0 && cap) atomicOr(&s_fl, cap);
  // rank among the equal IDs of this chunk: one ballot per ID bit, a lane
  // keeping the lanes whose bit matches its own
  uint64_t m = ballot(valid);
  for (int bt = 0; bt < g.key_bits; ++bt) {
    const bool set = (ev >> bt) & 1;
    const uint64_t ones = ballot(set);
    m &= set ? ones : ~ones;
  }
  const int rank = lanes_below(m);
  __syncthreads();

  // ---- stores only from here on -------------------------------------------
  // A pair's rank in its expert must lie below the expert's total, and its
  // row inside the buffer; with histograms that do not count these IDs (a
  // workspace changed between the two launches) it may not, and then the
  // pair is left unplaced (slot -1) and BAD_PLAN is set.
  uint32_t bad = 0;
  if (in) {
    int sl = -1;
    if (valid) {
      sl = cur[ev] + rank;
      const int r = sl - s_off[ev];
      if (!kFused && (r < 0 || r >= s_tot[ev])) {
        bad = MOE_STATUS_BAD_PLAN;
        sl = -1;
      } else if (g.ecap > 0 && r >= g.ecap) {
        sl = -1;  // a fixed capacity keeps the first cap pairs of each expert
      } else if (!kFused && (sl < 0 || sl >= g.r_max)) {
        bad = MOE_STATUS_BAD_PLAN;
        sl = -1;
      }
      if (sl >= 0) g.packed_src[sl] = static_cast<int32_t>(t.tok0 + i_loc / k);
    }
    g.slot[t.pair0 + i_loc] = sl;
  }
  if (!kFused) {
    if (b == 0 && tid == 0 && (s_off[E] < 0 || s_off[E] > g.r_max)) bad = MOE_STATUS_BAD_PLAN;
    if (ballot(bad != 0) && lane == 0) atomicOr(g.status, MOE_STATUS_BAD_PLAN);
  }

  // block 0: counts, offsets, per-rank table, status
  if (b == 0) {
    for (int e = tid; e < E; e += kThreads) {
      g.counts[e] = s_tot[e];
      g.offsets[e] = s_off[e];
    }
    if (tid == 0) {
      g.offsets[E] = s_off[E];
      // after the counting kernel, which cleared it, other blocks may OR
      // BAD_PLAN into the status word; a single-tile plan writes it alone
      if (kFused)
        *g.status = s_fl;
      else
        atomicOr(g.status, s_fl);
    }
    for (int r = tid; r < g.ep; r += kThreads) {
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

  // packed_src = -1 on the unused rows of each expert (at most A-1 pad rows,
  // or up to cap with a fixed capacity: the grid strides over E * that many
  // candidates) and on the tail rows
  const int per = g.ecap > 0 ? g.ecap : g.a - 1;
  if (per > 0) {
    const int cand = E * per;  // <= R_max < 2^31
    for (int q = b * kThreads + tid; q < cand; q += g.nblocks * kThreads) {
      const int e = q / per;
      const int used = g.ecap > 0 ? min(s_tot[e], g.ecap) : s_tot[e];
      const int64_t r = static_cast<int64_t>(s_off[e]) + used + (q - e * per);
      if (r < s_off[e + 1] && r >= 0 && r < g.r_max) g.packed_src[r] = -1;
    }
  }
  for (int64_t r = max(s_off[E], 0) + static_cast<int64_t>(b) * kThreads + tid; r < g.r_max;
       r += static_cast<int64_t>(g.nblocks) * kThreads)
    g.packed_src[r] = -1;
}

template <int KC>
void launch_k(const PlanArgs &g, bool fused, int e, int ranks, hipStream_t stream, bool count_only) {
  const size_t assign_lds =
      (static_cast<size_t>(4 + kWaves) * e + 2 + kTilePairs + 2 * kThreads) * sizeof(int);
  if (count_only) {
    const size_t count_lds = (static_cast<size_t>(e) + kTilePairs) * sizeof(int);
    plan_count_kernel<KC><<<dim3(g.ntiles, ranks), kThreads, count_lds, stream>>>(g);
  } else if (fused) {
    plan_assign_kernel<KC, true><<<dim3(g.nblocks, ranks), kThreads, assign_lds, stream>>>(g);
  } else {
    const size_t count_lds = (static_cast<size_t>(e) + kTilePairs) * sizeof(int);
    plan_count_kernel<KC><<<dim3(g.ntiles, ranks), kThreads, count_lds, stream>>>(g);
    plan_assign_kernel<KC, false><<<dim3(g.nblocks, ranks), kThreads, assign_lds, stream>>>(g);
  }
}

}  // namespace

namespace {

hipError_t launch_plan_impl(const moe_problem &p, int ranks, const int32_t *ids, const moe_plan &plan,
                            const PlanStrides &st, void *workspace, hipStream_t stream, bool count_only) {
  const PlanGeom geo = plan_geometry(p);
  PlanArgs g;
  g.ids = ids;
  g.n = p.n_tokens;
  g.npairs = geo.npairs;
  g.r_max = max_rows(p);
  g.cap = p.recv_capacity;
  g.ecap = static_cast<int>(p.expert_capacity);
  g.h = static_cast<uint32_t>(p.hidden);
  g.k = p.top_k;
  g.e = p.n_experts;
  g.ep = p.ep;
  g.a = p.pad_multiple;
  g.tile_tokens = geo.tile_tokens;
  g.ntiles = geo.ntiles;
  g.subs = geo.subs;
  g.nblocks = geo.ntiles * geo.subs;
  g.key_bits = geo.key_bits;
  g.counts = plan.expert_counts;
  g.offsets = plan.expert_offsets;
  g.dest_counts = plan.dest_counts;
  g.table = plan.rank_table;
  g.slot = plan.slot;
  g.packed_src = plan.packed_src;
  g.status = plan.status;
  g.hist = geo.single ? nullptr : static_cast<int32_t *>(workspace);
  g.tflags = geo.single ? nullptr
                        : reinterpret_cast<uint32_t *>(g.hist + static_cast<int64_t>(geo.ntiles) * p.n_experts);
  g.st_pairs = st.pairs;
  g.st_rows = st.rows;
  g.st_ws = st.workspace;
  g.st_counts = st.counts;
  g.st_offsets = st.offsets;
  g.st_dest = st.dest;
  g.st_table = st.table;
  switch (p.top_k) {
    case 1: launch_k<1>(g, geo.single, p.n_experts, ranks, stream, count_only); break;
    case 2: launch_k<2>(g, geo.single, p.n_experts, ranks, stream, count_only); break;
    case 4: launch_k<4>(g, geo.single, p.n_experts, ranks, stream, count_only); break;
    case 6: launch_k<6>(g, geo.single, p.n_experts, ranks, stream, count_only); break;
    case 8: launch_k<8>(g, geo.single, p.n_experts, ranks, stream, count_only); break;
    default: launch_k<0>(g, geo.single, p.n_experts, ranks, stream, count_only); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_plan_ranks(const moe_problem &p, int ranks, const int32_t *ids,
                             const moe_plan &plan, const PlanStrides &st, void *workspace,
                             hipStream_t stream) {
  return launch_plan_impl(p, ranks, ids, plan, st, workspace, stream, false);
}

hipError_t launch_plan_count(const moe_problem &p, const int32_t *ids, uint32_t *status,
                             void *workspace, hipStream_t stream) {
  // the workspace and the status word (cleared) are written; the other plan
  // arrays stay unset
  moe_plan plan{};
  plan.status = status;
  return launch_plan_impl(p, 1, ids, plan, PlanStrides{}, workspace, stream, true);
}

hipError_t launch_plan(const moe_problem &p, const int32_t *ids, const moe_plan &plan,
                       void *workspace, hipStream_t stream) {
  return launch_plan_ranks(p, 1, ids, plan, PlanStrides{}, workspace, stream);
}

}  // namespace moe
