// small_plan.hpp -- the part of the routing plan one 256-thread workgroup
// needs, computed in LDS, so that a kernel can plan and dispatch in one
// launch: from all the IDs of a small problem (at most 2048 (token, k)
// pairs), or in tiled mode from the tile histograms of plan.hip's counting
// kernel.
//
// What is computed is the plan of plan.hip, for problems without a fixed
// expert capacity (pages cited by title and section):
//   NKI permute_a2av API reference -- description (rows packed per
//     destination at cumsum offsets, the (4, EP) table of counts and
//     displacements in elements) and :param recv_capacity: (the bound each
//     destination's rows are checked against).
//   NeMo Automodel token_dispatcher API --
//     TokenDispatcherConfig.moe_router_expert_pad_multiple (each expert
//     padded to a multiple of A rows), _indices_to_multihot (-1 masks a
//     slot).
// Slots follow flat pair order t*k + j inside each expert.
//
// Design for gfx950.  Every workgroup of the launch reads all the IDs (at
// most 8 KB, served from L2 after the first workgroup) and needs no other
// workgroup's result.  It computes what it uses: each expert's count, the
// count of each expert among the pairs before its own tokens, the padded
// and unpadded offsets, and the slots of its own tokens' pairs only (at most
// 4 tokens, so at most 256 pairs: a pair's slot is its expert's offset, plus
// the earlier pairs of that expert before the workgroup's tokens, plus those
// among the workgroup's own earlier pairs).  Each wave finds the slots of
// its own token's pairs itself (own_slot), so they need no barrier; only the
// workgroup that reports the status gathers fault bits.  One LDS atomic per
// ID, no ballots, three barriers: one more in the workgroup that reports
// the status, and one more where E > 256.
//
// Tiled mode (larger problems, two launches).  The counting kernel of
// plan.hip first writes one histogram per count tile of T pairs (whole
// tokens) and the tile's fault bits.  A workgroup then needs no more than
// the histograms (each expert's total, and its count in the tiles before
// the workgroup's own tile) and the IDs of its own tile up to the end of its
// own pairs: at most T - 1 earlier pairs plus its own pairs.  The steps
// after the counting are the same in both modes.
#pragma once

#include "host_checks.hpp"
#include "moe_device.hpp"

namespace moe {

// kSmallPairs: pairs a small plan holds; kTileHist: histogram entries
// (tiles * E) a tiled plan reads (host_checks.hpp, which picks the mode)
constexpr int kSmallThreads = 256;   // one workgroup
constexpr int kSmallWaves = kSmallThreads / kWave;
constexpr int kSmallLoads = kSmallPairs / kSmallThreads;  // IDs per thread
constexpr int kSmallTargets = kSmallThreads;              // own pairs, one per thread
constexpr int kSmallIds = kSmallPairs + kSmallTargets;    // LDS IDs: tiled mode reads up to this many
constexpr int kRankBatch = 16;  // own IDs own_slot reads per batch, unconditionally
constexpr int kTileLoads = kSmallIds / kSmallThreads;     // IDs per thread in tiled mode
constexpr int kTileHistLoads = kTileHist / kSmallThreads;
static_assert(kMaxExperts <= 4 * kSmallThreads, "the expert scan gives each thread four experts");
static_assert(kSmallTargets >= kSmallWaves * kMaxTopK, "own pairs: up to one token per wave");

struct SmallPlanArgs {
  const int32_t *ids;  // [n][k]
  int n, k, e, ep, a;
  int ecap;            // fixed rows per expert (0: dropless, padded to A)
  int l;               // E / EP, experts per destination
  int64_t cap;         // recv_capacity (rows per destination)
  // tiled mode only
  const int32_t *hist;      // [ntiles][E] pairs per expert in each count tile
  const uint32_t *tflags;   // [ntiles]    BAD_ID / DUP_ID bits of each tile
  int ntiles, tile_tokens;  // ntiles * E <= kTileHist
};

// LDS arrays of a small plan (ints).
struct SmallPlanLds {
  int *ids;     // [kSmallIds] valid ID or -1, pairs lo .. (lo = 0 in small mode),
                // then kRankBatch entries that own_slot may read and ignore
  int *cnt;     // [E]   pairs per expert (while counting, small mode: those from p0 on)
  int *before;  // [E]   pairs per expert before p0
  int *off;     // [E+1] padded exclusive cumsum, off[E] = R_used
  int *cpre;    // [E+1] unpadded exclusive cumsum
};

__host__ __device__ constexpr size_t small_plan_lds_bytes(int e) {
  return (static_cast<size_t>(kSmallIds + kRankBatch) + 4 * static_cast<size_t>(e) + 2) * sizeof(int);
}

__device__ __forceinline__ SmallPlanLds small_plan_lds(int *smem, int e) {
  SmallPlanLds s;
  s.ids = smem;
  s.cnt = s.ids + kSmallIds + kRankBatch;
  s.before = s.cnt + e;
  s.off = s.before + e;
  s.cpre = s.off + e + 1;
  return s;
}

// Every ID of the problem, thread tid holding pairs u * 256 + tid (-1 past
// the end).  Separate from small_plan so that a caller can issue other loads
// before the IDs are first used.  Bounds-checked buffer loads, so no branch
// surrounds them.
__device__ __forceinline__ void small_plan_load(const SmallPlanArgs &g, int (&v)[kSmallLoads]) {
  const int np = g.n * g.k;
  const auto ids = buffer_rsrc(g.ids, static_cast<uint32_t>(np) * 4u);
#pragma unroll
  for (int u = 0; u < kSmallLoads; ++u) {
    const int i = u * kSmallThreads + threadIdx.x;
    const int x = __builtin_amdgcn_raw_buffer_load_b32(ids, i * 4, 0, kLoadDefault);
    v[u] = i < np ? x : -1;
  }
}

// Tiled mode: the IDs of pairs lo .. lo+len-1 (len <= kSmallIds), every
// tile histogram and every tile's fault bits.
struct TileLoads {
  int v[kTileLoads];
  int h[kTileHistLoads];
  uint32_t fl;
};

// Bounds-checked buffer loads (zero past each array's end), so no branch
// surrounds them.
__device__ __forceinline__ void tile_plan_load(const SmallPlanArgs &g, int lo, int len, TileLoads &l) {
  const int tid = threadIdx.x;
  const auto ids = buffer_rsrc(g.ids + lo, static_cast<uint32_t>(len) * 4u);
#pragma unroll
  for (int u = 0; u < kTileLoads; ++u) {
    const int i = u * kSmallThreads + tid;
    const int x = __builtin_amdgcn_raw_buffer_load_b32(ids, i * 4, 0, kLoadDefault);
    l.v[u] = i < len ? x : -1;
  }
  const auto hist = buffer_rsrc(g.hist, static_cast<uint32_t>(g.ntiles * g.e) * 4u);
#pragma unroll
  for (int u = 0; u < kTileHistLoads; ++u)
    l.h[u] = __builtin_amdgcn_raw_buffer_load_b32(hist, (u * kSmallThreads + tid) * 4, 0, kLoadDefault);
  const auto tfl = buffer_rsrc(g.tflags, static_cast<uint32_t>(g.ntiles) * 4u);
  uint32_t fl = 0;
#pragma unroll
  for (int u = 0; u < kTileHistLoads; ++u)  // ntiles <= kTileHist
    fl |= __builtin_amdgcn_raw_buffer_load_b32(tfl, (u * kSmallThreads + tid) * 4, 0, kLoadDefault);
  l.fl = fl;
}

namespace detail {

// Common end of both modes, after before[e] holds the pairs of expert e
// ahead of p0 and cnt[e] its total (TOTAL) or its pairs from p0 on: padded
// and unpadded scans, and, where `status`, capacity and the status bits (0
// otherwise).  `fl` holds this thread's fault bits so far.  Starts and ends
// with a barrier.
template <bool TOTAL>
__device__ uint32_t plan_finish(const SmallPlanArgs &g, const SmallPlanLds &s, uint32_t fl, bool status) {
  __shared__ int s_scan[2][kSmallWaves];
  __shared__ uint32_t s_fl;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int E = g.e;
  if (tid == 0) s_fl = 0;
  __syncthreads();

  // ---- totals; padded and unpadded exclusive scans (4 experts a thread) ---
  {
    const int e0 = 4 * tid;
    // segment sizes: c padded to A, or the fixed capacity; with a fixed
    // capacity the unpadded sums count the kept pairs, min(c, cap)
    int c[4], kc[4], p[4], sc = 0, sp = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c[q] = e0 + q < E ? s.cnt[e0 + q] + (TOTAL ? 0 : s.before[e0 + q]) : 0;
      if (g.ecap > 0) {
        kc[q] = min(c[q], g.ecap);
        p[q] = e0 + q < E ? g.ecap : 0;
        if (c[q] > g.ecap) fl |= MOE_STATUS_DROPPED;
      } else {
        kc[q] = c[q];
        // no integer division when there is no padding (a long dependent chain)
        p[q] = g.a == 1 ? c[q] : ((c[q] + g.a - 1) / g.a) * g.a;
      }
      sc += kc[q];
      sp += p[q];
    }
    const int ip = wave_incl_scan(sp), ic = wave_incl_scan(sc);
    int xp = ip - sp, xc = ic - sc, tp, tc;
    if (E <= 4 * kWave) {
      // wave 0 holds every expert: its totals are the problem's, and no
      // other wave's scan is needed (E is the same for the whole workgroup)
      tp = __builtin_amdgcn_readlane(ip, kWave - 1);
      tc = __builtin_amdgcn_readlane(ic, kWave - 1);
    } else {
      if (lane == kWave - 1) {
        s_scan[0][wave] = ip;
        s_scan[1][wave] = ic;
      }
      __syncthreads();
      tp = tc = 0;
#pragma unroll
      for (int w = 0; w < kSmallWaves; ++w) {
        xp += w < wave ? s_scan[0][w] : 0;
        xc += w < wave ? s_scan[1][w] : 0;
        tp += s_scan[0][w];
        tc += s_scan[1][w];
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (e0 + q < E) {
        s.cnt[e0 + q] = c[q];  // each thread rewrites only the experts it read
        s.off[e0 + q] = xp;
        s.cpre[e0 + q] = xc;
      }
      xp += p[q];
      xc += kc[q];
    }
    if (tid == 0) {
      s.off[E] = tp;
      s.cpre[E] = tc;
    }
  }
  __syncthreads();

  // ---- capacity of every destination; status --------------------------
  if (!status) return 0;  // uniform: the whole workgroup skips the gather
  const int L = g.l;
  for (int r = tid; r < g.ep; r += kSmallThreads)
    if (s.cpre[(r + 1) * L] - s.cpre[r * L] > g.cap) fl |= MOE_STATUS_CAPACITY;
  const uint64_t b0 = ballot(fl & MOE_STATUS_BAD_ID), b1 = ballot(fl & MOE_STATUS_DUP_ID),
                 b2 = ballot(fl & MOE_STATUS_CAPACITY), b3 = ballot(fl & MOE_STATUS_DROPPED);
  const uint32_t wfl = (b0 ? MOE_STATUS_BAD_ID : 0u) | (b1 ? MOE_STATUS_DUP_ID : 0u) |
                       (b2 ? MOE_STATUS_CAPACITY : 0u) | (b3 ? MOE_STATUS_DROPPED : 0u);
  if (lane == 0 && wfl) atomicOr(&s_fl, wfl);
  __syncthreads();
  return s_fl;
}

}  // namespace detail

// Packed row of own pair p (p0 <= p < p1) after small_plan or tile_plan, or
// -1 for a masked or invalid pair: its expert's offset, plus that expert's
// pairs before p0, plus its equal IDs among the own pairs ahead of p.  Reads
// only LDS that the plan's last barrier published, so a wave calls it for
// its own token's pairs with no further barrier.
//
// The pair's rank r in its expert must lie below the expert's count and its
// row inside the buffer [0, r_max).  From a plan of the IDs themselves it
// always does; in tiled mode the counts come from histograms in memory,
// and if those do not count these IDs the pair gets kBadSlot instead.
// With a fixed capacity `ecap`, a pair ranked at or past it is dropped (-1).
constexpr int kBadSlot = -2;

__device__ __forceinline__ int own_slot(const SmallPlanLds &s, int lo, int p0, int p, int r_max, int ecap) {
  const int e = s.ids[p - lo];
  if (e < 0) return -1;
  const int *own = s.ids + (p0 - lo);
  const int j = p - p0;
  int r = s.before[e];
  // kRankBatch LDS reads in flight at a time: every read of a batch is
  // issued, then one wait.  A read under its own condition would be compiled
  // into a read and a wait each.  The last batch may read up to
  // kRankBatch - 1 entries past p - lo (inside the ids array and its slack);
  // those are not counted.
  for (int q0 = 0; q0 < j; q0 += kRankBatch) {
    int w[kRankBatch];
#pragma unroll
    for (int q = 0; q < kRankBatch; ++q) w[q] = own[q0 + q];
#pragma unroll
    for (int q = 0; q < kRankBatch; ++q) r += q0 + q < j && w[q] == e ? 1 : 0;
  }
  if (r < 0 || r >= s.cnt[e]) return kBadSlot;
  if (ecap > 0 && r >= ecap) return -1;
  const int64_t row = static_cast<int64_t>(s.off[e]) + r;
  return row < 0 || row >= r_max ? kBadSlot : static_cast<int>(row);
}

// Fills cnt, off, cpre and ids for the whole problem and before (each
// expert's pairs ahead of p0, the workgroup's first pair); own_slot then
// gives the slots of the own pairs (whole tokens from p0, at most
// kSmallTargets pairs).  Where `status` (uniform in the workgroup), returns
// the status bits (BAD_ID, DUP_ID, CAPACITY), the same for every thread; 0
// otherwise.  Ends with a barrier.
__device__ uint32_t small_plan(const SmallPlanArgs &g, const SmallPlanLds &s, const int (&v)[kSmallLoads],
                               int p0, bool status) {
  const int tid = threadIdx.x;
  const int E = g.e;
  const int np = g.n * g.k;

  for (int e = tid; e < E; e += kSmallThreads) {
    s.cnt[e] = 0;
    s.before[e] = 0;
  }
  uint32_t fl = 0;
  int e_own[kSmallLoads];
#pragma unroll
  for (int u = 0; u < kSmallLoads; ++u) {
    const int i = u * kSmallThreads + tid;
    int e = v[u];
    if (e < -1 || e >= E) {
      fl |= MOE_STATUS_BAD_ID;
      e = -1;  // treated as masked
    }
    e_own[u] = e;
    if (i < np) s.ids[i] = e;
  }
  __syncthreads();

  // ---- counts, and counts before the own pairs: one atomic per ID ---------
#pragma unroll
  for (int u = 0; u < kSmallLoads; ++u) {
    const int i = u * kSmallThreads + tid;
    const int e = e_own[u];
    if (e >= 0) atomicAdd(i < p0 ? &s.before[e] : &s.cnt[e], 1);
  }
  // repeated IDs within a token (only where the status is written); up to
  // 8 IDs a token are read together into registers
  if (status) {
    for (int t = tid; t < g.n; t += kSmallThreads) {
      const int *row = s.ids + t * g.k;
      if (g.k <= 8) {
        // all 8 read unconditionally (t * k + 7 < kSmallPairs + 7, inside
        // the ids array), then masked
        int e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = row[j];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = j < g.k ? e[j] : -1;
#pragma unroll
        for (int j = 1; j < 8; ++j)
#pragma unroll
          for (int jj = 0; jj < j; ++jj)
            if (e[j] >= 0 && e[jj] == e[j]) fl |= MOE_STATUS_DUP_ID;
      } else {
        for (int j = 1; j < g.k; ++j) {
          const int e = row[j];
          if (e < 0) continue;
          for (int jj = 0; jj < j; ++jj)
            if (row[jj] == e) fl |= MOE_STATUS_DUP_ID;
        }
      }
    }
  }
  return detail::plan_finish<false>(g, s, fl, status);
}

__device__ __forceinline__ int tile_id(const SmallPlanArgs &g, int v) {
  return v < -1 || v >= g.e ? -1 : v;  // counted as masked (the tile's bits say BAD_ID)
}

// Tiled mode, first step: clears the counters and stores the IDs loaded by
// tile_plan_load(g, lo, len, l) into ids.  Ends with a barrier, so the IDs
// have arrived when it returns.
__device__ void tile_plan_stage(const SmallPlanArgs &g, const SmallPlanLds &s, const TileLoads &l, int len) {
  const int tid = threadIdx.x;
  for (int e = tid; e < g.e; e += kSmallThreads) {
    s.cnt[e] = 0;
    s.before[e] = 0;
  }
#pragma unroll
  for (int u = 0; u < kTileLoads; ++u) {
    const int i = u * kSmallThreads + tid;
    if (i < len) s.ids[i] = tile_id(g, l.v[u]);
  }
  __syncthreads();
}

// Tiled mode, after tile_plan_stage: lo is the first pair of count tile c0,
// the tile that holds pair p0 (p0 - lo < T, so the own pairs end at most
// kSmallIds pairs after lo).  Fills the same arrays as small_plan, with ids
// holding pairs lo .. p1-1.  Where `status`, the status bits are those of
// every tile (BAD_ID, DUP_ID) and CAPACITY; 0 otherwise.  Ends with a
// barrier.
__device__ uint32_t tile_plan(const SmallPlanArgs &g, const SmallPlanLds &s, const TileLoads &l, int lo,
                              int p0, int c0, bool status) {
  const int tid = threadIdx.x;
  const int E = g.e;

  // ---- totals from the histograms, and the count before tile c0; then the
  // pairs of tile c0 ahead of p0 ------------------------------------------
  // entry i = u * 256 + tid of [ntiles][E] is (tile i / E, expert i % E)
  const int dq = kSmallThreads / E, dr = kSmallThreads - dq * E;
  int tt = tid / E, e = tid - tt * E;
#pragma unroll
  for (int u = 0; u < kTileHistLoads; ++u) {
    const int c = l.h[u];  // 0 past the last entry
    if (c != 0) {
      atomicAdd(&s.cnt[e], c);
      if (tt < c0) atomicAdd(&s.before[e], c);
    }
    e += dr;
    tt += dq;
    if (e >= E) {
      e -= E;
      ++tt;
    }
  }
  const int ahead = p0 - lo;
#pragma unroll
  for (int u = 0; u < kTileLoads; ++u) {
    const int i = u * kSmallThreads + tid;
    const int ev = tile_id(g, l.v[u]);
    if (i < ahead && ev >= 0) atomicAdd(&s.before[ev], 1);
  }
  return detail::plan_finish<true>(g, s, l.fl, status);
}

}  // namespace moe
