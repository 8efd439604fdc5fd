// small_plan.hpp -- the routing plan of a small problem (at most 2048
// (token, k) pairs) computed inside one 256-thread workgroup, in LDS, so
// that a kernel can plan and dispatch in one launch.
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
// among the workgroup's own earlier pairs).  One LDS atomic per ID, no
// ballots, five barriers.
#pragma once

#include "moe_device.hpp"

namespace moe {

constexpr int kSmallPairs = 2048;    // pairs a small plan holds
constexpr int kSmallThreads = 256;   // one workgroup
constexpr int kSmallWaves = kSmallThreads / kWave;
constexpr int kSmallLoads = kSmallPairs / kSmallThreads;  // IDs per thread
constexpr int kSmallTargets = kSmallThreads;              // own pairs, one per thread
static_assert(kMaxExperts <= 4 * kSmallThreads, "the expert scan gives each thread four experts");
static_assert(kSmallTargets >= kSmallWaves * kMaxTopK, "own pairs: up to one token per wave");

struct SmallPlanArgs {
  const int32_t *ids;  // [n][k]
  int n, k, e, ep, a;
  int l;               // E / EP, experts per destination
  int64_t cap;         // recv_capacity (rows per destination)
};

// LDS arrays of a small plan (ints).
struct SmallPlanLds {
  int *ids;     // [kSmallPairs]   valid ID or -1
  int *tslot;   // [kSmallTargets] packed row of own pair p0 + j, or -1
  int *cnt;     // [E]   pairs per expert
  int *before;  // [E]   pairs per expert before p0
  int *off;     // [E+1] padded exclusive cumsum, off[E] = R_used
  int *cpre;    // [E+1] unpadded exclusive cumsum
};

__host__ __device__ constexpr size_t small_plan_lds_bytes(int e) {
  return (static_cast<size_t>(kSmallPairs) + kSmallTargets + 4 * static_cast<size_t>(e) + 2) *
         sizeof(int);
}

__device__ __forceinline__ SmallPlanLds small_plan_lds(int *smem, int e) {
  SmallPlanLds s;
  s.ids = smem;
  s.tslot = s.ids + kSmallPairs;
  s.cnt = s.tslot + kSmallTargets;
  s.before = s.cnt + e;
  s.off = s.before + e;
  s.cpre = s.off + e + 1;
  return s;
}

// Every ID of the problem, thread tid holding pairs u * 256 + tid (-1 past
// the end).  Separate from small_plan so that a caller can issue other loads
// before the IDs are first used.
__device__ __forceinline__ void small_plan_load(const SmallPlanArgs &g, int (&v)[kSmallLoads]) {
  const int np = g.n * g.k;
#pragma unroll
  for (int u = 0; u < kSmallLoads; ++u) {
    const int i = u * kSmallThreads + threadIdx.x;
    v[u] = i < np ? g.ids[i] : -1;
  }
}

// Fills cnt, off, cpre and ids for the whole problem and tslot[0 .. p1-p0)
// for the workgroup's own pairs [p0, p1) (p1 - p0 <= kSmallTargets, whole
// tokens).  Returns the status bits (BAD_ID, CAPACITY, and DUP_ID when
// check_dup), the same for every thread.  Ends with a barrier.
__device__ uint32_t small_plan(const SmallPlanArgs &g, const SmallPlanLds &s, const int (&v)[kSmallLoads],
                               int p0, int p1, bool check_dup) {
  __shared__ uint32_t s_fl;
  __shared__ int s_scan[2][kSmallWaves];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int E = g.e;
  const int np = g.n * g.k;

  for (int e = tid; e < E; e += kSmallThreads) {
    s.cnt[e] = 0;
    s.before[e] = 0;
  }
  if (tid == 0) s_fl = 0;
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
  if (check_dup) {
    for (int t = tid; t < g.n; t += kSmallThreads) {
      const int *row = s.ids + t * g.k;
      if (g.k <= 8) {
        int e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = j < g.k ? row[j] : -1;
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
  __syncthreads();

  // ---- totals; padded and unpadded exclusive scans (4 experts a thread) ---
  {
    const int e0 = 4 * tid;
    int c[4], p[4], sc = 0, sp = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c[q] = e0 + q < E ? s.cnt[e0 + q] + s.before[e0 + q] : 0;
      // no integer division when there is no padding (a long dependent chain)
      p[q] = g.a == 1 ? c[q] : ((c[q] + g.a - 1) / g.a) * g.a;
      sc += c[q];
      sp += p[q];
    }
    const int ip = wave_incl_scan(sp), ic = wave_incl_scan(sc);
    if (lane == kWave - 1) {
      s_scan[0][wave] = ip;
      s_scan[1][wave] = ic;
    }
    __syncthreads();
    int xp = ip - sp, xc = ic - sc, tp = 0, tc = 0;
#pragma unroll
    for (int w = 0; w < kSmallWaves; ++w) {
      xp += w < wave ? s_scan[0][w] : 0;
      xc += w < wave ? s_scan[1][w] : 0;
      tp += s_scan[0][w];
      tc += s_scan[1][w];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (e0 + q < E) {
        s.cnt[e0 + q] = c[q];  // each thread rewrites only the experts it read
        s.off[e0 + q] = xp;
        s.cpre[e0 + q] = xc;
      }
      xp += p[q];
      xc += c[q];
    }
    if (tid == 0) {
      s.off[E] = tp;
      s.cpre[E] = tc;
    }
  }
  __syncthreads();

  // ---- slots of the own pairs; capacity of every destination --------------
  {
    const int j = tid;
    if (j < p1 - p0) {
      const int pr = p0 + j;
      const int e = s.ids[pr];
      int sl = -1;
      if (e >= 0) {
        int r = s.before[e];
        // equal IDs among the own earlier pairs, 16 LDS reads in flight at a time
        for (int q0 = 0; q0 < j; q0 += 16) {
          int w[16];
#pragma unroll
          for (int q = 0; q < 16; ++q) w[q] = q0 + q < j ? s.ids[p0 + q0 + q] : -1;
#pragma unroll
          for (int q = 0; q < 16; ++q) r += w[q] == e ? 1 : 0;
        }
        sl = s.off[e] + r;
      }
      s.tslot[j] = sl;
    }
  }
  const int L = g.l;
  for (int r = tid; r < g.ep; r += kSmallThreads)
    if (s.cpre[(r + 1) * L] - s.cpre[r * L] > g.cap) fl |= MOE_STATUS_CAPACITY;
  const uint64_t b0 = ballot(fl & MOE_STATUS_BAD_ID), b1 = ballot(fl & MOE_STATUS_DUP_ID),
                 b2 = ballot(fl & MOE_STATUS_CAPACITY);
  const uint32_t wfl = (b0 ? MOE_STATUS_BAD_ID : 0u) | (b1 ? MOE_STATUS_DUP_ID : 0u) |
                       (b2 ? MOE_STATUS_CAPACITY : 0u);
  if (lane == 0 && wfl) atomicOr(&s_fl, wfl);
  __syncthreads();
  return s_fl;
}

}  // namespace moe
