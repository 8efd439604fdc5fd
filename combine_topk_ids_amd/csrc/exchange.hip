// exchange.hip -- the receive side of the expert-parallel exchange,
// simulated on one GPU that holds the shares of all EP ranks.
//
// What is computed (pages cited by title and section):
//   NKI permute_a2av API reference -- description: the receive layout is the
//     packed cumsum of the receive counts; the (4, EP) table's rows 2-3 hold
//     receive counts and displacements in elements; :return: a [C, H]
//     receive buffer holds each source's rows in rank order, then zero
//     rows.
//   DeepSpeed v0.19.4 function index, page 15 -- SplitPlan entries: one
//     all-to-all exchanges the [ep_size, E_local] count matrix; a rank
//     receives the matrix rows that cover its experts.
//   Mojo ep.dispatch_async.block.scaled.nv struct -- recv_count_ptrs (rows
//     received per expert).
//
// Steps, for EP ranks of N tokens each (rank s owns tokens s*N .. s*N+N-1):
//   1. every rank's own plan (the single-rank plan kernels, one launch with
//      blockIdx.y = rank, A = 1, no send-side capacity): counts per expert,
//      send counts per destination, send displacements (table rows 0-1),
//      and the pair's row in the rank's own packed order;
//   2. exchange_remap, one launch of two block ranges:
//      - blocks of pairs per source s (blockIdx.y = s): receive row = d*C +
//        (rows of d's buffer from sources before s) + (send row - start of
//        s's segment for d), kept if below C; the inverse map recv_src;
//      - blocks per destination d (blockIdx.y = d): the receive counts from
//        every source and their packed cumsum (table rows 2-3), the rows
//        offered to d, CAPACITY, what the counts all-to-all delivers to d
//        (its slice of every source's count matrix), and -1 over recv_src
//        past the rows in use.
// A pair's position inside its source's segment is the single-rank plan's,
// so the order inside a receive buffer is (source, expert, token, k) without
// any sort across ranks, and no output depends on atomic order.
#include "moe_device.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kPairsPerThread = 8;
constexpr int kPairsPerBlock = kThreads * kPairsPerThread;
constexpr int kTailRowsPerBlock = 4096;
constexpr int kMaxTailBlocks = 256;

struct ExchangeArgs {
  const int32_t *ids;           // [R][N*k]
  int32_t *slot;                // [R][N*k] send row in, receive row out
  const int32_t *counts;        // [R][E]
  const int32_t *send_counts;   // [R][R]
  const int32_t *offsets;       // [R][E+1] each rank's expert offsets (A = 1)
  int32_t *recv_expert_counts;  // [R][R][L]
  int32_t *recv_rows;           // [R]
  uint32_t *table;              // [R][4][R]
  int32_t *recv_src;            // [R][C]
  uint32_t *status;             // [R]
  int64_t n;                    // tokens per rank
  int64_t npairs;               // pairs per rank
  int64_t cap;                  // C
  uint32_t h;
  int k, e, r, l;
  int pair_blocks, dest_blocks;
};

// Exclusive prefix sum of v[0..n) in LDS (n <= 4 * kThreads), in place;
// returns the total.  Each thread scans 4 consecutive entries, then a DPP
// wave scan and one partial per wave carry the sums across.
__device__ int block_excl_scan4(int *v, int n, int *s_wave) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  int x[4], sum = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = 4 * tid + u;
    x[u] = i < n ? v[i] : 0;
    sum += x[u];
  }
  const int incl = wave_incl_scan(sum);
  if (lane == kWave - 1) s_wave[wave] = incl;
  __syncthreads();
  int run = incl - sum, total = 0;
#pragma unroll
  for (int w = 0; w < kThreads / kWave; ++w) {
    run += w < wave ? s_wave[w] : 0;
    total += s_wave[w];
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = 4 * tid + u;
    if (i < n) v[i] = run;
    run += x[u];
  }
  __syncthreads();
  return total;
}

// grid (pair_blocks + dest_blocks, R).  Blocks x < pair_blocks map the pairs
// of source rank s = blockIdx.y to receive rows; the others serve
// destination rank d = blockIdx.y: its metadata (first such block) and the
// -1 entries of recv_src past the rows in use.
__global__ __launch_bounds__(kThreads) void exchange_remap_kernel(ExchangeArgs g) {
  const int y = blockIdx.y;
  const int tid = threadIdx.x;
  const int R = g.r;
  __shared__ int s_v[kMaxExperts];  // per rank; EP <= E <= 1024
  __shared__ int s_wave[kThreads / kWave];
  if (static_cast<int>(blockIdx.x) < g.pair_blocks) {
    const int s = y;
    const int64_t p0 = static_cast<int64_t>(blockIdx.x) * kPairsPerBlock;
    const int32_t *ids = g.ids + s * g.npairs;
    int32_t *slot = g.slot + s * g.npairs;
    int sl[kPairsPerThread], ev[kPairsPerThread];
#pragma unroll
    for (int u = 0; u < kPairsPerThread; ++u) {
      const int64_t p = p0 + u * kThreads + tid;
      const bool in = p < g.npairs;
      sl[u] = in ? slot[p] : -1;
      ev[u] = in ? ids[p] : 0;
    }
    // receive row i = send row + (rows of d's buffer from sources before s)
    // - (start of s's segment for d in its own packed order)
    for (int d = tid; d < R; d += kThreads) {
      int before = 0;
      for (int q = 0; q < s; ++q) before += g.send_counts[static_cast<int64_t>(q) * R + d];
      s_v[d] = before - g.offsets[static_cast<int64_t>(s) * (g.e + 1) + d * g.l];
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPairsPerThread; ++u) {
      if (sl[u] < 0) continue;  // masked or invalid: stays -1
      const int64_t p = p0 + u * kThreads + tid;
      const int d = ev[u] / g.l;  // a routed pair's ID lies in [0, E)
      const int64_t i = static_cast<int64_t>(sl[u]) + s_v[d];
      if (i < g.cap) {
        const int64_t row = d * g.cap + i;  // < EP*C < 2^31: checked on the host
        g.recv_src[row] = static_cast<int32_t>(s * g.n + p / g.k);
        slot[p] = static_cast<int32_t>(row);
      } else {
        slot[p] = -1;  // past the buffer: dropped
      }
    }
    return;
  }
  // destination d: receive counts from every source, their packed cumsum
  const int d = y;
  const int xb = blockIdx.x - g.pair_blocks;
  for (int q = tid; q < R; q += kThreads) s_v[q] = g.send_counts[static_cast<int64_t>(q) * R + d];
  __syncthreads();
  int cnt[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) cnt[u] = 4 * tid + u < R ? s_v[4 * tid + u] : 0;
  const int64_t total = block_excl_scan4(s_v, R, s_wave);  // s_v: displacements
  if (xb == 0) {
    uint32_t *tab = g.table + static_cast<int64_t>(d) * 4 * R;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = 4 * tid + u;
      if (q < R) {
        tab[2 * R + q] = static_cast<uint32_t>(cnt[u]) * g.h;
        tab[3 * R + q] = static_cast<uint32_t>(s_v[q]) * g.h;  // < 2^32: checked on the host
      }
    }
    if (tid == 0) {
      g.recv_rows[d] = static_cast<int32_t>(total);
      if (total > g.cap) g.status[d] |= MOE_STATUS_CAPACITY;
    }
    // the counts all-to-all: d's slice of every source's count matrix
    int32_t *rec = g.recv_expert_counts + static_cast<int64_t>(d) * R * g.l;
    for (int i = tid; i < R * g.l; i += kThreads) {
      const int q = i / g.l, x = i - q * g.l;
      rec[i] = g.counts[static_cast<int64_t>(q) * g.e + d * g.l + x];
    }
  }
  // recv_src = -1 past the rows in use
  const int64_t used = min(total, g.cap);
  int32_t *src = g.recv_src + d * g.cap;
  const int64_t stride = static_cast<int64_t>(g.dest_blocks) * kThreads;
  for (int64_t i = used + static_cast<int64_t>(xb) * kThreads + tid; i < g.cap; i += stride) src[i] = -1;
}

}  // namespace

hipError_t launch_exchange_plan(const moe_problem &p, const int32_t *ids, const moe_exchange &x,
                                void *workspace, hipStream_t stream) {
  const ExchangeLayout L = exchange_layout(p);
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  const int R = p.ep;
  const moe_problem q = exchange_rank_problem(p);
  int32_t *offsets = reinterpret_cast<int32_t *>(ws + L.offsets);

  // 1. every rank's own plan, one launch
  moe_plan plan;
  plan.expert_counts = x.expert_counts;
  plan.expert_offsets = offsets;
  plan.dest_counts = x.send_counts;
  plan.rank_table = x.rank_table;
  plan.slot = x.recv_slot;
  plan.packed_src = reinterpret_cast<int32_t *>(ws + L.packed_src);
  plan.status = x.status;
  PlanStrides st;
  st.pairs = p.n_tokens * p.top_k;
  st.rows = p.n_tokens * p.top_k;  // R_max of a rank with A = 1
  st.workspace = static_cast<int64_t>(L.plan_ws_bytes / sizeof(int32_t));
  st.counts = p.n_experts;
  st.offsets = p.n_experts + 1;
  st.dest = R;
  st.table = 4 * R;
  hipError_t err = launch_plan_ranks(q, R, ids, plan, st, L.plan_ws_bytes ? ws + L.plan_ws : nullptr, stream);
  if (err != hipSuccess) return err;

  ExchangeArgs g;
  g.ids = ids;
  g.slot = x.recv_slot;
  g.counts = x.expert_counts;
  g.send_counts = x.send_counts;
  g.offsets = offsets;
  g.recv_expert_counts = x.recv_expert_counts;
  g.recv_rows = x.recv_rows;
  g.table = x.rank_table;
  g.recv_src = x.recv_src;
  g.status = x.status;
  g.n = p.n_tokens;
  g.npairs = p.n_tokens * p.top_k;
  g.cap = p.recv_capacity;
  g.h = static_cast<uint32_t>(p.hidden);
  g.k = p.top_k;
  g.e = p.n_experts;
  g.r = R;
  g.l = p.n_experts / R;
  g.pair_blocks = static_cast<int>((g.npairs + kPairsPerBlock - 1) / kPairsPerBlock);
  // at least one block per destination (its metadata), more for long tails
  const int64_t dest_blocks = (g.cap + kTailRowsPerBlock - 1) / kTailRowsPerBlock;
  g.dest_blocks = static_cast<int>(dest_blocks < 1 ? 1 : dest_blocks < kMaxTailBlocks ? dest_blocks
                                                                                      : kMaxTailBlocks);

  // 2. receive rows of every pair and their inverse; per destination: the
  //    receive counts and displacements, the counts all-to-all, the zero rows
  exchange_remap_kernel<<<dim3(g.pair_blocks + g.dest_blocks, R), kThreads, 0, stream>>>(g);
  return hipGetLastError();
}

hipError_t launch_exchange_combine(const moe_problem &p, const moe_exchange &x, const uint16_t *expert_out,
                                   const float *weights, uint16_t *out, hipStream_t stream) {
  // the reverse exchange and the weighted sum are one gather over the
  // stacked receive buffers: the single-buffer combine over all ranks' tokens
  moe_problem all = p;
  all.n_tokens = p.n_tokens * p.ep;
  moe_plan plan{};
  plan.slot = x.recv_slot;
  return launch_combine(all, plan, expert_out, p.recv_capacity * p.ep, weights, out, stream);
}

}  // namespace moe
