// exchange.hip -- the receive side of the expert-parallel exchange,
// simulated on one GPU that holds the shares of all EP ranks.
//
// What is computed (pages cited by title and section):
//   NKI permute_a2av API reference -- description: the receive layout is the
//     packed cumsum of the receive counts; the (4, EP) table's rows 2-3 hold
//     receive counts and displacements in elements; :return: a [C, H]
//     receive buffer of source-major packed rows followed by deterministic
//     zero padding.
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
//   2. exchange_scan (thread per destination d): walks the sources in order
//      over the send-count matrix column of d: rows of d's buffer that come
//      before source s, the receive counts and displacements (table rows
//      2-3), the rows offered to d, CAPACITY, and what the counts
//      all-to-all delivers to d (its slice of every source's count matrix);
//   3. exchange_remap (blocks of pairs per source, blockIdx.y = source):
//      receive row = d*C + (rows before source s in d's buffer) + (send row
//      - start of the source's segment for d), kept if below C; writes the
//      inverse map recv_src, and -1 over each buffer's zero rows.
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
  int32_t *pre;                 // [R][R] ([s][d]) rows of d's buffer before source s
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
  int pair_blocks, tail_blocks;
};

__global__ __launch_bounds__(kThreads) void exchange_scan_kernel(ExchangeArgs g) {
  const int d = blockIdx.x * kThreads + threadIdx.x;
  if (d >= g.r) return;
  const int R = g.r;
  uint32_t *tab = g.table + static_cast<int64_t>(d) * 4 * R;
  int64_t run = 0;
  for (int s = 0; s < R; ++s) {
    const int c = g.send_counts[static_cast<int64_t>(s) * R + d];
    g.pre[static_cast<int64_t>(s) * R + d] = static_cast<int32_t>(run);
    tab[2 * R + s] = static_cast<uint32_t>(c) * g.h;
    tab[3 * R + s] = static_cast<uint32_t>(run) * g.h;  // < 2^32: checked on the host
    run += c;
  }
  g.recv_rows[d] = static_cast<int32_t>(run);
  if (run > g.cap) g.status[d] |= MOE_STATUS_CAPACITY;
  // the counts all-to-all: d's slice of every source's count matrix
  int32_t *rec = g.recv_expert_counts + static_cast<int64_t>(d) * R * g.l;
  for (int s = 0; s < R; ++s)
    for (int x = 0; x < g.l; ++x)
      rec[s * g.l + x] = g.counts[static_cast<int64_t>(s) * g.e + d * g.l + x];
}

__global__ __launch_bounds__(kThreads) void exchange_remap_kernel(ExchangeArgs g) {
  const int s = blockIdx.y;
  const int tid = threadIdx.x;
  if (static_cast<int>(blockIdx.x) < g.pair_blocks) {
    __shared__ int s_base[kMaxExperts];  // per destination; EP <= E <= 1024
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
    // receive row i = send row + (rows before s in d's buffer) - (start of
    // s's segment for d in its own packed order)
    for (int d = tid; d < g.r; d += kThreads)
      s_base[d] = g.pre[static_cast<int64_t>(s) * g.r + d] -
                  g.offsets[static_cast<int64_t>(s) * (g.e + 1) + d * g.l];
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPairsPerThread; ++u) {
      if (sl[u] < 0) continue;  // masked or invalid: stays -1
      const int64_t p = p0 + u * kThreads + tid;
      const int d = ev[u] / g.l;  // a routed pair's ID lies in [0, E)
      const int64_t i = static_cast<int64_t>(sl[u]) + s_base[d];
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
  // zero rows of receive buffer d = blockIdx.y
  const int d = s;
  const int64_t used = min(static_cast<int64_t>(g.recv_rows[d]), g.cap);
  int32_t *src = g.recv_src + d * g.cap;
  const int64_t stride = static_cast<int64_t>(g.tail_blocks) * kThreads;
  for (int64_t i = used + static_cast<int64_t>(blockIdx.x - g.pair_blocks) * kThreads + tid; i < g.cap;
       i += stride)
    src[i] = -1;
}

size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

// Workspace: [R][E+1] offsets, [R][R] pre, [R][N*k] packed_src of the
// per-rank plans, then R copies of the single-rank plan workspace.
struct Layout {
  size_t offsets, pre, packed_src, plan_ws, total;
  size_t plan_ws_bytes;  // per rank
};

moe_problem rank_problem(const moe_problem &p) {
  moe_problem q = p;
  q.pad_multiple = 1;
  q.recv_capacity = INT64_MAX;  // capacity applies to receive buffers only
  q.flags = 0;
  return q;
}

Layout layout(const moe_problem &p) {
  const size_t R = static_cast<size_t>(p.ep);
  Layout L;
  size_t at = 0;
  L.offsets = at;
  at += align256(R * (p.n_experts + 1) * sizeof(int32_t));
  L.pre = at;
  at += align256(R * R * sizeof(int32_t));
  L.packed_src = at;
  at += align256(R * static_cast<size_t>(p.n_tokens) * p.top_k * sizeof(int32_t));
  L.plan_ws_bytes = plan_workspace_bytes(rank_problem(p));
  L.plan_ws = at;
  at += R * L.plan_ws_bytes;
  L.total = at;
  return L;
}

}  // namespace

size_t exchange_workspace_bytes(const moe_problem &p) { return layout(p).total; }

hipError_t launch_exchange_plan(const moe_problem &p, const int32_t *ids, const moe_exchange &x,
                                void *workspace, hipStream_t stream) {
  const Layout L = layout(p);
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  const int R = p.ep;
  const moe_problem q = rank_problem(p);
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
  g.pre = reinterpret_cast<int32_t *>(ws + L.pre);
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
  const int64_t tail_blocks = (g.cap + kTailRowsPerBlock - 1) / kTailRowsPerBlock;
  g.tail_blocks = static_cast<int>(tail_blocks < kMaxTailBlocks ? tail_blocks : kMaxTailBlocks);

  // 2. receive counts and displacements
  exchange_scan_kernel<<<(R + kThreads - 1) / kThreads, kThreads, 0, stream>>>(g);
  // 3. receive rows of every pair, their inverse, the zero rows
  const int gx = g.pair_blocks + g.tail_blocks;
  if (gx > 0) exchange_remap_kernel<<<dim3(gx, R), kThreads, 0, stream>>>(g);
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
  return launch_combine(all, plan, expert_out, weights, out, stream);
}

}  // namespace moe
