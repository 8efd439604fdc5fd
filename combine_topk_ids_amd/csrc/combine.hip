// combine.hip -- gather each token's expert outputs and sum them weighted by
// the gate values.
//
// What is computed (pages cited by title and section):
//   DeepSpeed v0.19.4 function index, page 15 -- the combine entry: expert
//     results of each token are gathered back and weighted by gate values.
//   NeMo Automodel token_dispatcher API -- token_unpermutation /
//     combine_preprocess (restore the pre-expert token order),
//     TokenDispatcherConfig.moe_router_dtype (weighted averaging in fp32).
//   Mojo shmem ep_comm module -- router_weights_wrapper_type (one fp32 gate
//     weight per (token, top-k slot)).
//
// out[t][c] = bf16_rne(acc), acc = +0 then acc = fma(w[t][j], Y[slot][c], acc)
// for j = 0..k-1 in order, skipping masked slots: the same fp32 rounding
// sequence on every element, so results do not depend on the launch shape.
// Without weights (rows gated at dispatch: DeepSpeed v0.19.4 function index,
// page 15, the entry on scaling rows by router scores) every w is 1.
//
// Design for gfx950.  One wave64 per (token, column slab); each lane owns 8
// consecutive columns (one 16-byte bf16 vector) of every 512-column chunk of
// the slab.  Slabs are 2048 columns when the expert rows are streamed
// (longer runs of each row per wave measured faster there), 1024 when they
// are read with cache-allocating loads, and 512 when 1024-column slabs would
// give the launch too few waves to fill the GPU (decode shapes).  The
// token's k slots and gate weights are loaded once, one per lane, and
// broadcast with readlane; all k row loads of the slab are issued before the
// first FMA, so each wave makes two round trips to memory (index loads, then
// row loads) and keeps k x 2 or 4 KiB in flight.  Every row is read through
// a buffer resource that spans that row alone, and a masked slot (or one
// outside the rows of expert_out) gets a resource of zero bytes: its loads
// return zeros without touching memory, so no row that no slot names is
// ever read, and expert_out may be NULL when no slot can name a row.
#include "moe_device.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Tuning knobs (build-time): 16-byte vectors per lane in a slab (columns
// per wave = 512 * vectors) with cache-allocating and with non-temporal row
// loads; the footprint of expert rows up to which they are read with
// ordinary (cache-allocating) loads -- rows written just before, e.g. by the
// expert GEMM or, for identity experts, by the dispatch, are then still in
// the 256 MB Infinity Cache -- and beyond which with non-temporal loads that
// do not churn the caches.
#ifndef MOE_COMBINE_VEC
#define MOE_COMBINE_VEC 2
#endif
#ifndef MOE_COMBINE_VEC_NT
#define MOE_COMBINE_VEC_NT 4
#endif
// fewest waves a cached-path launch should have; below it the slabs halve
#ifndef MOE_COMBINE_MIN_WAVES
#define MOE_COMBINE_MIN_WAVES 8192
#endif
#ifndef MOE_COMBINE_CACHED_BYTES
#define MOE_COMBINE_CACHED_BYTES (256ll << 20)
#endif

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kBatch = 8;   // top-k slots whose loads are issued together

struct CombineArgs {
  const uint16_t *y;
  const int32_t *slot;
  const float *w;
  uint16_t *out;
  int64_t n;
  int64_t rows;  // rows of y: a slot outside [0, rows) is read as masked
  int k, h;
  int slabs;  // waves per token
};

__device__ __forceinline__ void fma8(float (&acc)[8], float w, const u32x4 v) {
  acc[0] = __builtin_fmaf(w, bf16_lo(v.x), acc[0]);
  acc[1] = __builtin_fmaf(w, bf16_hi(v.x), acc[1]);
  acc[2] = __builtin_fmaf(w, bf16_lo(v.y), acc[2]);
  acc[3] = __builtin_fmaf(w, bf16_hi(v.y), acc[3]);
  acc[4] = __builtin_fmaf(w, bf16_lo(v.z), acc[4]);
  acc[5] = __builtin_fmaf(w, bf16_hi(v.z), acc[5]);
  acc[6] = __builtin_fmaf(w, bf16_lo(v.w), acc[6]);
  acc[7] = __builtin_fmaf(w, bf16_hi(v.w), acc[7]);
}

__device__ __forceinline__ u32x4 pack8(const float (&a)[8]) {
  u32x4 r;
  r.x = f32_to_bf16(a[0]) | (f32_to_bf16(a[1]) << 16);
  r.y = f32_to_bf16(a[2]) | (f32_to_bf16(a[3]) << 16);
  r.z = f32_to_bf16(a[4]) | (f32_to_bf16(a[5]) << 16);
  r.w = f32_to_bf16(a[6]) | (f32_to_bf16(a[7]) << 16);
  return r;
}

// KC > 0: k is the compile-time constant KC; KC == 0: runtime k, in batches.
// NT: non-temporal expert-row loads.  VEC: 16-byte vectors per lane per
// slab (512 * VEC columns per wave).
template <int KC, bool NT, int VEC>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs g) {
  constexpr int kVec = VEC;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int q = blockIdx.x * kWaves + wave;  // the grid size keeps q within int
  const int t = q / g.slabs;
  if (t >= g.n) return;
  const int slab = q - t * g.slabs;
  const int lane = lane_id();
  const int k = KC > 0 ? KC : g.k;
  const int nvec = g.h / 8;
  const int v0 = slab * kWave * kVec;
  const int64_t pair0 = static_cast<int64_t>(t) * k;
  const int my_slot = lane < k ? g.slot[pair0 + lane] : -1;
  // no weights: every gate is 1 (the rows were weighted at dispatch), and
  // fma(1, y, acc) is the correctly rounded y + acc
  const float my_w = lane < k ? (g.w ? g.w[pair0 + lane] : 1.0f) : 0.0f;

  float acc[kVec][8];
#pragma unroll
  for (int u = 0; u < kVec; ++u)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[u][i] = 0.0f;

  constexpr int KB = KC > 0 ? KC : kBatch;
  const uint32_t row_bytes = 2u * static_cast<uint32_t>(g.h);
  for (int j0 = 0; j0 < k; j0 += KB) {
    u32x4 v[KB][kVec];
    bool live[KB];
#pragma unroll
    for (int jj = 0; jj < KB; ++jj) {
      const int s = (KC > 0 || j0 + jj < k) ? __builtin_amdgcn_readlane(my_slot, j0 + jj) : -1;
      live[jj] = s >= 0 && s < g.rows;
      // the row alone, or nothing: loads past the resource return zeros and
      // touch no memory (also the columns past H in the last slab)
      const auto rsrc = buffer_rsrc(live[jj] ? g.y + static_cast<int64_t>(s) * g.h : g.y,
                                    live[jj] ? row_bytes : 0u);
#pragma unroll
      for (int u = 0; u < kVec; ++u)
        v[jj][u] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (v0 + u * kWave + lane) * 16, 0,
                                                         NT ? kLoadNT : kLoadDefault);
    }
#pragma unroll
    for (int jj = 0; jj < KB; ++jj) {
      if (!live[jj]) continue;
      const float wj = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_w), j0 + jj));
#pragma unroll
      for (int u = 0; u < kVec; ++u) fma8(acc[u], wj, v[jj][u]);
    }
  }
  u32x4 *dst = reinterpret_cast<u32x4 *>(g.out + static_cast<int64_t>(t) * g.h);
#pragma unroll
  for (int u = 0; u < kVec; ++u) {
    const int idx = v0 + u * kWave + lane;
    if (idx < nvec) __builtin_nontemporal_store(pack8(acc[u]), dst + idx);
  }
}

template <bool NT, int VEC>
void launch_k(const CombineArgs &g, int k, int grid, hipStream_t stream) {
  switch (k) {
    case 1: combine_kernel<1, NT, VEC><<<grid, kThreads, 0, stream>>>(g); break;
    case 2: combine_kernel<2, NT, VEC><<<grid, kThreads, 0, stream>>>(g); break;
    case 4: combine_kernel<4, NT, VEC><<<grid, kThreads, 0, stream>>>(g); break;
    case 6: combine_kernel<6, NT, VEC><<<grid, kThreads, 0, stream>>>(g); break;
    case 8: combine_kernel<8, NT, VEC><<<grid, kThreads, 0, stream>>>(g); break;
    default: combine_kernel<0, NT, VEC><<<grid, kThreads, 0, stream>>>(g); break;
  }
}

}  // namespace

hipError_t launch_combine(const moe_problem &p, const moe_plan &plan, const uint16_t *expert_out,
                          int64_t rows, const float *weights, uint16_t *out, hipStream_t stream) {
  CombineArgs g;
  g.y = expert_out;
  g.slot = plan.slot;
  g.w = weights;
  g.out = out;
  g.n = p.n_tokens;
  g.rows = expert_out ? rows : 0;
  g.k = p.top_k;
  g.h = p.hidden;
  // bytes of expert rows this launch reads (one row per valid pair at most)
  const int64_t rows_bytes = p.n_tokens * p.top_k * 2 * static_cast<int64_t>(p.hidden);
  const bool nt = rows_bytes > MOE_COMBINE_CACHED_BYTES;
  auto slabs_of = [&](int vec) { return (p.hidden + kWave * vec * 8 - 1) / (kWave * vec * 8); };
  int vec = nt ? MOE_COMBINE_VEC_NT : MOE_COMBINE_VEC;
  if (!nt && vec > 1 && p.n_tokens * slabs_of(vec) < MOE_COMBINE_MIN_WAVES) vec = 1;
  g.slabs = slabs_of(vec);
  const int64_t waves = p.n_tokens * g.slabs;
  const int grid = static_cast<int>((waves + kWaves - 1) / kWaves);
  if (grid == 0) return hipSuccess;
  if (nt)
    launch_k<true, MOE_COMBINE_VEC_NT>(g, p.top_k, grid, stream);
  else if (vec == 1)
    launch_k<false, 1>(g, p.top_k, grid, stream);
  else
    launch_k<false, MOE_COMBINE_VEC>(g, p.top_k, grid, stream);
  return hipGetLastError();
}

}  // namespace moe
