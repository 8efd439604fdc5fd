// Fuzz driver for libmoe's host-side rules (host_checks.cpp), built with
// address and undefined-behaviour sanitizers by tests/test_sanitizers.py.
// Problems are drawn from edge values of every field (zero, one, limits,
// their neighbours, int32/int64 extremes) and from random values; every
// check and size helper is called on each, with pointer arguments null,
// aligned and misaligned.  Besides the sanitizers' own checks it asserts the
// guarantees the kernels rely on for every problem check_problem accepts.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "host_checks.hpp"

namespace {

uint64_t rng_state = 0x9E3779B97F4A7C15ull;
uint64_t next_u64() {  // splitmix64
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

template <typename T, size_t N>
T pick(const T (&v)[N]) { return v[next_u64() % N]; }

int failures = 0;
#define EXPECT(c)                                                           \
  do {                                                                      \
    if (!(c)) {                                                             \
      if (failures++ < 20) fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #c); \
    }                                                                       \
  } while (0)

const int64_t kI64[] = {INT64_MIN, -1, 0, 1, 2, 3, 7, 8, 127, 128, 129, 2047, 2048, 2049, 4096,
                        16384, 65535, 65536, 1 << 20, (int64_t)1 << 30, INT32_MAX / 8,
                        INT32_MAX / 64, INT32_MAX - 1, INT32_MAX, (int64_t)INT32_MAX + 1,
                        (int64_t)1 << 40, INT64_MAX - 1, INT64_MAX};
const int32_t kI32[] = {INT32_MIN, -1, 0, 1, 2, 3, 4, 6, 8, 12, 16, 32, 63, 64, 65, 100, 127, 128,
                        129, 255, 256, 257, 1000, 1023, 1024, 1025, 4096, 7168, 65536, 1 << 20,
                        INT32_MAX - 1, INT32_MAX};

int64_t draw64() { return next_u64() % 4 ? pick(kI64) : (int64_t)next_u64(); }
int32_t draw32() { return next_u64() % 4 ? pick(kI32) : (int32_t)next_u64(); }

moe_problem draw_problem() {
  moe_problem p;
  p.n_tokens = next_u64() % 3 ? (int64_t)(next_u64() % 70000) : draw64();
  p.hidden = next_u64() % 3 ? (int32_t)(8u * (uint32_t)(next_u64() % 8193)) : draw32();
  p.n_experts = next_u64() % 3 ? 1 + (int32_t)(next_u64() % 1024) : draw32();
  p.top_k = next_u64() % 3 ? 1 + (int32_t)(next_u64() % 64) : draw32();
  p.ep = next_u64() % 3 ? 1 << (next_u64() % 6) : draw32();
  p.recv_capacity = next_u64() % 2 ? (int64_t)(next_u64() % 200000) : draw64();
  p.pad_multiple = next_u64() % 3 ? 1 + (int32_t)(next_u64() % 128) : draw32();
  p.fmt = next_u64() % 4 ? (int32_t)(next_u64() % 4) : draw32();
  p.flags = next_u64() % 4 ? (uint32_t)(next_u64() % 2) : (uint32_t)next_u64();
  p.expert_capacity = next_u64() % 2 ? 0 : (next_u64() % 2 ? (int64_t)(next_u64() % 5000) : draw64());
  return p;
}

void *ptr_of(int kind) {  // never dereferenced: only checked for null and alignment
  switch (kind) {
    case 0: return nullptr;
    case 1: return reinterpret_cast<void *>(uintptr_t{1} << 20);
    case 2: return reinterpret_cast<void *>((uintptr_t{1} << 20) + 4);
    default: return reinterpret_cast<void *>((uintptr_t{1} << 20) + 1);
  }
}
void *any_ptr() { return ptr_of((int)(next_u64() % 8 < 5 ? 1 : next_u64() % 4)); }

bool valid_code(int rc) {
  return rc == MOE_OK || rc == MOE_EINVAL || rc == MOE_EALIGN || rc == MOE_EOVERFLOW;
}

void check_accepted(const moe_problem &p) {
  using namespace moe;
  const int64_t r_max = max_rows(p);
  EXPECT(r_max >= 0 && r_max <= INT32_MAX);
  EXPECT(r_max * (int64_t)p.hidden < ((int64_t)1 << 32));
  EXPECT(p.n_tokens * p.top_k <= INT32_MAX);
  EXPECT(payload_row_bytes(p) > 0 && scale_row_bytes(p) >= 0);
  const PlanGeom g = plan_geometry(p);
  EXPECT(g.ntiles >= 1 && (int64_t)g.ntiles * g.tile_tokens >= p.n_tokens);
  EXPECT(g.tile_pairs <= kPlanTilePairs || g.tile_tokens == 1);
  EXPECT(g.subs >= 1 && (int64_t)g.subs * kPlanSubPairs >= (g.single ? g.npairs : g.tile_pairs));
  EXPECT((1 << g.key_bits) >= p.n_experts);
  const size_t ws = plan_workspace_bytes(p);
  EXPECT(ws % 256 == 0);
  EXPECT(g.single ? ws == 0 : ws >= (size_t)g.ntiles * (p.n_experts + 1) * 4);
  const PlanDispatchMode m = plan_dispatch_mode(p);
  if (m == PlanDispatchMode::kOneLaunch) EXPECT(p.n_tokens * p.top_k <= kSmallPairs);
  if (m == PlanDispatchMode::kTiled) EXPECT((int64_t)g.ntiles * p.n_experts <= kTileHist && r_max <= INT32_MAX);
  if (one_launch_direct(p)) {  // keys (expert << 11 | pair index) fit 21 bits
    EXPECT(m == PlanDispatchMode::kOneLaunch && p.pad_multiple == 1 && p.expert_capacity == 0);
    EXPECT(p.n_tokens * p.top_k <= kSmallPairs && kSmallPairs <= 2048 && p.n_experts <= 1024);
  }
  EXPECT(map_workspace_bytes(p) % 256 == 0);
  EXPECT((int64_t)map_blocks(p) * (kMapThreads / map_lanes_per_token(p.n_experts)) >= p.n_tokens);
}

void one_problem(const moe_problem &p) {
  using namespace moe::host;
  const int rc = check_problem(&p);
  EXPECT(valid_code(rc));
  if (rc == MOE_OK) check_accepted(p);
  const int rx = check_exchange(&p);
  EXPECT(valid_code(rx));
  if (rx == MOE_OK) {
    EXPECT(rc == MOE_OK);
    const moe::ExchangeLayout L = moe::exchange_layout(p);
    EXPECT(L.offsets <= L.packed_src && L.packed_src <= L.plan_ws && L.plan_ws <= L.total);
    EXPECT((int64_t)p.ep * p.recv_capacity <= INT32_MAX);
  }
  moe_plan plan;
  int32_t **fields[] = {&plan.expert_counts, &plan.expert_offsets, &plan.dest_counts, &plan.slot,
                        &plan.packed_src};
  for (int32_t **f : fields) *f = static_cast<int32_t *>(any_ptr());
  plan.rank_table = static_cast<uint32_t *>(any_ptr());
  plan.status = static_cast<uint32_t *>(any_ptr());
  moe_exchange x;
  int32_t **xf[] = {&x.expert_counts, &x.send_counts, &x.recv_expert_counts, &x.recv_rows,
                    &x.recv_slot, &x.recv_src};
  for (int32_t **f : xf) *f = static_cast<int32_t *>(any_ptr());
  x.rank_table = static_cast<uint32_t *>(any_ptr());
  x.status = static_cast<uint32_t *>(any_ptr());
  auto i32 = [] { return static_cast<const int32_t *>(any_ptr()); };
  auto u16 = [] { return static_cast<const uint16_t *>(any_ptr()); };
  auto f32 = [] { return static_cast<const float *>(any_ptr()); };
  const moe_problem *pp = next_u64() % 64 ? &p : nullptr;
  const moe_plan *pl = next_u64() % 64 ? &plan : nullptr;
  const moe_exchange *px = next_u64() % 64 ? &x : nullptr;
  int codes[] = {
      check_plan_args(pp, i32(), pl, any_ptr()),
      check_plan_and_dispatch_args(pp, i32(), pl, u16(), f32(), f32(), any_ptr(), any_ptr(), any_ptr()),
      check_dispatch_args(pp, pl, u16(), any_ptr(), any_ptr()),
      check_dispatch_scaled_args(pp, pl, u16(), f32(), any_ptr(), any_ptr()),
      check_dispatch_gated_args(pp, pl, u16(), f32(), any_ptr(), any_ptr()),
      check_combine_args(pp, pl, u16(), f32(), static_cast<const uint16_t *>(any_ptr())),
      check_exchange_plan_args(pp, i32(), px, any_ptr()),
      check_exchange_dispatch_args(pp, px, u16(), any_ptr(), any_ptr()),
      check_exchange_dispatch_scaled_args(pp, px, u16(), f32(), any_ptr(), any_ptr()),
      check_exchange_dispatch_gated_args(pp, px, u16(), f32(), any_ptr(), any_ptr()),
      check_exchange_combine_args(pp, px, u16(), f32(), static_cast<const uint16_t *>(any_ptr())),
      check_map_args(pp, static_cast<const uint8_t *>(any_ptr()), f32(), i32(), f32(),
                     static_cast<const uint32_t *>(any_ptr()), any_ptr()),
  };
  for (int c : codes) {
    EXPECT(valid_code(c));
    // an entry point never accepts a problem that check_problem refuses
    if (pp && rc != MOE_OK) EXPECT(c != MOE_OK);
  }
  if (!pp) for (int c : codes) EXPECT(c == MOE_EINVAL);
  for (int c = -6; c <= 1; ++c) EXPECT(error_text(c) != nullptr);
}

}  // namespace

int main(int argc, char **argv) {
  const long iters = argc > 1 ? atol(argv[1]) : 300000;
  for (long i = 0; i < iters; ++i) one_problem(draw_problem());
  // the shapes of the workloads, accepted
  const moe_problem shapes[] = {
      {128, 256, 2, 8, 4, 256, 1, MOE_FMT_BF16, 0, 0},
      {4096, 4096, 6, 64, 8, 24576, 128, MOE_FMT_BF16, 0, 0},
      {8192, 7168, 8, 256, 32, 65536, 1, MOE_FMT_FP8_E4M3_B128, 0, 0},
      {16384, 4096, 8, 128, 16, 131072, 128, MOE_FMT_BF16, 0, 0},
      {128, 7168, 8, 256, 8, 1024, 1, MOE_FMT_MXFP4_B32, 0, 0},
  };
  for (const moe_problem &p : shapes) {
    EXPECT(moe::host::check_problem(&p) == MOE_OK);
    one_problem(p);
  }
  const double cfs[] = {0.0, 0.5, 1.0, 1.25, 1e9, 1e300, INFINITY, -1.0, NAN, -0.0};
  for (double cf : cfs)
    for (int64_t n : kI64)
      for (int32_t k : kI32) {
        const int64_t c = moe::expert_capacity(n, k, 64, cf);
        EXPECT(c == MOE_EINVAL || c == MOE_EOVERFLOW || (c >= 0 && c <= INT32_MAX));
      }
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("host checks: %ld random problems and the workload shapes, no failures\n", iters);
  return 0;
}
