// dispatch.hip -- pack token rows into the expert-major buffer, optionally
// quantising them on the way.
//
// What is computed (pages cited by title and section):
//   NKI permute_a2av API reference -- description and :return: (rows packed
//     per destination; unused rows are zero bytes).
//   NeMo Automodel token_dispatcher API -- get_permuted_hidden_states_by_experts
//     (rows permuted into expert order by a fused kernel),
//     TokenDispatcherConfig.moe_router_expert_pad_multiple (pad rows).
//   Mojo shmem ep_comm module -- BF16TokenFormat (rows carried in bf16),
//     BlockwiseFP8TokenFormat (FP8 with one scale per block),
//     MXTokenFormat (MX FP4), EP_COPY_SRC_WIDTH (8 source elements per
//     thread per copy item), block_memcpy (vector loads and stores).
//   Formats: OCP 8-bit Floating Point (E4M3) and OCP MX v1.0 (E2M1, E8M0),
//     with the per-1x128 amax/448 fp32 scale of the FP8 recipe.
//
// Design for gfx950.  Token-stationary: one wave64 owns one column slab of
// one token, reads it once with 16-byte loads (8 bf16 per lane, 1 KiB per
// wave instruction), encodes it once, and writes the result to each of the
// token's k packed rows, so the cost does not depend on how skewed the
// routing is.  In the quantising formats a lane encodes 8 consecutive values
// (a 512-value slab per wave: the division-heavy FP8 encode wants many
// waves); an FP8 1x128 block spans one 16-lane DPP row (block maximum by
// quad, half-row and row mirrors), an MX 32-value block one quad.  Pad rows
// are zeroed by a second range of workgroups in the same launch, the
// optional tail by a third.
//
// The simulated expert-parallel exchange reuses the token waves unchanged:
// there the slot of a pair is its row in the stacked receive buffers of all
// ranks, and the third range writes the zero rows that end every receive
// buffer (NKI permute_a2av API reference, :return:).
//
// plan_dispatch_kernel plans and dispatches in one launch (NKI permute_a2av
// API reference, description: one call both lays out and permutes): each
// workgroup computes in LDS the part of the plan it needs (small_plan.hpp)
// while its slabs load, from all the IDs (at most 2048 pairs) or from the
// tile histograms of the plan's counting kernel (tiled mode).
#include "moe_device.hpp"
#include "moe_kernels.hpp"
#include "small_plan.hpp"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Tuning knobs (build-time): vectors per lane in a bf16 slab, bf16 elements
// per lane in the quantising formats (8 or 16), non-temporal payload stores.
#ifndef MOE_DISPATCH_VEC
#define MOE_DISPATCH_VEC 4
#endif
#ifndef MOE_QUANT_LANE_ELEMS
#define MOE_QUANT_LANE_ELEMS 8
#endif
#ifndef MOE_DISPATCH_NT_STORE
#define MOE_DISPATCH_NT_STORE 0
#endif
#ifndef MOE_QUANT_CHUNKS
#define MOE_QUANT_CHUNKS 1
#endif
// Zero rows after the used part of each segment: workgroups for them, their
// place in the grid (first or last), non-temporal stores.  Non-temporal
// tail stores measured faster (receive-buffer tails: 400 vs 436 us at 8
// ranks x 4096 tokens); on per-expert pad rows they slowed the combine that
// follows, so pad rows keep ordinary stores.
#ifndef MOE_TAIL_BLOCKS
#define MOE_TAIL_BLOCKS 512
#endif
#ifndef MOE_TAIL_FIRST
#define MOE_TAIL_FIRST 0
#endif
#ifndef MOE_TAIL_NT
#define MOE_TAIL_NT 1
#endif


constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kPadRowsPerWave = 4;
constexpr int kTailBlocks = MOE_TAIL_BLOCKS;

struct DispatchArgs {
  const uint16_t *x;
  const int32_t *slot;
  const float *w;  // [n][k] gates applied at dispatch (gated launches only)
  const float *gscale;  // [1] NVFP4 global encode scale
  const int32_t *counts;
  const int32_t *offsets;
  uint8_t *payload;
  uint8_t *scales;
  int64_t n;
  int64_t r_max;
  int64_t row_bytes;    // payload bytes per packed row
  int64_t scale_bytes;  // scale bytes per packed row
  int k, h, e;
  int slabs;  // waves per token
  int token_blocks, pad_blocks, tail_blocks;
  int pad_groups;  // pad-row groups of kPadRowsPerWave per expert
  // Zero rows at the end of each of `nseg` segments of seg_rows rows:
  // segment d keeps its first min(seg_used[d], seg_rows) rows.  One segment
  // (the whole buffer, used = R_used) for a single packed buffer; one per
  // receive buffer for the exchange.
  const int32_t *seg_used;  // null: one segment, used_rows rows used
  int nseg;
  int64_t seg_rows;
  int used_rows;
};

template <bool NT, typename V>
__device__ __forceinline__ void store(V *p, V v) {
  if (NT)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

// One wave handles one (token, column slab).  The k destination slots are
// loaded once, one per lane, together with the slab's data, and broadcast
// with readlane, so a wave makes a single round trip to memory before it
// starts storing.
// A slot outside the buffer's rows [0, r_max) is skipped like a masked one.
__device__ __forceinline__ int lane_slot(const DispatchArgs &g, int64_t t, int lane) {
  const int s = lane < g.k ? g.slot[t * g.k + lane] : -1;
  return s >= 0 && s < g.r_max ? s : -1;
}

// ---- bf16: copy the slab to every destination -------------------------------
constexpr int kBf16Vec = MOE_DISPATCH_VEC;  // 16-byte vectors per lane per slab

// quantising formats: each lane encodes LE consecutive values
constexpr int kLE = MOE_QUANT_LANE_ELEMS;           // 8 or 16
constexpr int kQC = MOE_QUANT_CHUNKS;               // chunks of kWave*kLE per wave
constexpr int kQuantSlab = kWave * kLE * kQC;       // values per wave
static_assert(kLE == 8 || kLE == 16, "8 or 16 values per lane");

// What one lane of a token wave reads: its 16-byte vectors of the slab
// (zeros past the row end) and, for gated copies, its gate (lane j holds
// the gate of pair (t, j)).  Loading is separate from encoding and storing
// so that a caller can issue these loads before other work.
constexpr int kRawVec = kBf16Vec > kQC * kLE / 8 ? kBf16Vec : kQC * kLE / 8;
struct RawSlab {
  u32x4 v[kRawVec];
  float w;
};

template <int FMT, bool GATED>
__device__ __forceinline__ RawSlab load_slab(const DispatchArgs &g, int64_t t, int slab) {
  const int lane = lane_id();
  const u32x4 *row = reinterpret_cast<const u32x4 *>(g.x + t * g.h);
  const u32x4 zero = {0u, 0u, 0u, 0u};
  RawSlab r;
  if (FMT == MOE_FMT_BF16) {
    const int nvec = g.h / 8;
    const int v0 = slab * kWave * kBf16Vec;
#pragma unroll
    for (int u = 0; u < kBf16Vec; ++u) {
      const int idx = v0 + u * kWave + lane;
      r.v[u] = idx < nvec ? __builtin_nontemporal_load(row + idx) : zero;
    }
  } else {
#pragma unroll
    for (int c = 0; c < kQC; ++c) {
      const int elem = slab * kQuantSlab + c * kWave * kLE + lane * kLE;
#pragma unroll
      for (int q = 0; q < kLE / 8; ++q)
        r.v[c * (kLE / 8) + q] = elem < g.h ? __builtin_nontemporal_load(row + elem / 8 + q) : zero;
    }
  }
  r.w = GATED && lane < g.k ? g.w[t * g.k + lane] : 0.0f;
  return r;
}

// load_slab through bounds-checked buffer loads, issued whether or not the
// wave has a token (live): a wave without one reads nothing and gets zeros.
// No branch surrounds the loads, so a kernel that issues other loads before
// these can wait for those alone.
template <int FMT, bool GATED>
__device__ __forceinline__ RawSlab load_slab_buf(const DispatchArgs &g, int64_t t, int slab, bool live) {
  const int lane = lane_id();
  const auto row = buffer_rsrc(live ? g.x + t * g.h : g.x, live ? 2u * static_cast<uint32_t>(g.h) : 0u);
  RawSlab r;
  if (FMT == MOE_FMT_BF16) {
    const int v0 = slab * kWave * kBf16Vec;
#pragma unroll
    for (int u = 0; u < kBf16Vec; ++u)
      r.v[u] = __builtin_amdgcn_raw_buffer_load_b128(row, (v0 + u * kWave + lane) * 16, 0, kLoadNT);
  } else {
#pragma unroll
    for (int c = 0; c < kQC; ++c) {
      const int elem = slab * kQuantSlab + c * kWave * kLE + lane * kLE;
#pragma unroll
      for (int q = 0; q < kLE / 8; ++q)
        r.v[c * (kLE / 8) + q] = __builtin_amdgcn_raw_buffer_load_b128(row, (elem / 8 + q) * 16, 0, kLoadNT);
    }
  }
  if (GATED) {
    const auto w = buffer_rsrc(g.w + (live ? t * g.k : 0), live ? 4u * static_cast<uint32_t>(g.k) : 0u);
    r.w = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(w, lane * 4, 0, kLoadDefault));
  } else {
    r.w = 0.0f;
  }
  return r;
}

// Chunk c of this lane's values as fp32.
__device__ __forceinline__ void unpack_lane(const RawSlab &r, int c, float (&f)[kLE]) {
#pragma unroll
  for (int q = 0; q < kLE / 8; ++q) {
    const u32x4 v = r.v[c * (kLE / 8) + q];
    uint4 r4;
    r4.x = v.x; r4.y = v.y; r4.z = v.z; r4.w = v.w;
    float h[8];
    unpack8(r4, h);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[q * 8 + i] = h[i];
  }
}

// Cache policy of the bf16 row stores: device scope (the sc1 bit).  Against
// default stores, the uniform workload's dispatch (4096 tokens x 6 rows of
// 8 KiB) ran 44.0 -> 43.1 us with it, and the Zipf and capacity workloads
// did not change.  The same bit made the FP8 dispatch 6-9% slower, so the
// quantising formats keep default stores.
constexpr int kStoreDevice = 16;
constexpr int kStoreNT = 2;

template <bool NT>
__device__ void slab_bf16(const DispatchArgs &g, int slab, int my_slot, const RawSlab &r) {
  const int lane = lane_id();
  const int nvec = g.h / 8;
  const int v0 = slab * kWave * kBf16Vec;
  const u32x4 *buf = r.v;
  for (int j = 0; j < g.k; ++j) {
    const int s = __builtin_amdgcn_readlane(my_slot, j);
    if (s < 0) continue;
    const auto dst = buffer_rsrc(g.payload + static_cast<int64_t>(s) * g.row_bytes, static_cast<uint32_t>(g.row_bytes));
#pragma unroll
    for (int u = 0; u < kBf16Vec; ++u) {
      const int idx = v0 + u * kWave + lane;
      if (idx < nvec) __builtin_amdgcn_raw_buffer_store_b128(buf[u], dst, idx * 16, 0, NT ? kStoreNT : kStoreDevice);
    }
  }
}

// ---- quantising formats -------------------------------------------------------

__device__ __forceinline__ uint32_t lane_absmax(const float (&f)[kLE]) {
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < kLE; ++i) am = max(am, __float_as_uint(f[i]) & 0x7FFFFFFFu);
  return am;
}

// ---- FP8 E4M3, one fp32 scale per 1x128 block -------------------------------
template <bool NT>
__device__ void slab_fp8(const DispatchArgs &g, int slab, int my_slot, const RawSlab &r) {
  const int lane = lane_id();
  float f[kQC][kLE];
#pragma unroll
  for (int c = 0; c < kQC; ++c) unpack_lane(r, c, f[c]);
  uint32_t w[kQC][kLE / 4];
  float sc[kQC];
#pragma unroll
  for (int c = 0; c < kQC; ++c) {
    // one 1x128 block = 128/kLE lanes: a 16-lane row (kLE 8) or 8 lanes (16)
    uint32_t am = quad_max(lane_absmax(f[c]));
    am = max(am, dpp<kRowHalfMirror>(am));
    if (kLE == 8) am = max(am, dpp<kRowMirror>(am));
    const float s = __uint_as_float(am) / 448.0f;
    // codes E4M3(fl32(x / s)): a reciprocal and one fused correction per value
    // (exact for every block maximum >= 2^-103), IEEE division below that,
    // zero codes for an all-zero block; hardware conversion in pairs
    float q[kLE];
    if (am >= kFp8FastMinBits) {
      const float r = 1.0f / s;
#pragma unroll
      for (int i = 0; i < kLE; ++i) q[i] = fp8_quotient_fast(f[c][i], s, r);
    } else if (am != 0) {
#pragma unroll
      for (int i = 0; i < kLE; ++i) q[i] = f[c][i] / s;
    } else {
#pragma unroll
      for (int i = 0; i < kLE; ++i) q[i] = 0.0f;
    }
#pragma unroll
    for (int qd = 0; qd < kLE / 4; ++qd)
      w[c][qd] = e4m3_pair_hw(q[4 * qd], q[4 * qd + 1]) | (e4m3_pair_hw(q[4 * qd + 2], q[4 * qd + 3]) << 16);
    sc[c] = s;
  }
  for (int j = 0; j < g.k; ++j) {
    const int d = __builtin_amdgcn_readlane(my_slot, j);
    if (d < 0) continue;
    uint8_t *prow = g.payload + static_cast<int64_t>(d) * g.row_bytes;
    float *srow = reinterpret_cast<float *>(g.scales + static_cast<int64_t>(d) * g.scale_bytes);
#pragma unroll
    for (int c = 0; c < kQC; ++c) {
      const int elem = slab * kQuantSlab + c * kWave * kLE + lane * kLE;
      if (elem < g.h) {
        if (kLE == 16)
          store<NT>(reinterpret_cast<u32x4 *>(prow + elem), u32x4{w[c][0], w[c][1], w[c][2], w[c][3]});
        else
          store<NT>(reinterpret_cast<u32x2 *>(prow + elem), u32x2{w[c][0], w[c][1]});
        if ((lane & (128 / kLE - 1)) == 0) store<NT>(srow + elem / 128, sc[c]);
      }
    }
  }
}

// ---- MX-FP4: E2M1 codes, one E8M0 scale per 32 values -----------------------
template <bool NT>
__device__ void slab_mx(const DispatchArgs &g, int slab, int my_slot, const RawSlab &r) {
  const int lane = lane_id();
  float f[kQC][kLE];
#pragma unroll
  for (int c = 0; c < kQC; ++c) unpack_lane(r, c, f[c]);
  uint32_t w[kQC][kLE / 8];
  uint8_t sbyte[kQC];
#pragma unroll
  for (int c = 0; c < kQC; ++c) {
    // one 32-value block = 32/kLE lanes: a quad (kLE 8) or a lane pair (16)
    uint32_t am = lane_absmax(f[c]);
    am = max(am, dpp<kQuadSwap1>(am));
    if (kLE == 8) am = max(am, dpp<kQuadSwap2>(am));
    const int X = mx_exponent(am);
    const float mul = __uint_as_float(static_cast<uint32_t>(127 - X) << 23);  // 2^-X
    const bool hw = ballot(nan_bits(am)) == 0;  // hardware codes unless a NaN
#pragma unroll
    for (int qd = 0; qd < kLE / 8; ++qd) {
      float q[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = f[c][8 * qd + i] * mul;
      const uint32_t v = e2m1_lane8(q, hw);
      w[c][qd] = am == 0 ? 0u : v;
    }
    sbyte[c] = am == 0 ? 0 : static_cast<uint8_t>(X + 127);
  }
  for (int j = 0; j < g.k; ++j) {
    const int d = __builtin_amdgcn_readlane(my_slot, j);
    if (d < 0) continue;
    uint8_t *prow = g.payload + static_cast<int64_t>(d) * g.row_bytes;
    uint8_t *srow = g.scales + static_cast<int64_t>(d) * g.scale_bytes;
#pragma unroll
    for (int c = 0; c < kQC; ++c) {
      const int elem = slab * kQuantSlab + c * kWave * kLE + lane * kLE;
      if (elem < g.h) {
        if (kLE == 16)
          store<NT>(reinterpret_cast<u32x2 *>(prow + elem / 2), u32x2{w[c][0], w[c][1]});
        else
          store<NT>(reinterpret_cast<uint32_t *>(prow + elem / 2), w[c][0]);
        if ((lane & (32 / kLE - 1)) == 0) store<NT>(srow + elem / 32, sbyte[c]);
      }
    }
  }
}

// ---- NVFP4: E2M1 codes, one E4M3 scale per 16 values, fp32 global scale -----
// (Mojo ep.dispatch_async.block.scaled.nv struct: NVFP4 transfer with global
// input scales.)  Per 16-value block (a lane pair): sf = E4M3(fl32(amax / 6)
// * gs), saturated at 448 (the hardware conversion is exact below 464), and
// codes E2M1(fl32(fl32(x * gs) / value(sf))) with IEEE division.
template <bool NT>
__device__ void slab_nvfp4(const DispatchArgs &g, int slab, int my_slot, const RawSlab &r) {
  static_assert(kLE == 8 && kQC == 1, "a 16-value block is one lane pair");
  const int lane = lane_id();
  const int elem = slab * kQuantSlab + lane * kLE;
  float f[kLE];
  unpack_lane(r, 0, f);
  uint32_t am = lane_absmax(f);
  am = max(am, dpp<kQuadSwap1>(am));
  const float gs = *g.gscale;
  const float ts = (__uint_as_float(am) / 6.0f) * gs;
  const uint32_t sf = e4m3_pair_hw(fminf(fmaxf(ts, -448.0f), 448.0f), 0.0f) & 0xFFu;
  const float sfv = e4m3_magnitude(sf & 0x7Fu);
  // hardware codes unless a NaN value or a global scale that makes one
  const bool hw = ballot(nan_bits(am)) == 0 && fabsf(gs) <= 0x1.fffffep127f;
  uint32_t w = 0;
  if (sfv != 0.0f) {
    float q[kLE];
#pragma unroll
    for (int i = 0; i < kLE; ++i) q[i] = (f[i] * gs) / sfv;
    w = e2m1_lane8(q, hw);
  }
  for (int j = 0; j < g.k; ++j) {
    const int d = __builtin_amdgcn_readlane(my_slot, j);
    if (d < 0) continue;
    if (elem < g.h) {
      uint8_t *prow = g.payload + static_cast<int64_t>(d) * g.row_bytes;
      uint8_t *srow = g.scales + static_cast<int64_t>(d) * g.scale_bytes;
      store<NT>(reinterpret_cast<uint32_t *>(prow + elem / 2), w);
      if ((lane & 1) == 0) store<NT>(srow + elem / 16, static_cast<uint8_t>(sf));
    }
  }
}

// ---- gated copies: row slot[t][j] holds encode(fl32(w[t][j] * x[t])) -------
// (DeepSpeed v0.19.4 function index, page 15: the entry on scaling token
// rows by their router scores ahead of the experts.)  The slab is read
// once; every copy is multiplied by its own gate and encoded on its own.  A
// block maximum of the products needs no new reduction: rounding is
// monotone, so max |fl32(w x_i)| = fl32(|w| max |x_i|).

__device__ __forceinline__ float bcast(float v, int j) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), j));
}

template <bool NT>
__device__ void slab_bf16_gated(const DispatchArgs &g, int slab, int my_slot, const RawSlab &r) {
  const int lane = lane_id();
  const int nvec = g.h / 8;
  const int v0 = slab * kWave * kBf16Vec;
  const float my_w = r.w;
  const u32x4 *buf = r.v;
  for (int j = 0; j < g.k; ++j) {
    const int s = __builtin_amdgcn_readlane(my_slot, j);
    if (s < 0) continue;
    const float wj = bcast(my_w, j);
    u32x4 *dst = reinterpret_cast<u32x4 *>(g.payload + static_cast<int64_t>(s) * g.row_bytes);
#pragma unroll
    for (int u = 0; u < kBf16Vec; ++u) {
      const int idx = v0 + u * kWave + lane;
      if (idx < nvec) {
        uint4 r4;
        r4.x = buf[u].x; r4.y = buf[u].y; r4.z = buf[u].z; r4.w = buf[u].w;
        float f[8];
        unpack8(r4, f);
        u32x4 o;
        o.x = f32_to_bf16(wj * f[0]) | (f32_to_bf16(wj * f[1]) << 16);
        o.y = f32_to_bf16(wj * f[2]) | (f32_to_bf16(wj * f[3]) << 16);
        o.z = f32_to_bf16(wj * f[4]) | (f32_to_bf16(wj * f[5]) << 16);
        o.w = f32_to_bf16(wj * f[6]) | (f32_to_bf16(wj * f[7]) << 16);
        store<NT>(dst + idx, o);
      }
    }
  }
}

// FP8: per copy s = fl32(fl32(|w| amax) / 448) and codes E4M3(fl32(v / s)),
// v = fl32(w x), with IEEE division (the reciprocal shortcut of the ungated
// path is exact only for the bf16 values it was checked on).
template <bool NT>
__device__ void slab_fp8_gated(const DispatchArgs &g, int slab, int my_slot, const RawSlab &r) {
  static_assert(kQC == 1, "gated encoders take one chunk per wave");
  const int lane = lane_id();
  const float my_w = r.w;
  const int elem = slab * kQuantSlab + lane * kLE;
  float f[kLE];
  unpack_lane(r, 0, f);
  uint32_t am = quad_max(lane_absmax(f));
  am = max(am, dpp<kRowHalfMirror>(am));
  if (kLE == 8) am = max(am, dpp<kRowMirror>(am));
  const float amax = __uint_as_float(am);
  for (int j = 0; j < g.k; ++j) {
    const int d = __builtin_amdgcn_readlane(my_slot, j);
    if (d < 0) continue;
    const float wj = bcast(my_w, j);
    const float amj = fabsf(wj) * amax;
    const float s = amj / 448.0f;  // 0 for a zero block, or when amj / 448 underflows
    uint32_t w4[kLE / 4];
    if (s != 0.0f) {
      float q[kLE];
#pragma unroll
      for (int i = 0; i < kLE; ++i) q[i] = (wj * f[i]) / s;
#pragma unroll
      for (int qd = 0; qd < kLE / 4; ++qd)
        w4[qd] = e4m3_pair_hw(q[4 * qd], q[4 * qd + 1]) | (e4m3_pair_hw(q[4 * qd + 2], q[4 * qd + 3]) << 16);
    } else {
#pragma unroll
      for (int qd = 0; qd < kLE / 4; ++qd) w4[qd] = 0u;
    }
    if (elem < g.h) {
      uint8_t *prow = g.payload + static_cast<int64_t>(d) * g.row_bytes;
      float *srow = reinterpret_cast<float *>(g.scales + static_cast<int64_t>(d) * g.scale_bytes);
      if (kLE == 16)
        store<NT>(reinterpret_cast<u32x4 *>(prow + elem), u32x4{w4[0], w4[1], w4[2], w4[3]});
      else
        store<NT>(reinterpret_cast<u32x2 *>(prow + elem), u32x2{w4[0], w4[1]});
      if ((lane & (128 / kLE - 1)) == 0) store<NT>(srow + elem / 128, s);
    }
  }
}

// MX-FP4: per copy X from fl32(|w| amax), codes E2M1(fl32(w x) * 2^-X).
template <bool NT>
__device__ void slab_mx_gated(const DispatchArgs &g, int slab, int my_slot, const RawSlab &r) {
  static_assert(kQC == 1, "gated encoders take one chunk per wave");
  const int lane = lane_id();
  const float my_w = r.w;
  const int elem = slab * kQuantSlab + lane * kLE;
  float f[kLE];
  unpack_lane(r, 0, f);
  uint32_t am = lane_absmax(f);
  am = max(am, dpp<kQuadSwap1>(am));
  if (kLE == 8) am = max(am, dpp<kQuadSwap2>(am));
  const float amax = __uint_as_float(am);
  const bool finite_x = ballot(nan_bits(am)) == 0;
  for (int j = 0; j < g.k; ++j) {
    const int d = __builtin_amdgcn_readlane(my_slot, j);
    if (d < 0) continue;
    const float wj = bcast(my_w, j);
    const float amj = fabsf(wj) * amax;
    const uint32_t ab = __float_as_uint(amj);
    const int X = mx_exponent(ab);
    const float mul = __uint_as_float(static_cast<uint32_t>(127 - X) << 23);  // 2^-X
    // hardware codes unless a NaN value, or a gate that makes one
    const bool hw = finite_x && fabsf(wj) <= 0x1.fffffep127f;
    uint32_t w8[kLE / 8];
#pragma unroll
    for (int qd = 0; qd < kLE / 8; ++qd) {
      float q[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = (wj * f[8 * qd + i]) * mul;
      const uint32_t v = e2m1_lane8(q, hw);
      w8[qd] = ab == 0 ? 0u : v;
    }
    if (elem < g.h) {
      uint8_t *prow = g.payload + static_cast<int64_t>(d) * g.row_bytes;
      uint8_t *srow = g.scales + static_cast<int64_t>(d) * g.scale_bytes;
      if (kLE == 16)
        store<NT>(reinterpret_cast<u32x2 *>(prow + elem / 2), u32x2{w8[0], w8[1]});
      else
        store<NT>(reinterpret_cast<uint32_t *>(prow + elem / 2), w8[0]);
      if ((lane & (32 / kLE - 1)) == 0)
        store<NT>(srow + elem / 32, static_cast<uint8_t>(ab == 0 ? 0 : X + 127));
    }
  }
}

// ---- zero fill of one packed row (payload and scales) -----------------------
template <bool NT>
__device__ void zero_row(const DispatchArgs &g, int64_t r) {
  const int lane = lane_id();
  u32x4 *p = reinterpret_cast<u32x4 *>(g.payload + r * g.row_bytes);
  const int nvec = static_cast<int>(g.row_bytes / 16);
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int i = lane; i < nvec; i += kWave) store<NT>(p + i, z);
  if (g.scale_bytes) {
    uint8_t *s = g.scales + r * g.scale_bytes;
    if ((g.scale_bytes & 3) == 0) {
      uint32_t *s4 = reinterpret_cast<uint32_t *>(s);
      for (int i = lane; i < g.scale_bytes / 4; i += kWave) store<NT>(s4 + i, 0u);
    } else {
      for (int i = lane; i < g.scale_bytes; i += kWave) store<NT>(s + i, static_cast<uint8_t>(0));
    }
  }
}

// Workgroups are handed to the 8 XCDs round-robin (block b runs on XCD
// b % 8), each XCD with its own L2.  Renumbering the token range so that
// consecutive logical blocks share an XCD keeps all waves of a token on one
// L2, where the partial-line writes of its scale rows (16 bytes per wave and
// copy) merge before they reach memory.
constexpr int kXcds = 8;

__device__ __forceinline__ int xcd_local_block(int b, int nblocks) {
  const int per = nblocks / kXcds, extra = nblocks % kXcds;
  const int x = b % kXcds, pos = b / kXcds;
  return x * per + min(x, extra) + pos;
}

// zero rows after the used part of every segment, by `blk` of tail_blocks
template <bool NT>
__device__ void zero_tails(const DispatchArgs &g, int blk, int wave) {
  const int64_t stride = static_cast<int64_t>(g.tail_blocks) * kWaves;
  for (int d = 0; d < g.nseg; ++d) {
    const int64_t u = g.seg_used ? g.seg_used[d] : g.used_rows;
    const int64_t used = max(min(u, g.seg_rows), int64_t{0});
    const int64_t base = d * g.seg_rows;
    for (int64_t r = used + static_cast<int64_t>(blk) * kWaves + wave; r < g.seg_rows; r += stride)
      zero_row<NT>(g, base + r);
  }
}

// Encode a loaded slab and store it to the token's k packed rows.
template <int FMT, bool NT, bool GATED>
__device__ __forceinline__ void emit_slab(const DispatchArgs &g, int slab, int my_slot, const RawSlab &r) {
  if (GATED) {  // not instantiated for NVFP4 (the host rejects it)
    if (FMT == MOE_FMT_BF16) slab_bf16_gated<NT>(g, slab, my_slot, r);
    else if (FMT == MOE_FMT_FP8_E4M3_B128) slab_fp8_gated<NT>(g, slab, my_slot, r);
    else slab_mx_gated<NT>(g, slab, my_slot, r);
  } else {
    if (FMT == MOE_FMT_BF16) slab_bf16<NT>(g, slab, my_slot, r);
    else if (FMT == MOE_FMT_FP8_E4M3_B128) slab_fp8<NT>(g, slab, my_slot, r);
    else if (FMT == MOE_FMT_NVFP4_B16) slab_nvfp4<NT>(g, slab, my_slot, r);
    else slab_mx<NT>(g, slab, my_slot, r);
  }
}

// The three workgroup ranges of a dispatch launch: token slabs, pad rows,
// zero tails.  `blk` < token_blocks + pad_blocks + tail_blocks.
template <int FMT, bool NT, bool GATED>
__device__ __forceinline__ void dispatch_body(const DispatchArgs &g, int blk, int wave) {
  if (MOE_TAIL_FIRST) {
    if (blk < g.tail_blocks) {
      zero_tails<NT || MOE_TAIL_NT>(g, blk, wave);
      return;
    }
    blk -= g.tail_blocks;
  }
  if (blk < g.token_blocks) {
    if (FMT != MOE_FMT_BF16) blk = xcd_local_block(blk, g.token_blocks);
    const int q = blk * kWaves + wave;  // the grid size keeps q within int
    const int t = q / g.slabs;
    if (t >= g.n) return;
    const int slab = q - t * g.slabs;
    // the token's slots (one per lane) and the slab: one round trip
    const int my_slot = lane_slot(g, t, lane_id());
    const RawSlab r = load_slab<FMT, GATED>(g, t, slab);
    emit_slab<FMT, NT, GATED>(g, slab, my_slot, r);
    return;
  }
  blk -= g.token_blocks;
  if (blk < g.pad_blocks) {
    const int q = blk * kWaves + wave;
    const int e = q / g.pad_groups;
    if (e >= g.e) return;
    const int grp = q - e * g.pad_groups;
    // unused rows [offsets[e] + counts[e], offsets[e+1]); with a fixed
    // capacity counts[e] may exceed the expert's rows (int64: no overflow);
    // never outside the buffer, whatever the plan arrays hold
    const int64_t hi = min(static_cast<int64_t>(g.offsets[e + 1]), g.r_max);
    const int64_t lo = max(min(static_cast<int64_t>(g.offsets[e]) + g.counts[e], hi), int64_t{0});
    const int64_t r0 = lo + static_cast<int64_t>(grp) * kPadRowsPerWave;
    const int64_t r1 = min(r0 + kPadRowsPerWave, hi);
    for (int64_t r = r0; r < r1; ++r) zero_row<NT>(g, r);
    return;
  }
  blk -= g.pad_blocks;
  if (!MOE_TAIL_FIRST) zero_tails<NT || MOE_TAIL_NT>(g, blk, wave);
}

template <int FMT, bool NT, bool GATED>
__global__ __launch_bounds__(kThreads) void dispatch_kernel(DispatchArgs g) {
  dispatch_body<FMT, NT, GATED>(g, blockIdx.x, __builtin_amdgcn_readfirstlane(threadIdx.x / kWave));
}

// ---- plan and dispatch in one launch ---------------------------------------
// Every workgroup issues the loads of the IDs and of its token slabs, then
// computes in LDS the part of the plan it needs (small_plan.hpp) while the
// slabs arrive, and encodes and stores its slabs with the slots it found.
// Small mode (at most kSmallPairs pairs): the plan from all the IDs.  Tiled
// mode (after plan_count_kernel): the plan from the tile histograms and the
// IDs of the workgroup's own count tile.  The loads are bounds-checked
// buffer loads with no branch around them, so the plan waits for its IDs
// alone and runs while the slabs are still in flight.
// Workgroup 0 writes the counts, offsets, table and status; the wave that
// holds slab 0 of a token writes that token's slots and packed_src rows;
// all workgroups stride over the pad and tail rows of packed_src; the
// workgroups past the token range zero pad and tail rows as in dispatch.
struct PlanDispatchArgs {
  DispatchArgs d;       // plan pointers are replaced by LDS in the kernel
  SmallPlanArgs sp;
  int32_t *counts, *offsets, *dest_counts, *slot, *packed_src;
  uint32_t *table, *status;
  uint32_t h;           // elements per row, for the table
  int r_max;
  int dispatch_blocks;  // workgroups of the three dispatch ranges
};

static_assert(kThreads == kSmallThreads, "one small plan per dispatch workgroup");
static_assert(MOE_TAIL_FIRST == 0, "the one-launch kernel places the token workgroups first");

// Workgroup 0's share of a one-launch plan: counts, offsets, the (4, EP)
// table and the status, from the plan in LDS.
template <bool TILED>
__device__ void write_plan_arrays(const PlanDispatchArgs &g, const SmallPlanLds &s, uint32_t fl) {
  const int E = g.sp.e, tid = threadIdx.x;
  for (int e = tid; e < E; e += kThreads) {
    g.counts[e] = s.cnt[e];
    g.offsets[e] = s.off[e];
  }
  if (tid == 0) {
    g.offsets[E] = s.off[E];
    // tiled: the counting kernel cleared the status word, and other
    // workgroups may OR BAD_PLAN into it; one launch: written here alone
    if constexpr (TILED)
      atomicOr(g.status, fl | (s.off[E] < 0 || s.off[E] > g.r_max ? MOE_STATUS_BAD_PLAN : 0u));
    else
      *g.status = fl;
  }
  const int L = g.sp.l;
  for (int rk = tid; rk < g.sp.ep; rk += kThreads) {
    const int lo = rk * L, hi = lo + L;
    const int S = s.cpre[hi] - s.cpre[lo];
    g.dest_counts[rk] = S;
    g.table[rk] = static_cast<uint32_t>(S) * g.h;
    g.table[g.sp.ep + rk] = static_cast<uint32_t>(s.cpre[lo]) * g.h;
    g.table[2 * g.sp.ep + rk] = static_cast<uint32_t>(s.off[hi] - s.off[lo]) * g.h;
    g.table[3 * g.sp.ep + rk] = static_cast<uint32_t>(s.off[lo]) * g.h;
  }
}

template <int FMT, bool NT, bool GATED, bool TILED>
__global__ __launch_bounds__(kThreads) void plan_dispatch_kernel(PlanDispatchArgs g) {
  extern __shared__ int smem[];
  const int E = g.sp.e, k = g.sp.k;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const DispatchArgs &d = g.d;
  const SmallPlanLds s = small_plan_lds(smem, E);

  const bool tok = b < d.token_blocks;
  const int blk = tok && FMT != MOE_FMT_BF16 ? xcd_local_block(b, d.token_blocks) : b;
  // the workgroup's own pairs: every pair of its (at most kWaves) tokens
  int p0 = 0, p1 = 0;
  if (tok) {
    const int t0 = (blk * kWaves) / d.slabs;
    const int t1 = min(g.sp.n - 1, (blk * kWaves + kWaves - 1) / d.slabs);
    if (t0 < g.sp.n) {
      p0 = t0 * k;
      p1 = (t1 + 1) * k;
    }
  }
  // tiled: pairs from the start of the count tile that holds p0
  const int c0 = TILED ? (p0 / k) / g.sp.tile_tokens : 0;
  const int tlo = c0 * g.sp.tile_tokens * k;

  // the IDs (and histograms), then this wave's token slab: all loads in
  // flight during the plan
  int v[kSmallLoads];
  TileLoads tl;
  if constexpr (TILED)
    tile_plan_load(g.sp, tlo, p1 - tlo, tl);
  else
    small_plan_load(g.sp, v);
  const int q = blk * kWaves + wave;  // the grid size keeps q within int
  const int t = tok ? q / d.slabs : 0;
  const int slab = q - t * d.slabs;
  const bool live = tok && t < g.sp.n;
  const RawSlab r = load_slab_buf<FMT, GATED>(d, t, slab, live);
  // the plan waits for its own loads only: the slab may still be in flight
  if constexpr (TILED) tile_plan_stage(g.sp, s, tl, p1 - tlo);
  // only workgroup 0 reports the status
  uint32_t fl;
  if constexpr (TILED)
    fl = tile_plan(g.sp, s, tl, tlo, p0, c0, b == 0);
  else
    fl = small_plan(g.sp, s, v, p0, b == 0);

  if (b == 0) write_plan_arrays<TILED>(g, s, fl);
  // the wave's own token's slots, found by the wave itself; they and the
  // token's packed_src rows are written by the wave of its slab 0.  A pair
  // the histograms do not account for (tiled mode, a workspace that does
  // not count these IDs) is left unplaced and reported.
  int my_slot = live && lane < k ? own_slot(s, TILED ? tlo : 0, p0, t * k + lane, g.r_max, g.sp.ecap) : -1;
  const bool bad = my_slot == kBadSlot;
  if (bad) my_slot = -1;
  if (live && slab == 0) {
    if (lane < k) {
      g.slot[t * k + lane] = my_slot;
      if (my_slot >= 0) g.packed_src[my_slot] = t;
    }
    if (TILED && ballot(bad) && lane == 0) atomicOr(g.status, MOE_STATUS_BAD_PLAN);
  }
  // packed_src = -1 on the unused rows of each expert and on the tail, never
  // outside the buffer
  const int stride = gridDim.x * kThreads;
  const int per = g.sp.ecap > 0 ? g.sp.ecap : g.sp.a - 1;  // unused rows an expert, at most
  for (int qq = b * kThreads + tid; qq < E * per; qq += stride) {
    const int e = qq / per;
    const int64_t row = static_cast<int64_t>(s.off[e]) + s.cnt[e] + (qq - e * per);
    if (row < s.off[e + 1] && row >= 0 && row < g.r_max) g.packed_src[row] = -1;
  }
  for (int row = max(s.off[E], 0) + b * kThreads + tid; row < g.r_max; row += stride)
    g.packed_src[row] = -1;

  if (live) {
    emit_slab<FMT, NT, GATED>(d, slab, my_slot, r);
  } else if (!tok && b < g.dispatch_blocks) {
    // pad and tail ranges, reading the plan from LDS
    DispatchArgs dp = d;
    dp.counts = s.cnt;
    dp.offsets = s.off;
    dp.seg_used = s.off + E;
    dispatch_body<FMT, NT, GATED>(dp, b, wave);
  }
}

// ---- one launch without padding: slots by counting smaller keys --------------
// With A = 1 the packed row of a valid pair is the number of valid pairs
// ahead of it in (expert, flat pair index) order: the stable counting sort
// of the plan, whose offsets are then the unpadded cumsum.  As 21-bit keys
// (expert << 11 | pair index; masked and invalid pairs get a key above
// every valid one) the row of pair p is the count of keys below p's key,
// which also ranks the equal IDs of one token.  A token workgroup counts
// these for its own pairs (those of its at most kWaves tokens) without LDS
// atomics (about 64 cycles each on this chip) and with one barrier: each
// wave holds a quarter of the keys (ID u * 256 + tid in register u), counts
// for every own pair the keys below it in that quarter with one ballot per
// register, and stores the count; after the barrier a pair's row is the sum
// of the four counts.  Workgroup 0 builds the whole plan in LDS all the
// same, for the counts, offsets, table, status and the packed_src tail,
// and stores no payload; the token workgroups are 1 .. token_blocks, then
// the tail workgroups.
constexpr uint32_t kNoKey = 0xFFFFFFFFu;
constexpr int kOwnMax = kWaves * kMaxTopK;  // own pairs of a workgroup, at most
static_assert(kSmallPairs <= 2048 && kMaxExperts <= 1024, "keys: 11 index bits, 10 expert bits");
static_assert(kOwnMax <= 4 * kWave, "own keys: four registers a lane");

// Key registers per thread (IDs u * kThreads + tid) for a one-launch problem.
__host__ __device__ constexpr int rank_regs(int64_t npairs) {
  return npairs <= kThreads ? 1 : npairs <= 4 * kThreads ? 4 : kSmallPairs / kThreads;
}

template <int FMT, bool NT, bool GATED, int NR>
__global__ __launch_bounds__(kThreads) void plan_dispatch_rank_kernel(PlanDispatchArgs g) {
  extern __shared__ int smem[];
  __shared__ int s_cnt[kWaves][kOwnMax];  // per wave: keys below each own pair
  __shared__ int s_used[kWaves];
  const int E = g.sp.e, k = g.sp.k;
  const int np = g.sp.n * k;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  if (b == 0) {
    const SmallPlanLds s = small_plan_lds(smem, E);
    int v[kSmallLoads];
    small_plan_load(g.sp, v);
    const uint32_t fl = small_plan(g.sp, s, v, 0, true);
    write_plan_arrays<false>(g, s, fl);
    for (int row = max(s.off[E], 0) + tid; row < g.r_max; row += kThreads) g.packed_src[row] = -1;
    return;
  }
  const DispatchArgs &d = g.d;
  const int bb = b - 1;
  const bool tok = bb < d.token_blocks;
  const int blk = tok && FMT != MOE_FMT_BF16 ? xcd_local_block(bb, d.token_blocks) : bb;
  // (token, slab) of this wave and the workgroup's own pairs (every pair of
  // its tokens).  With at least kWaves slabs a token, a token has
  // ceil(slabs / kWaves) workgroups of its own (token_blocks = N times
  // that), so the own pairs are the token's k; otherwise consecutive waves
  // take consecutive (token, slab) items and a workgroup spans up to
  // kWaves tokens.
  int t, slab, p0 = 0, p1 = 0;
  if (d.slabs >= kWaves) {
    const int wpt = (d.slabs + kWaves - 1) / kWaves;
    t = tok ? blk / wpt : 0;
    slab = (blk - t * wpt) * kWaves + wave;
    if (tok && t < g.sp.n) {
      p0 = t * k;
      p1 = p0 + k;
    }
  } else {
    const int q = blk * kWaves + wave;  // the grid size keeps q within int
    t = tok ? q / d.slabs : 0;
    slab = q - t * d.slabs;
    if (tok) {
      const int t0 = (blk * kWaves) / d.slabs;
      const int t1 = min(g.sp.n - 1, (blk * kWaves + kWaves - 1) / d.slabs);
      if (t0 < g.sp.n) {
        p0 = t0 * k;
        p1 = (t1 + 1) * k;
      }
    }
  }
  const int own_n = p1 - p0;  // <= kOwnMax
  const bool live = tok && t < g.sp.n && slab < d.slabs;

  // this thread's IDs, the workgroup's own IDs (pair p0 + r * 64 + lane in
  // register r) and the slab: bounds-checked loads, all in flight together
  const auto ids = buffer_rsrc(g.sp.ids, static_cast<uint32_t>(np) * 4u);
  int x[NR];
#pragma unroll
  for (int u = 0; u < NR; ++u)
    x[u] = __builtin_amdgcn_raw_buffer_load_b32(ids, (u * kThreads + tid) * 4, 0, kLoadDefault);
  const auto own_ids = buffer_rsrc(g.sp.ids + p0, 4u * static_cast<uint32_t>(own_n));
  int o[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) o[r] = __builtin_amdgcn_raw_buffer_load_b32(own_ids, (r * kWave + lane) * 4, 0, kLoadDefault);
  const auto tok_ids = buffer_rsrc(g.sp.ids + (live ? t * k : 0), live ? 4u * static_cast<uint32_t>(k) : 0u);
  const int own = __builtin_amdgcn_raw_buffer_load_b32(tok_ids, lane * 4, 0, kLoadDefault);  // pair (t, lane)
  const RawSlab raw = load_slab_buf<FMT, GATED>(d, t, slab, live);

  uint32_t key[NR];
  int used = 0;  // valid pairs among this wave's quarter
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    const int i = u * kThreads + tid;
    const bool ok = i < np && x[u] >= 0 && x[u] < E;
    key[u] = ok ? (static_cast<uint32_t>(x[u]) << 11) | static_cast<uint32_t>(i) : kNoKey;
    used += __popcll(ballot(ok));
  }
  uint32_t okey[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int j = r * kWave + lane, p = p0 + j;
    okey[r] = j < own_n && o[r] >= 0 && o[r] < E ? (static_cast<uint32_t>(o[r]) << 11) | static_cast<uint32_t>(p) : kNoKey;
  }
  // keys of this quarter below each own key: four own keys an iteration,
  // four independent chains of ballots (counts for lanes past own_n are
  // computed and not used)
  int cnt[4] = {0, 0, 0, 0};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int jn = min(own_n - r * kWave, kWave);
    for (int jj = 0; jj < jn; jj += 4) {
      uint32_t kq[4];
      int c[4] = {0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) kq[i] = __builtin_amdgcn_readlane(okey[r], min(jj + i, kWave - 1));
#pragma unroll
      for (int u = 0; u < NR; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) c[i] += __popcll(ballot(key[u] < kq[i]));
#pragma unroll
      for (int i = 0; i < 4; ++i) cnt[r] = lane == jj + i ? c[i] : cnt[r];
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (r * kWave + lane < own_n) s_cnt[wave][r * kWave + lane] = cnt[r];
  if (lane == 0) s_used[wave] = used;
  __syncthreads();

  // the own token's pairs (lane j < k): the row is the sum of the counts
  int my_slot = -1;
  if (live && lane < k && own >= 0 && own < E) {
    const int j = t * k + lane - p0;  // < own_n
    int row = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) row += s_cnt[w][j];
    if (row >= 0 && row < g.r_max) my_slot = row;
  }
  if (live && slab == 0 && lane < k) {
    g.slot[t * k + lane] = my_slot;
    if (my_slot >= 0) g.packed_src[my_slot] = t;
  }
  if (live) {
    emit_slab<FMT, NT, GATED>(d, slab, my_slot, raw);
  } else if (!tok && bb < g.dispatch_blocks) {
    // zero tail rows after R_used (no pad rows without padding)
    int u_all = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) u_all += s_used[w];
    DispatchArgs dp = d;
    dp.seg_used = nullptr;
    dp.used_rows = u_all;
    dispatch_body<FMT, NT, GATED>(dp, bb, wave);
  }
}

template <int FMT>
void launch_fmt(const DispatchArgs &g, int grid, hipStream_t stream) {
  if (FMT != MOE_FMT_NVFP4_B16 && g.w)
    dispatch_kernel<FMT, MOE_DISPATCH_NT_STORE != 0, FMT != MOE_FMT_NVFP4_B16><<<grid, kThreads, 0, stream>>>(g);
  else
    dispatch_kernel<FMT, MOE_DISPATCH_NT_STORE != 0, false><<<grid, kThreads, 0, stream>>>(g);
}

}  // namespace

namespace {

// Fields that depend only on the problem (format, sizes, token waves).
DispatchArgs base_args(const moe_problem &p, int64_t tokens, const int32_t *slot,
                       const uint16_t *hidden, void *payload, void *scales) {
  DispatchArgs g{};
  g.x = hidden;
  g.slot = slot;
  g.payload = static_cast<uint8_t *>(payload);
  g.scales = static_cast<uint8_t *>(scales);
  g.n = tokens;
  g.k = p.top_k;
  g.h = p.hidden;
  g.e = p.n_experts;
  if (p.fmt == MOE_FMT_BF16) {
    g.row_bytes = 2 * static_cast<int64_t>(p.hidden);
    g.scale_bytes = 0;
  } else if (p.fmt == MOE_FMT_FP8_E4M3_B128) {
    g.row_bytes = p.hidden;
    g.scale_bytes = 4 * static_cast<int64_t>(p.hidden / 128);
  } else if (p.fmt == MOE_FMT_NVFP4_B16) {
    g.row_bytes = p.hidden / 2;
    g.scale_bytes = p.hidden / 16;
  } else {
    g.row_bytes = p.hidden / 2;
    g.scale_bytes = p.hidden / 32;
  }
  const int slab_elems = p.fmt == MOE_FMT_BF16 ? kWave * kBf16Vec * 8 : kQuantSlab;
  g.slabs = (p.hidden + slab_elems - 1) / slab_elems;
  g.token_blocks = static_cast<int>((tokens * g.slabs + kWaves - 1) / kWaves);
  g.pad_groups = 1;  // keeps the division in the kernel defined without pads
  return g;
}

hipError_t launch_args(const DispatchArgs &g, int fmt, hipStream_t stream) {
  const int grid = g.token_blocks + g.pad_blocks + g.tail_blocks;
  if (grid == 0) return hipSuccess;
  if (fmt == MOE_FMT_BF16) launch_fmt<MOE_FMT_BF16>(g, grid, stream);
  else if (fmt == MOE_FMT_FP8_E4M3_B128) launch_fmt<MOE_FMT_FP8_E4M3_B128>(g, grid, stream);
  else if (fmt == MOE_FMT_NVFP4_B16) launch_fmt<MOE_FMT_NVFP4_B16>(g, grid, stream);
  else launch_fmt<MOE_FMT_MXFP4_B32>(g, grid, stream);
  return hipGetLastError();
}

// Dispatch into one packed buffer, with the plan at `slot`, `counts` and
// `offsets` (device memory, or LDS inside the one-launch kernel).
DispatchArgs single_buffer_args(const moe_problem &p, const int32_t *slot, const int32_t *counts,
                                const int32_t *offsets, const uint16_t *hidden, const float *gates,
                                const float *gscale, void *payload, void *scales) {
  DispatchArgs g = base_args(p, p.n_tokens, slot, hidden, payload, scales);
  g.w = gates;
  g.gscale = gscale;
  g.counts = counts;
  g.offsets = offsets;
  g.r_max = max_rows(p);
  // unused rows per expert: fewer than A with padding, up to cap with a fixed
  // capacity (rows [offsets[e] + counts[e], offsets[e+1]) either way)
  const int64_t pad_span = p.expert_capacity > 0 ? p.expert_capacity : p.pad_multiple - 1;
  const int pad_groups = static_cast<int>((pad_span + kPadRowsPerWave - 1) / kPadRowsPerWave);
  g.pad_blocks = pad_groups == 0 ? 0 : (p.n_experts * pad_groups + kWaves - 1) / kWaves;
  if (pad_groups > 0) g.pad_groups = pad_groups;
  g.seg_used = offsets ? offsets + p.n_experts : nullptr;  // R_used
  g.nseg = 1;
  g.seg_rows = g.r_max;
  g.tail_blocks = (p.flags & MOE_FLAG_ZERO_TAIL) && g.r_max > 0 ? kTailBlocks : 0;
  return g;
}

template <int FMT, bool TILED>
void launch_plan_dispatch_fmt(const PlanDispatchArgs &g, int grid, size_t lds, hipStream_t stream) {
  constexpr bool kNT = MOE_DISPATCH_NT_STORE != 0;
  if (FMT != MOE_FMT_NVFP4_B16 && g.d.w)
    plan_dispatch_kernel<FMT, kNT, FMT != MOE_FMT_NVFP4_B16, TILED><<<grid, kThreads, lds, stream>>>(g);
  else
    plan_dispatch_kernel<FMT, kNT, false, TILED><<<grid, kThreads, lds, stream>>>(g);
}

template <int FMT, int NR>
void launch_plan_dispatch_rank_nr(const PlanDispatchArgs &g, int grid, size_t lds, hipStream_t stream) {
  constexpr bool kNT = MOE_DISPATCH_NT_STORE != 0;
  if (FMT != MOE_FMT_NVFP4_B16 && g.d.w)
    plan_dispatch_rank_kernel<FMT, kNT, FMT != MOE_FMT_NVFP4_B16, NR><<<grid, kThreads, lds, stream>>>(g);
  else
    plan_dispatch_rank_kernel<FMT, kNT, false, NR><<<grid, kThreads, lds, stream>>>(g);
}

template <int FMT>
void launch_plan_dispatch_rank_fmt(const PlanDispatchArgs &g, int nr, int grid, size_t lds, hipStream_t stream) {
  if (nr == 1) launch_plan_dispatch_rank_nr<FMT, 1>(g, grid, lds, stream);
  else if (nr == 4) launch_plan_dispatch_rank_nr<FMT, 4>(g, grid, lds, stream);
  else launch_plan_dispatch_rank_nr<FMT, kSmallPairs / kThreads>(g, grid, lds, stream);
}

void launch_plan_dispatch_rank(const PlanDispatchArgs &g, int fmt, int nr, int grid, size_t lds, hipStream_t stream) {
  if (fmt == MOE_FMT_BF16) launch_plan_dispatch_rank_fmt<MOE_FMT_BF16>(g, nr, grid, lds, stream);
  else if (fmt == MOE_FMT_FP8_E4M3_B128) launch_plan_dispatch_rank_fmt<MOE_FMT_FP8_E4M3_B128>(g, nr, grid, lds, stream);
  else if (fmt == MOE_FMT_NVFP4_B16) launch_plan_dispatch_rank_fmt<MOE_FMT_NVFP4_B16>(g, nr, grid, lds, stream);
  else launch_plan_dispatch_rank_fmt<MOE_FMT_MXFP4_B32>(g, nr, grid, lds, stream);
}

// Ballots a wave of the counting one-launch kernel makes: (own pairs of a
// workgroup, at most) x (key registers).  Above kRankSteps the workgroup-wide
// plan in LDS is faster.
constexpr int kRankSteps = 512;
int rank_steps(const moe_problem &p, int slabs) {
  // tokens a workgroup can touch: one with whole workgroups per token
  const int64_t span = slabs >= kWaves ? 1 : (kWaves - 2 + slabs) / slabs + 1;
  const int64_t tokens = p.n_tokens < span ? p.n_tokens : span;
  return static_cast<int>(tokens * p.top_k * rank_regs(p.n_tokens * p.top_k));
}

template <bool TILED>
void launch_plan_dispatch_any(const PlanDispatchArgs &g, int fmt, int grid, size_t lds, hipStream_t stream) {
  if (fmt == MOE_FMT_BF16) launch_plan_dispatch_fmt<MOE_FMT_BF16, TILED>(g, grid, lds, stream);
  else if (fmt == MOE_FMT_FP8_E4M3_B128) launch_plan_dispatch_fmt<MOE_FMT_FP8_E4M3_B128, TILED>(g, grid, lds, stream);
  else if (fmt == MOE_FMT_NVFP4_B16) launch_plan_dispatch_fmt<MOE_FMT_NVFP4_B16, TILED>(g, grid, lds, stream);
  else launch_plan_dispatch_fmt<MOE_FMT_MXFP4_B32, TILED>(g, grid, lds, stream);
}

}  // namespace

hipError_t launch_dispatch(const moe_problem &p, const moe_plan &plan, const uint16_t *hidden,
                           const float *gates, const float *gscale, void *payload, void *scales,
                           hipStream_t stream) {
  const DispatchArgs g = single_buffer_args(p, plan.slot, plan.expert_counts, plan.expert_offsets,
                                            hidden, gates, gscale, payload, scales);
  return launch_args(g, p.fmt, stream);
}

hipError_t launch_plan_dispatch(const moe_problem &p, const int32_t *ids, const moe_plan &plan,
                                const uint16_t *hidden, const float *gates, const float *gscale,
                                void *payload, void *scales, void *workspace, hipStream_t stream) {
  const PlanDispatchMode mode = plan_dispatch_mode(p);
  PlanDispatchArgs g{};
  // plan pointers are taken from LDS inside the kernel
  g.d = single_buffer_args(p, nullptr, nullptr, nullptr, hidden, gates, gscale, payload, scales);
  g.sp.ids = ids;
  g.sp.n = static_cast<int>(p.n_tokens);
  g.sp.k = p.top_k;
  g.sp.e = p.n_experts;
  g.sp.ep = p.ep;
  g.sp.a = p.pad_multiple;
  g.sp.ecap = static_cast<int>(p.expert_capacity);
  g.sp.l = p.n_experts / p.ep;
  g.sp.cap = p.recv_capacity;
  g.counts = plan.expert_counts;
  g.offsets = plan.expert_offsets;
  g.dest_counts = plan.dest_counts;
  g.slot = plan.slot;
  g.packed_src = plan.packed_src;
  g.table = plan.rank_table;
  g.status = plan.status;
  g.h = static_cast<uint32_t>(p.hidden);
  g.r_max = static_cast<int>(max_rows(p));
  g.dispatch_blocks = g.d.token_blocks + g.d.pad_blocks + g.d.tail_blocks;
  const int grid = max(g.dispatch_blocks, 1);  // N = 0 still writes the plan
  const size_t lds = small_plan_lds_bytes(p.n_experts);
  if (mode == PlanDispatchMode::kOneLaunch) {
    if (one_launch_direct(p) && rank_steps(p, g.d.slabs) <= kRankSteps) {  // workgroup 0 plans
      PlanDispatchArgs gr = g;
      if (g.d.slabs >= kWaves) {  // whole workgroups per token
        gr.d.token_blocks = static_cast<int>(p.n_tokens) * ((g.d.slabs + kWaves - 1) / kWaves);
        gr.dispatch_blocks = gr.d.token_blocks + gr.d.pad_blocks + gr.d.tail_blocks;
      }
      launch_plan_dispatch_rank(gr, p.fmt, rank_regs(p.n_tokens * p.top_k), gr.dispatch_blocks + 1, lds, stream);
    } else
      launch_plan_dispatch_any<false>(g, p.fmt, grid, lds, stream);
    return hipGetLastError();
  }
  // tiled: the counting kernel has written the histograms and fault bits
  const PlanGeom geo = plan_geometry(p);
  g.sp.hist = static_cast<const int32_t *>(workspace);
  g.sp.tflags = reinterpret_cast<const uint32_t *>(g.sp.hist + static_cast<int64_t>(geo.ntiles) * p.n_experts);
  g.sp.ntiles = geo.ntiles;
  g.sp.tile_tokens = geo.tile_tokens;
  launch_plan_dispatch_any<true>(g, p.fmt, grid, lds, stream);
  return hipGetLastError();
}

hipError_t launch_exchange_dispatch(const moe_problem &p, const moe_exchange &x, const uint16_t *hidden,
                                    const float *gates, const float *gscale, void *payload, void *scales,
                                    hipStream_t stream) {
  const int64_t tokens = p.n_tokens * p.ep;
  DispatchArgs g = base_args(p, tokens, x.recv_slot, hidden, payload, scales);
  g.w = gates;
  g.gscale = gscale;
  g.r_max = p.recv_capacity * p.ep;
  g.pad_blocks = 0;  // no per-expert padding in receive buffers
  g.seg_used = x.recv_rows;
  g.nseg = p.ep;
  g.seg_rows = p.recv_capacity;
  g.tail_blocks = g.r_max > 0 ? kTailBlocks : 0;
  return launch_args(g, p.fmt, stream);
}

}  // namespace moe
