/*
 * oracle.c -- plain, slow CPU oracle for MoE token dispatch and combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this file's library.  It shares no
 * source with the HIP library (no header, helper, table or constant): every
 * format rule below is written out again from its published definition.
 *
 * What it computes, step by step, with the passage each step follows
 * (pages are cited by title and section):
 *
 *   plan      counts per expert, padded exclusive cumsum offsets, the (4, EP)
 *             counts/displacements table, status bits, and a stable slot per
 *             (token, k) pair.
 *             - NKI permute_a2av API reference: description (rows packed at
 *               cumsum(send_counts) offsets, (4, EP) uint32 table in
 *               elements), :param packed_source_indices: (source rows in
 *               [0, N), destination-major), :param recv_capacity: (dropless
 *               bound N*min(top_k, L); duplicate IDs void it).
 *             - NeMo Automodel token_dispatcher API: dispatch_postprocess
 *               (rows permuted by expert plus tokens per expert),
 *               TokenDispatcherConfig.moe_router_expert_pad_multiple (pad each
 *               expert to a multiple), _indices_to_multihot (-1 = masked).
 *             - DeepSpeed v0.19.4 function index, page 15: SplitPlan entry
 *               (per-expert histogram viewed as an [ep_size, E_local] matrix).
 *   dispatch  each packed row holds its source token's hidden row, encoded in
 *             bf16, blockwise FP8-E4M3 (one fp32 amax/448 scale per 1x128
 *             block) or MX-FP4 (E2M1 codes, one E8M0 scale per 32 values);
 *             pad rows are all zero bytes.
 *             - Mojo shmem ep_comm module: Structs BF16TokenFormat,
 *               BlockwiseFP8TokenFormat, MXTokenFormat.
 *             - DeepSpeed v0.19.4 function index, page 15: the dispatch entry
 *               (an inverted routing map turns the copy into one gather) --
 *               this oracle uses exactly that gather form.
 *             - OCP 8-bit Floating Point Specification (E4M3 with no
 *               infinities, max 448) and OCP Microscaling Formats v1.0 (E2M1
 *               element, E8M0 shared scale, X = floor(log2 amax) - emax).
 *   exchange  EP simulated ranks, each with its own N tokens: the count
 *             matrix each rank sends, the receive counts and displacements,
 *             and for every destination rank a receive buffer of C rows that
 *             holds, source rank by source rank, the rows each source sends
 *             it (in that source's packed order), then zero rows.
 *             - NKI permute_a2av API reference: description (the receive
 *               layout is the packed cumsum of recv_counts; the table's rows
 *               2-3 are receive counts and displacements) and :return: (C
 *               rows per rank: each source's rows in rank order, then zero
 *               rows).
 *             - DeepSpeed v0.19.4 function index, page 15: SplitPlan entries
 *               (one all-to-all of the [ep_size, E_local] count matrix; the
 *               rows a rank receives from it).
 *             - Mojo ep.dispatch_async.block.scaled.nv struct: recv_count_ptrs
 *               (tokens received per expert).
 *   capacity plan  fixed per-expert capacity: expert e owns rows
 *             e*cap .. e*cap+cap-1; its first cap pairs in flat order are
 *             kept, later ones dropped (slot -1, DROPPED flagged); unused
 *             rows of an expert are zero rows; cap = ceil(cf * N * k / E)
 *             for a capacity factor cf.
 *             - NeMo Automodel token_dispatcher API:
 *               TokenDispatcherConfig.moe_expert_capacity_factor (a capacity
 *               factor per expert; None means nothing is dropped) and the
 *               _DeepepManager capacity_factor argument.
 *             - DeepSpeed v0.19.4 function index, page 15: the dispatch entry
 *               (every routed token placed in its expert slot of an
 *               [e, c, m] buffer; the inverted map makes it one gather).
 *   routing map  a multihot [N, E] map (nonzero byte = routed) with dense
 *             probabilities [N, E] turned into the compact form: a token's
 *             routed experts in ascending order, their probabilities, -1 and
 *             0 in unused slots; more than k routed experts is flagged and
 *             the extra ones are ignored.
 *             - NeMo Automodel token_dispatcher API:
 *               _DeepepManager._indices_to_multihot (top-k indices with -1
 *               masks <-> multihot routing map and multihot probabilities),
 *               TokenDispatcherConfig.moe_hybridep_compact_routing (compact
 *               top-k indices or a dense Boolean routing map), and the
 *               conversion from top-k indices to the multihot routing map.
 *   gated dispatch  every copy (t, j) carries the token row multiplied by its
 *             gate, fl32(w[t,j] * x), encoded in the payload format; combine
 *             then sums the expert rows without weights.
 *             - DeepSpeed v0.19.4 function index, page 15: the entry on
 *               scaling token rows by their router scores ahead of the
 *               experts.
 *   NVFP4     E2M1 codes with one E4M3 scale per 16 values and one fp32
 *             global encode scale gs given by the caller: per block, the
 *             scale code sf = E4M3(fl32(fl32(amax / 6) * gs)) (saturating),
 *             and each code E2M1(fl32(fl32(x * gs) / value(sf))); a block
 *             whose scale is 0 has zero codes.  Decoding: q * value(sf) / gs.
 *             - Mojo ep.dispatch_async.block.scaled.nv struct: execute
 *               (tokens transferred in NVFP4; input_scales, the global
 *               input scales for NVFP4 quantization).
 *             - Mojo shmem ep_comm module: NVBlockScaledTokenFormat
 *               (block-scaled FP4), input_scales_wrapper_type.
 *             - The published NVFP4 format: E2M1 elements, 16-value blocks
 *               with E4M3 scales, one fp32 per-tensor scale.
 *   combine   out[t] = bf16(sum_j w[t,j] * Y[slot[t,j]]) accumulated in fp32
 *             in j order, one fused multiply-add per term.
 *             - DeepSpeed v0.19.4 function index, page 15: the combine entry
 *               (gather expert results back, weight by gate values).
 *             - NeMo Automodel token_dispatcher API:
 *               TokenDispatcherConfig.moe_router_dtype (fp32 routing and
 *               weighted averaging).
 *
 * Readings where the pages are silent (expert e lives on rank e / L; rows are
 * ordered expert-major, then token, then k; invalid IDs are masked and
 * flagged; duplicates are dispatched and flagged; zero blocks get zero codes
 * and zero scales; signs of zero are kept; rows a receive buffer cannot hold
 * are dropped and flagged) are listed with the design notes.
 *
 * Threads.  The loops over independent rows (dispatch: packed rows; combine:
 * tokens; plan step O5: experts, each walking the pairs for its own rows)
 * may run on several OpenMP threads.  Every row is still computed by exactly
 * the code above, on one thread, so the results do not depend on the thread
 * count (oracle_set_threads; the tests check 1 against several).
 *
 * Build: gcc -O2 -std=c99 -fPIC -shared -ffp-contract=off -fopenmp
 *        -o liboracle.so oracle.c -lm  (no fast-math: IEEE division and fmaf
 *        are required)
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_BAD_ID 1u
#define ORC_DUP_ID 2u
#define ORC_CAPACITY 4u
#define ORC_MAP_OVERFLOW 8u
#define ORC_DROPPED 16u

#define ORC_FMT_BF16 0
#define ORC_FMT_FP8 1
#define ORC_FMT_MX 2

/* Threads the row loops may use (>= 1), and how many they use now. */
void oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int oracle_threads(void) { return omp_get_max_threads(); }

/* ---------------------------------------------------------------- bf16 -- */

/* bf16 is the top half of an IEEE binary32: widening is exact. */
float oracle_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static double bf16_bits_value(uint32_t mag_bits) {
  /* value of a non-negative bf16 magnitude pattern; the pattern one past the
   * largest finite value (0x7F80) is treated as 2^128 so that "round to the
   * nearer neighbour" also decides overflow to infinity. */
  if (mag_bits >= 0x7F80u) return ldexp(1.0, 128);
  return (double)oracle_bf16_to_f32((uint16_t)mag_bits);
}

/* IEEE round-to-nearest-even from binary32 to bf16, decided by comparing the
 * distances to the two neighbouring bf16 values (not by the usual bias-add
 * trick).  NaN maps to the quiet NaN 0x7FC0 (non-finite data is outside the
 * contract; this only keeps the result a NaN). */
uint16_t oracle_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t sign = u & 0x80000000u;
  uint32_t mag = u & 0x7FFFFFFFu;
  if (mag > 0x7F800000u) return 0x7FC0;
  if (mag == 0x7F800000u) return (uint16_t)((sign | mag) >> 16);
  uint32_t lo = mag >> 16;        /* truncation toward zero */
  uint32_t hi = lo + 1;           /* next magnitude up      */
  double v = fabs((double)f);
  double dlo = v - bf16_bits_value(lo);
  double dhi = bf16_bits_value(hi) - v;
  uint32_t pick;
  if (dlo < dhi) pick = lo;
  else if (dhi < dlo) pick = hi;
  else pick = (lo & 1u) ? hi : lo; /* tie: even last mantissa bit */
  return (uint16_t)((sign >> 16) | pick);
}

/* --------------------------------------------------------- E4M3 (FN) ---- */

/* Value of a non-negative OCP E4M3 code 0..126 (S.EEEE.MMM, bias 7; code
 * 0x7F is NaN and is never produced).  E = 0 is subnormal: M/8 * 2^-6. */
double oracle_e4m3_value(int code) {
  int e = (code >> 3) & 15;
  int m = code & 7;
  if (e == 0) return ldexp((double)m / 8.0, -6);
  return ldexp(1.0 + (double)m / 8.0, e - 7);
}

/* Saturating round-to-nearest-even into OCP E4M3: clamp |v| to 448, then
 * take the nearest of the 127 finite magnitudes by brute force; on a tie
 * the even code wins.  The sign bit is kept (so -0 gives 0x80). */
uint8_t oracle_e4m3_encode(float v) {
  int neg = signbit(v) ? 1 : 0;
  double a = fabs((double)v);
  if (a > 448.0) a = 448.0;
  int best = 0;
  double bestd = a; /* distance to code 0 */
  for (int c = 1; c <= 126; c++) {
    double d = fabs(a - oracle_e4m3_value(c));
    if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      bestd = d;
    }
  }
  return (uint8_t)((neg << 7) | best);
}

/* ---------------------------------------------------------------- E2M1 -- */

static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double oracle_e2m1_value(int code) { return kE2M1[code & 7]; }

/* Saturating round-to-nearest-even into OCP E2M1 (S.EE.M, bias 1): clamp
 * |v| to 6, nearest of the 8 magnitudes, ties to the even code, sign kept. */
uint8_t oracle_e2m1_encode(float v) {
  int neg = signbit(v) ? 1 : 0;
  double a = fabs((double)v);
  if (a > 6.0) a = 6.0;
  int best = 0;
  double bestd = a;
  for (int c = 1; c < 8; c++) {
    double d = fabs(a - kE2M1[c]);
    if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      bestd = d;
    }
  }
  return (uint8_t)((neg << 3) | best);
}

/* -------------------------------------------------------------- sizes --- */

/* Static packed-row bound: every valid pair takes one row and every expert
 * adds fewer than A pad rows, so N*k + E*(A-1) rows always suffice. */
int64_t oracle_max_rows(int64_t n, int k, int e, int a) {
  return n * (int64_t)k + (int64_t)e * (int64_t)(a - 1);
}

/* ---------------------------------------------------------------- plan --- */

/* O1..O5: validate, count, padded offsets, (4, EP) table, stable slots.
 * Arrays: ids[n*k]; counts[E]; offsets[E+1]; dest_counts[EP]; table[4*EP]
 * (row-major: row 0 send counts, 1 send displacements, 2 padded segment
 * sizes, 3 padded segment offsets, all in elements = rows * H); slot[n*k];
 * packed_src[r_max]. */
void oracle_plan(int64_t n, int k, int e_cnt, int ep, int a, int64_t cap,
                 int64_t h, const int32_t *ids, int32_t *counts,
                 int32_t *offsets, int32_t *dest_counts, uint32_t *table,
                 int32_t *slot, int32_t *packed_src, uint32_t *status) {
  int64_t r_max = oracle_max_rows(n, k, e_cnt, a);
  int l = e_cnt / ep;
  uint32_t st = 0;

  /* O1 + O2: validity and counts, in flat pair order t*k + j. */
  for (int x = 0; x < e_cnt; x++) counts[x] = 0;
  for (int64_t t = 0; t < n; t++) {
    for (int j = 0; j < k; j++) {
      int32_t e = ids[t * k + j];
      if (e == -1) continue;                  /* masked slot */
      if (e < -1 || e >= e_cnt) {             /* out of range: mask, flag */
        st |= ORC_BAD_ID;
        continue;
      }
      for (int jj = 0; jj < j; jj++)
        if (ids[t * k + jj] == e) st |= ORC_DUP_ID;
      counts[e] += 1;
    }
  }

  /* O3: p_e = A * ceil(c_e / A); offsets = exclusive cumsum of p_e. */
  offsets[0] = 0;
  for (int x = 0; x < e_cnt; x++) {
    int32_t p = a * ((counts[x] + a - 1) / a);
    offsets[x + 1] = offsets[x] + p;
  }

  /* O4: per simulated destination rank r (experts r*L .. r*L+L-1). */
  uint32_t send_disp = 0, seg_disp = 0;
  for (int r = 0; r < ep; r++) {
    int64_t s = 0, p = 0;
    for (int x = r * l; x < (r + 1) * l; x++) {
      s += counts[x];
      p += offsets[x + 1] - offsets[x];
    }
    dest_counts[r] = (int32_t)s;
    if (s > cap) st |= ORC_CAPACITY;
    table[0 * ep + r] = (uint32_t)(s * h);
    table[1 * ep + r] = send_disp;
    table[2 * ep + r] = (uint32_t)(p * h);
    table[3 * ep + r] = seg_disp;
    send_disp += (uint32_t)(s * h);
    seg_disp += (uint32_t)(p * h);
  }

  /* O5: for each expert in turn, walk the pairs in flat order; each pair
   * routed there takes the expert's next free row, so rows inside an expert
   * follow (token, k) order.  Masked and invalid pairs keep slot -1; rows no
   * pair takes (pad rows, tail rows) keep packed_src -1. */
  for (int64_t r = 0; r < r_max; r++) packed_src[r] = -1;
  for (int64_t t = 0; t < n; t++) {
    for (int j = 0; j < k; j++) slot[t * k + j] = -1;
  }
#pragma omp parallel for schedule(dynamic, 1)
  for (int x = 0; x < e_cnt; x++) {
    int32_t next = offsets[x];
    for (int64_t t = 0; t < n; t++) {
      for (int j = 0; j < k; j++) {
        if (ids[t * k + j] == x) {
          slot[t * k + j] = next;
          packed_src[next] = (int32_t)t;
          next++;
        }
      }
    }
  }
  *status = st;
}

/* ------------------------------------------------------- capacity plan --- */

/* Per-expert capacity from a capacity factor: ceil(cf * N * k / E), computed
 * in double precision. */
int64_t oracle_expert_capacity(int64_t n, int k, int e, double cf) {
  return (int64_t)ceil(cf * (double)n * (double)k / (double)e);
}

/* C1..C5: validate and count as O1-O2; offsets[e] = e*cap; per rank r the
 * kept rows S_r = sum of min(c_e, cap) (table row 0, cumsum in row 1), the
 * fixed segment L*cap (row 2, cumsum in row 3), CAPACITY if some S_r > rcap;
 * slots: the i-th pair of expert e in flat order takes row e*cap + i while
 * i < cap, later pairs are dropped (slot -1, DROPPED); packed_src holds the
 * token of every kept row and -1 for the unused rows of each expert. */
void oracle_capacity_plan(int64_t n, int k, int e_cnt, int ep, int64_t rcap,
                          int64_t h, int64_t cap, const int32_t *ids,
                          int32_t *counts, int32_t *offsets,
                          int32_t *dest_counts, uint32_t *table,
                          int32_t *slot, int32_t *packed_src,
                          uint32_t *status) {
  int l = e_cnt / ep;
  uint32_t st = 0;
  for (int x = 0; x < e_cnt; x++) counts[x] = 0;
  for (int64_t t = 0; t < n; t++) {
    for (int j = 0; j < k; j++) {
      int32_t e = ids[t * k + j];
      if (e == -1) continue;
      if (e < -1 || e >= e_cnt) {
        st |= ORC_BAD_ID;
        continue;
      }
      for (int jj = 0; jj < j; jj++)
        if (ids[t * k + jj] == e) st |= ORC_DUP_ID;
      counts[e] += 1;
    }
  }
  for (int x = 0; x <= e_cnt; x++) offsets[x] = (int32_t)(x * cap);
  uint32_t send_disp = 0, seg_disp = 0;
  for (int r = 0; r < ep; r++) {
    int64_t kept = 0;
    for (int x = r * l; x < (r + 1) * l; x++) kept += counts[x] < cap ? counts[x] : cap;
    int64_t seg = (int64_t)l * cap;
    dest_counts[r] = (int32_t)kept;
    if (kept > rcap) st |= ORC_CAPACITY;
    table[0 * ep + r] = (uint32_t)(kept * h);
    table[1 * ep + r] = send_disp;
    table[2 * ep + r] = (uint32_t)(seg * h);
    table[3 * ep + r] = seg_disp;
    send_disp += (uint32_t)(kept * h);
    seg_disp += (uint32_t)(seg * h);
  }
  for (int64_t r = 0; r < (int64_t)e_cnt * cap; r++) packed_src[r] = -1;
  for (int64_t t = 0; t < n; t++)
    for (int j = 0; j < k; j++) slot[t * k + j] = -1;
  for (int x = 0; x < e_cnt; x++) {
    int64_t next = 0;
    for (int64_t t = 0; t < n; t++) {
      for (int j = 0; j < k; j++) {
        if (ids[t * k + j] != x) continue;
        if (next < cap) {
          slot[t * k + j] = (int32_t)(x * cap + next);
          packed_src[x * cap + next] = (int32_t)t;
        } else {
          st |= ORC_DROPPED;
        }
        next++;
      }
    }
  }
  *status = st;
}

/* ------------------------------------------------------------ exchange --- */

/* X1..X5 for EP simulated ranks; rank s owns tokens s*n .. s*n+n-1 of the
 * stacked arrays.  Arrays: ids[ep][n][k]; expert_counts[ep][E] (row s is the
 * count matrix rank s sends, viewed as [EP][L]); send_counts[ep][ep] ([s][d]:
 * rows s sends to d); recv_expert_counts[ep][ep][L] ([d][s][l]: rows d
 * receives from s for its local expert l); recv_rows[ep] (rows offered to
 * each receive buffer); table[ep][4][ep] (rank r: row 0 send counts, 1 send
 * displacements, 2 receive counts, 3 receive displacements, in elements);
 * recv_slot[ep][n][k] (receive row d*cap + i of each pair, -1 if masked,
 * invalid or dropped); recv_src[ep][cap] (global source token s*n + t of each
 * receive row, -1 in the zero tail); status[ep]. */
void oracle_exchange_plan(int64_t n, int k, int e_cnt, int ep, int64_t cap,
                          int64_t h, const int32_t *ids, int32_t *expert_counts,
                          int32_t *send_counts, int32_t *recv_expert_counts,
                          int32_t *recv_rows, uint32_t *table,
                          int32_t *recv_slot, int32_t *recv_src,
                          uint32_t *status) {
  int l = e_cnt / ep;

  /* X1: every rank validates and counts its own pairs in flat order. */
  for (int s = 0; s < ep; s++) {
    const int32_t *sid = ids + (int64_t)s * n * k;
    int32_t *cnt = expert_counts + (int64_t)s * e_cnt;
    uint32_t st = 0;
    for (int x = 0; x < e_cnt; x++) cnt[x] = 0;
    for (int64_t t = 0; t < n; t++) {
      for (int j = 0; j < k; j++) {
        int32_t e = sid[t * k + j];
        if (e == -1) continue;
        if (e < -1 || e >= e_cnt) {
          st |= ORC_BAD_ID;
          continue;
        }
        for (int jj = 0; jj < j; jj++)
          if (sid[t * k + jj] == e) st |= ORC_DUP_ID;
        cnt[e] += 1;
      }
    }
    status[s] = st;
  }

  /* X2: rows rank s sends to rank d = its pairs for d's L experts. */
  for (int s = 0; s < ep; s++) {
    for (int d = 0; d < ep; d++) {
      int64_t c = 0;
      for (int x = d * l; x < (d + 1) * l; x++) c += expert_counts[(int64_t)s * e_cnt + x];
      send_counts[(int64_t)s * ep + d] = (int32_t)c;
    }
  }

  /* X3: the counts all-to-all.  Rank d receives, from every rank s, the
   * part of s's count matrix that covers d's experts. */
  for (int d = 0; d < ep; d++) {
    int64_t total = 0;
    for (int s = 0; s < ep; s++) {
      for (int x = 0; x < l; x++)
        recv_expert_counts[((int64_t)d * ep + s) * l + x] =
            expert_counts[(int64_t)s * e_cnt + d * l + x];
      total += send_counts[(int64_t)s * ep + d];
    }
    recv_rows[d] = (int32_t)total;
    if (total > cap) status[d] |= ORC_CAPACITY;
  }

  /* X4: each rank's table; receive displacements are the packed cumsum of
   * its receive counts, source by source. */
  for (int r = 0; r < ep; r++) {
    uint32_t *tr = table + (int64_t)r * 4 * ep;
    uint32_t sd = 0, rd = 0;
    for (int q = 0; q < ep; q++) {
      uint32_t sc = (uint32_t)((int64_t)send_counts[(int64_t)r * ep + q] * h);
      uint32_t rc = (uint32_t)((int64_t)send_counts[(int64_t)q * ep + r] * h);
      tr[0 * ep + q] = sc;
      tr[1 * ep + q] = sd;
      tr[2 * ep + q] = rc;
      tr[3 * ep + q] = rd;
      sd += sc;
      rd += rc;
    }
  }

  /* X5: fill each receive buffer: sources in rank order; within a source,
   * its own packed order (its experts for d in turn, then token, then k).
   * The first cap rows are kept, later ones dropped; the rest of the buffer
   * is zero rows (recv_src -1). */
  for (int64_t i = 0; i < (int64_t)ep * n * k; i++) recv_slot[i] = -1;
  for (int d = 0; d < ep; d++) {
    int64_t next = 0;
    for (int s = 0; s < ep; s++) {
      const int32_t *sid = ids + (int64_t)s * n * k;
      for (int x = d * l; x < (d + 1) * l; x++) {
        for (int64_t t = 0; t < n; t++) {
          for (int j = 0; j < k; j++) {
            if (sid[t * k + j] != x) continue;
            if (next < cap) {
              recv_slot[((int64_t)s * n + t) * k + j] = (int32_t)((int64_t)d * cap + next);
              recv_src[(int64_t)d * cap + next] = (int32_t)((int64_t)s * n + t);
            }
            next++;
          }
        }
      }
    }
    for (int64_t i = next; i < cap; i++) recv_src[(int64_t)d * cap + i] = -1;
  }
}

/* ------------------------------------------------------------ encoders --- */

static int64_t payload_row_bytes(int fmt, int64_t h);
static int64_t scale_row_bytes(int fmt, int64_t h);

/* One row of h fp32 values into one packed row.  For FP8 the payload row
 * holds h code bytes and the scale row h/128 floats; for MX the payload row
 * holds h/2 bytes (element 2m in the low nibble, 2m+1 in the high one) and
 * the scale row h/32 E8M0 bytes. */
void oracle_encode_row_f32(int fmt, int64_t h, const float *v, void *payload,
                           void *scales) {
  if (fmt == ORC_FMT_BF16) {
    uint16_t *q = (uint16_t *)payload;
    for (int64_t i = 0; i < h; i++) q[i] = oracle_f32_to_bf16(v[i]);
    return;
  }
  if (fmt == ORC_FMT_FP8) {
    uint8_t *q = (uint8_t *)payload;
    float *sc = (float *)scales;
    for (int64_t b = 0; b < h / 128; b++) {
      float amax = 0.0f;
      for (int i = 0; i < 128; i++) {
        float a = fabsf(v[b * 128 + i]);
        if (a > amax) amax = a;
      }
      float s = amax / 448.0f;
      if (s == 0.0f) {
        for (int i = 0; i < 128; i++) q[b * 128 + i] = 0;
        sc[b] = 0.0f;
        continue;
      }
      for (int i = 0; i < 128; i++) q[b * 128 + i] = oracle_e4m3_encode(v[b * 128 + i] / s);
      sc[b] = s;
    }
    return;
  }
  /* MX-FP4 */
  uint8_t *q = (uint8_t *)payload;
  uint8_t *sc = (uint8_t *)scales;
  for (int64_t b = 0; b < h / 32; b++) {
    float amax = 0.0f;
    for (int i = 0; i < 32; i++) {
      float a = fabsf(v[b * 32 + i]);
      if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
      for (int i = 0; i < 16; i++) q[b * 16 + i] = 0;
      sc[b] = 0;
      continue;
    }
    int ex;
    frexpf(amax, &ex);          /* amax = m * 2^ex, m in [0.5, 1) */
    int xs = (ex - 1) - 2;      /* floor(log2 amax) - emax(E2M1) */
    if (xs < -127) xs = -127;
    if (xs > 127) xs = 127;
    sc[b] = (uint8_t)(xs + 127);
    for (int i = 0; i < 16; i++) {
      float v0 = ldexpf(v[b * 32 + 2 * i], -xs);
      float v1 = ldexpf(v[b * 32 + 2 * i + 1], -xs);
      q[b * 16 + i] =
          (uint8_t)(oracle_e2m1_encode(v0) | (oracle_e2m1_encode(v1) << 4));
    }
  }
}

/* One hidden row of h bf16 values: widened exactly to fp32, then encoded. */
void oracle_encode_row(int fmt, int64_t h, const uint16_t *x, void *payload,
                       void *scales) {
  float *v = (float *)malloc((size_t)(h > 0 ? h : 1) * sizeof(float));
  for (int64_t i = 0; i < h; i++) v[i] = oracle_bf16_to_f32(x[i]);
  oracle_encode_row_f32(fmt, h, v, payload, scales);
  free(v);
}

/* m hidden rows x[m][h], each encoded on its own (oracle_encode_row) into
 * payload row i and scale row i. */
void oracle_encode_rows(int fmt, int64_t m, int64_t h, const uint16_t *x,
                        uint8_t *payload, uint8_t *scales) {
  int64_t pb = payload_row_bytes(fmt, h), sb = scale_row_bytes(fmt, h);
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t i = 0; i < m; i++)
    oracle_encode_row(fmt, h, x + i * h, payload + i * pb, sb ? scales + i * sb : 0);
}

/* NVFP4 row: h/2 payload bytes (element 2m in the low nibble of byte m) and
 * h/16 E4M3 scale bytes, with global encode scale gs. */
void oracle_encode_row_nvfp4(int64_t h, const uint16_t *x, float gs,
                             uint8_t *payload, uint8_t *scales) {
  for (int64_t b = 0; b < h / 16; b++) {
    float amax = 0.0f;
    for (int i = 0; i < 16; i++) {
      float a = fabsf(oracle_bf16_to_f32(x[b * 16 + i]));
      if (a > amax) amax = a;
    }
    float d = amax / 6.0f;            /* ideal decode scale of the block */
    uint8_t sf = oracle_e4m3_encode(d * gs);
    double sv = oracle_e4m3_value(sf & 0x7F);
    scales[b] = sf;
    if (sv == 0.0) {
      for (int i = 0; i < 8; i++) payload[b * 8 + i] = 0;
      continue;
    }
    float sfv = (float)sv;            /* exact: every E4M3 value is an fp32 */
    for (int i = 0; i < 8; i++) {
      float v0 = (oracle_bf16_to_f32(x[b * 16 + 2 * i]) * gs) / sfv;
      float v1 = (oracle_bf16_to_f32(x[b * 16 + 2 * i + 1]) * gs) / sfv;
      payload[b * 8 + i] =
          (uint8_t)(oracle_e2m1_encode(v0) | (oracle_e2m1_encode(v1) << 4));
    }
  }
}

/* Gather-form dispatch in NVFP4 (as oracle_dispatch). */
void oracle_dispatch_nvfp4(int64_t h, int64_t r_max, int64_t r_used,
                           const int32_t *packed_src, const uint16_t *x, float gs,
                           uint8_t *payload, uint8_t *scales, int zero_tail) {
  int64_t pb = h / 2, sb = h / 16;
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t r = 0; r < r_max; r++) {
    if (r >= r_used && !zero_tail) continue;
    int32_t t = r < r_used ? packed_src[r] : -1;
    if (t < 0) {
      memset(payload + r * pb, 0, (size_t)pb);
      memset(scales + r * sb, 0, (size_t)sb);
    } else {
      oracle_encode_row_nvfp4(h, x + (int64_t)t * h, gs, payload + r * pb, scales + r * sb);
    }
  }
}

static int64_t payload_row_bytes(int fmt, int64_t h) {
  if (fmt == ORC_FMT_BF16) return 2 * h;
  if (fmt == ORC_FMT_FP8) return h;
  return h / 2;
}

static int64_t scale_row_bytes(int fmt, int64_t h) {
  if (fmt == ORC_FMT_BF16) return 0;
  if (fmt == ORC_FMT_FP8) return 4 * (h / 128);
  return h / 32;
}

/* O6, gather form: packed row r takes token packed_src[r], or zero bytes.
 * Rows in [r_used, r_max) are zeroed only when zero_tail is set, otherwise
 * left as they were. */
void oracle_dispatch(int fmt, int64_t h, int64_t r_max, int64_t r_used,
                     const int32_t *packed_src, const uint16_t *x,
                     uint8_t *payload, uint8_t *scales, int zero_tail) {
  int64_t pb = payload_row_bytes(fmt, h), sb = scale_row_bytes(fmt, h);
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t r = 0; r < r_max; r++) {
    if (r >= r_used && !zero_tail) continue;
    uint8_t *prow = payload + r * pb;
    uint8_t *srow = sb ? scales + r * sb : 0;
    int32_t t = r < r_used ? packed_src[r] : -1;
    if (t < 0) {
      memset(prow, 0, (size_t)pb);
      if (srow) memset(srow, 0, (size_t)sb);
    } else {
      oracle_encode_row(fmt, h, x + (int64_t)t * h, prow, srow);
    }
  }
}

/* Gated dispatch, scatter form: each valid pair (t, j) writes
 * encode(fl32(w[t,j] * x[t][c]) for every c) to packed row slot[t,j]; pad
 * rows (rows below r_used that no pair names) are zero bytes; rows in
 * [r_used, r_max) are zeroed only when zero_tail is set. */
void oracle_dispatch_gated(int fmt, int64_t n, int k, int64_t h, int64_t r_max,
                           int64_t r_used, const int32_t *slot, const float *w,
                           const uint16_t *x, uint8_t *payload, uint8_t *scales,
                           int zero_tail) {
  int64_t pb = payload_row_bytes(fmt, h), sb = scale_row_bytes(fmt, h);
  int64_t zero_to = zero_tail ? r_max : r_used;
  for (int64_t r = 0; r < zero_to; r++) {
    memset(payload + r * pb, 0, (size_t)pb);
    if (sb) memset(scales + r * sb, 0, (size_t)sb);
  }
  float *v = (float *)malloc((size_t)(h > 0 ? h : 1) * sizeof(float));
  for (int64_t t = 0; t < n; t++) {
    for (int j = 0; j < k; j++) {
      int32_t r = slot[t * k + j];
      if (r < 0) continue;
      float wt = w[t * k + j];
      for (int64_t c = 0; c < h; c++) v[c] = wt * oracle_bf16_to_f32(x[t * h + c]);
      oracle_encode_row_f32(fmt, h, v, payload + (int64_t)r * pb,
                            sb ? scales + (int64_t)r * sb : 0);
    }
  }
  free(v);
}

/* Multihot routing map -> compact top-k.  map[n][e_cnt] (nonzero = routed),
 * probs[n][e_cnt] or NULL; ids[n][k] gets the routed experts of each token
 * in ascending order, -1 after them; w[n][k] (if not NULL) their
 * probabilities, 0 after them.  A token with more than k routed experts
 * keeps its first k and sets ORC_MAP_OVERFLOW. */
void oracle_routing_map_to_topk(int64_t n, int e_cnt, int k, const uint8_t *map,
                                const float *probs, int32_t *ids, float *w,
                                uint32_t *status) {
  uint32_t st = 0;
  for (int64_t t = 0; t < n; t++) {
    int used = 0;
    for (int e = 0; e < e_cnt; e++) {
      if (!map[t * e_cnt + e]) continue;
      if (used == k) {
        st |= ORC_MAP_OVERFLOW;
        break;
      }
      ids[t * k + used] = e;
      if (w) w[t * k + used] = probs ? probs[t * e_cnt + e] : 1.0f;
      used++;
    }
    for (int j = used; j < k; j++) {
      ids[t * k + j] = -1;
      if (w) w[t * k + j] = 0.0f;
    }
  }
  *status = st;
}

/* O7: out[t][c] = bf16_rne( fmaf chain over j = 0..k-1 of w[t,j]*Y[slot][c] )
 * starting from +0.0f and skipping slots < 0.  w == NULL: every weight is 1
 * (the unweighted sum that follows a gated dispatch; fmaf(1, y, acc) is the
 * correctly rounded y + acc). */
void oracle_combine(int64_t n, int k, int64_t h, const int32_t *slot,
                    const float *w, const uint16_t *y, uint16_t *out) {
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < n; t++) {
    for (int64_t c = 0; c < h; c++) {
      float acc = 0.0f;
      for (int j = 0; j < k; j++) {
        int32_t s = slot[t * k + j];
        if (s < 0) continue;
        float wt = w ? w[t * k + j] : 1.0f;
        acc = fmaf(wt, oracle_bf16_to_f32(y[(int64_t)s * h + c]), acc);
      }
      out[t * h + c] = oracle_f32_to_bf16(acc);
    }
  }
}

/* ---------------------------------------------- array helpers for tests -- */

void oracle_f32_to_bf16_array(const float *in, uint16_t *out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_f32_to_bf16(in[i]);
}

void oracle_e4m3_encode_array(const float *in, uint8_t *out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_e4m3_encode(in[i]);
}

void oracle_e2m1_encode_array(const float *in, uint8_t *out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_e2m1_encode(in[i]);
}
