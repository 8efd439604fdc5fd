/*
 * moe.h -- C ABI of libmoe: MoE token dispatch and combine on one AMD
 * Instinct MI355X (gfx950).
 *
 * The library turns top-k expert IDs into a routing plan, packs token rows
 * into an expert-major buffer (optionally quantised to blockwise FP8,
 * MX-FP4 or NVFP4 on the way) and combines expert outputs back into token
 * order, weighted by the gate values.  Expert-parallel destination ranks
 * are simulated as contiguous segments of the one packed buffer, or, with
 * the moe_exchange_* calls, as separate receive buffers of several
 * simulated source ranks.
 *
 * Conventions for every entry point
 *   - Pointers named in a moe_plan, and every data pointer argument, are
 *     DEVICE pointers the caller allocated; the library never allocates,
 *     frees or synchronises, and keeps no state between calls.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it and the call returns at once; no host wait is
 *     made, so the calls can be captured into a HIP graph.
 *   - Return value: MOE_OK (0) or a negative MOE_E* code.  On an error
 *     nothing has been launched.  No C++ exception crosses this ABI.
 *   - Data-dependent faults (IDs out of range, repeated IDs within a token,
 *     a destination rank over recv_capacity) never fail a call: they set
 *     bits in plan->status on the device, and every row is still placed
 *     inside the static buffer (out-of-range IDs are treated as masked).
 *   - Calls on one stream are ordered; calls that share output buffers on
 *     different streams race, as with any kernel.
 *
 * Passages followed (pages cited by title and section):
 *   NKI permute_a2av API reference: description (rows packed per destination
 *     at cumsum(send_counts) offsets; a (4, EP) uint32 table of send counts,
 *     send displacements, receive counts and receive displacements, in
 *     elements), :param packed_source_indices: (int32 source rows in [0, N),
 *     destination-major), :param recv_capacity: (dropless bound
 *     N * min(top_k, L); duplicate IDs void it), :return: (the output
 *     buffer: rows in use, then rows of zeros).
 *   NeMo Automodel token_dispatcher API: dispatch_preprocess2 (compact
 *     token_indices[T, K] and token_probs[T, K]), dispatch_postprocess (rows
 *     permuted by expert plus tokens per expert), _indices_to_multihot (-1
 *     masks a slot), TokenDispatcherConfig.moe_router_expert_pad_multiple and
 *     .moe_router_dtype (fp32 weighted averaging).
 *   Mojo ep.dispatch_async.block.scaled.nv struct: execute (input_tokens
 *     [num_tokens, hidden_size], topk_ids [num_tokens, top_k]).
 *   Mojo shmem ep_comm module: BF16TokenFormat, BlockwiseFP8TokenFormat,
 *     MXTokenFormat, router_weights_wrapper_type (fp32 gate weight per
 *     (token, k)).
 *   DeepSpeed v0.19.4 function index, page 15: the combine entry (gather
 *     expert results back, weight by gate values) and the SplitPlan entry
 *     (per-expert histogram as an [ep_size, E_local] matrix).
 *   Formats: OCP 8-bit Floating Point Specification (E4M3, max 448, no
 *     infinities) and OCP Microscaling Formats v1.0 (E2M1 elements, E8M0
 *     scale, X = floor(log2 amax) - 2).
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_API __attribute__((visibility("default")))

/* ---- return codes ------------------------------------------------------ */
#define MOE_OK 0
#define MOE_EINVAL (-1)    /* null pointer, bad shape or divisibility       */
#define MOE_EALIGN (-2)    /* a row pointer is not 16-byte aligned          */
#define MOE_EOVERFLOW (-3) /* R_max*H >= 2^32 (table) or rows >= 2^31       */
#define MOE_EHIP (-4)      /* the HIP runtime reported a launch error       */
#define MOE_ESCRATCH (-5)  /* moe_plan_and_dispatch_noalloc: the problem's
                              workspace exceeds MOE_NOALLOC_SCRATCH_BYTES     */

/* ---- bits of plan->status (device, written by moe_dispatch_plan and by
 *      moe_plan_and_dispatch) ------------------------------------------ */
#define MOE_STATUS_BAD_ID 1u   /* an ID outside [-1, E): treated as masked   */
#define MOE_STATUS_DUP_ID 2u   /* an ID repeated within one token: routed    */
#define MOE_STATUS_CAPACITY 4u /* some rank receives more than recv_capacity */
/* (status of moe_routing_map_to_topk) a token routes to more than k experts:
 * its first k, in expert order, are kept */
#define MOE_STATUS_MAP_OVERFLOW 8u
/* (fixed expert capacity) some expert was routed more pairs than its
 * capacity: the later ones were dropped */
#define MOE_STATUS_DROPPED 16u
/* The plan's workspace did not describe these IDs: a pair's place, found
 * from the tile histograms that the counting launch left in the workspace,
 * fell outside its expert's rows or the buffer (the workspace, topk_ids or
 * the plan arrays were changed between the launches of one plan).  Such
 * pairs get slot -1 and nothing is written through them, every store stays
 * inside the caller's buffers, and the plan and payload are not valid. */
#define MOE_STATUS_BAD_PLAN 32u

/* ---- payload formats ---------------------------------------------------- */
typedef enum moe_fmt {
  /* bf16 rows copied bit for bit: payload uint16 [R_max][H], no scales.   */
  MOE_FMT_BF16 = 0,
  /* OCP E4M3 codes, one fp32 scale s = amax/448 per 1x128 block, code =
   * E4M3(x / s) rounded to nearest even and saturated; an all-zero block
   * has s = 0 and zero codes.  payload uint8 [R_max][H],
   * scales float [R_max][H/128].  Needs H % 128 == 0.                     */
  MOE_FMT_FP8_E4M3_B128 = 1,
  /* OCP MX-FP4: E2M1 codes with one E8M0 scale per 32 values,
   * X = clamp(floor(log2 amax) - 2, -127, 127), scale byte X + 127, code =
   * E2M1(x * 2^-X) rounded to nearest even and saturated; element 2m in the
   * low nibble of byte m; an all-zero block has scale byte 0 and zero
   * codes.  payload uint8 [R_max][H/2], scales uint8 [R_max][H/32].
   * Needs H % 32 == 0.                                                    */
  MOE_FMT_MXFP4_B32 = 2,
  /* NVFP4: E2M1 codes with one E4M3 scale per 16 values and one fp32 global
   * encode scale gs (a device value the caller passes to the *_scaled
   * dispatch calls): per block sf = E4M3(fl32(fl32(amax / 6) * gs)),
   * rounded to nearest even and saturated at 448; code = E2M1(fl32(fl32(x *
   * gs) / value(sf))) as for MX-FP4; a block whose scale is 0 has zero codes.
   * Decoding: code * value(sf) / gs.  payload uint8 [R_max][H/2] (element
   * 2m in the low nibble of byte m), scales uint8 [R_max][H/16] (E4M3
   * codes).  Needs H % 32 == 0.  (Mojo ep.dispatch_async.block.scaled.nv
   * struct: NVFP4 transfer and its global input scales; Mojo shmem ep_comm
   * module: NVBlockScaledTokenFormat.)                                      */
  MOE_FMT_NVFP4_B16 = 3
} moe_fmt;

/* ---- flags -------------------------------------------------------------- */
/* Also zero the tail rows [R_used, R_max) of payload and scales.  Without it
 * those rows are left as they were (pad rows inside R_used are always
 * zeroed). */
#define MOE_FLAG_ZERO_TAIL 1u

/* ---- problem description (host memory) ---------------------------------- */
typedef struct moe_problem {
  int64_t n_tokens;      /* N >= 0 token rows                                */
  int32_t hidden;        /* H > 0, H % 8 == 0 (16-byte bf16 rows); see fmt   */
  int32_t top_k;         /* k, 1 <= k <= min(E, 64)                          */
  int32_t n_experts;     /* E, 1 <= E <= 1024                                */
  int32_t ep;            /* EP simulated ranks, E % EP == 0; expert e lives
                            on rank e / (E/EP)                               */
  int64_t recv_capacity; /* C: rows a rank may receive before CAPACITY is
                            flagged; the dropless bound is N * min(k, E/EP)  */
  int32_t pad_multiple;  /* A >= 1: every expert's row count is padded up to
                            a multiple of A with zero rows                   */
  int32_t fmt;           /* a moe_fmt value                                  */
  uint32_t flags;        /* MOE_FLAG_*                                       */
  int64_t expert_capacity; /* 0: dropless (the layout above).  cap > 0: fixed
                            capacity -- expert e owns rows e*cap .. e*cap+cap-1
                            of an [E][cap] buffer (R_max = E*cap); its first
                            cap pairs in flat order are kept, later ones get
                            slot -1 (combine skips them) and set
                            MOE_STATUS_DROPPED; unused rows are zero rows;
                            needs pad_multiple == 1.  (NeMo Automodel
                            token_dispatcher API, TokenDispatcherConfig.
                            moe_expert_capacity_factor; DeepSpeed v0.19.4
                            function index, page 15, the dispatch entry's
                            [e, c, m] buffer.)  See moe_expert_capacity.   */
} moe_problem;

/* ---- routing plan (device pointers; written by moe_dispatch_plan) ------- */
typedef struct moe_plan {
  int32_t *expert_counts;  /* [E]   c_e: valid (token, k) pairs of expert e   */
  int32_t *expert_offsets; /* [E+1] exclusive cumsum of A*ceil(c_e/A);
                                    [E] = R_used rows in use (fixed capacity:
                                    e*cap)                                   */
  int32_t *dest_counts;    /* [EP]  S_r = sum of c_e over rank r's experts
                                    (fixed capacity: of the kept min(c_e, cap);
                                    rows 2-3 of the table then hold L*cap)  */
  uint32_t *rank_table;    /* [4][EP] row-major, in elements (rows * H):
                              0 send counts S_r*H, 1 their exclusive cumsum,
                              2 padded segment sizes P_r*H, 3 their exclusive
                              cumsum (P_r = sum of padded counts; with A = 1
                              rows 2-3 equal rows 0-1)                      */
  int32_t *slot;           /* [N][k] packed row of pair (t, j), -1 if masked
                              or invalid; rows of one expert follow flat pair
                              order t*k + j                                  */
  int32_t *packed_src;     /* [R_max] source token of each packed row, -1 for
                              pad and tail rows                              */
  uint32_t *status;        /* [1]   MOE_STATUS_* bits of this plan           */
} moe_plan;

/* ---- host-only helpers (no GPU work, safe without a device) ------------- */

/* MOE_OK if the problem is well formed, else the error code the entry
 * points would return for it.  The problem's fields are the ones the NKI
 * permute_a2av API reference states (description and parameters:
 * hidden_states [N, H], the routing, EP, recv_capacity), with E and the
 * pad multiple of the NeMo Automodel token_dispatcher API
 * (TokenDispatcherConfig). */
MOE_API int moe_check_problem(const moe_problem *p);

/* R_max = N*k + E*(A-1): rows of the static packed buffer (always >= R_used);
 * E*cap with a fixed expert capacity.  Negative error code if the problem is
 * invalid.  (NKI permute_a2av API reference, :param recv_capacity: and
 * :return: -- a static-shape buffer that every routing fits; NeMo Automodel
 * token_dispatcher API, TokenDispatcherConfig.moe_router_expert_pad_multiple
 * -- at most A-1 pad rows per expert.) */
MOE_API int64_t moe_max_rows(const moe_problem *p);

/* Capacity per expert for a capacity factor cf >= 0: ceil(cf * N * k / E),
 * computed in double precision; negative error code for invalid sizes. */
MOE_API int64_t moe_expert_capacity(int64_t n_tokens, int32_t top_k,
                                    int32_t n_experts, double capacity_factor);

/* Bytes of one payload row (2H, H or H/2) and of one scale row (0, 4*H/128,
 * H/32 or H/16).  Negative error code if the problem is invalid.  (Mojo shmem
 * ep_comm module: BF16TokenFormat, BlockwiseFP8TokenFormat, MXTokenFormat,
 * NVBlockScaledTokenFormat.) */
MOE_API int64_t moe_payload_row_bytes(const moe_problem *p);
MOE_API int64_t moe_scale_row_bytes(const moe_problem *p);

/* Device scratch bytes moe_dispatch_plan needs (0 if none; the pointer may
 * then be NULL).  This is this library's own scratch (the counting kernel's
 * tile histograms); the pages define no workspace.  The caller owns it; its contents need no initialisation
 * and are dead once the plan's kernels have run.  Returns 0 for an invalid
 * problem (moe_dispatch_plan reports the error). */
MOE_API size_t moe_workspace_bytes(const moe_problem *p);

/* ---- entry points -------------------------------------------------------- */

/* Routing plan from topk_ids (device int32 [N][k], -1 = masked): fills every
 * array of *plan.  (NKI permute_a2av API reference, description -- counts,
 * cumsum offsets and the (4, EP) table in elements -- and :param
 * recv_capacity: -- the per-rank bound, CAPACITY; NeMo Automodel
 * token_dispatcher API, dispatch_postprocess -- tokens per expert -- and
 * TokenDispatcherConfig.moe_router_expert_pad_multiple; DeepSpeed v0.19.4
 * function index, page 15, the SplitPlan entry -- the per-expert histogram
 * as an [ep_size, E_local] matrix.)  workspace: moe_workspace_bytes(p)
 * device bytes, 256-byte aligned.  Deterministic: no output depends on the
 * order in which atomic operations land. */
MOE_API int moe_dispatch_plan(const moe_problem *p, const int32_t *topk_ids,
                              const moe_plan *plan, void *workspace,
                              void *stream);

/* Pack token rows (NKI permute_a2av API reference, description and :return:
 * -- rows permuted into destination-major order, unused rows zero; NeMo
 * Automodel token_dispatcher API, get_permuted_hidden_states_by_experts;
 * Mojo shmem ep_comm module, the token formats named at moe_fmt):
 * hidden (device bf16 bits [N][H]) is read once per token;
 * each valid pair (t, j) writes encode(hidden[t]) to packed row
 * plan->slot[t*k+j] of payload (and its scale row of scales); pad rows of
 * every expert are written as zero bytes; rows past R_used are zeroed only
 * with MOE_FLAG_ZERO_TAIL.  payload/scales layouts are given by p->fmt;
 * scales must be NULL for MOE_FMT_BF16.  Reads slot, expert_counts and
 * expert_offsets of a plan made for the same problem; a slot outside
 * [0, R_max) is skipped and pad rows are never written outside the buffer,
 * whatever those arrays hold. */
MOE_API int moe_dispatch(const moe_problem *p, const moe_plan *plan,
                         const uint16_t *hidden, void *payload, void *scales,
                         void *stream);

/* Dispatch in a format that takes a global encode scale (MOE_FMT_NVFP4_B16;
 * the others return MOE_EINVAL): as moe_dispatch, with input_scale a device
 * pointer to the fp32 global encode scale gs.  moe_dispatch itself returns
 * MOE_EINVAL for such a format. */
MOE_API int moe_dispatch_scaled(const moe_problem *p, const moe_plan *plan,
                                const uint16_t *hidden, const float *input_scale,
                                void *payload, void *scales, void *stream);

/* Gated dispatch: as moe_dispatch, but each valid pair (t, j) writes
 * encode(fl32(topk_weights[t][j] * hidden[t][c]) for every c), the token row
 * pre-multiplied by its gate, to packed row slot[t][j] (DeepSpeed v0.19.4
 * function index, page 15, the entry on applying the router scores to the
 * token rows before the experts run).  Each copy is encoded on its own: for FP8
 * its block scale is fl32(fl32(|w| * amax) / 448) and its codes
 * E4M3(fl32(v / s)) with v = fl32(w * x); for MX-FP4 its exponent comes from
 * fl32(|w| * amax).  topk_weights: device float [N][k].  A combine of gated
 * rows passes NULL weights.  Not for MOE_FMT_NVFP4_B16 (MOE_EINVAL). */
MOE_API int moe_dispatch_gated(const moe_problem *p, const moe_plan *plan,
                               const uint16_t *hidden, const float *topk_weights,
                               void *payload, void *scales, void *stream);

/* Plan and dispatch in one call: the outputs of moe_dispatch_plan followed
 * by moe_dispatch (topk_weights NULL, input_scale NULL), moe_dispatch_gated
 * (topk_weights = the gates) or moe_dispatch_scaled (MOE_FMT_NVFP4_B16:
 * input_scale required, topk_weights must be NULL), byte for byte.  NKI
 * permute_a2av API reference, description: one call computes the layout
 * from the routing and permutes the rows into it.  How it runs
 * (moe_plan_and_dispatch_mode): problems with at most 2048 (token, k) pairs
 * run as one launch, in which every workgroup finds the rows of its own
 * pairs before its share of the dispatch (by counting sort keys when there
 * is no padding and no fixed capacity, else from the plan built in LDS);
 * larger ones whose count tiles times E is at most 2048 run the plan's
 * counting kernel and then one launch in which every workgroup finishes
 * the plan it needs from the tile histograms and dispatches; the rest run
 * the plan's kernels and then the dispatch.  A fixed expert capacity drops
 * the pairs ranked past it in the launch that places them.  Equivalent to
 * moe_plan_and_dispatch_begin followed by moe_plan_and_dispatch_end.
 * workspace: moe_workspace_bytes(p) bytes (none for the one-launch sizes).
 * Arguments, layouts and errors as in the calls it replaces. */
MOE_API int moe_plan_and_dispatch(const moe_problem *p, const int32_t *topk_ids,
                                  const moe_plan *plan, const uint16_t *hidden,
                                  const float *topk_weights, const float *input_scale,
                                  void *payload, void *scales, void *workspace,
                                  void *stream);

/* How moe_plan_and_dispatch runs problem p, as launches of its two halves
 * (negative error code for an invalid problem):                           */
#define MOE_PD_ONE_LAUNCH 1 /* _begin: nothing; _end: one launch that plans
                               and dispatches                               */
#define MOE_PD_TILED 2      /* _begin: the counting kernel (tile histograms
                               into workspace); _end: one launch that
                               finishes the plan and dispatches             */
#define MOE_PD_SEPARATE 3   /* _begin: the plan (as moe_dispatch_plan);
                               _end: the dispatch                           */
MOE_API int moe_plan_and_dispatch_mode(const moe_problem *p);

/* moe_plan_and_dispatch in two calls on one stream: _begin launches the
 * work that needs only topk_ids, _end the launch that reads hidden and
 * writes the payload (a single kernel, or none when there is nothing to
 * write).  _begin can therefore be issued as soon as the router has written
 * topk_ids.  _end must follow a _begin of the same problem and arguments
 * on the same stream: it reads what _begin wrote, and without it its
 * results are undefined.  Between the two, topk_ids, the plan arrays and
 * the workspace must not be changed (for MOE_PD_TILED the workspace carries
 * the tile histograms from _begin to _end).  The plan is complete only
 * after _end.  Both take the arguments of moe_plan_and_dispatch that they
 * name and check them as it does. */
MOE_API int moe_plan_and_dispatch_begin(const moe_problem *p, const int32_t *topk_ids,
                                        const moe_plan *plan, void *workspace,
                                        void *stream);
MOE_API int moe_plan_and_dispatch_end(const moe_problem *p, const int32_t *topk_ids,
                                      const moe_plan *plan, const uint16_t *hidden,
                                      const float *topk_weights, const float *input_scale,
                                      void *payload, void *scales, void *workspace,
                                      void *stream);

/* Combine (DeepSpeed v0.19.4 function index, page 15, the combine entry --
 * each token's expert outputs gathered back and weighted by the gate
 * values; NeMo Automodel token_dispatcher API,
 * TokenDispatcherConfig.moe_router_dtype -- the weighting in fp32):
 * out[t][c] = bf16_rne( fp32 fused multiply-add chain, starting
 * from +0 and running over j = 0..k-1 in order, of
 * topk_weights[t][j] * expert_out[slot[t][j]][c] ), skipping slots < 0.
 * expert_out: device bf16 bits [R_max][H]; only rows that some slot names
 * are read (each row through a bounds-checked load of that row alone, so a
 * masked slot reads nothing, and a slot outside [0, R_max) is skipped like a
 * masked one); it may be NULL when R_max = 0.  topk_weights: device float
 * [N][k], or NULL for weights of 1 (the unweighted sum that follows a gated
 * dispatch); out: device bf16 bits [N][H]. */
MOE_API int moe_combine(const moe_problem *p, const moe_plan *plan,
                        const uint16_t *expert_out, const float *topk_weights,
                        uint16_t *out, void *stream);

/* ---- exchange across EP simulated ranks ----------------------------------
 *
 * One GPU holds the shares of all EP ranks of an expert-parallel group: rank
 * s owns tokens s*N .. s*N+N-1 of stacked arrays ([EP][N][k], [EP][N][H]).
 * Each rank routes its own tokens; the exchange itself is simulated by
 * writing every rank's rows straight into the receive buffer of their
 * destination rank (expert e lives on rank e / L, L = E/EP).  A receive
 * buffer has C = recv_capacity rows: the rows of source rank 0, then of rank
 * 1, ..., each source's rows in its own packed order (expert, then token,
 * then k), then zero rows up to C.  Rows that would land at or past C are
 * dropped (their pairs get receive row -1, so combine skips them) and flag
 * MOE_STATUS_CAPACITY on the receiving rank.
 *
 * Problem fields: n_tokens = N per rank; ep = EP ranks, each both a source
 * and a destination; recv_capacity = C rows per receive buffer;
 * pad_multiple must be 1 (a source-major receive buffer has no per-expert
 * padding); flags may hold MOE_FLAG_ZERO_TAIL but the zero rows are always
 * written.  Also needed: EP*N*k*H < 2^32 (the table counts elements in
 * uint32) and EP*C < 2^31 (receive rows are int32).
 *
 * Passages: NKI permute_a2av API reference, description (the receive layout
 * is the packed cumsum of recv_counts; table rows 2-3 hold receive counts
 * and displacements) and :return: (a [C, H] buffer per rank: the rows of
 * each source in turn, then zero rows up to C); DeepSpeed v0.19.4 function index, page
 * 15, SplitPlan entries (one all-to-all of the [ep_size, E_local] count
 * matrix; the rows a rank receives from it); Mojo
 * ep.dispatch_async.block.scaled.nv struct, recv_count_ptrs (tokens
 * received per expert). */
typedef struct moe_exchange {
  int32_t *expert_counts;      /* [EP][E] pairs rank s routes to expert e; row
                                  s, viewed as [EP][L], is the count matrix
                                  rank s sends in the counts all-to-all      */
  int32_t *send_counts;        /* [EP][EP] [s][d]: rows rank s sends rank d  */
  int32_t *recv_expert_counts; /* [EP][EP][L] [d][s][l]: rows rank d receives
                                  from rank s for its local expert l (what
                                  the counts all-to-all delivers to d)       */
  int32_t *recv_rows;          /* [EP] rows offered to each receive buffer,
                                  the sum over s of send_counts[s][d]; more
                                  than C flags CAPACITY                      */
  uint32_t *rank_table;        /* [EP][4][EP] each rank's table, in elements
                                  (rows * H): 0 send counts, 1 send
                                  displacements (in the rank's own packed
                                  order), 2 receive counts from each source,
                                  3 receive displacements (exclusive cumsum
                                  of row 2)                                  */
  int32_t *recv_slot;          /* [EP][N][k] receive row d*C + i of pair
                                  (s, t, j): row i of rank d's buffer; -1 if
                                  masked, invalid or dropped                 */
  int32_t *recv_src;           /* [EP][C] global token s*N + t that each
                                  receive row holds, -1 for the zero rows    */
  uint32_t *status;            /* [EP] per rank: BAD_ID / DUP_ID for the IDs
                                  it routes, CAPACITY for its own buffer     */
} moe_exchange;

/* MOE_OK if p describes a valid exchange (see above), else the error code
 * the exchange entry points would return for it. */
MOE_API int moe_check_exchange(const moe_problem *p);

/* Device scratch bytes moe_exchange_plan needs (always > 0 for a valid
 * problem; 0 for an invalid one).  256-byte aligned, caller-owned, no
 * initialisation needed, dead once the plan's kernels have run. */
MOE_API size_t moe_exchange_workspace_bytes(const moe_problem *p);

/* Exchange plan from topk_ids (device int32 [EP][N][k], -1 = masked): fills
 * every array of *x.  Deterministic (no output depends on the order in
 * which atomic operations land). */
MOE_API int moe_exchange_plan(const moe_problem *p, const int32_t *topk_ids,
                              const moe_exchange *x, void *workspace,
                              void *stream);

/* Fill every receive buffer: hidden (device bf16 bits [EP][N][H]) is read
 * once per token; each kept pair writes encode(hidden[s][t]) to receive row
 * x->recv_slot[s][t][j] of recv_payload ([EP][C] rows of the format's
 * payload row) and recv_scales ([EP][C] scale rows; NULL for bf16); every
 * other row of every buffer is written as zero bytes.  Reads recv_slot and
 * recv_rows of an exchange plan made for the same problem. */
MOE_API int moe_exchange_dispatch(const moe_problem *p, const moe_exchange *x,
                                  const uint16_t *hidden, void *recv_payload,
                                  void *recv_scales, void *stream);

/* As moe_exchange_dispatch, for MOE_FMT_NVFP4_B16 with its global encode
 * scale (see moe_dispatch_scaled). */
MOE_API int moe_exchange_dispatch_scaled(const moe_problem *p,
                                         const moe_exchange *x,
                                         const uint16_t *hidden,
                                         const float *input_scale,
                                         void *recv_payload, void *recv_scales,
                                         void *stream);

/* As moe_exchange_dispatch, with every copy pre-multiplied by its gate as in
 * moe_dispatch_gated (not for MOE_FMT_NVFP4_B16); topk_weights: device
 * float [EP][N][k]. */
MOE_API int moe_exchange_dispatch_gated(const moe_problem *p,
                                        const moe_exchange *x,
                                        const uint16_t *hidden,
                                        const float *topk_weights,
                                        void *recv_payload, void *recv_scales,
                                        void *stream);

/* Reverse exchange and combine: out[s][t][c] = bf16_rne( fp32 fused
 * multiply-add chain over j = 0..k-1 in order, from +0, of
 * topk_weights[s][t][j] * expert_out[recv_slot[s][t][j]][c] ), skipping
 * receive rows < 0.  expert_out: device bf16 bits [EP][C][H], of which only
 * rows that some pair names are read; it may be NULL when C = 0 (no receive
 * row exists).  topk_weights: device float [EP][N][k], or NULL for weights
 * of 1; out: device bf16 bits [EP][N][H]. */
MOE_API int moe_exchange_combine(const moe_problem *p, const moe_exchange *x,
                                 const uint16_t *expert_out,
                                 const float *topk_weights, uint16_t *out,
                                 void *stream);

/* ---- dense routing-map input -------------------------------------------
 *
 * NeMo Automodel token_dispatcher API: _DeepepManager._indices_to_multihot
 * (top-k indices with -1 masks and probabilities <-> a multihot routing map
 * and multihot probabilities) and TokenDispatcherConfig.
 * moe_hybridep_compact_routing (routing given as compact top-k indices or as
 * a dense Boolean map).  The dense form is turned into the compact one that
 * moe_dispatch_plan and the combine take. */

/* Device scratch bytes moe_routing_map_to_topk needs (0 for N = 0 or an
 * invalid problem). */
MOE_API size_t moe_map_workspace_bytes(const moe_problem *p);

/* routing_map: device uint8 [N][E], nonzero = the token routes to that
 * expert; probs: device float [N][E] or NULL.  Writes topk_ids [N][k]: the
 * token's routed experts in ascending order, then -1; topk_weights [N][k]
 * (or NULL to skip): probs[t][e] of those experts (1 without probs), then 0;
 * status [1] (written, not accumulated): MOE_STATUS_MAP_OVERFLOW if some
 * token routes to more than k experts (it keeps its first k).  Uses
 * p->n_tokens, p->n_experts and p->top_k. */
MOE_API int moe_routing_map_to_topk(const moe_problem *p,
                                    const uint8_t *routing_map,
                                    const float *probs, int32_t *topk_ids,
                                    float *topk_weights, uint32_t *status,
                                    void *workspace, void *stream);

/* ---- plan and dispatch with no caller workspace ----------------------------
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.
 * moe_plan_and_dispatch_noalloc is moe_plan_and_dispatch with the plan's
 * workspace (the counting kernel's tile histograms and fault bits) taken
 * from a static device array of MOE_NOALLOC_SCRATCH_BYTES inside the
 * library instead of a caller buffer: same arguments otherwise, same
 * outputs byte for byte, same launches on `stream`.  It allocates nothing
 * and frees nothing.  The caller still passes every input and output.
 *   - A problem whose moe_workspace_bytes exceeds MOE_NOALLOC_SCRATCH_BYTES
 *     (more than 262,144 histogram entries: count tiles of at most 2048
 *     pairs times E + 1) returns MOE_ESCRATCH and launches nothing.
 *   - Each GPU holds its own copy of the array, from its first use until the
 *     process ends; its device address is looked up once per device (with
 *     that device current: the stream must belong to the current device).
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents (the counting kernel rewrites every entry it uses, so
 *     nothing needs clearing).  Calls that overlap on one GPU -- on two
 *     streams, or from two host threads without ordering -- race on it;
 *     calls on one stream are ordered and safe. */
#define MOE_NOALLOC_SCRATCH_BYTES (1u << 20)
MOE_API int moe_plan_and_dispatch_noalloc(const moe_problem *p, const int32_t *topk_ids,
                                          const moe_plan *plan, const uint16_t *hidden,
                                          const float *topk_weights, const float *input_scale,
                                          void *payload, void *scales, void *stream);

/* Static text for a return code. */
MOE_API const char *moe_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
