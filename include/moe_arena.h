/*
 * moe_arena.h -- C ABI of libmoe_arena.so: one routed-expert MoE layer running
 * against a partially resident expert arena, on an AMD Instinct MI355X (gfx950).
 *
 * The method (TideLM README, "How adaptive expert loading works"):
 *   item 1  every routed pick the router wants, resident or not, is recorded
 *           per (layer, expert), weighted by its routing score;
 *   item 2  the router only picks resident experts; a missing pick is replaced
 *           by the next-best resident expert for that token;
 *   item 3  hot reads copy a missing expert into a slot (a ring entry, or the
 *           slot of the coldest expert) so it becomes routable.
 * Rows are named by index rather than copied per expert, and the per-expert
 * results of a row are added in one fixed order (colibri cluster page, wire
 * protocol paragraphs on COLIEX01 v2 and on the fixed summation order).
 *
 * Conventions for every entry point:
 *   - Pointers are device memory owned by the caller unless marked (host).
 *     The library allocates nothing and never synchronises the device.
 *   - Every call only validates its arguments and enqueues work on the given
 *     HIP stream; results are ready when that stream reaches them.
 *   - All validation happens before the first HIP call, so a rejected call has
 *     no side effect.  No call aborts, prints or throws.
 *   - Calls are reentrant; two calls that share an output or a workspace must
 *     be ordered by the caller (same stream or events).
 *   - Inputs must be finite (no NaN or Inf in activations or weights).
 *   - The k picks of a token are always listed in ascending expert id; every
 *     order-dependent sum follows that order.
 *
 * Formats:
 *   bf16      : uint16_t bit pattern of a bfloat16.
 *   MXFP4 row : K/2 bytes of E2M1 codes (element 2i in the low nibble of byte
 *               i; code = sign<<3 | exponent<<1 | mantissa, exponent bias 1)
 *               followed, at byte K/2, by K/32 E8M0 scale bytes (value
 *               2^(byte-127)), one per 32 consecutive elements; a row occupies
 *               moe_mxfp4_row_bytes(K) bytes (padded to 16).  OCP MX v1.0.
 *               Activation rows are encoded with X = 2^(floor(log2 amax) - 2)
 *               clamped to 2^-127..2^127, round to nearest E2M1 value with ties
 *               to the even mantissa, saturation at +-6, sign bit copied from
 *               the input, and scale byte 0 with all-zero codes for a block
 *               whose amax is 0.
 *   MXFP6 row : the activation-format variant (act_format = MOE_ACT_MXFP6):
 *               K/32 blocks of 24 bytes of E2M3 codes (code = sign<<5 |
 *               exponent<<3 | mantissa, exponent bias 1; element i of a block
 *               at bits [6i, 6i+6) of its 24 bytes read as one little-endian
 *               number -- the operand layout of the block-scaled matrix
 *               instruction), followed, at byte 3K/4, by the K/32 E8M0 scale
 *               bytes; moe_act_row_bytes(K, MOE_ACT_MXFP6) bytes (padded to
 *               16).  Encoded like MXFP4 activation rows (same X, OCP MX v1.0
 *               FP6 E2M3 values, saturation at +-7.5).
 *   slot      : one SwiGLU expert, six sections, each starting on a 256-byte
 *               boundary (offsets from moe_slot_sections):
 *                 gate codes [I][H/2] | gate scales [I][H/32] |
 *                 up codes   [I][H/2] | up scales   [I][H/32] |
 *                 down codes [H][I/2] | down scales [H][I/32]
 *               A matrix's MXFP4 rows (row n: output n's weights, K/2 code
 *               bytes, K/32 scale bytes) are stored as follows.  Scales: row
 *               by row, [N][K/32].  Codes: in tiles of 16 rows x 64 code
 *               bytes (128 elements): byte j of row n sits at
 *                 (n/16)*16*(K/2) + (j/64)*1024 + (n%16)*w + j%64,
 *               w = min(64, K/2 - 64*(j/64)) (64, or the width of a last
 *               partial tile), so a tile's 16 row pieces are one 1 KB run
 *               (N, a multiple of 32, splits into whole 16-row blocks).
 *   arena     : S slots at arena + s*slot_stride; slot ids are global: arena
 *               slots first, hot-ring slots after them (TideLM README, "Settings
 *               worth knowing": the ring's slots are on top of the budget).
 *   expert_slot[e] : slot of expert e, or -1 if e is not routable.  Values
 *               outside [0, S) are treated as -1.  Distinct routable experts
 *               must have distinct slots.
 */
#ifndef MOE_ARENA_H
#define MOE_ARENA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MOE_OK 0
#define MOE_EINVAL -1        /* null pointer, negative or inconsistent size, misalignment */
#define MOE_EUNSUPPORTED -2  /* H or I not a multiple of 32, k > min(E, 32), E > 1024, S > 8192 */
#define MOE_EWORKSPACE -3    /* ws_bytes below moe_workspace_bytes(...) */
#define MOE_EHIP -4          /* a HIP launch or copy reported an error */
#define MOE_ESCRATCH -5      /* the batch needs more than the library's own scratch holds */
#define MOE_EIO -6           /* a history file could not be opened, read, written or renamed */
#define MOE_EFORMAT -7       /* a history file is not one of this shape, or is damaged */

/* Workspace selectors for moe_workspace_bytes. */
#define MOE_OP_ROUTE 0
#define MOE_OP_DEMAND 1
#define MOE_OP_EXPERTS 2
#define MOE_OP_HOT_PICK 3
#define MOE_OP_EXPERTS_SHARED 4  /* moe_experts_forward with a shared expert */
#define MOE_OP_ACT_MXFP6 0x10    /* or-ed into MOE_OP_EXPERTS(_SHARED): act_format MXFP6 */

#define MOE_MAX_E 1024
#define MOE_MAX_K 32
#define MOE_MAX_S 8192
#define MOE_MAX_RING_PAIRS 16384  /* L*E of a ring plan */
#define MOE_MAX_RING 1024         /* ring entries */
#define MOE_MAX_RING_PER_STEP 64  /* picks of one ring plan */

/* Human-readable text for a status code (static storage; never NULL). */
const char* moe_status_string(int status);

/* Bytes of one MXFP4 row of K elements (K % 32 == 0): K/2 + K/32 rounded up to 16. */
size_t moe_mxfp4_row_bytes(int K);

/* Activation formats (moe_route_args.act_format, moe_experts_args.act_format):
 * the activation rows xq and the experts' intermediate rows h in MXFP4 (the
 * default) or in MXFP6 (E2M3 elements: the activation-format variant; better
 * accuracy, 1.5x the activation bytes).  The weights are MXFP4 either way. */
#define MOE_ACT_MXFP4 0
#define MOE_ACT_MXFP6 1

/* Bytes of one activation row of K elements in a format: moe_mxfp4_row_bytes(K)
 * or 3K/4 + K/32 rounded up to 16 (MXFP6); 0 for K not a positive multiple of
 * 32 or an unknown format. */
size_t moe_act_row_bytes(int K, int act_format);

/* Byte size of one packed expert slot (the slot format above); 0 if H or I is
 * not a positive multiple of 32. */
size_t moe_slot_bytes(int H, int I);

/* Section offsets of a slot, in the order gate codes, gate scales, up codes,
 * up scales, down codes, down scales.  out6 (host) receives 6 values.
 * Returns MOE_OK, MOE_EINVAL (null out6) or MOE_EUNSUPPORTED. */
int moe_slot_sections(int H, int I, size_t* out6);

/* Workspace bytes an operation needs for the given shape (0 if none; the
 * workspace pointer may then be NULL).  op is one of MOE_OP_*; for the
 * experts' MXFP6 activation variant, MOE_OP_EXPERTS or MOE_OP_EXPERTS_SHARED
 * or-ed with MOE_OP_ACT_MXFP6.  Unused arguments are ignored.  Returns
 * (size_t)-1 for an invalid op or shape. */
size_t moe_workspace_bytes(int op, int T, int H, int E, int k, int I, int S);

/*
 * moe_route -- router scores, demand picks, masked top-k, bucketing, and
 * MXFP4 activations for one layer call.
 *
 * Steps (TideLM README, "How adaptive expert loading works", items 1-2):
 *   z[t,e]  = sum_h x[t,h] * w_router[e,h] + bias[e] in float64 (every
 *             product is exact): for T <= 64 and H <= 8192 the sum over h
 *             runs in chunks of 32 (a fused multiply-add chain over each
 *             chunk, ascending h); the chunk sums are added in runs of 16
 *             consecutive chunks and the run sums in ascending order; for
 *             larger batches it is the chain over h in steps of 4 of the
 *             float64 matrix instruction; then the bias.  Within each regime a
 *             token's z does not depend on the rest of the batch.
 *             Larger batches with H a multiple of 512 (H <= 8192) first compute every z on
 *             the bf16 matrix instruction (w split exactly into three bf16
 *             parts, float32 sums per 128-wide slice of h, float64 across
 *             slices) with a bound on its error, 34 * 8.13 * 2^-24 *
 *             ||x_t|| * max_e ||w_e|| (a model of the instruction's rounding:
 *             at most twice the error of 16 round-to-nearest additions);
 *             every token whose k-th and (k+1)-th logits -- over all experts
 *             or over the routable ones -- are within twice that bound is
 *             selected again after the experts that can still be picked (those
 *             not below its k-th value by more than twice the bound, in either
 *             order) get float64 logits (a fused multiply-add chain per lane
 *             over H/64 consecutive h, then a fixed-order wave sum); every
 *             other expert is provably out of its top-k.  So the picks are
 *             those of float64 logits.  Probabilities of the other
 *             tokens come from the bounded logits (typically ~1e-6 relative).
 *   p[t,:]  = softmax over all E experts of z[t,:] (float64).
 *   topk    = the k experts with the largest z (ties to the lower id), listed in
 *             ascending id, with score p[t,e]: the picks demand is recorded over.
 *   sel     = the min(k, |R|) routable experts with the largest z (same order
 *             rule), R = {e : 0 <= expert_slot[e] < S}; remaining entries are
 *             padded with expert -1, weight 0, slot -1.  A routable pick that
 *             was also wanted is kept; each miss is replaced by the next-best
 *             routable expert.
 *   sel_weight[t,j] = p[t,e_j] / sum_j' p[t,e_j'] over the present picks.
 *   bucketing: assignment a = t*k + j goes to slot sel_slot[t,j];
 *             slot_offsets[s] = number of assignments in slots < s (S+1 entries);
 *             perm lists assignments by slot, ascending a within a slot;
 *             perm[slot_offsets[S] .. T*k) = -1 (padded picks).
 *   xq      = each token row of x encoded as an MXFP4 row (format above).
 *
 * Inputs : x [T][H] bf16; w_router [E][H] float; bias [E] float (nullable =
 *          zero); expert_slot [E] int32.
 * Outputs: topk_expert, sel_expert, sel_slot [T][k] int32; topk_score,
 *          sel_weight [T][k] float; slot_offsets [S+1] int32; perm [T*k] int32;
 *          xq [T][moe_act_row_bytes(H, act_format)] uint8 (16-byte aligned).
 * Workspace: moe_workspace_bytes(MOE_OP_ROUTE, T, H, E, k, 0, S) bytes, 256-byte
 *          aligned.  Contents on return are unspecified, except the router's
 *          dot products (see reuse_logits).
 * T = 0 is valid (only slot_offsets is written, all zero).
 * stage_events (host array, nullable): MOE_STAGE_EVENTS events recorded on
 *          `stream` when T > 0: before the router logits, before selection,
 *          before bucket counting (with hist_row, larger batches count the
 *          demand's chunk sums there too), before the scatter, and after it -- so a
 *          caller can time each kernel stage.  For T <= 64, E <= 256 and
 *          H <= 8192, selection and bucketing run as one kernel and the last
 *          three events are recorded together after it.  A null entry is not
 *          recorded.
 *          Recording changes no result, but each record costs a few
 *          microseconds of stream time.
 * hist_row, delta (nullable): when hist_row is non-null the call also does
 *          moe_demand_accumulate's work for this batch (same definition, same
 *          float64 result): hist_row[e] += delta[e], delta (if non-null) gets
 *          the per-call demand.  For small batches this runs inside the
 *          selection kernel and saves a launch.
 * reuse_logits: nonzero skips the router's dot products: they are taken from
 *          the workspace, and xq is left as written, by the previous moe_route
 *          call made with the same T, H, E, x, w_router, xq and ws (nothing
 *          else may have written ws or xq since); expert_slot, S, bias and the
 *          output buffers may differ.  Selection, renormalisation and
 *          bucketing run as usual, so the results equal those of a call
 *          without the flag.  For a hot read: route again over a changed
 *          routable set without recomputing the products.  On every return
 *          with T > 0 the first T*E*8 bytes of ws hold them (float64 [T][E],
 *          x . w_router before the bias; for larger batches, the bounded
 *          bf16-instruction values except for the tokens recomputed exactly).
 *          With reuse_logits the selection certifies the stored values again
 *          against the new routable set.
 * act_format: MOE_ACT_MXFP4 (xq rows in MXFP4) or MOE_ACT_MXFP6 (MXFP6 rows,
 *          for the experts' activation-format variant); anything else is
 *          MOE_EINVAL.
 */
#define MOE_STAGE_EVENTS 5

typedef struct moe_route_args {
  int T, H, E, k, S;
  const uint16_t* x;
  const float* w_router;
  const float* bias;
  const int32_t* expert_slot;
  int32_t* topk_expert;
  float* topk_score;
  int32_t* sel_expert;
  float* sel_weight;
  int32_t* sel_slot;
  int32_t* slot_offsets;
  int32_t* perm;
  uint8_t* xq;
  void* ws;
  size_t ws_bytes;
  hipEvent_t* stage_events;
  double* hist_row;
  float* delta;
  int reuse_logits;
  int act_format;
} moe_route_args;

int moe_route(const moe_route_args* args, hipStream_t stream);

/*
 * moe_demand_accumulate -- record the router's demand for one layer call
 * (TideLM README, "How adaptive expert loading works", item 1: every pick the
 * router wants, resident or not, weighted by its routing score).
 *
 *   delta[e]    = sum over tokens t (ascending) of topk_score[t,j] where
 *                 topk_expert[t,j] == e, accumulated in float64 in a fixed order;
 *   hist_row[e] += delta[e]   (float64 running history of this layer).
 * Independent of the resident mask.  Entries of topk_expert outside [0, E) are
 * ignored.
 * Inputs : topk_expert [T][k] int32, topk_score [T][k] float.
 * In/out : hist_row [E] double (e.g. hist + layer*E).
 * Output : delta [E] float (nullable).
 * Workspace: moe_workspace_bytes(MOE_OP_DEMAND, T, 0, E, k, 0, 0) bytes.
 */
int moe_demand_accumulate(const int32_t* topk_expert, const float* topk_score, int T, int k,
                          int E, double* hist_row, float* delta, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/*
 * moe_experts_forward -- the grouped SwiGLU expert FFNs over arena slots and the
 * weighted combine (steps after bucketing).
 *
 * For every slot s with assignments, rows p in [slot_offsets[s], slot_offsets[s+1])
 * name assignment a = perm[p] of token t = a / k:
 *   g = xq[t] . Wg^T, u = xq[t] . Wu^T   (MXFP4 x MXFP4 products, float32 sums)
 *   h = silu(g) * u, silu(v) = v / (1 + exp(-v))
 *   y[a] = MXFP4(h) . Wd^T               (h encoded like an activation row, along I)
 * then out[t] = sum over j ascending (ascending expert id) of sel_weight[t,j] *
 * y[t*k+j], skipping picks with sel_slot[t,j] < 0, summed in float32 and
 * rounded to bf16.  y is kept in float32 by the small-batch kernels (T*k <
 * 2048, or H or I not a multiple of 512) and rounded to bf16 per element by
 * the pipelined kernels before the sum.
 * Only the slots that hold assignments are read.
 * shared_expert (nullable): one more SwiGLU expert in the slot format (256-byte
 *          aligned, moe_slot_bytes(H, I) bytes, anywhere in device memory),
 *          the layer's shared expert (colibri cluster page, shared-expert item:
 *          it takes every row, unweighted, and its row is added at one fixed
 *          point).  It runs on every token inside the same gate/up and down
 *          launches as the routed slots (one more work item), and out[t] =
 *          (the routed sum above) + y_shared[t], added after the last routed
 *          pick, in float32, before the one rounding to bf16.  With it, the
 *          workspace is moe_workspace_bytes(MOE_OP_EXPERTS_SHARED, ...) and
 *          the call runs even when S == 0.
 * act_format: the format of xq (as moe_route wrote it) and of h.  With
 *          MOE_ACT_MXFP6 the products take E2M3 activations against the MXFP4
 *          weights (the block-scaled instruction at the E2M1 x E2M3 setting;
 *          g, u and y otherwise as above, h encoded as an MXFP6 row), on both
 *          kernel families; H and I must be multiples of 512 and at most
 *          15872 (else MOE_EUNSUPPORTED).  Other values: MOE_EINVAL.
 *
 * Inputs : xq, slot_offsets, perm, sel_slot, sel_weight as written by moe_route
 *          for the same T, k, S; arena (256-byte aligned), slot_stride (multiple
 *          of 256, >= moe_slot_bytes(H, I)).  Indices out of range are skipped,
 *          never dereferenced.
 * Output : out [T][H] bf16.
 * Workspace: moe_workspace_bytes(MOE_OP_EXPERTS, T, H, 0, k, I, S) bytes
 *          (MOE_OP_EXPERTS_SHARED with a shared expert; either or-ed with
 *          MOE_OP_ACT_MXFP6 when act_format is MOE_ACT_MXFP6).
 * Any copy into a slot the call reads (arena_load_slot) must be ordered before
 * it: by the caller (hipStreamWaitEvent on the load's event), or, for one
 * slot, through defer_slot.
 * defer_slot, defer_event: -1 and NULL, or a slot in [0, S) whose bytes are
 *          still being written and the event recorded after that write (the
 *          hot read: arena_load_slot's `done`).  The call then runs the
 *          gate/up products of every other slot first, makes `stream` wait for
 *          defer_event, and runs that slot's and everything after them, so the
 *          copy overlaps the first part; the output is the same as a call made
 *          after the copy.  Batches taking the small-batch kernels (T*k <
 *          2048, or H or I not a multiple of 512) wait for the event before
 *          any work.  MOE_EINVAL for defer_slot outside [-1, S) or a deferred
 *          slot without an event.
 * stage_events (host array, nullable): MOE_STAGE_EVENTS events on `stream`
 *          when T > 0 and S > 0: [0] before the work list; [1] and [2] the
 *          start and the end of the gate/up kernel itself, taken from its
 *          dispatch (hipExtLaunchKernel), so their interval is that kernel's
 *          duration (with a deferred slot, of the gate/up pass over the other
 *          slots); [3] after the down kernel; [4] after the combine.  A null
 *          entry is not recorded.  Recording changes no result.
 */
typedef struct moe_experts_args {
  int T, H, I, k, S;
  const uint8_t* xq;
  const uint8_t* arena;
  size_t slot_stride;
  const int32_t* slot_offsets;
  const int32_t* perm;
  const int32_t* sel_slot;
  const float* sel_weight;
  uint16_t* out;
  void* ws;
  size_t ws_bytes;
  hipEvent_t* stage_events;
  int defer_slot;
  hipEvent_t defer_event;
  const uint8_t* shared_expert;
  int act_format;
} moe_experts_args;

int moe_experts_forward(const moe_experts_args* args, hipStream_t stream);

/*
 * moe_experts_forward_noalloc -- moe_experts_forward for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, kernels and results,
 * except that args->ws must be NULL and args->ws_bytes 0: the workspace is a
 * device array of MOE_NOALLOC_SCRATCH_BYTES (16 MiB) inside the library, one
 * copy per GPU, kept until the process ends.  The call allocates nothing and
 * calls no allocating routine; the array's device address is looked up once
 * per device (on the first call made with that device current) and reused.
 * `stream` must belong to the current device.
 * Limit: batches whose moe_workspace_bytes(...) for the call's op exceeds
 * MOE_NOALLOC_SCRATCH_BYTES are refused with MOE_ESCRATCH before any HIP call
 * (for example up to 900 assignments T*k at H = 4096: decode batches).
 * Every call on one GPU uses the same array and leaves its contents there:
 * calls that may overlap on one GPU (different streams, no ordering between
 * them) race and give wrong results; order them on one stream or with events.
 * Errors: as moe_experts_forward; MOE_EINVAL also for a non-null ws or a
 * nonzero ws_bytes; MOE_EHIP if the array's address cannot be found.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (16u << 20)

int moe_experts_forward_noalloc(const moe_experts_args* args, hipStream_t stream);

/*
 * arena_load_slot -- copy one expert, read by the host, into a slot or hot-ring
 * entry (TideLM README, "How adaptive expert loading works", item 3).
 *
 * Enqueues an asynchronous host-to-device copy of `bytes` bytes from host_src
 * (host; page-locked memory for a truly asynchronous copy) to
 * arena + slot*slot_stride on side_stream, then records `done` (nullable) on
 * it.  The caller makes the slot routable (expert_slot) only after `done`, so
 * a copy in flight or a failed copy leaves the expert non-routable and its
 * tokens are served by substitutes.  host_src must stay valid until `done`.
 * Errors: MOE_EINVAL for a null pointer, slot outside [0, num_slots), bytes 0
 * or above slot_stride, or slot_stride not a multiple of 256; MOE_EHIP if the
 * copy or the event record fails.
 */
int arena_load_slot(uint8_t* arena, size_t slot_stride, int num_slots, int slot,
                    const void* host_src, size_t bytes, hipStream_t side_stream, hipEvent_t done);

/*
 * moe_hot_pick -- the hot-read decision for one layer call (TideLM README,
 * "How adaptive expert loading works", item 3, GLM-5.3 bullet: a layer's
 * heaviest miss carrying at least 0.2 of a token's routing weight is read
 * before the layer's experts run and kept in place of the coldest expert).
 *
 *   share[t,j] = topk_score[t,j] / sum_j' topk_score[t,j'] over the token's
 *                unrestricted picks, in float64 with the sum in ascending j;
 *   out[0] = e*: among picks whose expert is not routable (expert_slot outside
 *            [0, S)) and whose share >= threshold, the one with the largest
 *            share, ties to the lower expert id, then the lower token; -1 if none;
 *   out[1] = c: among experts with 0 <= expert_slot[e] < n_arena (arena slots;
 *            hot-ring slots are never evicted), the one with the smallest
 *            hist_row[e], ties to the lower id; -1 if none.
 * Inputs : topk_expert, topk_score [T][k] as written by moe_route; expert_slot
 *          [E]; hist_row [E] double (the history after this call's demand).
 * Output : out [2] int32 (device).
 * Workspace: moe_workspace_bytes(MOE_OP_HOT_PICK, T, 0, 0, 0, 0, 0) bytes,
 *          256-byte aligned (16 B per token-pass workgroup, at most 256 of them;
 *          0 when T == 0).  Two kernels on `stream`: a token pass over
 *          min(ceil(T/256), 256) workgroups writes each one's best miss, then
 *          one workgroup takes the best of those and the coldest expert.
 *          Returns MOE_EWORKSPACE if ws_bytes is short, MOE_EINVAL for null or
 *          misaligned pointers (4 bytes for the int32/float arrays, 8 for
 *          hist_row, 256 for ws), a negative size or a threshold that is NaN or
 *          negative, MOE_EUNSUPPORTED past the k, E, S limits.
 * The caller reads out, copies expert e*'s bytes into c's slot with
 * arena_load_slot, sets expert_slot[e*] = old slot of c and expert_slot[c] = -1
 * (moe_hot_install does it on the device), routes again without demand, and
 * orders moe_experts_forward after the copy.
 */
int moe_hot_pick(const int32_t* topk_expert, const float* topk_score, int T, int k, int E,
                 const int32_t* expert_slot, int S, int n_arena, const double* hist_row,
                 double threshold, int32_t* out, void* ws, size_t ws_bytes,
                 hipStream_t stream);

/*
 * moe_hot_install -- applies a moe_hot_pick decision to the slot table on the
 * device (TideLM README, "How adaptive expert loading works", item 3, GLM-5.3
 * bullet: the loaded expert is kept in place of the coldest one), so the
 * layer's second routing can be enqueued without the host having read the
 * decision first.
 *
 *   with (e*, c) = pick[0..1]: if 0 <= e*, c < E, e* != c, expert_slot[e*] is
 *   not in [0, S) (a miss) and 0 <= expert_slot[c] < min(n_arena, S):
 *       s = expert_slot[c]; expert_slot[e*] = s; expert_slot[c] = -1;
 *       slot_out[0] = s;
 *   otherwise the table is left as it is and slot_out[0] = -1.
 * Inputs : pick [2] int32 (device; moe_hot_pick's out); expert_slot [E] int32
 *          (device; updated in place).
 * Output : slot_out [1] int32 (device, nullable).
 * One single-thread kernel on `stream`.  The caller orders it after
 * moe_hot_pick on the same stream, copies e*'s bytes into slot s with
 * arena_load_slot, and orders moe_experts_forward (slot s deferred) after the
 * copy; kernels that run between this call and that copy route to slot s but
 * must not read its bytes.
 * Errors: MOE_EINVAL for null or misaligned (4-byte) pointers, E <= 0, S < 0 or
 * n_arena < 0; MOE_EUNSUPPORTED past the E and S limits.
 */
int moe_hot_install(const int32_t* pick, int32_t* expert_slot, int E, int S, int n_arena,
                    int32_t* slot_out, hipStream_t stream);

/*
 * moe_replan -- re-plan of one arena shared by all layers (TideLM README, "How
 * adaptive expert loading works", item 1: the arena is re-planned from the
 * demand history, so a busy layer takes slots from a quiet one).  Host function:
 * every pointer is host memory, no HIP call is made.
 *
 *   Eviction: resident pairs (l,e) (expert_slot[l*E+e] >= 0) in ascending
 *   (hist, l, e); a pair is taken unless it would leave layer l with fewer than
 *   k resident experts; stop after n_swap pairs.
 *   Loading: non-resident pairs in descending hist, ties ascending (l, e); the
 *   first n_done of them, n_done = number evicted.
 *   The i-th loaded pair receives the i-th evicted pair's slot.
 * Inputs : hist [L][E] double, expert_slot [L][E] int32 (-1 = not resident).
 * Outputs: evict, load [n_swap][2] int32 (l, e) pairs (entries beyond n_done
 *          are unspecified); new_expert_slot [L][E] (must not alias the
 *          inputs); n_done (host int) = min(evictable pairs, non-resident
 *          pairs, n_swap).
 * The caller copies each loaded pair's bytes with arena_load_slot into its
 * slot (after any kernel reading the evicted expert has finished) and installs
 * new_expert_slot on the device after the copies' events.
 * Errors: MOE_EINVAL for null pointers, L, E, k <= 0, n_swap < 0, a NaN in
 * hist, or a slot id used twice; MOE_EUNSUPPORTED if E > MOE_MAX_E or k >
 * MOE_MAX_K.
 */
int moe_replan(const double* hist, const int32_t* expert_slot, int L, int E, int k, int n_swap,
               int32_t* evict, int32_t* load, int32_t* new_expert_slot, int* n_done);

/*
 * moe_ring_plan -- one step's plan for the hot ring (TideLM README, "How
 * adaptive expert loading works", item 3, DeepSeek bullet: after each step the
 * heaviest misses are read into a ring of slots of their own while the next
 * step runs, routable from the step after until the ring wraps; every lane's
 * misses feed one plan).  One kernel on `stream`, one workgroup.
 *
 *   Candidates: pairs p = l*E + e with expert_slot[p] < 0 (not routable),
 *   not held by any ring entry, and miss_weight[p] > 0 (finite).
 *   Picks: the first min(per_step, R) candidates by larger weight, then lower
 *   p.  Pick i takes ring entry r = (head + i) mod R (global slot
 *   ring_slot0 + r); the pair the entry held before is evicted, and if
 *   expert_slot routes it to that slot it is set to -1 at once (the slot is
 *   about to be overwritten).  The new pairs are NOT made routable here: the
 *   caller copies their bytes (arena_load_slot into slot ring_slot0 + r) and
 *   then calls moe_ring_install.
 * Inputs : miss_weight [L][E] float -- the step's demand per pair (e.g. the
 *          `delta` rows moe_route wrote for each layer of the step).
 * In/out : expert_slot [L][E] int32 (the layers' slot tables, one array);
 *          ring [1 + R] int32: ring[0] = head, ring[1 + r] = pair held by
 *          entry r or -1 (start from head 0 and all -1).
 * Output : plan [1 + 3*per_step] int32: plan[0] = number of picks n, then
 *          (r, l, e) per pick.
 * The kernel runs after the step's layers in stream order, so no kernel of the
 * step still reads an evicted slot; copies into the plan's slots must wait for
 * it (an event recorded after this call).
 * Errors: MOE_EINVAL for null or misaligned pointers (4 bytes), L, E, R <= 0,
 * ring_slot0 < 0 or per_step <= 0; MOE_EUNSUPPORTED for L*E >
 * MOE_MAX_RING_PAIRS, R > MOE_MAX_RING, per_step > MOE_MAX_RING_PER_STEP or
 * ring_slot0 + R > MOE_MAX_S.
 */
int moe_ring_plan(const float* miss_weight, int32_t* expert_slot, int L, int E, int32_t* ring,
                  int R, int ring_slot0, int per_step, int32_t* plan, hipStream_t stream);

/*
 * moe_ring_install -- make a ring plan's pairs routable once their bytes are
 * in place: for each pick (r, l, e) of `plan` (as moe_ring_plan wrote it)
 * whose ring entry still holds that pair (ring[1 + r] == l*E + e),
 * expert_slot[l*E + e] = ring_slot0 + r.  Entries taken over by a later plan
 * in the meantime are skipped.  Order it after the copies' events.
 * Errors: as moe_ring_plan (plan must be non-null and 4-byte aligned).
 */
int moe_ring_install(const int32_t* plan, int32_t* expert_slot, int L, int E,
                     const int32_t* ring, int R, int ring_slot0, hipStream_t stream);

/*
 * Demand history across restarts and the arena filled from it (TideLM README,
 * "How adaptive expert loading works", item 1: every pick the router wants is
 * recorded per (layer, expert) into a history that persists across restarts;
 * the arena is filled from it at boot and re-planned after each prompt's
 * prefill, every few hundred generated tokens and between requests;
 * "Settings worth knowing": the history lives in a state file, and a
 * sensitivity setting sets how fast the resident set follows new traffic).
 *
 * History file (little-endian):
 *   bytes 0-7   magic "MOEHIST" followed by the byte 0x01
 *   bytes 8-11  L (uint32), bytes 12-15 E (uint32)
 *   bytes 16-23 tokens (uint64): routed tokens the history has seen (the
 *               caller's count; stored and returned as is)
 *   then        L*E float64, row-major [L][E], each finite and >= 0
 *   last 8      FNV-1a 64-bit hash (offset basis 0xcbf29ce484222325, prime
 *               0x100000001b3) of every byte before it
 */

/* Writes hist [L][E] (host) to `path`: to path + ".tmp" first, then renamed
 * over `path`, so a reader never sees a partly written file.  MOE_EINVAL for
 * null pointers, L or E <= 0, or a negative, NaN or infinite entry; MOE_EIO if
 * a write or the rename fails.  Host only, no HIP call. */
int moe_history_save(const char* path, const double* hist, int L, int E, uint64_t tokens);

/* Reads a history written by moe_history_save into hist [L][E] (host) and, if
 * `tokens` is non-null, its token count.  MOE_EIO if the file cannot be
 * opened or read; MOE_EFORMAT for another magic, another L or E, a short or
 * long file, a hash mismatch or an entry that is negative, NaN or infinite;
 * hist and tokens are written only on MOE_OK.  Host only. */
int moe_history_load(const char* path, double* hist, int L, int E, uint64_t* tokens);

/* The arena filled from a history at boot: expert_slot [L][E] (host output)
 * holds min(n_slots, L*E) resident pairs.  Every layer first keeps its
 * min(k, E) hottest experts (within a layer: larger history, then lower
 * expert id), so routing can always make k picks; the remaining slots go to
 * the other pairs in the order (larger history, then rank inside their layer,
 * then lower layer) -- equal histories, a fresh all-zero one above all, are
 * shared round-robin between layers.  Slots 0, 1, ... are given to the chosen
 * pairs in ascending (layer, expert); every other entry is -1.  MOE_EINVAL for
 * null pointers, L, E, k <= 0, n_slots < L*min(k, E) or a NaN in hist;
 * MOE_EUNSUPPORTED for E > MOE_MAX_E or k > MOE_MAX_K.  Host only. */
int moe_boot_plan(const double* hist, int L, int E, int k, int n_slots, int32_t* expert_slot);

/* hist[i] *= factor for i < n (device array), on `stream`: the history's
 * forgetting before a re-plan (factor 1 keeps everything; a smaller factor
 * makes the resident set follow new traffic faster).  MOE_EINVAL for a null
 * or misaligned pointer (8 bytes) or a factor outside [0, 1]. */
int moe_history_scale(double* hist, size_t n, double factor, hipStream_t stream);

/*
 * moe_test_mxfp4_probe -- test-only: one wave runs one block-scaled MXFP4
 * matrix instruction on raw per-lane operands, so a test can check the
 * hardware's decoding of E2M1 codes and E8M0 scales and its lane layout.
 * shape 0: 16x16 output, contraction 128 (lane l: row or column l%16,
 * elements 32(l/16) .. +31), d[l][0..3] used; shape 1: 32x32 output,
 * contraction 64 (lane l: row or column l%32, elements 32(l/32) .. +31),
 * d[l][0..15] used.  a, b: [64 lanes][16 bytes] codes; a_scale, b_scale:
 * [64] scale bytes; d: [64 lanes][16] floats as the lanes hold them.
 * MOE_EINVAL for another shape, a null pointer or misalignment.
 */
int moe_test_mxfp4_probe(int shape, const uint8_t* a, const uint8_t* a_scale, const uint8_t* b,
                         const uint8_t* b_scale, float* d, hipStream_t stream);

/*
 * moe_test_stream_read -- test-only microbenchmark: the achievable memory read
 * rate on this device, against which the expert kernels' rooflines are also
 * read (the vendor peak is the other).  `grid` workgroups of 256 threads read
 * src[0, bytes) once, 16 bytes per thread per load, four loads in flight per
 * thread, consecutive threads on consecutive 16-byte units; each thread
 * writes the XOR of what it read to sink[workgroup * 256 + thread] (so the
 * loads cannot be dropped).  src: device memory, 16-byte aligned, bytes a
 * positive multiple of 16; sink: device memory of grid * 256 uint32, owned by
 * the caller.  MOE_EINVAL for a null pointer, misalignment, bytes not a
 * positive multiple of 16 or grid outside [1, 65536].
 */
int moe_test_stream_read(const void* src, size_t bytes, uint32_t* sink, int grid,
                         hipStream_t stream);

/*
 * moe_test_mfma_loop -- test-only microbenchmark: the achievable rate of the
 * v_mfma_scale_f32_32x32x64_f8f6f4 instruction (the pipelined expert kernels'
 * instruction) with E2M1 A and, by act_format, E2M1 (MOE_ACT_MXFP4) or E2M3
 * (MOE_ACT_MXFP6) B operands.  `grid` workgroups of 256 threads;
 * every wave runs `iters` rounds of 8 independent accumulator chains (one
 * instruction each, 2*32*32*64 flops), so the launch does
 * grid * 4 * iters * 8 * 131072 flops; each thread writes the sum of its
 * accumulators to sink[workgroup * 256 + thread].  sink: device memory of
 * grid * 256 floats.  MOE_EINVAL for a null sink, iters outside [1, 1<<20],
 * grid outside [1, 65536] or an unknown act_format.
 */
int moe_test_mfma_loop(int iters, int act_format, float* sink, int grid, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ARENA_H */
