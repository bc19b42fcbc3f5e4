/*
 * awq_moe.h -- C ABI of the AWQ int4 MoE expert stage for small-batch decode
 * (gfx950 / MI355X).
 *
 * The stage (PR #520 "[Perf][SM70] Narrow Qwen3.8 AWQ active grouped decode",
 * Purpose and Implementation; fork PR #12 "Add opt-in native-g32 AWQ QPN M1
 * dispatch", Purpose and stack): for M = 1..8 decode tokens, each with top-k
 * routed experts, compact the routed ids into active-expert segments, run
 * W13 (gate/up interleaved, K = hidden, N = 2*inter) with SwiGLU, run W2
 * (K = inter, N = hidden) and sum the expert outputs weighted by the router
 * weights. Weights are AWQ int4 with one {fp16 scale, u8 zero} record per
 * group of 32 along K, stored as 4-byte padded or 3-byte compact records
 * (PR #522 "Coalesce AWQ QPN W13 compact metadata loads and enable compact
 * metadata by default", Purpose).
 *
 * Conventions for every entry point:
 *  - Return AWQ_MOE_OK (0) or a negative error code. Arguments are checked on
 *    the host before anything is written or launched; on error nothing is
 *    written and nothing is launched (fail closed, as the pages' explicit
 *    requests do: PR #522, Default switch). awq_moe_last_error() then holds a
 *    message for the calling thread.
 *  - "device" pointers are HIP device memory owned by the caller; "host"
 *    pointers are ordinary host memory owned by the caller. The library never
 *    allocates device memory, never synchronises a stream and reads no
 *    environment variables, so the launching calls can be captured in a HIP
 *    graph.
 *  - stream is a hipStream_t passed as void* (NULL = the null stream). Kernels
 *    run asynchronously on it; a launch failure returns AWQ_MOE_EHIP.
 *  - Every call that reads a bank takes bank_bytes, the size of the caller's
 *    allocation, and fails with AWQ_MOE_ENOSPC when it is smaller than the
 *    layout of dims (so a bank packed for other dims is rejected before a
 *    kernel could read past it).
 *  - Concurrent calls that share an output or workspace buffer race.
 *
 * Bank layout (version 1; also stated in oracle/layout.py):
 *   Per expert block, four sections, each padded to 256 bytes: W13 units,
 *   W13 records, W2 units, W2 records (offsets from awq_moe_bank_layout_query).
 *   A unit = 16 bytes = the 32 4-bit values of group g of one output column:
 *   dword d (LE) holds k = 32g + 8d + p, p = 0..7, value p at bit
 *   4*(p>>1) + 16*(p&1). A record = bytes {scale lo, scale hi, zero} (+ a
 *   zero pad byte for 4-byte records). W13 column 2i is gate i, 2i+1 is up i.
 *   W13 (K = H, N = 2I) and W2 (K = I, N = H) use one tiled placement; with
 *   G = K/32 and L = 4*G, column n, group g:
 *     nt = n/16, c = n%16, quad = c/4, j = c%4, t = 4g + quad,
 *     unit at nt*256*G + (j*L + t)*16, record at nt*16*G*RB + (4t + j)*RB.
 *
 * Routing arrays (n = M*topk slots, flat slot s = t*topk + j):
 *   active_expert_ids[n]      segment -> expert id, ascending; -1 past num_active
 *   active_expert_offsets[n+1] row ranges of the segments; entries past
 *                             num_active hold V, the number of valid slots
 *   sorted_slots[n]           row -> flat slot; rows of one segment in
 *                             ascending slot order; invalid slots last
 *   num_active[1]             number of segments
 *   status[1]                 bit 0 set when some id was outside [0, E)
 *   Ids outside [0, E) are not an error of the call: their rows are left out
 *   of every segment and contribute 0 to the output.
 */
#ifndef AWQ_MOE_H
#define AWQ_MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AWQ_MOE_OK 0
#define AWQ_MOE_EINVAL (-1)       /* null pointer, misalignment, bad size or value */
#define AWQ_MOE_EUNSUPPORTED (-2) /* group size, record size or shape not served */
#define AWQ_MOE_ENOSPC (-3)       /* buffer smaller than the layout needs */
#define AWQ_MOE_EHIP (-4)         /* HIP runtime error (message has hipGetErrorString) */

#define AWQ_MOE_MAX_TOKENS 8      /* decode tokens per call, M in [1, 8] */
#define AWQ_MOE_MAX_TOPK 32
#define AWQ_MOE_MAX_HIDDEN 8192
#define AWQ_MOE_MAX_INTER 2048
#define AWQ_MOE_MAX_ROUTER_EXPERTS 4096
#define AWQ_MOE_MAX_ROUTER_ROWS 4096  /* rows of logits per awq_moe_router_topk call */
#define AWQ_MOE_STATUS_BAD_ID 1u
#define AWQ_MOE_PREFILL_MIN_TOKENS 9      /* indexed prefill tokens per call, M in [9, 4096] */
#define AWQ_MOE_PREFILL_MAX_TOKENS 4096
#define AWQ_MOE_PREFILL_MAX_EXPERTS 4096

typedef struct awq_moe_dims {
  int32_t num_experts; /* E >= 1 */
  int32_t hidden;      /* H: multiple of 32, <= AWQ_MOE_MAX_HIDDEN */
  int32_t inter;       /* I: local intermediate size, multiple of 32, <= AWQ_MOE_MAX_INTER */
  int32_t group_size;  /* must be 32 */
  int32_t meta_bytes;  /* 3 (compact records) or 4 (padded records) */
} awq_moe_dims;

typedef struct awq_moe_bank_layout {
  uint64_t w13_off;      /* section offsets inside one expert block */
  uint64_t w13_meta_off;
  uint64_t w2_off;
  uint64_t w2_meta_off;
  uint64_t expert_bytes; /* one expert block (multiple of 256) */
  uint64_t total_bytes;  /* num_experts * expert_bytes */
} awq_moe_bank_layout;

/* Fill *out with the bank layout of dims (host only). EINVAL on a null
 * pointer, EUNSUPPORTED on a shape this layout does not serve. */
int awq_moe_bank_layout_query(const awq_moe_dims* dims, awq_moe_bank_layout* out);

/* Pack logical AWQ weights into the bank layout (host -> host; pure,
 * deterministic, thread-safe). Builds the prepared banks the pages call
 * awq_sm70_prepare_compact for 3-byte records (PR #522, Default switch).
 * Orientation y = x W, all arrays C-contiguous host memory:
 *   q_gate, q_up [E][H][I] and q_down [E][I][H]: uint8, values 0..15
 *   s_gate, s_up [E][H/32][I], s_down [E][I/32][H]: fp16 bit patterns (finite)
 *   z_gate, z_up [E][H/32][I], z_down [E][I/32][H]: uint8 zeros (0..255)
 * bank: host buffer of bank_bytes >= total_bytes; every byte of the first
 * total_bytes is written (padding zero). The caller uploads it to device.
 * EINVAL on a q value > 15 or a non-finite scale (nothing written),
 * ENOSPC when bank_bytes is too small. */
int awq_moe_prepare(const awq_moe_dims* dims,
                    const uint8_t* q_gate, const uint8_t* q_up, const uint8_t* q_down,
                    const uint16_t* s_gate, const uint16_t* s_up, const uint16_t* s_down,
                    const uint8_t* z_gate, const uint8_t* z_up, const uint8_t* z_down,
                    void* bank, uint64_t bank_bytes);

/* Bytes of decode workspace for up to max_tokens tokens with topk experts
 * each (host only). */
int awq_moe_workspace_bytes(const awq_moe_dims* dims, int32_t max_tokens, int32_t topk,
                            uint64_t* out);

/* Decode workspace layout (bytes), for n = M*topk slots: the uint32 status
 * word at AWQ_MOE_WS_STATUS_OFFSET (bit 0: some id was outside [0, E)),
 * written by every W13 launch; the fp16 intermediate act[n][I], indexed by
 * flat slot, at AWQ_MOE_WS_ACT_OFFSET. A workspace sized for (max_tokens,
 * topk) serves any M <= max_tokens with the same topk; it needs no
 * initialisation. */
#define AWQ_MOE_WS_STATUS_OFFSET 0
#define AWQ_MOE_WS_ACT_OFFSET 256

/* Compact routed ids into active-expert segments (PR #520, Purpose: multi-row
 * active-expert segments with offsets-based scheduling; Implementation: the op
 * writes active_expert_ids and active_expert_offsets). All pointers device,
 * int32 topk_ids [M][topk] C-contiguous; outputs as described above, sized
 * for n = M*topk. M in [1, 8], topk in [1, 32]. */
int awq_moe_route_compact(const int32_t* topk_ids, int32_t M, int32_t topk, int32_t num_experts,
                          int32_t* active_expert_ids, int32_t* active_expert_offsets,
                          int32_t* sorted_slots, int32_t* num_active, uint32_t* status,
                          void* stream);

/* The whole stage for M = 1..8 tokens (PR #520 Purpose: 2 to 8 tokens; fork
 * PR #12 Purpose and stack: physical M = 1 with fp16 (1, hidden) x, int32
 * (1, k) ids and fp32 router weights).
 *   bank     device, 256-byte aligned; bank_bytes, the size of the caller's
 *            allocation, must be >= awq_moe_bank_layout_query(dims).total_bytes
 *            (ENOSPC otherwise: the kernels address experts by id and cannot
 *            see the allocation)
 *   x        device fp16 [M][H], 16-byte aligned
 *   topk_ids device int32 [M][topk]; topk_w device fp32 [M][topk] (used as given)
 *   out      device fp16 [M][H], 16-byte aligned, overwritten:
 *            out[t] = fp16_rne(sum_j topk_w[t][j] * W2_e(silu(x_t Wg_e) * (x_t Wu_e))),
 *            e = topk_ids[t][j] over the valid ids, accumulated in fp32 over
 *            the token's slots in ascending (expert, slot) order, so the
 *            result does not depend on the order of a token's top-k list.
 *   workspace device, 256-byte aligned, >= awq_moe_workspace_bytes(dims, M, topk);
 *            receives the status word and the fp16 intermediate.
 * Launches two kernels on stream: W13 + SwiGLU with one workgroup per
 * (slot, 16-column tile), then W2 + reduction with one workgroup per
 * (token, 16-column tile) that sums the token's slots itself. Slots that
 * share an expert read its tiles at about the same moment, so no routing
 * launch precedes them: a second read hits the L2 when it runs on the same
 * XCD and otherwise goes to the MALL or HBM (with 8 tokens drawing from
 * shared pools, W13 fetches about 1.4 times the distinct experts' bytes). */
int awq_moe_decode(const awq_moe_dims* dims, const void* bank, uint64_t bank_bytes, const uint16_t* x,
                   const int32_t* topk_ids, const float* topk_w, int32_t M, int32_t topk,
                   uint16_t* out, void* workspace, uint64_t workspace_bytes, void* stream);

/* awq_moe_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The workspace is a fixed scratch array
 * inside the library, AWQ_MOE_NOALLOC_SCRATCH_BYTES bytes per device, held
 * until the process ends; this call allocates nothing. Arguments, results and
 * kernels are those of awq_moe_decode (outputs are bit-identical), except:
 *   - ENOSPC when awq_moe_workspace_bytes(dims, M, topk) exceeds the scratch,
 *     i.e. when 256 + M*topk*inter*2 (rounded up to 256) > the maximum;
 *   - status: device uint32 [1] or NULL; when given, the status word of the
 *     call (bit 0: some id outside [0, E)) is copied there on stream.
 * Every call on one device shares that device's scratch (it keeps the last
 * call's contents and needs no clearing: each call writes what it reads), so
 * calls that overlap on one device race; serialise them on one stream. */
#define AWQ_MOE_NOALLOC_SCRATCH_BYTES (256 + 512 * 1024)
int awq_moe_decode_noalloc(const awq_moe_dims* dims, const void* bank, uint64_t bank_bytes, const uint16_t* x,
                           const int32_t* topk_ids, const float* topk_w, int32_t M, int32_t topk,
                           uint16_t* out, uint32_t* status, void* stream);

/* --- the per-M tactic table (kernel forms) ---
 * Each decode stage has several kernel forms; a constant table inside the
 * library picks one per token count M and record size (measured on the
 * rank layer; a form a shape cannot run falls back to a general rule).
 * Forms: W13 + SwiGLU 1 = lane pairs (each group split over two lanes),
 * 2 = single lanes (one 16-column tile per workgroup), 3 = single lanes,
 * two tiles per workgroup; W2 + reduction 1 = slot segments with the most
 * slots per wave, 2 = one instantiated step fewer (more waves). Form 1
 * runs the slot-segment kernel (one slot per wave from inter 288, which
 * needs top-k <= 16), from inter 544 to 1024 its two-groups-per-lane
 * variant (top-k <= 16), and otherwise a generic kernel; form 2 exists
 * where one step fewer slots per wave still fits 16 waves. 0 = the table's
 * choice. The pages' own tactic table (PR #520, Results: tile
 * tactics and the small-shape autotune) is the model. */
#define AWQ_MOE_W13_TABLE 0
#define AWQ_MOE_W13_PAIR 1
#define AWQ_MOE_W13_SINGLE 2
#define AWQ_MOE_W13_SINGLE_TWO_TILES 3
#define AWQ_MOE_W2_TABLE 0
#define AWQ_MOE_W2_SEG_MOST 1
#define AWQ_MOE_W2_SEG_FEWER 2

/* The forms awq_moe_decode uses for (dims, M, topk) (host only). */
int awq_moe_decode_table(const awq_moe_dims* dims, int32_t M, int32_t topk, int32_t* w13_form, int32_t* w2_form);

/* awq_moe_decode with the forms given instead of the table's (diagnostic:
 * per-form timing and parity). Arguments as for awq_moe_decode, plus
 * w13_form, w2_form (0 = the table's) and stages: 1 runs W13 + SwiGLU only
 * (topk_w and out unused), 2 runs W2 + reduction only, on the act the
 * workspace holds (x unused), 3 runs both. EUNSUPPORTED when a form cannot
 * run the shape. Every form gives the same result within the stage's
 * rounding (the reduction orders differ between lane pairs and single
 * lanes; two tiles per workgroup and the W2 forms are bit-identical to
 * their one-tile / most-slots counterparts). */
int awq_moe_decode_forms(const awq_moe_dims* dims, const void* bank, uint64_t bank_bytes, const uint16_t* x,
                         const int32_t* topk_ids, const float* topk_w, int32_t M, int32_t topk, uint16_t* out,
                         void* workspace, uint64_t workspace_bytes, int32_t w13_form, int32_t w2_form,
                         int32_t stages, void* stream);

/* --- stage exports, for stage-pair checks (fork PR #12, Numerical acceptance:
 * W2 checked on its own intermediate) and per-kernel timing. awq_moe_decode
 * is exactly awq_moe_w13_swiglu followed by awq_moe_w2_reduce on the same
 * workspace. */

/* W13 + SwiGLU for the routed ids topk_ids [M][topk] (device int32). Writes
 * the status word and act into workspace: act[s] =
 * fp16(silu(x_t Wg_e) * (x_t Wu_e)) for each valid flat slot s = t*topk + j
 * (rows of invalid slots are not written). One launch. */
int awq_moe_w13_swiglu(const awq_moe_dims* dims, const void* bank, uint64_t bank_bytes, const uint16_t* x,
                       const int32_t* topk_ids, int32_t M, int32_t topk,
                       void* workspace, uint64_t workspace_bytes, void* stream);

/* W2 + router-weighted reduction from the act in workspace (left there by
 * awq_moe_w13_swiglu for the same M and topk, or written by the caller;
 * workspace is only read). topk_ids device int32 [M][topk] and topk_w device
 * fp32 [M][topk] as for awq_moe_decode; out device fp16 [M][H], overwritten.
 * One launch. */
int awq_moe_w2_reduce(const awq_moe_dims* dims, const void* bank, uint64_t bank_bytes, const int32_t* topk_ids,
                      const float* topk_w, int32_t M, int32_t topk, const void* workspace,
                      uint64_t workspace_bytes, uint16_t* out, void* stream);

/* --- support for a stack of MoE layers (not part of the stage itself) --- */

/* Router top-k + softmax for M = 1..AWQ_MOE_MAX_ROUTER_ROWS rows of logits
 * (tokens, or the tokens of several layers whose logits are all known). The
 * pages leave the router
 * unchanged (fork PR #12, Purpose and stack); this is the library's reading:
 * per token, the topk largest fp32 logits, compared exactly (-0 == +0, NaN
 * below every number, ties to the lower expert id), listed by descending
 * logit, and w = softmax over the topk selected logits in fp32
 * (max-subtracted). All pointers device:
 *   logits   fp32 [M][num_experts], C-contiguous, 4-byte aligned
 *   topk_ids int32 [M][topk] out; topk_w fp32 [M][topk] out
 * num_experts in [1, AWQ_MOE_MAX_ROUTER_EXPERTS]; topk in [1, min(32,
 * num_experts)]. One launch (one wave per token). */
int awq_moe_router_topk(const float* logits, int32_t M, int32_t num_experts, int32_t topk,
                        int32_t* topk_ids, float* topk_w, void* stream);

/* One stacked pre-norm layer around the stage (the norm and the residual are
 * not on the pages; fork PR #12, Purpose and stack, leaves the rest of the
 * model unchanged): with x = r / sqrt(mean(r^2) + eps) per row and
 * out = the fp16 result of the stage on x (as awq_moe_decode computes it),
 *   r_next = fp16(r + out)     (fp32 add, one rounding)
 * Two launches, like awq_moe_decode: the W13 workgroups take their dot
 * products on r and scale each column's fp32 sum by 1/sqrt(mean(r^2) + eps)
 * (formed with the hardware reciprocal and reciprocal square root, within
 * about 2 ulp of fp32; the norm is a per-row scale; x is never rounded to
 * fp16, unlike the x of
 * awq_moe_residual_rmsnorm), computing the mean from the row they load
 * anyway; the W2 workgroups add the residual as they store. So no separate
 * norm or residual launch sits between two layers.
 *   r, r_next: device fp16 [M][hidden], 16-byte aligned, not overlapping;
 *   eps a normal float in [2^-126, 1]; the other arguments, the workspace and its contents
 *   (status word, act) as for awq_moe_decode. */
int awq_moe_decode_rmsnorm_residual(const awq_moe_dims* dims, const void* bank, uint64_t bank_bytes,
                                    const uint16_t* r, float eps, const int32_t* topk_ids, const float* topk_w,
                                    int32_t M, int32_t topk, uint16_t* r_next, void* workspace,
                                    uint64_t workspace_bytes, void* stream);

/* Residual update and parameter-free RMS norm between stacked layers (not on
 * the pages: fp16 residuals chained through many layers overflow without a
 * norm). Per row t of M = 1..8 rows, in fp32:
 *   r_next[t] = fp16_rne(r[t] + delta[t])      (delta NULL: r_next[t] = r[t])
 *   x[t]      = fp16_rne(r_next[t] / sqrt(mean(r_next[t]^2) + eps))
 * where 1/sqrt(...) is formed with the hardware reciprocal and reciprocal
 * square root (within about 2 ulp of fp32), so an x value may sit one fp16
 * ulp from the correctly rounded quotient; awq_moe_router_gemv forms its x
 * with the same formula, bit for bit.
 * r, delta, r_next, x: device fp16 [M][hidden], 16-byte aligned; hidden a
 * multiple of 8 in [8, AWQ_MOE_MAX_HIDDEN]; r_next and x must not overlap r,
 * delta or each other. eps a normal float in [2^-126, 1] (AWQ_MOE_EINVAL
 * otherwise). One launch. */
int awq_moe_residual_rmsnorm(const uint16_t* r, const uint16_t* delta, int32_t M, int32_t hidden,
                             float eps, uint16_t* r_next, uint16_t* x, void* stream);

/* awq_moe_residual_rmsnorm and awq_moe_router_topk in one launch (the two
 * per-token steps between stacked layers; one workgroup per token). The
 * results are bit-identical to the two calls; arguments and errors are the
 * union of theirs, with one M for both. */
int awq_moe_router_residual(const float* logits, int32_t M, int32_t num_experts, int32_t topk,
                            int32_t* topk_ids, float* topk_w, const uint16_t* r,
                            const uint16_t* delta, int32_t hidden, float eps, uint16_t* r_next,
                            uint16_t* x, void* stream);

/* Router GEMV between stacked layers (the router is not on the pages; fork PR
 * #12, Purpose and stack, leaves it unchanged): the residual step of
 * awq_moe_residual_rmsnorm (r_next, x, same arguments and rules), then
 *   logits[t][e] = sum_k x[t][k] * router_w[e][k]   (fp16 products, fp32 sums)
 * router_w: device fp16 [num_experts][hidden] (expert-major), 16-byte aligned;
 * logits: device fp32 [M][num_experts]. r_next and x are bit-identical to
 * awq_moe_residual_rmsnorm's. One launch; awq_moe_router_topk on logits then
 * gives the routing. */
int awq_moe_router_gemv(const uint16_t* r, const uint16_t* delta, int32_t M, int32_t hidden, float eps,
                        const uint16_t* router_w, int32_t num_experts, uint16_t* r_next, uint16_t* x,
                        float* logits, void* stream);

/* Indexed prefill: the same stage as awq_moe_decode (route, W13 + SwiGLU, W2,
 * router-weighted reduction; every reading of the decode stage holds) for
 * M in [9, 4096] tokens. PR #520 "[Perf][SM70] Narrow Qwen3.8 AWQ active
 * grouped decode", Tests: indexed prefill and grouped decode have disjoint
 * admission (boundary cases 8 and 9 tokens), so M <= 8 is EINVAL here and
 * M >= 9 is EINVAL in awq_moe_decode.
 *
 * Up to 64 tokens and 1,024 slots the call runs the decode kernels on all
 * of its tokens (two launches: W13 + SwiGLU per slot and tile, W2 per token
 * and tile), so it returns the bytes that awq_moe_decode gives on any split
 * of the tokens into calls of at most 8. Beyond, work is expert-major: each
 * distinct expert's weights are read once per call and applied to all of
 * its rows with matrix-core products, the dequantised weight kept exact as
 * the integer (q - z) and the group scale applied to the fp32 group result.
 * Row results go to an fp32 workspace and each token's rows are summed in
 * ascending (expert id, slot) order. Either way the output is
 * deterministic, bit-invariant to permuting a token's (id, weight) pairs,
 * and independent of which other tokens share the call.
 *
 * Arguments as in awq_moe_decode, with num_experts <= 4096 and
 * workspace_bytes >= awq_moe_prefill_workspace_bytes(dims, M, topk).
 * Workspace layout, with n = M*topk, X = ceil(n/32) + min(E, n),
 * W = ceil(n/64) + min(E, n) and P(b) = b rounded up to a multiple of 256,
 * each part starting where the previous one ends:
 *   [0, 256)   status u32 at 0 (bit 0: an id outside [0, E); its slot
 *              contributes 0), number of work items i32 at 4, number of
 *              wide work items i32 at 8;
 *   P(4n)      slot_row i32[n]: row of each slot, -1 for an invalid id;
 *   P(4n)      row_slot i32[n]: slot of each row (rows 0 .. valid slots - 1);
 *   P(8X)      work items i32[X][2]: {expert, first row | rows << 24}, rows
 *              <= 32, in ascending expert order, each expert's rows cut
 *              into chunks of 32 from its first row;
 *   P(8W)      wide work items i32[W][2]: the same format, ceil(c/64)
 *              items for an expert of c rows, each but the last of
 *              16*ceil(ceil(c/items)/16) rows;
 *   P(4BE), P(4B)  routing counts: with B = max(1, min(ceil(n/2048),
 *              65536/E)) workgroups, each slice's slots per expert i32[B][E]
 *              and a flag per slice (working state of the routing);
 *   P(2n*I)    fp16 act [n][inter] by row (not written when both products
 *              run in one launch: M >= 65 and inter <= 160);
 *   P(4n*H)    fp32 y [n][hidden] by row.
 * The rows of expert e are the contiguous range after the rows of all
 * lower experts (ascending expert order, as route_compact's segments); the
 * order of the rows inside that range is unspecified and no output depends
 * on it. The calls that run the decode kernels use the workspace in the
 * decode layout instead (status word at 0, act at 256) and write no routing
 * arrays. The workspace needs no initialisation. Two launches on `stream`
 * in the decode form; otherwise routing, W13 and W2 (one launch for both
 * from 65 tokens at inter <= 160), reduce, the routing taking two launches
 * above 16,384 slots; nothing is allocated and nothing synchronises, so the
 * call can be captured in a HIP graph. Calls that share a workspace must
 * not overlap. */
int awq_moe_prefill_workspace_bytes(const awq_moe_dims* dims, int32_t max_tokens, int32_t topk, uint64_t* out);
int awq_moe_prefill(const awq_moe_dims* dims, const void* bank, uint64_t bank_bytes, const uint16_t* x,
                    const int32_t* topk_ids, const float* topk_w, int32_t M, int32_t topk, uint16_t* out,
                    void* workspace, uint64_t workspace_bytes, void* stream);

/* Dequantise experts [expert_begin, expert_begin + expert_count) of the bank
 * into fp32 (diagnostic). Each value s * (q - z) is exact in fp32: q - z is an
 * integer in [-255, 15] and s an fp16, so the product needs at most 19
 * significant bits.
 *   which = 0: W13 [count][H][2I] (column 2i gate, 2i+1 up)
 *   which = 1: W2  [count][I][H]
 * out device fp32, C-contiguous. */
int awq_moe_dequant(const awq_moe_dims* dims, const void* bank, uint64_t bank_bytes, int32_t expert_begin,
                    int32_t expert_count, int32_t which, float* out, void* stream);

/* Message for the last error returned on the calling thread ("" if none). */
const char* awq_moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* AWQ_MOE_H */
