/*
 * epx.h -- C ABI of the MI355X (gfx950) MoE expert-parallel dispatch/combine
 * library (libepx.so).
 *
 * The operations follow "Balancing and Beyond: Communication-Centric
 * Optimizations in Expert Parallelism" (research digest) and the DeepEP
 * issues "[GH-ISSUE #250] Profiling when rank unbalance" and "Poor HybridEP
 * performance on dual-node 16x B300 GPUs". One call sequence serves one
 * source rank of an expert-parallel group on one GPU:
 *
 *   epx_get_layout   -- top-k routing -> counts, offsets and row positions
 *   epx_dispatch     -- token rows -> per-expert rows (Mode 1) or one row per
 *                       destination host (Mode 2 relay), bf16 or fp8
 *   epx_layout_dispatch -- the two above in one call (one launch for decode
 *                       batches, fewer launches for larger ones)
 *   epx_combine      -- k expert outputs per token -> weighted sum, bf16
 *   epx_relay_fanout, epx_combine_relay_partials, epx_combine_relay_finish
 *                    -- the relay's receive side and its two-level combine
 *   epx_plan_swaps   -- per-step expert swaps between GPUs of one host
 *
 * Conventions for every call:
 *  - Every array argument is a DEVICE pointer the caller allocated; the
 *    library allocates nothing and frees nothing. Its only state is the
 *    static scratch array of epx_layout_dispatch_noalloc (one per GPU), the
 *    per-thread measurement hook of epx_time_next_call and, in the
 *    bounds-checked build only, a device counter of skipped accesses.
 *    Activation pointers (x, recv, y, out) must be 16-byte aligned.
 *  - Calls are asynchronous and ordered on the HIP stream passed as `stream`
 *    (a hipStream_t; NULL = the null stream). No call synchronises the host,
 *    except epx_read_error.
 *  - Host-side argument checks fail with EPX_ERR_ARG or EPX_ERR_CAPACITY and
 *    then launch nothing. A failed kernel launch returns EPX_ERR_DEVICE.
 *  - An expert id outside [0, num_experts) is a device-side error: the
 *    layout counts such ids into totals[3]; dispatch and combine then write
 *    nothing; epx_read_error reports EPX_ERR_INDEX.
 *  - Supported sizes: 1 <= topk <= 64, topk <= num_experts <= 2048,
 *    num_experts % num_ranks == 0, num_ranks % num_hosts == 0,
 *    num_hosts <= 64, ranks per host <= 32, 0 <= my_rank < num_ranks,
 *    0 <= num_tokens <= 2^24 and num_tokens * topk < 2^31.
 */
#ifndef EPX_H
#define EPX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EPX_ABI_VERSION 4

#if defined(__GNUC__)
#define EPX_API __attribute__((visibility("default")))
#else
#define EPX_API
#endif

typedef enum {
    EPX_OK = 0,
    EPX_ERR_ARG = 1,      /* bad pointer, alignment, geometry or size     */
    EPX_ERR_INDEX = 2,    /* an expert id out of range (device-detected)  */
    EPX_ERR_CAPACITY = 3, /* an output buffer smaller than required       */
    EPX_ERR_DEVICE = 4,   /* a HIP launch or runtime call failed          */
    EPX_ERR_SCRATCH = 5   /* problem too large for the static scratch of
                             epx_layout_dispatch_noalloc                  */
} epx_status;

/* Size of the static scratch array behind epx_layout_dispatch_noalloc. */
#define EPX_NOALLOC_SCRATCH_BYTES (16u << 20)

/* Transport layout of dispatch (digest section 3.2, Figure 3).
 * PER_EXPERT: a token row for each of its destination experts (DeepEP's Mode 1).
 * HOST_RELAY: one copy per destination host, addressed to the same-index GPU
 *             on that host, plus an index to fan it out there (Mode 2 with
 *             de-redundancy). */
typedef enum { EPX_MODE_PER_EXPERT = 0, EPX_MODE_HOST_RELAY = 1 } epx_mode;

/* Row payloads. FP8_E4M3: OCP E4M3FN codes with one float32 scale per 128
 * channels (the BF16-to-FP8 conversion inside dispatch, digest section 3.1).
 * F32: float32 rows (relay partial sums only). */
typedef enum { EPX_BF16 = 0, EPX_FP8_E4M3 = 1, EPX_F32 = 2 } epx_dtype;

/* The problem of one source rank. Experts sit on ranks in contiguous
 * blocks (rank(e) = e / (num_experts/num_ranks)), ranks on hosts in
 * contiguous blocks (host(r) = r / (num_ranks/num_hosts)).
 *
 * Expert groups (per-expert overlap, digest section 3.3, Figure 4): with
 * num_groups = m > 1 the experts are split into m groups that are dispatched
 * and combined one after another; group g holds, on every rank, the local
 * experts i = e mod (E/R) with i / (E/R/m) == g, so every rank has work in
 * every group. m must divide E/R and the mode must be PER_EXPERT. 0 and 1
 * both mean no groups. */
typedef struct {
    int32_t num_tokens;   /* T: tokens of this source rank           */
    int32_t topk;         /* k: experts per token                     */
    int32_t num_experts;  /* E                                        */
    int32_t num_ranks;    /* R: expert-parallel ranks                 */
    int32_t num_hosts;    /* H: hosts the ranks are spread over       */
    int32_t my_rank;      /* s: this source rank                      */
    int32_t mode;         /* epx_mode                                 */
    int32_t num_groups;   /* m: expert groups (0 or 1: none)          */
} epx_problem;

/* Index of each layout array in the sizes reported by epx_layout_sizes. */
enum {
    EPX_L_EXPERT_COUNT = 0,  /* int32 [E]    copies per expert                                */
    EPX_L_EXPERT_OFFSET,     /* int32 [E+1]  exclusive prefix of expert_count                 */
    EPX_L_RANK_ROWS,         /* int32 [R]    copies per rank (sum over its experts)           */
    EPX_L_RANK_TOKENS,       /* int32 [R]    tokens with >= 1 expert on the rank              */
    EPX_L_RANK_OFFSET,       /* int32 [R+1]  = expert_offset[r * E/R]; -1 when m > 1          */
    EPX_L_HOST_TOKENS,       /* int32 [H]    tokens with >= 1 expert on the host (relay rows) */
    EPX_L_HOST_OFFSET,       /* int32 [H+1]  exclusive prefix of host_tokens                  */
    EPX_L_SLOT,              /* int32 [T*k]  per-expert row of pair (t, j)                    */
    EPX_L_ROW_TOKEN,         /* int32 [T*k]  source token of each per-expert row              */
    EPX_L_RELAY_SLOT,        /* int32 [T*H]  relay row of (t, h), -1 if t has no expert on h  */
    EPX_L_RELAY_TOKEN,       /* int32 [C]    source token of each relay row, -1 past the end  */
    EPX_L_FANOUT_EXPERT,     /* int32 [C*k]  expert j of the row's token if on the row's host */
    EPX_L_FANOUT_RANK_MASK,  /* uint32 [C]   bit (rank mod R/H) for each local rank to feed   */
    EPX_L_RELAY_DST_RANK,    /* int32 [H]    same-index GPU: h*(R/H) + my_rank mod (R/H)     */
    EPX_L_TOTALS,            /* int32 [4]    rows, relay rows, max expert count, bad ids      */
    EPX_L_GROUP_OFFSET,      /* int32 [m*R+1] first row of (group g, rank r) at g*R + r, total */
    EPX_L_WORKSPACE,         /* int32 [..]   scratch between the layout kernels (16-B aligned) */
    EPX_LAYOUT_NARRAYS
};

/* Device arrays of one layout. Row order (the digest fixes none):
 *  - per-expert rows: by expert, then token, then position j, so one
 *    expert's rows keep token order and one rank's rows are contiguous;
 *    with m > 1 groups, by group first: rows by (group, expert, token, j),
 *    so one group's rows are one range and, inside it, one rank's rows are
 *    contiguous (group_offset); expert_offset follows that order;
 *  - relay rows: by host, then token; a token's own host gets a row too.
 * C = T * min(k, H) is the relay row capacity (batch x k sizing of the
 * digest, section 3.4). The four relay arrays are written in HOST_RELAY mode
 * only and may be NULL in PER_EXPERT mode. */
typedef struct {
    int32_t *expert_count;
    int32_t *expert_offset;
    int32_t *rank_rows;
    int32_t *rank_tokens;
    int32_t *rank_offset;
    int32_t *host_tokens;
    int32_t *host_offset;
    int32_t *slot;
    int32_t *row_token;
    int32_t *relay_slot;
    int32_t *relay_token;
    int32_t *fanout_expert;
    uint32_t *fanout_rank_mask;
    int32_t *relay_dst_rank;
    int32_t *totals;
    int32_t *group_offset;
    int32_t *workspace;
} epx_layout;

/* Element counts (not bytes) of each layout array, indexed by EPX_L_*.
 * Host only; returns EPX_ERR_ARG for an unsupported problem. */
EPX_API epx_status epx_layout_sizes(const epx_problem *p, int64_t sizes_out[EPX_LAYOUT_NARRAYS]);

/* Counts, offsets and row positions for topk_idx [T, k] (int32, row-major):
 * copies per expert and per rank, distinct tokens per rank and per host
 * (digest sections 1-2; the per-rank receive counts of the DeepEP issue
 * "[GH-ISSUE #250] Profiling when rank unbalance"), their prefixes, the row
 * of every (token, expert) pair and, in HOST_RELAY mode, of every (token,
 * destination host) copy with its fan-out index (digest section 3.2, Mode 2,
 * Figure 3). The layout arrays are overwritten (no zeroing needed
 * beforehand); the workspace is scratch owned by the caller for the duration
 * of the call. Errors: EPX_ERR_ARG on the host (problem, pointers); ids
 * outside [0, E) are counted into totals[3] on the device and the other
 * arrays are then undefined (epx_read_error reports it). */
EPX_API epx_status epx_get_layout(const epx_problem *p, const int32_t *topk_idx,
                          const epx_layout *layout, void *stream);

/* Scatter token rows into the layout's destination rows: one copy per
 * destination expert (PER_EXPERT, the digest's Mode 1) or one copy per
 * destination host (HOST_RELAY, Mode 2 with de-redundancy; digest section
 * 3.2), optionally converted from bf16 to fp8 inside the dispatch (section
 * 3.1).
 *  x            bf16 [T, hidden], row-major
 *  out_dtype    EPX_BF16: recv is bf16 [capacity_rows, hidden];
 *               EPX_FP8_E4M3: recv is uint8 codes [capacity_rows, hidden] and
 *               recv_scales float32 [capacity_rows, hidden/128], where for
 *               token t and block b: scale = max|x[t, 128b:128b+128]| / 448
 *               (float32 division) and code = E4M3(x / scale) rounded to
 *               nearest even with saturation at +-448; an all-zero block has
 *               scale 0 and codes +-0.
 *  hidden       multiple of 8 (bf16) or of 128 (fp8)
 *  capacity_rows >= T*k (PER_EXPERT) or >= T*min(k, H) (HOST_RELAY)
 * Rows are written at the layout's slots (PER_EXPERT) or relay slots
 * (HOST_RELAY); other rows of recv are left untouched. The layout must come
 * from epx_get_layout (or epx_layout_dispatch) with the same problem, ordered
 * before this call; the host cannot check its contents, and a layout made
 * for another problem can hold rows past capacity_rows (the bounds-checked
 * build skips and counts such rows, see epx_checked_violations). Errors: EPX_ERR_ARG
 * (dtype, hidden, pointers, 16-byte alignment), EPX_ERR_CAPACITY (recv too
 * small); after a layout that saw bad ids nothing is written. */
EPX_API epx_status epx_dispatch(const epx_problem *p, const epx_layout *layout, const void *x,
                        int32_t hidden, int32_t out_dtype, void *recv, float *recv_scales,
                        int64_t capacity_rows, void *stream);

/* Combine (digest section 3.2, the combine step; section 3.4, buffers of
 * batch x k rows):
 * out[t, :] = bf16( sum_j topk_weights[t, j] * y[slot[t, j], :] ): the k
 * expert outputs of each token gathered from the per-expert rows of y
 * (bf16 [y_rows, hidden], y_rows >= T*k) and summed in float32 as
 * acc = fma(w, y, acc) for j = 0..k-1 from +0, rounded to bf16 (nearest
 * even). Weights are used as given. hidden must be a multiple of 8. The
 * layout must come from the same problem (as for epx_dispatch).
 * Errors: EPX_ERR_ARG (hidden, pointers, alignment), EPX_ERR_CAPACITY
 * (y_rows < T*k); after a layout that saw bad ids nothing is written. */
EPX_API epx_status epx_combine(const epx_problem *p, const epx_layout *layout, const void *y,
                       int64_t y_rows, const float *topk_weights, int32_t hidden, void *out,
                       void *stream);

/* Layout and dispatch in one call: the same results as epx_get_layout
 * followed by epx_dispatch on the same stream, bit for bit (every layout
 * array, recv and recv_scales; with ids outside [0, E) only totals[3] is
 * defined and nothing is dispatched). For the decode batches of the digest
 * (section 1: at most 128 tokens per GPU; section 5) the layout is small
 * enough that every dispatch workgroup recomputes the part of it that its
 * token needs, so the two steps run as one launch with no dependency between
 * workgroups: used when T <= 1024, T*k <= 4096, k <= 16 and E <= 512 (and
 * the kernel's LDS fits in 60 KB). Larger batches with k <= 16 and one
 * expert group (bf16 in either mode, fp8 in HOST_RELAY mode) take the
 * layout's count and scan launches and then one launch in which the row
 * assignment and the token copies run side by side (each token workgroup
 * derives its own rows from the scan); every other case makes the layout
 * and dispatch launches. Arguments, alignment
 * and capacity rules are those of the two calls; the layout's workspace may
 * go unused. Errors: those of either call, checked before anything is
 * launched. */
EPX_API epx_status epx_layout_dispatch(const epx_problem *p, const int32_t *topk_idx,
                                       const epx_layout *layout, const void *x, int32_t hidden,
                                       int32_t out_dtype, void *recv, float *recv_scales,
                                       int64_t capacity_rows, void *stream);

/* epx_layout_dispatch for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. The same arguments and the same results, bit for bit, except
 * that layout->workspace is not used (it may be NULL): the layout kernels'
 * scratch is instead a static device array inside the library,
 * EPX_NOALLOC_SCRATCH_BYTES (16 MiB) on every GPU the library runs on, held
 * until the process ends. Its device address is looked up on the first call
 * on each device (with that device current). Nothing in it has to start at
 * any value: every call overwrites what it reads.
 * Limit: the problem's workspace (epx_layout_sizes, EPX_L_WORKSPACE, int32
 * elements) must fit in the array, else EPX_ERR_SCRATCH before anything is
 * launched or any HIP call is made. At E = 256, top-8 that holds batches of
 * well over 100 000 tokens; decode batches (the single-launch sizes) do not
 * use it at all.
 * All calls on one GPU share its array, and it keeps the last call's
 * contents: calls that overlap on one GPU (other streams, other host
 * threads, graphs replayed concurrently) race and give undefined results.
 * Calls ordered on one stream are safe. No hipMalloc, hipFree or other
 * allocating routine is called. */
EPX_API epx_status epx_layout_dispatch_noalloc(const epx_problem *p, const int32_t *topk_idx,
                                               const epx_layout *layout, const void *x,
                                               int32_t hidden, int32_t out_dtype, void *recv,
                                               float *recv_scales, int64_t capacity_rows,
                                               void *stream);

/* ---- Expert groups (per-expert overlap, digest section 3.3, Figure 4).
 * The problem has num_groups = m > 1; call with group = 0 .. m-1.
 *
 * Dispatch of one group: epx_dispatch restricted to the pairs whose expert
 * is in `group`: recv[slot[t,j]] = x[t] (bf16, or fp8 codes + scales) for
 * those pairs only; rows of other groups are not touched. recv is the whole
 * per-expert buffer (capacity_rows >= T*k); group g's rows are
 * [group_offset[g*R], group_offset[(g+1)*R]). */
EPX_API epx_status epx_dispatch_group(const epx_problem *p, const epx_layout *layout,
                                      int32_t group, const void *x, int32_t hidden,
                                      int32_t out_dtype, void *recv, float *recv_scales,
                                      int64_t capacity_rows, void *stream);

/* Combine of one group, in ascending group order on one carry: for every
 * token with pairs in `group`, acc = (token had pairs in an earlier group) ?
 * carry[t] : +0; then for j ascending with expert idx[t,j] in the group,
 * acc = fmaf(w[t,j], y[slot[t,j]], acc); the result goes to carry[t]
 * (float32 [T, hidden]) if the token has pairs in a later group, else to
 * out[t] as bf16 (nearest even). After the last group every out row is
 * written once. Tokens without pairs in the group are not touched. With
 * m == 1 this is epx_combine and carry may be NULL. carry must be 16-byte
 * aligned; y and weights as in epx_combine. */
EPX_API epx_status epx_combine_group(const epx_problem *p, const epx_layout *layout,
                                     int32_t group, const void *y, int64_t y_rows,
                                     const float *topk_weights, int32_t hidden, float *carry,
                                     void *out, void *stream);

/* ---- Host relay, receive side and two-level combine (digest section 3.2,
 * Mode 2, Figure 3). Problem mode must be HOST_RELAY.
 * C = T * min(k, H) is the relay row capacity. ---- */

/* Fan-out at the same-index GPU of a host: every relay row r (token t) is
 * copied to the per-expert rows slot[t, j] of the token's experts j on that
 * host (fanout_expert[r, j] >= 0). dtype EPX_BF16: rows are bf16 [*, hidden];
 * EPX_FP8_E4M3: rows are uint8 codes [*, hidden] with float32 scales
 * [*, hidden/128] (relay_scales / recv_scales). relay_rows holds at least
 * relay_capacity_rows >= C rows, recv at least capacity_rows >= T*k. Applied
 * to the rows of a HOST_RELAY dispatch, recv equals what a PER_EXPERT dispatch
 * writes. */
EPX_API epx_status epx_relay_fanout(const epx_problem *p, const epx_layout *layout,
                                    const void *relay_rows, const float *relay_scales,
                                    int64_t relay_capacity_rows, int32_t hidden, int32_t dtype,
                                    void *recv, float *recv_scales, int64_t capacity_rows,
                                    void *stream);

/* Level 1, at the relay GPU: for relay row r = (t, h),
 * partials[r, :] = sum over j ascending with fanout_expert[r, j] >= 0 of
 * topk_weights[t, j] * y[slot[t, j], :], accumulated as fp32 fma from +0 and
 * stored as EPX_F32 (float32 [C, hidden]) or EPX_BF16 (rounded to nearest
 * even, bf16 [C, hidden], the compact return form). y as in epx_combine;
 * partial_capacity_rows >= C. */
EPX_API epx_status epx_combine_relay_partials(const epx_problem *p, const epx_layout *layout,
                                              const void *y, int64_t y_rows,
                                              const float *topk_weights, int32_t hidden,
                                              int32_t partial_dtype, void *partials,
                                              int64_t partial_capacity_rows, void *stream);

/* Level 2, at the source: out[t, :] = bf16( sum over hosts h ascending with
 * relay_slot[t, h] >= 0 of partials[relay_slot[t, h], :] ), fp32 adds from
 * +0, rounded to nearest even. */
EPX_API epx_status epx_combine_relay_finish(const epx_problem *p, const epx_layout *layout,
                                            const void *partials, int64_t partial_capacity_rows,
                                            int32_t partial_dtype, int32_t hidden, void *out,
                                            void *stream);

/* ---- Per-step intra-host expert swaps (digest section 3.1, Figure 2(b)).
 * Experts sit in slots: slot_expert[r * (E/R) + i] is the expert in slot i of
 * rank r (E/R slots per rank, ranks h*(R/H) .. (h+1)*(R/H)-1 on host h). The
 * load of a rank is the sum of expert_count over its slots (expert_count may
 * be a layout's EPX_L_EXPERT_COUNT). In every host the ranks are ordered by
 * load descending, then rank index; the i-th heaviest pairs with the i-th
 * lightest (i < (R/H)/2; an odd middle rank stays unpaired). Each pair takes
 * the single expert exchange that gives the smallest new pair maximum (ties:
 * smaller slot of the heavier rank, then smaller slot of the lighter rank)
 * and applies it only when the pair's maximum drops by max(tau, 1) tokens
 * or more; tau is the swap cost in token units (weight-move time over
 * per-token time).
 *
 * Device arrays: expert_count int32 [E] (non-negative, total < 2^31);
 * slot_expert_in / slot_expert_out int32 [E] (distinct buffers);
 * rank_load_before / rank_load_after int32 [R];
 * swaps int32 [H * ((R/H)/2) * 7], per pair host-major: heavy rank, its
 * expert, light rank, its expert, old maximum, new maximum, applied (0/1)
 * (may be NULL when R/H < 2); host_bad int32 [H].
 * A host whose slots hold an id outside [0, E) is not planned: its slots are
 * copied unchanged, its loads and records are -1 (applied 0) and host_bad[h]
 * is the number of such ids (0 for a planned host).
 * Limits: E <= 2048, H <= 64, R/H <= 32, tau >= 0; else EPX_ERR_ARG. */
EPX_API epx_status epx_plan_swaps(int32_t num_experts, int32_t num_ranks, int32_t num_hosts,
                                  const int32_t *expert_count, const int32_t *slot_expert_in,
                                  int32_t tau, int32_t *slot_expert_out,
                                  int32_t *rank_load_before, int32_t *rank_load_after,
                                  int32_t *swaps, int32_t *host_bad, void *stream);

/* Synchronises `stream`, then reads totals[3]: EPX_OK, or EPX_ERR_INDEX when
 * the last layout on this layout's arrays saw out-of-range expert ids (their
 * number in *bad_count if not NULL). For tests and debugging. */
EPX_API epx_status epx_read_error(const epx_layout *layout, int32_t *bad_count, void *stream);

/* Bounds-checked build (libepx_checked.so, the same sources compiled with
 * EPX_CHECKED; a debugging aid, not the product path): every row index that a
 * kernel computes, or reads from a layout, is checked against the buffer it
 * addresses (the capacities passed to the call; T*k and T*min(k, H) for the
 * layout's own arrays) before the access, and an index out of bounds skips
 * the access and is counted on the device (once per lane that skips, so the
 * count is not a number of rows). This call synchronises `stream`,
 * returns the count accumulated on the current device since the last call in
 * *count and resets it. In the release build (libepx.so) nothing is checked:
 * it returns EPX_ERR_ARG and *count = -1. Errors: EPX_ERR_ARG (count NULL, or
 * a release build), EPX_ERR_DEVICE. */
EPX_API epx_status epx_checked_violations(int64_t *count, void *stream);

/* Elementwise float32 -> E4M3FN with the rounding and saturation that the
 * fp8 dispatch uses (in [n] -> out [n], device arrays). A diagnostic entry
 * point for checking the conversion exhaustively. */
EPX_API epx_status epx_f32_to_e4m3(const float *in, uint8_t *out, int64_t n, void *stream);

/* Measurement hook. The kernels that the next library call made from this
 * host thread launches carry the two HIP events (hipEvent_t, created by the
 * caller with timing enabled) on their own dispatch packets
 * (hipExtLaunchKernel): `start_event` is recorded when that call's first
 * kernel begins and `stop_event` when its last kernel ends, so
 * hipEventElapsedTime gives the call's kernel time without the gaps that
 * event records placed around the call add. The hook applies to one call,
 * whatever it returns, and is cleared when that call returns; a call that
 * launches nothing (an error, an empty batch) leaves the events unrecorded.
 * Both NULL disarms it. Errors: EPX_ERR_ARG if exactly one is NULL. For
 * benchmarks and profiling; it changes no result. */
EPX_API epx_status epx_time_next_call(void *start_event, void *stop_event);

EPX_API const char *epx_status_string(epx_status s);
EPX_API int32_t epx_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EPX_H */
