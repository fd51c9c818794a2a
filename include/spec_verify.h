/*
 * spec_verify.h -- C ABI of the MI355X (gfx950) batched lossless draft
 * verification library, libspecverify.so.
 *
 * Operations:
 *
 *   spec_verify         speculative-sampling verification of a batch of draft
 *                       blocks against the target's logits.
 *   spec_verify_packed  the same over densely packed target rows (each
 *                       request's kept positions only).
 *   spec_verify_logits  the same with the draft distribution given as logits
 *                       (its softmax at the call's temperature).
 *   spec_verify_tree    greedy verification of a candidate tree (the
 *                       acceptance walk after the target's ancestor-masked
 *                       pass over the flattened tree).
 *   spec_schedule       confidence-scheduled verification depth: how many
 *                       drafts of each request to verify under a batch token
 *                       budget.
 *   spec_schedule_calibrated  the same on temperature-calibrated confidences.
 *   spec_dcut           ratio-budgeted verification depth: the budget ratio
 *                       with the best estimated progress per profiled cost,
 *                       its keep depths and the packed row offsets.
 *   spec_acceptance     per-position acceptance overlap alpha = sum min(p, q)
 *                       (= 1 - TV), the expected acceptance of each draft.
 *   spec_schedule_static  the static scheduler: a fixed length, or the leading
 *                       drafts whose confidence exceeds a threshold.
 *   spec_sts_fit        Sequential Temperature Scaling: per-position
 *                       temperatures fitted left to right on acceptance data;
 *                       spec_schedule_calibrated, spec_dcut and
 *                       spec_schedule_static apply them (calib_temps) as they
 *                       load confidences.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensors are row-major and contiguous.  Pointers named "device" point
 *   to memory on the current HIP device; host pointers are never read.
 * - `stream` is a hipStream_t passed as an opaque pointer (NULL = the null
 *   stream).  Calls are asynchronous: they validate their arguments on the
 *   host, enqueue kernels on `stream` and return.  Outputs are valid once the
 *   caller has synchronised the stream.  No call allocates or frees memory,
 *   synchronises, or keeps state between calls; every call may be captured
 *   into a HIP graph.
 * - Host-checkable errors (null pointers, bad sizes, bad temperature, bad
 *   dtype, misalignment, small workspace) return a status before anything is
 *   enqueued, and every output is left untouched.  A failed kernel launch
 *   returns SPEC_ERR_DEVICE.
 * - Data errors found on the device do not stop the batch: the affected
 *   request's outputs are set to -1 and the other requests are processed.
 * - The caller owns every buffer.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SPEC_OK = 0,
    SPEC_ERR_NULL_POINTER = 1,        /* a required pointer is NULL                     */
    SPEC_ERR_BAD_SHAPE = 2,           /* B, G, V, table or budget out of range           */
    SPEC_ERR_BAD_TEMPERATURE = 3,     /* temperature < 0, not finite, or too small       */
    SPEC_ERR_BAD_DTYPE = 4,           /* unknown dtype code                              */
    SPEC_ERR_WORKSPACE_TOO_SMALL = 5, /* workspace_bytes < the *_workspace_bytes query   */
    SPEC_ERR_UNSUPPORTED = 6,         /* valid but beyond this build's limits            */
    SPEC_ERR_DEVICE = 7,              /* HIP error while querying the device or launching */
    SPEC_ERR_MISALIGNED = 8,          /* a pointer is not aligned to its element type /
                                         the workspace is not 256-byte aligned           */
    SPEC_ERR_SCRATCH_TOO_SMALL = 9    /* spec_verify_noalloc: the shape needs more than
                                         SPEC_NOALLOC_SCRATCH_BYTES of workspace          */
} spec_status_t;

typedef enum { SPEC_DTYPE_F32 = 0, SPEC_DTYPE_BF16 = 1 } spec_dtype_t;

/* How the draft distribution is given: float32 probabilities, or logits of
 * the target's dtype whose softmax at the call's temperature is the draft
 * distribution. */
typedef enum { SPEC_DRAFT_PROBS = 0, SPEC_DRAFT_LOGITS = 1 } spec_draft_kind_t;

/* Modes of spec_schedule_static. */
typedef enum { SPEC_STATIC_FIXED = 0, SPEC_STATIC_THRESHOLD = 1 } spec_static_mode_t;

/*
 * Calibration (the calib_temps argument of spec_schedule_calibrated, spec_dcut
 * and spec_schedule_static): NULL, or a host array
 * of G finite, positive per-position temperatures T_k ("UraionSpec", section
 * "Sequential Temperature Scaling").  Confidence c[b,k] is then read as
 * c~ = float32(c^(1/T_k)), formed in double as 2^(log2(c) / T_k), before any
 * other use.  Validated on the host (SPEC_ERR_BAD_SHAPE) and passed by value.
 */

/* A hipStream_t, passed opaquely so that this header needs no HIP include. */
typedef void *spec_stream_t;

/* Limits of this build. */
#define SPEC_MAX_BATCH 65536          /* B <= 65536 for spec_verify                      */
#define SPEC_MAX_DRAFTS 255           /* G <= 255                                        */
#define SPEC_MAX_VOCAB (1 << 30)      /* V <= 2^30                                       */
#define SPEC_MAX_SCHEDULE_CANDIDATES 4096 /* B, B * G <= 4096 for spec_schedule, spec_dcut */
#define SPEC_MAX_RATIOS 8             /* budget ratios per spec_dcut call                */

/*
 * Optional diagnostics of spec_verify.  Each field may be NULL.
 *
 * The four arrays are for parity checks (they cost extra stores; keep them
 * NULL on a timed path).  Device pointers.  Entries that a request does not
 * compute are set to NaN; for a request with a data error every entry is NaN.
 * Temperature 0 writes none of them.
 *
 *   target_lse [B, G+1]  m_k/T + ln S_k of each read target row k <= len_b
 *   p_draft    [B, G]    p_k(x_k), the target probability of draft k, k < len_b
 *   q_draft    [B, G]    q_k(x_k) as read from draft_probs, k < len_b
 *   resid_mass [B]       R = sum_v max(p_j(v) - q_j(v), 0) at the rejection
 *                        row j; -1 when every verified draft was accepted
 *
 * row_pass_event is a hipEvent_t (opaque) created by the caller, for timing:
 * the call records it on `stream` right after the launch that reads the target
 * rows: after the row launch when the call makes two launches, else after its
 * single launch.  It costs one event record and no extra memory traffic.
 */
typedef struct {
    float *target_lse;
    float *p_draft;
    float *q_draft;
    float *resid_mass;
    void *row_pass_event;
} spec_verify_diag_t;

/*
 * Bytes of device workspace spec_verify needs for this shape (0 on invalid
 * arguments).  The same workspace serves every shape whose query is not larger.
 *
 * The workspace holds the per-row partial sums (target rows, and draft rows
 * for spec_verify_logits), the per-draft gathers and the per-request sub-tile
 * masses; every verify entry point takes it.  It must be zero-filled once before its first use (e.g.
 * allocated with a zeroing allocator); every completed call leaves it
 * zero-filled again, so one workspace can serve later calls of any shape
 * without clearing.  Calls that share one workspace must not overlap in time
 * (use one per stream).
 */
size_t spec_verify_workspace_bytes(int32_t B, int32_t G, int32_t V, spec_dtype_t target_dtype);

/*
 * spec_verify -- batched lossless speculative-sampling verification.
 *
 * Operation ("breaking down dspark and its lineage", sections "Speculative
 * decoding basics: drafting and verification" and "Preserving the target
 * distribution during verification"; "UraionSpec", section "Speculative
 * Decoding", Eq. (acceptance); "AngelSpec", sections 1 and 4.1):
 * for request b with verify length n = len_b,
 *   p_k = softmax(z[b,k,:] / T) for target rows k = 0..n (row k is the target's
 *         distribution after k accepted drafts; row n supplies the bonus token);
 *   draft k < n is accepted iff u[b,k] < p_k(x_k) / q[b,k,x_k]  (if
 *         q[b,k,x_k] <= 0: accepted iff p_k(x_k) > 0);
 *   j = the first rejected k, or n if none;
 *   if j < n the final token is drawn from r = max(p_j - q[b,j,:], 0),
 *   else from r = p_n;  y = min{v : sum_{w<=v} r(w) > u[b,G] * sum_w r(w)}
 *   (if r sums to zero, p_j is used; if no index qualifies, the largest v
 *   with r(v) > 0);
 *   out_accepted[b] = j;  out_tokens[b,:] = x[b,0..j-1], y, then -1.
 * Temperature 0 is the greedy limit: a_k = lowest index of the maximum of
 * row k (exact comparison); draft k is accepted iff x_k == a_k; y = a_j.
 *
 * Arguments (all device pointers unless stated):
 *   target_logits  [B, G+1, V] of target_dtype (F32 or BF16).  Only rows
 *                  k <= len_b of each request are read.
 *   draft_probs    [B, G, V] float, the distribution each draft token was
 *                  sampled from; used as given.  May be NULL if T == 0 or G == 0.
 *   draft_tokens   [B, G] int32 in [0, V).  May be NULL if G == 0.
 *   uniforms       [B, G+1] float in [0, 1): u[b,k], k < G, decides draft k;
 *                  u[b,G] is the final draw.  May be NULL if T == 0.
 *   verify_len     [B] int32 in [0, G], or NULL meaning G for every request.
 *   1 <= B <= SPEC_MAX_BATCH, 0 <= G <= SPEC_MAX_DRAFTS, 1 <= V <= SPEC_MAX_VOCAB.
 *   temperature    T == 0 (greedy) or 2^-126 <= T < inf.
 *   out_accepted   [B] int32: accepted drafts j in [0, len_b]; -1 = data error.
 *   out_tokens     [B, G+1] int32.
 *   diag           host pointer to a spec_verify_diag_t, or NULL.
 *   workspace      device, 256-byte aligned, zero-filled before first use, at
 *                  least spec_verify_workspace_bytes(B, G, V, target_dtype).
 *
 * Data errors (outputs of that request all -1): len_b outside [0, G]; a draft
 * token outside [0, V) at a verified position; a read target row that holds a
 * NaN, whose maximum is +inf, or which is entirely -inf.
 */
spec_status_t spec_verify(const void *target_logits, spec_dtype_t target_dtype,
                          const float *draft_probs, const int32_t *draft_tokens,
                          const float *uniforms, const int32_t *verify_len,
                          int32_t B, int32_t G, int32_t V, float temperature,
                          int32_t *out_accepted, int32_t *out_tokens,
                          const spec_verify_diag_t *diag,
                          void *workspace, size_t workspace_bytes, spec_stream_t stream);

/*
 * spec_verify_packed -- spec_verify over densely packed target rows.
 *
 * Operation ("AngelSpec", section 4.2, "Packing and correctness"): the kept
 * prefixes of all requests form one dense batch of target positions, and each
 * kept token is verified exactly as by spec_verify.  Request b's target rows
 * are packed rows row_offsets[b] .. row_offsets[b+1]-1, its positions 0..n_b in
 * order, so its verify length is n_b = row_offsets[b+1] - row_offsets[b] - 1.
 * The result equals spec_verify on the unpacked rows with verify_len = n.
 *
 * Arguments as for spec_verify, except:
 *   target_logits  [rows, V] of target_dtype; rows >= 1 is the number of rows
 *                  the buffer holds (rows past the last request are not read).
 *   row_offsets    [B+1] int32, device (e.g. spec_dcut's out_row_offsets).
 *   There is no verify_len.  Workspace: spec_verify_workspace_bytes(B, G, V, dtype).
 *   Diagnostics are indexed by (request, position) as for spec_verify.
 *
 * Data errors (outputs of that request all -1): row_offsets[b] < 0,
 * row_offsets[b+1] > rows, or n_b outside [0, G]; and the data errors of
 * spec_verify.
 */
spec_status_t spec_verify_packed(const void *target_logits, spec_dtype_t target_dtype, int32_t rows,
                                 const int32_t *row_offsets, const float *draft_probs,
                                 const int32_t *draft_tokens, const float *uniforms,
                                 int32_t B, int32_t G, int32_t V, float temperature,
                                 int32_t *out_accepted, int32_t *out_tokens,
                                 const spec_verify_diag_t *diag,
                                 void *workspace, size_t workspace_bytes, spec_stream_t stream);

/*
 * spec_verify_logits -- spec_verify with draft logits instead of draft
 * probabilities.
 *
 * Operation ("AngelSpec", section 2, Eq. 2; the verification rule as for
 * spec_verify): the draft distribution of position k is
 * q_k = softmax(draft_logits[b,k,:] / T) at the call's temperature, formed on
 * the device: the row pass also reduces every verified draft row (max and
 * exp-sum), the accept test uses q_k(x_k) from that normaliser, and the
 * residual max(p_j - q_j, 0) reads draft row j's logits.
 *
 * Arguments as for spec_verify, except draft_logits [B, G, V] of target_dtype
 * (rows k < len_b are read; may be NULL if T == 0 or G == 0) in place of
 * draft_probs.  Workspace: spec_verify_workspace_bytes.  diag->q_draft returns
 * q_k(x_k) computed from the logits.
 *
 * Data errors: those of spec_verify, and a verified draft row (k < len_b) that
 * holds a NaN, whose maximum is +inf, or which is entirely -inf.
 */
spec_status_t spec_verify_logits(const void *target_logits, spec_dtype_t target_dtype,
                                 const void *draft_logits, const int32_t *draft_tokens,
                                 const float *uniforms, const int32_t *verify_len,
                                 int32_t B, int32_t G, int32_t V, float temperature,
                                 int32_t *out_accepted, int32_t *out_tokens,
                                 const spec_verify_diag_t *diag,
                                 void *workspace, size_t workspace_bytes, spec_stream_t stream);

/*
 * spec_verify_tree -- greedy (temperature 0) verification of a candidate tree.
 *
 * Operation ("breaking down dspark and its lineage", section "Tree
 * attention"): the candidates of request b form a tree of M nodes; node 0 is
 * the root (the last committed token), node i >= 1 carries token
 * node_tokens[b,i] and parent parents[b,i] < i.  target_logits[b,i,:] is the
 * target's next-token distribution after the path root..i (one target pass over
 * the flattened tree with an ancestor-only mask).  From the root, the walk
 * moves to the child of the current node whose token equals the lowest-index
 * argmax of the current node's row (the lowest-numbered child if several
 * carry it) and stops when none does.  This emits exactly what greedy
 * decoding of the target would.
 *   out_accepted[b] = accepted path length;
 *   out_tokens[b,:] = the accepted tokens, then the argmax at the last node
 *                     (the bonus), then -1;
 *   out_path[b,:]   = the accepted node indices after the root, then -1.
 * Sampled acceptance over several candidates is not defined on the pages and
 * not provided.
 *
 * Arguments (device pointers): target_logits [B, M, V] of target_dtype;
 * parents, node_tokens [B, M] int32 (entry 0 ignored; may be NULL if M == 1);
 * 1 <= M <= SPEC_MAX_DRAFTS + 1; out_accepted [B], out_tokens [B, M],
 * out_path [B, M] int32; workspace of spec_verify_workspace_bytes(B, M - 1, V,
 * target_dtype).  One launch while B is at most half the workgroups the
 * device holds at once (the greedy row pass over every node row, then one
 * workgroup per request that waits for its rows' partials); else two launches
 * (the row pass, then the walks).
 *
 * Data errors (that request's outputs all -1): a parent outside [0, i) or a
 * token outside [0, V) at some node i >= 1; a visited row (the root or a node
 * on the accepted path) that holds a NaN, whose maximum is +inf, or which is
 * entirely -inf.
 */
spec_status_t spec_verify_tree(const void *target_logits, spec_dtype_t target_dtype,
                               const int32_t *parents, const int32_t *node_tokens,
                               int32_t B, int32_t M, int32_t V,
                               int32_t *out_accepted, int32_t *out_tokens, int32_t *out_path,
                               void *workspace, size_t workspace_bytes, spec_stream_t stream);

/*
 * Number of kernel launches spec_verify makes for this shape on the current
 * device, with 16-byte-aligned target_logits and verify_len NULL: for T > 0,
 * 1 (the row workgroups, a decision workgroup per request and the request
 * workgroups share one grid, also with verify lengths; spec_verify_logits,
 * with draft logits, makes 2: the pass over the read rows, then the
 * per-request pass); for T == 0, 1 when the per-request work
 * shares the row launch and 2 when it runs as a second launch.  -1 on invalid
 * arguments or a failed device query.  Host-only; enqueues nothing.
 */
int32_t spec_verify_launches(int32_t B, int32_t G, int32_t V, spec_dtype_t target_dtype, float temperature);

/* Workspace bytes held by spec_verify_noalloc's static scratch (per GPU). */
#define SPEC_NOALLOC_SCRATCH_BYTES (8u << 20)

/*
 * spec_verify_noalloc -- spec_verify for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same operation, arguments, outputs and errors as
 * spec_verify, without the workspace arguments.
 *
 * The workspace is a static device array of SPEC_NOALLOC_SCRATCH_BYTES inside
 * the library; each GPU the library runs on holds its own copy until the
 * process ends.  The call allocates nothing (no hipMalloc, no allocating
 * library routine); on its first use on a device it looks up that device's
 * address of the array.  Each call clears the part of the array it uses (a
 * fill kernel on `stream`) and then launches exactly what spec_verify does.
 *
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (on two streams, or from two host threads) race and must not be
 * made.  A shape whose spec_verify_workspace_bytes exceeds
 * SPEC_NOALLOC_SCRATCH_BYTES (about B = 490 requests at G = 15, V = 129280,
 * bf16) returns SPEC_ERR_SCRATCH_TOO_SMALL before anything is enqueued.
 */
spec_status_t spec_verify_noalloc(const void *target_logits, spec_dtype_t target_dtype,
                                  const float *draft_probs, const int32_t *draft_tokens,
                                  const float *uniforms, const int32_t *verify_len,
                                  int32_t B, int32_t G, int32_t V, float temperature,
                                  int32_t *out_accepted, int32_t *out_tokens,
                                  const spec_verify_diag_t *diag, spec_stream_t stream);

/* Bytes of device workspace spec_schedule needs (currently 0: it works in LDS). */
size_t spec_schedule_workspace_bytes(int32_t B, int32_t G);

/*
 * spec_schedule -- confidence-scheduled verification depth.
 *
 * Operation ("AngelSpec", section 4.2, Eq. 19-21 and the tie rule after them;
 * "UraionSpec", section "Hardware-Aware Prefix Scheduler", Algorithm 1;
 * "breaking down dspark and its lineage", section "Verify smarter, not longer"),
 * in float64:
 *   s[b,k] = prod_{t=0..k} c[b,t]  (survival of draft k+1);
 *   candidates (b,k) with s[b,k] > eps, ordered by s descending, then k
 *   ascending, then b ascending;
 *   len = 0, T = B, tau = B, best = tau / cost[T];
 *   for each candidate in order: skip it unless len_b == k; stop if
 *   T + 1 > token_budget; theta = (tau + s[b,k]) / cost[T+1]; if theta > best
 *   keep it (len_b = k+1, T += 1, tau += s[b,k], best = theta), else stop.
 * The result is bit-identical to that sequential loop in float64.
 * Confidences are used as given; spec_schedule_calibrated applies per-position
 * temperatures first.
 *
 * Arguments (device pointers unless stated):
 *   confidence          [B, G] float, per-draft acceptance estimates in [0, 1].
 *   cost_table          [table_len] float, cost of one verification step with
 *                       T positions, T = 0..table_len-1 (1/steps-per-second);
 *                       entries T = B..token_budget must be positive.
 *   B >= 1, G >= 0, B*G <= SPEC_MAX_SCHEDULE_CANDIDATES,
 *   B <= token_budget < table_len, eps finite.
 *   out_verify_len      [B] int32 in [0, G]: feed to spec_verify's verify_len.
 *   out_total_tokens    [1] int32: T = sum_b (len_b + 1).
 *   out_expected_tokens [1] float: tau = B + sum of kept survivals, or NULL.
 *   workspace           may be NULL when spec_schedule_workspace_bytes is 0.
 */
spec_status_t spec_schedule(const float *confidence, const float *cost_table, int32_t table_len,
                            int32_t B, int32_t G, int32_t token_budget, float eps,
                            int32_t *out_verify_len, int32_t *out_total_tokens,
                            float *out_expected_tokens,
                            void *workspace, size_t workspace_bytes, spec_stream_t stream);

/*
 * spec_schedule_calibrated -- spec_schedule on calibrated confidences
 * ("UraionSpec", section "Sequential Temperature Scaling", applied before the
 * prefix scheduler of section "Hardware-Aware Prefix Scheduler").
 *
 * Exactly spec_schedule with every confidence c[b,k] replaced by
 * c~ = float32(c^(1/T_k)) (see "Calibration" above), where calib_temps is a
 * host array of G finite, positive temperatures (e.g. spec_sts_fit's output,
 * copied to the host).  calib_temps == NULL is spec_schedule itself.  The
 * other arguments, outputs and errors are those of spec_schedule; an invalid
 * temperature returns SPEC_ERR_BAD_SHAPE before anything is enqueued.
 */
spec_status_t spec_schedule_calibrated(const float *confidence, const float *calib_temps,
                                       const float *cost_table, int32_t table_len,
                                       int32_t B, int32_t G, int32_t token_budget, float eps,
                                       int32_t *out_verify_len, int32_t *out_total_tokens,
                                       float *out_expected_tokens,
                                       void *workspace, size_t workspace_bytes, spec_stream_t stream);

/*
 * spec_dcut -- ratio-budgeted verification depth (D-cut).
 *
 * Operation ("AngelSpec", section 4.2, Eq. 20-24), in float64:
 *   score of request b's position k: s[b,0] = 1 (the bonus position) and
 *   s[b,k] = prod_{t<k} c[b,t], k = 1..G, with each confidence clamped into
 *   [0, 1] (NaN as 0);
 *   for each ratio rho_r: K_r = max(B, ceil(rho_r * B * (G+1))) (rho_r * B(G+1)
 *   formed exactly in double); the K_r best scores of the batch, equal scores
 *   ranked shallower position first, then lower b, are kept: a prefix of
 *   n_b^r + 1 positions of every request;
 *   U_r = sum_b sum_{k<=n_b^r} s[b,k], the estimated progress;
 *   the chosen ratio r* is the first with the largest U_r / cost_r;
 *   out_verify_len[b] = n_b^{r*}; out_row_offsets = the exclusive prefix of
 *   n_b + 1 (row_offsets[B] = K_{r*}), the packed layout spec_verify_packed reads.
 * Keep depths, offsets and K are exact.  U_r is summed per request in position
 * order, then over requests in a fixed tree order, so it can differ from a
 * sequential sum in the last bits; r* can then differ only between ratios
 * whose U / cost agree to about 1e-15 relative.
 *
 * Arguments:
 *   confidence       [B, G] float, device (may be NULL when G == 0).
 *   ratios           [num_ratios] float, host, each in (0, 1], e.g.
 *                    {0.25, 0.5, 0.75, 1}.
 *   ratio_cost       [num_ratios] float, host, each finite and > 0: the
 *                    profiled cost of one step at this batch size and ratio.
 *   1 <= num_ratios <= SPEC_MAX_RATIOS; B >= 1, G >= 0,
 *   B, B*G <= SPEC_MAX_SCHEDULE_CANDIDATES.
 *   out_verify_len   [B] int32, device: n_b in [0, G].
 *   out_row_offsets  [B+1] int32, device.
 *   out_ratio_index  [1] int32, device: r*.
 *   out_total_rows   [1] int32, device: K_{r*} = sum_b (n_b + 1).
 *   out_utility      [num_ratios] double, device, or NULL: U_r.
 *   calib_temps      see "Calibration" above (applied before the clamp).
 * Needs no workspace.
 */
spec_status_t spec_dcut(const float *confidence, int32_t B, int32_t G,
                        const float *ratios, const float *ratio_cost, int32_t num_ratios,
                        const float *calib_temps, int32_t *out_verify_len, int32_t *out_row_offsets,
                        int32_t *out_ratio_index, int32_t *out_total_rows,
                        double *out_utility, spec_stream_t stream);

/*
 * spec_acceptance -- per-position acceptance diagnostics.
 *
 * Operation ("AngelSpec", section 2, Eq. 2, 4 and 5; "UraionSpec", the
 * confidence head's training target): for every tested position k < len_b,
 *   alpha[b,k] = sum_v min(p_k(v), q_k(v)),  p_k = softmax(z[b,k,:] / T),
 * where q_k is draft[b,k,:] as given (SPEC_DRAFT_PROBS) or
 * softmax(draft[b,k,:] / T) (SPEC_DRAFT_LOGITS).  alpha is the expected
 * probability that draft k is accepted; TV(p_k, q_k) = 1 - alpha and the
 * confidence target c*_k = alpha.
 * NaN where k >= len_b, for every position of a request whose verify length is
 * outside [0, G], and where target row k or draft row k (logits) holds a NaN,
 * has maximum +inf or is entirely -inf.  Sums are fp32 per eight elements and
 * fp64 beyond (about 1e-6 absolute).
 *
 * Arguments (device pointers): target_logits [B, G+1, V] of target_dtype (rows
 * k < len_b are read); draft [B, G, V]: float32 probabilities, or logits of
 * target_dtype; verify_len [B] or NULL (= G); T finite, >= 2^-126;
 * out_alpha [B, G] float.  Shape limits as spec_verify.  Needs no workspace.
 */
spec_status_t spec_acceptance(const void *target_logits, spec_dtype_t target_dtype,
                              const void *draft, spec_draft_kind_t draft_kind,
                              const int32_t *verify_len, int32_t B, int32_t G, int32_t V,
                              float temperature, float *out_alpha, spec_stream_t stream);

/*
 * spec_schedule_static -- the static scheduler ("UraionSpec", the fallback
 * scheduler's fixed-length and static-threshold modes; "breaking down dspark
 * and its lineage", section "Verify smarter, not longer": threshold 0 is
 * fixed-length verification).
 *   SPEC_STATIC_FIXED:     len_b = min(max(fixed_len, 0), G) (confidence unused,
 *                          may be NULL);
 *   SPEC_STATIC_THRESHOLD: len_b = the number of leading drafts whose
 *                          (calibrated) confidence exceeds threshold, i.e. the
 *                          first k with c~[b,k] <= threshold, else G.
 * Outputs (device): out_verify_len [B]; out_total_tokens [1] = sum (len_b + 1)
 * or NULL; out_row_offsets [B+1] (the packed layout of spec_verify_packed) or
 * NULL.  1 <= B <= SPEC_MAX_BATCH, 0 <= G <= SPEC_MAX_DRAFTS; threshold not NaN.
 */
spec_status_t spec_schedule_static(const float *confidence, int32_t B, int32_t G, spec_static_mode_t mode,
                                   int32_t fixed_len, float threshold, const float *calib_temps,
                                   int32_t *out_verify_len, int32_t *out_total_tokens,
                                   int32_t *out_row_offsets, spec_stream_t stream);

/*
 * spec_sts_fit -- Sequential Temperature Scaling fit ("UraionSpec", section
 * "Sequential Temperature Scaling"): for k = 0..G-1 in order, over the grid
 * temps[0..num_temps-1], the expected calibration error with `bins`
 * equal-width bins on [0, 1] of a_n(T) = prefix_n * c[n,k]^(1/T) against the
 * cumulative labels y_n = [acc_len[n] > k] is
 *   ECE(T) = (1/N) sum_bins |sum_{n in bin} a_n - sum_{n in bin} y_n|,
 *   bin = min(floor(bins * a), bins - 1);
 * out_temps[k] = the first grid point with the least ECE, and prefix_n gains
 * c[n,k]^(1/T_k) (prefix starts at 1; powers in double as 2^(log2(c) * (1/T))).
 * Confidences are clamped into [0, 1] (NaN as 0).  Prediction sums are exact
 * in 2^-40 fixed point, so the result does not depend on the order of
 * accumulation.  The usual grid is 100 points, linspace(0.1, 10, 100), with
 * 15 bins.
 *
 * Arguments: confidence [N, G] float and acc_len [N] int32 (accepted drafts per
 * sample), device; temps host, each finite and > 0; 1 <= N < 2^23,
 * 1 <= num_temps <= 128, 1 <= bins <= 32 (so num_temps * bins <= 4096);
 * out_temps [G] float, device; workspace device, 256-byte aligned, at least
 * spec_sts_fit_workspace_bytes(N, G, num_temps, bins) (0 on invalid shapes).
 * 3 launches per position.
 */
size_t spec_sts_fit_workspace_bytes(int32_t N, int32_t G, int32_t num_temps, int32_t bins);
spec_status_t spec_sts_fit(const float *confidence, const int32_t *acc_len, int32_t N, int32_t G,
                           const float *temps, int32_t num_temps, int32_t bins, float *out_temps,
                           void *workspace, size_t workspace_bytes, spec_stream_t stream);

/* Static, NUL-terminated description of a status code. */
const char *spec_status_string(spec_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
