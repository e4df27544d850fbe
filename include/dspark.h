/*
 * dspark.h -- C ABI of the MI355X (gfx950) DSpark draft-head-and-verify chain.
 *
 * One decode step of DSpark's confidence-scheduled speculative decoding, as
 * five calls that run on the caller's HIP stream:
 *
 *   dspark_markov_draft   draft a gamma-token block with the Markov head
 *   dspark_confidence     confidence c_k and prefix survival a_{r,j}
 *                         (dspark_markov_draft_confidence: both in one call)
 *   dspark_schedule_topb  global top-B prefix selection (verify windows)
 *   dspark_pack_ragged    cu_seqlens packing rounded up to a capture tier
 *                         (dspark_schedule_pack: schedule and pack in one launch)
 *   dspark_verify         lossless rejection-sampling verification
 *
 * a sixth, dspark_advance, that carries a decode loop from one step to the
 * next on the device, two observability calls (dspark_observe,
 * dspark_analytic_accept), plus host/device utilities (W2 pre-packing, cost-table preparation,
 * workspace sizing and initialisation, status strings) and one diagnostic
 * call.
 *
 * Sources, cited by page title and section:
 *   [digest]  "DSpark: Confidence-Scheduled Speculative Decoding with
 *             Semi-Autoregressive Generation", technical digest
 *             (zhao9797.github.io).
 *   [sglang]  "SGLang integrates DSpark" blog (aihot.vn; Chinese copy at
 *             aihot.virxact.com).
 *   [vllm]    "vLLM adaptive verification with DSpark" (agentlenshq.com).
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked [host]. The caller allocates
 *     and owns every buffer; the library never allocates, frees or
 *     synchronises inside a call, and keeps no state besides a per-device
 *     cache of the compute-unit count.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Each
 *     call enqueues its kernels on it and returns at once; outputs are valid
 *     once the stream has reached that point.
 *   - Arrays are row-major and contiguous. Token ids are int32 in [0, V).
 *   - dtype selects the storage type of the large float inputs (U, W1, W2,
 *     h, target logits): DSPARK_F32 (float32) or DSPARK_BF16 (bfloat16 bit
 *     patterns, 2 bytes). All arithmetic is float32 (bf16 products are exact
 *     in fp32; sums accumulate in fp32).
 *   - Arguments are checked on the host. A failed check returns a negative
 *     dspark_status and launches nothing. Device-side preconditions (token ids
 *     in range, a monotone cost table) are not checked; violating them gives
 *     unspecified values but no out-of-bounds access for token ids (they are
 *     clamped into [0, V) before any indexing).
 *   - Limits: 1 <= gamma <= 16, R * (gamma + 1) <= 4096, 1 <= r <= 256 for
 *     bf16 and 1 <= r <= 128 for f32, V >= 1.
 *   - Random numbers: Philox4x64-10 (Salmon et al., SC'11) keyed by
 *     (seed, 0) with counter (k, req_ids[r], step, 0) for slot k of request
 *     r; its four 64-bit words drive, in order, the draft sample, the accept
 *     test, the residual resample and the bonus sample at slot k. A word x
 *     becomes the uniform (x >> 40) * 2^-24. Outputs are a pure function of
 *     the inputs and (seed, step, req_ids).
 *   - Calls that draw take the step as a value and, optionally, as a device
 *     word `step_dev` (uint64). When step_dev is not NULL the kernels read the
 *     step from it when they run and the value is ignored; a launch captured
 *     once in a graph then follows a counter that dspark_advance moves on.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSPARK_OK = 0,
  DSPARK_EINVAL = -1,     /* null pointer or bad argument                    */
  DSPARK_EDTYPE = -2,     /* unknown dtype                                   */
  DSPARK_ETIER = -3,      /* bad capture-tier list (empty, unsorted, <= 0)   */
  DSPARK_ESIZE = -4,      /* a size is outside the documented limits         */
  DSPARK_EWORKSPACE = -5, /* workspace missing or smaller than required      */
  DSPARK_EHIP = -6        /* a HIP runtime call or kernel launch failed      */
} dspark_status;

typedef enum { DSPARK_F32 = 0, DSPARK_BF16 = 1 } dspark_dtype;

/* [sglang] "Verify modes". */
typedef enum {
  DSPARK_VERIFY_STATIC = 0,    /* verify and commit the whole block          */
  DSPARK_VERIFY_COMPACT = 1,   /* verify and commit the packed window        */
  DSPARK_VERIFY_CAP_ACCEPT = 2 /* verify the whole block, commit the window  */
} dspark_verify_mode;

/* [digest] "Verification scheduling" (greedy early stop) and "Infra"
 * (unconstrained search over a budget array); [vllm] "DSpark
 * confidence-scheduling mechanism" (budget given from the host). */
typedef enum {
  DSPARK_SCHED_ARGMAX = 0, /* smallest K maximising Theta over the budget array */
  DSPARK_SCHED_GREEDY = 1, /* admit while Theta strictly increases               */
  DSPARK_SCHED_FIXED = 2   /* K given by the caller                              */
} dspark_sched_mode;

/* Which kernels dspark_markov_draft and dspark_markov_draft_confidence use
 * (dspark_set_draft_path). */
typedef enum {
  DSPARK_DRAFT_AUTO = 0,     /* the library's choice: the per-slot launches,
                                which measured faster on MI355X at every
                                workload shape                               */
  DSPARK_DRAFT_PER_SLOT = 1, /* always the per-slot GEMM + select launches   */
  DSPARK_DRAFT_RESIDENT = 2  /* the resident-W2 block kernel where the shape
                                allows it (see dspark_markov_draft), else
                                per-slot launches                            */
} dspark_draft_path;

/* Selector for dspark_workspace_bytes. */
typedef enum {
  DSPARK_CALL_MARKOV_DRAFT = 0,
  DSPARK_CALL_VERIFY = 1,
  DSPARK_CALL_ANALYTIC_ACCEPT = 2
} dspark_call;

/* ------------------------------------------------------------------------ */
/* Utilities                                                                 */
/* ------------------------------------------------------------------------ */

/* Human-readable text for a dspark_status value (static storage). */
const char* dspark_status_string(int status);

/* Bytes of workspace `call` needs for these sizes (0 for calls that need
 * none, and for invalid sizes). The verify workspace does not depend on M_cap:
 * a well-formed pack never has more than R * (gamma + 1) rows.
 *
 * Workspaces hold the counters the GEMM passes deal vocabulary tiles from. A
 * workspace must be initialised once, before its first use, with
 * dspark_workspace_init (or be zero-filled by other means); every completed
 * call leaves it initialised. A workspace serves one call at a time. */
size_t dspark_workspace_bytes(int call, int R, int gamma, int V, int r);

/* Zero-fill a workspace of ws_bytes bytes on `stream` (a kernel rather than a
 * memset, so it may be captured in a graph). DSPARK_EINVAL for a null ws,
 * DSPARK_EHIP if the launch fails. */
int dspark_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Device offset, in bytes, of the error word of a draft workspace for R and V:
 * a uint32 that a resident draft sets to 1 when one of its barrier waits ran
 * out (see dspark_markov_draft); 0 otherwise. dspark_workspace_init clears it.
 * Returns 0 for invalid sizes. */
size_t dspark_workspace_status_offset(int R, int V);

/* Process-wide choice of draft kernels (dspark_draft_path; default AUTO).
 * Both give outputs within the same tolerance of the definition; they are
 * not bit-identical (their partial sums merge in different orders). For
 * tests and measurement. Returns the previous choice, or DSPARK_EINVAL for
 * an unknown value (the choice is then unchanged). Not thread-safe against
 * concurrent draft calls. */
int dspark_set_draft_path(int path);

/* Bytes of the pre-packed W2 buffer for rank r, vocabulary V and dtype. */
size_t dspark_prepacked_w2_bytes(int r, int V, int dtype);

/* Re-lay the Markov projection W2 [r, V] ([digest] "Architecture (drafter)":
 * B = W1 W2, W2 in R^{r x V}) into the matrix-core operand order used by the
 * draft and verify kernels. Weights are static across steps, so this runs
 * once per model. W2 and W2p are device buffers of the given dtype; W2p must
 * hold dspark_prepacked_w2_bytes(r, V, dtype) bytes. Zero padding fills the
 * rank up to a multiple of 32 and the vocabulary up to a multiple of 64. */
int dspark_prepack_w2(const void* W2, int r, int V, int dtype, void* W2p, size_t W2p_bytes,
                      void* stream);

/* Host cost-table preparation ([sglang] "Cost-table profiling": additive step
 * time with M = bs + K verify tokens; [vllm] "Technical implementation & CUDA
 * graphs": profiled curves are forced monotone and graph padding makes them
 * staircases).
 *   raw_step_time_s [host, M_max+1]  profiled step time T(M), seconds
 *   tiers           [host, n_tiers]  ascending captured pack totals
 *   staircase       nonzero: T(M) is read at the smallest tier >= M (capped
 *                   at M_max) and M above the top tier is infeasible (0)
 *   sps_milli       [host, M_max+1]  out: floor(1000 / T + 0.5), i.e. steps
 *                   per second x 1000, after T has been made monotone by a
 *                   running maximum over M; 0 marks an infeasible M.
 * Returns DSPARK_ETIER for an empty/unsorted/non-positive tier list. */
int dspark_cost_table_prepare(const double* raw_step_time_s, int M_max, const int32_t* tiers,
                              int n_tiers, int staircase, uint32_t* sps_milli);

/* ------------------------------------------------------------------------ */
/* Hot calls                                                                 */
/* ------------------------------------------------------------------------ */

/* Draft one block with the Markov sequential head ([digest] "Architecture
 * (drafter)": p_k(v | x_0, x_<k) = softmax(U_k(v) + W1[x_{k-1}] W2 (v)),
 * sampled left to right; the anchor x_0 is the last committed token).
 *   U        [R, gamma, V]  base logits of slots 1..gamma (dtype)
 *   W1       [V, r]         Markov lookup factor (dtype)
 *   W2p      pre-packed W2  (dspark_prepack_w2)
 *   anchor   [R] int32      x_0
 *   req_ids  [R] uint32     Philox request ids
 *   tokens   [R, gamma] int32  out: x_1..x_gamma
 *   p_draft  [R, gamma] f32    out: draft probability of the sampled token
 *   lse_draft[R, gamma] f32    out: log-sum-exp of the slot's draft logits
 *   ws       workspace of dspark_workspace_bytes(DSPARK_CALL_MARKOV_DRAFT, ...)
 * Sampling: inverse CDF over ascending ids with a strict comparison,
 * x = min{v : C_v > u S}, on the draft uniform of slot k.
 *
 * Kernels (dspark_set_draft_path). Per slot: two launches, the GEMM pass
 * with the softmax partials and the draw. Resident: for bfloat16 with
 * 224 < r <= 256 (r a multiple of 8), R <= 256, V a multiple of 8, at most 10
 * vocabulary tiles of 64 per compute unit and 16-byte aligned U and W1, the
 * whole block is one launch with W2 held on chip for all gamma slots (one
 * workgroup per compute unit, grid-wide waits between a slot's products and
 * its draws); other shapes fall back to per-slot launches. A resident call
 * must not overlap another resident draft on the same device (their
 * workgroups would wait on each other); a wait that runs out sets an error
 * word in the workspace (dspark_workspace_status_offset) and the call
 * finishes with undefined outputs. */
int dspark_markov_draft(const void* U, const void* W1, const void* W2p, const int32_t* anchor,
                        uint64_t seed, uint64_t step, const uint64_t* step_dev,
                        const uint32_t* req_ids, int R, int gamma,
                        int V, int r, int dtype, int32_t* tokens, float* p_draft,
                        float* lse_draft, void* ws, size_t ws_bytes, void* stream);

/* dspark_markov_draft without a workspace argument, for callers that cannot
 * allocate (code under graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). The workspace is a device array of the library
 * (dspark_noalloc_scratch_bytes(): 8 MiB, one per device, held until the
 * process ends); the call allocates nothing. Arguments and outputs as in
 * dspark_markov_draft, bit for bit. Sizes whose draft workspace
 * (dspark_workspace_bytes(DSPARK_CALL_MARKOV_DRAFT, ...)) exceeds the array
 * return DSPARK_EWORKSPACE before anything is launched; DSPARK_EHIP if the
 * array's address cannot be found. Each call first clears the workspace's
 * counters with a small kernel on `stream`. All calls on one device share the
 * array: calls that overlap on one device race and give undefined outputs. */
int dspark_markov_draft_noalloc(const void* U, const void* W1, const void* W2p,
                                const int32_t* anchor, uint64_t seed, uint64_t step,
                                const uint64_t* step_dev, const uint32_t* req_ids, int R,
                                int gamma, int V, int r, int dtype, int32_t* tokens,
                                float* p_draft, float* lse_draft, void* stream);

/* Bytes of the device array behind dspark_markov_draft_noalloc. */
size_t dspark_noalloc_scratch_bytes(void);

/* Peak probes for the measurement (not part of the method): what this GPU
 * reaches beside the published peaks the rooflines are priced against.
 * dspark_probe_read: one grid-stride sweep of 16-byte nontemporal loads over
 *   src [bytes] (16-byte aligned, a multiple of 16 bytes), 4 workgroups of
 *   512 threads per CU; sink [1] uint32 scratch, written only on a constant
 *   the sweep never produces. Bytes read = bytes.
 * dspark_probe_mfma: grid workgroups of 4 waves, each wave iters rounds of 8
 *   independent v_mfma_f32_16x16x32_bf16; sink [256] float scratch as above.
 *   dspark_probe_mfma_flops(grid, iters) = the FLOP the launch performs.
 * Both enqueue one launch on `stream`; DSPARK_EINVAL / DSPARK_ESIZE for bad
 * arguments, before anything is launched. */
int dspark_probe_read(const void* src, size_t bytes, void* sink, void* stream);
int dspark_probe_mfma(void* sink, int grid, int iters, void* stream);
double dspark_probe_mfma_flops(int grid, int iters);

/* Confidence head and prefix survival ([digest] "Verification scheduling
 * (system side)"): c_k = sigmoid((w . [h_k ; W1[x_{k-1}]] + b) * inv_temp_k),
 * a_{r,k} = a_{r,k-1} * c_k in float32, a_{r,0} = 1.
 *   h        [R, gamma, d]  hidden states (dtype)
 *   W1       [V, r]         (dtype)
 *   anchor   [R], tokens [R, gamma]
 *   w        [d + r] f32    head weight, hidden part first
 *   b        head bias
 *   inv_temp [gamma] f32 or NULL (NULL: 1; the per-position inverse
 *            temperatures of sequential temperature scaling, dspark_sts_fit)
 *   conf, surv [R, gamma] f32  out
 *   logit    [R, gamma] f32 out or NULL: the logit before the temperature,
 *            z = w . [h_k ; W1[x_{k-1}]] + b (the input of dspark_sts_fit) */
int dspark_confidence(const void* h, const void* W1, const int32_t* anchor, const int32_t* tokens,
                      const float* w, float b, const float* inv_temp, int R, int gamma, int d,
                      int V, int r, int dtype, float* conf, float* surv, float* logit,
                      void* stream);

/* dspark_markov_draft and dspark_confidence in one call ([sglang] "Performance
 * optimisation and zero-overhead scheduling": the drafter's sampling path is
 * fused). The head for slot k needs only x_{k-1}, which slot k's GEMM pass
 * already reads, so that launch also scores the slot: in its prologue, with
 * its first tiles' loads in flight, one wave per request runs the head's two
 * dot products and the survival product. That is done when at most a quarter
 * of the GEMM's workgroups carry a request (e.g. 64 requests on an MI355X);
 * with more requests the head runs as one launch after the draft. Arguments
 * as in the two calls; the outputs equal theirs bit for bit either way (same
 * wave code, same order). Errors: those of both calls. */
int dspark_markov_draft_confidence(const void* U, const void* W1, const void* W2p,
                                   const int32_t* anchor, uint64_t seed, uint64_t step,
                                   const uint64_t* step_dev, const uint32_t* req_ids, int R,
                                   int gamma, int V, int r, int dtype, const void* h,
                                   const float* w, float b, const float* inv_temp, int d,
                                   int32_t* tokens, float* p_draft, float* lse_draft, float* conf,
                                   float* surv, float* logit, void* ws, size_t ws_bytes,
                                   void* stream);

/* Global top-B prefix scheduler ([vllm] "DSpark confidence-scheduling
 * mechanism"; [digest] "Verification scheduling" and "Infra"). Integer fixed
 * point, so any evaluation order gives the same result:
 *   a_q = floor(clamp(a, 0, 1) * 2^20) (NaN -> 0), made non-increasing along
 *   each request by a running minimum; keys ordered by (a_q desc, request asc,
 *   slot asc); tau_K = R * 2^20 + sum of the K largest a_q of the budget array;
 *   Theta_K = tau_K * sps_milli[R + K] (uint64); K in [0, min(B_cap, R*gamma,
 *   M_max - R)].
 *   ARGMAX: smallest K maximising Theta_K.  GREEDY: stop at the first K with
 *   Theta_{K+1} <= Theta_K.  FIXED: K = clamp(K_fixed).
 * The K selected slots are always the K best keys of the CURRENT survivals;
 * win_len[r] counts request r's selected slots (a prefix).
 *   surv        [R, gamma] f32
 *   surv_budget [R, gamma] f32 or NULL (NULL: surv), e.g. stale confidences
 *   sps_milli   [M_max + 1] u32 (device copy of dspark_cost_table_prepare)
 *   win_len     [R] int32 out;  K_out [1] int32 out
 * Runs as one workgroup; nothing is read back to the host. */
int dspark_schedule_topb(const float* surv, const float* surv_budget, const uint32_t* sps_milli,
                         int M_max, int R, int gamma, int B_cap, int mode, int K_fixed,
                         int32_t* win_len, int32_t* K_out, void* stream);

/* Ragged pack ([sglang] "Ragged verify under full CUDA graphs": windows packed
 * front to back into a cu_seqlens buffer whose total is rounded up to the
 * nearest captured tier; [vllm] "Configuration & reproduction": the largest
 * verify batch is (gamma + 1) * R).
 *   win_len [R] or NULL (NULL: gamma, the full block); values clamped to
 *           [0, gamma]
 *   tiers   [host, n_tiers <= 32] ascending
 *   M_cap   rows of the packed buffers, >= R * (gamma + 1)
 *   cu_seqlens [R+1]: cu[0] = 0, cu[r+1] = cu[r] + 1 + L_r
 *   packed_tokens/req/slot [M_cap]: row cu[r] + j holds x_j (j = 0: anchor),
 *           request r, slot j; rows >= M hold 0, -1, -1
 *   totals  [2]: M = cu[R] and M_pad = smallest tier >= M, or -1 if M
 *           exceeds every tier */
int dspark_pack_ragged(const int32_t* anchor, const int32_t* tokens, const int32_t* win_len,
                       int R, int gamma, const int32_t* tiers, int n_tiers, int M_cap,
                       int32_t* cu_seqlens, int32_t* packed_tokens, int32_t* packed_req,
                       int32_t* packed_slot, int32_t* totals, void* stream);

/* dspark_schedule_topb then dspark_pack_ragged in one launch (one workgroup;
 * the windows pass to the pack through shared memory). Arguments as in the two
 * calls. pack_windows != 0 packs the scheduled windows (compact verify);
 * pack_windows == 0 packs every window at gamma, as dspark_pack_ragged with
 * win_len NULL (static and cap-accept verify), while win_len and K_out still
 * receive the schedule. The outputs equal the two calls'. Errors: those of
 * both calls. */
int dspark_schedule_pack(const float* surv, const float* surv_budget, const uint32_t* sps_milli,
                         int M_max, int R, int gamma, int B_cap, int mode, int K_fixed,
                         int32_t* win_len, int32_t* K_out, const int32_t* anchor,
                         const int32_t* tokens, int pack_windows, const int32_t* tiers,
                         int n_tiers, int M_cap, int32_t* cu_seqlens, int32_t* packed_tokens,
                         int32_t* packed_req, int32_t* packed_slot, int32_t* totals,
                         void* stream);

/* Rejection-sampling verification ([digest] summary and "Architecture": the
 * longest conforming prefix is accepted by rejection sampling, lossless
 * because every draft probability is an exact softmax; [sglang] "Verify
 * modes"). Packed target row cu[r] + j holds the target's logits for slot
 * j + 1; a request has Lv = cu[r+1] - cu[r] - 1 verified slots.
 *   slot k accepted iff u_accept < p_t(x_k) / p_draft[r, k] (float32);
 *   A_full = leading accepted slots; commit window L = Lv (STATIC, COMPACT)
 *   or min(win_len[r], Lv) (CAP_ACCEPT); A = min(A_full, L);
 *   A < L: resample slot A+1 from max(0, p_t - p_d) (p_d recomputed from U,
 *          W1[x_A], W2 with lse_draft; from p_t if no residual mass is left);
 *   A = L: bonus token for slot L+1 from p_t.
 *   target_packed [M_cap, V] (dtype), cu_seqlens [R+1], anchor [R],
 *   tokens, p_draft, lse_draft [R, gamma] (from dspark_markov_draft),
 *   U [R, gamma, V], W1 [V, r], W2p (pre-packed), win_len [R] (CAP_ACCEPT
 *   only, else may be NULL)
 *   accept_len [R] out: A;  n_out [R] out: A + 1
 *   out_tokens [R, gamma + 1] out: x_1..x_A, the correction/bonus token, then
 *              -1 padding
 *   ceiling_len [R] out or NULL: A_full (the cap-accept ceiling)
 *   ws  workspace of dspark_workspace_bytes(DSPARK_CALL_VERIFY, ...) */
int dspark_verify(const void* target_packed, int M_cap, const int32_t* cu_seqlens,
                  const int32_t* anchor, const int32_t* tokens, const float* p_draft,
                  const float* lse_draft, const void* U, const void* W1, const void* W2p,
                  const int32_t* win_len, int mode, uint64_t seed, uint64_t step,
                  const uint64_t* step_dev, const uint32_t* req_ids, int R, int gamma, int V,
                  int r, int dtype, int32_t* accept_len, int32_t* out_tokens, int32_t* n_out,
                  int32_t* ceiling_len, void* ws, size_t ws_bytes, void* stream);

/* Decode-loop advance ([digest] "Infra": the verify budget is sized from
 * confidences two steps back, while candidates are ranked by the latest
 * survivals; [vllm] "Execution pipeline": budget from the previous step's
 * double-buffered confidences, slots assigned on the GPU without read-back).
 * One launch, after a step's dspark_verify, that prepares the next step:
 *   anchor[r] <- out_tokens[r, A] with A = accept_len[r] clamped to [0, gamma]
 *               (the correction or bonus token, the next x_0)
 *   *step_dev += 1                    (skipped if step_dev is NULL)
 *   surv_hist [n_hist, R, gamma] f32: level h <- level h - 1 (h >= 1),
 *               level 0 <- surv [R, gamma] (n_hist = 0: no history; surv_hist
 *               and surv may then be NULL)
 * After the call, level h holds the survivals of the step h + 1 steps before
 * the next one; passing level lag - 1 as surv_budget to dspark_schedule_topb
 * sizes the budget from confidences lag steps old. 0 <= n_hist <= 8.
 * anchor, accept_len and out_tokens are the [R], [R] and [R, gamma + 1]
 * buffers of the step just verified. */
int dspark_advance(int32_t* anchor, const int32_t* accept_len, const int32_t* out_tokens, int R,
                   int gamma, uint64_t* step_dev, float* surv_hist, const float* surv, int n_hist,
                   void* stream);

/* ------------------------------------------------------------------------ */
/* Observability                                                             */
/* ------------------------------------------------------------------------ */

/* Words (uint64) of an observability block for R requests, block length gamma
 * and n_bins calibration bins (1 <= n_bins <= 32); 0 for invalid sizes. */
size_t dspark_observe_words(int R, int gamma, int n_bins);

/* Add one step to an observability block ([sglang] "Observability": the
 * cap-accept ceiling, per-request confidence and calibration such as ECE;
 * [sglang] "Per-request differentiation on mixed traffic": windows and
 * utilisation against the ceiling; [digest] "Verification scheduling": c_k is
 * the pass probability of slot k given an accepted prefix). Inputs are the
 * step's device buffers: conf, surv [R, gamma] (dspark_confidence), win_len
 * [R] (dspark_schedule_topb), accept_len and ceiling_len [R] (dspark_verify),
 * cu_seqlens [R + 1] (dspark_pack_ragged). Per request r let A = accept_len,
 * C = ceiling_len, L = win_len, Lv = cu[r+1] - cu[r] - 1 (each clamped to
 * [0, gamma]). The block (uint64 words, zero it before the first step, e.g.
 * with dspark_workspace_init) accumulates:
 *   [0] steps  [1] requests x steps  [2] sum (A + 1)  [3] sum A  [4] sum C
 *   [5] sum L  [6] sum Lv  [7] reserved
 *   [8 + h * (gamma + 1) + v]  histograms h = 0: L, 1: A, 2: C, of value v
 *   [8 + 3 (gamma + 1) + q * R + r]  per request: q = 0: sum A, 1: sum C,
 *                                   2: sum L
 *   then calibration cells [kind][k - 1][bin][3] = (count, sum of
 *   floor(p * 2^32), hits), bin = floor(p * n_bins) (p clamped to [0, 1],
 *   the top edge in the last bin, NaN in bin 0):
 *     kind 0 (conditional): p = conf[r, k-1], hit = slot k accepted, for
 *                           k <= min(C + 1, Lv);
 *     kind 1 (prefix):      p = surv[r, k-1], hit = C >= k, for k <= Lv.
 * All counts are integers, so the block does not depend on thread order. ECE
 * = sum over bins |sum p - hits| / count. One workgroup; calls on one block
 * must be ordered (one stream). */
int dspark_observe(const float* conf, const float* surv, const int32_t* win_len,
                   const int32_t* accept_len, const int32_t* ceiling_len,
                   const int32_t* cu_seqlens, int R, int gamma, int n_bins, uint64_t* stats,
                   size_t stats_words, void* stream);

/* Analytic acceptance rate of every verified slot ([digest] "Verification
 * scheduling (system side)": the confidence head's target is
 * c*_k = 1 - 1/2 ||p_d,k - p_t,k||_1). For slot k <= Lv of request r:
 *   p_d = softmax(U[r, k-1] + W1[x_{k-1}] W2), normalised by lse_draft[r, k-1];
 *   p_t = softmax(target_packed[cu[r] + k - 1]);
 *   cstar[r, k-1] = sum_v min(p_d(v), p_t(v))  (= 1 - TV, float32 sums)
 * and NaN for slots past Lv. Arguments as for dspark_verify (tokens and
 * lse_draft from dspark_markov_draft); ws: dspark_workspace_bytes(
 * DSPARK_CALL_ANALYTIC_ACCEPT, ...) bytes, initialised. A diagnostic pass:
 * it reads every verified row of U and of the target once more. */
int dspark_analytic_accept(const void* target_packed, int M_cap, const int32_t* cu_seqlens,
                           const int32_t* anchor, const int32_t* tokens, const float* lse_draft,
                           const void* U, const void* W1, const void* W2p, int R, int gamma,
                           int V, int r, int dtype, float* cstar, void* ws, size_t ws_bytes,
                           void* stream);

/* The first of the two passes dspark_markov_draft runs for every slot, as a
 * call of its own (for callers that time or fuse it): the bias GEMM
 * W1[x_prev] W2 on the matrix cores plus U_k, reduced per 64-entry vocabulary
 * tile t to a softmax partial (max_v z, sum_v exp(z - max)) of request n (two
 * floats). The partials are request-major: with n_t = ceil(V / 64) tiles and
 * c = ceil(n_t / 256), request n's row starts at part + n * 256 c (float2
 * units) and tile t sits at (t % c) * 256 + t / c in it -- the order in which
 * the 256 threads of dspark_markov_select read them. U_k rows are ldU elements
 * apart; x_prev[n * xstride] is the previous token of request n. part must hold
 * dspark_workspace_bytes(DSPARK_CALL_MARKOV_DRAFT, R, 1, V, r) bytes and be an
 * initialised workspace. The call uses up the workspace's tile queue; the
 * dspark_markov_select call that consumes these partials restores it, so the
 * two calls alternate on one workspace. */
int dspark_markov_partials(const void* U_k, long long ldU, const void* W1, const void* W2p,
                           const int32_t* x_prev, int xstride, int R, int V, int r, int dtype,
                           void* part, size_t part_bytes, void* stream);

/* The second pass of a draft slot, as a call of its own: per request n, merge
 * the tile partials of dspark_markov_partials into (m, S), draw u * S with the
 * slot-k draft uniform of req_ids[n], find the tile where the cumulative mass
 * crosses it, recompute that tile with the same matrix-core code and finish
 * the inverse-CDF search. Writes tok_out[n * ostride] (the token),
 * p_out[n * ostride] (its draft probability) and lse_out[n * ostride]
 * (m + ln S). dspark_markov_draft is dspark_markov_partials followed by this
 * call, for k = 1..gamma. */
int dspark_markov_select(const void* U_k, long long ldU, const void* W1, const void* W2p,
                         const int32_t* x_prev, int xstride, const void* part, uint64_t seed,
                         uint64_t step, const uint64_t* step_dev, const uint32_t* req_ids, int k,
                         int R, int V, int r, int dtype, int32_t* tok_out, float* p_out,
                         float* lse_out, int ostride, void* stream);

/* ------------------------------------------------------------------------ */
/* Sequential temperature scaling                                            */
/* ------------------------------------------------------------------------ */

/* Workspace bytes of dspark_sts_fit (0 for invalid sizes: 1 <= gamma <= 16,
 * 1 <= n_grid <= 256, 1 <= n_bins <= 32, N * gamma <= 2^31). */
size_t dspark_sts_workspace_bytes(int N, int gamma, int n_grid, int n_bins);

/* Fit per-position inverse temperatures for the confidence head ([digest]
 * "Verification scheduling (system side)": sequential temperature scaling
 * calibrates the running products prod_{i<=k} c_i left to right by a 1-D
 * grid search minimising ECE). Over N samples (rows of z, y, mask):
 *   for k = 1..gamma: for every candidate beta_j of betas[n_grid],
 *     a_k = a_{k-1} * sigmoid(z[n, k-1] * beta_j)  (float32, a_0 = 1, the
 *           chosen betas of earlier positions fixed);
 *     ece[k-1, j] = ECE of the pairs (a_k, y[n, k-1]) with mask[n, k-1] != 0
 *           (mask NULL: every pair), n_bins equal-width bins on [0, 1] (p
 *           clamped, the top edge in the last bin): sum over bins of
 *           |sum a - sum y| / pairs, from integer bin sums of floor(p 2^32);
 *     inv_temp[k-1] = the first beta_j with the smallest ECE.
 *   z   [N, gamma] f32: the head's logits (dspark_confidence's logit output)
 *   y   [N, gamma] f32 in [0, 1]: labels for the prefix products, hard (the
 *       prefix of length k was accepted) or soft (e.g. prod_{i<=k} c*_i from
 *       dspark_analytic_accept)
 *   betas [n_grid] f32 > 0, device; inv_temp [gamma] out, ece [gamma, n_grid]
 *   out (NaN where a position has no pairs); ws: dspark_sts_workspace_bytes.
 * Pass inv_temp to dspark_confidence to apply the fit. 3 gamma + 1 launches,
 * no read-back. */
int dspark_sts_fit(const float* z, const float* y, const uint8_t* mask, int N, int gamma,
                   const float* betas, int n_grid, int n_bins, float* inv_temp, float* ece,
                   void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Vocabulary-sharded draft (per-rank calls)                                 */
/* ------------------------------------------------------------------------ */

/* [sglang] "Performance optimisation and zero-overhead scheduling": the block
 * drafter's matmul is sharded. Under tensor parallelism over the vocabulary,
 * rank g of G owns columns [v0, v0 + V_g) of W2 (pre-packed on its own with
 * dspark_prepack_w2 for V_g columns) and of U; W1 is whole on every rank and
 * token ids are global. One draft slot k on rank g is:
 *   1. dspark_markov_shard_partials -- the GEMM pass on the rank's columns;
 *   2. dspark_markov_shard_summary -- the rank's (m_g, S_g) per request;
 *   3. all-gather of the G summaries into [G, R, 2] (a collective);
 *   4. dspark_markov_shard_select  -- merge, owner test, in-shard search;
 *   5. all-reduce MAX of the token and SUM of the probability (a collective);
 *      every rank then holds x_k for slot k + 1.
 * The draw is the single-device draw: the threshold u S over the global
 * vocabulary in ascending id order, u the slot's draft uniform. */

/* dspark_markov_partials on rank g's V_g columns: U_k points at the rank's
 * first column (rows ldU elements apart), W2p is the rank's pre-packed
 * [r, V_g] slice, and the previous tokens are global ids in [0, V) that pick
 * rows of the whole W1 [V, r]. part: dspark_workspace_bytes(
 * DSPARK_CALL_MARKOV_DRAFT, R, 1, V_g, r) bytes, initialised. */
int dspark_markov_shard_partials(const void* U_k, long long ldU, const void* W1, const void* W2p,
                                 const int32_t* x_prev, int xstride, int R, int V_g, int V, int r,
                                 int dtype, void* part, size_t part_bytes, void* stream);

/* Per request n: summary[n] = (max over the rank's tiles, sum of exp(z - max))
 * as two floats, from the partials of dspark_markov_partials over V_g
 * columns (part: the workspace of dspark_markov_shard_partials, part_bytes its
 * size). */
int dspark_markov_shard_summary(const void* part, size_t part_bytes, int R, int V_g,
                                float* summary, void* stream);

/* Rank g's select for slot k. summaries [G, R, 2]: every rank's summary, rank
 * major. Every rank merges them in rank order into the global (m, S), forms
 * T = u S and the mass P_h before each rank h; the rank with
 * P_g <= T < P_{g+1} (the last rank for T >= P_{G-1}) searches its own tiles
 * for T - P_g, recomputing the crossing tile. Writes at n * ostride: tok_out =
 * the global id on the owning rank, -1 elsewhere; p_out = the id's draft
 * probability on the owning rank, 0 elsewhere; lse_out = m + ln S on every
 * rank. U_k, ldU, x_prev, xstride, part as for dspark_markov_select (U_k at
 * the rank's first column); V is the full vocabulary (W1 rows, token range).
 * Restores the partials workspace's tile queue, like dspark_markov_select.
 * 1 <= G <= 64, 0 <= g < G, v0 + V_g <= V. */
int dspark_markov_shard_select(const void* U_k, long long ldU, const void* W1, const void* W2p,
                               const int32_t* x_prev, int xstride, const void* part,
                               const float* summaries, int G, int g, int v0, uint64_t seed,
                               uint64_t step, const uint64_t* step_dev, const uint32_t* req_ids,
                               int k, int R, int V_g, int V, int r, int dtype, int32_t* tok_out,
                               float* p_out, float* lse_out, int ostride, void* stream);

/* ------------------------------------------------------------------------ */
/* Diagnostic                                                                */
/* ------------------------------------------------------------------------ */

/* Markov logits of one slot, written out in full: z[n, v] = U_k[n, v] +
 * W1[x_prev[n]] . W2[:, v] (float32), computed by the same matrix-core tile
 * code as dspark_markov_draft. U_k rows are `ldU` elements apart (gamma * V
 * for a slot of a [R, gamma, V] block). For tests; not on the hot path. */
int dspark_markov_logits(const void* U_k, long long ldU, const void* W1, const void* W2p,
                         const int32_t* x_prev, int R, int V, int r, int dtype, float* z,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
