/*
 * spec_verify.h -- C ABI of the batched speculative-decoding verification step
 * on AMD Instinct MI355X (gfx950).
 *
 * What is computed (pages cited by title and section):
 *  - aivaro.ru answer 289, "Как работает speculative decoding на уровне
 *    логитов, а не токенов?": section 5 step 3 and section 6 (accept a draft
 *    token with probability min(1, p_target/p_draft); after a rejection drop
 *    the later drafts and draw from max(0, p_target - p_draft)/Z), section 9
 *    (softmax of both rows, a uniform compared with "<", multinomial draw).
 *  - Hung-yi Lee lecture 16 notes, part "4、推测解码验证流程图": item 1
 *    (one target pass scores all positions), items 2-3 (position-by-position
 *    check, truncation at the first failure), item 4 (bonus token from the
 *    (K+1)-th target distribution when every draft passes).
 *  - aihero.vn "Speculative decoding": section "Chấp nhận bằng tỉ lệ, không chỉ
 *    bằng argmax" (q = draft, p = target at the same prefix; ratio test;
 *    residual), section "Cùng phân bố không có nghĩa cùng chuỗi mỗi lần"
 *    (temperature / top-k / top-p applied consistently; greedy decoding has
 *    its own check).
 *
 * For each sequence b with K_b draft tokens x_0..x_{K_b-1}:
 *   q_i = softmax(filter(draft_row_i / T)),  p_i = softmax(filter(target_row_i / T))
 *   accept x_i iff u_i < p_i(x_i) / q_i(x_i)   (strict; q_i(x)=0<p_i(x): accept)
 *   n = index of the first rejection, or K_b
 *   n < K_b: token n = inverse CDF of max(0, p_n - q_n) with u_{K_b}
 *   n = K_b: token n = inverse CDF of p_{K_b} with u_{K_b}      (bonus)
 * The inverse CDF takes the smallest id j (ascending ids) whose cumulative
 * weight exceeds u * Z. filter = top-k (values >= the k-th largest, ties kept)
 * then top-p (keep ids whose strictly-larger-logit mass is < top_p).
 * Greedy sequences (temperature 0, or the per-sequence mask) accept x_i iff it
 * equals argmax(target_row_i) (lowest id on ties) and emit argmax(target_row_n)
 * at position n; they never read draft rows or uniforms.
 *
 * Layout (all device pointers, row-major, rows contiguous with stride V):
 *   draft_logits  [sum_b K_b, V]        sequence b owns rows cu[b] .. cu[b+1]-1
 *   target_logits [sum_b (K_b+1), V]    rows cu[b]+b .. cu[b+1]+b
 *   draft_tokens  int32 [sum_b K_b]
 *   uniforms      float [sum_b (K_b+1)] slots 0..K_b-1 accept tests, slot K_b
 *                                       the resample-or-bonus draw
 *   out_tokens    int32 [sum_b (K_b+1)] tokens 0..n valid, the rest -1
 *   num_accepted  int32 [B]             n, or a negative per-sequence code
 * The dense entry point is the case cu[b] = b*K ([B,K,V], [B,K+1,V], ...).
 *
 * Ownership: the caller owns every buffer (inputs, outputs and the workspace);
 * the library allocates nothing, keeps no state between calls and enqueues all
 * work on `stream` without synchronising it. Calls that share a workspace must
 * be ordered (same stream, or synchronised). The one exception is
 * spec_verify_noalloc, whose workspace is a fixed array inside the library
 * (one per device, shared by every such call on that device).
 *
 * Errors: argument errors return a negative SV_E* code before any device work.
 * Data errors found on the device are reported per sequence in num_accepted
 * (SV_SEQ_*), with that sequence's out_tokens all -1 (for SV_SEQ_BAD_OFFSETS,
 * whose rows cannot be located, out_tokens is left unwritten).
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of the logit rows. */
typedef enum sv_dtype { SV_F32 = 0, SV_F16 = 1, SV_BF16 = 2 } sv_dtype;

/* Return codes of the entry points. */
#define SV_OK 0
#define SV_EINVAL (-1)       /* null pointer, negative size, K out of [0,64],
                                temperature < 0 / NaN / inf, top_p outside (0,1] */
#define SV_EDTYPE (-2)       /* dtype not one of sv_dtype */
#define SV_EWORKSPACE (-3)   /* workspace null, not 256-byte aligned, or smaller
                                than spec_verify_workspace_bytes() */
#define SV_EHIP (-4)         /* a HIP launch or event record failed */
#define SV_EUNSUPPORTED (-5) /* valid request outside this build's limits:
                                top_k above SV_MAX_TOP_K, V above 2^30, or
                                a grid of more than 2^24 blocks */
#define SV_ESCRATCH (-6)     /* spec_verify_noalloc: the call needs more than
                                the library's fixed scratch array holds
                                (SV_NOALLOC_SCRATCH_BYTES) */

/* Per-sequence codes written to num_accepted[b] instead of a count. */
#define SV_SEQ_BAD_TOKEN (-1)   /* a draft id outside [0, V) */
#define SV_SEQ_BAD_ROW (-2)     /* a used row holds NaN or +inf, or no finite
                                   value. The used rows are the draft and target
                                   rows of positions 0..n (n = the first
                                   rejection) and the bonus row when every draft
                                   passes; greedy sequences use no draft rows.
                                   Rows past the first rejection are never read */
#define SV_SEQ_BAD_OFFSETS (-3) /* ragged offsets: cu[b] > cu[b+1], outside
                                   [0, total_draft_rows], or K_b > 64 */
#define SV_SEQ_SYNC_TIMEOUT (-4) /* a bounded wait for the sequence's row
                                    statistics ran out; its outputs are not
                                    valid */

#define SV_MAX_K 64
#define SV_MAX_TOP_K 1024
#define SV_MAX_CHAINS 4
/* Bytes of the fixed scratch array spec_verify_noalloc uses on each device. */
#define SV_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* Human-readable text for a return code or per-sequence code. Never NULL. */
const char* spec_verify_strerror(int code);

/* Bytes of device workspace a call with these sizes needs (the same value for
 * spec_verify with total_draft_rows = B*K). An active top_k (0 < top_k < V,
 * top_k <= SV_MAX_TOP_K) adds per-chunk candidate records and per-row
 * results, top_p < 1 alone per-row results; a workspace sized with an active
 * top_k also serves calls with top-p alone or without filters. Returns 0 for
 * invalid sizes. */
size_t spec_verify_workspace_bytes(int B, int total_draft_rows, int V, int top_k,
                                   float top_p);

/* Zero-fill a workspace on `stream` (kernel fill, no memset node). A workspace
 * must be zero-filled once before its first use: blocks of one call hand
 * per-row partial results to each other through it, and a zero entry means
 * "not yet published". Every call returns those entries, its per-sequence
 * counters and (with filters) its candidate records and per-row results to
 * zero before it ends, so calls that share one workspace may differ
 * in B, K, V and dtype, as long as it is large enough for each of them. After a
 * call that reports SV_SEQ_SYNC_TIMEOUT or SV_SEQ_BAD_OFFSETS for any sequence,
 * zero-fill the workspace again. */
int spec_verify_workspace_init(void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Dense batch: B sequences with K drafts each.
 *   draft_logits  [B, K, V]   (may be NULL when K == 0 or temperature == 0)
 *   target_logits [B, K+1, V]
 *   draft_tokens  int32 [B, K] (may be NULL when K == 0)
 *   uniforms      float [B, K+1] in [0, 1) (may be NULL when temperature == 0)
 *   temperature   > 0 sampling, == 0 greedy for every sequence
 *   top_k         <= 0 or >= V: off;  top_p in (0, 1], 1: off
 *   out_tokens    int32 [B, K+1];  num_accepted int32 [B]
 * B == 0 returns SV_OK and launches nothing.
 * Device occupancy: without filters the call is one kernel whose draw blocks
 * wait (bounded) for row statistics that later blocks of the same grid
 * compute. For a dense batch with K >= 2 the draw blocks are placed ahead of
 * the last two positions' statistics when the device holds all of them at
 * once with a block per compute unit to spare; this assumes the call has the
 * device to itself. A kernel running beside it on another stream that keeps
 * compute units busy can make those waits run out: the sequences concerned
 * report SV_SEQ_SYNC_TIMEOUT (then zero-fill the workspace before reuse). The
 * compute-unit count and the kernel's occupancy are looked up once per device
 * and kept (facts about the device, no data of any call). */
int spec_verify(const void* draft_logits, const void* target_logits,
                const int32_t* draft_tokens, const float* uniforms, int B, int K,
                int V, float temperature, int top_k, float top_p, sv_dtype dtype,
                int32_t* out_tokens, int32_t* num_accepted, void* workspace,
                size_t workspace_bytes, hipStream_t stream);

/* spec_verify for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation. Arguments, outputs, return codes and per-sequence codes
 * are those of spec_verify; the workspace is a fixed array inside the library,
 * SV_NOALLOC_SCRATCH_BYTES on each device that calls it, held from the first
 * call on that device until the process ends. The call allocates nothing (no
 * hipMalloc, no allocating library routine); its first call on a device looks
 * up that device's copy of the array. Each call first clears the part of the
 * array it uses with a fill kernel on `stream` (no memset node), so nothing of
 * an earlier call carries over, not even after SV_SEQ_SYNC_TIMEOUT. Every call
 * on one device shares that device's array: calls that overlap on one GPU
 * (other streams or threads) race, and the caller must order them. Returns
 * SV_ESCRATCH, before any device work, when the call needs more than
 * SV_NOALLOC_SCRATCH_BYTES (its spec_verify_workspace_bytes): unfiltered and
 * top-p-alone calls fit up to B = 512, K = 16 at V = 128256; active top-k
 * does not fit at these vocabularies. */
int spec_verify_noalloc(const void* draft_logits, const void* target_logits,
                        const int32_t* draft_tokens, const float* uniforms, int B, int K,
                        int V, float temperature, int top_k, float top_p, sv_dtype dtype,
                        int32_t* out_tokens, int32_t* num_accepted, hipStream_t stream);

/* Ragged batch (per-sequence K_b, the dynamic-K setting of the lecture-16 notes,
 * "工程里的关键优化点" item 3): packed rows as described above.
 *   cu_draft   int32 [B+1] device offsets, cu[0] = 0, non-decreasing,
 *              cu[B] = total_draft_rows, K_b = cu[b+1]-cu[b] <= 64; a sequence
 *              whose own pair (cu[b], cu[b+1]) breaks this reports
 *              SV_SEQ_BAD_OFFSETS; if the array as a whole is not
 *              non-decreasing the other sequences' results are unspecified
 *   greedy     uint8 [B] device mask (nonzero: greedy), or NULL for none;
 *              temperature == 0 makes every sequence greedy. */
int spec_verify_ragged(const void* draft_logits, const void* target_logits,
                       const int32_t* draft_tokens, const float* uniforms,
                       const int32_t* cu_draft, const uint8_t* greedy, int B,
                       int total_draft_rows, int V, float temperature, int top_k,
                       float top_p, sv_dtype dtype, int32_t* out_tokens,
                       int32_t* num_accepted, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/* Optional side outputs of spec_verify_diag (every pointer may be NULL).
 *   row_max_*    raw logit maximum of each row's kept set
 *   row_logsum_* ln sum_{kept} exp((l - max)/T) of each row; the row's
 *                normaliser is exp(max/T) * exp(row_logsum)
 *   ratio        p_i(x_i)/q_i(x_i) per draft row (sampling sequences)
 *   resid_Z      per sequence: the mass the final inverse CDF normalised by
 *                (residual mass at n, or the bonus row's mass)
 *   stage_events n_stage_events events recorded on `stream` before the first
 *                kernel and after each kernel of the call (for timing); events
 *                beyond the kernel count are recorded after the last kernel.
 *                With filters the kernels are the row statistics pass, a
 *                per-row filter pass (threshold and kept-set normaliser) and
 *                the decision-and-draw pass; without filters all three run
 *                in one kernel.
 *   spin_limit   bound of a wait for row statistics (0: default); a small
 *                value forces the SV_SEQ_SYNC_TIMEOUT path in tests.
 *   beta, expected_accepted
 *                the acceptance statistics of the same rows, as
 *                spec_verify_accept_stats defines them: beta float
 *                [total_draft_rows], expected_accepted float [B]. Both or
 *                neither (else SV_EINVAL). Greedy sequences get NaN (a draft
 *                of theirs has no pass probability); K_b = 0 gives 0. When
 *                the call runs as one kernel (no top-k / top-p) a second
 *                kernel sums min(p, q) over every (draft, target) row pair
 *                from the first one's row statistics: two passes over the
 *                rows in all. With filters (or rows of more than 256 * 1024
 *                vectors) the acceptance statistics run as their own two
 *                passes after the verification, and a call that also has
 *                greedy sequences returns SV_EUNSUPPORTED. Stage events then
 *                mark the verification kernels as above, and every event past
 *                them is recorded after the acceptance statistics. */
typedef struct sv_diag {
  float* row_max_draft;
  float* row_logsum_draft;
  float* row_max_target;
  float* row_logsum_target;
  float* ratio;
  float* resid_Z;
  hipEvent_t* stage_events;
  int n_stage_events;
  int spin_limit;
  float* beta;
  float* expected_accepted;
} sv_diag;

/* Number of kernels a call launches for these settings (stage events = this+1). */
int spec_verify_num_stages(int top_k, float top_p);

/* spec_verify_ragged with side outputs (diag may be NULL). */
int spec_verify_diag(const void* draft_logits, const void* target_logits,
                     const int32_t* draft_tokens, const float* uniforms,
                     const int32_t* cu_draft, const uint8_t* greedy, int B,
                     int total_draft_rows, int V, float temperature, int top_k,
                     float top_p, sv_dtype dtype, int32_t* out_tokens,
                     int32_t* num_accepted, void* workspace,
                     size_t workspace_bytes, hipStream_t stream,
                     const sv_diag* diag);

/* Acceptance statistics of sampling verification (no draft ids, no uniforms):
 * how often drafts pass, the quantity a caller adapting K per sequence needs
 * (aivaro.ru answer 289 section 6: a draft token passes with probability
 * min(1, p/q) and the acceptance rate measures how close the draft is to the
 * target; aihero.vn "Speculative decoding" section "Khi thời gian tiết kiệm bị
 * chi phí ăn hết": measure useful tokens per round and the acceptance rate;
 * lecture-16 notes "工程里的关键优化点" item 3: K adapted to it).
 *   beta[d] = sum_x q_i(x) * min(1, p_i(x)/q_i(x)) = sum_x min(p_i(x), q_i(x))
 *       for draft row d = cu[b] + i and the target row of the same position,
 *       on the tempered, filtered rows: the probability that a draft drawn
 *       from q_i passes the ratio test. NaN if either row holds NaN or +inf or
 *       no finite value.
 *   expected_accepted[b] = sum_{j<K_b} prod_{i<=j} beta_i: the expected number
 *       of accepted drafts with the rows held fixed (the emitted count is one
 *       more: the correction or bonus token). 0 when K_b = 0; NaN if a beta of
 *       the sequence is NaN or the sequence's offsets are invalid (then the
 *       betas of its rows are unspecified).
 * Layout as spec_verify_ragged; target row K_b of each sequence (the bonus
 * row) is not read. cu_draft may be NULL: then every sequence has
 * K = total_draft_rows / B drafts (total_draft_rows must be a multiple of B,
 * K <= 64). temperature must be finite and > 0 (greedy verification has no
 * pass probability); top_k / top_p as spec_verify, and the same limits.
 * Outputs: beta float [total_draft_rows] (may be NULL when it is 0),
 * expected_accepted float [B], device memory. The workspace is sized by
 * spec_verify_workspace_bytes(B, total_draft_rows, V, top_k, top_p) and obeys
 * the same zero rules. Two passes over the rows: statistics, then the sums. */
int spec_verify_accept_stats(const void* draft_logits, const void* target_logits,
                             const int32_t* cu_draft, int B, int total_draft_rows, int V,
                             float temperature, int top_k, float top_p, sv_dtype dtype,
                             float* beta, float* expected_accepted, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* Several draft chains per sequence (the lecture-16 notes, part "1、第16講":
 * there can be several drafters; the pages give no rule, so the one used is
 * their own single step applied again, from aivaro.ru answer 289 section 6:
 * accepting x ~ q with probability min(1, p(x)/q(x)), else drawing from
 * max(0, p - q)/Z, is rejection sampling whose result follows p; after a
 * rejection the remainder max(0, p - q)/Z is the law the next candidate,
 * drawn independently, is tested against).
 * M chains of K drafts share each sequence's prefix; chain m's rows at
 * position j are conditioned on its own tokens 0..j-1, and the caller's target
 * rows of chains with equal prefixes must agree. Position j is checked against
 * the chains still alive (their tokens so far equal the emitted ones), in
 * chain order, starting from the lowest live chain's target row p_j: a
 * candidate is accepted iff u < r(x)/q_m(x), where r is the current law (p_j,
 * then each remainder). An accepted token keeps alive the chains that
 * proposed it. When every candidate is rejected the token is drawn from the
 * last remainder, by inverse CDF over ascending ids (the bonus position K
 * draws from p_K). top_k / top_p filter every row as in spec_verify (each
 * law is the row's kept-set distribution; aihero.vn "Speculative decoding",
 * section "Cùng phân bố không có nghĩa cùng chuỗi mỗi lần"). temperature 0
 * verifies greedily: the first live chain whose token is the argmax of p_j
 * (lowest id on ties) is accepted, and when none is the argmax is emitted
 * (the limit of the rule above when p_j is a point mass); draft rows and
 * uniforms are not read then (draft_logits and uniforms may be NULL).
 *   draft_logits  [B, M, K, V]     target_logits [B, M, K+1, V]
 *   draft_tokens  int32 [B, M, K]
 *   uniforms      float [B, K+1, M+1]: [b, j, m] tests chain m's candidate at
 *                 position j, [b, j, M] is the draw at j (used where the walk
 *                 stops)
 *   out_tokens    int32 [B, K+1] (-1 padded); num_accepted int32 [B] (n, or
 *                 SV_SEQ_BAD_TOKEN for any id outside [0, V), SV_SEQ_BAD_ROW
 *                 for a used row with NaN, +inf or no finite value,
 *                 SV_SEQ_SYNC_TIMEOUT if a bounded wait between the blocks of
 *                 the sequence ran out; then fill the workspace with zeros again)
 *   out_chain     int32 [B] or NULL: the lowest chain holding the emitted
 *                 prefix (the cache to keep), -1 with an error code
 * 1 <= M <= SV_MAX_CHAINS, 0 <= K <= SV_MAX_K, temperature finite and >= 0,
 * top_k and top_p with the meaning and limits of spec_verify,
 * rows of at most 2^18 vectors (16-byte vectors when V * element size is a
 * multiple of 16 and both arrays are 16-byte aligned, else elements; longer
 * rows return SV_EUNSUPPORTED). The
 * workspace (spec_verify_multi_workspace_bytes) obeys the zero rules of
 * spec_verify. Two kernels: the row statistics of every row, then the walk,
 * four blocks of 1024 threads per sequence, each on a quarter of the
 * vocabulary (one pass per rejection and per draw, the blocks exchanging
 * their sums through the workspace after each pass). The blocks of a sequence
 * wait for each other, so, as for spec_verify, the call assumes no other
 * kernel holds the device's compute units meanwhile; a wait that runs out
 * gives SV_SEQ_SYNC_TIMEOUT instead of a hang. */
size_t spec_verify_multi_workspace_bytes(int B, int M, int K, int V, int top_k, float top_p);
int spec_verify_multi(const void* draft_logits, const void* target_logits,
                      const int32_t* draft_tokens, const float* uniforms, int B, int M, int K,
                      int V, float temperature, int top_k, float top_p, sv_dtype dtype,
                      int32_t* out_tokens, int32_t* num_accepted, int32_t* out_chain,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Verification from LM-head hidden states: the same step as spec_verify, with
 * the logit rows formed inside the library as l = h W^T on the matrix cores
 * (bf16 operands, fp32 accumulation) and reduced in the GEMM epilogue, so the
 * bf16 [B, K, V] and [B, K+1, V] logit arrays are never written by a model
 * and read back (aivaro.ru answer 289 section 8 names the memory the draft and
 * target logits take; the lecture-16 notes: the target model scores every
 * drafted position in one pass, its logits being the last layer's output).
 * A sampling call stores the fp32 rows inside the workspace as the GEMM forms
 * them, and the final draw reads its rows (p_n, and q_n for a residual) there.
 *   hidden_draft   bf16 [B*K, d_draft]     draft model's last hidden states
 *   weight_draft   bf16 [V, d_draft]       draft LM head (may be NULL with hidden_draft when K == 0)
 *   hidden_target  bf16 [B*(K+1), d_target]
 *   weight_target  bf16 [V, d_target]
 *   draft_tokens   int32 [B, K]; uniforms float [B, K+1]; outputs as spec_verify.
 * temperature finite and >= 0; no top-k / top-p. Temperature 0 verifies
 * greedily (accept iff the draft id is the target row's argmax, the lowest id
 * on ties; the correction or bonus token is that argmax): no draft row is
 * formed, no row stored and no uniform read, so hidden_draft, weight_draft and
 * uniforms may be NULL and d_draft is not checked. d_draft (sampling) and
 * d_target are multiples of 8 (>= 8); the matrices given are 16-byte aligned.
 * Row-major throughout. The workspace is sized by
 * spec_verify_lmhead_workspace_bytes(B, K, V), 256-byte aligned; its first
 * spec_verify_lmhead_zero_bytes(B, K, V) bytes must be zero before the first
 * call (spec_verify_workspace_init) and are zero again after every call. The
 * logits ((B*K + B*(K+1)) * V floats, draft rows first) sit at the tail of the
 * workspace and hold the last sampling call's rows. One workspace serves calls
 * of any smaller B, K, V: their zero regions start at the front and their
 * logits end at the back. stage_events (may be NULL; n_stage_events of them,
 * caller-created) are recorded on `stream`: before the statistics GEMM (draft
 * and target rows, one launch), after it, after the merge of its partials,
 * and every further one after the decision and draw. Errors as spec_verify. */
size_t spec_verify_lmhead_workspace_bytes(int B, int K, int V);
size_t spec_verify_lmhead_zero_bytes(int B, int K, int V);
int spec_verify_lmhead(const void* hidden_draft, const void* weight_draft, int d_draft,
                       const void* hidden_target, const void* weight_target, int d_target,
                       const int32_t* draft_tokens, const float* uniforms, int B, int K, int V,
                       float temperature, int32_t* out_tokens, int32_t* num_accepted,
                       void* workspace, size_t workspace_bytes, hipStream_t stream,
                       hipEvent_t* stage_events, int n_stage_events);

/* spec_verify_lmhead with side outputs, for checking the logits the
 * decisions were made on (every pointer of diag may be NULL; diag may be NULL):
 *   logits_draft   float [B*K, V]      the draft rows' logits as the statistics
 *   logits_target  float [B*(K+1), V]  GEMM formed them (fp32 accumulation),
 *                                      before any reduction (a greedy call
 *                                      forms no draft logits)
 * Device memory owned by the caller, 16-byte aligned (else SV_EINVAL). A
 * sampling call stores these rows in place of the workspace's and its draw
 * reads them there, so they must not overlap the workspace or each other; a
 * greedy call writes logits_target only for this output. */
typedef struct sv_lmhead_diag {
  float* logits_draft;
  float* logits_target;
} sv_lmhead_diag;

int spec_verify_lmhead_diag(const void* hidden_draft, const void* weight_draft, int d_draft,
                            const void* hidden_target, const void* weight_target, int d_target,
                            const int32_t* draft_tokens, const float* uniforms, int B, int K,
                            int V, float temperature, int32_t* out_tokens, int32_t* num_accepted,
                            void* workspace, size_t workspace_bytes, hipStream_t stream,
                            hipEvent_t* stage_events, int n_stage_events,
                            const sv_lmhead_diag* diag);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
