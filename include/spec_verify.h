/*
 * spec_verify.h -- C ABI of the MI355X (gfx950) batched draft-verification
 * library.
 *
 * The operation. For every request b of a batch, a drafter has proposed
 * up to K tokens x_0..x_{K-1}; the target model has scored the whole block
 * in one pass, giving K+1 logit rows (one per drafted position plus the
 * position after the block). Of the K drafted tokens only the first k_b (the
 * request's verify budget) are checked. The library decides which drafted
 * tokens survive and draws the one token that follows them:
 *
 *   - Greedy verification (temperature == 0), as described in
 *     "Speculative decoding becomes standard: DSpark and multi-token
 *     drafters", section "Why draft-and-verify does not change the output",
 *     paragraph 1: keep drafted tokens while they equal the target's most
 *     likely token (lowest index among equal maxima), and at the first
 *     mismatch emit the target's own token; if all k_b agree, emit the
 *     target's token at position k_b.
 *   - Sampled verification (temperature T > 0), same section, paragraph 2
 *     (the rule of Leviathan, Kalman and Matias): with p_i = softmax(z_t/T)
 *     and q_i = softmax(z_d/T) over the full vocabulary, drafted token x_i
 *     survives when u < min(1, p_i(x_i)/q_i(x_i)); at the first rejection j
 *     the token is drawn from the renormalised residual max(0, p_j - q_j);
 *     if all k_b survive, a bonus token is drawn from p_{k_b}. Draws are
 *     inverse-CDF in vocabulary order.
 *   - Per-request budgets k_b (0 <= k_b <= K) model the confidence-driven
 *     scheduler of the same page, section "What DSpark adds", paragraph 2.
 *
 * Random numbers: Philox4x32-10 (Salmon et al., SC'11) with key = seed
 * (low word, high word) and counter = (b, i, 0, 0) for position i of request
 * b; output word 0 gives the acceptance uniform of position i, word 1 its
 * sampling uniform, each as (word >> 8) * 2^-24.
 *
 * Conventions shared by every entry point:
 *   - All tensors are caller-owned device memory; the library never frees
 *     or retains them past a call. The library owns only the context and its
 *     device workspace.
 *   - Work is enqueued on the caller's HIP stream (hipStream_t passed as
 *     void*, NULL = default stream) and the call returns without waiting.
 *   - Return values are sv_status codes; nothing is thrown across the ABI.
 *     Argument errors are detected on the host before anything is enqueued.
 *     Errors only visible on the device (a budget outside [0, K], a drafted
 *     token outside [0, V)) set bits of a device status word read by
 *     spec_verify_status; the kernels never read out of bounds because of
 *     them.
 *   - One context serves one stream at a time: calls that overlap in time
 *     on the same context race on its workspace.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct spec_verify_ctx spec_verify_ctx;

/* Storage type of the logit tensors. */
enum sv_dtype {
    SV_DTYPE_F32 = 0,   /* IEEE fp32 */
    SV_DTYPE_BF16 = 1   /* bfloat16: the upper 16 bits of an fp32 */
};

/* Return codes. */
enum sv_status {
    SV_OK = 0,
    SV_ERR_NULL = -1,    /* a required pointer is NULL */
    SV_ERR_ARG = -2,     /* a scalar argument is out of range */
    SV_ERR_DTYPE = -3,   /* unknown storage type */
    SV_ERR_ALIGN = -4,   /* a pointer is not aligned to its element size */
    SV_ERR_HIP = -5,     /* the HIP runtime reported an error */
    SV_ERR_NOMEM = -6,   /* device workspace allocation failed */
    SV_ERR_STATE = -7,   /* NULL or already freed context */
    SV_ERR_TOO_BIG = -8  /* spec_verify_run_noalloc: the call needs more
                            workspace than its static scratch holds */
};

/* Bits of the device status word (spec_verify_status). */
#define SV_FLAG_BAD_BUDGET 0x1u /* a budget was outside [0, K]; it was clamped */
#define SV_FLAG_BAD_TOKEN  0x2u /* a checked drafted token was outside [0, V);
                                   it was treated as rejected, its p and q as 0 */
#define SV_FLAG_SYNC_TIMEOUT 0x4u /* an internal consistency check failed (a
                                   wave's bounded wait for another wave of its
                                   own workgroup expired, or a decision was
                                   read before it was final); the outputs of
                                   that call are not valid. No wait depends on
                                   other workgroups being resident. */

/* Library limits. */
#define SV_MAX_BATCH 16384
#define SV_MAX_K 32
#define SV_MAX_VOCAB (1 << 20)

/* Size of the static device scratch of spec_verify_run_noalloc (per GPU). */
#define SV_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * spec_verify_init -- create a context for one device and one problem shape
 * (the batched verify step of "Speculative decoding becomes standard: DSpark
 * and multi-token drafters", section "Why draft-and-verify does not change
 * the output", with the per-request budgets of section "What DSpark adds",
 * paragraph 2).
 *   out        receives the context (set to NULL on failure).
 *   device     HIP device ordinal.
 *   max_batch  largest B a run will pass, 1..SV_MAX_BATCH.
 *   max_k      largest K a run will pass, 0..SV_MAX_K.
 *   vocab      V, the vocabulary size of every run, 1..SV_MAX_VOCAB.
 *   dtype      sv_dtype of the logits of every run.
 * Allocates and zeroes the device workspace (per-chunk partial statistics,
 * per-row argmax keys and per-request counters of greedy mode, status
 * word). The context owns it until spec_verify_free. Synchronous.
 * Errors: SV_ERR_NULL, SV_ERR_ARG, SV_ERR_DTYPE, SV_ERR_HIP, SV_ERR_NOMEM.
 */
int spec_verify_init(spec_verify_ctx** out, int device, int max_batch, int max_k,
                     int vocab, int dtype);

/*
 * spec_verify_run -- verify one batch (stream-ordered, no host sync): the
 * greedy rule ("Speculative decoding becomes standard: DSpark and
 * multi-token drafters", section "Why draft-and-verify does not change the
 * output", paragraph 1) when temperature == 0, else the rejection rule with
 * residual and bonus draws (same section, paragraph 2), over the budgeted
 * positions of each request (section "What DSpark adds", paragraph 2).
 *   target_logits     [B, K+1, V] row-major, storage ctx dtype (device).
 *   draft_logits      [B, K, V] row-major, same storage (device); may be
 *                     NULL when temperature == 0 (never read then).
 *   draft_tokens      int32 [B, K] drafted token ids (device); entries at
 *                     positions >= budgets[b] are never read.
 *   budgets           int32 [B] verify budgets k_b, 0 <= k_b <= K (device).
 *   B, K              batch size (0..max_batch; 0 is a no-op) and block
 *                     width (0..max_k).
 *   temperature       0 = greedy; > 0 = sampled; must be finite. Sampled
 *                     rows are reduced with c = log2(e) / T in fp32 and the
 *                     scaled maximum max(z) c, so |z| c must stay inside the
 *                     fp32 range (for logits below 1e4 in magnitude: T >= 1e-30).
 *   seed              Philox key of this call.
 *   out_tokens        int32 [B, K+1]: x_0..x_{j-1}, then the drawn token,
 *                     then -1 padding (device).
 *   out_num_accepted  int32 [B]: j, the number of drafted tokens kept.
 *   out_p_draft       float [B, K] or NULL: p_i(x_i) for i < k_b, NaN for
 *                     i >= k_b and in greedy mode (device).
 *   out_q_draft       float [B, K] or NULL: q_i(x_i), same layout.
 *   stream            hipStream_t or NULL.
 * The caller keeps ownership of every tensor. Request b uses Philox counter
 * (b, i, 0, 0); spec_verify_run_ex offsets b.
 * Pointers must be aligned to their element size; a 16-byte aligned logit
 * base with V * sizeof(element) a multiple of 16 takes the vector-load path
 * for every row. Rows b*(K+1)+i beyond i = k_b are never read.
 * Errors (host-detected, nothing enqueued): SV_ERR_STATE, SV_ERR_NULL,
 * SV_ERR_ARG, SV_ERR_ALIGN; SV_ERR_HIP if the launch fails.
 */
int spec_verify_run(spec_verify_ctx* ctx, const void* target_logits,
                    const void* draft_logits, const int32_t* draft_tokens,
                    const int32_t* budgets, int B, int K, float temperature,
                    uint64_t seed, int32_t* out_tokens, int32_t* out_num_accepted,
                    float* out_p_draft, float* out_q_draft, void* stream);

/*
 * spec_verify_run_ex -- spec_verify_run on a slice of a larger batch: row b
 * of the tensors is request request_base + b of the whole batch, and its
 * Philox counters are (request_base + b, i, 0, 0). Requests are independent,
 * so calls over disjoint slices with their own bases give the outputs of one
 * call over the whole batch, bit for bit (how the batch would be split across
 * GPUs, each taking a contiguous range of requests). Arguments as in
 * spec_verify_run; 0 <= request_base <= 2^32 - 1 - B, else SV_ERR_ARG.
 */
int spec_verify_run_ex(spec_verify_ctx* ctx, const void* target_logits,
                       const void* draft_logits, const int32_t* draft_tokens,
                       const int32_t* budgets, int B, int K, float temperature,
                       uint64_t seed, int64_t request_base, int32_t* out_tokens,
                       int32_t* out_num_accepted, float* out_p_draft,
                       float* out_q_draft, void* stream);

/*
 * spec_verify_run_noalloc -- spec_verify_run_ex without a context, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation). It calls no
 * hipMalloc or hipFree: its workspace is a static device array of
 * SV_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until the
 * process ends. It runs on the current HIP device; vocab and dtype are given
 * per call. Every call on one GPU shares that GPU's array: calls that overlap
 * in time on one GPU (on different streams, or from different threads) race
 * and their outputs are undefined; calls in stream order are safe (each call
 * clears the counters it needs with a fill kernel, no memset).
 *   vocab, dtype  as in spec_verify_init.
 *   out_status    uint32 [1] (device) or NULL: this call's SV_FLAG_BAD_BUDGET
 *                 and SV_FLAG_BAD_TOKEN bits (written, not accumulated).
 *   other arguments as in spec_verify_run_ex.
 * Three launches: the fill kernel, the streaming pass and, in sampled mode,
 * the draw pass.
 * Errors (nothing enqueued): SV_ERR_NULL, SV_ERR_ARG, SV_ERR_DTYPE,
 * SV_ERR_ALIGN; SV_ERR_TOO_BIG when the call's workspace (it grows with
 * min(B, 8192) * (K + 1) and the vocabulary's chunk count) exceeds the
 * static array, e.g. B = 512, K = 8, V = 151936 in bf16 or fp32 fits;
 * SV_ERR_HIP if a launch fails.
 */
int spec_verify_run_noalloc(int vocab, int dtype, const void* target_logits,
                            const void* draft_logits, const int32_t* draft_tokens,
                            const int32_t* budgets, int B, int K, float temperature,
                            uint64_t seed, int64_t request_base, int32_t* out_tokens,
                            int32_t* out_num_accepted, float* out_p_draft,
                            float* out_q_draft, uint32_t* out_status, void* stream);

/*
 * spec_verify_check_args -- the host-side argument check of spec_verify_run
 * for a context created with (max_batch, max_k, vocab, dtype), without a
 * context or a device. Pointers are only tested for NULL and alignment,
 * never dereferenced. Returns SV_OK or the code spec_verify_run would return.
 */
int spec_verify_check_args(int max_batch, int max_k, int vocab, int dtype,
                           const void* target_logits, const void* draft_logits,
                           const void* draft_tokens, const void* budgets, int B,
                           int K, float temperature, const void* out_tokens,
                           const void* out_num_accepted, const void* out_p_draft,
                           const void* out_q_draft);

/*
 * spec_verify_status -- wait for the device, return and clear the status
 * word (SV_FLAG_* bits accumulated by runs since the last call).
 * Errors: SV_ERR_STATE, SV_ERR_NULL, SV_ERR_HIP.
 */
int spec_verify_status(spec_verify_ctx* ctx, uint32_t* flags);

/*
 * spec_verify_philox_words -- write the Philox4x32-10 blocks the verifier
 * uses: out_words[(b*P + i)*4 + w] = word w of the block with key = seed and
 * counter = (b, i, 0, 0), for b < B, i < P (device buffer of 4*B*P uint32).
 * Stream-ordered. For checking the device generator against other
 * implementations. Errors: SV_ERR_NULL, SV_ERR_ARG, SV_ERR_HIP.
 */
int spec_verify_philox_words(uint64_t seed, int B, int P, uint32_t* out_words,
                             void* stream);

/*
 * spec_verify_timing -- per-pass device timing of later runs (off by
 * default). enable != 0: every later spec_verify_run on this context records
 * a HIP event pair on its stream around each pass it launches -- pass 0 the
 * streaming pass (row statistics; the greedy decisions and outputs), pass 1
 * the draw pass of sampled mode (accept decisions, first rejection,
 * residual or bonus draw, outputs) -- up to
 * 65536 passes, then recording stops. enable == 0 waits for and discards
 * what is recorded. The events are the context's; recording adds event
 * markers between the launches and nothing else.
 * Errors: SV_ERR_STATE, SV_ERR_HIP.
 */
int spec_verify_timing(spec_verify_ctx* ctx, int enable);

/*
 * spec_verify_timing_read -- wait for the recorded passes, write per pass p
 * (0 streaming, 1 draw) the number of launches counts[p] and the sum of their
 * durations total_ms[p] in milliseconds (host arrays of 2), and clear the
 * record (timing stays as set).
 * Errors: SV_ERR_STATE, SV_ERR_NULL, SV_ERR_HIP.
 */
int spec_verify_timing_read(spec_verify_ctx* ctx, int* counts, double* total_ms);

/*
 * spec_budget_schedule -- per-request verify budgets from per-position
 * confidences ("Speculative decoding becomes standard: DSpark and
 * multi-token drafters", section "What DSpark adds", paragraph 2: each
 * drafted position has a confidence, read as its chance of acceptance once
 * every earlier position of the block was accepted, and verify windows are
 * sized jointly over the batch, shrinking as load grows; the Analytics
 * Vidhya DSpark page, section "Gotchas and Issues": the cut is set afresh
 * for every batch, and a position is verified only if it is expected to
 * pay off). Stream-ordered, no host sync, no context and no workspace.
 *   confidences  float [B, K] row-major (device): c[b, i] for drafted
 *                position i of request b. NaN and negatives read as 0,
 *                values above 1 as 1.
 *   B, K         requests (0..SV_MAX_BATCH; 0 is a no-op) and drafted
 *                positions per request (0..SV_MAX_K).
 *   n_total      the batch's verify budget N >= 0: drafted positions to
 *                verify over all requests (the load sets it).
 *   tau          >= 0, finite: a position is verified only if its gain
 *                exceeds tau.
 *   out_budgets  int32 [B] (device): k_b, ready for spec_verify_run.
 * The gain of position k of request b is g = c[b,0] * c[b,1] * ... * c[b,k]
 * (the expected accepted tokens it adds), multiplied left to right in fp32.
 * The N largest gains above tau are verified, equal gains by position, then
 * request; k_b counts those of request b, always a prefix of its block.
 * sum_b k_b = min(N, number of gains above tau).
 * Errors (nothing enqueued): SV_ERR_ARG, SV_ERR_NULL, SV_ERR_ALIGN (pointers
 * not 4-byte aligned); SV_ERR_HIP if the launch fails.
 */
int spec_budget_schedule(const float* confidences, int B, int K, int n_total, float tau,
                         int32_t* out_budgets, void* stream);

/*
 * spec_head_stats -- row statistics of the shared output head, computed on
 * the matrix cores without writing the logits ("Speculative decoding becomes
 * standard: DSpark and multi-token drafters", section "What DSpark adds",
 * paragraph 1: the drafter reuses the target's output projection unchanged;
 * section "Why draft-and-verify does not change the output", paragraphs 1
 * and 2: a verify step needs each scored row's most likely token, or p(x)
 * and q(x) of the drafted token). Stream-ordered, no host sync.
 *   hidden      bf16 [R, H] row-major (device, 16-byte aligned): hidden
 *               states, one row per scored position (target or drafter).
 *   weight      bf16 [V, H] row-major (device, 16-byte aligned): the head.
 *   R, H, V     rows (>= 0; 0 is a no-op), hidden size (>= 8, a multiple of
 *               8) and vocabulary (1..SV_MAX_VOCAB).
 *   tokens      int32 [R] or NULL: the token whose logit out_ztok reports.
 *   temperature > 0: sampled statistics; 0: greedy (max and argmax only).
 *   out_max     float [R]: m = max_v z[r, v], z = hidden weight^T (fp32
 *               accumulation of exact bf16 products).
 *   out_sumexp  float [R] or NULL: sum_v 2^((z[r, v] - m) log2(e) / T)
 *               (sampled; NaN in greedy mode). p(x) = 2^((z_x - m) log2(e)/T)
 *               / sum.
 *   out_ztok    float [R] or NULL: z[r, tokens[r]], NaN if out of range.
 *   out_argmax  int32 [R] or NULL: the first argmax (greedy; -1 when sampled).
 *   workspace   device scratch of at least spec_head_workspace_bytes(R, V)
 *               bytes (16-byte aligned), caller-owned; calls that share it
 *               must not overlap.
 * Errors (nothing enqueued): SV_ERR_ARG, SV_ERR_NULL, SV_ERR_ALIGN;
 * SV_ERR_HIP if a launch fails.
 */
int spec_head_stats(const void* hidden, const void* weight, int R, int H, int V,
                    const int32_t* tokens, float temperature, float* out_max,
                    float* out_sumexp, float* out_ztok, int32_t* out_argmax,
                    void* workspace, size_t workspace_bytes, void* stream);

/* spec_head_workspace_bytes -- scratch spec_head_stats needs for (R, V):
 * one 16-byte partial per row and vocabulary split (for 1,536 rows or more
 * and V of at least 10,240: 40 per row plus at most ceil(V / 256) / 16 + 4).
 * 0 on bad arguments. Host only. */
size_t spec_head_workspace_bytes(int R, int V);

/*
 * spec_verify_hidden -- one verify step from hidden states through the shared
 * output head: the outputs of spec_verify_run on the logits z = h W^T,
 * without writing the logits of the scored rows anywhere ("Speculative
 * decoding becomes standard: DSpark and multi-token drafters", section "What
 * DSpark adds", paragraph 1: the drafter reuses the target's output
 * projection unchanged; section "Why draft-and-verify does not change the output",
 * paragraphs 1 and 2: the greedy and sampled rules; section "What DSpark
 * adds", paragraph 2: per-request budgets). Logits are fp32 accumulations of
 * exact bf16 products; p and q, the accept test, the Philox counters and the
 * inverse-CDF draw are those of spec_verify_run. Stream-ordered, no host
 * sync; five launches (plan, head statistics, decide, and in sampled mode
 * the head product over each request's draw rows and the draw). With at
 * least 512 requests (when the head's many-row product takes the draw rows)
 * that product leaves per-block draw masses instead of logits, so no logit
 * reaches memory; with fewer it writes the draw rows' fp32 logits to the
 * workspace.
 *   target_hidden  bf16 [B, K+1, H] row-major (device, 16-byte aligned).
 *   draft_hidden   bf16 [B, K, H] (device, 16-byte aligned); may be NULL
 *                  when temperature == 0 or K == 0.
 *   head           bf16 [V, H] row-major (device, 16-byte aligned).
 *   draft_tokens   int32 [B, K] (device); may be NULL when K == 0.
 *   budgets        int32 [B] (device), 0 <= k_b <= K.
 *   B, K, H, V     requests (0..SV_MAX_BATCH; 0 is a no-op), drafted
 *                  positions (0..SV_MAX_K), hidden size (>= 8, a multiple
 *                  of 8), vocabulary (1..SV_MAX_VOCAB).
 *   temperature    > 0 sampled, 0 greedy (drafter states and seed unused).
 *   seed           Philox key; counter (b, i, 0, 0) as in spec_verify_run.
 *   out_tokens     int32 [B, K+1]: x_0..x_{j-1}, y, then -1.
 *   out_num_accepted int32 [B]: j_b.
 *   out_p_draft, out_q_draft  float [B, K] or NULL: p_i(x_i), q_i(x_i) for
 *                  i < k_b, NaN elsewhere and in greedy mode.
 *   out_status     int32 [1] (device) or NULL: this call's SV_FLAG_BAD_BUDGET
 *                  and SV_FLAG_BAD_TOKEN bits (written, not accumulated). A
 *                  flagged request's outputs are undefined.
 *   workspace      device scratch of at least
 *                  spec_verify_hidden_workspace_bytes(B, K, V) bytes,
 *                  256-byte aligned, caller-owned; calls sharing it must not
 *                  overlap. Most of it is the fp32 logits of two rows per
 *                  request (8 B V bytes).
 * Errors (nothing enqueued): SV_ERR_ARG, SV_ERR_NULL, SV_ERR_ALIGN;
 * SV_ERR_HIP if a launch fails.
 */
int spec_verify_hidden(const void* target_hidden, const void* draft_hidden, const void* head,
                       const int32_t* draft_tokens, const int32_t* budgets, int B, int K, int H,
                       int V, float temperature, uint64_t seed, int32_t* out_tokens,
                       int32_t* out_num_accepted, float* out_p_draft, float* out_q_draft,
                       int32_t* out_status, void* workspace, size_t workspace_bytes,
                       void* stream);

/* spec_verify_hidden_workspace_bytes -- scratch spec_verify_hidden needs for
 * (B, K, V); 0 on bad arguments. Host only. */
size_t spec_verify_hidden_workspace_bytes(int B, int K, int V);

/*
 * spec_markov_draft -- the drafter's low-rank Markov head over a block of K
 * drafted positions ("Speculative decoding becomes standard: DSpark and
 * multi-token drafters", section "What DSpark adds", paragraph 1: the block
 * comes from a parallel backbone and a factorised rank-256 Markov model over
 * consecutive positions corrects it; "DSpark" (finds page): the deployed
 * sequential structure conditions only on the preceding token, through a
 * low-rank matrix). For i = 0..K-1 in
 * order: z_i = base_i + A[x_{i-1}] Bm^T, the bias an fp32 sum of exact bf16
 * products, the sum formed in fp32 and rounded once to bf16 (to nearest,
 * ties to even) and stored; x_i = the first (lowest index) argmax of the
 * stored row; x_{-1} = prev_tokens. The stored rows are drafter logits a
 * verify step can read. Stream-ordered, no host sync; K + 2 launches when r
 * is a multiple of 16 up to 256 and V a multiple of 8, else 1 + 2K.
 *   base_logits  bf16 [B, K, V] row-major (device, 16-byte aligned): the
 *                backbone's logits.
 *   markov_a     bf16 [V, r] (device, 16-byte aligned): the previous token's
 *                factor.
 *   markov_b     bf16 [V, r] (device, 16-byte aligned): the vocabulary factor.
 *   prev_tokens  int32 [B] (device): the last token of each sequence.
 *   B, K, r, V   requests (0..SV_MAX_BATCH; 0 is a no-op), positions
 *                (0..SV_MAX_K; 0 is a no-op), rank (>= 8, a multiple of 8),
 *                vocabulary (1..SV_MAX_VOCAB).
 *   out_logits   bf16 [B, K, V] (device, 16-byte aligned, not base_logits).
 *   out_tokens   int32 [B, K] (device): the drafted tokens.
 *   out_status   int32 [1] (device) or NULL: SV_FLAG_BAD_TOKEN if a previous
 *                token is outside [0, V) (written, not accumulated); that
 *                request's outputs are undefined.
 *   workspace    device scratch of at least
 *                spec_markov_draft_workspace_bytes(B, V) bytes, 256-byte
 *                aligned, caller-owned; calls sharing it must not overlap.
 *                It holds two token maps of B entries, three arrays of one
 *                8-byte first-argmax key per request (positions in turn),
 *                and one 8-byte first-argmax entry per request and
 *                vocabulary split for the product of other shapes; the bias
 *                rows never reach memory, and of the stored rows only each
 *                request's best 32 columns per position are read back.
 * Errors (nothing enqueued): SV_ERR_ARG, SV_ERR_NULL, SV_ERR_ALIGN;
 * SV_ERR_HIP if a launch fails.
 */
int spec_markov_draft(const void* base_logits, const void* markov_a, const void* markov_b,
                      const int32_t* prev_tokens, int B, int K, int r, int V, void* out_logits,
                      int32_t* out_tokens, int32_t* out_status, void* workspace,
                      size_t workspace_bytes, void* stream);

/* spec_markov_draft_workspace_bytes -- scratch spec_markov_draft needs for
 * (B, V); 0 on bad arguments. Host only. */
size_t spec_markov_draft_workspace_bytes(int B, int V);

/* spec_verify_free -- release the context (NULL-safe, idempotent on NULL).
 * Waits for the device before freeing the workspace. */
void spec_verify_free(spec_verify_ctx* ctx);

/* spec_verify_strerror -- static text for an sv_status code. */
const char* spec_verify_strerror(int code);

/* spec_verify_chunks -- number of vocabulary chunks a row is split into for
 * (vocab, dtype) in sampled mode (the unit of the workspace's per-chunk
 * records; greedy calls use chunks twice as long), or a negative sv_status
 * on bad arguments. Host only. */
int spec_verify_chunks(int vocab, int dtype);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
