/*
 * softembed.h -- C ABI of libsoftembed: DiffusionGemma's self-conditioning soft
 * embedding on AMD Instinct MI355X (gfx950).
 *
 * The operation (calvarado04.com/tag/vllm, section "Where the shapes stop
 * agreeing", the expected-token-embedding equation, and section "The fix", the
 * per-rank partial S^(r) and the normaliser gamma):
 *
 *     p_i      = softmax(logits_i)               over the FULL vocabulary [0, vocab)
 *     out_i,:  = gamma * sum_{v=s}^{e-1} p_iv * W_shard[v - s, :]
 *
 * One call on the slice [vocab_start, vocab_end) = [s, e) yields exactly one
 * tensor-parallel rank's partial gamma * S^(r).  Summing the calls of a
 * disjoint, exhaustive partition gives the full product (same section, the
 * partition equation).  There is no collective in this library.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All array pointers are DEVICE pointers (hipMalloc'd or equivalent) owned
 *    by the caller.  The library never allocates, frees, synchronises or reads
 *    device memory from the host.  Work is enqueued on `stream` (a hipStream_t;
 *    NULL = the null stream).  Outputs are valid once that stream is
 *    synchronised; inputs must stay alive and unmodified until then.
 *  - Matrices are row-major with a leading dimension (`ld_*`, in elements).
 *    Vocabulary-wide matrices (logits, probs) have column j = vocab id j and are
 *    read only at the columns an entry point documents.  The embedding shard
 *    has row 0 = vocab id `vocab_start`.
 *  - bf16 values are passed as uint16_t bit patterns (IEEE binary32 top half).
 *  - Outputs must not alias inputs or the workspace.
 *  - Every argument check happens synchronously on the host BEFORE anything is
 *    enqueued; on any error nothing is launched and the outputs are untouched.
 *  - Results are bitwise reproducible for the same inputs and shapes on the same
 *    kind of device: the work decomposition depends only on the shapes and the
 *    current device's compute-unit count (the contraction is split over the
 *    vocabulary into the number of pieces that minimises a makespan model of the
 *    shape on that many CUs), and every reduction runs in a fixed order.
 *  - The only global state is a per-device cache of that CU count, read once per
 *    device (std::call_once) from the HIP runtime; without a usable device the
 *    MI355X count, 256, is used.  Besides it, each thread has its own list of
 *    timing markers (se_set_launch_events), empty unless the thread arms it.
 *  - Logits must be finite (not checked on the device).
 *  - n_rows == 0 is a no-op that checks only sizes; its pointers may be NULL.
 *  - Calls are thread-safe and capture-safe (no allocation, no sync, no host
 *    read of device data): a caller may issue them from several threads on
 *    several streams, or capture them into a HIP graph and replay it.
 */
#ifndef SOFTEMBED_H
#define SOFTEMBED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SE_OK = 0,
    SE_ERR_NULL = 1,      /* a required pointer is NULL                                  */
    SE_ERR_SHAPE = 2,     /* negative/zero size where one is required, ld too small,      */
                          /* vocab or d above INT32_MAX, or a buffer the kernels address  */
                          /* with 32-bit byte offsets reaching 4 GiB (2^32 bytes):        */
                          /*  - the staged bf16 probabilities of the staged, step and    */
                          /*    one-pass calls, n_rows * ceil((e - s) / 128) * 256 bytes  */
                          /*    (at e - s = 262,144: at most 8,191 rows per call);        */
                          /*  - the shard slice, (e - s) * ld_w * element size (2 for     */
                          /*    bf16, 1 for e4m3 codes);                                  */
                          /*  - one 256-row tile of the probability operand of            */
                          /*    se_soft_embed / se_soft_embed_fused and their e4m3 forms, */
                          /*    255 * ld * element size + (e - s) * element size (fp32    */
                          /*    logits: 4, bf16 probabilities: 2);                        */
                          /*  - a one-pass slice of logits, (e - s) * 4 bytes.            */
                          /* Larger work is split into several calls by rows or slices.   */
    SE_ERR_SLICE = 3,     /* not 0 <= vocab_start <= vocab_end <= vocab, or the slice is  */
                          /* longer than the shard (vocab_end - vocab_start > w_rows)     */
    SE_ERR_ALIGN = 4,     /* pointer not 16-byte aligned, a row pitch not a multiple of   */
                          /* 16 bytes, vocab_start % 8 != 0, or d % 8 != 0                */
    SE_ERR_WORKSPACE = 5, /* workspace smaller than se_soft_embed_workspace_bytes()       */
    SE_ERR_HIP = 6        /* the HIP runtime reported an error when launching             */
} se_status;

/* Human-readable name of a status code (static storage). */
const char* se_status_string(se_status s);

/* Number of kernels / version, for diagnostics. */
const char* se_version(void);

/*
 * se_set_launch_events -- per-kernel timing markers for the calling thread.
 *
 * events: n_events HIP events (hipEvent_t, passed as void*), created by the caller
 * (with timing enabled, to read durations) and owned by it; they must stay valid until
 * the kernels that use them have run.  After this call, every kernel the calling thread
 * launches through this library takes the next two events of the list, in launch order:
 * the dispatch itself stamps the first with the kernel's start and the second with its
 * end (hipExtLaunchKernel), so the time between them is that kernel's own duration and
 * the stream carries no extra command.  Once fewer than two events remain, launches take
 * none.  An entry point that makes k launches thus uses 2k events.  n_events == 0
 * (events may then be NULL) disarms the markers.  The markers are thread-local: other
 * threads' calls are unaffected.  Not for use under graph capture.
 * Errors: SE_ERR_SHAPE if n_events < 0; SE_ERR_NULL if events is NULL with
 * n_events > 0.
 */
se_status se_set_launch_events(void* const* events, int32_t n_events);

/* Events handed to launches (two per launch) since the calling thread last armed them
 * with se_set_launch_events. */
int32_t se_launch_events_used(void);

/*
 * se_row_stats -- softmax statistics of each logits row over the full width.
 *
 * Definitions (agentlenshq DiffusionGemma overview, "sampling loop and
 * entropy-bound denoising": acceptance orders positions by confidence and the
 * convergence test uses a stable argmax and the mean per-token entropy; the
 * softmax itself is over the full vocabulary as on calvarado04.com, "Where the
 * shapes stop agreeing"):
 *     row_max[i]     = max_v l_iv
 *     row_argmax[i]  = smallest v with l_iv = row_max[i]
 *     row_lse[i]     = log sum_v exp(l_iv)                       (natural log)
 *     row_entropy[i] = -sum_v p_iv log p_iv, p = softmax(l_i)    (nats)
 *
 * logits:  fp32 [n_rows, ld_logits], columns [0, vocab) are read.
 * outputs: fp32 row_max/row_lse/row_entropy [n_rows], int32 row_argmax [n_rows].
 * n_rows == 0 is a no-op.  Requires vocab >= 1, ld_logits >= vocab,
 * logits 16-byte aligned and ld_logits % 4 == 0; outputs 4-byte aligned.
 */
se_status se_row_stats(const float* logits, int64_t ld_logits, int64_t n_rows, int64_t vocab,
                       float* row_max, float* row_lse, float* row_entropy,
                       int32_t* row_argmax, void* stream);

/*
 * se_probs_bf16 -- materialise the probability slice for the unfused path.
 *
 *     probs[i, v] = bf16_rne( exp(logits[i, v] - row_lse[i]) )   for v in [s, e)
 *
 * (calvarado04.com, "The fix": the probability slice is cast to the embedding
 * dtype before the product; rounding is to nearest, ties to even.)
 * Only columns [s, e) of probs are written.  row_lse comes from se_row_stats.
 * Requires 0 <= s <= e <= vocab, s % 8 == 0, ld_logits % 4 == 0,
 * ld_probs % 8 == 0, ld_* >= vocab, 16-byte aligned logits/probs.
 */
se_status se_probs_bf16(const float* logits, int64_t ld_logits, const float* row_lse,
                        int64_t n_rows, int64_t vocab, int64_t vocab_start, int64_t vocab_end,
                        uint16_t* probs, int64_t ld_probs, void* stream);

/*
 * se_soft_embed_workspace_bytes -- device workspace the two soft-embed entry
 * points need for this shape (0 when the contraction is not split).  It
 * depends on the shape and the current device's CU count, so query it with the
 * device current that the calls will run on.  Returns 0 for shapes the calls
 * would reject.
 */
size_t se_soft_embed_workspace_bytes(int64_t n_rows, int64_t vocab_start, int64_t vocab_end,
                                     int64_t d);

/*
 * se_soft_embed_splits -- the number S of vocabulary ranges the contraction cuts the
 * slice [s, e) into for this shape on the current device (split-K; 0 for shapes the
 * calls would reject or that have nothing to contract).  With nb = ceil((e - s) / 128)
 * blocks of 128 positions, range r holds the slice positions
 *     [128 floor(r nb / S), min(128 floor((r + 1) nb / S), e - s)),   r = 0 .. S-1.
 * Every contraction adds its ranges' partial products in the order r = 0 .. S-1; the
 * one-read calls (se_soft_embed_onepass, se_soft_embed_step_onepass) also normalise each
 * range's probabilities against that range's own maximum, so their roundings follow these
 * ranges.
 */
int64_t se_soft_embed_splits(int64_t n_rows, int64_t vocab_start, int64_t vocab_end, int64_t d);

/*
 * se_soft_embed -- gamma * P[:, s:e] W_shard[0:e-s, :] from materialised bf16
 * probabilities (calvarado04.com, "The fix": the slice of the gathered
 * probabilities times the local shard, then the normaliser).
 *
 * probs:   bf16 [n_rows, ld_probs]; columns [s, e) are read.
 * w_shard: bf16 [w_rows, ld_w]; rows [0, e - s) and columns [0, d) are read.
 *          Rows at or past e - s (the next rank's rows, or padding) are never
 *          read, so padding may hold anything.
 * out:     fp32 [n_rows, ld_out]; columns [0, d) are written (fp32 accumulate).
 * workspace: device buffer of at least se_soft_embed_workspace_bytes() bytes
 *          (may be NULL when that is 0); its contents are scratch.
 * An empty slice (s == e) writes zeros.  n_rows == 0 is a no-op.
 * Requires 0 <= s <= e <= vocab, e - s <= w_rows, s % 8 == 0, d % 8 == 0,
 * ld_probs % 8 == 0, ld_w % 8 == 0, ld_out % 4 == 0, ld_probs >= vocab,
 * ld_w >= d, ld_out >= d, 16-byte aligned pointers.
 */
se_status se_soft_embed(const uint16_t* probs, int64_t ld_probs, int64_t n_rows, int64_t vocab,
                        int64_t vocab_start, int64_t vocab_end,
                        const uint16_t* w_shard, int64_t w_rows, int64_t ld_w, int64_t d,
                        float gamma, float* out, int64_t ld_out,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * se_soft_embed_fused -- as se_soft_embed, but the bf16 probabilities are
 * rebuilt from the fp32 logits and row_lse inside the contraction, so the
 * probability matrix is never written to memory.  Same rounding as
 * se_probs_bf16 (bf16 nearest-even of exp(l - lse)), same accumulation.
 * Not the fast path on MI355X: each 256-column tile of the output pulls the fp32
 * logits through its compute unit again (4 bytes per probability, against 2 for
 * staged bf16), and the bytes all compute units pull together through L2 and HBM
 * bound this contraction; the same result comes faster from se_soft_embed_staged
 * (and, with the statistics, from se_soft_embed_step / se_soft_embed_step_onepass).
 *
 * logits:  fp32 [n_rows, ld_logits]; columns [s, e) are read.
 * row_lse: fp32 [n_rows] from se_row_stats over the FULL width [0, vocab).
 * Other arguments and requirements as se_soft_embed, with ld_logits % 4 == 0
 * and ld_logits >= vocab.
 */
se_status se_soft_embed_fused(const float* logits, int64_t ld_logits, const float* row_lse,
                              int64_t n_rows, int64_t vocab, int64_t vocab_start,
                              int64_t vocab_end,
                              const uint16_t* w_shard, int64_t w_rows, int64_t ld_w, int64_t d,
                              float gamma, float* out, int64_t ld_out,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * se_soft_embed_staged -- the result of se_soft_embed_fused, bit for bit, computed by
 * staging the bf16 probabilities of the slice in the workspace in a layout the
 * contraction streams in 1 KB runs ([super-step of 128 positions][row][128]).  On
 * MI355X at the pages' shapes the extra 2 * n_rows * (e - s) bytes written and read
 * back cost less than re-reading fp32 logits once per 256-column tile of the fused
 * kernel.  Arguments and errors as se_soft_embed_fused, with a workspace of
 * se_soft_embed_staged_workspace_bytes() bytes (16-byte aligned); an empty slice
 * writes zeros and needs no workspace.
 */
size_t se_soft_embed_staged_workspace_bytes(int64_t n_rows, int64_t vocab_start,
                                            int64_t vocab_end, int64_t d);

se_status se_soft_embed_staged(const float* logits, int64_t ld_logits, const float* row_lse,
                               int64_t n_rows, int64_t vocab, int64_t vocab_start,
                               int64_t vocab_end, const uint16_t* w_shard, int64_t w_rows,
                               int64_t ld_w, int64_t d, float gamma, float* out, int64_t ld_out,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * se_soft_embed_step -- one whole sampler step for a rank in one call: se_row_stats
 * over the full width [0, vocab) followed by se_soft_embed_fused on [s, e), with
 * outputs bit for bit those of the two calls.  The statistics kernel writes the
 * slice's bf16 probabilities (staged, as se_soft_embed_staged) right after each
 * row's statistics, and one launch boundary disappears.  The kernel keeps the slice's
 * first (up to) 4 groups of 16,384 positions in registers as they stream past, when they
 * are whole groups of the row; a slice within them (a tensor-parallel rank's share of a
 * large vocabulary at 4 or more ranks) is read only once, and the rest of a longer slice
 * is read again (from whatever cache level still holds it; at the pages' shapes that
 * second read misses the L2).
 * Arguments: those of se_row_stats and se_soft_embed_fused together (row_max,
 * row_lse, row_entropy and row_argmax are outputs here); workspace of
 * se_soft_embed_staged_workspace_bytes() bytes (16-byte aligned; none for an empty
 * slice).  Errors as those calls.
 */
se_status se_soft_embed_step(const float* logits, int64_t ld_logits, int64_t n_rows,
                             int64_t vocab, int64_t vocab_start, int64_t vocab_end,
                             const uint16_t* w_shard, int64_t w_rows, int64_t ld_w, int64_t d,
                             float gamma, float* out, int64_t ld_out, float* row_max,
                             float* row_lse, float* row_entropy, int32_t* row_argmax,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * se_soft_embed_step_noalloc -- se_soft_embed_step for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the workspace is a device array owned by the library, of
 * se_soft_embed_step_noalloc_max_bytes() bytes (128 MiB), one per GPU, held from the
 * moment the library's code is loaded on that GPU until the process ends.  Its device
 * address is looked up once per device on the first call there.  The call allocates
 * nothing and returns exactly what se_soft_embed_step returns for the same arguments with
 * that array as its workspace.
 * Arguments: those of se_soft_embed_step without the workspace.
 * Limit: shapes whose se_soft_embed_staged_workspace_bytes() exceeds the array return
 * SE_ERR_WORKSPACE and launch nothing (the one-rank shape, 256 rows by a 65,536-position
 * slice at d = 2,816, needs about 95 MiB; a whole 262,144-position vocabulary does not fit).
 * Every call on one GPU shares that GPU's array, so calls that overlap on one GPU (on
 * different streams or threads) race: serialise them.  Nothing in the array needs to
 * start at any value; it keeps the last call's contents.  SE_ERR_HIP if the array's
 * address cannot be obtained.  Other errors as se_soft_embed_step.
 */
size_t se_soft_embed_step_noalloc_max_bytes(void);

se_status se_soft_embed_step_noalloc(const float* logits, int64_t ld_logits, int64_t n_rows,
                                     int64_t vocab, int64_t vocab_start, int64_t vocab_end,
                                     const uint16_t* w_shard, int64_t w_rows, int64_t ld_w,
                                     int64_t d, float gamma, float* out, int64_t ld_out,
                                     float* row_max, float* row_lse, float* row_entropy,
                                     int32_t* row_argmax, void* stream);

/*
 * se_soft_embed_step_fp8 -- se_soft_embed_step against an e4m3 table with per-row
 * power-of-two scales (as se_quantize_table_fp8 writes them; the pages serve FP8
 * weights: agentlenshq overview of DiffusionGemma in vLLM, performance and
 * quantization).  Outputs are bit for bit those of se_row_stats followed by
 * se_soft_embed_fp8_fused.  With a 16-byte aligned w_scale the statistics pass stores each
 * slice probability times its row's scale and the contraction reads the codes as they are
 * (as se_soft_embed_step_onepass_fp8 does; the same bits wherever every stored probability
 * stays in bf16's normal range); otherwise the contraction turns the codes into bf16 rows.
 * Arguments: those of se_soft_embed_step with the table given as w_codes (uint8
 * [w_rows, ld_w]) and w_scale (fp32 [w_rows]) as in se_soft_embed_fp8; workspace of
 * se_soft_embed_staged_workspace_bytes() bytes.  Errors as se_soft_embed_step, and those
 * of se_soft_embed_fp8's table checks.
 */
se_status se_soft_embed_step_fp8(const float* logits, int64_t ld_logits, int64_t n_rows,
                                 int64_t vocab, int64_t vocab_start, int64_t vocab_end,
                                 const uint8_t* w_codes, const float* w_scale, int64_t w_rows,
                                 int64_t ld_w, int64_t d, float gamma, float* out,
                                 int64_t ld_out, float* row_max, float* row_lse,
                                 float* row_entropy, int32_t* row_argmax, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * se_soft_embed_step_onepass -- the same step as se_soft_embed_step (row statistics
 * over the full width [0, vocab), the slice's soft embedding against them) from ONE
 * read of the logits.  The row is cut into ranges: [0, s) and [e, vocab) in chunks,
 * and the slice in the contraction's split ranges.  Each range yields its maximum,
 * first argmax, Z_r = sum e^(l - m_r) and S1_r = sum e^(l - m_r)(l - m_r); each slice
 * range also writes its bf16 probabilities against its own maximum,
 * bf16_rne(e^(l - m_r)).  The ranges merge at the row maximum M,
 *     Z = sum_r e^(m_r - M) Z_r,  lse = M + ln Z,
 *     H = ln Z - sum_r e^(m_r - M) (S1_r + (m_r - M) Z_r) / Z,
 * and the contraction of split r is scaled by gamma e^(m_r - lse) before the splits are
 * summed in order: the partition identity of calvarado04.com, "The fix" (a sum over
 * disjoint vocabulary pieces), applied to softmax numerators.  Results agree with
 * se_soft_embed_step to rounding (argmax and row max exactly), are bitwise repeatable,
 * but are not bitwise those of the two-pass calls.
 * When the slice is empty, or one split range is longer than 24,576 positions (the
 * sweep holds a range in the registers of at most 8 wavefronts), the call is
 * se_soft_embed_step itself.
 * Arguments and errors as se_soft_embed_step, with a workspace of
 * se_soft_embed_step_onepass_workspace_bytes() bytes (16-byte aligned): the bf16
 * slice, the split partials and per-(range, row) statistics.
 */
size_t se_soft_embed_step_onepass_workspace_bytes(int64_t n_rows, int64_t vocab,
                                                  int64_t vocab_start, int64_t vocab_end,
                                                  int64_t d);

se_status se_soft_embed_step_onepass(const float* logits, int64_t ld_logits, int64_t n_rows,
                                     int64_t vocab, int64_t vocab_start, int64_t vocab_end,
                                     const uint16_t* w_shard, int64_t w_rows, int64_t ld_w,
                                     int64_t d, float gamma, float* out, int64_t ld_out,
                                     float* row_max, float* row_lse, float* row_entropy,
                                     int32_t* row_argmax, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * se_soft_embed_step_onepass_fp8 -- se_soft_embed_step_onepass against an e4m3 table with
 * per-row power-of-two scales 2^k_v, as se_quantize_table_fp8 writes them (the FP8
 * weights of the agentlenshq overview of DiffusionGemma in vLLM, section on performance
 * and quantization).  The sweep stores each slice probability times its table row's
 * scale, bf16_rne(e^(l - m_r) 2^k_v) = bf16_rne(e^(l - m_r)) 2^k_v, and the contraction
 * multiplies those by the codes themselves (every e4m3 value is exact in bf16): the
 * partition identity of calvarado04.com, "The fix", with each term's scale moved from the
 * table row to the probability.  The result is se_soft_embed_step_onepass's on the
 * dequantized table (codes times scales) bit for bit wherever every stored probability
 * stays in bf16's normal range (a probability below 2^-126 / 2^k_v may round differently;
 * such a term is below 2^-117 in magnitude).
 * Arguments as se_soft_embed_step_fp8, with w_scale 16-byte aligned, and a workspace of
 * se_soft_embed_step_onepass_workspace_bytes() bytes (16-byte aligned).  Shapes the sweep
 * cannot take (empty slice, a split range longer than 24,576 positions) run as
 * se_soft_embed_step_fp8 in the same workspace.  Errors as se_soft_embed_step_fp8, and
 * SE_ERR_ALIGN for a w_scale that is not 16-byte aligned.
 */
se_status se_soft_embed_step_onepass_fp8(const float* logits, int64_t ld_logits,
                                         int64_t n_rows, int64_t vocab, int64_t vocab_start,
                                         int64_t vocab_end, const uint8_t* w_codes,
                                         const float* w_scale, int64_t w_rows, int64_t ld_w,
                                         int64_t d, float gamma, float* out, int64_t ld_out,
                                         float* row_max, float* row_lse, float* row_entropy,
                                         int32_t* row_argmax, void* workspace,
                                         size_t workspace_bytes, void* stream);

/*
 * se_quantize_table_fp8 -- the e4m3 form of a bf16 embedding table (the pages serve
 * the model with FP8 weights: agentlenshq overview of DiffusionGemma in vLLM,
 * section on performance and quantization, quantized checkpoints).
 *
 * Per row v:  k_v = the smallest integer >= -126 with max_j |w[v, j]| <= 448 * 2^k_v
 *             (k_v = 0 for an all-zero row; 448 is the largest finite e4m3 value),
 *             row_scale[v] = 2^k_v (an exact power of two),
 *             codes[v, j]  = e4m3_rne(w[v, j] * 2^-k_v)   (OCP FP8 E4M3: 1 sign,
 *                            4 exponent bits with bias 7, 3 mantissa bits, no
 *                            infinities; nearest value, ties to even code; the sign
 *                            of a zero result is the input's).
 * code * scale is exactly representable in bf16, so the e4m3 table dequantizes
 * exactly to bf16.
 *
 * w: bf16 [rows, ld_w], columns [0, d) read; values must be finite.
 * codes: uint8 [rows, ld_codes], columns [0, d) written.  row_scale: fp32 [rows].
 * Errors: SE_ERR_SHAPE if rows < 0, d < 1, ld_w < d or ld_codes < d; SE_ERR_NULL for
 * a NULL pointer (rows > 0); SE_ERR_ALIGN unless d % 16 == 0, ld_w % 8 == 0,
 * ld_codes % 16 == 0, w and codes 16-byte and row_scale 4-byte aligned.
 * rows == 0 is a no-op.
 */
se_status se_quantize_table_fp8(const uint16_t* w, int64_t ld_w, int64_t rows, int64_t d,
                                uint8_t* codes, int64_t ld_codes, float* row_scale,
                                void* stream);

/*
 * se_soft_embed_fp8 / se_soft_embed_fp8_fused -- se_soft_embed / se_soft_embed_fused
 * with the shard in the e4m3 form of se_quantize_table_fp8:
 *
 *     out_i,: = gamma * sum_{v=s}^{e-1} p_iv * (codes[v - s, :] * w_scale[v - s])
 *
 * The table enters the bf16 MFMA contraction as code * scale, which is exact, so
 * the result equals se_soft_embed(_fused) on the dequantized bf16 table bit for bit
 * (same probabilities, same accumulation order).
 *
 * w_codes: uint8 [w_rows, ld_w], rows [0, e - s) and columns [0, d) read.
 * w_scale: fp32 [w_rows], entries [0, e - s) read; each must be a power of two in
 *          the normal range (as se_quantize_table_fp8 writes them).
 * Other arguments, the workspace and the errors as se_soft_embed(_fused), and in
 * addition: SE_ERR_NULL if w_scale is NULL; SE_ERR_ALIGN unless d % 16 == 0,
 * ld_w % 16 == 0 and w_scale is 4-byte aligned.
 */
se_status se_soft_embed_fp8(const uint16_t* probs, int64_t ld_probs, int64_t n_rows, int64_t vocab,
                            int64_t vocab_start, int64_t vocab_end, const uint8_t* w_codes,
                            const float* w_scale, int64_t w_rows, int64_t ld_w, int64_t d,
                            float gamma, float* out, int64_t ld_out, void* workspace,
                            size_t workspace_bytes, void* stream);

se_status se_soft_embed_fp8_fused(const float* logits, int64_t ld_logits, const float* row_lse,
                                  int64_t n_rows, int64_t vocab, int64_t vocab_start,
                                  int64_t vocab_end, const uint8_t* w_codes, const float* w_scale,
                                  int64_t w_rows, int64_t ld_w, int64_t d, float gamma,
                                  float* out, int64_t ld_out, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * se_soft_embed_onepass -- the soft embedding and the row statistics of a vocabulary
 * slice from ONE read of its logits (no se_row_stats pass first).  The softmax is
 * over the slice [s, e) itself:
 *
 *     q_iv     = e^(l_iv) / sum_{u=s}^{e-1} e^(l_iu)                 for v in [s, e)
 *     out_i,:  = gamma * sum_{v=s}^{e-1} q_iv * W_shard[v - s, :]
 *     row_max, row_argmax (a vocabulary id), row_lse, row_entropy: as se_row_stats,
 *     over columns [s, e)
 *
 * With [s, e) = [0, vocab) this is se_row_stats followed by se_soft_embed_fused.  On
 * a rank's slice it is the slice-local result that se_merge_slices combines across
 * slices (calvarado04.com, "The fix": the vocabulary-sharded layout; each rank then
 * needs only its own logits columns).  Internally the slice is cut into the
 * contraction's split ranges; each range's probabilities are taken against the
 * range's own maximum (bf16, round to nearest even), contracted in fp32, and the
 * ranges are merged with the rescaling rule e^(m_r - m) before dividing by the sum.
 *
 * logits: fp32 [n_rows, ld_logits], columns [s, e) read.  Other arguments as
 * se_soft_embed_fused, with row_max / row_lse / row_entropy (fp32) and row_argmax
 * (int32) of [n_rows] written, and a workspace of se_soft_embed_onepass_workspace_bytes
 * (it holds the bf16 probabilities of the slice, the split partials and per-split
 * statistics: about 2 * n_rows * (e - s) bytes plus the partials).
 * Errors as se_soft_embed_fused, and SE_ERR_SLICE for an empty slice (s == e);
 * SE_ERR_NULL / SE_ERR_ALIGN for a NULL or misaligned statistics output or workspace.
 */
size_t se_soft_embed_onepass_workspace_bytes(int64_t n_rows, int64_t vocab_start,
                                             int64_t vocab_end, int64_t d);

se_status se_soft_embed_onepass(const float* logits, int64_t ld_logits, int64_t n_rows,
                                int64_t vocab, int64_t vocab_start, int64_t vocab_end,
                                const uint16_t* w_shard, int64_t w_rows, int64_t ld_w, int64_t d,
                                float gamma, float* out, int64_t ld_out, float* row_max,
                                float* row_lse, float* row_entropy, int32_t* row_argmax,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * se_merge_slices -- combine the se_soft_embed_onepass results of T disjoint slices,
 * given in vocabulary order, into the result over their union (the full vocabulary
 * when the slices partition it).  With lse = ln sum_r e^(lse_r), slice r carries the
 * probability mass pi_r = e^(lse_r - lse) (calvarado04.com, "The fix": the partition
 * of the product over vocabulary slices, here with each slice normalised by itself):
 *
 *     out = sum_r pi_r out_r,            row_lse = lse,
 *     row_entropy = sum_r pi_r (H_r - ln pi_r),
 *     row_max = max_r max_r,  row_argmax = the argmax of the first slice reaching it.
 *
 * Slice r's output is the fp32 matrix [n_rows, d] at outs + r * part_stride (row pitch
 * ld_part); its statistics are part_max / part_lse / part_entropy / part_argmax
 * [r * n_rows + i].  Slices are added in order r = 0 .. n_parts-1 (fp32).
 * Errors: SE_ERR_SHAPE if n_parts < 1, n_rows < 0 or > 65535, d < 1, a pitch < d, or
 * part_stride < n_rows * ld_part; SE_ERR_NULL for a NULL pointer (n_rows > 0);
 * SE_ERR_ALIGN unless d, the pitches and part_stride are multiples of 4, outs / out
 * are 16-byte and the statistics arrays 4-byte aligned.  n_rows == 0 is a no-op.
 */
se_status se_merge_slices(const float* outs, int64_t n_parts, int64_t part_stride,
                          int64_t n_rows, int64_t d, int64_t ld_part, const float* part_max,
                          const float* part_lse, const float* part_entropy,
                          const int32_t* part_argmax, float* out, int64_t ld_out,
                          float* row_max, float* row_lse, float* row_entropy,
                          int32_t* row_argmax, void* stream);

/*
 * se_accept_converge -- entropy-bound acceptance and the convergence test of the
 * diffusion sampler, on the statistics se_row_stats produces (agentlenshq overview
 * of DiffusionGemma in vLLM, section on the sampling loop and entropy-bound
 * denoising: tokens are accepted from the most to the least confident until the
 * cumulative entropy exceeds a fixed budget; a canvas has converged when its argmax
 * prediction has been stable for several steps and its mean per-token entropy is
 * below a threshold, or when a step limit is reached).
 *
 * The rows are n_canvas canvases of canvas_len consecutive positions each
 * (row c * canvas_len + i is position i of canvas c).  Per canvas, one call:
 *   1. candidates = positions with accepted[] == 0, ordered by entropy ascending,
 *      ties by lower position;
 *   2. entropies enter as exact fixed-point integers q = round_half_even(H * 2^32)
 *      (2^-32 nat resolution), so cumulative sums are exact and order-free;
 *   3. the candidates taken are the prefix of that order before the first one whose
 *      cumulative sum exceeds entropy_budget * 2^32 (compared in double), but at
 *      least one when any candidate is left; they get newly_accepted = 1 and
 *      accepted = 1 (every other position: newly_accepted = 0);
 *   4. stable_count = (row_argmax == prev_argmax at every position) ?
 *      stable_count + 1 : 0;  prev_argmax = row_argmax;  step_count += 1;
 *   5. converged = (stable_count >= stable_steps && sum(q) < entropy_tau *
 *      canvas_len * 2^32) || step_count >= step_limit.
 * The budget, stable_steps, tau and step_limit values are the caller's: the pages
 * give none.
 *
 * row_entropy: fp32 [n_canvas * canvas_len] (nats); row_argmax: int32, same size.
 * State (in/out, caller-owned, initialise once per canvas: accepted = 0,
 * prev_argmax = -1, stable_count = 0, step_count = 0):
 *   accepted: uint8 [n_canvas * canvas_len]; prev_argmax: int32, same size;
 *   stable_count, step_count: int32 [n_canvas].
 * Outputs: newly_accepted: uint8 [n_canvas * canvas_len]; converged: uint8 [n_canvas].
 * Errors: SE_ERR_SHAPE if n_canvas < 0, canvas_len < 1 or > 1024, stable_steps < 1,
 * step_limit < 1, or entropy_budget / entropy_tau is NaN; SE_ERR_NULL for a NULL
 * pointer (n_canvas > 0); SE_ERR_ALIGN if an int32 or fp32 array is not 4-byte
 * aligned.  n_canvas == 0 is a no-op.
 */
se_status se_accept_converge(const float* row_entropy, const int32_t* row_argmax,
                             int64_t n_canvas, int64_t canvas_len, double entropy_budget,
                             int32_t stable_steps, double entropy_tau, int32_t step_limit,
                             uint8_t* accepted, int32_t* prev_argmax, int32_t* stable_count,
                             int32_t* step_count, uint8_t* newly_accepted, uint8_t* converged,
                             void* stream);

/*
 * se_reduce_partials -- E^sc = sum_r S^(r) over T partials that sit on one GPU
 * (calvarado04.com/tag/vllm, section "The fix": the per-rank partials are summed
 * by one all-reduce and the result is in the embedding dtype).  Each partial is
 * the output of one slice call (gamma already applied); part r is the fp32 matrix
 * [n_rows, d] at parts + r * part_stride with row pitch ld_part.  Parts are added
 * in the order r = 0 .. n_parts-1 in fp32.  The sum is written to out (fp32, row
 * pitch ld_out) and / or to out_bf16 (bf16 bits, round to nearest even, row pitch
 * ld_bf16); either output may be NULL, not both.
 * Errors: SE_ERR_SHAPE if n_parts < 1, n_rows < 0, d < 1, a pitch < d, or
 * part_stride < n_rows * ld_part; SE_ERR_NULL if parts is NULL or both outputs are
 * (n_rows > 0); SE_ERR_ALIGN if d or a pitch (or part_stride) is not a multiple of
 * 4, or parts / out is not 16-byte or out_bf16 not 8-byte aligned.  n_rows == 0
 * is a no-op.
 */
se_status se_reduce_partials(const float* parts, int64_t n_parts, int64_t part_stride,
                             int64_t n_rows, int64_t d, int64_t ld_part, float* out,
                             int64_t ld_out, uint16_t* out_bf16, int64_t ld_bf16, void* stream);

/*
 * se_mfma_loop -- measurement aid: the bf16 matrix-core rate this device sustains, the
 * achievable ceiling read beside the nominal peak when the contraction's roofline is
 * assessed (the nominal 2.5 PFLOP/s assumes the 2.4 GHz peak clock; under load the clock
 * runs lower).  Not part of the soft embedding.
 *
 * Launches `blocks` workgroups of 256 threads (4 waves).  Each wave runs 8 independent
 * chains of `iters` v_mfma_f32_32x32x16_bf16 (32 x 32 x 16, fp32 accumulate) on register
 * operands whose every element is bf16(unit) (unit's top 16 bits), reads no memory, and
 * stores one float per lane: the sum of its 8 x 16 accumulator elements, so
 *     out[b * 256 + t] = 8 * 16 * iters * (16 * bf16(unit)^2)   (fp32, exact when small).
 * Work per call: blocks * 4 * 8 * iters * 32,768 FLOP.
 * out: fp32 [blocks * 256], 4-byte aligned, written.
 * Errors: SE_ERR_SHAPE unless 1 <= blocks <= 65,536 and 1 <= iters <= 2^24; SE_ERR_NULL
 * if out is NULL; SE_ERR_ALIGN if out is not 4-byte aligned.
 */
se_status se_mfma_loop(float* out, int64_t blocks, int64_t iters, float unit, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SOFTEMBED_H */
