/*
 * snapkv.h - C ABI of the SnapKV prefill-time KV-cache compression library
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation (per prompt b of length L, per KV head h; P = L - W):
 *
 *   1. vote    s_h[j] = sum over the G = H_q/H_kv query heads of h's group and
 *              over the W observation-window rows i of the causal attention
 *              probability softmax_j'(q_i . k_j' / sqrt(D)), j' <= P + i,
 *              taken at key j < P;
 *   2. pool    c_h = s_h smoothed with a stride-1 window of kernel_size
 *              positions (average: window sum / kernel_size, positions
 *              outside [0, P) count as zero; max: in-range maximum);
 *   3. select  the top B - W positions of c_h (ties to the lower position),
 *              in ascending order, followed by the window positions P..L-1;
 *   4. gather  those rows of K and V into a B-entry compressed cache.
 *   A prompt with L <= B is kept whole (indices 0..L-1).
 *
 * Sources: glossary page "SnapKV(スナップケーブイ)", section "SnapKVの仕組み"
 * (observation window of the last 16-64 prompt tokens; per-head attention
 * scores aggregated; only a budget of B pairs kept; decode on the compressed
 * cache; pooling of neighbouring scores before selection), section
 * "実装と統合" (the four hyperparameters window_size, max_capacity_prompt,
 * kernel_size, pooling), FAQ Q1 (MHA and GQA models); paper page "SnapKV: LLM
 * Knows What You are Looking for Before Generation", abstract (selection of
 * clustered important KV positions for each attention head, from an
 * observation window at the end of the prompt) and section "기술적 접근법"
 * (max or average pooling, kernel 5-13, window 16-64, budget 1024-4096).
 * Where the pages are silent (softmax scale 1/sqrt(D); the causal row
 * includes the window's own keys; aggregation is a sum; the budget B counts
 * the W window rows; zero padding with division by kernel_size; lowest-index
 * ties) the plainest reading is taken.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - bf16 tensors are passed as raw device pointers to bfloat16 bit patterns.
 *   Layouts (row-major, innermost last):
 *     q_win  [batch, H_q, W, D]  queries of positions L-W..L-1 of each prompt
 *     k, v   [T, H_kv, D]        prompts packed back to back, T = sum(L_b)
 *     out_k, out_v [batch, H_kv, B, D]
 *     out_idx      [batch, H_kv, B] int32, positions relative to the prompt
 *   Query head q belongs to KV head q / G (contiguous groups).
 * - seq_lens is a HOST pointer to int32[batch]; it is read during the call only.
 * - Device pointers must be 16-byte aligned.
 * - The caller owns every buffer. The library allocates no memory and keeps no
 *   pointer after a call returns. Inputs are read-only.
 * - stream is a hipStream_t (NULL = the default stream). All device work is
 *   enqueued on it and the call returns without synchronising; outputs are
 *   valid once the stream has reached that point. Calls are re-entrant when
 *   they use distinct workspaces; two calls in flight must not share one.
 * - Errors are reported by status code only. Argument checks run entirely on
 *   the host before any HIP call: on SNAPKV_ERR_INVALID_ARGUMENT,
 *   SNAPKV_ERR_UNSUPPORTED or SNAPKV_ERR_WORKSPACE nothing is enqueued and no
 *   output is touched. SNAPKV_ERR_HIP reports a failed launch; outputs are
 *   then undefined. snapkv_last_error() gives the detail (per thread).
 */
#ifndef SNAPKV_H_
#define SNAPKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SNAPKV_OK 0
#define SNAPKV_ERR_INVALID_ARGUMENT 1
#define SNAPKV_ERR_UNSUPPORTED 2
#define SNAPKV_ERR_WORKSPACE 3
#define SNAPKV_ERR_HIP 4

#define SNAPKV_POOL_AVG 0 /* "avgpool" */
#define SNAPKV_POOL_MAX 1 /* "maxpool" */

#define SNAPKV_MAX_BATCH 256       /* prompts per call */
#define SNAPKV_MAX_ROWS 512        /* G * W, window rows scored per KV head */
#define SNAPKV_MAX_KERNEL 2049     /* largest pooling kernel */
#define SNAPKV_NUM_STAGES 4        /* stages: vote statistics, vote + pool,
                                      select, gather */

/*
 * Bytes of device workspace that snapkv_compress, snapkv_compress_staged and
 * snapkv_window_scores need for this shape (the same size serves all three).
 * The workspace holds intermediate results only (per-chunk softmax
 * statistics and pooled score vectors, each written before it is read): it
 * needs no initialisation and may be reused across calls and shapes, but not
 * by two calls in flight at once.
 * Returns SNAPKV_OK and writes *bytes, or an error status under the
 * validation rules of snapkv_compress.
 */
int32_t snapkv_workspace_size(int32_t batch, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim,
                              const int32_t* seq_lens, int32_t window,
                              size_t* bytes);

/*
 * Compress one layer's prompt KV cache (steps 1-4 above) with
 * SNAPKV_NUM_STAGES consecutive kernels on `stream`: vote statistics, vote
 * with pooling, selection, gather. When snapkv_score_kernels reports 1 or 3
 * for the shape, the first two run as one kernel whose work items exchange
 * the row statistics through the workspace and wait, bounded, for each
 * other; its results are bit-identical to the two kernels'.
 *
 *   window       W >= 1, the observation window (pages: 16-64)
 *   kernel_size  odd, 1 <= kernel_size <= SNAPKV_MAX_KERNEL; 1 = no pooling
 *                (pages: 5-13)
 *   pool_mode    SNAPKV_POOL_AVG or SNAPKV_POOL_MAX
 *   budget       B > W, entries kept per head including the W window rows
 *                (pages: 1024-4096, and 256)
 *   workspace    at least snapkv_workspace_size bytes of device memory
 *
 * Every output element is written: for prompt b and head h the first
 * n = min(L_b, B) entries hold the kept rows and their ascending indices,
 * the rest are zero rows with index -1. Gathered rows are bit copies of K/V.
 * Results do not depend on how the work is scheduled: repeated calls give
 * identical bits.
 *
 * Errors: SNAPKV_ERR_INVALID_ARGUMENT for a null pointer, a misaligned
 * device pointer, batch outside [1, SNAPKV_MAX_BATCH], heads < 1 or
 * num_q_heads % num_kv_heads != 0, window < 1, budget <= window, an even or
 * non-positive kernel_size, an unknown pool_mode, a seq_len < 1, or more than
 * 2^31-1 packed tokens; SNAPKV_ERR_UNSUPPORTED for head_dim not in {64, 128},
 * G * W > SNAPKV_MAX_ROWS or kernel_size > SNAPKV_MAX_KERNEL;
 * SNAPKV_ERR_WORKSPACE when workspace_bytes is below snapkv_workspace_size;
 * SNAPKV_ERR_HIP when a kernel launch fails.
 */
int32_t snapkv_compress(int32_t batch, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim,
                        const void* q_win, const void* k, const void* v,
                        const int32_t* seq_lens, int32_t window,
                        int32_t kernel_size, int32_t pool_mode, int32_t budget,
                        void* out_k, void* out_v, int32_t* out_idx,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * How snapkv_compress (and its _staged, _int4 and _fp8 forms) runs the vote
 * statistics and the vote on this shape, on the current device:
 *   1  one kernel, snapkv_score_fused, whose work items keep their keys in
 *      LDS between the two (head_dim 128, num_q_heads / num_kv_heads * window
 *      <= 256, at most 512 keys per work item, kernel_size <= 33);
 *   3  one kernel, snapkv_score_fused_stream, whose work items read their
 *      keys twice (other shapes);
 *   2  two kernels, snapkv_score_stats and snapkv_score_vote.
 * The one-kernel forms are taken when the call has at most one scoring work
 * item per compute unit of the device, so that every item can be resident
 * at once: their items exchange the row statistics through the workspace
 * and wait, bounded, for each other. All three give identical bits. While
 * the environment variable SNAPKV_NO_FUSED_SCORE is set to a non-empty value
 * other than "0" (read at every call), it is always 2.
 * Concurrency: the one-kernel forms count on having the device's compute
 * units to themselves while they run; the results never depend on it. Each
 * wait is bounded (about a second of polling; SNAPKV_SPIN_LIMIT, read at
 * every call, lowers the number of polls, e.g. to exercise this path): an
 * item that stops waiting computes the statistics it did not receive itself,
 * with the same arithmetic, and the selection recounts its first radix digit
 * when a histogram may have missed its clearing, so the outputs are the same
 * bits as with no wait given up; only the time grows. A process that runs
 * compressions on several streams of one device at once may set
 * SNAPKV_NO_FUSED_SCORE, or SNAPKV_COOPERATIVE (read at every call), which
 * launches them as cooperative kernels so that the runtime guarantees every
 * work item a compute unit (about 19 us more per call on MI355X), to avoid
 * those slow calls.
 * snapkv_compress_from_lse always runs the vote kernel alone. Writes
 * *kernels and returns SNAPKV_OK, or an error status under the shape rules
 * of snapkv_compress (SNAPKV_ERR_INVALID_ARGUMENT also for a NULL
 * `kernels`).
 */
int32_t snapkv_score_kernels(int32_t batch, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim,
                             const int32_t* seq_lens, int32_t window,
                             int32_t kernel_size, int32_t* kernels);

/*
 * Whether snapkv_compress (and its _staged, _from_lse, _int4 and _fp8
 * forms) runs the selection inside the gather on this shape, on the current
 * device: 1 when each gather work item runs its head's selection itself
 * (snapkv_gather_select: every prefix L - W is at most 32768 positions and
 * the gather's work items, of 32 or 64 rows, fit the device one per compute
 * unit), so the selection stage launches nothing; else 0 (snapkv_select,
 * then snapkv_gather). Results are identical either way. While the
 * environment variable SNAPKV_NO_FUSED_SELECT is set to a non-empty value
 * other than "0" (read at every call), it is always 0. Writes *fused
 * and returns SNAPKV_OK, or an error status under the shape rules of
 * snapkv_compress (SNAPKV_ERR_INVALID_ARGUMENT also for a NULL `fused` or
 * budget <= window).
 */
int32_t snapkv_gather_selects(int32_t batch, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim,
                              const int32_t* seq_lens, int32_t window,
                              int32_t budget, int32_t* fused);

/*
 * Which kernels snapkv_compress's selection stage (stage 2 of
 * snapkv_compress_staged) launches on this shape, on the current device
 * (the per-head selection of the pages' step 3: glossary page
 * "SnapKV(スナップケーブイ)", section "SnapKVの仕組み"):
 *   0  none: no prompt is compressed, or the selection runs inside the
 *      gather (snapkv_gather_selects = 1);
 *   1  snapkv_select, one workgroup per (prompt, KV head), every prefix
 *      L - W at most 32768 positions;
 *   2  snapkv_select_slices, the sliced selection of longer prefixes as one
 *      launch whose 4096-position slice workgroups exchange the digit
 *      histograms through flags (every slice workgroup of the call fits the
 *      device one per compute unit);
 *   3  the sliced selection as three kernels (snapkv_select_digit<2>,
 *      snapkv_select_digit<3>, snapkv_select_count), otherwise, or while
 *      SNAPKV_NO_FUSED_SELECT is set to a non-empty value other than "0".
 * Results are identical in every case. Writes *kernels and returns
 * SNAPKV_OK, or an error status under the shape rules of snapkv_compress
 * (SNAPKV_ERR_INVALID_ARGUMENT also for a NULL `kernels` or budget <= window).
 */
int32_t snapkv_select_kernels(int32_t batch, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim,
                              const int32_t* seq_lens, int32_t window,
                              int32_t budget, int32_t* kernels);

/*
 * snapkv_compress for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * no workspace argument; the intermediates go to a fixed scratch area of
 * SNAPKV_STATIC_SCRATCH_BYTES inside the library, one per device, held from
 * the first call on that device until the process ends. The call allocates
 * nothing (no hipMalloc, no allocating library routine); the caller still
 * passes the inputs and outputs, as for snapkv_compress. Results are
 * identical to snapkv_compress's. The area needs no clearing: every word a
 * call reads is written by that call first, or only counts when it carries
 * the call's own mark.
 * All calls on one device share its area: calls that overlap in time on one
 * device (two streams, two threads) race and give undefined results; the
 * caller serialises them.
 * Errors as for snapkv_compress; SNAPKV_ERR_WORKSPACE when the shape needs
 * more scratch than SNAPKV_STATIC_SCRATCH_BYTES (snapkv_workspace_size gives
 * the need; e.g. 5.3 MB for one 70B-shaped layer at 131072 tokens, 11 MB for
 * eight 8B-shaped prompts of up to 32768 tokens), checked before any HIP
 * call; SNAPKV_ERR_HIP when the area's address cannot be looked up.
 */
#define SNAPKV_STATIC_SCRATCH_BYTES (32u << 20)

int32_t snapkv_compress_static(int32_t batch, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim,
                               const void* q_win, const void* k, const void* v,
                               const int32_t* seq_lens, int32_t window,
                               int32_t kernel_size, int32_t pool_mode,
                               int32_t budget, void* out_k, void* out_v,
                               int32_t* out_idx, void* stream);

/*
 * snapkv_compress (window_lse NULL) or snapkv_compress_from_lse (window_lse
 * as there) that also hands out the pooled scores its selection read, for
 * checking the path's scores against a reference (the scores of step 2 above
 * as they come out of whichever scoring kernels snapkv_score_kernels names
 * for the shape):
 *
 *   out_scores  device float32 [batch, H_kv, scores_len], 16-byte aligned;
 *               entry j < P_b of prompt b with L_b > budget holds c_h[j],
 *               every other entry (prompts kept whole, positions past P_b)
 *               is written as 0.
 *   scores_len  >= max_b(L_b - W) and >= 1.
 *
 * The compressed cache is identical to snapkv_compress's (or
 * snapkv_compress_from_lse's); one more kernel copies the scores out of the
 * workspace after the gather. Errors as for those calls;
 * SNAPKV_ERR_INVALID_ARGUMENT also for a null or misaligned out_scores or a
 * scores_len that is too small.
 */
int32_t snapkv_compress_with_scores(int32_t batch, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim,
                                    const void* q_win, const void* k,
                                    const void* v, const int32_t* seq_lens,
                                    int32_t window, const float* window_lse,
                                    int32_t kernel_size, int32_t pool_mode,
                                    int32_t budget, void* out_k, void* out_v,
                                    int32_t* out_idx, float* out_scores,
                                    int32_t scores_len, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * snapkv_compress with optional per-stage timing: the same kernels (named by
 * snapkv_stage_name) and identical results. When stage_events is not NULL it
 * points to 2 * SNAPKV_NUM_STAGES caller-owned hipEvent_t: the dispatch of
 * stage s records stage_events[2*s] when its kernel starts and
 * stage_events[2*s+1] when it ends (a stage without work records both back
 * to back), so elapsed times are the kernels' own durations. With a fused
 * score kernel (snapkv_score_kernels = 1 or 3) stage 0 times that kernel
 * and stage 1 has no work; with the selection inside the gather
 * (snapkv_gather_selects = 1) stage 3 times snapkv_gather_select and stage 2
 * has no work; otherwise stage 2 spans the selection kernel(s) that
 * snapkv_select_kernels names.
 * Errors as for snapkv_compress.
 */
int32_t snapkv_compress_staged(int32_t batch, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim,
                               const void* q_win, const void* k,
                               const void* v, const int32_t* seq_lens,
                               int32_t window, int32_t kernel_size,
                               int32_t pool_mode, int32_t budget,
                               void* out_k, void* out_v, int32_t* out_idx,
                               void* workspace, size_t workspace_bytes,
                               void* stream, void* const* stage_events);

/*
 * snapkv_compress for a caller whose own prefill attention already produced
 * the softmax normaliser of every observation-window row (glossary page
 * "SnapKV(スナップケーブイ)", FAQ Q3: the scores are computed together with
 * the ordinary prefill, at almost no extra cost). The window-statistics pass
 * is skipped:
 *
 *   window_lse  device float32 [batch, H_q, W], row-major: for prompt b,
 *               query head q and window row i (position P + i), the natural
 *               log of sum_{j <= P + i} exp(q . k_j / sqrt(D)) over the
 *               prompt's keys (what flash-attention kernels report as the
 *               log-sum-exp of a row). 4-byte aligned. Read only. Only the
 *               rows of prompts that are compressed (L_b > B) are read and
 *               they must be finite; entries of other prompts are ignored.
 *
 * Results equal snapkv_compress's up to the normalisers' rounding (the
 * votes are computed from them; selections are identical wherever the
 * pooled scores are not within that rounding of a tie). Other arguments,
 * the workspace and errors as for snapkv_compress; SNAPKV_ERR_INVALID_ARGUMENT
 * also for a null or misaligned window_lse. It runs the kernels of
 * snapkv_compress with the first (the statistics pass) replaced by a small
 * one that clears the vote's histogram in the workspace, or, when every vote
 * work item can be resident at once (as for the one-kernel scoring forms of
 * snapkv_score_kernels, with the same concurrency rules and switches), by
 * nothing: the vote kernel's first item per head clears the histograms and
 * the others check its flag (bounded wait) before adding to them.
 */
int32_t snapkv_compress_from_lse(int32_t batch, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 const void* q_win, const void* k,
                                 const void* v, const int32_t* seq_lens,
                                 int32_t window, const float* window_lse,
                                 int32_t kernel_size, int32_t pool_mode,
                                 int32_t budget, void* out_k, void* out_v,
                                 int32_t* out_idx, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * snapkv_compress with the compressed cache stored at 4 bits per value
 * (Scissorhands page, section "4ビット量子化との併用" and its FAQ on
 * quantisation: token reduction and a 4-bit value width are separate levers
 * that combine). The selection is snapkv_compress's (identical out_idx);
 * each kept K or V row x of one head (D values) is stored as
 *
 *   scale = amax / 7,  code_d = rint(x_d * (7 / amax)) in [-7, 7]
 *
 * with amax = max_d |x_d|, in float32 with round-to-nearest-even (rint ties
 * to even); x_d ~= code_d * scale within scale / 2. A zero row has codes 0
 * and scale 0. K and V must be finite.
 *
 *   out_kq, out_vq  device uint8 [batch, H_kv, B, D/2]: codes as two's-
 *                   complement nibbles, element 2i in the low nibble of byte i
 *   out_ks, out_vs  device float32 [batch, H_kv, B]: the rows' scales
 *   window_lse      NULL (the statistics pass runs) or as for
 *                   snapkv_compress_from_lse
 *
 * Slots past min(L_b, B) hold codes 0, scale 0 and index -1. Other
 * arguments, the workspace and errors as for snapkv_compress (the scale
 * buffers must also be non-null and 16-byte aligned; a non-null window_lse
 * 4-byte aligned).
 */
int32_t snapkv_compress_int4(int32_t batch, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim,
                             const void* q_win, const void* k, const void* v,
                             const int32_t* seq_lens, int32_t window,
                             const float* window_lse, int32_t kernel_size,
                             int32_t pool_mode, int32_t budget,
                             uint8_t* out_kq, float* out_ks, uint8_t* out_vq,
                             float* out_vs, int32_t* out_idx, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * snapkv_compress with the kept rows stored at 8 bits per value in the OCP
 * FP8 E4M3 format (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, largest finite value 448), the format MI355X's matrix cores
 * read: per kept K or V row, scale = amax / 448 and code_d =
 * E4M3(x_d * (448 / amax)), the product in float32 and the conversion
 * rounding to nearest even (code * scale is within 2^-4 of x_d relative, or
 * 2^-10 * scale below 2^-6 * scale). A zero row has codes 0 and scale 0.
 *
 *   out_kq, out_vq  device uint8 [batch, H_kv, B, D]: E4M3 bytes
 *   out_ks, out_vs  device float32 [batch, H_kv, B]
 *
 * Everything else as for snapkv_compress_int4 (same selection, index list,
 * padding, optional window_lse and errors).
 */
int32_t snapkv_compress_fp8(int32_t batch, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim,
                            const void* q_win, const void* k, const void* v,
                            const int32_t* seq_lens, int32_t window,
                            const float* window_lse, int32_t kernel_size,
                            int32_t pool_mode, int32_t budget,
                            uint8_t* out_kq, float* out_ks, uint8_t* out_vq,
                            float* out_vs, int32_t* out_idx, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * The pooled scores c_h (steps 1-2) of every prompt with P = L - W >= 1,
 * whatever its length relative to a budget; raw scores when kernel_size = 1.
 *
 *   out_scores  device float32 [batch, H_kv, scores_len]; entry j < P_b of
 *               prompt b holds c_h[j], every other entry is written as 0.
 *   scores_len  >= max_b(L_b - W) and >= 1.
 *
 * The values are bit-identical to the ones snapkv_compress selects from on
 * the same inputs. Errors as for snapkv_compress; SNAPKV_ERR_INVALID_ARGUMENT
 * also for a scores_len that is too small.
 */
int32_t snapkv_window_scores(int32_t batch, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim,
                             const void* q_win, const void* k,
                             const int32_t* seq_lens, int32_t window,
                             int32_t kernel_size, int32_t pool_mode,
                             float* out_scores, int32_t scores_len,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * Decode-step attention over a KV cache, to run decoding on the compressed
 * cache (glossary page "SnapKV(スナップケーブイ)", section "SnapKVの仕組み",
 * step 4: the decode phase uses the compressed cache; paper page, results:
 * the generation speed-up at 16K input tokens) or, for comparison, on the
 * uncompressed one. For prompt b and query head q of KV head h = q / G:
 *
 *   out[b, q, :] = sum_t softmax_t(q[b, q, :] . k_t / sqrt(D)) v_t
 *
 * over the cache_lens[b] rows t of head h (no mask; the token being generated
 * is attended only if the caller has appended it to the cache).
 *
 *   q        device bf16 [batch, H_q, D]
 *   layout   SNAPKV_CACHE_COMPRESSED: k_cache, v_cache bf16
 *              [batch, H_kv, capacity, D] (snapkv_compress's out_k / out_v
 *              with capacity = B), rows 0 .. cache_lens[b]-1 read;
 *            SNAPKV_CACHE_PACKED: bf16 [T, H_kv, D] with the prompts back to
 *              back, T = sum(cache_lens) (the prefill cache); capacity unused
 *   cache_lens  HOST int32[batch], each >= 1 (and <= capacity when compressed)
 *   out      device float32 [batch, H_q, D]
 *   workspace   at least snapkv_decode_workspace_size bytes (per-chunk
 *            partial softmax and done marks; no initialisation, not shared
 *            by calls in flight)
 *
 * Rows are split into chunks (a multiple of 128 rows, about 1024 chunk items
 * per call). When no prompt has more than 16 chunks (a compressed cache) the
 * step is one kernel: each chunk item publishes its partial and a done mark
 * tagged with the call, and an item that finds all marks of its head merges
 * the head's chunks (no item waits for another); otherwise two kernels,
 * chunk partials then a merge (snapkv_decode_kernels reports which). Both forms
 * compute in float32 from the bf16 inputs with the same fixed summation
 * orders, so they give identical bits, and so do repeated calls. Conventions
 * and error behaviour as for snapkv_compress: SNAPKV_ERR_INVALID_ARGUMENT
 * for null or misaligned pointers, batch outside [1, SNAPKV_MAX_BATCH], bad
 * head counts, an unknown layout, a cache length < 1 or above capacity;
 * SNAPKV_ERR_UNSUPPORTED for head_dim not in {64, 128} or more than 8 query
 * heads per KV head; SNAPKV_ERR_WORKSPACE for a small workspace.
 */
#define SNAPKV_CACHE_COMPRESSED 0
#define SNAPKV_CACHE_PACKED 1

int32_t snapkv_decode_workspace_size(int32_t batch, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim,
                                     int32_t layout, int32_t capacity,
                                     const int32_t* cache_lens, size_t* bytes);

int32_t snapkv_decode_attention(int32_t batch, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim,
                                const void* q, const void* k_cache,
                                const void* v_cache, int32_t layout,
                                int32_t capacity, const int32_t* cache_lens,
                                float* out, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * snapkv_decode_attention with the step's device time: start_event and
 * stop_event (hipEvent_t created by the caller, or NULL) are recorded by the
 * dispatches themselves at the first kernel's start and the last kernel's
 * end, so hipEventElapsedTime between them is the step's GPU time, free of
 * host launch cost. Same arguments, results and errors otherwise.
 */
int32_t snapkv_decode_attention_timed(int32_t batch, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim,
                                      const void* q, const void* k_cache,
                                      const void* v_cache, int32_t layout,
                                      int32_t capacity, const int32_t* cache_lens,
                                      float* out, void* workspace,
                                      size_t workspace_bytes, void* stream,
                                      void* start_event, void* stop_event);

/*
 * How many kernels snapkv_decode_attention launches for this shape (1 or 2,
 * into *kernels), without launching anything. Errors as for
 * snapkv_decode_workspace_size.
 */
int32_t snapkv_decode_kernels(int32_t batch, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim,
                              int32_t layout, int32_t capacity,
                              const int32_t* cache_lens, int32_t* kernels);

/*
 * Prefill attention with the window normalisers as a by-product, for a
 * caller without a prefill kernel of its own (glossary page
 * "SnapKV(スナップケーブイ)", FAQ Q3: the window scores can come out of the
 * ordinary prefill attention at almost no extra cost). Causal attention of
 * every prompt row at scale 1/sqrt(D), computed with bf16 MFMAs and float32
 * softmax and accumulation: for prompt b, query head q of KV head h = q / G
 * and row i,
 *
 *   out[i] = sum_{j <= i} softmax_j(q_i . k_j / sqrt(D)) v_j
 *
 *   q        device bf16 [T, H_q, D], the prompts' queries packed back to back
 *   k, v     device bf16 [T, H_kv, D] (as for snapkv_compress)
 *   out      device bf16 [T, H_q, D] (each row rounded once to bf16)
 *   window_lse  device float32 [batch, H_q, W] or NULL: for the last W rows
 *            of each prompt (row L - W + i), the natural log of
 *            sum_{j <= row} exp(q . k_j / sqrt(D)), exactly the input of
 *            snapkv_compress_from_lse; NaN for rows before a prompt's start
 *            (L < W). 4-byte aligned.
 *   q_win    device bf16 [batch, H_q, W, D] or NULL: copies of those rows'
 *            queries, the q_win argument of the compression calls (zero
 *            rows before a prompt's start).
 *   window   W >= 1 when window_lse or q_win is given (ignored otherwise)
 *
 * One kernel on `stream`; repeated calls give identical bits. Conventions
 * and errors as for snapkv_compress: SNAPKV_ERR_INVALID_ARGUMENT for null or
 * misaligned pointers, a bad batch, head counts or seq_len, or window < 1
 * with a window output; SNAPKV_ERR_UNSUPPORTED for head_dim not in {64, 128}
 * or batch * num_q_heads > 65535; SNAPKV_ERR_HIP when the launch fails.
 */
int32_t snapkv_prefill_attention(int32_t batch, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 const void* q, const void* k, const void* v,
                                 const int32_t* seq_lens, int32_t window,
                                 void* out, float* window_lse, void* q_win,
                                 void* stream);

/* Static text of a status code ("ok", "invalid argument", ...). */
const char* snapkv_status_string(int32_t status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* snapkv_last_error(void);

/* Name of stage s of snapkv_compress_staged (its kernel's name), or NULL
 * when s is out of range. */
const char* snapkv_stage_name(int32_t stage);

#ifdef __cplusplus
}
#endif

#endif /* SNAPKV_H_ */
