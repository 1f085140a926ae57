/*
 * idx.h -- C ABI of the MI355X (gfx950) DeepSeek-V4.1 Indexer hot path.
 *
 * The operations follow the Indexer as stated on three web pages, cited by
 * page and section:
 *   [IDX]  "DeepSeek V4.1" -- class Indexer, forward (atlas.klimoza.dev,
 *          models/deepseek-v4.1 .../attention/indexer/index-keys)
 *   [CMP]  "Module compress" -- API docs of a CPU reference
 *          (docs.atlascybernetics.ai, spark_model/layers/deepseek_v41_ref/compress)
 *   [VLLM] "launcher/docker-images/dsv41-flash/patches/attention.py" -- vLLM
 *          DeepseekV4 attention patch (git.kilork.org)
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are device memory owned by the caller; the
 *     library never allocates device memory and keeps no state between calls
 *     other than the launch-timing hook (idx_timing_arm).  Calls may come
 *     from several host threads; the timing hook itself is single-threaded.
 *   - bf16 tensors are passed as their 16-bit patterns (uint16_t).
 *   - stream is a hipStream_t (NULL = the default stream); every launch is
 *     asynchronous on it and calls on one stream run in call order.
 *   - Arguments are validated on the host before anything is launched; on a
 *     validation failure nothing is launched and IDX_EINVAL /
 *     IDX_EUNSUPPORTED is returned.  IDX_EHIP reports a launch error.
 *     Values inside device arrays (compress_lens, candidate ids) are read on
 *     the device and clamped as documented; they cannot be validated on the
 *     host without a synchronisation.
 *   - Inputs must be finite; block maxima of at most 2^120 keep every
 *     dequantised value finite.  NaN or Inf inputs give unspecified results.
 *
 * fp4 key row (68 bytes, [VLLM, _indexer_k_cache_head_dim] fixes the size):
 *   bytes 0..63  the 128 e2m1 codes, two per byte, element 2i in the low
 *                nibble of byte i (bit 3 of a code = sign);
 *   bytes 64..67 the e8m0 exponents e_j + 127 of blocks j = 0..3 (32 values
 *                each).  Element i dequantises to code_value * 2^e_(i/32).
 * A key cache is [B][Tcap][68] bytes: sequence b's rows are contiguous and
 * start at byte b * k_batch_stride_rows * 68.
 */
#ifndef IDX_H
#define IDX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    IDX_OK = 0,
    IDX_EINVAL = 1,       /* bad pointer, size or shape */
    IDX_EUNSUPPORTED = 2, /* valid but not implemented (e.g. index_head_dim != 128) */
    IDX_EHIP = 3          /* a HIP launch failed */
} idx_status;

/* Human-readable name of a status code (static string). */
const char *idx_status_string(idx_status s);

/* Library version string (static). */
const char *idx_version(void);

/*
 * Launch timing of the score kernel (measurement support, not a page
 * operation).  idx_timing_arm(slot) makes the next score launch of this
 * process (idx_score, idx_score_topk or their paged forms, any stream) record the start and end
 * of that kernel's execution into HIP event pair `slot` (0 <= slot < 256),
 * through hipExtLaunchKernel, so no marker packet is added to the stream;
 * the pair is created on first use on the current device and kept until
 * the process ends.  idx_timing_read(slot, ms) waits for the pair's end
 * event and writes the kernel's duration in milliseconds.  Not thread-safe:
 * one thread arms and launches.  IDX_EINVAL for a slot out of range or never
 * armed, IDX_EHIP when an event call fails.
 */
idx_status idx_timing_arm(int slot);
idx_status idx_timing_read(int slot, float *ms);

/*
 * idx_fp4_quant -- block-32 e2m1 / e8m0 quantise-dequantise of 128-wide rows
 * ([IDX, forward: fp4_act_quant on q and k]; [CMP, fp4_quant_e8m0_inplace,
 * to_e2m1_rne]).  Per block of 32 values: amax raised to at least 6*2^-126,
 * scale 2^e with e the smallest integer such that 6*2^e >= amax, each value
 * rounded to the nearest e2m1 point of x/2^e with ties to the even code and
 * its sign kept.
 *   x          device, [n_rows][128] bf16, 16-byte aligned
 *   rows68     device, [n_rows][68] output key rows (layout above), 4-byte
 *              aligned
 *   roundtrip  device, [n_rows][128] bf16 output (dequantised values), 16-byte
 *              aligned, or NULL
 * n_rows >= 0 (0 launches nothing).  A misaligned pointer gives IDX_EINVAL.
 */
idx_status idx_fp4_quant(const uint16_t *x, int64_t n_rows, uint8_t *rows68, uint16_t *roundtrip,
                         void *stream);

/*
 * idx_q_rope_quant -- the query side of the step ([IDX, forward: q split
 * into heads, apply_rotary_emb(q[..., -rd:], freqs_cis[start_pos:end_pos]),
 * fp4_act_quant(q), weights = weights_proj(x) * softmax_scale *
 * n_heads^-0.5]; [VLLM, fused_indexer_q_rope_quant] does the three in one
 * step).  Row r = b*S + s sits at position start_pos + s.  Per head: RoPE
 * on the last rd dims as interleaved pairs (x0, x1) rotated by (c, s) =
 * cos_sin[pos][i]: (x0*c - x1*s, x0*s + x1*c), each product and sum
 * rounded in fp32, result bf16 (as idx_publish_keys); then the block-32
 * quantiser of idx_fp4_quant.  Weights: bf16(fp32(w_raw) * w_scale).
 *   q            device, [B*S][H][D] bf16 before RoPE, 16-byte aligned
 *   w_raw        device, [B*S][H] bf16 (weights_proj output)
 *   cos_sin      device, [P][rd/2][2] fp32, 8-byte aligned;
 *                start_pos + S - 1 < P
 *   q_rows       device, [B*S][H][68] quantised heads, 4-byte aligned
 *   q_roundtrip  device, [B*S][H][D] bf16 dequantised heads, 16-byte
 *                aligned, or NULL.  It is a valid q for idx_score: the
 *                quantiser maps it to the same values (the same scores);
 *                idx_score_q4 takes q_rows directly
 *   w_out        device, [B*S][H] bf16, the w of idx_score
 * Requires D == 128 and rd even with 0 <= rd <= D.
 */
idx_status idx_q_rope_quant(const uint16_t *q, const uint16_t *w_raw, float w_scale,
                            const float *cos_sin, int P, int B, int S, int H, int D, int rd,
                            int start_pos, uint8_t *q_rows, uint16_t *q_roundtrip,
                            uint16_t *w_out, void *stream);

/*
 * idx_score -- rectified, weighted head sum of fp4 q against the fp4 keys
 * ([IDX, forward: the einsum of q and index_k, relu, times weights, sum over
 * heads, compress_lens mask, level-two candidate mask]).
 *   scores[r][t] = sum_{h=0..H-1} relu(qhat[r][h] . khat[b][t]) * w[r][h]
 * with r = b*S + s, qhat the fp4 round trip of q (done in the kernel),
 * khat the dequantised key row t of sequence b.  The head sum is fp32 in
 * one fixed association: heads [0, H/2) and [H/2, H) are each summed
 * ascending, one fused multiply-add per head starting from +0, and the
 * score is the low sum plus the high sum (one rounded add).  Each per-head
 * dot product is exact (it then matches an exact reference bit for bit)
 * when, for that head and key, the four block exponent sums e_q,j + e_k,j
 * of the blocks with a non-zero partial product differ by at most 9: every
 * block partial is an integer below 4608 in units of 2^(e_q,j + e_k,j - 2),
 * so the sum then fits fp32's 24 bits.  Block maxima of every row within a
 * factor 2^4 of each other suffice; outside that the dots are rounded in an
 * order the matrix core fixes.
 *   q              device, [B*S][H][D] bf16, RoPE already applied, 16-byte
 *                  aligned
 *   w              device, [B*S][H] bf16, weights_proj output already
 *                  multiplied by D^-0.5 * H^-0.5
 *   k_cache        device, key rows, 4-byte aligned, sequence stride
 *                  k_batch_stride_rows >= T
 *   compress_lens  device, [B*S] int32: row r scores positions t < cl[r]
 *                  (values clamped to [0, T])
 *   cand_blocks    device, [B*S][n_cand] int32 block ids (level two), or
 *                  NULL.  When given, every t < T is first set to -inf and
 *                  only positions t < cl[r] inside the listed blocks of
 *                  cand_block_size positions are scored; ids < 0 or
 *                  >= ceil(T/cand_block_size) are skipped.  An id listed
 *                  twice is scored twice (same values) and counted twice in
 *                  key_hist, so with key_hist the ids must be distinct.
 *   scores         device, [B*S][ld] fp32, ld >= T.  Entries t >= cl[r] are
 *                  left unspecified without cand_blocks (callers mask by cl).
 *   key_hist       device, [B*S][2048] uint32, or NULL.  When given, the
 *                  call adds to it, per row, the count of the scores it
 *                  wrote by the top 11 bits of their order key (the key maps
 *                  -0 to +0, then flips negative floats and sets the sign of
 *                  positive ones).  It must hold zeros before the call:
 *                  idx_clear_key_hist clears it once, and every idx_topk
 *                  that consumes it leaves it zeroed again.  idx_topk takes
 *                  it to skip its first pass; positions it does not count
 *                  are -inf there.  The top-k calls check its total: a row
 *                  whose histogram does not count exactly its scored
 *                  positions (one filled twice, or by another call) is
 *                  ranked from its scores alone, more slowly.  A histogram
 *                  with the right total but taken on other scores is not
 *                  detected.
 * Requires D == 128 and H in {32, 64}.  T == 0 launches nothing.
 */
idx_status idx_score(const uint16_t *q, const uint16_t *w, const uint8_t *k_cache,
                     int64_t k_batch_stride_rows, int B, int S, int H, int D, int T,
                     const int32_t *compress_lens, const int32_t *cand_blocks, int n_cand,
                     int cand_block_size, float *scores, int64_t ld, uint32_t *key_hist,
                     void *stream);

/*
 * idx_score_topk -- idx_score followed by idx_topk in one launch, for rows of
 * at most 8192 positions (prefill rows, short contexts): one workgroup
 * scores a whole row into on-chip memory and ranks it there, so the scores
 * never travel through device memory unless asked for.  Without scores, a
 * row with compress_lens[r] <= index_topk is written in closed form and not
 * scored at all ([VLLM, _fill_short_context_topk_indices]: its result does
 * not depend on the scores).  Arguments and
 * results as idx_score (no candidates, no histogram) and idx_topk (no
 * workspace): out gets, per row, min(index_topk, T) positions in position
 * order, t + offset where t < compress_lens[r], else -1.
 *   scores  device, [B*S][ld] fp32, or NULL: when given, also receives the
 *           scores exactly as idx_score writes them
 * Requires D == 128, H in {32, 64} and T <= 8192 (IDX_EUNSUPPORTED
 * otherwise).
 */
idx_status idx_score_topk(const uint16_t *q, const uint16_t *w, const uint8_t *k_cache,
                          int64_t k_batch_stride_rows, int B, int S, int H, int D, int T,
                          const int32_t *compress_lens, int index_topk, int32_t offset,
                          int32_t *out, int64_t ld_out, float *scores, int64_t ld, void *stream);

/*
 * Paged key cache ([VLLM, DeepseekV4IndexerCache.get_kv_cache_spec]: pages of
 * 64 compressed positions, 64 * compress_ratio tokens, reached through a
 * per-sequence block table).  Row t of sequence b lives in slot t % 64 of
 * physical page block_table[b][t / 64]; slot s of page p is the 68-byte row
 * at k_pages + p * page_stride + 68 * s.
 *   k_pages      device, the page pool
 *   page_stride  bytes between pages, >= 64 * 68 and a multiple of 4 (the
 *                pool itself 4-byte aligned)
 *   n_pages      pages in the pool; an id outside [0, n_pages) is never
 *                dereferenced: its keys score as zero rows (idx_score_paged)
 *                or its row is not written (idx_publish_keys_paged)
 *   block_table  device, [B][bt_stride] int32 physical page ids, read for
 *                the pages that hold positions t < min(compress_lens[r], T)
 *                (score) or the published rows (publish)
 *   bt_stride    >= ceil(T / 64) (score) or ceil(Tcap / 64) (publish)
 * Everything else, and every result, is as for the contiguous call of the
 * same name; the results are bit-identical to it on the same rows.  In
 * candidate mode an invalid id likewise scores as zero rows.  When there is
 * work (score: B, S, T > 0; publish: B * G > 0), a null block_table,
 * n_pages <= 0, page_stride < 64 * 68 or a bt_stride below the bound gives
 * IDX_EINVAL before any launch.
 */

/* idx_score on a paged key cache.  With cand_blocks (level two) the row's
 * page ids are held on chip, which bounds T to 131072 (IDX_EUNSUPPORTED
 * beyond). */
idx_status idx_score_paged(const uint16_t *q, const uint16_t *w, const uint8_t *k_pages,
                           int64_t page_stride, int n_pages, const int32_t *block_table,
                           int64_t bt_stride, int B, int S, int H, int D, int T,
                           const int32_t *compress_lens, const int32_t *cand_blocks, int n_cand,
                           int cand_block_size, float *scores, int64_t ld, uint32_t *key_hist,
                           void *stream);

/* idx_score_topk on a paged key cache ([IDX, forward: score, then the final
 * topk]; pages as above).  T <= 8192 as for idx_score_topk
 * (IDX_EUNSUPPORTED otherwise); without scores, rows with compress_lens <=
 * index_topk are written in closed form and read no page. */
idx_status idx_score_topk_paged(const uint16_t *q, const uint16_t *w, const uint8_t *k_pages,
                                int64_t page_stride, int n_pages, const int32_t *block_table,
                                int64_t bt_stride, int B, int S, int H, int D, int T,
                                const int32_t *compress_lens, int index_topk, int32_t offset,
                                int32_t *out, int64_t ld_out, float *scores, int64_t ld,
                                void *stream);

/*
 * idx_score_q4, idx_score_topk_q4 -- idx_score and idx_score_topk with the
 * query heads given already quantised ([VLLM, fused_indexer_q_rope_quant]
 * hands its fp4 output to the indexer op): q_rows [B*S][H][68], the rows of
 * idx_fp4_quant / idx_q_rope_quant, 4-byte aligned, in place of q.  Every
 * other argument and every result as for the call without _q4; the scores
 * equal those of idx_score given the rows' bf16 round trip.
 */
idx_status idx_score_q4(const uint8_t *q_rows, const uint16_t *w, const uint8_t *k_cache,
                        int64_t k_batch_stride_rows, int B, int S, int H, int D, int T,
                        const int32_t *compress_lens, const int32_t *cand_blocks, int n_cand,
                        int cand_block_size, float *scores, int64_t ld, uint32_t *key_hist,
                        void *stream);
idx_status idx_score_topk_q4(const uint8_t *q_rows, const uint16_t *w, const uint8_t *k_cache,
                             int64_t k_batch_stride_rows, int B, int S, int H, int D, int T,
                             const int32_t *compress_lens, int index_topk, int32_t offset,
                             int32_t *out, int64_t ld_out, float *scores, int64_t ld,
                             void *stream);

/*
 * idx_score_qrope, idx_score_topk_qrope -- the query step inside the score
 * launch ([IDX, forward]: RoPE on the query heads' last rd dims at position
 * start_pos + s, fp4_act_quant of the heads, weights_proj output times
 * softmax_scale * n_heads^-0.5; [VLLM, fused_indexer_q_rope_quant]):
 * idx_q_rope_quant followed by idx_score_q4 / idx_score_topk_q4 on its
 * rows and weights, in one launch and with the same results bit for bit.
 * q holds the heads before RoPE, w_raw the raw weights, w_scale the
 * weights' factor, cos_sin, P, rd and start_pos as for idx_q_rope_quant
 * (rd even, 0 <= rd <= 128; when rd > 0, cos_sin 8-byte aligned with every
 * position start_pos + s, s < S, below P).  Every other argument and result
 * as for idx_score (no candidate blocks) and idx_score_topk.  An invalid
 * query-step argument gives IDX_EINVAL before any launch.
 */
idx_status idx_score_qrope(const uint16_t *q, const uint16_t *w_raw, float w_scale,
                           const float *cos_sin, int P, int rd, int start_pos,
                           const uint8_t *k_cache, int64_t k_batch_stride_rows, int B, int S,
                           int H, int D, int T, const int32_t *compress_lens, float *scores,
                           int64_t ld, uint32_t *key_hist, void *stream);
idx_status idx_score_topk_qrope(const uint16_t *q, const uint16_t *w_raw, float w_scale,
                                const float *cos_sin, int P, int rd, int start_pos,
                                const uint8_t *k_cache, int64_t k_batch_stride_rows, int B, int S,
                                int H, int D, int T, const int32_t *compress_lens, int index_topk,
                                int32_t offset, int32_t *out, int64_t ld_out, float *scores,
                                int64_t ld, void *stream);

/*
 * FP8 key cache ([VLLM, _indexer_k_cache_head_dim]: the FP8 indexer cache
 * row is 128 fp8 bytes plus one fp32 scale per 128 values, 132 bytes;
 * [VLLM, DeepseekV4Indexer.__init__]: quant_block_size 128, scale_fmt
 * "ue8m0").  Row layout:
 *   bytes 0..127    OCP e4m3 codes of elements 0..127 (bit 7 = sign)
 *   bytes 128..131  the scale 2^e as a little-endian fp32
 * e is the smallest integer with 448 * 2^e >= amax (amax of the 128 values,
 * at least 448 * 2^-126), each value is the nearest e4m3 point of x / 2^e
 * with ties to the even code, sign kept (the e2m1 rule of idx_fp4_quant
 * with e4m3's maximum 448 and a block of 128).  The query heads go through
 * the same quantiser.
 */

/* idx_fp8_quant -- 128-wide bf16 rows (16-byte aligned) -> 132-byte rows
 * (4-byte aligned), and optionally their bf16 round trip (16-byte aligned,
 * or NULL).  n_rows >= 0; misaligned pointers give IDX_EINVAL. */
idx_status idx_fp8_quant(const uint16_t *x, int64_t n_rows, uint8_t *rows132, uint16_t *roundtrip,
                         void *stream);

/*
 * idx_score_fp8 -- idx_score on the FP8 cache: k_cache holds 132-byte rows
 * (sequence stride k_batch_stride_rows rows), q is quantised per head by the
 * FP8 quantiser in the kernel, the dots run on the matrix core's e4m3 form.
 * Every other argument and result as idx_score.  Unlike the fp4 rows, a
 * 128-term e4m3 dot is not exact in fp32: each dot is rounded in the order
 * the matrix core fixes, so the scores agree with an exactly rounded
 * reference to within a few fp32 roundings per head, not bit for bit.
 * Requires D == 128 and H in {32, 64}.
 */
idx_status idx_score_fp8(const uint16_t *q, const uint16_t *w, const uint8_t *k_cache,
                         int64_t k_batch_stride_rows, int B, int S, int H, int D, int T,
                         const int32_t *compress_lens, const int32_t *cand_blocks, int n_cand,
                         int cand_block_size, float *scores, int64_t ld, uint32_t *key_hist,
                         void *stream);

/* idx_publish_keys_fp8 -- idx_publish_keys into an FP8 cache (132-byte rows,
 * 4-byte aligned): the same key (wk, k_norm, RoPE), quantised by the FP8
 * quantiser.  Arguments and errors as idx_publish_keys. */
idx_status idx_publish_keys_fp8(const uint16_t *latent, const uint16_t *wk, const float *gamma,
                                const float *cos_sin, int P, int B, int G, int Din, int D, int rd,
                                float eps, int start_pos, int ratio, uint8_t *k_cache,
                                int64_t k_batch_stride_rows, int Tcap, void *stream);

/*
 * idx_clear_key_hist -- zero a [R][2048] uint32 score histogram (device) on
 * the stream, before the first idx_score accumulates into it (idx_topk
 * resets it after each use).
 */
idx_status idx_clear_key_hist(uint32_t *key_hist, int R, void *stream);

/*
 * Bytes of device workspace idx_topk needs for R rows of width T.
 */
size_t idx_topk_workspace_size(int R, int T, int index_topk);

/*
 * idx_topk -- per-row top-k in position order ([IDX, forward: topk of
 * min(index_topk, end_pos//ratio), sort by position, -1 where not below
 * compress_lens, plus offset]).  Row r ranks positions t in [0, T) by
 * (masked score descending, t ascending), where positions t >= cl[r] count
 * as -inf and -0 equals +0; it keeps the first k_out = min(index_topk, T),
 * and writes them by ascending t as t + offset when t < cl[r], else -1.
 * When index_topk >= T the result is the closed form of
 * [VLLM, _fill_short_context_topk_indices] plus the offset.
 *   scores         device, [R][ld] fp32
 *   compress_lens  device, [R] int32 (clamped to [0, T])
 *   key_hist       device, [R][2048] from idx_score on these scores and
 *                  compress_lens, or NULL (then the first digit is counted
 *                  here).  The call reads it and resets it to zero (in
 *                  stream order), ready for the next idx_score.  A row whose
 *                  histogram total is not its count of positions below
 *                  compress_lens (clamped to [0, T]) is ranked without it;
 *                  rows wider than 262144 never use it.
 *   out            device, [R][ld_out] int32, ld_out >= k_out; only the first
 *                  k_out entries of each row are written
 *   k_out          host, or NULL: receives the row width min(index_topk, T)
 *                  once the arguments pass their checks
 *   ws, ws_bytes   device workspace of at least idx_topk_workspace_size bytes
 *                  (may be NULL when that size is 0)
 * NaN scores give unspecified results.
 */
idx_status idx_topk(const float *scores, int64_t ld, int R, int T, const int32_t *compress_lens,
                    uint32_t *key_hist, int index_topk, int32_t offset, int32_t *out,
                    int64_t ld_out, int32_t *k_out, void *ws, size_t ws_bytes, void *stream);

/*
 * idx_topk_noalloc -- idx_topk for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Arguments, results and errors as idx_topk, without the
 * workspace: it comes from a static device array of the library, of
 * idx_topk_noalloc_max_workspace() bytes (16 MiB), one per GPU the library
 * runs on, held until the process ends.  A call whose idx_topk workspace
 * would exceed it returns IDX_EUNSUPPORTED before any launch (e.g. more
 * than 7 rows of 262144 positions).  The call allocates nothing.  Every
 * call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (other streams, other host threads) race and give undefined results;
 * calls in one stream's order are safe.  The kernels initialise whatever
 * part of the array they read, so a call does not depend on the previous
 * contents.
 */
idx_status idx_topk_noalloc(const float *scores, int64_t ld, int R, int T,
                            const int32_t *compress_lens, uint32_t *key_hist, int index_topk,
                            int32_t offset, int32_t *out, int64_t ld_out, int32_t *k_out,
                            void *stream);
size_t idx_topk_noalloc_max_workspace(void);

/*
 * idx_topk_candidates -- idx_topk for a level-two row, whose finite scores
 * all lie in its candidate blocks (as idx_score with the same cand_blocks
 * writes them; [IDX, forward: the level-two mask, then the final topk]).
 * The result equals idx_topk's on the full row: when at least k_out
 * candidate positions lie below compress_lens the row is ranked among them
 * only; otherwise every finite position is kept plus the lowest other
 * positions, as the full ranking does.
 *   cand_blocks  device, [R][n_cand] int32 block ids in strictly
 *                ascending order apart from skipped ids
 *                (idx_select_candidate_blocks' output); ids < 0 or
 *                >= ceil(T/cand_block_size) are skipped
 *   key_hist     device, [R][2048] from idx_score with these cand_blocks on
 *                these scores and compress_lens, or NULL (then the first
 *                digit is counted here).  Read and reset to zero, as by
 *                idx_topk.
 *   scores, compress_lens, index_topk, offset, out, ld_out, k_out: as
 *                idx_topk
 * Requires T <= 65536, n_cand <= 2048 and n_cand * cand_block_size <= 8192
 * (IDX_EUNSUPPORTED otherwise).
 */
idx_status idx_topk_candidates(const float *scores, int64_t ld, int R, int T,
                               const int32_t *compress_lens, const int32_t *cand_blocks,
                               int n_cand, int cand_block_size, uint32_t *key_hist,
                               int index_topk, int32_t offset, int32_t *out, int64_t ld_out,
                               int32_t *k_out, void *stream);

/*
 * The top-k of rows split along their positions (T-split): one owner per
 * slice of consecutive positions (a GPU of a context-parallel group, say)
 * ranks its slice, the slices' (position, score) lists are gathered, and
 * idx_merge_topk ranks their union.  The result is idx_topk's on the whole
 * rows ([IDX, forward: topk of min(index_topk, end_pos//ratio), sort by
 * position, -1 where not below compress_lens, plus offset]): a position in a
 * row's top k is beaten by fewer than k positions of the row, so it is in its
 * slice's top k, and the union of the slices' lists is ranked by the same
 * (score descending, position ascending) order.
 *
 * Bytes of device workspace idx_topk_pairs needs.
 */
size_t idx_topk_pairs_workspace_size(int R, int T_slice, int index_topk);

/*
 * idx_topk_pairs -- the top-k of one slice of each row, as pairs.  The slice
 * holds row positions [slice_start, slice_start + T_slice); its scores are
 * scores[r][0 .. T_slice) (a pointer to the slice's first column).
 *   scores          device, [R][ld] fp32, ld >= T_slice
 *   compress_lens   device, [R] int32: the rows' own lengths (positions
 *                   t >= compress_lens[r] of the row count as -inf); the
 *                   slice's are clamp(cl - slice_start, 0, T_slice)
 *   key_hist        device, [R][2048] from idx_score of this slice with the
 *                   slice's compress_lens, or NULL; read and reset as by
 *                   idx_topk
 *   pos_out         device, [R][ld_out] int32, ld_out >= k_out =
 *                   min(index_topk, T_slice): the slice's top k_out row
 *                   positions in ascending order, -1 where not below
 *                   compress_lens (idx_topk of the slice with offset
 *                   slice_start)
 *   score_out       device, [R][ld_out] fp32: the score of each listed
 *                   position, -inf for -1
 *   k_out           host, or NULL: receives k_out
 *   ws, ws_bytes    device workspace, at least idx_topk_pairs_workspace_size
 * Requires slice_start >= 0 and slice_start + T_slice < 2^31 (IDX_EINVAL
 * otherwise).  NaN scores give unspecified results.
 */
idx_status idx_topk_pairs(const float *scores, int64_t ld, int R, int T_slice, int slice_start,
                          const int32_t *compress_lens, uint32_t *key_hist, int index_topk,
                          int32_t *pos_out, float *score_out, int64_t ld_out, int32_t *k_out,
                          void *ws, size_t ws_bytes, void *stream);

/*
 * idx_merge_topk -- the rows' top-k from their slices' pairs.  List g of row
 * r holds n pairs at pos[g*list_stride + r*ld + j], score[...same], j < n:
 * idx_topk_pairs of slice g, the slices in ascending position order and
 * none overlapping (a shorter list padded with position -1).  Entries with
 * position -1 are skipped.  Row r: with c = clamp(compress_lens[r], 0, T)
 * <= k_out = min(index_topk, T), the closed form (t + offset for t < c,
 * then -1); otherwise the k_out listed pairs first by (score descending, -0
 * equal to +0; position ascending), written by ascending position as
 * position + offset (-1 for a position >= c).  Lists that are the slices'
 * top-k lists hold at least k_out valid pairs whenever c > k_out; with fewer,
 * every valid pair is written and the rest of the row is -1.
 *   pos, score      device, int32 / fp32 as above (may be NULL when n == 0)
 *   G               lists per row, >= 1; G * n <= 32768 (IDX_EUNSUPPORTED)
 *   list_stride     >= (R - 1) * ld + n when G > 1, ld >= n
 *   compress_lens   device, [R] int32
 *   T               the rows' width
 *   out             device, [R][ld_out] int32, ld_out >= k_out
 *   k_out           host, or NULL: receives k_out
 * NaN scores give unspecified results.
 */
idx_status idx_merge_topk(const int32_t *pos, const float *score, int G, int n,
                          int64_t list_stride, int64_t ld, int R, const int32_t *compress_lens,
                          int T, int index_topk, int32_t offset, int32_t *out, int64_t ld_out,
                          int32_t *k_out, void *stream);

/*
 * Bytes of device workspace idx_select_candidate_blocks needs.
 */
size_t idx_select_workspace_size(int R, int T, int candidate_topk_blocks, int cand_block_size);

/*
 * idx_select_candidate_blocks -- level one of the two-level selection
 * ([IDX, forward: select_candidate_blocks]; [CMP, select_candidate_blocks],
 * whose body the pages do not give).  Reading implemented here: block j
 * covers positions [j*cbs, (j+1)*cbs) clipped to T, its score is the maximum
 * of its scores at positions t < cl[r] (-inf when it has none); the blocks
 * are ranked like idx_topk with k = candidate_topk_blocks, compress_lens
 * ceil(cl[r]/cbs) and offset 0.
 *   scores     device, [R][ld] fp32 (level-one scores)
 *   block_ids  device, [R][ld_ids] int32, ld_ids >= min(ctb, ceil(T/cbs));
 *              ascending block ids, -1 for a kept block without reachable
 *              positions.  The keep mask of the pages is the union of the
 *              listed blocks.
 */
idx_status idx_select_candidate_blocks(const float *scores, int64_t ld, int R, int T,
                                       const int32_t *compress_lens, int candidate_topk_blocks,
                                       int cand_block_size, int32_t *block_ids, int64_t ld_ids,
                                       void *ws, size_t ws_bytes, void *stream);

/*
 * idx_publish_keys -- index-key publish of a key-owning layer ([IDX,
 * forward: k = k_norm(wk(latent)), RoPE on the last rope_head_dim dims,
 * fp4_act_quant, write into k_cache]; [VLLM, DeepseekV4Indexer._produce_k]).
 * For sequence b and group g:
 *   y  = wk . latent[b][g]     fp32, one fma per input feature in order,
 *                              rounded to bf16 (the bf16 Linear output)
 *   z  = bf16((y * inv) * gamma), inv = 1/sqrt(sum_o y_o^2 / D + eps)
 *        (sum in order with fma; sqrt and division correctly rounded)
 *   RoPE on dims [D-rd, D) as interleaved pairs (x0, x1) with (c, s) =
 *        cos_sin[pos][i]: (x0*c - x1*s, x0*s + x1*c), products and sums
 *        rounded in fp32, result bf16
 *   quantise as idx_fp4_quant and write the 68-byte row.
 * Slots: start_pos == 0 (prefill) puts group g at position g*ratio, row g;
 * start_pos > 0 (decode, G must be 1) puts the completed group at position
 * start_pos + 1 - ratio, row start_pos / ratio.
 *   latent     device, [B][G][Din] bf16
 *   wk         device, [D][Din] bf16
 *   gamma      device, [D] fp32 (k_norm weight)
 *   cos_sin    device, [P][rd/2][2] fp32; every position used must be < P
 *   k_cache    device, 4-byte aligned; written rows must be < Tcap
 * Requires D == 128, rd even with 0 <= rd <= D, Din >= 1, ratio >= 1.
 */
idx_status idx_publish_keys(const uint16_t *latent, const uint16_t *wk, const float *gamma,
                            const float *cos_sin, int P, int B, int G, int Din, int D, int rd,
                            float eps, int start_pos, int ratio, uint8_t *k_cache,
                            int64_t k_batch_stride_rows, int Tcap, void *stream);

/* idx_publish_keys into a paged key cache ([IDX, forward: the key-owning
 * layer's store at start_pos // ratio]; pages as above): row t < Tcap goes
 * to slot t % 64 of page block_table[b][t / 64]; a page id outside
 * [0, n_pages) is not written.  Arguments and errors otherwise as
 * idx_publish_keys. */
idx_status idx_publish_keys_paged(const uint16_t *latent, const uint16_t *wk, const float *gamma,
                                  const float *cos_sin, int P, int B, int G, int Din, int D,
                                  int rd, float eps, int start_pos, int ratio, uint8_t *k_pages,
                                  int64_t page_stride, int n_pages, const int32_t *block_table,
                                  int64_t bt_stride, int Tcap, void *stream);

/*
 * idx_score_topk_candidates -- the level-two pass of the two-level indexer
 * ([IDX, forward]: scores of this layer's own weights, the non-candidate
 * positions masked with -inf, then the top-k): idx_score in candidate mode,
 * then idx_topk_candidates, with the scores kept per candidate slot instead
 * of per position.  Slot v (0 <= v < n_cand * cand_block_size) is position
 * cand_blocks[r][v / cbs] * cbs + v % cbs; slot_scores[r][v] receives its
 * score (ld >= n_cand * cand_block_size; slots without a reachable position
 * hold unspecified values), so no -inf fill of the row is needed.
 * cand_blocks as idx_topk_candidates takes them (strictly ascending apart
 * from skipped ids).  The other arguments, the indices, k_out and the
 * histogram's handling are those of the two calls, and the indices equal
 * theirs bit for bit.  The
 * top-k's checks run before the score launches (IDX_EUNSUPPORTED where
 * idx_topk_candidates would return it).
 */
idx_status idx_score_topk_candidates(const uint16_t *q, const uint16_t *w, const uint8_t *k_cache,
                                     int64_t k_batch_stride_rows, int B, int S, int H, int D,
                                     int T, const int32_t *compress_lens,
                                     const int32_t *cand_blocks, int n_cand, int cand_block_size,
                                     float *slot_scores, int64_t ld, uint32_t *key_hist,
                                     int index_topk, int32_t offset, int32_t *out, int64_t ld_out,
                                     int32_t *k_out, void *stream);

/*
 * idx_two_level_topk -- what follows the level-one select in a two-level
 * step ([IDX, forward]: the top-k of the candidate source layer's scores,
 * and the other layer's scores of the candidate blocks with their own
 * top-k): idx_topk of the level-one scores into out1, then
 * idx_score_topk_candidates into out2, with the same results bit for bit.
 * The two rankings do not depend on each other, so when level one takes the
 * split path (32768 < T <= 131072, key_hist given) and level two the
 * 1024-thread candidate ranking (n_cand * cand_block_size > 2048,
 * index_topk < T, key_hist2 given), they run side by side in one launch,
 * after level one's first split kernel and the candidate score; otherwise
 * the two calls run in order.
 *   scores, ld, key_hist, out1, ld_out1, ws, ws_bytes: idx_topk's arguments
 *           for level one (key_hist is reset for the next score call; ws as
 *           idx_topk_workspace_size gives)
 *   q .. ld_out2: idx_score_topk_candidates' arguments for level two (w2 its
 *           head weights, out2 its indices, key_hist2 its histogram)
 * The two histograms must be distinct buffers when both are given
 * (IDX_EINVAL otherwise): the rankings read and reset them side by side.
 * index_topk and offset serve both levels.  Every check of both calls runs
 * before anything launches.
 */
idx_status idx_two_level_topk(const float *scores, int64_t ld, uint32_t *key_hist, int32_t *out1,
                              int64_t ld_out1, void *ws, size_t ws_bytes, const uint16_t *q,
                              const uint16_t *w2, const uint8_t *k_cache,
                              int64_t k_batch_stride_rows, int B, int S, int H, int D, int T,
                              const int32_t *compress_lens, const int32_t *cand_blocks,
                              int n_cand, int cand_block_size, float *slot_scores, int64_t ld2,
                              uint32_t *key_hist2, int index_topk, int32_t offset, int32_t *out2,
                              int64_t ld_out2, void *stream);

/*
 * idx_score_select_blocks -- idx_score then idx_select_candidate_blocks on
 * the scores just written: the level-one pass of the two-level indexer
 * ([IDX, forward]: the candidate source layer scores every key, then
 * select_candidate_blocks keeps its best blocks for the next layer).
 * Arguments, outputs and errors are those of the two calls (ws sized by
 * idx_select_workspace_size); the outputs equal theirs bit for bit.  When
 * cand_block_size divides the score launch's chunk and the row has at most
 * 1024 blocks, the score launch also writes the block maxima (from the
 * chunk's scores in LDS) and one wave per row ranks them, so no pass reads
 * the scores back (cand_block_size a power of two in [16, 1024]; other
 * sizes run the two calls).
 */
idx_status idx_score_select_blocks(const uint16_t *q, const uint16_t *w, const uint8_t *k_cache,
                                   int64_t k_batch_stride_rows, int B, int S, int H, int D, int T,
                                   const int32_t *compress_lens, float *scores, int64_t ld,
                                   uint32_t *key_hist, int candidate_topk_blocks,
                                   int cand_block_size, int32_t *block_ids, int64_t ld_ids,
                                   void *ws, size_t ws_bytes, void *stream);

/*
 * idx_publish_score -- idx_publish_keys then idx_score for a decode step
 * that publishes its completed group ([IDX, forward]: the key-owning layer
 * stores k = k_norm(wk(latent)) with RoPE and the fp4 round trip at
 * start_pos // ratio before the score reads the cache; [VLLM]: "K write
 * must land before indexer_op reads the cache").  One query row and one
 * group per sequence (S = G = 1).  When the new key is the last scored
 * position (start_pos // ratio == T - 1, the usual decode step), both run
 * in one launch: one extra workgroup per sequence publishes the row and
 * scores that key itself, and the other workgroups score positions
 * [0, T - 1), so the publish overlaps the score.  Otherwise the two calls
 * run one after the other on the stream.  Arguments, results and errors as
 * the two calls (latent [B][1][Din], k_cache rows of 68 bytes with stride
 * k_batch_stride_rows, which also bounds the published row); the cache row,
 * the scores and key_hist equal those of the two calls bit for bit for the
 * documented inputs.  Din <= 2048 for the single launch.
 */
idx_status idx_publish_score(const uint16_t *latent, const uint16_t *wk, const float *gamma,
                             const float *cos_sin, int P, int Din, int rd, float eps,
                             int start_pos, int ratio, const uint16_t *q, const uint16_t *w,
                             uint8_t *k_cache, int64_t k_batch_stride_rows, int B, int H, int D,
                             int T, const int32_t *compress_lens, float *scores, int64_t ld,
                             uint32_t *key_hist, void *stream);

/*
 * idx_publish_score_fp8 -- idx_publish_score on an FP8 key cache: the
 * steps idx_publish_keys_fp8 then idx_score_fp8 ([IDX, forward]: the
 * key-owning layer's store before the score reads the cache; the FP8 row of
 * [VLLM, _indexer_k_cache_head_dim], 128 e4m3 bytes and an fp32 ue8m0
 * scale).  The same single launch when the new key is the last scored
 * position, the two calls on the stream otherwise.  k_cache rows are 132
 * bytes with stride k_batch_stride_rows.  Arguments, results and errors as
 * the two calls; the cache row, the scores and key_hist equal theirs bit for
 * bit for the documented inputs.  Din <= 2048 for the single launch.
 */
idx_status idx_publish_score_fp8(const uint16_t *latent, const uint16_t *wk, const float *gamma,
                                 const float *cos_sin, int P, int Din, int rd, float eps,
                                 int start_pos, int ratio, const uint16_t *q, const uint16_t *w,
                                 uint8_t *k_cache, int64_t k_batch_stride_rows, int B, int H,
                                 int D, int T, const int32_t *compress_lens, float *scores,
                                 int64_t ld, uint32_t *key_hist, void *stream);

/*
 * idx_publish_score_paged -- idx_publish_score on a paged key cache
 * ([IDX, forward]: the key-owning layer's store before the score reads the
 * cache; pages as idx_score_paged: row t of sequence b in slot t % 64 of
 * page block_table[b][t / 64]).  The same single launch when the new key
 * is the last scored position; otherwise idx_publish_keys_paged then
 * idx_score_paged on the stream.  The published row's page id outside
 * [0, n_pages) is not written, and that key is scored as the zero row the
 * paged score reads there.  The block table must cover rows [0, max(T,
 * start_pos / ratio + 1)).  Arguments, results and errors as those two
 * calls; the page, the scores and key_hist equal theirs bit for bit for the
 * documented inputs.  Din <= 2048 for the single launch.
 */
idx_status idx_publish_score_paged(const uint16_t *latent, const uint16_t *wk,
                                   const float *gamma, const float *cos_sin, int P, int Din,
                                   int rd, float eps, int start_pos, int ratio,
                                   const uint16_t *q, const uint16_t *w, uint8_t *k_pages,
                                   int64_t page_stride, int n_pages, const int32_t *block_table,
                                   int64_t bt_stride, int B, int H, int D, int T,
                                   const int32_t *compress_lens, float *scores, int64_t ld,
                                   uint32_t *key_hist, void *stream);

/*
 * idx_yarn_cos_sin -- host-side RoPE table for idx_publish_keys and
 * idx_q_rope_quant ([CMP, yarn_freqs_cis]: precompute_freqs_cis with YaRN;
 * the YaRN method of Peng et al.).  Pair i of the rd rotated dims has the
 * plain frequency theta^(-2i/rd).  With orig_len > 0 and factor != 1 it is
 * blended towards plain/factor by a linear ramp in i, 0 up to lo and 1 from
 * hi, where lo = floor(d(beta_fast)), hi = ceil(d(beta_slow)) kept inside
 * [0, rd - 1] (hi == lo widens the ramp to 0.001), and d(b) is the real
 * dimension at which a pair turns b times over orig_len positions.  Angles,
 * cosines and sines in double, stored fp32.
 *   out  host, [P][rd/2][2] fp32 (cos, sin)
 * IDX_EINVAL for P < 0, rd odd or <= 0, theta <= 1, factor <= 0, orig_len < 0,
 * a non-positive beta when the ramp is used, or a null out with P > 0;
 * IDX_EUNSUPPORTED for rd > 2048.
 */
idx_status idx_yarn_cos_sin(int P, int rd, double theta, double factor, int orig_len,
                            double beta_fast, double beta_slow, float *out);

#ifdef __cplusplus
}
#endif

#endif /* IDX_H */
