/*
 * oracle.c -- plain, slow CPU oracle for the DeepSeek-V4.1 Indexer hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or helper with the
 * HIP library; the two meet only through the seeded inputs.
 *
 * Sources (web pages; cited by page and section, never by line):
 *   [IDX]  "DeepSeek V4.1" -- class Indexer (__init__, forward) and
 *          SharedAttentionRuntime (atlas.klimoza.dev, models/deepseek-v4.1,
 *          .../attention/indexer/index-keys).
 *   [CMP]  "Module compress" -- API docs of the Rust CPU reference module
 *          (docs.atlascybernetics.ai, spark_model/layers/deepseek_v41_ref/compress).
 *   [VLLM] "launcher/docker-images/dsv41-flash/patches/attention.py" -- a vLLM
 *          DeepseekV4 attention patch (git.kilork.org, sm121 launcher).
 *
 * Every function computes the plain definition of its step: exact integer
 * arithmetic where the method is exact, one fixed fp32 operation order where
 * the contract fixes one.  No blocking, fusion or reordering.
 *
 * Provenance of the one order that is not the pages': the pages sum the
 * rectified, weighted head scores in bf16 torch ops and fix no association.
 * The fp32 head sum here (heads [0, ceil(H/2)) and [ceil(H/2), H) each
 * summed ascending, then one add) is a contract shared with the GPU
 * library; its split into two chains was chosen to match how the matrix
 * core leaves a key's heads in the two halves of a wavefront.  A hand-worked
 * golden (tests/golden/head_order.txt) tells this association apart from a
 * single chain, a pairwise tree and the other plausible splits.
 *
 * The RoPE table is not here: oracle/__init__.py builds it in float64 numpy
 * (yarn_cos_sin), and every function below takes it as an input.
 *
 * Parity status of each function is recorded in the file header of
 * oracle/__init__.py and in the design notes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ROW_BYTES 68 /* 64 bytes of e2m1 codes + 4 e8m0 bytes: [VLLM, _indexer_k_cache_head_dim] */
#define HEAD_DIM 128 /* index_head_dim */
#define BLOCK 32     /* fp4 block size: one e8m0 byte per 32 values [VLLM, _indexer_k_cache_head_dim] */

/* ------------------------------------------------------------------ bf16 */

static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round a finite float to bf16, nearest with ties to even, from the
 * definition: compare the 16 dropped bits with the half-way pattern. */
static uint16_t f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t hi = u >> 16, lo = u & 0xffffu;
    if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u)))
        hi += 1;
    return (uint16_t)hi;
}

/* ------------------------------------------------------- fp4 quantiser */

/* The e2m1 grid, indexed by the 3-bit magnitude code. */
static const double E2M1_GRID[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* [CMP, to_e2m1_rne]: round a magnitude onto the e2m1 grid, nearest point,
 * ties to the even code.  Brute force over the eight grid points. */
static int e2m1_code_of_magnitude(double y)
{
    int best = 0;
    double bd = fabs(y - E2M1_GRID[0]);
    for (int c = 1; c < 8; ++c) {
        double d = fabs(y - E2M1_GRID[c]);
        /* ties only occur between neighbouring codes, one even and one odd */
        if (d < bd || (d == bd && (c % 2) == 0)) {
            bd = d;
            best = c;
        }
    }
    return best;
}

/* [CMP, fp4_quant_e8m0_inplace]: the block scale is the power-of-two
 * ceiling of amax/6, amax first raised to at least 6*2^-126.  Returns the
 * exponent e of that power: the smallest integer with 6*2^e >= amax, found
 * with exact double comparisons. */
static int e8m0_exponent(float amax)
{
    double a = (double)amax;
    double floor_ = 6.0 * ldexp(1.0, -126);
    if (a < floor_)
        a = floor_;
    int E;
    frexp(a, &E); /* a in [2^(E-1), 2^E) */
    int e = E - 4;
    while (ldexp(6.0, e) < a)
        ++e;
    return e;
}

/* Quantise one block of 32 bf16 values.  codes[i] gets the 4-bit e2m1 code
 * (bit 3 = sign of the input, kept also when the magnitude rounds to zero),
 * rt[i] the dequantised value code*2^e as bf16.  Returns e. */
static int quant_block(const uint16_t *x, uint8_t *codes, uint16_t *rt)
{
    float amax = 0.0f;
    for (int i = 0; i < BLOCK; ++i) {
        float v = fabsf(bf16_to_f32(x[i]));
        if (v > amax)
            amax = v;
    }
    int e = e8m0_exponent(amax);
    for (int i = 0; i < BLOCK; ++i) {
        float v = bf16_to_f32(x[i]);
        double y = ldexp(fabs((double)v), -e); /* exact: v has 8 significant bits */
        int c = e2m1_code_of_magnitude(y);
        int neg = signbit(v) ? 1 : 0;
        codes[i] = (uint8_t)(c | (neg << 3));
        if (rt) {
            double val = ldexp(E2M1_GRID[c], e);
            float fv = (float)(neg ? -val : val);
            rt[i] = f32_to_bf16(fv); /* exact for in-range inputs (at most 2 significant bits) */
        }
    }
    return e;
}

/* Row layout (a reading; the pages fix only the 68-byte size): bytes 0..63
 * hold the 128 codes two per byte, element 2i in the low nibble of byte i;
 * byte 64+j holds the biased exponent e_j+127 of block j. */
static void quant_row(const uint16_t *x, uint8_t *row, uint16_t *rt)
{
    uint8_t codes[HEAD_DIM];
    for (int j = 0; j < HEAD_DIM / BLOCK; ++j) {
        int e = quant_block(x + j * BLOCK, codes + j * BLOCK, rt ? rt + j * BLOCK : NULL);
        row[64 + j] = (uint8_t)(e + 127);
    }
    for (int i = 0; i < 64; ++i)
        row[i] = (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));
}

/* [IDX, forward: fp4_act_quant on k and q]; [CMP, fp4_quant_e8m0_inplace].
 * x: [n_rows][128] bf16 -> rows: [n_rows][68]; rt (optional): [n_rows][128]. */
void orc_fp4_quant_rows(const uint16_t *x, int64_t n_rows, uint8_t *rows, uint16_t *rt)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_rows; ++r)
        quant_row(x + r * HEAD_DIM, rows + r * ROW_BYTES, rt ? rt + r * HEAD_DIM : NULL);
}

/* ------------------------------------------------------- exact q.k dot */

/* Signed twice-value of a nibble: 2*grid value is an integer in
 * {0,1,2,3,4,6,8,12}. */
static int nibble_twice(int nib)
{
    static const int TW[8] = {0, 1, 2, 3, 4, 6, 8, 12};
    int v = TW[nib & 7];
    return (nib & 8) ? -v : v;
}

typedef struct {
    int8_t tw[HEAD_DIM]; /* twice-values */
    int e[HEAD_DIM / BLOCK];
} decoded_row;

static void decode_row(const uint8_t *row, decoded_row *d)
{
    for (int i = 0; i < 64; ++i) {
        d->tw[2 * i] = (int8_t)nibble_twice(row[i] & 0xf);
        d->tw[2 * i + 1] = (int8_t)nibble_twice(row[i] >> 4);
    }
    for (int j = 0; j < HEAD_DIM / BLOCK; ++j)
        d->e[j] = (int)row[64 + j] - 127;
}

/* [IDX, forward: the einsum of q against index_k].  The product of two
 * dequantised rows, computed exactly: per block an integer sum of
 * twice-value products (units of 2^(eq+ek-2)), the four blocks combined in
 * 64-bit integers on a common exponent, then one rounding to fp32.  *inexact
 * is incremented when that rounding is not exact. */
static float exact_dot(const decoded_row *q, const decoded_row *k, int64_t *inexact)
{
    int64_t P[4];
    int E[4];
    int emin = 1 << 30, any = 0;
    for (int j = 0; j < 4; ++j) {
        int64_t s = 0;
        for (int i = 0; i < BLOCK; ++i)
            s += (int64_t)q->tw[j * BLOCK + i] * (int64_t)k->tw[j * BLOCK + i];
        P[j] = s;
        E[j] = q->e[j] + k->e[j];
        if (s != 0) {
            any = 1;
            if (E[j] < emin)
                emin = E[j];
        }
    }
    if (!any)
        return 0.0f;
    int spread_ok = 1;
    int64_t N = 0;
    for (int j = 0; j < 4; ++j) {
        if (P[j] == 0)
            continue;
        int sh = E[j] - emin;
        if (sh > 30) {
            spread_ok = 0;
            break;
        }
        N += P[j] * ((int64_t)1 << sh);
    }
    if (!spread_ok) {
        /* exponent spread too wide for the 64-bit path: flag and fall back */
        long double v = 0.0L;
        for (int j = 0; j < 4; ++j)
            v += ldexpl((long double)P[j], E[j] - 2);
        (*inexact)++;
        return (float)v;
    }
    double dv = ldexp((double)N, emin - 2); /* exact: |N| < 2^45 */
    float f = (float)dv;
    if ((double)f != dv)
        (*inexact)++;
    return f;
}

/* Per-head dots d[r][h][t] for t < T (test export for pinning the dot).
 * q: [R][H][128] bf16 (quantised here), kc: [B][Tcap][68] with batch
 * stride kstride rows, query row r belongs to sequence r / S. */
int64_t orc_head_dots(const uint16_t *q, const uint8_t *kc, int64_t kstride, int B, int S, int H,
                      int T, float *d)
{
    (void)B;
    int64_t R = (int64_t)B * S, inexact = 0;
    for (int64_t r = 0; r < R; ++r) {
        int64_t b = r / S;
        for (int h = 0; h < H; ++h) {
            uint8_t qrow[ROW_BYTES];
            decoded_row dq;
            quant_row(q + (r * H + h) * HEAD_DIM, qrow, NULL);
            decode_row(qrow, &dq);
            for (int t = 0; t < T; ++t) {
                decoded_row dk;
                decode_row(kc + (b * kstride + t) * ROW_BYTES, &dk);
                d[(r * H + h) * (int64_t)T + t] = exact_dot(&dq, &dk, &inexact);
            }
        }
    }
    return inexact;
}

/* ---------------------------------------------------------------- score */

/* [IDX, forward: relu, times weights, sum over heads] in the fp32 order both
 * sides share: heads [0, hs) and [hs, H), hs = ceil(H/2), each summed
 * ascending by one fmaf per head from +0, then lo + hi (one rounded add,
 * canonical +0). */
static float head_sum(const float *dh, const uint16_t *wrow, int H)
{
    const int hsplit = (H + 1) / 2;
    float lo = 0.0f, hi = 0.0f;
    for (int h = 0; h < hsplit; ++h)
        lo = fmaf(fmaxf(dh[h], 0.0f), bf16_to_f32(wrow[h]), lo);
    for (int h = hsplit; h < H; ++h)
        hi = fmaf(fmaxf(dh[h], 0.0f), bf16_to_f32(wrow[h]), hi);
    return (lo + hi) + 0.0f;
}

static int in_candidates(const int32_t *cand, int n_cand, int cbs, int t)
{
    int blk = t / cbs;
    for (int j = 0; j < n_cand; ++j)
        if (cand[j] == blk)
            return 1;
    return 0;
}

/* [IDX, forward]: index_score[r][t] = sum_h relu(q_h . k_t) * w_h, with
 *   - q quantised here (fp4_act_quant of q), k given as 68-byte rows;
 *   - the head sum in fp32 in one fixed order both sides share: heads
 *     [0, hs) and [hs, H), hs = ceil(H/2), each summed ascending by one
 *     fmaf per head from +0, then lo + hi (one rounded add);
 *   - the causal mask t >= cl[r] -> -inf ([IDX, forward: compress_lens]);
 *   - with cand != NULL (level two): t < cl[r] outside the blocks listed in
 *     cand[r][0..n_cand) -> -inf ([IDX, forward: masked_fill of ~candidates]).
 * q: [R][H][128] bf16, w: [R][H] bf16 (already scaled), R = B*S,
 * scores: [R][ld] fp32, every t < T written.  Returns the number of dots
 * whose fp32 rounding was inexact (0 for the documented input range). */
int64_t orc_score(const uint16_t *q, const uint16_t *w, const uint8_t *kc, int64_t kstride, int B,
                  int S, int H, int T, const int32_t *cl, const int32_t *cand, int n_cand, int cbs,
                  float *scores, int64_t ld)
{
    int64_t R = (int64_t)B * S, inexact_total = 0;
    decoded_row *dq = (decoded_row *)malloc(sizeof(decoded_row) * (size_t)H);
    for (int64_t r = 0; r < R; ++r) {
        int64_t b = r / S;
        for (int h = 0; h < H; ++h) {
            uint8_t qrow[ROW_BYTES];
            quant_row(q + (r * H + h) * HEAD_DIM, qrow, NULL);
            decode_row(qrow, &dq[h]);
        }
        int64_t inexact = 0;
#pragma omp parallel for schedule(static) reduction(+ : inexact)
        for (int t = 0; t < T; ++t) {
            float *out = &scores[r * ld + t];
            if (t >= cl[r]) {
                *out = -INFINITY;
                continue;
            }
            if (cand && !in_candidates(cand + r * (int64_t)n_cand, n_cand, cbs, t)) {
                *out = -INFINITY;
                continue;
            }
            decoded_row dk;
            decode_row(kc + (b * kstride + t) * ROW_BYTES, &dk);
            float dh[1024];
            for (int h = 0; h < H; ++h)
                dh[h] = exact_dot(&dq[h], &dk, &inexact);
            *out = head_sum(dh, w + r * H, H);
        }
        inexact_total += inexact;
    }
    free(dq);
    return inexact_total;
}

/* ----------------------------------------------------------------- top-k */

typedef struct {
    float s;
    int32_t t;
} ranked;

/* score descending, then position ascending (the lowest-index tie rule);
 * -0 and +0 compare equal. */
static int cmp_rank(const void *a, const void *b)
{
    const ranked *x = (const ranked *)a, *y = (const ranked *)b;
    if (x->s > y->s)
        return -1;
    if (x->s < y->s)
        return 1;
    return (x->t > y->t) - (x->t < y->t);
}

static int cmp_i32(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* One row of [IDX, forward: the final top-k]: rank all T positions by
 * (masked score desc, position asc) with t >= cl masked to -inf, keep the
 * first min(k, T), re-sort them by position, and emit t + offset for
 * t < cl and -1 otherwise.  tmp: T ranked, idx: min(k,T) ints. */
static void topk_row(const float *s, int T, int cl, int k, int32_t offset, int32_t *out,
                     ranked *tmp, int32_t *idx)
{
    int kout = k < T ? k : T;
    for (int t = 0; t < T; ++t) {
        tmp[t].s = (t < cl) ? s[t] : -INFINITY;
        tmp[t].t = t;
    }
    qsort(tmp, (size_t)T, sizeof(ranked), cmp_rank);
    for (int i = 0; i < kout; ++i)
        idx[i] = tmp[i].t;
    qsort(idx, (size_t)kout, sizeof(int32_t), cmp_i32);
    for (int i = 0; i < kout; ++i)
        out[i] = (idx[i] < cl) ? idx[i] + offset : -1;
}

/* scores: [R][ld]; out: [R][ld_out], min(k, T) entries per row written. */
void orc_topk(const float *scores, int64_t ld, int R, int T, const int32_t *cl, int k,
              int32_t offset, int32_t *out, int64_t ld_out)
{
#pragma omp parallel
    {
        ranked *tmp = (ranked *)malloc(sizeof(ranked) * (size_t)(T > 0 ? T : 1));
        int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
#pragma omp for schedule(dynamic, 1)
        for (int r = 0; r < R; ++r)
            topk_row(scores + (int64_t)r * ld, T, cl[r], k, offset, out + (int64_t)r * ld_out, tmp,
                     idx);
        free(tmp);
        free(idx);
    }
}

/* ------------------------------------------------- candidate block select */

/* [IDX, forward: select_candidate_blocks]; [CMP, select_candidate_blocks].
 * The body is not on the pages.  Reading: block j covers positions
 * [j*cbs, (j+1)*cbs) clipped to T; its score is the maximum of its masked
 * scores (t >= cl -> -inf); the blocks are then ranked exactly like the
 * top-k above with k = ctb, compress_lens ceil(min(cl,T)/cbs) and offset 0.
 * ids: [R][ld_ids], min(ctb, nb) ascending block ids per row, -1 for a kept
 * block with no reachable position. */
void orc_select_blocks(const float *scores, int64_t ld, int R, int T, const int32_t *cl, int ctb,
                       int cbs, int32_t *ids, int64_t ld_ids)
{
    int nb = (T + cbs - 1) / cbs;
#pragma omp parallel
    {
        float *bmax = (float *)malloc(sizeof(float) * (size_t)(nb > 0 ? nb : 1));
        ranked *tmp = (ranked *)malloc(sizeof(ranked) * (size_t)(nb > 0 ? nb : 1));
        int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nb > 0 ? nb : 1));
#pragma omp for schedule(dynamic, 1)
        for (int r = 0; r < R; ++r) {
            int c = cl[r] < T ? cl[r] : T;
            for (int j = 0; j < nb; ++j) {
                float m = -INFINITY;
                for (int t = j * cbs; t < (j + 1) * cbs && t < T; ++t) {
                    float v = (t < c) ? scores[(int64_t)r * ld + t] : -INFINITY;
                    if (v > m)
                        m = v;
                }
                bmax[j] = m;
            }
            int clb = (c + cbs - 1) / cbs;
            topk_row(bmax, nb, clb, ctb, 0, ids + (int64_t)r * ld_ids, tmp, idx);
        }
        free(bmax);
        free(tmp);
        free(idx);
    }
}

/* ------------------------------------------------------------ key publish */

/* The key for one latent, before quantisation ([IDX, forward: the
 * index-key publish]): y = wk . latent (fp32, one fmaf per input feature in
 * order, from +0, rounded to bf16 as the bf16 Linear output);
 * RMSNorm: ss = sum of y_o^2 (fmaf, o ascending), inv = 1/sqrt(ss/D + eps)
 * (correctly rounded), z_o = bf16((y_o*inv)*gamma_o); RoPE on the last rd
 * dims as interleaved pairs (x0, x1) rotated by (c, s):
 * (x0*c - x1*s, x0*s + x1*c), each product and sum rounded in fp32,
 * then bf16.  z: [128] bf16. */
/* [IDX, forward: apply_rotary_emb on the last rd dims]: interleaved pairs
 * (x0, x1) = (z[D-rd+2i], z[D-rd+2i+1]) rotated by (c, s) = cs_row[i]:
 * (x0*c - x1*s, x0*s + x1*c), each product and sum rounded in fp32 (no
 * fused multiply-add), then bf16.  z: [128] bf16, in place. */
static void rope_row(uint16_t *z, const float *cs_row, int rd)
{
    int base = HEAD_DIM - rd;
    for (int i = 0; i < rd / 2; ++i) {
        float x0 = bf16_to_f32(z[base + 2 * i]), x1 = bf16_to_f32(z[base + 2 * i + 1]);
        float c = cs_row[2 * i], s = cs_row[2 * i + 1];
        float a = x0 * c, bb = x1 * s, cc = x0 * s, dd = x1 * c;
        z[base + 2 * i] = f32_to_bf16(a - bb);
        z[base + 2 * i + 1] = f32_to_bf16(cc + dd);
    }
}

static void publish_prequant(const uint16_t *latent, const uint16_t *wk, const float *gamma,
                             const float *cs_row, int Din, int rd, float eps, uint16_t *z)
{
    float y[HEAD_DIM];
    for (int o = 0; o < HEAD_DIM; ++o) {
        float acc = 0.0f;
        for (int i = 0; i < Din; ++i)
            acc = fmaf(bf16_to_f32(wk[(int64_t)o * Din + i]), bf16_to_f32(latent[i]), acc);
        y[o] = bf16_to_f32(f32_to_bf16(acc));
    }
    float ss = 0.0f;
    for (int o = 0; o < HEAD_DIM; ++o)
        ss = fmaf(y[o], y[o], ss);
    float inv = 1.0f / sqrtf(ss / (float)HEAD_DIM + eps);
    for (int o = 0; o < HEAD_DIM; ++o) {
        float v = y[o] * inv;
        v = v * gamma[o];
        z[o] = f32_to_bf16(v);
    }
    rope_row(z, cs_row, rd);
}

/* Position and cache row of group g ([IDX, forward]: in prefill group j sits
 * at position j*ratio and fills row j; in decode the completed group sits at
 * start_pos+1-ratio and fills row start_pos/ratio). */
static void publish_slot(int start_pos, int ratio, int g, int *pos, int *row)
{
    if (start_pos == 0) {
        *pos = g * ratio;
        *row = g;
    } else {
        *pos = start_pos + 1 - ratio;
        *row = start_pos / ratio + g;
    }
}

/* latent: [B][G][Din] bf16, wk: [128][Din] bf16, gamma: [128] fp32,
 * cos_sin: [P][rd/2][2] fp32.  Writes kc[b][row] (68 bytes).  prequant
 * (optional): [B][G][128] bf16 keys before quantisation, for pinning. */
void orc_publish(const uint16_t *latent, const uint16_t *wk, const float *gamma,
                 const float *cos_sin, int P, int B, int G, int Din, int rd, float eps,
                 int start_pos, int ratio, uint8_t *kc, int64_t kstride, uint16_t *prequant)
{
    (void)P;
#pragma omp parallel for schedule(static)
    for (int64_t bg = 0; bg < (int64_t)B * G; ++bg) {
        int64_t b = bg / G;
        int g = (int)(bg % G);
        int pos, row;
        publish_slot(start_pos, ratio, g, &pos, &row);
        uint16_t z[HEAD_DIM];
        publish_prequant(latent + bg * Din, wk, gamma, cos_sin + (int64_t)pos * rd, Din, rd, eps,
                         z);
        if (prequant)
            memcpy(prequant + bg * HEAD_DIM, z, sizeof(z));
        quant_row(z, kc + (b * kstride + row) * ROW_BYTES, NULL);
    }
}

/* ------------------------------------------------------ query RoPE + quant */

/* The query side of the step ([IDX, forward]: q split into heads,
 * apply_rotary_emb(q[..., -rd:], freqs_cis[start_pos:end_pos]),
 * fp4_act_quant(q), weights = weights_proj(x) * (softmax_scale *
 * n_heads^-0.5); [VLLM, fused_indexer_q_rope_quant] does the three in one
 * step).  Row r = b*S + s sits at position start_pos + s.
 *   q: [R][H][128] bf16 before RoPE; w_raw: [R][H] bf16; scale: fp32
 *   cos_sin: [P][rd/2][2] fp32
 *   rows: [R][H][68] quantised heads; rt (optional): [R][H][128] their bf16
 *   round trip; prequant (optional): [R][H][128] bf16 after RoPE, before
 *   quantisation; w_out: [R][H] bf16, bf16(fp32(w_raw) * scale). */
void orc_q_rope_quant(const uint16_t *q, const uint16_t *w_raw, float scale, const float *cos_sin,
                      int P, int B, int S, int H, int rd, int start_pos, uint8_t *rows,
                      uint16_t *rt, uint16_t *prequant, uint16_t *w_out)
{
    (void)P;
    int64_t R = (int64_t)B * S;
#pragma omp parallel for schedule(static)
    for (int64_t rh = 0; rh < R * H; ++rh) {
        int64_t r = rh / H;
        int pos = start_pos + (int)(r % S);
        uint16_t z[HEAD_DIM];
        memcpy(z, q + rh * HEAD_DIM, sizeof(z));
        rope_row(z, cos_sin + (int64_t)pos * rd, rd);
        if (prequant)
            memcpy(prequant + rh * HEAD_DIM, z, sizeof(z));
        quant_row(z, rows + rh * ROW_BYTES, rt ? rt + rh * HEAD_DIM : NULL);
        w_out[rh] = f32_to_bf16(bf16_to_f32(w_raw[rh]) * scale);
    }
}

/* ------------------------------------------------------- FP8 key cache */

/* The FP8 indexer cache ([VLLM, _indexer_k_cache_head_dim]: 128 fp8 bytes
 * and one fp32 scale per 128 values, 132-byte rows; [VLLM,
 * DeepseekV4Indexer.__init__]: quant_block_size 128, scale_fmt "ue8m0").
 * Readings: the fp8 format is OCP e4m3 (finite maximum 448); the ue8m0 scale
 * of a 128-value block is the power of two 2^e with e the smallest integer
 * such that 448 * 2^e >= amax, amax first raised to at least 448 * 2^-126
 * (the e2m1 rule of [CMP, fp4_quant_e8m0_inplace] with e4m3's maximum in
 * place of e2m1's); values are rounded to the nearest e4m3 point of x/2^e,
 * ties to the even code, sign kept; the query heads go through the same
 * quantiser. */
#define FP8_ROW_BYTES 132
#define E4M3_MAX 448.0

/* Value of a non-negative e4m3 code 0..126 (code 127 is NaN): exponent
 * field E (bias 7), mantissa m: subnormal m * 2^-9 for E = 0, else
 * (8 + m) * 2^(E - 10). */
static double e4m3_value(int c)
{
    int E = c >> 3, m = c & 7;
    return E == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), E - 10);
}

/* Nearest non-negative e4m3 code to y (0 <= y <= 448), ties to the even
 * code: the codes order like their values, so the two neighbours of y are
 * found by bisection and compared. */
static int e4m3_code_of_magnitude(double y)
{
    int lo = 0, hi = 126; /* e4m3_value(lo) <= y <= e4m3_value(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (e4m3_value(mid) <= y)
            lo = mid;
        else
            hi = mid;
    }
    double dl = y - e4m3_value(lo), dh = e4m3_value(hi) - y;
    if (dl < dh)
        return lo;
    if (dh < dl)
        return hi;
    return (lo % 2 == 0) ? lo : hi;
}

/* Scale exponent of a 128-value block: the smallest e with 448 * 2^e >=
 * amax, amax raised to at least 448 * 2^-126; exact double comparisons. */
static int ue8m0_exponent_fp8(float amax)
{
    double a = (double)amax, floor_ = E4M3_MAX * ldexp(1.0, -126);
    if (a < floor_)
        a = floor_;
    int E;
    frexp(a, &E); /* a in [2^(E-1), 2^E) */
    int e = E - 10;
    while (ldexp(E4M3_MAX, e) < a)
        ++e;
    return e;
}

/* Row layout: bytes 0..127 the e4m3 codes of elements 0..127 (bit 7 =
 * sign), bytes 128..131 the scale 2^e as a little-endian fp32. */
static void quant_row_fp8(const uint16_t *x, uint8_t *row, uint16_t *rt)
{
    float amax = 0.0f;
    for (int i = 0; i < HEAD_DIM; ++i) {
        float v = fabsf(bf16_to_f32(x[i]));
        if (v > amax)
            amax = v;
    }
    int e = ue8m0_exponent_fp8(amax);
    for (int i = 0; i < HEAD_DIM; ++i) {
        float v = bf16_to_f32(x[i]);
        int c = e4m3_code_of_magnitude(ldexp(fabs((double)v), -e)); /* exact scaling */
        int neg = signbit(v) ? 1 : 0;
        row[i] = (uint8_t)(c | (neg << 7));
        if (rt) {
            double val = ldexp(e4m3_value(c), e);
            rt[i] = f32_to_bf16((float)(neg ? -val : val)); /* exact: 4 significant bits */
        }
    }
    float scale = ldexpf(1.0f, e);
    memcpy(row + HEAD_DIM, &scale, 4);
}

/* x: [n_rows][128] bf16 -> rows: [n_rows][132]; rt (optional): [n_rows][128]. */
void orc_fp8_quant_rows(const uint16_t *x, int64_t n_rows, uint8_t *rows, uint16_t *rt)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_rows; ++r)
        quant_row_fp8(x + r * HEAD_DIM, rows + r * FP8_ROW_BYTES, rt ? rt + r * HEAD_DIM : NULL);
}

typedef struct {
    double v[HEAD_DIM]; /* e4m3 values, scale not applied */
    int e;
} decoded_row_fp8;

static void decode_row_fp8(const uint8_t *row, decoded_row_fp8 *d)
{
    for (int i = 0; i < HEAD_DIM; ++i) {
        int c = row[i];
        double v = e4m3_value(c & 0x7f);
        d->v[i] = (c & 0x80) ? -v : v;
    }
    float scale;
    memcpy(&scale, row + HEAD_DIM, 4);
    int E;
    frexpf(scale, &E);
    d->e = E - 1; /* scale = 2^e */
}

/* [IDX, forward: the einsum of q against index_k] on fp8 rows: the sum of
 * the 128 products of e4m3 values is exact in double (each product has at
 * most 8 significant bits between 2^-18 and 2^17.6, so the sum needs at
 * most 43 bits), then it is scaled by 2^(eq + ek) and rounded once to fp32. */
static float exact_dot_fp8(const decoded_row_fp8 *q, const decoded_row_fp8 *k, int64_t *inexact)
{
    double s = 0.0;
    for (int i = 0; i < HEAD_DIM; ++i)
        s += q->v[i] * k->v[i];
    double d = ldexp(s, q->e + k->e);
    float f = (float)d;
    if ((double)f != d)
        (*inexact)++;
    return f;
}

/* Per-head fp8 dots d[r][h][t] (test export).  q: [R][H][128] bf16,
 * quantised here; kc: [B][Tcap][132].  Returns the count of dots whose fp32
 * rounding was inexact (rounding is expected here, unlike fp4). */
int64_t orc_head_dots_fp8(const uint16_t *q, const uint8_t *kc, int64_t kstride, int B, int S,
                          int H, int T, float *d)
{
    int64_t R = (int64_t)B * S, inexact = 0;
    for (int64_t r = 0; r < R; ++r) {
        int64_t b = r / S;
        for (int h = 0; h < H; ++h) {
            uint8_t qrow[FP8_ROW_BYTES];
            decoded_row_fp8 dq, dk;
            quant_row_fp8(q + (r * H + h) * HEAD_DIM, qrow, NULL);
            decode_row_fp8(qrow, &dq);
            for (int t = 0; t < T; ++t) {
                decode_row_fp8(kc + (b * kstride + t) * FP8_ROW_BYTES, &dk);
                d[(r * H + h) * (int64_t)T + t] = exact_dot_fp8(&dq, &dk, &inexact);
            }
        }
    }
    return inexact;
}

/* orc_score on the FP8 cache: q quantised per head by the fp8 quantiser,
 * keys [B][Tcap][132]; masks and the head sum as orc_score. */
int64_t orc_score_fp8(const uint16_t *q, const uint16_t *w, const uint8_t *kc, int64_t kstride,
                      int B, int S, int H, int T, const int32_t *cl, const int32_t *cand,
                      int n_cand, int cbs, float *scores, int64_t ld)
{
    int64_t R = (int64_t)B * S, inexact_total = 0;
    decoded_row_fp8 *dq = (decoded_row_fp8 *)malloc(sizeof(decoded_row_fp8) * (size_t)H);
    for (int64_t r = 0; r < R; ++r) {
        int64_t b = r / S;
        for (int h = 0; h < H; ++h) {
            uint8_t qrow[FP8_ROW_BYTES];
            quant_row_fp8(q + (r * H + h) * HEAD_DIM, qrow, NULL);
            decode_row_fp8(qrow, &dq[h]);
        }
        int64_t inexact = 0;
#pragma omp parallel for schedule(static) reduction(+ : inexact)
        for (int t = 0; t < T; ++t) {
            float *out = &scores[r * ld + t];
            if (t >= cl[r] || (cand && !in_candidates(cand + r * (int64_t)n_cand, n_cand, cbs, t))) {
                *out = -INFINITY;
                continue;
            }
            decoded_row_fp8 dk;
            decode_row_fp8(kc + (b * kstride + t) * FP8_ROW_BYTES, &dk);
            float dh[1024];
            for (int h = 0; h < H; ++h)
                dh[h] = exact_dot_fp8(&dq[h], &dk, &inexact);
            *out = head_sum(dh, w + r * H, H);
        }
        inexact_total += inexact;
    }
    free(dq);
    return inexact_total;
}
