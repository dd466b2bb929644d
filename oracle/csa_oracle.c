/*
 * csa_oracle.c -- plain, slow, obviously-correct CPU reference for the
 * Compressed Sparse Attention (CSA) / Heavily Compressed Attention (HCA) /
 * DeepSeek Sparse Attention (DSA) hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library shares
 * no code, header, table or constant generator with it.
 *
 * Sources (the Hugging Face Transformers model pages):
 *   [V4-HA]   "DeepSeek-V4", section "Hybrid attention (§2.3)"
 *   [V4-MASK] "DeepSeek-V4", section "Attention mask layout"
 *   [V4-CACHE]"DeepSeek-V4", section "Cache layers"
 *   [V4-CFG]  "DeepSeek-V4", DeepseekV4Config parameter list
 *   [V32-DSA] "DeepSeek-V3.2", section "DeepSeek Sparse Attention (DSA)"
 *
 * Arithmetic: fp32 storage and fp32 arithmetic, every sum taken sequentially
 * in index order (no blocking, no reassociation).  RoPE angles are formed in
 * fp64 and their cosine/sine rounded once to fp32.  Where the GPU library
 * stores bf16, the caller asks this oracle to round to bf16 (round to nearest
 * even) at the same point.
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes): the index-score form (weighted sum of ReLU'd per-head dot
 * products), the gated-softmax pooling of the compressor, the 2m overlap
 * window, the pool-entry RoPE position pos0 + w*m, the sink as an extra
 * softmax denominator term, output de-rotation only when dv == D, and zero
 * output for a row with no visible key and no sink.
 *
 * "parity unpinned" (no value on the pages fixes them; pinned only by the
 * invariants in the test-suite): the ReLU in the index score, the gating
 * form of the compressor, the pool-entry RoPE position, the choice of theta
 * per layer and the softmax scale.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_BAD_ARG 1

/* ---------------------------------------------------------------------------
 * bf16 storage rounding: keep the top 16 bits of the fp32 pattern, rounding to
 * nearest with ties to even.  Finite inputs only.
 * ------------------------------------------------------------------------- */
static float round_to_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u = u + 0x7fffu + lsb;
    u &= 0xffff0000u;
    float r;
    memcpy(&r, &u, 4);
    return r;
}

float orc_round_bf16(float x) { return round_to_bf16(x); }

void orc_round_bf16_array(float *a, long n)
{
    for (long e = 0; e < n; ++e) a[e] = round_to_bf16(a[e]);
}

/* ---------------------------------------------------------------------------
 * RoPE ([V4-HA] partial RoPE on the trailing qk_rope_head_dim channels,
 * interleaved pairs; [V4-CFG] rope_theta / compress_rope_theta).
 * Pair i (0 <= i < rope_dim/2) is the channel pair (D-rope_dim+2i,
 * D-rope_dim+2i+1).  Its frequency is theta^(-2i/rope_dim); the angle at
 * position p is p times that frequency.
 * ------------------------------------------------------------------------- */
/* freq: per-pair frequencies (e.g. YaRN's, below), or NULL for the plain
 * theta^(-2i/rope_dim). */
static void rope_cos_sin(double theta, int rope_dim, long pos, int i,
                         const double *freqs, float *c, float *s)
{
    double freq = freqs ? freqs[i] : pow(theta, -2.0 * (double)i / (double)rope_dim);
    double angle = (double)pos * freq;
    *c = (float)cos(angle);
    *s = (float)sin(angle);
}

/* cs[p][i][0] = cos, cs[p][i][1] = sin, for p in [0, n_pos). */
void orc_rope_table_f(float *cs, int n_pos, int rope_dim, double theta, const double *freqs)
{
    int half = rope_dim / 2;
    for (long p = 0; p < n_pos; ++p)
        for (int i = 0; i < half; ++i)
            rope_cos_sin(theta, rope_dim, p, i, freqs, &cs[(p * half + i) * 2],
                         &cs[(p * half + i) * 2 + 1]);
}

void orc_rope_table(float *cs, int n_pos, int rope_dim, double theta)
{
    orc_rope_table_f(cs, n_pos, rope_dim, theta, NULL);
}

/* ---------------------------------------------------------------------------
 * YaRN-scaled frequencies ([V4-CFG] compress_rope_theta is used together with
 * rope scaling for YaRN; rope_parameters carry the scaling for a longer
 * max_position_embeddings).  The pages name the method only; its steps here
 * are those of the published YaRN method ("NTK-by-parts" interpolation, Peng
 * et al. 2023) in the per-pair-index form of the Transformers RoPE utilities:
 *   1. f_i = theta^(-2i/d) for the d/2 pairs (d = rope_dim).
 *   2. Over the original context L a pair turns L f_i / (2 pi) times; the
 *      (fractional) pair index at which that count equals r is
 *      i(r) = d ln(L / (2 pi r)) / (2 ln theta).
 *   3. low = floor(i(beta_fast)) clamped at 0, high = ceil(i(beta_slow))
 *      clamped at d - 1; if they coincide high is moved up by 0.001.
 *   4. ramp_i = clamp((i - low) / (high - low), 0, 1).
 *   5. f'_i = (f_i / factor) ramp_i + f_i (1 - ramp_i): fast pairs (many
 *      turns over L) keep their frequency, slow pairs are interpolated by the
 *      factor, the ones between blend linearly in i.
 * The magnitude correction YaRN also defines is a scalar on the logits and is
 * not part of the table (the table stays a pure rotation).
 * ------------------------------------------------------------------------- */
void orc_yarn_freqs(double *freqs, int rope_dim, double theta, double factor,
                    long original_max_pos, double beta_fast, double beta_slow)
{
    const double two_pi = 2.0 * acos(-1.0);
    double d = (double)rope_dim;
    double i_fast = d * log((double)original_max_pos / (two_pi * beta_fast)) / (2.0 * log(theta));
    double i_slow = d * log((double)original_max_pos / (two_pi * beta_slow)) / (2.0 * log(theta));
    double low = floor(i_fast), high = ceil(i_slow);
    if (low < 0.0) low = 0.0;
    if (high > d - 1.0) high = d - 1.0;
    if (high == low) high += 0.001;
    for (int i = 0; i < rope_dim / 2; ++i) {
        double f = pow(theta, -2.0 * (double)i / d);
        double ramp = ((double)i - low) / (high - low);
        if (ramp < 0.0) ramp = 0.0;
        if (ramp > 1.0) ramp = 1.0;
        freqs[i] = (f / factor) * ramp + f * (1.0 - ramp);
    }
}

/* Rotate the trailing rope_dim channels of v (length D) by +pos (sign=+1) or
 * by -pos (sign=-1): the pair (a, b) becomes (a*c - b*s, a*s + b*c) with
 * s = sin(sign*angle). */
static void rope_apply(float *v, int D, int rope_dim, double theta, const double *freqs,
                       long pos, int sign)
{
    int base = D - rope_dim;
    for (int i = 0; i < rope_dim / 2; ++i) {
        float c, s;
        rope_cos_sin(theta, rope_dim, pos, i, freqs, &c, &s);
        if (sign < 0) s = -s;
        float a = v[base + 2 * i];
        float b = v[base + 2 * i + 1];
        float na = a * c - b * s;
        float nb = a * s + b * c;
        v[base + 2 * i] = na;
        v[base + 2 * i + 1] = nb;
    }
}

/* Public helper so the tests can pin the rotation itself: n rows of length
 * D, row r rotated at sign*pos[r]. */
void orc_rope_apply_f(float *v, long n, int D, int rope_dim, double theta,
                      const double *freqs, const long *pos, int sign)
{
    for (long r = 0; r < n; ++r)
        rope_apply(v + r * D, D, rope_dim, theta, freqs, pos[r], sign);
}

void orc_rope_apply(float *v, long n, int D, int rope_dim, double theta,
                    const long *pos, int sign)
{
    orc_rope_apply_f(v, n, D, rope_dim, theta, NULL, pos, sign);
}

/* ---------------------------------------------------------------------------
 * Compressor ([V4-HA] CSA pool with overlapping windows at rate m, HCA pool
 * with non-overlapping windows at rate m'; [V4-CACHE] the compressor keeps a
 * buffer / pool / count, plus overlap state for CSA and a parallel indexer
 * compressor at index_head_dim).
 *
 * One sequence.  x, gate: [S][D]; slot_bias: [(1+overlap)*m][D] or NULL;
 * gate NULL means all logits zero.  pool: [S/m][D].
 * Entry w pools tokens j in [max(0,(w-overlap)*m), (w+1)*m); for every
 * channel c the weights are softmax_j(gate[j][c] + slot_bias[j-(w-overlap)*m][c]).
 * Then the trailing rope_dim channels are rotated to position pos0 + w*m,
 * then the entry is rounded to bf16 if round_bf16 is set.
 * ------------------------------------------------------------------------- */
int orc_compress_f(const float *x, const float *gate, const float *slot_bias,
                   float *pool, int S, int D, int m, int overlap, int rope_dim,
                   double theta, const double *freqs, long pos0, int round_bf16)
{
    if (m < 1 || S < 0 || D < 1 || (overlap != 0 && overlap != 1) ||
        rope_dim < 0 || rope_dim > D || (rope_dim & 1))
        return ORC_BAD_ARG;
    int T = S / m;
    int span = (1 + overlap) * m;
#pragma omp parallel for schedule(static)
    for (int w = 0; w < T; ++w) {
        long first_slot_pos = (long)(w - overlap) * m; /* token of slot 0 */
        long j0 = first_slot_pos < 0 ? 0 : first_slot_pos;
        long j1 = (long)(w + 1) * m;
        float *logit = (float *)malloc(sizeof(float) * span);
        float *out = pool + (long)w * D;
        for (int c = 0; c < D; ++c) {
            int n = 0;
            float mx = -INFINITY;
            for (long j = j0; j < j1; ++j) {
                float a = 0.0f;
                if (gate) a += gate[j * D + c];
                if (slot_bias) a += slot_bias[(j - first_slot_pos) * D + c];
                logit[n++] = a;
                if (a > mx) mx = a;
            }
            float den = 0.0f;
            for (int q = 0; q < n; ++q) den += expf(logit[q] - mx);
            float acc = 0.0f;
            for (int q = 0; q < n; ++q) {
                float wgt = expf(logit[q] - mx) / den;
                acc += wgt * x[(j0 + q) * D + c];
            }
            out[c] = acc;
        }
        if (rope_dim > 0)
            rope_apply(out, D, rope_dim, theta, freqs, pos0 + (long)w * m, +1);
        if (round_bf16)
            for (int c = 0; c < D; ++c) out[c] = round_to_bf16(out[c]);
        free(logit);
    }
    return ORC_OK;
}

int orc_compress(const float *x, const float *gate, const float *slot_bias,
                 float *pool, int S, int D, int m, int overlap, int rope_dim,
                 double theta, long pos0, int round_bf16)
{
    return orc_compress_f(x, gate, slot_bias, pool, S, D, m, overlap, rope_dim, theta,
                          NULL, pos0, round_bf16);
}

/* ---------------------------------------------------------------------------
 * Readiness ([V4-MASK]): query at absolute position t may use pool entry w
 * only once w's source window has closed, i.e. w < (t+1)/m (integer
 * division), and never beyond the T entries that exist.
 * ------------------------------------------------------------------------- */
static long ready_count(long t, int m, int T)
{
    long r = (t + 1) / m;
    if (t + 1 < 0) r = 0;
    if (r > T) r = T;
    if (r < 0) r = 0;
    return r;
}

long orc_ready_count(long t, int m, int T) { return ready_count(t, m, T); }

/* ---------------------------------------------------------------------------
 * Lightning-Indexer score ([V4-HA] indexer scoring queries against the pool,
 * eqs. 13-17; [V4-CFG] index_n_heads n_h^I (eq. 14), index_head_dim c^I;
 * [V32-DSA] low-head-count score between a query and earlier keys, a dot
 * product against a single-head key, per-head weights).
 *
 * Rows r in [0, n_rows): query at absolute position tpos[r], heads qI[r][j][c]
 * (n_heads x head_dim), per-head weights wI[r][j].  Keys kI[w][c], w < T.
 *   score[r][w] = sum_j wI[r][j] * max(0, sum_c qI[r][j][c] * kI[w][c])
 * for w < R(t); +0.0f is added so a negative zero becomes +0.  Entries with
 * w >= R(t) are written as -inf (never selectable).
 * ------------------------------------------------------------------------- */
int orc_index_scores(const float *qI, const float *wI, const long *tpos,
                     int n_rows, const float *kI, int T, int n_heads,
                     int head_dim, int m, float *scores)
{
    if (m < 1 || T < 0 || n_heads < 1 || head_dim < 1) return ORC_BAD_ARG;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < n_rows; ++r) {
        long R = ready_count(tpos[r], m, T);
        const float *qrow = qI + (long)r * n_heads * head_dim;
        for (long w = 0; w < T; ++w) {
            if (w >= R) {
                scores[(long)r * T + w] = -INFINITY;
                continue;
            }
            float s = 0.0f;
            for (int j = 0; j < n_heads; ++j) {
                float dot = 0.0f;
                for (int c = 0; c < head_dim; ++c)
                    dot += qrow[(long)j * head_dim + c] * kI[w * head_dim + c];
                float relu = dot > 0.0f ? dot : 0.0f;
                s += wI[(long)r * n_heads + j] * relu;
            }
            scores[(long)r * T + w] = s + 0.0f;
        }
    }
    return ORC_OK;
}

/* ---------------------------------------------------------------------------
 * Top-k ([V4-CFG] index_topk, eq. 17; [V4-MASK] the indexer emits the -1
 * sentinel for slots it cannot fill before enough entries are ready).
 * Candidates w < R(t).  Order by score descending, equal scores by lower
 * index first; keep the first min(k, R(t)); emit those indices in ascending
 * order, then -1 for the remaining slots.
 * ------------------------------------------------------------------------- */
typedef struct {
    float score;
    int index;
} cand_t;

static int cand_cmp(const void *pa, const void *pb)
{
    const cand_t *a = (const cand_t *)pa, *b = (const cand_t *)pb;
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
    return (a->index > b->index) - (a->index < b->index);
}

static int int_cmp(const void *pa, const void *pb)
{
    int a = *(const int *)pa, b = *(const int *)pb;
    return (a > b) - (a < b);
}

int orc_topk(const float *scores, const long *tpos, int n_rows, int T, int k,
             int m, int *idx)
{
    if (k < 1 || m < 1 || T < 0) return ORC_BAD_ARG;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < n_rows; ++r) {
        long R = ready_count(tpos[r], m, T);
        cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (R > 0 ? R : 1));
        for (long w = 0; w < R; ++w) {
            c[w].score = scores[(long)r * T + w];
            c[w].index = (int)w;
        }
        qsort(c, (size_t)R, sizeof(cand_t), cand_cmp);
        long keep = R < k ? R : k;
        int *out = idx + (long)r * k;
        for (long q = 0; q < keep; ++q) out[q] = c[q].index;
        qsort(out, (size_t)keep, sizeof(int), int_cmp);
        for (long q = keep; q < k; ++q) out[q] = -1;
        free(c);
    }
    return ORC_OK;
}

/* ---------------------------------------------------------------------------
 * Core attention ([V4-HA] shared K=V multi-query attention with one KV head,
 * partial RoPE on q, de-rotation of the output rope slice at -t (eq. 26), a
 * learnable per-head sink (eq. 27), the sliding-window K=V branch
 * concatenated with the compressed entries; [V4-MASK] the mask columns;
 * [V32-DSA] attention restricted to the selected tokens).
 *
 * Rows r: query q[r][h][c] (H x D) at absolute position tpos[r].
 * Visible keys, in this order:
 *   window: positions s in (t-window, t] held in kv_win (row s-win_pos0,
 *           when 0 <= s-win_pos0 < L_win), already rotated at s;
 *   pool:   idx != NULL: pool rows idx[r][j] != -1 (j ascending);
 *           idx == NULL: all pool rows w < R(t) (HCA, dense over ready
 *           entries).  Pool rows are already rotated.
 * Per head h: q~ = q rotated at +t; l_j = scale * <q~, key_j>;
 * M = max(z_h, max_j l_j) (z_h absent without a sink);
 * den = exp(z_h - M) + sum_j exp(l_j - M); o = sum_j exp(l_j - M)/den * key_j[:dv];
 * if dv == D the trailing rope_dim channels of o are rotated at -t.
 * A row with no visible key and no sink gives o = 0.
 * ------------------------------------------------------------------------- */
int orc_attention_f(const float *q, const long *tpos, int n_rows, int H, int D,
                    int dv, const float *kv_win, long win_pos0, int L_win,
                    int window, const float *pool, int T, const int *idx, int k,
                    int m, const float *sink, int rope_dim, double theta,
                    const double *freqs, float scale, float *out)
{
    if (H < 1 || D < 1 || (dv != D && dv != D - rope_dim) || rope_dim < 0 ||
        rope_dim > D || (rope_dim & 1) || window < 0 || m < 1 || T < 0)
        return ORC_BAD_ARG;
    if (idx) {
        for (long e = 0; e < (long)n_rows * k; ++e)
            if (idx[e] < -1 || idx[e] >= T) return ORC_BAD_ARG;
    }
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int r = 0; r < n_rows; ++r) {
        for (int h = 0; h < H; ++h) {
            long t = tpos[r];
            /* gather the visible key rows, window branch first */
            long max_keys = (long)window + (idx ? k : T);
            const float **keys =
                (const float **)malloc(sizeof(float *) * (max_keys > 0 ? max_keys : 1));
            long nk = 0;
            for (long s = t - window + 1; s <= t; ++s) {
                long row = s - win_pos0;
                if (s < 0 || row < 0 || row >= L_win || !kv_win) continue;
                keys[nk++] = kv_win + row * D;
            }
            if (idx) {
                for (int j = 0; j < k; ++j) {
                    int w = idx[(long)r * k + j];
                    if (w >= 0) keys[nk++] = pool + (long)w * D;
                }
            } else {
                long R = ready_count(t, m, T);
                for (long w = 0; w < R; ++w) keys[nk++] = pool + w * D;
            }

            float *qr = (float *)malloc(sizeof(float) * D);
            float *logit = (float *)malloc(sizeof(float) * (nk > 0 ? nk : 1));
            float *o = (float *)malloc(sizeof(float) * D);
            memcpy(qr, q + ((long)r * H + h) * D, sizeof(float) * D);
            if (rope_dim > 0) rope_apply(qr, D, rope_dim, theta, freqs, t, +1);

            float M = sink ? sink[h] : -INFINITY;
            for (long j = 0; j < nk; ++j) {
                float dot = 0.0f;
                for (int c = 0; c < D; ++c) dot += qr[c] * keys[j][c];
                logit[j] = scale * dot;
                if (logit[j] > M) M = logit[j];
            }
            float den = sink ? expf(sink[h] - M) : 0.0f;
            for (long j = 0; j < nk; ++j) den += expf(logit[j] - M);

            /* o[c] accumulates over j in list order for every channel c */
            for (int c = 0; c < D; ++c) o[c] = 0.0f;
            if (den > 0.0f) {
                for (long j = 0; j < nk; ++j) {
                    float p = expf(logit[j] - M) / den;
                    for (int c = 0; c < dv; ++c) o[c] += p * keys[j][c];
                }
            }
            if (dv == D && rope_dim > 0) rope_apply(o, D, rope_dim, theta, freqs, t, -1);
            memcpy(out + ((long)r * H + h) * dv, o, sizeof(float) * dv);
            free(qr);
            free(logit);
            free(o);
            free(keys);
        }
    }
    return ORC_OK;
}

int orc_attention(const float *q, const long *tpos, int n_rows, int H, int D,
                  int dv, const float *kv_win, long win_pos0, int L_win,
                  int window, const float *pool, int T, const int *idx, int k,
                  int m, const float *sink, int rope_dim, double theta,
                  float scale, float *out)
{
    return orc_attention_f(q, tpos, n_rows, H, D, dv, kv_win, win_pos0, L_win, window,
                           pool, T, idx, k, m, sink, rope_dim, theta, NULL, scale, out);
}
