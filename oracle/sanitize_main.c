/*
 * sanitize_main.c -- drives every entry point of csa_oracle.c over small
 * seeded inputs and their edge cases, for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitize.py compiles and runs
 * it).  TEST INFRASTRUCTURE ONLY, like the oracle itself.
 *
 * Cases: ragged sequences (S not a multiple of m), overlap on and off, gate
 * and slot bias absent or present, no whole window (T = 0), rows whose ready
 * count is 0, below k and above k, index rows with -1 padding, a window that
 * starts before token 0, dv = D and dv = D - rope_dim, with and without the
 * sink, YaRN frequencies.  Each call's status is checked; the outputs are
 * only required to be finite where the definition makes them finite.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void orc_rope_table_f(float *cs, int n_pos, int rope_dim, double theta, const double *freqs);
void orc_yarn_freqs(double *freqs, int rope_dim, double theta, double factor,
                    long original_max_pos, double beta_fast, double beta_slow);
void orc_rope_apply_f(float *v, long n, int D, int rope_dim, double theta,
                      const double *freqs, const long *pos, int sign);
int orc_compress_f(const float *x, const float *gate, const float *slot_bias, float *pool,
                   int S, int D, int m, int overlap, int rope_dim, double theta,
                   const double *freqs, long pos0, int round_bf16);
long orc_ready_count(long t, int m, int T);
int orc_index_scores(const float *qI, const float *wI, const long *tpos, int n_rows,
                     const float *kI, int T, int n_heads, int head_dim, int m, float *scores);
int orc_topk(const float *scores, const long *tpos, int n_rows, int T, int k, int m, int *idx);
int orc_attention_f(const float *q, const long *tpos, int n_rows, int H, int D, int dv,
                    const float *kv_win, long win_pos0, int L_win, int window,
                    const float *pool, int T, const int *idx, int k, int m,
                    const float *sink, int rope_dim, double theta, const double *freqs,
                    float scale, float *out);

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;

/* splitmix64 step mapped to [-1, 1) */
static float urand(void)
{
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
    return (float)((double)(z >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}

static float *fill(long n)
{
    /* exact-size allocations, so that any read past the end is reported */
    float *a = (float *)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
    for (long i = 0; i < n; ++i) a[i] = urand();
    return a;
}

static int failures = 0;

static void expect(int cond, const char *what)
{
    if (!cond) {
        fprintf(stderr, "FAILED: %s\n", what);
        ++failures;
    }
}

static void case_rope(void)
{
    const int n_pos = 37, rd = 16;
    double *fr = (double *)malloc(sizeof(double) * rd / 2);
    orc_yarn_freqs(fr, rd, 1e4, 8.0, 64, 32.0, 1.0);
    float *cs = fill((long)n_pos * rd);
    orc_rope_table_f(cs, n_pos, rd, 1e4, NULL);
    orc_rope_table_f(cs, n_pos, rd, 1e4, fr);
    for (long i = 0; i < (long)n_pos * rd; ++i) expect(isfinite(cs[i]), "rope table finite");
    const int D = 24;
    float *v = fill(5L * D);
    long pos[5] = {0, 1, 7, 36, 1000000};
    orc_rope_apply_f(v, 5, D, rd, 1e4, NULL, pos, +1);
    orc_rope_apply_f(v, 5, D, rd, 1e4, fr, pos, -1);
    free(v);
    free(cs);
    free(fr);
}

static void case_compress(int S, int D, int m, int overlap, int rope_dim, int gate,
                          int bias, int bf16)
{
    const int T = S / m;
    float *x = fill((long)S * D);
    float *g = gate ? fill((long)S * D) : NULL;
    float *sb = bias ? fill((long)(1 + overlap) * m * D) : NULL;
    float *pool = fill((long)T * D);
    expect(orc_compress_f(x, g, sb, pool, S, D, m, overlap, rope_dim, 1.6e5, NULL, 3, bf16) == 0,
           "compress status");
    for (long i = 0; i < (long)T * D; ++i) expect(isfinite(pool[i]), "compress finite");
    free(x);
    free(g);
    free(sb);
    free(pool);
}

static void case_index_topk(int n_rows, int T, int nh, int hd, int m, int k, long t0)
{
    float *q = fill((long)n_rows * nh * hd);
    float *w = fill((long)n_rows * nh);
    float *kI = fill((long)T * hd);
    long *tpos = (long *)malloc(sizeof(long) * (size_t)n_rows);
    for (int r = 0; r < n_rows; ++r) tpos[r] = t0 + 3L * r;
    float *sc = fill((long)n_rows * T);
    int *idx = (int *)malloc(sizeof(int) * (size_t)n_rows * k);
    expect(orc_index_scores(q, w, tpos, n_rows, kI, T, nh, hd, m, sc) == 0, "scores status");
    expect(orc_topk(sc, tpos, n_rows, T, k, m, idx) == 0, "topk status");
    for (int r = 0; r < n_rows; ++r) {
        long R = orc_ready_count(tpos[r], m, T);
        for (int j = 0; j < k; ++j) {
            int e = idx[(long)r * k + j];
            expect(j < R ? (e >= 0 && e < R) : e == -1, "topk entry range");
        }
    }
    free(q);
    free(w);
    free(kI);
    free(tpos);
    free(sc);
    free(idx);
}

static void case_attention(int n_rows, int H, int D, int rope_dim, int latent, int T, int k,
                           int m, int window, int with_idx, int with_sink, long t0)
{
    const int dv = latent ? D - rope_dim : D;
    const long win_pos0 = t0 - window > 0 ? t0 - window : 0;
    const int L_win = (int)(t0 + n_rows - win_pos0);
    float *q = fill((long)n_rows * H * D);
    float *kv = window ? fill((long)L_win * D) : NULL;
    float *pool = fill((long)(T > 0 ? T : 0) * D);
    float *sink = with_sink ? fill(H) : NULL;
    long *tpos = (long *)malloc(sizeof(long) * (size_t)n_rows);
    int *idx = NULL;
    for (int r = 0; r < n_rows; ++r) tpos[r] = t0 + r;
    if (with_idx) {
        idx = (int *)malloc(sizeof(int) * (size_t)n_rows * k);
        for (int r = 0; r < n_rows; ++r) {
            long R = orc_ready_count(tpos[r], m, T);
            for (int j = 0; j < k; ++j) idx[(long)r * k + j] = j < R ? (int)(R - 1 - j) : -1;
        }
    }
    float *out = fill((long)n_rows * H * dv);
    expect(orc_attention_f(q, tpos, n_rows, H, D, dv, kv, win_pos0, L_win, window, pool, T,
                           idx, with_idx ? k : 0, m, sink, rope_dim, 1.6e5, NULL,
                           1.0f / sqrtf((float)D), out) == 0,
           "attention status");
    for (long i = 0; i < (long)n_rows * H * dv; ++i) expect(isfinite(out[i]), "attention finite");
    free(q);
    free(kv);
    free(pool);
    free(sink);
    free(tpos);
    free(idx);
    free(out);
}

int main(void)
{
#ifdef ORC_SANITIZE_SELFTEST
    {
        /* the harness itself: a read one element past an allocation must be reported */
        float *a = fill(4);
        volatile float v = a[4];
        (void)v;
        free(a);
    }
#endif
    case_rope();
    /* compressor: overlap windows (CSA), plain windows (HCA), token copies, ragged, T = 0 */
    case_compress(4 * 9 + 3, 32, 4, 1, 8, 1, 0, 1);
    case_compress(4 * 9, 32, 4, 1, 0, 1, 1, 0);
    case_compress(16 * 3 + 5, 24, 16, 0, 8, 1, 1, 1);
    case_compress(11, 16, 1, 0, 16, 0, 0, 0);
    case_compress(3, 16, 4, 1, 8, 1, 1, 1);
    case_compress(0, 16, 4, 0, 0, 0, 0, 0);
    /* indexer and top-k: rows before any entry is ready, R < k, R > k */
    case_index_topk(7, 20, 3, 8, 4, 5, 0);
    case_index_topk(5, 33, 2, 16, 1, 8, 10);
    case_index_topk(3, 0, 2, 8, 4, 4, 5);
    /* attention: CSA (idx + window + sink), latent output, HCA dense, DSA (no window),
       a window that starts at token 0, a row that sees nothing without a sink */
    case_attention(4, 3, 32, 8, 0, 9, 4, 4, 6, 1, 1, 40);
    case_attention(3, 2, 40, 8, 1, 12, 5, 4, 4, 1, 1, 47);
    case_attention(3, 2, 32, 8, 0, 2, 0, 16, 8, 0, 1, 40);
    case_attention(3, 2, 32, 8, 1, 30, 6, 1, 0, 1, 0, 20);
    case_attention(2, 2, 16, 4, 0, 3, 2, 4, 5, 1, 1, 2);
    case_attention(1, 1, 16, 4, 0, 4, 2, 4, 0, 1, 0, 0);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer run: all cases clean\n");
    return 0;
}
