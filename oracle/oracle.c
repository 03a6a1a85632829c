/*
 * oracle.c -- plain fp64 CPU oracle for the forward pass of a stack of
 * post-LN transformer encoder layers with causal and key-padding masking.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
 * statement of what the GPU library computes.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no source, header or build step with the GPU library, and the GPU library
 * never calls it.
 *
 * What it follows (the pages are three project write-ups on one subject):
 *  - "KernelForge", "Why it matters": the workload is a small stack
 *    (2-4 layers) of encoder layers run with causal masking and a padding
 *    mask together; "What we built": causal and key-padding masks are
 *    applied in the same attention.
 *  - "Hyper-optimized megakernel-hybrid transformer inference",
 *    "Challenges": the layer is the PyTorch reference encoder layer, whose
 *    LayerNorm is the textbook mean/variance normalisation.
 *  - "KernelForge", "How the LLM is used": GELU uses the exact error
 *    function, never a polynomial approximation of erf.
 *  - "KernelForge", "Results": correctness at 100k tokens was checked
 *    against a streamed exact reference, i.e. one that never holds the
 *    L x L score matrix.  This oracle streams in the same sense: it keeps
 *    one row of scores (length <= L) per thread.
 *
 * Each layer computes (x is one token row, d = d_model, H heads,
 * dh = d / H, f = FFN width):
 *     qkv = x W_qkv^T + b_qkv                 rows of W_qkv: q | k | v,
 *                                             head h owns columns h*dh..
 *     s_j = (q_h . k_h[j]) / sqrt(dh)         for allowed keys j
 *     a_h = sum_j softmax(s)_j v_h[j]
 *     x1  = LN(x + a W_o^T + b_o)
 *     x   = LN(x1 + GELU(x1 W_1^T + b_1) W_2^T + b_2)
 * with key j allowed for query i of sequence b iff j <= i and j < len_b.
 * Every query row, padded ones (i >= len_b) included, is computed by this
 * same formula.  LN(z) = (z - mean) / sqrt(var + eps) * gamma + beta with
 * the biased (1/d) variance.  GELU(h) = h/2 * (1 + erf(h / sqrt(2))).
 *
 * All arithmetic is IEEE double with libm exp/erf/sqrt; compile with
 * -O2 -fno-fast-math -ffp-contract=off.  Every output element is produced
 * by exactly one thread in a fixed loop order, so the result does not
 * depend on the thread count.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

typedef struct {
    const double *w_qkv, *b_qkv; /* [3d, d], [3d] */
    const double *w_o, *b_o;     /* [d, d],  [d]  */
    const double *ln1_g, *ln1_b; /* [d] */
    const double *w_1, *b_1;     /* [f, d],  [f]  */
    const double *w_2, *b_2;     /* [d, f],  [d]  */
    const double *ln2_g, *ln2_b; /* [d] */
} orc_layer;

void orc_set_threads(int n) { if (n > 0) omp_set_num_threads(n); }
int orc_max_threads(void) { return omp_get_max_threads(); }

/* Y[t, o] = b[o] + sum_{c ascending} A[t, c] * W[o, c]   (nn.Linear). */
void orc_linear(long T, int n_in, int n_out, const double *A, const double *W,
                const double *b, double *Y)
{
    long t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < T; t++) {
        const double *a = A + t * n_in;
        double *y = Y + t * n_out;
        for (int o = 0; o < n_out; o++) {
            const double *w = W + (long)o * n_in;
            double acc = 0.0;
            for (int c = 0; c < n_in; c++) acc += a[c] * w[c];
            y[o] = acc + (b ? b[o] : 0.0);
        }
    }
}

/* Masked multi-head attention over packed projections.
 * qkv: [B, L, 3d] (q | k | v per row), o: [B, L, d] (heads concatenated).
 * Returns 0, or -1 if some len_b lies outside [1, L]. */
int orc_attention(int B, int L, int H, int d, const int *lens,
                  const double *qkv, double *o)
{
    for (int b = 0; b < B; b++)
        if (lens[b] < 1 || lens[b] > L) return -1;
    const int dh = d / H;
    const double rs = sqrt((double)dh);
    const long rows = (long)B * H * L;
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)L);
        double *acc = (double *)malloc(sizeof(double) * (size_t)dh);
        if (!s || !acc) {
#pragma omp atomic write
            bad = 1;
        }
        long r;
#pragma omp for schedule(dynamic, 8)
        for (r = 0; r < rows; r++) {
            if (!s || !acc) continue;
            const int i = (int)(r % L);
            const int h = (int)((r / L) % H);
            const int b = (int)(r / ((long)L * H));
            const int last = (i < lens[b] - 1) ? i : lens[b] - 1; /* keys 0..last */
            const double *q = qkv + ((long)b * L + i) * 3 * d + (long)h * dh;
            double m = -INFINITY;
            for (int j = 0; j <= last; j++) {
                const double *k = qkv + ((long)b * L + j) * 3 * d + d + (long)h * dh;
                double dot = 0.0;
                for (int t = 0; t < dh; t++) dot += q[t] * k[t];
                s[j] = dot / rs;
                if (s[j] > m) m = s[j];
            }
            double l = 0.0;
            for (int j = 0; j <= last; j++) {
                s[j] = exp(s[j] - m);
                l += s[j];
            }
            for (int t = 0; t < dh; t++) acc[t] = 0.0;
            for (int j = 0; j <= last; j++) {
                const double *v = qkv + ((long)b * L + j) * 3 * d + 2 * d + (long)h * dh;
                for (int t = 0; t < dh; t++) acc[t] += s[j] * v[t];
            }
            double *out = o + ((long)b * L + i) * d + (long)h * dh;
            for (int t = 0; t < dh; t++) out[t] = acc[t] / l;
        }
        free(s);
        free(acc);
    }
    return bad ? -2 : 0;
}

/* Row-wise LayerNorm, two passes: mean, then biased variance. */
void orc_layernorm(long T, int d, const double *z, const double *g,
                   const double *b, double eps, double *out)
{
    long t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < T; t++) {
        const double *zr = z + t * d;
        double *yr = out + t * d;
        double mean = 0.0;
        for (int c = 0; c < d; c++) mean += zr[c];
        mean /= d;
        double var = 0.0;
        for (int c = 0; c < d; c++) var += (zr[c] - mean) * (zr[c] - mean);
        var /= d;
        const double inv = 1.0 / sqrt(var + eps);
        for (int c = 0; c < d; c++) yr[c] = (zr[c] - mean) * inv * g[c] + b[c];
    }
}

/* GELU with the exact error function. */
void orc_gelu(long n, const double *h, double *g)
{
    long i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; i++) g[i] = 0.5 * h[i] * (1.0 + erf(h[i] / sqrt(2.0)));
}

/* Attention sub-block tail: X1 = LN(X + o W_o^T + b_o).  z is scratch [T, d]. */
void orc_out_ln(long T, int d, const double *X, const double *o,
                const double *w_o, const double *b_o, const double *g,
                const double *beta, double eps, double *z, double *X1)
{
    orc_linear(T, d, d, o, w_o, b_o, z);
    long i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < T * d; i++) z[i] = X[i] + z[i];
    orc_layernorm(T, d, z, g, beta, eps, X1);
}

/* FFN sub-block: X2 = LN(X1 + GELU(X1 W_1^T + b_1) W_2^T + b_2).
 * hbuf is scratch [T, f], z is scratch [T, d]. */
void orc_ffn_ln(long T, int d, int f, const double *X1, const double *w_1,
                const double *b_1, const double *w_2, const double *b_2,
                const double *g, const double *beta, double eps, double *hbuf,
                double *z, double *X2)
{
    orc_linear(T, d, f, X1, w_1, b_1, hbuf);
    orc_gelu(T * f, hbuf, hbuf);
    orc_linear(T, f, d, hbuf, w_2, b_2, z);
    long i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < T * d; i++) z[i] = X1[i] + z[i];
    orc_layernorm(T, d, z, g, beta, eps, X2);
}

/* Whole stack.  x, y: [B, L, d].  Returns 0, -1 on a bad length or shape,
 * -2 when scratch memory cannot be had. */
int orc_forward(int n_layers, int d, int H, int f, int B, int L, double eps,
                const orc_layer *layers, const double *x, const int *lens,
                double *y)
{
    if (n_layers < 1 || d < 1 || H < 1 || d % H != 0 || f < 1 || B < 1 || L < 1)
        return -1;
    const long T = (long)B * L;
    double *X = (double *)malloc(sizeof(double) * (size_t)(T * d));
    double *X1 = (double *)malloc(sizeof(double) * (size_t)(T * d));
    double *z = (double *)malloc(sizeof(double) * (size_t)(T * d));
    double *o = (double *)malloc(sizeof(double) * (size_t)(T * d));
    double *qkv = (double *)malloc(sizeof(double) * (size_t)(T * 3 * d));
    double *hb = (double *)malloc(sizeof(double) * (size_t)(T * f));
    int rc = 0;
    if (!X || !X1 || !z || !o || !qkv || !hb) { rc = -2; goto done; }
    memcpy(X, x, sizeof(double) * (size_t)(T * d));
    for (int l = 0; l < n_layers; l++) {
        const orc_layer *p = &layers[l];
        orc_linear(T, d, 3 * d, X, p->w_qkv, p->b_qkv, qkv);
        rc = orc_attention(B, L, H, d, lens, qkv, o);
        if (rc) goto done;
        orc_out_ln(T, d, X, o, p->w_o, p->b_o, p->ln1_g, p->ln1_b, eps, z, X1);
        orc_ffn_ln(T, d, f, X1, p->w_1, p->b_1, p->w_2, p->b_2, p->ln2_g,
                   p->ln2_b, eps, hb, z, X);
    }
    memcpy(y, X, sizeof(double) * (size_t)(T * d));
done:
    free(X); free(X1); free(z); free(o); free(qkv); free(hb);
    return rc;
}
