/*
 * oracle.c -- plain, slow, fp64 CPU oracle of the windowed atom-attention
 * block (encoder and decoder stage, AF3 and ESMFold2 style).
 *
 * TEST INFRASTRUCTURE ONLY: used by the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark, never by the product library. It shares
 * no code with the HIP implementation.
 *
 * Sources (all "Required behavior" unless stated):
 *   [W]  windowed_atom_attention -- Local atom attention, encoder pooling and
 *        decoder skip/readout
 *   [AF] AlphaFold 3 Atom Attention Encoder (also its Worked example)
 *   [EF] ESMFold 2 Atom Attention Encoder   (also its Worked example)
 *
 * The method is an exact computation, so this file is its plain definition:
 * every sum is a straight loop in index order, in double precision, on the
 * stored input values. Work is split over atoms with OpenMP; that changes no
 * arithmetic. Parity pins for every step live in tests/ (closed forms from
 * the two worked examples, invariants, brute force and special cases that
 * reduce to library routines).
 */
#include "oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Scalar and vector primitives                                        */
/* ------------------------------------------------------------------ */

/* Logistic function. [W]/[EF] define sigmoid(z) = 1/(1+e^-z); for z < 0 the
 * algebraically equal e^z/(1+e^z) is used so that very negative inputs give
 * their (possibly subnormal) value instead of 1/inf; [W] asks that such
 * tails are kept. */
static double sigmoid(double z)
{
    if (z >= 0.0)
        return 1.0 / (1.0 + exp(-z));
    double e = exp(z);
    return e / (1.0 + e);
}

/* SiLU(z) = z * sigmoid(z)  ([EF]). */
static double silu(double z) { return z * sigmoid(z); }

/* Population LayerNorm without affine terms, eps inside the root ([W], the
 * AF3 style bullet; [AF]). */
static void layer_norm(const double *v, int64_t n, double eps, double *out)
{
    double mean = 0.0;
    for (int64_t i = 0; i < n; ++i)
        mean += v[i];
    mean /= (double)n;
    double var = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double d = v[i] - mean;
        var += d * d;
    }
    var /= (double)n;
    double r = 1.0 / sqrt(var + eps);
    for (int64_t i = 0; i < n; ++i)
        out[i] = (v[i] - mean) * r;
}

/* RMS normalisation without affine terms: v / sqrt(mean(v^2) + eps)
 * ([W] ESMFold2 bullets; [EF]). */
static void rms_norm(const double *v, int64_t n, double eps, double *out)
{
    double ms = 0.0;
    for (int64_t i = 0; i < n; ++i)
        ms += v[i] * v[i];
    ms /= (double)n;
    double r = 1.0 / sqrt(ms + eps);
    for (int64_t i = 0; i < n; ++i)
        out[i] = v[i] * r;
}

/* y[o] = sum_i x[i] * W[i][o]; W has nin rows of stride ldw. Parameters are
 * stored [in][out] so that a projection reads "x @ W" as on the pages. */
static void vec_mat(const double *x, int64_t nin, const double *w, int64_t ldw,
                    int64_t nout, double *y)
{
    for (int64_t o = 0; o < nout; ++o) {
        double acc = 0.0;
        for (int64_t i = 0; i < nin; ++i)
            acc += x[i] * w[i * ldw + o];
        y[o] = acc;
    }
}

/* ------------------------------------------------------------------ */
/* Conditioning                                                        */
/* ------------------------------------------------------------------ */

/* AF3 adaptive-norm parameters of stage j (0 query, 1 key/value,
 * 2 transition): with chat = LN(c) * cond_scale[j],
 *   sigma_j = sigmoid(chat @ w_scale[j] + b_scale[j]),  mu_j = chat @ w_shift[j].
 * ([W] AF3 style bullet; [AF]) */
static void af3_adaptive_params(const orc_dims *d, const orc_params *p,
                                const double *c, double eps, int j,
                                double *sigma, double *mu, double *tmp_s)
{
    const int64_t S = d->S, C = d->C;
    layer_norm(c, S, eps, tmp_s);
    for (int64_t s = 0; s < S; ++s)
        tmp_s[s] *= p->cond_scale[j * S + s];
    vec_mat(tmp_s, S, p->w_scale + j * S * C, C, C, sigma);
    for (int64_t i = 0; i < C; ++i)
        sigma[i] = sigmoid(sigma[i] + p->b_scale[j * C + i]);
    vec_mat(tmp_s, S, p->w_shift + j * S * C, C, C, mu);
}

/* A_j(z) = LN(z) * sigma_j + mu_j  ([W] AF3 style bullet; [AF]). */
static void af3_adaptive_norm(const double *z, int64_t C, double eps,
                              const double *sigma, const double *mu,
                              double *out)
{
    layer_norm(z, C, eps, out);
    for (int64_t i = 0; i < C; ++i)
        out[i] = out[i] * sigma[i] + mu[i];
}

/* AF3 residual gate j (0 attention, 1 transition) from the raw (sanitised,
 * not normalised) condition: sigmoid(c @ w_residual_gate[j] +
 * b_residual_gate[j]). ([W]; [AF]) */
static void af3_residual_gate(const orc_dims *d, const orc_params *p,
                              const double *c, int j, double *out)
{
    const int64_t S = d->S, C = d->C;
    vec_mat(c, S, p->w_residual_gate + j * S * C, C, C, out);
    for (int64_t i = 0; i < C; ++i)
        out[i] = sigmoid(out[i] + p->b_residual_gate[j * C + i]);
}

/* ESMFold2 modulation: SiLU(c) contracted with w_mod[S,6,C] gives six
 * vectors in the order attention shift, scale, gate, transition shift,
 * scale, gate. out is [6][C]. ([W] ESMFold2 bullets; [EF]) */
static void esm_modulation(const orc_dims *d, const orc_params *p,
                           const double *c, double *out, double *tmp_s)
{
    const int64_t S = d->S, C = d->C;
    for (int64_t s = 0; s < S; ++s)
        tmp_s[s] = silu(c[s]);
    for (int i = 0; i < 6; ++i)
        vec_mat(tmp_s, S, p->w_mod + (int64_t)i * C, 6 * C, C, out + i * C);
}

/* ESMFold2 modulated norm: RMS(x) * (1 + scale) + shift. */
static void esm_modulated_norm(const double *x, int64_t C, double eps,
                               const double *shift, const double *scale,
                               double *out)
{
    rms_norm(x, C, eps, out);
    for (int64_t i = 0; i < C; ++i)
        out[i] = out[i] * (1.0 + scale[i]) + shift[i];
}

/* Half-split rotary: q * cos + rotate_half(q) * sin with
 * rotate_half([q1, q2]) = [-q2, q1]  ([W], [EF]). D is even. */
static void rotary(double *q, int64_t D, const double *cs, const double *sn,
                   double *tmp)
{
    const int64_t h = D / 2;
    for (int64_t i = 0; i < D; ++i) {
        double rot = (i < h) ? -q[i + h] : q[i - h];
        tmp[i] = q[i] * cs[i] + rot * sn[i];
    }
    memcpy(q, tmp, (size_t)D * sizeof(double));
}

/* ------------------------------------------------------------------ */
/* Masks                                                               */
/* ------------------------------------------------------------------ */

/* Atom usability: valid, atom_to_token in [0,T), and that token valid
 * ([W]; [AF]; [EF]). token_valid is read only for an in-range token. */
static int atom_usable(const orc_dims *d, const orc_inputs *in, int64_t b,
                       int64_t a)
{
    const int64_t n = b * d->A + a;
    if (!in->valid[n])
        return 0;
    int64_t t = in->atom_to_token[n];
    if (t < 0 || t >= d->T)
        return 0;
    return in->token_valid[b * d->T + t] ? 1 : 0;
}

/* Slot permission: key id in [0,A), query and key usable, window_mask True,
 * and |key - query| <= radius when radius >= 0 (an index window). ([W]) */
static int slot_allowed(const orc_dims *d, const uint8_t *usable,
                        const int64_t *key_index, const uint8_t *window_mask,
                        int64_t radius, int64_t b, int64_t a, int64_t k)
{
    const int64_t A = d->A, K = d->K;
    if (!usable[b * A + a])
        return 0;
    int64_t j = key_index[(b * A + a) * K + k];
    if (j < 0 || j >= A)
        return 0;
    if (!usable[b * A + j])
        return 0;
    if (!window_mask[(b * A + a) * K + k])
        return 0;
    if (radius >= 0) {
        int64_t dist = j > a ? j - a : a - j;
        if (dist > radius)
            return 0;
    }
    return 1;
}

/* ------------------------------------------------------------------ */
/* Slot attention for one query atom                                   */
/* ------------------------------------------------------------------ */

/* For query (b,a): allowed slots, logits Q.K/sqrt(D) (+ AF3 pair bias
 * (LN(pair) * pair_scale) @ w_pair, one value per head), masked softmax over
 * the allowed slots (each slot its own term, duplicates included; a row with
 * no allowed slot gets all-zero weights), and o = sum_k w_k V[key_k].
 * ([W]; [AF]; [EF]) */
static void slot_attention_row(const orc_dims *d, int style, double eps,
                               int64_t radius, const uint8_t *usable,
                               const double *q, const double *k,
                               const double *v, const int64_t *key_index,
                               const uint8_t *window_mask, const double *pair,
                               const double *pair_scale, const double *w_pair,
                               int64_t b, int64_t a, double *attention,
                               double *o, uint8_t *allowed_out,
                               double *scratch)
{
    const int64_t A = d->A, K = d->K, H = d->H, D = d->D, V = d->V;
    const int64_t HD = H * D;
    const int64_t n = b * A + a;
    /* scratch layout: allowed flags [K], bias [K][H], logits [K], pair LN [V] */
    double *allow = scratch;
    double *bias = allow + K;
    double *logit = bias + K * H;
    double *pn = logit + K;

    for (int64_t s = 0; s < K; ++s) {
        int ok = slot_allowed(d, usable, key_index, window_mask, radius, b, a, s);
        allow[s] = ok ? 1.0 : 0.0;
        if (allowed_out)
            allowed_out[n * K + s] = (uint8_t)ok;
        for (int64_t h = 0; h < H; ++h)
            bias[s * H + h] = 0.0;
        if (ok && style == ORC_AF3) {
            layer_norm(pair + (n * K + s) * V, V, eps, pn);
            for (int64_t x = 0; x < V; ++x)
                pn[x] *= pair_scale[x];
            vec_mat(pn, V, w_pair, H, H, bias + s * H);
        }
    }

    const double inv_sqrt_d = 1.0 / sqrt((double)D);
    for (int64_t h = 0; h < H; ++h) {
        int any = 0;
        double mx = -INFINITY;
        for (int64_t s = 0; s < K; ++s) {
            if (allow[s] == 0.0)
                continue;
            int64_t j = key_index[n * K + s];
            const double *qv = q + n * HD + h * D;
            const double *kv = k + (b * A + j) * HD + h * D;
            double dot = 0.0;
            for (int64_t e = 0; e < D; ++e)
                dot += qv[e] * kv[e];
            logit[s] = dot * inv_sqrt_d + bias[s * H + h];
            if (!any || logit[s] > mx)
                mx = logit[s];
            any = 1;
        }
        double *orow = o + n * HD + h * D;
        for (int64_t e = 0; e < D; ++e)
            orow[e] = 0.0;
        double *arow = attention + ((b * H + h) * A + a) * K;
        if (!any) {
            for (int64_t s = 0; s < K; ++s)
                arow[s] = 0.0;
            continue;
        }
        double den = 0.0;
        for (int64_t s = 0; s < K; ++s)
            if (allow[s] != 0.0)
                den += exp(logit[s] - mx);
        for (int64_t s = 0; s < K; ++s) {
            if (allow[s] == 0.0) {
                arow[s] = 0.0;
                continue;
            }
            double w = exp(logit[s] - mx) / den;
            arow[s] = w;
            int64_t j = key_index[n * K + s];
            const double *vv = v + (b * A + j) * HD + h * D;
            for (int64_t e = 0; e < D; ++e)
                orow[e] += w * vv[e];
        }
    }
}

static size_t slot_scratch_len(const orc_dims *d)
{
    return (size_t)(d->K + d->K * d->H + d->K + d->V + 8);
}

/* ------------------------------------------------------------------ */
/* Argument checks                                                     */
/* ------------------------------------------------------------------ */

static int dims_ok(const orc_dims *d)
{
    return d && d->B >= 1 && d->A >= 1 && d->T >= 1 && d->K >= 1 &&
           d->C >= 1 && d->S >= 1 && d->H >= 1 && d->D >= 1 && d->V >= 1 &&
           d->M >= 1 && d->U >= 1;
}

int orc_threads(int nthreads)
{
    return nthreads > 0 ? nthreads : omp_get_max_threads();
}

int orc_slot_attention(const orc_dims *dims, int style, double eps,
                       int64_t radius, const uint8_t *usable,
                       const double *q, const double *k, const double *v,
                       const int64_t *key_index, const uint8_t *window_mask,
                       const double *pair, const double *pair_scale,
                       const double *w_pair, double *attention, double *o,
                       uint8_t *allowed, int nthreads)
{
    if (!dims_ok(dims) || (style != ORC_AF3 && style != ORC_ESMFOLD2) ||
        !(eps > 0.0) || !isfinite(eps) || radius < -1 || !usable || !q ||
        !k || !v || !key_index || !window_mask || !attention || !o)
        return -1;
    if (style == ORC_AF3 && (!pair || !pair_scale || !w_pair))
        return -1;
    const int64_t N = dims->B * dims->A;
    const int nt = orc_threads(nthreads);
#pragma omp parallel num_threads(nt)
    {
        double *scratch = (double *)malloc(slot_scratch_len(dims) * sizeof(double));
#pragma omp for schedule(dynamic, 16)
        for (int64_t n = 0; n < N; ++n)
            slot_attention_row(dims, style, eps, radius, usable, q, k, v,
                               key_index, window_mask, pair, pair_scale,
                               w_pair, n / dims->A, n % dims->A, attention, o,
                               allowed, scratch);
        free(scratch);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Whole block                                                         */
/* ------------------------------------------------------------------ */

int orc_block(const orc_dims *d, int style, int stage, double eps,
              int64_t radius, const orc_inputs *in, const orc_params *p,
              const uint8_t *select, orc_outputs *out, int nthreads)
{
    if (!dims_ok(d) || !in || !p || !out)
        return -1;
    if (style != ORC_AF3 && style != ORC_ESMFOLD2)
        return -1;
    if (stage != ORC_ENCODER && stage != ORC_DECODER)
        return -1;
    if (!(eps > 0.0) || !isfinite(eps) || radius < -1)
        return -1;
    if (style == ORC_ESMFOLD2 && (d->D % 2) != 0)
        return -1;
    if (!in->atom || !in->condition || !in->valid || !in->token_valid ||
        !in->window_mask || !in->atom_to_token || !in->key_index)
        return -1;
    if (!p->w_q || !p->w_k || !p->w_v || !p->w_value_gate ||
        !p->w_attention_out || !p->w_ff_gate || !p->w_ff_up || !p->w_ff_out)
        return -1;
    if (style == ORC_AF3 &&
        (!in->pair || !p->cond_scale || !p->w_scale || !p->b_scale ||
         !p->w_shift || !p->w_residual_gate || !p->b_residual_gate ||
         !p->b_q || !p->pair_scale || !p->w_pair))
        return -1;
    if (style == ORC_ESMFOLD2 && (!in->rope_cos || !in->rope_sin || !p->w_mod))
        return -1;
    if (stage == ORC_ENCODER && (!p->w_pool || !out->token_output))
        return -1;
    if (stage == ORC_DECODER &&
        (!in->token || !p->w_token || !p->readout_scale || !p->w_readout ||
         !out->position_update || (style == ORC_ESMFOLD2 && !p->readout_bias)))
        return -1;
    if (!out->hidden || !out->attention)
        return -1;

    const int64_t B = d->B, A = d->A, T = d->T, K = d->K, C = d->C, S = d->S;
    const int64_t H = d->H, D = d->D, M = d->M, U = d->U;
    const int64_t HD = H * D, N = B * A;
    const int nt = orc_threads(nthreads);

    uint8_t *usable = (uint8_t *)calloc((size_t)N, 1);
    uint8_t *need_out = (uint8_t *)calloc((size_t)N, 1);
    uint8_t *need_proj = (uint8_t *)calloc((size_t)N, 1);
    uint8_t *tok_want = (uint8_t *)calloc((size_t)(B * T), 1);
    double *x0 = (double *)calloc((size_t)(N * C), sizeof(double));
    double *cc = (double *)calloc((size_t)(N * S), sizeof(double));
    double *qi = (double *)calloc((size_t)(N * C), sizeof(double));
    double *kvi = (double *)calloc((size_t)(N * C), sizeof(double));
    double *Q = (double *)calloc((size_t)(N * HD), sizeof(double));
    double *Kp = (double *)calloc((size_t)(N * HD), sizeof(double));
    double *Vp = (double *)calloc((size_t)(N * HD), sizeof(double));
    double *G = (double *)calloc((size_t)(N * HD), sizeof(double));
    double *O = (double *)calloc((size_t)(N * HD), sizeof(double));
    double *X1 = (double *)calloc((size_t)(N * C), sizeof(double));
    if (!usable || !need_out || !need_proj || !tok_want || !x0 || !cc ||
        !qi || !kvi || !Q || !Kp || !Vp || !G || !O || !X1) {
        free(usable); free(need_out); free(need_proj); free(tok_want);
        free(x0); free(cc); free(qi); free(kvi); free(Q); free(Kp);
        free(Vp); free(G); free(O); free(X1);
        return -2;
    }

    /* Step 1: usability of every atom. */
    for (int64_t n = 0; n < N; ++n)
        usable[n] = (uint8_t)atom_usable(d, in, n / A, n % A);

    /* Which rows to compute. For the encoder a chosen usable atom pulls in
     * every usable atom of its token so that the token mean is complete. */
    for (int64_t n = 0; n < N; ++n)
        need_out[n] = select ? (select[n] != 0) : 1;
    if (stage == ORC_ENCODER && select) {
        for (int64_t n = 0; n < N; ++n)
            if (need_out[n] && usable[n])
                tok_want[(n / A) * T + in->atom_to_token[n]] = 1;
        for (int64_t n = 0; n < N; ++n)
            if (usable[n] && tok_want[(n / A) * T + in->atom_to_token[n]])
                need_out[n] = 1;
    }
    for (int64_t n = 0; n < N; ++n) {
        if (!need_out[n])
            continue;
        need_proj[n] = 1;
        const int64_t b = n / A;
        for (int64_t s = 0; s < K; ++s) {
            int64_t j = in->key_index[n * K + s];
            if (j >= 0 && j < A)
                need_proj[b * A + j] = 1;
        }
    }

    /* Steps 2-6, per atom: sanitise, decoder entry, conditioning, modulated
     * norms, Q/K/V/value-gate projections, ESMFold2 head RMS + rotary. */
#pragma omp parallel num_threads(nt)
    {
        double *tmp_s = (double *)malloc((size_t)(S + 8) * sizeof(double));
        double *sig = (double *)malloc((size_t)(C + 8) * sizeof(double));
        double *mu = (double *)malloc((size_t)(C + 8) * sizeof(double));
        double *mods = (double *)malloc((size_t)(6 * C + 8) * sizeof(double));
        double *tmp_d = (double *)malloc((size_t)(D + 8) * sizeof(double));
#pragma omp for schedule(dynamic, 16)
        for (int64_t n = 0; n < N; ++n) {
            if (!need_proj[n])
                continue;
            const int64_t b = n / A;
            double *x = x0 + n * C;
            double *c = cc + n * S;
            /* Unusable atoms start from zeros: their payload (maybe NaN/Inf)
             * is never read into arithmetic ([W] sanitising bullet). */
            if (usable[n]) {
                for (int64_t i = 0; i < C; ++i)
                    x[i] = in->atom[n * C + i];
                for (int64_t s = 0; s < S; ++s)
                    c[s] = in->condition[n * S + s];
                if (stage == ORC_DECODER) {
                    /* Decoder entry: skip + gather(token @ w_token), bias-free. */
                    const int64_t t = in->atom_to_token[n];
                    const double *tok = in->token + (b * T + t) * d->U;
                    for (int64_t i = 0; i < C; ++i) {
                        double acc = 0.0;
                        for (int64_t u = 0; u < d->U; ++u)
                            acc += tok[u] * p->w_token[u * C + i];
                        x[i] += acc;
                    }
                }
            }
            double *qin = qi + n * C;
            double *kvin = kvi + n * C;
            if (style == ORC_AF3) {
                af3_adaptive_params(d, p, c, eps, 0, sig, mu, tmp_s);
                af3_adaptive_norm(x, C, eps, sig, mu, qin);
                af3_adaptive_params(d, p, c, eps, 1, sig, mu, tmp_s);
                af3_adaptive_norm(x, C, eps, sig, mu, kvin);
            } else {
                esm_modulation(d, p, c, mods, tmp_s);
                esm_modulated_norm(x, C, eps, mods + 0 * C, mods + 1 * C, qin);
                memcpy(kvin, qin, (size_t)C * sizeof(double));
            }
            vec_mat(qin, C, p->w_q, HD, HD, Q + n * HD);
            if (style == ORC_AF3)
                for (int64_t i = 0; i < HD; ++i)
                    Q[n * HD + i] += p->b_q[i];
            vec_mat(kvin, C, p->w_k, HD, HD, Kp + n * HD);
            vec_mat(kvin, C, p->w_v, HD, HD, Vp + n * HD);
            vec_mat(qin, C, p->w_value_gate, HD, HD, G + n * HD);
            for (int64_t i = 0; i < HD; ++i)
                G[n * HD + i] = sigmoid(G[n * HD + i]);
            if (style == ORC_ESMFOLD2) {
                const double *cs = in->rope_cos + n * D;
                const double *sn = in->rope_sin + n * D;
                for (int64_t h = 0; h < H; ++h) {
                    double *qh = Q + n * HD + h * D;
                    double *kh = Kp + n * HD + h * D;
                    rms_norm(qh, D, eps, qh);
                    rms_norm(kh, D, eps, kh);
                    rotary(qh, D, cs, sn, tmp_d);
                    rotary(kh, D, cs, sn, tmp_d);
                }
            }
        }
        free(tmp_s); free(sig); free(mu); free(mods); free(tmp_d);
    }

    /* Steps 7-8: masked slot softmax and value mix, for the output rows. */
#pragma omp parallel num_threads(nt)
    {
        double *scratch = (double *)malloc(slot_scratch_len(d) * sizeof(double));
#pragma omp for schedule(dynamic, 16)
        for (int64_t n = 0; n < N; ++n) {
            if (!need_out[n])
                continue;
            slot_attention_row(d, style, eps, radius, usable, Q, Kp, Vp,
                               in->key_index, in->window_mask, in->pair,
                               p->pair_scale, p->w_pair, n / A, n % A,
                               out->attention, O, out->allowed, scratch);
        }
        free(scratch);
    }

    /* Steps 9-11 per atom: value gate, output projection, gated attention
     * residual, modulated transition, gated transition residual, mask, and
     * the decoder readout. */
#pragma omp parallel num_threads(nt)
    {
        double *tmp_s = (double *)malloc((size_t)(S + 8) * sizeof(double));
        double *sig = (double *)malloc((size_t)(C + 8) * sizeof(double));
        double *mu = (double *)malloc((size_t)(C + 8) * sizeof(double));
        double *gate = (double *)malloc((size_t)(C + 8) * sizeof(double));
        double *mods = (double *)malloc((size_t)(6 * C + 8) * sizeof(double));
        double *ug = (double *)malloc((size_t)(HD + 8) * sizeof(double));
        double *u = (double *)malloc((size_t)(C + 8) * sizeof(double));
        double *z = (double *)malloc((size_t)(C + 8) * sizeof(double));
        double *hg = (double *)malloc((size_t)(M + 8) * sizeof(double));
        double *hu = (double *)malloc((size_t)(M + 8) * sizeof(double));
        double *tr = (double *)malloc((size_t)(C + 8) * sizeof(double));
        double *ln = (double *)malloc((size_t)(C + 8) * sizeof(double));
#pragma omp for schedule(dynamic, 16)
        for (int64_t n = 0; n < N; ++n) {
            if (!need_out[n])
                continue;
            const double *x = x0 + n * C;
            const double *c = cc + n * S;
            double *x1 = X1 + n * C;
            /* value gate per channel, flattened head-major (h*D + d) */
            for (int64_t i = 0; i < HD; ++i)
                ug[i] = O[n * HD + i] * G[n * HD + i];
            vec_mat(ug, HD, p->w_attention_out, C, C, u);
            if (style == ORC_AF3) {
                af3_residual_gate(d, p, c, 0, gate);
            } else {
                esm_modulation(d, p, c, mods, tmp_s);
                memcpy(gate, mods + 2 * C, (size_t)C * sizeof(double));
            }
            for (int64_t i = 0; i < C; ++i)
                x1[i] = x[i] + gate[i] * u[i];
            /* transition on the NEW state */
            if (style == ORC_AF3) {
                af3_adaptive_params(d, p, c, eps, 2, sig, mu, tmp_s);
                af3_adaptive_norm(x1, C, eps, sig, mu, z);
            } else {
                esm_modulated_norm(x1, C, eps, mods + 3 * C, mods + 4 * C, z);
            }
            vec_mat(z, C, p->w_ff_gate, M, M, hg);
            vec_mat(z, C, p->w_ff_up, M, M, hu);
            for (int64_t i = 0; i < M; ++i)
                hg[i] = silu(hg[i]) * hu[i];
            vec_mat(hg, M, p->w_ff_out, C, C, tr);
            if (style == ORC_AF3)
                af3_residual_gate(d, p, c, 1, gate);
            else
                memcpy(gate, mods + 5 * C, (size_t)C * sizeof(double));
            double *hid = out->hidden + n * C;
            for (int64_t i = 0; i < C; ++i)
                hid[i] = usable[n] ? x1[i] + gate[i] * tr[i] : 0.0;
            if (stage == ORC_DECODER) {
                /* Readout: (LN(hidden) * readout_scale [+ readout_bias]) @
                 * w_readout, masked; a coordinate update. */
                double *pu = out->position_update + n * 3;
                if (!usable[n]) {
                    pu[0] = pu[1] = pu[2] = 0.0;
                } else {
                    layer_norm(hid, C, eps, ln);
                    for (int64_t i = 0; i < C; ++i) {
                        ln[i] *= p->readout_scale[i];
                        if (style == ORC_ESMFOLD2)
                            ln[i] += p->readout_bias[i];
                    }
                    vec_mat(ln, C, p->w_readout, 3, 3, pu);
                }
            }
        }
        free(tmp_s); free(sig); free(mu); free(gate); free(mods); free(ug);
        free(u); free(z); free(hg); free(hu); free(tr); free(ln);
    }

    /* Encoder: exact per-token mean of ReLU(hidden @ w_pool) over usable
     * assigned atoms; a token with none is zero. */
    if (stage == ORC_ENCODER) {
        for (int64_t bt = 0; bt < B * T; ++bt) {
            const int64_t b = bt / T, t = bt % T;
            int complete = 1;
            int64_t count = 0;
            for (int64_t a = 0; a < A; ++a) {
                int64_t n = b * A + a;
                if (usable[n] && in->atom_to_token[n] == t) {
                    ++count;
                    if (!need_out[n])
                        complete = 0;
                }
            }
            if (out->done_token)
                out->done_token[bt] = (uint8_t)complete;
            if (!complete)
                continue;
            double *to = out->token_output + bt * U;
            for (int64_t x = 0; x < U; ++x)
                to[x] = 0.0;
            if (count == 0)
                continue;
            double *proj = (double *)malloc((size_t)U * sizeof(double));
            for (int64_t a = 0; a < A; ++a) {
                int64_t n = b * A + a;
                if (!(usable[n] && in->atom_to_token[n] == t))
                    continue;
                vec_mat(out->hidden + n * C, C, p->w_pool, U, U, proj);
                for (int64_t x = 0; x < U; ++x)
                    to[x] += proj[x] > 0.0 ? proj[x] : 0.0;
            }
            for (int64_t x = 0; x < U; ++x)
                to[x] /= (double)count;
            free(proj);
        }
    } else if (out->done_token) {
        memset(out->done_token, 0, (size_t)(B * T));
    }

    /* optional intermediates */
    if (out->usable)
        memcpy(out->usable, usable, (size_t)N);
    if (out->done_atom)
        memcpy(out->done_atom, need_out, (size_t)N);
    if (out->x0)
        memcpy(out->x0, x0, (size_t)(N * C) * sizeof(double));
    if (out->q_in)
        memcpy(out->q_in, qi, (size_t)(N * C) * sizeof(double));
    if (out->kv_in)
        memcpy(out->kv_in, kvi, (size_t)(N * C) * sizeof(double));
    if (out->q)
        memcpy(out->q, Q, (size_t)(N * HD) * sizeof(double));
    if (out->k)
        memcpy(out->k, Kp, (size_t)(N * HD) * sizeof(double));
    if (out->v)
        memcpy(out->v, Vp, (size_t)(N * HD) * sizeof(double));
    if (out->g)
        memcpy(out->g, G, (size_t)(N * HD) * sizeof(double));
    if (out->o)
        memcpy(out->o, O, (size_t)(N * HD) * sizeof(double));
    if (out->x1)
        memcpy(out->x1, X1, (size_t)(N * C) * sizeof(double));

    free(usable); free(need_out); free(need_proj); free(tok_want);
    free(x0); free(cc); free(qi); free(kvi); free(Q); free(Kp); free(Vp);
    free(G); free(O); free(X1);
    return 0;
}
