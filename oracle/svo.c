/*
 * svo.c -- CPU oracle for the single-forward speculative verification step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the test suite, the package's smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header or constant
 * with the GPU library.
 *
 * Plain, slow and direct: dense mask matrix, two-pass softmax per row over
 * the visible keys, full per-slot softmax, serial scans.  All arithmetic is
 * float64; inputs arrive as float32 (bf16 inputs are upcast exactly by the
 * caller).  Sources followed (page title, then section / equation):
 *   - "SimSD: Simple Speculative Decoding in Diffusion Language Models"
 *     (papernotes.org): 关键设计 1 (paired data/mask layout), 关键设计 2
 *     (temporal mask A_ij, the four-case equation), 关键设计 3 (RoPE copy
 *     alignment), 关键设计 4 (acceptance alpha_r in draft order, longest
 *     accepted prefix, in-place resample at the first rejection).
 *   - "S2D2: Fast Decoding for Diffusion LLMs via Training-Free
 *     Self-Speculation": 前置知识 "推测解码" (accept with min(1, q/p), resample
 *     at the first rejection from the residual) and 方法步骤 (5) (residual
 *     distribution (P_ver - P_draft)^+).
 *   - The Portuguese SimSD summary (gist.science), sections 1-4, which
 *     restate the layout, mask and RoPE rule.
 *   - "SPOT: Enhancing Speculative Decoding for Diffusion Language Models
 *     via Commit-Order Prediction": 前置知识 "Gumbel-Max 技巧与随机耦合"
 *     (argmax of log-probability plus Gumbel noise samples the distribution;
 *     a noise table shared by draft and target couples the two samples) and
 *     核心创新 / 方法步骤详情 (noise indexed by absolute output position; given
 *     the noise the target transition is deterministic; an edge is accepted
 *     when the draft state equals the target's; otherwise the target's own
 *     result is committed; T = 0 is the greedy transition).
 *   - "S2D2": 方法步骤详情 (4), the routing decision: the expected accepted
 *     prefix length K = sum_k prod_{i<=k} alpha_i with a margin-based
 *     (indicator of margin >= threshold) or entropy-based (exp(-beta H~))
 *     estimate of each alpha_i.
 *   - "SimSD", 关键设计 4 (a block with fewer undecoded positions than the
 *     draft length is finished by ordinary denoising) and 损失函数 / 训练策略
 *     (the prompt's K/V are cached), with the block-diffusion prior of
 *     "SPOT", 前置知识 (finished blocks join the cached prefix): the commit
 *     step, the cache append and the paged prompt cache at the end of this
 *     file.
 * Readings where the pages are silent:
 *   prompt carries step label 0 and counts as data; D~_k shares tau(k) with
 *   D_k; positions are 0..P-1 for the prompt and P+k for both D_k and D~_k;
 *   rotate-half RoPE with inv_freq_i = theta^(-2i/d); scale 1/sqrt(d) by
 *   default; q-head h reads kv-head h / (Hq/Hkv); accept iff u < alpha
 *   (strict); alpha = 1 when the draft probability of the proposed token is
 *   zero; inverse-CDF resampling in ascending token order with u[gamma];
 *   Z = 0 falls back to the target distribution; a full accept emits no extra
 *   token; the confidence that orders commit positions is max_v p_theta(v)
 *   of the untempered model distribution at every temperature (the token at
 *   the chosen position is the coupled choice); a state with no masked slot
 *   commits nothing and ends a tree walk.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define SVO_OK 0
#define SVO_BAD_TAU -1
#define SVO_BAD_ARG -2

int svo_version(void) { return 1; }

void svo_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int svo_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* tau must be a permutation of 1..B.  Returns 1 if so. */
static int tau_is_permutation(const int32_t *tau, int B) {
    int ok = 1;
    char *seen = (char *)calloc((size_t)B + 1, 1);
    for (int k = 0; k < B; ++k) {
        int t = tau[k];
        if (t < 1 || t > B || seen[t]) { ok = 0; break; }
        seen[t] = 1;
    }
    free(seen);
    return ok;
}

/*
 * Temporal-causal mask (SimSD 关键设计 2, equation A_ij).
 * Key/row order: [prompt 0..P-1 | D_1..D_B | D~_1..D~_B].  M is [2B][P+2B],
 * row i = response row (i < B: D_{i+1}; i >= B: D~_{i-B+1}).
 * Every position carries a kind (data or mask) and a step label: the prompt
 * is data with label 0, D_k and D~_k both carry tau(k).  A row sees a column
 * exactly when one of the equation's four cases holds.
 */
int svo_mask(int B, int P, const int32_t *tau, uint8_t *M) {
    if (B < 1 || P < 0) return SVO_BAD_ARG;
    if (!tau_is_permutation(tau, B)) return SVO_BAD_TAU;
    const int ncol = P + 2 * B;
    for (int i = 0; i < 2 * B; ++i) {
        const int row_is_data = i < B;
        const int ti = tau[i % B];
        for (int j = 0; j < ncol; ++j) {
            int col_is_data, tj;
            if (j < P) { col_is_data = 1; tj = 0; }
            else { const int c = j - P; col_is_data = c < B; tj = tau[c % B]; }
            int vis = 0;
            if (row_is_data && col_is_data && tj <= ti) vis = 1;          /* i,j in D      */
            else if (row_is_data && !col_is_data && tj > ti) vis = 1;     /* i in D, j in D~ */
            else if (!row_is_data && col_is_data && tj < ti) vis = 1;     /* i in D~, j in D */
            else if (!row_is_data && !col_is_data && tj >= ti) vis = 1;   /* i,j in D~     */
            M[(size_t)i * ncol + j] = (uint8_t)vis;
        }
    }
    return SVO_OK;
}

/*
 * Rotary position embedding, rotate-half convention, in place on
 * x[n][heads][d] (float64); row r is rotated at position pos[r].
 * Pair (i, i + d/2) turns by angle pos * theta^(-2i/d).
 */
void svo_rope(double *x, int64_t n, int heads, int d, const double *pos, double theta) {
    const int half = d / 2;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        for (int h = 0; h < heads; ++h) {
            double *v = x + ((size_t)r * heads + h) * d;
            for (int i = 0; i < half; ++i) {
                const double w = pow(theta, -2.0 * i / d);
                const double phi = pos[r] * w;
                const double c = cos(phi), s = sin(phi);
                const double a = v[i], b = v[i + half];
                v[i] = a * c - b * s;
                v[i + half] = a * s + b * c;
            }
        }
    }
}

/*
 * Masked attention of the 2B response rows of ONE sequence.
 *   q      [2B][Hq][d]   (pre-RoPE if theta > 0)
 *   k_new  [2B][Hkv][d]  (pre-RoPE if theta > 0), v_new [2B][Hkv][d]
 *   k_cache, v_cache [Hkv][P][d] (prompt keys already rotated)
 *   tau    [B], out [2B][Hq][d] float64.
 * Response row r (D_{r+1} or D~_{r-B+1}) sits at position P + (r mod B)
 * (SimSD 关键设计 3: the mask slot reuses its data slot's index).  With
 * theta <= 0 the inputs are taken as already rotated.  scale <= 0 means
 * 1/sqrt(d).  Keys: prompt, then the 2B response keys, masked by svo_mask.
 */
static int attn_dense(const float *q, const float *k_new, const float *v_new,
                      const float *k_cache, const float *v_cache, const uint8_t *M,
                      int R, int B, int P, int Hq, int Hkv, int d, double theta, double scale,
                      double *out);

int svo_attn(const float *q, const float *k_new, const float *v_new,
             const float *k_cache, const float *v_cache, const int32_t *tau,
             int B, int P, int Hq, int Hkv, int d, double theta, double scale,
             double *out) {
    if (B < 1 || P < 0 || Hq < 1 || Hkv < 1 || d < 2 || (d & 1) || Hq % Hkv) return SVO_BAD_ARG;
    const int R = 2 * B, ncol = P + 2 * B;
    uint8_t *M = (uint8_t *)malloc((size_t)R * ncol);
    int rc = svo_mask(B, P, tau, M);
    if (rc) { free(M); return rc; }
    rc = attn_dense(q, k_new, v_new, k_cache, v_cache, M, R, B, P, Hq, Hkv, d, theta, scale, out);
    free(M);
    return rc;
}

/*
 * Multi-copy verification attention of ONE sequence ("SPOT", 方法步骤详情 /
 * 核心方法 第三步: the target runs one batched forward over the root and all
 * draft states, (1+D)L positions, each state a copy of the block; 前置知识
 * "块扩散语言模型": attention is bidirectional inside a block and causal
 * across blocks).  Row r belongs to copy r / L and sits at position
 * P + (r mod L) (every copy is the same block); it sees every prompt key and
 * the L keys of its own copy, none of another copy's.
 *   q [C*L][Hq][d], k_new/v_new [C*L][Hkv][d] (copy-major, pre-RoPE if
 *   theta > 0), k_cache/v_cache [Hkv][P][d], out [C*L][Hq][d] float64.
 */
int svo_attn_copies(const float *q, const float *k_new, const float *v_new,
                    const float *k_cache, const float *v_cache, int L, int C, int P, int Hq,
                    int Hkv, int d, double theta, double scale, double *out) {
    if (L < 1 || C < 1 || P < 0 || Hq < 1 || Hkv < 1 || d < 2 || (d & 1) || Hq % Hkv) return SVO_BAD_ARG;
    const int R = C * L, ncol = P + R;
    uint8_t *M = (uint8_t *)malloc((size_t)R * ncol);
    for (int i = 0; i < R; ++i)
        for (int j = 0; j < ncol; ++j)
            M[(size_t)i * ncol + j] = (uint8_t)(j < P || (j - P) / L == i / L);
    const int rc = attn_dense(q, k_new, v_new, k_cache, v_cache, M, R, L, P, Hq, Hkv, d, theta, scale, out);
    free(M);
    return rc;
}

/*
 * Attention of R response rows under a dense visibility matrix M[R][P + R]
 * (prompt columns first); row r and response key r sit at position
 * P + (r mod B).
 */
static int attn_dense(const float *q, const float *k_new, const float *v_new,
                      const float *k_cache, const float *v_cache, const uint8_t *M,
                      int R, int B, int P, int Hq, int Hkv, int d, double theta, double scale,
                      double *out) {
    const int ncol = P + R, g = Hq / Hkv;
    double *qd = (double *)malloc(sizeof(double) * (size_t)R * Hq * d);
    double *kd = (double *)malloc(sizeof(double) * (size_t)R * Hkv * d);
    double *pos = (double *)malloc(sizeof(double) * (size_t)R);
    for (size_t t = 0; t < (size_t)R * Hq * d; ++t) qd[t] = q[t];
    for (size_t t = 0; t < (size_t)R * Hkv * d; ++t) kd[t] = k_new[t];
    for (int r = 0; r < R; ++r) pos[r] = (double)P + (double)(r % B);
    if (theta > 0) {
        svo_rope(qd, R, Hq, d, pos, theta);
        svo_rope(kd, R, Hkv, d, pos, theta);
    }
    if (scale <= 0) scale = 1.0 / sqrt((double)d);

#pragma omp parallel
    {
        double *sc = (double *)malloc(sizeof(double) * (size_t)ncol);
#pragma omp for schedule(dynamic, 1) collapse(2)
        for (int h = 0; h < Hq; ++h) {
            for (int i = 0; i < R; ++i) {
                const int kvh = h / g;
                const double *qi = qd + ((size_t)i * Hq + h) * d;
                const uint8_t *Mi = M + (size_t)i * ncol;
                double mx = -INFINITY;
                for (int j = 0; j < ncol; ++j) {
                    if (!Mi[j]) continue;
                    double dot = 0.0;
                    if (j < P) {
                        const float *kj = k_cache + ((size_t)kvh * P + j) * d;
                        for (int e = 0; e < d; ++e) dot += qi[e] * (double)kj[e];
                    } else {
                        const double *kj = kd + ((size_t)(j - P) * Hkv + kvh) * d;
                        for (int e = 0; e < d; ++e) dot += qi[e] * kj[e];
                    }
                    sc[j] = scale * dot;
                    if (sc[j] > mx) mx = sc[j];
                }
                double den = 0.0;
                for (int j = 0; j < ncol; ++j) {
                    if (!Mi[j]) continue;
                    sc[j] = exp(sc[j] - mx);
                    den += sc[j];
                }
                double *oi = out + ((size_t)i * Hq + h) * d;
                for (int e = 0; e < d; ++e) oi[e] = 0.0;
                for (int j = 0; j < ncol; ++j) {
                    if (!Mi[j]) continue;
                    const double w = sc[j] / den;
                    if (j < P) {
                        const float *vj = v_cache + ((size_t)kvh * P + j) * d;
                        for (int e = 0; e < d; ++e) oi[e] += w * (double)vj[e];
                    } else {
                        const float *vj = v_new + ((size_t)(j - P) * Hkv + kvh) * d;
                        for (int e = 0; e < d; ++e) oi[e] += w * (double)vj[e];
                    }
                }
            }
        }
        free(sc);
    }
    free(qd); free(kd); free(pos);
    return SVO_OK;
}

/* Softmax of one logits row in float64: p[v] = exp(l[v] - m) / s with
 * m = max l and s = sum_v exp(l[v] - m).  p may be NULL (only m, s). */
void svo_softmax(const float *l, int64_t V, double *p, double *m_out, double *s_out) {
    double m = -INFINITY;
    for (int64_t v = 0; v < V; ++v) if ((double)l[v] > m) m = l[v];
    double s = 0.0;
    for (int64_t v = 0; v < V; ++v) s += exp((double)l[v] - m);
    if (p) for (int64_t v = 0; v < V; ++v) p[v] = exp((double)l[v] - m) / s;
    if (m_out) *m_out = m;
    if (s_out) *s_out = s;
}

/*
 * Residual resample at the first rejected slot (S2D2 方法步骤 (5): the
 * residual (P_target - P_draft)^+; SimSD 关键设计 4: the target resamples the
 * rejected position in place).  r(v) = max(0, p_theta(v) - p_phi(v)),
 * Z = sum r.  The token is the smallest v whose running sum (ascending token
 * order) exceeds u * Z.  If Z == 0 the target distribution p_theta is used
 * instead.  If rounding leaves no running sum above u * Z, the last token
 * with positive mass is taken.  Optional outputs: cdf[V] (running sums of the
 * distribution actually used), *Z_out, *used_target (1 if Z == 0).
 */
int64_t svo_residual(const float *l, const float *pphi, int64_t V, double u,
                     double *cdf, double *Z_out, int *used_target) {
    double m, s;
    svo_softmax(l, V, NULL, &m, &s);
    double Z = 0.0;
    for (int64_t v = 0; v < V; ++v) {
        const double pt = exp((double)l[v] - m) / s;
        const double r = pt - (double)pphi[v];
        if (r > 0) Z += r;
    }
    const int use_t = !(Z > 0.0);
    double tot = 0.0;
    if (use_t) for (int64_t v = 0; v < V; ++v) tot += exp((double)l[v] - m) / s;
    else tot = Z;
    const double thr = u * tot;
    double run = 0.0;
    int64_t pick = -1, last_pos = -1;
    for (int64_t v = 0; v < V; ++v) {
        const double pt = exp((double)l[v] - m) / s;
        double mass = use_t ? pt : pt - (double)pphi[v];
        if (mass < 0) mass = 0;
        run += mass;
        if (cdf) cdf[v] = run;
        if (mass > 0) last_pos = v;
        if (pick < 0 && run > thr) pick = v;
    }
    if (pick < 0) pick = last_pos;
    if (Z_out) *Z_out = tot;
    if (used_target) *used_target = use_t;
    return pick;
}

/* Tempered logits row (sampling at temperature T: the target distribution
 * is softmax(l / T)).  z[v] = l[v] * inv_t, the product rounded to float32,
 * with inv_t = 1/T rounded to float32 by the caller; T = 1 (inv_t = 1)
 * leaves the row unchanged. */
static void temper_row(const float *l, int64_t V, float inv_t, float *z) {
    for (int64_t v = 0; v < V; ++v) z[v] = l[v] * inv_t;
}

/*
 * Acceptance for `batch` sequences (SimSD 关键设计 4).
 *   logits, probs [batch][B][V] indexed by slot (the slot's D~ row);
 *   inv_t: 1/T in float32; the target distribution of a slot is the softmax
 *   of its tempered logits row (temper_row); the draft probabilities are the
 *   caller's, already at the drafter's temperature;
 *   tokens [batch][B] draft token per slot; tau [batch][B];
 *   u [batch][gamma+1]: u[r-1] tests draft step r, u[gamma] drives the resample.
 * Draft step r (1..gamma) verifies slot o_r with tau(o_r) = r:
 *   alpha_r = min(1, p_theta(x) / p_phi(x)), x = tokens[o_r], accept iff
 *   u[r-1] < alpha_r.  L = number of leading accepted steps.
 * Outputs: accept_len[batch] = L; out_tokens[batch][B]: the draft token where
 *   tau <= L, the resampled token where tau == L+1 (only if L < gamma), -1
 *   elsewhere; alpha[batch][gamma] (float64, every step, draft order);
 *   resample_slot[batch] (-1 if none) -- may be NULL.
 * Returns 0, or a negative code for the first bad sequence.
 */
int svo_accept(const float *logits, const float *probs, const int32_t *tokens,
               const int32_t *tau, const float *u, int batch, int B, int gamma,
               int64_t V, float inv_t, int32_t *accept_len, int32_t *out_tokens, double *alpha,
               int32_t *resample_slot) {
    if (batch < 0 || B < 1 || gamma < 1 || gamma > B || V < 1) return SVO_BAD_ARG;
    if (!(inv_t > 0.f) || !isfinite(inv_t)) return SVO_BAD_ARG;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < batch; ++b) {
        const int32_t *tb = tau + (size_t)b * B;
        const int32_t *xb = tokens + (size_t)b * B;
        const float *ub = u + (size_t)b * (gamma + 1);
        int32_t *ob = out_tokens + (size_t)b * B;
        if (!tau_is_permutation(tb, B)) {
#pragma omp critical
            err = SVO_BAD_TAU;
            continue;
        }
        int bad = 0;
        for (int k = 0; k < B; ++k) if (xb[k] < 0 || xb[k] >= V) bad = 1;
        if (bad) {
#pragma omp critical
            err = SVO_BAD_ARG;
            continue;
        }
        int order[64 + 1];
        int *o = (B <= 64) ? order : (int *)malloc(sizeof(int) * ((size_t)B + 1));
        float *z = (float *)malloc(sizeof(float) * (size_t)V);  /* tempered row */
        for (int k = 0; k < B; ++k) o[tb[k]] = k;   /* o[r] = slot decoded at step r */
        int L = -1;
        for (int r = 1; r <= gamma; ++r) {
            const int k = o[r];
            temper_row(logits + ((size_t)b * B + k) * V, V, inv_t, z);
            const float *pk = probs + ((size_t)b * B + k) * V;
            double m, s;
            svo_softmax(z, V, NULL, &m, &s);
            const int x = xb[k];
            const double pt = exp((double)z[x] - m) / s;
            const double pd = (double)pk[x];
            double a = (pd > 0.0) ? pt / pd : 1.0;
            if (a > 1.0) a = 1.0;
            if (alpha) alpha[(size_t)b * gamma + (r - 1)] = a;
            if (L < 0 && !((double)ub[r - 1] < a)) L = r - 1;
        }
        if (L < 0) L = gamma;
        accept_len[b] = L;
        for (int k = 0; k < B; ++k) ob[k] = (tb[k] <= L) ? xb[k] : -1;
        int rs = -1;
        if (L < gamma) {
            rs = o[L + 1];
            temper_row(logits + ((size_t)b * B + rs) * V, V, inv_t, z);
            const float *pk = probs + ((size_t)b * B + rs) * V;
            ob[rs] = (int32_t)svo_residual(z, pk, V, (double)ub[gamma], NULL, NULL, NULL);
        }
        if (resample_slot) resample_slot[b] = rs;
        free(z);
        if (o != order) free(o);
    }
    return err;
}

/*
 * Target choice of one slot under shared-noise verification ("SPOT", 前置知识
 * "Gumbel-Max 技巧与随机耦合"; 方法步骤详情: given the noise table the target
 * transition is a deterministic function).  At temperature T > 0 the choice
 * is argmax_v (l[v] / T + g[v]) with g the slot's row of the noise table;
 * T = 0 is the greedy choice argmax_v l[v].  This argmax decides an integer,
 * so it is taken in the kernel's precision: the score is one float32 fused
 * multiply-add fmaf(l[v], inv_t, g[v]) with inv_t = 1.0f / T rounded to
 * float32, and equal scores go to the smallest v.  inv_t <= 0 selects the
 * greedy choice (g is not read and may be NULL).
 */
int64_t svo_coupled_choice(const float *l, const float *g, int64_t V, float inv_t) {
    int64_t best = 0;
    float bs = (inv_t > 0.f) ? fmaf(l[0], inv_t, g[0]) : l[0];
    for (int64_t v = 1; v < V; ++v) {
        const float sc = (inv_t > 0.f) ? fmaf(l[v], inv_t, g[v]) : l[v];
        if (sc > bs) { bs = sc; best = v; }
    }
    return best;
}

/*
 * Shared-noise verification of a batch ("SPOT", 核心创新 "耦合噪声验证" and
 * 方法步骤详情 验证; the draft order and slot layout of "SimSD", 关键设计 1 and
 * 4).  Draft step r = 1..gamma verifies the slot o_r with tau(o_r) = r: it is
 * accepted iff the draft token equals the target's own choice at that slot
 * (the states after the step are equal; the commit position is fixed by
 * tau).  L = number of leading accepted steps; at the first rejection the
 * target's own choice is committed.
 *   logits [batch][B][V], gumbel [batch][B][V] (the noise-table row of each
 *   slot's absolute position; may be NULL when temperature == 0), tokens and
 *   tau [batch][B].  temperature > 0: coupled sampling; == 0: greedy.
 * Outputs: accept_len[batch]; out_tokens[batch][B] = draft token where
 *   tau <= L, the target's choice where tau == L+1 (only if L < gamma), -1
 *   elsewhere; target_tokens[batch][B] (may be NULL) = the target's choice at
 *   every verified slot (tau <= gamma), -1 elsewhere.
 * Returns 0, or a negative code for the first bad sequence.
 */
int svo_accept_coupled(const float *logits, const float *gumbel, const int32_t *tokens,
                       const int32_t *tau, int batch, int B, int gamma, int64_t V, float temperature,
                       int32_t *accept_len, int32_t *out_tokens, int32_t *target_tokens) {
    if (batch < 0 || B < 1 || gamma < 1 || gamma > B || V < 1 || !(temperature >= 0.f)) return SVO_BAD_ARG;
    if (temperature > 0.f && !gumbel) return SVO_BAD_ARG;
    const float inv_t = (temperature > 0.f) ? 1.0f / temperature : 0.f;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < batch; ++b) {
        const int32_t *tb = tau + (size_t)b * B;
        const int32_t *xb = tokens + (size_t)b * B;
        int32_t *ob = out_tokens + (size_t)b * B;
        if (!tau_is_permutation(tb, B)) {
#pragma omp critical
            err = SVO_BAD_TAU;
            continue;
        }
        int order[64 + 1];
        int *o = (B <= 64) ? order : (int *)malloc(sizeof(int) * ((size_t)B + 1));
        for (int k = 0; k < B; ++k) o[tb[k]] = k;   /* o[r] = slot decoded at step r */
        int64_t choice[64];
        int64_t *c = (B <= 64) ? choice : (int64_t *)malloc(sizeof(int64_t) * (size_t)B);
        for (int k = 0; k < B; ++k) {
            c[k] = -1;
            if (tb[k] > gamma) continue;   /* not verified in this call */
            const size_t row = (size_t)b * B + k;
            c[k] = svo_coupled_choice(logits + row * V, gumbel ? gumbel + row * V : NULL, V, inv_t);
        }
        int L = gamma;
        for (int r = 1; r <= gamma; ++r) {
            const int k = o[r];
            if ((int64_t)xb[k] != c[k]) { L = r - 1; break; }
        }
        accept_len[b] = L;
        for (int k = 0; k < B; ++k) ob[k] = (tb[k] <= L) ? xb[k] : -1;
        if (L < gamma) ob[o[L + 1]] = (int32_t)c[o[L + 1]];
        if (target_tokens)
            for (int k = 0; k < B; ++k) target_tokens[(size_t)b * B + k] = (int32_t)c[k];
        if (c != choice) free(c);
        if (o != order) free(o);
    }
    return err;
}

/*
 * Verify-routing estimator of one batch ("S2D2", 方法步骤详情 (4): the expected
 * accepted prefix length K = sum_{k=1}^{L} prod_{i=1}^{k} alpha_i, with
 * alpha_i estimated from the draft distribution either by its margin,
 * 1[m_i >= tau_margin], or by its entropy, exp(-beta * H~_i)).
 * Per slot, with p the slot's draft distribution (float64 arithmetic):
 *   m  = p_(1) - p_(2), the two largest entries (m = p_(1) when V = 1);
 *   H~ = -(sum_v p_v ln p_v) / ln V, terms with p_v = 0 vanish (H~ = 0 when
 *        V = 1).
 * The steps are taken in draft order r = 1..gamma (slot o_r with tau(o_r) =
 * r), the positions the verification would check, so
 *   khat = sum_{k=1}^{gamma} prod_{r=1}^{k} alpha_{o_r}.
 * estimator 0: margin with param = tau_margin; 1: entropy with param = beta.
 * Outputs khat[batch] and alpha_hat[batch][gamma] (draft order; may be NULL).
 */
int svo_route(const float *probs, const int32_t *tau, int batch, int B, int gamma, int64_t V,
              int estimator, double param, double *khat, double *alpha_hat) {
    if (batch < 0 || B < 1 || gamma < 1 || gamma > B || V < 1 || (estimator != 0 && estimator != 1))
        return SVO_BAD_ARG;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < batch; ++b) {
        const int32_t *tb = tau + (size_t)b * B;
        if (!tau_is_permutation(tb, B)) {
#pragma omp critical
            err = SVO_BAD_TAU;
            continue;
        }
        int order[64 + 1];
        int *o = (B <= 64) ? order : (int *)malloc(sizeof(int) * ((size_t)B + 1));
        for (int k = 0; k < B; ++k) o[tb[k]] = k;   /* o[r] = slot decoded at step r */
        double prod = 1.0, sum = 0.0;
        for (int r = 1; r <= gamma; ++r) {
            const float *p = probs + ((size_t)b * B + o[r]) * V;
            double a;
            if (estimator == 0) {
                double p1 = -1.0, p2 = 0.0;
                for (int64_t v = 0; v < V; ++v) {
                    const double x = (double)p[v];
                    if (x > p1) { p2 = p1; p1 = x; }
                    else if (x > p2) p2 = x;
                }
                if (p2 < 0.0) p2 = 0.0;
                a = (p1 - p2 >= param) ? 1.0 : 0.0;
            } else {
                double h = 0.0;
                for (int64_t v = 0; v < V; ++v) {
                    const double x = (double)p[v];
                    if (x > 0.0) h -= x * log(x);
                }
                const double hn = (V > 1) ? h / log((double)V) : 0.0;
                a = exp(-param * hn);
            }
            if (alpha_hat) alpha_hat[(size_t)b * gamma + (r - 1)] = a;
            prod *= a;
            sum += prod;
        }
        khat[b] = sum;
        if (o != order) free(o);
    }
    return err;
}

/*
 * Prompt rows of ONE sequence from its cache, for callers that keep the
 * prompt K (or V) in pages.  The pages say only that the prompt's K/V are
 * cached ("SimSD", 损失函数 / 训练策略: a KV cache makes the prefix cost
 * linear; the block-diffusion prior in "SPOT", 前置知识: finished blocks are
 * cached and later blocks attend to them).  Paging is a storage layout for
 * that cache, not something the pages prescribe: row j of the sequence is
 * row j % page_size of page table_row[j / page_size], pages laid out
 * [n_pages][Hkv][page_size][d].
 * out [Hkv][P][d].  Returns SVO_BAD_ARG for a page id outside [0, n_pages).
 */
int svo_gather_prefix(const float *pages, const int32_t *table_row, int P, int page_size, int n_pages,
                      int Hkv, int d, float *out) {
    if (P < 0 || page_size < 1 || n_pages < 1 || Hkv < 1 || d < 1) return SVO_BAD_ARG;
    for (int j = 0; j < P; ++j) {
        const int pg = table_row[j / page_size];
        if (pg < 0 || pg >= n_pages) return SVO_BAD_ARG;
        for (int h = 0; h < Hkv; ++h)
            memcpy(out + ((size_t)h * P + j) * d,
                   pages + (((size_t)pg * Hkv + h) * page_size + j % page_size) * d, sizeof(float) * d);
    }
    return SVO_OK;
}

/*
 * Commit step of one verification round, per sequence ("SimSD", 关键设计 4:
 * the accepted prefix is kept, the first rejected position is resampled in
 * place, the rest is discarded; when fewer undecoded positions R remain in
 * the block than the draft length gamma, the block is finished by ordinary
 * target denoising).
 *   out_tokens   [batch][B]: the verification output, the committed token of
 *                each slot or -1 (accepted slots and the resampled slot carry
 *                a token).
 *   block_tokens [batch][B], in/out: the block's tokens, -1 where still
 *                masked; every committed token is written into its slot.
 *   remaining [batch] = R, the masked slots left after the commit;
 *   state [batch] = 2 when R == 0 (the block is finished and joins the
 *   prefix), 1 when 0 < R < gamma (fall back to target denoising), else 0;
 *   n_append [batch] = B when the block is finished (its B rows are appended
 *   to the prompt cache), else 0.
 */
int svo_commit(const int32_t *out_tokens, int32_t *block_tokens, int batch, int B, int gamma,
               int32_t *remaining, int32_t *state, int32_t *n_append) {
    if (batch < 0 || B < 1 || gamma < 1 || gamma > B) return SVO_BAD_ARG;
    for (int b = 0; b < batch; ++b) {
        int R = 0;
        for (int k = 0; k < B; ++k) {
            const size_t i = (size_t)b * B + k;
            if (out_tokens[i] >= 0) block_tokens[i] = out_tokens[i];
            if (block_tokens[i] < 0) ++R;
        }
        remaining[b] = R;
        state[b] = (R == 0) ? 2 : (R < gamma ? 1 : 0);
        n_append[b] = (R == 0) ? B : 0;
    }
    return SVO_OK;
}

/*
 * Append rows to the prompt cache of each sequence (the cache of
 * svo_gather_prefix; the finished block joins the prefix).  Sequence b
 * appends rows 0 .. n_append[b]-1 of its source rows (k_rows / v_rows
 * [batch][src_stride][Hkv][d]) at positions prefix_lens[b] + i, then
 * prefix_lens[b] += n_append[b].  With theta > 0 the key of row i is rotated
 * at its position prefix_lens[b] + i before it is stored (the cache holds
 * rotated keys, as the attention's prompt keys are).  k_out / v_out receive
 * the stored rows as float64 [batch][src_stride][Hkv][d] (rows past
 * n_append[b] untouched) and pages are not written here: the caller places
 * row i of sequence b at page table[b][(P_b + i) / page_size], row
 * (P_b + i) % page_size.  status[b] = 1 (and nothing appended) when the
 * rows would pass `capacity` rows (max_pages * page_size for a paged cache,
 * the row stride for a contiguous one), else 0.
 */
int svo_kv_append(const float *k_rows, const float *v_rows, int src_stride, const int32_t *n_append,
                  int32_t *prefix_lens, int batch, int capacity, int Hkv, int d, double theta,
                  double *k_out, double *v_out, int32_t *status) {
    if (batch < 0 || src_stride < 1 || Hkv < 1 || d < 2 || (d & 1) || capacity < 0) return SVO_BAD_ARG;
    for (int b = 0; b < batch; ++b) {
        const int n = n_append[b], P = prefix_lens[b];
        if (n < 0 || n > src_stride || P < 0) return SVO_BAD_ARG;
        if ((long long)P + n > capacity) { status[b] = 1; continue; }
        status[b] = 0;
        for (int i = 0; i < n; ++i) {
            const size_t row = ((size_t)b * src_stride + i) * Hkv * d;
            for (int e = 0; e < Hkv * d; ++e) {
                k_out[row + e] = (double)k_rows[row + e];
                v_out[row + e] = (double)v_rows[row + e];
            }
            if (theta > 0) {
                const double pos = (double)P + (double)i;
                svo_rope(k_out + row, 1, Hkv, d, &pos, theta);
            }
        }
        prefix_lens[b] = P + n;
    }
    return SVO_OK;
}

/*
 * Verification of a draft tree ("SPOT", 核心方法, second step: a tree of
 * draft states, each child its parent plus one commit (position, token);
 * 方法步骤详情, 验证: one forward gives the target's own next commit at the
 * root and at every draft state, edges equal to it are accepted, otherwise
 * the target's own commit is made).  Per sequence, nodes 0..N-1 with node 0
 * the root state:
 *   parent[n] (node 0's is ignored), node_pos[n], node_tok[n]: node n is its
 *     parent plus the commit of node_tok[n] at position node_pos[n];
 *   target_pos[n]: the position the target's own policy commits next at
 *     state n (an input: the policy belongs to the model);
 *   logits[n][V], gumbel[n][V]: the target's logits at that position in
 *     node n's copy and the noise row of its absolute position (gumbel may
 *     be NULL when temperature == 0).
 * The target's own token at n is svo_coupled_choice of its row.  From the
 * root, the walk moves to the child (smallest index if several) whose
 * commit equals the target's own commit at the current node, and stops when
 * none does.
 * Outputs: path_len[b] = accepted edges L; path[b][0..L] = the nodes of the
 * walk (root first), -1 after; commit_pos[b], commit_tok[b] = the target's
 * own commit at the last node; target_tok[b][n] = the target's own token at
 * every node.  Returns SVO_BAD_ARG for a parent index outside [0, n).
 */
int svo_tree_verify(const float *logits, const float *gumbel, const int32_t *parent, const int32_t *node_pos,
                    const int32_t *node_tok, const int32_t *target_pos, int batch, int N, int64_t V,
                    float temperature, int32_t *path_len, int32_t *path, int32_t *commit_pos,
                    int32_t *commit_tok, int32_t *target_tok) {
    if (batch < 0 || N < 1 || V < 1 || !(temperature >= 0.f)) return SVO_BAD_ARG;
    const float inv_t = temperature > 0.f ? 1.0f / temperature : 0.0f;  /* 0: greedy */
    for (int b = 0; b < batch; ++b) {
        const int32_t *pb = parent + (size_t)b * N;
        for (int n = 1; n < N; ++n)
            if (pb[n] < 0 || pb[n] >= n) return SVO_BAD_ARG;
        int32_t *tt = target_tok + (size_t)b * N;
        for (int n = 0; n < N; ++n) {
            const size_t row = (size_t)b * N + n;
            tt[n] = (int32_t)svo_coupled_choice(logits + row * V, gumbel ? gumbel + row * V : NULL, V, inv_t);
        }
        const int32_t *tp = target_pos + (size_t)b * N;
        const int32_t *np = node_pos + (size_t)b * N, *nt = node_tok + (size_t)b * N;
        int32_t *pa = path + (size_t)b * N;
        for (int n = 0; n < N; ++n) pa[n] = -1;
        int cur = 0, L = 0;
        pa[0] = 0;
        while (L < N - 1) {  /* a walk down a tree has at most N - 1 edges */
            int next = -1;
            for (int c = 1; c < N; ++c)
                if (pb[c] == cur && np[c] == tp[cur] && nt[c] == tt[cur]) { next = c; break; }
            if (next < 0) break;
            cur = next;
            pa[++L] = cur;
        }
        path_len[b] = L;
        commit_pos[b] = tp[cur];
        commit_tok[b] = tt[cur];
    }
    return SVO_OK;
}

/*
 * Confidence of one slot ("SPOT", 前置知识 "块扩散语言模型": a decoding step
 * commits the masked position of highest confidence; "动态阈值解码": the
 * confidence is c_s = max_v p_theta,s(v)).  With p = softmax(l):
 * max_v p_v = 1 / sum_v exp(l_v - max l).  All in float64.  The confidence
 * reads the model's distribution p_theta itself at every temperature (the
 * page's formula carries no temperature).
 */
double svo_confidence(const float *l, int64_t V) {
    double m = -INFINITY;
    for (int64_t v = 0; v < V; ++v)
        if ((double)l[v] > m) m = (double)l[v];
    if (m == -INFINITY) return 0.0;  /* every entry masked: no mass anywhere */
    double s = 0.0;
    for (int64_t v = 0; v < V; ++v) s += exp((double)l[v] - m);
    return 1.0 / s;
}

/*
 * The target's own transition at one block state ("SPOT", 方法步骤详情, 验证:
 * Phi_0 at T = 0, Phi_G for the fixed noise table G at T > 0; with the rule
 * of "动态阈值解码" for the set-commit decoder).
 *   state[L]: the block, a token >= 0 at each decided slot, -1 where masked;
 *   logits[L][V]: the target's logits at every slot of this state's copy
 *     (rows of decided slots are not read);
 *   gumbel[L][V]: the noise-table rows of the block's absolute positions
 *     (NULL when inv_t <= 0);
 *   threshold: every masked slot whose confidence exceeds it (strictly) is
 *     committed; when none does, the single masked slot of highest
 *     confidence is, the smallest slot among equal confidences.  A threshold
 *     >= 1 can never be exceeded (c <= 1): the one-commit decoder.
 * The token at a committed slot is the target's own choice there,
 * svo_coupled_choice of its row (greedy when inv_t <= 0).
 * Outputs: commit[L] = that token at each committed slot, -1 elsewhere;
 *   conf[L] (may be NULL) = the confidence of each masked slot, -1 at
 *   decided slots.  Returns the number of committed slots (0 when the state
 *   has no masked slot).
 */
int svo_transition(const float *logits, const float *gumbel, const int32_t *state, int L, int64_t V, float inv_t,
                   float threshold, int32_t *commit, double *conf) {
    int best = -1, n = 0;
    double bc = 0.0;
    for (int s = 0; s < L; ++s) {
        commit[s] = -1;
        if (conf) conf[s] = -1.0;
        if (state[s] >= 0) continue;
        const double c = svo_confidence(logits + (size_t)s * V, V);
        if (conf) conf[s] = c;
        if (best < 0 || c > bc) { best = s; bc = c; }
        if (c > (double)threshold) {
            commit[s] = (int32_t)svo_coupled_choice(logits + (size_t)s * V, gumbel ? gumbel + (size_t)s * V : NULL,
                                                    V, inv_t);
            ++n;
        }
    }
    if (n == 0 && best >= 0) {
        commit[best] = (int32_t)svo_coupled_choice(logits + (size_t)best * V,
                                                   gumbel ? gumbel + (size_t)best * V : NULL, V, inv_t);
        n = 1;
    }
    return n;
}

/*
 * The walk down a tree of block states given the target's own commit at
 * every state ("SPOT", 核心方法, third step: state-equality checks edge by
 * edge, the one prefix path that agrees with the target's own trajectory is
 * accepted; 方法步骤详情, 验证: otherwise the target's own result is
 * committed).  Per sequence, nodes 0..N-1, node 0 the root:
 *   parent[N] (node 0's ignored; parent[n] in [0, n));
 *   state[N][L]: each node's block (-1 masked);
 *   commit[N][L]: the target's own commit at each node (svo_transition).
 * From the root the walk moves to the child (smallest index if several)
 * whose state equals the current state with the current commit applied; it
 * stops at a node with no masked slot (a finished block has nothing left to
 * commit) or where no child matches.  At most N - 1 edges.
 * Outputs: path_len[b], path[b][N] (nodes of the walk, root first, -1
 * after), next_state[b][L] = the last node's state with its commit applied.
 */
int svo_state_walk(const int32_t *parent, const int32_t *state, const int32_t *commit, int batch, int N, int L,
                   int32_t *path_len, int32_t *path, int32_t *next_state) {
    if (batch < 0 || N < 1 || L < 1) return SVO_BAD_ARG;
    for (int b = 0; b < batch; ++b) {
        const int32_t *pb = parent + (size_t)b * N;
        for (int n = 1; n < N; ++n)
            if (pb[n] < 0 || pb[n] >= n) return SVO_BAD_ARG;
        const int32_t *sb = state + (size_t)b * N * L, *cb = commit + (size_t)b * N * L;
        int32_t *pa = path + (size_t)b * N;
        for (int n = 0; n < N; ++n) pa[n] = -1;
        int cur = 0, len = 0;
        pa[0] = 0;
        while (len < N - 1) {
            const int32_t *y = sb + (size_t)cur * L, *cm = cb + (size_t)cur * L;
            int open = 0;
            for (int s = 0; s < L; ++s) open |= (y[s] < 0);
            if (!open) break;
            int next = -1;
            for (int c = 1; c < N && next < 0; ++c) {
                if (pb[c] != cur) continue;
                const int32_t *z = sb + (size_t)c * L;
                int eq = 1;
                for (int s = 0; s < L && eq; ++s) eq = (z[s] == (cm[s] >= 0 ? cm[s] : y[s]));
                if (eq) next = c;
            }
            if (next < 0) break;
            cur = next;
            pa[++len] = cur;
        }
        path_len[b] = len;
        const int32_t *y = sb + (size_t)cur * L, *cm = cb + (size_t)cur * L;
        for (int s = 0; s < L; ++s) next_state[(size_t)b * L + s] = cm[s] >= 0 ? cm[s] : y[s];
    }
    return SVO_OK;
}

/*
 * Verification of a tree of block states: the target's own transition at
 * every node (svo_transition) followed by the walk (svo_state_walk).
 *   logits [batch][N][L][V]: the target's logits at every slot of every
 *     node's copy; gumbel [batch][L][V]: the noise rows of the block's
 *     absolute positions, shared by all copies (NULL when temperature == 0);
 *   parent [batch][N], state [batch][N][L].
 * Outputs as svo_state_walk, plus commit [batch][N][L] and conf
 * [batch][N][L] (may be NULL) per node as svo_transition.
 */
int svo_tree_states(const float *logits, const float *gumbel, const int32_t *parent, const int32_t *state, int batch,
                    int N, int L, int64_t V, float temperature, float threshold, int32_t *path_len, int32_t *path,
                    int32_t *next_state, int32_t *commit, double *conf) {
    if (batch < 0 || N < 1 || L < 1 || V < 1 || !(temperature >= 0.f) || threshold != threshold) return SVO_BAD_ARG;
    const float inv_t = temperature > 0.f ? 1.0f / temperature : 0.0f;
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int b = 0; b < batch; ++b)
        for (int n = 0; n < N; ++n) {
            const size_t node = (size_t)b * N + n;
            svo_transition(logits + node * L * V, gumbel ? gumbel + (size_t)b * L * V : NULL, state + node * L, L, V,
                           inv_t, threshold, commit + node * L, conf ? conf + node * L : NULL);
        }
    return svo_state_walk(parent, state, commit, batch, N, L, path_len, path, next_state);
}
