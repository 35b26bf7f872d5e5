/*
 * spec_verify_oracle.c -- plain CPU oracle for the verify step of speculative
 * sampling (modified rejection sampling).
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this code.  The GPU library never calls it and shares
 * no source with it.
 *
 * Style: one thread, IEEE fp64 for every value, every sum taken sequentially in
 * vocabulary order, one step of the method after the other in the order the
 * pages give.  Nothing is blocked, fused or reordered.  bf16 inputs are widened
 * exactly (bf16 -> fp32 -> fp64); fp32 uniforms are widened exactly.
 *
 * What is computed, with the passage each step follows:
 *
 *   [P1] "Speculative Decoding（投機的デコーディング）— 小さなモデルでLLM推論を高速化する"
 *        (disassemble-channel.com/speculative-decoding-theory/)
 *   [P2] "論文解説: Fast Inference from Transformers via Speculative Decoding"
 *        (0h-n0.github.io/posts/paper-2211-17192)
 *   [P3] "投機的デコーディングとは：同時リクエストが多いと遅くなる理由"
 *        (zvxbase.com/blog/speculative-decoding-draft-length-by-load/)
 *   [P4] "LLM推測デコーディング最適化実踐" (toolsku.com), section 検証アルゴリズムの実装
 *
 *   - p_i = softmax(z_p[i] / T), q_i = softmax(z_q[i] / T), one T for target and
 *     draft: P2 code sketch (softmax of logits / temperature on both models);
 *     P4 section 検証アルゴリズムの実装 (same).  Target has gamma+1 rows (P4, the
 *     slice of the last gamma+1 positions), draft has gamma rows.
 *   - accept draft i with probability min(1, p_i(x_i) / q_i(x_i)); with a
 *     supplied uniform u this is "accept iff u < min(1, p/q)": P1 section
 *     ステップ3: 受理・棄却判定 (alpha_i equation) and the simulation's
 *     comparison of a uniform draw against the acceptance probability; P2
 *     section 投機的サンプリングアルゴリズム (accept equation).
 *   - stop at the first rejection, keep the accepted prefix, discard the rest:
 *     P1 section ステップ3 (bullet list after the alpha_i equation).
 *   - on a rejection at position k, sample from
 *     p'(x) = max(0, p_k(x) - q_k(x)) / sum_x' max(0, p_k(x') - q_k(x')):
 *     P1 section 修正分布の定義 (the p' equation); P2 section 投機的サンプリング
 *     アルゴリズム (modified-distribution equation).  If that sum is zero the
 *     P1 simulation falls back to p (section Pythonによるシミュレーション実装);
 *     this oracle does the same and raises a flag.
 *   - if every draft is accepted, sample a bonus token from target row gamma:
 *     P1 section ステップ3 (bonus sentence, garbled in the extraction) and the
 *     simulation's final draw from p; P4 (bonus drawn from the last target row).
 *   - T == 0 is greedy: draft i is accepted iff it equals argmax p_i, and the
 *     emitted replacement / bonus is argmax of the target row: P2 section
 *     実装のポイント (greedy decoding reduces acceptance to an argmax match); P3
 *     worked example in section 先読みは、一回の順伝播で進むトークンを増やす.
 *
 *   - optional top-k / top-p filtering (only the deployment example of P4,
 *     section vLLM推測デコーディング設定, names top_p; the semantics are a
 *     reading): both filters apply to every target and draft row of the
 *     request, temperature first, then top-k, then top-p on what top-k kept;
 *     the rule above then runs on the renormalised distributions.
 *
 * Readings where the pages are silent (each one is listed in the design notes):
 *   R1 strict comparison u < a;  R2 no epsilon guards (q(x) = 0 gives ratio
 *   +inf if p(x) > 0, else 0);  R4 zero residual mass falls back to p_k;
 *   R5 sampling is the inverse CDF in vocabulary order with one supplied uniform:
 *   the smallest v with u*Z < P(v), P(v) = w[0] + ... + w[v]; if rounding leaves
 *   no such v the last v with w[v] > 0 is taken;  R6 one u_sample per request;
 *   R7 accepted_count = number of accepted drafts (0..gamma_b); out[0..k] holds
 *   the emitted tokens, later entries are -1;  R8 argmax ties go to the lowest
 *   index;  R9 T is per request, T == 0 selects greedy;  R10 greedy requests do
 *   not read draft logits or uniforms;  R11 the bonus uses target row gamma_b;
 *   R12 ragged requests use rows 0..gamma_b only.
 *
 * Near-boundary flags (for parity comparison, not part of the method):
 *   bit 0  some decided position i has |u_i - a_i| < 1e-6
 *   bit 1  u_sample lies within 1e-6 of an end of the sampled token's interval
 *          [C(v-1), C(v)) of the normalised CDF C = P / Z (P 修正分布の定義:
 *          the residual is sampled after normalisation)
 *   bit 2  the zero-residual-mass fallback was used
 *   bit 3  a top-p cut lies within 1e-6 (of the kept mass) of a value group
 *   bit 4  not bit 1, but the same distance measured in probability units,
 *          (u - C(v-1)) * Z or (C(v) - u) * Z, is below 1e-6: the residual's
 *          mass Z = sum of max(0, p - q) is so small that a break of its CDF
 *          moves by more than 1e-6 of Z when p - q is formed in single
 *          precision (an absolute error of a few 1e-8 per token).  Never set
 *          for a draw from p (Z = 1).
 * In a tree, a position's current target after rejections is
 * max(0, p - c q) / Z_j; bits 0 and 1 use the normalised bands above, and
 * bit 4 marks a uniform outside them but within 1e-6 once the distance is
 * multiplied by the current target's unnormalised mass (the product of the
 * normalisers Z_j so far).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "spec_verify_oracle.h"

#define BAND 1e-6

/* ------------------------------------------------------------------ input access */
static double widen(const void *base, int dtype, size_t idx)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[idx];
    /* bf16: the 16 stored bits are the top half of an fp32 value */
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

typedef struct {
    const void *base;
    int dtype;
    size_t off; /* element offset of the row */
    int V;
} row_t;

static double z_at(const row_t *r, int v) { return widen(r->base, r->dtype, r->off + (size_t)v); }

static row_t target_row(const void *t, int dtype, int gamma, int V, int b, int i)
{
    row_t r = {t, dtype, ((size_t)b * (size_t)(gamma + 1) + (size_t)i) * (size_t)V, V};
    return r;
}

static row_t draft_row(const void *d, int dtype, int gamma, int V, int b, int i)
{
    row_t r = {d, dtype, ((size_t)b * (size_t)gamma + (size_t)i) * (size_t)V, V};
    return r;
}

/* ------------------------------------------------------------------ softmax(z / T) */
/* m = max_v z[v];  e(v) = exp((z[v] - m) / T);  p(v) = e(v) / s, s = sum_v e(v).
 * Subtracting the maximum changes nothing mathematically and keeps exp finite.
 *
 * Optional filtering (top-k, then top-p), applied alike to every target and
 * draft row of a request: tau_k is the k-th largest logit; F(t) = sum of e(v)
 * over z[v] >= t; tau_p is the largest logit value t with
 * F(t) >= top_p * F(tau_k) (equal logits enter together).  Tokens with
 * z[v] < tau = max(tau_k, tau_p) get probability 0 and s sums the rest. */
typedef struct {
    double m, s, T, tau;
    int near_cut; /* the top-p cut lies within 1e-6 (of the kept mass) of a value group */
} softmax_t;

static int cmp_desc(const void *a, const void *b)
{
    double x = *(const double *)a, y = *(const double *)b;
    return (x < y) - (x > y);
}

static softmax_t softmax_stats(const row_t *r, double T, int top_k, double top_p)
{
    softmax_t st;
    st.T = T;
    st.tau = -INFINITY;
    st.near_cut = 0;
    st.m = z_at(r, 0);
    for (int v = 1; v < r->V; ++v) {
        double z = z_at(r, v);
        if (z > st.m) st.m = z;
    }
    const int use_k = top_k > 0 && top_k < r->V;
    const int use_p = top_p < 1.0;
    if (use_k || use_p) {
        double *zs = (double *)malloc(sizeof(double) * (size_t)r->V);
        for (int v = 0; v < r->V; ++v) zs[v] = z_at(r, v);
        qsort(zs, (size_t)r->V, sizeof(double), cmp_desc);
        double tau_k = use_k ? zs[top_k - 1] : -INFINITY;
        double tau = tau_k;
        if (use_p) {
            double Fk = 0.0;
            for (int v = 0; v < r->V; ++v)
                if (zs[v] >= tau_k) Fk += exp((zs[v] - st.m) / T);
            double target = top_p * Fk, cum = 0.0;
            int i = 0;
            while (i < r->V) {
                double t = zs[i], before = cum;
                while (i < r->V && zs[i] == t) cum += exp((zs[i++] - st.m) / T);
                if (cum >= target) {
                    if ((target - before) < 1e-6 * Fk || (cum - target) < 1e-6 * Fk) st.near_cut = 1;
                    if (t > tau) tau = t;
                    break;
                }
            }
        }
        st.tau = tau;
        free(zs);
    }
    st.s = 0.0;
    for (int v = 0; v < r->V; ++v) {
        double z = z_at(r, v);
        if (z >= st.tau) st.s += exp((z - st.m) / T);
    }
    return st;
}

static double prob(const row_t *r, const softmax_t *st, int v)
{
    double z = z_at(r, v);
    if (z < st->tau) return 0.0;
    return exp((z - st->m) / st->T) / st->s;
}

/* ------------------------------------------------------------------ argmax */
static int argmax_lowest(const row_t *r)
{
    int best = 0;
    double bz = z_at(r, 0);
    for (int v = 1; v < r->V; ++v) {
        double z = z_at(r, v);
        if (z > bz) { /* strict: equal values keep the earlier index */
            bz = z;
            best = v;
        }
    }
    return best;
}

/* ------------------------------------------------------------------ acceptance */
/* a = min(1, p(x) / q(x)), no epsilon guard. */
static double accept_probability(double px, double qx)
{
    if (qx == 0.0) return px > 0.0 ? 1.0 : 0.0;
    double ratio = px / qx;
    return ratio < 1.0 ? ratio : 1.0;
}

/* ------------------------------------------------------------------ inverse CDF */
/* Smallest v with u*Z < w[0] + ... + w[v]; Z = w[0] + ... + w[V-1].
 * Returns the token; writes Z and the distance of u from the ends of the chosen
 * token's normalised CDF interval. */
static int inverse_cdf(const double *w, int V, double u, double *Z_out, double *margin)
{
    double Z = 0.0;
    for (int v = 0; v < V; ++v) Z += w[v];
    *Z_out = Z;
    double target = u * Z;
    double acc = 0.0;
    int tok = -1;
    double lo = 0.0, hi = 0.0;
    for (int v = 0; v < V; ++v) {
        double before = acc;
        acc += w[v];
        if (target < acc) {
            tok = v;
            lo = before;
            hi = acc;
            break;
        }
    }
    if (tok < 0) { /* rounding left u*Z at or above the running total */
        for (int v = V - 1; v >= 0; --v)
            if (w[v] > 0.0) { tok = v; break; }
        if (tok < 0) tok = V - 1;
        *margin = 0.0;
        return tok;
    }
    double c_lo = lo / Z, c_hi = hi / Z;
    double m1 = u - c_lo, m2 = c_hi - u;
    *margin = m1 < m2 ? m1 : m2;
    return tok;
}

/* ------------------------------------------------------------------ one request */
static void verify_request(const oracle_args *a, int b, double *w)
{
    const int gamma = a->gamma, V = a->V, dt = a->dtype;
    const int g = a->lens ? a->lens[b] : gamma;
    const double T = (double)a->temperature[b];
    const int tk = a->top_k ? a->top_k[b] : 0;
    const double tp = a->top_p ? (double)a->top_p[b] : 1.0;
    const int nrows = 2 * gamma + 1;
    oracle_trace *tr = a->trace;
    int32_t *out = a->out_tokens + (size_t)b * (size_t)(gamma + 1);
    for (int i = 0; i <= gamma; ++i) out[i] = -1;
    int flags = 0;
    double acc_margin = INFINITY, cdf_margin = INFINITY, Zrep = NAN;

    if (T == 0.0) {
        /* greedy: accept while the draft equals the target arg-max */
        int tmax[ORACLE_GAMMA_MAX + 1];
        for (int i = 0; i <= g; ++i) {
            row_t r = target_row(a->target, dt, gamma, V, b, i);
            tmax[i] = argmax_lowest(&r);
            if (tr && tr->row_argmax) tr->row_argmax[(size_t)b * (gamma + 1) + i] = tmax[i];
        }
        int k = g;
        for (int i = 0; i < g; ++i) {
            if (a->draft_tokens[(size_t)b * gamma + i] != tmax[i]) { k = i; break; }
        }
        for (int i = 0; i < k; ++i) out[i] = a->draft_tokens[(size_t)b * gamma + i];
        out[k] = tmax[k];
        a->accepted_count[b] = k;
    } else {
        /* softmax statistics of every row the method uses */
        softmax_t sp[ORACLE_GAMMA_MAX + 1], sq[ORACLE_GAMMA_MAX];
        for (int i = 0; i <= g; ++i) {
            row_t r = target_row(a->target, dt, gamma, V, b, i);
            sp[i] = softmax_stats(&r, T, tk, tp);
            if (sp[i].near_cut) flags |= 8;
            if (tr && tr->row_max) tr->row_max[(size_t)b * nrows + i] = sp[i].m;
            if (tr && tr->row_sum) tr->row_sum[(size_t)b * nrows + i] = sp[i].s;
        }
        for (int i = 0; i < g; ++i) {
            row_t r = draft_row(a->draft, dt, gamma, V, b, i);
            sq[i] = softmax_stats(&r, T, tk, tp);
            if (sq[i].near_cut) flags |= 8;
            if (tr && tr->row_max) tr->row_max[(size_t)b * nrows + gamma + 1 + i] = sq[i].m;
            if (tr && tr->row_sum) tr->row_sum[(size_t)b * nrows + gamma + 1 + i] = sq[i].s;
        }
        /* accept / reject in order; stop at the first rejection */
        int k = g;
        for (int i = 0; i < g; ++i) {
            int x = a->draft_tokens[(size_t)b * gamma + i];
            row_t rp = target_row(a->target, dt, gamma, V, b, i);
            row_t rq = draft_row(a->draft, dt, gamma, V, b, i);
            double px = prob(&rp, &sp[i], x);
            double qx = prob(&rq, &sq[i], x);
            double ai = accept_probability(px, qx);
            double u = (double)a->u_accept[(size_t)b * gamma + i];
            if (tr && tr->p_draft) tr->p_draft[(size_t)b * gamma + i] = px;
            if (tr && tr->q_draft) tr->q_draft[(size_t)b * gamma + i] = qx;
            if (tr && tr->accept_prob) tr->accept_prob[(size_t)b * gamma + i] = ai;
            double d = fabs(u - ai);
            if (d < acc_margin) acc_margin = d;
            if (!(u < ai)) { k = i; break; }
        }
        for (int i = 0; i < k; ++i) out[i] = a->draft_tokens[(size_t)b * gamma + i];
        a->accepted_count[b] = k;

        /* the distribution of the emitted token at position k */
        row_t rp = target_row(a->target, dt, gamma, V, b, k);
        if (k < g) {
            row_t rq = draft_row(a->draft, dt, gamma, V, b, k);
            for (int v = 0; v < V; ++v) {
                double diff = prob(&rp, &sp[k], v) - prob(&rq, &sq[k], v);
                w[v] = diff > 0.0 ? diff : 0.0;
            }
        } else {
            for (int v = 0; v < V; ++v) w[v] = prob(&rp, &sp[k], v);
        }
        double Z = 0.0;
        for (int v = 0; v < V; ++v) Z += w[v];
        if (Z == 0.0) { /* fallback to p_k */
            flags |= 4;
            for (int v = 0; v < V; ++v) w[v] = prob(&rp, &sp[k], v);
        }
        double m;
        out[k] = inverse_cdf(w, V, (double)a->u_sample[b], &Zrep, &m);
        cdf_margin = m;
        if (m < BAND) flags |= 2;              /* normalised CDF band */
        else if (m * Zrep < BAND) flags |= 16; /* the same band in probability units */
        if (acc_margin < BAND) flags |= 1;
    }
    if (tr && tr->residual_mass) tr->residual_mass[b] = Zrep;
    if (tr && tr->flags) tr->flags[b] = flags;
    if (tr && tr->accept_margin) tr->accept_margin[b] = acc_margin;
    if (tr && tr->cdf_margin) tr->cdf_margin[b] = cdf_margin;
}

/* ------------------------------------------------------------------ entry point */
int oracle_spec_verify(const oracle_args *a)
{
    if (!a || !a->target || !a->out_tokens || !a->accepted_count || !a->u_sample || !a->temperature)
        return -1;
    if (a->B < 1 || a->gamma < 0 || a->gamma > ORACLE_GAMMA_MAX || a->V < 1) return -1;
    if (a->dtype != ORACLE_F32 && a->dtype != ORACLE_BF16) return -1;
    if (a->gamma > 0 && !a->draft_tokens) return -1;
    for (int b = 0; b < a->B; ++b) {
        float T = a->temperature[b];
        int g = a->lens ? a->lens[b] : a->gamma;
        if (!(T >= 0.0f) || isinf(T)) return -1;
        if (g < 0 || g > a->gamma) return -1;
        if (T > 0.0f && g > 0 && (!a->draft || !a->u_accept)) return -1;
        if (a->top_k && a->top_k[b] < 0) return -1;
        if (a->top_p && !(a->top_p[b] > 0.0f && a->top_p[b] <= 1.0f)) return -1;
        for (int i = 0; i < g; ++i) {
            int x = a->draft_tokens[(size_t)b * a->gamma + i];
            if (x < 0 || x >= a->V) return -1;
        }
    }
    double *w = (double *)malloc(sizeof(double) * (size_t)a->V);
    if (!w) return -2;
    for (int b = 0; b < a->B; ++b) verify_request(a, b, w);
    free(w);
    return 0;
}

/* ================================================================== tree verification */
/* Verification of a tree of drafts (several candidates per position).
 *
 * The pages draw the tree (P4, section Eagleツリー推測の原理: several candidate
 * paths verified together) but verify it with a lossy probability threshold,
 * so the lossless rule used here is a reading: the children of a position were
 * drawn independently from that position's draft distribution q, and they are
 * tested in increasing node index, each against the current target: the first
 * child against p, and after a rejection the next child against the modified
 * distribution max(0, p_cur - q) / sum (P1 section 修正分布の定義 applied again,
 * with the position's q).  The first accepted child is emitted and verification
 * continues at its position; if every child is rejected, or the position has no
 * child, the token is drawn from the current target by the inverse CDF (R5)
 * with u_sample.  One child per position is exactly the linear method.  T == 0
 * accepts the first child equal to the target arg-max and emits the arg-max
 * otherwise.
 *
 * Layout: node n (0 <= n < N_b) has parent[n] in [-1, n) (-1: the verified
 * prefix) and token[n].  Position 0 is the prefix, position n + 1 is node n.
 * target [B][max_nodes + 1][V]: row j is the target at position j.
 * draft  [B][max_nodes][V]: row j is the q the children of position j were drawn
 * from (a position with children is the prefix or a node n < N_b - 1, so j < N_b).
 */
static void verify_tree_request(const oracle_tree_args *a, int b, double *p, double *q, double *cur)
{
    const int Nmax = a->max_nodes, V = a->V, dt = a->dtype;
    const int N = a->num_nodes ? a->num_nodes[b] : Nmax;
    const double T = (double)a->temperature[b];
    const int32_t *parent = a->parent + (size_t)b * Nmax;
    const int32_t *token = a->tokens + (size_t)b * Nmax;
    int32_t *out = a->out_tokens + (size_t)b * (Nmax + 1);
    int32_t *onodes = a->out_nodes + (size_t)b * Nmax;
    for (int i = 0; i <= Nmax; ++i) out[i] = -1;
    for (int i = 0; i < Nmax; ++i) onodes[i] = -1;
    int flags = 0;
    int depth = 0, pos = 0;
    for (;;) {
        row_t rp = {a->target, dt, ((size_t)b * (size_t)(Nmax + 1) + (size_t)pos) * (size_t)V, V};
        if (T == 0.0) {
            int am = argmax_lowest(&rp), hit = -1;
            for (int n = pos; n < N; ++n)
                if (parent[n] == pos - 1 && token[n] == am) { hit = n; break; }
            if (hit < 0) { out[depth] = am; break; }
            out[depth] = am;
            onodes[depth] = hit;
            ++depth;
            pos = hit + 1;
            continue;
        }
        softmax_t sp = softmax_stats(&rp, T, 0, 1.0);
        for (int v = 0; v < V; ++v) { p[v] = prob(&rp, &sp, v); cur[v] = p[v]; }
        /* cur's unnormalised mass in probability units (the product of the
         * normalisers so far): bit 4 measures the bands in these units */
        double scale = 1.0;
        int hit = -1, have_q = 0;
        for (int n = pos; n < N && hit < 0; ++n) {
            if (parent[n] != pos - 1) continue;
            if (!have_q) {
                row_t rq = {a->draft, dt, ((size_t)b * (size_t)Nmax + (size_t)pos) * (size_t)V, V};
                softmax_t sq = softmax_stats(&rq, T, 0, 1.0);
                for (int v = 0; v < V; ++v) q[v] = prob(&rq, &sq, v);
                have_q = 1;
            }
            const int x = token[n];
            const double an = accept_probability(cur[x], q[x]);
            const double u = (double)a->u_accept[(size_t)b * Nmax + n];
            if (fabs(u - an) < BAND) flags |= 1;
            else if (fabs(u - an) * scale < BAND) flags |= 16;
            if (u < an) { hit = n; break; }
            /* rejected: the next child is tested against max(0, cur - q) / sum */
            double Z = 0.0;
            for (int v = 0; v < V; ++v) {
                double d = cur[v] - q[v];
                cur[v] = d > 0.0 ? d : 0.0;
                Z += cur[v];
            }
            if (Z == 0.0) { /* fallback to the position's p, as in the linear case */
                for (int v = 0; v < V; ++v) cur[v] = p[v];
                flags |= 4;
                scale = 1.0;
            } else {
                for (int v = 0; v < V; ++v) cur[v] /= Z;
                scale *= Z;
            }
        }
        if (hit >= 0) {
            out[depth] = token[hit];
            onodes[depth] = hit;
            ++depth;
            pos = hit + 1;
            continue;
        }
        double Zc, margin;
        out[depth] = inverse_cdf(cur, V, (double)a->u_sample[b], &Zc, &margin);
        if (margin < BAND) flags |= 2;
        else if (margin * scale < BAND) flags |= 16;
        break;
    }
    a->accepted_count[b] = depth;
    if (a->flags) a->flags[b] = flags;
}

int oracle_spec_verify_tree(const oracle_tree_args *a)
{
    if (!a || !a->target || !a->parent || !a->tokens || !a->u_sample || !a->temperature || !a->out_tokens ||
        !a->out_nodes || !a->accepted_count)
        return -1;
    if (a->B < 1 || a->max_nodes < 0 || a->V < 1) return -1;
    if (a->dtype != ORACLE_F32 && a->dtype != ORACLE_BF16) return -1;
    for (int b = 0; b < a->B; ++b) {
        const float T = a->temperature[b];
        const int N = a->num_nodes ? a->num_nodes[b] : a->max_nodes;
        if (!(T >= 0.0f) || isinf(T)) return -1;
        if (N < 0 || N > a->max_nodes) return -1;
        if (T > 0.0f && N > 0 && (!a->draft || !a->u_accept)) return -1;
        for (int n = 0; n < N; ++n) {
            const int pa = a->parent[(size_t)b * a->max_nodes + n], x = a->tokens[(size_t)b * a->max_nodes + n];
            if (pa < -1 || pa >= n || x < 0 || x >= a->V) return -1;
        }
    }
    double *buf = (double *)malloc(sizeof(double) * 3 * (size_t)a->V);
    if (!buf) return -2;
    for (int b = 0; b < a->B; ++b) verify_tree_request(a, b, buf, buf + a->V, buf + 2 * (size_t)a->V);
    free(buf);
    return 0;
}
