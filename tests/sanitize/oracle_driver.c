/*
 * oracle_driver.c -- runs the CPU oracle (test infrastructure) over seeded
 * random cases with every buffer allocated to its exact size, for a build
 * under AddressSanitizer and UndefinedBehaviorSanitizer.  It checks memory
 * safety and a few structural facts of the outputs, not the values (those
 * are pinned by the Python oracle tests).  Exit status 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "spec_verify_oracle.h"

static uint64_t rng_state;

static uint64_t next_u64(void) { /* splitmix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static double uniform01(void) { return (double)(next_u64() >> 11) * (1.0 / 9007199254740992.0); }

static float logit(double scale) { /* roughly normal: sum of four uniforms */
    double s = uniform01() + uniform01() + uniform01() + uniform01() - 2.0;
    return (float)(scale * s * 1.7);
}

static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static void fill_logits(void *dst, size_t n, int dtype, double scale, int poison_every) {
    for (size_t i = 0; i < n; ++i) {
        float z = logit(scale);
        if (poison_every && (i % (size_t)poison_every) == 0) z = -INFINITY;
        if (dtype == ORACLE_F32) {
            ((float *)dst)[i] = z;
        } else {
            uint32_t bits;
            memcpy(&bits, &z, 4);
            ((uint16_t *)dst)[i] = (uint16_t)(bits >> 16);
        }
    }
}

static int failures = 0;

static void expect(int cond, const char *what, int case_id) {
    if (!cond) {
        fprintf(stderr, "case %d: %s\n", case_id, what);
        ++failures;
    }
}

static void linear_case(int id, int B, int gamma, int V, int dtype, int ragged, int mixed_T, int filt) {
    const size_t elt = dtype == ORACLE_F32 ? 4 : 2;
    const size_t nt = (size_t)B * (gamma + 1) * V, nd = (size_t)B * gamma * V;
    void *target = xmalloc(nt * elt), *draft = xmalloc(nd * elt);
    fill_logits(target, nt, dtype, 3.0, id % 3 == 0 ? 97 : 0);
    fill_logits(draft, nd, dtype, 3.0, 0);
    int32_t *tokens = xmalloc(sizeof(int32_t) * (size_t)B * gamma);
    float *ua = xmalloc(sizeof(float) * (size_t)B * gamma), *us = xmalloc(sizeof(float) * (size_t)B);
    float *T = xmalloc(sizeof(float) * (size_t)B);
    int32_t *lens = ragged ? xmalloc(sizeof(int32_t) * (size_t)B) : NULL;
    int32_t *topk = filt ? xmalloc(sizeof(int32_t) * (size_t)B) : NULL;
    float *topp = filt ? xmalloc(sizeof(float) * (size_t)B) : NULL;
    for (int b = 0; b < B; ++b) {
        us[b] = (float)uniform01();
        T[b] = mixed_T ? (float)((next_u64() % 3) * 0.5) : 1.0f;
        if (lens) lens[b] = (int32_t)(next_u64() % (uint64_t)(gamma + 1));
        if (topk) topk[b] = (int32_t)(next_u64() % (uint64_t)(V + 2));  /* 0 and >= V: off */
        if (topp) topp[b] = (float)(1.0 - 0.999 * uniform01());         /* (0, 1], 1: off */
        for (int i = 0; i < gamma; ++i) {
            tokens[(size_t)b * gamma + i] = (int32_t)(next_u64() % (uint64_t)V);
            ua[(size_t)b * gamma + i] = (float)uniform01();
        }
    }
    int32_t *count = xmalloc(sizeof(int32_t) * (size_t)B), *out = xmalloc(sizeof(int32_t) * (size_t)B * (gamma + 1));
    const size_t rows = (size_t)B * (2 * gamma + 1);
    oracle_trace tr;
    tr.p_draft = xmalloc(sizeof(double) * (size_t)B * gamma);
    tr.q_draft = xmalloc(sizeof(double) * (size_t)B * gamma);
    tr.accept_prob = xmalloc(sizeof(double) * (size_t)B * gamma);
    tr.row_max = xmalloc(sizeof(double) * rows);
    tr.row_sum = xmalloc(sizeof(double) * rows);
    tr.row_argmax = xmalloc(sizeof(int32_t) * (size_t)B * (gamma + 1));
    tr.residual_mass = xmalloc(sizeof(double) * (size_t)B);
    tr.flags = xmalloc(sizeof(int32_t) * (size_t)B);
    tr.accept_margin = xmalloc(sizeof(double) * (size_t)B);
    tr.cdf_margin = xmalloc(sizeof(double) * (size_t)B);
    oracle_args a;
    memset(&a, 0, sizeof a);
    a.target = target;
    a.draft = draft;
    a.dtype = dtype;
    a.draft_tokens = tokens;
    a.u_accept = ua;
    a.u_sample = us;
    a.temperature = T;
    a.lens = lens;
    a.top_k = topk;
    a.top_p = topp;
    a.B = B;
    a.gamma = gamma;
    a.V = V;
    a.accepted_count = count;
    a.out_tokens = out;
    a.trace = (id % 2) ? &tr : NULL;
    const int rc = oracle_spec_verify(&a);
    expect(rc == 0, "oracle_spec_verify failed", id);
    for (int b = 0; rc == 0 && b < B; ++b) {
        const int g = lens ? lens[b] : gamma;
        expect(count[b] >= 0 && count[b] <= g, "accepted count outside [0, g]", id);
        const int32_t tok = out[(size_t)b * (gamma + 1) + count[b]];
        expect(tok >= 0 && tok < V, "emitted token outside the vocabulary", id);
        for (int t = count[b] + 1; t <= gamma; ++t) expect(out[(size_t)b * (gamma + 1) + t] == -1, "padding", id);
    }
    free(target);
    free(draft);
    free(tokens);
    free(ua);
    free(us);
    free(T);
    free(lens);
    free(topk);
    free(topp);
    free(count);
    free(out);
    free(tr.p_draft);
    free(tr.q_draft);
    free(tr.accept_prob);
    free(tr.row_max);
    free(tr.row_sum);
    free(tr.row_argmax);
    free(tr.residual_mass);
    free(tr.flags);
    free(tr.accept_margin);
    free(tr.cdf_margin);
}

static void tree_case(int id, int B, int N, int V, int dtype) {
    const size_t elt = dtype == ORACLE_F32 ? 4 : 2;
    const size_t nt = (size_t)B * (N + 1) * V, nd = (size_t)B * N * V;
    void *target = xmalloc(nt * elt), *draft = xmalloc(nd * elt);
    fill_logits(target, nt, dtype, 2.5, 0);
    fill_logits(draft, nd, dtype, 2.5, 0);
    int32_t *parent = xmalloc(sizeof(int32_t) * (size_t)B * N), *tok = xmalloc(sizeof(int32_t) * (size_t)B * N);
    int32_t *nn = xmalloc(sizeof(int32_t) * (size_t)B);
    float *ua = xmalloc(sizeof(float) * (size_t)B * N), *us = xmalloc(sizeof(float) * (size_t)B);
    float *T = xmalloc(sizeof(float) * (size_t)B);
    for (int b = 0; b < B; ++b) {
        nn[b] = (int32_t)(next_u64() % (uint64_t)(N + 1));
        us[b] = (float)uniform01();
        T[b] = (float)((next_u64() % 3) * 0.6);
        for (int n = 0; n < N; ++n) {
            parent[(size_t)b * N + n] = n == 0 ? -1 : (int32_t)(next_u64() % (uint64_t)(n + 1)) - 1;
            tok[(size_t)b * N + n] = (int32_t)(next_u64() % (uint64_t)V);
            ua[(size_t)b * N + n] = (float)uniform01();
        }
    }
    int32_t *count = xmalloc(sizeof(int32_t) * (size_t)B), *out = xmalloc(sizeof(int32_t) * (size_t)B * (N + 1));
    int32_t *nodes = xmalloc(sizeof(int32_t) * (size_t)B * N), *flags = xmalloc(sizeof(int32_t) * (size_t)B);
    oracle_tree_args a;
    memset(&a, 0, sizeof a);
    a.target = target;
    a.draft = draft;
    a.dtype = dtype;
    a.parent = parent;
    a.tokens = tok;
    a.num_nodes = nn;
    a.u_accept = ua;
    a.u_sample = us;
    a.temperature = T;
    a.B = B;
    a.max_nodes = N;
    a.V = V;
    a.accepted_count = count;
    a.out_tokens = out;
    a.out_nodes = nodes;
    a.flags = flags;
    const int rc = oracle_spec_verify_tree(&a);
    expect(rc == 0, "oracle_spec_verify_tree failed", id);
    for (int b = 0; rc == 0 && b < B; ++b) expect(count[b] >= 0 && count[b] <= nn[b], "tree path length", id);
    free(target);
    free(draft);
    free(parent);
    free(tok);
    free(nn);
    free(ua);
    free(us);
    free(T);
    free(count);
    free(out);
    free(nodes);
    free(flags);
}

int main(void) {
    rng_state = 20261202u;
    int id = 0;
    static const int shapes[][3] = {{1, 0, 1}, {3, 1, 1}, {2, 4, 7}, {4, 8, 64}, {2, 31, 33}, {3, 5, 1000}, {2, 3, 4099}};
    for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s)
        for (int dtype = 0; dtype < 2; ++dtype)
            for (int variant = 0; variant < 4; ++variant)
                linear_case(id++, shapes[s][0], shapes[s][1], shapes[s][2], dtype, variant & 1, variant >= 2,
                            variant == 3);
    for (int dtype = 0; dtype < 2; ++dtype) {
        tree_case(id++, 3, 1, 50, dtype);
        tree_case(id++, 4, 12, 300, dtype);
        tree_case(id++, 2, 40, 97, dtype);
    }
    /* invalid arguments are rejected before anything is computed */
    oracle_args bad;
    memset(&bad, 0, sizeof bad);
    bad.B = 1;
    bad.gamma = 1;
    bad.V = 4;
    expect(oracle_spec_verify(&bad) == -1, "NULL arrays accepted", id++);
    bad.gamma = ORACLE_GAMMA_MAX + 1;
    expect(oracle_spec_verify(&bad) == -1, "gamma above the maximum accepted", id++);
    {
        float target[2 * 4] = {0}, draft[4] = {0}, ua[1] = {0.5f}, us[1] = {0.5f}, T[1] = {1.0f}, tp[1] = {1.5f};
        int32_t tok[1] = {4}, tk[1] = {-1}, cnt[1], out[2];
        oracle_args a;
        memset(&a, 0, sizeof a);
        a.target = target;
        a.draft = draft;
        a.dtype = ORACLE_F32;
        a.draft_tokens = tok;
        a.u_accept = ua;
        a.u_sample = us;
        a.temperature = T;
        a.B = 1;
        a.gamma = 1;
        a.V = 4;
        a.accepted_count = cnt;
        a.out_tokens = out;
        expect(oracle_spec_verify(&a) == -1, "draft id outside the vocabulary accepted", id++);
        tok[0] = 1;
        expect(oracle_spec_verify(&a) == 0, "a valid call rejected", id++);
        a.top_k = tk;
        expect(oracle_spec_verify(&a) == -1, "negative top_k accepted", id++);
        a.top_k = NULL;
        a.top_p = tp;
        expect(oracle_spec_verify(&a) == -1, "top_p above 1 accepted", id++);
    }
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("oracle driver: %d cases ok\n", id);
    return 0;
}
