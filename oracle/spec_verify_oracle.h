/*
 * spec_verify_oracle.h -- interface of the plain CPU oracle (test infrastructure
 * only; the GPU library neither includes nor links this file).
 */
#ifndef SPEC_VERIFY_ORACLE_H
#define SPEC_VERIFY_ORACLE_H

#include <stdint.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_GAMMA_MAX 32

typedef struct {
    /* every pointer may be NULL; sizes in elements */
    double *p_draft;       /* [B*gamma] p_i(x_i); untouched where not evaluated      */
    double *q_draft;       /* [B*gamma] q_i(x_i)                                     */
    double *accept_prob;   /* [B*gamma] min(1, p/q)                                  */
    double *row_max;       /* [B*(2*gamma+1)] target rows 0..gamma, then draft rows  */
    double *row_sum;       /* [B*(2*gamma+1)] sum_v exp((z - max)/T)                 */
    int32_t *row_argmax;   /* [B*(gamma+1)] greedy target rows                       */
    double *residual_mass; /* [B] mass of the sampled distribution (NaN if greedy)   */
    int32_t *flags;        /* [B] bit0 accept band, bit1 normalised CDF band,
                              bit2 fallback, bit3 a top-p cut within the band,
                              bit4 CDF band in probability units only          */
    double *accept_margin; /* [B] min |u_i - a_i| over decided positions             */
    double *cdf_margin;    /* [B] distance of u_sample from its CDF interval's ends  */
} oracle_trace;

typedef struct {
    const void *target;          /* [B][gamma+1][V] fp32 or bf16 bits, row-major      */
    const void *draft;           /* [B][gamma][V]                                     */
    int dtype;                   /* ORACLE_F32 / ORACLE_BF16                          */
    const int32_t *draft_tokens; /* [B][gamma]                                        */
    const float *u_accept;       /* [B][gamma]                                        */
    const float *u_sample;       /* [B]                                               */
    const float *temperature;    /* [B], 0 = greedy request                           */
    const int32_t *lens;         /* [B] draft lengths or NULL (= gamma)               */
    const int32_t *top_k;        /* [B] keep the k largest logits (0 or >= V: off), or NULL */
    const float *top_p;          /* [B] keep the top mass fraction p (>= 1: off), or NULL  */
    int B, gamma, V;
    int32_t *accepted_count;     /* out [B]                                           */
    int32_t *out_tokens;         /* out [B][gamma+1]                                  */
    oracle_trace *trace;         /* optional                                          */
} oracle_args;

/* 0 on success, -1 invalid arguments, -2 out of memory. */
int oracle_spec_verify(const oracle_args *a);

/* Tree of drafts (see the comment above verify_tree_request). */
typedef struct {
    const void *target;          /* [B][max_nodes+1][V]: row j = target at position j   */
    const void *draft;           /* [B][max_nodes][V]: row j = q at position j           */
    int dtype;
    const int32_t *parent;       /* [B][max_nodes], -1 = the prefix, else < n            */
    const int32_t *tokens;       /* [B][max_nodes]                                       */
    const int32_t *num_nodes;    /* [B] or NULL (= max_nodes)                            */
    const float *u_accept;       /* [B][max_nodes], one per node                         */
    const float *u_sample;       /* [B]                                                  */
    const float *temperature;    /* [B], 0 = greedy                                      */
    int B, max_nodes, V;
    int32_t *accepted_count;     /* out [B]: nodes on the accepted path                  */
    int32_t *out_tokens;         /* out [B][max_nodes+1]: path tokens, then the drawn one */
    int32_t *out_nodes;          /* out [B][max_nodes]: path node indices, -1 after      */
    int32_t *flags;              /* out [B] or NULL: bit0 accept band, bit1 CDF band,
                                    bit2 zero-mass fallback, bit4 a band in units of
                                    the current target's unnormalised mass only     */
} oracle_tree_args;

int oracle_spec_verify_tree(const oracle_tree_args *a);

#endif
