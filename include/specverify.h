/*
 * specverify.h -- C ABI of libspecverify, the verify step of speculative
 * sampling (modified rejection sampling) on AMD MI355X (gfx950).
 *
 * What one call computes, per request b of a batch of B (the pages:
 *   [P1] "Speculative Decoding（投機的デコーディング）— 小さなモデルでLLM推論を高速化する",
 *   [P2] "論文解説: Fast Inference from Transformers via Speculative Decoding",
 *   [P3] "投機的デコーディングとは：同時リクエストが多いと遅くなる理由",
 *   [P4] "LLM推測デコーディング最適化実踐"):
 *
 *   1. p_i = softmax(z_p[b,i,:] / T) for the gamma_b+1 target rows and
 *      q_i = softmax(z_q[b,i,:] / T) for the gamma_b draft rows, one T for both
 *      (P2 code sketch; P4 section 検証アルゴリズムの実装).
 *   2. draft token x_i is accepted iff u_accept[b,i] < min(1, p_i(x_i)/q_i(x_i))
 *      (P1 section ステップ3: 受理・棄却判定; P2 section 投機的サンプリング
 *      アルゴリズム, accept equation).
 *   3. k = index of the first rejection (gamma_b if none); drafts 0..k-1 are
 *      emitted, later drafts are discarded (P1 section ステップ3).
 *   4. if k < gamma_b the token at position k is drawn from
 *      max(0, p_k - q_k) / sum max(0, p_k - q_k) (P1 section 修正分布の定義;
 *      P2 modified-distribution equation); if that mass is exactly zero the draw
 *      falls back to p_k (P1 simulation code).  If k == gamma_b a bonus token
 *      is drawn from p_{gamma_b} (P1 section ステップ3; P4 bonus draw).
 *      The draw is the inverse CDF in vocabulary order with the one supplied
 *      uniform u_sample[b]: the smallest v with u*Z < w[0] + ... + w[v].
 *   5. T == 0 selects greedy verification: x_i is accepted iff it equals the
 *      lowest-index arg-max of target row i, and the token at position k is the
 *      arg-max of target row k (P2 section 実装のポイント; P3 worked example in
 *      section 先読みは、一回の順伝播で進むトークンを増やす).  Greedy requests
 *      read neither draft logits nor uniforms.
 *
 * Outputs: accepted_count[b] = k (number of accepted drafts, 0..gamma_b);
 * out_tokens[b][0..k] = the k accepted drafts followed by the sampled token;
 * out_tokens[b][k+1..gamma] = -1.
 *
 * Conventions for every entry point:
 *   - Pointers named *_logits, draft_tokens, u_*, accepted_count, out_tokens,
 *     workspace and the temperature / draft_lens / top_k / top_p arrays are
 *     DEVICE pointers (hipMalloc'd or torch tensors on the GPU).  The caller
 *     owns all of them; the library allocates nothing and keeps no state.
 *   - Layouts are dense row-major: target_logits [B][gamma+1][V],
 *     draft_logits [B][gamma][V], draft_tokens / u_accept [B][gamma],
 *     u_sample / accepted_count [B], out_tokens [B][gamma+1].  Logits may be
 *     any element-aligned address; 16-byte aligned rows take the fast path.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and the call returns without synchronising.  Outputs are valid once the
 *     stream reaches that point.
 *   - Arguments are checked on the host before anything is enqueued; a failed
 *     check returns SV_EINVAL / SV_EWORKSPACE and touches nothing.  A failed
 *     launch returns SV_EHIP.  Values that live in device memory (uniforms in
 *     [0, 1), per-request T >= 0 and finite) are the caller's contract and are
 *     not checked; memory safety does not depend on them.  For T > 0 every
 *     row's scaled maximum |max(z) * log2(e) / T| must stay below 2^28 (for
 *     example T >= 1e-5 with |z| <= 1000; the tests run T from 1e-3 to 50 with
 *     logits up to about 150 in magnitude).  A draft length
 *     outside [0, gamma] is clamped to that range, and a draft token id outside
 *     [0, V) is treated as rejected at its position.  Logits must be finite on
 *     every row that the method reads (padding rows of ragged requests are
 *     never read and may hold anything).
 *   - Two calls may run concurrently only with distinct workspaces.
 *   - Results are deterministic: identical inputs give bit-identical outputs.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element type of the logits */
typedef enum { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

/* return codes */
enum {
    SV_OK = 0,
    SV_EINVAL = -1,     /* bad pointer, size, dtype or temperature           */
    SV_EWORKSPACE = -2, /* workspace NULL, misaligned (256 B) or too small    */
    SV_EHIP = -3,       /* a HIP launch or runtime call failed                */
    SV_ESCRATCH = -4    /* spec_verify_noalloc: the call needs more scratch
                           than SV_NOALLOC_SCRATCH_BYTES                     */
};

/* largest supported draft length gamma */
#define SV_GAMMA_MAX 32

/* Bytes of device workspace one call with these sizes needs (0 if the sizes are
 * invalid).  The workspace must be 256-byte aligned; its contents on entry do
 * not matter. */
size_t spec_verify_workspace_bytes(int B, int gamma, int V, int dtype);

/* Uniform batch: every request has gamma drafts and the same temperature.
 * temperature: host scalar, >= 0 and finite; 0 = greedy for every request
 *   (then draft_logits and u_accept may be NULL).
 * B >= 1, 0 <= gamma <= SV_GAMMA_MAX, V >= 1, dtype one of sv_dtype. */
int spec_verify(const void *target_logits, const void *draft_logits,
                const int32_t *draft_tokens, const float *u_accept,
                const float *u_sample, float temperature, int B, int gamma,
                int V, int dtype, int32_t *accepted_count,
                int32_t *out_tokens, void *workspace, size_t workspace_bytes,
                void *stream);

/* Optional per-call diagnostics for tests and profiling (device pointers, any
 * may be NULL; pass a NULL sv_debug in timed runs).  Entries that a request
 * does not produce (e.g. draft probabilities of greedy requests, positions
 * after the first rejection) are left untouched. */
typedef struct {
    double *p_draft;       /* [B][gamma] p_i(x_i)                                   */
    double *q_draft;       /* [B][gamma] q_i(x_i)                                   */
    double *accept_prob;   /* [B][gamma] min(1, p_i(x_i)/q_i(x_i))                   */
    float *row_max;        /* [B][2*gamma+1] max logit; target rows 0..gamma first   */
    double *row_sum;       /* [B][2*gamma+1] sum_v exp((z_v - max)/T)                */
    int32_t *row_argmax;   /* [B][gamma+1] lowest-index arg-max of greedy target rows */
    double *residual_mass; /* [B] Z, the mass of the distribution sampled at k       */
    void *k1_events[2];    /* hipEvent_t pair recorded around the row-statistics
                              kernel on `stream` (both or neither; the one-workgroup
                              kernel of a small request, which is the whole step)  */
} sv_debug;

/* spec_verify with diagnostics (dbg may be NULL): the same kernels as
 * spec_verify (one host temperature for the batch), so that k1_events time the
 * row-statistics kernel the uniform entry point runs (the one-workgroup kernel
 * for requests of at most 12288 logits, where the step is that one kernel).
 * Arguments, layouts and errors as spec_verify and spec_verify_ex. */
int spec_verify_dbg(const void *target_logits, const void *draft_logits,
                    const int32_t *draft_tokens, const float *u_accept,
                    const float *u_sample, float temperature, int B, int gamma,
                    int V, int dtype, int32_t *accepted_count,
                    int32_t *out_tokens, void *workspace, size_t workspace_bytes,
                    void *stream, const sv_debug *dbg);

/* Ragged / mixed batch.
 * temperature: DEVICE array [B]; 0 = greedy request, else > 0 and finite.
 * draft_lens:  DEVICE array [B] of gamma_b in [0, gamma], or NULL (= gamma);
 *              gamma is then the padding stride of the draft dimension.
 * dbg: NULL or diagnostics as above.
 * draft_logits and u_accept must be non-NULL when gamma > 0 (greedy requests
 * do not read them). */
int spec_verify_ex(const void *target_logits, const void *draft_logits,
                   const int32_t *draft_tokens, const float *u_accept,
                   const float *u_sample, const float *temperature,
                   const int32_t *draft_lens, int B, int gamma, int V,
                   int dtype, int32_t *accepted_count, int32_t *out_tokens,
                   void *workspace, size_t workspace_bytes, void *stream,
                   const sv_debug *dbg);

/* Largest vocabulary accepted by spec_verify_filtered: the filter's masses are
 * 64-bit fixed-point integers with 61 - ceil(log2 V) fractional bits, so a row's
 * truncation loss stays below 2^-21 of its top token's mass. */
#define SV_FILTER_MAX_V (1 << 20)

/* Top-k / top-p filtered verification: spec_verify_ex with every target and
 * draft row of a filtered request truncated before steps 2-4.  The pages name
 * top_p only as a serving parameter (P4, section vLLM推測デコーディング設定:
 * temperature 0.7 with top_p 0.9) and give no rule; the rule used here is:
 *   - temperature first, then top-k, then top-p, the same cut on every row of
 *     the request (target and draft alike);
 *   - top-k keeps the tokens whose logit is >= the k-th largest logit of the
 *     row (equal logits are kept together, so ties can keep more than k);
 *   - top-p then keeps the tokens whose logit is >= the largest logit value t
 *     such that the tokens with logit >= t hold at least a fraction top_p of
 *     the probability that top-k kept (equal logits enter and leave together);
 *   - p_i, q_i are renormalised over the kept tokens; a cut token has
 *     probability 0, and a draft token with q_i(x) = 0 is accepted iff
 *     p_i(x) > 0.  Residual, bonus and fallback use the renormalised rows.
 * top_k: DEVICE [B] or NULL; k in [1, V-1] filters, any other value (0, >= V,
 *        negative) leaves top-k off for that request.
 * top_p: DEVICE [B] or NULL; p in (0, 1) filters, any other value (1, <= 0,
 *        > 1, NaN) leaves top-p off for that request.
 * Greedy requests (T == 0) ignore both: the arg-max is never cut.  With both
 * arrays NULL this is spec_verify_ex.  V <= SV_FILTER_MAX_V when either array is
 * given (else SV_EINVAL).  Stochastic rows of filtered requests must not hold
 * NaN.  The workspace is sized by spec_verify_filtered_workspace_bytes (larger
 * than spec_verify_workspace_bytes: it holds the filter's per-row candidate
 * lists); the other arguments are those of spec_verify_ex.  Diagnostics report
 * the filtered quantities: row_sum is the kept mass, p_draft / q_draft the
 * renormalised probabilities. */
/* Bytes of device workspace one spec_verify_filtered call with these sizes
 * needs (0 if the sizes are invalid or V > SV_FILTER_MAX_V); 256-byte aligned,
 * contents on entry do not matter. */
size_t spec_verify_filtered_workspace_bytes(int B, int gamma, int V, int dtype);

int spec_verify_filtered(const void *target_logits, const void *draft_logits,
                         const int32_t *draft_tokens, const float *u_accept,
                         const float *u_sample, const float *temperature,
                         const int32_t *draft_lens, const int32_t *top_k,
                         const float *top_p, int B, int gamma, int V, int dtype,
                         int32_t *accepted_count, int32_t *out_tokens,
                         void *workspace, size_t workspace_bytes, void *stream,
                         const sv_debug *dbg);

/* Largest tree and vocabulary accepted by spec_verify_tree. */
#define SV_TREE_MAX_NODES 256
#define SV_TREE_MAX_V (1 << 20)

/* Tree (multi-candidate) verification.  The pages draw a tree of drafts (P4,
 * section Eagleツリー推測の原理: several candidate paths verified together) but
 * verify it with a lossy probability threshold; the rule here is a reading that
 * keeps every emitted token distributed as the target:
 *   - node n (0 <= n < N_b) has parent node_parent[b][n] in [-1, n) (-1: the
 *     verified prefix) and token node_tokens[b][n]; position 0 is the prefix
 *     and position n + 1 is node n;
 *   - the children of a position are independent draws from that position's
 *     draft distribution q; they are tested in increasing node index, the
 *     first against p, each later one against max(0, p_cur - q) / sum, the
 *     modified distribution left by the previous rejection (P1 section
 *     修正分布の定義 applied again), with u_accept[b][n] (strict <, R2 for q = 0);
 *   - the first accepted child is emitted and the walk continues at its
 *     position; when every child is rejected, or the position has none, the
 *     token is drawn from the current target by the inverse CDF (step 4's
 *     rule) with u_sample[b]; a zero residual mass falls back to the
 *     position's p;
 *   - T == 0 follows the first child equal to the lowest-index arg-max of the
 *     target and emits the arg-max where none does.
 * A tree in which every position has at most one child is exactly the linear
 * method.
 * target_logits: DEVICE [B][max_nodes + 1][V], row j = target at position j.
 * draft_logits:  DEVICE [B][max_nodes][V], row j = q at position j (rows of
 *                positions without children are read but not used: finite).
 * node_parent, node_tokens, u_accept: DEVICE [B][max_nodes].
 * num_nodes:     DEVICE [B] node count N_b (clamped to [0, max_nodes]), or NULL
 *                (= max_nodes).
 * u_sample:      DEVICE [B]; temperature: DEVICE [B] (0 = greedy).
 * Outputs: accepted_count[b] = nodes on the accepted path; out_tokens
 * [B][max_nodes + 1]: the path's tokens then the drawn token, -1 after;
 * out_nodes [B][max_nodes]: the path's node indices, -1 after.
 * A parent outside [-1, n) makes the node nobody's child; a token outside
 * [0, V) is rejected when tested and never dereferenced.  0 <= max_nodes <=
 * SV_TREE_MAX_NODES, V <= SV_TREE_MAX_V.  The workspace is sized by
 * spec_verify_tree_workspace_bytes.
 * Row statistics: with max_nodes >= 8 the walk computes them for the
 * positions it visits only (two launches: a clear of the exchange words, the
 * walk); smaller trees take them from one streaming pass over every row, then
 * walk.  The environment variable SPECVERIFY_TREE_STATS, read on each call,
 * forces one way ("walk" or "rows"; for testing): the results agree to
 * rounding either way. */
size_t spec_verify_tree_workspace_bytes(int B, int max_nodes, int V, int dtype);

int spec_verify_tree(const void *target_logits, const void *draft_logits,
                     const int32_t *node_parent, const int32_t *node_tokens,
                     const int32_t *num_nodes, const float *u_accept,
                     const float *u_sample, const float *temperature, int B,
                     int max_nodes, int V, int dtype, int32_t *accepted_count,
                     int32_t *out_tokens, int32_t *out_nodes, void *workspace,
                     size_t workspace_bytes, void *stream);

/* Draft-side sampling: one token per row of softmax(logits[r] / T_r), drawn by
 * the inverse CDF in vocabulary order with the supplied uniform u[r]: the
 * smallest v with u*Z < w[0] + ... + w[v] (the categorical draw that drafting
 * performs before verification: P2 code sketch, multinomial over
 * softmax(logits / temperature); P4 section 検証アルゴリズムの実装).  T_r == 0
 * gives the lowest-index arg-max.  Two kernels: the per-sub-chunk statistics
 * (2048 tokens each) over several workgroups per row, then one wave per row
 * that scans them and reads one sub-chunk again.
 * logits:       DEVICE [R][V] dt, row-major
 * u:            DEVICE [R] in [0, 1)
 * temperature:  host scalar used when `temperatures` is NULL (>= 0, finite)
 * temperatures: DEVICE [R] per-row temperatures, or NULL
 * tokens:       DEVICE out [R]
 * workspace:    spec_sample_workspace_bytes(R, V, dtype) bytes, 256-byte aligned
 * Errors as for spec_verify. */
size_t spec_sample_workspace_bytes(int R, int V, int dtype);
int spec_sample(const void *logits, const float *u, float temperature,
                const float *temperatures, int R, int V, int dtype,
                int32_t *tokens, void *workspace, size_t workspace_bytes,
                void *stream);

/* Draft-side sampling from filtered rows: one token per row of softmax(logits[r]
 * / T_r) truncated by top_k[r] / top_p[r] under the rule of spec_verify_filtered
 * (the sampler a serving system runs before filtered verification), by the
 * same inverse CDF with u[r].  temperatures: DEVICE [R] (0 = arg-max, which no
 * filter changes); top_k, top_p: DEVICE [R] or NULL, out-of-range values switch
 * the filter off for that row.  V <= SV_FILTER_MAX_V.  The workspace is sized by
 * spec_sample_filtered_workspace_bytes. */
size_t spec_sample_filtered_workspace_bytes(int R, int V, int dtype);
int spec_sample_filtered(const void *logits, const float *u, const float *temperatures,
                         const int32_t *top_k, const float *top_p, int R, int V, int dtype,
                         int32_t *tokens, void *workspace, size_t workspace_bytes,
                         void *stream);

/* ---- Adaptive draft length (host only, no GPU work) ----------------------
 * Policies that pick the next gamma from the accepted counts of past steps
 * (P3 section vLLM は利用者が書く表で、SGLang は実行中に観測した受理の長さで
 * 先読み数を変える; P4 section 動的推測戦略).  The caller owns the state; all
 * arguments are HOST memory.
 *   SV_GAMMA_BY_BATCH    gamma from a table of batch-size ranges (defaults
 *                        1-64 -> 3, 65-128 -> 1, 129-512 -> 0; past the table,
 *                        its last entry); observe() is a no-op.
 *   SV_GAMMA_EMA         per batch-size bucket (upper bounds 1, 2, 4, 8, 16,
 *                        31) an exponential moving average (weight 0.2) of the
 *                        mean accepted count; next = round(avg) + 1 clamped to
 *                        [1, 7]; 7 before the bucket has data; batches >= 32
 *                        use 1.
 *   SV_GAMMA_RATE_WINDOW mean of the last 100 per-step acceptance rates
 *                        (mean accepted count / gamma used); above 0.85 gamma
 *                        grows by one (max 8), below 0.65 it shrinks by one
 *                        (min 2); starts at 5.
 * Fields may be edited after init to change the defaults.  Functions return
 * SV_EINVAL on a NULL policy, B < 1 or an unknown kind; spec_gamma_next returns
 * the draft length (>= 0) otherwise. */
enum { SV_GAMMA_BY_BATCH = 0, SV_GAMMA_EMA = 1, SV_GAMMA_RATE_WINDOW = 2 };
#define SV_GAMMA_POLICY_SLOTS 16
#define SV_GAMMA_WINDOW_MAX 256

typedef struct {
    int kind;
    /* SV_GAMMA_BY_BATCH */
    int n_ranges;
    int range_max_batch[SV_GAMMA_POLICY_SLOTS];
    int range_gamma[SV_GAMMA_POLICY_SLOTS];
    /* SV_GAMMA_EMA */
    int n_buckets;
    int bucket_max_batch[SV_GAMMA_POLICY_SLOTS];
    double ema[SV_GAMMA_POLICY_SLOTS];
    int ema_count[SV_GAMMA_POLICY_SLOTS];
    double ema_weight;
    int steps_min, steps_max;
    int fixed_from_batch, fixed_steps;
    /* SV_GAMMA_RATE_WINDOW */
    int window, hist_len, hist_pos;
    double history[SV_GAMMA_WINDOW_MAX];
    double raise_above, lower_below;
    int gamma_min, gamma_max, gamma_current;
} sv_gamma_policy;

int spec_gamma_policy_init(sv_gamma_policy *policy, int kind);
int spec_gamma_next(const sv_gamma_policy *policy, int batch_size);
int spec_gamma_observe(sv_gamma_policy *policy, const int32_t *accepted_count,
                       int B, int gamma_used);

/* ---- No-allocation variant ---------------------------------------------
 * For callers that cannot allocate device memory or take a workspace argument:
 * code under HIP graph capture that must not call hipMalloc, tight serving
 * loops, harnesses that forbid allocation.  spec_verify_noalloc computes
 * exactly what spec_verify computes, with the same kernels, but its scratch
 * memory is a fixed array inside the library (SV_NOALLOC_SCRATCH_BYTES per
 * GPU, held until the process ends) instead of a caller's workspace.  Its
 * device address is looked up once per GPU, on the first call made with that
 * GPU current.  The call allocates nothing and calls no allocating routine.
 * Limit: a call whose spec_verify_workspace_bytes(B, gamma, V, dtype) exceeds
 * SV_NOALLOC_SCRATCH_BYTES returns SV_ESCRATCH and touches nothing.  Every call
 * on one GPU uses that GPU's one array: calls that overlap on one GPU (two
 * streams, or two host threads) race and must be serialised by the caller.
 * Arguments and results are those of spec_verify. */
#define SV_NOALLOC_SCRATCH_BYTES (4 << 20)
int spec_verify_noalloc(const void *target_logits, const void *draft_logits,
                        const int32_t *draft_tokens, const float *u_accept,
                        const float *u_sample, float temperature, int B, int gamma,
                        int V, int dtype, int32_t *accepted_count,
                        int32_t *out_tokens, void *stream);

/* Static description of a return code. */
const char *spec_verify_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
