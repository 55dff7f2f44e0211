/*
 * moe_oracle.h -- plain, slow CPU reference for one sparsely-gated MoE layer
 * evaluated over one speculative-decoding verification pass of N tokens.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this library: only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no source with the GPU library.
 *
 * What it computes, and where that is defined:
 *   - gate logits, top-k, softmax over the k, weighted sum of expert outputs:
 *     "Deep Dive into Mixture of Experts: From 1991 to DeepSeek-V3",
 *     section 2 ("2017: The Sparse-Gating Leap", the moe_layer sketch);
 *   - always-on shared experts added with weight one: same page, section 5
 *     ("DeepSeek-V3 and the Current State of the Art", deepseek_moe_layer);
 *   - the dense mixture (every expert weighted, every expert run): same page,
 *     section 1 ("1991: Where It Started");
 *   - per-slot engine (each selected expert read once per token) versus
 *     deduplicating engine (read once per pass) and their requested bytes:
 *     "Speculative Decoding for Mixture-of-Experts Models: Expert Bytes,
 *     Kernel Bandwidth and the Best Draft Length", abstract.
 * Readings the pages leave open (SwiGLU experts, tie rule, precisions) are
 * listed in the comments of moe_oracle.cpp next to the code that takes them.
 *
 * Arithmetic: fp64 accumulation everywhere.  bf16 weights are passed as their
 * raw 16-bit patterns.  All arrays are row-major and host-resident.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* weight element type */
#define ORACLE_F32 0
#define ORACLE_BF16 1

/* near-tie flags written by oracle_route */
#define ORACLE_FLAG_BOUNDARY 1u /* gap between k-th and (k+1)-th logit < tie_eps */
#define ORACLE_FLAG_ORDER 2u    /* two adjacent selected logits closer than tie_eps */

typedef struct oracle_shape {
  int32_t d;      /* d_model */
  int32_t E;      /* routed experts */
  int32_t k;      /* experts selected per token */
  int32_t f;      /* d_ff of every expert */
  int32_t S;      /* always-on shared experts */
  int32_t wdtype; /* ORACLE_F32 or ORACLE_BF16 */
} oracle_shape;

/* Expert weights.  Routed expert e: W1 = w13[e][0] ([f][d]), W3 = w13[e][1]
 * ([f][d]), W2 = w2[e] ([d][f]).  Shared expert s: the same in ws13 / ws2.
 * Element type per wdtype (bf16 as uint16 bit patterns). */
typedef struct oracle_weights {
  const void *w13, *w2, *ws13, *ws2;
} oracle_weights;

/* Round an fp32 value to bf16, nearest with ties to even; returns the 16-bit
 * pattern.  NaN maps to a quiet NaN. */
uint16_t oracle_bf16_rne(float x);

/* Round an fp64 value to bf16 in one step, nearest with ties to even (no
 * intermediate fp32 rounding); values at or beyond the overflow midpoint
 * become infinity.  Returns the 16-bit pattern; NaN maps to a quiet NaN. */
uint16_t oracle_bf16_rne_f64(double x);

/* Logits L[t][e] = sum_i x[t][i] * gate_w[e][i], fp64, index order. */
int oracle_gate_logits(const oracle_shape *s, const float *gate_w, const float *x,
                       int32_t n_tokens, double *logits);

/* Top-k + softmax over the k.  idx[t][j]: j-th expert in the order
 * (fp64 logit descending, expert index ascending).  w[t][j] in fp64
 * from the fp64 logits.  margin[t] = L_(k) - L_(k+1) (+inf if k == E).
 * flags[t] per ORACLE_FLAG_*.  logits/margin/flags may be NULL. */
int oracle_route(const oracle_shape *s, const float *gate_w, const float *x,
                 int32_t n_tokens, double tie_eps, double *logits, int32_t *idx,
                 double *w, double *margin, uint8_t *flags);

/* oracle_route with a per-expert bias [E] added to the logits before the
 * top-k; the softmax over the k takes the biased values (DeepSeek-style
 * sketch).  logits receives the biased logits. */
int oracle_route_biased(const oracle_shape *s, const float *gate_w, const float *bias,
                        const float *x, int32_t n_tokens, double tie_eps, double *logits,
                        int32_t *idx, double *w, double *margin, uint8_t *flags);

/* One SwiGLU expert on one token: out[d] = W2 * r(silu(W1 xt) . (W3 xt)),
 * xt = r(x), r = bf16 rounding for bf16 weights and the identity for fp32.
 * W1/W3/W2 point at that expert's matrices, element type per wdtype. */
int oracle_expert(const oracle_shape *s, const void *W1, const void *W3,
                  const void *W2, const float *x, double *out);

/* Full layer for a given routing.  engine 0 = per-slot, 1 = dedup.
 * y[t] = sum_j w[t][j] * expert_{idx[t][j]}(x_t)  (slot order)
 *        + sum_s shared_s(x_t).
 * bytes[0] = routed expert bytes the engine requests, bytes[1] = shared
 * expert bytes; *n_unique = number of distinct routed experts in the pass.
 * n_threads >= 1 splits the expert evaluations over std::threads; results
 * do not depend on it.  bytes / n_unique may be NULL. */
int oracle_layer(const oracle_shape *s, const oracle_weights *wts, const float *x,
                 int32_t n_tokens, const int32_t *idx, const double *w, int32_t engine,
                 int32_t n_threads, double *y, uint64_t *bytes, int32_t *n_unique);

/* The layer with dedup inside token groups: tokens group_start[g] ..
 * group_start[g+1]-1 form group g (group_start[0] = 0, group_start[G] = N,
 * strictly increasing).  y as oracle_layer; bytes[0] = sum_g U_g B_e,
 * bytes[1] = S B_e; n_unique[g] = U_g (may be NULL). */
int oracle_layer_grouped(const oracle_shape *s, const oracle_weights *wts, const float *x,
                         int32_t n_tokens, int32_t n_groups, const int32_t *group_start,
                         const int32_t *idx, const double *w, int32_t n_threads, double *y,
                         uint64_t *bytes, int32_t *n_unique);

/* Dense mixture: y[t] = sum_e softmax(L_t)_e * expert_e(x_t) + shared. */
int oracle_dense_mixture(const oracle_shape *s, const float *gate_w,
                         const oracle_weights *wts, const float *x, int32_t n_tokens,
                         double *y);

/* Requested bytes of one pass: B_e = 3 d f s_w; per-slot N k B_e, dedup
 * U B_e, shared S B_e. */
int oracle_pass_bytes(const oracle_shape *s, const int32_t *idx, int32_t n_tokens,
                      uint64_t *perslot, uint64_t *dedup, uint64_t *shared,
                      int32_t *n_unique);

/* Routing-trace compaction: counts[e] = slots choosing e; offs = exclusive
 * prefix of counts (E+1 entries); list = slot ids t*k+j grouped by expert,
 * ascending within an expert; uniq = the experts with counts > 0, ascending;
 * *n_unique = their number.  uniq needs E entries, list N*k. */
int oracle_compact(const oracle_shape *s, const int32_t *idx, int32_t n_tokens,
                   int32_t *counts, int32_t *offs, int32_t *list, int32_t *uniq,
                   int32_t *n_unique);

/* ---- speculative-decoding verification round ("Building a Terminal Based
 * LLM Inference Internals Explorer - Part 3: Speculative Decoding", sections
 * "The Accept/Reject Mechanism", "A Worked Example" and "Sampling vs
 * Greedy").
 *
 * Inverse-CDF sampler: weights w_j >= 0 are quantized to integers
 * floor(w_j * 2^40); with W their sum and r a uniform 32-bit integer, the
 * sample is the smallest index c whose inclusive prefix sum exceeds
 * floor(W r / 2^32).  Returns -1 when W == 0. */
int32_t oracle_sample_index(const float *weights, int32_t V, uint32_t r);

/* One round for one sequence.
 *   p      [gamma+1][V] verifier distributions (row gamma: the bonus position)
 *   q      [gamma][V]   draft distributions (sampling mode; NULL for greedy)
 *   x      [gamma]      draft tokens
 *   u      [gamma]      uniforms in [0, 1) for the accept tests (sampling)
 *   r                   32-bit uniform for the correction / bonus sample
 *   mode               0 greedy, 1 sampling
 * Outputs *n_acc (accepted draft tokens, 0..gamma) and tokens [gamma+1]: the
 * accepted prefix, then the correction (first rejection) or bonus token, then
 * -1.  Returns 0, or -1 on bad arguments. */
/* Softmax of logits / temperature, then top-p (nucleus) filtering and
 * renormalisation (see moe_oracle.cpp, reading V6).  probs [V] fp64 out;
 * boundary_gap may be NULL. */
int oracle_filter_probs(int32_t V, const float *logits, double temperature, double top_p,
                        double *probs, double *boundary_gap);

int oracle_verify_gate(int32_t gamma, int32_t V, int32_t mode, const float *p, const float *q,
                       const int32_t *x, const float *u, uint32_t r, int32_t *n_acc,
                       int32_t *tokens);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ORACLE_H */
