/*
 * moe_oracle.cpp -- plain CPU reference for the MoE verify-pass layer.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the CPU
 * baseline of the benchmark, never by the product path.  Written for
 * readability, not speed: loops in the order of the definitions, fp64
 * accumulation, no blocking, no fusion.
 *
 * Sources (web pages; sections as titled there):
 *  [MoE]  "Deep Dive into Mixture of Experts: From 1991 to DeepSeek-V3"
 *         s1 "1991: Where It Started"            -- dense mixture
 *         s2 "2017: The Sparse-Gating Leap"      -- logits, top-k, softmax
 *                                                   over the k, weighted sum
 *         s5 "DeepSeek-V3 and the Current State of the Art"
 *                                                -- shared experts, weight 1
 *  [SDM]  "Speculative Decoding for Mixture-of-Experts Models: Expert Bytes,
 *         Kernel Bandwidth and the Best Draft Length", abstract
 *                                                -- per-slot vs dedup bytes
 *
 * Readings taken where the pages are silent (each also used by the tests):
 *  R1  experts are SwiGLU FFNs, W2 (silu(W1 x) . W3 x), no biases; the pages
 *      only write experts[idx](x).
 *  R2  top-k order is (logit descending, expert index ascending); slot 0 is
 *      the largest, as a topk routine returns it.  The pages fix no
 *      precision, so the order is taken on the logits themselves, here
 *      their fp64 sums (within a few units of 1e-16 of the exact products'
 *      sum at these sizes).  Near-ties (gap < tie_eps) are flagged: only
 *      there can a computation in lower precision order them differently.
 *  R3  the softmax is over the k selected logits (the sketch's comment says
 *      it is renormalised over just the top-k).
 *  R4  bf16 weight configs round the token to bf16 before the experts and the
 *      SwiGLU product to bf16 before W2: each is one rounding to nearest,
 *      ties to even, of the value being rounded (the fp32 token; the
 *      product's fp64 value, with no fp32 step between); fp32 configs round
 *      nothing.
 *  R5  the dense mixture of s1 uses the same softmax gate over all E experts.
 *  R6  the per-expert bias of the DeepSeek-style sketch (s5) is added to the
 *      logits before the top-k, and the softmax over the k takes the biased
 *      values, as the sketch writes it.
 *  R7  dedup within token groups (several sequences verified in one pass):
 *      each group reads each of its distinct experts once, so a pass
 *      requests sum over groups of U_g expert reads; one group is the dedup
 *      engine, one token per group reads what the per-slot engine reads.
 */
#include "moe_oracle.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <thread>
#include <vector>

namespace {

bool shape_ok(const oracle_shape *s) {
  return s && s->d > 0 && s->E > 0 && s->k > 0 && s->k <= s->E && s->f > 0 &&
         s->S >= 0 && (s->wdtype == ORACLE_F32 || s->wdtype == ORACLE_BF16);
}

size_t elem_bytes(const oracle_shape *s) { return s->wdtype == ORACLE_BF16 ? 2 : 4; }

/* value of the n-th element of a weight array of the shape's type */
double weight_at(const oracle_shape *s, const void *base, size_t n) {
  if (s->wdtype == ORACLE_F32) return (double)((const float *)base)[n];
  uint32_t bits = (uint32_t)((const uint16_t *)base)[n] << 16;
  float v;
  std::memcpy(&v, &bits, 4);
  return (double)v;
}

float bf16_bits_to_float(uint16_t h) {
  uint32_t bits = (uint32_t)h << 16;
  float v;
  std::memcpy(&v, &bits, 4);
  return v;
}

/* R4: the rounding applied to activations on bf16 configs, one step from v */
double act_round(const oracle_shape *s, double v) {
  if (s->wdtype == ORACLE_F32) return v;
  return (double)bf16_bits_to_float(oracle_bf16_rne_f64(v));
}

double silu(double z) { return z / (1.0 + std::exp(-z)); }

const void *offset_weights(const oracle_shape *s, const void *base, size_t elems) {
  return (const void *)((const char *)base + elems * elem_bytes(s));
}

/* pointers to W1, W3, W2 of routed expert e (shared=false) or shared expert e */
void expert_mats(const oracle_shape *s, const oracle_weights *wts, int e, bool shared,
                 const void **W1, const void **W3, const void **W2) {
  size_t fd = (size_t)s->f * (size_t)s->d;
  const void *w13 = shared ? wts->ws13 : wts->w13;
  const void *w2 = shared ? wts->ws2 : wts->w2;
  *W1 = offset_weights(s, w13, (size_t)e * 2 * fd);
  *W3 = offset_weights(s, w13, ((size_t)e * 2 + 1) * fd);
  *W2 = offset_weights(s, w2, (size_t)e * fd);
}

/* R2: does expert a come before expert b in the selection order? */
bool before(const double *key, int a, int b) {
  if (key[a] != key[b]) return key[a] > key[b];
  return a < b;
}

/* Run a list of independent jobs over n_threads std::threads. */
template <class Job>
void run_jobs(size_t n_jobs, int n_threads, const Job &job) {
  if (n_threads <= 1 || n_jobs <= 1) {
    for (size_t i = 0; i < n_jobs; ++i) job(i);
    return;
  }
  size_t nt = std::min<size_t>((size_t)n_threads, n_jobs);
  std::vector<std::thread> pool;
  for (size_t w = 0; w < nt; ++w)
    pool.emplace_back([&, w]() {
      for (size_t i = w; i < n_jobs; i += nt) job(i);
    });
  for (auto &th : pool) th.join();
}

/* [MoE] s2 from the logits on: top-k under R2, softmax over the k (R3),
 * margin and near-tie flags.  L is [n_tokens][E] fp64. */
void route_from_logits(const oracle_shape *s, const std::vector<double> &L, int32_t n_tokens,
                       double tie_eps, double *logits, int32_t *idx, double *w,
                       double *margin, uint8_t *flags) {
  const int E = s->E, k = s->k;
  if (logits) std::memcpy(logits, L.data(), L.size() * sizeof(double));

  for (int t = 0; t < n_tokens; ++t) {
    const double *Lt = &L[(size_t)t * E];
    const double *key = Lt;

    /* [MoE] s2: top_k_vals, top_k_idx = topk(logits, k).  Selection by
     * repeated search for the best remaining expert under R2. */
    std::vector<int> order;
    std::vector<bool> taken(E, false);
    int rounds = (k < E) ? k + 1 : k; /* one more for the margin */
    for (int r = 0; r < rounds; ++r) {
      int best = -1;
      for (int e = 0; e < E; ++e)
        if (!taken[e] && (best < 0 || before(key, e, best))) best = e;
      taken[best] = true;
      order.push_back(best);
    }
    for (int j = 0; j < k; ++j) idx[(size_t)t * k + j] = order[j];

    /* [MoE] s2: top_k_weights = softmax(top_k_vals), renormalised over the k */
    double vmax = Lt[order[0]];
    double denom = 0.0;
    for (int j = 0; j < k; ++j) denom += std::exp(Lt[order[j]] - vmax);
    for (int j = 0; j < k; ++j) w[(size_t)t * k + j] = std::exp(Lt[order[j]] - vmax) / denom;

    double m = (k < E) ? Lt[order[k - 1]] - Lt[order[k]]
                       : std::numeric_limits<double>::infinity();
    if (margin) margin[t] = m;
    if (flags) {
      uint8_t fl = 0;
      if (m < tie_eps) fl |= ORACLE_FLAG_BOUNDARY;
      for (int j = 0; j + 1 < k; ++j)
        if (Lt[order[j]] - Lt[order[j + 1]] < tie_eps) fl |= ORACLE_FLAG_ORDER;
      flags[t] = fl;
    }
  }
}

uint64_t expert_bytes(const oracle_shape *s) {
  return 3ull * (uint64_t)s->d * (uint64_t)s->f * elem_bytes(s);
}

/* One job = one expert evaluation on one token: routed expert e for slot
 * `slot` of token t, or shared expert `slot` (e unused) when shared. */
struct Job {
  int t, slot, e;
  bool shared;
};

/* [SDM] dedup over the tokens t0 .. t1-1: every distinct selected expert,
 * ascending, with all (token, slot) pairs of the range that chose it.
 * Appends the jobs and returns the number of distinct experts. */
int32_t dedup_jobs(const oracle_shape *s, const int32_t *idx, int t0, int t1,
                   std::vector<Job> *jobs) {
  const int k = s->k;
  int32_t U = 0;
  for (int e = 0; e < s->E; ++e) {
    bool used = false;
    for (int t = t0; t < t1; ++t)
      for (int j = 0; j < k; ++j)
        if (idx[(size_t)t * k + j] == e) {
          jobs->push_back({t, j, e, false});
          used = true;
        }
    if (used) ++U;
  }
  return U;
}

/* Runs the routed jobs plus every shared expert on every token, then
 * [MoE] s2 / s5: y = sum over slots of weight * expert output, then the
 * shared experts (weight 1); slot order whatever order the jobs came in. */
void evaluate_layer(const oracle_shape *s, const oracle_weights *wts, const float *x, int N,
                    const double *w, std::vector<Job> jobs, int n_threads, double *y) {
  const int d = s->d, k = s->k, S = s->S;
  /* o[t][j] = expert_{idx[t][j]}(x_t);  osh[t][s] = shared_s(x_t) */
  std::vector<double> o((size_t)N * k * d), osh((size_t)N * S * d);
  /* [MoE] s5: shared experts run on every token, read once per pass */
  for (int sh = 0; sh < S; ++sh)
    for (int t = 0; t < N; ++t) jobs.push_back({t, sh, sh, true});

  run_jobs(jobs.size(), n_threads, [&](size_t i) {
    const Job &jb = jobs[i];
    const void *W1, *W3, *W2;
    expert_mats(s, wts, jb.e, jb.shared, &W1, &W3, &W2);
    double *dst = jb.shared ? &osh[((size_t)jb.t * S + jb.slot) * d]
                            : &o[((size_t)jb.t * k + jb.slot) * d];
    oracle_expert(s, W1, W3, W2, x + (size_t)jb.t * d, dst);
  });

  for (int t = 0; t < N; ++t)
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j) acc += w[(size_t)t * k + j] * o[((size_t)t * k + j) * d + c];
      for (int sh = 0; sh < S; ++sh) acc += osh[((size_t)t * S + sh) * d + c];
      y[(size_t)t * d + c] = acc;
    }
}

}  // namespace

extern "C" {

uint16_t oracle_bf16_rne_f64(double x) {
  const uint16_t sign = std::signbit(x) ? 0x8000u : 0u;
  if (std::isnan(x)) return (uint16_t)(sign | 0x7FC0u);
  const double a = std::fabs(x);
  if (std::isinf(a)) return (uint16_t)(sign | 0x7F80u);
  if (a == 0.0) return sign;
  /* bf16 keeps 8 significant bits: in [2^(e-1), 2^e) its values are the
   * multiples of 2^(e-8), and below 2^-126 the multiples of 2^-133 (its
   * subnormals).  Scale a to units of that spacing (exact: a power of two),
   * split off the fraction (exact), and take the nearer multiple, the even
   * one on a tie. */
  int e = 0;
  (void)std::frexp(a, &e);                 /* a = m * 2^e, 1/2 <= m < 1 */
  const int q = std::max(e - 8, -133);
  const double units = std::ldexp(a, -q);  /* < 2^8 */
  const double lo = std::floor(units);
  const double frac = units - lo;
  double r = lo;
  if (frac > 0.5 || (frac == 0.5 && std::fmod(lo, 2.0) != 0.0)) r = lo + 1.0;
  const double v = std::ldexp(r, q);
  const double max_bf16 = std::ldexp(255.0, 120);  /* 0x7F7F */
  if (v > max_bf16) return (uint16_t)(sign | 0x7F80u);
  const float fv = (float)v;               /* exact: v is a bf16 value */
  uint32_t bits;
  std::memcpy(&bits, &fv, 4);
  return (uint16_t)(sign | (uint16_t)(bits >> 16));
}

uint16_t oracle_bf16_rne(float x) {
  uint32_t bits;
  std::memcpy(&bits, &x, 4);
  if (std::isnan(x)) return (uint16_t)((bits >> 16) | 0x0040u);
  return oracle_bf16_rne_f64((double)x);   /* fp32 -> fp64 is exact */
}

int oracle_gate_logits(const oracle_shape *s, const float *gate_w, const float *x,
                       int32_t n_tokens, double *logits) {
  if (!shape_ok(s) || !gate_w || !x || !logits || n_tokens < 0) return -1;
  /* [MoE] s2: logits = x @ gate_weights, one score per expert */
  for (int t = 0; t < n_tokens; ++t)
    for (int e = 0; e < s->E; ++e) {
      double acc = 0.0;
      for (int i = 0; i < s->d; ++i)
        acc += (double)x[(size_t)t * s->d + i] * (double)gate_w[(size_t)e * s->d + i];
      logits[(size_t)t * s->E + e] = acc;
    }
  return 0;
}

int oracle_route(const oracle_shape *s, const float *gate_w, const float *x,
                 int32_t n_tokens, double tie_eps, double *logits, int32_t *idx,
                 double *w, double *margin, uint8_t *flags) {
  if (!shape_ok(s) || !gate_w || !x || !idx || !w || n_tokens < 0) return -1;
  std::vector<double> L((size_t)n_tokens * s->E);
  oracle_gate_logits(s, gate_w, x, n_tokens, L.data());
  route_from_logits(s, L, n_tokens, tie_eps, logits, idx, w, margin, flags);
  return 0;
}

int oracle_route_biased(const oracle_shape *s, const float *gate_w, const float *bias,
                        const float *x, int32_t n_tokens, double tie_eps, double *logits,
                        int32_t *idx, double *w, double *margin, uint8_t *flags) {
  if (!shape_ok(s) || !gate_w || !bias || !x || !idx || !w || n_tokens < 0) return -1;
  std::vector<double> L((size_t)n_tokens * s->E);
  oracle_gate_logits(s, gate_w, x, n_tokens, L.data());
  /* [MoE] s5, DeepSeek-style routing sketch: logits = x @ gate_weights + bias,
   * and the biased logits feed both the top-k and the softmax (R6) */
  for (int t = 0; t < n_tokens; ++t)
    for (int e = 0; e < s->E; ++e) L[(size_t)t * s->E + e] += (double)bias[e];
  route_from_logits(s, L, n_tokens, tie_eps, logits, idx, w, margin, flags);
  return 0;
}

int oracle_expert(const oracle_shape *s, const void *W1, const void *W3, const void *W2,
                  const float *x, double *out) {
  if (!shape_ok(s) || !W1 || !W3 || !W2 || !x || !out) return -1;
  const int d = s->d, f = s->f;
  /* R4: the token as the experts see it */
  std::vector<double> xt(d);
  for (int i = 0; i < d; ++i) xt[i] = act_round(s, (double)x[i]);
  /* R1: a = silu(W1 xt) * (W3 xt), rounded per R4 */
  std::vector<double> a(f);
  for (int r = 0; r < f; ++r) {
    double h = 0.0, g = 0.0;
    for (int i = 0; i < d; ++i) {
      h += weight_at(s, W1, (size_t)r * d + i) * xt[i];
      g += weight_at(s, W3, (size_t)r * d + i) * xt[i];
    }
    a[r] = act_round(s, silu(h) * g);
  }
  /* out = W2 a */
  for (int c = 0; c < d; ++c) {
    double acc = 0.0;
    for (int r = 0; r < f; ++r) acc += weight_at(s, W2, (size_t)c * f + r) * a[r];
    out[c] = acc;
  }
  return 0;
}

int oracle_layer(const oracle_shape *s, const oracle_weights *wts, const float *x,
                 int32_t n_tokens, const int32_t *idx, const double *w, int32_t engine,
                 int32_t n_threads, double *y, uint64_t *bytes, int32_t *n_unique) {
  if (!shape_ok(s) || !wts || !wts->w13 || !wts->w2 || !x || !idx || !w || !y ||
      n_tokens < 0 || (engine != 0 && engine != 1))
    return -1;
  if (s->S > 0 && (!wts->ws13 || !wts->ws2)) return -1;
  const int k = s->k, N = n_tokens;
  for (size_t i = 0; i < (size_t)N * k; ++i)
    if (idx[i] < 0 || idx[i] >= s->E) return -1;
  const uint64_t Be = expert_bytes(s);

  std::vector<Job> jobs;
  uint64_t routed_bytes = 0;
  int32_t U = 0;
  if (engine == 0) {
    /* [SDM] per-slot: every (token, slot) reads its expert */
    for (int t = 0; t < N; ++t)
      for (int j = 0; j < k; ++j) {
        jobs.push_back({t, j, idx[(size_t)t * k + j], false});
        routed_bytes += Be;
      }
    std::vector<bool> seen(s->E, false);
    for (size_t i = 0; i < (size_t)N * k; ++i)
      if (!seen[idx[i]]) { seen[idx[i]] = true; ++U; }
  } else {
    /* [SDM] dedup: each distinct selected expert is read once per pass */
    U = dedup_jobs(s, idx, 0, N, &jobs);
    routed_bytes = (uint64_t)U * Be;
  }
  evaluate_layer(s, wts, x, N, w, jobs, n_threads, y);
  if (bytes) {
    bytes[0] = routed_bytes;
    bytes[1] = (uint64_t)s->S * Be;
  }
  if (n_unique) *n_unique = U;
  return 0;
}

int oracle_layer_grouped(const oracle_shape *s, const oracle_weights *wts, const float *x,
                         int32_t n_tokens, int32_t n_groups, const int32_t *group_start,
                         const int32_t *idx, const double *w, int32_t n_threads, double *y,
                         uint64_t *bytes, int32_t *n_unique) {
  if (!shape_ok(s) || !wts || !wts->w13 || !wts->w2 || !x || !idx || !w || !y ||
      !group_start || n_tokens < 0 || n_groups < 1)
    return -1;
  if (s->S > 0 && (!wts->ws13 || !wts->ws2)) return -1;
  if (group_start[0] != 0 || group_start[n_groups] != n_tokens) return -1;
  for (int g = 0; g < n_groups; ++g)
    if (group_start[g + 1] <= group_start[g]) return -1;
  for (size_t i = 0; i < (size_t)n_tokens * s->k; ++i)
    if (idx[i] < 0 || idx[i] >= s->E) return -1;
  const uint64_t Be = expert_bytes(s);

  /* R7: the dedup formulation applied to each group's tokens on its own */
  std::vector<Job> jobs;
  uint64_t routed_bytes = 0;
  for (int g = 0; g < n_groups; ++g) {
    const int32_t Ug = dedup_jobs(s, idx, group_start[g], group_start[g + 1], &jobs);
    routed_bytes += (uint64_t)Ug * Be;
    if (n_unique) n_unique[g] = Ug;
  }
  evaluate_layer(s, wts, x, n_tokens, w, jobs, n_threads, y);
  if (bytes) {
    bytes[0] = routed_bytes;
    bytes[1] = (uint64_t)s->S * Be;
  }
  return 0;
}

int oracle_dense_mixture(const oracle_shape *s, const float *gate_w,
                         const oracle_weights *wts, const float *x, int32_t n_tokens,
                         double *y) {
  if (!shape_ok(s) || !gate_w || !wts || !x || !y || n_tokens < 0) return -1;
  if (s->S > 0 && (!wts->ws13 || !wts->ws2)) return -1;
  const int d = s->d, E = s->E, S = s->S;
  std::vector<double> L((size_t)n_tokens * E), out(d);
  oracle_gate_logits(s, gate_w, x, n_tokens, L.data());
  for (int t = 0; t < n_tokens; ++t) {
    /* [MoE] s1: the gate weights every expert and every expert runs (R5) */
    double vmax = L[(size_t)t * E];
    for (int e = 1; e < E; ++e) vmax = std::max(vmax, L[(size_t)t * E + e]);
    double denom = 0.0;
    for (int e = 0; e < E; ++e) denom += std::exp(L[(size_t)t * E + e] - vmax);
    std::vector<double> acc(d, 0.0);
    for (int e = 0; e < E; ++e) {
      double p = std::exp(L[(size_t)t * E + e] - vmax) / denom;
      const void *W1, *W3, *W2;
      expert_mats(s, wts, e, false, &W1, &W3, &W2);
      oracle_expert(s, W1, W3, W2, x + (size_t)t * d, out.data());
      for (int c = 0; c < d; ++c) acc[c] += p * out[c];
    }
    for (int sh = 0; sh < S; ++sh) {
      const void *W1, *W3, *W2;
      expert_mats(s, wts, sh, true, &W1, &W3, &W2);
      oracle_expert(s, W1, W3, W2, x + (size_t)t * d, out.data());
      for (int c = 0; c < d; ++c) acc[c] += out[c];
    }
    for (int c = 0; c < d; ++c) y[(size_t)t * d + c] = acc[c];
  }
  return 0;
}

int oracle_pass_bytes(const oracle_shape *s, const int32_t *idx, int32_t n_tokens,
                      uint64_t *perslot, uint64_t *dedup, uint64_t *shared,
                      int32_t *n_unique) {
  if (!shape_ok(s) || !idx || n_tokens < 0) return -1;
  const uint64_t Be = 3ull * (uint64_t)s->d * (uint64_t)s->f * elem_bytes(s);
  std::vector<bool> seen(s->E, false);
  int32_t U = 0;
  for (size_t i = 0; i < (size_t)n_tokens * s->k; ++i) {
    if (idx[i] < 0 || idx[i] >= s->E) return -1;
    if (!seen[idx[i]]) { seen[idx[i]] = true; ++U; }
  }
  /* [SDM] per-slot reads once per token and slot; dedup once per pass */
  if (perslot) *perslot = (uint64_t)n_tokens * (uint64_t)s->k * Be;
  if (dedup) *dedup = (uint64_t)U * Be;
  if (shared) *shared = (uint64_t)s->S * Be;
  if (n_unique) *n_unique = U;
  return 0;
}

int oracle_compact(const oracle_shape *s, const int32_t *idx, int32_t n_tokens,
                   int32_t *counts, int32_t *offs, int32_t *list, int32_t *uniq,
                   int32_t *n_unique) {
  if (!shape_ok(s) || !idx || !counts || !offs || !list || !uniq || !n_unique ||
      n_tokens < 0)
    return -1;
  const int E = s->E;
  const size_t slots = (size_t)n_tokens * s->k;
  for (size_t i = 0; i < slots; ++i)
    if (idx[i] < 0 || idx[i] >= E) return -1;
  int32_t U = 0, pos = 0;
  for (int e = 0; e < E; ++e) {
    offs[e] = pos;
    int32_t c = 0;
    for (size_t i = 0; i < slots; ++i)
      if (idx[i] == e) list[pos + c++] = (int32_t)i;
    counts[e] = c;
    pos += c;
    uniq[e] = -1;
    if (c > 0) uniq[U++] = e;
  }
  offs[E] = pos;
  *n_unique = U;
  return 0;
}

/* ---- verification round
 *
 * Readings (the page's code draws with torch.rand / torch.multinomial; here
 * the random numbers come in as arguments):
 *   V1 p and q are the models' distributions after the caller's temperature
 *      and top-p filtering, the same settings on both sides, as the page
 *      requires for the ratio to be meaningful;
 *   V2 a draft token is accepted when u < min(1, p(x) / q(x)) and q(x) > 0;
 *      u q(x) < p(x) says the same without a division, and the products of
 *      two fp32 values are exact in fp64;
 *   V3 sampling from the normalised residual max(0, p - q) is an inverse-CDF
 *      draw over its quantized weights (oracle_sample_index): normalising is
 *      the scaling of the target by W;
 *   V4 a residual that quantizes to zero everywhere (p and q equal to within
 *      2^-40) draws the correction from p itself;
 *   V5 greedy mode accepts a draft token when it is the verifier's argmax
 *      (ties to the lowest index) and emits the verifier's argmax at the
 *      first mismatch, or at the bonus position. */
int32_t oracle_sample_index(const float *weights, int32_t V, uint32_t r) {
  if (!weights || V <= 0) return -1;
  const double scale = 1099511627776.0; /* 2^40 */
  uint64_t W = 0;
  for (int32_t j = 0; j < V; ++j) {
    const double w = weights[j] > 0.f ? (double)weights[j] : 0.0;
    W += (uint64_t)std::floor(w * scale);
  }
  if (W == 0) return -1;
  const uint64_t target = (uint64_t)(((unsigned __int128)W * r) >> 32);
  uint64_t prefix = 0;
  for (int32_t j = 0; j < V; ++j) {
    const double w = weights[j] > 0.f ? (double)weights[j] : 0.0;
    prefix += (uint64_t)std::floor(w * scale);
    if (prefix > target) return j;
  }
  return -1; /* not reached: prefix ends at W > target */
}

/* V6: the verifier's and the draft's distributions from their logits, as
 * the page's verify phase builds them: softmax of logits / temperature, then
 * top-p (nucleus) filtering -- the shortest run of tokens in the order
 * (probability descending, index ascending) whose probability reaches top_p,
 * the token that reaches it included, renormalised; the rest get zero.
 * top_p >= 1 keeps every token.  fp64 throughout.  *boundary_gap (if given)
 * receives the smallest margin of the decision (below): small values mark
 * rows whose kept set a lower precision could change. */
int oracle_filter_probs(int32_t V, const float *logits, double temperature, double top_p,
                        double *probs, double *boundary_gap) {
  if (V <= 0 || !logits || !probs || !(temperature > 0.0) || !(top_p > 0.0)) return -1;
  std::vector<double> z((size_t)V);
  double m = -std::numeric_limits<double>::infinity();
  for (int32_t j = 0; j < V; ++j) {
    z[j] = (double)logits[j] / temperature;
    if (z[j] > m) m = z[j];
  }
  double S = 0.0;
  for (int32_t j = 0; j < V; ++j) {
    z[j] = std::exp(z[j] - m);
    S += z[j];
  }
  for (int32_t j = 0; j < V; ++j) probs[j] = z[j] / S;
  if (boundary_gap) *boundary_gap = std::numeric_limits<double>::infinity();
  if (top_p >= 1.0) return 0;
  std::vector<int32_t> order((size_t)V);
  for (int32_t j = 0; j < V; ++j) order[j] = j;
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b) { return probs[a] > probs[b]; });
  double kept = 0.0;
  int32_t n_kept = 0;
  while (n_kept < V) {
    kept += probs[order[n_kept]];
    ++n_kept;
    if (kept >= top_p) break;
  }
  if (boundary_gap) {
    /* how close the row is to keeping a different set at lower precision:
     * the kept mass against top_p on both sides of the last kept token,
     * and the relative distance from the last kept probability to the
     * nearest different probability above and below it (an exact tie is
     * ordered by index in any precision; a near one may not be) */
    const double last = probs[order[n_kept - 1]];
    const double before = kept - last;
    double gap = std::min(std::fabs(top_p - before), std::fabs(kept - top_p));
    const double scale = last > 0.0 ? last : 1.0;
    for (int32_t r = n_kept; r < V; ++r)
      if (probs[order[r]] != last) {
        gap = std::min(gap, (last - probs[order[r]]) / scale);
        break;
      }
    for (int32_t r = n_kept - 1; r >= 0; --r)
      if (probs[order[r]] != last) {
        gap = std::min(gap, (probs[order[r]] - last) / scale);
        break;
      }
    *boundary_gap = gap;
  }
  double total = 0.0;
  for (int32_t r = 0; r < n_kept; ++r) total += probs[order[r]];
  std::vector<char> keep((size_t)V, 0);
  for (int32_t r = 0; r < n_kept; ++r) keep[order[r]] = 1;
  for (int32_t j = 0; j < V; ++j) probs[j] = keep[j] ? probs[j] / total : 0.0;
  return 0;
}

static int32_t argmax_lowest(const float *row, int32_t V) {
  int32_t best = 0;
  for (int32_t j = 1; j < V; ++j)
    if (row[j] > row[best]) best = j;
  return best;
}

int oracle_verify_gate(int32_t gamma, int32_t V, int32_t mode, const float *p, const float *q,
                       const int32_t *x, const float *u, uint32_t r, int32_t *n_acc,
                       int32_t *tokens) {
  if (gamma < 0 || V <= 0 || !p || !n_acc || !tokens || (gamma > 0 && !x)) return -1;
  if (mode != 0 && mode != 1) return -1;
  if (mode == 1 && gamma > 0 && (!q || !u)) return -1;
  for (int32_t i = 0; i < gamma; ++i)
    if (x[i] < 0 || x[i] >= V) return -1;
  for (int32_t i = 0; i <= gamma; ++i) tokens[i] = -1;
  std::vector<float> residual((size_t)V);
  for (int32_t i = 0; i < gamma; ++i) {
    const float *pi = p + (size_t)i * V;
    bool accept;
    if (mode == 0) {
      accept = argmax_lowest(pi, V) == x[i]; /* V5 */
    } else {
      const float *qi = q + (size_t)i * V;
      const double pv = pi[x[i]], qv = qi[x[i]];
      accept = qv > 0.0 && (double)u[i] * qv < pv; /* V2 */
    }
    if (accept) {
      tokens[i] = x[i];
      continue;
    }
    /* first rejection: the round ends with the verifier's own token */
    *n_acc = i;
    if (mode == 0) {
      tokens[i] = argmax_lowest(pi, V);
      return 0;
    }
    const float *qi = q + (size_t)i * V;
    for (int32_t j = 0; j < V; ++j) {
      const float d = pi[j] - qi[j];
      residual[j] = d > 0.f ? d : 0.f; /* max(0, p - q) */
    }
    int32_t c = oracle_sample_index(residual.data(), V, r); /* V3 */
    if (c < 0) c = oracle_sample_index(pi, V, r);           /* V4 */
    tokens[i] = c;
    return 0;
  }
  /* every draft token survived: the bonus token from the last position */
  *n_acc = gamma;
  const float *pb = p + (size_t)gamma * V;
  tokens[gamma] = mode == 0 ? argmax_lowest(pb, V) : oracle_sample_index(pb, V, r);
  return 0;
}

}  // extern "C"
