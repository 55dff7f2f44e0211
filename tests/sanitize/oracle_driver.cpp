// Drives every function of the CPU oracle (oracle/moe_oracle.h) on small
// seeded inputs, and on rejected arguments, for AddressSanitizer and UBSan
// builds.  It checks only what needs no reference: status codes, that
// outputs are finite, and that the two engines agree; the values
// themselves are pinned by the Python tests.  Exit status 0 = all held.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "moe_oracle.h"

static int g_fail = 0;
#define CHECK(c)                                                     \
  do {                                                               \
    if (!(c)) {                                                      \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++g_fail;                                                      \
    }                                                                \
  } while (0)

int main() {
  std::mt19937 rng(7);
  std::normal_distribution<float> nd(0.f, 1.f);
  for (int wd : {ORACLE_F32, ORACLE_BF16}) {
    const oracle_shape s{32, 8, 3, 32, 1, wd};
    const size_t fd = (size_t)s.f * s.d;
    const int n = 5;
    std::vector<float> gate((size_t)s.E * s.d), x((size_t)n * s.d), bias(s.E);
    for (auto &v : gate) v = nd(rng);
    for (auto &v : x) v = nd(rng);
    for (auto &v : bias) v = 0.3f * nd(rng);
    std::vector<float> wf((size_t)(s.E + s.S) * 3 * fd);
    for (auto &v : wf) v = 0.1f * nd(rng);
    std::vector<uint16_t> wb(wf.size());
    for (size_t i = 0; i < wf.size(); ++i) wb[i] = oracle_bf16_rne(wf[i]);
    const char *base = wd == ORACLE_F32 ? (const char *)wf.data() : (const char *)wb.data();
    const size_t es = wd == ORACLE_F32 ? 4 : 2;
    const oracle_weights w{base, base + (size_t)s.E * 2 * fd * es,
                           base + (size_t)s.E * 3 * fd * es,
                           base + ((size_t)s.E * 3 + 2 * s.S) * fd * es};
    std::vector<double> logits((size_t)n * s.E), wt((size_t)n * s.k), margin(n);
    std::vector<int32_t> idx((size_t)n * s.k);
    std::vector<uint8_t> flags(n);
    CHECK(oracle_gate_logits(&s, gate.data(), x.data(), n, logits.data()) == 0);
    CHECK(oracle_route(&s, gate.data(), x.data(), n, 1e-4, logits.data(), idx.data(), wt.data(),
                       margin.data(), flags.data()) == 0);
    CHECK(oracle_route_biased(&s, gate.data(), bias.data(), x.data(), n, 1e-4, logits.data(),
                              idx.data(), wt.data(), margin.data(), flags.data()) == 0);
    std::vector<double> y0((size_t)n * s.d), y1(y0.size()), y2(y0.size()), y3(y0.size());
    uint64_t b0[2], b1[2], b2[2];
    int32_t u0 = 0, u1 = 0, ug[3] = {0, 0, 0};
    CHECK(oracle_layer(&s, &w, x.data(), n, idx.data(), wt.data(), 0, 1, y0.data(), b0, &u0) == 0);
    CHECK(oracle_layer(&s, &w, x.data(), n, idx.data(), wt.data(), 1, 3, y1.data(), b1, &u1) == 0);
    const int32_t gs[4] = {0, 2, 3, 5};
    CHECK(oracle_layer_grouped(&s, &w, x.data(), n, 3, gs, idx.data(), wt.data(), 2, y2.data(),
                               b2, ug) == 0);
    CHECK(y0 == y1 && y1 == y2 && u0 == u1 && ug[0] + ug[1] + ug[2] >= u1);
    for (double v : y0) CHECK(std::isfinite(v));
    std::vector<double> out(s.d);
    CHECK(oracle_expert(&s, w.w13, (const char *)w.w13 + fd * es, w.w2, x.data(), out.data()) == 0);
    CHECK(oracle_dense_mixture(&s, gate.data(), &w, x.data(), n, y3.data()) == 0);
    uint64_t ps = 0, dd = 0, sh = 0;
    int32_t U = 0;
    CHECK(oracle_pass_bytes(&s, idx.data(), n, &ps, &dd, &sh, &U) == 0 && U == u0);
    std::vector<int32_t> counts(s.E), offs(s.E + 1), list((size_t)n * s.k), uniq(s.E);
    CHECK(oracle_compact(&s, idx.data(), n, counts.data(), offs.data(), list.data(), uniq.data(),
                         &U) == 0 && offs[s.E] == n * s.k);
    // rejected arguments
    const int32_t bad_gs[4] = {0, 4, 3, 5};  // not increasing
    CHECK(oracle_layer_grouped(&s, &w, x.data(), n, 3, bad_gs, idx.data(), wt.data(), 1,
                               y2.data(), b2, ug) != 0);
    std::vector<int32_t> oob(idx);
    oob[0] = s.E;
    CHECK(oracle_layer(&s, &w, x.data(), n, oob.data(), wt.data(), 0, 1, y0.data(), b0, &u0) != 0);
    CHECK(oracle_pass_bytes(&s, oob.data(), n, &ps, &dd, &sh, &U) != 0);
  }
  // the verification round and the sampler
  const int V = 1000, gamma = 4;
  std::vector<float> p((size_t)(gamma + 1) * V), q((size_t)gamma * V), u(gamma);
  std::uniform_real_distribution<float> ud(0.f, 1.f);
  for (auto &v : p) v = ud(rng) / V;
  for (auto &v : q) v = ud(rng) / V;
  for (auto &v : u) v = ud(rng);
  std::vector<int32_t> xt = {1, 2, 3, 999}, tok(gamma + 1);
  int32_t na = -1;
  for (int mode : {0, 1}) {
    CHECK(oracle_verify_gate(gamma, V, mode, p.data(), q.data(), xt.data(), u.data(), 12345u,
                             &na, tok.data()) == 0);
    CHECK(na >= 0 && na <= gamma && tok[na] >= 0 && tok[na] < V);
  }
  xt[2] = V;
  CHECK(oracle_verify_gate(gamma, V, 1, p.data(), q.data(), xt.data(), u.data(), 1u, &na,
                           tok.data()) != 0);
  CHECK(oracle_sample_index(p.data(), V, 0u) >= 0 && oracle_sample_index(p.data(), V, ~0u) < V);
  std::vector<double> fp(V);
  double gap = 0.0;
  for (double top_p : {0.3, 0.9, 1.0}) {
    CHECK(oracle_filter_probs(V, p.data(), 0.7, top_p, fp.data(), &gap) == 0);
    double sum = 0.0;
    for (double v : fp) sum += v;
    CHECK(std::fabs(sum - 1.0) < 1e-9);
  }
  CHECK(oracle_filter_probs(V, p.data(), 0.0, 0.9, fp.data(), nullptr) != 0);
  std::printf("oracle driver: %d failed checks\n", g_fail);
  return g_fail == 0 ? 0 : 1;
}
