// abi.cpp -- the C ABI of include/moe_verify.h: argument validation,
// workspace sizing, the launch sequence of each call and the optional
// per-kernel event timing.  Kernels live in router.hip and expert.hip
// (the dedup compaction, done inside the up kernel, in compact.h).
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>
#include <vector>

#include "kernels.h"
#include "verify.h"
#include "moe_verify.h"

namespace {

using moe::align_up;

constexpr size_t kAlign = 256;
// The first kHead bytes of every workspace belong to arrival counters
// (routing, stack pass, verification round); no call writes data there, so
// one zero fill before a workspace's first use serves any sequence of calls.
constexpr size_t kHead = 256;

int check_shape(const moe_shape *s) {
  if (!s) return MOE_ERR_INVALID_ARG;
  if (s->d_model <= 0 || s->d_ff <= 0 || s->n_experts <= 0 || s->top_k <= 0)
    return MOE_ERR_INVALID_ARG;
  if (s->top_k > s->n_experts || s->top_k > MOE_MAX_TOPK) return MOE_ERR_INVALID_ARG;
  if (s->n_experts > MOE_MAX_EXPERTS) return MOE_ERR_INVALID_ARG;
  if (s->n_shared < 0 || s->n_shared > MOE_MAX_SHARED) return MOE_ERR_INVALID_ARG;
  if (s->wdtype != MOE_F32 && s->wdtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (s->d_model % 32 != 0 || s->d_ff % 32 != 0) return MOE_ERR_UNSUPPORTED;
  // 16-row tiles index rows with 32-bit ints
  if ((int64_t)s->d_model * s->d_ff > (int64_t)1 << 30) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_tokens(const moe_shape *s, int32_t n) {
  if (n < 1 || n > MOE_MAX_TOKENS) return MOE_ERR_INVALID_ARG;
  if ((int64_t)n * s->top_k > MOE_MAX_SLOTS) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

bool aligned(const void *p) { return ((uintptr_t)p % kAlign) == 0; }

size_t wbytes(const moe_shape *s) { return s->wdtype == MOE_BF16 ? 2 : 4; }

// rows of the per-instance activation / output buffers: N*k routed + S*N shared
size_t entry_rows(const moe_shape *s, int n) {
  return (size_t)n * s->top_k + (size_t)s->n_shared * n;
}

// [arrival counters (one per layer, in the head) | partial logits
//  [L][splits][N][E]]
size_t route_ws(const moe_shape *s, int n, int L = 1) {
  return kHead + align_up((size_t)L * moe::gate_splits(s->d_model) * n * s->n_experts *
                               sizeof(float), kAlign);
}

// one compaction record (per token group of the dedup engine)
size_t cmp_ws(const moe_shape *s, int n) {
  moe::CompactLayout L{s->n_experts, n * s->top_k};
  return align_up((size_t)L.total() * sizeof(int32_t), kAlign);
}

// Token groups: 1 <= G <= MOE_MAX_GROUPS, gs[0] = 0, gs[G] = n, increasing.
int check_groups(int32_t n, int32_t G, const int32_t *gs) {
  if (G < 1 || G > MOE_MAX_GROUPS || !gs) return MOE_ERR_INVALID_ARG;
  if (gs[0] != 0 || gs[G] != n) return MOE_ERR_INVALID_ARG;
  for (int g = 0; g < G; ++g)
    if (gs[g + 1] <= gs[g]) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

size_t abuf_ws(const moe_shape *s, int n) {
  return align_up(entry_rows(s, n) * s->d_ff * wbytes(s), kAlign);
}

size_t obuf_ws(const moe_shape *s, int n) {
  return align_up(entry_rows(s, n) * s->d_model * sizeof(float), kAlign);
}

// Workspace query / size check shared by the device calls.  Returns
// MOE_OK and sets *launch when the call should go ahead.
int workspace_gate(void *ws, size_t *ws_bytes, size_t need, bool *launch) {
  *launch = false;
  if (!ws_bytes) return MOE_ERR_INVALID_ARG;
  if (!ws) {
    *ws_bytes = need;
    return MOE_OK;
  }
  if (!aligned(ws)) return MOE_ERR_INVALID_ARG;
  if (*ws_bytes < need) return MOE_ERR_WORKSPACE;
  *launch = true;
  return MOE_OK;
}

// ---- per-kernel event timing
struct EventPair {
  int kind;
  hipEvent_t start, stop;
};

struct Timing {
  std::mutex mu;
  int mask = 0;
  std::vector<EventPair> pending;
  std::vector<hipEvent_t> pool;

  hipEvent_t take() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    // timing only: no system-scope fence when the event is recorded, so
    // the pair does not add a cache write-back and invalidation around the
    // kernel it brackets (nothing reads memory through these events)
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    return e;
  }
};

Timing &timing() {
  static Timing t;
  return t;
}

template <class F>
hipError_t timed(int kind, hipStream_t st, F &&launch) {
  Timing &tm = timing();
  if (!(tm.mask & (1 << kind))) return launch();
  hipEvent_t a, b;
  {
    std::lock_guard<std::mutex> lk(tm.mu);
    a = tm.take();
    b = tm.take();
  }
  if (!a || !b) return hipErrorOutOfMemory;
  hipError_t err = hipEventRecord(a, st);
  if (err == hipSuccess) err = launch();
  if (err == hipSuccess) err = hipEventRecord(b, st);
  std::lock_guard<std::mutex> lk(tm.mu);
  tm.pending.push_back({kind, a, b});
  return err;
}

int status_of(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

int check_weights(const moe_shape *s, const moe_expert_weights *w) {
  if (!w || !w->w13 || !w->w2) return MOE_ERR_INVALID_ARG;
  if (w->layout != MOE_LAYOUT_ROWS && w->layout != MOE_LAYOUT_TILED) return MOE_ERR_INVALID_ARG;
  if (s->n_shared > 0 && (!w->ws13 || !w->ws2)) return MOE_ERR_INVALID_ARG;
  if (s->n_shared == 0 && (w->ws13 || w->ws2)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// Expert-pass workspace after the head: [G * L compaction records (dedup) |
// abuf of every layer | obuf of every layer].
size_t expert_ws(const moe_shape *s, int n, int G, int L, bool dedup) {
  return (dedup ? (size_t)G * L * cmp_ws(s, n) : 0) + (size_t)L * abuf_ws(s, n) +
         (size_t)L * obuf_ws(s, n);
}

// Weights of L layers: layer l at l * (bytes of one layer's array).
struct LayerWeights {
  const void *w13, *w2, *ws13, *ws2;
  int layout;
};

// Launches up, down and combine for L layers (L = 1: one layer) on the
// routing idx / tw ([L][N][k]); G token groups with boundaries gs (host) for
// the dedup engine (G = 1 with gs = {0, n}: the whole pass; L > 1 needs
// G = 1).  Arguments are already validated and ws is big enough.
int launch_pass(const moe_shape *s, const LayerWeights &w, int L, const float *x, int32_t n,
                int32_t G, const int32_t *gs, const int32_t *idx, const float *tw, float *y,
                int32_t *n_unique, bool dedup, void *ws, hipStream_t st) {
  const size_t rec_bytes = cmp_ws(s, n);
  const size_t c_bytes = dedup ? (size_t)G * L * rec_bytes : 0;
  const size_t a_bytes = (size_t)L * abuf_ws(s, n);
  unsigned char *base = (unsigned char *)ws;
  const bool bf16 = s->wdtype == MOE_BF16;
  const size_t fd = (size_t)s->d_model * s->d_ff * wbytes(s);

  moe::ExpertArgs a{};
  a.w13 = w.w13;
  a.w2 = w.w2;
  a.ws13 = w.ws13;
  a.ws2 = w.ws2;
  a.x = x;
  a.idx = idx;
  a.w = tw;
  a.y = y;
  a.cmp = dedup ? (int32_t *)base : nullptr;
  a.abuf = base + c_bytes;
  a.obuf = (float *)(base + c_bytes + a_bytes);
  a.cmp_out = dedup ? (int32_t *)base : nullptr;
  a.n_unique = n_unique;
  a.d = s->d_model;
  a.f = s->d_ff;
  a.E = s->n_experts;
  a.k = s->top_k;
  a.S = s->n_shared;
  a.N = n;
  a.dedup = dedup ? (G > 1 ? 2 : 1) : 0;
  a.tiled = w.layout == MOE_LAYOUT_TILED ? 1 : 0;
  const int slots = n * s->top_k;
  a.G = G;
  a.rec_ints = (int)(rec_bytes / sizeof(int32_t));
  // The dedup grid holds U_max = min(E, N*k) routed instances; folded, it
  // holds ceil(U_max / 2) and a workgroup runs a second instance only when
  // U exceeds that.  Folding pays while U stays below the fold (fewer
  // absent workgroups to dispatch) and costs a second tile per workgroup
  // when U nears U_max, so it is used only where the instance space is large
  // against the k experts every token selects: E >= 8k and a fold of at
  // least 2k.  Token groups fold one by one.
  const bool large = s->n_experts >= 8 * s->top_k;
  auto folded = [&](int m) { return (dedup && large && (m + 1) / 2 >= 2 * s->top_k) ? (m + 1) / 2 : m; };
  int routed = 0, grid_routed = 0;
  for (int g = 0; g < G; ++g) {
    const int gslots = (gs[g + 1] - gs[g]) * s->top_k;
    const int m = gslots < s->n_experts ? gslots : s->n_experts;
    a.gstart[g] = gs[g];
    a.ibase[g] = routed;
    a.fbase[g] = grid_routed;
    routed += m;
    grid_routed += folded(m);
  }
  a.gstart[G] = gs[G];
  a.ibase[G] = routed;
  a.fbase[G] = grid_routed;
  a.n_routed = dedup ? routed : slots;
  a.fold = (G == 1 && folded(routed) < routed) ? folded(routed) : 0;
  a.L = L;
  a.lw13 = 2 * fd * s->n_experts;
  a.lw2 = fd * s->n_experts;
  a.lws13 = 2 * fd * s->n_shared;
  a.lws2 = fd * s->n_shared;

  hipError_t err = hipSuccess;
  a.lds_bytes = moe::expert_lds_bytes(n, s->d_model, bf16, true, s->n_experts, s->top_k);
  err = timed(MOE_K_UP, st, [&] { return moe::launch_up(a, bf16, st); });
  if (err == hipSuccess) {
    a.lds_bytes = moe::expert_lds_bytes(n, s->d_ff, bf16, false, s->n_experts, s->top_k);
    err = timed(MOE_K_DOWN, st, [&] { return moe::launch_down(a, bf16, st); });
  }
  if (err == hipSuccess)
    err = timed(MOE_K_COMBINE, st, [&] { return moe::launch_combine(a, st); });
  return status_of(err);
}

// G token groups with boundaries gs (host) for the dedup engine; G = 1 with
// gs = {0, n} is the whole pass.
int expert_pass(const moe_shape *s, const moe_expert_weights *w, const float *x, int32_t n,
                int32_t G, const int32_t *gs, const int32_t *idx, const float *tw, float *y,
                int32_t *n_unique, bool dedup, void *ws, size_t *ws_bytes, void *stream) {
  int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if ((rc = check_tokens(s, n)) != MOE_OK) return rc;
  if ((rc = check_weights(s, w)) != MOE_OK) return rc;
  if ((rc = check_groups(n, G, gs)) != MOE_OK) return rc;
  if (!x || !idx || !tw || !y) return MOE_ERR_INVALID_ARG;
  bool launch;
  if ((rc = workspace_gate(ws, ws_bytes, kHead + expert_ws(s, n, G, 1, dedup), &launch)) !=
          MOE_OK ||
      !launch)
    return rc;
  const LayerWeights lw{w->w13, w->w2, w->ws13, w->ws2, w->layout};
  return launch_pass(s, lw, 1, x, n, G, gs, idx, tw, y, n_unique, dedup,
                     (unsigned char *)ws + kHead, (hipStream_t)stream);
}

// Gate + top-k + softmax for L layers (gate_w [L][E][d], bias [L][E] or
// NULL, outputs [L][N][...]); ws holds route_ws(s, n, L) bytes with the
// arrival counters zero.
int launch_route(const moe_shape *s, int L, const float *gate_w, const float *bias,
                 const float *x, int32_t n, float *logits, int32_t *idx, float *tw,
                 float *margin, void *ws, hipStream_t st) {
  moe::RouteArgs a{};
  a.gate_w = gate_w;
  a.bias = bias;
  a.x = x;
  a.N = n;
  a.d = s->d_model;
  a.E = s->n_experts;
  a.k = s->top_k;
  a.L = L;
  a.splits = moe::gate_splits(s->d_model);
  a.done = (unsigned *)ws;
  a.part = (float *)((unsigned char *)ws + kHead);
  a.logits = logits;
  a.idx = idx;
  a.w = tw;
  a.margin = margin;
  hipError_t err = timed(MOE_K_GATE, st, [&] { return moe::launch_gate(a, st); });
  if (err == hipSuccess && !moe::route_fused(n, s->d_model, s->n_experts))
    err = timed(MOE_K_TOPK, st, [&] { return moe::launch_topk(a, st); });
  return status_of(err);
}

bool overlaps(const void *a, const void *b, size_t n_a, size_t n_b) {
  const char *x = (const char *)a, *y = (const char *)b;
  return x < y + n_b && y < x + n_a;
}

// The filter over one or two row sets (rows_b may be 0): validation, the
// workspace gate, the launches.
int verify_probs(int32_t rows_a, const float *logits_a, float *probs_a, int32_t rows_b,
                 const float *logits_b, float *probs_b, int32_t vocab, float temperature,
                 float top_p, void *ws, size_t *ws_bytes, void *stream) {
  if (vocab < 1 || vocab > MOE_MAX_VOCAB || rows_a < 1 || !logits_a || !probs_a || rows_b < 0)
    return MOE_ERR_INVALID_ARG;
  if (rows_b > 0 && (!logits_b || !probs_b)) return MOE_ERR_INVALID_ARG;
  if (!(temperature > 0.f) || !(temperature < INFINITY) || !(top_p > 0.f) || !(top_p <= 1.f))
    return MOE_ERR_INVALID_ARG;
  const size_t na = (size_t)rows_a * vocab * sizeof(float);
  const size_t nb = (size_t)rows_b * vocab * sizeof(float);
  // no output may overlap an input or the other output
  if (overlaps(probs_a, logits_a, na, na)) return MOE_ERR_INVALID_ARG;
  if (rows_b > 0 && (overlaps(probs_b, logits_b, nb, nb) || overlaps(probs_a, logits_b, na, nb) ||
                     overlaps(probs_b, logits_a, nb, na) || overlaps(probs_a, probs_b, na, nb)))
    return MOE_ERR_INVALID_ARG;
  const int64_t rows = (int64_t)rows_a + rows_b;
  if (rows > 65535) return MOE_ERR_UNSUPPORTED;  // rows are a grid dimension
  bool launch;
  int rc;
  if ((rc = workspace_gate(ws, ws_bytes, kHead + moe::filter_ws_bytes((int)rows, vocab),
                           &launch)) != MOE_OK ||
      !launch)
    return rc;
  hipStream_t st = (hipStream_t)stream;
  const hipError_t err = timed(MOE_K_FILTER, st, [&] {
    return moe::launch_filter(rows_a, logits_a, probs_a, rows_b, logits_b, probs_b, vocab,
                              temperature, top_p, (unsigned char *)ws + kHead, st);
  });
  return status_of(err);
}

}  // namespace

extern "C" {

int moe_route(const moe_shape *s, const float *gate_w, const float *x, int32_t n,
              float *logits, int32_t *topk_idx, float *topk_w, float *margin, void *ws,
              size_t *ws_bytes, void *stream) {
  return moe_route_biased(s, gate_w, nullptr, x, n, logits, topk_idx, topk_w, margin, ws,
                          ws_bytes, stream);
}

int moe_route_biased(const moe_shape *s, const float *gate_w, const float *bias,
                     const float *x, int32_t n, float *logits, int32_t *topk_idx,
                     float *topk_w, float *margin, void *ws, size_t *ws_bytes, void *stream) {
  int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if ((rc = check_tokens(s, n)) != MOE_OK) return rc;
  if (!gate_w || !x || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
  bool launch;
  if ((rc = workspace_gate(ws, ws_bytes, route_ws(s, n), &launch)) != MOE_OK || !launch)
    return rc;
  return launch_route(s, 1, gate_w, bias, x, n, logits, topk_idx, topk_w, margin, ws,
                      (hipStream_t)stream);
}

int moe_stack_pass(const moe_shape *s, int32_t L, const moe_stack_weights *w, const float *x,
                   int32_t n, int32_t engine, int32_t *topk_idx, float *topk_w, float *y,
                   int32_t *n_unique, void *ws, size_t *ws_bytes, void *stream) {
  int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if ((rc = check_tokens(s, n)) != MOE_OK) return rc;
  if (L < 1 || L > MOE_MAX_LAYERS) return MOE_ERR_INVALID_ARG;
  if (engine != MOE_ENGINE_PERSLOT && engine != MOE_ENGINE_DEDUP) return MOE_ERR_INVALID_ARG;
  if (!w || !w->gate_w || !x || !topk_idx || !topk_w || !y) return MOE_ERR_INVALID_ARG;
  const moe_expert_weights ew{w->w13, w->w2, w->ws13, w->ws2, w->layout};
  if ((rc = check_weights(s, &ew)) != MOE_OK) return rc;
  const bool dedup = engine == MOE_ENGINE_DEDUP;
  const size_t r_bytes = route_ws(s, n, L);
  bool launch;
  if ((rc = workspace_gate(ws, ws_bytes, r_bytes + expert_ws(s, n, 1, L, dedup), &launch)) !=
          MOE_OK ||
      !launch)
    return rc;
  hipStream_t st = (hipStream_t)stream;
  rc = launch_route(s, L, w->gate_w, w->bias, x, n, nullptr, topk_idx, topk_w, nullptr, ws, st);
  if (rc != MOE_OK) return rc;
  const int32_t whole[2] = {0, n};
  const LayerWeights lw{w->w13, w->w2, w->ws13, w->ws2, w->layout};
  return launch_pass(s, lw, L, x, n, 1, whole, topk_idx, topk_w, y, n_unique, dedup,
                     (unsigned char *)ws + r_bytes, st);
}

int moe_verify_gate(int32_t n_seq, int32_t gamma, int32_t vocab, int32_t mode,
                    const float *p_verify, const float *q_draft, const int32_t *draft_tokens,
                    const float *u_accept, const uint32_t *r_sample, int32_t *n_accepted,
                    int32_t *out_tokens, void *ws, size_t *ws_bytes, void *stream) {
  if (n_seq < 1 || n_seq > MOE_MAX_SEQ || gamma < 0 || gamma > MOE_MAX_DRAFT || vocab < 1 ||
      vocab > MOE_MAX_VOCAB)
    return MOE_ERR_INVALID_ARG;
  if (mode != MOE_VERIFY_GREEDY && mode != MOE_VERIFY_SAMPLING) return MOE_ERR_INVALID_ARG;
  if (!p_verify || !n_accepted || !out_tokens || (gamma > 0 && !draft_tokens))
    return MOE_ERR_INVALID_ARG;
  if (mode == MOE_VERIFY_SAMPLING && (!r_sample || (gamma > 0 && (!q_draft || !u_accept))))
    return MOE_ERR_INVALID_ARG;
  // [arrival counters | partial results [n_seq][chunks][gamma + 1] uint64]
  const size_t need = kHead + align_up((size_t)n_seq * moe::verify_chunks(vocab) *
                                            (size_t)(gamma + 1) * sizeof(uint64_t),
                                        kAlign);
  bool launch;
  int rc;
  if ((rc = workspace_gate(ws, ws_bytes, need, &launch)) != MOE_OK || !launch) return rc;
  hipStream_t st = (hipStream_t)stream;
  const hipError_t err = timed(MOE_K_VERIFY, st, [&] {
    return moe::launch_verify(n_seq, gamma, vocab, mode, p_verify,
                              mode == MOE_VERIFY_SAMPLING ? q_draft : nullptr, draft_tokens,
                              u_accept, r_sample, n_accepted, out_tokens, ws, st);
  });
  return status_of(err);
}

int moe_verify_probs(int32_t rows, int32_t vocab, const float *logits, float temperature,
                     float top_p, float *probs, void *ws, size_t *ws_bytes, void *stream) {
  return verify_probs(rows, logits, probs, 0, nullptr, nullptr, vocab, temperature, top_p, ws,
                      ws_bytes, stream);
}

int moe_verify_probs_pair(int32_t rows_p, const float *logits_p, float *probs_p, int32_t rows_q,
                          const float *logits_q, float *probs_q, int32_t vocab,
                          float temperature, float top_p, void *ws, size_t *ws_bytes,
                          void *stream) {
  if (rows_q < 1) return MOE_ERR_INVALID_ARG;
  return verify_probs(rows_p, logits_p, probs_p, rows_q, logits_q, probs_q, vocab, temperature,
                      top_p, ws, ws_bytes, stream);
}

int moe_filter_spin_limit(uint32_t polls) {
  moe::set_filter_spin_limit(polls);
  return MOE_OK;
}

int moe_expert_pass_perslot(const moe_shape *s, const moe_expert_weights *w, const float *x,
                            int32_t n, const int32_t *idx, const float *tw, float *y,
                            void *ws, size_t *ws_bytes, void *stream) {
  const int32_t whole[2] = {0, n};
  return expert_pass(s, w, x, n, 1, whole, idx, tw, y, nullptr, false, ws, ws_bytes, stream);
}

int moe_expert_pass_dedup(const moe_shape *s, const moe_expert_weights *w, const float *x,
                          int32_t n, const int32_t *idx, const float *tw, float *y,
                          int32_t *n_unique, void *ws, size_t *ws_bytes, void *stream) {
  const int32_t whole[2] = {0, n};
  return expert_pass(s, w, x, n, 1, whole, idx, tw, y, n_unique, true, ws, ws_bytes, stream);
}

int moe_expert_pass_dedup_grouped(const moe_shape *s, const moe_expert_weights *w,
                                  const float *x, int32_t n, int32_t n_groups,
                                  const int32_t *group_start, const int32_t *idx,
                                  const float *tw, float *y, int32_t *n_unique, void *ws,
                                  size_t *ws_bytes, void *stream) {
  return expert_pass(s, w, x, n, n_groups, group_start, idx, tw, y, n_unique, true, ws,
                     ws_bytes, stream);
}

int moe_pack_weights(const moe_shape *s, int32_t n_sets, const void *w13_rows,
                     const void *w2_rows, void *w13_tiled, void *w2_tiled, void *stream) {
  int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if (n_sets < 0) return MOE_ERR_INVALID_ARG;
  if ((w13_rows == nullptr) != (w13_tiled == nullptr)) return MOE_ERR_INVALID_ARG;
  if ((w2_rows == nullptr) != (w2_tiled == nullptr)) return MOE_ERR_INVALID_ARG;
  const size_t eb = wbytes(s);
  const size_t fd = (size_t)s->d_model * s->d_ff * eb;
  auto overlap = [](const void *a, size_t na, const void *b, size_t nb) {
    const char *pa = (const char *)a, *pb = (const char *)b;
    return pa < pb + nb && pb < pa + na;
  };
  if (w13_rows && overlap(w13_rows, 2 * fd * n_sets, w13_tiled, 2 * fd * n_sets))
    return MOE_ERR_INVALID_ARG;
  if (w2_rows && overlap(w2_rows, fd * n_sets, w2_tiled, fd * n_sets)) return MOE_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  const bool bf16 = s->wdtype == MOE_BF16;
  hipError_t err = hipSuccess;
  if (w13_rows)  // W1 and W3: 2 n matrices of [f][d]
    err = moe::launch_pack(w13_rows, w13_tiled, s->d_ff, s->d_model, 2LL * n_sets, bf16, st);
  if (err == hipSuccess && w2_rows)  // W2: n matrices of [d][f]
    err = moe::launch_pack(w2_rows, w2_tiled, s->d_model, s->d_ff, (long long)n_sets, bf16, st);
  return status_of(err);
}

int moe_pass_bytes(const moe_shape *s, const int32_t *idx, int32_t n, uint64_t *perslot,
                   uint64_t *dedup, uint64_t *shared, int32_t *n_unique) {
  int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if ((rc = check_tokens(s, n)) != MOE_OK) return rc;
  if (!idx) return MOE_ERR_INVALID_ARG;
  const int E = s->n_experts;
  std::vector<unsigned char> seen((size_t)E, 0);
  int32_t U = 0;
  const size_t slots = (size_t)n * s->top_k;
  for (size_t i = 0; i < slots; ++i) {
    const int32_t e = idx[i];
    if (e < 0 || e >= E) return MOE_ERR_INVALID_ARG;
    if (!seen[(size_t)e]) {
      seen[(size_t)e] = 1;
      ++U;
    }
  }
  const uint64_t be = 3ull * (uint64_t)s->d_model * (uint64_t)s->d_ff * wbytes(s);
  if (perslot) *perslot = (uint64_t)slots * be;
  if (dedup) *dedup = (uint64_t)U * be;
  if (shared) *shared = (uint64_t)s->n_shared * be;
  if (n_unique) *n_unique = U;
  return MOE_OK;
}

int moe_pass_bytes_grouped(const moe_shape *s, const int32_t *idx, int32_t n, int32_t G,
                           const int32_t *gs, uint64_t *dedup, int32_t *n_unique) {
  int rc = check_shape(s);
  if (rc != MOE_OK) return rc;
  if ((rc = check_tokens(s, n)) != MOE_OK) return rc;
  if ((rc = check_groups(n, G, gs)) != MOE_OK) return rc;
  if (!idx) return MOE_ERR_INVALID_ARG;
  uint64_t total = 0;
  for (int g = 0; g < G; ++g) {
    uint64_t b = 0;
    int32_t u = 0;
    rc = moe_pass_bytes(s, idx + (size_t)gs[g] * s->top_k, gs[g + 1] - gs[g], nullptr, &b,
                        nullptr, &u);
    if (rc != MOE_OK) return rc;
    total += b;
    if (n_unique) n_unique[g] = u;
  }
  if (dedup) *dedup = total;
  return MOE_OK;
}

const char *moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int moe_timing_enable(int mask) {
  Timing &tm = timing();
  std::lock_guard<std::mutex> lk(tm.mu);
  tm.mask = mask & ((1 << MOE_K_COUNT) - 1);
  return MOE_OK;
}

int moe_timing_read(double *ms, int64_t *launches) {
  Timing &tm = timing();
  std::lock_guard<std::mutex> lk(tm.mu);
  int rc = MOE_OK;
  for (const EventPair &p : tm.pending) {
    float el = 0.f;
    if (hipEventSynchronize(p.stop) != hipSuccess ||
        hipEventElapsedTime(&el, p.start, p.stop) != hipSuccess) {
      rc = MOE_ERR_HIP;
    } else {
      if (ms) ms[p.kind] += (double)el;
      if (launches) launches[p.kind] += 1;
    }
    tm.pool.push_back(p.start);
    tm.pool.push_back(p.stop);
  }
  tm.pending.clear();
  return rc;
}

}  // extern "C"
