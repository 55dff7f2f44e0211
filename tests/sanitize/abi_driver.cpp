// Host-side driver of the C ABI (include/moe_verify.h) for AddressSanitizer
// and UBSan builds on the CPU.  The kernel launchers are replaced by stubs
// that check the launch descriptors the ABI builds and launch nothing, so
// argument validation, workspace sizing, group and layer tables and the host
// byte accounting all run for real without a GPU.  Device pointers are host
// addresses that nothing dereferences.  Exit status 0 = every check held.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "kernels.h"
#include "moe_verify.h"
#include "verify.h"

static int g_fail = 0;
#define CHECK(c)                                                     \
  do {                                                               \
    if (!(c)) {                                                      \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++g_fail;                                                      \
    }                                                                \
  } while (0)

namespace moe {
static int g_launches = 0;

int verify_chunks(int V) { return (V + 2047) / 2048; }

hipError_t launch_gate(const RouteArgs &a, hipStream_t) {
  CHECK(a.L >= 1 && a.L <= MOE_MAX_LAYERS && a.N >= 1 && a.splits == gate_splits(a.d));
  CHECK(a.gate_w && a.x && a.idx && a.w && a.done && a.part);
  ++g_launches;
  return hipSuccess;
}
static int g_topk_launches = 0;
hipError_t launch_topk(const RouteArgs &a, hipStream_t) {
  CHECK(!route_fused(a.N, a.d, a.E));
  ++g_topk_launches;
  ++g_launches;
  return hipSuccess;
}
static void check_expert(const ExpertArgs &a) {
  CHECK(a.G >= 1 && a.G <= MOE_MAX_GROUPS && a.L >= 1 && a.L <= MOE_MAX_LAYERS);
  CHECK(a.gstart[0] == 0 && a.gstart[a.G] == a.N && a.ibase[0] == 0);
  for (int g = 0; g < a.G; ++g) {
    const int slots = (a.gstart[g + 1] - a.gstart[g]) * a.k;
    CHECK(a.gstart[g + 1] > a.gstart[g]);
    CHECK(a.ibase[g + 1] - a.ibase[g] == (slots < a.E ? slots : a.E));
  }
  CHECK(a.n_routed == (a.dedup ? a.ibase[a.G] : a.N * a.k));
  CHECK(a.dedup == 0 || a.dedup == (a.G > 1 ? 2 : 1));
  CHECK(a.L == 1 || a.G == 1);
  CHECK((a.cmp != nullptr) == (a.dedup != 0) && a.abuf && a.obuf && a.y && a.x);
  CHECK((size_t)a.rec_ints * 4 % 256 == 0 && a.rec_ints >= 2 + 3 * a.E + a.N * a.k);
  // the dynamic LDS the launch asks for is within the limit set on the kernel
  CHECK(a.lds_bytes > 0 && a.lds_bytes <= expert_lds_bound(a.N > kTile));
  // grid slots per token group: the group's instances, or half of them
  // rounded up where its dedup grid folds (E >= 8k, half >= 2k)
  CHECK(a.fbase[0] == 0);
  for (int g = 0; g < a.G; ++g) {
    const int m = a.ibase[g + 1] - a.ibase[g], f = a.fbase[g + 1] - a.fbase[g];
    const bool fold = a.dedup != 0 && a.E >= 8 * a.k && (m + 1) / 2 >= 2 * a.k;
    CHECK(f == (fold ? (m + 1) / 2 : m));
  }
  // folded dedup grid: one group, half the routed slots (so two passes
  // cover U_max), E >= 8k and a fold of at least 2k
  if (a.fold != 0) {
    CHECK(a.dedup == 1 && a.G == 1);
    CHECK(a.fold == (a.n_routed + 1) / 2 && 2 * a.fold >= a.n_routed);
    CHECK(a.E >= 8 * a.k && a.fold >= 2 * a.k);
  } else if (a.dedup == 1) {
    CHECK(a.E < 8 * a.k || (a.n_routed + 1) / 2 < 2 * a.k);
  }
}
hipError_t launch_up(const ExpertArgs &a, bool, hipStream_t) {
  check_expert(a);
  // a record-writing workgroup's scratch fits the dynamic LDS of the launch
  CHECK(a.dedup == 0 || a.lds_bytes >= record_lds_ints(a.E, a.N * a.k) * (int)sizeof(int));
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_down(const ExpertArgs &a, bool, hipStream_t) { check_expert(a); ++g_launches; return hipSuccess; }
hipError_t launch_combine(const ExpertArgs &a, hipStream_t) { check_expert(a); ++g_launches; return hipSuccess; }
hipError_t launch_pack(const void *, void *, int R, int K, long long n, bool, hipStream_t) {
  CHECK(R > 0 && K > 0 && n >= 0);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_verify(int n_seq, int gamma, int V, int mode, const float *p, const float *,
                         const int32_t *, const float *, const uint32_t *, int32_t *n_acc,
                         int32_t *out, void *ws, hipStream_t) {
  CHECK(n_seq >= 1 && gamma >= 0 && V >= 1 && (mode == 0 || mode == 1) && p && n_acc && out && ws);
  ++g_launches;
  return hipSuccess;
}
size_t filter_ws_bytes(int rows, int V) { return (size_t)rows * (V / 4096 + 1) * 4200; }
static unsigned g_spin_limit = 0;
void set_filter_spin_limit(unsigned polls) { g_spin_limit = polls; }
hipError_t launch_filter(int rows_a, const float *lg_a, float *out_a, int rows_b,
                         const float *lg_b, float *out_b, int V, float T, float top_p, void *ws,
                         hipStream_t) {
  CHECK(rows_a >= 1 && rows_b >= 0 && V >= 1 && lg_a && out_a && ws && T > 0.f && top_p > 0.f &&
        top_p <= 1.f);
  CHECK(rows_b == 0 || (lg_b && out_b));
  CHECK(rows_a + rows_b <= 65535);
  ++g_launches;
  return hipSuccess;
}
}  // namespace moe

static void *fake(size_t off = 0) { return (void *)(uintptr_t)(0x100000 + off); }

struct Buf {  // 256-byte aligned host buffer standing in for a workspace
  void *p = nullptr;
  explicit Buf(size_t n) { p = std::aligned_alloc(256, (n + 255) / 256 * 256 + 256); }
  ~Buf() { std::free(p); }
};

int main() {
  // the workloads' shapes, and a narrow gate with many experts whose routing
  // takes one launch at small N and two at N = 64 (the partials fit 64 KB,
  // the LDS copy of the logits does not)
  const moe_shape shapes[] = {{256, 8, 2, 512, 0, MOE_F32}, {2048, 64, 6, 1408, 2, MOE_BF16},
                              {7168, 256, 8, 2048, 1, MOE_BF16}, {4096, 8, 2, 14336, 0, MOE_BF16},
                              {256, 256, 8, 512, 0, MOE_BF16}};
  for (const moe_shape &s : shapes) {
    const int topk_before = moe::g_topk_launches;
    const moe_expert_weights w{fake(), fake(), s.n_shared ? fake() : nullptr,
                               s.n_shared ? fake() : nullptr, MOE_LAYOUT_TILED};
    for (int n : {1, 3, 16, 17, 64}) {
      if (n * s.top_k > MOE_MAX_SLOTS) continue;
      size_t need = 0;
      CHECK(moe_route(&s, (float *)fake(), (float *)fake(), n, nullptr, (int32_t *)fake(),
                      (float *)fake(), nullptr, nullptr, &need, nullptr) == MOE_OK);
      {
        Buf ws(need);
        size_t have = need;
        CHECK(moe_route_biased(&s, (float *)fake(), (float *)fake(), (float *)fake(), n,
                               nullptr, (int32_t *)fake(), (float *)fake(), nullptr, ws.p,
                               &have, nullptr) == MOE_OK);
        have = need - 1;
        CHECK(moe_route(&s, (float *)fake(), (float *)fake(), n, nullptr, (int32_t *)fake(),
                        (float *)fake(), nullptr, ws.p, &have, nullptr) == MOE_ERR_WORKSPACE);
      }
      // per-slot, dedup and grouped passes with every group count up to n
      for (int G = 0; G <= (n < MOE_MAX_GROUPS ? n : MOE_MAX_GROUPS); ++G) {
        std::vector<int32_t> gs;
        if (G > 0) {
          for (int g = 0; g <= G; ++g) gs.push_back((int32_t)((long long)g * n / G));
        }
        size_t nb = 0;
        int rc;
        if (G == 0)
          rc = moe_expert_pass_perslot(&s, &w, (float *)fake(), n, (int32_t *)fake(),
                                       (float *)fake(), (float *)fake(), nullptr, &nb, nullptr);
        else
          rc = moe_expert_pass_dedup_grouped(&s, &w, (float *)fake(), n, G, gs.data(),
                                             (int32_t *)fake(), (float *)fake(),
                                             (float *)fake(), nullptr, nullptr, &nb, nullptr);
        CHECK(rc == MOE_OK && nb > 0);
        Buf ws(nb);
        size_t have = nb;
        if (G == 0)
          rc = moe_expert_pass_perslot(&s, &w, (float *)fake(), n, (int32_t *)fake(),
                                       (float *)fake(), (float *)fake(), ws.p, &have, nullptr);
        else
          rc = moe_expert_pass_dedup_grouped(&s, &w, (float *)fake(), n, G, gs.data(),
                                             (int32_t *)fake(), (float *)fake(),
                                             (float *)fake(), (int32_t *)fake(), ws.p, &have,
                                             nullptr);
        CHECK(rc == MOE_OK);
      }
      // the stack pass at 1, 2 and the most layers, both engines
      const moe_stack_weights sw{(float *)fake(), nullptr, fake(), fake(),
                                 s.n_shared ? fake() : nullptr, s.n_shared ? fake() : nullptr,
                                 MOE_LAYOUT_TILED};
      for (int L : {1, 2, MOE_MAX_LAYERS})
        for (int eng : {MOE_ENGINE_PERSLOT, MOE_ENGINE_DEDUP}) {
          size_t nb = 0;
          CHECK(moe_stack_pass(&s, L, &sw, (float *)fake(), n, eng, (int32_t *)fake(),
                               (float *)fake(), (float *)fake(), nullptr, nullptr, &nb,
                               nullptr) == MOE_OK);
          Buf ws(nb);
          size_t have = nb;
          CHECK(moe_stack_pass(&s, L, &sw, (float *)fake(), n, eng, (int32_t *)fake(),
                               (float *)fake(), (float *)fake(), (int32_t *)fake(), ws.p,
                               &have, nullptr) == MOE_OK);
        }
      // host byte accounting reads real host routing
      std::vector<int32_t> idx((size_t)n * s.top_k);
      for (size_t i = 0; i < idx.size(); ++i) idx[i] = (int32_t)((i * 7 + i / s.top_k) % s.n_experts);
      uint64_t ps = 0, dd = 0, sh = 0;
      int32_t U = 0;
      CHECK(moe_pass_bytes(&s, idx.data(), n, &ps, &dd, &sh, &U) == MOE_OK);
      const int32_t whole[2] = {0, n};
      uint64_t dg = 0;
      int32_t Ug = 0;
      CHECK(moe_pass_bytes_grouped(&s, idx.data(), n, 1, whole, &dg, &Ug) == MOE_OK);
      CHECK(dg == dd && Ug == U && U <= n * s.top_k && (uint64_t)U * 3 * s.d_model * s.d_ff <= dd);
    }
    // the narrow many-expert gate routes N = 64 in two launches, N = 1 in one
    if (s.d_model == 256 && s.n_experts == 256) {
      CHECK(moe::g_topk_launches > topk_before);
      CHECK(moe::route_fused(1, 256, 256) && !moe::route_fused(64, 256, 256));
    }
  }
  // rejected arguments
  const moe_shape s = shapes[1];
  const int32_t bad_groups[][4] = {{1, 4, 0, 0}, {0, 2, 2, 4}, {0, 3, 2, 4}};
  for (auto &g : bad_groups)
    CHECK(moe_pass_bytes_grouped(&s, (int32_t *)fake(), 4, 3, g, nullptr, nullptr) ==
          MOE_ERR_INVALID_ARG);
  std::vector<int32_t> oob = {0, 1, 2, 3, 4, 64};
  CHECK(moe_pass_bytes(&s, oob.data(), 1, nullptr, nullptr, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
  size_t nb = 0;
  CHECK(moe_stack_pass(&s, MOE_MAX_LAYERS + 1, nullptr, nullptr, 4, 0, nullptr, nullptr, nullptr,
                       nullptr, nullptr, &nb, nullptr) == MOE_ERR_INVALID_ARG);
  // the verification round
  for (int gamma : {0, 1, 8, MOE_MAX_DRAFT}) {
    CHECK(moe_verify_gate(4, gamma, 102400, 1, (float *)fake(), (float *)fake(),
                          (int32_t *)fake(), (float *)fake(), (uint32_t *)fake(),
                          (int32_t *)fake(), (int32_t *)fake(), nullptr, &nb, nullptr) == MOE_OK);
    Buf ws(nb);
    size_t have = nb;
    CHECK(moe_verify_gate(4, gamma, 102400, 1, (float *)fake(), (float *)fake(),
                          (int32_t *)fake(), (float *)fake(), (uint32_t *)fake(),
                          (int32_t *)fake(), (int32_t *)fake(), ws.p, &have, nullptr) == MOE_OK);
  }
  CHECK(moe_pack_weights(&s, 2, fake(), fake(), fake(1 << 30), fake(3u << 29), nullptr) == MOE_OK);
  CHECK(moe_verify_probs(36, 129280, (float *)fake(), 0.7f, 0.9f, (float *)fake(1u << 30),
                         nullptr, &nb, nullptr) == MOE_OK && nb > 0);
  {
    Buf ws(nb);
    size_t have = nb;
    CHECK(moe_verify_probs(36, 129280, (float *)fake(), 0.7f, 0.9f, (float *)fake(1u << 30),
                           ws.p, &have, nullptr) == MOE_OK);
  }
  CHECK(moe_verify_probs(2, 1000, (float *)fake(), 0.7f, 0.9f, (float *)fake(100), nullptr, &nb,
                         nullptr) == MOE_ERR_INVALID_ARG);  // overlapping
  // the pair: both row sets through one launch sequence, workspace for all rows
  size_t nb2 = 0;
  CHECK(moe_verify_probs_pair(36, (float *)fake(), (float *)fake(1u << 30), 32,
                              (float *)fake(2u << 30), (float *)fake(3u << 30), 129280, 0.7f, 0.9f,
                              nullptr, &nb2, nullptr) == MOE_OK && nb2 > nb);
  {
    Buf ws(nb2);
    size_t have = nb2;
    CHECK(moe_verify_probs_pair(36, (float *)fake(), (float *)fake(1u << 30), 32,
                                (float *)fake(2u << 30), (float *)fake(3u << 30), 129280, 0.7f,
                                0.9f, ws.p, &have, nullptr) == MOE_OK);
  }
  CHECK(moe_verify_probs_pair(36, (float *)fake(), (float *)fake(1u << 30), 32,
                              (float *)fake(2u << 30), (float *)fake(1u << 30), 129280, 0.7f, 0.9f,
                              nullptr, &nb2, nullptr) == MOE_ERR_INVALID_ARG);  // outputs overlap
  // the filter's barrier limit: passed through, 0 restores the default
  CHECK(moe_filter_spin_limit(3) == MOE_OK && moe::g_spin_limit == 3);
  CHECK(moe_filter_spin_limit(0) == MOE_OK && moe::g_spin_limit == 0);
  std::printf("abi driver: %d launches described, %d failed checks\n", moe::g_launches, g_fail);
  return g_fail == 0 ? 0 : 1;
}
