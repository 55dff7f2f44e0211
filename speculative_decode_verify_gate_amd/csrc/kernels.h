// kernels.h -- internal launch interface between the C ABI (abi.cpp) and the
// gfx950 kernels.  Not installed; the public interface is include/moe_verify.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_verify.h"

namespace moe {

// Geometry shared by the launchers and the workspace sizing in abi.cpp.
constexpr int kWave = 64;
constexpr int kTile = 16;               // MFMA output tile is 16 rows x 16 tokens
constexpr int kWavesPerBlock = 4;       // expert kernels: waves per 16-row tile

constexpr int kGateKPerBlock = 256;     // gate logits: K elements per workgroup
constexpr int kLdsBudget = 36 * 1024;   // staged activations per workgroup, when a
                                        // token group's K window fits it (four
                                        // workgroups per CU); wider windows take
                                        // up to expert_lds_bound(true)
constexpr int kLdsPad = 8;              // elements of padding per staged row
constexpr int kSpc = 4;                 // expert kernels: MFMA steps per K chunk

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Offsets (int32 elements) of the compaction record at the head of the dedup
// workspace; the layout is part of the public contract.
struct CompactLayout {
  int E, slots;
  __host__ __device__ int u() const { return 0; }
  __host__ __device__ int counts() const { return 1; }
  __host__ __device__ int offs() const { return 1 + E; }
  __host__ __device__ int uniq() const { return 2 + 2 * E; }
  __host__ __device__ int list() const { return 2 + 3 * E; }
  __host__ __device__ int total() const { return 2 + 3 * E + slots; }
};

// LDS ints the compaction-record writer needs for E experts and `slots`
// routing entries: a count per expert (then its offset), the valid expert
// of each slot, and per expert a bit mask of its slots.
__host__ __device__ constexpr int record_lds_ints(int E, int slots) {
  return E + slots + E * ((slots + 31) / 32);
}

struct ExpertArgs {
  const void *w13, *w2, *ws13, *ws2;
  const float *x;         // [N][d]
  const int32_t *idx;     // [N][k]
  const float *w;         // [N][k] routing weights
  float *y;               // [N][d] layer output
  const int32_t *cmp;     // compaction record (dedup) or nullptr
  void *abuf;             // [N*k + S*N][f] SwiGLU outputs, weight element type
  float *obuf;            // [N*k + S*N][d] expert outputs
  int32_t *cmp_out;       // dedup up kernel: where workgroup 0 writes the record
  int32_t *n_unique;      // dedup up kernel: U for the caller, or nullptr
  int d, f, E, k, S, N;
  int tiled;              // weight layout: 0 row-major, 1 MOE_LAYOUT_TILED
  int dedup;              // 0: instance i is slot i; 1: instance u is the
                          //    u-th distinct selected expert; 2: the same
                          //    within each token group of the tables below
  int n_routed;           // routed instances (U_max for the dedup engine)
  int fold;               // dedup, one group: routed instance slots per
                          // layer in the grid (slot v runs v, then v + fold
                          // if present), or 0: one slot per routed instance
                          // (grouped passes use fbase instead)
  int lds_bytes;          // dynamic LDS per workgroup
  // Dedup within token groups: tokens gstart[g] .. gstart[g+1]-1 form group
  // g, whose distinct experts are routed instances ibase[g] .. ibase[g+1]-1
  // and whose compaction record starts rec_ints int32 after group g-1's.
  // Read only when dedup == 2; the plain engines run with G = 1.
  int G;
  int rec_ints;
  // A stack of L layers (L = 1: one layer): layer l's weights start
  // l * lw13 / lw2 / lws13 / lws2 bytes into the arrays, its routing,
  // compaction record (rec_ints int32 apart), U, rows, and y follow the
  // previous layer's.
  int L;
  size_t lw13, lw2, lws13, lws2;
  int gstart[MOE_MAX_GROUPS + 1];
  int ibase[MOE_MAX_GROUPS + 1];
  // Grouped dedup: group g's routed slots in the grid start at fbase[g]
  // (fbase[g+1] - fbase[g] is its instance count ibase[g+1] - ibase[g], or
  // half of it rounded up when the group's grid is folded).
  int fbase[MOE_MAX_GROUPS + 1];
};

// Routing.  Partial logits of all splits at most this many bytes: one launch
// (the last gate workgroup also runs the top-k); otherwise gate + top-k.
constexpr int kFusedRouteBytes = 64 * 1024;

// A stack of L layers routes the same N tokens through L gates; every
// array below then holds L consecutive per-layer blocks (L = 1: one layer).
struct RouteArgs {
  const float *gate_w, *x;    // [L][E][d], [N][d]
  const float *bias;          // [L][E] added to the logits, or nullptr
  int N, d, E, k, splits, L;
  float *part;                // [L][splits][N][E] partial logits
  unsigned *done;             // [L] arrival counters (one launch): zero on entry and exit
  float *logits;              // [L][N][E] or nullptr
  int32_t *idx;               // [L][N][k]
  float *w;                   // [L][N][k]
  float *margin;              // [L][N] or nullptr
};

// Row length of a token's logits in the router's LDS: E rounded up to whole
// 16-byte vectors.
__host__ __device__ inline int logit_ld(int E) { return (E + 3) & ~3; }
constexpr int kFusedRouteLds = 32 * 1024;  // one-launch routing: [N][E] logits in LDS

inline int gate_splits(int d) { return (d + kGateKPerBlock - 1) / kGateKPerBlock; }

// One launch routes the pass when the partials that its last workgroup sums
// and that workgroup's LDS copy of the logits are small enough.
inline bool route_fused(int N, int d, int E) {
  return (size_t)gate_splits(d) * N * E * sizeof(float) <= (size_t)kFusedRouteBytes &&
         (size_t)N * logit_ld(E) * sizeof(float) <= (size_t)kFusedRouteLds;
}

hipError_t launch_gate(const RouteArgs &a, hipStream_t st);
hipError_t launch_topk(const RouteArgs &a, hipStream_t st);

// Expert pass = up kernel (in the dedup engine it also compacts the
// routing), down kernel, combine kernel.  bf16 selects bf16 weights, else
// fp32.
hipError_t launch_up(const ExpertArgs &a, bool bf16, hipStream_t st);
hipError_t launch_down(const ExpertArgs &a, bool bf16, hipStream_t st);
hipError_t launch_combine(const ExpertArgs &a, hipStream_t st);
// Row-major -> MOE_LAYOUT_TILED for n_mats matrices of R x K.
hipError_t launch_pack(const void *src, void *dst, int R, int K, long long n_mats, bool bf16,
                       hipStream_t st);

// Dynamic LDS for the expert kernels at this token count: the partial sums
// (16-token tiles, which read their token columns directly), or K windows of
// up to min(N, 64) staged token rows.
inline int expert_lds_bytes(int N, int K, bool bf16, bool up, int E, int k) {
  const int eb = bf16 ? 2 : 4;
  const int ctmax = N > kTile ? 4 : 1;
  // the partial sums of 16-token tiles, or, in a record-writing workgroup of
  // the up kernel, the compaction scratch (at most a pass's N k slots)
  const size_t record = up ? (size_t)record_lds_ints(E, N * k) * sizeof(int) : 0;
  if (ctmax == 1) {
    const size_t partials = (size_t)(up ? 2 : 1) * kWavesPerBlock * kWave * 16;
    return (int)(partials > record ? partials : record);
  }
  const int step = bf16 ? 32 : 16;
  const int chunk = kSpc * step;
  const int rows = ctmax * kTile;
  const int kpad = (K + kWavesPerBlock * chunk - 1) / (kWavesPerBlock * chunk) *
                   (kWavesPerBlock * chunk);
  // the whole K for as many token rows as an instance can have (at most N
  // unless a caller's routing repeats an expert within a token)
  const int rows_n = N < rows ? N : rows;
  const size_t whole = (size_t)rows_n * (kpad + kLdsPad) * eb;
  // at least one chunk per wave for a full token group, and room for the
  // waves' partial sums
  const size_t least = (size_t)rows * (kWavesPerBlock * chunk + kLdsPad) * eb;
  // two weight streams: W1 and W3 (up), or a pair of W2 tiles (wide down)
  const size_t partials = (size_t)2 * kWavesPerBlock * ctmax * kWave * 16;
  size_t bytes = whole < (size_t)kLdsBudget ? whole : (size_t)kLdsBudget;
  if (bytes < least) bytes = least;
  if (bytes < partials) bytes = partials;
  if (bytes < record) bytes = record;
  return (int)bytes;
}

// The most expert_lds_bytes() can ask for, over every shape: 16-token tiles
// (wide = false) or the LDS-staged wide tiles (wide = true).  The kernels'
// dynamic-LDS limit is set to it, and every launch is checked against it.
constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int expert_lds_bound(bool wide) {
  return wide ? cmax(cmax(kLdsBudget, 4 * kTile * (kWavesPerBlock * kSpc * 32 + kLdsPad) * 2),
                     cmax(4 * kTile * (kWavesPerBlock * kSpc * 16 + kLdsPad) * 4,
                          2 * kWavesPerBlock * 4 * kWave * 16))
              : cmax(2 * kWavesPerBlock * kWave * 16,
                     record_lds_ints(MOE_MAX_EXPERTS, MOE_MAX_SLOTS) * (int)sizeof(int));
}
static_assert(expert_lds_bound(true) >=
                  record_lds_ints(MOE_MAX_EXPERTS, MOE_MAX_SLOTS) * (int)sizeof(int),
              "a wide up kernel's LDS must also hold the compaction scratch");

}  // namespace moe
