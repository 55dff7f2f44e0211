// router.hip -- gate logits, top-k and softmax over the k on gfx950.
//
// "Deep Dive into Mixture of Experts: From 1991 to DeepSeek-V3", section 2:
// logits = x @ gate_weights, keep the k largest, weights = softmax of the k
// selected values.  Ties are broken toward the lower expert index.
//
// Two launches.  The gate GEMM [N x d] x [d x E] streams the fp32 gate matrix
// once with fp32 MFMA (16 experts x 16 tokens per tile), split over K so
// that enough workgroups stream it; each split writes fp32 partial logits.
// The top-k kernel sums the partials in a fixed order (deterministic), then a
// single wavefront per token runs k rounds of a (value desc, index asc)
// argmax butterfly across the 64 lanes.
#include <math.h>

#include "kernels.h"

namespace moe {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGateWaves = 4;
constexpr int kGateKPerWave = kGateKPerBlock / kGateWaves;  // 64 = 4 steps of 16
constexpr int kMaxColTiles = 4;                              // N <= 64

// Partial logits of one 16-expert tile over one K split.
// part[split][t][e] = sum over the split's K range of x[t][i] * gate_w[e][i].
__global__ __launch_bounds__(256) void gate_kernel(const float *__restrict__ gate_w,
                                                   const float *__restrict__ x, int N, int d,
                                                   int E, float *__restrict__ part) {
  const int n_et = (E + kTile - 1) / kTile;
  const int et = blockIdx.x % n_et;
  const int split = blockIdx.x / n_et;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;  // A row (expert) / B column (token) of this lane
  const int g = lane >> 4;  // K group of this lane
  const int n_ct = (N + kTile - 1) / kTile;

  const int k_begin = split * kGateKPerBlock + wave * kGateKPerWave;
  const int expert = et * kTile + r;

  f32x4 acc[kMaxColTiles];
#pragma unroll
  for (int ct = 0; ct < kMaxColTiles; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Each step covers 16 K elements: lane group g holds elements 4g..4g+3 of
  // the step, and fp32 MFMA number v consumes element v of every group.
#pragma unroll
  for (int s = 0; s < kGateKPerWave / 16; ++s) {
    const int k0 = k_begin + s * 16;
    if (k0 >= d) break;
    f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
    if (expert < E) a = *(const f32x4 *)(gate_w + (size_t)expert * d + k0 + 4 * g);
#pragma unroll
    for (int ct = 0; ct < kMaxColTiles; ++ct) {
      if (ct < n_ct) {
        const int tok = ct * kTile + r;
        f32x4 b = f32x4{0.f, 0.f, 0.f, 0.f};
        if (tok < N) b = *(const f32x4 *)(x + (size_t)tok * d + k0 + 4 * g);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, acc[ct], 0, 0, 0);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, acc[ct], 0, 0, 0);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, acc[ct], 0, 0, 0);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, acc[ct], 0, 0, 0);
      }
    }
  }

  // Sum the four waves' partials in wave order.
  __shared__ f32x4 red[kGateWaves][kMaxColTiles][64];
#pragma unroll
  for (int ct = 0; ct < kMaxColTiles; ++ct)
    if (ct < n_ct) red[wave][ct][lane] = acc[ct];
  __syncthreads();
  if (wave < n_ct) {
    const int ct = wave;
    f32x4 s = red[0][ct][lane];
#pragma unroll
    for (int w = 1; w < kGateWaves; ++w) s += red[w][ct][lane];
    // lane holds rows (experts) 4g..4g+3 of the tile for token column r
    const int tok = ct * kTile + r;
    if (tok < N) {
      float *dst = part + ((size_t)split * N + tok) * E;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int e = et * kTile + 4 * g + v;
        if (e < E) dst[e] = s[v];
      }
    }
  }
}

__device__ inline bool ranks_before(float v1, int e1, float v2, int e2) {
  return v1 > v2 || (v1 == v2 && e1 < e2);
}

constexpr int kMaxExpertsPerLane = MOE_MAX_EXPERTS / 64;

// One wavefront per token.
__global__ __launch_bounds__(64) void topk_kernel(const float *__restrict__ part, int splits,
                                                  int N, int E, int k,
                                                  float *__restrict__ logits,
                                                  int32_t *__restrict__ idx,
                                                  float *__restrict__ w,
                                                  float *__restrict__ margin) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  float v[kMaxExpertsPerLane];
  bool taken[kMaxExpertsPerLane];
  const int n_q = (E + 63) / 64;
#pragma unroll
  for (int q = 0; q < kMaxExpertsPerLane; ++q) v[q] = 0.f;
  // Sum the K-split partials in split order.  Loads of 8 splits (for every
  // expert of the lane) are issued together so the partials, written by the
  // gate kernel on other XCDs, cost one memory round trip per 8 splits.
  for (int sp0 = 0; sp0 < splits; sp0 += 8) {
    float pv[kMaxExpertsPerLane][8];
#pragma unroll
    for (int q = 0; q < kMaxExpertsPerLane; ++q) {
      if (q < n_q) {
        const int e = min(q * 64 + lane, E - 1);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int sp = min(sp0 + u, splits - 1);
          pv[q][u] = part[((size_t)sp * N + t) * E + e];
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kMaxExpertsPerLane; ++q)
      if (q < n_q) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (sp0 + u < splits) v[q] += pv[q][u];
      }
  }
#pragma unroll
  for (int q = 0; q < kMaxExpertsPerLane; ++q) {
    const int e = q * 64 + lane;
    taken[q] = !(e < E);
    if (e < E) {
      if (logits) logits[(size_t)t * E + e] = v[q];
    } else {
      v[q] = -INFINITY;
    }
  }

  __shared__ float sel_v[MOE_MAX_TOPK + 1];
  __shared__ int sel_e[MOE_MAX_TOPK + 1];
  const int rounds = (k < E) ? k + 1 : k;
  for (int rd = 0; rd < rounds; ++rd) {
    // best untaken candidate of this lane
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < kMaxExpertsPerLane; ++q) {
      const int e = q * 64 + lane;
      if (!taken[q] && (be == 0x7fffffff || ranks_before(v[q], e, bv, be))) {
        bv = v[q];
        be = e;
      }
    }
    // butterfly: every lane ends with the same (unique) winner
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oe = __shfl_xor(be, off, 64);
      if (oe != 0x7fffffff && (be == 0x7fffffff || ranks_before(ov, oe, bv, be))) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) {
#pragma unroll
      for (int q = 0; q < kMaxExpertsPerLane; ++q)
        if (q == (be >> 6)) taken[q] = true;
    }
    if (lane == 0) {
      sel_v[rd] = bv;
      sel_e[rd] = be;
    }
  }
  __syncthreads();
  if (lane < k) {
    const float v0 = sel_v[0];
    float denom = 0.f;
    for (int j = 0; j < k; ++j) denom += expf(sel_v[j] - v0);
    idx[(size_t)t * k + lane] = sel_e[lane];
    w[(size_t)t * k + lane] = expf(sel_v[lane] - v0) / denom;
  }
  if (lane == 0 && margin) margin[t] = (k < E) ? sel_v[k - 1] - sel_v[k] : INFINITY;
}

}  // namespace

int gate_splits(int d) { return (d + kGateKPerBlock - 1) / kGateKPerBlock; }

hipError_t launch_gate(const float *gate_w, const float *x, int N, int d, int E, float *part,
                       hipStream_t st) {
  const int n_et = (E + kTile - 1) / kTile;
  const int blocks = n_et * gate_splits(d);
  hipLaunchKernelGGL(gate_kernel, dim3(blocks), dim3(256), 0, st, gate_w, x, N, d, E, part);
  return hipGetLastError();
}

hipError_t launch_topk(const float *part, int splits, int N, int E, int k, float *logits,
                       int32_t *idx, float *w, float *margin, hipStream_t st) {
  hipLaunchKernelGGL(topk_kernel, dim3(N), dim3(64), 0, st, part, splits, N, E, k, logits,
                     idx, w, margin);
  return hipGetLastError();
}

}  // namespace moe
