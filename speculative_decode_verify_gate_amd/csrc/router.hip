// router.hip -- gate logits, top-k and softmax over the k on gfx950.
//
// "Deep Dive into Mixture of Experts: From 1991 to DeepSeek-V3", section 2:
// logits = x @ gate_weights, keep the k largest, weights = softmax of the k
// selected values.  Ties are broken toward the lower expert index.  The
// DeepSeek-style variant of section 5 adds a per-expert bias to the logits
// (after the split partials are summed); selection and softmax then take
// the biased values.
//
// The gate GEMM [N x d] x [d x E] streams the fp32 gate matrix once with
// fp32 MFMA (16 experts x 16 tokens per tile), split over K so that enough
// workgroups stream it; each split yields fp32 partial logits.  Logits are
// the partials summed in split order (deterministic).  Top-k: a wavefront
// per token takes k + 1 rounds of a wavefront-wide argmax in the order
// (value descending, index ascending): round j yields slot j, round k the
// margin.
//
// When all partials of a pass are small (at most 64 KB), one launch does
// everything: the gate workgroups hand their partials over with
// device-coherent stores and the last one to arrive sums them and runs the
// top-k for every token.  Larger gates (e.g. 256 experts x 7168) use a second
// launch for the top-k.
#include <math.h>

#include "coherent.h"
#include "kernels.h"

namespace moe {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGateWaves = 4;
constexpr int kGateKPerWave = kGateKPerBlock / kGateWaves;  // 64 = 4 steps of 16
constexpr int kMaxColTiles = 4;                              // N <= 64
constexpr int kMaxExpertsPerLane = MOE_MAX_EXPERTS / 64;
constexpr int kFusedGateThreads = 512;     // one-launch routing: threads per workgroup
constexpr int kGateScratch = kGateWaves * kMaxColTiles * 64 * 16;  // the waves' partial sums

// Logits sit in LDS at logit_ld(E) per token; the selection reads only
// indices below E.

// Order-preserving 32-bit key of a logit (signed compare: larger value,
// larger key), -0 taken as +0.  kDead, below every key of a value that is
// not a NaN, marks an expert already taken (or past E).
__device__ inline int logit_key(float v) {
  int b = __float_as_int(v);
  if (b == (int)0x80000000) b = 0;
  return b < 0 ? (b ^ 0x7FFFFFFF) : b;
}
__device__ inline float key_logit(int key) { return __int_as_float(key < 0 ? key ^ 0x7FFFFFFF : key); }
constexpr int kDead = (int)0x80000000;

// k from lane i - SHIFT of the same 16-lane row (DPP row_shr), kDead for
// the first SHIFT lanes of a row.
template <int SHIFT>
__device__ inline int row_shr_key(int k) {
  return __builtin_amdgcn_update_dpp(kDead, k, 0x110 + SHIFT, 0xf, 0xf, false);
}

// Largest key over the wavefront, returned to every lane: a max over each
// 16-lane row by shifted DPP moves (lane 16r + 15 ends with its row's max),
// then the four row maxima read out and combined.
__device__ inline int wave_max_key(int k) {
  k = max(k, row_shr_key<1>(k));
  k = max(k, row_shr_key<2>(k));
  k = max(k, row_shr_key<4>(k));
  k = max(k, row_shr_key<8>(k));
  const int r0 = __builtin_amdgcn_readlane(k, 15), r1 = __builtin_amdgcn_readlane(k, 31);
  const int r2 = __builtin_amdgcn_readlane(k, 47), r3 = __builtin_amdgcn_readlane(k, 63);
  return max(max(r0, r1), max(r2, r3));
}

// i from lane i - SHIFT of the same 16-lane row, kNone for the first SHIFT
// lanes of a row; the smallest over the wavefront, returned to every lane.
constexpr int kNone = 0x7FFFFFFF;
template <int SHIFT>
__device__ inline int row_shr_idx(int i) {
  return __builtin_amdgcn_update_dpp(kNone, i, 0x110 + SHIFT, 0xf, 0xf, false);
}
__device__ inline int wave_min_idx(int i) {
  i = min(i, row_shr_idx<1>(i));
  i = min(i, row_shr_idx<2>(i));
  i = min(i, row_shr_idx<4>(i));
  i = min(i, row_shr_idx<8>(i));
  const int r0 = __builtin_amdgcn_readlane(i, 15), r1 = __builtin_amdgcn_readlane(i, 31);
  const int r2 = __builtin_amdgcn_readlane(i, 47), r3 = __builtin_amdgcn_readlane(i, 63);
  return min(min(r0, r1), min(r2, r3));
}

// Top-k selection of n_tok tokens whose logits sit in LDS (L[t][ld], ld =
// logit_ld(E)), by the nth threads of the caller.  A wavefront takes a
// token: lane l holds the keys of experts l, l+64, l+128, l+192, and each
// round takes the largest remaining key over the wavefront and, among the
// remaining experts holding it, the lowest index (a second wavefront
// reduction, a min over the indices that hold it): the next slot in the
// order (logit descending, index ascending).  Rounds 0..k-1 fill the slots, round k
// gives the margin.  TPW tokens per wavefront go through the rounds
// together, so their dependent steps overlap.  sel_v / sel_e: LDS
// [n_tok][MOE_MAX_TOPK + 1].  QM: 64-expert quarters compiled for
// (E <= 64 QM).
template <int QM, int TPW>
__device__ inline void argmax_select(const float *L, int n_tok, const RouteArgs &a, int tid,
                                     int nth, float (*sel_v)[MOE_MAX_TOPK + 1],
                                     int (*sel_e)[MOE_MAX_TOPK + 1]) {
  const int E = a.E;
  const int k = a.k;
  const int ld = logit_ld(E);
  const int lane = tid & 63, wave = tid >> 6, nw = nth >> 6;
  const int rounds = k < E ? k + 1 : k;
  for (int tb = wave; tb < n_tok; tb += nw * TPW) {  // uniform per wavefront
    int key[TPW][QM];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      const int t = tb + tt * nw;
#pragma unroll
      for (int q = 0; q < QM; ++q) {
        const int e = q * 64 + lane;
        key[tt][q] = (t < n_tok && e < E) ? logit_key(L[(size_t)t * ld + e]) : kDead;
      }
    }
    for (int r = 0; r < rounds; ++r) {
      int m[TPW];
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) {
        m[tt] = key[tt][0];
#pragma unroll
        for (int q = 1; q < QM; ++q) m[tt] = max(m[tt], key[tt][q]);
      }
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) m[tt] = wave_max_key(m[tt]);
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) {
        // the lowest expert holding the maximum; when only NaN logits
        // remain (no key equals the maximum), the lowest remaining expert
        int cand = kNone;
#pragma unroll
        for (int q = QM - 1; q >= 0; --q)
          if (key[tt][q] == m[tt] && m[tt] != kDead) cand = q * 64 + lane;
        int e = wave_min_idx(cand);
        if (e == kNone) {
#pragma unroll
          for (int q = QM - 1; q >= 0; --q)
            if (q * 64 + lane < E && key[tt][q] != kDead) cand = q * 64 + lane;
          e = wave_min_idx(cand);
          if (e == kNone) e = -1;
        }
        const int t = tb + tt * nw;
#pragma unroll
        for (int q = 0; q < QM; ++q)
          if (q * 64 + lane == e) key[tt][q] = kDead;
        if (lane == 0 && t < n_tok && e >= 0) {
          sel_e[t][r] = e;
          sel_v[t][r] = key_logit(m[tt]);
        }
      }
    }
  }
}

template <int QM>
__device__ inline void argmax_select_q(const float *L, int n_tok, const RouteArgs &a, int tid,
                                       int nth, float (*sel_v)[MOE_MAX_TOPK + 1],
                                       int (*sel_e)[MOE_MAX_TOPK + 1]) {
  const int per_wave = (n_tok + (nth >> 6) - 1) / (nth >> 6);  // tokens per wavefront
  if (per_wave >= 4)
    argmax_select<QM, 4>(L, n_tok, a, tid, nth, sel_v, sel_e);
  else if (per_wave >= 2)
    argmax_select<QM, 2>(L, n_tok, a, tid, nth, sel_v, sel_e);
  else
    argmax_select<QM, 1>(L, n_tok, a, tid, nth, sel_v, sel_e);
}

// Top-k, softmax over the k, margin and (if asked) the logits of n_tok
// tokens whose logits sit in LDS; t0 is the global index of token 0.
__device__ inline void select_topk(const float *L, int n_tok, int t0, const RouteArgs &a,
                                   int tid, int nth, float (*sel_v)[MOE_MAX_TOPK + 1],
                                   int (*sel_e)[MOE_MAX_TOPK + 1]) {
  const int E = a.E, k = a.k;
  if (a.logits) {
    const int ld = logit_ld(E);
    for (int i = tid; i < n_tok * E; i += nth) {
      const int t = i / E;
      a.logits[(size_t)t0 * E + i] = L[(size_t)t * ld + (i - t * E)];
    }
  }
  if (E <= 64)
    argmax_select_q<1>(L, n_tok, a, tid, nth, sel_v, sel_e);
  else if (E <= 128)
    argmax_select_q<2>(L, n_tok, a, tid, nth, sel_v, sel_e);
  else
    argmax_select_q<4>(L, n_tok, a, tid, nth, sel_v, sel_e);
  __syncthreads();
  for (int p = tid; p < n_tok * k; p += nth) {
    const int t = p / k;
    const int j = p - t * k;
    const float v0 = sel_v[t][0];
    float denom = 0.f;
    for (int i = 0; i < k; ++i) denom += expf(sel_v[t][i] - v0);
    a.idx[(size_t)(t0 + t) * k + j] = sel_e[t][j];
    a.w[(size_t)(t0 + t) * k + j] = expf(sel_v[t][j] - v0) / denom;
    if (j == 0 && a.margin)
      a.margin[t0 + t] = (k < E) ? sel_v[t][k - 1] - sel_v[t][k] : INFINITY;
  }
  __syncthreads();
}

// Partial logits of one 16-expert tile over one K split,
// part[split][t][e] = sum over the split's K range of x[t][i] * gate_w[e][i];
// with FUSED, the last workgroup of the layer also finishes its routing.
// A stack of L layers (the same tokens through every layer's gate) runs as
// L consecutive ranges of workgroups, each with its own gate, bias,
// partials, arrival counter and outputs.
template <bool FUSED>
__global__ __launch_bounds__(FUSED ? kFusedGateThreads : 256) void gate_kernel(RouteArgs a) {
  const int N = a.N, d = a.d, E = a.E;
  const int n_et = (E + kTile - 1) / kTile;
  // layers of a stack are consecutive ranges of n_et * splits workgroups
  const int per_layer = n_et * a.splits;
  const int layer = blockIdx.x / per_layer;
  const int bid = blockIdx.x - layer * per_layer;
  const int et = bid % n_et;
  const int split = bid / n_et;
  const float *gate_w = a.gate_w + (size_t)layer * E * d;
  float *part = a.part + (size_t)layer * a.splits * N * E;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;  // A row (expert) / B column (token) of this lane
  const int g = lane >> 4;  // K group of this lane
  const int n_ct = (N + kTile - 1) / kTile;

  const int k_begin = split * kGateKPerBlock + wave * kGateKPerWave;
  const int expert = et * kTile + r;
  const bool mma_wave = wave < kGateWaves;

  f32x4 acc[kMaxColTiles];
#pragma unroll
  for (int ct = 0; ct < kMaxColTiles; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Each step covers 16 K elements: lane group g holds elements 4g..4g+3 of
  // the step, and fp32 MFMA number v consumes element v of every group.
#pragma unroll
  for (int s = 0; s < kGateKPerWave / 16; ++s) {
    const int k0 = k_begin + s * 16;
    if (!mma_wave || k0 >= d) break;
    f32x4 av = f32x4{0.f, 0.f, 0.f, 0.f};
    if (expert < E) av = *(const f32x4 *)(gate_w + (size_t)expert * d + k0 + 4 * g);
#pragma unroll
    for (int ct = 0; ct < kMaxColTiles; ++ct) {
      if (ct < n_ct) {
        const int tok = ct * kTile + r;
        f32x4 b = f32x4{0.f, 0.f, 0.f, 0.f};
        if (tok < N) b = *(const f32x4 *)(a.x + (size_t)tok * d + k0 + 4 * g);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.x, b.x, acc[ct], 0, 0, 0);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.y, b.y, acc[ct], 0, 0, 0);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.z, b.z, acc[ct], 0, 0, 0);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.w, b.w, acc[ct], 0, 0, 0);
      }
    }
  }

  // Sum the four waves' partials in wave order.
  __shared__ __align__(16) unsigned char scratch[kGateScratch];
  f32x4 (*red)[kMaxColTiles][64] = (f32x4 (*)[kMaxColTiles][64])scratch;
  if (mma_wave) {
#pragma unroll
    for (int ct = 0; ct < kMaxColTiles; ++ct)
      if (ct < n_ct) red[wave][ct][lane] = acc[ct];
  }
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
        if (e < E) {
          if (FUSED)
            store_coherent(dst + e, s[v]);
          else
            dst[e] = s[v];
        }
      }
    }
  }
  if (!FUSED) return;

  // ---- the last workgroup to finish sums the partials and routes
  __shared__ int s_last;
  wait_stores();
  __syncthreads();
  if (tid == 0) {
    // arrivals counted in the caller's workspace (zero before first use);
    // the last workgroup puts it back to zero for the next call
    s_last = atomicAdd(a.done + layer, 1u) == (unsigned)per_layer - 1;
    if (s_last) atomicExch(a.done + layer, 0u);
  }
  __syncthreads();
  if (!s_last) return;
  extern __shared__ __align__(16) float Ls[];  // [N][logit_ld(E)] logits
  const int splits = a.splits;
  const int NE = N * E;
  const int ld = logit_ld(E);
  const int nth = blockDim.x;
  for (int i = tid; i < N * (ld - E); i += nth) {
    const int t = i / (ld - E);
    Ls[t * ld + E + (i - t * (ld - E))] = -INFINITY;
  }
  for (int i0 = 0; i0 < NE; i0 += 4 * nth) {
    // the loads of 4 logits x 8 splits are issued before any is summed
    for (int sp0 = 0; sp0 < splits; sp0 += 8) {
      float pv[4][8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = min(i0 + q * nth + tid, NE - 1);
#pragma unroll
        for (int u = 0; u < 8; ++u)
          pv[q][u] = load_coherent(part + (size_t)min(sp0 + u, splits - 1) * NE + i);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = i0 + q * nth + tid;
        if (i < NE) {
          const int t = i / E;
          const int e = i - t * E;
          float acc_l = (sp0 == 0) ? 0.f : Ls[t * ld + e];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (sp0 + u < splits) acc_l += pv[q][u];
          if (sp0 + 8 >= splits && a.bias) acc_l += a.bias[(size_t)layer * E + e];
          Ls[t * ld + e] = acc_l;
        }
      }
    }
  }
  __syncthreads();
  __shared__ float sel_v[MOE_MAX_TOKENS][MOE_MAX_TOPK + 1];
  __shared__ int sel_e[MOE_MAX_TOKENS][MOE_MAX_TOPK + 1];
  select_topk(Ls, N, layer * N, a, tid, nth, sel_v, sel_e);
}

// Unfused top-k, one workgroup per token.  Wave w sums the partials of
// splits w, w+4, w+8, ... (all loads of a lane issued together: one memory
// round trip for up to 32 splits); the four wave sums are added in wave
// order, then every thread ranks at most one expert.
__global__ __launch_bounds__(256) void topk_kernel(RouteArgs a) {
  constexpr int kBatch = 8;  // splits per wave and batch
  const int t = blockIdx.x;
  const int layer = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int N = a.N, E = a.E, splits = a.splits;
  const int ld = logit_ld(E);
  __shared__ __align__(16) float Ls[MOE_MAX_EXPERTS];
  __shared__ float ws_sum[kGateWaves][MOE_MAX_EXPERTS];
  __shared__ float sel_v[1][MOE_MAX_TOPK + 1];
  __shared__ int sel_e[1][MOE_MAX_TOPK + 1];
  const int n_q = (E + 63) / 64;
  float v[kMaxExpertsPerLane];
#pragma unroll
  for (int q = 0; q < kMaxExpertsPerLane; ++q) v[q] = 0.f;
  for (int sp0 = wave; sp0 < splits; sp0 += kGateWaves * kBatch) {
    float pv[kMaxExpertsPerLane][kBatch];
#pragma unroll
    for (int q = 0; q < kMaxExpertsPerLane; ++q) {
      if (q < n_q) {
        const int e = min(q * 64 + lane, E - 1);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int sp = min(sp0 + u * kGateWaves, splits - 1);
          pv[q][u] = a.part[(((size_t)layer * splits + sp) * N + t) * E + e];
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kMaxExpertsPerLane; ++q)
      if (q < n_q) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
          if (sp0 + u * kGateWaves < splits) v[q] += pv[q][u];
      }
  }
#pragma unroll
  for (int q = 0; q < kMaxExpertsPerLane; ++q) {
    const int e = q * 64 + lane;
    if (e < E) ws_sum[wave][e] = v[q];
  }
  __syncthreads();
  if (tid < ld) {
    float l = -INFINITY;
    if (tid < E) {
      l = ws_sum[0][tid];
#pragma unroll
      for (int w = 1; w < kGateWaves; ++w) l += ws_sum[w][tid];
      if (a.bias) l += a.bias[(size_t)layer * E + tid];
    }
    Ls[tid] = l;
  }
  __syncthreads();
  select_topk(Ls, 1, layer * N + t, a, tid, blockDim.x, sel_v, sel_e);
}

}  // namespace

hipError_t launch_gate(const RouteArgs &a, hipStream_t st) {
  const int n_et = (a.E + kTile - 1) / kTile;
  const int blocks = n_et * a.splits * a.L;
  if (route_fused(a.N, a.d, a.E)) {
    const size_t lds = (size_t)a.N * logit_ld(a.E) * sizeof(float);
    hipLaunchKernelGGL(gate_kernel<true>, dim3(blocks), dim3(kFusedGateThreads), lds, st, a);
  } else {
    hipLaunchKernelGGL(gate_kernel<false>, dim3(blocks), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const RouteArgs &a, hipStream_t st) {
  hipLaunchKernelGGL(topk_kernel, dim3(a.N, a.L), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
