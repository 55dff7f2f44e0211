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
// the partials summed in split order (deterministic).  Top-k: every
// (token, expert) pair finds its rank under (value desc, index asc) by
// counting, in LDS, the experts ahead of it; ranks below k are the slots.
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
constexpr int kFusedGateThreads = 256;     // one-launch routing: threads per workgroup
// gate workgroup LDS shared by the wave sums and the routing's partial ranks
constexpr int kGateScratch =
    (kGateWaves * kMaxColTiles * 64 * 16 > (kFusedGateThreads / 64) * MOE_MAX_EXPERTS * 4)
        ? kGateWaves * kMaxColTiles * 64 * 16
        : (kFusedGateThreads / 64) * MOE_MAX_EXPERTS * 4;

// Logits sit in LDS at logit_ld(E) per token.  The padding holds -inf at
// indices >= E, which never ranks ahead of a real expert: it is not greater
// than any logit, and on equality with a -inf logit the lower (real) index
// wins.

// Order key of expert e with logit v: order-preserving bits of v (with -0
// taken as +0) above the complemented index, so keys compare like (logit
// descending, index ascending) -- a strict total order in which a token's
// rank of e is the number of its keys greater than e's.  Padding entries
// (e >= E) get key 0, below every real key.
__device__ inline uint64_t order_key(float v, int e) {
  uint32_t b = __float_as_uint(v);
  if ((b << 1) == 0u) b = 0u;                       // -0 and +0 compare equal
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)b << 32) | (uint32_t)~e;
}

// Top-k + softmax of n_tok tokens whose logits sit in LDS (L[t][ld], ld =
// logit_ld(E)), by the nth threads of the caller.  Lane l of a wavefront
// owns experts l, l+64, l+128, l+192 of a token; every key of the token is
// broadcast from its owner lane (readlane, no memory round trip) and
// compared with the lane's own keys, counting those ahead.  With fewer
// tokens than wavefronts, each token's keys are split over several
// wavefronts and the partial counts added in LDS; with more, a wavefront
// takes TPW tokens at once so their compare chains overlap.  Ranks 0..k-1
// are the selection in slot order; rank k gives the margin.  sel_v / sel_e:
// LDS [n_tok][MOE_MAX_TOPK + 1].  t0 is the global index of token 0.
// QM: 64-expert quarters compiled for (E <= 64 QM).
template <int QM, int TPW>
__device__ inline void rank_and_select(const float *L, int n_tok, int t0, const RouteArgs &a,
                                       int tid, int nth, float (*sel_v)[MOE_MAX_TOPK + 1],
                                       int (*sel_e)[MOE_MAX_TOPK + 1],
                                       int (*part_rank)[MOE_MAX_EXPERTS]) {
  const int E = a.E;
  const int k = a.k;
  const int ld = logit_ld(E);
  const int lane = tid & 63, wave = tid >> 6, nw = nth >> 6;
  const int nq = (E + 63) >> 6;
  const int wpt = n_tok >= nw ? 1 : nw / n_tok;  // wavefronts per token
  const int slice = wave % wpt;                  // this wavefront's share of the keys
  const int tstride = nw / wpt;                  // tokens started per round
  const int jn = (E + wpt - 1) / wpt;
  const int j0 = slice * jn, j1 = min(E, j0 + jn);
  // Split mode (wpt > 1) makes one round, in which a wavefront whose token
  // index is past n_tok only takes part in the barrier.
  for (int tb = wave / wpt; wpt > 1 || tb < n_tok; tb += tstride * TPW) {
    float v[TPW][QM];
    uint64_t key[TPW][QM];
    int rank[TPW][QM];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      const int t = tb + tt * tstride;
#pragma unroll
      for (int q = 0; q < QM; ++q) {
        const int e = q * 64 + lane;
        const bool ok = t < n_tok && q < nq && e < E;
        v[tt][q] = ok ? L[(size_t)t * ld + e] : -INFINITY;
        key[tt][q] = ok ? order_key(v[tt][q], e) : 0ull;
        rank[tt][q] = 0;
      }
    }
#pragma unroll
    for (int qq = 0; qq < QM; ++qq) {
      const int ja = max(j0 - qq * 64, 0), jb = min(j1 - qq * 64, 64);
      if (qq >= nq || ja >= jb) continue;  // uniform
      uint32_t hi[TPW], lo[TPW];
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) {
        hi[tt] = (uint32_t)(key[tt][qq] >> 32);
        lo[tt] = (uint32_t)key[tt][qq];
      }
      for (int j = ja; j < jb; ++j) {
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
          const uint64_t kj = ((uint64_t)__builtin_amdgcn_readlane(hi[tt], j) << 32) |
                              (uint32_t)__builtin_amdgcn_readlane(lo[tt], j);
#pragma unroll
          for (int q = 0; q < QM; ++q) rank[tt][q] += kj > key[tt][q] ? 1 : 0;
        }
      }
    }
    if (wpt > 1) {
      // one token per wavefront group: add the groups' slices
#pragma unroll
      for (int q = 0; q < QM; ++q) part_rank[wave][q * 64 + lane] = rank[0][q];
      __syncthreads();
      if (slice == 0 && tb < n_tok) {
#pragma unroll
        for (int q = 0; q < QM; ++q) {
          rank[0][q] = 0;
          for (int w = 0; w < wpt; ++w) rank[0][q] += part_rank[wave + w][q * 64 + lane];
        }
      }
    }
    if (slice == 0) {
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) {
        const int t = tb + tt * tstride;
#pragma unroll
        for (int q = 0; q < QM; ++q) {
          const int e = q * 64 + lane;
          if (t < n_tok && q < nq && e < E) {
            if (rank[tt][q] <= k) {
              sel_v[t][rank[tt][q]] = v[tt][q];
              sel_e[t][rank[tt][q]] = e;
            }
            if (a.logits) a.logits[(size_t)(t0 + t) * E + e] = v[tt][q];
          }
        }
      }
    }
    if (wpt > 1) break;
  }
}

template <int QM>
__device__ inline void rank_and_select_q(const float *L, int n_tok, int t0, const RouteArgs &a,
                                         int tid, int nth, float (*sel_v)[MOE_MAX_TOPK + 1],
                                         int (*sel_e)[MOE_MAX_TOPK + 1],
                                         int (*part_rank)[MOE_MAX_EXPERTS]) {
  const int per_wave = (n_tok + (nth >> 6) - 1) / (nth >> 6);  // tokens per wavefront
  if (per_wave >= 4)
    rank_and_select<QM, 4>(L, n_tok, t0, a, tid, nth, sel_v, sel_e, part_rank);
  else if (per_wave >= 2)
    rank_and_select<QM, 2>(L, n_tok, t0, a, tid, nth, sel_v, sel_e, part_rank);
  else
    rank_and_select<QM, 1>(L, n_tok, t0, a, tid, nth, sel_v, sel_e, part_rank);
}

// part_rank: LDS [nth / 64][MOE_MAX_EXPERTS] ints, free during the call.
__device__ inline void select_topk(const float *L, int n_tok, int t0, const RouteArgs &a,
                                   int tid, int nth, float (*sel_v)[MOE_MAX_TOPK + 1],
                                   int (*sel_e)[MOE_MAX_TOPK + 1],
                                   int (*part_rank)[MOE_MAX_EXPERTS]) {
  const int E = a.E, k = a.k;
  if (E <= 64)
    rank_and_select_q<1>(L, n_tok, t0, a, tid, nth, sel_v, sel_e, part_rank);
  else if (E <= 128)
    rank_and_select_q<2>(L, n_tok, t0, a, tid, nth, sel_v, sel_e, part_rank);
  else
    rank_and_select_q<4>(L, n_tok, t0, a, tid, nth, sel_v, sel_e, part_rank);
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

  // Sum the four waves' partials in wave order.  The buffer is reused for
  // the partial ranks of the routing.
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
  select_topk(Ls, N, layer * N, a, tid, nth, sel_v, sel_e, (int (*)[MOE_MAX_EXPERTS])scratch);
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
  __shared__ int part_rank[kGateWaves][MOE_MAX_EXPERTS];
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
  select_topk(Ls, 1, layer * N + t, a, tid, blockDim.x, sel_v, sel_e, part_rank);
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
