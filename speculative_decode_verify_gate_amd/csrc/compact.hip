// compact.hip -- routing-trace compaction for the deduplicating engine.
//
// "Speculative Decoding for Mixture-of-Experts Models: Expert Bytes, Kernel
// Bandwidth and the Best Draft Length", abstract: a deduplicating engine reads
// each selected expert once per pass.  To do so it needs, per distinct
// expert, the list of (token, slot) pairs that chose it.  One workgroup builds
// that record in LDS from the N*k routing entries (N*k <= 512):
//   1. every slot sets its bit in a per-expert 512-bit membership mask
//      (LDS atomic OR: order-independent, so the result is deterministic);
//   2. counts are mask popcounts; one wavefront scans counts and presence
//      flags to get offsets and the ascending unique-expert list;
//   3. a slot's rank inside its expert's list is the popcount of the mask
//      bits below it, so lists come out in (token, slot) order.
#include "kernels.h"

namespace moe {
namespace {

constexpr int kMaskWords = MOE_MAX_SLOTS / 32;  // 16

__global__ __launch_bounds__(512) void compact_kernel(const int32_t *__restrict__ idx,
                                                      int slots, int E,
                                                      int32_t *__restrict__ cmp,
                                                      int32_t *__restrict__ n_unique) {
  __shared__ uint32_t mask[MOE_MAX_EXPERTS][kMaskWords];
  __shared__ int cnt[MOE_MAX_EXPERTS];
  __shared__ int offs[MOE_MAX_EXPERTS + 1];
  __shared__ int upos[MOE_MAX_EXPERTS + 1];
  const int tid = threadIdx.x;
  const int words = (slots + 31) / 32;
  const CompactLayout L{E, slots};

  for (int i = tid; i < E * kMaskWords; i += blockDim.x) (&mask[0][0])[i] = 0u;
  __syncthreads();
  for (int s = tid; s < slots; s += blockDim.x) {
    const int e = idx[s];
    if (e >= 0 && e < E) atomicOr(&mask[e][s >> 5], 1u << (s & 31));
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) {
    int c = 0;
    for (int wd = 0; wd < words; ++wd) c += __popc(mask[e][wd]);
    cnt[e] = c;
  }
  __syncthreads();

  // exclusive scans of counts and of presence flags by the first wavefront;
  // lane l owns experts 4l .. 4l+3 (E <= 256)
  if (tid < 64) {
    int c4[4], p4[4], cs = 0, ps = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid * 4 + q;
      c4[q] = (e < E) ? cnt[e] : 0;
      p4[q] = (c4[q] > 0) ? 1 : 0;
      cs += c4[q];
      ps += p4[q];
    }
    int ci = cs, pi = ps;  // inclusive wave scan of the per-lane sums
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int co = __shfl_up(ci, off, 64);
      const int po = __shfl_up(pi, off, 64);
      if (tid >= off) {
        ci += co;
        pi += po;
      }
    }
    int cex = ci - cs, pex = pi - ps;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid * 4 + q;
      if (e < E) {
        offs[e] = cex;
        upos[e] = pex;
      }
      cex += c4[q];
      pex += p4[q];
    }
    if (tid == 63) {
      offs[E] = ci;
      upos[E] = pi;
    }
  }
  __syncthreads();

  for (int e = tid; e < E; e += blockDim.x) {
    cmp[L.counts() + e] = cnt[e];
    cmp[L.offs() + e] = offs[e];
    if (cnt[e] > 0) cmp[L.uniq() + upos[e]] = e;
    // entries past U mark "no instance": an expert block reads uniq[u] alone
    if (e >= upos[E]) cmp[L.uniq() + e] = -1;
  }
  if (tid == 0) {
    cmp[L.offs() + E] = offs[E];
    cmp[L.u()] = upos[E];
    if (n_unique) *n_unique = upos[E];
  }
  for (int s = tid; s < slots; s += blockDim.x) {
    const int e = idx[s];
    if (e >= 0 && e < E) {
      const int wd = s >> 5;
      int rank = __popc(mask[e][wd] & ((1u << (s & 31)) - 1u));
      for (int q = 0; q < wd; ++q) rank += __popc(mask[e][q]);
      cmp[L.list() + offs[e] + rank] = s;
    }
  }
}

}  // namespace

hipError_t launch_compact(const int32_t *idx, int N, int k, int E, int32_t *cmp,
                          int32_t *n_unique, hipStream_t st) {
  hipLaunchKernelGGL(compact_kernel, dim3(1), dim3(512), 0, st, idx, N * k, E, cmp, n_unique);
  return hipGetLastError();
}

}  // namespace moe
