// verify.hip -- one speculative-decoding verification round per sequence on
// gfx950: accept/reject of the drafted tokens against the verifier's
// distributions, then the verifier's correction or bonus token.
//
// "Building a Terminal Based LLM Inference Internals Explorer - Part 3:
// Speculative Decoding", sections "The Accept/Reject Mechanism", "A Worked
// Example" and "Sampling vs Greedy":
//   sampling: draft token i is kept when u_i < min(1, p_i(x_i) / q_i(x_i))
//             (and q_i(x_i) > 0); at the first rejection the round ends with a
//             draw from max(0, p_i - q_i) normalised; if every draft token is
//             kept, a bonus token is drawn from p at position gamma;
//   greedy:   a draft token is kept when it is the verifier's argmax; the
//             round ends with the verifier's argmax at the first mismatch,
//             or at the bonus position.
// The random numbers are inputs.  Every decision is exact: u q(x) < p(x) in
// fp64 (products of two fp32 values are exact there), and the draw is an
// inverse CDF over integer weights floor(w * 2^40) with target
// floor(W r / 2^32), so sums do not depend on their order.
//
// Layout of the work: a workgroup takes a 2048-entry chunk of the vocabulary
// of one sequence, each thread 8 consecutive entries (two 16-byte loads
// where the rows allow).  Sampling: each
// workgroup finds the first rejection itself (2 gamma scalar loads) and
// writes the integer weight sum of its chunk of the row to draw from.
// Greedy: a workgroup per (position, chunk) writes the chunk's argmax as one
// 64-bit key (value bits above the complemented index, so the largest key is
// the largest value at the lowest index).  The last workgroup of a sequence
// to finish (arrival counter in the workspace) finishes the round: the
// argmax decisions (all keys loaded at once, LDS 64-bit max per position),
// or the chunk holding the draw target and, inside it, the entry, by
// block-wide integer prefix sums.
#include <stdint.h>

#include <atomic>
#include <chrono>
#include <random>

#include "coherent.h"
#include "kernels.h"
#include "verify.h"

namespace moe {
namespace {

constexpr int kVThreads = 256;
constexpr int kVPer = 8;                       // entries per thread per row
constexpr int kVChunk = kVThreads * kVPer;     // 2048
constexpr double kQuant = 1099511627776.0;     // 2^40
constexpr int kUnitsGreedy = 4;                // units per workgroup, at most
constexpr int kUnitsSampling = 4;
constexpr int kWavesV = kVThreads / 64;

__device__ inline uint64_t quantize(float w) {
  return w > 0.f ? (uint64_t)((double)w * kQuant) : 0ull;
}

// Key of value v at index j: larger value first, then lower index.  -0 and
// +0 are equal values, so they get one key and the lower index wins.
__device__ inline uint64_t argmax_key(float v, int j) {
  uint32_t b = __float_as_uint(v);
  if ((b << 1) == 0u) b = 0u;                       // -0 as +0
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);  // order-preserving
  return ((uint64_t)b << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
}
__device__ inline int key_index(uint64_t k) { return (int)(0xFFFFFFFFu - (uint32_t)k); }

__device__ inline uint64_t shfl_xor64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
  const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}
__device__ inline uint64_t shfl_up64(uint64_t v, int d) {
  const uint32_t lo = __shfl_up((uint32_t)v, d, 64);
  const uint32_t hi = __shfl_up((uint32_t)(v >> 32), d, 64);
  return ((uint64_t)hi << 32) | lo;
}

// Block-wide sum / max of one uint64 per thread (all threads get it).
template <bool MAX>
__device__ inline uint64_t block_reduce(uint64_t v, uint64_t *scratch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint64_t o = shfl_xor64(v, m);
    v = MAX ? (o > v ? o : v) : v + o;
  }
  __syncthreads();
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  uint64_t r = scratch[0];
  for (int w = 1; w < kVThreads / 64; ++w) r = MAX ? (scratch[w] > r ? scratch[w] : r) : r + scratch[w];
  return r;
}

// Inclusive block-wide prefix sum of one uint64 per thread (in thread
// order); *total receives the block sum.
__device__ inline uint64_t block_scan(uint64_t v, uint64_t *scratch, uint64_t *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint64_t o = shfl_up64(v, d);
    if (lane >= d) v += o;
  }
  __syncthreads();
  if (lane == 63) scratch[wave] = v;
  __syncthreads();
  uint64_t before = 0, all = 0;
  for (int w = 0; w < kVThreads / 64; ++w) {
    if (w < wave) before += scratch[w];
    all += scratch[w];
  }
  *total = all;
  return v + before;
}

// NU block-wide sums / maxima at once, one barrier: thread u < NU gets
// result u (others get 0).
template <bool MAX, int NU>
__device__ inline uint64_t block_reduce_many(const uint64_t (&v)[NU], uint64_t (*scratch)[kWavesV]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    uint64_t x = v[u];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const uint64_t o = shfl_xor64(x, m);
      x = MAX ? (o > x ? o : x) : x + o;
    }
    if (lane == 0) scratch[u][wave] = x;
  }
  __syncthreads();
  uint64_t r = 0;
  if ((int)threadIdx.x < NU) {
    r = scratch[threadIdx.x][0];
    for (int w = 1; w < kWavesV; ++w) {
      const uint64_t y = scratch[threadIdx.x][w];
      r = MAX ? (y > r ? y : r) : r + y;
    }
  }
  return r;
}

struct VerifyArgs {
  int n_seq, gamma, V, mode, chunks;
  int upb;         // units (chunk, or position x chunk) per workgroup
  const float *p, *q, *u;
  const int32_t *x;
  const uint32_t *r;
  int32_t *n_acc, *out;
  unsigned *done;  // [n_seq] arrival counters: zero on entry and exit
  uint64_t *part;  // [n_seq][gamma + 1][chunks] (sampling: [n_seq][chunks])
};

// First rejected draft position of sequence s in sampling mode (gamma if
// none); every thread gets it.
__device__ inline int first_rejection(const VerifyArgs &a, int s, int *sh) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    bool reject = false;
    if (tid < a.gamma) {
      const int i = tid;
      const int x = a.x[s * a.gamma + i];
      reject = true;  // a token outside the vocabulary is rejected unread
      if (x >= 0 && x < a.V) {
        const size_t row = ((size_t)s * (a.gamma + 1) + i) * a.V;
        const size_t qrow = ((size_t)s * a.gamma + i) * a.V;
        const double pv = a.p[row + x], qv = a.q[qrow + x];
        const double u = a.u[s * a.gamma + i];
        reject = !(qv > 0.0 && u * qv < pv);
      }
    }
    const uint64_t m = __ballot(reject);
    if (tid == 0) *sh = m ? __ffsll((unsigned long long)m) - 1 : a.gamma;
  }
  __syncthreads();
  return *sh;
}

// Weight of vocabulary entry j of the row the sampling draw uses: the
// residual at a rejection, the bonus distribution otherwise, or (fallback,
// residual quantized to zero) the verifier distribution itself.
__device__ inline uint64_t draw_weight(const VerifyArgs &a, int s, int istar, bool fallback,
                                       int j) {
  const float pv = a.p[((size_t)s * (a.gamma + 1) + istar) * a.V + j];
  if (istar == a.gamma || fallback) return quantize(pv);
  const float qv = a.q[((size_t)s * a.gamma + istar) * a.V + j];
  const float d = pv - qv;
  return quantize(d > 0.f ? d : 0.f);
}

// Entries j0 .. j0+kVPer-1 of a row, 0 past V: two 16-byte loads when vec
// (V a multiple of 4 and 16-byte aligned rows, so a group of 4 is all in
// or all out of the row), else one by one.
__device__ inline void load_run(const float *row, int V, int j0, bool vec, float (&v)[kVPer]) {
  static_assert(kVPer == 8, "two groups of four");
  if (vec) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int j = j0 + 4 * h;
      const float4 t = j < V ? *(const float4 *)(row + j) : make_float4(0.f, 0.f, 0.f, 0.f);
      v[4 * h] = t.x;
      v[4 * h + 1] = t.y;
      v[4 * h + 2] = t.z;
      v[4 * h + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < kVPer; ++e) v[e] = j0 + e < V ? row[j0 + e] : 0.f;
  }
}

__global__ __launch_bounds__(kVThreads) void verify_kernel(VerifyArgs a) {
  const int s = blockIdx.y, tid = threadIdx.x;
  const int G = a.gamma;
  const bool sampling = a.mode == MOE_VERIFY_SAMPLING;
  // a workgroup takes upb consecutive units: chunks (sampling) or
  // (position, chunk) pairs in position-major order (greedy)
  const int units = sampling ? a.chunks : a.chunks * (G + 1);
  const int u0 = blockIdx.x * a.upb;
  const unsigned arrivals = gridDim.x;
  __shared__ uint64_t scratch[kWavesV];
  __shared__ uint64_t many[kUnitsGreedy > kUnitsSampling ? kUnitsGreedy : kUnitsSampling][kWavesV];
  __shared__ int sh_i;
  __shared__ int sh_last;
  __shared__ int xs[MOE_MAX_DRAFT + 1];  // this sequence's draft tokens
  // loaded now, used only by the workgroup that finishes the round
  if (tid < G) xs[tid] = a.x[s * G + tid];
  const uint64_t rr = sampling ? (uint64_t)a.r[s] : 0ull;
  int istar = G;
  // rows start at multiples of V entries: 16-byte aligned when V is a
  // multiple of 4 and the arrays are
  const bool vec = (a.V & 3) == 0 && (((uintptr_t)a.p | (uintptr_t)a.q) & 15) == 0;

  // ---- this workgroup's partial results (all loads issued before any use)
  if (sampling) {
    istar = first_rejection(a, s, &sh_i);
    const float *prow = a.p + ((size_t)s * (G + 1) + istar) * a.V;
    const float *qrow = istar < G ? a.q + ((size_t)s * G + istar) * a.V : prow;
    float pv[kUnitsSampling][kVPer], qv[kUnitsSampling][kVPer];
#pragma unroll
    for (int uu = 0; uu < kUnitsSampling; ++uu) {
      const int unit = u0 + uu;
      // past the workgroup's units: an index past the row, so zeros
      const int j0 = uu < a.upb && unit < units ? unit * kVChunk + tid * kVPer : a.V;
      load_run(prow, a.V, j0, vec, pv[uu]);
      load_run(qrow, a.V, istar < G ? j0 : a.V, vec, qv[uu]);
    }
    uint64_t sum[kUnitsSampling];
#pragma unroll
    for (int uu = 0; uu < kUnitsSampling; ++uu) {
      sum[uu] = 0;
#pragma unroll
      for (int k = 0; k < kVPer; ++k) {
        const float d = istar < G ? pv[uu][k] - qv[uu][k] : pv[uu][k];  // residual / bonus
        sum[uu] += quantize(d > 0.f ? d : 0.f);
      }
    }
    const uint64_t r = block_reduce_many<false, kUnitsSampling>(sum, many);
    if (tid < a.upb && u0 + tid < units) store_coherent64(a.part + (size_t)s * a.chunks + u0 + tid, r);
  } else {
    float pv[kUnitsGreedy][kVPer];
#pragma unroll
    for (int uu = 0; uu < kUnitsGreedy; ++uu) {
      const int unit = u0 + uu;
      const bool live = uu < a.upb && unit < units;
      const int row_i = live ? unit / a.chunks : 0, c = live ? unit - row_i * a.chunks : 0;
      const float *row = a.p + ((size_t)s * (G + 1) + row_i) * a.V;
      load_run(row, a.V, live ? c * kVChunk + tid * kVPer : a.V, vec, pv[uu]);
    }
    uint64_t best[kUnitsGreedy];
#pragma unroll
    for (int uu = 0; uu < kUnitsGreedy; ++uu) {
      const int unit = u0 + uu;
      const int c = unit % a.chunks;
      best[uu] = 0;
#pragma unroll
      for (int k = 0; k < kVPer; ++k) {
        const int j = c * kVChunk + tid * kVPer + k;
        const bool ok = uu < a.upb && unit < units && j < a.V;
        const uint64_t key = ok ? argmax_key(pv[uu][k], j) : 0ull;
        best[uu] = key > best[uu] ? key : best[uu];
      }
    }
    const uint64_t r = block_reduce_many<true, kUnitsGreedy>(best, many);
    if (tid < a.upb && u0 + tid < units) store_coherent64(a.part + (size_t)s * units + u0 + tid, r);
  }

  // ---- the last workgroup of the sequence finishes the round
  wait_stores();
  __syncthreads();
  if (tid == 0) {
    sh_last = atomicAdd(a.done + s, 1u) == arrivals - 1;
    if (sh_last) atomicExch(a.done + s, 0u);
  }
  __syncthreads();
  if (!sh_last) return;

  int32_t *out = a.out + (size_t)s * (G + 1);
  if (!sampling) {
    // all (position, chunk) keys at once: one LDS max per position
    __shared__ unsigned long long best[MOE_MAX_DRAFT + 1];
    __shared__ int sh_n;
    for (int i = tid; i <= G; i += kVThreads) best[i] = 0ull;
    __syncthreads();
    for (int f = tid; f < units; f += kVThreads) {
      const uint64_t k = load_coherent64(a.part + (size_t)s * units + f);
      atomicMax(&best[f / a.chunks], (unsigned long long)k);
    }
    __syncthreads();
    // kept drafts: the leading positions whose argmax is the draft token
    if (tid < 64) {
      const bool miss = tid < G && key_index(best[tid]) != xs[tid];
      const uint64_t m = __ballot(miss);
      if (tid == 0) sh_n = m ? __ffsll((unsigned long long)m) - 1 : G;
    }
    __syncthreads();
    const int n = sh_n;
    for (int i = tid; i <= G; i += kVThreads)
      out[i] = i < n ? xs[i] : (i == n ? key_index(best[n]) : -1);
    if (tid == 0) a.n_acc[s] = n;
    return;
  }

  // total weight: the chunk sums (or, if the residual vanished, the
  // verifier's own row, summed here by this workgroup alone)
  // Each thread keeps its first chunk sum for the scan below, which then
  // needs no second round trip when the row has at most kVThreads chunks.
  uint64_t W = 0, cs_first = 0;
  for (int cc = tid; cc < a.chunks; cc += kVThreads) {
    const uint64_t v = load_coherent64(a.part + (size_t)s * a.chunks + cc);
    if (cc == tid) cs_first = v;
    W += v;
  }
  W = block_reduce<false>(W, scratch);
  const bool fallback = W == 0 && istar < G;
  if (fallback) {
    W = 0;
    for (int j = tid; j < a.V; j += kVThreads) W += draw_weight(a, s, istar, true, j);
    W = block_reduce<false>(W, scratch);
  }
  const uint64_t hi = __umul64hi(W, rr), lo = W * rr;
  const uint64_t target = (hi << 32) | (lo >> 32);  // floor(W r / 2^32) < W

  // the chunk holding the target: block-wide prefix sums of the chunk sums,
  // kVThreads chunks at a time
  __shared__ int sh_chunk;
  __shared__ uint64_t sh_before;
  if (tid == 0) sh_chunk = -1;
  uint64_t run = 0;
  for (int c0 = 0; c0 < a.chunks; c0 += kVThreads) {
    const int cc = c0 + tid;
    uint64_t cs = 0;
    if (cc < a.chunks) {
      if (!fallback) {
        cs = c0 == 0 ? cs_first : load_coherent64(a.part + (size_t)s * a.chunks + cc);
      } else {
        for (int k = 0; k < kVChunk; ++k) {
          const int j = cc * kVChunk + k;
          if (j < a.V) cs += draw_weight(a, s, istar, true, j);
        }
      }
    }
    uint64_t total;
    const uint64_t incl = block_scan(cs, scratch, &total);
    if (cs > 0 && run + incl > target && run + incl - cs <= target) {
      sh_chunk = cc;
      sh_before = run + incl - cs;
    }
    __syncthreads();
    if (sh_chunk >= 0) break;
    run += total;
  }
  // inside that chunk (no chunk when every weight is zero: the draw has no
  // token, -1): each thread's kVPer consecutive weights, one block-wide
  // prefix sum of their sums in thread (= index) order, then the thread
  // whose run holds the target walks its entries in order
  __shared__ int sh_pick;
  if (tid == 0) sh_pick = -1;
  __syncthreads();
  if (sh_chunk >= 0) {
    const int j0 = sh_chunk * kVChunk + tid * kVPer;
    uint64_t w[kVPer], sum = 0;
#pragma unroll
    for (int k = 0; k < kVPer; ++k) {
      const int j = j0 + k;
      w[k] = j < a.V ? draw_weight(a, s, istar, fallback, j) : 0ull;
      sum += w[k];
    }
    uint64_t total;
    const uint64_t incl = block_scan(sum, scratch, &total);
    uint64_t at = sh_before + incl - sum;  // weight of the chunk's entries before this thread's
    if (sum > 0 && at <= target && at + sum > target) {
      // the first entry whose inclusive prefix passes the target
      for (int k = 0; k < kVPer; ++k) {
        if (at + w[k] > target) {
          sh_pick = j0 + k;
          break;
        }
        at += w[k];
      }
    }
  }
  __syncthreads();
  for (int i = tid; i <= G; i += kVThreads)
    out[i] = i < istar ? xs[i] : (i == istar ? sh_pick : -1);
  if (tid == 0) a.n_acc[s] = istar;
}

// ---- the distributions from the logits (the verify phase of the same page:
// softmax(logits / temperature), then top-p filtering, the same settings for
// the verifier and the draft).
//   top-p: the tokens kept are the shortest run in the order (probability
//   descending, index ascending) whose probability reaches top_p, the token
//   that reaches it included.  The decision uses integer masses
//   floor(P * 2^52) against ceil(top_p * W), W their total, so it is exact
//   and independent of summation order: a radix select over the
//   probability bits (non-negative floats order like their bits, and P <= 1
//   leaves bits 31-30 zero) finds the probability K of the last kept token;
//   of the tokens tied at K (all of equal mass) the first ones in index
//   order are kept, i.e. those up to an index cut.  The kept tokens are
//   renormalised by their mass.
// Work split: a row is cut into kFChunk-entry chunks, one workgroup each,
// so a few rows still fill the chip, each thread holding four 16-byte
// groups of consecutive entries.  The phases of a row:
//   stat:   chunk max m_c and sum of exp(z - m_c), z = logit / T;
//   prob:   the row's max and sum (a fixed-order reduction of the chunks'
//           pairs, so every workgroup of the row gets the same bits) and
//           P = exp(z - M) / S.  Without top-p P is the output.  With it,
//           the chunk's mass histogram of bits 29-22 is added into the
//           row's (64-bit integer atomics: the sum does not depend on their
//           order), and the bin where the mass counted from the top reaches
//           ceil(top_p W) is selected;
//   gather: the chunk's entries in the selected bin (candidates) appended
//           to the row's candidate list; the last kept token is found among
//           them: for a short list by ranking every candidate in the order
//           and a running sum of the masses in that order, else by K (bits
//           21-11, then 10-0), the number of ties at K to keep and, when
//           only some are kept, the index cut (bits 23-12, then 11-0 of the
//           tied indices, by counts);
//   write:  the kept entries renormalised, the rest zeroed.
// Two schedules run these phases with the same arithmetic, so they give the
// same bits:
//   one launch (rows <= kFusedRows, chunks <= kFusedChunks, and a grid the
//     chip holds at once, with one chunk per workgroup or else two): each
//     workgroup keeps its chunks from the logits load to the output store
//     (the first in registers, a second in LDS), and the row's workgroups
//     meet three times, on synchronisation words tagged with the call
//     (nothing needs clearing between calls).  After stat every workgroup
//     polls all the chunks' statistics and reduces them itself; after the
//     histogram (each workgroup's bins in a slot of its own) the row's first
//     workgroup sums them, selects the bin and hands it to every
//     workgroup's line;
//     after the gather (each chunk's candidates in a stretch of its own,
//     their count on its line) every workgroup polls the counts and ranks a
//     short list itself, while a long list is resolved by the first
//     workgroup and handed out.  The logits are read once and the output
//     written once.  Workgroups are dispatched in index order (a row's
//     chunks are consecutive), so the earliest unfinished row always has
//     all its workgroups placed or placeable: every wait ends.  A wait that
//     still gives up (after about a second) writes NaN over its chunk of
//     the output.
//   four launches (otherwise): stat; prob, whose row's last workgroup
//     selects the bin and hands M and S on; gather, whose row's last
//     workgroup resolves; write.  Each launch reads the logits again and
//     recomputes P with the handed-on M and S; no P is stored between
//     launches.  Each launch issues its logits loads before the loads of
//     what the previous launch handed on, so the two round trips overlap.
// Whatever workgroups hand over to each other inside one launch is written
// and read with coherent accesses.
constexpr int kFThreads = 256;
constexpr int kFGroups = 4;                 // 16-byte groups per thread
constexpr int kFPer = 4 * kFGroups;         // 16 entries per thread
constexpr int kFChunk = kFThreads * kFPer;  // 4096 entries per workgroup
constexpr int kFWaves = kFThreads / 64;
constexpr int kFirstShift = 22;             // first level: bits 29-22, 256 bins
// One launch: up to this many rows and chunks per row (every workgroup
// reads the row's chunk statistics).
constexpr int kFusedRows = MOE_FILTER_ONE_LAUNCH_ROWS;
constexpr int kFusedChunks = MOE_FILTER_ONE_LAUNCH_VOCAB / kFChunk;
static_assert(MOE_FILTER_ONE_LAUNCH_VOCAB % kFChunk == 0, "whole chunks");
constexpr unsigned kSpinLimit = 1u << 20;  // polls of a row barrier before it gives up (default)

struct FilterArgs {
  int V, chunks;
  float temperature;
  double top_p;
  // Two row sets in one launch (the verifier's rows and the draft's, with
  // the same settings): rows 0 .. rows_a-1 are rows of logits / probs, the
  // rest rows of logits_b / probs_b.  The per-row workspace arrays are
  // indexed by the launch's row.
  int rows_a;
  const float *logits, *logits_b;
  float *probs, *probs_b;
  float2 *stat;        // [rows][chunks]: (chunk max, sum of exp relative to it)
  uint64_t *rowhist;   // [rows][256] first-level mass histogram
  uint64_t *cand;      // [rows][V] candidates: probability bits | index << 32
  uint64_t *state;     // [rows][8]: prefix, mask, mass above, target; K, index cut, kept
                       // mass; the row's M and S (float bits, S in the high half)
  unsigned *count;     // [rows][4]: arrivals (prob, gather), candidates
  unsigned *sync;      // one launch: [rows][4 chunks] 128-byte synchronisation lines
  uint64_t tag;        // one launch: this call's tag (distinct per call, halves non-zero)
  unsigned spin;       // one launch: polls of a row barrier before it gives up
  uint64_t *hpart;     // one launch: [rows][chunks][256] the chunks' first-level histograms
};

__device__ inline const float *logits_row(const FilterArgs &a, int row) {
  return row < a.rows_a ? a.logits + (size_t)row * a.V
                        : a.logits_b + (size_t)(row - a.rows_a) * a.V;
}
__device__ inline float *probs_row(const FilterArgs &a, int row) {
  return row < a.rows_a ? a.probs + (size_t)row * a.V : a.probs_b + (size_t)(row - a.rows_a) * a.V;
}

// The filter's integer mass of a probability: floor(P * 2^52).  Every
// fp32 P >= 2^-29 is then exact (24 significant bits), the rest lose less
// than 2^-52 each, and a row's total (sum of P about 1) fits 64 bits: the
// decision is exact on the fp32 probabilities even over 2^24 entries.
constexpr double kMassQuant = 4503599627370496.0;  // 2^52
__device__ inline uint64_t mass_of(float p) { return (uint64_t)((double)p * kMassQuant); }

template <class T, class Op>
__device__ inline T block_all(T v, T *scratch, Op op) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = op(v, (T)__shfl_xor(v, m, 64));
  __syncthreads();
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  T r = scratch[0];
  for (int w = 1; w < kFWaves; ++w) r = op(r, scratch[w]);
  return r;
}

// Exclusive prefix of a per-thread count over the workgroup (thread order)
// and the workgroup's total.
__device__ inline uint32_t block_exclusive(uint32_t n, uint32_t &total) {
  __shared__ uint32_t wtot[kFWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = n;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t t = __shfl_up(inc, d, 64);
    if (lane >= d) inc += t;
  }
  __syncthreads();
  if (lane == 63) wtot[wave] = inc;
  __syncthreads();
  uint32_t before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kFWaves; ++w) {
    before += w < wave ? wtot[w] : 0u;
    total += wtot[w];
  }
  return before + inc - n;
}

// Entry of this thread's group g: c0 + (g * kFThreads + tid) * 4 (+ 0..3).
__device__ inline int entry_of(int c0, int g) { return c0 + (g * kFThreads + (int)threadIdx.x) * 4; }

// This workgroup's chunk, `fill` past the row: 16-byte loads when the row
// is 16-byte aligned and V a multiple of 4 (then a group is all in or all
// out of the row), else per entry.
__device__ inline void load_chunk(const float *row, int V, int c0, float (&v)[kFPer], float fill) {
  const bool vec = (V & 3) == 0 && ((uintptr_t)row & 15) == 0;
#pragma unroll
  for (int g = 0; g < kFGroups; ++g) {
    const int j = entry_of(c0, g);
    if (vec) {
      const float4 t = j < V ? *(const float4 *)(row + j) : make_float4(fill, fill, fill, fill);
      v[4 * g] = t.x;
      v[4 * g + 1] = t.y;
      v[4 * g + 2] = t.z;
      v[4 * g + 3] = t.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * g + e] = j + e < V ? row[j + e] : fill;
    }
  }
}

__device__ inline void store_chunk(float *row, int V, int c0, const float (&v)[kFPer]) {
  const bool vec = (V & 3) == 0 && ((uintptr_t)row & 15) == 0;
#pragma unroll
  for (int g = 0; g < kFGroups; ++g) {
    const int j = entry_of(c0, g);
    if (vec) {
      if (j < V) *(float4 *)(row + j) = make_float4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j + e < V) row[j + e] = v[4 * g + e];
    }
  }
}

// The chunk's max of z = logit * (1 / T) and sum of exp(z - max).  The
// product is one rounding more than a division, but monotone in the logit
// (equal logits stay equal), and the same in every phase.  The filter's
// arithmetic is not contracted into fused multiply-adds: whether the
// compiler fuses z - M depends on what else uses z in the kernel, so each
// product, difference and sum is rounded on its own, the same way in every
// kernel.
__device__ inline float2 chunk_stat(const float (&v)[kFPer], float temperature, float *fs) {
#pragma clang fp contract(off)
  const float inv_t = 1.0f / temperature;
  float z[kFPer];
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < kFPer; ++k) {
    z[k] = v[k] * inv_t;
    m = fmaxf(m, z[k]);
  }
  m = block_all(m, fs, [](float x, float y) { return fmaxf(x, y); });
  float S = 0.f;
  if (m != -INFINITY) {
#pragma unroll
    for (int k = 0; k < kFPer; ++k) S += expf(z[k] - m);
  }
  S = block_all(S, fs, [](float x, float y) { return x + y; });
  return make_float2(m, S);
}

__device__ inline uint64_t ms_bits(float2 ms) {
  return (uint64_t)__float_as_uint(ms.x) | ((uint64_t)__float_as_uint(ms.y) << 32);
}
__device__ inline float2 ms_of(uint64_t b) {
  return make_float2(__uint_as_float((uint32_t)b), __uint_as_float((uint32_t)(b >> 32)));
}

// The row's max and sum of exponentials from the chunks' (max, sum): a
// fixed-order reduction, so every workgroup of the row gets the same bits.
// COH: the pairs were written in this launch (coherent loads).
template <bool COH>
__device__ inline float2 row_stat(const float2 *st, int chunks, float *fs) {
#pragma clang fp contract(off)
  float2 mine[(kFusedChunks + kFThreads - 1) / kFThreads];
  float m = -INFINITY;
  int i = 0;
  for (int c = threadIdx.x; c < chunks; c += kFThreads, ++i) {
    const float2 t = COH ? ms_of(load_coherent64((const uint64_t *)(st + c))) : st[c];
    if (COH) mine[i] = t;
    m = fmaxf(m, t.x);
  }
  m = block_all(m, fs, [](float x, float y) { return fmaxf(x, y); });
  float S = 0.f;
  i = 0;
  for (int c = threadIdx.x; c < chunks; c += kFThreads, ++i) {
    const float2 t = COH ? mine[i] : st[c];
    if (t.x != -INFINITY) S += t.y * expf(t.x - m);
  }
  S = block_all(S, fs, [](float x, float y) { return x + y; });
  return make_float2(m, S);
}

// P of a logit given the row's max M and sum S of exp(z - M): every phase
// computes it with this one expression, so all of them get the same bits.
// exp(z - M) <= 1 and 1 / S <= 1 (S >= 1: the max's own term), so P <= 1
// and its bits 31-30 are zero; a -inf fill (past the row) gives 0.
__device__ inline float prob_of(float logit, float temperature, float2 ms) {
#pragma clang fp contract(off)
  return expf(logit * (1.0f / temperature) - ms.x) * (1.0f / ms.y);
}

// Selection over NB mass bins h (bits [shift, shift + log2 NB) of the
// probability, in global memory written by this launch's other workgroups
// and read coherently, or in LDS): the bin where the mass counted from the
// top reaches the target.  Updates prefix / mask / above; returns the
// bin's mass.  With top_p > 0 (the first level, whose histogram holds
// every entry) the target is first set to ceil(top_p * W), W the total.
template <int NB, bool GLOBAL>
__device__ inline uint64_t select_level(const uint64_t *h, int shift, uint64_t &target,
                                        uint32_t &prefix, uint32_t &mask, uint64_t &above,
                                        double top_p = 0.0) {
  constexpr int PT = NB / kFThreads;  // consecutive bins per thread
  static_assert(PT >= 1 && NB % kFThreads == 0, "bins per thread");
  __shared__ uint64_t wsum[kFWaves];
  __shared__ uint32_t s_digit;
  __shared__ uint64_t s_above, s_bin;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t own[PT], tot = 0;
#pragma unroll
  for (int i = 0; i < PT; ++i) own[i] = GLOBAL ? load_coherent64(h + tid * PT + i) : h[tid * PT + i];
#pragma unroll
  for (int i = 0; i < PT; ++i) tot += own[i];
  uint64_t suf = tot;  // inclusive sum over the lanes >= this lane of the wave
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t lo = __shfl_down((uint32_t)suf, d, 64);
    const uint32_t hi = __shfl_down((uint32_t)(suf >> 32), d, 64);
    if (lane + d < 64) suf += ((uint64_t)hi << 32) | lo;
  }
  __syncthreads();
  if (lane == 0) wsum[wave] = suf;  // the wave's total
  __syncthreads();
  uint64_t W = 0, later = 0;  // total; mass of the later waves' bins
#pragma unroll
  for (int w = 0; w < kFWaves; ++w) {
    W += wsum[w];
    later += w > wave ? wsum[w] : 0ull;
  }
  uint64_t tg = target;
  if (top_p > 0.0) {
    tg = (uint64_t)ceil(top_p * (double)W);
    tg = tg < 1 ? 1 : tg;
  }
  uint64_t c = above + later + (suf - tot);  // mass of the bins above this thread's
#pragma unroll
  for (int i = PT - 1; i >= 0; --i) {
    if (c < tg && c + own[i] >= tg) {  // exactly one bin of the row
      s_digit = (uint32_t)(tid * PT + i);
      s_above = c;
      s_bin = own[i];
    }
    c += own[i];
  }
  __syncthreads();
  target = tg;
  prefix |= s_digit << shift;
  mask |= (uint32_t)(NB - 1) << shift;
  above = s_above;
  return s_bin;
}

// Over NB count bins h in LDS, in ascending bin order: the bin where the
// running count, starting at base, reaches rank (1-based).  Sets base to
// the count below that bin.
template <int NB>
__device__ inline uint32_t rank_bin(const uint32_t *h, uint32_t rank, uint32_t &base) {
  constexpr int PT = NB / kFThreads;
  __shared__ uint32_t s_digit, s_base;
  uint32_t own[PT], tot = 0;
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    own[i] = h[threadIdx.x * PT + i];
    tot += own[i];
  }
  uint32_t total;
  uint32_t c = base + block_exclusive(tot, total);  // count below this thread's bins
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    if (c < rank && c + own[i] >= rank) {
      s_digit = threadIdx.x * PT + i;
      s_base = c;
    }
    c += own[i];
  }
  __syncthreads();
  base = s_base;
  return s_digit;
}

// After this workgroup's hand-over stores and atomics: true in the last
// workgroup of the row to arrive (n arrivals in all).
__device__ inline bool arrive_last(unsigned *ctr, unsigned n) {
  __shared__ int s_last;
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) s_last = atomicAdd(ctr, 1u) == n - 1;
  __syncthreads();
  return s_last != 0;
}

// The chunk's first-level mass histogram (bits 29-22 of P), one LDS copy
// per wave in lh (kFWaves x 256), added into the row's bins rh.
__device__ inline void add_chunk_hist(const float (&p)[kFPer], unsigned long long *lh,
                                      uint64_t *rh) {
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int i = tid; i < kFWaves * 256; i += kFThreads) lh[i] = 0ull;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kFPer; ++k)
    if (p[k] > 0.f)
      atomicAdd(&lh[wave * 256 + ((__float_as_uint(p[k]) >> kFirstShift) & 255u)],
                (unsigned long long)mass_of(p[k]));
  __syncthreads();
  static_assert(kFWaves == 4 && kFThreads == 256, "one bin per thread, four copies");
  const uint64_t t = lh[tid] + lh[256 + tid] + lh[512 + tid] + lh[768 + tid];
  if (t) atomicAdd((unsigned long long *)&rh[tid], (unsigned long long)t);
}

// The chunk's entries in the selected bin appended to the row's candidate
// list (its length counted at *n_cand).
__device__ inline void append_candidates(const float (&p)[kFPer], int c0, uint32_t prefix,
                                         uint32_t mask, uint64_t *cand, unsigned *n_cand) {
  const int tid = threadIdx.x;
  uint32_t mine = 0;
#pragma unroll
  for (int k = 0; k < kFPer; ++k)
    mine += ((__float_as_uint(p[k]) & mask) == prefix && p[k] > 0.f) ? 1u : 0u;
  uint32_t total;
  const uint32_t off = block_exclusive(mine, total);
  __shared__ uint32_t s_base;
  if (tid == 0) s_base = total ? atomicAdd(n_cand, total) : 0u;
  __syncthreads();
  uint32_t at = s_base + off;
#pragma unroll
  for (int g = 0; g < kFGroups; ++g) {
    const int j = entry_of(c0, g);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t key = __float_as_uint(p[4 * g + e]);
      if ((key & mask) == prefix && p[4 * g + e] > 0.f)
        store_coherent64(cand + at++, (uint64_t)key | ((uint64_t)(j + e) << 32));
    }
  }
}

// The boundary from at most kDirect candidates (candidate i is cand(i), a
// coherent load): each
// candidate's rank in the order (probability descending, index ascending)
// by counting the candidates before it, their masses in that order, a
// running sum, and the first rank at which the mass above the bin plus the
// running sum reaches the target: that token is the last one kept, its
// probability is K and its index the cut (the ties at K after it in the
// order have larger indices).  The one thread that finds it writes K, the
// cut and the kept mass to out[0..2].
// ord and by_rank are LDS arrays of kDirect entries each.
constexpr uint32_t kDirect = 512;
template <class Load>
__device__ inline void resolve_direct(Load cand, uint32_t n, uint64_t above,
                                      uint64_t target, unsigned long long *ord,
                                      unsigned long long *by_rank, uint64_t *out) {
  __shared__ uint64_t scratch[kWavesV];
  const int tid = threadIdx.x;
  for (uint32_t i = tid; i < n; i += kFThreads) {
    const uint64_t e = cand(i);
    ord[i] = ((uint64_t)(uint32_t)e << 32) | (0xFFFFFFFFu - (uint32_t)(e >> 32));
  }
  __syncthreads();
  for (uint32_t i = tid; i < n; i += kFThreads) {
    const uint64_t o = ord[i];
    uint32_t r = 0;
    for (uint32_t q = 0; q < n; ++q) r += ord[q] > o ? 1u : 0u;  // keys are distinct
    by_rank[r] = o;
  }
  __syncthreads();
  static_assert(kDirect == 2 * kFThreads, "two ranks per thread");
  const uint32_t r0 = 2 * tid, r1 = r0 + 1;
  const uint64_t m0 = r0 < n ? mass_of(__uint_as_float((uint32_t)(by_rank[r0] >> 32))) : 0;
  const uint64_t m1 = r1 < n ? mass_of(__uint_as_float((uint32_t)(by_rank[r1] >> 32))) : 0;
  uint64_t all;
  const uint64_t before = above + block_scan(m0 + m1, scratch, &all) - (m0 + m1);
  // exactly one rank crosses: the bin holds the crossing, so the running
  // sum over all candidates reaches the target
  uint32_t last = 0xFFFFFFFFu;
  uint64_t kept = 0;
  if (r0 < n && before < target && before + m0 >= target) {
    last = r0;
    kept = before + m0;
  } else if (r1 < n && before + m0 < target && before + m0 + m1 >= target) {
    last = r1;
    kept = before + m0 + m1;
  }
  if (last != 0xFFFFFFFFu) {
    const uint64_t o = by_rank[last];
    out[0] = o >> 32;
    out[1] = 0xFFFFFFFFu - (uint32_t)o;
    out[2] = kept;
  }
}

// The boundary from the row's n candidates (cand(i), coherent loads), the selection
// of the first level given: K, the index cut and the kept mass to out[0..2]
// (written by thread 0 on the radix path).  lh: 1024 LDS entries (the
// direct path's two arrays; the radix path's 256 mass bins, then 256
// count bins).  Radix levels are 8 bits wide, so each takes one bin per
// thread: K from bits 21-14, 13-6 and 7-0 (bits 7-6 already fixed, so
// the bins outside them stay empty), the index cut from bits 23-16, 15-8
// and 7-0 of the tied indices.
template <class Load>
__device__ inline void resolve_row(Load cand, uint32_t n, uint32_t prefix,
                                   uint32_t mask, uint64_t above, uint64_t target,
                                   unsigned long long *lh, uint64_t *out) {
  if (n <= kDirect) {
    resolve_direct(cand, n, above, target, lh, lh + kDirect, out);
    return;
  }
  uint32_t *lc = (uint32_t *)lh;
  const int tid = threadIdx.x;
  uint64_t bin = 0;
#pragma unroll 1
  for (int shift = 14; shift >= 0; shift = shift > 6 ? shift - 8 : shift - 6) {
    lh[tid] = 0ull;
    __syncthreads();
    for (uint32_t i = tid; i < n; i += kFThreads) {
      const uint32_t key = (uint32_t)cand(i);
      if ((key & mask) == prefix)
        atomicAdd(&lh[(key >> shift) & 255u], (unsigned long long)mass_of(__uint_as_float(key)));
    }
    __syncthreads();
    bin = select_level<256, false>((const uint64_t *)lh, shift, target, prefix, mask, above);
    __syncthreads();  // every thread has read its bin
  }
  const uint32_t K = prefix;                       // the last kept probability's bits
  const uint64_t mk = mass_of(__uint_as_float(K));  // > 0: the target lies in positive mass
  const uint64_t ties = bin / mk;                  // all of equal mass mk
  const uint64_t keep = (target - above + mk - 1) / mk;
  uint32_t cut = 0xFFFFFFFFu;  // every tie kept
  if (keep < ties) {
    // the keep-th smallest index among the ties, 8 index bits at a time
    uint32_t ip = 0, im = 0, base = 0;
#pragma unroll 1
    for (int shift = 16; shift >= 0; shift -= 8) {
      lc[tid] = 0u;
      __syncthreads();
      for (uint32_t i = tid; i < n; i += kFThreads) {
        const uint64_t e = cand(i);
        const uint32_t j = (uint32_t)(e >> 32);
        if ((uint32_t)e == K && (j & im) == ip) atomicAdd(&lc[(j >> shift) & 255u], 1u);
      }
      __syncthreads();
      ip |= rank_bin<256>(lc, (uint32_t)keep, base) << shift;
      im |= 255u << shift;
      __syncthreads();  // every thread has read its bin
    }
    cut = ip;
  }
  if (tid == 0) {
    out[0] = K;
    out[1] = cut;
    out[2] = above + keep * mk;  // the kept mass
  }
}

// The chunk's output: P kept (P > K, or P = K at an index up to the cut)
// renormalised by the kept mass, the rest zero.
__device__ inline void write_chunk(float *out, int V, int c0, float (&p)[kFPer], uint64_t kbits,
                                   uint64_t cut64, uint64_t kept) {
  const float pk = __uint_as_float((uint32_t)kbits);  // the last kept probability
  const uint32_t cut = (uint32_t)cut64;                // ties kept up to this index
  const float total = (float)((double)kept / kMassQuant);
#pragma unroll
  for (int g = 0; g < kFGroups; ++g) {
    const uint32_t j = (uint32_t)entry_of(c0, g);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = p[4 * g + e];
      const bool keep = x > pk || (x == pk && x > 0.f && j + e <= cut);
      p[4 * g + e] = keep ? x / total : 0.f;
    }
  }
  store_chunk(out, V, c0, p);
}

// ---- four launches

__global__ __launch_bounds__(kFThreads) void filter_stat_kernel(FilterArgs a) {
  const int row = blockIdx.y, c = blockIdx.x;
  __shared__ float fs[kFWaves];
  float v[kFPer];
  load_chunk(logits_row(a, row), a.V, c * kFChunk, v, -INFINITY);
  const float2 cs = chunk_stat(v, a.temperature, fs);
  if (threadIdx.x == 0) a.stat[(size_t)row * a.chunks + c] = cs;
  // the row's histogram and counters start at zero for the later launches
  if (a.top_p < 1.0 && c == 0) {
    a.rowhist[(size_t)row * 256 + threadIdx.x] = 0;
    if (threadIdx.x < 4) a.count[(size_t)row * 4 + threadIdx.x] = 0u;
  }
}

// HIST: top_p < 1 (the first-level histogram and selection follow); the
// plain softmax instantiation reserves no histogram LDS.
template <bool HIST>
__global__ __launch_bounds__(kFThreads) void filter_prob_kernel(FilterArgs a) {
  const int row = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  __shared__ float fs[kFWaves];
  float v[kFPer];
  const int c0 = c * kFChunk;
  load_chunk(logits_row(a, row), a.V, c0, v, -INFINITY);
  const float2 ms = row_stat<false>(a.stat + (size_t)row * a.chunks, a.chunks, fs);
#pragma unroll
  for (int k = 0; k < kFPer; ++k) v[k] = prob_of(v[k], a.temperature, ms);
  if (!HIST) {
    store_chunk(probs_row(a, row), a.V, c0, v);
    return;
  }
  __shared__ unsigned long long lh[kFWaves * 256];
  uint64_t *rh = a.rowhist + (size_t)row * 256;
  add_chunk_hist(v, lh, rh);
  if (!arrive_last(a.count + (size_t)row * 4, a.chunks)) return;
  uint32_t prefix = 0, mask = 0xC0000000u;  // bits 31-30 are zero for every entry
  uint64_t above = 0, target = 0;
  select_level<256, true>(rh, kFirstShift, target, prefix, mask, above, a.top_p);
  if (tid == 0) {
    uint64_t *st = a.state + (size_t)row * 8;
    st[0] = prefix;
    st[1] = mask;
    st[2] = above;
    st[3] = target;
    st[7] = ms_bits(ms);
  }
}

__global__ __launch_bounds__(kFThreads) void filter_gather_kernel(FilterArgs a) {
  const int row = blockIdx.y, c = blockIdx.x;
  __shared__ unsigned long long lh[2 * kDirect];
  float p[kFPer];
  const int c0 = c * kFChunk;
  load_chunk(logits_row(a, row), a.V, c0, p, -INFINITY);
  uint64_t *st = a.state + (size_t)row * 8;
  const uint32_t prefix = (uint32_t)st[0], mask = (uint32_t)st[1];
  const float2 ms = ms_of(st[7]);
#pragma unroll
  for (int k = 0; k < kFPer; ++k) p[k] = prob_of(p[k], a.temperature, ms);
  uint64_t *cand = a.cand + (size_t)row * a.V;
  append_candidates(p, c0, prefix, mask, cand, a.count + (size_t)row * 4 + 2);
  if (!arrive_last(a.count + (size_t)row * 4 + 1, a.chunks)) return;
  const uint32_t n = __hip_atomic_load(a.count + (size_t)row * 4 + 2, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  resolve_row([cand](uint32_t i) { return load_coherent64(cand + i); }, n, prefix, mask, st[2],
              st[3], lh, st + 4);
}

__global__ __launch_bounds__(kFThreads) void filter_write_kernel(FilterArgs a) {
  const int row = blockIdx.y, c = blockIdx.x;
  const int c0 = c * kFChunk;
  float p[kFPer];
  load_chunk(logits_row(a, row), a.V, c0, p, -INFINITY);
  const uint64_t *st = a.state + (size_t)row * 8;
  const float2 ms = ms_of(st[7]);
#pragma unroll
  for (int k = 0; k < kFPer; ++k) p[k] = prob_of(p[k], a.temperature, ms);
  write_chunk(probs_row(a, row), a.V, c0, p, st[4], st[5], st[6]);
}

// ---- one launch

// Synchronisation lines of a row, 128 bytes each.  Device-scope accesses to
// one line queue behind each other at the memory side, so what many
// workgroups poll is spread over lines.  Nothing clears them: every word a
// waiter accepts carries the call's 64-bit tag (FilterArgs::tag, distinct
// for every call of the process, both 32-bit halves non-zero), so what an
// earlier call or other data left there is never taken for this call's.  A
// value shares its 64-bit words with the tag: the low half holds the value,
// the high half one half of the tag, and a slot is accepted when both its
// words carry their halves.  Per chunk c and workgroup w of the row (a
// workgroup holds one or two consecutive chunks):
//   stat[c]   words 0-1: chunk c's max and sum (float bits) | tag halves
//   count[c]  words 0-1: chunk c's number of candidates | tag halves
//   hist[w]   word 0: the tag, once workgroup w's histogram slot is written
//   out[w]    polled only by workgroup w, four tagged 32-bit values each:
//             words 0-3 the selected bin (from the row's first workgroup,
//             which sums the histograms), words 4-7 the boundary of a long
//             candidate list (from the same workgroup)
constexpr int kLineWords = 32;  // 128 bytes
constexpr int kRowLines = 4;    // stat, count, hist, out: lines per chunk
constexpr int kStatLine = 0, kCountLine = 1, kHistLine = 2, kOutLine = 3;
__device__ inline unsigned *row_lines(const FilterArgs &a, int row) {
  return a.sync + (size_t)row * kRowLines * a.chunks * kLineWords;
}
__device__ inline uint64_t *line_of(unsigned *lines, int kind, int n, int c) {
  return (uint64_t *)(lines + (size_t)(kind * n + c) * kLineWords);
}
__device__ inline uint64_t with_tag(uint32_t v, uint32_t half) {
  return (uint64_t)v | ((uint64_t)half << 32);
}

// A value and the call's tag in two words of line c (one 64-bit store each).
__device__ inline void put_tagged(uint64_t *w, uint32_t v0, uint32_t v1, uint64_t tag) {
  store_coherent64(w, with_tag(v0, (uint32_t)tag));
  store_coherent64(w + 1, with_tag(v1, (uint32_t)(tag >> 32)));
}

// Wait (bounded) until line t of `kind` holds a tagged value for every
// t < n; thread t < n gets its line's two value halves.  False if the wait
// gave up (the same in every thread).
__device__ inline bool wait_tagged(unsigned *lines, int kind, unsigned n, uint64_t tag,
                                   unsigned spin, uint32_t &v0, uint32_t &v1) {
  const uint64_t *p = threadIdx.x < n ? line_of(lines, kind, (int)n, threadIdx.x) : nullptr;
  uint64_t w0 = 0, w1 = 0;
  bool ok = p == nullptr;
  for (unsigned i = 0;; ++i) {
    if (!ok) {
      w0 = load_coherent64(p);
      w1 = load_coherent64(p + 1);
      ok = (uint32_t)(w0 >> 32) == (uint32_t)tag && (uint32_t)(w1 >> 32) == (uint32_t)(tag >> 32);
    }
    if (__syncthreads_and(ok)) break;
    if (i + 1 >= spin) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  v0 = (uint32_t)w0;
  v1 = (uint32_t)w1;
  return true;
}

// Wait (bounded) until word `word` of line t of `kind` equals the tag, for
// every t < count (n lines of each kind).
__device__ inline bool wait_flags(unsigned *lines, int kind, unsigned n, unsigned count, int word,
                                  uint64_t tag, unsigned spin) {
  const uint64_t *p =
      threadIdx.x < count ? line_of(lines, kind, (int)n, threadIdx.x) + word : nullptr;
  bool ok = p == nullptr;
  for (unsigned i = 0;; ++i) {
    if (!ok) ok = load_coherent64(p) == tag;
    if (__syncthreads_and(ok)) break;
    if (i + 1 >= spin) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  return true;
}

// The first workgroup's result for each of the row's `count` workgroups:
// four 32-bit values, each in a word of its own with a half of the tag
// (words [first, first + 4) of each out line), so no store has to land
// before another.
__device__ inline void hand_out(unsigned *lines, unsigned n, unsigned count, int first,
                                const uint32_t (&v)[4], uint64_t tag) {
  for (unsigned i = threadIdx.x; i < count; i += kFThreads) {
    uint64_t *o = line_of(lines, kOutLine, (int)n, i) + first;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      store_coherent64(o + k, with_tag(v[k], (uint32_t)(k & 1 ? tag >> 32 : tag)));
  }
}

// Workgroup c's share of a hand-out: wait (bounded) until the four words
// carry the tag, then every thread gets the values.  False if the wait gave
// up.
__device__ inline bool take_out(unsigned *lines, unsigned n, int c, int first, uint64_t tag,
                                unsigned spin, uint32_t (&v)[4]) {
  __shared__ uint32_t s_v[4];
  __shared__ int s_ok;
  if (threadIdx.x == 0) {
    const uint64_t *o = line_of(lines, kOutLine, (int)n, c) + first;
    int ok = 1;
    for (unsigned i = 0;; ++i) {
      bool all = true;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint64_t x = load_coherent64(o + k);
        s_v[k] = (uint32_t)x;
        all = all && (uint32_t)(x >> 32) == (uint32_t)(k & 1 ? tag >> 32 : tag);
      }
      if (all) break;
      if (i + 1 >= spin) {
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    s_ok = ok;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) v[k] = s_v[k];
  return s_ok != 0;
}

// A wait gave up: the output of workgroup wg's chunks (the first `mine` of
// its CPW) is NaN, so the failure shows.
template <int CPW>
__device__ inline void poison_chunks(float *out, int V, int wg, int mine) {
  float nan[kFPer];
#pragma unroll
  for (int k = 0; k < kFPer; ++k) nan[k] = __builtin_nanf("");
#pragma unroll
  for (int j = 0; j < CPW; ++j)
    if (j < mine) store_chunk(out, V, (wg * CPW + j) * kFChunk, nan);
}

template <bool HIST, int CPW>
__device__ __attribute__((always_inline)) inline void filter_fused(const FilterArgs &a) {
  static_assert(CPW == 1 || CPW == 2, "one or two chunks per workgroup");
  const int row = blockIdx.y, wg = blockIdx.x, tid = threadIdx.x;
  const unsigned n = (unsigned)a.chunks;    // 4096-entry chunks of the row
  const unsigned nw = (n + CPW - 1) / CPW;  // the row's workgroups
  // this workgroup's chunks: wg * CPW (entries from c0) and, with two per
  // workgroup, the next one when the row has it (the same in every thread,
  // so the per-chunk steps keep the workgroup's barriers together)
  const int c0 = wg * CPW * kFChunk;
  const bool two = CPW == 2 && (unsigned)(wg * CPW + 1) < n;
  const int mine = two ? 2 : 1;
  const uint64_t tag = a.tag;
  unsigned *lines = row_lines(a, row);
  __shared__ float fs[kFWaves];
  __shared__ unsigned long long lds[2 * kDirect];  // histogram copies, then the resolve's arrays
  static_assert(2 * kDirect >= kFWaves * 256, "the histogram copies fit");
  static_assert(kFusedChunks <= kFThreads, "a chunk per thread in the waits");
  __shared__ uint64_t res[3];                      // K, index cut, kept mass
  __shared__ uint32_t off[kFusedChunks + 1];       // candidate offsets of the chunks
  // the second chunk's probabilities between the phases (top-p, two chunks
  // per workgroup), element k of thread t at k * kFThreads + t: the first
  // chunk stays in registers
  __shared__ float hold[HIST && CPW == 2 ? kFPer * kFThreads : 1];
  float v[kFPer], u[kFPer];
  load_chunk(logits_row(a, row), a.V, c0, v, -INFINITY);
  // (past the row: -inf fill, probability 0)
  if constexpr (CPW == 2) load_chunk(logits_row(a, row), a.V, c0 + kFChunk, u, -INFINITY);
  float *out = probs_row(a, row);
  // the chunks' statistics: each workgroup reduces all of them itself (the
  // fixed-order reduction of the four-launch schedule)
  {
    const float2 cs = chunk_stat(v, a.temperature, fs);
    if (tid == 0)
      put_tagged(line_of(lines, kStatLine, n, wg * CPW), __float_as_uint(cs.x),
                 __float_as_uint(cs.y), tag);
  }
  if constexpr (CPW == 2) {
    if (two) {
      const float2 cs = chunk_stat(u, a.temperature, fs);
      if (tid == 0)
        put_tagged(line_of(lines, kStatLine, n, wg * CPW + 1), __float_as_uint(cs.x),
                   __float_as_uint(cs.y), tag);
    }
  }
  wait_stores();
  uint32_t lo0 = 0, lo1 = 0;
  if (!wait_tagged(lines, kStatLine, n, tag, a.spin, lo0, lo1))
    return poison_chunks<CPW>(out, a.V, wg, mine);
  float2 ms;
  {
    const float2 t = tid < (int)n ? make_float2(__uint_as_float(lo0), __uint_as_float(lo1))
                                  : make_float2(-INFINITY, 0.f);
    float m = block_all(t.x, fs, [](float x, float y) { return fmaxf(x, y); });
    float S;
    {
#pragma clang fp contract(off)
      S = (tid < (int)n && t.x != -INFINITY) ? t.y * expf(t.x - m) : 0.f;
    }
    S = block_all(S, fs, [](float x, float y) { return x + y; });
    ms = make_float2(m, S);
  }
#pragma unroll
  for (int k = 0; k < kFPer; ++k) v[k] = prob_of(v[k], a.temperature, ms);
  if constexpr (CPW == 2) {
#pragma unroll
    for (int k = 0; k < kFPer; ++k) u[k] = prob_of(u[k], a.temperature, ms);
  }
  if (!HIST) {
    store_chunk(out, a.V, c0, v);
    if (two) store_chunk(out, a.V, c0 + kFChunk, u);
    return;
  }
  // the workgroup's histogram (its chunks' bins: integer masses, so how the
  // chunks are grouped does not change the row's sums) into its own slot;
  // the row's first workgroup sums the slots, selects the bin and hands it
  // out
  uint64_t *part = a.hpart + (size_t)row * a.chunks * 256;
  {
    const int wave = tid >> 6;
    for (int i = tid; i < kFWaves * 256; i += kFThreads) lds[i] = 0ull;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kFPer; ++k)
      if (v[k] > 0.f)
        atomicAdd(&lds[wave * 256 + ((__float_as_uint(v[k]) >> kFirstShift) & 255u)],
                  (unsigned long long)mass_of(v[k]));
    if constexpr (CPW == 2) {
#pragma unroll
      for (int k = 0; k < kFPer; ++k) {
        if (u[k] > 0.f)
          atomicAdd(&lds[wave * 256 + ((__float_as_uint(u[k]) >> kFirstShift) & 255u)],
                    (unsigned long long)mass_of(u[k]));
        hold[k * kFThreads + tid] = u[k];
      }
    }
    __syncthreads();
    store_coherent64(part + (size_t)wg * 256 + tid,
                     lds[tid] + lds[256 + tid] + lds[512 + tid] + lds[768 + tid]);
    wait_stores();
    __syncthreads();
    if (tid == 0) store_coherent64(line_of(lines, kHistLine, n, wg), tag);
  }
  uint32_t prefix = 0, mask = 0xC0000000u | (255u << kFirstShift);
  uint64_t above = 0, target = 0;
  uint64_t w[2];
  if (wg == 0) {
    if (!wait_flags(lines, kHistLine, n, nw, 0, tag, a.spin)) return poison_chunks<CPW>(out, a.V, wg, mine);
    uint64_t h = 0;  // the row's bin tid: the slots' counts (eight loads in flight)
    for (unsigned q0 = 0; q0 < nw; q0 += 8) {
      uint64_t t[8];
#pragma unroll
      for (unsigned j = 0; j < 8; ++j)
        t[j] = q0 + j < nw ? load_coherent64(part + (size_t)(q0 + j) * 256 + tid) : 0ull;
#pragma unroll
      for (unsigned j = 0; j < 8; ++j) h += t[j];
    }
    __syncthreads();  // every thread has read its copy bins
    lds[tid] = h;
    __syncthreads();
    uint32_t pf = 0, mk = 0xC0000000u;
    select_level<256, false>((const uint64_t *)lds, kFirstShift, target, pf, mk, above, a.top_p);
    prefix = pf;
    // above < target <= W < 2^53: their high words leave room for the bin
    const uint32_t hv[4] = {(uint32_t)above, (uint32_t)(above >> 32) | ((pf >> kFirstShift) << 24),
                            (uint32_t)target, (uint32_t)(target >> 32)};
    hand_out(lines, n, nw, 0, hv, tag);
  } else {
    uint32_t hv[4];
    if (!take_out(lines, n, wg, 0, tag, a.spin, hv)) return poison_chunks<CPW>(out, a.V, wg, mine);
    above = (uint64_t)hv[0] | ((uint64_t)(hv[1] & 0xFFFFFFu) << 32);
    prefix = (hv[1] >> 24) << kFirstShift;
    target = (uint64_t)hv[2] | ((uint64_t)hv[3] << 32);
  }
  // each chunk's candidates (entries in the bin) into its own stretch of
  // the row's list, their number into its count line
  uint64_t *cand = a.cand + (size_t)row * a.V;
  auto emit = [&](const float (&p)[kFPer], int c) {
    uint32_t cnt = 0;
#pragma unroll
    for (int k = 0; k < kFPer; ++k)
      cnt += ((__float_as_uint(p[k]) & mask) == prefix && p[k] > 0.f) ? 1u : 0u;
    uint32_t total;
    uint32_t at = block_exclusive(cnt, total);
    const int e0 = c * kFChunk;
#pragma unroll
    for (int g = 0; g < kFGroups; ++g) {
      const int j = entry_of(e0, g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = __float_as_uint(p[4 * g + e]);
        if ((key & mask) == prefix && p[4 * g + e] > 0.f)
          store_coherent64(cand + e0 + at++, (uint64_t)key | ((uint64_t)(j + e) << 32));
      }
    }
    wait_stores();
    __syncthreads();
    if (tid == 0) put_tagged(line_of(lines, kCountLine, n, c), total, total, tag);
  };
  emit(v, wg * CPW);
  if constexpr (CPW == 2) {
    if (two) {
      float t[kFPer];
#pragma unroll
      for (int k = 0; k < kFPer; ++k) t[k] = hold[k * kFThreads + tid];
      emit(t, wg * CPW + 1);
    }
  }
  wait_stores();
  if (!wait_tagged(lines, kCountLine, n, tag, a.spin, lo0, lo1))
    return poison_chunks<CPW>(out, a.V, wg, mine);
  uint32_t nc;
  {
    const uint32_t k_t = tid < (int)n ? lo0 : 0u;
    const uint32_t o = block_exclusive(k_t, nc);
    if (tid < (int)n) off[tid] = o;
    if (tid == 0) off[n] = nc;
    __syncthreads();
  }
  // candidate i: the chunk whose stretch holds it (binary search of the
  // offsets), then its place in the stretch
  auto load = [&](uint32_t i) {
    uint32_t lo = 0, hi = n;  // off[lo] <= i < off[hi]
    while (hi - lo > 1) {
      const uint32_t mid = (lo + hi) / 2;
      if (off[mid] <= i) lo = mid;
      else hi = mid;
    }
    return load_coherent64(cand + (size_t)lo * kFChunk + (i - off[lo]));
  };
  if (nc <= kDirect) {
    // a short list: every workgroup ranks it itself
    resolve_direct(load, nc, above, target, lds, lds + kDirect, res);
    __syncthreads();
    w[0] = res[0] | (res[1] << 32);
    w[1] = res[2];
  } else if (wg == 0) {
    // a long list: the first workgroup resolves it and hands the result out
    resolve_row(load, nc, prefix, mask, above, target, lds, res);
    __syncthreads();
    w[0] = res[0] | (res[1] << 32);
    w[1] = res[2];
    const uint32_t rv[4] = {(uint32_t)res[0], (uint32_t)res[1], (uint32_t)res[2],
                            (uint32_t)(res[2] >> 32)};
    hand_out(lines, n, nw, 4, rv, tag);
  } else {
    uint32_t rv[4];
    if (!take_out(lines, n, wg, 4, tag, a.spin, rv)) return poison_chunks<CPW>(out, a.V, wg, mine);
    w[0] = (uint64_t)rv[0] | ((uint64_t)rv[1] << 32);
    w[1] = (uint64_t)rv[2] | ((uint64_t)rv[3] << 32);
  }
  write_chunk(out, a.V, c0, v, (uint32_t)w[0], w[0] >> 32, w[1]);
  if constexpr (CPW == 2) {
    if (two) {
      float t[kFPer];
#pragma unroll
      for (int k = 0; k < kFPer; ++k) t[k] = hold[k * kFThreads + tid];
      write_chunk(out, a.V, c0 + kFChunk, t, (uint32_t)w[0], w[0] >> 32, w[1]);
    }
  }
}

template <bool HIST>
__global__ __launch_bounds__(kFThreads) void filter_fused_kernel(FilterArgs a) {
  filter_fused<HIST, 1>(a);
}

// Two chunks per workgroup (the second one's probabilities held in LDS),
// for grids past the one-chunk kernel's capacity (a call of 68 rows of
// 102,400 or 129,280 entries): half the workgroups, each holding twice the
// entries.
template <bool HIST>
__global__ __launch_bounds__(kFThreads) void filter_fused_pair_kernel(FilterArgs a) {
  filter_fused<HIST, 2>(a);
}

}  // namespace

int filter_chunks(int V) { return (V + kFChunk - 1) / kFChunk; }

bool filter_one_launch(int rows, int V) {
  return rows <= kFusedRows && filter_chunks(V) <= kFusedChunks;
}

namespace {

// A tag for one call of the one-launch filter: a process-wide counter from
// a random start, mixed (splitmix64), both halves made non-zero.  Distinct
// for every call of the process; a word left by another process or by
// other data matches it by chance with odds of about 2^-64.
uint64_t next_tag() {
  static std::atomic<uint64_t> counter{[] {
    std::random_device rd;
    return ((uint64_t)rd() << 32) ^ rd() ^
           (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
  }()};
  uint64_t z = counter.fetch_add(0x9E3779B97F4A7C15ull, std::memory_order_relaxed);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  if ((uint32_t)z == 0) z |= 1u;
  if ((z >> 32) == 0) z |= 1ull << 32;
  return z;
}

// Polls of a row barrier before a one-launch workgroup gives up.
std::atomic<unsigned> g_spin{kSpinLimit};

// Workgroups of the one-launch kernel the current device holds at once (0
// if unknown).  Beyond that, rows wait for earlier rows to finish before
// their workgroups are placed: still correct, but slower.  Measured (V =
// 32,000 to 129,280, top_p = 0.9), the one launch is faster than the four
// up to this many workgroups and slower beyond it.
// kind: 0 the softmax-only kernel, 1 the top-p kernel, 2 and 3 the same
// with two chunks per workgroup.
int fused_capacity(int kind) {
  constexpr int kDevices = 64;
  static std::atomic<int> cache[4][kDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevices) return 0;
  int cap = cache[kind][dev].load(std::memory_order_relaxed);
  if (cap > 0) return cap;
  int per_cu = 0, cus = 0;
  const void *k = kind == 0   ? (const void *)filter_fused_kernel<false>
                  : kind == 1 ? (const void *)filter_fused_kernel<true>
                  : kind == 2 ? (const void *)filter_fused_pair_kernel<false>
                              : (const void *)filter_fused_pair_kernel<true>;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kFThreads, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  cap = per_cu * cus;
  cache[kind][dev].store(cap, std::memory_order_relaxed);
  return cap;
}

}  // namespace

void set_filter_spin_limit(unsigned polls) {
  g_spin.store(polls ? polls : kSpinLimit, std::memory_order_relaxed);
}

size_t filter_ws_bytes(int rows, int V) {
  const size_t ch = (size_t)filter_chunks(V);
  return align_up((size_t)rows * ch * sizeof(float2), 256) +
         align_up((size_t)rows * 256 * sizeof(uint64_t), 256) +

         align_up((size_t)rows * V * sizeof(uint64_t), 256) +
         align_up((size_t)rows * 8 * sizeof(uint64_t), 256) +
         align_up((size_t)rows * 4 * sizeof(unsigned), 256) +
         (filter_one_launch(rows, V)
              ? align_up((size_t)rows * kRowLines * ch * kLineWords * sizeof(unsigned), 256) +
                    (size_t)rows * ch * 256 * sizeof(uint64_t)
              : 0);
}


hipError_t launch_filter(int rows_a, const float *logits_a, float *probs_a, int rows_b,
                         const float *logits_b, float *probs_b, int V, float temperature,
                         float top_p, void *ws, hipStream_t st) {
  const int rows = rows_a + rows_b;
  FilterArgs a{};
  a.V = V;
  a.chunks = filter_chunks(V);
  a.temperature = temperature;
  a.top_p = top_p;
  a.rows_a = rows_a;
  a.logits = logits_a;
  a.probs = probs_a;
  a.logits_b = logits_b;
  a.probs_b = probs_b;
  unsigned char *b = (unsigned char *)ws;
  a.stat = (float2 *)b;
  b += align_up((size_t)rows * a.chunks * sizeof(float2), 256);
  a.rowhist = (uint64_t *)b;
  b += align_up((size_t)rows * 256 * sizeof(uint64_t), 256);
  a.cand = (uint64_t *)b;
  b += align_up((size_t)rows * V * sizeof(uint64_t), 256);
  a.state = (uint64_t *)b;
  b += align_up((size_t)rows * 8 * sizeof(uint64_t), 256);
  a.count = (unsigned *)b;
  b += align_up((size_t)rows * 4 * sizeof(unsigned), 256);
  a.sync = (unsigned *)b;
  b += align_up((size_t)rows * kRowLines * a.chunks * kLineWords * sizeof(unsigned), 256);
  a.hpart = (uint64_t *)b;
  a.spin = g_spin.load(std::memory_order_relaxed);
  const dim3 grid(a.chunks, rows);
  if (filter_one_launch(rows, V)) {
    // the first kernel whose grid the chip holds at once: one chunk per
    // workgroup, else two
    const bool hist = top_p < 1.f;
    const int pairs = (a.chunks + 1) / 2;
    const dim3 grid2(pairs, rows);
    if ((long long)rows * a.chunks <= fused_capacity(hist ? 1 : 0)) {
      a.tag = next_tag();
      if (hist)
        hipLaunchKernelGGL(filter_fused_kernel<true>, grid, dim3(kFThreads), 0, st, a);
      else
        hipLaunchKernelGGL(filter_fused_kernel<false>, grid, dim3(kFThreads), 0, st, a);
      return hipGetLastError();
    }
    if ((long long)rows * pairs <= fused_capacity(hist ? 3 : 2)) {
      a.tag = next_tag();
      if (hist)
        hipLaunchKernelGGL(filter_fused_pair_kernel<true>, grid2, dim3(kFThreads), 0, st, a);
      else
        hipLaunchKernelGGL(filter_fused_pair_kernel<false>, grid2, dim3(kFThreads), 0, st, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL(filter_stat_kernel, grid, dim3(kFThreads), 0, st, a);
  if (top_p < 1.f) {
    hipLaunchKernelGGL(filter_prob_kernel<true>, grid, dim3(kFThreads), 0, st, a);
    hipLaunchKernelGGL(filter_gather_kernel, grid, dim3(kFThreads), 0, st, a);
    hipLaunchKernelGGL(filter_write_kernel, grid, dim3(kFThreads), 0, st, a);
  } else {
    hipLaunchKernelGGL(filter_prob_kernel<false>, grid, dim3(kFThreads), 0, st, a);
  }
  return hipGetLastError();
}

int verify_chunks(int V) { return (V + kVChunk - 1) / kVChunk; }

hipError_t launch_verify(int n_seq, int gamma, int V, int mode, const float *p, const float *q,
                         const int32_t *x, const float *u, const uint32_t *r, int32_t *n_acc,
                         int32_t *out, void *ws, hipStream_t st) {
  VerifyArgs a{};
  a.n_seq = n_seq;
  a.gamma = gamma;
  a.V = V;
  a.mode = mode;
  a.chunks = verify_chunks(V);
  a.p = p;
  a.q = q;
  a.u = u;
  a.x = x;
  a.r = r;
  a.n_acc = n_acc;
  a.out = out;
  a.done = (unsigned *)ws;
  a.part = (uint64_t *)((unsigned char *)ws + 256);
  // about 64 workgroups per sequence: the whole chip for a few sequences,
  // without piling every chunk's arrival onto one counter
  const bool sampling = mode == MOE_VERIFY_SAMPLING;
  const int units = sampling ? a.chunks : a.chunks * (gamma + 1);
  const int cap = sampling ? kUnitsSampling : kUnitsGreedy;
  a.upb = (units + 63) / 64;
  a.upb = a.upb < 1 ? 1 : (a.upb > cap ? cap : a.upb);
  const int per_seq = (units + a.upb - 1) / a.upb;
  hipLaunchKernelGGL(verify_kernel, dim3(per_seq, n_seq), dim3(kVThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
