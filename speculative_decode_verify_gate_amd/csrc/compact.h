// compact.h -- routing-trace compaction for the deduplicating engine, done
// inside the up kernel's workgroups.
//
// "Speculative Decoding for Mixture-of-Experts Models: Expert Bytes, Kernel
// Bandwidth and the Best Draft Length", abstract: a deduplicating engine
// reads each selected expert once per pass, so it needs, per distinct
// expert, the (token, slot) entries that chose it.  The N*k <= 512 routing
// entries are few, so every up-kernel workgroup derives what it needs from
// them directly (no separate launch):
//   local_instance: the u-th distinct valid expert (ascending) and its
//                   entries in slot order, from a 256-bit presence mask and
//                   wave ballots;
//   write_record:   one workgroup also writes the full compaction record for
//                   the down kernel and the caller (counts, offsets, unique
//                   list, grouped slot list, U).
// Both are deterministic: masks are built with order-independent bit ORs and
// counts with integer adds, and list order is slot order.
#pragma once

#include "kernels.h"

namespace moe {

// The u-th distinct valid expert of the routing entries idx[0 .. slots) in
// ascending order, or -1 when there are at most u of them.  The entries are
// slots slot0 .. slot0+slots-1 of the pass (a group of whole tokens; slot0
// is a multiple of k); the expert's entries (slot s = t*k + j, in
// increasing s) go to ent_row[] (s) and ent_tok[] (s / k), their number to
// *m, and the number of distinct valid experts (U) to *n_distinct.  All
// threads of the workgroup call it (it contains barriers) and get the same
// results.  slots <= 2 * blockDim.x.
template <class Row, class Tok>
__device__ inline int local_instance(const int32_t *__restrict__ idx, int slots, int slot0,
                                     int E, int k, int u, Row *ent_row, Tok *ent_tok, int *m,
                                     int *n_distinct) {
  constexpr int kWords = MOE_MAX_EXPERTS / 32;
  constexpr int kMaxWaves = 16;
  __shared__ uint32_t pres[kWords];
  __shared__ int wcnt[2][kMaxWaves];
  __shared__ int s_e, s_u;
  const int tid = threadIdx.x;
  const int nth = blockDim.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nw = nth >> 6;

  if (tid < kWords) pres[tid] = 0u;
  int es[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int s = p * nth + tid;
    const int v = s < slots ? idx[s] : -1;
    es[p] = (v >= 0 && v < E) ? v : -1;
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 2; ++p)
    if (es[p] >= 0) atomicOr(&pres[es[p] >> 5], 1u << (es[p] & 31));
  __syncthreads();
  if (tid == 0) {
    int e = -1, left = u, all = 0;
    for (int w = 0; w < kWords; ++w) {
      uint32_t bits = pres[w];
      const int c = __popc(bits);
      all += c;
      if (e >= 0) continue;
      if (left < c) {
        for (int i = 0; i < left; ++i) bits &= bits - 1u;  // drop the lowest bits
        e = w * 32 + __ffs(bits) - 1;
      } else {
        left -= c;
      }
    }
    s_e = e;
    s_u = all;
  }
  __syncthreads();
  const int e = s_e;
  *n_distinct = s_u;
  if (e < 0) return -1;

  // entries of e in slot order: per pass, a wave's matches are counted with
  // a ballot and placed after the matches of earlier waves and passes
  uint64_t bal[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    bal[p] = __ballot(es[p] == e);
    if (lane == 0) wcnt[p][wave] = __popcll(bal[p]);
  }
  __syncthreads();
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int base = 0, total = 0;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    int before = 0, all = 0;
    for (int w = 0; w < nw; ++w) {
      before += (w < wave) ? wcnt[p][w] : 0;
      all += wcnt[p][w];
    }
    if (es[p] == e) {
      const int pos = base + before + __popcll(bal[p] & below);
      const int s = slot0 + p * nth + tid;
      ent_row[pos] = (Row)s;
      ent_tok[pos] = (Tok)(s / k);
    }
    base += all;
    total += all;
  }
  *m = total;
  __syncthreads();
  return e;
}

// The full compaction record of the routing entries idx[0 .. slots), which
// are slots slot0 .. slot0+slots-1 of the pass (layout CompactLayout,
// documented in moe_verify.h; the list holds pass slot ids), and U to
// *n_unique (if given).  Called by one workgroup of at least E threads;
// scratch is record_lds_ints(E, slots) ints of LDS that the caller does not
// use meanwhile.  Everything is parallel over experts or slots: offsets and
// the distinct list come from one workgroup-wide exclusive scan of (count,
// present), and a slot's place among its expert's slots is the number of
// set bits below it in that expert's slot mask.
__device__ inline void write_record(const int32_t *__restrict__ idx, int slots, int slot0,
                                    int E, int32_t *__restrict__ cmp,
                                    int32_t *__restrict__ n_unique, int *scratch) {
  constexpr int kMaxWaves = 16;
  __shared__ int wsum[kMaxWaves];
  const CompactLayout L{E, slots};
  const int words = (slots + 31) >> 5;
  int *cnt = scratch;                                // [E] counts, then offsets
  int *ev = cnt + E;                                 // [slots] expert of each slot (-1: none)
  uint32_t *mask = (uint32_t *)(ev + slots);         // [E][words] each expert's slots
  const int tid = threadIdx.x;
  const int nth = blockDim.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  for (int e = tid; e < E; e += nth) cnt[e] = 0;
  for (int i = tid; i < E * words; i += nth) mask[i] = 0u;
  for (int s = tid; s < slots; s += nth) {
    const int v = idx[s];
    ev[s] = (v >= 0 && v < E) ? v : -1;
  }
  __syncthreads();
  for (int s = tid; s < slots; s += nth) {
    const int e = ev[s];
    if (e < 0) continue;
    atomicAdd(&cnt[e], 1);
    atomicOr(&mask[e * words + (s >> 5)], 1u << (s & 31));
  }
  __syncthreads();
  // exclusive scan over experts (thread e holds expert e) of count | present
  // << 16; the counts sum to at most MOE_MAX_SLOTS, so the halves stay apart
  const int c = tid < E ? cnt[tid] : 0;
  const int mine = c | ((c > 0 ? 1 : 0) << 16);
  int v = mine;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  if (lane == kWave - 1) wsum[wave] = v;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < (nth >> 6); ++w) {
    before += (w < wave) ? wsum[w] : 0;
    all += wsum[w];
  }
  const int excl = before + v - mine;
  const int up = all >> 16;
  if (tid < E) {
    const int off = excl & 0xffff;
    cnt[tid] = off;  // only this thread read cnt[tid]
    cmp[L.counts() + tid] = c;
    cmp[L.offs() + tid] = off;
    if (c > 0) cmp[L.uniq() + (excl >> 16)] = tid;
  }
  for (int q = up + tid; q < E; q += nth) cmp[L.uniq() + q] = -1;
  if (tid == 0) {
    cmp[L.offs() + E] = all & 0xffff;
    cmp[L.u()] = up;
    if (n_unique) *n_unique = up;
  }
  __syncthreads();
  // a slot's place in its expert's list: its expert's slots below it
  for (int s = tid; s < slots; s += nth) {
    const int e = ev[s];
    if (e < 0) continue;
    const uint32_t *me = mask + e * words;
    int rank = __popc(me[s >> 5] & ((1u << (s & 31)) - 1u));
    for (int w = 0; w < (s >> 5); ++w) rank += __popc(me[w]);
    cmp[L.list() + cnt[e] + rank] = slot0 + s;
  }
  __syncthreads();  // scratch is free again
}

}  // namespace moe
