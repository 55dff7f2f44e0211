// expert.hip -- SwiGLU expert FFNs over the expert instances of one pass.
//
// An expert instance is one expert's weights applied to a list of tokens:
//   per-slot engine: instance i is routing slot i = t*k + j, one token; the
//                    expert is streamed once per (token, slot);
//   dedup engine:    instance u is the u-th distinct selected expert with all
//                    the (token, slot) entries that chose it; the expert is
//                    streamed once per pass (or once per token group, when
//                    the pass is split into groups such as sequences);
//   both engines:    shared expert s is one instance over all N tokens.
// ("Speculative Decoding for Mixture-of-Experts Models: Expert Bytes, Kernel
// Bandwidth and the Best Draft Length", abstract; shared experts: "Deep Dive
// into Mixture of Experts: From 1991 to DeepSeek-V3", section 5.)
//
// Up kernel:   A = rows of W1 and W3 ([f][d]), B = the instance's tokens
//              (fp32 x rounded to bf16), out = bf16(silu(h) * g) per token.
// Down kernel: A = rows of W2 ([d][f]), B = the up kernel's rows, out = fp32
//              rows of the expert output buffer, one per (instance entry).
//
// Decode-time MoE is bound by weight bytes (the same page, section 6), so the
// kernels are laid out to stream weights:
//  - a workgroup owns one 16-row MFMA tile of one instance; its four waves
//    take the K dimension in 4-step chunks, round-robin, so every workgroup
//    is short (one tile) and there are many of them to balance the chip;
//  - each lane streams 16-byte vectors (4 lanes cover 64 contiguous bytes of
//    a row per load), with the next chunk always in flight (register double
//    buffering in branch-free code, so waits are exact);
//  - the instance's tokens are the MFMA B operand (16 tokens per tile, up to
//    4 tiles), staged once per K window in LDS and read with ds_read_b128;
//  - the four waves' partial sums are added in wave order through LDS, and
//    the MFMA (v_mfma_f32_16x16x32_bf16; fp32: 16x16x4) sums each output over
//    K in a fixed step order that does not depend on which other tokens share
//    the tile, so a token gets the same bits alone (per-slot) or batched with
//    others (dedup).
#include <math.h>

#include "compact.h"
#include "kernels.h"

namespace moe {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <bool BF16>
struct WT;

template <>
struct WT<true> {
  static constexpr int kBytes = 2;
  static constexpr int kStep = 32;    // K per MFMA step: 4 lane groups x 8 elements
  static constexpr int kPerLane = 8;  // one 16-byte vector per lane per step
  __device__ static inline f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

template <>
struct WT<false> {
  static constexpr int kBytes = 4;
  static constexpr int kStep = 16;    // 4 lane groups x 4 elements
  static constexpr int kPerLane = 4;
  __device__ static inline f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    const f32x4 fa = __builtin_bit_cast(f32x4, a);
    const f32x4 fb = __builtin_bit_cast(f32x4, b);
    // element v of every lane group forms the K = 4 slice of MFMA number v
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.x, fb.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.y, fb.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.z, fb.z, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(fa.w, fb.w, c, 0, 0, 0);
    return c;
  }
};

__device__ inline u32x4 ldg16(const unsigned char *p) { return *(const u32x4 *)p; }

// Weights in the tiled layout are read exactly once per use, in contiguous
// 1 KB fragments: nontemporal loads keep them from displacing the staged
// activations and expert rows that are re-read.
__device__ inline u32x4 ldg16_once(const unsigned char *p) {
  return __builtin_nontemporal_load((const u32x4 *)p);
}

constexpr int kBlock = kWavesPerBlock * kWave;    // threads per workgroup
static_assert(kBlock >= MOE_MAX_EXPERTS, "the record writer takes one expert per thread");

// With 16-token tiles (CTMAX == 1) the B operand is not staged in LDS: every
// lane loads its own token column's 16 bytes (8 bf16 or 4 fp32 elements) per
// MFMA step straight from the L2-resident rows -- fp32 x for the up kernel
// (rounded to bf16 in registers for bf16 weights), the up kernel's rows for
// the down kernel -- in the same pipelined stream as the weights, so the
// workgroup never stops for staging.  Wider tiles (N > 16) stage K windows
// of their token rows in LDS.
// Waves per SIMD the register allocation must leave room for: three for the
// up kernel's direct tiles (two weight sets, two B sets, in flight), four
// for the down kernel's; wide tiles are bounded by their staged LDS anyway.
template <bool UP, int CTMAX>
constexpr int kMinWaves = CTMAX == 1 ? (UP ? 3 : 4) : 2;

// Wide down tiles are paired: a workgroup streams two consecutive 16-row
// tiles of W2 against one staged window of its instance's activation rows,
// as the up kernel streams W1 and W3 against one window of tokens, so the
// staging is paid once per 32 output rows.
template <bool UP, int CTMAX>
constexpr bool kPairDown = !UP && CTMAX > 1;
template <bool UP, int CTMAX>
constexpr bool kTwoStreams = UP || kPairDown<UP, CTMAX>;

// Short reductions (SK, down kernel only): with K = d_ff under 32 MFMA
// steps -- one GPU's share of a layer whose experts are split along d_ff
// -- a 16-row tile is a few kilobytes and splitting its K over four waves
// leaves most of them idle.  Then each wave owns two consecutive 16-row
// tiles over the whole of K (the two-stream path), a workgroup covers
// 2 * kWavesPerBlock tiles, and each wave stores its own outputs: every
// output is still summed over K in step order by one wave, the same for a
// token alone or in a tile of 16.
constexpr int kShortKSteps = 32;
template <bool UP, int CTMAX, bool SK>
constexpr int kTilesPerBlock = SK ? 2 * kWavesPerBlock : (kPairDown<UP, CTMAX> ? 2 : 1);

// Kernel variants: the plain engines, dedup within token groups, and a stack
// of layers (all layers' instances in one grid, layer-major).
constexpr int kPlain = 0, kGrouped = 1, kStack = 2;

// One tile (instance bid / RT, row tile bid % RT) of layer `layer` (0
// unless stacked).  In the dedup up kernel, writer >= 0 first writes the
// compaction record of token group `writer` (one workgroup per group).  The
// dedup engine's routed instances also report U, the number of distinct
// experts of the pass (of the token group, when grouped), to *n_distinct.
template <bool BF16, bool UP, int CTMAX, bool TILED, int VAR, bool SK>
__device__ __attribute__((always_inline)) inline void expert_tile(const ExpertArgs &a, int layer,
                                                                  int bid, int writer,
                                                                  int *ent_row, int *ent_tok,
                                                                  int *n_distinct) {
  static_assert(!(UP && SK), "short reductions are the down kernel's");
  constexpr bool DIRECT = CTMAX == 1;
  constexpr bool PAIR = kPairDown<UP, CTMAX> || SK;  // two W2 tiles per wave
  constexpr bool TWO = UP || PAIR;  // a second weight stream (W3, or W2's next tile)
  constexpr int TPB = kTilesPerBlock<UP, CTMAX, SK>;  // 16-row tiles per workgroup
  constexpr int CS = SK ? 1 : kWavesPerBlock;         // a wave's chunk stride
  constexpr int NB = (UP && BF16) ? 2 : 1;  // 16-byte B loads per lane and step
  using T = WT<BF16>;
  constexpr int SPC = kSpc;
  constexpr int NW = kWavesPerBlock;
  constexpr int CHUNK = SPC * T::kStep;             // K elements per chunk
  constexpr int EB = T::kBytes;
  constexpr int GROUP = CTMAX * kTile;              // tokens per MFMA pass
  constexpr int ITEM = 16 / EB;                     // elements per 16-byte item

  extern __shared__ __align__(16) unsigned char lds[];  // staged tokens / partials

  const int R = UP ? a.f : a.d;  // output rows
  const int K = UP ? a.d : a.f;  // reduction length
  const int RT = R / kTile / TPB;  // workgroups per instance
  // A stack runs each layer's grid in turn: its own weights, routing,
  // compaction record, U and buffers; the tokens are shared.  Only the stack
  // instantiation offsets the per-layer arrays.
  const int32_t *idx = a.idx;
  const int32_t *cmp = a.cmp;
  int32_t *cmp_out = a.cmp_out;
  int32_t *n_unique = a.n_unique;
  const unsigned char *w13 = (const unsigned char *)a.w13;
  const unsigned char *w2 = (const unsigned char *)a.w2;
  const unsigned char *ws13 = (const unsigned char *)a.ws13;
  const unsigned char *ws2 = (const unsigned char *)a.ws2;
  unsigned char *abuf = (unsigned char *)a.abuf;
  float *obuf = a.obuf;
  if (VAR == kStack) {
    const size_t rows = (size_t)a.N * (a.k + a.S);
    idx += (size_t)layer * a.N * a.k;
    if (cmp) cmp += (size_t)layer * a.rec_ints;
    if (cmp_out) cmp_out += (size_t)layer * a.rec_ints;
    if (n_unique) n_unique += layer;
    w13 += (size_t)layer * a.lw13;
    w2 += (size_t)layer * a.lw2;
    if (ws13) ws13 += (size_t)layer * a.lws13;
    if (ws2) ws2 += (size_t)layer * a.lws2;
    abuf += (size_t)layer * rows * a.f * EB;
    obuf += (size_t)layer * rows * a.d;
  }
  const int inst = bid / RT;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // this wave's first 16-row tile (SK: two per wave; else the workgroup's)
  const int rt = (bid - inst * RT) * TPB + (SK ? 2 * wave : 0);
  const int r = lane & 15;
  const int g = lane >> 4;
  const CompactLayout CL{a.E, a.N * a.k};
  const size_t fd = (size_t)a.f * (size_t)a.d;

  // ---- the instance's expert: one dependent load before the weight stream.
  // Instances are ordered shared experts first, then routed ones (slot u, or
  // the u-th distinct expert of a token group, groups in order), so the
  // fixed shared work is dispatched first.  The dedup up kernel finds its
  // instance in the routing itself (workgroup g < G also writes group g's
  // compaction record for the down kernel and the caller); the down kernel
  // reads it from that record.
  int e = -1, shared_s = -1, m = 0;
  bool have_entries = false;
  const int32_t *rec = nullptr;  // the instance's compaction record (dedup down)
  // The group tables are read only by the grouped instantiation (dedup ==
  // 2), so the plain engines' prologue has no extra argument loads.
  constexpr bool grouped = VAR == kGrouped;
  int u = inst - a.S;
  if (UP && a.dedup && writer >= 0) {
    const int b = writer;
    const int t0 = grouped ? a.gstart[b] : 0;
    const int t1 = grouped ? a.gstart[b + 1] : a.N;
    write_record(idx + t0 * a.k, (t1 - t0) * a.k, t0 * a.k, a.E,
                 cmp_out + (size_t)b * a.rec_ints, n_unique ? n_unique + b : nullptr,
                 (int *)lds);
  }
  int grp = 0;
  if (grouped && u >= 0) {
    // the group whose instance range holds u (bases ascend; ibase[0] = 0)
    int hi = a.G;
    while (hi - grp > 1) {
      const int mid = (grp + hi) >> 1;
      if (u >= a.ibase[mid]) grp = mid; else hi = mid;
    }
    u -= a.ibase[grp];
  }
  if (inst < a.S) {
    shared_s = inst;
  } else if (UP && a.dedup) {
    const int t0 = grouped ? a.gstart[grp] : 0;
    const int t1 = grouped ? a.gstart[grp + 1] : a.N;
    e = local_instance(idx + t0 * a.k, (t1 - t0) * a.k, t0 * a.k, a.E, a.k, u, ent_row,
                       ent_tok, &m, n_distinct);
    if (e < 0) return;  // past the group's U
    have_entries = true;
  } else {
    // one load either way: the u-th distinct expert of the record, or slot u
    const int32_t *src = idx;
    if (a.dedup) {
      rec = cmp + (grouped ? (size_t)grp * a.rec_ints : 0);
      src = rec + CL.uniq();
      *n_distinct = rec[CL.u()];
    }
    e = src[u];
    if (e < 0 || e >= a.E) return;  // past the group's U (dedup) or an empty slot
  }
  const unsigned char *wA, *wB = nullptr;
  {
    const unsigned char *base13 = shared_s < 0 ? w13 : ws13;
    const unsigned char *base2 = shared_s < 0 ? w2 : ws2;
    const size_t ex = (size_t)(shared_s < 0 ? e : shared_s);
    if (UP) {
      wA = base13 + ex * 2 * fd * EB;
      wB = wA + fd * EB;
    } else {
      wA = base2 + ex * fd * EB;
      wB = wA;  // paired: the next 16-row tile of the same W2
    }
  }
  const int nsteps = K / T::kStep;
  const int nchunks = (nsteps + SPC - 1) / SPC;
  const int lane_k = g * T::kPerLane;
  // Where this lane's 16 bytes of step `step` start.  Row-major: row
  // 16 rt + r, columns kStep*step + lane_k.  Tiled: fragment (rt, step) is
  // 1 KB and the lane's unit is its lane index (the layout stores exactly the
  // MFMA A-operand order), so a wave's load is one contiguous kilobyte.
  const unsigned char *rowA, *rowB = nullptr;
  const int rtB = PAIR ? rt + 1 : rt;  // the second stream's tile
  if (TILED) {
    rowA = wA + ((size_t)rt * nsteps * kWave + lane) * 16;
    if (TWO) rowB = wB + ((size_t)rtB * nsteps * kWave + lane) * 16;
  } else {
    rowA = wA + ((size_t)(rt * kTile + r) * K + lane_k) * EB;
    if (TWO) rowB = wB + ((size_t)(rtB * kTile + r) * K + lane_k) * EB;
  }
  const size_t step_bytes = TILED ? (size_t)kWave * 16 : (size_t)T::kStep * EB;

  // Issue the 16-byte weight loads of one chunk.  Branch-free on purpose: the
  // compiler can then count outstanding loads exactly and wait only for the
  // chunk being consumed while the next one is in flight.  Steps past the end
  // of K (last chunk only) re-read the last step; compute() ignores them.
  auto issue = [&](int ch, u32x4 (&d1)[SPC], u32x4 (&d3)[SPC]) {
#pragma unroll
    for (int s = 0; s < SPC; ++s) {
      const int step = min(ch * SPC + s, nsteps - 1);
      const size_t off = (size_t)step * step_bytes;
      if (TILED) {
        d1[s] = ldg16_once(rowA + off);
        if (TWO) d3[s] = ldg16_once(rowB + off);
      } else {
        d1[s] = ldg16(rowA + off);
        if (TWO) d3[s] = ldg16(rowB + off);
      }
    }
  };
  // DIRECT: this lane's B operand of one chunk (its token column's row at
  // `bsrc`, NB x 16 bytes per step), same clamping as the weights
  const unsigned char *bsrc = nullptr;
  constexpr int BEB = UP ? 4 : EB;  // bytes per B element in memory (x is fp32)
  auto issue_b = [&](int ch, u32x4 (&db)[SPC][NB]) {
#pragma unroll
    for (int s = 0; s < SPC; ++s) {
      const int step = min(ch * SPC + s, nsteps - 1);
#pragma unroll
      for (int h = 0; h < NB; ++h)
        db[s][h] = ldg16(bsrc + (size_t)step * T::kStep * BEB + h * 16);
    }
  };

  u32x4 ra1[SPC], ra3[SPC], rb1[SPC], rb3[SPC];
  u32x4 rab[SPC][NB], rbb[SPC][NB];  // DIRECT B operands of the two chunk sets
  // the first chunk of this wave leaves before the token lists are read
  // (every window holds at least NW chunks, so chunk `wave` is in window 0)
  const int first = SK ? 0 : wave;
  if (first < nchunks) issue(first, ra1, ra3);

  // ---- token entries of the instance
  if (have_entries) {
    // already placed by local_instance
  } else if (shared_s >= 0) {
    m = a.N;
    for (int c = tid; c < m; c += kBlock) {
      ent_row[c] = a.N * a.k + shared_s * a.N + c;
      ent_tok[c] = c;
    }
  } else if (a.dedup) {
    m = rec[CL.counts() + e];
    const int base = rec[CL.offs() + e];
    for (int c = tid; c < m; c += kBlock) {
      const int row = rec[CL.list() + base + c];
      ent_row[c] = row;
      ent_tok[c] = row / a.k;
    }
  } else {
    m = 1;
    if (tid == 0) {
      ent_row[0] = u;
      ent_tok[0] = u / a.k;
    }
  }
  if (DIRECT) __syncthreads();  // lanes read their columns' entries below

  for (int c0 = 0; c0 < m; c0 += GROUP) {
    const int mg = min(m - c0, GROUP);
    const int n_ct = (mg + kTile - 1) / kTile;
    // K window staged in LDS: a multiple of NW chunks (at least NW); DIRECT
    // stages nothing and takes all of K as one window
    int cpw = DIRECT ? (nchunks + NW - 1) / NW * NW
                     : ((a.lds_bytes / (mg * EB)) - kLdsPad) / CHUNK / NW * NW;
    cpw = max(NW, min(cpw, (nchunks + NW - 1) / NW * NW));
    const int KW = cpw * CHUNK;
    const int stride = KW + kLdsPad;  // elements per staged row

    f32x4 acc1[CTMAX], acc3[CTMAX];
#pragma unroll
    for (int ct = 0; ct < CTMAX; ++ct) {
      acc1[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc3[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // Stage rows [c0, c0+mg) of the B operand for K range [k0, k0+KW).
    // Loads are batched (IB per thread) before any LDS write so a thread has
    // several requests in flight instead of one round trip per item.
    auto stage_window = [&](int k0) {
      constexpr int IB = (UP && BF16) ? 4 : 8;
      const int kw = min(KW, K - k0);
      const int items = kw / ITEM;
      const int total = mg * items;
      for (int base = 0; base < total; base += IB * kBlock) {
        u32x4 v[IB];
#pragma unroll
        for (int u = 0; u < IB; ++u) {
          const int it = min(base + u * kBlock + tid, total - 1);
          const int c = it / items;
          const int kk = k0 + (it - c * items) * ITEM;
          if (UP) {
            const float *src = a.x + (size_t)ent_tok[c0 + c] * K + kk;
            if (BF16) {
              const f32x4 lo = *(const f32x4 *)src;
              const f32x4 hi = *(const f32x4 *)(src + 4);
              bf16x8 b;
              b[0] = (__bf16)lo.x; b[1] = (__bf16)lo.y; b[2] = (__bf16)lo.z; b[3] = (__bf16)lo.w;
              b[4] = (__bf16)hi.x; b[5] = (__bf16)hi.y; b[6] = (__bf16)hi.z; b[7] = (__bf16)hi.w;
              v[u] = __builtin_bit_cast(u32x4, b);
            } else {
              v[u] = *(const u32x4 *)src;
            }
          } else {
            v[u] = ldg16((const unsigned char *)abuf +
                         ((size_t)ent_row[c0 + c] * K + kk) * EB);
          }
        }
#pragma unroll
        for (int u = 0; u < IB; ++u) {
          const int it = base + u * kBlock + tid;
          if (it < total) {
            const int c = it / items;
            const int q = it - c * items;
            *(u32x4 *)(lds + ((size_t)c * stride + q * ITEM) * EB) = v[u];
          }
        }
      }
    };

    // MFMAs of one chunk.  The B fragment of a lane is token column
    // ct*16 + r; columns past the group read a valid row and are zeroed.
    auto compute = [&](int ch, const u32x4 (&s1)[SPC], const u32x4 (&s3)[SPC],
                       const u32x4 (&sb)[SPC][NB]) {
      const int kin = (ch % cpw) * CHUNK;  // offset inside the window
#pragma unroll
      for (int s = 0; s < SPC; ++s) {
        if (ch * SPC + s < nsteps) {
          const int off = kin + s * T::kStep + lane_k;
#pragma unroll
          for (int ct = 0; ct < CTMAX; ++ct) {
            if (ct == 0 || ct < n_ct) {
              const int col = ct * kTile + r;
              const int row = min(col, mg - 1);
              u32x4 b;
              if (DIRECT) {
                if (NB == 2) {
                  // 8 fp32 of x rounded to bf16 (nearest even), as when staged
                  const f32x4 lo = __builtin_bit_cast(f32x4, sb[s][0]);
                  const f32x4 hi = __builtin_bit_cast(f32x4, sb[s][NB - 1]);
                  bf16x8 v;
                  v[0] = (__bf16)lo.x; v[1] = (__bf16)lo.y; v[2] = (__bf16)lo.z; v[3] = (__bf16)lo.w;
                  v[4] = (__bf16)hi.x; v[5] = (__bf16)hi.y; v[6] = (__bf16)hi.z; v[7] = (__bf16)hi.w;
                  b = __builtin_bit_cast(u32x4, v);
                } else {
                  b = sb[s][0];
                }
              } else {
                b = *(const u32x4 *)(lds + ((size_t)row * stride + off) * EB);
              }
              if (col >= mg) b = u32x4{0u, 0u, 0u, 0u};
              acc1[ct] = T::mma(s1[s], b, acc1[ct]);
              if (TWO) acc3[ct] = T::mma(s3[s], b, acc3[ct]);
            }
          }
        }
      }
    };

    if (DIRECT) {
      // this lane's token column: row of the group's entry min(r, mg-1)
      const int ent = c0 + min(r, mg - 1);
      if (UP)
        bsrc = (const unsigned char *)(a.x + (size_t)ent_tok[ent] * K + lane_k);
      else
        bsrc = (const unsigned char *)abuf + ((size_t)ent_row[ent] * K + lane_k) * EB;
    }
    for (int w0 = 0; w0 < nchunks; w0 += cpw) {
      const int w1 = min(w0 + cpw, nchunks);
      int c = w0 + first;  // this wave's chunks: c, c + CS, ... < w1
      if (!(c0 == 0 && w0 == 0) && c < w1) issue(c, ra1, ra3);
      if (DIRECT) {
        if (c < w1) issue_b(c, rab);
      } else {
        __syncthreads();  // readers of the previous window are done
        stage_window(w0 * CHUNK);
        __syncthreads();
      }
      if (c < w1) {
        // steady state: two chunks per iteration, next chunk always in flight
        for (; c + 2 * CS < w1; c += 2 * CS) {
          issue(c + CS, rb1, rb3);
          if (DIRECT) issue_b(c + CS, rbb);
          compute(c, ra1, ra3, rab);
          issue(c + 2 * CS, ra1, ra3);
          if (DIRECT) issue_b(c + 2 * CS, rab);
          compute(c + CS, rb1, rb3, rbb);
        }
        if (c + CS < w1) {
          issue(c + CS, rb1, rb3);
          if (DIRECT) issue_b(c + CS, rbb);
          compute(c, ra1, ra3, rab);
          compute(c + CS, rb1, rb3, rbb);
        } else {
          compute(c, ra1, ra3, rab);
        }
      }
    }

    if (SK) {
      // each wave holds the whole sums of its two tiles: lane rows 4g..4g+3
      // of each, token column r of every token tile
#pragma unroll
      for (int ct = 0; ct < CTMAX; ++ct) {
        const int col = ct * kTile + r;
        if (ct < n_ct && col < mg) {
          float *o = obuf + (size_t)ent_row[c0 + col] * a.d + rt * kTile + 4 * g;
          *(f32x4 *)o = acc1[ct];
          *(f32x4 *)(o + kTile) = acc3[ct];
        }
      }
      if (!DIRECT) __syncthreads();  // the staged rows are read before the next group's
      continue;
    }

    // ---- the four waves' partial sums, added in wave order; wave ct then
    // finishes token tile ct (lane holds rows 4g..4g+3 for token column r)
    __syncthreads();  // every wave is done with the staged rows
    f32x4 *red = (f32x4 *)lds;  // [TWO ? 2 : 1][NW][CTMAX][64]
#pragma unroll
    for (int ct = 0; ct < CTMAX; ++ct) {
      if (ct < n_ct) {
        red[(wave * CTMAX + ct) * kWave + lane] = acc1[ct];
        if (TWO) red[((NW + wave) * CTMAX + ct) * kWave + lane] = acc3[ct];
      }
    }
    __syncthreads();
    if (wave < n_ct) {
      const int ct = wave;
      f32x4 h = red[ct * kWave + lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) h += red[(w * CTMAX + ct) * kWave + lane];
      f32x4 gg = f32x4{0.f, 0.f, 0.f, 0.f};
      if (TWO) {
        gg = red[(NW * CTMAX + ct) * kWave + lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) gg += red[((NW + w) * CTMAX + ct) * kWave + lane];
      }
      const int col = ct * kTile + r;
      if (col < mg) {
        const int orow = ent_row[c0 + col];
        const int row0 = rt * kTile + 4 * g;
        if (UP) {
          float act[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) act[v] = h[v] / (1.0f + expf(-h[v])) * gg[v];
          unsigned char *dst = abuf + ((size_t)orow * a.f + row0) * EB;
          if (BF16) {
            bf16x4 b;
            b[0] = (__bf16)act[0]; b[1] = (__bf16)act[1];
            b[2] = (__bf16)act[2]; b[3] = (__bf16)act[3];
            *(u32x2 *)dst = __builtin_bit_cast(u32x2, b);
          } else {
            *(f32x4 *)dst = f32x4{act[0], act[1], act[2], act[3]};
          }
        } else {
          *(f32x4 *)(obuf + (size_t)orow * a.d + row0) = h;
          if (PAIR) *(f32x4 *)(obuf + (size_t)orow * a.d + row0 + kTile) = gg;
        }
      }
    }
    __syncthreads();  // partials are overwritten by the next token group
  }
}

// The dedup engine's grid is sized for U_max = min(E, N*k) distinct
// experts because U is known only on the device.  With a.fold > 0 the
// routed part (of every layer, when stacked; of every token group, when
// grouped, by the tables fbase / ibase) is folded: workgroup (slot v, row tile rt) runs distinct
// expert v, then v + fold if v + fold < U (fold = ceil(U_max / 2)), so the
// grid holds half the absent instances and, while U <= fold, every
// workgroup runs one tile.  The first tile learns U on the way: from the
// presence mask it builds (up) or from the compaction record (down).
template <bool BF16, bool UP, int CTMAX, bool TILED, int VAR, bool SK>
__global__ __launch_bounds__(256, (kMinWaves<UP, CTMAX>)) void expert_kernel(ExpertArgs a) {
  __shared__ int ent_row[MOE_MAX_SLOTS];
  __shared__ int ent_tok[MOE_MAX_SLOTS];
  // workgroups per instance (paired wide down tiles: half the 16-row tiles;
  // short reductions: an eighth)
  const int RT = (UP ? a.f : a.d) / kTile / kTilesPerBlock<UP, CTMAX, SK>;
  int U = 0;
  if (VAR == kGrouped) {
    // groups fold one by one: group g's routed slots in the grid are
    // fbase[g] .. fbase[g+1]-1, its instances ibase[g] .. ibase[g+1]-1
    const int writer = (int)blockIdx.x < a.G ? (int)blockIdx.x : -1;
    const int slot = blockIdx.x / RT, rt = blockIdx.x - slot * RT;
    if (slot < a.S) {
      expert_tile<BF16, UP, CTMAX, TILED, VAR, SK>(a, 0, blockIdx.x, writer, ent_row, ent_tok, &U);
      return;
    }
    const int v = slot - a.S;
    int g = 0, hi = a.G;  // the group whose grid slots hold v (bases ascend)
    while (hi - g > 1) {
      const int mid = (g + hi) >> 1;
      if (v >= a.fbase[mid]) g = mid; else hi = mid;
    }
    const int vl = v - a.fbase[g];
    const int fg = a.fbase[g + 1] - a.fbase[g], mg = a.ibase[g + 1] - a.ibase[g];
    const int bid = (a.S + a.ibase[g] + vl) * RT + rt;
    expert_tile<BF16, UP, CTMAX, TILED, VAR, SK>(a, 0, bid, writer, ent_row, ent_tok, &U);
    if (fg < mg && vl + fg < U)
      expert_tile<BF16, UP, CTMAX, TILED, VAR, SK>(a, 0, bid + fg * RT, -1, ent_row, ent_tok, &U);
    return;
  }
  const bool folded = a.fold > 0;
  int layer = 0, bid = blockIdx.x;
  if (VAR == kStack) {
    const int bpl = ((folded ? a.fold : a.n_routed) + a.S) * RT;  // workgroups per layer
    layer = bid / bpl;
    bid -= layer * bpl;
  }
  expert_tile<BF16, UP, CTMAX, TILED, VAR, SK>(a, layer, bid, bid == 0 ? 0 : -1, ent_row, ent_tok,
                                           &U);
  if (!folded) return;
  const int slot = bid / RT;
  if (slot < a.S || slot - a.S + a.fold >= U) return;
  expert_tile<BF16, UP, CTMAX, TILED, VAR, SK>(a, layer, bid + a.fold * RT, -1, ent_row, ent_tok, &U);
}

template <bool BF16, bool UP, int CTMAX, bool TILED, int VAR, bool SK>
hipError_t launch_expert_kernel(const ExpertArgs &a, long long blocks, hipStream_t st) {
  // the dynamic-LDS limit of each kernel, once per kernel: the most any
  // shape asks of it (the wide tiles may exceed the default 64 KB)
  static const hipError_t set = hipFuncSetAttribute(
      (const void *)expert_kernel<BF16, UP, CTMAX, TILED, VAR, SK>,
      hipFuncAttributeMaxDynamicSharedMemorySize, expert_lds_bound(CTMAX > 1));
  if (set != hipSuccess) return set;
  hipLaunchKernelGGL((expert_kernel<BF16, UP, CTMAX, TILED, VAR, SK>), dim3((unsigned)blocks),
                     dim3(kBlock), a.lds_bytes, st, a);
  return hipGetLastError();
}

template <bool BF16, bool UP, bool TILED, int VAR>
hipError_t launch_expert_layout(const ExpertArgs &a, hipStream_t st) {
  const int R = UP ? a.f : a.d;
  const int K = UP ? a.d : a.f;
  const int routed = VAR == kGrouped ? a.fbase[a.G] : (a.fold > 0 ? a.fold : a.n_routed);
  const bool wide = a.N > kTile;
  // a short reduction gives every wave two whole tiles (eight per
  // workgroup), when the rows make whole workgroups
  const bool sk = !UP && K / WT<BF16>::kStep < kShortKSteps &&
                  (R / kTile) % (2 * kWavesPerBlock) == 0;
  // else wide down tiles are paired (d is a multiple of 32, so they pair up)
  const int tpb = sk ? 2 * kWavesPerBlock : (!UP && wide ? 2 : 1);
  const long long blocks = (long long)a.L * (routed + a.S) * (R / kTile) / tpb;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.lds_bytes < 0 || a.lds_bytes > expert_lds_bound(wide)) return hipErrorInvalidValue;
  if constexpr (!UP) {
    if (sk)
      return wide ? launch_expert_kernel<BF16, UP, 4, TILED, VAR, true>(a, blocks, st)
                  : launch_expert_kernel<BF16, UP, 1, TILED, VAR, true>(a, blocks, st);
  }
  return wide ? launch_expert_kernel<BF16, UP, 4, TILED, VAR, false>(a, blocks, st)
              : launch_expert_kernel<BF16, UP, 1, TILED, VAR, false>(a, blocks, st);
}

template <bool BF16, bool UP, int VAR>
hipError_t launch_expert_var(const ExpertArgs &a, hipStream_t st) {
  return a.tiled ? launch_expert_layout<BF16, UP, true, VAR>(a, st)
                 : launch_expert_layout<BF16, UP, false, VAR>(a, st);
}

template <bool BF16, bool UP>
hipError_t launch_expert(const ExpertArgs &a, hipStream_t st) {
  if (a.L > 1) return launch_expert_var<BF16, UP, kStack>(a, st);
  if (a.dedup == 2) return launch_expert_var<BF16, UP, kGrouped>(a, st);
  return launch_expert_var<BF16, UP, kPlain>(a, st);
}

// Row-major -> tiled, one thread per 16-byte unit of the output.  Unit u of a
// matrix: fragment u / 64 = (rt, step), lane L = u % 64 -> source row
// 16 rt + L % 16, columns STEP step + (L / 16) STEP/4 (see moe_verify.h).
template <int STEP, int EB>
__global__ __launch_bounds__(256) void pack_kernel(const unsigned char *__restrict__ src,
                                                   unsigned char *__restrict__ dst, int R, int K,
                                                   long long n_mats) {
  const long long units_per_mat = (long long)R * K * EB / 16;
  const long long total = units_per_mat * n_mats;
  const int nsteps = K / STEP;
  for (long long u = (long long)blockIdx.x * blockDim.x + threadIdx.x; u < total;
       u += (long long)gridDim.x * blockDim.x) {
    const long long mat = u / units_per_mat;
    const long long q = u - mat * units_per_mat;
    const long long frag = q / 64;
    const int L = (int)(q - frag * 64);
    const int rt = (int)(frag / nsteps);
    const int step = (int)(frag - (long long)rt * nsteps);
    const int row = rt * kTile + (L % 16);
    const int col = step * STEP + (L / 16) * (STEP / 4);
    const unsigned char *s = src + ((size_t)mat * R * K + (size_t)row * K + col) * EB;
    *(u32x4 *)(dst + (size_t)u * 16) = *(const u32x4 *)s;
  }
}

// y[t] = sum_j w[t][j] * o[t*k+j] + sum_s o[N*k + s*N + t], in slot order,
// fp32.  The rows read do not depend on the routing values, so every load a
// thread needs (its k+S expert rows, the k indices and weights) is issued
// before the first is used: one memory round trip.
// A stack's layers are blockIdx.z, each with its own rows, routing and y.
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ obuf,
                                                      const int32_t *__restrict__ idx,
                                                      const float *__restrict__ w, int N, int k,
                                                      int S, int d, int E,
                                                      float *__restrict__ y) {
  constexpr int J = MOE_MAX_TOPK + MOE_MAX_SHARED;
  const int t = blockIdx.y;
  const size_t layer = blockIdx.z;
  obuf += layer * N * (k + S) * d;
  idx += layer * N * k;
  w += layer * N * k;
  y += layer * N * d;
  const int c = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (c >= d) return;
  f32x4 ov[J];
  int ej[MOE_MAX_TOPK];
  float wj[MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (j < k + S) {
      const int row = (j < k) ? t * k + j : N * k + (j - k) * N + t;
      ov[j] = *(const f32x4 *)(obuf + (size_t)row * d + c);
    }
  }
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    if (j < k) {
      ej[j] = idx[t * k + j];
      wj[j] = w[t * k + j];
    }
  }
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (j < k) {
      if (ej[j] >= 0 && ej[j] < E) acc += wj[j] * ov[j];
    } else if (j < k + S) {
      acc += ov[j];
    }
  }
  *(f32x4 *)(y + (size_t)t * d + c) = acc;
}

}  // namespace

hipError_t launch_up(const ExpertArgs &a, bool bf16, hipStream_t st) {
  return bf16 ? launch_expert<true, true>(a, st) : launch_expert<false, true>(a, st);
}

hipError_t launch_down(const ExpertArgs &a, bool bf16, hipStream_t st) {
  return bf16 ? launch_expert<true, false>(a, st) : launch_expert<false, false>(a, st);
}

hipError_t launch_pack(const void *src, void *dst, int R, int K, long long n_mats, bool bf16,
                       hipStream_t st) {
  const long long units = (long long)R * K * (bf16 ? 2 : 4) / 16 * n_mats;
  if (units == 0) return hipSuccess;
  const long long want = (units + 255) / 256;
  const int blocks = (int)(want < 65536 ? want : 65536);
  if (bf16)
    hipLaunchKernelGGL((pack_kernel<32, 2>), dim3(blocks), dim3(256), 0, st,
                       (const unsigned char *)src, (unsigned char *)dst, R, K, n_mats);
  else
    hipLaunchKernelGGL((pack_kernel<16, 4>), dim3(blocks), dim3(256), 0, st,
                       (const unsigned char *)src, (unsigned char *)dst, R, K, n_mats);
  return hipGetLastError();
}

hipError_t launch_combine(const ExpertArgs &a, hipStream_t st) {
  dim3 grid((a.d / 4 + 255) / 256, a.N, a.L);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, st, a.obuf, a.idx, a.w, a.N, a.k, a.S,
                     a.d, a.E, a.y);
  return hipGetLastError();
}

}  // namespace moe
