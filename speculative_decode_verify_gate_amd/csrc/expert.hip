// expert.hip -- SwiGLU expert FFNs over the expert instances of one pass.
//
// An expert instance is one expert's weights applied to a list of tokens:
//   per-slot engine: instance i is routing slot i = t*k + j, one token; the
//                    expert is streamed once per (token, slot);
//   dedup engine:    instance u is the u-th distinct selected expert with all
//                    the (token, slot) entries that chose it; the expert is
//                    streamed once per pass;
//   both engines:    shared expert s is one instance over all N tokens.
// ("Speculative Decoding for Mixture-of-Experts Models: Expert Bytes, Kernel
// Bandwidth and the Best Draft Length", abstract; shared experts: "Deep Dive
// into Mixture of Experts: From 1991 to DeepSeek-V3", section 5.)
//
// Up kernel:   A = rows of W1 and W3 ([f][d]), B = the instance's tokens
//              (fp32 x rounded to bf16), out = bf16(silu(h) * g) per token.
// Down kernel: A = rows of W2 ([d][f]), B = the up kernel's rows, out = fp32
//              per (instance entry) rows of the expert output buffer.
//
// Decode-time MoE is bound by weight bytes (the same page, section 6), so the
// kernels are laid out to stream weights:
//  - a workgroup owns one instance and 64 output rows; each wave owns one
//    16-row MFMA tile and streams those rows over the whole K with 16-byte
//    loads (4 lanes cover 64 contiguous bytes of a row per load), two chunks
//    in flight through register double buffering;
//  - the instance's tokens are the MFMA B operand (16 tokens per tile, up
//    to 4 tiles): staged once per K window in LDS, read with ds_read_b128,
//    never re-read from global per row tile;
//  - the MFMA v_mfma_f32_16x16x32_bf16 (fp32: 16x16x4) sums each output
//    element over K in a fixed step order that does not depend on which
//    other tokens share the tile, so a token gets the same bits whether it
//    is alone (per-slot) or batched with others (dedup).
#include <math.h>

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

// Steps per register chunk: the up kernel streams two matrices.
template <bool UP, int CTMAX>
struct Chunking {
  static constexpr int kSteps = UP ? 8 : (CTMAX == 1 ? 16 : 8);
};

template <bool BF16, bool UP, int CTMAX>
__global__ __launch_bounds__(256) void expert_kernel(ExpertArgs a) {
  using T = WT<BF16>;
  constexpr int SPC = Chunking<UP, CTMAX>::kSteps;
  constexpr int CHUNK = SPC * T::kStep;             // K elements per chunk
  constexpr int EB = T::kBytes;
  constexpr int GROUP = CTMAX * kTile;              // tokens per MFMA pass
  constexpr int ITEM = 16 / EB;                     // elements per 16-byte item

  extern __shared__ __align__(16) unsigned char lds[];  // staged token rows
  __shared__ int ent_row[MOE_MAX_SLOTS];
  __shared__ int ent_tok[MOE_MAX_SLOTS];

  const int R = UP ? a.f : a.d;  // output rows
  const int K = UP ? a.d : a.f;  // reduction length
  const int RG = (R + kRowsPerBlock - 1) / kRowsPerBlock;
  const int inst = blockIdx.x / RG;
  const int rgrp = blockIdx.x - inst * RG;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;
  const int g = lane >> 4;
  const CompactLayout CL{a.E, a.N * a.k};
  const size_t fd = (size_t)a.f * (size_t)a.d;

  // ---- the instance: expert matrices and token entries (uniform per block)
  int m;
  const unsigned char *wA, *wB = nullptr;
  int list_base = 0, shared_s = -1;
  if (inst < a.n_routed) {
    int e;
    if (!a.dedup) {
      e = a.idx[inst];
      if (e < 0 || e >= a.E) return;
      m = 1;
    } else {
      if (inst >= a.cmp[CL.u()]) return;
      e = a.cmp[CL.uniq() + inst];
      m = a.cmp[CL.counts() + e];
      list_base = a.cmp[CL.offs() + e];
    }
    if (UP) {
      wA = (const unsigned char *)a.w13 + (size_t)e * 2 * fd * EB;
      wB = wA + fd * EB;
    } else {
      wA = (const unsigned char *)a.w2 + (size_t)e * fd * EB;
    }
  } else {
    shared_s = inst - a.n_routed;
    if (shared_s >= a.S) return;
    m = a.N;
    if (UP) {
      wA = (const unsigned char *)a.ws13 + (size_t)shared_s * 2 * fd * EB;
      wB = wA + fd * EB;
    } else {
      wA = (const unsigned char *)a.ws2 + (size_t)shared_s * fd * EB;
    }
  }
  for (int c = tid; c < m; c += blockDim.x) {
    int row;
    if (shared_s >= 0)
      row = a.N * a.k + shared_s * a.N + c;
    else
      row = a.dedup ? a.cmp[CL.list() + list_base + c] : inst;
    ent_row[c] = row;
    ent_tok[c] = (shared_s >= 0) ? c : row / a.k;
  }

  const int rt = rgrp * kWavesPerBlock + wave;  // this wave's 16-row tile
  const bool active = rt * kTile < R;
  const int nsteps = K / T::kStep;
  const int nchunks = (nsteps + SPC - 1) / SPC;
  const unsigned char *rowA = wA + (size_t)(rt * kTile + r) * K * EB;
  const unsigned char *rowB = UP ? wB + (size_t)(rt * kTile + r) * K * EB : nullptr;
  const int lane_k = g * T::kPerLane;

  for (int c0 = 0; c0 < m; c0 += GROUP) {
    const int mg = min(m - c0, GROUP);
    // K window staged in LDS: as many whole chunks as fit for mg rows
    int KW = ((a.lds_bytes / (mg * EB)) - kLdsPad) / CHUNK * CHUNK;
    KW = min(KW, nchunks * CHUNK);
    const int cpw = KW / CHUNK;
    const int stride = KW + kLdsPad;  // elements per staged row

    f32x4 acc1[CTMAX], acc3[CTMAX];
#pragma unroll
    for (int ct = 0; ct < CTMAX; ++ct) {
      acc1[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc3[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    u32x4 ra1[SPC], ra3[SPC], rb1[SPC], rb3[SPC];

    auto load_chunk = [&](int ch, u32x4 (&d1)[SPC], u32x4 (&d3)[SPC]) {
#pragma unroll
      for (int s = 0; s < SPC; ++s) {
        if (ch * SPC + s < nsteps) {
          const size_t off = (size_t)(ch * CHUNK + s * T::kStep + lane_k) * EB;
          d1[s] = ldg16(rowA + off);
          if (UP) d3[s] = ldg16(rowB + off);
        }
      }
    };

    auto stage_window = [&](int w) {
      const int k0 = w * KW;
      const int kw = min(KW, K - k0);
      const int items = kw / ITEM;
      for (int it = tid; it < mg * items; it += blockDim.x) {
        const int c = it / items;
        const int q = it - c * items;
        const int kk = k0 + q * ITEM;
        u32x4 v;
        if (UP) {
          const float *src = a.x + (size_t)ent_tok[c0 + c] * K + kk;
          if (BF16) {
            const f32x4 lo = *(const f32x4 *)src;
            const f32x4 hi = *(const f32x4 *)(src + 4);
            bf16x8 b;
            b[0] = (__bf16)lo.x; b[1] = (__bf16)lo.y; b[2] = (__bf16)lo.z; b[3] = (__bf16)lo.w;
            b[4] = (__bf16)hi.x; b[5] = (__bf16)hi.y; b[6] = (__bf16)hi.z; b[7] = (__bf16)hi.w;
            v = __builtin_bit_cast(u32x4, b);
          } else {
            v = *(const u32x4 *)src;
          }
        } else {
          v = ldg16((const unsigned char *)a.abuf + ((size_t)ent_row[c0 + c] * K + kk) * EB);
        }
        *(u32x4 *)(lds + ((size_t)c * stride + q * ITEM) * EB) = v;
      }
    };

    auto compute_chunk = [&](int ch, const u32x4 (&s1)[SPC], const u32x4 (&s3)[SPC]) {
      const int kin = (ch % cpw) * CHUNK;  // offset inside the window
#pragma unroll
      for (int s = 0; s < SPC; ++s) {
        if (ch * SPC + s < nsteps) {
          const int off = kin + s * T::kStep + lane_k;
#pragma unroll
          for (int ct = 0; ct < CTMAX; ++ct) {
            if (ct * kTile < mg) {
              const int col = ct * kTile + r;
              u32x4 b = u32x4{0u, 0u, 0u, 0u};
              if (col < mg) b = *(const u32x4 *)(lds + ((size_t)col * stride + off) * EB);
              acc1[ct] = T::mma(s1[s], b, acc1[ct]);
              if (UP) acc3[ct] = T::mma(s3[s], b, acc3[ct]);
            }
          }
        }
      }
    };

    auto step = [&](int ch, u32x4 (&c1)[SPC], u32x4 (&c3)[SPC], u32x4 (&n1)[SPC],
                    u32x4 (&n3)[SPC]) {
      if (ch % cpw == 0) {
        __syncthreads();  // readers of the previous window are done
        stage_window(ch / cpw);
        __syncthreads();
      }
      if (active && ch + 1 < nchunks) load_chunk(ch + 1, n1, n3);
      if (active) compute_chunk(ch, c1, c3);
    };

    if (active) load_chunk(0, ra1, ra3);
    for (int ch = 0; ch < nchunks; ch += 2) {
      step(ch, ra1, ra3, rb1, rb3);
      if (ch + 1 < nchunks) step(ch + 1, rb1, rb3, ra1, ra3);
    }

    // ---- epilogue: lane holds rows 4g..4g+3 of its tile for token column r
    if (active) {
      const int row0 = rt * kTile + 4 * g;
#pragma unroll
      for (int ct = 0; ct < CTMAX; ++ct) {
        const int col = ct * kTile + r;
        if (ct * kTile < mg && col < mg) {
          const int orow = ent_row[c0 + col];
          if (UP) {
            float act[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float h = acc1[ct][v];
              act[v] = h / (1.0f + expf(-h)) * acc3[ct][v];
            }
            unsigned char *dst = (unsigned char *)a.abuf + ((size_t)orow * a.f + row0) * EB;
            if (BF16) {
              bf16x4 b;
              b[0] = (__bf16)act[0]; b[1] = (__bf16)act[1];
              b[2] = (__bf16)act[2]; b[3] = (__bf16)act[3];
              *(u32x2 *)dst = __builtin_bit_cast(u32x2, b);
            } else {
              *(f32x4 *)dst = f32x4{act[0], act[1], act[2], act[3]};
            }
          } else {
            *(f32x4 *)(a.obuf + (size_t)orow * a.d + row0) = acc1[ct];
          }
        }
      }
    }
    __syncthreads();  // LDS rows are restaged by the next token group
  }
}

template <bool BF16, bool UP>
hipError_t launch_expert(const ExpertArgs &a, hipStream_t st) {
  const int R = UP ? a.f : a.d;
  const int RG = (R + kRowsPerBlock - 1) / kRowsPerBlock;
  const int blocks = (a.n_routed + a.S) * RG;
  if (blocks == 0) return hipSuccess;
  const bool wide = a.N > kTile;
  // allow more than the default 64 KB of dynamic LDS, once per kernel
  static const hipError_t set_wide = hipFuncSetAttribute(
      (const void *)expert_kernel<BF16, UP, 4>, hipFuncAttributeMaxDynamicSharedMemorySize,
      kLdsBudget);
  static const hipError_t set_narrow = hipFuncSetAttribute(
      (const void *)expert_kernel<BF16, UP, 1>, hipFuncAttributeMaxDynamicSharedMemorySize,
      kLdsBudget);
  if (set_wide != hipSuccess) return set_wide;
  if (set_narrow != hipSuccess) return set_narrow;
  if (wide)
    hipLaunchKernelGGL((expert_kernel<BF16, UP, 4>), dim3(blocks), dim3(256), a.lds_bytes, st,
                       a);
  else
    hipLaunchKernelGGL((expert_kernel<BF16, UP, 1>), dim3(blocks), dim3(256), a.lds_bytes, st,
                       a);
  return hipGetLastError();
}

// y[t] = sum_j w[t][j] * o[t*k+j] + sum_s o[N*k + s*N + t], slot order, fp32.
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ obuf,
                                                      const int32_t *__restrict__ idx,
                                                      const float *__restrict__ w, int N, int k,
                                                      int S, int d, int E,
                                                      float *__restrict__ y) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (c >= d) return;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int e = idx[t * k + j];
    if (e < 0 || e >= E) continue;
    const float wt = w[t * k + j];
    const f32x4 o = *(const f32x4 *)(obuf + (size_t)(t * k + j) * d + c);
    acc += wt * o;
  }
  for (int s = 0; s < S; ++s) acc += *(const f32x4 *)(obuf + (size_t)(N * k + s * N + t) * d + c);
  *(f32x4 *)(y + (size_t)t * d + c) = acc;
}

}  // namespace

int expert_lds_bytes(int N, int K, bool bf16, bool up) {
  const int eb = bf16 ? 2 : 4;
  const int ctmax = N > kTile ? 4 : 1;
  const int step = bf16 ? 32 : 16;
  const int spc = up ? 8 : (ctmax == 1 ? 16 : 8);
  const int chunk = spc * step;
  const int kpad = (K + chunk - 1) / chunk * chunk;
  const int rows = ctmax * kTile;
  const size_t whole = (size_t)rows * (kpad + kLdsPad) * eb;
  const size_t least = (size_t)rows * (chunk + kLdsPad) * eb;
  size_t bytes = whole < (size_t)kLdsBudget ? whole : (size_t)kLdsBudget;
  if (bytes < least) bytes = least;
  return (int)bytes;
}

hipError_t launch_up(const ExpertArgs &a, bool bf16, hipStream_t st) {
  return bf16 ? launch_expert<true, true>(a, st) : launch_expert<false, true>(a, st);
}

hipError_t launch_down(const ExpertArgs &a, bool bf16, hipStream_t st) {
  return bf16 ? launch_expert<true, false>(a, st) : launch_expert<false, false>(a, st);
}

hipError_t launch_combine(const float *obuf, const int32_t *idx, const float *w, int N, int k,
                          int S, int d, int E, float *y, hipStream_t st) {
  dim3 grid((d / 4 + 255) / 256, N);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, st, obuf, idx, w, N, k, S, d, E, y);
  return hipGetLastError();
}

}  // namespace moe
