/*
 * moe_verify.h -- C ABI of the MI355X (gfx950) MoE verify-pass library.
 *
 * One sparsely-gated MoE layer evaluated over one speculative-decoding
 * verification pass of N tokens: gate logits, top-k selection, softmax over
 * the k selected logits, SwiGLU expert FFNs combined by those weights, plus
 * always-on shared experts.  Two engines compute the same layer output:
 *   per-slot -- every (token, slot) streams its expert's weights, so a pass
 *               requests N*k expert-sized reads;
 *   dedup    -- every distinct selected expert is streamed once per pass and
 *               applied to all tokens that chose it (U expert-sized reads).
 * Sources: "Deep Dive into Mixture of Experts: From 1991 to DeepSeek-V3",
 * sections 2 (top-k sparse gating) and 5 (shared experts); "Speculative
 * Decoding for Mixture-of-Experts Models: Expert Bytes, Kernel Bandwidth and
 * the Best Draft Length", abstract (per-slot versus deduplicating engines,
 * requested bytes); "Building a Terminal Based LLM Inference Internals
 * Explorer - Part 3: Speculative Decoding", section "The Flow" (one verify
 * pass scores the newest token plus the gamma drafts, so n = gamma + 1).
 *
 * Conventions shared by every call:
 *  - All tensors are dense row-major.  Device pointers are owned by the
 *    caller; the library never allocates, frees or synchronises in these
 *    calls.  Work is enqueued on `stream` (a hipStream_t passed as void*,
 *    NULL = the null stream) and is complete when the stream is.
 *  - Every call returns a moe_status.  Arguments are validated on the host
 *    before anything is enqueued; on an error nothing is enqueued and no
 *    output is written.  A failed launch returns MOE_ERR_HIP.
 *  - Workspace: the device calls take (workspace, workspace_bytes).  With
 *    workspace == NULL the call stores the bytes it needs for this shape and
 *    token count in *workspace_bytes and returns MOE_OK without launching.
 *    Otherwise *workspace_bytes is the size supplied; a smaller size than
 *    needed returns MOE_ERR_WORKSPACE.  A workspace must be 256-byte
 *    aligned and may not be shared by calls that can run concurrently.
 *    The first 256 bytes of every workspace (the head) hold arrival
 *    counters (moe_route, moe_route_biased, moe_stack_pass and
 *    moe_verify_gate count there the workgroups that have finished): they
 *    must be zero before the workspace's first use, and every call leaves
 *    them zero.  No call writes anything else there (data such as the
 *    compaction record starts at byte 256), so one zero fill of the head
 *    serves any later sequence of calls, of any kind and size, on the
 *    same workspace.
 *  - Routing entries passed to the expert passes must lie in [0, E); that
 *    cannot be checked on the host without a copy, so an out-of-range entry
 *    is treated on the device as an empty slot (no weights read, zero
 *    contribution) rather than read out of bounds.
 *  - Limits: 1 <= N <= MOE_MAX_TOKENS, 1 <= k <= min(E, MOE_MAX_TOPK),
 *    N*k <= MOE_MAX_SLOTS, E <= MOE_MAX_EXPERTS, 0 <= S <= MOE_MAX_SHARED,
 *    d_model and d_ff multiples of 32 (so each lane moves whole 16-byte
 *    vectors), violations return MOE_ERR_INVALID_ARG (count limits) or
 *    MOE_ERR_UNSUPPORTED (alignment limits).
 */
#ifndef MOE_VERIFY_H
#define MOE_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status_code {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, count out of range, bad dtype */
  MOE_ERR_UNSUPPORTED = -2, /* well-formed but outside what the kernels do */
  MOE_ERR_WORKSPACE = -3,   /* workspace smaller than required */
  MOE_ERR_HIP = -4          /* a HIP runtime call or launch failed */
};

/* expert weight element type (the gate and activations are always fp32) */
enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 };

#define MOE_MAX_TOKENS 64
#define MOE_MAX_TOPK 16
#define MOE_MAX_SLOTS 512
#define MOE_MAX_EXPERTS 256
#define MOE_MAX_SHARED 4
#define MOE_MAX_GROUPS 64  /* token groups of a grouped dedup pass */
#define MOE_MAX_LAYERS 64  /* layers of one moe_stack_pass call */
#define MOE_MAX_SEQ 64     /* sequences per verification-round call */
#define MOE_MAX_DRAFT 63   /* drafted tokens per sequence and round */
#define MOE_MAX_VOCAB (1 << 24)
/* The logits filter may run as one launch up to these sizes (rows of one
 * call, vocabulary), else as four; both give the same bits. */
#define MOE_FILTER_ONE_LAUNCH_ROWS 128
#define MOE_FILTER_ONE_LAUNCH_VOCAB 262144

/* Engines of moe_stack_pass. */
#define MOE_ENGINE_PERSLOT 0
#define MOE_ENGINE_DEDUP 1

/* Verification-round modes (moe_verify_gate). */
#define MOE_VERIFY_GREEDY 0
#define MOE_VERIFY_SAMPLING 1

typedef struct moe_shape {
  int32_t d_model;   /* d: hidden width */
  int32_t n_experts; /* E: routed experts */
  int32_t top_k;     /* k: experts selected per token */
  int32_t d_ff;      /* f: inner width of every expert */
  int32_t n_shared;  /* S: always-on shared experts (weight 1) */
  int32_t wdtype;    /* moe_dtype of the expert weights */
} moe_shape;

/* Layout of every expert matrix W with R rows and K columns (W1, W3: R = f,
 * K = d; W2: R = d, K = f):
 *   MOE_LAYOUT_ROWS   row-major [R][K].
 *   MOE_LAYOUT_TILED  16-row x STEP-column fragments stored contiguously in
 *                     the order the MFMA consumes them, STEP = 32 for bf16 and
 *                     16 for fp32: fragment (rt, s) occupies the 1024 bytes at
 *                     offset (rt * K/STEP + s) * 1024 of the matrix, and its
 *                     16-byte unit L (0..63) holds W[16 rt + L % 16]
 *                     [STEP s + (L / 16) * STEP/4 .. + STEP/4).  Same size as
 *                     ROWS; moe_pack_weights() converts.  Every weight load of
 *                     the expert kernels is then one contiguous 1 KB block.
 * Each matrix starts where it starts in the row-major arrays below. */
enum moe_layout { MOE_LAYOUT_ROWS = 0, MOE_LAYOUT_TILED = 1 };

/* Expert weights, device pointers, element type wdtype.
 *   w13  [E][2][f][d]  w13[e][0] is W1 (gate projection), w13[e][1] is W3
 *                      (up projection)
 *   w2   [E][d][f]     W2 (down projection)
 *   ws13 [S][2][f][d], ws2 [S][d][f]  shared experts; NULL iff S == 0.
 *   layout             moe_layout of all four arrays.
 * Expert e computes  W2 * (silu(W1 xt) . (W3 xt))  with xt = x rounded to
 * bf16 (nearest-even) and the product rounded to bf16 before W2 when
 * wdtype == MOE_BF16; nothing is rounded for MOE_F32.  Accumulation is fp32. */
typedef struct moe_expert_weights {
  const void *w13;
  const void *w2;
  const void *ws13;
  const void *ws2;
  int32_t layout;
} moe_expert_weights;

/* Convert n_sets expert sets from MOE_LAYOUT_ROWS to MOE_LAYOUT_TILED:
 * w13_rows [n][2][f][d] -> w13_tiled, w2_rows [n][d][f] -> w2_tiled (device
 * pointers, element type wdtype, outputs must not overlap the inputs).
 * Either pair may be NULL to skip it.  Asynchronous on stream; a one-time
 * preparation of resident weights, not part of a pass. */
int moe_pack_weights(const moe_shape *shape, int32_t n_sets, const void *w13_rows,
                     const void *w2_rows, void *w13_tiled, void *w2_tiled, void *stream);

/* Gate + top-k + softmax over the k ("Deep Dive into Mixture of Experts",
 * section 2: logits = x @ gate_weights, top_k of the logits, softmax of the
 * selected values).
 *   gate_w   [E][d] fp32 device (row e scores expert e)
 *   x        [N][d] fp32 device hidden states of the pass
 *   logits   [N][E] fp32 device output, or NULL
 *   topk_idx [N][k] int32 device output: slot j holds the j-th expert in the
 *            order (logit descending, expert index ascending)
 *   topk_w   [N][k] fp32 device output: exp(L_j - L_0) / sum_i exp(L_i - L_0)
 *   margin   [N]    fp32 device output L_(k) - L_(k+1) (+inf if k == E), or
 *            NULL; a small margin marks a near-tie at the selection boundary. */
int moe_route(const moe_shape *shape, const float *gate_w, const float *x,
              int32_t n_tokens, float *logits, int32_t *topk_idx, float *topk_w,
              float *margin, void *workspace, size_t *workspace_bytes, void *stream);

/* moe_route with the per-expert bias of the DeepSeek-style routing sketch
 * ("Deep Dive into Mixture of Experts", section 5: logits = x @ gate_weights
 * + bias, then top_k and softmax of the selected values):
 *   bias [E] fp32 device, added to every token's logits after the gate
 *        product; the selection, the margin, the softmax over the k and the
 *        logits output all take the biased values.  NULL is moe_route.
 * Other arguments, workspace and errors as for moe_route. */
int moe_route_biased(const moe_shape *shape, const float *gate_w, const float *bias,
                     const float *x, int32_t n_tokens, float *logits, int32_t *topk_idx,
                     float *topk_w, float *margin, void *workspace, size_t *workspace_bytes,
                     void *stream);

/* Per-slot expert pass ("Speculative Decoding for Mixture-of-Experts
 * Models", abstract: a per-slot engine reads each selected expert once per
 * token).  Every (token t, slot j) streams expert topk_idx[t][j]; shared
 * experts are streamed once for all tokens.
 *   x        [N][d] fp32 device
 *   topk_idx [N][k] int32 device, topk_w [N][k] fp32 device (any routing,
 *            e.g. the output of moe_route)
 *   y        [N][d] fp32 device output:
 *            y[t] = sum_j topk_w[t][j] * expert_{topk_idx[t][j]}(x_t)
 *                   + sum_s shared_s(x_t), summed in slot order. */
int moe_expert_pass_perslot(const moe_shape *shape, const moe_expert_weights *weights,
                            const float *x, int32_t n_tokens, const int32_t *topk_idx,
                            const float *topk_w, float *y, void *workspace,
                            size_t *workspace_bytes, void *stream);

/* Deduplicating expert pass (same abstract: a deduplicating engine reads each
 * selected expert once per pass).  Same arguments and the same y as the
 * per-slot pass; in addition
 *   n_unique [1] int32 device output (or NULL): U, the number of distinct
 *            valid experts in topk_idx.
 * The workspace holds, from byte 256 on, the routing-trace compaction,
 * int32 each (indices counted from that byte):
 *   [0]                 U
 *   [1 .. E]            counts[e]: slots that chose expert e
 *   [E+1 .. 2E+1]       offs[e]: exclusive prefix sum of counts (E+1 values)
 *   [2E+2 .. 3E+1]      uniq[u]: the experts with counts > 0, ascending,
 *                       then -1 for u >= U
 *   [3E+2 .. 3E+1+N*k]  list: slot ids t*k+j grouped by expert in uniq
 *                       order, ascending within an expert
 * valid once the stream has completed the call. */
int moe_expert_pass_dedup(const moe_shape *shape, const moe_expert_weights *weights,
                          const float *x, int32_t n_tokens, const int32_t *topk_idx,
                          const float *topk_w, float *y, int32_t *n_unique,
                          void *workspace, size_t *workspace_bytes, void *stream);

/* Deduplicating expert pass inside token groups, e.g. the sequences of a
 * batch verified in one pass: each group streams each of its distinct
 * experts once ("Speculative Decoding for Mixture-of-Experts Models",
 * abstract, applied per group), so the pass requests sum_g U_g expert reads,
 * between the union's U and N*k.  Same y as the other passes.
 *   n_groups     G, 1 <= G <= MOE_MAX_GROUPS
 *   group_start  [G+1] int32 HOST array: group g is tokens group_start[g] ..
 *                group_start[g+1]-1; group_start[0] = 0, group_start[G] =
 *                N, strictly increasing (else MOE_ERR_INVALID_ARG).  Read
 *                during the call only.
 *   n_unique     [G] int32 device output (or NULL): U_g per group.
 * The workspace holds, from byte 256 on, G compaction records, record g at
 * byte offset 256 + g * R, R = the 256-byte-aligned size of one record (the layout of
 * moe_expert_pass_dedup's with N*k list entries, of which group g fills its
 * own slots; list entries are slot ids t*k+j of the whole pass).  G = 1 with
 * group_start = {0, N} is moe_expert_pass_dedup; one token per group
 * streams what the per-slot pass streams. */
int moe_expert_pass_dedup_grouped(const moe_shape *shape, const moe_expert_weights *weights,
                                  const float *x, int32_t n_tokens, int32_t n_groups,
                                  const int32_t *group_start, const int32_t *topk_idx,
                                  const float *topk_w, float *y, int32_t *n_unique,
                                  void *workspace, size_t *workspace_bytes, void *stream);

/* A stack of L layers of one shape, each array holding the layers back to
 * back (device pointers):
 *   gate_w [L][E][d] fp32;  bias [L][E] fp32 or NULL (moe_route_biased's
 *   bias per layer);  w13 [L][E][2][f][d], w2 [L][E][d][f], ws13
 *   [L][S][2][f][d], ws2 [L][S][d][f] (NULL iff S == 0), element type
 *   wdtype, all in `layout`. */
typedef struct moe_stack_weights {
  const float *gate_w;
  const float *bias;
  const void *w13;
  const void *w2;
  const void *ws13;
  const void *ws2;
  int32_t layout;
} moe_stack_weights;

/* One verify pass of the same N tokens through every layer of a stack of
 * L independent MoE layers (1 <= L <= MOE_MAX_LAYERS), fused: one routing
 * launch for all L gates, then one up, one down and one combine launch over
 * every layer's expert instances ("Speculative Decoding for Mixture-of-
 * Experts Models", abstract: a pass's step time is its bytes over the
 * kernels' bandwidth plus a fixed time, which the fused launches pay once
 * per stack instead of once per layer).  Layer l computes exactly what
 * moe_route_biased (moe_route when bias is NULL) followed by the chosen
 * engine's expert pass computes on layer l's weights, bit for bit.
 *   x         [N][d] fp32 device, the input of every layer
 *   engine    MOE_ENGINE_PERSLOT or MOE_ENGINE_DEDUP
 *   topk_idx  [L][N][k] int32 device output, topk_w [L][N][k] fp32 output
 *   y         [L][N][d] fp32 device output
 *   n_unique  [L] int32 device output (dedup), or NULL
 * Workspace: the head (arrival counters, as for every call), the routing
 * partials, then the expert-pass buffers; query and errors as for the
 * other calls. */
int moe_stack_pass(const moe_shape *shape, int32_t n_layers, const moe_stack_weights *weights,
                   const float *x, int32_t n_tokens, int32_t engine, int32_t *topk_idx,
                   float *topk_w, float *y, int32_t *n_unique, void *workspace,
                   size_t *workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * moe_stack_pass with the library's own workspace instead of a caller's.
 * The workspace is a static device array of MOE_NOALLOC_SCRATCH_BYTES that
 * every GPU the library runs on holds until the process ends; the call
 * allocates nothing.  Arguments, outputs and results are moe_stack_pass's
 * (bit for bit); a pass whose workspace would exceed the array returns
 * MOE_ERR_WORKSPACE before anything is enqueued (the V2-Lite-shaped stack of
 * 26 layers at 16 tokens needs about 38 MB, one V3-shaped layer at 64
 * tokens about 21 MB).  All calls on one GPU share its array: calls that
 * can overlap on one GPU (other streams, other host threads) race, so the
 * caller serialises them. */
#define MOE_NOALLOC_SCRATCH_BYTES (64 << 20)
int moe_stack_pass_noalloc(const moe_shape *shape, int32_t n_layers,
                           const moe_stack_weights *weights, const float *x, int32_t n_tokens,
                           int32_t engine, int32_t *topk_idx, float *topk_w, float *y,
                           int32_t *n_unique, void *stream);

/* Requested expert bytes of one pass, on the host (same abstract: step time
 * is the bytes each kernel requests over its effective bandwidth).
 * B_e = 3 * d * f * sizeof(weight); perslot = N*k*B_e, dedup = U*B_e,
 * shared = S*B_e, n_unique = U.  topk_idx_host is host memory; an entry
 * outside [0, E) returns MOE_ERR_INVALID_ARG.  Any output pointer may be
 * NULL.  Synchronous, pure, thread-safe. */
int moe_pass_bytes(const moe_shape *shape, const int32_t *topk_idx_host, int32_t n_tokens,
                   uint64_t *perslot_bytes, uint64_t *dedup_bytes, uint64_t *shared_bytes,
                   int32_t *n_unique);

/* moe_pass_bytes of a grouped dedup pass: dedup_bytes = sum_g U_g * B_e and
 * n_unique[g] = U_g (host array of G, or NULL), for the groups of
 * moe_expert_pass_dedup_grouped.  Host memory only; synchronous, pure,
 * thread-safe; an entry outside [0, E) or bad groups return
 * MOE_ERR_INVALID_ARG. */
int moe_pass_bytes_grouped(const moe_shape *shape, const int32_t *topk_idx_host,
                           int32_t n_tokens, int32_t n_groups, const int32_t *group_start,
                           uint64_t *dedup_bytes, int32_t *n_unique);

/* One speculative-decoding verification round for each of n_seq sequences
 * ("Building a Terminal Based LLM Inference Internals Explorer - Part 3:
 * Speculative Decoding", sections "The Accept/Reject Mechanism", "A Worked
 * Example" and "Sampling vs Greedy"): the step after the verify pass.
 *   p_verify     [n_seq][gamma+1][V] fp32 device: the verifier's
 *                distributions at the gamma drafted positions and at the
 *                bonus position, after the caller's temperature / top-p
 *                filtering (the same filtering as the draft's;
 *                moe_verify_probs computes both from the models' logits)
 *   q_draft      [n_seq][gamma][V] fp32 device: the draft's full
 *                distributions (sampling; ignored and may be NULL for greedy)
 *   draft_tokens [n_seq][gamma] int32 device, each in [0, V)
 *   u_accept     [n_seq][gamma] fp32 device uniforms in [0, 1) (sampling)
 *   r_sample     [n_seq] uint32 device uniforms (sampling)
 *   n_accepted   [n_seq] int32 device output: drafted tokens kept (0..gamma)
 *   out_tokens   [n_seq][gamma+1] int32 device output: the kept drafts, then
 *                the verifier's correction (first rejection) or bonus token,
 *                then -1
 * Sampling keeps draft token i when q_i(x_i) > 0 and u_i q_i(x_i) < p_i(x_i)
 * (u_i < min(1, p/q)); at the first rejection it draws from max(0, p_i - q_i)
 * normalised, after a fully kept round from p at the bonus position.  A draw
 * is an inverse CDF over integer weights floor(w * 2^40): the smallest index
 * whose inclusive prefix sum exceeds floor(W r / 2^32), W the weight total;
 * a residual that is zero at that precision draws from p_i instead.  Greedy
 * keeps a draft token when it is the verifier's argmax (ties to the lowest
 * index; -0 and +0 are equal values) and ends with the verifier's argmax;
 * p_verify must hold no NaN in that mode.  Greedy reads nothing of p but
 * each row's argmax, which softmax, temperature and top-p keep, so the
 * verifier's logits may be passed as p_verify directly in that mode.
 * Results are deterministic and exact (no dependence on summation order).
 * Limits: 1 <= n_seq <= MOE_MAX_SEQ, 0 <= gamma <= MOE_MAX_DRAFT,
 * 1 <= V <= MOE_MAX_VOCAB.  A draft token outside [0, V) cannot be checked
 * on the host; the device treats it as rejected (never read).  Workspace as
 * for the other calls (its head holds one arrival counter per sequence). */
int moe_verify_gate(int32_t n_seq, int32_t gamma, int32_t vocab, int32_t mode,
                    const float *p_verify, const float *q_draft, const int32_t *draft_tokens,
                    const float *u_accept, const uint32_t *r_sample, int32_t *n_accepted,
                    int32_t *out_tokens, void *workspace, size_t *workspace_bytes, void *stream);

/* The distributions a verification round compares, from the models'
 * logits ("Building a Terminal Based LLM Inference Internals Explorer -
 * Part 3: Speculative Decoding", sections "The Accept/Reject Mechanism" and
 * "The Flow": softmax of logits / temperature, then top-p filtering, with
 * the same settings for the verifier and the draft):
 *   logits [rows][V] fp32 device (each row with at least one finite logit;
 *          -inf masks a token; logit / temperature must be finite in fp32)
 *   probs  [rows][V] fp32 device output: P = softmax(logits / temperature);
 *          with top_p < 1 only the shortest run of tokens in the order
 *          (P descending, index ascending) whose probability reaches top_p
 *          is kept (the token that reaches it included), renormalised; the
 *          rest are 0.  The kept set is decided on integer masses
 *          floor(P * 2^52) against ceil(top_p * their total), exactly and
 *          independent of summation order.  probs may not overlap logits.
 * 0 < temperature (finite), 0 < top_p <= 1, 1 <= rows, 1 <= V <=
 * MOE_MAX_VOCAB; violations return MOE_ERR_INVALID_ARG (more than 65535
 * rows: MOE_ERR_UNSUPPORTED).  Workspace as for the other calls: after the
 * head come per-row statistics, which each call initialises itself, and a
 * candidate list of up to V 8-byte entries per row, so its size is about
 * twice that of the logits (the head is not used).  With at most
 * MOE_FILTER_ONE_LAUNCH_ROWS rows, V <= MOE_FILTER_ONE_LAUNCH_VOCAB and a
 * grid of rows x ceil(V / 4096) workgroups that the device holds at once
 * (else rows x ceil(V / 8192), two 4096-entry chunks per workgroup), the
 * filter is one launch whose workgroups meet at row barriers (their
 * words in the workspace carry a tag of the call, so nothing is cleared
 * between calls), else four launches; both give the same bits.  The
 * barriers' waits are bounded: should a row's workgroups fail to meet
 * within about a second (not expected: they are dispatched in index order,
 * a row's consecutively), that row's outputs are NaN.
 * Feed the verifier's rows as p_verify and the draft's as q_draft. */
int moe_verify_probs(int32_t rows, int32_t vocab, const float *logits, float temperature,
                     float top_p, float *probs, void *workspace, size_t *workspace_bytes,
                     void *stream);

/* The same filtering for both distributions a round compares, in one
 * sequence of launches ("Building a Terminal Based LLM Inference Internals
 * Explorer - Part 3: Speculative Decoding", section "The Flow": the
 * verifier's and the draft's logits go through the same temperature and
 * top-p settings):
 *   logits_p [rows_p][V] -> probs_p [rows_p][V], and
 *   logits_q [rows_q][V] -> probs_q [rows_q][V], fp32 device,
 * each row exactly as moe_verify_probs computes it (the outputs are bit for
 * bit those of two moe_verify_probs calls).  1 <= rows_p, 1 <= rows_q,
 * rows_p + rows_q <= 65535 (else MOE_ERR_UNSUPPORTED); no output may
 * overlap an input or the other output (the inputs may overlap each
 * other); other arguments and the workspace as for moe_verify_probs, for
 * rows_p + rows_q rows.  Violations return MOE_ERR_INVALID_ARG. */
int moe_verify_probs_pair(int32_t rows_p, const float *logits_p, float *probs_p, int32_t rows_q,
                          const float *logits_q, float *probs_q, int32_t vocab,
                          float temperature, float top_p, void *workspace,
                          size_t *workspace_bytes, void *stream);

/* For tests of the one-launch filter's failure path: the number of polls
 * after which a workgroup waiting at a row barrier of moe_verify_probs /
 * moe_verify_probs_pair gives up and writes NaN over its chunks of the
 * output (0 restores the default, about a second of polling).  A small
 * limit makes workgroups give up while the others are still on their way,
 * so some outputs come out NaN; every call still ends.  Applies to calls
 * made after it, process-wide; the four-launch filter and every other call
 * have no such waits.  Always MOE_OK. */
int moe_filter_spin_limit(uint32_t polls);

/* Human-readable name of a status code (static storage). */
const char *moe_status_string(int status);

/* Per-kernel timing, for measurement.  While enabled, every kernel of a
 * selected kind that the calls above launch is bracketed by a pair of HIP
 * events recorded on the call's stream, and moe_timing_read() adds up the
 * elapsed time per kernel kind.  The events are created without a
 * system-scope fence (they only time), yet each pair still adds some idle
 * time around its kernel, so select only the kinds being measured.
 * Kernel kinds (bit positions of the mask, indices into the arrays): */
enum moe_kernel_kind {
  MOE_K_GATE = 0,    /* gate logits, split over K; when the partial logits of
                        the pass fit 64 KB this launch also does the top-k */
  MOE_K_TOPK = 1,    /* top-k + softmax per token (larger gates only) */
  MOE_K_COMPACT = 2, /* reserved: the dedup up kernel compacts the routing
                        itself, so no launch of this kind is made */
  MOE_K_UP = 3,      /* W1/W3 + SwiGLU over all expert instances */
  MOE_K_DOWN = 4,    /* W2 over all expert instances */
  MOE_K_COMBINE = 5, /* weighted sum in slot order + shared experts */
  MOE_K_VERIFY = 6,  /* verification round (moe_verify_gate) */
  MOE_K_FILTER = 7,  /* softmax + top-p filtering (moe_verify_probs) */
  MOE_K_COUNT = 8
};
/* mask: bit (1 << kind) selects a kernel kind; 0 disables timing.  Not
 * meant for concurrent use from several host threads. */
int moe_timing_enable(int mask);
/* Waits for every recorded event pair, adds their elapsed times to ms[kind],
 * their number to launches[kind] (arrays of MOE_K_COUNT), and clears the
 * record.  Either array may be NULL. */
int moe_timing_read(double *ms, int64_t *launches);

#ifdef __cplusplus
}
#endif

#endif /* MOE_VERIFY_H */
