// verify.h -- launch interface of the verification round (verify.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Vocabulary chunks of one verification round (2048 entries each).
int verify_chunks(int V);

// Workspace: 256 bytes of arrival counters (zero before first use, left
// zero) + n_seq * chunks * (gamma + 1) uint64 partial results.
hipError_t launch_verify(int n_seq, int gamma, int V, int mode, const float *p, const float *q,
                         const int32_t *x, const float *u, const uint32_t *r, int32_t *n_acc,
                         int32_t *out, void *ws, hipStream_t st);

// softmax(logits / temperature) then top-p filtering (rows x V fp32 in and
// out), chunked over the chip through a workspace of filter_ws_bytes(rows_a
// + rows_b, V): rows_a rows of logits_a into probs_a and rows_b (may be 0)
// rows of logits_b into probs_b, with the same settings, in one sequence of
// launches: one when filter_one_launch(rows, V) and the grid fits the device
// at once, else four.
size_t filter_ws_bytes(int rows, int V);
// Polls of a row barrier before a one-launch workgroup gives up and writes
// NaN over its chunks (0: the default, about a second).
void set_filter_spin_limit(unsigned polls);
bool filter_one_launch(int rows, int V);
hipError_t launch_filter(int rows_a, const float *logits_a, float *probs_a, int rows_b,
                         const float *logits_b, float *probs_b, int V, float temperature,
                         float top_p, void *ws, hipStream_t st);

}  // namespace moe
