// Launchers shared between the library's translation units.
#pragma once

#include <hip/hip_runtime.h>

#include "favor_plan.hpp"

namespace favor {

// Records ev[i] (if given) before the i-th kernel of a call and after the last one.
struct Marks {
  hipEvent_t* ev;
  int n;
  bool mark(int i, hipStream_t st) const {
    return ev == nullptr || i >= n || hipEventRecord(ev[i], st) == hipSuccess;
  }
};

// The feature map of the queries (side 0, row stabilisers) or keys (side 1, one stabiliser
// per (batch, kv head)) as float32 [rows][m], stabilisers in natural-log units in c.  With
// Lo > L each head gets Lo rows of phi (and of c for queries), rows L..Lo-1 written as zero.
favor_status launch_features(const Plan& s, int side, const void* X, const float* W, float* phi, float* c,
                             hipStream_t st, int Lo = 0);

// The key-side range summaries of a bidirectional plan as float32 partials:
// gs [BH][T][d+1][m] (value rows in the permuted order vperm within each 32-column tile, row d
// the ones column) and gc [BH][T][m], the per-feature stabilisers in log2 units, with
// gs = sum over the range's positions of 2^(e - gc) [v, 1], e = log2(e) (w . k - |k|^2 / 2).
favor_status launch_key_summaries(const Plan& s, const void* K, const void* V, const float* W, float* gs,
                                  float* gc, hipStream_t st);

// Attention with the ReLU feature map, on the softmax forward's kernels in their ReLU mode:
// bidirectional, the key side's range summaries of ReLU(W k) [v, 1] (no stabilisers), then
// a readout of ReLU(W q) against them; causal, the segment summaries, their exclusive
// prefix and the chunk kernel.  Rows with a zero denominator are written as zeros.
// Workspace: relu_workspace_bytes(s) bytes laid out as the plan's.
size_t relu_workspace_bytes(const Plan& s);
favor_status launch_relu_attention(const Plan& s, const void* Q, const void* K, const void* V, const float* W,
                                   void* out, char* ws, hipStream_t st);

// The causal pass of bf16 problems after the key side has written the segment summaries:
// the exclusive scan with per-feature stabilisers, then the chunked pass (features over the
// waves for d = 64, value columns and feature groups for d = 128) and its repair pass, for
// the shapes causal_v_supported accepts.
bool causal_v_supported(const Plan& s);
favor_status launch_causal_scan_pf(const Plan& s, char* ws, hipStream_t st);
favor_status launch_causal_v(const Plan& s, const void* Q, const void* K, const void* V, const float* W, void* out,
                             char* ws, hipStream_t st);

// Bidirectional float32 forward: the key side per (kv head, range, 32-feature tile), then
// the readout with the feature tiles over the waves (ranges merged in the readout).
// Whether launch_small_f32 runs *s as one launch (key side, grid barrier, readout) on the
// current device.
bool small_f32_fused(const Plan& s);

favor_status launch_small_f32(const Plan& s, const float* Q, const float* K, const float* V, const float* W,
                              float* out, char* ws, hipStream_t st, const Marks& mk);

}  // namespace favor
