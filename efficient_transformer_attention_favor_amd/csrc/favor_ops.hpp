// Launchers shared between the library's translation units.
#pragma once

#include <hip/hip_runtime.h>

#include "favor_plan.hpp"

namespace favor {

// The feature map of the queries (side 0, row stabilisers) or keys (side 1, one stabiliser
// per (batch, kv head)) as float32 [rows][m], stabilisers in natural-log units in c.  With
// Lo > L each head gets Lo rows of phi (and of c for queries), rows L..Lo-1 written as zero.
favor_status launch_features(const Plan& s, int side, const void* X, const float* W, float* phi, float* c,
                             hipStream_t st, int Lo = 0);

// The ReLU feature map ReLU(W x) / sqrt(m) of the queries (side 0) or keys (side 1) as
// float32 [rows][m], Lo rows per head as above.
favor_status launch_relu_features(const Plan& s, int side, const void* X, const float* W, float* phi,
                                  hipStream_t st, int Lo = 0);

// The key-side range summaries of a bidirectional plan as float32 partials:
// gs [BH][T][d+1][m] (value rows in the permuted order vperm within each 32-column tile, row d
// the ones column) and gc [BH][T][m], the per-feature stabilisers in log2 units, with
// gs = sum over the range's positions of 2^(e - gc) [v, 1], e = log2(e) (w . k - |k|^2 / 2).
favor_status launch_key_summaries(const Plan& s, const void* K, const void* V, const float* W, float* gs,
                                  float* gc, hipStream_t st);

}  // namespace favor
