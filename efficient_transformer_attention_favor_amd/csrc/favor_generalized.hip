// Kernelised attention with a feature map other than softmax's (the favor_attn_fwd_generalized
// entry point).
//
// "Rethinking Attention with Performers" (review page), section "ABSTRACT": FAVOR+ can also
// model kernelisable attention mechanisms beyond softmax.  The same linear-order evaluation
// D^-1 A V, A = phi(Q) phi(K)^T ("KDEformer" review page, "提出的方法" for D^-1 A V), holds
// for any non-negative feature map; here phi(x) = ReLU(W x) / sqrt(m) (FAVOR_FEATURE_RELU),
// whose kernel is the first-order arc-cosine kernel.  Without an exponential there is no
// stabiliser, and a row whose weights are all zero (every feature of its query, or of its
// keys, zero) gets a zero output.
//
// Implementation: the softmax forward's kernels in their ReLU mode, so the features stay on
// chip (bf16 problems: fp16 W contraction, bf16 features and products, float32
// accumulation).  Bidirectional: S = phi(K)^T [V, 1] per position range, then out =
// phi(Q) S_v / phi(Q) S_1.  Causal: the segment summaries, their exclusive prefix, and the
// chunk kernel's 32-position blocks (carry plus masked intra-block product).
#include <hip/hip_runtime.h>

#include "favor_ops.hpp"
#include "favor_plan.hpp"

namespace favor {
namespace {

favor_status gen_plan(const favor_problem* p, int32_t fn, Plan* s) {
  if (p == nullptr) return FAVOR_ERR_INVALID_ARG;
  const favor_status st = make_plan(p, s);
  if (st != FAVOR_OK) return st;
  return fn == FAVOR_FEATURE_RELU ? FAVOR_OK : FAVOR_ERR_UNSUPPORTED;
}

}  // namespace
}  // namespace favor

extern "C" size_t favor_generalized_workspace_bytes(const favor_problem* p, int32_t fn) {
  favor::Plan s;
  if (favor::gen_plan(p, fn, &s) != FAVOR_OK) return 0;
  return favor::relu_workspace_bytes(s);
}

extern "C" favor_status favor_attn_fwd_generalized(const favor_problem* p, int32_t fn, const void* Q, const void* K,
                                                   const void* V, const float* W, void* out, void* workspace,
                                                   size_t workspace_bytes, void* stream) {
  favor::Plan s;
  const favor_status st = favor::gen_plan(p, fn, &s);
  if (st != FAVOR_OK) return st;
  if (Q == nullptr || K == nullptr || V == nullptr || W == nullptr || out == nullptr) return FAVOR_ERR_INVALID_ARG;
  if (workspace == nullptr || workspace_bytes < favor::relu_workspace_bytes(s) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return FAVOR_ERR_WORKSPACE;
  return favor::launch_relu_attention(s, Q, K, V, W, out, static_cast<char*>(workspace),
                                      static_cast<hipStream_t>(stream));
}
