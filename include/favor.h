/*
 * favor.h -- C ABI of the MI355X (gfx950) FAVOR+ attention library (libfavor.so).
 *
 * FAVOR+ ("Rethinking Attention with Performers", sections "요약", "ABSTRACT" and
 * "제안 방법") estimates softmax attention softmax(Q K^T) V in linear time and space with
 * positive orthogonal random features:
 *
 *     phi(x) = exp(W x - |x|^2 / 2 - c) / sqrt(m)                 W: m x d feature matrix
 *     out_i  = phi(q_i)^T S_v / phi(q_i)^T S_1,   S = phi(K)^T [V, 1]   (bidirectional)
 *     out_i  = the same with S summed over positions j <= i only            (causal)
 *
 * i.e. the row-normalised D^-1 A_hat V of the implied attention matrix
 * A_hat = phi(Q) phi(K)^T (notation of the KDEformer review, section "提出的方法").
 * The stabiliser c cancels between numerator and denominator: the library picks it per
 * query row (row maximum) and per kv head (global maximum).  No 1/sqrt(d) temperature is
 * applied: callers who want one fold d^-1/4 into Q and K.
 *
 * Head layout ("Fast Transformer Decoding: One Write-Head is All You Need", section
 * "提出的方法"): heads_q query heads share heads_kv key/value heads; query head hq reads
 * kv head hq / (heads_q / heads_kv).  W is per kv head (heads_w == heads_kv) or shared
 * (heads_w == 1).
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers, contiguous, row-major, innermost dimension
 *    last:  Q [batch][heads_q][seq_len][head_dim],  K and V [batch][heads_kv][seq_len][head_dim],
 *    W [heads_w][num_features][head_dim] (float32, host-generated),
 *    out [batch][heads_q][seq_len][head_dim].  Q, K, V and out share `dtype`.
 *  - The caller owns every buffer; the library allocates and frees no device memory.
 *    Scratch space is the caller's `workspace`, at least favor_workspace_bytes() bytes,
 *    256-byte aligned.  Host-side state is limited to a cached compute-unit count per
 *    device and a launch counter (see favor_attn_fwd).
 *  - `stream` is a hipStream_t (NULL = default stream).  Work is queued asynchronously;
 *    no entry point synchronises the host.
 *  - Arguments are checked before any HIP call.  On an error status nothing has been
 *    queued and `out` is untouched.  FAVOR_ERR_HIP reports a failed kernel launch.
 *  - Results are deterministic: the same inputs and problem give bitwise-identical
 *    output (fixed-order reductions, no floating-point atomics).
 *  - Accumulation is float32.  For bf16 problems the exponent W x is contracted in fp16
 *    (W * log2(e) rounded to fp16, the bf16 inputs converted exactly), the features and
 *    the summary in bf16; float32 problems use float32 throughout.
 *  - `out` must not alias Q, K, V, W or the workspace.
 */
#ifndef FAVOR_H
#define FAVOR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FAVOR_ABI_VERSION 1

typedef enum {
  FAVOR_OK = 0,
  FAVOR_ERR_INVALID_ARG = 1,  /* null pointer, non-positive size, bad head layout       */
  FAVOR_ERR_UNSUPPORTED = 2,  /* head_dim, num_features, dtype, mode or chunk not built  */
  FAVOR_ERR_WORKSPACE = 3,    /* workspace smaller than favor_workspace_bytes(), or NULL */
  FAVOR_ERR_HIP = 4           /* a kernel launch failed                                  */
} favor_status;

typedef enum { FAVOR_F32 = 0, FAVOR_BF16 = 1 } favor_dtype;
typedef enum { FAVOR_BIDIRECTIONAL = 0, FAVOR_CAUSAL = 1 } favor_mode;

/* Problem description.  Supported: head_dim in {64, 128}; num_features a multiple of 64
 * in [64, 512]; heads_q % heads_kv == 0; heads_w in {1, heads_kv}; seq_len >= 1;
 * batch * heads_q * seq_len * head_dim < 2^31; one head's seq_len * head_dim elements under
 * 2^31 bytes; batch * heads_q <= 65535 (otherwise
 * FAVOR_ERR_UNSUPPORTED).  chunk (causal only) is the intra-chunk block C of the chunked
 * prefix scan: the positions of one chunk see each other through a masked C x C product
 * tril(phi(Q_c) phi(K_c)^T) [V_c, 1] and the earlier chunks through the carried state
 * S_<c, which is updated once per chunk.  0 (library default, 32) or one of 32, 64, 128,
 * 256; C above 32 is built for bf16 problems with head_dim 64 (and C = 256 for
 * num_features <= 256), other causal problems take 0 or 32 (otherwise
 * FAVOR_ERR_UNSUPPORTED).  The sequence segments that run in parallel are multiples of C.
 * The result does not depend on C beyond rounding.  Ignored for bidirectional problems. */
typedef struct {
  int32_t batch, heads_q, heads_kv, heads_w;
  int32_t seq_len, head_dim, num_features;
  int32_t dtype; /* favor_dtype */
  int32_t mode;  /* favor_mode  */
  int32_t chunk;
} favor_problem;

/* Bytes of workspace favor_attn_fwd needs for *p (0 if *p is invalid). */
size_t favor_workspace_bytes(const favor_problem* p);

/* Kernel slots of one favor_attn_fwd call: the key/value summary per position range (or
 * segment); the prefix scan of the segment summaries (causal; empty for bidirectional
 * problems); the query readout (bidirectional) or chunked causal pass.  A one-launch
 * float32 call fills the first slot only. */
#define FAVOR_FWD_KERNELS 3

/* Number of kernels one favor_attn_fwd call for *p queues on the current device (1, 2, 4
 * or 6; 0 if *p is invalid).  Reads the device's compute-unit count (a HIP query); without
 * a usable device the one-launch path is off and the count says so. */
int32_t favor_attn_fwd_launches(const favor_problem* p);

/* FAVOR+ forward (Performer page, "제안 방법"): out = D^-1 A_hat V in linear order,
 * bidirectional or causal (inclusive mask j <= i) per p->mode.  Queues 2 (bidirectional)
 * or 4 (causal: key-side summaries, their prefix scan, the chunked pass and its repair
 * launch; 6 where d = 128 with m > 256 in bf16 or float32, whose chunked pass and repair
 * run once per feature range) kernels on `stream`.  A float32 bidirectional problem whose
 * key-side units (kv head x position range x 32 features) and 32-row query tiles each
 * number at most the device's compute units runs as ONE kernel: the key side, a grid-wide
 * barrier on a 64-bit word in the workspace (tagged per launch from a host counter, so
 * it needs no clearing), then the readout.  Its wait is bounded; rows of a launch whose
 * barrier gave up (not every workgroup resident, e.g. beside other work holding the
 * compute units) are written as NaN.  Two such calls in flight at once on one device must
 * not share a workspace.  The environment variable FAVOR_BARRIER_POLLS_FOR_TESTS (a test
 * hook, read per call) lowers the barrier's poll limit so that path can be exercised. */
favor_status favor_attn_fwd(const favor_problem* p, const void* Q, const void* K, const void* V,
                            const float* W, void* out, void* workspace, size_t workspace_bytes,
                            void* stream);

/* favor_attn_fwd with timing marks: events[i] (hipEvent_t, created by the caller) is
 * recorded on `stream` before the i-th kernel and events[FAVOR_FWD_KERNELS] after the
 * last, so hipEventElapsedTime(events[i], events[i+1]) is the duration of kernel slot i
 * (an empty slot's two events are recorded back to back).
 * n_events must be at least FAVOR_FWD_KERNELS + 1 (else FAVOR_ERR_INVALID_ARG); a failed
 * event record returns FAVOR_ERR_HIP.  The kernels are the same as favor_attn_fwd's. */
favor_status favor_attn_fwd_timed(const favor_problem* p, const void* Q, const void* K,
                                  const void* V, const float* W, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream, void* const* events,
                                  int32_t n_events);

/* favor_attn_fwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels, with
 * the workspace taken from a device array inside the library instead of the caller's.
 * That array holds FAVOR_NOALLOC_SCRATCH_BYTES (64 MiB) on each device the library runs
 * on, for the life of the process; a problem whose favor_workspace_bytes() exceeds it is
 * rejected with FAVOR_ERR_WORKSPACE (nothing queued).  The entry point allocates nothing:
 * no hipMalloc, hipFree or allocating library call.  Its first call on a device looks up
 * that device's array address (hipGetSymbolAddress, FAVOR_ERR_HIP if that fails).  `stream`
 * must belong to the current device (else FAVOR_ERR_INVALID_ARG); NULL is the current
 * device's default stream.  Every call on a device shares that device's array: calls that
 * overlap on one device (on different streams, or from several host threads without
 * ordering) race and give undefined results; calls ordered on one stream do not.  No part
 * of the array needs to start zeroed.  Other arguments, layouts and errors as for
 * favor_attn_fwd. */
#define FAVOR_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
favor_status favor_attn_fwd_noalloc(const favor_problem* p, const void* Q, const void* K, const void* V,
                                    const float* W, void* out, void* stream);

/* The positive feature map alone (Performer page, "제안 방법"), as a float32 tensor:
 *   side 0 (queries): X = Q, rows = batch*heads_q*seq_len, c per row (the row maximum of
 *                     the exponent), c_out [rows];
 *   side 1 (keys):    X = K, rows = batch*heads_kv*seq_len, one c per (batch, kv head)
 *                     (the maximum over that head), c_out [batch*heads_kv].
 * phi_out [rows][num_features] = exp(W x - |x|^2/2 - c) / sqrt(m), with the natural-log
 * stabiliser c written to c_out.  W of row x is the one its kv head uses; p->mode and
 * p->chunk are ignored.  phi_out and c_out are device pointers owned by the caller
 * (float32, sizes as above).  Queues 1 kernel (side 0) or 4 (side 1) on `stream`;
 * side 1 uses c_out as scratch until its last kernel.  Diagnostic entry point: the
 * attention kernels compute the same features on chip and never write them out. */
favor_status favor_features(const favor_problem* p, int32_t side, const void* X, const float* W,
                            float* phi_out, float* c_out, void* stream);

/* Kernelised attention with another non-negative feature map (Performer page, "ABSTRACT":
 * FAVOR+ also models kernelisable attention beyond softmax): out = D^-1 A V with
 * A = phi(Q) phi(K)^T, the inclusive causal mask in FAVOR_CAUSAL mode, evaluated in linear
 * order like favor_attn_fwd.  fn selects phi:
 *   FAVOR_FEATURE_RELU  phi(x) = ReLU(W x) / sqrt(m)  (the first-order arc-cosine kernel).
 * A row whose weights are all zero gets a zero output.  Arguments, layouts and errors as
 * for favor_attn_fwd (an unknown fn is FAVOR_ERR_UNSUPPORTED, also p->chunk as there); the
 * workspace (favor_generalized_workspace_bytes(p, fn) bytes, 256-byte aligned) holds the
 * float32 range or segment summaries, as favor_attn_fwd's does.  The features stay on chip;
 * the arithmetic is favor_attn_fwd's (bf16 problems: fp16 W contraction, bf16 features and
 * products, float32 accumulation).  Queues 2 (bidirectional) or 3-4 (causal: key side,
 * prefix scan, one or two chunked passes) kernels on `stream`. */
typedef enum { FAVOR_FEATURE_RELU = 1 } favor_feature_fn;
size_t favor_generalized_workspace_bytes(const favor_problem* p, int32_t fn);
favor_status favor_attn_fwd_generalized(const favor_problem* p, int32_t fn, const void* Q, const void* K,
                                        const void* V, const float* W, void* out, void* workspace,
                                        size_t workspace_bytes, void* stream);

/* Random feature matrix drawn on the device from a seed: W [heads_w][num_features][head_dim]
 * float32 (device pointer, caller-owned).  Orthogonal random features (Performer page,
 * "제안 방법": random features with orthogonal rows lower the estimator's variance) when
 * orthogonal = 1: per block of head_dim rows, a standard Gaussian head_dim x head_dim
 * matrix whose rows are orthonormalised by modified Gram-Schmidt in row order (float64)
 * and rescaled by the lengths of the Gaussian rows; rows past num_features in the last
 * block are dropped.  orthogonal = 0: the Gaussian rows themselves (i.i.d. features).
 * The Gaussians come from a counter-based stream that depends on the seed only:
 * Philox4x32-10 (Salmon et al., SC 2011) with key (seed mod 2^32, seed div 2^32) on
 * counter (p mod 2^32, p div 2^32, 0, 0) for the p-th pair, Box-Muller on two 53-bit
 * uniforms taken from the output's 64-bit halves; number e = ((h nblocks + b) d + i) d + j
 * fills head h, block b, row i, column j.  The same seed gives the same W on every device.
 * 1 <= head_dim <= 128 (else FAVOR_ERR_UNSUPPORTED), 1 <= num_features, heads_w <= 65536,
 * orthogonal in {0, 1}, W not null (else FAVOR_ERR_INVALID_ARG).  Queues 1 kernel
 * (heads_w * ceil(num_features / head_dim) workgroups) on `stream`. */
favor_status favor_draw_features(int32_t heads_w, int32_t num_features, int32_t head_dim, uint64_t seed,
                                 int32_t orthogonal, float* W, void* stream);

/* Causal decoding, one new position per (batch, head) per call.
 *
 * The causal mode is a running sum over positions (FAVOR+ in linear order, Performer page,
 * "제안 방법"; the inclusive mask j <= i), so one step of incremental decoding needs only
 * the summary of the positions so far, an m x (d+1) matrix per kv head, instead of the
 * whole key/value history whose reloading bounds incremental decoding (MQA page,
 * "ABSTRACT"; under multi-query heads one summary serves all G query heads of a kv head).
 *
 * State (device memory, caller-owned, favor_decode_state_bytes(p) bytes, 256-byte
 * aligned): float32 S[batch*heads_kv][m][d+1], float32 c[batch*heads_kv][8] and uint32
 * n[batch*heads_kv][8], one c and n per slice s of m/8 features (rows s m/8 .. (s+1) m/8 - 1
 * of S, updated in parallel), with, for feature f of slice s,
 *   S_f = sum_{j so far} 2^(e_j,f - c_s) [v_j, 1],  e_j,f = log2(e) (w_f . k_j - |k_j|^2 / 2),
 * i.e. the summary in log2 units scaled by 2^-c_s, and n_s the number of positions added
 * (the same in every slice).  c_s starts at the first key's largest exponent over the
 * slice's features and only grows (the slice is rescaled when it does).  A zero-filled
 * buffer is the empty state.
 *
 * favor_attn_decode: q [batch][heads_q][d], k and v [batch][heads_kv][d] (the new
 * position), W as for favor_attn_fwd, out [batch][heads_q][d] (device pointers; q, k, v,
 * out in p->dtype).  p->mode must be FAVOR_CAUSAL and p->seq_len 1; p->chunk is ignored.
 * Adds the new position to the state, then writes out = phi(q) S_v / phi(q) S_1 (so the
 * new position attends to itself and to every earlier one).  Queues 2 kernels on
 * `stream`; concurrent calls on one state race.  Errors as for favor_attn_fwd (a null
 * pointer is FAVOR_ERR_INVALID_ARG; nothing is queued on an error). */
size_t favor_decode_state_bytes(const favor_problem* p);

/* Prompt prefill for decoding: writes the state (layout above) that holds the prompt's L =
 * p->seq_len positions, i.e. the state favor_attn_decode would reach after decoding them
 * one by one (up to rounding), with c_s the largest key exponent of the prompt over the
 * features of slice s and n = L.
 * p->mode must be FAVOR_CAUSAL (the state belongs to a causal sequence); the state buffer
 * has favor_decode_state_bytes of the same problem with seq_len 1 and is overwritten
 * whole.  K, V [batch][heads_kv][L][d] and W as for favor_attn_fwd.  The workspace
 * (favor_decode_prefill_workspace_bytes(p) bytes, 256-byte aligned) holds the key side's
 * float32 range partials.  Runs the forward pass's key-side kernel, then one merge kernel
 * per call on `stream`.  Errors as for favor_attn_fwd. */
size_t favor_decode_prefill_workspace_bytes(const favor_problem* p);
favor_status favor_decode_prefill(const favor_problem* p, const void* K, const void* V, const float* W,
                                  float* state, void* workspace, size_t workspace_bytes, void* stream);
favor_status favor_attn_decode(const favor_problem* p, const void* q, const void* k, const void* v,
                               const float* W, float* state, void* out, void* stream);

/* Gradients of FAVOR+ with respect to Q, K and V (W fixed): for an upstream gradient dout
 * of out = favor_attn_fwd(Q, K, V, W) in the problem's mode, the gradients of
 * sum(dout * out).  The pages give no backward pass: it follows from the linear-order
 * definition (Performer page, "제안 방법"; out = D^-1 A_hat V, KDEformer page, "提出的方法")
 * by the chain rule, with the multi-query head map (a kv head's dK and dV sum over its
 * query heads).  Causal problems (inclusive mask j <= i) run over chunks of 64 positions
 * with prefix sums of the key summaries and suffix sums of the query-side ones; p->chunk is
 * validated as for the forward and otherwise ignored.
 * dout, dQ like Q, dK and dV like K (device pointers, p->dtype; float32 arithmetic inside).
 * The workspace (favor_bwd_workspace_bytes(p) bytes, 256-byte aligned, caller-owned) holds
 * the float32 feature matrices phi(Q), phi(K) and their gradients, about
 * 4 m (B Hq L + B Hkv L) floats, and for causal problems also the per-chunk summaries,
 * about 2 (B Hq + B Hkv) (L / 64) m (d+1) floats.  Errors as for favor_attn_fwd.  Queues
 * about 20 kernels (causal: 25 + 2 heads_q / heads_kv) on `stream`. */
size_t favor_bwd_workspace_bytes(const favor_problem* p);
favor_status favor_attn_bwd(const favor_problem* p, const void* Q, const void* K, const void* V,
                            const float* W, const void* dout, void* dQ, void* dK, void* dV,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code; never NULL. */
const char* favor_status_string(favor_status s);

/* FAVOR_ABI_VERSION of the built library. */
int32_t favor_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FAVOR_H */
