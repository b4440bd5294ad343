// Host-side problem validation, launch geometry and workspace layout.  No HIP calls, so
// the argument checks of every entry point run (and are tested) without a GPU.
#include "favor_plan.hpp"

namespace favor {

namespace {

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

}  // namespace

favor_status make_plan(const favor_problem* p, Plan* s) {
  if (p == nullptr || s == nullptr) return FAVOR_ERR_INVALID_ARG;
  if (p->batch < 1 || p->heads_q < 1 || p->heads_kv < 1 || p->heads_w < 1 || p->seq_len < 1 ||
      p->head_dim < 1 || p->num_features < 1)
    return FAVOR_ERR_INVALID_ARG;
  if (p->heads_q % p->heads_kv != 0) return FAVOR_ERR_INVALID_ARG;
  if (p->heads_w != 1 && p->heads_w != p->heads_kv) return FAVOR_ERR_INVALID_ARG;
  if (p->dtype != FAVOR_F32 && p->dtype != FAVOR_BF16) return FAVOR_ERR_UNSUPPORTED;
  if (p->mode != FAVOR_BIDIRECTIONAL && p->mode != FAVOR_CAUSAL) return FAVOR_ERR_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128) return FAVOR_ERR_UNSUPPORTED;
  if (p->num_features % 64 != 0 || p->num_features > 512) return FAVOR_ERR_UNSUPPORTED;
  if (p->chunk != 0 && p->chunk != 32 && p->chunk != 64 && p->chunk != 128 && p->chunk != 256)
    return FAVOR_ERR_UNSUPPORTED;
  // intra-chunk blocks above 32 positions: bf16 with d = 64 only, C = 256 up to m = 256
  if (p->mode == FAVOR_CAUSAL && p->chunk > 32 &&
      (p->dtype != FAVOR_BF16 || p->head_dim != 64 || (p->chunk == 256 && p->num_features > 256)))
    return FAVOR_ERR_UNSUPPORTED;
  const long long elems_q = (long long)p->batch * p->heads_q * p->seq_len * p->head_dim;
  const long long elems_kv = (long long)p->batch * p->heads_kv * p->seq_len * p->head_dim;
  if (elems_q >= (1LL << 31) || elems_kv >= (1LL << 31)) return FAVOR_ERR_UNSUPPORTED;
  // one head's bytes index a buffer descriptor (a signed 32-bit byte count)
  const long long esize = p->dtype == FAVOR_F32 ? 4 : 2;
  if ((long long)p->seq_len * p->head_dim * esize >= (1LL << 31)) return FAVOR_ERR_UNSUPPORTED;
  // (batch, head) pairs index the second grid dimension of several launches
  if ((long long)p->batch * p->heads_q > 65535) return FAVOR_ERR_UNSUPPORTED;

  Plan& q = *s;
  q.B = p->batch;
  q.Hq = p->heads_q;
  q.Hkv = p->heads_kv;
  q.Hw = p->heads_w;
  q.L = p->seq_len;
  q.d = p->head_dim;
  q.m = p->num_features;
  q.dtype = p->dtype;
  q.mode = p->mode;
  q.chunk = p->mode == FAVOR_CAUSAL ? (p->chunk == 0 ? 32 : p->chunk) : 0;
  q.G = q.Hq / q.Hkv;
  q.BH = q.B * q.Hkv;
  q.NFT = q.m / kTile;
  q.NDT = q.d / kTile + 1;

  // Position ranges per kv head.  Bidirectional: about kKeyTarget key-side workgroups
  // (one per range and 64-feature slice), each range at least 128 positions.  Causal:
  // segments (a multiple of the chunk) chosen by the cost model below.  The split depends
  // on the problem only, which keeps the reduction order -- and so the result bits --
  // independent of the device.
  const int nfs = q.m / kFeatPerWave;
  int T, unit;
  if (q.mode == FAVOR_CAUSAL) {
    // Segment count by a cost model in units of one 32-position block step: the chunk
    // kernel runs one workgroup per CU (about twice the time per step of the key side;
    // four times where d = 128 with m > 256 runs it as two launches over feature ranges),
    // the key side one wave per segment and 64-feature slice, taken as one wave per SIMD
    // (bf16 d = 64 runs two), segments in groups of kSegGroup per workgroup.  The segment summaries cross HBM about four
    // times (written by the key side, read and rewritten as prefixes by the scan, read by
    // the chunk kernel); kSumUnitBytes of that traffic count as one unit.  Ties go to fewer
    // segments.
    unit = q.chunk;
    const int max_t = ceil_div(q.L, unit);
    const long long chunk_w = (q.d == 128 && q.m > 256) ? 4 : 2;
    const long long sum_bytes = 4LL * sizeof(float) * (q.d + 1) * q.m * q.BH;  // per segment
    long long best = -1;
    T = 1;
    for (int t = 1; t <= max_t; ++t) {
      const int r = ceil_div(ceil_div(q.L, t), unit) * unit;
      if (ceil_div(q.L, r) != t) continue;  // the same split as a smaller t
      const long long steps = r / kTile;
      const long long chunk_rounds = ceil_div((long long)q.B * q.Hq * t, kCUs);
      const long long key_waves = (long long)q.BH * ceil_div(t, kSegGroup) * kSegGroup * nfs;
      const long long key_rounds = ceil_div(key_waves, 4LL * kCUs);
      const long long cost = (chunk_w * chunk_rounds + key_rounds) * steps + sum_bytes * t / kSumUnitBytes;
      if (best < 0 || cost < best) {
        best = cost;
        T = t;
      }
    }
  } else if (q.dtype == FAVOR_F32) {
    // float32: about kSmallKeyTarget key-side workgroups of one 32-feature tile each, every
    // range at least 4 x 32 positions (one block per wave), and at most kSmallRanges ranges:
    // each range the readout merges costs it about one dependent round of loads
    unit = 4 * kTile;
    T = ceil_div(kSmallKeyTarget, (long long)q.BH * (q.m / kTile));
    const int max_t = ceil_div(q.L, unit);
    if (T > max_t) T = max_t;
    if (T > kSmallRanges) T = kSmallRanges;
  } else {
    unit = 4 * kTile;
    T = (int)((kKeyTarget + (long long)q.BH * nfs / 2) / ((long long)q.BH * nfs));
    const int max_t = ceil_div(q.L, unit);
    if (T > max_t) T = max_t;
  }
  if (T < 1) T = 1;
  q.R = ceil_div(ceil_div(q.L, T), unit) * unit;
  q.T = ceil_div(q.L, q.R);

  size_t off = 0;
  q.off_gs = off;
  off = align256(off + sizeof(float) * (size_t)(q.d + 1) * q.m * q.BH * q.T);
  q.off_gc = off;
  off = align256(off + sizeof(float) * (size_t)q.m * q.BH * q.T);
  q.off_p = off;
  if (q.mode == FAVOR_CAUSAL) off = align256(off + sizeof(float) * (size_t)(q.d + 1) * q.m * q.BH * q.T);
  q.off_pc = off;
  if (q.mode == FAVOR_CAUSAL) off = align256(off + sizeof(float) * (size_t)q.m * q.BH * q.T);
  q.off_wide = off;
  if (q.mode == FAVOR_CAUSAL) off = align256(off + sizeof(int) * (size_t)q.B * q.Hq * q.T);
  q.off_part = off;
  if (q.mode == FAVOR_CAUSAL && q.d == 128 && q.m > 256)
    off = align256(off + sizeof(float) * (size_t)q.B * q.Hq * q.L * (q.d + 4));
  q.img = q.mode == FAVOR_BIDIRECTIONAL && q.dtype == FAVOR_BF16 && q.T == 1 && q.m <= kImgMP;
  q.off_img_w = q.off_img_s = q.off_img_cb = off;
  if (q.img) {
    off = align256(off + img_w_bytes(q.d, q.m) * q.Hw);
    q.off_img_s = off;
    off = align256(off + img_s_bytes(q.d) * q.BH);
    q.off_img_cb = off;
    off = align256(off + img_cb_bytes(q.m) * q.BH);
  }
  q.off_bar = off;
  if (q.dtype == FAVOR_F32 && q.mode == FAVOR_BIDIRECTIONAL) off = align256(off + sizeof(unsigned long long) * (1 + kCUs));
  q.bytes = off;
  return FAVOR_OK;
}

}  // namespace favor
