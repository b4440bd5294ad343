// Host-side problem validation, launch geometry and workspace layout.  No HIP calls.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/favor.h"

namespace favor {

constexpr int kWave = 64;          // wavefront width on CDNA
constexpr int kTile = 32;          // MFMA tile edge (32x32 accumulators)
constexpr int kFeatPerWave = 64;   // features owned by one wave in the key-side kernels
constexpr int kKeyTarget = 256;     // key-side workgroups a pass aims for (4 waves each, 8 for bf16 d = 64)
constexpr int kCUs = 256;           // compute units of the MI355X (launch-geometry model only)
constexpr int kSegGroup = 4;        // causal segments per key-side workgroup in the cost model
constexpr long long kSumUnitBytes = 12LL << 20;  // summary traffic worth one block step (causal cost model)
constexpr int kReadoutTarget = 256; // readout workgroups a pass aims for
constexpr int kSmallKeyTarget = 512;  // float32 key-side workgroups (one 32-feature tile each)
constexpr int kSmallRanges = 4;       // float32 position ranges per kv head at most
// Ready-to-copy LDS images for the bf16 bidirectional readout (one position range per kv
// head): fp16 W rows of d+8, bf16 S'^T rows of kImgMP+8 (d+2 rows: values, ones, zeros),
// and two 16-byte bias operands per feature.  Sizes are whole 1 KB blocks (LDS DMA unit).
constexpr int kImgMP = 256;
#if defined(__HIP__)
#define FAVOR_HD __host__ __device__
#else
#define FAVOR_HD
#endif
FAVOR_HD constexpr size_t img_w_bytes(int d, int m) { return (size_t)m * (d + 8) * 2; }
FAVOR_HD constexpr size_t img_s_bytes(int d) { return (((size_t)(d + 2) * (kImgMP + 8) * 2) + 1023) & ~size_t(1023); }
FAVOR_HD constexpr size_t img_cb_bytes(int m) { return (size_t)m * 32; }

struct Plan {
  int B, Hq, Hkv, Hw, L, d, m, dtype, mode, chunk;
  int G;    // query heads per kv head
  int BH;   // batch * heads_kv
  int T;    // position ranges per kv head (bidirectional) or segments (causal)
  int R;    // positions per range / segment (multiple of the chunk)
  int NFT;  // feature tiles: m / 32
  int NDT;  // value-column tiles incl. the ones column: d / 32 + 1
  size_t off_gs;       // [BH][T][d+1][m] range / segment summaries (float)
  size_t off_gc;       // [BH][T][m] their per-feature stabilisers (log2 units)
  size_t off_p;        // [BH][T][d+1][m] exclusive prefixes of the segment summaries (causal)
  size_t off_pc;       // [BH][T][m] per-feature stabilisers of the exclusive prefixes (causal)
  size_t off_wide;     // [B Hq][T] int: segment met a block of widely spread keys (causal)
  size_t off_part;     // [B Hq L][d+4] per-row partials of two feature ranges (causal, d = 128, m > 256)
  bool img;            // bf16 bidirectional, one range per head, m <= kImgMP: LDS images
  size_t off_img_w;    // [Hw] fp16 W images
  size_t off_img_s;    // [BH] bf16 S'^T images
  size_t off_img_cb;   // [BH] bias-operand images
  size_t off_bar;      // one-launch float32 path's grid barrier: epoch word + kCUs arrival flags (64-bit)
  size_t bytes;        // total workspace bytes
};

// Fills *plan from *p; returns FAVOR_OK or the validation error (no HIP calls).
favor_status make_plan(const favor_problem* p, Plan* plan);

}  // namespace favor
