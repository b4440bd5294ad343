// Host-side problem validation, launch geometry and workspace layout.  No HIP calls.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/favor.h"

namespace favor {

constexpr int kWave = 64;          // wavefront width on CDNA
constexpr int kTile = 32;          // MFMA tile edge (32x32 accumulators)
constexpr int kFeatPerWave = 64;   // features owned by one wave in the key-side kernels
constexpr int kKeyTarget = 256;     // key-side workgroups (4 waves each) a pass aims for
constexpr int kSegmentTarget = 512; // causal chunk-kernel workgroups a pass aims for
constexpr int kReadoutTarget = 256; // readout workgroups a pass aims for

struct Plan {
  int B, Hq, Hkv, Hw, L, d, m, dtype, mode, chunk;
  int G;    // query heads per kv head
  int BH;   // batch * heads_kv
  int T;    // position ranges per kv head (bidirectional) or segments (causal)
  int R;    // positions per range / segment (multiple of the chunk)
  int NFT;  // feature tiles: m / 32
  int NDT;  // value-column tiles incl. the ones column: d / 32 + 1
  size_t tile_elems;   // m * (d + 32): floats of one fragment-native summary
  size_t off_gs;       // [BH][T][d+1][m] range / segment summaries (float)
  size_t off_gc;       // [BH][T][m] their per-feature stabilisers (log2 units)
  size_t off_p;        // [BH][T] exclusive prefixes, fragment-native (causal)
  size_t off_cstar;    // [BH] global stabiliser per kv head (causal)
  size_t bytes;        // total workspace bytes
};

// Fills *plan from *p; returns FAVOR_OK or the validation error (no HIP calls).
favor_status make_plan(const favor_problem* p, Plan* plan);

}  // namespace favor
