// Launch arguments shared by the prefill kernels.
#pragma once

#include "bf_common.h"

namespace bifocal {

constexpr int kMaxSeqPerLaunch = 48;

// Key-tile records written once per call by the key preparation pass and copied
// verbatim into LDS by the bf16 prefill kernel.  One record per (KV head, tile of
// kRecKeys keys of one sequence):
//   kr  [kRecKeys][128]  fp16  R(f(j) - j) K_j                 8192 B
//   kc  [kRecKeys][16]   fp16  hi/lo of the selected pairs     1024 B
//   vt  [128][kRecKeys]  fp16  V^T * 2^-e_v                    8192 B
// Keys past the end of the sequence are zero.
constexpr int kRecKeys = 32;
constexpr size_t kRecKr = 8192, kRecKc = 1024, kRecVt = 8192;
constexpr size_t kRecBytes = kRecKr + kRecKc + kRecVt;
static_assert(kRecBytes == kKeyTileBytes && kRecKeys == kKeyTileKeys, "workspace sizing");

struct SeqInfo {
  int32_t start;  // first token of the sequence in the packed [T, H, D] tensors
  int32_t len;    // L_b
  int32_t G;      // max(1, ceil(L_b / w_pretrained))
  uint32_t gmul;  // floor(x / G) = (x * gmul) >> gshift for 0 <= x < 2^24
  uint32_t gshift;
  int32_t tile_base;  // index of the sequence's first key-tile record
  int32_t pad[2];
};

struct PrefillArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* lse;          // [Hq, T] or null
  const float2* tab;   // position table (cos, sin) [n][D/2]
  const int32_t* sel;  // [Hkv][kSelStride]: corrected RoPE pairs, operand exponents
  uint8_t* rec;        // key-tile records [Hkv][tiles_total] (bf16 path)
  double theta;        // RoPE base (angles evaluated in the kernels: continuous positions)
  int32_t T, Hq, Hkv, D, w0, nseq, max_qblocks, tiles_total;
  float scale;         // softmax scale (natural-log domain)
  // Pair set and score rule of the launch: 0 = bifocal (each causal pair by its own
  // rule); the three passes of the inclusion-exclusion form: 1 = remote scores over
  // all causal pairs, 2 = remote scores over the window pairs, 3 = local scores over
  // the window pairs.
  int32_t mode;
  int32_t out_f32;     // O written as float32 (the passes' intermediates) instead of dtype
  // Remote positions: 0 = floor(x / G) (the method), 1 = x / G (continuous: the
  // frequency-interpolation variant of the pages' ablation)
  int32_t interp;
  SeqInfo seq[kMaxSeqPerLaunch];
  // Query blocks of the matrix-core kernel, heaviest first across the launch's sequences
  // and no workgroup without rows: with the sequences sorted by their query-block counts
  // c_0 >= c_1 >= ... (c_n = 0), level k holds the blocks qb in [c_{k+1}, c_k) of the
  // k + 1 longest sequences, qb descending, then sequence.  lvl_start[k] is the index of
  // level k's first (sequence, block) pair, lvl_start[n] the number of pairs; lvl_qb[k] =
  // c_k; lvl_seq[s] the launch-local index of the s-th longest sequence.
  int32_t nlvl;
  int32_t lvl_start[kMaxSeqPerLaunch + 1];
  int32_t lvl_qb[kMaxSeqPerLaunch];
  int32_t lvl_seq[kMaxSeqPerLaunch];
};

}  // namespace bifocal
