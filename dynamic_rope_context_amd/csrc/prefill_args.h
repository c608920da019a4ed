// Launch arguments shared by the prefill kernels.
#pragma once

#include "bf_common.h"

namespace bifocal {

constexpr int kMaxSeqPerLaunch = 48;

struct SeqInfo {
  int32_t start;  // first token of the sequence in the packed [T, H, D] tensors
  int32_t len;    // L_b
  int32_t G;      // max(1, ceil(L_b / w_pretrained))
  uint32_t gmul;  // floor(x / G) = (x * gmul) >> gshift for 0 <= x < 2^24
  uint32_t gshift;
  int32_t pad[3];
};

struct PrefillArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* lse;          // [Hq, T] or null
  const float2* tab;   // position table (cos, sin) [n][D/2]
  const int32_t* sel;  // [Hkv][kSelPairs] RoPE pairs given the hi/lo correction
  int32_t T, Hq, Hkv, D, w0, nseq, max_qblocks, pad0;
  float scale;         // softmax scale (natural-log domain)
  float pad1;
  SeqInfo seq[kMaxSeqPerLaunch];
};

}  // namespace bifocal
