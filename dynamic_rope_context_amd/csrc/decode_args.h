// Launch arguments of the decode kernels.
#pragma once

#include "bf_common.h"

namespace bifocal {

struct DecodeArgs {
  const void* q;       // [Hq, D]
  const void* K;       // [S, Hkv, D]
  const void* V;       // [S, Hkv, D]
  const float2* tab;   // position table [n][D/2]
  float* part;         // [Hq][nsplit][D + 2] (acc..., m, l) in the base-2 domain
  void* o;             // [Hq, D]
  float* lse;          // [Hq] or null
  int32_t pos, Hq, Hkv, w0, G, nsplit, kps;  // kps: keys per split
  int32_t npart;                             // partials per query head left for the combine
  DivMagic gdiv;                             // floor(x / G) without a divide
  float scale_log2;                          // softmax scale * log2(e)
};

}  // namespace bifocal
