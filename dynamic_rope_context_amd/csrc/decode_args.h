// Launch arguments of the decode kernels.
#pragma once

#include "bf_common.h"

namespace bifocal {

// Vector (VALU) split kernel + separate combine: fp32 caches and D = 64.
struct DecodeArgs {
  const void* q;       // [Hq, D]
  const void* K;       // [S, Hkv, D]
  const void* V;       // [S, Hkv, D]
  const float2* tab;   // position table [n][D/2]
  float* part;         // [Hq][nsplit][D + 2] (acc..., m, l) in the base-2 domain
  void* o;             // [Hq, D]
  float* lse;          // [Hq] or null
  int32_t pos, Hq, Hkv, w0, G, nsplit, kps;  // kps: keys per split
  DivMagic gdiv;                             // floor(x / G) without a divide
  float scale_log2;                          // softmax scale * log2(e)
};

// Matrix-core kernel (bf16, D = 128) over a batch of sequences.
constexpr int kDecodeMaxBatch = 64;  // sequences per launch (larger batches are chunked)

struct DecSeq {
  int32_t pos;     // the query's position; keys 0 .. pos
  uint32_t gmul;   // floor(x / G) = (x * gmul) >> gshift, G from pos + 1
  uint32_t gshift;
  int32_t G;
};

// Variants of the attention computed (decode and prefill): the method, continuous
// remote positions x / G (frequency interpolation), or the local window alone.
enum { kVariantBifocal = 0, kVariantInterp = 1, kVariantWindow = 2 };

struct DecodeBatchArgs {
  const void* q;            // [B, Hq, D]
  const void* K;            // [B, S, Hkv, D]
  const void* V;            // [B, S, Hkv, D]
  float* part;              // [B][Hq][nwg][D + 2] (acc..., m, l), base-2 domain
  void* o;                  // [B, Hq, D]
  float* lse;               // [B, Hq] or null
  int64_t seq_stride;       // elements between two sequences' caches (S * Hkv * D)
  double theta;
  int32_t b_base;           // first sequence of this launch
  int32_t nseq;             // sequences in this launch
  int32_t Hq, Hkv, w0;
  int32_t nsplit, nwg;      // waves (splits) per (sequence, KV head); nwg = nsplit / 4
                            // workgroups, nwg <= kDecodeMaxParts
  float scale_log2;         // softmax scale * log2(e)
  int32_t variant;          // kVariant*
  // The workspace's position-table header and the rows the table region holds in this
  // call's layout: the partials sit past them and may overwrite rows a larger earlier
  // table held, so the kernel lowers the header's row count to n_cap (hdr null: the
  // partials are not in a workspace).
  TableHeader* hdr;
  int32_t n_cap;
  DecSeq seq[kDecodeMaxBatch];
};

}  // namespace bifocal
