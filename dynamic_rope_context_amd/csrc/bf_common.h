// Shared device/host definitions for the bifocal RoPE attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bifocal {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) 16-byte global loads and stores, for data that one call
// reads or writes once, in accesses whose lanes together cover whole cache lines: the
// cache hierarchy does not keep such lines.  On the decode sweep over the cache and on
// rope_apply's in-place pass they take 5-7% off the time.  Stores that cover only part
// of a line stay cached (the L2 merges them; streamed, they reach HBM as partial
// writes).
__device__ __forceinline__ u32x4 ld_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st_stream(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// ---------------------------------------------------------------------------
// Position table kept in the workspace.
//
// tab[p][m] = (cos(p * theta_m), sin(p * theta_m)) for p in [0, n_valid), float32
// values rounded once from float64.  It serves both branches' needs:
//   * standard RoPE at position p,
//   * the correction rotation of the remote branch, R(f(x) - x) = R(-(x - f(x))),
//     read at n = x - f(x) with the sine negated.  Indexing by n rather than by x
//     keeps the table independent of G, so one table serves every sequence of a
//     ragged batch and every decode step (RoPE rotations compose additively; the
//     pages' on-the-fly correction rotation, technical summary section 2).
// ---------------------------------------------------------------------------
struct TableHeader {
  uint64_t magic;      // kTableMagic once a table is complete
  double theta;
  int32_t D;
  int32_t n_valid;     // positions covered
  uint32_t pad[58];
};
static_assert(sizeof(TableHeader) == 256, "header is one 256-byte slot");

constexpr uint64_t kTableMagic = 0x42464f43414c5442ull;  // "BTLACOFB"

// Workspace layout: [header 256 B][table rows 0 .. n_cap-1][per-call records][op scratch].
// The table offset does not depend on the operation, so prefill and decode calls can
// share one workspace and its table; the records (prefill key tiles) and the op scratch
// are carved from the end, and the table takes the room that is left.
struct WsLayout {
  size_t table_off, rec_off, scratch_off, scratch_bytes;
  int32_t n_cap;  // positions the table region can hold
};

constexpr int kDecodeMaxSplits = 512;     // partials per query head (vector decode path)
constexpr int kDecodeMaxParts = 128;      // partials per (sequence, query head), matrix-core path
constexpr int kSelPairs = 4;  // RoPE pairs per KV head given the hi/lo correction
// Per-KV-head record written by the prefill pre-pass: the kSelPairs corrected pairs, then
// the power-of-two exponents e that keep the fp16 operands in range (remote queries of
// the group, remote keys, values: each operand is multiplied by 2^-e before its fp16
// rounding, and the product is scaled back exactly).
constexpr int kSelExpQ = kSelPairs, kSelExpK = kSelPairs + 1, kSelExpV = kSelPairs + 2;
constexpr int kSelStride = 8;
constexpr size_t kKeyTileBytes = 17408;  // one prefill key-tile record (32 keys, D = 128)
constexpr int kKeyTileKeys = 32;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline size_t table_row_bytes(int D) { return (size_t)(D / 2) * 2 * sizeof(float); }

// Op scratch: decode partials (the larger of one sequence's vector path partials and
// nseq sequences' matrix-core partials), or prefill pair maxima + selected pairs.
// fp32 intermediates of the three inclusion-exclusion passes: O_x [T, Hq, D] and
// LSE_x [Hq, T] for x = A, B, C.
inline size_t ie_bytes(int64_t T, int Hq, int D) {
  return 3 * (align_up((size_t)T * Hq * D * sizeof(float), 256) +
              align_up((size_t)Hq * T * sizeof(float), 256));
}
// Prefill pre-pass maxima: per (head, RoPE pair) of Q, K and V.
inline size_t pair_max_bytes(int Hq, int Hkv) {
  return align_up((size_t)(Hq + 2 * Hkv) * 64 * sizeof(uint32_t), 256);
}
inline size_t scratch_bytes(int op, int Hq, int Hkv, int D, int64_t nseq = 1) {
  if (op == 3) op = 1;  // the inclusion-exclusion prefill shares the prefill scratch
  if (op == 2) {
    if (nseq < 1) nseq = 1;
    const size_t vec = (size_t)Hq * kDecodeMaxSplits * (D + 2) * sizeof(float);
    const size_t mfma = (size_t)nseq * Hq * kDecodeMaxParts * (D + 2) * sizeof(float);
    return align_up(vec > mfma ? vec : mfma, 256);
  }
  if (op == 1) {
    return pair_max_bytes(Hq, Hkv) + align_up((size_t)Hkv * kSelStride * sizeof(int32_t), 256);
  }
  return 0;
}

// Key-tile records of a prefill call with `tiles` tiles per KV head.
inline size_t records_bytes(int Hkv, int64_t tiles) {
  return align_up((size_t)Hkv * (size_t)tiles * kKeyTileBytes, 256);
}
// Upper bound of the tiles of any batch of `num_seqs` sequences and `total` tokens.
inline int64_t max_tiles(int64_t total, int64_t num_seqs) {
  return (total + kKeyTileKeys - 1) / kKeyTileKeys + num_seqs;
}

inline WsLayout ws_layout(int op, int Hq, int Hkv, int D, size_t ws_bytes, size_t rec_bytes,
                          int64_t nseq = 1) {
  WsLayout l;
  l.table_off = 256;
  l.scratch_bytes = scratch_bytes(op, Hq, Hkv, D, nseq);
  const size_t ws = ws_bytes / 256 * 256;
  const size_t tail = l.scratch_bytes + rec_bytes;
  l.scratch_off = ws > tail ? ws - l.scratch_bytes : 0;
  l.rec_off = ws > tail ? ws - tail : 0;
  const size_t room = l.rec_off > l.table_off ? l.rec_off - l.table_off : 0;
  const size_t n = room / table_row_bytes(D);
  l.n_cap = n > (size_t)INT32_MAX ? INT32_MAX : (int32_t)n;
  return l;
}

inline size_t ws_bytes_for(int op, int max_len, int64_t total, int64_t num_seqs, int Hq, int Hkv,
                           int D) {
  size_t rec = (op == 1 || op == 3) ? records_bytes(Hkv, max_tiles(total, num_seqs)) : 0;
  if (op == 3) rec += ie_bytes(total, Hq, D);
  return 256 + align_up((size_t)max_len * table_row_bytes(D), 256) + rec +
         scratch_bytes(op, Hq, Hkv, D, op == 2 ? num_seqs : 1);
}

// ---------------------------------------------------------------------------
// Scalar helpers
// ---------------------------------------------------------------------------

// sin and cos of a float64 angle 0 <= a < 2^30: the angle is first reduced to
// [-pi, pi] with a two-part 2*pi (Cody-Waite; the reduction error stays below 1e-11
// for the position ranges used here), so the library routine takes its short path
// instead of the large-argument reduction.
__device__ __forceinline__ void sincos_reduced(double a, double* s, double* c) {
  constexpr double kTwoPiHi = 6.283185307179586;
  constexpr double kTwoPiLo = 2.4492935982947064e-16;
  const double k = rint(a * 0.15915494309189535);
  const double r = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, a));
  sincos(r, s, c);
}
// (cos, sin) of the angle n * theta_m, formed and reduced in float64, rounded once
// to float32 (the values a position-table row holds, for any real position n).
__device__ __forceinline__ float2 angle_cs(double n, double invf) {
  double s, c;
  sincos_reduced(n * invf, &s, &c);
  return make_float2((float)c, (float)s);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// Two floats -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
// One float -> fp16 bits, round to nearest even, through the scalar conversion.  Every
// fp16 operand of the remote branch (main operands and the hi/lo split) goes through
// this one function so that the split always completes the exact hi value the main
// MFMA used; the packed two-value form, when the compiler chose it for some operands
// only, broke that match.
__device__ __forceinline__ uint32_t f16_bits_of(float a) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a);
}
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return f16_bits_of(a) | (f16_bits_of(b) << 16);
}
// 2^x with the hardware instruction (inputs far below -126 flush to 0, which is what a
// softmax weight that small should be).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// theta_m = theta^(-2m/D) and the angle p * theta_m in float64.
__device__ __forceinline__ double inv_freq64(double theta, int m, int D) {
  return pow(theta, -2.0 * (double)m / (double)D);
}

// f(x) = floor(x / G) and n(x) = x - f(x) for x >= 0.
__device__ __forceinline__ int alias_pos(int x, int G) { return x / G; }

// Division by G without a divide: for 0 <= x < 2^24, floor(x / G) =
// (x * M) >> S with S = 24 + ceil(log2 G) and M = ceil(2^S / G).  (x*M/2^S exceeds
// x/G by less than 2^24 / 2^S <= 1/G, which cannot reach the next integer.)
struct DivMagic {
  uint32_t mul;
  uint32_t shift;
};
inline DivMagic div_magic(uint32_t G) {
  uint32_t l = 0;
  while ((1u << l) < G) ++l;
  const uint32_t S = 24 + l;
  const uint64_t M = ((1ull << S) + G - 1) / G;
  return DivMagic{(uint32_t)M, S};
}
__device__ __forceinline__ int alias_fast(int x, DivMagic m) {
  return (int)(((uint64_t)(uint32_t)x * m.mul) >> m.shift);
}
constexpr int kMaxPositions = 1 << 24;  // positions the magic division covers

}  // namespace bifocal
