// Bifocal decode on gfx950 matrix cores: a batch of queries, one per sequence, over
// bf16 standard-RoPE caches, D = 128.
//
// Jet-Long technical summary, "Methodology" section 2 (on-the-fly correction
// rotation): the cache keeps keys with standard RoPE at their exact positions and is
// never rewritten.  A remote key j is scored against R(f(j) - j) K_j, i.e. the stored
// key rotated in fp32 registers by the angles of n = j - f(j), and the query rotated
// once by R(f(pos) - pos); rotations compose additively, so this is RoPE at the
// aliased positions f(x) = floor(x/G) of section 1, with G from the sequence's current
// length pos + 1.  Keys inside the window (pos - j < w0) are scored with the stored
// bytes as they are.
//
// Layout (per wave, 16 keys per block, 16x16 matrix-core shapes):
//   * S = Q K^T with the query heads as MFMA rows and the block's keys as columns
//     (v_mfma_f32_16x16x32): lane (key l, group k) of the B operand holds channels
//     32s + 8k + e of its key, so a channel and its RoPE partner (c + 64) sit in the
//     same lane, steps s and s + 2.
//   * Remote scores need fp32 accuracy (the fp32 rotation is not representable in one
//     16-bit operand): keys and query are split into fp16 hi + lo parts and three
//     MFMAs add hi*hi + hi*lo + lo*hi (the lo*lo term is below fp32 rounding).
//   * Angles: the keys of a block have consecutive n = j - f(j) (steps of 0 or 1), so
//     R(n) = R(n0) R(n - n0) with n - n0 < 16.  Each lane of a wave owns one RoPE pair
//     and evaluates cos/sin(n0 theta_m) in fp64 once per block (rounded once to fp32,
//     the values a precomputed table would hold); the 16 offset rows R(d) are built
//     once per workgroup.  No table is read, so decode needs no table in the workspace.
//   * O^T = V^T P^T (v_mfma_f32_16x16x16_bf16): the block's V rows are transposed
//     through a per-wave LDS tile (pairs of keys packed per 32-bit word), P goes
//     through a small LDS row buffer.
//   * Online softmax in the base-2 domain with a lazy running max per head.
//   * Two waves per SIMD (at most 256 registers each) so that one wave's loads are in
//     flight while the other computes.
// Key blocks are dealt to the waves of a (sequence, KV head) round-robin: at any time
// the waves of the whole grid read one contiguous window of the caches, which keeps
// the DRAM access pattern a sweep.  The four waves of a workgroup merge their states
// in LDS and write one partial (acc[D], m, l) per query head; a second kernel merges
// the partials of each head by their log-sum-exp and writes O and LSE.  (Merging in
// the last workgroup to finish instead puts a chain of uncached round trips at the end
// of the grid, which measured slower than the second launch.)
#include "bf_common.h"
#include "decode_args.h"
#include "mfma_util.h"

namespace bifocal {

namespace dm {
constexpr int D = 128;
constexpr int BK = 16;           // keys per block
constexpr int NWD = 4;           // waves per workgroup (one split each)
constexpr float kLazy = 8.f;     // allowed growth of the running max before a rescale
}  // namespace dm

// fp16 hi/lo of 8 consecutive values, packed as two MFMA operands: hi = RNE(y) by the
// packed conversion, lo = RNE(y - hi) with hi read back from the packed word (the asm
// keeps the compiler from re-deriving hi with separate scalar conversions).
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split8(const float* y, u32x4& hi, u32x4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const f16x2_t hv = {(_Float16)y[2 * e], (_Float16)y[2 * e + 1]};
    uint32_t hb = __builtin_bit_cast(uint32_t, hv);
    asm volatile("" : "+v"(hb));
    const f16x2_t hr = __builtin_bit_cast(f16x2_t, hb);
    const f16x2_t lv = {(_Float16)(y[2 * e] - (float)hr.x), (_Float16)(y[2 * e + 1] - (float)hr.y)};
    h[e] = hb;
    l[e] = __builtin_bit_cast(uint32_t, lv);
  }
  hi = u32x4{h[0], h[1], h[2], h[3]};
  lo = u32x4{l[0], l[1], l[2], l[3]};
}

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4 mfma16_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16k16_bf16(uint2 a, uint2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4_t, a),
                                                   __builtin_bit_cast(bf16x4_t, b), c, 0, 0, 0);
}
// Max / sum over the 16 lanes of a DPP row.
__device__ __forceinline__ float row_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x121, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x122, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xf, 0xf, false)));
  return fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xf, 0xf, false)));
}
__device__ __forceinline__ float row_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x121, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x122, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xf, 0xf, false));
  return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xf, 0xf, false));
}

template <int REP>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
decode_mfma_kernel(DecodeBatchArgs a) {
  using namespace dm;
  // per wave: V^T tile [128 channels][16 keys] (8-byte segments swizzled by row), P^T
  // rows [16 heads][16 keys], standard query rows [8 heads][128] + one zero row, and
  // the angle row R(n0) of the current block (lane = RoPE pair)
  __shared__ __align__(16) uint16_t s_vt[NWD][D * BK];
  __shared__ __align__(16) uint16_t s_p[NWD][16 * BK];
  __shared__ __align__(16) uint16_t s_q[NWD][9 * D];
  __shared__ __align__(16) float2 s_row[NWD][64];
  // offset rows R(d), d = 0..15, padded by 16 B
  __shared__ __align__(16) float2 s_dt[BK][64 + 2];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, kq = lane >> 4;  // MFMA column / row, K group

  // Workgroup -> (sequence, group of NWD splits, KV head)
  const int id = blockIdx.x;
  const int g = id % a.Hkv;
  const int wgi = (id / a.Hkv) % a.nwg;
  const int bl = id / (a.Hkv * a.nwg);
  const int b = a.b_base + bl;
  const int w = wgi * NWD + wave;  // this wave's split
  const int pos = a.seq[bl].pos;
  const DivMagic gdiv{a.seq[bl].gmul, a.seq[bl].gshift};
  const int variant = a.variant;
  // continuous remote positions (interpolation variant): n(x) = x - x/G = x rpos
  const double rpos = (double)(a.seq[bl].G - 1) / (double)a.seq[bl].G;
  // window-only variant: keys from the block holding pos - w0 + 1
  const int jb = variant == kVariantWindow ? (max(0, pos - a.w0 + 1) / BK) * BK : 0;
  const int nblk = (pos - jb) / BK + 1;  // blocks holding keys jb .. pos
  const int nsplit = a.nsplit;
  // this wave's blocks: w, w + nsplit, w + 2 nsplit, ... < nblk
  const int cnt = w < nblk ? (nblk - 1 - w) / nsplit + 1 : 0;

  // keys j <= last_remote are remote (none in the window-only variant)
  const int last_remote = variant == kVariantWindow ? -1 : pos - a.w0;
  const float c2 = a.scale_log2;
  const uint32_t rs = (uint32_t)a.Hkv * D;  // elements between consecutive cache rows
  const uint16_t* kg = (const uint16_t*)a.K + (size_t)b * a.seq_stride + (size_t)g * D;
  const uint16_t* vg = (const uint16_t*)a.V + (size_t)b * a.seq_stride + (size_t)g * D;
  // Block loads, one block ahead: K (key l16, channels 32s + 8kq + e) and V (keys 2kp,
  // 2kp+1 of channel group cg = 16 channels).  Keys past pos are clamped to pos (their
  // scores are masked).
  const int kp = lane & 7, cg = lane >> 3;
  struct Blk {
    uint4 k[4];
    uint4 v[2][2];
  };
  auto load_blk = [&](int i, Blk& x) __attribute__((always_inline)) {
    const int j0 = jb + (w + i * nsplit) * BK;
    // 64-bit offset of the block (uniform), 32-bit offsets of the lanes within it.  A
    // wave without blocks still loads one (the static wait counts): its j0 lies past
    // pos, so the base is clamped to pos too and every lane offset stays in [0, 15].
    const int jbase = min(j0, pos);
    const uint16_t* kb = kg + (size_t)jbase * rs;
    const uint16_t* vb = vg + (size_t)jbase * rs;
    const int jk = min(j0 + l16, pos);
    const uint16_t* kr = kb + (uint32_t)(jk - jbase) * rs + 8 * kq;
#pragma unroll
    for (int s = 0; s < 4; ++s) x.k[s] = *reinterpret_cast<const uint4*>(kr + 32 * s);
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int jv = min(j0 + 2 * kp + k2, pos);
      const uint16_t* vr = vb + (uint32_t)(jv - jbase) * rs + 16 * cg;
#pragma unroll
      for (int c = 0; c < 2; ++c) x.v[k2][c] = *reinterpret_cast<const uint4*>(vr + 8 * c);
    }
  };

  // The query and the first block's loads go out before the set-up work below (angles,
  // query rotation); the block's loads stay in flight across its barrier.
  uint4 raw[4];
  {
    const uint16_t* qp = (const uint16_t*)a.q + ((size_t)b * a.Hq + g * REP + min(l16, REP - 1)) * D;
#pragma unroll
    for (int s = 0; s < 4; ++s) raw[s] = *reinterpret_cast<const uint4*>(qp + 32 * s + 8 * kq);
  }
  Blk buf0, buf1;
  load_blk(0, buf0);  // unconditional (clamped to pos): keeps the wait counts static

  const double invf = inv_freq64(a.theta, lane, D);  // lane = RoPE pair
  float2* row = s_row[wave];

  // ---- angles: offset rows (shared) and the query's row --------------------------------
#pragma unroll
  for (int r = wave; r < BK; r += NWD)
    s_dt[r][lane] = angle_cs(variant == kVariantInterp ? r * rpos : (double)r, invf);
  row[lane] = angle_cs(variant == kVariantInterp ? pos * rpos : (double)(pos - alias_fast(pos, gdiv)),
                       invf);

  // ---- query operands (A: rows = query heads, lanes l16 >= REP zero) ------------------
  // lane (head l16, group kq) holds channels 32s + 8kq + e, s = 0..3
  u32x4 qh[4], ql[4];
  {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      if (l16 >= REP) raw[s] = make_uint4(0u, 0u, 0u, 0u);
    uint16_t* sq = s_q[wave];
    if (l16 < REP)
#pragma unroll
      for (int s = 0; s < 4; ++s) *reinterpret_cast<uint4*>(sq + l16 * D + 32 * s + 8 * kq) = raw[s];
    if (l16 == 15)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        *reinterpret_cast<uint4*>(sq + 8 * D + 32 * s + 8 * kq) = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float y1[8], y2[8];
      const float4* tr = reinterpret_cast<const float4*>(row + 32 * s + 8 * kq);
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const float4 cs = tr[e2];
        rot_neg(bf16_at(raw[s], 2 * e2), bf16_at(raw[s + 2], 2 * e2), cs.x, cs.y, y1[2 * e2],
                y2[2 * e2]);
        rot_neg(bf16_at(raw[s], 2 * e2 + 1), bf16_at(raw[s + 2], 2 * e2 + 1), cs.z, cs.w,
                y1[2 * e2 + 1], y2[2 * e2 + 1]);
      }
      split8(y1, qh[s], ql[s]);
      split8(y2, qh[s + 2], ql[s + 2]);
    }
  }
  const uint16_t* sq_row = s_q[wave] + (l16 < REP ? l16 : 8) * D + 8 * kq;
  // offset rows complete (LDS only: a plain __syncthreads would also wait for the
  // block loads in flight)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  f32x4 oacc[8];  // O^T blocks [16 channels][16 head columns]
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[4], l_run[4];  // heads 4*kq + r, base-2 domain; l per lane (summed at the end)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_run[r] = -1e30f;
    l_run[r] = 0.f;
  }

  uint16_t* vt = s_vt[wave];
  uint16_t* pt = s_p[wave];
  // Blocks alternate between two load buffers (no register copy between blocks).
  auto block = [&](int i, const Blk& cur, Blk& nxt) __attribute__((always_inline)) {
    const int j0 = jb + (w + i * nsplit) * BK;  // <= pos
    const int jk = j0 + l16;
    const bool any_remote = j0 <= last_remote;
    const bool any_local = j0 + BK - 1 > last_remote;
    // unconditional (the last block reloads itself): a static count of loads in
    // flight keeps the waits below from draining the prefetch
    load_blk(min(i + 1, cnt - 1), nxt);

    // ---- V^T tile: keys (2kp, 2kp+1) of channels 16cg .. 16cg+15, one word each --------
    // row dd: four 8-byte segments of 4 keys; segment q sits at q ^ ((dd >> 2) & 3)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint32_t* a0 = reinterpret_cast<const uint32_t*>(&cur.v[0][c]);
      const uint32_t* a1 = reinterpret_cast<const uint32_t*>(&cur.v[1][c]);
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int dd = 16 * cg + 8 * c + 2 * ww + hh;
          const uint32_t word = __byte_perm(a0[ww], a1[ww], hh ? 0x7632 : 0x5410);
          const int seg = (kp >> 1) ^ ((dd >> 2) & 3);
          *reinterpret_cast<uint32_t*>(vt + dd * BK + 4 * seg + 2 * (kp & 1)) = word;
        }
      }
    }

    // ---- scores S[h][key] -------------------------------------------------------------
    f32x4 sr = f32x4{0.f, 0.f, 0.f, 0.f}, sl = f32x4{0.f, 0.f, 0.f, 0.f};
    if (any_remote) {
      const int jkc = min(jk, pos);
      // n of the block's first key and the offset row of this lane's key: floor map
      // (n steps by 0 or 1 per key) or continuous map (n = j rpos, offset row j - j0)
      const int n0 = j0 - alias_fast(j0, gdiv);
      const int dk = variant == kVariantInterp ? jkc - j0 : (jkc - alias_fast(jkc, gdiv)) - n0;
      // R(n0) of the block: lane = pair (the wave's previous reads of the row are
      // complete: LDS operations of a wave execute in order)
      row[lane] = angle_cs(variant == kVariantInterp ? j0 * rpos : (double)n0, invf);
      const float2* drow = &s_dt[dk][8 * kq];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float y1[8], y2[8];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          // R(n0 + d): compose the block row with the offset row
          const float4 c0 = *reinterpret_cast<const float4*>(row + 32 * s + 8 * kq + 2 * e2);
          const float4 cd = *reinterpret_cast<const float4*>(drow + 32 * s + 2 * e2);
          const float4 cs = make_float4(c0.x * cd.x - c0.y * cd.y, c0.y * cd.x + c0.x * cd.y,
                                        c0.z * cd.z - c0.w * cd.w, c0.w * cd.z + c0.z * cd.w);
          rot_neg(bf16_at(cur.k[s], 2 * e2), bf16_at(cur.k[s + 2], 2 * e2), cs.x, cs.y,
                  y1[2 * e2], y2[2 * e2]);
          rot_neg(bf16_at(cur.k[s], 2 * e2 + 1), bf16_at(cur.k[s + 2], 2 * e2 + 1), cs.z, cs.w,
                  y1[2 * e2 + 1], y2[2 * e2 + 1]);
        }
        u32x4 h1, l1, h2, l2;
        split8(y1, h1, l1);
        split8(y2, h2, l2);
        sr = mfma16_f16(qh[s], h1, sr);
        sr = mfma16_f16(qh[s], l1, sr);
        sr = mfma16_f16(ql[s], h1, sr);
        sr = mfma16_f16(qh[s + 2], h2, sr);
        sr = mfma16_f16(qh[s + 2], l2, sr);
        sr = mfma16_f16(ql[s + 2], h2, sr);
      }
    }
    if (any_local) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 qs = *reinterpret_cast<const u32x4*>(sq_row + 32 * s);
        sl = mfma16_bf16(qs, __builtin_bit_cast(u32x4, cur.k[s]), sl);
      }
    }
    const bool use_local = pos - jk < a.w0;
    // window-only variant: keys before the window are dropped, not re-scored
    const bool valid = jk <= pos && (variant != kVariantWindow || use_local);
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = valid ? (use_local ? sl[r] : sr[r]) : -INFINITY;

    // ---- online softmax (heads 4kq + r: row group kq of the result) ---------------------
    float bm[4];
    bool need = false;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      bm[r] = fmaxf(m_run[r], row_max(sc[r]) * c2);
      need |= bm[r] > m_run[r] + kLazy;
    }
    if (__ballot(need)) {
      float f[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float mn = bm[r] > m_run[r] + kLazy ? bm[r] : m_run[r];
        f[r] = fast_exp2(m_run[r] - mn);
        l_run[r] *= f[r];
        m_run[r] = mn;
      }
      // O^T column l16 belongs to head l16: its factor lives in row group l16 >> 2,
      // register l16 & 3
      const int src = 16 * ((l16 >> 2) & 3);
      float fc = 1.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float fr = __shfl(f[r], src);
        if ((l16 & 3) == r) fc = fr;
      }
#pragma unroll
      for (int db = 0; db < 8; ++db) oacc[db] *= fc;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = fast_exp2(__fmaf_rn(sc[r], c2, -m_run[r]));
      l_run[r] += p;
      const int h = 4 * kq + r;
      if (h < REP) pt[h * BK + l16] = (uint16_t)(pack_bf16(p, 0.f) & 0xffffu);
    }

    // ---- O^T += V^T P^T (K = the block's 16 keys) -----------------------------------------
    const uint2 pb = *reinterpret_cast<const uint2*>(pt + (l16 & 15) * BK + 4 * kq);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int d = 16 * db + l16;
      const int seg = kq ^ ((d >> 2) & 3);
      const uint2 va = *reinterpret_cast<const uint2*>(vt + d * BK + 4 * seg);
      oacc[db] = mfma16k16_bf16(va, pb, oacc[db]);
    }
  };
  int i = 0;
  for (; i + 1 < cnt; i += 2) {
    block(i, buf0, buf1);
    block(i + 1, buf1, buf0);
  }
  if (i < cnt) block(i, buf0, buf1);

  // ---- merge the four waves (splits) of this workgroup, write one partial per head -----
  float lt[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) lt[r] = row_sum(l_run[r]);
  __shared__ float s_ml[NWD][16][2];
  __shared__ __align__(16) float s_acc[NWD][8][D];  // [wave][head][channel]
  if (l16 == 0)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s_ml[wave][4 * kq + r][0] = cnt > 0 ? m_run[r] : -INFINITY;
      s_ml[wave][4 * kq + r][1] = cnt > 0 ? lt[r] : 0.f;
    }
  if (l16 < REP) {  // O^T column l16 = head l16: rows 16db + 4kq + r
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) s_acc[wave][l16][16 * db + 4 * kq + r] = oacc[db][r];
  }
  __syncthreads();
  const int nwg = a.nwg;
  const size_t head0 = (size_t)b * a.Hq + (size_t)g * REP;  // first query head of the group
  for (int e = threadIdx.x; e < REP * D; e += 256) {
    const int h = e / D, d = e - h * D;
    float mx = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NWD; ++ww) mx = fmaxf(mx, s_ml[ww][h][0]);
    float o = 0.f, l = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < NWD; ++ww) {
        const float ms = s_ml[ww][h][0];
        const float wt = ms == -INFINITY ? 0.f : fast_exp2(ms - mx);
        o += wt * s_acc[ww][h][d];
        l += wt * s_ml[ww][h][1];
      }
    }
    float* dst = a.part + ((head0 + h) * nwg + wgi) * (D + 2);
    dst[d] = o;
    if (d == 0) {
      dst[D] = mx;
      dst[D + 1] = l;
    }
  }
}

// Merge the partials of each (sequence, query head): O = sum_s w_s acc_s / sum_s w_s l_s
// with w_s = 2^(m_s - max m), LSE = ln 2 (max m + log2 sum_s w_s l_s).  One workgroup per
// (sequence, query head, 32 channels); every load is issued up front (one memory round
// trip), then the maxima, weights and weighted sums are reduced in registers and LDS.
__global__ void __launch_bounds__(256) decode_mfma_combine_kernel(DecodeBatchArgs a) {
  constexpr int D = dm::D;
  constexpr int KP = kDecodeMaxParts / 8;  // partials per lane group of 32
  __shared__ float s_w[kDecodeMaxParts];
  __shared__ float s_red[8][33];
  const int tid = threadIdx.x, grp = tid >> 5, c = tid & 31;
  const int d0 = 32 * blockIdx.y;
  const int nwg = a.nwg;
  const size_t head = (size_t)a.b_base * a.Hq + blockIdx.x;
  const float* base = a.part + head * nwg * (D + 2);
  float mv = -INFINITY, lv = 0.f;
  if (tid < nwg) {
    mv = base[(size_t)tid * (D + 2) + D];
    lv = base[(size_t)tid * (D + 2) + D + 1];
  }
  float acc[KP];
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    const int s = grp + 8 * k;
    acc[k] = s < nwg ? base[(size_t)s * (D + 2) + d0 + c] : 0.f;
  }
  // max over the partials (64-lane waves, then the four waves)
  float mx = mv;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((tid & 63) == 0) s_red[tid >> 6][32] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(s_red[0][32], s_red[1][32]), fmaxf(s_red[2][32], s_red[3][32]));
  const float wt = mv == -INFINITY ? 0.f : exp2f(mv - mx);
  if (tid < nwg) s_w[tid] = wt;
  float ls = wt * lv;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ls += __shfl_xor(ls, o);
  __syncthreads();  // s_w complete, s_red[.][32] consumed
  if ((tid & 63) == 0) s_red[tid >> 6][32] = ls;
  float o = 0.f;
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    const int s = grp + 8 * k;
    if (s < nwg) o += s_w[s] * acc[k];
  }
  s_red[grp][c] = o;
  __syncthreads();
  if (tid < 32) {
    const float l = s_red[0][32] + s_red[1][32] + s_red[2][32] + s_red[3][32];
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) v += s_red[q][tid];
    ((uint16_t*)a.o)[head * D + d0 + tid] = (uint16_t)f32_to_bf16_bits(v / l);
    if (a.lse && blockIdx.y == 0 && tid == 0) a.lse[head] = (mx + log2f(l)) * 0.69314718055994530942f;
  }
}

hipError_t launch_decode_mfma(const DecodeBatchArgs& a, int rep, hipStream_t stream) {
  const dim3 grid(a.nseq * a.nwg * a.Hkv);
  switch (rep) {
    case 1: hipLaunchKernelGGL(decode_mfma_kernel<1>, grid, dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(decode_mfma_kernel<2>, grid, dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL(decode_mfma_kernel<4>, grid, dim3(256), 0, stream, a); break;
    case 8: hipLaunchKernelGGL(decode_mfma_kernel<8>, grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_mfma_combine_kernel, dim3(a.nseq * a.Hq, dm::D / 32), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace bifocal
