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
//   * S^T = K Q^T with the block's keys as MFMA rows and the query heads as columns
//     (v_mfma_f32_16x16x32): lane (key l, group k) of the A operand holds channels
//     32s + 8k + e of its key, so a channel and its RoPE partner (c + 64) sit in the
//     same lane, steps s and s + 2.  The result gives lane (head h, group k) keys
//     4k .. 4k+3 of head h: the layout of P^T as the B operand of the PV product, so
//     the probabilities never leave the registers, and a head's row max and sum take
//     two lane swaps.
//   * Remote scores need fp32 accuracy (the fp32 rotation is not representable in one
//     16-bit operand): keys and query are split into fp16 hi + lo parts and three
//     MFMAs add hi*hi + hi*lo + lo*hi (the lo*lo term is below fp32 rounding).
//   * Angles: the keys of a block have consecutive n = j - f(j) (steps of 0 or 1), so
//     R(n) = R(n0) R(n - n0) with n - n0 < 16.  Each lane of a wave owns one RoPE pair
//     and holds cos/sin(n0 theta_m) of the wave's current block in fp64, rounded to fp32
//     per block (the values a precomputed table would hold, to within fp32 rounding);
//     the 16 offset rows R(d) are built once per workgroup, as fp64 powers of R(1).
//     Consecutive blocks of a wave lie nsplit*16 keys apart, so n0 advances by one of
//     two integers (the floor map moves by q or q + 1, with q = floor(nsplit*16 / G)):
//     the fp64 angle pair advances by the angle-addition formula with one of two step
//     rotations evaluated once per workgroup, and the drift after thousands of steps
//     stays near 1e-12, far below fp32 rounding.  No table is read, so decode needs no
//     table in the workspace.
//   * O^T = V^T P^T (v_mfma_f32_16x16x16_bf16): the block's V rows go to a per-wave
//     LDS tile as loaded, and the transposing LDS read (ds_read_b64_tr_b16) hands each
//     lane four keys of one channel, the V^T operand.
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
constexpr float kLazySum = 256.f;  // 2^kLazy
}  // namespace dm

// fp16 hi/lo of 8 consecutive values, packed as two MFMA operands: hi = RNE(y) by the
// packed conversion, lo = RNE(y - hi).  y - hi is exact in fp32 (hi is y rounded to 11
// bits, or inf on overflow, when the difference is -inf as well), so one mixed-precision
// FMA per half, fp16 hi times -1 plus fp32 y rounded once to fp16, gives the same bits
// as converting hi back and subtracting, in one instruction instead of three.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split8(const float* y, u32x4& hi, u32x4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const f16x2_t hv = {(_Float16)y[2 * e], (_Float16)y[2 * e + 1]};
    h[e] = __builtin_bit_cast(uint32_t, hv);
    asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(l[e]) : "v"(h[e]), "v"(y[2 * e]));
    asm("v_fma_mixhi_f16 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "+v"(l[e]) : "v"(h[e]), "v"(y[2 * e + 1]));
  }
  hi = u32x4{h[0], h[1], h[2], h[3]};
  lo = u32x4{l[0], l[1], l[2], l[3]};
}

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
// ds_read_b64_tr_b16 at an address in LDS (p points into a __shared__ array): within each
// group of 16 lanes, lane i receives element i & 3 of the 8-byte chunks that lanes i/4,
// 4 + i/4, 8 + i/4 and 12 + i/4 of its group point to (a 4 x 4 transpose of 16-bit
// elements per 16-lane group).
__device__ __forceinline__ v4i16 lds_read_tr16(uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds_u8*)p);
}
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
// Max / sum of lane i and lane i ^ 16 (rows of 16 lanes swapped in pairs), and sums
// of lane i and lane i ^ 32, with the permlane swaps (no LDS round trip).
__device__ __forceinline__ float max_lane_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_lane_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_lane_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
template <int REP>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
decode_mfma_kernel(DecodeBatchArgs a) {
  using namespace dm;
  // per wave: V tile [16 keys][128 channels] (32-byte blocks swizzled by row), P^T
  // rows [16 heads][16 keys], standard query rows [8 heads][128] + one zero row, and
  // the angle row R(n0) of the current block (lane = RoPE pair)
  __shared__ __align__(16) uint16_t s_vt[NWD][D * BK];
  __shared__ __align__(16) uint16_t s_q[NWD][9 * D];
  __shared__ __align__(16) float2 s_row[NWD][64];
  // offset rows R(d), d = 0..15, padded by 16 B
  __shared__ __align__(16) float2 s_dt[BK][64 + 2];
  // angles computed once per workgroup: the offset rows' base step and the block
  // recurrence's step (fp64), the query's row (fp32)
  __shared__ __align__(16) double2 s_base[64], s_step[64];
  __shared__ __align__(16) float2 s_qrow[64];
  // K tile of the current block per wave: 16 rows x 256 bytes (after the key loop, the
  // wave's part of the merge buffer)
  __shared__ __align__(16) uint8_t s_kt[NWD][BK * D * 2];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, kq = lane >> 4;  // MFMA column / row, K group
  if (a.hdr && blockIdx.x == 0 && threadIdx.x == 0) {
    // table rows past this layout's capacity are overwritten by the partials below:
    // a later prefill on the same workspace must not trust them
    volatile TableHeader* h = a.hdr;
    if (h->n_valid > a.n_cap) h->n_valid = a.n_cap;
  }

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
  // Block loads, one block ahead, to registers.  K and V alike: load t takes keys
  // 4t .. 4t+3 of the block, each a whole 256-byte row (lane: key 4t + (lane >> 4),
  // 16-byte chunk lane & 15), so one load reads four contiguous row segments; loads that
  // give each key 64 bytes stream about a tenth slower, and V loads of 128 bytes per key
  // about 1% slower.  The K chunks then go through the wave's LDS tile to the
  // matrix-core layout (chunk c of key r at position c ^ r of its LDS row, which keeps
  // both the writes and the reads free of bank conflicts); the V chunks go to the V tile.
  // Keys past pos are clamped to pos (their scores are masked).
  struct Blk {
    u32x4 k[4];  // native vectors: plain register moves, no struct copies
    u32x4 v[4];
  };
  // Byte offsets of this lane's loads within a block of 16 whole keys (key rows rs
  // elements apart), fixed for the wave
  uint32_t koff[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) koff[t] = ((4 * t + (lane >> 4)) * rs + 8 * (lane & 15)) * 2u;
  auto load_blk = [&](int i, Blk& x) __attribute__((always_inline)) {
    const int j0 = jb + (w + i * nsplit) * BK;
    // 64-bit offset of the block (uniform), 32-bit offsets of the lanes within it.  A
    // wave without blocks still loads one (the static wait counts): its j0 lies past
    // pos, so the base is clamped to pos too and every lane offset stays in [0, 15].
    const int jbase = min(j0, pos);
    const uint8_t* kb = reinterpret_cast<const uint8_t*>(kg + (size_t)jbase * rs);
    const uint8_t* vb = reinterpret_cast<const uint8_t*>(vg + (size_t)jbase * rs);
    uint32_t ko[4];
    if (j0 + BK - 1 <= pos) {  // every key of the block exists (all but the last block)
#pragma unroll
      for (int t = 0; t < 4; ++t) ko[t] = koff[t];
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        ko[t] = ((uint32_t)(min(j0 + 4 * t + (lane >> 4), pos) - jbase) * rs + 8 * (lane & 15)) * 2u;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) x.k[t] = ld_stream(kb + ko[t]);
#pragma unroll
    for (int t = 0; t < 4; ++t) x.v[t] = ld_stream(vb + ko[t]);
  };
  // K of a block through the wave's LDS tile: lane (key l16, group kq), step s =
  // channels 32s + 8kq .. +7 (chunk 4s + kq).  The wave's LDS operations run in order, so
  // the reads see this block's writes and the next block's writes follow these reads.
  uint8_t* kt = s_kt[wave];
  auto stage_k = [&](const Blk& x, uint4* k) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r = 4 * t + (lane >> 4);
      *reinterpret_cast<u32x4*>(kt + 256 * r + 16 * ((lane & 15) ^ r)) = x.k[t];
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 y = *reinterpret_cast<const u32x4*>(kt + 256 * l16 + 16 * ((4 * s + kq) ^ l16));
      k[s] = make_uint4(y[0], y[1], y[2], y[3]);
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

  // ---- angles ----------------------------------------------------------------------------
  // Each wave takes one float64 sincos per lane for its first block; three angles are
  // shared by the workgroup, one wave each: the offset rows' base step (wave 0), the
  // query's row (wave 1) and the block recurrence's step (wave 2).  The offset rows are
  // float64 powers of the base step and R(step - 1) = R(step) R(-1), so a wave evaluates
  // two sincos instead of eight (products of a few unit rotations stay within 1e-15 of
  // the sincos values, far below fp32 rounding).
  const int jstep = nsplit * BK;
  const int dstep = jstep - alias_fast(jstep, gdiv);  // n0 step when f moves by floor(jstep/G)
  const double da = variant == kVariantInterp ? jstep * rpos : (double)dstep;
  double ac, as;  // fp64 angle of the current block (first block: w)
  {
    const int jw = jb + w * BK;
    const double a0 = variant == kVariantInterp ? jw * rpos : (double)(jw - alias_fast(jw, gdiv));
    sincos_reduced(a0 * invf, &as, &ac);
  }
  if (wave == 0) {
    double sn, cs;  // base step: 1 (floor map) or G-1/G (continuous map)
    sincos_reduced((variant == kVariantInterp ? rpos : 1.0) * invf, &sn, &cs);
    s_base[lane] = make_double2(cs, sn);
  } else if (wave == 1) {
    s_qrow[lane] = angle_cs(variant == kVariantInterp ? pos * rpos
                                                     : (double)(pos - alias_fast(pos, gdiv)),
                            invf);
  } else if (wave == 2) {
    double sn, cs;
    sincos_reduced(da * invf, &sn, &cs);
    s_step[lane] = make_double2(cs, sn);
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // shared angles written
  auto cmul = [](double2 x, double2 y) __attribute__((always_inline)) {
    return make_double2(x.x * y.x - x.y * y.y, x.x * y.y + x.y * y.x);
  };
  const double2 b1 = s_base[lane];
  const double2 st = s_step[lane];
  const double ca = st.x, sa = st.y;
  // R(da - 1) = R(da) conj(R(1)) (floor map; the continuous map never takes it)
  const double cb = ca * b1.x + sa * b1.y, sb = sa * b1.x - ca * b1.y;
  {
    // offset rows d = wave + 4k: B^d with B the base step
    const double2 p2 = cmul(b1, b1), p4 = cmul(p2, p2);
    double2 r = wave == 0 ? make_double2(1.0, 0.0) : wave == 1 ? b1 : wave == 2 ? p2 : cmul(p2, b1);
#pragma unroll
    for (int k = 0; k < BK / NWD; ++k) {
      s_dt[wave + NWD * k][lane] = make_float2((float)r.x, (float)r.y);
      r = cmul(r, p4);
    }
  }

  // ---- query operands (B: columns = query heads, lanes l16 >= REP zero) ---------------
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
      const float4* tr = reinterpret_cast<const float4*>(s_qrow + 32 * s + 8 * kq);
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
  // running max of head l16 (base-2 domain, equal in the lane's four key groups) and
  // the lane's share of its row sum (keys 4kq .. 4kq+3 of every block; summed at the end)
  float m_run = -1e30f, l_run = 0.f;

  uint8_t* vtb = reinterpret_cast<uint8_t*>(s_vt[wave]);
  // Blocks alternate between two load buffers (no register copy between blocks): block
  // i + 1's loads go out first and stay in flight while block i is scored.
  auto block = [&](int i, const Blk& cur, Blk& nxt) __attribute__((always_inline)) {
    const int j0 = jb + (w + i * nsplit) * BK;  // <= pos
    const int jk = j0 + l16;
    const bool any_remote = j0 <= last_remote;
    const int n0 = j0 - alias_fast(j0, gdiv);  // n of the block's first key (floor map)
    const bool any_local = j0 + BK - 1 > last_remote;
    // unconditional (the last block reloads itself): a static count of loads in
    // flight keeps the waits below from draining the prefetch
    load_blk(min(i + 1, cnt - 1), nxt);
    uint4 kr4[4];
    stage_k(cur, kr4);

    // ---- V tile, rows as loaded: row = key, 32-byte block b (16 channels) of row r at
    // position b ^ (r & 7); load t of lane (key 4t + lane/16, chunk lane mod 16) is one
    // 16-byte half of such a block (conflict-free: a row's 16 chunks cover all banks)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r = 4 * t + (lane >> 4), ch = lane & 15;
      *reinterpret_cast<u32x4*>(vtb + 256 * r + 32 * ((ch >> 1) ^ (r & 7)) + 16 * (ch & 1)) =
          cur.v[t];
    }

    // ---- scores S^T[key][head] ----------------------------------------------------------
    f32x4 sr = f32x4{0.f, 0.f, 0.f, 0.f}, sl = f32x4{0.f, 0.f, 0.f, 0.f};
    if (any_remote) {
      const int jkc = min(jk, pos);
      // offset row of this lane's key: floor map (n steps by 0 or 1 per key) or
      // continuous map (n = j rpos, offset row j - j0)
      const int dk = variant == kVariantInterp ? jkc - j0 : (jkc - alias_fast(jkc, gdiv)) - n0;
      // R(n0) of the block: lane = pair (the wave's previous reads of the row are
      // complete: LDS operations of a wave execute in order)
      row[lane] = make_float2((float)ac, (float)as);
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
          rot_neg(bf16_at(kr4[s], 2 * e2), bf16_at(kr4[s + 2], 2 * e2), cs.x, cs.y,
                  y1[2 * e2], y2[2 * e2]);
          rot_neg(bf16_at(kr4[s], 2 * e2 + 1), bf16_at(kr4[s + 2], 2 * e2 + 1), cs.z, cs.w,
                  y1[2 * e2 + 1], y2[2 * e2 + 1]);
        }
        u32x4 h1, l1, h2, l2;
        split8(y1, h1, l1);
        split8(y2, h2, l2);
        sr = mfma16_f16(h1, qh[s], sr);
        sr = mfma16_f16(l1, qh[s], sr);
        sr = mfma16_f16(h1, ql[s], sr);
        sr = mfma16_f16(h2, qh[s + 2], sr);
        sr = mfma16_f16(l2, qh[s + 2], sr);
        sr = mfma16_f16(h2, ql[s + 2], sr);
      }
    }
    if (any_local) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 qs = *reinterpret_cast<const u32x4*>(sq_row + 32 * s);
        sl = mfma16_bf16(__builtin_bit_cast(u32x4, kr4[s]), qs, sl);
      }
    }
    // S^T: lane (head l16, group kq) holds keys j0 + 4kq + r, r = 0..3, of head l16
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = j0 + 4 * kq + r;
      const bool use_local = pos - j < a.w0;
      // window-only variant: keys before the window are dropped, not re-scored
      const bool valid = j <= pos && (variant != kVariantWindow || use_local);
      sc[r] = valid ? (use_local ? sl[r] : sr[r]) : -INFINITY;
    }

    // ---- online softmax of head l16 -------------------------------------------------------
    // Probabilities against the running max first; the head's max only when a lane's
    // four probabilities sum past 2^kLazy (each is at most the sum, so otherwise no score
    // passed m_run by more than kLazy and the lazy rule keeps m_run).
    float pr[4];
    auto probs = [&]() __attribute__((always_inline)) {
      float t = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[r] = fast_exp2(__fmaf_rn(sc[r], c2, -m_run));
        t += pr[r];
      }
      return t;
    };
    float tsum = probs();
    if (__ballot(!(tsum <= kLazySum))) {
      float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      mx = max_lane_xor16(max_lane_xor32(mx));  // the head's four key groups
      const float bm = fmaxf(m_run, mx * c2);
      const bool need = bm > m_run + kLazy;
      if (__ballot(need)) {
        // O^T column l16 is head l16: the lane's own factor
        const float mn = need ? bm : m_run;
        const float f = fast_exp2(m_run - mn);
        l_run *= f;
        m_run = mn;
#pragma unroll
        for (int db = 0; db < 8; ++db) oacc[db] *= f;
      }
      tsum = probs();
    }
    l_run += tsum;

    // ---- O^T += V^T P^T (K = the block's 16 keys): P^T is already in operand layout ------
    const uint2 pb = make_uint2(pack_bf16(pr[0], pr[1]), pack_bf16(pr[2], pr[3]));
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      // transposing read: lane j of group kq gives 4 channels 16db + 4(j & 3) .. of key
      // 4kq + j/4, and lane (channel 16db + l16, group kq) receives keys 4kq .. 4kq+3 of
      // its channel, the V^T operand
      const int r = 4 * kq + (l16 >> 2);
      const v4i16 t = lds_read_tr16(vtb + 256 * r + 32 * (db ^ (r & 7)) + 8 * (l16 & 3));
      oacc[db] = mfma16k16_bf16(__builtin_bit_cast(uint2, t), pb, oacc[db]);
    }

    // ---- advance the block angle to this wave's next block --------------------------------
    const int j1 = j0 + jstep;
    if (j1 <= last_remote) {
      const bool alt = variant != kVariantInterp && (j1 - alias_fast(j1, gdiv)) - n0 != dstep;
      const double c = alt ? cb : ca, sn = alt ? sb : sa;
      const double t = ac * c - as * sn;
      as = fma(as, c, ac * sn);
      ac = t;
    }
  };
  int i = 0;
  for (; i + 1 < cnt; i += 2) {
    block(i, buf0, buf1);
    block(i + 1, buf1, buf0);
  }
  if (i < cnt) block(i, buf0, buf1);

  // ---- merge the four waves (splits) of this workgroup, write one partial per head -----
  const float lt = sum_lane_xor16(sum_lane_xor32(l_run));  // the head's four key groups
  __shared__ float s_ml[NWD][16][2];
  // [wave][head][channel] over the K tiles: each wave writes the part that was its own
  // tile, after its own last reads of it
  float(*s_acc)[8][D] = reinterpret_cast<float(*)[8][D]>(&s_kt[0][0]);
  static_assert(sizeof(s_kt[0]) == sizeof(float) * 8 * D, "merge buffer = K tile per wave");
  if (kq == 0) {
    s_ml[wave][l16][0] = cnt > 0 ? m_run : -INFINITY;
    s_ml[wave][l16][1] = cnt > 0 ? lt : 0.f;
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
