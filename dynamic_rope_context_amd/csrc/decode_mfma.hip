// Bifocal decode on gfx950 matrix cores: one query at position pos, bf16 cache, D = 128.
//
// Jet-Long technical summary, "Methodology" section 2 (on-the-fly correction
// rotation): the cache keeps keys with standard RoPE at their exact positions and is
// never rewritten.  A remote key j is scored against R(f(j) - j) K_j, i.e. the stored
// key rotated in fp32 registers by the table entry at n = j - f(j), and the query
// rotated once by R(f(pos) - pos); rotations compose additively, so this is RoPE at the
// aliased positions f(x) = floor(x/G) of section 1.  Keys inside the window (pos - j <
// w0) are scored with the stored bytes as they are.
//
// Layout (per wave, 16 keys per block, 16x16 matrix-core shapes):
//   * S = Q K^T with the query heads as MFMA rows and the block's keys as columns
//     (v_mfma_f32_16x16x32): lane (key l, group k) of the B operand holds channels
//     32s + 8k + e of its key, so a channel and its RoPE partner (c + 64) sit in the
//     same lane, steps s and s + 2.
//   * Remote scores need fp32 accuracy (the fp32 rotation is not representable in one
//     16-bit operand): keys and query are split into fp16 hi + lo parts and three
//     MFMAs add hi*hi + hi*lo + lo*hi (the lo*lo term is below fp32 rounding).
//   * O^T = V^T P^T (v_mfma_f32_16x16x16_bf16): the block's V rows are transposed
//     through a per-wave LDS tile (pairs of keys packed per 32-bit word), P goes
//     through a small LDS row buffer.
//   * Online softmax in the base-2 domain with a lazy running max per head.
//   * Two waves per SIMD (at most 256 registers each) so that one wave's loads are in
//     flight while the other computes.
// Each wave streams its own contiguous range of keys; the four waves of a workgroup
// merge their states in LDS and write one partial (acc[D], m, l) per query head, and
// decode_combine_kernel merges the workgroups.
#include "bf_common.h"
#include "decode_args.h"
#include "mfma_util.h"

namespace bifocal {

namespace dm {
constexpr int D = 128;
constexpr int BKD = 32;          // keys per block
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
decode_mfma_kernel(DecodeArgs a) {
  using namespace dm;
  constexpr int BK = 16;  // keys per block
  // per wave: V^T tile [128 channels][16 keys] (8-byte segments swizzled by row), P^T
  // rows [16 heads][16 keys], standard query rows [8 heads][128] + one zero row
  __shared__ __align__(16) uint16_t s_vt[NWD][D * BK];
  __shared__ __align__(16) uint16_t s_p[NWD][16 * BK];
  __shared__ __align__(16) uint16_t s_q[NWD][9 * D];
  // table rows 0..15 (angles of the key offsets inside a block), rows padded by 16 B
  __shared__ __align__(16) float2 s_dt[BK][64 + 2];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, kq = lane >> 4;  // MFMA column / row, K group

  // Workgroup -> (KV head, group of NWD splits); consecutive workgroups go to different
  // XCDs and the splits of one XCD cover a contiguous key range for every head, so the
  // table rows of that range are fetched into one L2 and shared by all heads.
  const int nwg = a.nsplit / NWD;     // workgroups per head (multiple of 8)
  const int per_xcd = nwg >> 3;
  const int id = blockIdx.x;
  const int xcd = id & 7;
  const int k_in = id >> 3;
  const int g = k_in % a.Hkv;
  const int wsplit = (xcd * per_xcd + k_in / a.Hkv) * NWD + wave;

  const int pos = a.pos;
  const int last_remote = pos - a.w0;  // keys j <= last_remote are remote
  const float c2 = a.scale_log2;
  const uint16_t* __restrict__ Kp = (const uint16_t*)a.K;
  const uint16_t* __restrict__ Vp = (const uint16_t*)a.V;
  const float2* __restrict__ tab = a.tab;
  const uint32_t rs = (uint32_t)a.Hkv * D;  // elements between consecutive cache rows
  const uint16_t* kg = Kp + (size_t)g * D;
  const uint16_t* vg = Vp + (size_t)g * D;

  // ---- query operands (A: rows = query heads, lanes l16 >= REP zero) ------------------
  // lane (head l16, group kq) holds channels 32s + 8kq + e, s = 0..3
  u32x4 qh[4], ql[4];
  {
    const uint16_t* qp = (const uint16_t*)a.q + (size_t)(g * REP + min(l16, REP - 1)) * D;
    uint4 raw[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      raw[s] = *reinterpret_cast<const uint4*>(qp + 32 * s + 8 * kq);
      if (l16 >= REP) raw[s] = make_uint4(0u, 0u, 0u, 0u);
    }
    uint16_t* sq = s_q[wave];
    if (l16 < REP)
#pragma unroll
      for (int s = 0; s < 4; ++s) *reinterpret_cast<uint4*>(sq + l16 * D + 32 * s + 8 * kq) = raw[s];
    if (l16 == 15)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        *reinterpret_cast<uint4*>(sq + 8 * D + 32 * s + 8 * kq) = make_uint4(0u, 0u, 0u, 0u);
    const int nq = pos - alias_fast(pos, a.gdiv);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float y1[8], y2[8];
      const float4* tr = reinterpret_cast<const float4*>(tab + (size_t)nq * 64 + 32 * s + 8 * kq);
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
  for (int i = threadIdx.x; i < BK * 32; i += 256) {  // rows <= pos are built
    const int r = i >> 5, c = i & 31;
    *reinterpret_cast<float4*>(&s_dt[r][2 * c]) =
        reinterpret_cast<const float4*>(tab + (size_t)min(r, pos) * 64)[c];
  }
  __syncthreads();

  // ---- this wave's key range --------------------------------------------------------
  const int j_begin = wsplit * a.kps;
  const int j_end = min(j_begin + a.kps, pos + 1);
  const int nblk = j_end > j_begin ? (j_end - j_begin + BK - 1) / BK : 0;

  f32x4 oacc[8];  // O^T blocks [16 channels][16 head columns]
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[4], l_run[4];  // heads 4*kq + r, base-2 domain; l per lane (summed at the end)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_run[r] = -1e30f;
    l_run[r] = 0.f;
  }

  // Block loads, one block ahead: K (key l16, channels 32s + 8kq + e), V (keys 2kp,
  // 2kp+1 of channel group cg = 16 channels) and the correction-table row of the key
  // (pairs 32s + 8kq + e, s < 2).
  const int kp = lane & 7, cg = lane >> 3;
  struct Blk {
    uint4 k[4];
    uint4 v[2][2];
    float4 t[8];
  };
  auto load_blk = [&](int b, Blk& x) __attribute__((always_inline)) {
    const int j0 = j_begin + b * BK;
    const int jk = min(j0 + l16, pos);
    const uint16_t* kr = kg + (uint32_t)jk * rs + 8 * kq;
#pragma unroll
    for (int s = 0; s < 4; ++s) x.k[s] = *reinterpret_cast<const uint4*>(kr + 32 * s);
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int jv = min(j0 + 2 * kp + k2, pos);
      const uint16_t* vr = vg + (uint32_t)jv * rs + 16 * cg;
#pragma unroll
      for (int c = 0; c < 2; ++c) x.v[k2][c] = *reinterpret_cast<const uint4*>(vr + 8 * c);
    }
    // The block's keys have consecutive n = j - f(j) (steps of 0 or 1): their angles
    // are n0 + d with d < 16; the row of n0 is loaded here (one row per block, shared
    // by all lanes), the rows of d sit in LDS.  Unconditional (unused for blocks
    // without remote keys): a fixed number of loads per block lets every wait count
    // only the loads it needs.
    const int j0c = min(j0, pos);
    const float4* tr =
        reinterpret_cast<const float4*>(tab + (size_t)(j0c - alias_fast(j0c, a.gdiv)) * 64 + 8 * kq);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) x.t[4 * s + e2] = tr[16 * s + e2];
  };

  uint16_t* vt = s_vt[wave];
  uint16_t* pt = s_p[wave];
  // Blocks alternate between two load buffers (no register copy between blocks).
  auto block = [&](int b, const Blk& cur, Blk& nxt) __attribute__((always_inline)) {
    const int j0 = j_begin + b * BK;
    const int jk = j0 + l16;
    const bool any_remote = j0 <= last_remote;
    const bool any_local = j0 + BK - 1 > last_remote;
    // unconditional (the last block reloads itself): a static count of loads in
    // flight keeps the waits below from draining the prefetch
    load_blk(min(b + 1, nblk - 1), nxt);

    // ---- V^T tile: keys (2kp, 2kp+1) of channels 16cg .. 16cg+15, one word each --------
    // row dd: four 8-byte segments of 4 keys; segment q sits at q ^ ((dd >> 2) & 3)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint32_t* a0 = reinterpret_cast<const uint32_t*>(&cur.v[0][c]);
      const uint32_t* a1 = reinterpret_cast<const uint32_t*>(&cur.v[1][c]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int dd = 16 * cg + 8 * c + 2 * w + hh;
          const uint32_t word = __byte_perm(a0[w], a1[w], hh ? 0x7632 : 0x5410);
          const int seg = (kp >> 1) ^ ((dd >> 2) & 3);
          *reinterpret_cast<uint32_t*>(vt + dd * BK + 4 * seg + 2 * (kp & 1)) = word;
        }
      }
    }

    // ---- scores S[h][key] -------------------------------------------------------------
    f32x4 sr = f32x4{0.f, 0.f, 0.f, 0.f}, sl = f32x4{0.f, 0.f, 0.f, 0.f};
    if (any_remote) {
      const int j0c = min(j0, pos), jkc = min(jk, pos);
      const int dk = (jkc - alias_fast(jkc, a.gdiv)) - (j0c - alias_fast(j0c, a.gdiv));
      const float2* drow = &s_dt[dk][8 * kq];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float y1[8], y2[8];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          // R(n0 + d): compose the block row with the offset row
          const float4 c0 = cur.t[4 * s + e2];
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
    const bool valid = jk <= pos;
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
  Blk buf0, buf1;
  if (nblk > 0) load_blk(0, buf0);
  int b = 0;
  for (; b + 1 < nblk; b += 2) {
    block(b, buf0, buf1);
    block(b + 1, buf1, buf0);
  }
  if (b < nblk) block(b, buf0, buf1);

  // ---- merge the four waves (splits) of this workgroup, write one partial per head -----
  float lt[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) lt[r] = row_sum(l_run[r]);
  __shared__ float s_ml[NWD][16][2];
  __shared__ __align__(16) float s_acc[NWD][8][D];  // [wave][head][channel]
  if (l16 == 0)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s_ml[wave][4 * kq + r][0] = nblk > 0 ? m_run[r] : -INFINITY;
      s_ml[wave][4 * kq + r][1] = nblk > 0 ? lt[r] : 0.f;
    }
  if (l16 < REP) {  // O^T column l16 = head l16: rows 16db + 4kq + r
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) s_acc[wave][l16][16 * db + 4 * kq + r] = oacc[db][r];
  }
  __syncthreads();
  const int wg_split = wsplit / NWD;
  const int nwg_all = a.nsplit / NWD;
  for (int e = threadIdx.x; e < REP * D; e += 256) {
    const int h = e / D, d = e - h * D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWD; ++w) mx = fmaxf(mx, s_ml[w][h][0]);
    float o = 0.f, l = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NWD; ++w) {
        const float ms = s_ml[w][h][0];
        const float wt = ms == -INFINITY ? 0.f : fast_exp2(ms - mx);
        o += wt * s_acc[w][h][d];
        l += wt * s_ml[w][h][1];
      }
    }
    float* dst = a.part + ((size_t)(g * REP + h) * nwg_all + wg_split) * (D + 2);
    dst[d] = o;
    if (d == 0) {
      dst[D] = mx;
      dst[D + 1] = l;
    }
  }
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int rep, hipStream_t stream) {
  const dim3 grid(a.nsplit / dm::NWD * a.Hkv);
  switch (rep) {
    case 1: hipLaunchKernelGGL(decode_mfma_kernel<1>, grid, dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(decode_mfma_kernel<2>, grid, dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL(decode_mfma_kernel<4>, grid, dim3(256), 0, stream, a); break;
    case 8: hipLaunchKernelGGL(decode_mfma_kernel<8>, grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace bifocal
