// Bifocal prefill on gfx950 matrix cores: bf16 inputs, fp32 accumulation.
//
// What it computes (Jet-Long technical summary, "Methodology" sections 1 and 2):
// causal GQA attention where key j <= i is scored with standard RoPE when i - j < w0
// (local window) and with RoPE at the aliased positions f(i), f(j), f(x) = floor(x/G),
// G = max(1, ceil(L / w_pretrained)), otherwise.  The pages merge three FlashAttention
// passes by inclusion-exclusion with LogSumExp statistics; since that merge equals
// per-pair routing, each pair's score is selected by its distance and fed to ONE
// online softmax, with no mask matrix: tiles are classified from indices alone.
//
// Design for CDNA4 (one workgroup = one KV head x a block of query positions for all
// Hq/Hkv query heads of the group; 8 waves, each wave 32 query rows):
//   * S^T = K Q^T and O^T = V^T P^T with v_mfma_f32_32x32x16: the query is the MFMA
//     column, so every query row lives in one lane pair (l, l^32) and P goes from
//     the score accumulator to the PV operand without a trip through LDS.
//   * K/V tiles of 64 keys are staged through LDS (double-buffered, one barrier per
//     tile) and shared by all query heads of the group.  V is stored transposed so
//     that the PV operand is two 8-byte LDS reads.
//   * Tiles are classified from indices: REMOTE (every pair outside the window) take
//     the remote-only path, LOCAL (every pair inside) the standard path, and the few
//     STRADDLE tiles compute both score sets and select per element.
//   * Local scores use the exact bf16 input bytes (bf16 MFMA), so G = 1 reproduces
//     plain causal attention.  Remote scores need the correction rotation R(f(x) - x)
//     (section 2, rotations compose additively), applied in fp32 registers once per
//     key tile for the whole group and once per query row; the rotated operands are
//     rounded to fp16 (same MFMA rate as bf16 on gfx950, 3 more mantissa bits), and
//     for the 4 RoPE pairs per KV head with the largest |q||k| bound a hi/lo split adds
//     one K=16 MFMA step (hi*lo + lo*hi) so that outlier channels do not lose the
//     low-order bits of their products.
//   * Online softmax in the base-2 domain with a lazy running max (rescale only when
//     the max grows by more than 8), row sums kept per lane half.
#include <type_traits>

#include "bf_common.h"
#include "prefill_args.h"

namespace bifocal {

namespace mf {
constexpr int D = 128;
constexpr int BK = 64;        // keys per tile
constexpr int NW = 8;         // waves per workgroup (32 query rows each)
constexpr int ROWS = 256;     // query rows (head, position) per workgroup
constexpr int KS_LD = D + 8;  // LDS row stride (16-bit elements) of the K arrays: 272 B
constexpr int VT_LD = BK + 4; // LDS row stride of transposed V: 136 B
constexpr int KC_LD = 16;     // LDS row of the hi/lo correction operand: 32 B
constexpr float kLazy = 8.f;  // allowed growth of the running max before a rescale

struct Stage {
  uint16_t ks[BK * KS_LD];  // standard keys, bf16 bits
  uint16_t kr[BK * KS_LD];  // remote keys R(f(j)-j) K_j, fp16 bits
  uint16_t kc[BK * KC_LD];  // [lo of 8 selected channels | hi of them], fp16 bits
  uint16_t vt[D * VT_LD];   // V^T, bf16 bits
};
constexpr size_t kSmem = 2 * sizeof(Stage);

enum { kRemote = 0, kStraddle = 1, kLocal = 2 };
}  // namespace mf

// R(-n) with the table entry (cos, sin) of n: (x1, x2) -> (x1 c + x2 s, x2 c - x1 s).
// Written with explicit roundings so that every caller gets identical bits.
__device__ __forceinline__ void rot_neg(float x1, float x2, float c, float s, float& y1,
                                        float& y2) {
  y1 = __fmaf_rn(x1, c, __fmul_rn(x2, s));
  y2 = __fmaf_rn(x2, c, -__fmul_rn(x1, s));
}

__device__ __forceinline__ uint32_t f16_bits(_Float16 h) {
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}
// fp16 hi part (round to nearest even) and the fp16 remainder.
__device__ __forceinline__ void split_f16(float y, uint32_t& hi, uint32_t& lo) {
  const _Float16 h = (_Float16)y;
  const _Float16 l = (_Float16)(y - (float)h);
  hi = f16_bits(h);
  lo = f16_bits(l);
}
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return f16_bits((_Float16)a) | (f16_bits((_Float16)b) << 16);
}

__device__ __forceinline__ f32x16 mfma_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_at(const uint4& w, int e) {
  const uint32_t x = e < 2 ? w.x : e < 4 ? w.y : e < 6 ? w.z : w.w;
  return (e & 1) ? bf16_hi(x) : bf16_lo(x);
}

// ---------------------------------------------------------------------------
// Pre-pass: per (head, RoPE pair) maximum of the squared pair norm over all tokens.
// Pair norms are rotation invariant, so the maxima over the standard-RoPE inputs
// bound the remote (rotated) operands too.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) pair_max_zero_kernel(uint32_t* mx, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) mx[i] = 0u;
}

__global__ void __launch_bounds__(256) pair_max_kernel(const uint16_t* __restrict__ X, int T,
                                                       int H, int tok_per_block,
                                                       uint32_t* __restrict__ mx) {
  const int hm = blockIdx.x * 256 + threadIdx.x;  // head * 64 + pair
  if (hm >= H * 64) return;
  const int h = hm >> 6, m = hm & 63;
  const int t0 = blockIdx.y * tok_per_block;
  const int t1 = min(T, t0 + tok_per_block);
  float best = 0.f;
  for (int t = t0; t < t1; ++t) {
    const uint16_t* row = X + ((size_t)t * H + h) * mf::D;
    const float a = __uint_as_float((uint32_t)row[m] << 16);
    const float b = __uint_as_float((uint32_t)row[m + 64] << 16);
    best = fmaxf(best, a * a + b * b);
  }
  atomicMax(mx + hm, __float_as_uint(best));  // non-negative floats order as integers
}

// Top kSelPairs pairs per KV head by the bound max|k_m| * max_h |q_{h,m}| (squared).
__global__ void pair_select_kernel(const uint32_t* __restrict__ mxq,
                                   const uint32_t* __restrict__ mxk, int Hq, int Hkv,
                                   int32_t* __restrict__ sel) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= Hkv) return;
  const int rep = Hq / Hkv;
  float bound[64];
  for (int m = 0; m < 64; ++m) {
    float q = 0.f;
    for (int r = 0; r < rep; ++r) q = fmaxf(q, __uint_as_float(mxq[(g * rep + r) * 64 + m]));
    bound[m] = q * __uint_as_float(mxk[g * 64 + m]);
  }
  int chosen[kSelPairs];
  for (int p = 0; p < kSelPairs; ++p) {
    int best = -1;
    float bv = -1.f;
    for (int m = 0; m < 64; ++m) {
      bool used = false;
      for (int q = 0; q < p; ++q) used |= chosen[q] == m;
      if (!used && bound[m] > bv) {
        bv = bound[m];
        best = m;
      }
    }
    chosen[p] = best;
  }
  for (int p = 0; p < kSelPairs; ++p) sel[g * kSelPairs + p] = chosen[p];
}

// ---------------------------------------------------------------------------
// Main kernel
// ---------------------------------------------------------------------------
template <int REP>
__global__ void __launch_bounds__(512) prefill_mfma_kernel(PrefillArgs args) {
  using namespace mf;
  extern __shared__ __align__(16) uint8_t smem_raw[];
  Stage* stg = reinterpret_cast<Stage*>(smem_raw);

  constexpr int BMPOS = ROWS / REP;       // query positions per workgroup
  constexpr int PBLK = BMPOS / 32;        // 32-row position blocks per head

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;              // 0 .. NW-1: one 32-query block each
  const int ln = lane & 31;               // MFMA column / row within a 32-block
  const int hf = lane >> 5;               // lane half

  // Workgroup -> (KV head, sequence, query block).  KV head is the fastest index so
  // that the workgroups of one head share an XCD's L2; query blocks run longest-first.
  const int Hkv = args.Hkv;
  const int nseq = args.nseq;
  const int g = blockIdx.x % Hkv;
  const int rest = blockIdx.x / Hkv;
  const int b = rest % nseq;
  const int qb = args.max_qblocks - 1 - rest / nseq;
  const int L = args.seq[b].len;
  const int i0 = qb * BMPOS;
  if (i0 >= L) return;
  const int start = args.seq[b].start;
  const int G = args.seq[b].G;
  const int Hq = args.Hq;
  const int i_end = min(L, i0 + BMPOS);  // exclusive
  // G = 1: the aliased positions are the true ones, every pair is "local".
  const int w0 = G == 1 ? (1 << 30) : args.w0;

  const uint16_t* __restrict__ Qp = (const uint16_t*)args.Q;
  const uint16_t* __restrict__ Kp = (const uint16_t*)args.K;
  const uint16_t* __restrict__ Vp = (const uint16_t*)args.V;
  const float2* __restrict__ tab = args.tab;

  // ---- this wave's 32-query block -------------------------------------------------
  const int qhead = g * REP + wave / PBLK;
  const int qi = i0 + 32 * (wave % PBLK) + ln;  // query position of this lane's column
  const int qrow_i = min(qi, L - 1);
  const uint16_t* qrow = Qp + ((size_t)(start + qrow_i) * Hq + qhead) * D;

  // ---- tile ranges --------------------------------------------------------------
  const int nkt = (i_end - 1) / BK + 1;
  int ktA, ktB;  // [0,ktA) remote, [ktA,ktB) straddle, [ktB,nkt) local
  {
    const long long x = (long long)i0 - w0 - (BK - 1);
    ktA = x >= 0 ? (int)(x / BK) + 1 : 0;
    const long long y = (long long)(i_end - 1) - w0;
    ktB = y >= 0 ? (int)(y / BK) + 1 : 0;
    ktA = min(ktA, nkt);
    ktB = min(max(ktB, ktA), nkt);
  }

  // ---- query operands -------------------------------------------------------------
  // B operand of S^T = K Q^T: lane (column ln, half hf) holds channels 16s + 8hf + e.
  u32x4 qop[8];   // remote phase: fp16 of R(f(i)-i) q; local phase: bf16 q
  u32x4 qcor;     // hi (half 0) or lo (half 1) of the 8 selected remote channels
  auto load_q_std = [&](u32x4* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 8; ++s)
      dst[s] = *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * hf);
  };
  auto load_q_remote = [&]() __attribute__((always_inline)) {
    const int n = qrow_i - alias_pos(qrow_i, G);
    uint4 raw[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) raw[s] = *reinterpret_cast<const uint4*>(qrow + 16 * s + 8 * hf);
    const float2* trow = tab + (size_t)n * 64;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float y1[8], y2[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 cs = trow[16 * s + 8 * hf + e];
        rot_neg(bf16_at(raw[s], e), bf16_at(raw[s + 4], e), cs.x, cs.y, y1[e], y2[e]);
      }
      qop[s] = u32x4{pack_f16(y1[0], y1[1]), pack_f16(y1[2], y1[3]), pack_f16(y1[4], y1[5]),
                     pack_f16(y1[6], y1[7])};
      qop[s + 4] = u32x4{pack_f16(y2[0], y2[1]), pack_f16(y2[2], y2[3]), pack_f16(y2[4], y2[5]),
                         pack_f16(y2[6], y2[7])};
    }
    uint32_t part[8];
#pragma unroll
    for (int p = 0; p < kSelPairs; ++p) {
      const int m = args.sel[g * kSelPairs + p];
      const float x1 = __uint_as_float((uint32_t)qrow[m] << 16);
      const float x2 = __uint_as_float((uint32_t)qrow[m + 64] << 16);
      const float2 cs = trow[m];
      float y1, y2;
      rot_neg(x1, x2, cs.x, cs.y, y1, y2);
      uint32_t h1, l1, h2, l2;
      split_f16(y1, h1, l1);
      split_f16(y2, h2, l2);
      part[p] = hf ? l1 : h1;
      part[p + 4] = hf ? l2 : h2;
    }
    qcor = u32x4{part[0] | (part[1] << 16), part[2] | (part[3] << 16),
                 part[4] | (part[5] << 16), part[6] | (part[7] << 16)};
  };

  // ---- K/V staging: global -> registers -> LDS --------------------------------------
  // K: thread (key kr_ = tid/8, eighth kq = tid%8) holds channels 8kq..8kq+7 and their
  //    RoPE partners 64+8kq..; V: thread (key pair vr = tid%32, chunk vc = tid/32) holds
  //    channels 8vc..8vc+7 of keys 2vr, 2vr+1; the hi/lo correction of key tid/4, pair
  //    tid%4 is done by the first 256 threads.
  const int kr_ = tid >> 3, kq = tid & 7;
  const int vr = tid & 31, vc = tid >> 5;
  const int cr = (tid >> 2) & 63, cp = tid & 3;
  const bool c_thread = tid < 4 * BK;
  const int my_sel = args.sel[g * kSelPairs + cp];
  uint4 kraw[2], vraw[2];
  uint32_t ccor[2];   // selected pair (x1, x2) of key cr, pair my_sel, bf16 bits
  auto stage_load = [&](int kt) __attribute__((always_inline)) {
    const int j0 = kt * BK;
    {
      const int j = min(j0 + kr_, L - 1);
      const uint16_t* row = Kp + ((size_t)(start + j) * Hkv + g) * D + 8 * kq;
      kraw[0] = *reinterpret_cast<const uint4*>(row);
      kraw[1] = *reinterpret_cast<const uint4*>(row + 64);
    }
    if (c_thread) {
      const int j = min(j0 + cr, L - 1);
      const uint16_t* row = Kp + ((size_t)(start + j) * Hkv + g) * D;
      ccor[0] = row[my_sel];
      ccor[1] = row[my_sel + 64];
    }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int j = min(j0 + 2 * vr + k2, L - 1);
      vraw[k2] = *reinterpret_cast<const uint4*>(Vp + ((size_t)(start + j) * Hkv + g) * D + 8 * vc);
    }
  };
  auto stage_store = [&](int kt, int mode, Stage& st) __attribute__((always_inline)) {
    const int j0 = kt * BK;
    if (mode != kRemote) {
      uint16_t* dst = st.ks + kr_ * KS_LD + 8 * kq;
      *reinterpret_cast<uint4*>(dst) = kraw[0];
      *reinterpret_cast<uint4*>(dst + 64) = kraw[1];
    }
    if (mode != kLocal) {
      {
        const int j = min(j0 + kr_, L - 1);
        const int n = j - alias_pos(j, G);
        const float4* trow = reinterpret_cast<const float4*>(tab + (size_t)n * 64 + 8 * kq);
        float y1[8], y2[8];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const float4 cs = trow[e2];  // pairs 8kq + 2e2, +1
          rot_neg(bf16_at(kraw[0], 2 * e2), bf16_at(kraw[1], 2 * e2), cs.x, cs.y, y1[2 * e2],
                  y2[2 * e2]);
          rot_neg(bf16_at(kraw[0], 2 * e2 + 1), bf16_at(kraw[1], 2 * e2 + 1), cs.z, cs.w,
                  y1[2 * e2 + 1], y2[2 * e2 + 1]);
        }
        uint16_t* dst = st.kr + kr_ * KS_LD + 8 * kq;
        *reinterpret_cast<uint4*>(dst) =
            make_uint4(pack_f16(y1[0], y1[1]), pack_f16(y1[2], y1[3]), pack_f16(y1[4], y1[5]),
                       pack_f16(y1[6], y1[7]));
        *reinterpret_cast<uint4*>(dst + 64) =
            make_uint4(pack_f16(y2[0], y2[1]), pack_f16(y2[2], y2[3]), pack_f16(y2[4], y2[5]),
                       pack_f16(y2[6], y2[7]));
      }
      // hi/lo of the selected pair cp for key cr: [lo ch0..7 | hi ch0..7],
      // channel k = pair (k % 4), component (k / 4).
      if (c_thread) {
        const int j = min(j0 + cr, L - 1);
        const int n = j - alias_pos(j, G);
        const float2 cs = tab[(size_t)n * 64 + my_sel];
        float y1, y2;
        rot_neg(__uint_as_float(ccor[0] << 16), __uint_as_float(ccor[1] << 16), cs.x, cs.y, y1,
                y2);
        uint32_t h1, l1, h2, l2;
        split_f16(y1, h1, l1);
        split_f16(y2, h2, l2);
        uint16_t* row = st.kc + cr * KC_LD;
        row[cp] = (uint16_t)l1;
        row[4 + cp] = (uint16_t)l2;
        row[8 + cp] = (uint16_t)h1;
        row[12 + cp] = (uint16_t)h2;
      }
    }
    // V^T: vt[d][key], keys (2vr, 2vr+1) packed per 32-bit word
    {
      const uint32_t* a0 = reinterpret_cast<const uint32_t*>(&vraw[0]);  // key 2vr, d 8vc..+7
      const uint32_t* a1 = reinterpret_cast<const uint32_t*>(&vraw[1]);  // key 2vr+1
      uint32_t* dst = reinterpret_cast<uint32_t*>(st.vt) + vr;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int d = 8 * vc + 2 * w;
        dst[(d * VT_LD) / 2] = __byte_perm(a0[w], a1[w], 0x5410);
        dst[((d + 1) * VT_LD) / 2] = __byte_perm(a0[w], a1[w], 0x7632);
      }
    }
  };

  // ---- softmax state and output accumulators --------------------------------------
  f32x16 oacc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};  // O^T blocks [d block]
  float m_run = -1e30f, l_run = 0.f;
  const float c2 = args.scale * 1.4426950408889634f;  // scale * log2(e)

  auto tile_mode = [&](int kt) { return kt < ktA ? kRemote : kt < ktB ? kStraddle : kLocal; };

  // One tile of BK keys in two 32-key halves (mb): scores, online softmax, PV.
  auto compute = [&](int kt, const Stage& st, auto mode_c, bool need_mask)
      __attribute__((always_inline)) {
    constexpr int mode = decltype(mode_c)::value;
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
    if constexpr (mode == kLocal) {
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(st.ks + (32 * mb + ln) * KS_LD + 16 * s + 8 * hf);
          sacc[mb] = mfma_bf16(a, qop[s], sacc[mb]);
        }
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(st.kr + (32 * mb + ln) * KS_LD + 16 * s + 8 * hf);
          sacc[mb] = mfma_f16(a, qop[s], sacc[mb]);
        }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(st.kc + (32 * mb + ln) * KC_LD + 8 * hf);
        sacc[mb] = mfma_f16(a, qcor, sacc[mb]);
      }
    }
    if constexpr (mode == kStraddle) {
      // local scores with the exact bf16 operands, selected per pair by distance
      u32x4 qs[8];
      load_q_std(qs);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        f32x16 sl = f32x16{};
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(st.ks + (32 * mb + ln) * KS_LD + 16 * s + 8 * hf);
          sl = mfma_bf16(a, qs[s], sl);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = kt * BK + 32 * mb + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (qi - j < w0) sacc[mb][r] = sl[r];
        }
      }
    }

    // ---- online softmax (per query column, both lane halves) ----
    if (need_mask) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = kt * BK + 32 * mb + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (j > qi || j >= L) sacc[mb][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float cand = fmaxf(m_run, mx * c2);
    const bool need = cand > m_run + kLazy;
    if (__ballot(need)) {
      const float m_new = need ? cand : m_run;
      const float f = exp2f(m_run - m_new);
      l_run *= f;
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db] *= f;
      m_run = m_new;
    }
    const float mneg = -m_run;
    float lsum = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(__fmaf_rn(sacc[mb][r], c2, mneg));
        sacc[mb][r] = p;
        lsum += p;
      }
    l_run += lsum;

    // ---- O^T += V^T P^T (four K=16 steps) ----
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const f32x16& sv = sacc[mb];
        const u32x4 pb = u32x4{pack_bf16(sv[8 * t + 0], sv[8 * t + 1]), pack_bf16(sv[8 * t + 2], sv[8 * t + 3]),
                               pack_bf16(sv[8 * t + 4], sv[8 * t + 5]), pack_bf16(sv[8 * t + 6], sv[8 * t + 7])};
        const int kofs = 32 * mb + 16 * t + 4 * hf;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const uint16_t* vrow = st.vt + (32 * db + ln) * VT_LD + kofs;
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 8);
          oacc[db] = mfma_bf16(u32x4{lo.x, lo.y, hi.x, hi.y}, pb, oacc[db]);
        }
      }
  };

  // ---- main loop: remote tiles, then straddling tiles, then local tiles ----------
  auto iteration = [&](int kt, auto mode_c) __attribute__((always_inline)) {
    constexpr int mode = decltype(mode_c)::value;
    __syncthreads();
    if (kt + 1 < nkt) stage_load(kt + 1);
    const bool need_mask = mode != kRemote && kt * BK + BK - 1 > i0;  // diagonal / tail
    compute(kt, stg[kt & 1], mode_c, need_mask);
    if (kt + 1 < nkt) stage_store(kt + 1, tile_mode(kt + 1), stg[(kt + 1) & 1]);
  };
  if (ktB > 0) load_q_remote();
  stage_load(0);
  stage_store(0, tile_mode(0), stg[0]);
  int kt = 0;
  for (; kt < ktA; ++kt) iteration(kt, std::integral_constant<int, kRemote>());
  for (; kt < ktB; ++kt) iteration(kt, std::integral_constant<int, kStraddle>());
  load_q_std(qop);
  for (; kt < nkt; ++kt) iteration(kt, std::integral_constant<int, kLocal>());

  // ---- epilogue: O = O^T / l, LSE ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qi < L) {
    const float inv = 1.f / l_tot;
    uint16_t* orow = (uint16_t*)args.O + ((size_t)(start + qi) * Hq + qhead) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * db + 8 * q4 + 4 * hf;
        const f32x16& o = oacc[db];
        *reinterpret_cast<uint2*>(orow + d) =
            make_uint2(pack_bf16(o[4 * q4] * inv, o[4 * q4 + 1] * inv),
                       pack_bf16(o[4 * q4 + 2] * inv, o[4 * q4 + 3] * inv));
      }
    if (args.lse && hf == 0)
      args.lse[(size_t)qhead * args.T + start + qi] = (m_run + log2f(l_tot)) * 0.69314718055994530942f;
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_pair_select(const void* Q, const void* K, int T, int Hq, int Hkv,
                              uint32_t* mx /*[(Hq+Hkv)*64]*/, int32_t* sel, hipStream_t stream) {
  const int n = (Hq + Hkv) * 64;
  hipLaunchKernelGGL(pair_max_zero_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, mx, n);
  const int tpb = 256;  // tokens per block
  const int ty = (T + tpb - 1) / tpb;
  if (ty > 0) {
    hipLaunchKernelGGL(pair_max_kernel, dim3((Hq * 64 + 255) / 256, ty), dim3(256), 0, stream,
                       (const uint16_t*)Q, T, Hq, tpb, mx);
    hipLaunchKernelGGL(pair_max_kernel, dim3((Hkv * 64 + 255) / 256, ty), dim3(256), 0, stream,
                       (const uint16_t*)K, T, Hkv, tpb, mx + Hq * 64);
  }
  hipLaunchKernelGGL(pair_select_kernel, dim3((Hkv + 63) / 64), dim3(64), 0, stream, mx,
                     mx + Hq * 64, Hq, Hkv, sel);
  return hipGetLastError();
}

template <int REP>
static hipError_t launch_mfma_rep(const PrefillArgs& args, hipStream_t stream) {
  static bool attr_set = false;  // benign race: every caller sets the same value
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)prefill_mfma_kernel<REP>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)mf::kSmem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int blocks = args.Hkv * args.nseq * args.max_qblocks;
  hipLaunchKernelGGL(prefill_mfma_kernel<REP>, dim3(blocks), dim3(512), mf::kSmem, stream, args);
  return hipGetLastError();
}

hipError_t launch_prefill_mfma(const PrefillArgs& args, hipStream_t stream) {
  switch (args.Hq / args.Hkv) {
    case 1: return launch_mfma_rep<1>(args, stream);
    case 2: return launch_mfma_rep<2>(args, stream);
    case 4: return launch_mfma_rep<4>(args, stream);
    case 8: return launch_mfma_rep<8>(args, stream);
    default: return hipErrorInvalidValue;
  }
}

int prefill_mfma_positions_per_block(int rep) { return mf::ROWS / rep; }

}  // namespace bifocal
