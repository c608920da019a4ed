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
// Hq/Hkv query heads of the group; 8 waves, each wave 32 query rows, two per SIMD):
//   * S^T = K Q^T and O^T = V^T P^T with v_mfma_f32_32x32x16: the query is the MFMA
//     column, so every query row lives in one lane pair (l, l^32) and P goes from
//     the score accumulator to the PV operand without a trip through LDS.
//   * A key-preparation pass writes, once per call, a record per (KV head, 32-key
//     tile): the keys rotated to their remote positions (fp16), the hi/lo operand of
//     the selected pairs, and V transposed.  The main kernel copies records (remote
//     tiles) or K rows (local tiles) into an eight-slot LDS ring with LDS-DMA, six
//     tiles ahead, shared by all query heads of the group; the waves meet at a barrier
//     after every second tile.
//   * Tiles are classified from indices: the workgroup walks a remote pass (tiles with
//     remote pairs) and a local pass (tiles with window pairs); the few tiles that
//     straddle the window edge are visited by both passes, each masking the other
//     class, so every pair is scored once by its own rule.
//   * Local scores use the exact bf16 input bytes (bf16 MFMA), so G = 1 reproduces
//     plain causal attention.  Remote scores need the correction rotation R(f(x) - x)
//     (section 2, rotations compose additively), applied in fp32 registers once per
//     key and call (key preparation) and once per query row; the rotated operands are
//     rounded to fp16 (same MFMA rate as bf16 on gfx950, 3 more mantissa bits), and
//     for the 4 RoPE pairs per KV head with the largest |q||k| bound a hi/lo split adds
//     one K=16 MFMA step (hi*lo + lo*hi) so that outlier channels do not lose the
//     low-order bits of their products.  Operands near the fp16 range are first scaled
//     by exact powers of two chosen from the pre-pass maxima (undone in the softmax
//     scale and the output), so no input a bf16 tensor can hold overflows them.
//   * Online softmax in the base-2 domain with a lazy running max (rescale only when
//     the max grows by more than 8), row sums kept per lane half.  P and V^T enter the
//     PV product as fp16: with the lazy max a probability reaches 2^8, and a bf16 P
//     (8 significant bits) would put up to 2^-9 of relative error into the row sum, the
//     largest single term of the LSE error; fp16 keeps 11 bits at the same MFMA rate.
//   * The same kernel also runs the three passes of the pages' inclusion-exclusion
//     form (mode 1: remote over all causal pairs, 2: remote over the window, 3: local
//     over the window) and the continuous-position variant (remote angles x/G - x
//     evaluated in float64 instead of read from the table).
#include <type_traits>

#include "bf_common.h"
#include "mfma_util.h"
#include "prefill_args.h"

namespace bifocal {

namespace mf {
constexpr int D = 128;
constexpr int BK = 32;        // keys per tile (one 32-row MFMA block)
constexpr int NW = 8;         // waves per workgroup (32 query rows each)
constexpr int ROWS = 256;     // query rows (head, position) per workgroup
constexpr int KS_LD = D + 8;  // LDS row stride (16-bit elements) of the key operand: 272 B
// The key operand of a tile (remote fp16 copy or standard bf16 rows) occupies 32 rows
// of 17 16-byte chunks (one chunk of padding per row keeps the 128-bit operand reads
// conflict-free), filled by nine 1 KiB LDS-DMA transfers.
constexpr int K_CHUNKS = BK * (KS_LD / 8);  // 544
constexpr int K_DMA = 9;                    // 1 KiB transfers per key operand
// V^T rows (one per channel d) hold the tile's 32 keys as four 16-byte chunks; chunk c
// carries the keys one PV operand lane needs, {16t+4h .. +3, 16t+8+4h .. +3} for
// c = 2t + h, and sits at position c ^ ((d >> 2) & 3) so that the 16 lanes served
// together by a 128-bit LDS read hit 16 different bank groups.
constexpr int VT_LD = BK;
// hi/lo operand rows: 32 B = two chunks, chunk h at position h ^ ((key >> 3) & 1).
constexpr int KC_LD = 16;
constexpr float kLazy = 8.f;  // allowed growth of the running max before a rescale
constexpr float kLazySum = 256.f;  // 2^kLazy

struct Stage {
  uint16_t k[K_DMA * 512];  // key operand: remote fp16 or standard bf16, padded rows
  uint16_t kc[BK * KC_LD];  // [lo of 8 selected channels | hi of them], fp16 bits
  uint16_t vt[D * VT_LD];   // V^T 2^-e_v, fp16 bits, swizzled chunks (see VT_LD)
};
static_assert(sizeof(Stage) == 18432, "stage = 18 KiB");
constexpr int NSTAGE = 8;          // LDS ring of virtual tiles
// Tiles issued ahead of the one being computed.  The workgroup meets at a barrier
// after every second tile, so a slot is refilled two tiles after its last use.
constexpr int PREF = NSTAGE - 2;
constexpr size_t kSmem = NSTAGE * sizeof(Stage);

}  // namespace mf

// ---------------------------------------------------------------------------
// Pre-pass: per (head, RoPE pair) maximum of the squared pair norm over all tokens.
// Pair norms are rotation invariant, so the maxima over the standard-RoPE inputs
// bound the remote (rotated) operands too.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) pair_max_zero_kernel(uint32_t* mx, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) mx[i] = 0u;
}

// Thread (token lane tl, chunk lane cl): chunk ch = 64 blockIdx.x + cl of the H * 8
// chunks of a token (head ch / 8, pairs 8 (ch % 8) .. +7: two 16-byte streaming loads of
// the row halves), tokens t0 + tl, t0 + tl + 4, ...  A wave reads 64 consecutive chunks
// of one token (2 KiB contiguous); the four token lanes meet in LDS before the atomics.
__global__ void __launch_bounds__(256) pair_max_kernel(const uint16_t* __restrict__ X, int T,
                                                       int H, int tok_per_block,
                                                       uint32_t* __restrict__ mx) {
  __shared__ float s_best[4][64][9];
  const int tl = threadIdx.x >> 6, cl = threadIdx.x & 63;
  const int ch = blockIdx.x * 64 + cl;
  const bool live = ch < H * 8;
  const int h = ch >> 3, c = ch & 7;
  const int t0 = blockIdx.y * tok_per_block;
  const int t1 = min(T, t0 + tok_per_block);
  float best[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (live) {
    for (int t = t0 + tl; t < t1; t += 4) {
      const uint16_t* row = X + ((size_t)t * H + h) * mf::D + 8 * c;
      const u32x4 a = ld_stream(row), b = ld_stream(row + 64);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = __uint_as_float(e & 1 ? a[e >> 1] & 0xffff0000u : a[e >> 1] << 16);
        const float y = __uint_as_float(e & 1 ? b[e >> 1] & 0xffff0000u : b[e >> 1] << 16);
        best[e] = fmaxf(best[e], x * x + y * y);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) s_best[tl][cl][e] = best[e];
  __syncthreads();
  // thread (e, cl) for e < 4 and e + 4: one pair of the chunk each
  const int cl2 = threadIdx.x & 63, e0 = threadIdx.x >> 6;
  const int ch2 = blockIdx.x * 64 + cl2;
  if (ch2 < H * 8) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = e0 + 4 * k;
      const float m = fmaxf(fmaxf(s_best[0][cl2][e], s_best[1][cl2][e]),
                            fmaxf(s_best[2][cl2][e], s_best[3][cl2][e]));
      // non-negative floats order as integers
      atomicMax(mx + (ch2 >> 3) * 64 + 8 * (ch2 & 7) + e, __float_as_uint(m));
    }
  }
}

// Smallest e >= 0 with sqrt(m) * 2^-e < 2^15, for a maximum squared pair norm m: every
// component of a pair (rotated or not) scaled by 2^-e then fits fp16 (max 65504).
__device__ __forceinline__ int fp16_range_exp(float m) {
  if (!(m > 0x1p30f)) return 0;
  if (!(m < INFINITY)) return 64;
  int x;
  frexpf(m, &x);  // m < 2^x
  return (x - 29) >> 1;
}

// Argmax over the 64 lanes of a wave (lane = RoPE pair); the lowest pair wins a tie.
__device__ __forceinline__ void wave_argmax(float v, int& bi, float& bv) {
  bv = v;
  bi = threadIdx.x & 63;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(bv, o);
    const int oi = __shfl_xor(bi, o);
    if (ov > bv || (ov == bv && oi < bi)) {
      bv = ov;
      bi = oi;
    }
  }
}

// Per KV head (one wave, lane = RoPE pair m):
//  * the kSelPairs pairs with the largest sum_h |q_h,m|^2 * |k_m|^2 (maxima over the
//    tokens) get the hi/lo correction on both sides for every query head of the group
//    (the key-tile records carry their key remainders): the sum ranks first the pairs
//    that are large in the key, whose rounding errors reach every head;
//  * the operand exponents of the group's remote queries, remote keys and values.
__global__ void __launch_bounds__(64) pair_select_kernel(const uint32_t* __restrict__ mxq,
                                                         const uint32_t* __restrict__ mxk,
                                                         const uint32_t* __restrict__ mxv,
                                                         int Hq, int Hkv,
                                                         int32_t* __restrict__ sel) {
  const int g = blockIdx.x, m = threadIdx.x;
  const int rep = Hq / Hkv;
  int32_t* rec = sel + g * kSelStride;
  float q = 0.f, qsum = 0.f;
  for (int r = 0; r < rep; ++r) {
    const float x = __uint_as_float(mxq[(g * rep + r) * 64 + m]);
    q = fmaxf(q, x);
    qsum += x;
  }
  const float kk = __uint_as_float(mxk[g * 64 + m]);
  float vv = __uint_as_float(mxv[g * 64 + m]);
  const float bound = qsum * kk;  // >= 0
  bool taken = false;
  for (int p = 0; p < kSelPairs; ++p) {
    int bi;
    float bv;
    wave_argmax(taken ? -1.f : bound, bi, bv);
    if (m == 0) rec[p] = bi;
    if (m == bi) taken = true;
  }
  float qm = q, km = kk;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    qm = fmaxf(qm, __shfl_xor(qm, o));
    km = fmaxf(km, __shfl_xor(km, o));
    vv = fmaxf(vv, __shfl_xor(vv, o));
  }
  if (m == 0) {
    rec[kSelExpQ] = fp16_range_exp(qm);
    rec[kSelExpK] = fp16_range_exp(km);
    rec[kSelExpV] = fp16_range_exp(vv);
  }
}

// ---------------------------------------------------------------------------
// Key preparation: once per call, each key tile of each KV head is turned into the
// record the main kernel copies into LDS verbatim (layout in prefill_args.h): the
// remote copy R(f(j) - j) K_j 2^-e_k rounded to fp16, the hi/lo correction of the
// selected pairs, and V^T 2^-e_v in fp16 (the PV operands are fp16: P keeps 11
// significant bits instead of 8).  A key is rotated once here instead of once per query block that
// reads it.  One workgroup (256 threads) per (tile, KV head).
// ---------------------------------------------------------------------------
// INTERP: continuous remote positions (angles evaluated in fp64 here, no table); a
// separate instantiation keeps the table path's register allocation small.
template <bool INTERP>
__global__ void __launch_bounds__(256) key_prep_kernel(PrefillArgs args) {
  using namespace mf;
  __shared__ __align__(16) uint16_t sv[BK][D + 8];
  __shared__ __align__(16) float sy[BK][D + 4];  // rotated keys, natural channel order
  __shared__ double s_invf[D / 2];  // theta_m (continuous remote positions only)
  const int g = blockIdx.y;
  const int t_local = blockIdx.x;
  const int base0 = args.seq[0].tile_base;
  int b = 0;
  for (int q = 1; q < args.nseq; ++q)
    if (args.seq[q].tile_base - base0 <= t_local) b = q;
  const int kt = t_local - (args.seq[b].tile_base - base0);
  const int L = args.seq[b].len;
  const int start = args.seq[b].start;
  const int G = args.seq[b].G;
  const DivMagic gdiv{args.seq[b].gmul, args.seq[b].gshift};
  const int Hkv = args.Hkv;
  const uint16_t* __restrict__ Kp = (const uint16_t*)args.K;
  const uint16_t* __restrict__ Vp = (const uint16_t*)args.V;
  const float2* __restrict__ tab = args.tab;
  uint8_t* rec = args.rec + ((size_t)g * args.tiles_total + args.seq[b].tile_base + kt) * kRecBytes;
  uint16_t* kr = reinterpret_cast<uint16_t*>(rec);
  uint16_t* kc = reinterpret_cast<uint16_t*>(rec + kRecKr);
  uint16_t* vt = reinterpret_cast<uint16_t*>(rec + kRecKr + kRecKc);

  const int tid = threadIdx.x;
  const int k = tid >> 3, p = tid & 7;  // key of the tile; pairs 8p .. 8p+7
  constexpr bool interp = INTERP;
  const double rpos = (double)(G - 1) / (double)G;  // continuous: n(x) = x - x/G = x rpos
  if constexpr (interp) {
    if (tid < D / 2) s_invf[tid] = inv_freq64(args.theta, tid, D);
    __syncthreads();
  }
  const int j = kt * BK + k;
  const bool valid = j < L;
  const size_t row_off = ((size_t)(start + min(j, L - 1)) * Hkv + g) * D;
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  // exact power-of-two operand scales (1 unless an input is near the fp16 range)
  const float ks = __builtin_ldexpf(1.f, -args.sel[g * kSelStride + kSelExpK]);
  const float vs = __builtin_ldexpf(1.f, -args.sel[g * kSelStride + kSelExpV]);
  {
    const uint4 v0 = valid ? *reinterpret_cast<const uint4*>(Vp + row_off + 8 * p) : zero;
    const uint4 v1 = valid ? *reinterpret_cast<const uint4*>(Vp + row_off + 64 + 8 * p) : zero;
    uint4 h0, h1;
    h0.x = pack_f16(bf16_at(v0, 0) * vs, bf16_at(v0, 1) * vs);
    h0.y = pack_f16(bf16_at(v0, 2) * vs, bf16_at(v0, 3) * vs);
    h0.z = pack_f16(bf16_at(v0, 4) * vs, bf16_at(v0, 5) * vs);
    h0.w = pack_f16(bf16_at(v0, 6) * vs, bf16_at(v0, 7) * vs);
    h1.x = pack_f16(bf16_at(v1, 0) * vs, bf16_at(v1, 1) * vs);
    h1.y = pack_f16(bf16_at(v1, 2) * vs, bf16_at(v1, 3) * vs);
    h1.z = pack_f16(bf16_at(v1, 4) * vs, bf16_at(v1, 5) * vs);
    h1.w = pack_f16(bf16_at(v1, 6) * vs, bf16_at(v1, 7) * vs);
    *reinterpret_cast<uint4*>(&sv[k][8 * p]) = h0;
    *reinterpret_cast<uint4*>(&sv[k][64 + 8 * p]) = h1;
  }
  // G = 1 in the bifocal mode: every pair is local, the remote copy is never read (the
  // inclusion-exclusion passes read it whatever G is)
  if (G > 1 || args.mode != 0) {
    if (valid) {
      const uint4 a = *reinterpret_cast<const uint4*>(Kp + row_off + 8 * p);
      const uint4 c = *reinterpret_cast<const uint4*>(Kp + row_off + 64 + 8 * p);
      const float4* trow =
          reinterpret_cast<const float4*>(tab + (size_t)(j - alias_fast(j, gdiv)) * 64 + 8 * p);
      float y1[8], y2[8];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        float4 cs;
        if (interp) {
          const float2 c0 = angle_cs(j * rpos, s_invf[8 * p + 2 * e2]);
          const float2 c1 = angle_cs(j * rpos, s_invf[8 * p + 2 * e2 + 1]);
          cs = make_float4(c0.x, c0.y, c1.x, c1.y);
        } else {
          cs = trow[e2];
        }
        rot_neg(bf16_at(a, 2 * e2), bf16_at(c, 2 * e2), cs.x, cs.y, y1[2 * e2], y2[2 * e2]);
        rot_neg(bf16_at(a, 2 * e2 + 1), bf16_at(c, 2 * e2 + 1), cs.z, cs.w, y1[2 * e2 + 1],
                y2[2 * e2 + 1]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y1[e] *= ks;
        y2[e] *= ks;
      }
      float* r1 = &sy[k][8 * p];
      float* r2 = &sy[k][64 + 8 * p];
      *reinterpret_cast<float4*>(r1) = make_float4(y1[0], y1[1], y1[2], y1[3]);
      *reinterpret_cast<float4*>(r1 + 4) = make_float4(y1[4], y1[5], y1[6], y1[7]);
      *reinterpret_cast<float4*>(r2) = make_float4(y2[0], y2[1], y2[2], y2[3]);
      *reinterpret_cast<float4*>(r2 + 4) = make_float4(y2[4], y2[5], y2[6], y2[7]);
    } else {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        *reinterpret_cast<uint4*>(&sy[k][64 * q + 8 * p]) = zero;
        *reinterpret_cast<uint4*>(&sy[k][64 * q + 8 * p + 4]) = zero;
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint32_t h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        h[e] = pack_f16(sy[k][64 * q + 8 * p + 2 * e], sy[k][64 * q + 8 * p + 2 * e + 1]);
      *reinterpret_cast<uint4*>(kr + k * D + 64 * q + 8 * p) = make_uint4(h[0], h[1], h[2], h[3]);
    }
    if (tid < 4 * BK) {
      // hi/lo of selected pair cp of key ck: [lo ch0..7 | hi ch0..7], channel
      // q = pair (q % 4), component (q / 4)
      const int ck = tid >> 2, cp = tid & 3;
      const int m = args.sel[g * kSelStride + cp];
      uint32_t h1, l1, h2, l2;  // zero past the sequence's end (staged zeros)
      split_f16(sy[ck][m], h1, l1);
      split_f16(sy[ck][m + 64], h2, l2);
      uint16_t* crow = kc + ck * 16;
      const int lo_at = 8 * ((ck >> 3) & 1), hi_at = 8 - lo_at;  // swizzled chunks
      crow[lo_at + cp] = (uint16_t)l1;
      crow[lo_at + 4 + cp] = (uint16_t)l2;
      crow[hi_at + cp] = (uint16_t)h1;
      crow[hi_at + 4 + cp] = (uint16_t)h2;
    }
  }
  __syncthreads();
  // V^T [d][32 keys] in 16-byte chunks: physical chunk pc of row d holds logical chunk
  // c = pc ^ ((d >> 2) & 3), i.e. keys {16t+4h .. +3, 16t+8+4h .. +3} with c = 2t + h.
#pragma unroll
  for (int q = tid; q < D * 4; q += 256) {
    const int d = q >> 2, pc = q & 3;
    const int c = pc ^ ((d >> 2) & 3);
    const int k0 = 16 * (c >> 1) + 4 * (c & 1);
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 2; ++e)
      w[e] = (uint32_t)sv[k0 + 2 * e][d] | ((uint32_t)sv[k0 + 2 * e + 1][d] << 16);
#pragma unroll
    for (int e = 0; e < 2; ++e)
      w[2 + e] = (uint32_t)sv[k0 + 8 + 2 * e][d] | ((uint32_t)sv[k0 + 8 + 2 * e + 1][d] << 16);
    *reinterpret_cast<uint4*>(vt + d * BK + 8 * pc) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// ---------------------------------------------------------------------------
// Main kernel
// ---------------------------------------------------------------------------
// Wait until at most N vector-memory operations of this wave are outstanding and all
// its LDS operations are done, then meet the other waves.  Raw barrier: the ordinary
// workgroup barrier also drains every LDS-DMA transfer in flight (vmcnt 0), which
// would cut the prefetch depth to zero.  The empty asm statements keep the compiler
// from moving memory operations across.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));  // vmcnt(N) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// The same with a count per wave: wave 0 issues more transfers per tile (the ninth
// key-operand KiB and the hi/lo correction rows) than the other waves.
template <int N0, int N>
__device__ __forceinline__ void wait_vm_barrier_w(int wave) {
  static_assert(N0 >= 0 && N0 < 64 && N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  if (wave == 0)
    __builtin_amdgcn_s_waitcnt((N0 & 15) | (7 << 4) | ((N0 >> 4) << 14));
  else
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The same with the wave's role known at compile time.
template <int N0, int N, bool W0>
__device__ __forceinline__ void wait_vm_barrier_s() {
  static_assert(N0 >= 0 && N0 < 64 && N >= 0 && N < 64, "vmcnt range");
  constexpr int M = W0 ? N0 : N;
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((M & 15) | (7 << 4) | ((M >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int REP>
__global__ void __launch_bounds__(512) prefill_mfma_kernel(PrefillArgs args) {
  using namespace mf;
  extern __shared__ __align__(16) uint8_t smem_raw[];

  constexpr int BMPOS = ROWS / REP;       // query positions per workgroup
  constexpr int PBLK = BMPOS / 32;        // 32-row position blocks per head

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0 .. NW-1
  const int ln = lane & 31;               // MFMA column / row within a 32-block
  const int hf = lane >> 5;               // lane half

  // Workgroup -> (KV head, sequence, query block).  KV head is the fastest index so
  // that the workgroups of one head share an XCD's L2; (sequence, block) pairs run
  // heaviest-first over the launch's levels, and every workgroup has rows.
  const int Hkv = args.Hkv;
  const int g = blockIdx.x % Hkv;
  const int pid = blockIdx.x / Hkv;
  int lv = 0;
  while (lv + 1 < args.nlvl && args.lvl_start[lv + 1] <= pid) ++lv;
  const int r_in = pid - args.lvl_start[lv];
  const int qb = args.lvl_qb[lv] - 1 - r_in / (lv + 1);
  const int b = args.lvl_seq[r_in % (lv + 1)];
  const int L = args.seq[b].len;
  const int i0 = qb * BMPOS;
  const int start = args.seq[b].start;
  const int G = args.seq[b].G;
  const DivMagic gdiv{args.seq[b].gmul, args.seq[b].gshift};
  const int Hq = args.Hq;
  const int i_end = min(L, i0 + BMPOS);  // exclusive
  const int mode = args.mode;
  // G = 1: the aliased positions are the true ones, every pair is "local".  The
  // remote-over-all-causal-pairs pass classifies with w0 = 0 (every pair remote).
  const int w0 = mode == 0 ? (G == 1 ? (1 << 30) : args.w0) : (mode == 1 ? 0 : args.w0);

  const uint16_t* __restrict__ Qp = (const uint16_t*)args.Q;
  const uint16_t* __restrict__ Kp = (const uint16_t*)args.K;
  const float2* __restrict__ tab = args.tab;
  // continuous remote positions: n(x) = x - x/G, angles evaluated here (theta_m in LDS)
  const bool interp = args.interp != 0;
  const double rpos = (double)(G - 1) / (double)G;
  __shared__ double s_invf[D / 2];
  if (interp) {
    if (tid < D / 2) s_invf[tid] = inv_freq64(args.theta, tid, D);
    __syncthreads();  // no transfer is in flight yet
  }

  // ---- this wave's 32-query block -------------------------------------------------
  const int qhead = g * REP + wave / PBLK;
  const int qi = i0 + 32 * (wave % PBLK) + ln;  // query position of this lane's column
  const int qrow_i = min(qi, L - 1);
  const uint16_t* qrow = Qp + ((size_t)(start + qrow_i) * Hq + qhead) * D;

  // ---- tile ranges --------------------------------------------------------------
  // Physical key tiles [0,ktA) are remote for every query of the block, [ktB,nkt) local,
  // [ktA,ktB) straddle the window edge.  The block walks a sequence of virtual tiles:
  // a remote pass over [0,ktB), then a local pass over [ktA,nkt); on straddling tiles
  // each pass masks the pairs of the other class, so every pair is scored once, by its
  // own rule, in one online softmax.  The inclusion-exclusion passes walk: remote over
  // [0,nkt) with causal masks (mode 1), remote over the window tiles [ktA,nkt) with the
  // window mask (mode 2), local over [ktA,nkt) (mode 3).
  const int nkt = (i_end - 1) / BK + 1;
  int ktA, ktB;
  {
    const long long x = (long long)i0 - w0 - (BK - 1);
    ktA = x >= 0 ? (int)(x / BK) + 1 : 0;
    const long long y = (long long)(i_end - 1) - w0;
    ktB = y >= 0 ? (int)(y / BK) + 1 : 0;
    ktA = min(ktA, nkt);
    ktB = min(max(ktB, ktA), nkt);
  }
  // remote pass: physical tiles [r0, r0 + nr); local pass: [ktA, ktA + nl)
  const int r0 = mode == 2 ? ktA : 0;
  const int nr = mode == 0 ? ktB : (mode == 3 ? 0 : nkt - r0);
  const int nl = (mode == 0 || mode == 3) ? nkt - ktA : 0;
  const int nvt = nr + nl;
  auto vt_kt = [&](int v) __attribute__((always_inline)) { return v < nr ? r0 + v : ktA + (v - nr); };

  // ---- query operands -------------------------------------------------------------
  // B operand of S^T = K Q^T: lane (column ln, half hf) holds channels 16s + 8hf + e.
  // Local pass: the bf16 query.  Remote pass: the fp16 of R(f(i)-i) q 2^-e_q.
  u32x4 qop[8];
  u32x4 qcor;     // hi (half 0) or lo (half 1) of the 8 channels of the both-sided pairs
  auto load_q_std = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 8; ++s) qop[s] = *reinterpret_cast<const u32x4*>(qrow + 16 * s + 8 * hf);
  };
  const float qs = __builtin_ldexpf(1.f, -args.sel[g * kSelStride + kSelExpQ]);
  // Runs before any transfer into the LDS ring, whose space holds the rotated rows of
  // each wave meanwhile (float32) for the gather of the corrected pairs' channels; the
  // workgroup meets twice.
  auto load_q_remote = [&]() __attribute__((always_inline)) {
    constexpr int QS_LD = D + 4;  // floats per staged row
    float* stg = reinterpret_cast<float*>(smem_raw) + wave * (32 * QS_LD) + ln * QS_LD;
    const int n = qrow_i - alias_fast(qrow_i, gdiv);
    uint4 raw[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) raw[s] = *reinterpret_cast<const uint4*>(qrow + 16 * s + 8 * hf);
    const float2* trow = tab + (size_t)n * 64;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float y1[8], y2[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 cs = interp ? angle_cs(qrow_i * rpos, s_invf[16 * s + 8 * hf + e])
                                 : trow[16 * s + 8 * hf + e];
        rot_neg(bf16_at(raw[s], e), bf16_at(raw[s + 4], e), cs.x, cs.y, y1[e], y2[e]);
        y1[e] *= qs;
        y2[e] *= qs;
      }
      // channels 16s + 8hf + e (s < 4) and their partners (operand s + 4)
      qop[s] = u32x4{pack_f16(y1[0], y1[1]), pack_f16(y1[2], y1[3]), pack_f16(y1[4], y1[5]),
                     pack_f16(y1[6], y1[7])};
      qop[s + 4] = u32x4{pack_f16(y2[0], y2[1]), pack_f16(y2[2], y2[3]), pack_f16(y2[4], y2[5]),
                         pack_f16(y2[6], y2[7])};
      float* r1 = stg + 16 * s + 8 * hf;
      float* r2 = r1 + 64;
      *reinterpret_cast<float4*>(r1) = make_float4(y1[0], y1[1], y1[2], y1[3]);
      *reinterpret_cast<float4*>(r1 + 4) = make_float4(y1[4], y1[5], y1[6], y1[7]);
      *reinterpret_cast<float4*>(r2) = make_float4(y2[0], y2[1], y2[2], y2[3]);
      *reinterpret_cast<float4*>(r2 + 4) = make_float4(y2[4], y2[5], y2[6], y2[7]);
    }
    __syncthreads();
    uint32_t part[8];
#pragma unroll
    for (int p = 0; p < kSelPairs; ++p) {
      const int m = args.sel[g * kSelStride + p];
      uint32_t h1, l1, h2, l2;
      split_f16(stg[m], h1, l1);
      split_f16(stg[m + 64], h2, l2);
      part[p] = hf ? l1 : h1;
      part[p + 4] = hf ? l2 : h2;
    }
    qcor = u32x4{part[0] | (part[1] << 16), part[2] | (part[3] << 16),
                 part[4] | (part[5] << 16), part[6] | (part[7] << 16)};
    __syncthreads();  // every wave has read its rows before the ring is refilled
  };

  // ---- staging: LDS-DMA straight from the key-tile records / K rows ----------------
  // Wave w moves key-operand transfer w (wave 0 also transfer 8, the hi/lo operand of
  // remote tiles) and V^T kilobyte w.  Lane l of key transfer i fills padded position
  // p = 64 i + l: row p / 17, chunk p % 17 (chunk 16 and rows past 31 are padding and
  // take a harmless dummy copy).  Every wave issues at least two transfers per virtual
  // tile, which the vmcnt bound of the loop relies on.
  const uint8_t* rec_seq =
      args.rec + ((size_t)g * args.tiles_total + args.seq[b].tile_base) * kRecBytes;
  const uint16_t* kseq = Kp + ((size_t)start * Hkv + g) * D;
  const uint32_t krow_stride = (uint32_t)Hkv * D;  // elements between tokens
  // Per lane of key transfers wave and 8: byte offset in a record (remote tiles) and
  // the padded row / chunk (local tiles); addresses are a uniform base plus a 32-bit
  // lane offset, which keeps no 64-bit pointers live per lane.
  uint32_t krec_off[2], krow_r[2], kcol_b[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int p = 64 * (q == 0 ? wave : 8) + lane;
    const int r = p / 17, c = p % 17;
    const bool real = c < 16 && r < BK;
    krow_r[q] = real ? r : 0;
    kcol_b[q] = real ? 16 * c : 0;
    krec_off[q] = krow_r[q] * 256 + kcol_b[q];
  }
  const uint32_t lane16 = 16 * lane;
  const uint32_t krow_bytes = 2 * krow_stride;
  // REMSRC: the caller knows that tile v is a remote tile before the end (v < nr)
  // W0: the caller is wave 0, which also moves the ninth key-operand KiB and the hi/lo
  // correction rows
  auto issue = [&](int v, int so, auto remsrc_c, auto w0_c) __attribute__((always_inline)) {
    constexpr bool REMSRC = decltype(remsrc_c)::value;
    constexpr bool W0 = decltype(w0_c)::value;
    if (!REMSRC) v = min(v, nvt - 1);  // past the end: repeat the last tile (keeps the vmcnt count)
    const int kt = REMSRC ? r0 + v : vt_kt(v);
    uint8_t* st = smem_raw + so;
    const uint8_t* rec = rec_seq + (size_t)kt * kRecBytes;
    if (REMSRC || v < nr) {
      dma16_at(rec, krec_off[0], st + offsetof(Stage, k) + 1024 * wave);
      if constexpr (W0) {
        dma16_at(rec, krec_off[1], st + offsetof(Stage, k) + 1024 * 8);
        dma16_at(rec, kRecKr + lane16, st + offsetof(Stage, kc));
      }
    } else {
      const uint8_t* kb = reinterpret_cast<const uint8_t*>(kseq);
#pragma unroll
      for (int q = 0; q < 2; ++q)
        if (q == 0 || W0) {
          const uint32_t j = min((uint32_t)(kt * BK) + krow_r[q], (uint32_t)(L - 1));
          dma16_at(kb, j * krow_bytes + kcol_b[q], st + offsetof(Stage, k) + 1024 * (q == 0 ? wave : 8));
        }
    }
    dma16_at(rec, (kRecKr + kRecKc + 1024 * wave) + lane16, st + offsetof(Stage, vt) + 1024 * wave);
  };
  constexpr int kStageBytes = (int)sizeof(Stage);
  auto slot = [&](int v) __attribute__((always_inline)) { return (v % NSTAGE) * kStageBytes; };

  // ---- softmax state and output accumulators --------------------------------------
  f32x16 oacc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};  // O^T blocks [d block]
  float m_run = -1e30f, l_run = 0.f;
  const float c2l = args.scale * 1.4426950408889634f;  // scale * log2(e): local scores
  // remote scores come from operands scaled by 2^-e_q and 2^-e_k
  const float c2r = __builtin_ldexpf(c2l, args.sel[g * kSelStride + kSelExpQ] +
                                              args.sel[g * kSelStride + kSelExpK]);

  // Scores S^T (32 keys x this wave's 32 queries) of one virtual tile.
  auto qk_remote = [&](int so) __attribute__((always_inline)) -> f32x16 {
    const Stage& st = *reinterpret_cast<const Stage*>(smem_raw + so);
    f32x16 sacc = f32x16{};
    const uint16_t* krow = st.k + ln * KS_LD + 8 * hf;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      sacc = mfma_f16(*reinterpret_cast<const u32x4*>(krow + 16 * s), qop[s], sacc);
    const uint16_t* crow = st.kc + ln * KC_LD + 8 * (hf ^ ((ln >> 3) & 1));
    return mfma_f16(*reinterpret_cast<const u32x4*>(crow), qcor, sacc);
  };
  auto qk_local = [&](int so) __attribute__((always_inline)) -> f32x16 {
    const Stage& st = *reinterpret_cast<const Stage*>(smem_raw + so);
    f32x16 sacc = f32x16{};
    const uint16_t* krow = st.k + ln * KS_LD + 8 * hf;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      sacc = mfma_bf16(*reinterpret_cast<const u32x4*>(krow + 16 * s), qop[s], sacc);
    return sacc;
  };

  // Online softmax with a lazy running max m_run (base 2): m_run moves only when a row's
  // scores pass it by more than kLazy, so probabilities stay at most 2^kLazy.
  // Masks: MK = 1: remote pass over a straddling tile, keep i - j >= w0.  MK = 2: local
  // pass over a straddling or diagonal tile, keep 0 <= i - j < w0 (window and causality
  // in one unsigned compare).
  auto apply_mask = [&](int v, f32x16& sacc, auto mk_c) __attribute__((always_inline)) {
    constexpr int MK = decltype(mk_c)::value;
    if constexpr (MK != 0) {
      const int kt = vt_kt(v);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = kt * BK + 8 * (r >> 2) + 4 * hf + (r & 3);
        const bool drop = MK == 1 ? qi - j < w0 : (uint32_t)(qi - j) >= (uint32_t)w0;
        if (drop) sacc[r] = -INFINITY;
      }
    }
  };
  // The lazy rule on the tile's row max: a new m_run when the max passes it by more than
  // kLazy, with the output and row sum rescaled to it.
  auto rescale = [&](const f32x16& sacc, float c2) __attribute__((always_inline)) {
    float mx = sacc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
    mx = max_lane_xor32(mx);
    const float cand = fmaxf(m_run, mx * c2);
    const bool need = cand > m_run + kLazy;
    if (__ballot(need)) {
      const float m_new = need ? cand : m_run;
      const float f = fast_exp2(m_run - m_new);
      l_run *= f;
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db] *= f;
      m_run = m_new;
    }
  };
  // Probabilities against m_run in the PV operand layout (fp16, round to nearest even)
  // and the sum of this lane's 16 of them.  The row sum adds the same rounded
  // probabilities that PV multiplies (two per v_dot2 against (1, 1), fp32 accumulation),
  // so numerator and denominator agree.
  auto softmax_exp = [&](const f32x16& sacc, uint32_t* pk, float c2) __attribute__((always_inline)) -> float {
    const float mneg = -m_run;
    const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
    float t0 = 0.f, t1 = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = fast_exp2(__fmaf_rn(sacc[r], c2, mneg));
      const float p1 = fast_exp2(__fmaf_rn(sacc[r + 1], c2, mneg));
      const f16x2 ph = {(_Float16)p0, (_Float16)p1};
      pk[r / 2] = __builtin_bit_cast(uint32_t, ph);
      float& acc = (r & 2) ? t1 : t0;
      acc = __builtin_amdgcn_fdot2(ph, ones, acc, false);
    }
    return t0 + t1;
  };
  // O^T += V^T P^T over the tile's 32 keys.
  auto pv = [&](const uint32_t* pk, int so) __attribute__((always_inline)) {
    const Stage& st = *reinterpret_cast<const Stage*>(smem_raw + so);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const u32x4 pb = u32x4{pk[4 * t], pk[4 * t + 1], pk[4 * t + 2], pk[4 * t + 3]};
      const uint16_t* vrow = st.vt + ln * VT_LD + 8 * ((2 * t + hf) ^ ((ln >> 2) & 3));
#pragma unroll
      for (int db = 0; db < 4; ++db)
        oacc[db] = mfma_f16(*reinterpret_cast<const u32x4*>(vrow + 32 * VT_LD * db), pb, oacc[db]);
    }
  };

  // ---- software-pipelined loop over virtual tiles ----------------------------------
  // Iteration v: later tiles are in flight (LDS-DMA), v+1 is scored (MFMA) while v
  // goes through the softmax (VALU) and PV (MFMA).  The waves meet after odd
  // iterations only: the barrier closing iteration v (odd) must see tiles up to v+3
  // landed (read in iterations v+1 and v+2); the younger transfers (tiles v+4 ..
  // v+PREF, at least two per tile) may still be in flight.  Iteration v refills the
  // slot of tile v-2, whose last reader (iteration v-2) is behind a barrier.
  constexpr int kVmAhead = 2 * (PREF - 3);    // waves 1..7: two transfers per tile
  constexpr int kVmAhead0 = 3 * (PREF - 3);   // wave 0: three (local tile) or four
  // The tile walk, compiled once for wave 0 and once for the other waves (wave 0 moves
  // more per tile), so that no transfer or wait tests the wave.
  auto walk = [&](auto w0_c) __attribute__((always_inline)) {
    if (nr > 0) load_q_remote();
    else load_q_std();
  #pragma unroll
    for (int u = 0; u < PREF; ++u) issue(u, u * kStageBytes, std::false_type(), w0_c);
    wait_vm_barrier_s<kVmAhead0, kVmAhead, decltype(w0_c)::value>();  // tiles 0 .. 2 in LDS
    f32x16 s_cur = nr > 0 ? qk_remote(0) : qk_local(0);

    // Tile v+1 always has an LDS slot holding valid data (issue() repeats the last tile),
    // so its scores are computed unconditionally and simply unused past the end.  Two
    // score register sets alternate between consecutive tiles (no copy per tile).
    auto step = [&](int v, const f32x16& s_in, f32x16& s_out, auto qkrem_c, auto mk_c,
                    auto remsrc_c) __attribute__((always_inline)) {
      constexpr bool QKREM = decltype(qkrem_c)::value;  // class of tile v+1's scores
      issue(v + PREF, slot(v + PREF), remsrc_c, w0_c);
      // Tile v+1's score MFMAs and tile v's exponentials (independent of each other) share
      // one basic block and interleave.
      f32x16 sc = s_in;
      // class of tile v (wave-uniform; remote wherever the issued tiles are)
      const float c2 = decltype(remsrc_c)::value || v < nr ? c2r : c2l;
      apply_mask(v, sc, mk_c);
      s_out = QKREM ? qk_remote(slot(v + 1)) : qk_local(slot(v + 1));
      // Probabilities against the current m_run first, the row max only when needed: a
      // lane's probabilities are each at most their sum, so sums of at most 2^kLazy mean
      // that no score passed m_run by more than kLazy (the lazy rule keeps m_run).  Larger
      // sums (the first tiles of a row, a rising max) take the rule on the tile's max and
      // recompute the probabilities.
      uint32_t pk[8];
      float t = softmax_exp(sc, pk, c2);
      if (__builtin_expect(__ballot(!(t <= kLazySum)) != 0, 0)) {
        rescale(sc, c2);
        t = softmax_exp(sc, pk, c2);
      }
      l_run += t;
      pv(pk, slot(v));
      if (v & 1) wait_vm_barrier_s<kVmAhead0, kVmAhead, decltype(w0_c)::value>();
    };
    f32x16 s_alt;
    auto run = [&](int& v, int end, auto qkrem_c, auto mk_c, auto remsrc_c)
        __attribute__((always_inline)) {
      for (; v + 1 < end; v += 2) {
        step(v, s_cur, s_alt, qkrem_c, mk_c, remsrc_c);
        step(v + 1, s_alt, s_cur, qkrem_c, mk_c, remsrc_c);
      }
      if (v < end) {
        step(v, s_cur, s_alt, qkrem_c, mk_c, remsrc_c);
        s_cur = s_alt;
        ++v;
      }
    };
    using kRem = std::true_type;
    using kLoc = std::false_type;
    using kNoMask = std::integral_constant<int, 0>;
    using kRemMask = std::integral_constant<int, 1>;
    using kLocMask = std::integral_constant<int, 2>;
    // Phases of the virtual-tile walk (each loop body is specialised):
    //   remote unmasked [0, ktA) | remote straddling [ktA, ktB) | local straddling
    //   | local unmasked | local diagonal; the last remote tile switches the query operand.
    const int kt_diag = i0 >= BK - 1 ? (i0 - (BK - 1)) / BK + 1 : 0;  // first diagonal tile
    const int v_loc_plain = nr + (ktB - ktA);           // first local tile past the window edge
    const int v_diag = nr + (max(kt_diag, ktA) - ktA);  // first local tile needing causality
    const int v_rem_mask = ktA - r0;                    // first remote tile needing a mask
    int v = 0;
    if (mode == 2) {
      run(v, nr - 1, kRem(), kLocMask(), std::false_type());
    } else {
      // while the tiles issued (v + PREF) are remote, the transfers skip the class test
      run(v, min(min(v_rem_mask, nr - 1), nr - PREF), kRem(), kNoMask(), std::true_type());
      run(v, min(v_rem_mask, nr - 1), kRem(), kNoMask(), std::false_type());
      run(v, nr - 1, kRem(), kRemMask(), std::false_type());
    }
    if (nr > 0) {  // last remote tile: the next scores are local (or past the end)
      load_q_std();
      if (mode == 2) run(v, v + 1, kLoc(), kLocMask(), std::false_type());
      else if (v >= v_rem_mask) run(v, v + 1, kLoc(), kRemMask(), std::false_type());
      else run(v, v + 1, kLoc(), kNoMask(), std::false_type());
    }
    run(v, min(v_loc_plain, nvt), kLoc(), kLocMask(), std::false_type());
    run(v, min(v_diag, nvt), kLoc(), kNoMask(), std::false_type());
    run(v, nvt, kLoc(), kLocMask(), std::false_type());
  };
  if (wave == 0) walk(std::true_type());
  else walk(std::false_type());
  // Transfers issued past the last tile must land before this workgroup's LDS is
  // handed to another one.
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(7 << 4);  // vmcnt(0) lgkmcnt(0)

  // ---- epilogue: O = O^T / l, LSE ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qi < L) {
    // O = (V 2^-e_v)^T P^T 2^e_v / l.  Cached stores: each one covers 16 bytes of a row,
    // and the L2 merges them into whole lines (streaming stores wrote four times the
    // bytes of O to HBM).
    const float inv = __builtin_ldexpf(1.f, args.sel[g * kSelStride + kSelExpV]) / l_tot;
    const size_t orow_off = ((size_t)(start + qi) * Hq + qhead) * D;
    if (args.out_f32) {
      float* orow = (float*)args.O + orow_off;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d = 32 * db + 8 * q4 + 4 * hf;
          const f32x16& o = oacc[db];
          *reinterpret_cast<float4*>(orow + d) = make_float4(o[4 * q4] * inv, o[4 * q4 + 1] * inv,
                                                             o[4 * q4 + 2] * inv, o[4 * q4 + 3] * inv);
        }
    } else {
      uint16_t* orow = (uint16_t*)args.O + orow_off;
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
    }
    if (args.lse && hf == 0)
      args.lse[(size_t)qhead * args.T + start + qi] = (m_run + log2f(l_tot)) * 0.69314718055994530942f;
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_pair_select(const void* Q, const void* K, const void* V, int T, int Hq,
                              int Hkv, uint32_t* mx /*[(Hq+2Hkv)*64]*/, int32_t* sel,
                              hipStream_t stream) {
  const int n = (Hq + 2 * Hkv) * 64;
  hipLaunchKernelGGL(pair_max_zero_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, mx, n);
  const int tpb = 256;  // tokens per block
  const int ty = (T + tpb - 1) / tpb;
  if (ty > 0) {
    hipLaunchKernelGGL(pair_max_kernel, dim3((Hq * 8 + 63) / 64, ty), dim3(256), 0, stream,
                       (const uint16_t*)Q, T, Hq, tpb, mx);
    hipLaunchKernelGGL(pair_max_kernel, dim3((Hkv * 8 + 63) / 64, ty), dim3(256), 0, stream,
                       (const uint16_t*)K, T, Hkv, tpb, mx + Hq * 64);
    hipLaunchKernelGGL(pair_max_kernel, dim3((Hkv * 8 + 63) / 64, ty), dim3(256), 0, stream,
                       (const uint16_t*)V, T, Hkv, tpb, mx + (Hq + Hkv) * 64);
  }
  hipLaunchKernelGGL(pair_select_kernel, dim3(Hkv), dim3(64), 0, stream, mx,
                     mx + Hq * 64, mx + (Hq + Hkv) * 64, Hq, Hkv, sel);
  return hipGetLastError();
}

template <int REP>
static hipError_t launch_mfma_rep(const PrefillArgs& args, hipStream_t stream) {
  // set on every launch (idempotent, a host-side call): the library keeps no state
  hipError_t e = hipFuncSetAttribute((const void*)prefill_mfma_kernel<REP>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)mf::kSmem);
  if (e != hipSuccess) return e;
  const int blocks = args.Hkv * args.lvl_start[args.nlvl];
  hipLaunchKernelGGL(prefill_mfma_kernel<REP>, dim3(blocks), dim3(512), mf::kSmem, stream, args);
  return hipGetLastError();
}

hipError_t launch_prefill_mfma(const PrefillArgs& args, int chunk_tiles, hipStream_t stream) {
  if (chunk_tiles > 0) {
    if (args.interp)
      hipLaunchKernelGGL(key_prep_kernel<true>, dim3(chunk_tiles, args.Hkv), dim3(256), 0, stream,
                         args);
    else
      hipLaunchKernelGGL(key_prep_kernel<false>, dim3(chunk_tiles, args.Hkv), dim3(256), 0, stream,
                         args);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
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
