// Bifocal decode, vector path (fp32 caches, and D = 64): one query at position pos over
// a standard-RoPE KV cache (gfx950).  bf16 caches with D = 128 take the matrix-core
// kernel instead.
//
// Jet-Long technical summary, "Methodology" section 2 (on-the-fly correction
// rotation): the cache keeps keys with standard RoPE at their exact positions and is
// never rewritten; the remote branch rotates the active query and each stored key by
// R(f(x) - x) in registers, which lands them at the aliased positions f(x) = floor(x/G)
// of section 1 because RoPE rotations compose additively.  G comes from the current
// length pos + 1, so it changes as generation crosses multiples of w_pretrained.
//
// Split-KV: the cache range 0..pos is cut into splits; one workgroup streams one
// (KV head, split) with 128-bit loads, 16 lanes per key, each lane holding D/16
// channels of one key.  The RoPE partner channel (m +/- D/2) sits 8 lanes away and
// is fetched with a DPP row rotation.  Scores, the correction rotation and the
// softmax run in float32.  Each workgroup writes (m, l, acc[D]) per query head; a
// combine kernel merges the splits with log-sum-exp weights.
#include <type_traits>

#include "bf_common.h"
#include "decode_args.h"

namespace bifocal {

// DPP row rotation within 16-lane rows.
template <int N>
__device__ __forceinline__ float ror16(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x120 + N, 0xf, 0xf, false));
}

template <typename TIn>
struct Row;  // load CPL channels of a row as float

template <>
struct Row<uint16_t> {
  template <int CPL>
  __device__ __forceinline__ static void load(const uint16_t* p, float* out) {
    if constexpr (CPL == 8) {
      const uint4 w = *reinterpret_cast<const uint4*>(p);
      out[0] = bf16_lo(w.x); out[1] = bf16_hi(w.x);
      out[2] = bf16_lo(w.y); out[3] = bf16_hi(w.y);
      out[4] = bf16_lo(w.z); out[5] = bf16_hi(w.z);
      out[6] = bf16_lo(w.w); out[7] = bf16_hi(w.w);
    } else {
      const uint2 w = *reinterpret_cast<const uint2*>(p);
      out[0] = bf16_lo(w.x); out[1] = bf16_hi(w.x);
      out[2] = bf16_lo(w.y); out[3] = bf16_hi(w.y);
    }
  }
};

template <>
struct Row<float> {
  template <int CPL>
  __device__ __forceinline__ static void load(const float* p, float* out) {
#pragma unroll
    for (int c = 0; c < CPL; c += 4) {
      const float4 w = *reinterpret_cast<const float4*>(p + c);
      out[c] = w.x; out[c + 1] = w.y; out[c + 2] = w.z; out[c + 3] = w.w;
    }
  }
};

template <typename TIn, int D, int REP>
__global__ void __launch_bounds__(256) decode_split_kernel(DecodeArgs a) {
  constexpr int CPL = D / 16;   // channels per lane
  constexpr int H2 = D / 2;
  constexpr int U = 4;          // wave iterations (4 keys each) loaded ahead
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = lane >> 4;    // key slot within the wave iteration
  const int t = lane & 15;      // channel chunk
  const bool first_half = t < 8;
  const int c0 = CPL * t;       // first channel of this lane
  const int m0 = c0 % H2;       // first RoPE pair of this lane

  // Workgroup -> (KV head, split).  Consecutive workgroups go to different XCDs; the
  // splits of one XCD cover a contiguous key range for every head, so the table rows
  // of that range are fetched into that XCD's L2 once and shared by all heads.
  const int id = blockIdx.x;
  const int per_xcd = a.nsplit >> 3;  // nsplit is a multiple of 8
  const int xcd = id & 7;
  const int k_in = id >> 3;
  const int g = k_in % a.Hkv;
  const int split = xcd * per_xcd + k_in / a.Hkv;

  const int pos = a.pos;
  const int G = a.G;
  const TIn* __restrict__ Kp = (const TIn*)a.K;
  const TIn* __restrict__ Vp = (const TIn*)a.V;
  const float2* __restrict__ tab = a.tab;

  // Query rows of this KV head: standard copy and remote copy R(f(pos) - pos) q.
  float qs[REP][CPL], qr[REP][CPL];
  {
    const int nq = pos - alias_fast(pos, a.gdiv);
    const TIn* qp = (const TIn*)a.q;
#pragma unroll
    for (int h = 0; h < REP; ++h) {
      const TIn* row = qp + (size_t)(g * REP + h) * D;
      float own[CPL], par[CPL];
      Row<TIn>::template load<CPL>(row + c0, own);
      Row<TIn>::template load<CPL>(row + (first_half ? c0 + H2 : c0 - H2), par);
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const float2 cs = tab[(size_t)nq * H2 + m0 + c];
        qs[h][c] = own[c];
        // R(-n): x1' = x1 c + x2 s, x2' = x2 c - x1 s
        qr[h][c] = first_half ? own[c] * cs.x + par[c] * cs.y : own[c] * cs.x - par[c] * cs.y;
      }
    }
  }

  float m_run[REP], l_run[REP], acc[REP][CPL];
#pragma unroll
  for (int h = 0; h < REP; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[h][c] = 0.f;
  }

  const int kpw = a.kps >> 2;  // keys per wave
  const int j_wave = split * a.kps + wave * kpw;
  const int j_stop = min(j_wave + kpw, pos + 1);
  const size_t row_stride = (size_t)a.Hkv * D;
  const float sgn = first_half ? 1.f : -1.f;

  // Remote-ness is monotone in j (remote iff j <= pos - w0), so whole chunks of
  // 4*U keys are usually all remote or all local; only the chunk that crosses the
  // window edge takes the per-lane select.
  enum { kRemote = 0, kLocal = 1, kMixed = 2 };
  auto chunk = [&](const int jb, auto mode_c) {
    constexpr int mode = decltype(mode_c)::value;
    float kv[U][CPL], vv[U][CPL];
    float2 cs[U][CPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jb + 4 * u + grp;
      const int jc = j <= pos ? j : pos;  // clamp: masked below
      const TIn* kr = Kp + (size_t)jc * row_stride + (size_t)g * D + c0;
      const TIn* vr = Vp + (size_t)jc * row_stride + (size_t)g * D + c0;
      Row<TIn>::template load<CPL>(kr, kv[u]);
      Row<TIn>::template load<CPL>(vr, vv[u]);
      if constexpr (mode != kLocal) {
        const int n = jc - alias_fast(jc, a.gdiv);
        const float4* tp = reinterpret_cast<const float4*>(tab + (size_t)n * H2 + m0);
#pragma unroll
        for (int c = 0; c < CPL; c += 2) {
          const float4 w = tp[c / 2];
          cs[u][c] = make_float2(w.x, w.y);
          cs[u][c + 1] = make_float2(w.z, w.w);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jb + 4 * u + grp;
      const bool in_range = j < j_stop;
      const bool remote = (pos - j) >= a.w0;
      float kk[CPL];
      if constexpr (mode == kLocal) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) kk[c] = kv[u][c];
      } else {
        // correction rotation R(f(j) - j) of the key: the partner channel is 8 lanes away
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const float partner = ror16<8>(kv[u][c]);
          const float rot = kv[u][c] * cs[u][c].x + partner * (sgn * cs[u][c].y);
          kk[c] = (mode == kMixed && !remote) ? kv[u][c] : rot;
        }
      }
      float sc[REP];
#pragma unroll
      for (int h = 0; h < REP; ++h) {
        float d = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          float qv;
          if constexpr (mode == kRemote) qv = qr[h][c];
          else if constexpr (mode == kLocal) qv = qs[h][c];
          else qv = remote ? qr[h][c] : qs[h][c];
          d += qv * kk[c];
        }
        d += ror16<8>(d);
        d += ror16<4>(d);
        d += ror16<2>(d);
        d += ror16<1>(d);
        sc[h] = in_range ? d * a.scale_log2 : -INFINITY;
      }
#pragma unroll
      for (int h = 0; h < REP; ++h) {
        if (sc[h] > m_run[h]) {  // rescale only when the running max grows
          const float corr = exp2f(m_run[h] - sc[h]);
          l_run[h] *= corr;
#pragma unroll
          for (int c = 0; c < CPL; ++c) acc[h][c] *= corr;
          m_run[h] = sc[h];
        }
        const float p = in_range ? exp2f(sc[h] - m_run[h]) : 0.f;
        l_run[h] += p;
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[h][c] += p * vv[u][c];
      }
    }
  };
  const int last_remote = pos - a.w0;  // keys j <= last_remote are remote
  for (int jb = j_wave; jb < j_stop; jb += 4 * U) {
    const int je = jb + 4 * U - 1;
    if (je <= last_remote)
      chunk(jb, std::integral_constant<int, kRemote>());
    else if (jb > last_remote)
      chunk(jb, std::integral_constant<int, kLocal>());
    else
      chunk(jb, std::integral_constant<int, kMixed>());
  }

  // Merge the 16 streams (4 waves x 4 key slots) of this workgroup through LDS.
  __shared__ float s_acc[16][REP][D];
  __shared__ float s_ml[16][REP][2];
  const int stream = wave * 4 + grp;
#pragma unroll
  for (int h = 0; h < REP; ++h) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) s_acc[stream][h][c0 + c] = acc[h][c];
    if (t == 0) {
      s_ml[stream][h][0] = m_run[h];
      s_ml[stream][h][1] = l_run[h];
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < REP * D; e += 256) {
    const int h = e / D, d = e - h * D;
    float mx = -INFINITY;
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) mx = fmaxf(mx, s_ml[s2][h][0]);
    float o = 0.f, l = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2) {
        const float ms = s_ml[s2][h][0];
        const float w = ms == -INFINITY ? 0.f : exp2f(ms - mx);
        o += w * s_acc[s2][h][d];
        l += w * s_ml[s2][h][1];
      }
    }
    float* dst = a.part + ((size_t)(g * REP + h) * a.nsplit + split) * (D + 2);
    dst[d] = o;
    if (d == 0) {
      dst[D] = mx;
      dst[D + 1] = l;
    }
  }
}

// Merge the partials of each query head: O = sum_s w_s acc_s / sum_s w_s l_s with
// w_s = 2^(m_s - max m); LSE = ln 2 * (max m + log2 sum_s w_s l_s).  One workgroup per
// (query head, 32 channels): eight groups of 32 lanes sweep the partials, each lane one
// channel, and meet in LDS.
template <typename TOut, int D>
__global__ void __launch_bounds__(256) decode_combine_kernel(DecodeArgs a) {
  __shared__ float s_w[kDecodeMaxSplits];
  __shared__ float s_red[8][33];
  const int h = blockIdx.x;
  const int d0 = 32 * blockIdx.y;
  const int tid = threadIdx.x;
  const int ns = a.nsplit;
  const float* base = a.part + (size_t)h * ns * (D + 2);
  // max of the partial maxima (every thread scans a strided slice, then the block)
  float mx = -INFINITY;
  for (int s = tid; s < ns; s += 256) mx = fmaxf(mx, base[(size_t)s * (D + 2) + D]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((tid & 63) == 0) s_red[tid >> 6][32] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(s_red[0][32], s_red[1][32]), fmaxf(s_red[2][32], s_red[3][32]));
  float lsum = 0.f;
  for (int s = tid; s < ns; s += 256) {
    const float ms = base[(size_t)s * (D + 2) + D];
    const float w = ms == -INFINITY ? 0.f : exp2f(ms - mx);
    s_w[s] = w;
    lsum += w * base[(size_t)s * (D + 2) + D + 1];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) lsum += __shfl_xor(lsum, o);
  __syncthreads();  // s_w complete, s_red[.][32] consumed
  if ((tid & 63) == 0) s_red[tid >> 6][32] = lsum;
  __syncthreads();
  lsum = s_red[0][32] + s_red[1][32] + s_red[2][32] + s_red[3][32];
  const int grp = tid >> 5, c = tid & 31;
  float o = 0.f;
  for (int s = grp; s < ns; s += 8) o += s_w[s] * base[(size_t)s * (D + 2) + d0 + c];
  s_red[grp][c] = o;
  __syncthreads();
  if (tid < 32) {
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) v += s_red[q][tid];
    const float val = v / lsum;
    if constexpr (sizeof(TOut) == 2)
      ((uint16_t*)a.o)[(size_t)h * D + d0 + tid] = (uint16_t)f32_to_bf16_bits(val);
    else
      ((float*)a.o)[(size_t)h * D + d0 + tid] = val;
    if (a.lse && blockIdx.y == 0 && tid == 0) a.lse[h] = (mx + log2f(lsum)) * 0.69314718055994530942f;
  }
}

template <typename TIn, int D>
static hipError_t launch_decode_t(const DecodeArgs& a, int rep, hipStream_t stream) {
  dim3 grid(a.nsplit * a.Hkv);
  switch (rep) {
    case 1: hipLaunchKernelGGL((decode_split_kernel<TIn, D, 1>), grid, dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_split_kernel<TIn, D, 2>), grid, dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((decode_split_kernel<TIn, D, 4>), grid, dim3(256), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((decode_split_kernel<TIn, D, 8>), grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<TIn, D>), dim3(a.Hq, D / 32), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int rep, int D, bool bf16, hipStream_t stream) {
  if (bf16) return D == 64 ? launch_decode_t<uint16_t, 64>(a, rep, stream)
                           : launch_decode_t<uint16_t, 128>(a, rep, stream);
  return D == 64 ? launch_decode_t<float, 64>(a, rep, stream)
                 : launch_decode_t<float, 128>(a, rep, stream);
}

}  // namespace bifocal
