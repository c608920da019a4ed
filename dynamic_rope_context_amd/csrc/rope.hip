// rope_apply: in-place RoPE at (aliased) positions, x[t,h,:] <- R(floor(p_t / G)) x[t,h,:].
//
// With G = 1 this is standard RoPE, which builds the inputs the attention calls
// expect: queries and cached keys carry standard RoPE at exact absolute positions
// (Jet-Long technical summary, "Methodology" section 2).  With G > 1 the vectors land
// on the aliased grid f(x) = floor(x / G) of section 1.  Rotate-half pairing: channel m
// with m + D/2; the angle f(p) * theta_m is formed in float64 and its cos/sin rounded
// once to float32, then every head of the token is rotated with it in float32.
//
// Streaming kernel (HBM-bound: every element is read and written once).  A workgroup
// takes a block of tokens: first the (cos, sin) of each (token, pair) of the block go to
// LDS (theta_m once per workgroup, one float64 sincos per pair and token, not per head),
// then each thread rotates 8 consecutive pairs of one (token, head) with 16-byte loads
// and stores of both halves.  For bf16 they are streaming (non-temporal: 4-5% faster
// than cached ones); the eight lanes of a head half cover whole 128-byte lines.  Head dims whose half is not a multiple of 8 pairs, or rows
// that are not 16-byte aligned, take a one-pair-per-thread kernel.
#include "bf_common.h"

namespace bifocal {

namespace rp {
constexpr int TB = 4;        // tokens per workgroup (1, 2, 4, 8, 16 measured: 4 is fastest)
constexpr int THREADS = 256;
}  // namespace rp

template <typename T>
struct Chunk8;  // 8 consecutive elements as float, with 16-byte (bf16) or 2x16-byte loads
template <>
struct Chunk8<uint16_t> {
  __device__ __forceinline__ static void load(const uint16_t* p, float* v) {
    const u32x4 w = ld_stream(p);
    const uint32_t u[4] = {w[0], w[1], w[2], w[3]};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bf16_lo(u[e]);
      v[2 * e + 1] = bf16_hi(u[e]);
    }
  }
  __device__ __forceinline__ static void store(uint16_t* p, const float* v) {
    uint32_t u[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      u[e] = f32_to_bf16_bits(v[2 * e]) | (f32_to_bf16_bits(v[2 * e + 1]) << 16);
    st_stream(p, u32x4{u[0], u[1], u[2], u[3]});
  }
};
template <>
struct Chunk8<float> {
  __device__ __forceinline__ static void load(const float* p, float* v) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ static void store(float* p, const float* v) {
    // cached: each store covers half of a 32-byte run, which the L2 merges
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
};

template <typename T>
__global__ void __launch_bounds__(rp::THREADS) rope_apply_chunked_kernel(
    T* __restrict__ x, const int32_t* __restrict__ pos, int pos0, int T_, int H, int D,
    double theta, int G) {
  using namespace rp;
  __shared__ double s_invf[128];
  __shared__ float2 s_cs[TB][128];
  const int half = D / 2;
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * TB;
  for (int m = tid; m < half; m += THREADS) s_invf[m] = inv_freq64(theta, m, D);
  __syncthreads();
  for (int i = tid; i < TB * half; i += THREADS) {
    const int tt = i / half, m = i - tt * half;
    const int t = t0 + tt;
    if (t < T_) {
      const int p = pos ? pos[t] : pos0 + t;
      s_cs[tt][m] = angle_cs((double)alias_pos(p, G), s_invf[m]);
    }
  }
  __syncthreads();
  const int chunks = half / 8;             // 8-pair chunks per (token, head)
  const int per_tok = H * chunks;
  for (int i = tid; i < TB * per_tok; i += THREADS) {
    const int tt = i / per_tok;
    const int t = t0 + tt;
    if (t >= T_) break;                    // i grows with tt
    const int r = i - tt * per_tok;
    const int h = r / chunks, c = r - h * chunks;
    T* row = x + ((size_t)t * H + h) * D + 8 * c;
    float a[8], b[8];
    Chunk8<T>::load(row, a);
    Chunk8<T>::load(row + half, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float2 cs = s_cs[tt][8 * c + e];
      const float x1 = a[e], x2 = b[e];
      a[e] = x1 * cs.x - x2 * cs.y;
      b[e] = x2 * cs.x + x1 * cs.y;
    }
    Chunk8<T>::store(row, a);
    Chunk8<T>::store(row + half, b);
  }
}

// One thread per (token, pair): any even D, any alignment of the element type.
template <typename T>
__device__ __forceinline__ float ld(const T* p);
template <>
__device__ __forceinline__ float ld<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p) {
  return __uint_as_float((uint32_t)(*p) << 16);
}
template <typename T>
__device__ __forceinline__ void st(T* p, float v);
template <>
__device__ __forceinline__ void st<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void st<uint16_t>(uint16_t* p, float v) {
  *p = (uint16_t)f32_to_bf16_bits(v);
}

template <typename T>
__global__ void __launch_bounds__(256) rope_apply_kernel(T* __restrict__ x,
                                                         const int32_t* __restrict__ pos,
                                                         int pos0, int T_, int H, int D,
                                                         double theta, int G) {
  const int half = D / 2;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long t = idx / half;
  const int m = (int)(idx - t * half);
  if (t >= T_) return;
  const int p = pos ? pos[t] : pos0 + (int)t;
  const float2 cs = angle_cs((double)alias_pos(p, G), inv_freq64(theta, m, D));
  T* row = x + (size_t)t * H * D;
  for (int h = 0; h < H; ++h) {
    T* v = row + (size_t)h * D;
    const float x1 = ld(v + m), x2 = ld(v + m + half);
    st(v + m, x1 * cs.x - x2 * cs.y);
    st(v + m + half, x2 * cs.x + x1 * cs.y);
  }
}

hipError_t launch_rope_apply(void* x, const int32_t* pos, int pos0, int T_, int H, int D,
                             double theta, int G, bool bf16, hipStream_t stream) {
  const size_t esz = bf16 ? 2 : 4;
  const bool chunked = (D / 2) % 8 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
                       ((size_t)D / 2 * esz) % 16 == 0;
  if (chunked) {
    const int blocks = (T_ + rp::TB - 1) / rp::TB;
    if (bf16)
      hipLaunchKernelGGL(rope_apply_chunked_kernel<uint16_t>, dim3(blocks), dim3(rp::THREADS), 0,
                         stream, (uint16_t*)x, pos, pos0, T_, H, D, theta, G);
    else
      hipLaunchKernelGGL(rope_apply_chunked_kernel<float>, dim3(blocks), dim3(rp::THREADS), 0,
                         stream, (float*)x, pos, pos0, T_, H, D, theta, G);
    return hipGetLastError();
  }
  const long long threads = (long long)T_ * (D / 2);
  const int blocks = (int)((threads + 255) / 256);
  if (bf16)
    hipLaunchKernelGGL(rope_apply_kernel<uint16_t>, dim3(blocks), dim3(256), 0, stream,
                       (uint16_t*)x, pos, pos0, T_, H, D, theta, G);
  else
    hipLaunchKernelGGL(rope_apply_kernel<float>, dim3(blocks), dim3(256), 0, stream, (float*)x,
                       pos, pos0, T_, H, D, theta, G);
  return hipGetLastError();
}

}  // namespace bifocal
