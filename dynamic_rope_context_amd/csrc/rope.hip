// rope_apply: in-place RoPE at (aliased) positions, x[t,h,:] <- R(floor(p_t / G)) x[t,h,:].
//
// With G = 1 this is standard RoPE, which builds the inputs the attention calls
// expect: queries and cached keys carry standard RoPE at exact absolute positions
// (Jet-Long technical summary, "Methodology" section 2).  With G > 1 the vectors land
// on the aliased grid f(x) = floor(x / G) of section 1.
//
// One thread per (token, pair): the angle f(p) * theta_m is formed in float64 and its
// cos/sin rounded once to float32, then every head of the token is rotated with it in
// float32 (rotate-half pairing: channel m with m + D/2).
#include "bf_common.h"

namespace bifocal {

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
  const int f = alias_pos(p, G);
  double s64, c64;
  sincos_reduced((double)f * inv_freq64(theta, m, D), &s64, &c64);
  const float c = (float)c64, s = (float)s64;
  T* row = x + (size_t)t * H * D;
  for (int h = 0; h < H; ++h) {
    T* v = row + (size_t)h * D;
    const float x1 = ld(v + m), x2 = ld(v + m + half);
    st(v + m, x1 * c - x2 * s);
    st(v + m + half, x2 * c + x1 * s);
  }
}

hipError_t launch_rope_apply(void* x, const int32_t* pos, int pos0, int T_, int H, int D,
                             double theta, int G, bool bf16, hipStream_t stream) {
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
