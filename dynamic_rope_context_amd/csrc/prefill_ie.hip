// Inclusion-exclusion merge of three attention passes (gfx950).
//
// Jet-Long technical summary, "Methodology" section 2 (inference efficiency mechanisms):
// the pages compute the bifocal attention as three FlashAttention passes whose
// LogSumExp statistics are merged so that the remote window is not counted twice:
// A = local scores over the window pairs, B = remote scores over all causal pairs,
// C = remote scores over the window pairs, and Z = Z_B - Z_C + Z_A.  The fused kernels
// select each pair's rule instead; this literal form exists to measure that fusion and
// to cross-check it on the GPU.
//
// Per (token, head): m = max(LSE_A, LSE_B, LSE_C), w_x = exp(LSE_x - m),
// z = w_B - w_C + w_A, O = (w_B O_B - w_C O_C + w_A O_A) / z, LSE = m + ln z.
// HBM-bound: reads three fp32 [T, Hq, D] outputs and three [Hq, T] LSE rows, writes
// O in bf16 and LSE.
#include "bf_common.h"

namespace bifocal {

__global__ void __launch_bounds__(256) ie_merge_kernel(const float4* __restrict__ oa,
                                                       const float4* __restrict__ ob,
                                                       const float4* __restrict__ oc,
                                                       const float* __restrict__ la,
                                                       const float* __restrict__ lb,
                                                       const float* __restrict__ lc,
                                                       uint2* __restrict__ o, float* lse, int T,
                                                       int Hq) {
  constexpr int D4 = 128 / 4;  // float4 groups per row
  const size_t n4 = (size_t)T * Hq * D4;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const size_t row = i / D4;  // t * Hq + h
    const int h = (int)(row % Hq);
    const size_t t = row / Hq;
    const size_t li = (size_t)h * T + t;
    const float xa = la[li], xb = lb[li], xc = lc[li];
    const float m = fmaxf(xa, fmaxf(xb, xc));
    const float wa = expf(xa - m), wb = expf(xb - m), wc = expf(xc - m);
    const float z = (wb - wc) + wa;
    const float iz = 1.f / z;
    const float4 va = oa[i], vb = ob[i], vc = oc[i];
    const float r0 = ((wb * vb.x - wc * vc.x) + wa * va.x) * iz;
    const float r1 = ((wb * vb.y - wc * vc.y) + wa * va.y) * iz;
    const float r2 = ((wb * vb.z - wc * vc.z) + wa * va.z) * iz;
    const float r3 = ((wb * vb.w - wc * vc.w) + wa * va.w) * iz;
    o[i] = make_uint2(f32_to_bf16_bits(r0) | (f32_to_bf16_bits(r1) << 16),
                      f32_to_bf16_bits(r2) | (f32_to_bf16_bits(r3) << 16));
    if (lse && i % D4 == 0) lse[li] = m + logf(z);
  }
}

hipError_t launch_ie_merge(const float* oa, const float* ob, const float* oc, const float* la,
                           const float* lb, const float* lc, void* o, float* lse, int T, int Hq,
                           hipStream_t stream) {
  const size_t n4 = (size_t)T * Hq * 32;
  size_t blocks = (n4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(ie_merge_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const float4*)oa, (const float4*)ob, (const float4*)oc, la, lb, lc,
                     (uint2*)o, lse, T, Hq);
  return hipGetLastError();
}

}  // namespace bifocal
