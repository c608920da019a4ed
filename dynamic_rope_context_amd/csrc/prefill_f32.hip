// Bifocal prefill in float32 (VALU), for float32 inputs and any head ratio.
//
// One wave per (sequence, block of 64 query rows, query head); thread t owns query
// row i = 64*qb + t.  Per the Jet-Long technical summary ("Methodology" section 1),
// key j <= i is scored with standard RoPE when i - j < w0 and with RoPE at the aliased
// positions f(i), f(j) otherwise, f(x) = floor(x / G), G from the sequence length.
// Inputs carry standard RoPE; the remote vectors come from the correction rotation
// R(f(x) - x) (section 2), applied here in float32 from the position table.  All keys
// of a row share one online softmax, which is the exact result the pages' three-pass
// inclusion-exclusion merge produces.
#include "bf_common.h"
#include "prefill_args.h"

namespace bifocal {

namespace {
constexpr int kRows = 64;   // query rows per block (one per thread)
constexpr int kKeys = 32;   // keys staged per tile
}

// R(-n) from the table row n: (x1, x2) -> (x1 c + x2 s, x2 c - x1 s).
__device__ __forceinline__ void rot_back(float& a, float& b, float2 cs) {
  const float x1 = a, x2 = b;
  a = x1 * cs.x + x2 * cs.y;
  b = x2 * cs.x - x1 * cs.y;
}

template <int D>
__global__ void __launch_bounds__(64) prefill_f32_kernel(PrefillArgs args) {
  constexpr int H2 = D / 2;
  constexpr int LD = D + 1;  // padded row stride: conflict-free per-thread rows
  extern __shared__ float smem[];
  float* q_loc = smem;                       // [kRows][LD]
  float* q_rem = q_loc + kRows * LD;         // [kRows][LD]
  float* acc = q_rem + kRows * LD;           // [kRows][LD]
  float* k_loc = acc + kRows * LD;           // [kKeys][D]
  float* k_rem = k_loc + kKeys * D;          // [kKeys][D]
  float* v_s = k_rem + kKeys * D;            // [kKeys][D]

  const int tid = threadIdx.x;
  const int h = blockIdx.y;
  const int nseq = args.nseq;
  const int b = blockIdx.x % nseq;
  const int qb = args.max_qblocks - 1 - blockIdx.x / nseq;  // longest rows first
  const int L = args.seq[b].len;
  if (qb * kRows >= L) return;
  const int start = args.seq[b].start;
  const int G = args.seq[b].G;
  const int rep = args.Hq / args.Hkv;
  const int g = h / rep;
  const float* __restrict__ Q = (const float*)args.Q;
  const float* __restrict__ K = (const float*)args.K;
  const float* __restrict__ V = (const float*)args.V;
  const float2* __restrict__ tab = args.tab;
  const int w0 = args.w0;

  const int i = qb * kRows + tid;
  const bool valid = i < L;
  const int i_last = min(L, (qb + 1) * kRows) - 1;

  // Query row: standard RoPE as given, and the remote copy R(f(i) - i) q.
  {
    const float* qrow = Q + ((size_t)(start + (valid ? i : 0)) * args.Hq + h) * D;
    const int n = valid ? i - alias_pos(i, G) : 0;
    for (int m = 0; m < H2; ++m) {
      float a = qrow[m], c = qrow[m + H2];
      q_loc[tid * LD + m] = a;
      q_loc[tid * LD + m + H2] = c;
      rot_back(a, c, tab[(size_t)n * H2 + m]);
      q_rem[tid * LD + m] = a;
      q_rem[tid * LD + m + H2] = c;
    }
    for (int d = 0; d < D; ++d) acc[tid * LD + d] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  const float scale = args.scale;

  for (int j0 = 0; j0 <= i_last; j0 += kKeys) {
    __syncthreads();
    // Stage keys j0 .. j0+kKeys-1: standard copy, remote copy, values.
    for (int e = tid; e < kKeys * H2; e += 64) {
      const int kk = e / H2, m = e - kk * H2;
      const int j = j0 + kk;
      float a = 0.f, c = 0.f, va = 0.f, vc = 0.f;
      if (j < L) {
        const float* krow = K + ((size_t)(start + j) * args.Hkv + g) * D;
        const float* vrow = V + ((size_t)(start + j) * args.Hkv + g) * D;
        a = krow[m];
        c = krow[m + H2];
        va = vrow[m];
        vc = vrow[m + H2];
      }
      k_loc[kk * D + m] = a;
      k_loc[kk * D + m + H2] = c;
      v_s[kk * D + m] = va;
      v_s[kk * D + m + H2] = vc;
      const int n = j < L ? j - alias_pos(j, G) : 0;
      rot_back(a, c, tab[(size_t)n * H2 + m]);
      k_rem[kk * D + m] = a;
      k_rem[kk * D + m + H2] = c;
    }
    __syncthreads();
    if (!valid) continue;
    const int kmax = min(kKeys, i - j0 + 1);
    for (int kk = 0; kk < kmax; ++kk) {
      const int j = j0 + kk;
      const bool local = (i - j) < w0;
      const float* qv = local ? q_loc + tid * LD : q_rem + tid * LD;
      const float* kv = local ? k_loc + kk * D : k_rem + kk * D;
      float s = 0.f;
      for (int d = 0; d < D; ++d) s += qv[d] * kv[d];
      s *= scale;
      const float m_new = fmaxf(m_run, s);
      const float corr = expf(m_run - m_new);
      const float p = expf(s - m_new);
      l_run = l_run * corr + p;
      float* a = acc + tid * LD;
      const float* vv = v_s + kk * D;
      for (int d = 0; d < D; ++d) a[d] = a[d] * corr + p * vv[d];
      m_run = m_new;
    }
  }
  if (!valid) return;
  float* O = (float*)args.O + ((size_t)(start + i) * args.Hq + h) * D;
  const float inv = 1.f / l_run;
  for (int d = 0; d < D; ++d) O[d] = acc[tid * LD + d] * inv;
  if (args.lse) args.lse[(size_t)h * args.T + start + i] = m_run + logf(l_run);
}

template <int D>
static hipError_t launch_f32_d(const PrefillArgs& args, hipStream_t stream) {
  const size_t sm = (3 * kRows * (D + 1) + 3 * kKeys * D) * sizeof(float);
  // set on every launch (idempotent, a host-side call): the library keeps no state
  hipError_t e = hipFuncSetAttribute((const void*)prefill_f32_kernel<D>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
  if (e != hipSuccess) return e;
  dim3 grid(args.max_qblocks * args.nseq, args.Hq);
  hipLaunchKernelGGL(prefill_f32_kernel<D>, grid, dim3(64), sm, stream, args);
  return hipGetLastError();
}

hipError_t launch_prefill_f32(const PrefillArgs& args, hipStream_t stream) {
  return args.D == 64 ? launch_f32_d<64>(args, stream) : launch_f32_d<128>(args, stream);
}

int prefill_f32_rows_per_block() { return kRows; }

}  // namespace bifocal
