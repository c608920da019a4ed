// RoPE / correction-angle table generator (gfx950).
//
// Fills tab[p][m] = (cos(p*theta_m), sin(p*theta_m)) for p < n_cap, angles formed in
// float64 from the integer position and rounded once to float32.  The same table
// gives standard RoPE at p and, read at n = x - floor(x/G) with the sine negated, the
// correction rotation R(f(x) - x) that moves a standard-RoPE vector at x to the
// aliased position f(x) (Jet-Long technical summary, "Methodology" section 1 for f,
// section 2 "on-the-fly correction rotation" for the additive composition).
//
// The table persists in the caller's workspace behind a header.  A build is two
// launches on the caller's stream: every block of the build kernel reads the header
// first and leaves at once when it already describes (theta, D) with enough
// positions; otherwise the blocks fill the rows.  A one-thread publish kernel then
// writes the header (stream order makes every row of the build visible to it and to
// later kernels).  No block waits for another and nothing is counted, so a build
// costs its arithmetic only.
#include "bf_common.h"

namespace bifocal {

__device__ __forceinline__ bool table_valid(const volatile TableHeader* h, int D, double theta,
                                            int n_needed) {
  return h->magic == kTableMagic && h->theta == theta && h->D == D && h->n_valid >= n_needed;
}

__global__ void __launch_bounds__(256) table_build_kernel(const TableHeader* hdr, float2* tab,
                                                          int n_build, int n_needed, int D,
                                                          double theta) {
  __shared__ int s_skip;
  if (threadIdx.x == 0) s_skip = table_valid(hdr, D, theta, n_needed) ? 1 : 0;
  __syncthreads();
  if (s_skip) return;

  // theta_m once per block (D/2 <= 128 values): a float64 pow per entry would cost
  // more than the sine and cosine together
  __shared__ double s_invf[128];
  const int half = D / 2;
  for (int m = threadIdx.x; m < half; m += blockDim.x) s_invf[m] = inv_freq64(theta, m, D);
  __syncthreads();
  const size_t total = (size_t)n_build * half;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int p = (int)(idx / half);
    const int m = (int)(idx - (size_t)p * half);
    const double a = (double)p * s_invf[m];
    double s, c;
    sincos_reduced(a, &s, &c);
    tab[idx] = make_float2((float)c, (float)s);
  }
}

__global__ void table_publish_kernel(TableHeader* hdr, int n_cap, int n_build, int n_needed,
                                     int D, double theta) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  volatile TableHeader* h = hdr;
  if (table_valid(h, D, theta, n_needed)) {
    // Rows past this call's capacity may be overwritten by its scratch: forget them
    // (n_needed <= n_cap, so this never turns the table invalid for this call).
    if (h->n_valid > n_cap) h->n_valid = n_cap;
    return;
  }
  // the build kernel of this call filled rows 0 .. n_build-1
  h->magic = 0;
  h->theta = theta;
  h->D = D;
  h->n_valid = n_build;
  h->magic = kTableMagic;
}

// Enqueue the table check/build (the full grid: a valid header sends every block home
// after one load).
hipError_t launch_table_ensure(void* ws, const WsLayout& lay, int D, double theta, int n_needed,
                               hipStream_t stream) {
  TableHeader* hdr = reinterpret_cast<TableHeader*>(ws);
  float2* tab = reinterpret_cast<float2*>(reinterpret_cast<char*>(ws) + lay.table_off);
  // Build ahead of need (to the next multiple of 64K positions, within capacity) so
  // that calls walking forward one position at a time rarely rebuild.
  const long long want = ((long long)n_needed + 65535) / 65536 * 65536;
  const int n_build = (int)(want < lay.n_cap ? want : lay.n_cap);
  size_t total = (size_t)n_build * (D / 2);
  int blocks = (int)((total + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(table_build_kernel, dim3(blocks), dim3(256), 0, stream, hdr, tab, n_build,
                     n_needed, D, theta);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(table_publish_kernel, dim3(1), dim3(64), 0, stream, hdr, lay.n_cap, n_build,
                     n_needed, D, theta);
  return hipGetLastError();
}

}  // namespace bifocal
