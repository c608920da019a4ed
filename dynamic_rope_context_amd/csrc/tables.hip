// RoPE / correction-angle table generator (gfx950).
//
// Fills tab[p][m] = (cos(p*theta_m), sin(p*theta_m)) for p < n_cap, angles formed in
// float64 from the integer position and rounded once to float32.  The same table
// gives standard RoPE at p and, read at n = x - floor(x/G) with the sine negated, the
// correction rotation R(f(x) - x) that moves a standard-RoPE vector at x to the
// aliased position f(x) (Jet-Long technical summary, "Methodology" section 1 for f,
// section 2 "on-the-fly correction rotation" for the additive composition).
//
// The table persists in the caller's workspace behind a header.  Every block reads
// the header first and leaves at once when it already describes (theta, D) with
// enough positions, so a launch on a valid table costs one header read per block.
// When a build runs, the last block to finish publishes the header; blocks count
// themselves with a token-tagged 64-bit counter so that stale workspace contents
// can never be mistaken for a finished count.
#include "bf_common.h"

namespace bifocal {

__global__ void __launch_bounds__(256) table_ensure_kernel(TableHeader* hdr, float2* tab,
                                                           int n_cap, int n_build, int n_needed,
                                                           int D, double theta, uint32_t token) {
  __shared__ int s_skip;
  if (threadIdx.x == 0) {
    volatile TableHeader* h = hdr;
    const bool ok = h->magic == kTableMagic && h->theta == theta && h->D == D;
    s_skip = ok && h->n_valid >= n_needed ? 1 : 0;
    // Rows past this call's capacity may be overwritten by its scratch: forget them.
    // (n_needed <= n_cap, so lowering n_valid to n_cap never changes a skip decision.)
    if (ok && blockIdx.x == 0 && h->n_valid > n_cap) h->n_valid = n_cap;
  }
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

  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long* cnt = reinterpret_cast<unsigned long long*>(&hdr->done);
    unsigned long long old = *(volatile unsigned long long*)cnt, assumed, nv;
    do {
      assumed = old;
      nv = ((assumed >> 32) == token) ? assumed + 1ull
                                      : (((unsigned long long)token << 32) | 1ull);
      old = atomicCAS(cnt, assumed, nv);
    } while (old != assumed);
    const unsigned count = (unsigned)(nv & 0xffffffffull);
    if (count == gridDim.x) {
      __threadfence();
      volatile TableHeader* h = hdr;
      h->magic = 0;
      __threadfence();
      h->theta = theta;
      h->D = D;
      h->n_valid = n_build;
      __threadfence();
      h->magic = kTableMagic;
      __threadfence();
    }
  }
}

// Enqueue the table check/build.  `full` selects a grid that builds quickly; a
// one-block launch still builds (slowly) if the header turns out to be stale.
hipError_t launch_table_ensure(void* ws, const WsLayout& lay, int D, double theta, int n_needed,
                               bool full, uint32_t token, hipStream_t stream) {
  TableHeader* hdr = reinterpret_cast<TableHeader*>(ws);
  float2* tab = reinterpret_cast<float2*>(reinterpret_cast<char*>(ws) + lay.table_off);
  // Build ahead of need (to the next multiple of 64K positions, within capacity) so
  // that decode steps walking forward one position at a time rarely rebuild.
  const long long want = ((long long)n_needed + 65535) / 65536 * 65536;
  const int n_build = (int)(want < lay.n_cap ? want : lay.n_cap);
  size_t total = (size_t)n_build * (D / 2);
  int blocks = full ? (int)((total + 255) / 256) : 1;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(table_ensure_kernel, dim3(blocks), dim3(256), 0, stream, hdr, tab,
                     lay.n_cap, n_build, n_needed, D, theta, token);
  return hipGetLastError();
}

}  // namespace bifocal
