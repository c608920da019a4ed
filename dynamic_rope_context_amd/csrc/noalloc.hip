// bifocal_decode_noalloc: one bf16 decode step that allocates nothing and takes no
// workspace, for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// The matrix-core decode needs device memory beyond its inputs and outputs only for its
// split partials (acc[D], m, l per query head and split).  Here they live in a file-scope
// device array of fixed size, one copy per GPU, held until the process ends.  Its device
// address is looked up once per device (the host-side name of the array is not a device
// address) and kept in a small per-device table.  Every call on a GPU shares that GPU's
// array, so calls that overlap on one GPU race; calls ordered on one stream do not.  The
// partials are written before they are read, so nothing needs clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "bf_common.h"

extern "C" {
#include "../../include/bifocal.h"
}

namespace bifocal {
bf_status decode_fixed_partials(const void* q, const void* Kcache, const void* Vcache, void* o,
                                float* lse, int32_t pos, int32_t Hq, int32_t Hkv, int32_t D,
                                int32_t w0, int32_t w_pretrained, double theta,
                                float softmax_scale, bf_dtype dt, float* part, size_t part_bytes,
                                bf_stream stream);
}  // namespace bifocal

// 4 MiB: 64 query heads x 128 splits x (128 + 2) floats fit with room to spare.
static __device__ __align__(256) uint8_t scratch[BIFOCAL_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_status[kMaxDevices];

}  // namespace

extern "C" bf_status bifocal_decode_noalloc(const void* q, const void* Kcache, const void* Vcache,
                                            void* o, float* lse, int32_t pos, int32_t Hq,
                                            int32_t Hkv, int32_t D, int32_t w0,
                                            int32_t w_pretrained, double theta,
                                            float softmax_scale, bf_dtype dt, bf_stream stream) {
  // argument errors first, before any HIP call
  const bf_status chk = bifocal::decode_fixed_partials(q, Kcache, Vcache, o, lse, pos, Hq, Hkv,
                                                       D, w0, w_pretrained, theta, softmax_scale,
                                                       dt, nullptr, 0, stream);
  if (chk != BF_OK) return chk;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BF_EHIP;
  if (stream) {
    // the array's address is per device: the stream must run on the current device
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess) return BF_EHIP;
    if ((int)sdev != dev) return BF_EINVAL;
  }
  std::call_once(g_once[dev], [dev] {
    g_status[dev] = hipGetSymbolAddress(&g_scratch[dev], HIP_SYMBOL(scratch));
  });
  if (g_status[dev] != hipSuccess || !g_scratch[dev]) return BF_EHIP;
  return bifocal::decode_fixed_partials(q, Kcache, Vcache, o, lse, pos, Hq, Hkv, D, w0,
                                        w_pretrained, theta, softmax_scale, dt,
                                        static_cast<float*>(g_scratch[dev]),
                                        BIFOCAL_NOALLOC_SCRATCH_BYTES, stream);
}
