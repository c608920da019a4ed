// Host stand-ins for the kernel launchers of libbifocal, for the sanitizer build of the
// C-ABI layer (tests/test_host_sanitizers.py).  Built host-only; every pointer the ABI
// passes to a "launch" is host memory in that test.  Each stand-in touches (reads and
// writes) every byte its kernel would access through the arguments it is given, so
// AddressSanitizer reports any workspace carving or argument bookkeeping that points
// outside the caller's buffers.  Nothing here runs on, or describes, the GPU path's
// arithmetic.
#include <hip/hip_runtime.h>

#include <cstring>

#include "../dynamic_rope_context_amd/csrc/bf_common.h"
#include "../dynamic_rope_context_amd/csrc/decode_args.h"
#include "../dynamic_rope_context_amd/csrc/prefill_args.h"

namespace {
volatile unsigned char g_sink;
void touch(const void* p, size_t n) {
  if (!p || !n) return;
  const unsigned char* c = static_cast<const unsigned char*>(p);
  unsigned char x = 0;
  for (size_t i = 0; i < n; ++i) x ^= c[i];
  g_sink = x;
}
void touch_w(void* p, size_t n) {
  if (p && n) std::memset(p, 0x5a, n);
}
}  // namespace

namespace bifocal {

hipError_t launch_table_ensure(void* ws, const WsLayout& lay, int D, double, int n_needed,
                               hipStream_t) {
  touch_w(ws, sizeof(TableHeader));
  // the build writes up to the next multiple of 65536 rows within the table region
  const long long want = ((long long)n_needed + 65535) / 65536 * 65536;
  const long long n_build = want < lay.n_cap ? want : lay.n_cap;
  touch_w(static_cast<char*>(ws) + lay.table_off, (size_t)n_build * table_row_bytes(D));
  return hipSuccess;
}

hipError_t launch_rope_apply(void* x, const int32_t* pos, int, int T_, int H, int D, double, int,
                             bool bf16, hipStream_t) {
  touch_w(x, (size_t)T_ * H * D * (bf16 ? 2 : 4));
  if (pos) touch(pos, (size_t)T_ * sizeof(int32_t));
  return hipSuccess;
}

hipError_t launch_pair_select(const void* Q, const void* K, const void* V, int T, int Hq, int Hkv,
                              uint32_t* mx, int32_t* sel, hipStream_t) {
  touch(Q, (size_t)T * Hq * 128 * 2);
  touch(K, (size_t)T * Hkv * 128 * 2);
  touch(V, (size_t)T * Hkv * 128 * 2);
  touch_w(mx, (size_t)(Hq + 2 * Hkv) * 64 * sizeof(uint32_t));
  touch_w(sel, (size_t)Hkv * kSelStride * sizeof(int32_t));
  return hipSuccess;
}

static void touch_prefill(const PrefillArgs& a, size_t esz, bool records) {
  for (int i = 0; i < a.nseq; ++i) {
    const size_t s = a.seq[i].start, L = a.seq[i].len;
    touch(static_cast<const char*>(a.Q) + s * a.Hq * a.D * esz, L * a.Hq * a.D * esz);
    touch(static_cast<const char*>(a.K) + s * a.Hkv * a.D * esz, L * a.Hkv * a.D * esz);
    touch(static_cast<const char*>(a.V) + s * a.Hkv * a.D * esz, L * a.Hkv * a.D * esz);
    const size_t osz = a.out_f32 ? 4 : esz;
    touch_w(static_cast<char*>(a.O) + s * a.Hq * a.D * osz, L * a.Hq * a.D * osz);
    if (a.lse)
      for (int h = 0; h < a.Hq; ++h) touch_w(a.lse + (size_t)h * a.T + s, L * sizeof(float));
    touch(a.tab, L * (size_t)(a.D / 2) * sizeof(float2));
    if (records) {
      const size_t tiles = (L + kRecKeys - 1) / kRecKeys;
      for (int g = 0; g < a.Hkv; ++g)
        touch_w(a.rec + ((size_t)g * a.tiles_total + a.seq[i].tile_base) * kRecBytes,
                tiles * kRecBytes);
    }
  }
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, int, hipStream_t) {
  touch(a.sel, (size_t)a.Hkv * kSelStride * sizeof(int32_t));
  touch_prefill(a, 2, true);
  // every grid position decodes to a real (sequence, query block)
  const int rows = 256 / (a.Hq / a.Hkv);
  for (int pid = 0; pid < a.lvl_start[a.nlvl]; ++pid) {
    int lv = 0;
    while (lv + 1 < a.nlvl && a.lvl_start[lv + 1] <= pid) ++lv;
    const int r = pid - a.lvl_start[lv];
    const int qb = a.lvl_qb[lv] - 1 - r / (lv + 1);
    const int b = a.lvl_seq[r % (lv + 1)];
    if (b < 0 || b >= a.nseq || qb < 0 || qb * rows >= a.seq[b].len) return hipErrorInvalidValue;
  }
  return hipSuccess;
}

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t) {
  touch_prefill(a, 4, false);
  return hipSuccess;
}

int prefill_f32_rows_per_block() { return 64; }
int prefill_mfma_positions_per_block(int rep) { return 256 / rep; }

hipError_t launch_ie_merge(const float* oa, const float* ob, const float* oc, const float* la,
                           const float* lb, const float* lc, void* o, float* lse, int T, int Hq,
                           hipStream_t) {
  const size_t n = (size_t)T * Hq * 128;
  touch(oa, n * 4);
  touch(ob, n * 4);
  touch(oc, n * 4);
  touch(la, (size_t)T * Hq * 4);
  touch(lb, (size_t)T * Hq * 4);
  touch(lc, (size_t)T * Hq * 4);
  touch_w(o, n * 2);
  if (lse) touch_w(lse, (size_t)T * Hq * 4);
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, int rep, int D, bool bf16, hipStream_t) {
  const size_t esz = bf16 ? 2 : 4;
  const size_t Hkv = a.Hq / rep;
  touch(a.q, (size_t)a.Hq * D * esz);
  touch(a.K, (size_t)(a.pos + 1) * Hkv * D * esz);
  touch(a.V, (size_t)(a.pos + 1) * Hkv * D * esz);
  touch(a.tab, (size_t)(a.pos + 1) * (D / 2) * sizeof(float2));
  touch_w(a.part, (size_t)a.Hq * a.nsplit * (D + 2) * sizeof(float));
  touch_w(a.o, (size_t)a.Hq * D * esz);
  if (a.lse) touch_w(a.lse, (size_t)a.Hq * sizeof(float));
  return hipSuccess;
}

hipError_t launch_decode_mfma(const DecodeBatchArgs& a, int, hipStream_t) {
  for (int i = 0; i < a.nseq; ++i) {
    const size_t b = a.b_base + i;
    const size_t keys = (size_t)a.seq[i].pos + 1;
    touch(static_cast<const char*>(a.q) + b * a.Hq * 128 * 2, (size_t)a.Hq * 128 * 2);
    touch(static_cast<const char*>(a.K) + b * a.seq_stride * 2, keys * a.Hkv * 128 * 2);
    touch(static_cast<const char*>(a.V) + b * a.seq_stride * 2, keys * a.Hkv * 128 * 2);
    touch_w(static_cast<char*>(a.o) + b * a.Hq * 128 * 2, (size_t)a.Hq * 128 * 2);
    if (a.lse) touch_w(a.lse + b * a.Hq, (size_t)a.Hq * sizeof(float));
  }
  touch_w(a.part, (size_t)a.nseq * a.Hq * a.nwg * (128 + 2) * sizeof(float));
  if (a.hdr) touch_w(a.hdr, sizeof(TableHeader));
  return hipSuccess;
}

}  // namespace bifocal
