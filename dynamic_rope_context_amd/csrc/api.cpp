// C ABI of the bifocal RoPE attention library: argument validation, workspace
// layout, per-sequence group size, and kernel dispatch on the caller's stream.
// Every argument check happens before the first enqueue, so an error leaves all
// buffers untouched.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "bf_common.h"
#include "prefill_args.h"
#include "decode_args.h"

extern "C" {
#include "../../include/bifocal.h"
}

namespace bifocal {
hipError_t launch_table_ensure(void* ws, const WsLayout& lay, int D, double theta, int n_needed,
                               hipStream_t stream);
hipError_t launch_rope_apply(void* x, const int32_t* pos, int pos0, int T_, int H, int D,
                             double theta, int G, bool bf16, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillArgs& args, hipStream_t stream);
hipError_t launch_prefill_mfma(const PrefillArgs& args, int chunk_tiles, hipStream_t stream);
hipError_t launch_pair_select(const void* Q, const void* K, const void* V, int T, int Hq,
                              int Hkv, uint32_t* mx, int32_t* sel, hipStream_t stream);
int prefill_f32_rows_per_block();
int prefill_mfma_positions_per_block(int rep);

hipError_t launch_decode(const DecodeArgs& a, int rep, int D, bool bf16, hipStream_t stream);
hipError_t launch_decode_mfma(const DecodeBatchArgs& a, int rep, hipStream_t stream);
hipError_t launch_ie_merge(const float* oa, const float* ob, const float* oc, const float* la,
                           const float* lb, const float* lc, void* o, float* lse, int T, int Hq,
                           hipStream_t stream);
}  // namespace bifocal

using namespace bifocal;

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int32_t group_size(int64_t L, int32_t w_pre) {
  if (L < 0 || w_pre < 1) return 0;
  const int64_t G = (L + w_pre - 1) / w_pre;
  return (int32_t)std::max<int64_t>(1, G);
}

// The table check/build: every block of the full grid reads the header and leaves at
// once when the workspace already holds a table for (theta, D) with enough rows, so a
// repeated call costs one short launch; the host keeps no record of workspaces.
bf_status ensure_table(void* ws, const WsLayout& lay, int D, double theta, int n_needed,
                       hipStream_t stream) {
  return launch_table_ensure(ws, lay, D, theta, n_needed, stream) == hipSuccess ? BF_OK : BF_EHIP;
}

// Shared by bifocal_prefill (ie = false) and bifocal_prefill_ie (ie = true: the three
// inclusion-exclusion passes into fp32 intermediates, then the merge).
bf_status prefill_impl(const void* Q, const void* K, const void* V, void* O, float* lse,
                       const int32_t* cu_seqlens, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                       int32_t w0, int32_t w_pretrained, double theta, float softmax_scale,
                       bf_dtype dt, void* ws, size_t ws_bytes, bf_stream stream, bool ie,
                       int32_t variant = BF_VARIANT_BIFOCAL) {
  if (!cu_seqlens || B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || w0 < 1 || w_pretrained < 1 ||
      !(theta > 0.0) || !std::isfinite(theta) || !std::isfinite(softmax_scale))
    return BF_EINVAL;
  if (dt != BF_F32 && dt != BF_BF16) return BF_EINVAL;
  if (cu_seqlens[0] != 0) return BF_EINVAL;
  int32_t max_len = 0;
  for (int b = 0; b < B; ++b) {
    if (cu_seqlens[b + 1] < cu_seqlens[b]) return BF_EINVAL;
    max_len = std::max(max_len, cu_seqlens[b + 1] - cu_seqlens[b]);
  }
  const int32_t T = cu_seqlens[B];
  if (D != 64 && D != 128) return BF_EUNSUPPORTED;
  // positions must stay within the division-free alias range, and one sequence's rows
  // within 32-bit element offsets
  if (max_len >= kMaxPositions || (int64_t)max_len * std::max(Hq, Hkv) * D >= (1ll << 31))
    return BF_EUNSUPPORTED;
  const int rep = Hq / Hkv;
  if (dt == BF_BF16 && (D != 128 || (rep != 1 && rep != 2 && rep != 4 && rep != 8)))
    return BF_EUNSUPPORTED;
  if (ie && dt != BF_BF16) return BF_EUNSUPPORTED;
  if (variant < BF_VARIANT_BIFOCAL || variant > BF_VARIANT_WINDOW) return BF_EINVAL;
  if (variant != BF_VARIANT_BIFOCAL && dt != BF_BF16) return BF_EUNSUPPORTED;
  if (T == 0) return BF_OK;
  if (!Q || !K || !V || !O) return BF_EINVAL;
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) ||
      (lse && !aligned(lse, 4)))
    return BF_EINVAL;
  if (!ws || !aligned(ws, 256)) return BF_EWORKSPACE;
  // key-tile records (bf16 path): one per KV head and 32-key tile of every sequence
  int64_t tiles = 0;
  if (dt == BF_BF16)
    for (int b = 0; b < B; ++b)
      tiles += (cu_seqlens[b + 1] - cu_seqlens[b] + kKeyTileKeys - 1) / kKeyTileKeys;
  if (tiles > INT32_MAX) return BF_EUNSUPPORTED;
  const size_t rec_bytes = dt == BF_BF16 ? records_bytes(Hkv, tiles) : 0;
  const WsLayout lay =
      ws_layout(BF_OP_PREFILL, Hq, Hkv, D, ws_bytes, rec_bytes + (ie ? ie_bytes(T, Hq, D) : 0));
  if (lay.scratch_off == 0 || lay.n_cap < max_len) return BF_EWORKSPACE;

  hipStream_t st = (hipStream_t)stream;
  bf_status s = ensure_table(ws, lay, D, theta, max_len, st);
  if (s != BF_OK) return s;

  char* wsb = reinterpret_cast<char*>(ws);
  uint32_t* mx = reinterpret_cast<uint32_t*>(wsb + lay.scratch_off);
  int32_t* sel = reinterpret_cast<int32_t*>(wsb + lay.scratch_off + pair_max_bytes(Hq, Hkv));
  if (dt == BF_BF16) {
    if (launch_pair_select(Q, K, V, T, Hq, Hkv, mx, sel, st) != hipSuccess) return BF_EHIP;
  }

  PrefillArgs a{};
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.lse = lse;
  a.tab = reinterpret_cast<const float2*>(wsb + lay.table_off);
  a.sel = sel;
  a.rec = reinterpret_cast<uint8_t*>(wsb + lay.rec_off);
  a.tiles_total = (int32_t)tiles;
  a.T = T;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.w0 = w0;
  a.scale = softmax_scale > 0.f ? softmax_scale : (float)(1.0 / std::sqrt((double)D));
  a.theta = theta;
  a.interp = variant == BF_VARIANT_INTERP ? 1 : 0;
  a.mode = variant == BF_VARIANT_WINDOW ? 3 : 0;  // window-only: the local pass alone
  // inclusion-exclusion intermediates (pass A: local/window, B: remote/causal,
  // C: remote/window), after the records
  float* ie_o[3] = {nullptr, nullptr, nullptr};
  float* ie_l[3] = {nullptr, nullptr, nullptr};
  if (ie) {
    char* p = wsb + lay.rec_off + rec_bytes;
    for (int x = 0; x < 3; ++x) {
      ie_o[x] = reinterpret_cast<float*>(p);
      p += align_up((size_t)T * Hq * D * sizeof(float), 256);
      ie_l[x] = reinterpret_cast<float*>(p);
      p += align_up((size_t)Hq * T * sizeof(float), 256);
    }
  }
  const int rows = dt == BF_BF16 ? prefill_mfma_positions_per_block(rep)
                                 : prefill_f32_rows_per_block();
  int32_t tile_base = 0;
  for (int b0 = 0; b0 < B; b0 += kMaxSeqPerLaunch) {
    int n = 0, maxq = 0, chunk_tiles = 0;
    for (int b = b0; b < std::min(B, b0 + kMaxSeqPerLaunch); ++b) {
      const int L = cu_seqlens[b + 1] - cu_seqlens[b];
      if (L == 0) continue;
      const int nt = (L + kKeyTileKeys - 1) / kKeyTileKeys;
      a.seq[n].tile_base = tile_base;
      tile_base += nt;
      chunk_tiles += nt;
      a.seq[n].start = cu_seqlens[b];
      a.seq[n].len = L;
      a.seq[n].G = group_size(L, w_pretrained);
      const DivMagic dm = div_magic((uint32_t)a.seq[n].G);
      a.seq[n].gmul = dm.mul;
      a.seq[n].gshift = dm.shift;
      maxq = std::max(maxq, (L + rows - 1) / rows);
      ++n;
    }
    if (n == 0) continue;
    a.nseq = n;
    a.max_qblocks = maxq;
    {
      // levels of the matrix-core grid: sequences by query-block count, longest first
      int ord[kMaxSeqPerLaunch], cnt[kMaxSeqPerLaunch];
      for (int i = 0; i < n; ++i) {
        ord[i] = i;
        cnt[i] = (a.seq[i].len + rows - 1) / rows;
      }
      std::stable_sort(ord, ord + n, [&](int x, int y) { return cnt[x] > cnt[y]; });
      a.nlvl = n;
      a.lvl_start[0] = 0;
      for (int k = 0; k < n; ++k) {
        a.lvl_seq[k] = ord[k];
        a.lvl_qb[k] = cnt[ord[k]];
        const int next = k + 1 < n ? cnt[ord[k + 1]] : 0;
        a.lvl_start[k + 1] = a.lvl_start[k] + (a.lvl_qb[k] - next) * (k + 1);
      }
    }
    if (!ie) {
      hipError_t e = dt == BF_BF16 ? launch_prefill_mfma(a, chunk_tiles, st)
                                   : launch_prefill_f32(a, st);
      if (e != hipSuccess) return BF_EHIP;
      continue;
    }
    static const int kModes[3] = {3, 1, 2};  // passes A, B, C
    a.out_f32 = 1;
    for (int x = 0; x < 3; ++x) {
      a.mode = kModes[x];
      a.O = ie_o[x];
      a.lse = ie_l[x];
      // the key records are written once per chunk, by the first pass
      if (launch_prefill_mfma(a, x == 0 ? chunk_tiles : 0, st) != hipSuccess) return BF_EHIP;
    }
  }
  if (ie && launch_ie_merge(ie_o[0], ie_o[1], ie_o[2], ie_l[0], ie_l[1], ie_l[2], O, lse, T, Hq,
                            st) != hipSuccess)
    return BF_EHIP;
  return BF_OK;
}

}  // namespace

extern "C" {

const char* bifocal_status_string(int32_t s) {
  switch (s) {
    case BF_OK: return "ok";
    case BF_EINVAL: return "invalid argument";
    case BF_EUNSUPPORTED: return "unsupported configuration";
    case BF_EWORKSPACE: return "workspace missing or too small";
    case BF_EHIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

int32_t bifocal_group_size(int64_t L, int32_t w_pretrained) { return group_size(L, w_pretrained); }

size_t bifocal_workspace_bytes(int32_t op, int32_t max_len, int64_t total_tokens,
                               int32_t num_seqs, int32_t Hq, int32_t Hkv, int32_t D) {
  if (op < 0 || op > 3 || max_len < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv || (D != 64 && D != 128))
    return 0;
  if (op == BF_OP_ROPE) return 0;
  if ((op == BF_OP_PREFILL || op == BF_OP_PREFILL_IE) && (total_tokens < max_len || num_seqs < 1 ||
                              total_tokens > (int64_t)num_seqs * max_len))
    return 0;
  if (op == BF_OP_DECODE && num_seqs < 0) return 0;
  return ws_bytes_for(op, max_len, total_tokens, num_seqs, Hq, Hkv, D);
}

bf_status rope_apply(void* x, const int32_t* pos, int32_t pos0, int32_t T, int32_t H, int32_t D,
                     double theta, int32_t G, bf_dtype dt, bf_stream stream) {
  if (T < 0 || H < 1 || D < 2 || (D & 1) || G < 1 || !(theta > 0.0) || !std::isfinite(theta))
    return BF_EINVAL;
  if (dt != BF_F32 && dt != BF_BF16) return BF_EINVAL;
  if (D > 256) return BF_EUNSUPPORTED;
  if (T == 0) return BF_OK;
  if (!x) return BF_EINVAL;
  if (!pos && (pos0 < 0 || (int64_t)pos0 + T - 1 > INT32_MAX)) return BF_EINVAL;
  if (!aligned(x, dt == BF_BF16 ? 2 : 4) || (pos && !aligned(pos, 4))) return BF_EINVAL;
  hipError_t e = launch_rope_apply(x, pos, pos0, T, H, D, theta, G, dt == BF_BF16,
                                   (hipStream_t)stream);
  return e == hipSuccess ? BF_OK : BF_EHIP;
}

bf_status bifocal_prefill(const void* Q, const void* K, const void* V, void* O, float* lse,
                          const int32_t* cu_seqlens, int32_t B, int32_t Hq, int32_t Hkv,
                          int32_t D, int32_t w0, int32_t w_pretrained, double theta,
                          float softmax_scale, bf_dtype dt, void* ws, size_t ws_bytes,
                          bf_stream stream) {
  return prefill_impl(Q, K, V, O, lse, cu_seqlens, B, Hq, Hkv, D, w0, w_pretrained, theta,
                      softmax_scale, dt, ws, ws_bytes, stream, false);
}

bf_status bifocal_prefill_variant(const void* Q, const void* K, const void* V, void* O, float* lse,
                                  const int32_t* cu_seqlens, int32_t B, int32_t Hq, int32_t Hkv,
                                  int32_t D, int32_t w0, int32_t w_pretrained, double theta,
                                  float softmax_scale, int32_t variant, bf_dtype dt, void* ws,
                                  size_t ws_bytes, bf_stream stream) {
  return prefill_impl(Q, K, V, O, lse, cu_seqlens, B, Hq, Hkv, D, w0, w_pretrained, theta,
                      softmax_scale, dt, ws, ws_bytes, stream, false, variant);
}

bf_status bifocal_prefill_ie(const void* Q, const void* K, const void* V, void* O, float* lse,
                             const int32_t* cu_seqlens, int32_t B, int32_t Hq, int32_t Hkv,
                             int32_t D, int32_t w0, int32_t w_pretrained, double theta,
                             float softmax_scale, bf_dtype dt, void* ws, size_t ws_bytes,
                             bf_stream stream) {
  return prefill_impl(Q, K, V, O, lse, cu_seqlens, B, Hq, Hkv, D, w0, w_pretrained, theta,
                      softmax_scale, dt, ws, ws_bytes, stream, true);
}

}  // extern "C"

namespace {

// Shared by bifocal_decode (one sequence), bifocal_decode_batch and the variants.  With
// fixed_part set (the no-allocation entry point), the matrix-core path keeps its partials
// there (fixed_part_bytes of room) instead of in a workspace, and other paths are refused.
bf_status decode_impl(const void* q, const void* Kcache, const void* Vcache, void* o, float* lse,
                      const int32_t* pos, int32_t B, int64_t S, int32_t Hq, int32_t Hkv,
                      int32_t D, int32_t w0, int32_t w_pretrained, double theta,
                      float softmax_scale, bf_dtype dt, void* ws, size_t ws_bytes,
                      bf_stream stream, int32_t variant = BF_VARIANT_BIFOCAL,
                      float* fixed_part = nullptr, size_t fixed_part_bytes = 0,
                      bool validate_only = false) {
  if (B < 0 || (B > 0 && (!q || !Kcache || !Vcache || !o || !pos)) || S < 1 || Hq < 1 ||
      Hkv < 1 || Hq % Hkv || w0 < 1 || w_pretrained < 1 || !(theta > 0.0) ||
      !std::isfinite(theta) || !std::isfinite(softmax_scale))
    return BF_EINVAL;
  if (dt != BF_F32 && dt != BF_BF16) return BF_EINVAL;
  if (variant < BF_VARIANT_BIFOCAL || variant > BF_VARIANT_WINDOW) return BF_EINVAL;
  if (D != 64 && D != 128) return BF_EUNSUPPORTED;
  if (variant != BF_VARIANT_BIFOCAL && (dt != BF_BF16 || D != 128)) return BF_EUNSUPPORTED;
  const int rep = Hq / Hkv;
  if (rep != 1 && rep != 2 && rep != 4 && rep != 8) return BF_EUNSUPPORTED;
  int32_t max_pos = -1;
  for (int32_t b = 0; b < B; ++b) {
    if (pos[b] < 0 || pos[b] >= S) return BF_EINVAL;
    max_pos = std::max(max_pos, pos[b]);
  }
  if (B == 0) return BF_OK;
  if (!aligned(q, 16) || !aligned(Kcache, 16) || !aligned(Vcache, 16) ||
      !aligned(o, dt == BF_BF16 ? 2 : 4) || (lse && !aligned(lse, 4)))
    return BF_EINVAL;
  const int32_t n_keys = max_pos + 1;
  if (n_keys >= kMaxPositions) return BF_EUNSUPPORTED;
  const size_t part_row = (size_t)(D + 2) * sizeof(float);  // one partial
  WsLayout lay{};
  if (fixed_part || validate_only) {
    if (dt != BF_BF16 || D != 128) return BF_EUNSUPPORTED;
    // at least one partial per (sequence, query head) of a launch must fit
    if ((size_t)std::min<int32_t>(B, kDecodeMaxBatch) * Hq * part_row > fixed_part_bytes)
      return BF_EWORKSPACE;
  } else {
    if (!ws || !aligned(ws, 256)) return BF_EWORKSPACE;
    lay = ws_layout(BF_OP_DECODE, Hq, Hkv, D, ws_bytes, 0, B);
    if (lay.scratch_off == 0 || lay.n_cap < n_keys) return BF_EWORKSPACE;
  }
  if (validate_only) return BF_OK;

  hipStream_t st = (hipStream_t)stream;
  char* wsb = reinterpret_cast<char*>(ws);
  const double scale = softmax_scale > 0.f ? softmax_scale : 1.0 / std::sqrt((double)D);
  const float scale_log2 = (float)(scale * 1.4426950408889634);
  const size_t esz = dt == BF_BF16 ? 2 : 4;
  const int64_t seq_stride = S * Hkv * D;  // elements

  if (dt == BF_BF16 && D == 128) {
    // Matrix-core kernel: angles evaluated in the kernel (no table), then the combine.
    // Split count: about two workgroups per CU over the whole launch, at least eight
    // 16-key blocks per wave when the sequences are long enough.
    DecodeBatchArgs a{};
    a.q = q;
    a.K = Kcache;
    a.V = Vcache;
    a.part = fixed_part ? fixed_part : reinterpret_cast<float*>(wsb + lay.scratch_off);
    a.o = o;
    a.lse = lse;
    a.seq_stride = seq_stride;
    a.theta = theta;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.w0 = w0;
    a.scale_log2 = scale_log2;
    a.variant = variant;
    a.hdr = fixed_part ? nullptr : reinterpret_cast<TableHeader*>(ws);
    a.n_cap = lay.n_cap;
    for (int32_t b0 = 0; b0 < B; b0 += kDecodeMaxBatch) {
      const int nb = std::min<int32_t>(kDecodeMaxBatch, B - b0);
      int32_t mp = 0;
      for (int i = 0; i < nb; ++i) mp = std::max(mp, pos[b0 + i]);
      // key blocks per sequence (window-only: those of the last w0 keys)
      const int64_t nblk = variant == BF_VARIANT_WINDOW ? std::min<int64_t>(mp, w0) / 16 + 2
                                                        : mp / 16 + 1;
      int64_t nwg = (512 + (int64_t)nb * Hkv - 1) / ((int64_t)nb * Hkv);
      nwg = std::min<int64_t>(nwg, std::max<int64_t>(1, nblk / (4 * 8)));
      nwg = std::max<int64_t>(1, std::min<int64_t>(nwg, kDecodeMaxParts));
      if (fixed_part)  // fewer splits when the fixed buffer holds fewer partials
        nwg = std::max<int64_t>(
            1, std::min<int64_t>(nwg, (int64_t)(fixed_part_bytes / ((size_t)nb * Hq * part_row))));
      a.b_base = b0;
      a.nseq = nb;
      a.nwg = (int32_t)nwg;
      a.nsplit = (int32_t)nwg * 4;
      for (int i = 0; i < nb; ++i) {
        const int32_t G = group_size((int64_t)pos[b0 + i] + 1, w_pretrained);
        const DivMagic m = div_magic((uint32_t)G);
        a.seq[i] = DecSeq{pos[b0 + i], m.mul, m.shift, G};
      }
      if (launch_decode_mfma(a, rep, st) != hipSuccess) return BF_EHIP;
    }
    return BF_OK;
  }

  if (fixed_part) return BF_EUNSUPPORTED;  // unreachable: checked above
  // Vector path: one split launch + combine per sequence, sharing the table and the
  // partials buffer (stream order).
  bf_status s = ensure_table(ws, lay, D, theta, n_keys, st);
  if (s != BF_OK) return s;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t nk = pos[b] + 1;
    // Split the cache so that ~2048 workgroups stream it; splits are whole multiples of
    // 64 keys and their count a multiple of 8 (one slice per XCD).
    int nsplit = (2048 + Hkv - 1) / Hkv;
    nsplit = std::min(kDecodeMaxSplits, std::max(8, (nsplit + 7) / 8 * 8));
    int kps = (nk + nsplit - 1) / nsplit;
    kps = (kps + 63) / 64 * 64;
    nsplit = (nk + kps - 1) / kps;
    nsplit = (nsplit + 7) / 8 * 8;
    if (nsplit > kDecodeMaxSplits) return BF_EUNSUPPORTED;
    DecodeArgs a{};
    a.q = reinterpret_cast<const char*>(q) + (size_t)b * Hq * D * esz;
    a.K = reinterpret_cast<const char*>(Kcache) + (size_t)b * seq_stride * esz;
    a.V = reinterpret_cast<const char*>(Vcache) + (size_t)b * seq_stride * esz;
    a.tab = reinterpret_cast<const float2*>(wsb + lay.table_off);
    a.part = reinterpret_cast<float*>(wsb + lay.scratch_off);
    a.o = reinterpret_cast<char*>(o) + (size_t)b * Hq * D * esz;
    a.lse = lse ? lse + (size_t)b * Hq : nullptr;
    a.pos = pos[b];
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.w0 = w0;
    a.G = group_size((int64_t)pos[b] + 1, w_pretrained);
    a.gdiv = div_magic((uint32_t)a.G);
    a.nsplit = nsplit;
    a.kps = kps;
    a.scale_log2 = scale_log2;
    if (launch_decode(a, rep, D, dt == BF_BF16, st) != hipSuccess) return BF_EHIP;
  }
  return BF_OK;
}

}  // namespace

namespace bifocal {
// bifocal_decode with its partials in a caller-given device buffer (no workspace).  With
// part = null, only the argument checks run (no HIP call): the status they return.
bf_status decode_fixed_partials(const void* q, const void* Kcache, const void* Vcache, void* o,
                                float* lse, int32_t pos, int32_t Hq, int32_t Hkv, int32_t D,
                                int32_t w0, int32_t w_pretrained, double theta,
                                float softmax_scale, bf_dtype dt, float* part, size_t part_bytes,
                                bf_stream stream) {
  if (pos < 0 || pos == INT32_MAX) return BF_EINVAL;
  return decode_impl(q, Kcache, Vcache, o, lse, &pos, 1, (int64_t)pos + 1, Hq, Hkv, D, w0,
                     w_pretrained, theta, softmax_scale, dt, nullptr, 0, stream,
                     BF_VARIANT_BIFOCAL, part, part ? part_bytes : BIFOCAL_NOALLOC_SCRATCH_BYTES,
                     part == nullptr);
}
}  // namespace bifocal

extern "C" {

bf_status bifocal_decode(const void* q, const void* Kcache, const void* Vcache, void* o,
                         float* lse, int32_t pos, int32_t Hq, int32_t Hkv, int32_t D, int32_t w0,
                         int32_t w_pretrained, double theta, float softmax_scale, bf_dtype dt,
                         void* ws, size_t ws_bytes, bf_stream stream) {
  if (pos < 0 || pos == INT32_MAX) return BF_EINVAL;
  return decode_impl(q, Kcache, Vcache, o, lse, &pos, 1, (int64_t)pos + 1, Hq, Hkv, D, w0,
                     w_pretrained, theta, softmax_scale, dt, ws, ws_bytes, stream);
}

bf_status bifocal_decode_variant(const void* q, const void* Kcache, const void* Vcache, void* o,
                                 float* lse, const int32_t* pos, int32_t B, int32_t S, int32_t Hq,
                                 int32_t Hkv, int32_t D, int32_t w0, int32_t w_pretrained,
                                 double theta, float softmax_scale, int32_t variant, bf_dtype dt,
                                 void* ws, size_t ws_bytes, bf_stream stream) {
  return decode_impl(q, Kcache, Vcache, o, lse, pos, B, S, Hq, Hkv, D, w0, w_pretrained, theta,
                     softmax_scale, dt, ws, ws_bytes, stream, variant);
}

bf_status bifocal_decode_batch(const void* q, const void* Kcache, const void* Vcache, void* o,
                               float* lse, const int32_t* pos, int32_t B, int32_t S, int32_t Hq,
                               int32_t Hkv, int32_t D, int32_t w0, int32_t w_pretrained,
                               double theta, float softmax_scale, bf_dtype dt, void* ws,
                               size_t ws_bytes, bf_stream stream) {
  return decode_impl(q, Kcache, Vcache, o, lse, pos, B, S, Hq, Hkv, D, w0, w_pretrained, theta,
                     softmax_scale, dt, ws, ws_bytes, stream);
}

}  // extern "C"
