/*
 * bifocal.h -- C ABI of the MI355X (gfx950) Dynamic Bifocal RoPE attention library.
 *
 * The method (Jet-Long, "Efficient Long-Context Extension with Dynamic Bifocal
 * RoPE"; technical summary on gist.science, "Methodology" sections 1 and 2):
 * causal grouped-query attention in which each query-key pair is scored one of
 * two ways.  Keys within a sliding window of w0 positions of the query use
 * standard RoPE; every other key uses RoPE at aliased positions f(x) = floor(x/G)
 * with G = max(1, ceil(L / w_pretrained)) from the current sequence length L.
 * Both score sets enter one online softmax (the pages' inclusion-exclusion merge
 * of three FlashAttention passes, realised here as a per-pair selection).  The
 * remote branch gets its phases from a correction rotation R(f(x) - x) applied
 * on the fly to queries and keys that carry standard RoPE, so a KV cache built
 * with standard RoPE is read as is and never rewritten.
 *
 * Conventions shared by every call
 *   - Pointers marked (device) are device pointers; (host) are host pointers.
 *   - Tensors are contiguous with the head dimension innermost:
 *       Q, O: [T, Hq, D];  K, V: [T, Hkv, D];  decode cache: [S, Hkv, D].
 *     Pointers to bf16/f32 tensors must be 16-byte aligned.
 *   - RoPE pairs channel m with m + D/2 (rotate-half); theta_m = theta^(-2m/D);
 *     angles are formed in float64 from integer positions; cos/sin are rounded
 *     once to float32.
 *   - The caller owns every buffer.  The library never allocates or frees device
 *     memory and never synchronises: work is enqueued on the given stream.
 *   - The workspace (device, caller-owned, size from bifocal_workspace_bytes) keeps a
 *     position table between calls; calls that share a workspace must be ordered
 *     (same stream or explicit events).  A workspace's first use needs no
 *     initialisation: its table carries a validity header the kernels check.
 *   - Argument errors are returned before anything is enqueued and nothing is
 *     written.  BF_EHIP reports a failed launch (hipGetLastError after the launch);
 *     faults inside kernels surface at the caller's next stream synchronisation.
 *   - Supported head dims: D in {64, 128}.  Hq must be a multiple of Hkv.
 *   - Lengths: a prefill sequence's length L and a decode step's pos + 1 must be below
 *     2^24 (the range in which the aliased position floor(x / G) is formed with a
 *     multiply and shift, exactly), and a prefill sequence's L * max(Hq, Hkv) * D below
 *     2^31 (32-bit row offsets); BF_EUNSUPPORTED otherwise.
 *   - Thread safety: concurrent calls are safe on distinct workspaces.
 */
#ifndef BIFOCAL_H_
#define BIFOCAL_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BF_OK = 0,
  BF_EINVAL = 1,       /* bad argument: null pointer, bad size, misaligned pointer */
  BF_EUNSUPPORTED = 2, /* valid but not implemented: head dim, GQA ratio, dtype     */
  BF_EWORKSPACE = 3,   /* workspace missing or smaller than bifocal_workspace_bytes  */
  BF_EHIP = 4          /* a HIP launch or runtime call failed                        */
} bf_status;

typedef enum { BF_F32 = 0, BF_BF16 = 1 } bf_dtype;

typedef enum { BF_OP_ROPE = 0, BF_OP_PREFILL = 1, BF_OP_DECODE = 2, BF_OP_PREFILL_IE = 3 } bf_op;

/*
 * Attention variants (bifocal_prefill_variant, bifocal_decode_variant):
 *   BF_VARIANT_BIFOCAL  the method: remote pairs at f(x) = floor(x / G).
 *   BF_VARIANT_INTERP   remote pairs at the continuous positions x / G: frequency
 *                       interpolation, the alternative the pages' ablation compares
 *                       aliasing against ("aliasing vs interpolation").
 *   BF_VARIANT_WINDOW   the local window alone (0 <= i - j < w0, standard RoPE), the
 *                       shape of a sliding-window layer in the hybrid models the pages
 *                       discuss (Jet-Nemotron); remote pairs are dropped.
 */
typedef enum { BF_VARIANT_BIFOCAL = 0, BF_VARIANT_INTERP = 1, BF_VARIANT_WINDOW = 2 } bf_variant;

/* HIP stream handle; 0 is the default stream. */
typedef struct ihipStream_t* bf_stream;

/*
 * rope_apply -- in-place RoPE at (aliased) positions: x[t,h,:] <- R(floor(p_t / G)) x[t,h,:].
 *   G = 1 is standard RoPE, which is how a caller builds Q_std and the K cache the
 *   two attention calls expect (the pages' cache stores keys with standard RoPE at
 *   exact absolute positions; "Methodology" section 2).  G > 1 moves vectors to the
 *   aliased grid of section 1 (used for checks and for materialising remote keys).
 *   x    (device) [T, H, D] in dtype dt, rotated in place (float32 arithmetic).
 *   pos  (device) [T] int32 positions >= 0, or NULL for p_t = pos0 + t.
 *   Errors: BF_EINVAL if x is NULL, T < 0, H < 1, D not even, G < 1, theta <= 0,
 *           pos0 < 0 with pos NULL; BF_EUNSUPPORTED for D > 256.  T = 0 is a no-op.
 */
bf_status rope_apply(void* x, const int32_t* pos, int32_t pos0, int32_t T, int32_t H, int32_t D,
                     double theta, int32_t G, bf_dtype dt, bf_stream stream);

/*
 * bifocal_prefill -- causal bifocal attention over packed variable-length sequences.
 *   Sequence b owns tokens cu_seqlens[b] .. cu_seqlens[b+1]-1 and local positions
 *   0 .. L_b-1; its G_b = max(1, ceil(L_b / w_pretrained)) (section 1, computed here
 *   per sequence, never passed in).  For query i and key j <= i of the same sequence:
 *   local (i - j < w0):  s = scale * <Q_i, K_j>                  (standard RoPE)
 *   remote (otherwise):  s = scale * <R(f(i)-i) Q_i, R(f(j)-j) K_j> (RoPE at f(i), f(j))
 *   O_i = sum_j softmax_j(s) V_j;  lse_i = ln sum_j exp(s_ij).
 *   Q   (device) [T, Hq, D]  standard RoPE at local positions.
 *   K   (device) [T, Hkv, D] standard RoPE at local positions.
 *   V   (device) [T, Hkv, D].
 *   O   (device) [T, Hq, D] output, dtype dt (fully overwritten).
 *   lse (device) [Hq, T] float32 output, or NULL.
 *   cu_seqlens (host) [B+1] int32, non-decreasing, cu_seqlens[0] = 0, cu_seqlens[B] = T.
 *   w0 >= 1 (window size), w_pretrained >= 1, theta > 0, softmax_scale <= 0 selects 1/sqrt(D).
 *   dt = BF_BF16: bf16 in/out, bf16/fp16 MFMA with fp32 accumulation; the remote
 *     branch uses fp16 operands plus a hi/lo correction on the 4 RoPE pairs per KV
 *     head with the largest magnitude bound (chosen by a pre-pass over Q and K).
 *     Requires D = 128 and Hq/Hkv in {1, 2, 4, 8}.  Inputs must be finite: for NaN or
 *     infinity in Q, K or V the outputs are unspecified.
 *   dt = BF_F32: float32 in/out and arithmetic (VALU); D in {64, 128}, any Hq/Hkv.
 *   ws, ws_bytes: workspace (device) of at least
 *     bifocal_workspace_bytes(BF_OP_PREFILL, max_b L_b, T, B, Hq, Hkv, D).  Besides the
 *     position table it holds, for bf16, one record per KV head and 32-key tile (the
 *     keys rotated to their aliased positions once per call, their hi/lo operand, and
 *     V transposed), so its size grows with T.
 *   Errors: BF_EINVAL (null pointer, bad cu_seqlens, w0 < 1, ...), BF_EUNSUPPORTED,
 *           BF_EWORKSPACE; T = 0 is a no-op.
 */
bf_status bifocal_prefill(const void* Q, const void* K, const void* V, void* O, float* lse,
                          const int32_t* cu_seqlens, int32_t B, int32_t Hq, int32_t Hkv,
                          int32_t D, int32_t w0, int32_t w_pretrained, double theta,
                          float softmax_scale, bf_dtype dt, void* ws, size_t ws_bytes,
                          bf_stream stream);

/*
 * bifocal_prefill_variant -- bifocal_prefill for an attention variant (bf_variant).
 *   BF_VARIANT_BIFOCAL is bifocal_prefill.  BF_VARIANT_INTERP and BF_VARIANT_WINDOW run
 *   the bf16 matrix-core path only (dt = BF_BF16, D = 128, else BF_EUNSUPPORTED); the
 *   continuous remote angles are evaluated in float64 in the kernels (one rounding to
 *   float32, like table entries).  Arguments, layouts, workspace and errors as for
 *   bifocal_prefill; BF_EINVAL for an unknown variant.
 */
bf_status bifocal_prefill_variant(const void* Q, const void* K, const void* V, void* O, float* lse,
                                  const int32_t* cu_seqlens, int32_t B, int32_t Hq, int32_t Hkv,
                                  int32_t D, int32_t w0, int32_t w_pretrained, double theta,
                                  float softmax_scale, int32_t variant, bf_dtype dt, void* ws,
                                  size_t ws_bytes, bf_stream stream);

/*
 * bifocal_prefill_ie -- the same attention as bifocal_prefill, computed literally as
 * the pages' three passes merged by inclusion-exclusion of their LogSumExp statistics
 * (section 2, inference efficiency): A = local scores over the window pairs
 * (0 <= i - j < w0), B = remote scores over all causal pairs, C = remote scores over the
 * window pairs; then
 *   Z = e^{LSE_B} - e^{LSE_C} + e^{LSE_A},
 *   O = (e^{LSE_B} O_B - e^{LSE_C} O_C + e^{LSE_A} O_A) / Z,   lse = ln Z.
 *   The passes run the bf16 matrix-core kernel in three modes and keep O_x in fp32;
 *   a merge kernel forms O (bf16) and lse.  Meant for measuring the fused selection
 *   against the literal form and for cross-checking it; bifocal_prefill is faster.
 *   Arguments, layouts and errors as for bifocal_prefill; dt must be BF_BF16
 *   (BF_EUNSUPPORTED otherwise).  Where Z_B and Z_C nearly cancel, the merge loses
 *   the corresponding relative precision (not so for rows whose causal keys all lie
 *   in the window: there passes B and C are bitwise equal and O = O_A).
 *   ws, ws_bytes: workspace of at least
 *     bifocal_workspace_bytes(BF_OP_PREFILL_IE, max_b L_b, T, B, Hq, Hkv, D), which adds
 *     3 * (T * Hq * D + Hq * T) floats of intermediates to the prefill workspace.
 */
bf_status bifocal_prefill_ie(const void* Q, const void* K, const void* V, void* O, float* lse,
                             const int32_t* cu_seqlens, int32_t B, int32_t Hq, int32_t Hkv,
                             int32_t D, int32_t w0, int32_t w_pretrained, double theta,
                             float softmax_scale, bf_dtype dt, void* ws, size_t ws_bytes,
                             bf_stream stream);

/*
 * bifocal_decode -- one generation step over a standard-RoPE KV cache.
 *   The query sits at position pos and attends to cache entries 0 .. pos; G is taken
 *   from the current length pos + 1 (so it grows as generation crosses multiples of
 *   w_pretrained, without touching the cache: section 2, on-the-fly correction
 *   rotation applied to the active query and the stored keys).  Scores as in
 *   bifocal_prefill with i = pos.  Keys are rotated in float32 registers; the softmax
 *   runs in float32.
 *   q      (device) [Hq, D] standard RoPE at pos.
 *   Kcache (device) [S, Hkv, D] standard RoPE at absolute positions, S >= pos + 1.
 *   Vcache (device) [S, Hkv, D].
 *   o      (device) [Hq, D] output, dtype dt.   lse (device) [Hq] float32, or NULL.
 *   dt: BF_BF16 or BF_F32 for q, caches and o.  D in {64, 128}; Hq/Hkv in {1, 2, 4, 8}.
 *     bf16 with D = 128 runs on the matrix cores: remote scores use fp16 hi/lo operands
 *     of the rotated fp32 keys and query (error well below bf16 rounding), local scores
 *     the stored bf16 operands, and the correction angles are evaluated in the kernel
 *     (the workspace table is not read).  Other cases run on the vector units in fp32.
 *   ws, ws_bytes: workspace (device) of at least
 *     bifocal_workspace_bytes(BF_OP_DECODE, pos + 1, 0, 1, Hq, Hkv, D).
 *   Errors: BF_EINVAL (null pointer, pos < 0, w0 < 1, ...), BF_EUNSUPPORTED, BF_EWORKSPACE.
 */
bf_status bifocal_decode(const void* q, const void* Kcache, const void* Vcache, void* o,
                         float* lse, int32_t pos, int32_t Hq, int32_t Hkv, int32_t D, int32_t w0,
                         int32_t w_pretrained, double theta, float softmax_scale, bf_dtype dt,
                         void* ws, size_t ws_bytes, bf_stream stream);

/*
 * bifocal_decode_batch -- one generation step for each of B sequences of different
 * lengths (ragged batch decode).
 *   Sequence b's query sits at position pos[b] and attends to entries 0 .. pos[b] of its
 *   own cache; its G_b = max(1, ceil((pos[b] + 1) / w_pretrained)) is taken per sequence
 *   (section 1 with the sequence's current length), so sequences on either side of a
 *   multiple of w_pretrained use different groupings in the same call.  Each sequence
 *   is computed exactly as bifocal_decode would compute it alone.
 *   q      (device) [B, Hq, D] standard RoPE at pos[b].
 *   Kcache (device) [B, S, Hkv, D] standard RoPE at absolute positions (S rows per
 *          sequence; rows past pos[b] are not read).
 *   Vcache (device) [B, S, Hkv, D].
 *   o      (device) [B, Hq, D] output.   lse (device) [B, Hq] float32, or NULL.
 *   pos    (host) [B], 0 <= pos[b] < S.
 *   dt, D, Hq/Hkv as for bifocal_decode.  B = 0 is a no-op.
 *   ws, ws_bytes: workspace (device) of at least
 *     bifocal_workspace_bytes(BF_OP_DECODE, max_b pos[b] + 1, 0, B, Hq, Hkv, D).
 *   Errors: BF_EINVAL (null pointer, B < 0, S < 1, pos[b] outside [0, S), ...),
 *           BF_EUNSUPPORTED, BF_EWORKSPACE.
 */
bf_status bifocal_decode_batch(const void* q, const void* Kcache, const void* Vcache, void* o,
                               float* lse, const int32_t* pos, int32_t B, int32_t S, int32_t Hq,
                               int32_t Hkv, int32_t D, int32_t w0, int32_t w_pretrained,
                               double theta, float softmax_scale, bf_dtype dt, void* ws,
                               size_t ws_bytes, bf_stream stream);

/*
 * bifocal_decode_variant -- bifocal_decode_batch for an attention variant (bf_variant).
 *   BF_VARIANT_BIFOCAL is bifocal_decode_batch.  The other variants need dt = BF_BF16 and
 *   D = 128 (BF_EUNSUPPORTED otherwise); BF_VARIANT_WINDOW reads only the last w0 cache
 *   rows of each sequence.  Arguments, layouts, workspace and errors as for
 *   bifocal_decode_batch; BF_EINVAL for an unknown variant.
 */
bf_status bifocal_decode_variant(const void* q, const void* Kcache, const void* Vcache, void* o,
                                 float* lse, const int32_t* pos, int32_t B, int32_t S, int32_t Hq,
                                 int32_t Hkv, int32_t D, int32_t w0, int32_t w_pretrained,
                                 double theta, float softmax_scale, int32_t variant, bf_dtype dt,
                                 void* ws, size_t ws_bytes, bf_stream stream);

/*
 * bifocal_decode_noalloc -- bifocal_decode for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * no workspace argument, nothing allocated, freed or synchronised.
 *   The split partials live in a device array of BIFOCAL_NOALLOC_SCRATCH_BYTES that the
 *   library holds on each GPU it runs on until the process ends (its address is looked up
 *   on the first call on a device).  Every call on a GPU shares that array: calls that
 *   overlap on one GPU race; calls ordered on one stream are safe.
 *   Arguments, layouts and results as for bifocal_decode, on the matrix-core path only:
 *   dt = BF_BF16 and D = 128 (BF_EUNSUPPORTED otherwise).  When the array holds fewer
 *   partials than the usual split count wants (Hq above about 64), the step uses fewer
 *   splits; BF_EWORKSPACE if even one partial per query head does not fit.  stream must
 *   belong to the current device (BF_EINVAL otherwise); BF_EHIP if the array's address
 *   cannot be found.
 */
#define BIFOCAL_NOALLOC_SCRATCH_BYTES (4u << 20)
bf_status bifocal_decode_noalloc(const void* q, const void* Kcache, const void* Vcache, void* o,
                                 float* lse, int32_t pos, int32_t Hq, int32_t Hkv, int32_t D,
                                 int32_t w0, int32_t w_pretrained, double theta,
                                 float softmax_scale, bf_dtype dt, bf_stream stream);

/*
 * bifocal_workspace_bytes -- workspace size for an operation.
 *   max_len: the longest sequence a prefill will see, or the largest pos + 1 for decode.
 *   total_tokens, num_seqs: prefill (both ops): the largest T and B of the calls that will use the
 *     workspace (max_len <= total_tokens <= num_seqs * max_len).  Decode: num_seqs is the
 *     largest batch B (0 counts as 1), total_tokens is ignored.
 *   Returns 0 for invalid arguments.
 */
size_t bifocal_workspace_bytes(int32_t op, int32_t max_len, int64_t total_tokens,
                               int32_t num_seqs, int32_t Hq, int32_t Hkv, int32_t D);

/* bifocal_status_string -- static text for a status code (never NULL). */
const char* bifocal_status_string(int32_t status);

/*
 * bifocal_group_size -- G = max(1, ceil(L / w_pretrained)) as the kernels use it
 * (section 1); returns 0 if L < 0 or w_pretrained < 1.
 */
int32_t bifocal_group_size(int64_t L, int32_t w_pretrained);

#ifdef __cplusplus
}
#endif

#endif /* BIFOCAL_H_ */
