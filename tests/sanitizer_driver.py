"""Calls every entry point of a host-only build of the C-ABI layer (kernel launches
replaced by the stand-ins of tests/sanitizer_stubs.cpp) with valid and invalid arguments.
Every buffer is host memory of exactly the size the call needs (the workspaces exactly
what bifocal_workspace_bytes returns), so the sanitizers see any access past them.
Run by tests/test_host_sanitizers.py in a process with the AddressSanitizer runtime
preloaded; prints "ok" and exits 0 when every status is the expected one."""
import ctypes
import sys

OK, EINVAL, EUNSUP, EWS, EHIP = 0, 1, 2, 3, 4
vp, i32, i64, sz, f32, f64 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                              ctypes.c_float, ctypes.c_double)

lib = ctypes.CDLL(sys.argv[1])
libc = ctypes.CDLL(None)
lib.rope_apply.argtypes = [vp, vp, i32, i32, i32, i32, f64, i32, i32, vp]
lib.bifocal_prefill.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f64, f32,
                                i32, vp, sz, vp]
lib.bifocal_prefill_ie.argtypes = lib.bifocal_prefill.argtypes
lib.bifocal_prefill_variant.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                        f64, f32, i32, i32, vp, sz, vp]
lib.bifocal_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f64, f32, i32,
                               vp, sz, vp]
lib.bifocal_decode_batch.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                     f64, f32, i32, vp, sz, vp]
lib.bifocal_decode_variant.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                       f64, f32, i32, i32, vp, sz, vp]
lib.bifocal_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f64,
                                       f32, i32, vp]
lib.bifocal_workspace_bytes.argtypes = [i32, i32, i64, i32, i32, i32, i32]
lib.bifocal_workspace_bytes.restype = sz
for f in ("rope_apply", "bifocal_prefill", "bifocal_prefill_ie", "bifocal_prefill_variant",
          "bifocal_decode", "bifocal_decode_batch", "bifocal_decode_variant",
          "bifocal_decode_noalloc"):
    getattr(lib, f).restype = i32
libc.posix_memalign.argtypes = [ctypes.POINTER(vp), sz, sz]
libc.free.argtypes = [vp]

bufs = []


def buf(n):
    """n bytes, 256-byte aligned, exactly n long for the sanitizer."""
    p = vp()
    assert libc.posix_memalign(ctypes.byref(p), 256, max(int(n), 1)) == 0
    ctypes.memset(p, 0, max(int(n), 1))
    bufs.append(p)
    return p.value


def expect(got, want, what):
    if got != want:
        print(f"FAIL {what}: status {got}, expected {want}")
        sys.exit(1)


def ints(vals):
    return ctypes.cast((ctypes.c_int32 * len(vals))(*vals), vp)


# rope_apply
for dt, esz, D in ((1, 2, 128), (0, 4, 64), (1, 2, 100)):
    T, H = 37, 3
    x = buf(T * H * D * esz)
    expect(lib.rope_apply(x, None, 5, T, H, D, 1e6, 3, dt, None), OK, "rope_apply")
    expect(lib.rope_apply(x, buf(T * 4), 0, T, H, D, 1e6, 1, dt, None), OK, "rope_apply pos")
expect(lib.rope_apply(None, None, 0, 3, 1, 8, 1e4, 1, 1, None), EINVAL, "rope_apply null")

# prefill: ragged, bf16 (matrix-core) and fp32, with exact workspaces
for dt, esz, D, Hq, Hkv in ((1, 2, 128, 8, 2), (1, 2, 128, 8, 8), (0, 4, 64, 6, 2),
                            (0, 4, 128, 4, 4)):
    for lens in ((100, 1, 700), (0, 257, 0, 31), tuple((37 * i) % 150 + 1 for i in range(53))):
        cu = [0]
        for L in lens:
            cu.append(cu[-1] + L)
        T, B, mx = cu[-1], len(lens), max(lens)
        Q, K, V, O = (buf(T * Hq * D * esz), buf(T * Hkv * D * esz), buf(T * Hkv * D * esz),
                      buf(T * Hq * D * esz))
        lse = buf(T * Hq * 4)
        for op, fn in ((1, lib.bifocal_prefill), (3, lib.bifocal_prefill_ie)):
            if op == 3 and dt != 1:
                continue
            n = lib.bifocal_workspace_bytes(op, mx, T, B, Hq, Hkv, D)
            ws = buf(n)
            expect(fn(Q, K, V, O, lse, ints(cu), B, Hq, Hkv, D, 20, 64, 1e6, 0.0, dt, ws, n, None),
                   OK, f"prefill op {op} dt {dt} lens {lens[:4]}")
            expect(fn(Q, K, V, O, lse, ints(cu), B, Hq, Hkv, D, 20, 64, 1e6, 0.0, dt, ws, 4096,
                      None), EWS, "prefill workspace short")
        if dt == 1:
            n = lib.bifocal_workspace_bytes(1, mx, T, B, Hq, Hkv, D)
            for variant in (1, 2):
                expect(lib.bifocal_prefill_variant(Q, K, V, O, None, ints(cu), B, Hq, Hkv, D, 20,
                                                   64, 1e6, 0.0, variant, dt, buf(n), n, None),
                       OK, f"prefill variant {variant}")

# decode: matrix-core (bf16, D = 128) and vector paths, single and batched, exact workspaces
for dt, esz, D, Hq, Hkv in ((1, 2, 128, 32, 8), (1, 2, 64, 8, 2), (0, 4, 128, 4, 4)):
    S = 3001
    q, Kc, Vc, o = (buf(Hq * D * esz), buf(S * Hkv * D * esz), buf(S * Hkv * D * esz),
                    buf(Hq * D * esz))
    for pos in (0, 999, 3000):
        n = lib.bifocal_workspace_bytes(2, pos + 1, 0, 1, Hq, Hkv, D)
        expect(lib.bifocal_decode(q, Kc, Vc, o, buf(Hq * 4), pos, Hq, Hkv, D, 100, 1000, 1e6, 0.0,
                                  dt, buf(n), n, None), OK, f"decode dt {dt} D {D} pos {pos}")
    B, S = 70, 97
    pos = [(13 * b) % S for b in range(B)]
    qb, Kb, Vb, ob = (buf(B * Hq * D * esz), buf(B * S * Hkv * D * esz), buf(B * S * Hkv * D * esz),
                      buf(B * Hq * D * esz))
    n = lib.bifocal_workspace_bytes(2, max(pos) + 1, 0, B, Hq, Hkv, D)
    expect(lib.bifocal_decode_batch(qb, Kb, Vb, ob, buf(B * Hq * 4), ints(pos), B, S, Hq, Hkv, D,
                                    16, 40, 1e4, 0.0, dt, buf(n), n, None), OK, "decode batch")
    if dt == 1 and D == 128:
        for variant in (1, 2):
            expect(lib.bifocal_decode_variant(qb, Kb, Vb, ob, None, ints(pos), B, S, Hq, Hkv, D, 16,
                                              40, 1e4, 0.0, variant, dt, buf(n), n, None),
                   OK, f"decode variant {variant}")
    expect(lib.bifocal_decode(q, Kc, Vc, o, None, 5000, Hq, Hkv, D, 100, 1000, 1e6, 0.0, dt,
                              buf(64), 64, None), EWS, "decode workspace short")

# no-allocation decode: argument errors before any HIP call
q, Kc, Vc, o = buf(32 * 128 * 2), buf(100 * 8 * 128 * 2), buf(100 * 8 * 128 * 2), buf(32 * 256)
expect(lib.bifocal_decode_noalloc(q, Kc, Vc, o, None, -1, 32, 8, 128, 16, 40, 1e4, 0.0, 1, None),
       EINVAL, "noalloc pos")
expect(lib.bifocal_decode_noalloc(q, Kc, Vc, o, None, 50, 32, 8, 64, 16, 40, 1e4, 0.0, 1, None),
       EUNSUP, "noalloc D")

for p in bufs:
    libc.free(p)
print("ok")
