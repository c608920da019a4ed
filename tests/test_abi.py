"""The C-ABI library on the CPU: it loads, exports every declared symbol, and rejects
bad arguments before touching the GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bifocal.h")
LIB = os.path.join(ROOT, "dynamic_rope_context_amd", "libbifocal.so")

BF_OK, BF_EINVAL, BF_EUNSUPPORTED, BF_EWORKSPACE = 0, 1, 2, 3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"^\s*#.*$", "", text, flags=re.M)
    return sorted(set(re.findall(r"\b(\w+)\s*\(", text)) - {"defined", "if", "sizeof"})


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libbifocal.so is not built (run __graft_entry__.build())")
    import dynamic_rope_context_amd as b
    return b.lib()


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("bifocal_prefill", "bifocal_decode", "rope_apply", "bifocal_workspace_bytes",
              "bifocal_status_string", "bifocal_group_size", "bifocal_prefill_ie",
              "bifocal_decode_batch", "bifocal_prefill_variant", "bifocal_decode_variant",
              "bifocal_decode_noalloc"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} declared in bifocal.h but not exported"


def test_status_strings(lib):
    for s in range(5):
        assert lib.bifocal_status_string(s)
    assert lib.bifocal_status_string(99) == b"unknown status"


def test_group_size_export(lib):
    assert lib.bifocal_group_size(131072, 32768) == 4
    assert lib.bifocal_group_size(131073, 32768) == 5
    assert lib.bifocal_group_size(1, 32768) == 1
    assert lib.bifocal_group_size(0, 32768) == 1
    assert lib.bifocal_group_size(98427, 32768) == 4
    assert lib.bifocal_group_size(40001, 32768) == 2
    assert lib.bifocal_group_size(-1, 32768) == 0
    assert lib.bifocal_group_size(5, 0) == 0


def test_workspace_bytes(lib):
    n = lib.bifocal_workspace_bytes(1, 131072, 131072, 1, 32, 8, 128)
    assert n >= 131072 * 64 * 8          # the position table alone
    assert lib.bifocal_workspace_bytes(2, 131072, 0, 0, 32, 8, 128) > 0
    assert lib.bifocal_workspace_bytes(1, 10, 10, 1, 3, 2, 128) == 0   # Hq % Hkv != 0
    assert lib.bifocal_workspace_bytes(1, 10, 10, 1, 4, 2, 96) == 0    # unsupported D
    assert lib.bifocal_workspace_bytes(7, 10, 10, 1, 4, 2, 128) == 0
    assert lib.bifocal_workspace_bytes(1, 10, 30, 2, 4, 2, 128) == 0   # T > B * max_len
    assert lib.bifocal_workspace_bytes(1, 10, 5, 1, 4, 2, 128) == 0    # T < max_len


def _prefill(lib, **kw):
    args = dict(Q=16, K=16, V=16, O=16, lse=0, cu=None, B=1, Hq=4, Hkv=1, D=128, w0=4,
                w_pre=16, theta=1e4, scale=0.0, dt=1, ws=256, ws_bytes=1 << 30)
    args.update(kw)
    cu = args["cu"] if args["cu"] is not None else [0, 64]
    cu_ptr = None
    if cu != 0:
        arr = (ctypes.c_int32 * len(cu))(*cu)
        cu_ptr = ctypes.cast(arr, ctypes.c_void_p)
    return lib.bifocal_prefill(args["Q"], args["K"], args["V"], args["O"], args["lse"],
                               cu_ptr, args["B"], args["Hq"], args["Hkv"], args["D"],
                               args["w0"], args["w_pre"], args["theta"], args["scale"],
                               args["dt"], args["ws"], args["ws_bytes"], None)


def test_prefill_rejects_bad_arguments_before_launch(lib):
    # every case returns before any HIP call (the pointers are fake)
    assert _prefill(lib, w0=0) == BF_EINVAL
    assert _prefill(lib, w_pre=0) == BF_EINVAL
    assert _prefill(lib, theta=-1.0) == BF_EINVAL
    assert _prefill(lib, Hq=3, Hkv=2) == BF_EINVAL
    assert _prefill(lib, cu=[1, 64]) == BF_EINVAL
    assert _prefill(lib, cu=[0, 64, 32], B=2) == BF_EINVAL
    assert _prefill(lib, cu=0) == BF_EINVAL
    assert _prefill(lib, D=96) == BF_EUNSUPPORTED
    assert _prefill(lib, D=64) == BF_EUNSUPPORTED           # bf16 path needs D = 128
    assert _prefill(lib, Hq=12, Hkv=4) == BF_EUNSUPPORTED   # bf16 path: ratio 3
    assert _prefill(lib, Q=0) == BF_EINVAL
    assert _prefill(lib, Q=8) == BF_EINVAL                  # misaligned
    assert _prefill(lib, ws=0) == BF_EWORKSPACE
    assert _prefill(lib, ws=128) == BF_EWORKSPACE           # misaligned workspace
    assert _prefill(lib, ws_bytes=4096) == BF_EWORKSPACE
    assert _prefill(lib, dt=7) == BF_EINVAL
    assert _prefill(lib, cu=[0, 0], Q=0) == BF_OK           # empty batch: nothing to do


def test_prefill_ie_rejects_bad_arguments_before_launch(lib):
    def call(**kw):
        a = dict(Q=16, K=16, V=16, O=16, lse=0, B=1, Hq=4, Hkv=1, D=128, w0=4, w_pre=16,
                 theta=1e4, scale=0.0, dt=1, ws=256, ws_bytes=1 << 30, cu=[0, 64])
        a.update(kw)
        arr = (ctypes.c_int32 * len(a["cu"]))(*a["cu"])
        return lib.bifocal_prefill_ie(a["Q"], a["K"], a["V"], a["O"], a["lse"],
                                      ctypes.cast(arr, ctypes.c_void_p), a["B"], a["Hq"],
                                      a["Hkv"], a["D"], a["w0"], a["w_pre"], a["theta"],
                                      a["scale"], a["dt"], a["ws"], a["ws_bytes"], None)
    assert call(dt=0) == BF_EUNSUPPORTED      # the three-pass form is bf16 only
    assert call(w0=0) == BF_EINVAL
    assert call(Hq=12, Hkv=4) == BF_EUNSUPPORTED
    assert call(ws=0) == BF_EWORKSPACE
    assert call(ws_bytes=1 << 16) == BF_EWORKSPACE
    assert call(cu=[0, 0], Q=0) == BF_OK


def test_prefill_ie_workspace_adds_intermediates(lib):
    one = lib.bifocal_workspace_bytes(1, 4096, 8192, 2, 32, 8, 128)
    ie = lib.bifocal_workspace_bytes(3, 4096, 8192, 2, 32, 8, 128)
    assert ie >= one + 3 * (8192 * 32 * 128 * 4 + 32 * 8192 * 4)
    assert lib.bifocal_workspace_bytes(3, 4096, 100, 2, 32, 8, 128) == 0   # T < max_len


def _decode(lib, **kw):
    a = dict(q=16, K=16, V=16, o=16, lse=0, pos=100, Hq=4, Hkv=1, D=128, w0=4, w_pre=16,
             theta=1e4, scale=0.0, dt=1, ws=256, ws_bytes=1 << 30)
    a.update(kw)
    return lib.bifocal_decode(a["q"], a["K"], a["V"], a["o"], a["lse"], a["pos"], a["Hq"],
                              a["Hkv"], a["D"], a["w0"], a["w_pre"], a["theta"], a["scale"],
                              a["dt"], a["ws"], a["ws_bytes"], None)


def test_decode_rejects_bad_arguments_before_launch(lib):
    assert _decode(lib, pos=-1) == BF_EINVAL
    assert _decode(lib, q=0) == BF_EINVAL
    assert _decode(lib, w0=0) == BF_EINVAL
    assert _decode(lib, Hq=6, Hkv=4) == BF_EINVAL
    assert _decode(lib, Hq=12, Hkv=4) == BF_EUNSUPPORTED
    assert _decode(lib, D=80) == BF_EUNSUPPORTED
    assert _decode(lib, K=24) == BF_EINVAL
    assert _decode(lib, ws=0) == BF_EWORKSPACE
    assert _decode(lib, ws_bytes=1 << 12) == BF_EWORKSPACE


def _decode_noalloc(lib, **kw):
    a = dict(q=16, K=16, V=16, o=16, lse=0, pos=100, Hq=4, Hkv=1, D=128, w0=4, w_pre=16,
             theta=1e4, scale=0.0, dt=1)
    a.update(kw)
    return lib.bifocal_decode_noalloc(a["q"], a["K"], a["V"], a["o"], a["lse"], a["pos"],
                                      a["Hq"], a["Hkv"], a["D"], a["w0"], a["w_pre"], a["theta"],
                                      a["scale"], a["dt"], None)


def test_decode_noalloc_rejects_bad_arguments_before_any_hip_call(lib):
    # the checks run before the device lookup, so they work without a GPU
    assert _decode_noalloc(lib, pos=-1) == BF_EINVAL
    assert _decode_noalloc(lib, q=0) == BF_EINVAL
    assert _decode_noalloc(lib, w0=0) == BF_EINVAL
    assert _decode_noalloc(lib, Hq=6, Hkv=4) == BF_EINVAL
    assert _decode_noalloc(lib, Hq=12, Hkv=4) == BF_EUNSUPPORTED
    assert _decode_noalloc(lib, D=64) == BF_EUNSUPPORTED       # matrix-core path only
    assert _decode_noalloc(lib, dt=0) == BF_EUNSUPPORTED       # bf16 only
    assert _decode_noalloc(lib, K=24) == BF_EINVAL
    # one partial per query head must fit the fixed array
    assert _decode_noalloc(lib, Hq=8192, Hkv=1024) == BF_EWORKSPACE


def _decode_batch(lib, **kw):
    a = dict(q=16, K=16, V=16, o=16, lse=0, pos=[100, 7, 300], B=None, S=512, Hq=4, Hkv=1,
             D=128, w0=4, w_pre=16, theta=1e4, scale=0.0, dt=1, ws=256, ws_bytes=1 << 30)
    a.update(kw)
    pos = a["pos"]
    B = len(pos) if a["B"] is None else a["B"]
    ptr = None
    if pos is not None:
        arr = (ctypes.c_int32 * max(len(pos), 1))(*pos)
        ptr = ctypes.cast(arr, ctypes.c_void_p)
    return lib.bifocal_decode_batch(a["q"], a["K"], a["V"], a["o"], a["lse"], ptr, B, a["S"],
                                    a["Hq"], a["Hkv"], a["D"], a["w0"], a["w_pre"], a["theta"],
                                    a["scale"], a["dt"], a["ws"], a["ws_bytes"], None)


def test_decode_batch_rejects_bad_arguments_before_launch(lib):
    assert _decode_batch(lib, pos=[100, -1]) == BF_EINVAL
    assert _decode_batch(lib, pos=[100, 512]) == BF_EINVAL      # pos >= S
    assert _decode_batch(lib, pos=None, B=2) == BF_EINVAL
    assert _decode_batch(lib, B=-1) == BF_EINVAL
    assert _decode_batch(lib, S=0) == BF_EINVAL
    assert _decode_batch(lib, q=0) == BF_EINVAL
    assert _decode_batch(lib, w0=0) == BF_EINVAL
    assert _decode_batch(lib, Hq=12, Hkv=4) == BF_EUNSUPPORTED
    assert _decode_batch(lib, D=96) == BF_EUNSUPPORTED
    assert _decode_batch(lib, V=24) == BF_EINVAL                # misaligned
    assert _decode_batch(lib, ws=0) == BF_EWORKSPACE
    assert _decode_batch(lib, ws_bytes=1 << 12) == BF_EWORKSPACE
    assert _decode_batch(lib, pos=[], q=0, K=0, V=0, o=0) == BF_OK   # empty batch


def test_decode_workspace_grows_with_batch(lib):
    one = lib.bifocal_workspace_bytes(2, 4096, 0, 1, 32, 8, 128)
    assert lib.bifocal_workspace_bytes(2, 4096, 0, 0, 32, 8, 128) == one
    many = lib.bifocal_workspace_bytes(2, 4096, 0, 16, 32, 8, 128)
    assert many >= 16 * 32 * 128 * 130 * 4 > one
    assert lib.bifocal_workspace_bytes(2, 4096, 0, -1, 32, 8, 128) == 0


def test_variants_reject_bad_arguments_before_launch(lib):
    def pre(variant, dt=1, D=128):
        arr = (ctypes.c_int32 * 2)(0, 64)
        return lib.bifocal_prefill_variant(16, 16, 16, 16, 0, ctypes.cast(arr, ctypes.c_void_p),
                                           1, 4, 1, D, 4, 16, 1e4, 0.0, variant, dt, 256, 1 << 30,
                                           None)

    def dec(variant, dt=1, D=128):
        arr = (ctypes.c_int32 * 2)(100, 7)
        return lib.bifocal_decode_variant(16, 16, 16, 16, 0, ctypes.cast(arr, ctypes.c_void_p), 2,
                                          512, 4, 1, D, 4, 16, 1e4, 0.0, variant, dt, 256,
                                          1 << 12, None)
    assert pre(3) == BF_EINVAL and pre(-1) == BF_EINVAL
    assert pre(1, dt=0) == BF_EUNSUPPORTED and pre(2, dt=0) == BF_EUNSUPPORTED
    assert dec(7) == BF_EINVAL
    assert dec(1, dt=0) == BF_EUNSUPPORTED and dec(2, D=64) == BF_EUNSUPPORTED
    assert dec(1) == BF_EWORKSPACE   # valid variant, workspace too small


def test_positions_beyond_the_alias_range_are_rejected(lib):
    # floor(x / G) is evaluated by multiply-shift, exact below 2^24 positions
    assert _prefill(lib, cu=[0, 1 << 24]) == BF_EUNSUPPORTED
    assert _decode(lib, pos=(1 << 24) - 1) == BF_EUNSUPPORTED
    assert _decode_batch(lib, pos=[5, (1 << 24) - 1], S=1 << 24) == BF_EUNSUPPORTED


def test_rope_apply_rejects_bad_arguments(lib):
    f = lib.rope_apply
    assert f(16, None, 0, 10, 2, 7, 1e4, 1, 1, None) == BF_EINVAL     # odd D
    assert f(16, None, 0, 10, 2, 8, 1e4, 0, 1, None) == BF_EINVAL     # G < 1
    assert f(16, None, 0, 10, 2, 8, 0.0, 1, 1, None) == BF_EINVAL     # theta
    assert f(None, None, 0, 10, 2, 8, 1e4, 1, 1, None) == BF_EINVAL   # null x
    assert f(16, None, -1, 10, 2, 8, 1e4, 1, 1, None) == BF_EINVAL    # pos0 < 0
    assert f(16, None, 0, 10, 2, 512, 1e4, 1, 1, None) == BF_EUNSUPPORTED
    assert f(16, None, 0, 0, 2, 8, 1e4, 1, 1, None) == BF_OK          # empty


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import dynamic_rope_context_amd as b
    monkeypatch.setattr(b, "lib_path", str(tmp_path / "missing.so"))
    monkeypatch.setattr(b, "_lib_handle", None)
    with pytest.raises(ImportError):
        b.lib()


def test_binding_checks_caller_buffers_before_any_call():
    # wrong output shapes or dtypes are rejected before a pointer reaches the library
    import torch
    import dynamic_rope_context_amd as b
    Q = torch.zeros(8, 4, 128, dtype=torch.bfloat16)
    K = torch.zeros(8, 1, 128, dtype=torch.bfloat16)
    with pytest.raises(b.BifocalError):
        b.bifocal_prefill(Q, K, K, [0, 8], 4, 16, 1e4, out=torch.zeros(8, 4, 64, dtype=torch.bfloat16))
    with pytest.raises(b.BifocalError):
        b.bifocal_prefill(Q, K, K, [0, 8], 4, 16, 1e4, lse=torch.zeros(8, 4))
    with pytest.raises(b.BifocalError):
        b.bifocal_prefill(Q, K.float(), K, [0, 8], 4, 16, 1e4)
    q = torch.zeros(4, 128, dtype=torch.bfloat16)
    with pytest.raises(b.BifocalError):
        b.bifocal_decode(q, K, K, 5, 4, 16, 1e4, out=torch.zeros(4, 128))
    with pytest.raises(b.BifocalError):
        b.bifocal_decode_batch(q[None], K[None], K[None], [5], 4, 16, 1e4,
                               lse=torch.zeros(2, 4))
    with pytest.raises(b.BifocalError):
        b.bifocal_decode_variant(q[None], K[None], K[None], [5], 4, 16, 1e4, variant="yarn")
