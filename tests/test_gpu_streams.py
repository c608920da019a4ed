"""The calls on a non-default stream and under HIP-graph capture: the library only
enqueues kernels on the caller's stream (no allocation, copy, memset or
synchronisation), so a captured call replays to the eager result bit for bit.  Each
graph is replayed several times with other eager work and synchronisations in between,
and every replay is checked."""
import sys

import numpy as np
import pytest
import torch

import workloads as W
from helpers import decode_inputs, prefill_inputs, std_query

pytestmark = pytest.mark.gpu

TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def bf():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import dynamic_rope_context_amd as m
    m.lib()  # raises if the library is missing
    return m


def dev(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(TDT[dt]).cuda()


def _prefill_setup(bf, dt, D):
    w = W.Workload("graphp", "prefill", dt, Hq=8, Hkv=2, D=D, w0=40, w_pretrained=128,
                   theta=1e4, seqlens=(700, 90), outliers=4, seed=401)
    Q, K, V, cu = prefill_inputs(w)
    Qd, Kd, Vd = dev(Q, dt), dev(K, dt), dev(V, dt)
    c = [int(x) for x in cu]
    T = c[-1]
    out = torch.empty_like(Qd)
    lse = torch.empty((w.Hq, T), dtype=torch.float32, device="cuda")
    ws = bf.Workspace.for_op(bf.OP_PREFILL, max(w.seqlens), w.Hq, w.Hkv, D, total_tokens=T,
                             num_seqs=len(w.seqlens))
    call = lambda: bf.bifocal_prefill(Qd, Kd, Vd, c, w.w0, w.w_pretrained, w.theta, out=out,
                                      lse=lse, workspace=ws)
    return call, out, lse


def _decode_setup(bf, dt, D):
    w = W.Workload("graphd", "decode", dt, Hq=8, Hkv=2, D=D, w0=40, w_pretrained=128,
                   theta=1e4, cache_len=1500, decode_steps=1, outliers=4, seed=402)
    q_raw, Kc, Vc = decode_inputs(w)
    pos = 1499
    qd = dev(std_query(q_raw[0], pos, w.theta, dt), dt)
    Kd, Vd = dev(Kc, dt), dev(Vc, dt)
    out = torch.empty_like(qd)
    lse = torch.empty((w.Hq,), dtype=torch.float32, device="cuda")
    ws = bf.Workspace.for_op(bf.OP_DECODE, 1500, w.Hq, w.Hkv, D)
    call = lambda: bf.bifocal_decode(qd, Kd, Vd, pos, w.w0, w.w_pretrained, w.theta, out=out,
                                     lse=lse, workspace=ws)
    return call, out, lse


SETUPS = {"prefill": _prefill_setup, "decode": _decode_setup}
CASES = [("prefill", "bf16", 128), ("prefill", "f32", 64), ("decode", "bf16", 128),
         ("decode", "f32", 64)]


@pytest.mark.parametrize("what,dt,D", CASES)
def test_non_default_stream(bf, what, dt, D):
    say("stream", what, dt, D)
    call, out, lse = SETUPS[what](bf, dt, D)
    call()
    torch.cuda.synchronize()
    o_ref, l_ref = out.clone(), lse.clone()
    out.zero_()
    lse.zero_()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call()
    s.synchronize()
    assert torch.equal(out, o_ref) and torch.equal(lse, l_ref)


@pytest.mark.parametrize("what,dt,D", CASES)
def test_graph_replays_match_eager(bf, what, dt, D):
    say("graph", what, dt, D)
    call, out, lse = SETUPS[what](bf, dt, D)
    call()  # eager: also sets the kernels' launch attributes before any capture
    torch.cuda.synchronize()
    o_ref, l_ref = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device="cuda")
    for r in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        scratch.mul_(1.0001)  # other eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref), (what, r)
        assert torch.equal(lse, l_ref), (what, r)
        call()  # an eager call between replays
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref), (what, "eager", r)


def test_prefill_without_workspace_costs_no_more_than_with_one(bf):
    # A call given no workspace allocates one (on the launch stream) and builds the
    # position table in it: the table check runs on its full grid, so a fresh workspace
    # costs one table build (tens of microseconds), not a serial rebuild.  At the 32K
    # G = 1 layer shape each such call takes at most 1.1x a call on a ready workspace.
    w = W.get("qwen3_1p7b_32k_g1")
    q, k, v = W.raw_inputs_torch(w, "cuda")
    bf.rope_apply(q, w.theta)
    bf.rope_apply(k, w.theta)
    cu = [0, w.total_tokens]
    out = torch.empty_like(q)
    ws = bf.Workspace.for_op(bf.OP_PREFILL, w.total_tokens, w.Hq, w.Hkv, w.D)
    args = (q, k, v, cu, w.w0, w.w_pretrained, w.theta)

    def timed(**kw):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        bf.bifocal_prefill(*args, out=out, want_lse=False, **kw)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)
    for _ in range(2):  # warm-up, including the allocator's first blocks of this size
        timed(workspace=ws)
        timed()
    ref = min(timed(workspace=ws) for _ in range(3))
    fresh = [timed() for _ in range(2)]
    say(f"  with a workspace {ref:.3f} ms; without: {fresh}")
    assert max(fresh) <= 1.1 * ref, (ref, fresh)
