"""GPU parity: the HIP path through the C ABI against the CPU oracle, element by
element, on seeded inputs at sizes the oracle finishes in seconds (several tiles,
ragged tails, every supported GQA ratio, window/group edge cases)."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle.bifocal_ref import (bifocal_decode_ref, bifocal_prefill_ref, group_size,
                                rope_apply_ref, rope_rotate)
from helpers import (BF16_TOL, F32_TOL, decode_inputs, errors, ie_conditioning,
                     prefill_inputs, std_query, to_dtype, within)

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


def host(t):
    return t.float().cpu().numpy()


def run_prefill(bf, w, Q, K, V, cu):
    O, lse = bf.bifocal_prefill(dev(Q, w.dtype), dev(K, w.dtype), dev(V, w.dtype),
                                [int(c) for c in cu], w.w0, w.w_pretrained, w.theta)
    torch.cuda.synchronize()
    return host(O), lse.cpu().numpy()


def check_prefill(bf, w, Q, K, V, cu, tol, rows_per_seq=None):
    Og, Lg = run_prefill(bf, w, Q, K, V, cu)
    ref = bifocal_prefill_ref(Q, K, V, cu, w.w0, w.w_pretrained, w.theta,
                              rows_per_seq=rows_per_seq)
    worst = {}
    for b, (rows, O, LSE) in enumerate(ref):
        if O is None:
            continue
        s = int(cu[b])
        e = errors(Og[s + rows], O, Lg[:, s + rows].T, LSE)
        say(f"  seq {b}: L={int(cu[b+1]-cu[b])} G={group_size(int(cu[b+1]-cu[b]), w.w_pretrained)}"
            f" {e}")
        for k, v in e.items():
            worst[k] = max(worst.get(k, 0.0), v)
        assert within(e, tol), (b, e, tol)
        assert np.all(np.isfinite(Og[s + rows]))
    return worst


# ---------------------------------------------------------------------------
# rope_apply
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dt,G,use_pos,D", [("bf16", 1, False, 128), ("bf16", 3, True, 128),
                                            ("f32", 1, True, 128), ("f32", 4, False, 128),
                                            ("bf16", 2, True, 64), ("bf16", 1, False, 100),
                                            ("f32", 5, True, 36)])
def test_rope_apply_matches_oracle(bf, dt, G, use_pos, D):
    # D = 64, 128: 8-pair chunks with 16-byte accesses; D = 100, 36: one pair per thread
    say(f"rope_apply dt={dt} G={G} pos_array={use_pos} D={D}")
    rng = np.random.default_rng(7)
    T, H, theta = 300, 3, 1e6
    x = to_dtype(rng.standard_normal((T, H, D)).astype(np.float32), dt)
    pos = rng.integers(0, 131072, size=T).astype(np.int32) if use_pos else None
    p = pos if use_pos else np.arange(T) + 1000
    xd = dev(x, dt)
    bf.rope_apply(xd, theta, pos=torch.from_numpy(pos).cuda() if use_pos else None,
                  pos0=0 if use_pos else 1000, G=G)
    torch.cuda.synchronize()
    got = host(xd).astype(np.float64)
    exact = rope_apply_ref(x, p, theta, G)
    if dt == "bf16":
        # one bf16 rounding of a float32 rotation: within a bf16 ulp of the exact value,
        # plus the float32 error of x1 c - x2 s, which is relative to the inputs and not
        # to the result (it shows where the two products nearly cancel)
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(exact), 1e-30))) - 7)
        x64 = x.astype(np.float64)
        mag = np.abs(x64[..., :D // 2]) + np.abs(x64[..., D // 2:])
        mag = np.concatenate([mag, mag], axis=-1)
        assert np.all(np.abs(got - exact) <= ulp + 4 * 2.0 ** -24 * mag)
    else:
        mag = np.abs(x[..., :D // 2]).max() + np.abs(x[..., D // 2:]).max()
        assert np.max(np.abs(got - exact)) <= 4e-7 * mag


@pytest.mark.parametrize("dt,T,H,D", [("bf16", 61, 40, 128), ("f32", 61, 40, 128),
                                      ("bf16", 17, 64, 64), ("f32", 9, 33, 128),
                                      ("bf16", 1, 262145, 128)])
def test_rope_apply_many_heads(bf, dt, T, H, D):
    # several rounds of loads per workgroup (8 tokens x H x D/16 chunks beyond 8 (bf16)
    # or 4 (fp32) per thread), ragged token blocks, and H * D past 2^25, which takes the
    # one-pair-per-thread kernel
    say(f"rope_apply many heads dt={dt} T={T} H={H} D={D}")
    rng = np.random.default_rng(11)
    theta, G = 1e6, 3
    x = to_dtype(rng.standard_normal((T, H, D)).astype(np.float32), dt)
    pos = rng.integers(0, 131072, size=T).astype(np.int32)
    xd = dev(x, dt)
    bf.rope_apply(xd, theta, pos=torch.from_numpy(pos).cuda(), G=G)
    torch.cuda.synchronize()
    got = host(xd).astype(np.float64)
    exact = rope_apply_ref(x, pos, theta, G)
    x64 = x.astype(np.float64)
    mag = np.abs(x64[..., :D // 2]) + np.abs(x64[..., D // 2:])
    mag = np.concatenate([mag, mag], axis=-1)
    if dt == "bf16":
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(exact), 1e-30))) - 7)
        assert np.all(np.abs(got - exact) <= ulp + 4 * 2.0 ** -24 * mag)
    else:
        assert np.max(np.abs(got - exact)) <= 4e-7 * mag.max()


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------

def test_prefill_tiny_f32_workload(bf):
    w = W.get("tiny_f32")
    say("prefill", w)
    Q, K, V, cu = prefill_inputs(w)
    check_prefill(bf, w, Q, K, V, cu, F32_TOL)


def test_prefill_f32_ragged_d128(bf):
    w = W.Workload("f32_ragged", "prefill", "f32", Hq=6, Hkv=2, D=128, w0=50, w_pretrained=64,
                   theta=1e6, seqlens=(100, 333, 1, 64), outliers=4, seed=77)
    say("prefill", w)
    Q, K, V, cu = prefill_inputs(w)
    check_prefill(bf, w, Q, K, V, cu, F32_TOL)


BF16_CASES = [
    # name, Hq, Hkv, seqlens, w_pretrained, w0, outliers
    ("rep4_g4", 8, 2, (1000,), 256, 100, 4),
    ("rep1_ragged", 4, 4, (700, 45, 1333), 300, 64, 0),
    ("rep2_ragged", 8, 4, (513, 64, 1), 128, 200, 4),
    ("rep8_w0_1", 16, 2, (777,), 200, 1, 0),
    ("rep4_g1", 4, 1, (500,), 600, 64, 0),
    ("rep4_wide_window", 8, 2, (2500,), 512, 1000, 4),
    ("rep4_w0_ge_L", 4, 1, (300,), 64, 400, 4),
    # 3 KV heads, 12 query heads: 24 and 96 eight-pair chunks per token, so the
    # pair-maximum pre-pass runs partly filled chunk blocks
    ("rep4_hkv3", 12, 3, (900, 37), 256, 128, 4),
]


@pytest.mark.parametrize("case", BF16_CASES, ids=[c[0] for c in BF16_CASES])
def test_prefill_bf16_matches_oracle(bf, case):
    name, Hq, Hkv, seqlens, w_pre, w0, outl = case
    w = W.Workload(name, "prefill", "bf16", Hq=Hq, Hkv=Hkv, D=128, w0=w0, w_pretrained=w_pre,
                   theta=1e6, seqlens=seqlens, outliers=outl, seed=900 + len(name))
    say("prefill", w)
    Q, K, V, cu = prefill_inputs(w)
    check_prefill(bf, w, Q, K, V, cu, BF16_TOL)


def test_prefill_bf16_aligned_outliers_stress(bf):
    # the q heads of a group share the KV head's outlier channels: the hi/lo split on
    # the selected pairs is what keeps the remote scores accurate here
    w = W.Workload("aligned", "prefill", "bf16", Hq=8, Hkv=2, D=128, w0=64, w_pretrained=512,
                   theta=1e6, seqlens=(2048,), outliers=0, seed=4242)
    say("prefill aligned outliers", w)
    Q, K, V, cu = prefill_inputs(w)
    rng = np.random.default_rng(5)
    q, k, v = W.raw_prefill_inputs(w)
    for g in range(w.Hkv):
        ch = rng.choice(128, size=4, replace=False)
        for c in ch:
            k[:, g, c] *= 8
            for r in range(4):
                q[:, g * 4 + r, c] *= 8
    from helpers import std_rope_local
    Q = to_dtype(std_rope_local(q, cu, w.theta), "bf16")
    K = to_dtype(std_rope_local(k, cu, w.theta), "bf16")
    check_prefill(bf, w, Q, K, V, cu, BF16_TOL)


def test_prefill_bf16_g1_is_vanilla_bitwise(bf):
    # G = 1: every pair uses standard RoPE whatever w0 is, so w0 = 1 and w0 >= L must give
    # identical bits (same kernel path), and both must match the oracle.
    w = W.Workload("g1", "prefill", "bf16", Hq=8, Hkv=2, D=128, w0=1, w_pretrained=4096,
                   theta=1e6, seqlens=(1500,), seed=31)
    Q, K, V, cu = prefill_inputs(w)
    O1, L1 = run_prefill(bf, w, Q, K, V, cu)
    O2, L2 = run_prefill(bf, dataclasses.replace(w, w0=5000), Q, K, V, cu)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    check_prefill(bf, w, Q, K, V, cu, BF16_TOL)


def test_prefill_bf16_deterministic(bf):
    w = W.Workload("det", "prefill", "bf16", Hq=8, Hkv=2, D=128, w0=100, w_pretrained=300,
                   theta=1e6, seqlens=(900, 333), outliers=4, seed=12)
    Q, K, V, cu = prefill_inputs(w)
    O1, L1 = run_prefill(bf, w, Q, K, V, cu)
    O2, L2 = run_prefill(bf, w, Q, K, V, cu)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_prefill_empty_batch_is_noop(bf):
    Q = torch.zeros((0, 4, 128), dtype=torch.bfloat16, device="cuda")
    K = torch.zeros((0, 1, 128), dtype=torch.bfloat16, device="cuda")
    O, lse = bf.bifocal_prefill(Q, K, K, [0, 0], 4, 16, 1e4)
    assert O.shape == (0, 4, 128)


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dt,D,Hq,Hkv", [("bf16", 128, 8, 2), ("f32", 128, 4, 4),
                                         ("bf16", 64, 8, 1), ("f32", 64, 16, 2)])
def test_decode_matches_oracle(bf, dt, D, Hq, Hkv):
    w = W.Workload("dec", "decode", dt, Hq=Hq, Hkv=Hkv, D=D, w0=100, w_pretrained=1000,
                   theta=1e6, cache_len=3000, decode_steps=4, outliers=4, seed=55)
    say("decode", w)
    q_raw, Kc, Vc = decode_inputs(w)
    Kd, Vd = dev(Kc, dt), dev(Vc, dt)
    ws = bf.Workspace.for_op(bf.OP_DECODE, 3000, Hq, Hkv, D)
    tol = BF16_TOL if dt == "bf16" else F32_TOL
    for step, pos in enumerate((0, 5, 99, 100, 999, 1000, 2001, 2999)):
        q = std_query(q_raw[step % q_raw.shape[0]], pos, w.theta, dt)
        o, lse = bf.bifocal_decode(dev(q, dt), Kd, Vd, pos, w.w0, w.w_pretrained, w.theta,
                                   workspace=ws)
        torch.cuda.synchronize()
        Or, Lr = bifocal_decode_ref(q, Kc, Vc, pos, w.w0, w.w_pretrained, w.theta)
        e = errors(host(o), Or, lse.cpu().numpy(), Lr)
        say(f"  pos={pos} G={group_size(pos + 1, w.w_pretrained)} {e}")
        assert within(e, tol), (pos, e)


def test_decode_equals_prefill_last_row(bf):
    # the cache is read as is: decode at pos equals row pos of a prefill of length pos+1
    w = W.Workload("cross", "prefill", "bf16", Hq=8, Hkv=2, D=128, w0=64, w_pretrained=256,
                   theta=1e6, seqlens=(1200,), outliers=4, seed=99)
    Q, K, V, cu = prefill_inputs(w)
    for pos in (1199, 700, 255, 256):
        Og, Lg = run_prefill(bf, dataclasses.replace(w, seqlens=(pos + 1,)), Q[:pos + 1],
                             K[:pos + 1], V[:pos + 1], [0, pos + 1])
        o, lse = bf.bifocal_decode(dev(Q[pos], "bf16"), dev(K, "bf16"), dev(V, "bf16"), pos,
                                   w.w0, w.w_pretrained, w.theta)
        torch.cuda.synchronize()
        e = errors(host(o), Og[pos], lse.cpu().numpy(), Lg[:, pos])
        say(f"  pos={pos} decode vs prefill row: {e}")
        assert within(e, BF16_TOL)


# ---------------------------------------------------------------------------
# batched (ragged) decode and the length boundary
# ---------------------------------------------------------------------------

def _batch_caches(w, B, S):
    """B independently seeded caches [B,S,Hkv,D] and raw queries [B,Hq,D]."""
    qs, Ks, Vs = [], [], []
    for b in range(B):
        q_raw, Kc, Vc = decode_inputs(dataclasses.replace(w, seed=w.seed + 10 * b), S=S)
        qs.append(q_raw[0])
        Ks.append(Kc)
        Vs.append(Vc)
    return np.stack(qs), np.stack(Ks), np.stack(Vs)


@pytest.mark.parametrize("dt,D,Hq,Hkv", [("bf16", 128, 32, 8), ("bf16", 128, 8, 1),
                                         ("f32", 128, 4, 4), ("bf16", 64, 8, 2),
                                         ("bf16", 128, 32, 16), ("bf16", 128, 24, 12)])
def test_decode_batch_matches_oracle(bf, dt, D, Hq, Hkv):
    # ragged positions: G = 1, 1, 2, 3, 3 at w_pretrained 1000; window edges and a
    # one-key cache
    w = W.Workload("decb", "decode", dt, Hq=Hq, Hkv=Hkv, D=D, w0=100, w_pretrained=1000,
                   theta=1e6, cache_len=3000, decode_steps=1, outliers=4, seed=77)
    positions = [0, 999, 1000, 2001, 2999, 100, 57]
    B, S = len(positions), 3000
    say("decode batch", w, positions)
    q_raw, Kc, Vc = _batch_caches(w, B, S)
    q = np.stack([std_query(q_raw[b], positions[b], w.theta, dt) for b in range(B)])
    o, lse = bf.bifocal_decode_batch(dev(q, dt), dev(Kc, dt), dev(Vc, dt), positions, w.w0,
                                     w.w_pretrained, w.theta)
    torch.cuda.synchronize()
    og, lg = host(o), lse.cpu().numpy()
    tol = BF16_TOL if dt == "bf16" else F32_TOL
    for b, pos in enumerate(positions):
        Or, Lr = bifocal_decode_ref(q[b], Kc[b], Vc[b], pos, w.w0, w.w_pretrained, w.theta)
        e = errors(og[b], Or, lg[b], Lr)
        say(f"  seq {b} pos={pos} G={group_size(pos + 1, w.w_pretrained)} {e}")
        assert within(e, tol), (b, pos, e)


def test_decode_batch_sequences_do_not_interact(bf):
    # a sequence's result does not depend on the other members of its batch
    w = W.Workload("decb2", "decode", "bf16", Hq=16, Hkv=4, D=128, w0=64, w_pretrained=512,
                   theta=1e6, cache_len=2048, decode_steps=1, seed=91)
    positions = [2047, 600, 1500]
    q_raw, Kc, Vc = _batch_caches(w, 3, 2048)
    q = np.stack([std_query(q_raw[b], positions[b], w.theta, "bf16") for b in range(3)])
    qd, Kd, Vd = dev(q, "bf16"), dev(Kc, "bf16"), dev(Vc, "bf16")
    o_all, l_all = bf.bifocal_decode_batch(qd, Kd, Vd, positions, w.w0, w.w_pretrained, w.theta)
    o_one, l_one = bf.bifocal_decode_batch(qd[1:2].contiguous(), Kd[1:2].contiguous(),
                                           Vd[1:2].contiguous(), positions[1:2], w.w0,
                                           w.w_pretrained, w.theta)
    torch.cuda.synchronize()
    Or, Lr = bifocal_decode_ref(q[1], Kc[1], Vc[1], positions[1], w.w0, w.w_pretrained, w.theta)
    for o, l in ((o_all[1], l_all[1]), (o_one[0], l_one[0])):
        e = errors(host(o), Or, l.cpu().numpy(), Lr)
        say(f"  seq 1 {e}")
        assert within(e, BF16_TOL), e


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_decode_across_length_boundary(bf, dt):
    # w_pretrained 256: G is 4 up to L = 1024 and 5 from L = 1025 on; the cache is the
    # same bytes throughout (standard RoPE at absolute positions), only G changes
    w = W.Workload("bound", "decode", dt, Hq=8, Hkv=2, D=128, w0=48, w_pretrained=256,
                   theta=1e4, cache_len=1100, decode_steps=8, outliers=4, seed=123)
    q_raw, Kc, Vc = decode_inputs(w)
    Kd, Vd = dev(Kc, dt), dev(Vc, dt)
    ws = bf.Workspace.for_op(bf.OP_DECODE, 1100, w.Hq, w.Hkv, w.D, num_seqs=4)
    tol = BF16_TOL if dt == "bf16" else F32_TOL
    positions = [1021, 1022, 1023, 1024, 1025, 1026, 1099]
    assert [group_size(p + 1, 256) for p in positions] == [4, 4, 4, 5, 5, 5, 5]
    qs = [std_query(q_raw[i % 8], p, w.theta, dt) for i, p in enumerate(positions)]
    refs = [bifocal_decode_ref(q, Kc, Vc, p, w.w0, w.w_pretrained, w.theta)
            for q, p in zip(qs, positions)]
    for q, p, (Or, Lr) in zip(qs, positions, refs):  # one step at a time
        o, lse = bf.bifocal_decode(dev(q, dt), Kd, Vd, p, w.w0, w.w_pretrained, w.theta,
                                   workspace=ws)
        torch.cuda.synchronize()
        e = errors(host(o), Or, lse.cpu().numpy(), Lr)
        say(f"  pos={p} G={group_size(p + 1, 256)} {e}")
        assert within(e, tol), (p, e)
    # both sides of the boundary in one batched call over copies of the same cache
    sel = [2, 3, 4, 0]
    qb = np.stack([qs[i] for i in sel])
    Kb = Kd.unsqueeze(0).expand(len(sel), -1, -1, -1).contiguous()
    Vb = Vd.unsqueeze(0).expand(len(sel), -1, -1, -1).contiguous()
    o, lse = bf.bifocal_decode_batch(dev(qb, dt), Kb, Vb, [positions[i] for i in sel], w.w0,
                                     w.w_pretrained, w.theta, workspace=ws)
    torch.cuda.synchronize()
    for k, i in enumerate(sel):
        e = errors(host(o[k]), refs[i][0], lse[k].cpu().numpy(), refs[i][1])
        say(f"  batch member {k} pos={positions[i]} {e}")
        assert within(e, tol), (positions[i], e)


# ---------------------------------------------------------------------------
# the literal three-pass inclusion-exclusion form
# ---------------------------------------------------------------------------

IE_CASES = [c for c in BF16_CASES if c[0] in ("rep4_g4", "rep2_ragged", "rep8_w0_1", "rep4_g1",
                                                "rep4_wide_window", "rep4_w0_ge_L")]


@pytest.mark.parametrize("case", IE_CASES, ids=[c[0] for c in IE_CASES])
def test_prefill_ie_matches_oracle_and_fused(bf, case):
    # The merge Z = Z_B - Z_C + Z_A cancels where most of the remote mass lies in the
    # window while the local scores there are small (outlier channels make that
    # common): the passes' own errors (bf16 probabilities: relative 2^-9 per term) then
    # grow by cond = Z_B / Z.  Rows with cond <= 1.5 (most of them) must meet the bf16
    # tolerance; the others a bound that grows with cond.  A wrong pass would show in
    # the well-conditioned rows.
    name, Hq, Hkv, seqlens, w_pre, w0, outl = case
    w = W.Workload(name, "prefill", "bf16", Hq=Hq, Hkv=Hkv, D=128, w0=w0, w_pretrained=w_pre,
                   theta=1e6, seqlens=seqlens, outliers=outl, seed=700 + len(name))
    say("prefill ie", w)
    Q, K, V, cu = prefill_inputs(w)
    cuts = [int(c) for c in cu]
    Qd, Kd, Vd = dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16")
    O3, L3 = bf.bifocal_prefill_ie(Qd, Kd, Vd, cuts, w.w0, w.w_pretrained, w.theta)
    O1, L1 = bf.bifocal_prefill(Qd, Kd, Vd, cuts, w.w0, w.w_pretrained, w.theta)
    torch.cuda.synchronize()
    O3, L3, O1, L1 = host(O3), L3.cpu().numpy(), host(O1), L1.cpu().numpy()
    assert np.all(np.isfinite(O3)) and np.all(np.isfinite(L3))
    ref = bifocal_prefill_ref(Q, K, V, cu, w.w0, w.w_pretrained, w.theta)
    for b, (rows, O, LSE) in enumerate(ref):
        if O is None:
            continue
        s0, s1 = int(cu[b]), int(cu[b + 1])
        cond = ie_conditioning(Q[s0:s1], K[s0:s1], rows, w.w0, w.w_pretrained, w.theta)
        good = cond <= 1.5  # [rows, Hq]
        vmax = float(np.abs(V[s0:s1]).max())
        d_o = np.abs(O3[s0 + rows].astype(np.float64) - O).max(axis=2)
        d_l = np.abs(L3[:, s0 + rows].T - LSE)
        d_of = np.abs(O3[s0 + rows].astype(np.float64) - O1[s0 + rows]).max(axis=2)
        say(f"  seq {b}: cond max {cond.max():.3g}, {np.mean(good) * 100:.1f}% of (row, head) "
            f"with cond <= 1.5; well-conditioned max |dO| {d_o[good].max():.3g} mean "
            f"{np.abs(O3[s0 + rows] - O)[good].mean():.3g} max |dLSE| {d_l[good].max():.3g}; "
            f"three-pass vs fused max |dO| {d_of[good].max():.3g}")
        assert d_o[good].max() <= BF16_TOL["max_abs"]
        assert np.abs(O3[s0 + rows] - O)[good].mean() <= BF16_TOL["mean_abs"]
        assert d_l[good].max() <= BF16_TOL["lse_abs"]
        assert d_of[good].max() <= BF16_TOL["max_abs"]
        # everywhere: each pass's sums carry the bf16 rounding of its probabilities
        # (relative 2^-8 at worst), which the merge scales by the conditioning
        assert np.all(d_l <= BF16_TOL["lse_abs"] + 2.0 ** -7 * cond)
        assert np.all(d_o <= BF16_TOL["max_abs"] + 2.0 ** -7 * cond * vmax)


# ---------------------------------------------------------------------------
# variants: continuous remote positions and window-only layers
# ---------------------------------------------------------------------------

VARIANT_CASES = [
    # name, Hq, Hkv, seqlens, w_pretrained, w0, outliers
    ("v_rep4_g4", 8, 2, (1000,), 256, 100, 4),
    ("v_rep2_ragged", 8, 4, (513, 64, 1), 128, 200, 4),
    ("v_rep8_g3", 16, 2, (777,), 300, 50, 0),
    ("v_rep1_g1", 4, 4, (300,), 512, 64, 0),
]


@pytest.mark.parametrize("variant", ["interp", "window"])
@pytest.mark.parametrize("case", VARIANT_CASES, ids=[c[0] for c in VARIANT_CASES])
def test_prefill_variant_matches_oracle(bf, variant, case):
    name, Hq, Hkv, seqlens, w_pre, w0, outl = case
    w = W.Workload(name, "prefill", "bf16", Hq=Hq, Hkv=Hkv, D=128, w0=w0, w_pretrained=w_pre,
                   theta=1e6, seqlens=seqlens, outliers=outl, seed=600 + len(name))
    say("prefill", variant, w)
    Q, K, V, cu = prefill_inputs(w)
    O, lse = bf.bifocal_prefill_variant(dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16"),
                                        [int(c) for c in cu], w.w0, w.w_pretrained, w.theta,
                                        variant=variant)
    torch.cuda.synchronize()
    Og, Lg = host(O), lse.cpu().numpy()
    for b, (rows, Or, Lr) in enumerate(bifocal_prefill_ref(Q, K, V, cu, w.w0, w.w_pretrained,
                                                           w.theta, variant=variant)):
        if Or is None:
            continue
        s0 = int(cu[b])
        e = errors(Og[s0 + rows], Or, Lg[:, s0 + rows].T, Lr)
        say(f"  seq {b}: G={group_size(int(cu[b + 1] - cu[b]), w.w_pretrained)} {e}")
        assert within(e, BF16_TOL), (b, e)


def test_prefill_interp_g1_equals_method_bitwise(bf):
    w = W.Workload("g1i", "prefill", "bf16", Hq=8, Hkv=2, D=128, w0=40, w_pretrained=4096,
                   theta=1e6, seqlens=(900,), seed=41)
    Q, K, V, cu = prefill_inputs(w)
    args = (dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16"), [int(c) for c in cu], w.w0,
            w.w_pretrained, w.theta)
    O1, L1 = bf.bifocal_prefill(*args)
    O2, L2 = bf.bifocal_prefill_variant(*args, variant="interp")
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


@pytest.mark.parametrize("variant", ["interp", "window"])
def test_decode_variant_matches_oracle(bf, variant):
    w = W.Workload("decv", "decode", "bf16", Hq=16, Hkv=4, D=128, w0=100, w_pretrained=700,
                   theta=1e6, cache_len=3000, decode_steps=1, outliers=4, seed=81)
    positions = [2999, 1400, 699, 700, 99, 0, 2048]
    q_raw, Kc, Vc = _batch_caches(w, len(positions), 3000)
    q = np.stack([std_query(q_raw[b], positions[b], w.theta, "bf16")
                  for b in range(len(positions))])
    o, lse = bf.bifocal_decode_variant(dev(q, "bf16"), dev(Kc, "bf16"), dev(Vc, "bf16"),
                                       positions, w.w0, w.w_pretrained, w.theta, variant=variant)
    torch.cuda.synchronize()
    og, lg = host(o), lse.cpu().numpy()
    for b, pos in enumerate(positions):
        Or, Lr = bifocal_decode_ref(q[b], Kc[b], Vc[b], pos, w.w0, w.w_pretrained, w.theta,
                                    variant=variant)
        e = errors(og[b], Or, lg[b], Lr)
        say(f"  {variant} seq {b} pos={pos} G={group_size(pos + 1, w.w_pretrained)} {e}")
        assert within(e, BF16_TOL), (variant, pos, e)


# ---------------------------------------------------------------------------
# an explicit softmax scale (flatter and sharper than 1/sqrt(D))
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("scale", [0.03, 0.2])
@pytest.mark.parametrize("dt,D", [("bf16", 128), ("f32", 64)])
def test_explicit_softmax_scale(bf, dt, D, scale):
    w = W.Workload("scale", "prefill", dt, Hq=8, Hkv=2, D=D, w0=40, w_pretrained=128,
                   theta=1e4, seqlens=(600, 77), outliers=0, seed=311)
    say("prefill, softmax_scale", scale, w)
    Q, K, V, cu = prefill_inputs(w)
    O, lse = bf.bifocal_prefill(dev(Q, dt), dev(K, dt), dev(V, dt), [int(c) for c in cu],
                                w.w0, w.w_pretrained, w.theta, softmax_scale=scale)
    torch.cuda.synchronize()
    Og, Lg = host(O), lse.cpu().numpy()
    tol = BF16_TOL if dt == "bf16" else F32_TOL
    ref = bifocal_prefill_ref(Q, K, V, cu, w.w0, w.w_pretrained, w.theta, scale=scale)
    for b, (rows, Or, Lr) in enumerate(ref):
        s0 = int(cu[b])
        e = errors(Og[s0 + rows], Or, Lg[:, s0 + rows].T, Lr)
        say(f"  seq {b} {e}")
        assert within(e, tol), (b, e)
    # decode over a cache with the same scale (matrix-core path for bf16 D = 128,
    # vector path otherwise)
    wd = W.Workload("scaled", "decode", dt, Hq=8, Hkv=2, D=D, w0=40, w_pretrained=128,
                    theta=1e4, cache_len=900, decode_steps=2, outliers=0, seed=312)
    q_raw, Kc, Vc = decode_inputs(wd)
    for step, pos in enumerate((899, 130)):
        q = std_query(q_raw[step], pos, wd.theta, dt)
        o, l = bf.bifocal_decode(dev(q, dt), dev(Kc, dt), dev(Vc, dt), pos, wd.w0,
                                 wd.w_pretrained, wd.theta, softmax_scale=scale)
        torch.cuda.synchronize()
        Or, Lr = bifocal_decode_ref(q, Kc, Vc, pos, wd.w0, wd.w_pretrained, wd.theta,
                                    scale=scale)
        e = errors(host(o), Or, l.cpu().numpy(), Lr)
        say(f"  decode pos={pos} {e}")
        assert within(e, tol), (pos, e)


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("f32", 64)])
def test_outputs_without_lse_are_identical(bf, dt, D):
    # lse = NULL only skips the LSE stores: O is bit for bit the same
    w = W.Workload("nolse", "prefill", dt, Hq=8, Hkv=2, D=D, w0=30, w_pretrained=100,
                   theta=1e4, seqlens=(400, 33), outliers=4, seed=313)
    say("outputs without lse", dt, D)
    Q, K, V, cu = prefill_inputs(w)
    Qd, Kd, Vd = dev(Q, dt), dev(K, dt), dev(V, dt)
    c = [int(x) for x in cu]
    calls = [("prefill", lambda want: bf.bifocal_prefill(Qd, Kd, Vd, c, w.w0, w.w_pretrained,
                                                         w.theta, want_lse=want))]
    if dt == "bf16":
        calls.append(("prefill_ie", lambda want: bf.bifocal_prefill_ie(
            Qd, Kd, Vd, c, w.w0, w.w_pretrained, w.theta, want_lse=want)))
    qb = Qd[:3].contiguous()
    Kb = torch.stack([Kd[:300], Kd[:300], Kd[:300]]).contiguous()
    Vb = torch.stack([Vd[:300], Vd[:300], Vd[:300]]).contiguous()
    calls.append(("decode", lambda want: bf.bifocal_decode(Qd[299], Kd, Vd, 299, w.w0,
                                                           w.w_pretrained, w.theta,
                                                           want_lse=want)))
    calls.append(("decode_batch", lambda want: bf.bifocal_decode_batch(
        qb, Kb, Vb, [299, 150, 0], w.w0, w.w_pretrained, w.theta, want_lse=want)))
    for name, fn in calls:
        o1, l1 = fn(True)
        o2, l2 = fn(False)
        torch.cuda.synchronize()
        assert l1 is not None and l2 is None
        assert torch.equal(o1, o2), name
        assert bool(torch.isfinite(l1).all()), name


# ---------------------------------------------------------------------------
# launch chunking: more sequences than one launch takes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_prefill_many_sequences_chunked(bf, dt):
    # 53 sequences (more than one launch's 48), with empty ones in between and G from
    # 1 to 3
    lens = tuple([0] + [(37 * i) % 150 + 1 for i in range(50)] + [0, 300])
    w = W.Workload("many", "prefill", dt, Hq=4, Hkv=2, D=128, w0=20, w_pretrained=100,
                   theta=1e6, seqlens=lens, outliers=0, seed=17)
    say("prefill many sequences", dt, len(lens))
    Q, K, V, cu = prefill_inputs(w)
    check_prefill(bf, w, Q, K, V, cu, BF16_TOL if dt == "bf16" else F32_TOL)


def test_prefill_bf16_outlier_stress_many_short_sequences(bf):
    # The workloads' outlier layout (4 independently seeded x8 channels in every query head
    # and in every KV head: 12 outlier channels per group here) over 24 short sequences: the
    # hi/lo correction covers only 4 RoPE pairs per KV head, so most outlier pairs are
    # scored with fp16 operands alone.  Held to the bf16 tolerance as every other case.
    lens = tuple([(37 * i) % 150 + 1 for i in range(24)])
    w = W.Workload("stress", "prefill", "bf16", Hq=4, Hkv=2, D=128, w0=20, w_pretrained=100,
                   theta=1e6, seqlens=lens, outliers=4, seed=17)
    Q, K, V, cu = prefill_inputs(w)
    check_prefill(bf, w, Q, K, V, cu, BF16_TOL)


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("f32", 64)])
def test_decode_batch_chunked(bf, dt, D):
    # 70 sequences (more than one launch's 64) with short caches of their own lengths
    w = W.Workload("decmany", "decode", dt, Hq=8, Hkv=2, D=D, w0=16, w_pretrained=40,
                   theta=1e4, cache_len=96, decode_steps=1, seed=23)
    positions = [(13 * b) % 96 for b in range(70)]
    q_raw, Kc, Vc = _batch_caches(w, 70, 96)
    q = np.stack([std_query(q_raw[b], positions[b], w.theta, dt) for b in range(70)])
    o, lse = bf.bifocal_decode_batch(dev(q, dt), dev(Kc, dt), dev(Vc, dt), positions, w.w0,
                                     w.w_pretrained, w.theta)
    torch.cuda.synchronize()
    og, lg = host(o), lse.cpu().numpy()
    tol = BF16_TOL if dt == "bf16" else F32_TOL
    worst = {}
    for b, pos in enumerate(positions):
        Or, Lr = bifocal_decode_ref(q[b], Kc[b], Vc[b], pos, w.w0, w.w_pretrained, w.theta)
        e = errors(og[b], Or, lg[b], Lr)
        for k, v in e.items():
            worst[k] = max(worst.get(k, 0.0), v)
        assert within(e, tol), (b, pos, e)
    say(f"  70 sequences, worst {worst}")


# ---------------------------------------------------------------------------
# the position table cached in the workspace
# ---------------------------------------------------------------------------

def test_table_cache_rebuilds_when_stale(bf):
    # a workspace full of garbage, then reused with another theta and a longer sequence:
    # every call must see a table for its own (theta, D, length)
    w = W.Workload("tab", "prefill", "f32", Hq=4, Hkv=2, D=64, w0=16, w_pretrained=64,
                   theta=1e4, seqlens=(300,), outliers=0, seed=5)
    ws = bf.Workspace.for_op(bf.OP_PREFILL, 5000, 4, 2, 64, total_tokens=5000)
    g = torch.Generator(device="cpu").manual_seed(3)
    ws.buf.copy_(torch.randint(0, 256, ws.buf.shape, generator=g, dtype=torch.uint8))
    for theta, L in ((1e4, 300), (5e5, 300), (5e5, 2100), (1e4, 4000)):
        wt = dataclasses.replace(w, theta=theta, seqlens=(L,))
        Q, K, V, cu = prefill_inputs(wt)
        O, lse = bf.bifocal_prefill(dev(Q, "f32"), dev(K, "f32"), dev(V, "f32"), [0, L], wt.w0,
                                    wt.w_pretrained, theta, workspace=ws)
        torch.cuda.synchronize()
        rows = np.unique(np.r_[np.arange(0, L, 97), L - 1])
        ref = bifocal_prefill_ref(Q, K, V, cu, wt.w0, wt.w_pretrained, theta, rows_per_seq=[rows])
        e = errors(host(O)[rows], ref[0][1], lse.cpu().numpy()[:, rows].T, ref[0][2])
        say(f"  theta={theta:g} L={L}: {e}")
        assert within(e, F32_TOL), (theta, L, e)


# ---------------------------------------------------------------------------
# operands beyond the fp16 range, and one workspace shared by prefill and decode
# ---------------------------------------------------------------------------

def test_prefill_operands_beyond_fp16_range(bf):
    # Raw channels of about 1e5 (bf16 holds them; fp16 overflows at 65504) in a query
    # pair, a key pair and a value channel.  The remote operands and V^T are scaled by
    # exact powers of two before their fp16 rounding, so nothing overflows.  The huge
    # query and key pairs meet tiny partners on the other side (so the scores stay of
    # ordinary size); the huge value channel is compared relative to its size.
    w = W.Workload("range", "prefill", "bf16", Hq=4, Hkv=2, D=128, w0=40, w_pretrained=128,
                   theta=1e6, seqlens=(600,), outliers=0, seed=808)
    q, k, v = W.raw_prefill_inputs(w)
    q[:, :, 3] *= 1e5
    k[:, :, 3] *= 1e-5
    k[:, :, 67] *= 1e-5
    k[:, :, 10] *= 1e5
    q[:, :, 10] *= 1e-5
    q[:, :, 74] *= 1e-5
    v[:, :, 20] *= 1e5
    cu = w.cu_seqlens
    from helpers import std_rope_local
    Q = to_dtype(std_rope_local(q, cu, w.theta), "bf16")
    K = to_dtype(std_rope_local(k, cu, w.theta), "bf16")
    V = to_dtype(v, "bf16")
    assert np.abs(Q).max() > 65504 and np.abs(K).max() > 65504 and np.abs(V).max() > 65504
    Og, Lg = run_prefill(bf, w, Q, K, V, cu)
    assert np.all(np.isfinite(Og)) and np.all(np.isfinite(Lg))
    (rows, Or, Lr), = bifocal_prefill_ref(Q, K, V, cu, w.w0, w.w_pretrained, w.theta)
    normal = np.ones(128, dtype=bool)
    normal[20] = False
    e = errors(Og[rows][..., normal], Or[..., normal], Lg[:, rows].T, Lr)
    # channel 20 against its own scale: the bf16 bound 2e-2 is 5e-3 of the largest |V| of
    # a unit-normal channel (about 4)
    d20 = float(np.abs(Og[rows][..., 20] - Or[..., 20]).max())
    rel20 = d20 / float(np.abs(V[..., 20]).max())
    say(f"  beyond fp16 range: {e}, value channel 20: max |dO| {d20:.3g} = {rel20:.3g} of max |V|")
    assert within(e, BF16_TOL), e
    assert rel20 <= 5e-3, rel20


def test_prefill_decode_prefill_share_one_workspace(bf):
    # A decode-sized workspace also serves prefills that fit it.  The decode partials sit
    # past the rows of its own layout's table region, over rows a longer prefill built
    # earlier; the next prefill must rebuild them, not trust them.
    Hq, Hkv = 8, 2
    ws = bf.Workspace.for_op(bf.OP_DECODE, 1000, Hq, Hkv, 128)
    w = W.Workload("shared", "prefill", "bf16", Hq=Hq, Hkv=Hkv, D=128, w0=64, w_pretrained=300,
                   theta=1e6, seqlens=(1500,), outliers=4, seed=606)
    Q, K, V, cu = prefill_inputs(w)
    Qd, Kd, Vd = dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16")
    rows = np.unique(np.r_[np.arange(0, 1500, 37), 1499, 1250, 1251])
    for step, w_pre in enumerate((300, None, 250)):
        if w_pre is None:
            pos = 999
            o, l = bf.bifocal_decode(Qd[pos], Kd, Vd, pos, 64, 300, w.theta, workspace=ws)
            torch.cuda.synchronize()
            Or, Lr = bifocal_decode_ref(Q[pos], K, V, pos, 64, 300, w.theta)
            e = errors(host(o), Or, l.cpu().numpy(), Lr)
        else:
            wp = dataclasses.replace(w, w_pretrained=w_pre)
            O, lse = bf.bifocal_prefill(Qd, Kd, Vd, [0, 1500], wp.w0, w_pre, w.theta,
                                        workspace=ws)
            torch.cuda.synchronize()
            (rr, Or, Lr), = bifocal_prefill_ref(Q, K, V, cu, wp.w0, w_pre, w.theta,
                                                rows_per_seq=[rows])
            e = errors(host(O)[rows], Or, lse.cpu().numpy()[:, rows].T, Lr)
        say(f"  step {step} ({'decode' if w_pre is None else f'prefill G={group_size(1500, w_pre)}'}): {e}")
        assert within(e, BF16_TOL), (step, e)


def test_position_table_rows_match_reference(bf):
    # The workspace keeps [256 B header][rows p: D/2 x (cos, sin) float32] after a call.
    # Each entry must be the float64 value rounded once to float32 (at most one float32
    # ulp off where the float64 result sits next to a rounding boundary), and read at
    # n = x - f(x) with the sine negated it must give the correction rotation R(f(x) - x).
    from oracle.bifocal_ref import rope_tables_ref
    w = W.Workload("table", "prefill", "bf16", Hq=4, Hkv=2, D=128, w0=50, w_pretrained=700,
                   theta=1e6, seqlens=(3000,), outliers=0, seed=41)
    G = group_size(3000, w.w_pretrained)
    Q, K, V, cu = prefill_inputs(w)
    ws = bf.Workspace.for_op(bf.OP_PREFILL, 3000, w.Hq, w.Hkv, w.D, total_tokens=3000)
    bf.bifocal_prefill(dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16"), [0, 3000], w.w0,
                       w.w_pretrained, w.theta, workspace=ws)
    torch.cuda.synchronize()
    off = ws.ptr - ws.buf.data_ptr()
    raw = ws.buf[off:off + ws.nbytes].cpu().numpy()
    magic = int(raw[:8].view(np.uint64)[0])
    theta = float(raw[8:16].view(np.float64)[0])
    D, n_valid = (int(x) for x in raw[16:24].view(np.int32))
    say(f"  header: magic {magic:#x} theta {theta:g} D {D} rows {n_valid}")
    assert theta == w.theta and D == 128 and n_valid >= 3000
    tab = raw[256:256 + n_valid * 64 * 8].view(np.float32).reshape(n_valid, 64, 2)
    c, s, cc, sc = rope_tables_ref(n_valid, 128, w.theta, G)
    for got, want in ((tab[..., 0], c), (tab[..., 1], s)):
        w32 = want.astype(np.float32)
        ulp = np.spacing(np.abs(w32))
        assert np.all(np.abs(got - w32) <= ulp)
        assert np.mean(got == w32) >= 0.9999
    x = np.arange(3000)
    n = x - x // G
    for got, want in ((tab[n, :, 0], cc[:3000]), (-tab[n, :, 1], sc[:3000])):
        w32 = want.astype(np.float32)
        assert np.all(np.abs(got - w32) <= np.spacing(np.abs(w32)))


def test_decode_split_count_invariance(bf):
    # The split count follows the launch: one sequence alone gets 39 workgroups per KV
    # head here, the same sequence in a batch of eight gets 8.  Both results must meet the
    # bf16 tolerance against the oracle and agree with each other within it.
    w = W.Workload("splits", "decode", "bf16", Hq=32, Hkv=8, D=128, w0=256, w_pretrained=5000,
                   theta=1e6, cache_len=20000, decode_steps=1, outliers=4, seed=515)
    q_raw, Kc, Vc = decode_inputs(w)
    pos = 19999
    q = std_query(q_raw[0], pos, w.theta, "bf16")
    qd, Kd, Vd = dev(q, "bf16"), dev(Kc, "bf16"), dev(Vc, "bf16")
    o1, l1 = bf.bifocal_decode(qd, Kd, Vd, pos, w.w0, w.w_pretrained, w.theta)
    B = 8
    o8, l8 = bf.bifocal_decode_batch(qd.unsqueeze(0).expand(B, -1, -1).contiguous(),
                                     Kd.unsqueeze(0).expand(B, -1, -1, -1).contiguous(),
                                     Vd.unsqueeze(0).expand(B, -1, -1, -1).contiguous(),
                                     [pos] * B, w.w0, w.w_pretrained, w.theta)
    torch.cuda.synchronize()
    Or, Lr = bifocal_decode_ref(q, Kc, Vc, pos, w.w0, w.w_pretrained, w.theta)
    e1 = errors(host(o1), Or, l1.cpu().numpy(), Lr)
    e8 = errors(host(o8[3]), Or, l8[3].cpu().numpy(), Lr)
    d = errors(host(o1), host(o8[3]).astype(np.float64), l1.cpu().numpy(),
               l8[3].cpu().numpy().astype(np.float64))
    say(f"  alone {e1}; in a batch of 8 {e8}; between them {d}")
    for e in (e1, e8, d):
        assert within(e, BF16_TOL), e
    assert all(torch.equal(o8[0], o8[b]) for b in range(1, B))
