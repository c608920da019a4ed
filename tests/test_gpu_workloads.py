"""GPU parity at the full workload sizes, in the launch configuration the benchmark
times: every output row is computed on the GPU, and sampled rows (first/last rows,
rows around w0, tile and aliasing-group boundaries, uniform draws) of every head are
compared with the CPU oracle, which computes each row from its definition."""
import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle.bifocal_ref import bifocal_decode_ref, bifocal_rows, group_size, rope_apply_ref
from helpers import (BF16_TOL, decode_inputs, errors, ie_conditioning, prefill_inputs,
                     std_query, std_rope_local, to_dtype, within)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def bf():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import dynamic_rope_context_amd as m
    m.lib()
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).cuda()


def _prefill_case(bf, name, n_uniform, ie=False, variant="bifocal", min_rows=512, w0=None):
    w = W.get(name)
    if w0 is not None:  # another window on the same inputs (w0 >= L: every pair local)
        import dataclasses
        w = dataclasses.replace(w, w0=w0)
    say(f"{name}: building inputs on the CPU")
    Q, K, V, cu = prefill_inputs(w)
    say(f"{name}: GPU prefill" + (" (three-pass inclusion-exclusion form)" if ie else "")
        + (f" (variant {variant})" if variant != "bifocal" else ""))
    args = (dev(Q), dev(K), dev(V), [int(c) for c in cu], w.w0, w.w_pretrained, w.theta)
    if variant != "bifocal":
        O, lse = bf.bifocal_prefill_variant(*args, variant=variant)
    else:
        O, lse = (bf.bifocal_prefill_ie if ie else bf.bifocal_prefill)(*args)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(O).all())
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        L = e - s
        G = group_size(L, w.w_pretrained)
        rows = W.sample_rows(L, w.w0, n_uniform, seed=w.seed + b, tile=64,
                             extra=(G * 1000 - 1, G * 1000, w.w0 + 63, w.w0 + 64))
        assert len(rows) >= min_rows, len(rows)
        Og = O[s + rows].float().cpu().numpy()
        Lg = lse[:, s + rows].T.cpu().numpy()
        say(f"{name}: oracle on {len(rows)} rows x {w.Hq} heads of sequence {b} (L={L}, G={G})")
        Or, Lr = bifocal_rows(Q[s:e], K[s:e], V[s:e], rows, w.w0, w.w_pretrained, w.theta,
                              variant=variant)
        if not ie:
            err = errors(Og, Or, Lg, Lr)
            say(f"{name}: seq {b} {err}")
            assert within(err, BF16_TOL), err
            continue
        # three-pass form: bf16 tolerance where the merge is well conditioned
        # (cond = Z_B / Z <= 1.5), a bound growing with cond elsewhere
        cond = ie_conditioning(Q[s:e], K[s:e], rows, w.w0, w.w_pretrained, w.theta)
        good = cond <= 1.5
        vmax = float(np.abs(V[s:e]).max())
        d_o = np.abs(Og.astype(np.float64) - Or).max(axis=2)
        d_l = np.abs(Lg - Lr)
        say(f"{name}: seq {b} three-pass: cond max {cond.max():.3g}, "
            f"{np.mean(good) * 100:.1f}% well conditioned; there max |dO| {d_o[good].max():.3g}, "
            f"mean {np.abs(Og - Or)[good].mean():.3g}, max |dLSE| {d_l[good].max():.3g}")
        assert d_o[good].max() <= BF16_TOL["max_abs"]
        assert np.abs(Og - Or)[good].mean() <= BF16_TOL["mean_abs"]
        assert d_l[good].max() <= BF16_TOL["lse_abs"]
        assert np.all(d_l <= BF16_TOL["lse_abs"] + 2.0 ** -7 * cond)
        assert np.all(d_o <= BF16_TOL["max_abs"] + 2.0 ** -7 * cond * vmax)


# At least 512 sampled rows of every sequence, all query heads (first and last rows, rows
# around w0, tile and aliasing-group boundaries, uniform draws); 128 for the variant and
# the three-pass form.


def test_qwen3_1p7b_32k_g1(bf):
    _prefill_case(bf, "qwen3_1p7b_32k_g1", 480)


def test_qwen3_4b_128k(bf):
    _prefill_case(bf, "qwen3_4b_128k", 480)


def test_qwen3_8b_ragged(bf):
    _prefill_case(bf, "qwen3_8b_ragged", 480)


def test_qwen3_4b_128k_interp_variant(bf):
    # continuous remote positions x / G at full size (angles evaluated in the kernels)
    _prefill_case(bf, "qwen3_4b_128k", 100, variant="interp", min_rows=128)


def test_qwen3_4b_128k_vanilla_mode(bf):
    # the benchmark's vanilla comparator: the same call with w0 = L (every pair local,
    # i.e. causal attention with standard RoPE)
    _prefill_case(bf, "qwen3_4b_128k", 100, min_rows=128, w0=131072)


def test_qwen3_4b_128k_three_pass(bf):
    # the pages' literal form (three passes merged by their LSEs) at full size
    _prefill_case(bf, "qwen3_4b_128k", 100, ie=True, min_rows=128)


def test_qwen3_8b_decode_128k(bf):
    w = W.get("qwen3_8b_decode_128k")
    say("decode: building the cache on the CPU")
    q_raw, Kc, Vc = decode_inputs(w)
    Kd, Vd = dev(Kc), dev(Vc)
    ws = bf.Workspace.for_op(bf.OP_DECODE, w.cache_len, w.Hq, w.Hkv, w.D)
    positions = w.decode_positions()
    checked = {0, 1, len(positions) // 2, len(positions) - 1}
    for step, pos in enumerate(positions):
        q = std_query(q_raw[step], int(pos), w.theta, "bf16")
        o, lse = bf.bifocal_decode(dev(q), Kd, Vd, int(pos), w.w0, w.w_pretrained, w.theta,
                                   workspace=ws)
        if step in checked:
            torch.cuda.synchronize()
            Or, Lr = bifocal_decode_ref(q, Kc, Vc, int(pos), w.w0, w.w_pretrained, w.theta)
            err = errors(o.float().cpu().numpy(), Or, lse.cpu().numpy(), Lr)
            say(f"decode step {step} pos={int(pos)} G={group_size(int(pos) + 1, w.w_pretrained)}"
                f" {err}")
            assert within(err, BF16_TOL), err
    torch.cuda.synchronize()


def test_qwen3_8b_decode_128k_vanilla_mode(bf):
    # the benchmark's vanilla decode comparator: w0 past the position (every key local)
    import dataclasses
    w = dataclasses.replace(W.get("qwen3_8b_decode_128k"), w0=1 << 20)
    say("vanilla decode: building the cache on the CPU")
    q_raw, Kc, Vc = decode_inputs(w)
    Kd, Vd = dev(Kc), dev(Vc)
    ws = bf.Workspace.for_op(bf.OP_DECODE, w.cache_len, w.Hq, w.Hkv, w.D)
    positions = w.decode_positions()
    for step in (0, len(positions) - 1):
        pos = int(positions[step])
        q = std_query(q_raw[step], pos, w.theta, "bf16")
        o, lse = bf.bifocal_decode(dev(q), Kd, Vd, pos, w.w0, w.w_pretrained, w.theta,
                                   workspace=ws)
        torch.cuda.synchronize()
        Or, Lr = bifocal_decode_ref(q, Kc, Vc, pos, w.w0, w.w_pretrained, w.theta)
        err = errors(o.float().cpu().numpy(), Or, lse.cpu().numpy(), Lr)
        say(f"vanilla decode step {step} pos={pos} {err}")
        assert within(err, BF16_TOL), err


def test_qwen3_8b_decode_across_boundary(bf):
    # 258 consecutive steps from position 131071 (G = 4) to 131328 (G = 5 from 131072 on),
    # over one cache that is never rewritten; then both sides of the boundary in one
    # batched call
    w = W.get("qwen3_8b_decode_boundary")
    say("decode boundary: building the cache on the CPU")
    q_raw, Kc, Vc = decode_inputs(w)
    Kd, Vd = dev(Kc), dev(Vc)
    ws = bf.Workspace.for_op(bf.OP_DECODE, w.cache_len, w.Hq, w.Hkv, w.D, num_seqs=2)
    positions = w.decode_positions()
    assert int(positions[0]) == 131071 and int(positions[-1]) == 131328
    checked = {0, 1, 2, len(positions) - 1}
    qs = {}
    for step, pos in enumerate(positions):
        q = std_query(q_raw[step], int(pos), w.theta, "bf16")
        o, lse = bf.bifocal_decode(dev(q), Kd, Vd, int(pos), w.w0, w.w_pretrained, w.theta,
                                   workspace=ws)
        if step in checked:
            qs[step] = q
            torch.cuda.synchronize()
            Or, Lr = bifocal_decode_ref(q, Kc, Vc, int(pos), w.w0, w.w_pretrained, w.theta)
            err = errors(o.float().cpu().numpy(), Or, lse.cpu().numpy(), Lr)
            say(f"decode step {step} pos={int(pos)} G={group_size(int(pos) + 1, w.w_pretrained)}"
                f" {err}")
            assert within(err, BF16_TOL), err
    torch.cuda.synchronize()
    Kb = Kd.unsqueeze(0).expand(2, -1, -1, -1).contiguous()
    Vb = Vd.unsqueeze(0).expand(2, -1, -1, -1).contiguous()
    pb = [int(positions[0]), int(positions[1])]
    qb = np.stack([qs[0], qs[1]])
    o, lse = bf.bifocal_decode_batch(dev(qb), Kb, Vb, pb, w.w0, w.w_pretrained, w.theta,
                                     workspace=ws)
    torch.cuda.synchronize()
    for k, pos in enumerate(pb):
        Or, Lr = bifocal_decode_ref(qb[k], Kc, Vc, pos, w.w0, w.w_pretrained, w.theta)
        err = errors(o[k].float().cpu().numpy(), Or, lse[k].cpu().numpy(), Lr)
        say(f"batched pos={pos} G={group_size(pos + 1, w.w_pretrained)} {err}")
        assert within(err, BF16_TOL), err


@pytest.mark.parametrize("G", [1, 4])
def test_rope_apply_qwen3_4b_128k_query(bf, G):
    # rope_apply in place on the 128K workload's query tensor [131072, 32, 128] bf16, the
    # launch the benchmark times (G = 1: standard RoPE at positions 0 .. T-1; G = 4: the
    # aliased positions of this length), checked on up to 512 sampled tokens (the first and last 64) x all heads
    w = W.get("qwen3_4b_128k")
    T = w.total_tokens
    q, _, _ = W.raw_inputs_torch(w, "cuda")
    rng = np.random.default_rng(w.seed + 17)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(T - 64, T),
                                     rng.integers(64, T - 64, size=384)]))
    idx = torch.from_numpy(rows.astype(np.int64)).cuda()
    x = q.index_select(0, idx).float().cpu().numpy()  # the exact bf16 inputs of the rows
    say(f"rope_apply 128K query tensor G={G}: {len(rows)} sampled tokens x {w.Hq} heads")
    bf.rope_apply(q, w.theta, G=G)
    torch.cuda.synchronize()
    got = q.index_select(0, idx).float().cpu().numpy().astype(np.float64)
    exact = rope_apply_ref(x, rows, w.theta, G)
    D = w.D
    x64 = x.astype(np.float64)
    mag = np.abs(x64[..., :D // 2]) + np.abs(x64[..., D // 2:])
    mag = np.concatenate([mag, mag], axis=-1)
    # one bf16 rounding of a float32 rotation, as in the small rope_apply tests
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(exact), 1e-30))) - 7)
    assert np.all(np.abs(got - exact) <= ulp + 4 * 2.0 ** -24 * mag)


def test_decode_batch_8x16k(bf):
    # the batched decode the benchmark times: 8 sequences of the 128K decode layer's
    # shape, each with its own 16384-row cache (the 128K workload's cache rows cut into
    # 8 sequences, standard RoPE at each sequence's own positions), all queries at
    # position 16383, in one bifocal_decode_batch call; every sequence against the oracle
    w = W.get("qwen3_8b_decode_128k")
    B, S = 8, 16384
    q_raw, k_raw, v_raw = W.raw_decode_inputs(w, S=B * S)
    cu = [b * S for b in range(B + 1)]
    say("batched decode 8 x 16K: building the caches on the CPU")
    Kc = to_dtype(std_rope_local(k_raw, cu, w.theta), "bf16").reshape(B, S, w.Hkv, w.D)
    Vc = to_dtype(v_raw, "bf16").reshape(B, S, w.Hkv, w.D)
    qb = np.stack([std_query(q_raw[b], S - 1, w.theta, "bf16") for b in range(B)])
    positions = [S - 1] * B
    ws = bf.Workspace.for_op(bf.OP_DECODE, S, w.Hq, w.Hkv, w.D, num_seqs=B)
    o, lse = bf.bifocal_decode_batch(dev(qb), dev(Kc), dev(Vc), positions, w.w0, w.w_pretrained,
                                     w.theta, workspace=ws)
    torch.cuda.synchronize()
    for b in range(B):
        Or, Lr = bifocal_decode_ref(qb[b], Kc[b], Vc[b], S - 1, w.w0, w.w_pretrained, w.theta)
        err = errors(o[b].float().cpu().numpy(), Or, lse[b].cpu().numpy(), Lr)
        say(f"batched sequence {b} pos={S - 1} G={group_size(S, w.w_pretrained)} {err}")
        assert within(err, BF16_TOL), err
