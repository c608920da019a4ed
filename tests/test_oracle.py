"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: the loop-only twin with
explicit rotation matrices, a library routine (torch SDPA in float64), a
closed form, or an identity stated on the pages (three-pass inclusion-
exclusion merge, additive composition of rotations, in-grid remote angles).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from oracle.bifocal_ref import (alias, bifocal_decode_ref, bifocal_prefill_ref, bifocal_rows,
                                group_size, inv_freq, rope_apply_ref, rope_rotate,
                                rope_tables_ref)


# --------------------------------------------------------------------------
# independent helpers (complex-number RoPE, masked softmax, SDPA wrapper)
# --------------------------------------------------------------------------

def rope_complex(x, pos, theta):
    """RoPE as complex multiplication: z_m = x_m + i x_{m+D/2} times e^{i p theta_m}."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    h = D // 2
    freqs = np.array([theta ** (-(2.0 * m) / D) for m in range(h)])
    z = x[..., :h] + 1j * x[..., h:]
    z = z * np.exp(1j * np.asarray(pos, dtype=np.float64)[:, None, None] * freqs[None, None, :])
    return np.concatenate([z.real, z.imag], axis=-1)


def sdpa_f64(Q, K, V, scale=None):
    """torch SDPA, causal, float64 on CPU; GQA by repeating KV heads.  [L,H,D] layout."""
    Hq, Hkv = Q.shape[1], K.shape[1]
    rep = Hq // Hkv
    q = torch.from_numpy(np.ascontiguousarray(np.asarray(Q, np.float64).transpose(1, 0, 2)))
    k = torch.from_numpy(np.ascontiguousarray(np.asarray(K, np.float64).transpose(1, 0, 2)))
    v = torch.from_numpy(np.ascontiguousarray(np.asarray(V, np.float64).transpose(1, 0, 2)))
    k = k.repeat_interleave(rep, dim=0)
    v = v.repeat_interleave(rep, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale)
    return o.numpy().transpose(1, 0, 2)


def masked_softmax_pass(Qv, Kv, V, mask, scale):
    """One attention pass with an explicit boolean mask; returns (O, LSE) per [i, h]."""
    L, Hq, D = Qv.shape
    rep = Hq // Kv.shape[1]
    O = np.zeros((L, Hq, D))
    LSE = np.full((L, Hq), -np.inf)
    for h in range(Hq):
        g = h // rep
        s = scale * (Qv[:, h, :] @ Kv[:, g, :].T)
        s = np.where(mask, s, -np.inf)
        m = np.max(s, axis=1, keepdims=True)
        ok = np.isfinite(m[:, 0])
        e = np.where(np.isfinite(s), np.exp(s - np.where(ok[:, None], m, 0.0)), 0.0)
        z = e.sum(axis=1)
        LSE[ok, h] = (m[:, 0] + np.log(np.where(ok, z, 1.0)))[ok]
        O[ok, h, :] = (e[ok] / z[ok, None]) @ V[:, g, :]
    return O, LSE


def std_inputs(L, Hq, Hkv, D, theta, seed, scale_raw=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((L, Hq, D)) * scale_raw
    k = rng.standard_normal((L, Hkv, D)) * scale_raw
    v = rng.standard_normal((L, Hkv, D))
    pos = np.arange(L)
    return rope_complex(q, pos, theta), rope_complex(k, pos, theta), v


# --------------------------------------------------------------------------
# group size, aliasing map, in-grid invariant (Methodology section 1)
# --------------------------------------------------------------------------

def test_group_size_closed_forms():
    # the five workload shapes: ceil(L / w_pretrained)
    assert group_size(512, 128) == 4
    assert group_size(32768, 32768) == 1
    assert group_size(131072, 32768) == 4
    assert group_size(98427, 32768) == 4
    assert group_size(40001, 32768) == 2
    assert group_size(1, 32768) == 1
    assert group_size(32769, 32768) == 2
    assert group_size(131073, 32768) == 5
    assert int(alias(131071, 4)) == 32767          # last remote angle sits on w_pretrained - 1


def test_group_size_matches_real_ceiling():
    for L in range(1, 400):
        for w in (1, 2, 3, 5, 7, 16, 33, 128):
            assert group_size(L, w) == max(1, math.ceil(L / w))


@pytest.mark.parametrize("w", [1, 2, 3, 7, 16, 32, 128])
def test_remote_positions_stay_on_pretrained_grid(w):
    # every remote pair (j <= i - w0) maps to 0 <= f(j) <= f(i) <= w - 1, and G is
    # minimal: with G - 1 the last position would leave the grid.
    for L in range(1, 2049):
        G = group_size(L, w)
        f = alias(np.arange(L), G)
        assert f[0] == 0 and f[-1] <= w - 1
        assert np.all(np.diff(f) >= 0)
        if G > 1:
            assert (L - 1) // (G - 1) >= w


# --------------------------------------------------------------------------
# RoPE itself
# --------------------------------------------------------------------------

def test_inv_freq_closed_form():
    w = inv_freq(1e6, 128)
    assert w[0] == 1.0
    assert abs(w[32] - 1e6 ** -0.5) < 1e-18
    assert abs(w[-1] - 1e6 ** (-126 / 128)) < 1e-20


def test_rope_matches_complex_formulation():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, 3, 16))
    pos = rng.integers(0, 200000, size=50)
    np.testing.assert_allclose(rope_rotate(x, pos, 1e6), rope_complex(x, pos, 1e6),
                               rtol=0, atol=1e-12)


def test_rope_d2_closed_form():
    # D = 2: theta_0 = 1, so position p rotates (1, 0) to (cos p, sin p)
    for p in (0, 1, 5, 1000, 131071):
        r = rope_rotate(np.array([[[1.0, 0.0]]]), [p], 1e4)
        assert abs(r[0, 0, 0] - math.cos(p)) < 1e-12 and abs(r[0, 0, 1] - math.sin(p)) < 1e-12


def test_rope_relative_position_property():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((1, 1, 32))
    y = rng.standard_normal((1, 1, 32))
    base = float(np.sum(rope_rotate(x, [7], 1e4) * rope_rotate(y, [3], 1e4)))
    for t in (0, 11, 5000, 120000):
        s = float(np.sum(rope_rotate(x, [7 + t], 1e4) * rope_rotate(y, [3 + t], 1e4)))
        assert abs(s - base) < 1e-9


def test_correction_rotation_composes_additively():
    # R(f(x) - x) R(x) = R(f(x)) (Methodology section 2, correction rotation)
    rng = np.random.default_rng(3)
    n, D, G = 3000, 64, 4
    x = rng.standard_normal((n, 1, D))
    pos = np.arange(n) * 37 + 11
    std = rope_rotate(x, pos, 1e6)
    corrected = rope_rotate(std, alias(pos, G) - pos, 1e6)
    direct = rope_complex(x, alias(pos, G), 1e6)
    # angles reach ~1.1e5 rad, where one float64 ulp of the angle is ~1.5e-11
    np.testing.assert_allclose(corrected, direct, rtol=0, atol=1e-10)


def _tables_from_unit_vectors(n_pos, D, theta, G):
    """(cos, sin) columns read off RoPE (complex form) applied to the unit vectors e_m:
    rotating e_m by angle a puts cos a in channel m and sin a in channel m + D/2."""
    h = D // 2
    eye = np.eye(D)[:h]                                    # e_0 .. e_{h-1}
    p = np.arange(n_pos)
    out = []
    for pos in (p, p // G - p):                            # standard, correction
        r = rope_complex(np.broadcast_to(eye, (n_pos, h, D)), pos, theta)  # [n, m, D]
        out.append(r[:, np.arange(h), np.arange(h)])        # channel m of e_m's image
        out.append(r[:, np.arange(h), np.arange(h) + h])    # channel m + D/2
    return out


@pytest.mark.parametrize("D,theta,G", [(64, 1e6, 4), (128, 1e4, 3), (8, 50.0, 1)])
def test_rope_tables_match_rotated_unit_vectors(D, theta, G):
    # the table generator's reference, both column pairs, against RoPE applied to unit
    # vectors; the correction columns compose with the standard rotation to f(p)
    n = 300
    ref = rope_tables_ref(n, D, theta, G)
    for got, want in zip(ref, _tables_from_unit_vectors(n, D, theta, G)):
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    c, s, cc, sc = ref
    p = np.arange(n)
    a_f = (p // G)[:, None] * inv_freq(theta, D)[None, :]
    # R(f(p) - p) R(p) = R(f(p)): angle addition with the standard columns
    np.testing.assert_allclose(cc * c - sc * s, np.cos(a_f), atol=1e-12)
    np.testing.assert_allclose(sc * c + cc * s, np.sin(a_f), atol=1e-12)


def test_rope_tables_d2_closed_form():
    # D = 2, theta_0 = 1: the angles are the positions themselves
    c, s, cc, sc = rope_tables_ref(10, 2, 1e4, 3)
    for p in range(10):
        assert abs(c[p, 0] - math.cos(p)) < 1e-15 and abs(s[p, 0] - math.sin(p)) < 1e-15
        assert abs(cc[p, 0] - math.cos(p // 3 - p)) < 1e-15
        assert abs(sc[p, 0] - math.sin(p // 3 - p)) < 1e-15


@pytest.mark.parametrize("mistake", ["std_from_aliased", "correction_sign", "swap_cos_sin"])
def test_rope_tables_planted_mistakes_are_caught(monkeypatch, mistake):
    import oracle.bifocal_ref as ref
    orig = ref.rope_tables_ref

    def bad(n_pos, D, theta, G):
        c, s, cc, sc = orig(n_pos, D, theta, G)
        if mistake == "std_from_aliased":       # standard columns built from f(p)
            a = (np.arange(n_pos) // G)[:, None] * inv_freq(theta, D)[None, :]
            return np.cos(a), np.sin(a), cc, sc
        if mistake == "correction_sign":        # R(p - f(p)) instead of R(f(p) - p)
            return c, s, cc, -sc
        return s, c, cc, sc                     # swap_cos_sin
    monkeypatch.setattr(ref, "rope_tables_ref", bad)
    monkeypatch.setitem(globals(), "rope_tables_ref", bad)
    with pytest.raises(AssertionError):
        test_rope_tables_match_rotated_unit_vectors(64, 1e6, 4)


def test_rope_apply_ref_aliases_positions():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((40, 2, 8))
    pos = np.arange(40)
    np.testing.assert_allclose(rope_apply_ref(x, pos, 1e4, G=3),
                               rope_complex(x, pos // 3, 1e4), atol=1e-12)
    np.testing.assert_allclose(rope_apply_ref(x, pos, 1e4, G=1), rope_complex(x, pos, 1e4),
                               atol=1e-12)


# --------------------------------------------------------------------------
# bifocal attention
# --------------------------------------------------------------------------

def _to_lists(a):
    return np.asarray(a, dtype=np.float64).tolist()


@pytest.mark.parametrize("L,D,Hq,Hkv", [(12, 4, 2, 1), (12, 8, 1, 1)])
def test_oracle_matches_brute_force_exhaustive(L, D, Hq, Hkv):
    Q, K, V = std_inputs(L, Hq, Hkv, D, 50.0, seed=L * 10 + D)
    Ql, Kl, Vl = _to_lists(Q), _to_lists(K), _to_lists(V)
    for w_pre in range(1, L + 1):
        for w0 in range(1, L + 2):
            Ob, Lb = brute.brute_attention(Ql, Kl, Vl, w0, w_pre, 50.0)
            Oo, Lo = bifocal_rows(Q, K, V, np.arange(L), w0, w_pre, 50.0)
            np.testing.assert_allclose(Oo, np.array(Ob), rtol=0, atol=1e-12)
            np.testing.assert_allclose(Lo, np.array(Lb), rtol=0, atol=1e-12)


@pytest.mark.parametrize("L,w0,w_pre", [(37, 5, 10), (40, 1, 9), (33, 40, 4), (29, 7, 29)])
def test_oracle_matches_brute_force_ragged(L, w0, w_pre):
    Q, K, V = std_inputs(L, 4, 2, 8, 1e4, seed=L + w0)
    Ob, Lb = brute.brute_attention(_to_lists(Q), _to_lists(K), _to_lists(V), w0, w_pre, 1e4)
    Oo, Lo = bifocal_rows(Q, K, V, np.arange(L), w0, w_pre, 1e4)
    np.testing.assert_allclose(Oo, np.array(Ob), rtol=0, atol=1e-12)
    np.testing.assert_allclose(Lo, np.array(Lb), rtol=0, atol=1e-12)


def test_closed_form_d2_example():
    # D = 2 (angle = position in radians), raw q = raw k = (1, 0), L = 4,
    # w_pretrained = 2 -> G = 2, f = [0, 0, 1, 1], w0 = 2.  Row 3 sees
    # j = 3, 2 locally (cos 0, cos 1) and j = 1, 0 remotely at f(3) - f(j) = 1.
    L, s = 4, 1.0 / math.sqrt(2)
    raw_q = np.tile(np.array([1.0, 0.0]), (L, 1, 1))
    pos = np.arange(L)
    Q = rope_complex(raw_q, pos, 1e4)
    K = Q.copy()
    V = np.arange(L * 2, dtype=np.float64).reshape(L, 1, 2)
    O, LSE = bifocal_rows(Q, K, V, [3], w0=2, w_pretrained=2, theta=1e4)
    sc = [s * math.cos(1), s * math.cos(1), s * math.cos(1), s * 1.0]
    lse = math.log(sum(math.exp(x) for x in sc))
    assert abs(LSE[0, 0] - lse) < 1e-13
    o = [sum(math.exp(sc[j] - lse) * V[j, 0, d] for j in range(4)) for d in range(2)]
    np.testing.assert_allclose(O[0, 0], o, atol=1e-13)
    # vanilla RoPE would give cos 3, cos 2, cos 1, 1 for the same row
    O1, LSE1 = bifocal_rows(Q, K, V, [3], w0=4, w_pretrained=2, theta=1e4)
    lse1 = math.log(sum(math.exp(s * math.cos(d)) for d in (3, 2, 1, 0)))
    assert abs(LSE1[0, 0] - lse1) < 1e-13


@pytest.mark.parametrize("L,w_pre", [(64, 64), (100, 128), (96, 96)])
def test_g1_equals_vanilla_sdpa(L, w_pre):
    # L <= w_pretrained: G = 1, both branches are classic RoPE, so the result is
    # plain causal attention on the inputs as given.
    Q, K, V = std_inputs(L, 4, 2, 16, 1e6, seed=L)
    O, LSE = bifocal_rows(Q, K, V, np.arange(L), w0=7, w_pretrained=w_pre, theta=1e6)
    np.testing.assert_allclose(O, sdpa_f64(Q, K, V), rtol=0, atol=1e-12)


@pytest.mark.parametrize("L,w_pre,G", [(64, 16, 4), (90, 31, 3), (77, 77, 1)])
def test_w0_one_equals_pure_aliased_attention(L, w_pre, G):
    # w0 = 1: only the diagonal is local, and there f(i) - f(i) = 0 = i - i, so
    # every pair is effectively remote: SDPA on inputs moved to aliased positions.
    assert group_size(L, w_pre) == G
    Q, K, V = std_inputs(L, 4, 1, 16, 1e4, seed=L + 1)
    pos = np.arange(L)
    Qa = rope_complex(Q, pos // G - pos, 1e4)
    Ka = rope_complex(K, pos // G - pos, 1e4)
    O, LSE = bifocal_rows(Q, K, V, pos, w0=1, w_pretrained=w_pre, theta=1e4)
    np.testing.assert_allclose(O, sdpa_f64(Qa, Ka, V), rtol=0, atol=1e-12)


def test_w0_at_least_L_equals_vanilla():
    L = 70
    Q, K, V = std_inputs(L, 2, 1, 8, 1e4, seed=5)
    O, _ = bifocal_rows(Q, K, V, np.arange(L), w0=L, w_pretrained=10, theta=1e4)
    np.testing.assert_allclose(O, sdpa_f64(Q, K, V), rtol=0, atol=1e-12)


@pytest.mark.parametrize("L,w0,w_pre,scale_raw", [(80, 9, 20, 1.0), (128, 16, 32, 2.0),
                                                 (50, 3, 7, 0.5)])
def test_inclusion_exclusion_three_pass_merge(L, w0, w_pre, scale_raw):
    # Methodology section 2: local-window pass with base q/k (A), full causal pass
    # with remote q/k (B), local-window pass with remote q/k (C), merged with
    # LogSumExp statistics: Z = Z_B - Z_C + Z_A.
    Q, K, V = std_inputs(L, 4, 2, 16, 1e4, seed=L + w0, scale_raw=scale_raw)
    scale = 1.0 / 4.0
    G = group_size(L, w_pre)
    pos = np.arange(L)
    Qr = rope_complex(Q, pos // G - pos, 1e4)
    Kr = rope_complex(K, pos // G - pos, 1e4)
    dist = pos[:, None] - pos[None, :]
    win = (dist >= 0) & (dist < w0)
    causal = dist >= 0
    OA, LA = masked_softmax_pass(Q, K, V, win, scale)
    OB, LB = masked_softmax_pass(Qr, Kr, V, causal, scale)
    OC, LC = masked_softmax_pass(Qr, Kr, V, win, scale)
    m = np.maximum(np.maximum(LA, LB), LC)
    zA, zB, zC = np.exp(LA - m), np.exp(LB - m), np.exp(LC - m)
    Z = zB - zC + zA
    O_ie = (zB[..., None] * OB - zC[..., None] * OC + zA[..., None] * OA) / Z[..., None]
    LSE_ie = m + np.log(Z)
    O, LSE = bifocal_rows(Q, K, V, pos, w0, w_pre, 1e4, scale=scale)
    # conditioning: rows whose keys all lie in the window have Z_B == Z_C exactly
    # in exact arithmetic; compare with a tolerance relative to Z_B / Z.
    cond = np.maximum(1.0, zB / Z)
    assert np.all(np.abs(LSE - LSE_ie) <= 1e-12 * cond * 10)
    assert np.all(np.abs(O - O_ie) <= 1e-11 * cond[..., None] * 10)


# --------------------------------------------------------------------------
# variants: continuous remote positions ("interp") and window-only layers
# --------------------------------------------------------------------------

@pytest.mark.parametrize("variant", ["interp", "window"])
@pytest.mark.parametrize("L,w0,w_pre", [(13, 3, 4), (16, 1, 5), (11, 12, 3), (14, 6, 14)])
def test_variants_match_brute_force(variant, L, w0, w_pre):
    Q, K, V = std_inputs(L, 4, 2, 8, 1e4, seed=L + 3 * w0)
    Ob, Lb = brute.brute_attention(_to_lists(Q), _to_lists(K), _to_lists(V), w0, w_pre, 1e4,
                                   variant=variant)
    Oo, Lo = bifocal_rows(Q, K, V, np.arange(L), w0, w_pre, 1e4, variant=variant)
    np.testing.assert_allclose(Oo, np.array(Ob), rtol=0, atol=1e-12)
    np.testing.assert_allclose(Lo, np.array(Lb), rtol=0, atol=1e-12)


def test_interp_with_g1_is_the_method():
    # G = 1: x / G = floor(x / G) = x, both variants are vanilla RoPE attention
    Q, K, V = std_inputs(60, 4, 2, 16, 1e4, seed=61)
    O1, L1 = bifocal_rows(Q, K, V, np.arange(60), 7, 64, 1e4)
    O2, L2 = bifocal_rows(Q, K, V, np.arange(60), 7, 64, 1e4, variant="interp")
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    np.testing.assert_allclose(O2, sdpa_f64(Q, K, V), rtol=0, atol=1e-12)


@pytest.mark.parametrize("L,w_pre,G", [(64, 16, 4), (90, 31, 3)])
def test_interp_w0_one_equals_attention_at_scaled_positions(L, w_pre, G):
    # w0 = 1: every off-diagonal pair is remote and scored at the real positions x / G;
    # on the diagonal i/G - i/G = 0 = i - i.  So this is SDPA on inputs moved from x to
    # x / G (rotation by x/G - x).
    assert group_size(L, w_pre) == G
    Q, K, V = std_inputs(L, 4, 1, 16, 1e4, seed=L + 5)
    pos = np.arange(L)
    Qs = rope_complex(Q, pos / G - pos, 1e4)
    Ks = rope_complex(K, pos / G - pos, 1e4)
    O, _ = bifocal_rows(Q, K, V, pos, w0=1, w_pretrained=w_pre, theta=1e4, variant="interp")
    np.testing.assert_allclose(O, sdpa_f64(Qs, Ks, V), rtol=0, atol=1e-12)


def test_interp_differs_from_aliasing_when_g_above_1():
    # a planted-mistake guard: with G = 4 the two remote maps disagree
    Q, K, V = std_inputs(48, 2, 1, 8, 1e4, seed=7)
    O1, _ = bifocal_rows(Q, K, V, np.arange(48), 4, 12, 1e4)
    O2, _ = bifocal_rows(Q, K, V, np.arange(48), 4, 12, 1e4, variant="interp")
    assert np.max(np.abs(O1 - O2)) > 1e-3


@pytest.mark.parametrize("L,w0", [(50, 9), (64, 1), (40, 40), (33, 100)])
def test_window_equals_banded_sdpa(L, w0):
    # window-only layer: SDPA with a banded causal mask (0 <= i - j < w0) on the inputs as
    # given; w0 >= L is plain causal attention, w0 = 1 returns V_i
    Q, K, V = std_inputs(L, 4, 2, 16, 1e4, seed=L * w0)
    O, LSE = bifocal_rows(Q, K, V, np.arange(L), w0, 8, 1e4, variant="window")
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    band = torch.from_numpy((i - j >= 0) & (i - j < w0))
    q = torch.from_numpy(np.ascontiguousarray(Q.transpose(1, 0, 2)))
    k = torch.from_numpy(np.ascontiguousarray(np.repeat(K, 2, axis=1).transpose(1, 0, 2)))
    v = torch.from_numpy(np.ascontiguousarray(np.repeat(V, 2, axis=1).transpose(1, 0, 2)))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=band)
    np.testing.assert_allclose(O, ref.numpy().transpose(1, 0, 2), rtol=0, atol=1e-12)
    if w0 == 1:
        np.testing.assert_allclose(O, np.repeat(V, 2, axis=1), rtol=0, atol=1e-14)
    if w0 >= L:
        np.testing.assert_allclose(O, sdpa_f64(Q, K, V), rtol=0, atol=1e-12)


def test_variant_decode_equals_prefill_row():
    Q, K, V = std_inputs(120, 4, 2, 16, 1e4, seed=12)
    for variant in ("interp", "window"):
        for pos in (0, 17, 63, 119):
            Od, Ld = bifocal_decode_ref(Q[pos], K, V, pos, w0=10, w_pretrained=30, theta=1e4,
                                        variant=variant)
            Op, Lp = bifocal_rows(Q[:pos + 1], K[:pos + 1], V[:pos + 1], [pos], 10, 30, 1e4,
                                  variant=variant)
            np.testing.assert_allclose(Od, Op[0], atol=1e-13)
            np.testing.assert_allclose(Ld, Lp[0], atol=1e-13)


def test_decode_equals_prefill_row():
    L = 150
    Q, K, V = std_inputs(L, 4, 2, 16, 1e4, seed=9)
    for pos in (0, 5, 63, 64, 99, 149):
        Od, Ld = bifocal_decode_ref(Q[pos], K, V, pos, w0=10, w_pretrained=40, theta=1e4)
        # a prefill of length pos + 1 has the same G as decode at pos
        Op, Lp = bifocal_rows(Q[:pos + 1], K[:pos + 1], V[:pos + 1], [pos], 10, 40, 1e4)
        np.testing.assert_allclose(Od, Op[0], atol=1e-13)
        np.testing.assert_allclose(Ld, Lp[0], atol=1e-13)


def test_prefill_varlen_matches_per_sequence():
    lens = [30, 1, 47]
    cu = np.concatenate([[0], np.cumsum(lens)])
    Q, K, V = std_inputs(sum(lens), 2, 1, 8, 1e4, seed=11)
    res = bifocal_prefill_ref(Q, K, V, cu, w0=4, w_pretrained=12, theta=1e4)
    for b, (rows, O, LSE) in enumerate(res):
        s, e = cu[b], cu[b + 1]
        Ob, Lb = brute.brute_attention(_to_lists(Q[s:e]), _to_lists(K[s:e]), _to_lists(V[s:e]),
                                       4, 12, 1e4)
        np.testing.assert_allclose(O, np.array(Ob), atol=1e-12)
        np.testing.assert_allclose(LSE, np.array(Lb), atol=1e-12)


def test_local_scores_depend_only_on_distance():
    # shifting every absolute position by t leaves a pure-local (w0 >= L) result unchanged
    rng = np.random.default_rng(12)
    L = 40
    q = rng.standard_normal((L, 2, 8))
    k = rng.standard_normal((L, 1, 8))
    v = rng.standard_normal((L, 1, 8))
    outs = []
    for t in (0, 1000, 77777):
        Q = rope_complex(q, np.arange(L) + t, 1e4)
        K = rope_complex(k, np.arange(L) + t, 1e4)
        # feed as a sequence whose own positions are 0..L-1: undo the shift on input
        Q0 = rope_complex(Q, -t * np.ones(L), 1e4)
        K0 = rope_complex(K, -t * np.ones(L), 1e4)
        outs.append(bifocal_rows(Q0, K0, v, np.arange(L), L, L, 1e4)[0])
    np.testing.assert_allclose(outs[0], outs[1], atol=1e-10)
    np.testing.assert_allclose(outs[0], outs[2], atol=1e-10)


# --------------------------------------------------------------------------
# planted mistakes: each must be caught by one of the pins above
# --------------------------------------------------------------------------

def _pins_pass():
    try:
        test_oracle_matches_brute_force_ragged(37, 5, 10)
        test_w0_one_equals_pure_aliased_attention(64, 16, 4)
        test_g1_equals_vanilla_sdpa(64, 64)
        test_closed_form_d2_example()
        test_inclusion_exclusion_three_pass_merge(80, 9, 20, 1.0)
    except AssertionError:
        return False
    return True


def _rotate_flipped(x, pos, theta):
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq(theta, D)[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = x[..., : D // 2], x[..., D // 2:]
    return np.concatenate([x1 * c + x2 * s, x2 * c - x1 * s], axis=-1)


def _rotate_interleaved(x, pos, theta):
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq(theta, D)[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    out[..., 1::2] = x[..., 1::2] * c + x[..., 0::2] * s
    return out


@pytest.mark.parametrize("mutation", ["ceil_to_floor", "alias_off_by_one", "sin_sign",
                                      "pairing_interleaved", "window_off_by_one",
                                      "gqa_index", "query_offset"])
def test_planted_mistakes_are_caught(monkeypatch, mutation):
    """Plant one plausible mistake in the oracle and check that a pin fails."""
    import oracle.bifocal_ref as ref
    assert _pins_pass()
    if mutation == "ceil_to_floor":
        monkeypatch.setattr(ref, "group_size", lambda L, w: max(1, L // w))
    elif mutation == "alias_off_by_one":
        monkeypatch.setattr(ref, "alias", lambda x, G: (np.asarray(x, dtype=np.int64) + 1) // G)
    elif mutation == "sin_sign":
        monkeypatch.setattr(ref, "rope_rotate", _rotate_flipped)
    elif mutation == "pairing_interleaved":
        monkeypatch.setattr(ref, "rope_rotate", _rotate_interleaved)
    else:
        orig = ref.bifocal_rows
        if mutation == "window_off_by_one":
            def bad(Q, K, V, rows, w0, *a, **k):
                return orig(Q, K, V, rows, w0 + 1, *a, **k)
        elif mutation == "gqa_index":
            def bad(Q, K, V, *a, **k):
                return orig(Q, np.ascontiguousarray(K[:, ::-1]),
                            np.ascontiguousarray(V[:, ::-1]), *a, **k)
        else:  # query_offset
            def bad(*a, **k):
                return orig(*a, q_offset=1, **k)
        # the pins call bifocal_rows through this module's global name
        monkeypatch.setitem(globals(), "bifocal_rows", bad)
    assert not _pins_pass(), f"planted mistake {mutation!r} was not caught by any pin"
