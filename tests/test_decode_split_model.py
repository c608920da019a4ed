"""The split-KV decode's partial/merge arithmetic, on the CPU: keys in 16-key blocks dealt
round-robin to the splits, each split keeping a base-2 running max (raised only when it
grows by more than 8), a row sum and an output accumulator; four splits merged per
workgroup, then the workgroups merged by their maxima (the two levels of the matrix-core
decode).  The merged result must not depend on the split count: for 4 to 512 splits it
must equal the float64 softmax of the same scores to float rounding.  Scores come from
the oracle's definition (remote pairs at the aliased positions)."""
import math

import numpy as np
import pytest

import workloads as W
from helpers import decode_inputs, std_query
from oracle.bifocal_ref import alias, bifocal_decode_ref, group_size, rope_rotate

LAZY = 8.0


def _scores(q, K, pos, w0, w_pre, theta):
    """Scaled scores of one decode row, float64 (the oracle's per-pair definition)."""
    L = pos + 1
    G = group_size(L, w_pre)
    j = np.arange(L)
    k_raw = rope_rotate(K[:L], -j, theta)
    q_raw = rope_rotate(q[None], [-pos], theta)[0]
    k_rem = rope_rotate(k_raw, alias(j, G), theta)
    q_rem = rope_rotate(q_raw[None], [pos // G], theta)[0]
    rep = q.shape[0] // K.shape[1]
    D = q.shape[-1]
    s_loc = np.einsum("hd,jhd->hj", q, np.repeat(np.asarray(K[:L], np.float64), rep, axis=1))
    s_rem = np.einsum("hd,jhd->hj", q_rem, np.repeat(k_rem, rep, axis=1))
    local = (pos - j) < w0
    return np.where(local[None, :], s_loc, s_rem) / math.sqrt(D)


def _split_merge(s2, V, nsplit, block=16, waves=4):
    """s2: [H, L] scores in the base-2 domain; V: [L, H, D].  Returns (O, LSE)."""
    H, L = s2.shape
    nblk = (L + block - 1) // block
    parts = []
    for w in range(nsplit):
        m = np.full(H, -np.inf)
        l = np.zeros(H)
        acc = np.zeros((H, V.shape[-1]))
        for b in range(w, nblk, nsplit):
            sl = slice(b * block, min(L, (b + 1) * block))
            bm = s2[:, sl].max(axis=1)
            cand = np.maximum(m, bm)
            new = np.where(cand > m + LAZY, cand, m)
            f = np.exp2(np.where(np.isfinite(m), m - new, -np.inf))
            l, acc, m = l * f, acc * f[:, None], new
            p = np.exp2(s2[:, sl] - m[:, None])
            l = l + p.sum(axis=1)
            acc = acc + np.einsum("hj,jhd->hd", p, V[sl])
        parts.append((m, l, acc))
    # workgroups of `waves` splits, then across workgroups
    def merge(ps):
        mx = np.max([p[0] for p in ps], axis=0)
        with np.errstate(invalid="ignore"):  # splits without keys: m = -inf
            wts = [np.where(np.isfinite(p[0]), np.exp2(p[0] - mx), 0.0) for p in ps]
        return (mx, sum(w * p[1] for w, p in zip(wts, ps)),
                sum(w[:, None] * p[2] for w, p in zip(wts, ps)))
    groups = [merge(parts[i:i + waves]) for i in range(0, nsplit, waves)]
    m, l, acc = merge(groups)
    return acc / l[:, None], (m + np.log2(l)) * math.log(2.0)


@pytest.mark.parametrize("pos", [100, 2999])
def test_decode_split_count_does_not_change_the_result(pos):
    w = W.Workload("splitmodel", "decode", "f32", Hq=8, Hkv=2, D=64, w0=100, w_pretrained=700,
                   theta=1e6, cache_len=3000, decode_steps=1, outliers=4, seed=21)
    q_raw, Kc, Vc = decode_inputs(w)
    q = std_query(q_raw[0], pos, w.theta, "f32").astype(np.float64)
    s = _scores(q, Kc, pos, w.w0, w.w_pretrained, w.theta)
    Or, Lr = bifocal_decode_ref(q, Kc, Vc, pos, w.w0, w.w_pretrained, w.theta)
    np.testing.assert_allclose(np.log(np.exp(s - s.max(1, keepdims=True)).sum(1)) + s.max(1), Lr,
                               atol=1e-10)  # the scores are the oracle's
    V = np.asarray(Vc[:pos + 1], np.float64).repeat(4, axis=1)
    for nsplit in (4, 8, 36, 128, 512):
        O, L = _split_merge(s / math.log(2.0), V, nsplit)
        np.testing.assert_allclose(O, Or, atol=1e-10)
        np.testing.assert_allclose(L, Lr, atol=1e-10)
