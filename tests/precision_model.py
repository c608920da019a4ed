"""CPU model of the bf16 prefill kernel's rounding steps (test infrastructure).

It replays, for chosen query rows of one sequence, every place where the matrix-core
prefill rounds a value, and leaves out everything that is exact to float64 accuracy:

* the correction rotation R(f(x) - x) applied in float32 with float32 (cos, sin) of the
  integer offset n = x - f(x) (the position table: float64 angle, one rounding), as a
  fused multiply-add after one float32 product;
* the remote operands rounded to fp16 (round to nearest even); for a set of RoPE pairs
  chosen per KV head from the largest max_h |q_h|^2 * max |k|^2 over the sequence
  (ties to the lower pair), the fp16 remainder lo = fp16(y - hi) on both sides, and the
  score terms hi*lo + lo*hi of those channels;
* local scores from the bf16 input bytes as they are (exact products);
* the base-2 online softmax over 32-key tiles in the kernel's visiting order (remote
  pass over every tile holding remote keys, then the local pass), with the lazy running
  max (raised only when a tile's max exceeds it by more than 8), float32 arguments of
  the exponentials, the probabilities rounded to the PV operand type and the row sum
  taken over the rounded probabilities;
* the output rounded to bf16.

Scores and sums accumulate in float64 here (the matrix cores accumulate in float32, a
far smaller error than the 11-bit operands).  The model shares nothing with the HIP
sources; it follows the arithmetic the kernel's comments describe, so that a change of
the precision scheme can be weighed on the CPU before it is built.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

from oracle.bifocal_ref import group_size, inv_freq
from workloads import round_to_bf16

BK = 32          # keys per tile
LAZY = 8.0       # growth of the running max (log2 units) tolerated before a rescale


@dataclasses.dataclass(frozen=True)
class Scheme:
    """Precision choices of the remote scores and the probabilities.

    pairs: RoPE pairs per KV head whose fp16 remainders enter the remote scores on both
      sides (hi*lo + lo*hi), chosen from max_h |q_h|^2 * max |k|^2 over the group.
    q_pairs: pairs per query head (chosen from that head's max |q_h|^2 * max |k|^2) whose
      query remainder enters against the key's fp16 value (lo*hi only).
    k_only: the per-KV-head pairs give only the key remainder against the query's fp16
      value (hi*lo), their query side is left to q_pairs.
    p_type: "bf16" or "f16", the type of P in the PV product and in the row sum.
    """
    pairs: int = 4
    p_type: str = "bf16"
    q_pairs: int = 0
    k_only: bool = False     # the per-KV-head pairs correct the key side only (lo of k)
    kv_sum: bool = False     # per-KV-head pairs by sum_h |q_h|^2 * |k|^2 instead of max_h

def _f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def _f16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float16).astype(np.float64)


def _bf16(x):
    return round_to_bf16(np.asarray(x, dtype=np.float32)).astype(np.float64)


def table_rows(n, D: int, theta: float):
    """(cos, sin) of n * theta_m, float64 angle rounded once to float32: [len(n), D/2]."""
    a = np.asarray(n, dtype=np.float64)[:, None] * inv_freq(theta, D)[None, :]
    return _f32(np.cos(a)), _f32(np.sin(a))


def rotate_remote(x, n, theta: float):
    """R(-n) x in float32 as the kernel does it: y1 = fma(x1, c, x2 s), y2 = fma(x2, c, -x1 s).
    x: [N, H, D] float32 values; n: [N] integer offsets.  Returns float64 [N, H, D]."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    c, s = table_rows(n, D, theta)
    c, s = c[:, None, :], s[:, None, :]
    x1, x2 = x[..., :D // 2], x[..., D // 2:]
    y1 = _f32(x1 * c + _f32(x2 * s))
    y2 = _f32(x2 * c - _f32(x1 * s))
    return np.concatenate([y1, y2], axis=-1)


def pair_bounds(Q, K):
    """max over tokens of each RoPE pair's squared norm, float32: ([Hq, D/2], [Hkv, D/2])."""
    Q = np.asarray(Q, dtype=np.float32)
    K = np.asarray(K, dtype=np.float32)
    h = Q.shape[-1] // 2
    mq = (Q[..., :h] * Q[..., :h] + Q[..., h:] * Q[..., h:]).max(axis=0)
    mk = (K[..., :h] * K[..., :h] + K[..., h:] * K[..., h:]).max(axis=0)
    return mq, mk


def _top(bound, n: int, exclude=()):
    order = sorted((m for m in range(len(bound)) if m not in exclude),
                   key=lambda m: (-float(bound[m]), m))
    return order[:n]


def select_pairs(Q, K, npairs: int, by_sum: bool = False):
    """Per KV head, the npairs RoPE pairs with the largest max_h |q_h|^2 * max |k|^2, or
    with by_sum the largest sum_h max |q_h|^2 * max |k|^2 (pair squared norms in float32
    over all tokens of the call), ties to the lower pair.  Returns [Hkv, npairs]."""
    mq, mk = pair_bounds(Q, K)
    Hq, Hkv = mq.shape[0], mk.shape[0]
    rep = Hq // Hkv
    out = np.zeros((Hkv, npairs), dtype=np.int64)
    for g in range(Hkv):
        qq = mq[g * rep:(g + 1) * rep]
        out[g] = _top((qq.sum(axis=0) if by_sum else qq.max(axis=0)) * mk[g], npairs)
    return out


def select_query_pairs(Q, K, kv_pairs, nq: int, exclude_kv: bool = True):
    """Per query head, up to nq pairs with the largest max |q_h|^2 * max |k|^2, not among
    its KV head's kv_pairs (unless exclude_kv is false) and not taken by a lower query
    head of the same group (heads in order; a pair sits in one head's set only).
    Returns a list of Hq lists."""
    mq, mk = pair_bounds(Q, K)
    Hq, Hkv = mq.shape[0], mk.shape[0]
    rep = Hq // Hkv
    out = []
    for g in range(Hkv):
        taken = set(int(m) for m in kv_pairs[g]) if exclude_kv else set()
        for r in range(rep):
            mine = _top(mq[g * rep + r] * mk[g], nq, exclude=taken)
            taken.update(mine)
            out.append(mine)
    return out


def _split_operands(y, sel_channels):
    """fp16 hi of every channel, and the fp16 remainder of the selected channels (zero
    elsewhere).  y: [..., D]; sel_channels: [D] bool."""
    hi = _f16(y)
    lo = np.where(sel_channels, _f16(y - hi), 0.0)
    return hi, lo


def _online_softmax(s_rem, s_loc, remote, local, Vg, c2, p_round, nkt):
    """The kernel's online softmax over the virtual tiles (remote pass over tiles 0..nkt-1,
    then the local pass), vectorised: the lazy running max is a scan over the tile maxima,
    and each tile's rounded probabilities are rescaled to the final max afterwards (the
    kernel's running rescale, up to float32 rounding of the factors).  Returns the
    unnormalised output [R, D], the row sum [R] and the final max [R]."""
    R = s_rem.shape[0]
    st = np.concatenate([np.where(remote, s_rem, -np.inf).reshape(R, nkt, BK),
                         np.where(local, s_loc, -np.inf).reshape(R, nkt, BK)], axis=1)
    valid = np.concatenate([remote.reshape(R, nkt, BK), local.reshape(R, nkt, BK)], axis=1)
    mxc = _f32(st.max(axis=2) * c2)                      # [R, 2 nkt]; -inf on empty tiles
    m = np.full(R, -1e30)
    m_t = np.empty((R, 2 * nkt))
    for t in range(2 * nkt):
        cand = np.maximum(m, mxc[:, t])
        m = np.where(cand > m + LAZY, cand, m)
        m_t[:, t] = m
    with np.errstate(invalid="ignore"):
        p = np.where(valid, _f32(np.exp2(_f32(st * c2 - m_t[:, :, None]))), 0.0)
    pr = p_round(p) * np.exp2(m_t - m[:, None])[:, :, None]  # to the final max
    l = pr.sum(axis=(1, 2))
    V2 = np.concatenate([Vg, Vg], axis=0)                  # keys of both passes
    acc = pr.reshape(R, 2 * nkt * BK) @ V2
    return acc, l, m


def emulate_rows(Q, K, V, rows, w0: int, w_pretrained: int, theta: float, scheme: Scheme,
                 pairs=None, q_pairs=None, scale=None, row_block: int = 64):
    """O [R, Hq, D] (bf16 values) and LSE [R, Hq] of the kernel model at the given query
    rows of one sequence (Q, K, V: [L, H, D] float32 arrays of bf16 values, standard RoPE
    at positions 0 .. L-1).  pairs: [Hkv, n] selected pairs (default: select_pairs over
    this sequence); q_pairs: [Hq, n] query-side pairs (default: select_query_pairs)."""
    Q = np.asarray(Q, dtype=np.float32)
    K = np.asarray(K, dtype=np.float32)
    V = np.asarray(V, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    L, Hq, D = Q.shape
    Hkv = K.shape[1]
    rep = Hq // Hkv
    h = D // 2
    G = group_size(L, w_pretrained)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    c2 = float(np.float32(scale * 1.4426950408889634))
    if pairs is None:
        pairs = (select_pairs(Q, K, scheme.pairs, by_sum=scheme.kv_sum) if scheme.pairs
                 else np.zeros((Hkv, 0), int))
    if q_pairs is None:
        q_pairs = (select_query_pairs(Q, K, pairs, scheme.q_pairs,
                                      exclude_kv=not scheme.k_only) if scheme.q_pairs
                   else [[] for _ in range(Hq)])
    p_round = _bf16 if scheme.p_type == "bf16" else _f16
    R = len(rows)
    O = np.zeros((R, Hq, D))
    LSE = np.zeros((R, Hq))
    order = np.argsort(rows)
    for b0 in range(0, R, row_block):
        idx = order[b0:b0 + row_block]
        rb = rows[idx]
        jmax = int(rb.max()) + 1
        nkt = (jmax + BK - 1) // BK
        J = nkt * BK
        pos = np.arange(J)
        Kp = np.zeros((J, Hkv, D), dtype=np.float32)
        Kp[:jmax] = K[:jmax]
        Vp = np.zeros((J, Hkv, D))
        Vp[:jmax] = V[:jmax]
        k_rem = rotate_remote(Kp, pos - pos // G, theta)
        q_rem = rotate_remote(Q[rb], rb - rb // G, theta)
        dist = rb[:, None] - pos[None, :]
        causal = dist >= 0
        local = causal & (dist < w0)
        remote = causal & ~local
        for g in range(Hkv):
            selc = np.zeros(D, dtype=bool)
            for m in pairs[g]:
                selc[m] = selc[m + h] = True
            kh, kl = _split_operands(k_rem[:, g, :], selc)
            kstd = Kp[:, g, :].astype(np.float64)
            for r in range(rep):
                hq = g * rep + r
                selq = np.zeros(D, dtype=bool) if scheme.k_only else selc.copy()
                for m in q_pairs[hq]:
                    selq[m] = selq[m + h] = True
                qh, ql = _split_operands(q_rem[:, hq, :], selq)
                s_rem = _f32(qh @ kh.T + qh @ kl.T + ql @ kh.T)
                s_loc = _f32(Q[rb, hq, :].astype(np.float64) @ kstd.T)
                acc, l, m = _online_softmax(s_rem, s_loc, remote, local, Vp[:, g, :], c2,
                                            p_round, nkt)
                O[idx, hq, :] = _bf16(acc / l[:, None])
                LSE[idx, hq] = (m + np.log2(l)) * math.log(2.0)
    return O, LSE
