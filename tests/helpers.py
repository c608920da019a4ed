"""Shared test helpers: inputs built on the CPU with the oracle's float64 RoPE, and
error metrics.  Nothing here comes from the HIP path."""
from __future__ import annotations

import numpy as np

import workloads
from oracle.bifocal_ref import alias, group_size, rope_rotate

BF16_TOL = dict(max_abs=2e-2, mean_abs=2e-3, lse_abs=5e-3)
F32_TOL = dict(max_abs=1e-4)


def std_rope_local(x_raw: np.ndarray, cu_seqlens, theta: float, chunk: int = 8192) -> np.ndarray:
    """Standard RoPE at each sequence's local positions, float64 math, float32 result."""
    out = np.empty(x_raw.shape, dtype=np.float32)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        for c0 in range(s, e, chunk):
            c1 = min(e, c0 + chunk)
            out[c0:c1] = rope_rotate(x_raw[c0:c1], np.arange(c0 - s, c1 - s), theta)
    return out


def to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Values as the kernel dtype stores them (bf16 rounding to nearest even), as float32."""
    return workloads.round_to_bf16(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


def prefill_inputs(w: workloads.Workload, seqlens=None, outliers=None):
    """Q_std, K_std, V (float32 arrays holding dtype-exact values) and cu_seqlens."""
    if seqlens is not None or outliers is not None:
        import dataclasses
        w = dataclasses.replace(w, seqlens=tuple(seqlens) if seqlens is not None else w.seqlens,
                                outliers=w.outliers if outliers is None else outliers)
    cu = w.cu_seqlens
    q, k, v = workloads.raw_prefill_inputs(w)
    Q = to_dtype(std_rope_local(q, cu, w.theta), w.dtype)
    K = to_dtype(std_rope_local(k, cu, w.theta), w.dtype)
    V = to_dtype(v, w.dtype)
    return Q, K, V, cu


def decode_inputs(w: workloads.Workload, S=None):
    """K/V caches [S,Hkv,D] with standard RoPE at absolute positions, and the raw queries
    of the decode steps (RoPE'd per step by the caller with std_query)."""
    q, k, v = workloads.raw_decode_inputs(w, S=S)
    S = k.shape[0]
    Kc = to_dtype(std_rope_local(k, [0, S], w.theta), w.dtype)
    Vc = to_dtype(v, w.dtype)
    return q, Kc, Vc


def std_query(q_raw_step: np.ndarray, pos: int, theta: float, dtype: str) -> np.ndarray:
    return to_dtype(rope_rotate(q_raw_step[None], [pos], theta)[0].astype(np.float32), dtype)


def errors(o_gpu, o_ref, lse_gpu=None, lse_ref=None):
    d = np.abs(np.asarray(o_gpu, dtype=np.float64) - np.asarray(o_ref, dtype=np.float64))
    out = dict(max_abs=float(d.max()), mean_abs=float(d.mean()))
    if lse_gpu is not None:
        out["lse_abs"] = float(np.max(np.abs(np.asarray(lse_gpu, np.float64) - lse_ref)))
    return out


def within(err: dict, tol: dict) -> bool:
    return all(err[k] <= v for k, v in tol.items() if k in err)


def ie_conditioning(Q_std, K_std, rows, w0: int, w_pretrained: int, theta: float,
                    scale=None, key_block: int = 16384) -> np.ndarray:
    """Conditioning of the three-pass inclusion-exclusion merge at the given rows of one
    sequence: max(1, Z_B / Z) per (row, query head), with Z_B the remote-score sum over
    all causal keys and Z the bifocal sum (Z = Z_B - Z_C + Z_A).  Errors of the passes
    (relative to their own sums) reach the merged result multiplied by this factor.
    Computed in float64 from the oracle's rotations; returns [len(rows), Hq]."""
    rows = np.asarray(rows, dtype=np.int64)
    L, Hq, D = Q_std.shape
    Hkv = K_std.shape[1]
    rep = Hq // Hkv
    sc = 1.0 / np.sqrt(D) if scale is None else scale
    G = group_size(L, w_pretrained)
    n_all = alias(np.arange(L), G) - np.arange(L)
    Qs = np.asarray(Q_std[rows], dtype=np.float64)
    Qr = rope_rotate(Qs, n_all[rows], theta)
    out = np.empty((len(rows), Hq))
    for g in range(Hkv):
        qs = Qs[:, g * rep:(g + 1) * rep].reshape(-1, D)
        qr = Qr[:, g * rep:(g + 1) * rep].reshape(-1, D)
        ri = np.repeat(rows, rep)
        lse = {k: np.full(len(ri), -np.inf) for k in "ABCZ"}
        for j0 in range(0, L, key_block):
            j1 = min(L, j0 + key_block)
            ks = np.asarray(K_std[j0:j1, g], dtype=np.float64)
            kr = rope_rotate(np.asarray(K_std[j0:j1, g:g + 1]), n_all[j0:j1], theta)[:, 0]
            s_loc = sc * qs @ ks.T
            s_rem = sc * qr @ kr.T
            dist = ri[:, None] - np.arange(j0, j1)[None, :]
            causal = dist >= 0
            win = causal & (dist < w0)
            for k, s_, m_ in (("A", s_loc, win), ("B", s_rem, causal), ("C", s_rem, win),
                              ("Z", np.where(win, s_loc, s_rem), causal)):
                x = np.where(m_, s_, -np.inf)
                lse[k] = np.logaddexp(lse[k], np.logaddexp.reduce(x, axis=1))
        out[:, g * rep:(g + 1) * rep] = np.maximum(1.0, np.exp(lse["B"] - lse["Z"])).reshape(
            len(rows), rep)
    return out
