"""CPU oracle for Dynamic Bifocal RoPE attention (Jet-Long) -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this module.  The product path (the HIP library and its
Python binding) never calls it, and this module imports nothing from the
product path.

What it computes is the plain definition of the method, in float64:

* Group size and aliasing map (technical summary on gist.science,
  "Methodology" section 1 "Dynamic Bifocal RoPE", the group-size formula and
  the floor-division map): G = max(1, ceil(L / w_pretrained)) from the current
  sequence length L, and f(x) = floor(x / G).
* Local window (same section, first bullet): a key j with i - j < w0 is scored
  with classic RoPE at the true positions i and j.
* Remote window (same section, second bullet): every other causal key is
  scored with RoPE at the aliased positions f(i) and f(j) (discrete position
  aliasing, no frequency interpolation).
* One softmax over all causal keys of a query with those per-pair scores.  The
  pages reach this with three FlashAttention passes merged by inclusion-
  exclusion and LogSumExp statistics ("Methodology" section 2, "Inclusion-
  exclusion attention merge"); the merged result is exactly per-pair routed
  attention, which is what is written here.  The three-pass form is checked
  against this one in the tests.
* Inputs follow the pages' cache convention ("Methodology" section 2,
  "On-the-fly correction rotation"): queries and keys arrive with standard
  RoPE at their exact absolute positions.  The raw vectors are recovered here
  by rotating back by the absolute position, then re-rotated to whichever
  position the pair's branch uses.

Readings taken where the pages are silent (each one is a parameter or a
documented constant here):

* RoPE pairing is rotate-half: channel m pairs with m + D/2, frequency
  theta_m = theta ** (-2 m / D), angle p * theta_m, all in float64.
* The window is sliding: local iff 0 <= i - j <= w0 - 1 (w0 keys including the
  diagonal).
* The remote query uses the same map as the keys (query offset 0): the query
  sits at f(i).  ``q_offset`` exists to show the alternative; default 0.
* The L that sets G is the whole sequence's length for prefill (every row of a
  sequence shares one G) and pos + 1 for decode.
* The softmax scale defaults to 1/sqrt(D); LSE is the natural log of the sum of
  exp(scaled scores).

Variants (``variant`` argument; the default is the method itself):

* ``"interp"``: the remote branch uses the continuous positions x / G instead of
  floor(x / G): frequency interpolation in the style the pages' ablation compares
  against ("aliasing vs interpolation", in the experimental results).  Everything
  else (window, softmax) is unchanged.
* ``"window"``: only the local window is attended (0 <= i - j < w0, classic RoPE),
  the shape of the sliding-window layers of hybrid models the pages mention
  (Jet-Nemotron); the remote pairs are dropped rather than re-scored.

Parity pins (tests/test_oracle.py): brute force with explicit rotation
matrices on tiny inputs; the three-pass inclusion-exclusion identity; G = 1
equals vanilla causal RoPE attention (torch SDPA, float64); w0 = 1 equals pure
aliased attention (torch SDPA on aliased rotations); every remote angle stays
on the pretrained grid; rotations compose additively; RoPE against a
complex-number formulation; decode equals the last prefill row; the table reference
(``rope_tables_ref``, both column pairs) against RoPE applied to unit vectors, with the
correction columns composing with the standard ones to the aliased angle.

Parity unpinned where the pages fix nothing: they print no worked numeric example,
so the readings above (rotate-half pairing, the sliding window, query offset 0) are
checked for being computed as stated, not for being the pages' intent.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "group_size", "alias", "inv_freq", "rope_rotate", "rope_apply_ref",
    "bifocal_rows", "bifocal_prefill_ref", "bifocal_decode_ref", "rope_tables_ref",
]


# ---------------------------------------------------------------------------
# Positions: group size and aliasing (Methodology section 1)
# ---------------------------------------------------------------------------

def group_size(L: int, w_pretrained: int) -> int:
    """G = max(1, ceil(L / w_pretrained)), in integer arithmetic."""
    if w_pretrained < 1:
        raise ValueError("w_pretrained must be >= 1")
    return max(1, (int(L) + int(w_pretrained) - 1) // int(w_pretrained))


def alias(x, G: int):
    """f(x) = floor(x / G) for non-negative integer positions."""
    return np.asarray(x, dtype=np.int64) // int(G)


# ---------------------------------------------------------------------------
# RoPE in float64
# ---------------------------------------------------------------------------

def inv_freq(theta: float, D: int) -> np.ndarray:
    """theta_m = theta ** (-2m / D), m = 0 .. D/2 - 1 (float64)."""
    m = np.arange(D // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * m / np.float64(D))


def rope_rotate(x: np.ndarray, pos, theta: float) -> np.ndarray:
    """Rotate each pair (x_m, x_{m+D/2}) of ``x`` by the angle pos * theta_m.

    x: [T, H, D] (any float dtype, computed in float64); pos: [T] positions
    (may be negative or fractional: the rotation by -p undoes the rotation by p).
    Returns float64.
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq(theta, D)[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1 = x[..., : D // 2]
    x2 = x[..., D // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_apply_ref(x: np.ndarray, pos, theta: float, G: int = 1) -> np.ndarray:
    """What ``rope_apply`` computes: x <- R(floor(p / G)) x (G = 1: standard RoPE)."""
    return rope_rotate(x, alias(pos, G), theta)


def rope_tables_ref(n_pos: int, D: int, theta: float, G: int):
    """Reference cos/sin of the standard angle p*theta_m and of the correction
    angle (f(p) - p)*theta_m for p in [0, n_pos); float64, [n_pos, D/2] each.

    The correction rotation R(f(p) - p) maps a standard-RoPE vector at p to the
    aliased position f(p), because RoPE rotations compose additively
    (Methodology section 2, "On-the-fly correction rotation")."""
    p = np.arange(n_pos, dtype=np.float64)
    f = alias(np.arange(n_pos), G).astype(np.float64)
    w = inv_freq(theta, D)
    a_std = p[:, None] * w[None, :]
    a_cor = (f - p)[:, None] * w[None, :]
    return np.cos(a_std), np.sin(a_std), np.cos(a_cor), np.sin(a_cor)


# ---------------------------------------------------------------------------
# Bifocal attention: per-pair routed softmax (Methodology sections 1 and 2)
# ---------------------------------------------------------------------------

VARIANTS = ("bifocal", "interp", "window")


def _remote_positions(x, G: int, variant: str):
    """Positions of the remote branch: floor(x / G) (the method) or x / G ("interp")."""
    x = np.asarray(x, dtype=np.int64)
    if variant == "interp":
        return x.astype(np.float64) / G
    return alias(x, G)


def bifocal_rows(Q_std: np.ndarray, K_std: np.ndarray, V: np.ndarray, rows, w0: int,
                 w_pretrained: int, theta: float, scale: Optional[float] = None,
                 q_offset: int = 0, row_block: int = 64, heads: Optional[Sequence[int]] = None,
                 L: Optional[int] = None, q_given_rows: bool = False, variant: str = "bifocal"
                 ) -> Tuple[np.ndarray, np.ndarray]:
    """Output and LSE of the selected query rows of ONE sequence.

    Q_std: [L, Hq, D] (or [len(rows), Hq, D] with ``q_given_rows``), K_std / V:
    [L, Hkv, D], standard RoPE at absolute positions 0 .. L-1 (any float dtype;
    upcast to float64).  ``rows``: query positions to evaluate.  ``L`` overrides
    the length that sets G (defaults to the number of keys given).  Returns
    O [len(rows), len(heads), D] and LSE [len(rows), len(heads)] in float64.
    """
    Lk = K_std.shape[0]
    L = Lk if L is None else int(L)
    Hq, D = Q_std.shape[1], Q_std.shape[2]
    Hkv = K_std.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if w0 < 1:
        raise ValueError("w0 must be >= 1")
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant!r}")
    rep = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    heads = list(range(Hq)) if heads is None else list(heads)
    rows = np.asarray(rows, dtype=np.int64)

    G = group_size(L, w_pretrained)
    R = len(rows)
    jmax = int(rows.max()) + 1 if R else 0       # causal: no query needs keys past its row
    if jmax > Lk:
        raise ValueError("a query row lies beyond the keys given")
    kv_heads = sorted({h // rep for h in heads})
    pos = np.arange(jmax, dtype=np.int64)
    # Raw vectors: undo the standard RoPE carried by the inputs.
    k_raw = rope_rotate(K_std[:jmax, kv_heads], -pos, theta)
    k_loc = rope_rotate(k_raw, pos, theta)                 # classic RoPE at j
    k_rem = rope_rotate(k_raw, _remote_positions(pos, G, variant), theta)  # RoPE at f(j)
    v = np.asarray(V[:jmax, kv_heads], dtype=np.float64)
    slot = {g: n for n, g in enumerate(kv_heads)}

    q_sel = np.asarray(Q_std if q_given_rows else Q_std[rows], dtype=np.float64)  # [R,Hq,D]
    q_raw = rope_rotate(q_sel, -rows, theta)
    q_loc = rope_rotate(q_raw, rows, theta)                # classic RoPE at i
    q_rem = rope_rotate(q_raw, _remote_positions(rows, G, variant) + q_offset, theta)  # f(i)

    O = np.zeros((R, len(heads), D), dtype=np.float64)
    LSE = np.zeros((R, len(heads)), dtype=np.float64)
    jj = np.arange(jmax, dtype=np.int64)
    for b0 in range(0, R, row_block):
        rb = slice(b0, min(R, b0 + row_block))
        ii = rows[rb][:, None]                              # [r, 1]
        dist = ii - jj[None, :]                             # i - j
        causal = dist >= 0
        local = causal & (dist < w0)                        # sliding window of w0 keys
        for hi, h in enumerate(heads):
            g = slot[h // rep]
            s_loc = q_loc[rb, h, :] @ k_loc[:, g, :].T
            s_rem = q_rem[rb, h, :] @ k_rem[:, g, :].T
            s = scale * np.where(local, s_loc, s_rem)
            s = np.where(local if variant == "window" else causal, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            z = e.sum(axis=1, keepdims=True)
            O[rb, hi, :] = (e / z) @ v[:, g, :]
            LSE[rb, hi] = (m + np.log(z))[:, 0]
    return O, LSE


def bifocal_prefill_ref(Q_std, K_std, V, cu_seqlens, w0: int, w_pretrained: int, theta: float,
                        scale: Optional[float] = None, rows_per_seq=None, heads=None,
                        q_offset: int = 0, variant: str = "bifocal"):
    """Packed variable-length prefill: sequence b owns tokens cu[b] .. cu[b+1]-1 and
    local positions 0 .. L_b - 1; each sequence has its own G.

    ``rows_per_seq``: optional list of local row indices per sequence (None = all).
    Returns a list of (rows, O, LSE) per sequence, rows being local positions."""
    out = []
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        rows = np.arange(e - s) if rows_per_seq is None else np.asarray(rows_per_seq[b])
        if e == s or len(rows) == 0:
            out.append((rows, None, None))
            continue
        O, LSE = bifocal_rows(Q_std[s:e], K_std[s:e], V[s:e], rows, w0, w_pretrained, theta,
                              scale=scale, heads=heads, q_offset=q_offset, variant=variant)
        out.append((rows, O, LSE))
    return out


def bifocal_decode_ref(q_std, K_cache, V_cache, pos: int, w0: int, w_pretrained: int,
                       theta: float, scale: Optional[float] = None, heads=None,
                       variant: str = "bifocal"):
    """One decode step: query at position ``pos`` over cache entries 0 .. pos,
    with G from the current length pos + 1.  q_std: [Hq, D] standard RoPE at pos;
    K_cache / V_cache: [S >= pos+1, Hkv, D] standard RoPE at absolute positions.
    Returns O [Hq, D], LSE [Hq] (float64)."""
    L = int(pos) + 1
    O, LSE = bifocal_rows(np.asarray(q_std)[None], K_cache[:L], V_cache[:L], [pos], w0,
                          w_pretrained, theta, scale=scale, heads=heads, L=L,
                          q_given_rows=True, variant=variant)
    return O[0], LSE[0]
