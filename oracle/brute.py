"""Loop-only twin of the bifocal oracle -- TEST INFRASTRUCTURE ONLY.

Written independently of ``bifocal_ref`` (shares no helper with it) so that
one can pin the other on tiny inputs.  Everything is plain Python floats and
explicit D x D rotation matrices built entry by entry:

* R(p) is block-diagonal in the rotate-half basis: for each m < D/2 it rotates
  the plane spanned by channels m and m + D/2 by p * theta ** (-2m/D).
* A query at position i and a key at position j are first brought back to raw
  vectors with R(-i), R(-j) (the inputs carry standard RoPE at absolute
  positions, as the cache does in the pages' "on-the-fly correction rotation"
  paragraph), then scored at (i, j) if i - j < w0 and at (floor(i/G),
  floor(j/G)) otherwise, G = max(1, ceil(L / w_pretrained)) (technical
  summary, "Methodology" section 1).
* Softmax over j <= i with an explicit running sum, LSE = ln(sum exp).
* Variants: ``"interp"`` scores remote pairs at (i / G, j / G) as real numbers;
  ``"window"`` keeps only the pairs with i - j < w0.

Only meant for L up to a few dozen and D up to 8.
"""
from __future__ import annotations

import math


def _rot_matrix(p: float, D: int, theta: float):
    Rm = [[0.0] * D for _ in range(D)]
    h = D // 2
    for m in range(h):
        a = p * theta ** (-2.0 * m / D)
        c, s = math.cos(a), math.sin(a)
        Rm[m][m] = c
        Rm[m][m + h] = -s
        Rm[m + h][m] = s
        Rm[m + h][m + h] = c
    return Rm


def _matvec(Rm, x):
    return [sum(Rm[r][c] * x[c] for c in range(len(x))) for r in range(len(Rm))]


def brute_attention(Q, K, V, w0: int, w_pretrained: int, theta: float, scale=None,
                    variant: str = "bifocal"):
    """Q: nested lists [L][Hq][D]; K, V: [L][Hkv][D].  Returns (O [L][Hq][D], LSE [L][Hq])."""
    L = len(Q)
    Hq, D = len(Q[0]), len(Q[0][0])
    Hkv = len(K[0])
    rep = Hq // Hkv
    G = 1
    while G * w_pretrained < L:          # smallest G >= 1 with G * w_pretrained >= L
        G += 1
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    O = [[[0.0] * D for _ in range(Hq)] for _ in range(L)]
    LSE = [[0.0] * Hq for _ in range(L)]
    for i in range(L):
        for h in range(Hq):
            g = h // rep
            q_raw = _matvec(_rot_matrix(-i, D, theta), Q[i][h])
            scores = []
            for j in range(i + 1):
                if variant == "window" and i - j >= w0:
                    continue
                k_raw = _matvec(_rot_matrix(-j, D, theta), K[j][g])
                if i - j < w0:
                    pi, pj = i, j
                elif variant == "interp":
                    pi, pj = i / G, j / G
                else:
                    pi, pj = i // G, j // G
                qv = _matvec(_rot_matrix(pi, D, theta), q_raw)
                kv = _matvec(_rot_matrix(pj, D, theta), k_raw)
                scores.append(scale * sum(a * b for a, b in zip(qv, kv)))
            mx = max(scores)
            tot = 0.0
            for s in scores:
                tot += math.exp(s - mx)
            lse = mx + math.log(tot)
            LSE[i][h] = lse
            js = [j for j in range(i + 1) if not (variant == "window" and i - j >= w0)]
            for j, s in zip(js, scores):
                w = math.exp(s - lse)
                for d in range(D):
                    O[i][h][d] += w * V[j][g][d]
    return O, LSE
