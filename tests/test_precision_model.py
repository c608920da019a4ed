"""The bf16 prefill's precision scheme, weighed on the CPU with a model of its rounding
steps (tests/precision_model.py) against the float64 oracle, on the workloads' own input
distribution: i.i.d. normal q/k/v with 4 independently seeded x8 outlier channels per
query head and per KV head (the Qwen3-4B 128K and ragged workloads' layout), at
GQA ratios 2 and 4.

The bound checked is the LSE tolerance of the bf16 parity tests, 5e-3, on every case.
The scheme: fp16 remote operands and fp16 probabilities; the 4 RoPE pairs per KV head
with the largest sum over the group's query heads of |q_h|^2 |k|^2 corrected on both
sides (for every head).  An outlier channel (x8) makes both rounding errors of its
products large (each is relative to |q_c k_c|); ranking the pairs by the sum over the
heads puts the key outliers, whose errors reach every head, first.  Measured on the GPU
over all rows of the layout cases below, the kernel reaches at most 4.60e-3 (the model
gives the same figures to within 1e-5), and 2.62e-3 over 528 rows x 32 heads of the
Qwen3-4B 128K workload (too slow for this suite), where the same 4 pairs ranked by the
maximum over the heads instead reached 6.0e-3.  A query-side correction of 8 more pairs
per head lowered the worst layout case only to 4.52e-3 for one more matrix product per
remote tile.  The model is first tied to the oracle (with every remote channel corrected
and fp16 probabilities it must agree to a few 1e-4) and to the kernel's measured
behaviour (with bf16 probabilities it must show the 4.9e-3 the kernel measured on the
smoke workload)."""
import numpy as np
import pytest

import workloads as W
from helpers import prefill_inputs
from oracle.bifocal_ref import bifocal_rows
from precision_model import Scheme, emulate_rows, select_pairs

KERNEL = Scheme(pairs=4, p_type="f16", kv_sum=True)  # the matrix-core prefill
EARLIER_F16 = Scheme(pairs=4, p_type="f16")
EARLIER = Scheme(pairs=4, p_type="bf16")   # bf16 probabilities
EXACT = Scheme(pairs=64, p_type="f16")     # every remote channel corrected
LSE_BOUND = 5e-3  # the bf16 parity tests' LSE tolerance

SMOKE = W.Workload("smoke", "prefill", "bf16", Hq=8, Hkv=2, D=128, w0=64, w_pretrained=256,
                   theta=1e6, seqlens=(1000, 77), outliers=4, seed=2024)


def _errors(w, scheme, n_uniform=None):
    """Worst (max |dO|, mean |dO|, max |dLSE|) of the model against the oracle over the
    sequences of w (all rows, or sampled rows)."""
    Q, K, V, cu = prefill_inputs(w)
    pairs = select_pairs(Q, K, scheme.pairs, by_sum=scheme.kv_sum)  # over the whole call
    worst = [0.0, 0.0, 0.0]
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        L = s1 - s0
        rows = np.arange(L) if n_uniform is None else W.sample_rows(L, w.w0, n_uniform, seed=b)
        Or, Lr = bifocal_rows(Q[s0:s1], K[s0:s1], V[s0:s1], rows, w.w0, w.w_pretrained, w.theta)
        O, LSE = emulate_rows(Q[s0:s1], K[s0:s1], V[s0:s1], rows, w.w0, w.w_pretrained,
                              w.theta, scheme, pairs=pairs)
        d = np.abs(O - Or)
        worst = [max(worst[0], d.max()), max(worst[1], d.mean()),
                 max(worst[2], np.abs(LSE - Lr).max())]
    return worst


def test_model_with_exact_scores_matches_oracle():
    # only the output and probability roundings left: the model's masks, tile order and
    # softmax must reproduce the oracle closely
    mx, mean, lse = _errors(SMOKE, EXACT)
    assert lse < 6e-4 and mx < 1e-2 and mean < 1e-3, (mx, mean, lse)


def test_model_reproduces_the_earlier_kernel_margin():
    # bf16 probabilities: the kernel measured max |dLSE| 4.94e-3 on this workload
    _, _, lse = _errors(SMOKE, EARLIER)
    assert 4.5e-3 < lse < 5.5e-3, lse


def test_kernel_scheme_on_smoke_workload():
    mx, mean, lse = _errors(SMOKE, KERNEL)
    assert lse <= LSE_BOUND and mx <= 2e-2 and mean <= 2e-3, (mx, mean, lse)


def test_kernel_scheme_on_many_short_sequences():
    lens = tuple([(37 * i) % 150 + 1 for i in range(24)])
    w = W.Workload("stress", "prefill", "bf16", Hq=4, Hkv=2, D=128, w0=20, w_pretrained=100,
                   theta=1e6, seqlens=lens, outliers=4, seed=17)
    mx, mean, lse = _errors(w, KERNEL)
    assert lse <= LSE_BOUND and mx <= 2e-2 and mean <= 2e-3, (mx, mean, lse)


@pytest.mark.parametrize("rep", [2, 4])
@pytest.mark.parametrize("seed", [1, 2, 3, 4, 5])
def test_kernel_scheme_on_workload_outlier_layout(rep, seed):
    # G = 4 (L = 2048, w_pretrained = 512), a window of 128 keys, four KV heads
    w = W.Workload("layout", "prefill", "bf16", Hq=4 * rep, Hkv=4, D=128, w0=128,
                   w_pretrained=512, theta=1e6, seqlens=(2048,), outliers=4, seed=seed)
    mx, mean, lse = _errors(w, KERNEL, n_uniform=200)
    assert lse <= LSE_BOUND and mx <= 2e-2 and mean <= 2e-3, (mx, mean, lse)
