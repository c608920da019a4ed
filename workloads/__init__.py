"""Seeded synthetic workloads shared by the tests, the benchmark and the oracle checks.

This module only draws random numbers and describes shapes.  It holds none
of the attention or RoPE arithmetic: the standard-RoPE step that turns the
raw query/key draws into the kernel inputs is done by whoever consumes them
(the CPU oracle in the tests, ``rope_apply`` on the GPU in the benchmark).

Workload shapes follow the Qwen3 models the Jet-Long pages evaluate on
(Qwen3-1.7B / 4B / 8B, native 32K window extended to 128K; technical
summary, "Experimental results").  No model weights or benchmark data are
involved: every tensor is i.i.d. normal noise, optionally with a few
"outlier" channels scaled up to stress the dynamic range of the remote
(aliased) scoring branch.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get", "raw_prefill_inputs", "raw_decode_inputs",
    "outlier_channels", "f32_to_bf16_bits", "bf16_bits_to_f32", "round_to_bf16",
    "sample_rows",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "prefill" or "decode"
    dtype: str                # "f32" or "bf16"
    Hq: int
    Hkv: int
    D: int
    w0: int
    w_pretrained: int
    theta: float
    seqlens: Tuple[int, ...] = ()   # prefill: one length per sequence
    cache_len: int = 0              # decode: keys held by the cache at the last step
    decode_steps: int = 0           # decode: consecutive steps ending at cache_len-1
    outliers: int = 0               # outlier channels per head (raw values x outlier_scale)
    outlier_scale: float = 8.0
    seed: int = 0

    @property
    def total_tokens(self) -> int:
        return sum(self.seqlens) if self.kind == "prefill" else self.cache_len

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int32)

    def decode_positions(self) -> np.ndarray:
        """Positions of the timed decode steps: the last one sees the full cache."""
        return np.arange(self.cache_len - self.decode_steps, self.cache_len, dtype=np.int64)


WORKLOADS = {
    # CPU-seconds reference in fp32: G = ceil(512/128) = 4.
    "tiny_f32": Workload("tiny_f32", "prefill", "f32", Hq=2, Hkv=1, D=64, w0=32,
                         w_pretrained=128, theta=1e4, seqlens=(512,), seed=1000),
    # Qwen3-1.7B attention layer, L = w_pretrained so G = 1: must equal vanilla RoPE attention.
    "qwen3_1p7b_32k_g1": Workload("qwen3_1p7b_32k_g1", "prefill", "bf16", Hq=16, Hkv=8, D=128,
                                  w0=4096, w_pretrained=32768, theta=1e6, seqlens=(32768,),
                                  seed=2000),
    # Qwen3-4B attention layer at 128K: G = 4, outlier channels.
    "qwen3_4b_128k": Workload("qwen3_4b_128k", "prefill", "bf16", Hq=32, Hkv=8, D=128, w0=4096,
                              w_pretrained=32768, theta=1e6, seqlens=(131072,), outliers=4,
                              seed=3000),
    # Qwen3-8B single-batch decode over a 128K standard-RoPE cache, 256 consecutive steps.
    "qwen3_8b_decode_128k": Workload("qwen3_8b_decode_128k", "decode", "bf16", Hq=32, Hkv=8,
                                     D=128, w0=4096, w_pretrained=32768, theta=1e6,
                                     cache_len=131072, decode_steps=256, seed=4000),
    # The same decode layer generating across the length boundary L = 4 * 32768 + 1, where G
    # goes from 4 to 5 while the cache stays as stored (positions 131071 .. 131328).
    "qwen3_8b_decode_boundary": Workload("qwen3_8b_decode_boundary", "decode", "bf16", Hq=32,
                                         Hkv=8, D=128, w0=4096, w_pretrained=32768, theta=1e6,
                                         cache_len=131329, decode_steps=258, seed=4100),
    # Qwen3-8B ragged prefill: two sequences with their own G (4 and 2), ragged tails.
    "qwen3_8b_ragged": Workload("qwen3_8b_ragged", "prefill", "bf16", Hq=32, Hkv=8, D=128,
                                w0=8192, w_pretrained=32768, theta=1e6,
                                seqlens=(98427, 40001), outliers=4, seed=5000),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def outlier_channels(seed: int, n_heads: int, D: int, count: int) -> np.ndarray:
    """[n_heads, count] distinct channel indices per head, drawn from ``seed``."""
    rng = _rng(seed)
    if count == 0:
        return np.zeros((n_heads, 0), dtype=np.int64)
    return np.stack([rng.choice(D, size=count, replace=False) for _ in range(n_heads)])


def _normal(seed: int, shape, chunk: int = 1 << 24) -> np.ndarray:
    """Standard normal fp32 draws; filled in chunks so that large tensors stay cheap."""
    rng = _rng(seed)
    out = np.empty(int(np.prod(shape)), dtype=np.float32)
    for s in range(0, out.size, chunk):
        e = min(out.size, s + chunk)
        out[s:e] = rng.standard_normal(e - s, dtype=np.float32)
    return out.reshape(shape)


def _apply_outliers(x: np.ndarray, chans: np.ndarray, scale: float) -> None:
    # x: [T, H, D]; per head, the chosen raw channels are multiplied by `scale`.
    for h in range(chans.shape[0]):
        for c in chans[h]:
            x[:, h, c] *= np.float32(scale)


def raw_prefill_inputs(w: Workload, T: Optional[int] = None):
    """Raw (pre-RoPE) q, k and v for a prefill workload, fp32.

    Seeds: q = seed+1, k = seed+2, v = seed+3, outlier choice = seed+4 (q heads)
    and seed+5 (kv heads).  ``T`` truncates the token count (used for reduced
    test sizes with the same value distribution).
    """
    T = w.total_tokens if T is None else T
    q = _normal(w.seed + 1, (T, w.Hq, w.D))
    k = _normal(w.seed + 2, (T, w.Hkv, w.D))
    v = _normal(w.seed + 3, (T, w.Hkv, w.D))
    if w.outliers:
        _apply_outliers(q, outlier_channels(w.seed + 4, w.Hq, w.D, w.outliers), w.outlier_scale)
        _apply_outliers(k, outlier_channels(w.seed + 5, w.Hkv, w.D, w.outliers), w.outlier_scale)
    return q, k, v


def raw_decode_inputs(w: Workload, S: Optional[int] = None):
    """Raw cache keys/values [S, Hkv, D] and one raw query per decode step [steps, Hq, D]."""
    S = w.cache_len if S is None else S
    k = _normal(w.seed + 2, (S, w.Hkv, w.D))
    v = _normal(w.seed + 3, (S, w.Hkv, w.D))
    q = _normal(w.seed + 1, (max(1, w.decode_steps), w.Hq, w.D))
    if w.outliers:
        _apply_outliers(q, outlier_channels(w.seed + 4, w.Hq, w.D, w.outliers), w.outlier_scale)
        _apply_outliers(k, outlier_channels(w.seed + 5, w.Hkv, w.D, w.outliers), w.outlier_scale)
    return q, k, v


# ---------------------------------------------------------------------------
# bfloat16 plumbing (storage format only; round-to-nearest-even from fp32)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even; NaN stays NaN."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Values rounded to bf16 (via fp32), returned as fp32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


def sample_rows(L: int, w0: int, n_uniform: int, seed: int, tile: int = 64,
                extra: Tuple[int, ...] = ()) -> np.ndarray:
    """Query rows to compare at long L: first/last rows, rows around w0, tile and
    aliasing-group boundaries, plus uniform draws."""
    rows = set(range(min(L, 16)))
    rows.update(range(max(0, L - 16), L))
    for c in (w0 - 2, w0 - 1, w0, w0 + 1, w0 + 2, tile - 1, tile, 2 * tile + 1, L // 2,
              L // 2 + 1, L - tile - 1, L - tile):
        if 0 <= c < L:
            rows.add(c)
    rows.update(int(e) for e in extra if 0 <= e < L)
    rng = _rng(seed)
    rows.update(int(r) for r in rng.integers(0, L, size=n_uniform))
    return np.array(sorted(rows), dtype=np.int64)


# ---------------------------------------------------------------------------
# Device-side draws for the benchmark (same distributions, torch's generator)
# ---------------------------------------------------------------------------

def raw_inputs_torch(w: Workload, device="cuda", T: Optional[int] = None, dtype=None):
    """Raw q [T,Hq,D] (or [decode_steps,Hq,D] for decode), k, v [T,Hkv,D] drawn on the
    device with torch.Generator(seed); outlier channels chosen as in the numpy path.
    Values are rounded to ``dtype`` (default: the workload's dtype)."""
    import torch
    dt = dtype or (torch.bfloat16 if w.dtype == "bf16" else torch.float32)
    T = (w.total_tokens if T is None else T)
    nq = T if w.kind == "prefill" else max(1, w.decode_steps)
    out = []
    for off, shape, hkey in ((1, (nq, w.Hq, w.D), 4), (2, (T, w.Hkv, w.D), 5),
                             (3, (T, w.Hkv, w.D), None)):
        g = torch.Generator(device=device)
        g.manual_seed(w.seed + off)
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if w.outliers and hkey is not None:
            ch = outlier_channels(w.seed + hkey, shape[1], w.D, w.outliers)
            for h in range(shape[1]):
                x[:, h, torch.as_tensor(ch[h], device=device)] *= w.outlier_scale
        out.append(x.to(dt))
    return tuple(out)
