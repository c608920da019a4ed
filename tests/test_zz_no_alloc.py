"""The no-allocation decode entry point (bifocal_decode_noalloc) through the C ABI: two
calls in a row, the second smaller, each equal to bifocal_decode on the same inputs (same
split count, so bit for bit) and within the bf16 tolerance of the oracle."""
import sys

import numpy as np
import pytest
import torch

import workloads as W
from oracle.bifocal_ref import bifocal_decode_ref
from helpers import BF16_TOL, decode_inputs, errors, std_query, within

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).cuda()


def test_noalloc_decode_matches_workspace_decode():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import dynamic_rope_context_amd as bf
    bf.lib()
    cases = [  # Hq, Hkv, cache length, position, G > 1 with remote keys
        (32, 8, 6000, 5999, 1000),
        (8, 2, 700, 333, 128),
    ]
    for Hq, Hkv, S, pos, w_pre in cases:
        w = W.Workload("noalloc", "decode", "bf16", Hq=Hq, Hkv=Hkv, D=128, w0=64,
                       w_pretrained=w_pre, theta=1e6, cache_len=S, decode_steps=1, outliers=4,
                       seed=S)
        say(f"no-alloc decode Hq={Hq} Hkv={Hkv} S={S} pos={pos}")
        q_raw, Kc, Vc = decode_inputs(w)
        q = std_query(q_raw[0], pos, w.theta, "bf16")
        qd, Kd, Vd = dev(q), dev(Kc), dev(Vc)
        o_na = torch.empty((Hq, 128), dtype=torch.bfloat16, device="cuda")
        l_na = torch.empty((Hq,), dtype=torch.float32, device="cuda")
        o_na, l_na = bf.bifocal_decode_noalloc(qd, Kd, Vd, pos, w.w0, w.w_pretrained, w.theta,
                                               out=o_na, lse=l_na)
        o_ws, l_ws = bf.bifocal_decode(qd, Kd, Vd, pos, w.w0, w.w_pretrained, w.theta)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws)
        Or, Lr = bifocal_decode_ref(q, Kc, Vc, pos, w.w0, w.w_pretrained, w.theta)
        e = errors(o_na.float().cpu().numpy(), Or, l_na.cpu().numpy(), Lr)
        say(f"  against the oracle: {e}")
        assert within(e, BF16_TOL), e
