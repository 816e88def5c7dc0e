"""The allocation-free forward (dualkv_fwd_noalloc, for callers that cannot
allocate) against dualkv_fwd on the same inputs: the kernels are the same and
the forward's result does not depend on the order of its work list, so O and
LSE must agree bitwise. Two calls in a row on one GPU, the second smaller, so
the second reuses the fixed scratch array the first one filled."""
import sys

import numpy as np
import pytest
import torch

from exact_shared_prefix_amd import binding
from exact_shared_prefix_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # larger first, then smaller: ragged with an empty response, GQA 4, d = 128
    dict(P=1000, lengths=[300, 0, 517, 64, 1], Hq=8, Hkv=2, d=128, seed=81),
    dict(P=100, lengths=[50, 20], Hq=4, Hkv=2, d=64, seed=82),
]


def _run(c):
    inp = make_inputs(c["P"], c["lengths"], c["Hq"], c["Hkv"], c["d"], seed=c["seed"])
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in (inp.q, inp.k, inp.v))
    pk = binding.Packing(inp.P, inp.lengths)
    o_ref, lse_ref = binding.fwd(q, k, v, pk, inp.scale)
    o = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(lse_ref, float("nan"))
    binding.fwd_noalloc(q, k, v, pk, inp.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu(), o_ref.cpu(), lse_ref.cpu()


def test_noalloc_forward_matches_workspace_forward_twice():
    for i, c in enumerate(CASES):
        print(f"case no-alloc call {i}: {c}", flush=True)
        sys.stdout.flush()
        o, lse, o_ref, lse_ref = _run(c)
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), i
        assert torch.equal(lse, lse_ref), i
        assert np.all(np.isfinite(o.float().numpy())), i
