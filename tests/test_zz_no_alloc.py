"""The allocation-free forward (moe_decode_forward_noalloc) against the
forward with a caller's workspace, through the C ABI: the same kernels on
the same inputs, so the outputs, selections and weights must be equal bit
for bit -- on two calls in a row, the second with fewer rows, and on both
paths (m <= 32 and the grouped m > 32)."""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_decode_amd import moe_decode as md
from mixture_experts_decode_amd import synth
from mixture_experts_decode_amd.device import DeviceLayer, to_device
from tests.test_gpu_parity import TOL, check, say, small

pytestmark = pytest.mark.gpu


def _both(dl, x_np, m):
    spec = dl.spec
    x = to_device(np.ascontiguousarray(x_np[:m]), "cuda")
    st = torch.cuda.current_stream().cuda_stream
    res = []
    for noalloc in (False, True):
        out = dl.new_out(m)
        idx = torch.full((m, spec.top_k), -1, dtype=torch.int32, device="cuda")
        w = torch.full((m, spec.top_k), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            md.moe_decode_forward_noalloc(dl.plan, dl.weights, x.data_ptr(), m, out.data_ptr(),
                                          idx.data_ptr(), w.data_ptr(), st)
        else:
            dl.forward(x, m, out, idx, w)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()))
    return res


@pytest.mark.parametrize("rows,mmax", [((8, 3), 8), ((64, 40), 64)])
def test_noalloc_matches_the_workspace_forward(rows, mmax):
    spec = small(hidden=256, num_experts=12, top_k=3, inter=192, shared=True, shared_gated=True,
                 shared_inter=160, rows=(mmax,))
    layer = synth.make_layer(spec, seed=901 + mmax)
    x = layer.x(0)
    ref = oracle.forward(layer, x)
    dl = DeviceLayer(layer)
    for m in rows:                              # two calls in a row, the second smaller
        say(f"[gpu] noalloc m={m} (max_rows {mmax})")
        (o1, i1, w1), (o2, i2, w2) = _both(dl, x, m)
        assert np.array_equal(o1, o2) and np.array_equal(i1, i2) and np.array_equal(w1, w2)
        got = (o2.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        check(spec, got, i2, w2, ref, m, TOL["bf16"], f"noalloc m={m}")
    del dl
    torch.cuda.empty_cache()
