"""The allocation-free head step (haste_head_step_noalloc: its workspace is
the library's static device scratch) against haste_head_step with a caller
workspace, through the C ABI: two allocation-free calls in a row, the second
on a smaller problem (the scratch still holds the first call's contents), and
each against the oracle.  dWh and the top-K come from the same deterministic
kernels and must be equal bit for bit; dX and the loss are fp32 atomic sums
whose order varies, so they agree to a small multiple of fp32 rounding."""
import pytest
import torch

import oracle
import workloads as wl
from _gpu import DEV, Dev, check, check_loss, to_f64

pytestmark = pytest.mark.gpu

CASES = (  # (sizes, top-K): the second smaller than the first
    (dict(B=96, D=256, H=2048, L=64, G=16, F=32), 5),
    (dict(B=40, D=128, H=512, L=64, G=16, F=32), 0),
)


@pytest.fixture(scope="module")
def H():
    from sparse_output_layer_amd import haste
    haste.lib()
    return haste


def _call(H, d, c, topk, noalloc):
    b = d.bce(0, 1.0 / c.B)
    if topk:
        b.topk_val = torch.full((c.B, topk), 7.0, dtype=torch.float32, device=DEV)
        b.topk_idx = torch.full((c.B, topk), 7, dtype=torch.int32, device=DEV)
    dWh = torch.full_like(d.Wh, 3.0)
    dX = torch.full((c.B, c.D), 5.0, dtype=torch.float32, device=DEV)
    if noalloc:
        H.haste_head_step_noalloc(d.X, d.Wh, b, dWh, dX)
    else:
        H.haste_head_step(d.X, d.Wh, b, dWh, dX)
    return b, dWh, dX


def test_head_step_noalloc_two_calls(H):
    inps = [wl.make_inputs(wl.tiny("noalloc", **case)) for case, _ in CASES]
    devs = [Dev(i) for i in inps]
    ref = [_call(H, d, i.cfg, k, False) for d, i, (_, k) in zip(devs, inps, CASES)]
    torch.cuda.synchronize()
    got = []
    for d, i, (case, k) in zip(devs, inps, CASES):
        print(f"no-alloc head step {case} top-{k}", flush=True)
        got.append(_call(H, d, i.cfg, k, True))
    torch.cuda.synchronize()
    for inp, (_, k), (b0, w0, x0), (b1, w1, x1) in zip(inps, CASES, ref, got):
        c = inp.cfg
        assert torch.equal(w0, w1), "dWh differs"
        assert float((x0 - x1).abs().max()) <= 1e-5 * float(x0.abs().max()), "dX differs"
        l0, l1 = b0.loss.item(), b1.loss.item()
        assert abs(l0 - l1) <= 1e-6 * abs(l0), (l0, l1)
        if k:
            assert torch.equal(b0.topk_val, b1.topk_val) and torch.equal(b0.topk_idx, b1.topk_idx)
        r = oracle.step(inp.X_f64(), inp.Wh_f64(), inp.idx, inp.W_f64(), inp.row_ptr,
                        inp.labels, c.L, c.G, 1.0 / c.B)
        check("noalloc dWh", to_f64(w1), r.dWh, r.dWh_abs, "bf16", nterms=c.B)
        check("noalloc dX", to_f64(x1), r.dX_head, r.dX_head_abs, "bf16", nterms=c.H)
        check_loss("noalloc loss", l1, r.loss_head, "bf16")
