"""Per-row top-K (top-K page, section "Method": per-bucket top-K' and a merge,
with K' = K) against the oracle, through the C ABI: tail and head separately
(fwd, fused step, split dW step), then merged over the whole output space."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from _gpu import DEV, Dev, check_topk

pytestmark = pytest.mark.gpu

CASES = [
    dict(B=40, D=96, H=48, L=200, G=16, F=32, K=5),
    dict(B=33, D=128, H=64, L=70000, G=64, F=64, K=5),     # three buckets of the tail
    dict(B=70, D=200, H=56, L=300, G=32, F=128, K=8),
    dict(B=17, D=64, H=40, L=3, G=16, F=32, K=5),           # fewer tail labels than K
    dict(B=9, D=64, H=64, L=1024, G=16, F=16, K=1, dtype="f32"),
]


@pytest.fixture(scope="module")
def H():
    from sparse_output_layer_amd import haste
    haste.lib()
    return haste


def _ids(c):
    return "B{B}-L{L}-G{G}-K{K}".format(**c) + ("-f32" if c.get("dtype") == "f32" else "")


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_topk(H, case):
    print("case", case, flush=True)
    case = dict(case)
    K = case.pop("K")
    inp = wl.make_inputs(wl.tiny("tk", **case))
    c = inp.cfg
    s = 1.0 / c.B
    d = Dev(inp)
    dt = c.dtype
    X, Wt, Wh = inp.X_f64(), inp.W_f64(), inp.Wh_f64()
    Zt, Zta = oracle.tail_logits(X, inp.idx, Wt, c.L, c.G, want_abs=True)
    Zh, Zha = oracle.head_logits(X, Wh, want_abs=True)

    def outs():
        return (torch.full((c.B, K), 7.0, dtype=torch.float32, device=DEV),
                torch.full((c.B, K), 7, dtype=torch.int32, device=DEV))

    def bce(off, tv, ti):
        b = d.bce(off, s)
        b.topk_val, b.topk_idx = tv, ti
        return b

    # tail: forward, fused step, split dW step
    results = {}
    tv, ti = outs()
    H.haste_tail_fwd(d.X, d.idx, d.W, c.L, c.G, bce=bce(c.H, tv, ti))
    results["tail fwd"] = (tv, ti)
    tv, ti = outs()
    H.haste_tail_step(d.X, d.idx, d.W, c.L, c.G, bce(c.H, tv, ti), torch.empty_like(d.W),
                      torch.empty(c.B, c.D, dtype=torch.float32, device=DEV))
    results["tail step"] = (tv, ti)
    tv, ti = outs()
    b5 = bce(c.H, tv, ti)
    ws = torch.empty(H.haste_tail_workspace_bytes(d.X, d.idx, c.L, c.G, b5), dtype=torch.uint8,
                     device=DEV)
    H.haste_tail_prepare(d.X, d.idx, c.L, c.G, b5, ws)
    H.haste_tail_step_dw(d.X, d.idx, d.W, c.L, c.G, b5, torch.empty_like(d.W), ws)
    results["tail split dW"] = (tv, ti)
    torch.cuda.synchronize()
    for name, (tv, ti) in results.items():
        check_topk(name, tv.cpu().numpy(), ti.cpu().numpy(), Zt, Zta, K, dt, id0=c.H)

    # head: forward and fused step
    hv, hi = outs()
    H.haste_head_fwd(d.X, d.Wh, bce=bce(0, hv, hi))
    torch.cuda.synchronize()
    check_topk("head fwd", hv.cpu().numpy(), hi.cpu().numpy(), Zh, Zha, K, dt, id0=0)
    hv, hi = outs()
    H.haste_head_step(d.X, d.Wh, bce(0, hv, hi), torch.empty_like(d.Wh),
                      torch.empty(c.B, c.D, dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    check_topk("head step", hv.cpu().numpy(), hi.cpu().numpy(), Zh, Zha, K, dt, id0=0)

    # whole output space: head and tail lists merged
    tv, ti = results["tail step"]
    mv, mi = H.haste_topk_merge(hv, hi, tv, ti)
    torch.cuda.synchronize()
    check_topk("merged", mv.cpu().numpy(), mi.cpu().numpy(), np.concatenate([Zh, Zt], axis=1),
               np.concatenate([Zha, Zta], axis=1), K, dt, id0=0)
