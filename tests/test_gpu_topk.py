"""Per-row top-K (top-K page, section "Method": per-bucket top-K' and a merge,
with K' = K) against the oracle, through the C ABI: tail and head separately
(fwd, fused step, split dW step), then merged over the whole output space."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from _gpu import DEV, Dev, check_topk, topk_tol

pytestmark = pytest.mark.gpu

CASES = [
    dict(B=40, D=96, H=48, L=200, G=16, F=32, K=5),
    dict(B=33, D=128, H=64, L=70000, G=64, F=64, K=5),     # three buckets of the tail
    dict(B=70, D=200, H=56, L=300, G=32, F=128, K=8),
    dict(B=50, D=256, H=64, L=5000, G=64, F=128, K=5),     # groups of 64 in two label slices
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
        tie_free, _ = check_topk(name, tv.cpu().numpy(), ti.cpu().numpy(), Zt, Zta, K, dt, id0=c.H,
                                 nterms=c.F)
        assert tie_free >= c.B // 2, (name, tie_free)

    # head: forward and fused step
    hv, hi = outs()
    H.haste_head_fwd(d.X, d.Wh, bce=bce(0, hv, hi))
    torch.cuda.synchronize()
    check_topk("head fwd", hv.cpu().numpy(), hi.cpu().numpy(), Zh, Zha, K, dt, id0=0, nterms=c.D)
    hv, hi = outs()
    H.haste_head_step(d.X, d.Wh, bce(0, hv, hi), torch.empty_like(d.Wh),
                      torch.empty(c.B, c.D, dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    check_topk("head step", hv.cpu().numpy(), hi.cpu().numpy(), Zh, Zha, K, dt, id0=0, nterms=c.D)

    # whole output space: head and tail lists merged
    tv, ti = results["tail step"]
    mv, mi = H.haste_topk_merge(hv, hi, tv, ti)
    torch.cuda.synchronize()
    check_topk("merged", mv.cpu().numpy(), mi.cpu().numpy(), np.concatenate([Zh, Zt], axis=1),
               np.concatenate([Zha, Zta], axis=1), K, dt, id0=0,
               nterms=np.concatenate([np.full(c.H, c.D), np.full(c.L, c.F)]))


APPROX = [
    # tail: (K, K', buckets); head last
    dict(B=24, D=128, H=64, L=70000, G=64, F=64, K=5, KP=2, NB=7),
    dict(B=20, D=96, H=48, L=1000, G=16, F=32, K=8, KP=1, NB=50),
    dict(B=16, D=96, H=48, L=600, G=32, F=64, K=5, KP=5, NB=3),      # exact on custom buckets
    dict(B=12, D=64, H=64, L=300, G=16, F=32, K=4, KP=2, NB=4, head=True),
    # one bucket per label group with K' = 1: stage 1 runs inside the logits pass
    dict(B=40, D=128, H=48, L=4000, G=16, F=64, K=5, KP=1, NB=250),
    dict(B=70, D=200, H=48, L=3000, G=64, F=32, K=8, KP=1, NB=47),
    dict(B=33, D=768, H=48, L=2000, G=32, F=128, K=3, KP=1, NB=63, step=True),
    # the merge's lane layouts (8 and 64 lanes per group), several group
    # segments with a ragged last one, two row blocks with a ragged last one
    dict(B=20, D=64, H=48, L=30000, G=32, F=32, K=4, KP=1, NB=938),
    dict(B=300, D=64, H=48, L=40000, G=16, F=32, K=5, KP=1, NB=2500),
]


def _check_two_stage(name, got_v, got_i, z, zabs, K, kp, seg, dtype, id0, nterms):
    """Against the oracle's two-stage top-K (top-K page, "Method") on the same
    buckets.  Ranks are decided with the fp32 summation bound of the kernels'
    logits (the same bf16 inputs, fp32 accumulation of nterms products):
    t = 2 * nterms * 2^-24 * sum|x w| per logit.  Where a bucket's K'-th and
    (K'+1)-th oracle logits lie within their two bounds, the kernels may pick
    either: such rows are checked for validity only.  Returns the number of
    rows compared by id."""
    rows, N = z.shape
    u = 2.0 ** -24
    ov, oi = oracle.topk_two_stage(z, K, kp, seg, id_offset=id0)
    vtol = topk_tol(zabs.max(axis=1), dtype)

    def rt(b, ids):            # rank tolerance of the logits of these ids in row b
        return 2 * nterms * u * zabs[b, np.asarray(ids) - id0]

    amb = np.zeros(rows, bool)
    surv = 0
    for c0 in range(0, N, seg):
        c1 = min(c0 + seg, N)
        surv += min(kp, c1 - c0)
        if c1 - c0 > kp:
            bv, bi = oracle.topk(z[:, c0:c1], kp + 1, id_offset=id0 + c0)
            for b in range(rows):
                t2 = rt(b, bi[b, kp - 1:kp + 1])
                amb[b] |= bv[b, kp - 1] - bv[b, kp] <= t2.sum()
    n = min(K, surv)
    got_v = np.asarray(got_v, np.float64)
    got_i = np.asarray(got_i, np.int64)
    for b in range(rows):
        ids = got_i[b]
        assert np.all(ids[:n] >= id0) and np.all(ids[:n] < id0 + N), f"{name}: row {b}: {ids}"
        assert np.all(ids[n:] == -1) and np.all(np.isneginf(got_v[b, n:])), f"{name}: row {b} padding"
        assert len(set(ids[:n].tolist())) == n, f"{name}: row {b} repeats an id"
        for k in range(n):
            assert abs(got_v[b, k] - z[b, ids[k] - id0]) <= vtol[b], f"{name}: row {b} pos {k} value"
            if k:
                assert got_v[b, k] <= got_v[b, k - 1], f"{name}: row {b} not descending"
        if amb[b]:
            continue
        m = min(n + 1, ov.shape[1])
        valid = oi[b, :m] >= 0
        tk = np.zeros(m)
        tk[valid] = rt(b, oi[b, :m][valid])
        for k in range(n):
            assert abs(got_v[b, k] - ov[b, k]) <= vtol[b], f"{name}: row {b} pos {k}: {got_v[b, k]} vs {ov[b, k]}"
            sep_hi = k == 0 or ov[b, k - 1] - ov[b, k] > tk[k - 1] + tk[k]
            sep_lo = k + 1 >= m or not valid[k + 1] or ov[b, k] - ov[b, k + 1] > tk[k] + tk[k + 1]
            if sep_hi and sep_lo:
                assert ids[k] == oi[b, k], f"{name}: row {b} pos {k}: id {ids[k]} vs oracle {oi[b, k]}"
    return int((~amb).sum())


@pytest.mark.parametrize("case", APPROX, ids=[
    "B{B}-L{L}-K{K}-Kp{KP}-nb{NB}".format(**c) + ("-head" if c.get("head") else "") +
    ("-step" if c.get("step") else "") for c in APPROX])
def test_topk_two_stage(H, case):
    print("case", case, flush=True)
    case = dict(case)
    K, KP, NB, head = case.pop("K"), case.pop("KP"), case.pop("NB"), case.pop("head", False)
    step = case.pop("step", False)
    inp = wl.make_inputs(wl.tiny("tk2", **case))
    c = inp.cfg
    d = Dev(inp)
    X, Wt, Wh = inp.X_f64(), inp.W_f64(), inp.Wh_f64()
    tv = torch.full((c.B, K), 7.0, dtype=torch.float32, device=DEV)
    ti = torch.full((c.B, K), 7, dtype=torch.int32, device=DEV)
    b = d.bce(0 if head else c.H, 1.0 / c.B)
    b.topk_val, b.topk_idx, b.topk_kprime, b.topk_buckets = tv, ti, KP, NB
    if head:
        z, za = oracle.head_logits(X, Wh, want_abs=True)
        H.haste_head_fwd(d.X, d.Wh, bce=b)
        n, id0, nterms = c.H, 0, c.D
    else:
        z, za = oracle.tail_logits(X, inp.idx, Wt, c.L, c.G, want_abs=True)
        if step:
            H.haste_tail_step(d.X, d.idx, d.W, c.L, c.G, b, torch.empty_like(d.W),
                              torch.empty(c.B, c.D, dtype=torch.float32, device=DEV))
        else:
            H.haste_tail_fwd(d.X, d.idx, d.W, c.L, c.G, bce=b)
        n, id0, nterms = c.L, c.H, c.F
    torch.cuda.synchronize()
    seg = oracle.topk_seg_len(n, NB)
    done = _check_two_stage("two-stage", tv.cpu().numpy(), ti.cpu().numpy(), z, za, K, KP, seg,
                            c.dtype, id0, nterms)
    print(f"rows compared by id: {done} of {c.B}", flush=True)
    assert done >= c.B // 2
