"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Small shapes are compared element by element; they span several MFMA tiles,
several 64-row chunks and ragged tails (rows, labels, features).  Integer
outputs (group-major positives, index validation, merged top-K ids) must be
bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from _gpu import DEV, TOL_BF16, Dev, check, check_loss, dev_array, to_f64

pytestmark = pytest.mark.gpu

CASES = [
    dict(B=40, D=96, H=48, L=200, G=16, F=32),
    dict(B=64, D=128, H=64, L=512, G=32, F=64),
    dict(B=70, D=200, H=56, L=300, G=64, F=128),
    dict(B=128, D=768, H=256, L=2000, G=16, F=128),
    dict(B=33, D=1024, H=96, L=700, G=64, F=64, idx_dist="skew10"),
    dict(B=65, D=768, H=128, L=1000, G=64, F=128, pos_per_row=7),
    dict(B=130, D=768, H=136, L=1500, G=32, F=128),
    # groups of 16 on wide inputs: 32-row dX chunks at D = 1024, 64-row
    # chunks at D = 544, and a batch of at most 32 rows
    dict(B=40, D=1024, H=64, L=600, G=16, F=64),
    dict(B=96, D=544, H=64, L=800, G=16, F=32),
    dict(B=20, D=448, H=48, L=400, G=16, F=128),
    # the scatter form of dX (groups of 32 and more on inputs of at least
    # 12F features): groups of 32, and a ragged batch with groups of 64
    dict(B=50, D=512, H=64, L=900, G=32, F=32),
    dict(B=90, D=800, H=64, L=1300, G=64, F=64),
    # degenerate shapes: one row and fewer labels than a group; full fan-in
    # (F = D); exactly one group of 64 at F = D = 128
    dict(B=1, D=64, H=16, L=10, G=16, F=32),
    dict(B=3, D=32, H=8, L=100, G=32, F=32),
    dict(B=64, D=128, H=64, L=64, G=64, F=128),
]


def _ids(c):
    return "B{B}-D{D}-L{L}-G{G}-F{F}".format(**c)


@pytest.fixture(scope="module")
def H():
    from sparse_output_layer_amd import haste
    haste.lib()
    return haste


def _ref(inp):
    c = inp.cfg
    return oracle.step(inp.X_f64(), inp.Wh_f64(), inp.idx, inp.W_f64(), inp.row_ptr,
                       inp.labels, c.L, c.G, 1.0 / c.B)


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_bf16_tail_and_head(H, case):
    print("case", case, flush=True)
    inp = wl.make_inputs(wl.tiny("par", **case))
    c = inp.cfg
    s = 1.0 / c.B
    r = _ref(inp)
    d = Dev(inp)
    bf = torch.bfloat16

    # tail forward: logits and loss
    Z = torch.empty(c.B, c.L, dtype=bf, device=DEV)
    b = d.bce(c.H, s)
    H.haste_tail_fwd(d.X, d.idx, d.W, c.L, c.G, Z=Z, bce=b)
    torch.cuda.synchronize()
    check("tail Z", to_f64(Z), r.Zt, r.Zt_abs, "bf16", nterms=c.F)
    check_loss("tail fwd loss", b.loss.item(), r.loss_tail, "bf16")

    # fused tail step
    dW = torch.full_like(d.W, 7.0)
    dX = torch.full((c.B, c.D), 3.0, dtype=torch.float32, device=DEV)
    b = d.bce(c.H, s)
    H.haste_tail_step(d.X, d.idx, d.W, c.L, c.G, b, dW, dX)
    torch.cuda.synchronize()
    check_loss("tail step loss", b.loss.item(), r.loss_tail, "bf16")
    check("tail dW", to_f64(dW[:c.L]), r.dWt, r.dWt_abs, "bf16", nterms=c.B)
    assert torch.all(dW[c.L:] == 0), "padded label rows of dW must be exactly zero"
    ng = c.n_groups
    check("tail dX", to_f64(dX), r.dX_tail, r.dX_tail_abs, "bf16", nterms=ng * c.G)
    # deterministic weight gradient (no atomics on dW)
    dW2 = torch.empty_like(d.W)
    dX2 = torch.empty_like(dX)
    H.haste_tail_step(d.X, d.idx, d.W, c.L, c.G, d.bce(c.H, s, loss=False), dW2, dX2)
    torch.cuda.synchronize()
    assert torch.equal(dW, dW2)

    # lean form: the dX pass recomputes dz instead of reading the dW pass's tiles
    dW6 = torch.empty_like(d.W)
    dX6 = torch.empty_like(dX)
    b6 = d.bce(c.H, s)
    H.haste_tail_step(d.X, d.idx, d.W, c.L, c.G, b6, dW6, dX6, lean=True)
    torch.cuda.synchronize()
    check_loss("lean step loss", b6.loss.item(), r.loss_tail, "bf16")
    assert torch.equal(dW6, dW)
    check("lean step dX", to_f64(dX6), r.dX_tail, r.dX_tail_abs, "bf16", nterms=ng * c.G)

    # split form of the step (prepare, dW, dX), as the benchmark runs it, both forms
    for lean in (False, True):
        b5 = d.bce(c.H, s)
        ws = torch.empty(H.haste_tail_workspace_bytes(d.X, d.idx, c.L, c.G, b5, lean=lean),
                         dtype=torch.uint8, device=DEV)
        dW5 = torch.empty_like(d.W)
        dX5 = torch.full_like(dX, 2.0)
        H.haste_tail_prepare(d.X, d.idx, c.L, c.G, b5, ws, lean=lean)
        H.haste_tail_step_dw(d.X, d.idx, d.W, c.L, c.G, b5, dW5, ws, lean=lean)
        H.haste_tail_step_dx(d.X, d.idx, d.W, c.L, c.G, b5, dX5, ws, accumulate_dX=True, lean=lean)
        torch.cuda.synchronize()
        check_loss(f"split step loss (lean={lean})", b5.loss.item(), r.loss_tail, "bf16")
        assert torch.equal(dW5, dW)
        check(f"split step dX (lean={lean})", to_f64(dX5) - 2.0, r.dX_tail, r.dX_tail_abs, "bf16",
              nterms=ng * c.G)

    # the feature order formed once (haste_tail_prepare_layout) and taken
    # from the workspace by every later call (HASTE_TAIL_LAYOUT_READY): the
    # same results, bit for bit, over two steps on one workspace
    b8 = d.bce(c.H, s)
    ws = torch.empty(H.haste_tail_workspace_bytes(d.X, d.idx, c.L, c.G, b8), dtype=torch.uint8,
                     device=DEV)
    H.haste_tail_prepare_layout(d.X, d.idx, c.L, c.G, ws)
    for rep in range(2):
        b8 = d.bce(c.H, s)
        dW8 = torch.empty_like(d.W)
        dX8 = torch.zeros_like(dX)
        H.haste_tail_prepare(d.X, d.idx, c.L, c.G, b8, ws)
        H.haste_tail_step_dw(d.X, d.idx, d.W, c.L, c.G, b8, dW8, ws, layout_ready=True)
        H.haste_tail_step_dx(d.X, d.idx, d.W, c.L, c.G, b8, dX8, ws, accumulate_dX=True)
        torch.cuda.synchronize()
        assert torch.equal(dW8, dW), f"layout-ready step {rep}: dW differs"
        check_loss(f"layout-ready step loss {rep}", b8.loss.item(), r.loss_tail, "bf16")
        check(f"layout-ready step dX {rep}", to_f64(dX8), r.dX_tail, r.dX_tail_abs, "bf16",
              nterms=ng * c.G)
    # the forward in a workspace of haste_tail_fwd_workspace_bytes (no dz tiles)
    bf_ = d.bce(c.H, s)
    wsf = torch.empty(H.haste_tail_fwd_workspace_bytes(d.X, d.idx, c.L, c.G, bf_), dtype=torch.uint8,
                      device=DEV)
    assert wsf.numel() < ws.numel()
    Zf = torch.empty_like(Z)
    H.haste_tail_fwd(d.X, d.idx, d.W, c.L, c.G, Z=Zf, bce=bf_, workspace=wsf)
    torch.cuda.synchronize()
    assert torch.equal(Zf, Z)
    check_loss("tail fwd loss (forward workspace)", bf_.loss.item(), r.loss_tail, "bf16")

    # fused SGD step: W_out = W - lr * dW, bit for bit the update after the
    # step; against the oracle's W - lr * dW within one bf16 rounding plus
    # lr times the dW tolerance; dX and the loss as the plain step
    lr = 0.5
    Wo = torch.full_like(d.W, 9.0)
    dX7 = torch.empty_like(dX)
    b7 = d.bce(c.H, s)
    H.haste_tail_step_sgd(d.X, d.idx, d.W, c.L, c.G, b7, lr, Wo, dX7)
    Wu = torch.empty_like(d.W)
    H.haste_sgd_update(d.W, dW, lr, Wu)
    torch.cuda.synchronize()
    assert torch.equal(Wo, Wu), "fused and unfused SGD updates differ"
    check_loss("SGD step loss", b7.loss.item(), r.loss_tail, "bf16")
    check("SGD step dX", to_f64(dX7), r.dX_tail, r.dX_tail_abs, "bf16", nterms=ng * c.G)
    Wt64 = inp.W_f64()
    ref = oracle.sgd(Wt64[:c.L], r.dWt, lr)
    got = to_f64(Wo[:c.L])
    # W_out's bf16 rounding, plus lr times (dW's tolerance + dW's bf16 rounding)
    bound = 2.0 ** -8 * np.abs(ref) + lr * (TOL_BF16[0] * r.dWt_abs + TOL_BF16[1] +
                                           2.0 ** -8 * np.abs(r.dWt)) + 1e-30
    bad = np.abs(got - ref) > bound
    assert not bad.any(), f"SGD W_out: {bad.sum()} elements off, worst {np.abs(got - ref)[bad].max()}"
    assert torch.equal(Wo[c.L:], d.W[c.L:]), "padded rows keep W"

    # tail backward, recomputing dz from the positives (no loss added)
    dW3 = torch.empty_like(d.W)
    dX3 = torch.zeros_like(dX)
    b3 = d.bce(c.H, s)
    H.haste_tail_bwd(d.X, d.idx, d.W, c.L, c.G, dW3, dX3, bce=b3)
    torch.cuda.synchronize()
    assert b3.loss.item() == 0.0
    assert torch.equal(dW3, dW)
    check("tail bwd dX", to_f64(dX3), r.dX_tail, r.dX_tail_abs, "bf16", nterms=ng * c.G)
    dX3.zero_()
    H.haste_tail_bwd(d.X, d.idx, d.W, c.L, c.G, dW3, dX3, bce=d.bce(c.H, s), lean=True)
    torch.cuda.synchronize()
    assert torch.equal(dW3, dW)
    check("lean bwd dX", to_f64(dX3), r.dX_tail, r.dX_tail_abs, "bf16", nterms=ng * c.G)

    # tail backward with a given dZ (bf16), accumulating into dX
    dZ_bits = wl.bf16_bits_from_f32(r.dZt.astype(np.float32))
    dZ64 = wl.f64_from_bf16_bits(dZ_bits)
    dZt = dev_array(dZ_bits, "bf16")
    dW4 = torch.empty_like(d.W)
    dX4 = torch.ones_like(dX)
    H.haste_tail_bwd(d.X, d.idx, d.W, c.L, c.G, dW4, dX4, dZ=dZt, accumulate_dX=True)
    torch.cuda.synchronize()
    rW, rWa = oracle.tail_dW(inp.X_f64(), inp.idx, dZ64, c.L, c.G)
    rX, rXa = oracle.tail_dX(inp.idx, inp.W_f64(), dZ64, c.D, c.L, c.G)
    check("tail bwd(dZ) dW", to_f64(dW4[:c.L]), rW, rWa, "bf16", nterms=c.B)
    check("tail bwd(dZ) dX", to_f64(dX4) - 1.0, rX, rXa, "bf16", nterms=ng * c.G)
    # the lean form reads the given dZ in place instead of copying it into tiles
    dW4l = torch.empty_like(d.W)
    dX4l = torch.empty_like(dX)
    H.haste_tail_bwd(d.X, d.idx, d.W, c.L, c.G, dW4l, dX4l, dZ=dZt, lean=True)
    torch.cuda.synchronize()
    check("lean tail bwd(dZ) dW", to_f64(dW4l[:c.L]), rW, rWa, "bf16", nterms=c.B)
    check("lean tail bwd(dZ) dX", to_f64(dX4l), rX, rXa, "bf16", nterms=ng * c.G)

    # head: forward logits + loss, fused step accumulating into the tail's dX
    Zh = torch.empty(c.B, c.H, dtype=bf, device=DEV)
    bh = d.bce(0, s)
    H.haste_head_fwd(d.X, d.Wh, Zh=Zh, bce=bh)
    torch.cuda.synchronize()
    check("head Z", to_f64(Zh), r.Zh, r.Zh_abs, "bf16", nterms=c.D)
    check_loss("head loss", bh.loss.item(), r.loss_head, "bf16")
    dWh = torch.empty_like(d.Wh)
    bh = d.bce(0, s)
    H.haste_head_step(d.X, d.Wh, bh, dWh, dX, accumulate_dX=True)
    torch.cuda.synchronize()
    check_loss("head step loss", bh.loss.item(), r.loss_head, "bf16")
    check("head dW", to_f64(dWh), r.dWh, r.dWh_abs, "bf16", nterms=c.B)
    check("step dX (head+tail)", to_f64(dX), r.dX, r.dX_abs, "bf16", nterms=ng * c.G + c.H)
    # head backward with a given dZh
    dZh_bits = wl.bf16_bits_from_f32(r.dZh.astype(np.float32))
    dZh64 = wl.f64_from_bf16_bits(dZh_bits)
    dWh2 = torch.empty_like(d.Wh)
    dXh = torch.empty_like(dX)
    H.haste_head_bwd(d.X, d.Wh, dWh2, dXh, dZh=dev_array(dZh_bits, "bf16"))
    torch.cuda.synchronize()
    rWh, rWha = oracle.head_dW(inp.X_f64(), dZh64)
    rXh, rXha = oracle.head_dX(inp.Wh_f64(), dZh64)
    check("head bwd(dZ) dW", to_f64(dWh2), rWh, rWha, "bf16", nterms=c.B)
    check("head bwd(dZ) dX", to_f64(dXh), rXh, rXha, "bf16", nterms=c.H)

    # integers: group-major positives, bit-exact
    gp, ent = H.haste_tail_group_positives(c.B, c.D, c.L, c.G, c.F, d.bce(c.H, s))
    rp, re_ = oracle.group_positives(inp.row_ptr, inp.labels, c.H, c.L, c.G)
    torch.cuda.synchronize()
    assert np.array_equal(gp.cpu().numpy(), rp)
    assert np.array_equal(ent.cpu().numpy()[:re_.size], re_)


def test_fp32_c1_full(H):
    """The tiny fp32 workload, every output, at the fp32 tolerance."""
    inp = wl.make_inputs("c1")
    c = inp.cfg
    s = 1.0 / c.B
    r = _ref(inp)
    d = Dev(inp)
    f = torch.float32
    Z = torch.empty(c.B, c.L, dtype=f, device=DEV)
    b = d.bce(c.H, s)
    H.haste_tail_fwd(d.X, d.idx, d.W, c.L, c.G, Z=Z, bce=b)
    dW = torch.empty_like(d.W)
    dX = torch.empty(c.B, c.D, dtype=f, device=DEV)
    b2 = d.bce(c.H, s)
    H.haste_tail_step(d.X, d.idx, d.W, c.L, c.G, b2, dW, dX)
    Zh = torch.empty(c.B, c.H, dtype=f, device=DEV)
    bh = d.bce(0, s)
    H.haste_head_fwd(d.X, d.Wh, Zh=Zh, bce=bh)
    dWh = torch.empty_like(d.Wh)
    bh2 = d.bce(0, s)
    H.haste_head_step(d.X, d.Wh, bh2, dWh, dX, accumulate_dX=True)
    torch.cuda.synchronize()
    check("Z", to_f64(Z), r.Zt, r.Zt_abs, "f32")
    check_loss("tail loss", b.loss.item(), r.loss_tail, "f32")
    check_loss("tail step loss", b2.loss.item(), r.loss_tail, "f32")
    check("dW", to_f64(dW), r.dWt, r.dWt_abs, "f32")
    check("Zh", to_f64(Zh), r.Zh, r.Zh_abs, "f32")
    check_loss("head loss", bh.loss.item(), r.loss_head, "f32")
    check("dWh", to_f64(dWh), r.dWh, r.dWh_abs, "f32")
    check("dX", to_f64(dX), r.dX, r.dX_abs, "f32")


def test_fp32_ragged_groups_of_three(H):
    inp = wl.make_inputs("c1", L=203, G=3, F=7)
    c = inp.cfg
    s = 0.37
    r = oracle.step(inp.X_f64(), inp.Wh_f64(), inp.idx, inp.W_f64(), inp.row_ptr, inp.labels,
                    c.L, c.G, s)
    d = Dev(inp)
    dW = torch.empty_like(d.W)
    dX = torch.empty(c.B, c.D, dtype=torch.float32, device=DEV)
    b = d.bce(c.H, s)
    H.haste_tail_step(d.X, d.idx, d.W, c.L, c.G, b, dW, dX)
    torch.cuda.synchronize()
    check("dW", to_f64(dW[:c.L]), r.dWt, r.dWt_abs, "f32")
    assert torch.all(dW[c.L:] == 0)
    check("dX", to_f64(dX), r.dX_tail, r.dX_tail_abs, "f32")
    check_loss("loss", b.loss.item(), r.loss_tail, "f32")


def test_validate_indices(H):
    inp = wl.make_inputs(wl.tiny("v", L=640, G=16, F=32, D=96))
    idx = inp.idx.copy()
    t = torch.from_numpy(idx).to(DEV)
    assert H.haste_tail_validate(t, 96, 640, 16).item() == -1
    bad = idx.copy()
    bad[17, 3], bad[17, 4] = bad[17, 4], bad[17, 3]      # unsorted row
    bad[30, 0] = 96                                      # out of range
    t = torch.from_numpy(bad).to(DEV)
    assert H.haste_tail_validate(t, 96, 640, 16).item() == 17
    bad[17] = idx[17]
    t = torch.from_numpy(bad).to(DEV)
    assert H.haste_tail_validate(t, 96, 640, 16).item() == 30


def test_topk_merge_exact(H):
    rng = np.random.default_rng(4)
    B, K = 37, 5
    va = np.round(rng.standard_normal((B, 40)) * 2) / 2
    ids = np.arange(80).reshape(2, 40)
    # each side's own top-K (oracle order), then merge both on the GPU
    av, ai = oracle.topk(va, K, id_offset=0)
    vb = np.round(rng.standard_normal((B, 40)) * 2) / 2
    bv, bi = oracle.topk(vb, K, id_offset=40)
    ov, oi = H.haste_topk_merge(*(torch.tensor(x, dtype=dt, device=DEV) for x, dt in
                                  ((av, torch.float32), (ai, torch.int32),
                                   (bv, torch.float32), (bi, torch.int32))))
    full = np.concatenate([va, vb], 1)
    rv, ri = oracle.topk(full, K, ids=ids.reshape(-1))
    assert np.array_equal(oi.cpu().numpy(), ri)
    assert np.array_equal(ov.cpu().numpy(), rv.astype(np.float32))


@pytest.mark.parametrize("B,L,G,per_row,dup,dtype", [
    (3, 40, 16, 0, False, torch.bfloat16),       # no positives at all
    (70, 300, 64, 4, True, torch.bfloat16),      # duplicates, ragged last group
    (1100, 5000, 16, 5, True, torch.bfloat16),   # more keys than one LDS chunk
    (2000, 9000, 32, 6, True, torch.bfloat16),   # 7,557 keys: a 30 x 30 grid of rank tiles
    (600, 777, 3, 7, True, torch.float32),       # fp32 desc, groups of three
])
def test_group_positives_edges(H, B, L, G, per_row, dup, dtype):
    """Group-major positives, bit-exact against the oracle: labels below and
    above the tail range, empty rows, a label listed twice in a row (both
    entries kept, in input order), and key counts spanning several chunks."""
    print("group positives", B, L, G, per_row, dup, flush=True)
    rng = np.random.default_rng(B * 7 + L)
    off = 50
    counts = rng.integers(0, per_row + 1, size=B) if per_row else np.zeros(B, np.int64)
    labels = []
    for b in range(B):
        row = list(rng.integers(0, off + L + 30, size=int(counts[b])))
        if dup and row:
            row.append(row[0])
        labels += row
    row_ptr = np.zeros(B + 1, np.int32)
    for b in range(B):
        n = int(counts[b]) + (1 if dup and counts[b] else 0)
        row_ptr[b + 1] = row_ptr[b] + n
    labels = np.array(labels, np.int32)
    assert labels.size == row_ptr[-1]
    rp, re_ = oracle.group_positives(row_ptr, labels, off, L, G)
    bce = H.Bce(torch.from_numpy(row_ptr).to(DEV), torch.from_numpy(labels).to(DEV), off, 1.0)
    gp, ent = H.haste_tail_group_positives(B, 128, L, G, 32, bce, dtype=dtype)
    torch.cuda.synchronize()
    assert np.array_equal(gp.cpu().numpy(), rp)
    assert np.array_equal(ent.cpu().numpy()[:re_.size], re_)


FANIN1 = [
    dict(B=40, D=96, H=48, L=300, G=1, F=32),
    dict(B=70, D=768, H=64, L=1500, G=1, F=128),
    dict(B=33, D=1024, H=64, L=700, G=1, F=64, idx_dist="skew10"),
]


@pytest.mark.parametrize("case", FANIN1, ids=[_ids(c) for c in FANIN1])
def test_bf16_fixed_fan_in_forward(H, case):
    """G = 1 (every label its own F indices; the per-label fixed fan-in the
    HASTE page compares against): logits and loss of haste_tail_fwd against
    the oracle, which at G = 1 is the fixed fan-in loop (pin P1)."""
    print("case", case, flush=True)
    inp = wl.make_inputs(wl.tiny("g1", **case))
    c = inp.cfg
    s = 1.0 / c.B
    X, Wt = inp.X_f64(), inp.W_f64()
    Zr, Zra = oracle.tail_logits(X, inp.idx, Wt, c.L, c.G, want_abs=True)
    Y = oracle.positive_mask(inp.row_ptr, inp.labels, c.H, c.L)
    _, lt = oracle.bce(Zr, Y, s)
    d = Dev(inp)
    Z = torch.empty(c.B, c.L, dtype=torch.bfloat16, device=DEV)
    b = d.bce(c.H, s)
    H.haste_tail_fwd(d.X, d.idx, d.W, c.L, c.G, Z=Z, bce=b)
    torch.cuda.synchronize()
    check("G=1 Z", to_f64(Z), Zr, Zra, "bf16", nterms=c.F)
    check_loss("G=1 loss", b.loss.item(), float(lt.sum()), "bf16")
    b2 = d.bce(c.H, s)
    H.haste_tail_fwd(d.X, d.idx, d.W, c.L, c.G, bce=b2)     # loss only, no Z
    torch.cuda.synchronize()
    check_loss("G=1 loss (no Z)", b2.loss.item(), float(lt.sum()), "bf16")


FANIN1_STEP = [
    dict(B=40, D=96, H=48, L=300, G=1, F=32),
    dict(B=70, D=768, H=64, L=1500, G=1, F=128),
    dict(B=33, D=960, H=64, L=700, G=1, F=64, idx_dist="skew10"),
    dict(B=130, D=200, H=64, L=77, G=1, F=64, pos_per_row=6),
]


@pytest.mark.parametrize("case", FANIN1_STEP, ids=[_ids(c) for c in FANIN1_STEP])
def test_bf16_fixed_fan_in_step(H, case):
    """G = 1 training step (haste_tail_step): loss, dW and dX against the
    oracle at G = 1; dW twice, bit for bit (no atomics on it)."""
    print("case", case, flush=True)
    inp = wl.make_inputs(wl.tiny("g1s", **case))
    c = inp.cfg
    s = 1.0 / c.B
    X, Wt = inp.X_f64(), inp.W_f64()
    Zr, _ = oracle.tail_logits(X, inp.idx, Wt, c.L, c.G, want_abs=False)
    Y = oracle.positive_mask(inp.row_ptr, inp.labels, c.H, c.L)
    dZ, lt = oracle.bce(Zr, Y, s)
    rW, rWa = oracle.tail_dW(X, inp.idx, dZ, c.L, c.G)
    rX, rXa = oracle.tail_dX(inp.idx, Wt, dZ, c.D, c.L, c.G)
    d = Dev(inp)
    outs = []
    for _ in range(2):
        dW = torch.full_like(d.W, 3.0)
        dX = torch.full((c.B, c.D), 5.0, dtype=torch.float32, device=DEV)
        b = d.bce(c.H, s)
        H.haste_tail_step(d.X, d.idx, d.W, c.L, c.G, b, dW, dX)
        torch.cuda.synchronize()
        outs.append((dW, dX, b.loss.item()))
    dW, dX, loss = outs[0]
    check_loss("G=1 step loss", loss, float(lt.sum()), "bf16")
    check("G=1 step dW", to_f64(dW[:c.L]), rW, rWa, "bf16", nterms=c.B)
    check("G=1 step dX", to_f64(dX), rX, rXa, "bf16", nterms=c.L)
    assert torch.equal(outs[0][0], outs[1][0]), "G=1 dW differs between calls"


def test_mfma_probe_runs(H):
    """The measurement probe (not a step of the layer) launches and completes;
    its flop count is blocks x 4 waves x iters x 16 MFMAs of 16x16x32x2."""
    print("case mfma probe", flush=True)
    sink = torch.zeros(1, dtype=torch.float32, device=DEV)
    flops = H.haste_probe_mfma(8, 4, sink)
    torch.cuda.synchronize()
    assert flops == 8 * 4 * 4 * 16 * (16 * 16 * 32 * 2)
    assert sink.item() == 0.0


def _far_below_zero(case, zmean=-15.0):
    """A workload whose every logit lies far below zero (about zmean): X
    shifted positive, all weights negative.  No positives, so the loss is a
    sum of tiny softplus terms, each about e^zmean."""
    inp = wl.make_inputs(wl.tiny("neg", pos_per_row=0, **case))
    c = inp.cfg
    x = np.abs(wl.f64_from_bf16_bits(inp.X)) + 0.5
    inp.X = wl.bf16_bits_from_f32(x.astype(np.float32))
    ex = float(np.mean(wl.f64_from_bf16_bits(inp.X)))
    for name, n in (("W", c.F), ("Wh", c.D)):
        w = wl.f64_from_bf16_bits(getattr(inp, name))
        w = -(1.0 + np.abs(w) / c.w_std) * (-zmean / (n * ex * (1.0 + np.sqrt(2.0 / np.pi))))
        setattr(inp, name, wl.bf16_bits_from_f32(w.astype(np.float32)))
    return inp


@pytest.mark.parametrize("case", [dict(B=64, D=128, H=64, L=500, G=16, F=32),
                                  dict(B=48, D=256, H=64, L=700, G=64, F=64)],
                         ids=["G16", "G64"])
def test_loss_with_logits_far_below_zero(H, case):
    """Each softplus term is about 3e-7 here, below the spacing of floats
    near 1: the loss must not round the (1 + e^-|z|) factors against 1.
    Tail forward, tail step and head step, within reading C16's relative
    bound alone (the losses are far below its absolute slack of 1e-6)."""
    print("case far below zero", case, flush=True)
    inp = _far_below_zero(case)
    c = inp.cfg
    s = 1.0 / c.B
    r = _ref(inp)
    assert np.max(r.Zt) < -5.0 and np.max(r.Zh) < -5.0
    d = Dev(inp)

    def _rel(name, got, ref):
        err = abs(got - ref) / ref
        print(f"  far below zero, {name}: relative error {err:.2e}", flush=True)
        assert err <= 1e-4, f"{name}: got {got} ref {ref}"

    b = d.bce(c.H, s)
    H.haste_tail_fwd(d.X, d.idx, d.W, c.L, c.G, bce=b)
    torch.cuda.synchronize()
    _rel("tail fwd loss", b.loss.item(), r.loss_tail)
    dW = torch.empty_like(d.W)
    dX = torch.empty((c.B, c.D), dtype=torch.float32, device=DEV)
    b = d.bce(c.H, s)
    H.haste_tail_step(d.X, d.idx, d.W, c.L, c.G, b, dW, dX)
    torch.cuda.synchronize()
    _rel("tail step loss", b.loss.item(), r.loss_tail)
    bh = d.bce(0, s)
    dWh = torch.empty_like(d.Wh)
    H.haste_head_step(d.X, d.Wh, bh, dWh, dX, accumulate_dX=True)
    torch.cuda.synchronize()
    _rel("head step loss", bh.loss.item(), r.loss_head)


@pytest.mark.parametrize("case", [dict(B=37, D=100, H=40, L=300, G=16, F=32),
                                  dict(B=70, D=203, H=40, L=500, G=64, F=64)],
                         ids=["D100-G16", "D203-G64"])
def test_feature_count_not_a_multiple_of_eight(H, case):
    """The tail alone (the bf16 head takes D in multiples of 8 only) on rows of
    X that are not whole 16-byte pieces, and a feature count that is not a
    whole number of the dX kernels' feature tiles.  Forward, one-call step
    and the split step."""
    print("case odd D", case, flush=True)
    inp = wl.make_inputs(wl.tiny("odd", **case))
    c = inp.cfg
    s = 1.0 / c.B
    r = _ref(inp)
    d = Dev(inp)
    ng = c.n_groups
    Z = torch.empty(c.B, c.L, dtype=torch.bfloat16, device=DEV)
    b = d.bce(c.H, s)
    H.haste_tail_fwd(d.X, d.idx, d.W, c.L, c.G, Z=Z, bce=b)
    torch.cuda.synchronize()
    check("odd-D tail Z", to_f64(Z), r.Zt, r.Zt_abs, "bf16", nterms=c.F)
    check_loss("odd-D tail fwd loss", b.loss.item(), r.loss_tail, "bf16")
    dW = torch.empty_like(d.W)
    dX = torch.empty((c.B, c.D), dtype=torch.float32, device=DEV)
    b = d.bce(c.H, s)
    H.haste_tail_step(d.X, d.idx, d.W, c.L, c.G, b, dW, dX)
    torch.cuda.synchronize()
    check_loss("odd-D step loss", b.loss.item(), r.loss_tail, "bf16")
    check("odd-D dW", to_f64(dW[:c.L]), r.dWt, r.dWt_abs, "bf16", nterms=c.B)
    check("odd-D dX", to_f64(dX), r.dX_tail, r.dX_tail_abs, "bf16", nterms=ng * c.G)
    b5 = d.bce(c.H, s)
    ws = torch.empty(H.haste_tail_workspace_bytes(d.X, d.idx, c.L, c.G, b5), dtype=torch.uint8,
                     device=DEV)
    dW5 = torch.empty_like(d.W)
    dX5 = torch.zeros_like(dX)
    H.haste_tail_prepare(d.X, d.idx, c.L, c.G, b5, ws)
    H.haste_tail_step_dw(d.X, d.idx, d.W, c.L, c.G, b5, dW5, ws)
    H.haste_tail_step_dx(d.X, d.idx, d.W, c.L, c.G, b5, dX5, ws, accumulate_dX=True)
    torch.cuda.synchronize()
    assert torch.equal(dW5, dW)
    check("odd-D split dX", to_f64(dX5), r.dX_tail, r.dX_tail_abs, "bf16", nterms=ng * c.G)


@pytest.mark.parametrize("case", [dict(B=70, D=200, H=56, L=300, G=64, F=128),
                                  dict(B=40, D=96, H=48, L=200, G=16, F=32),
                                  dict(B=33, D=1024, H=96, L=700, G=64, F=64)],
                         ids=["G64-F128-dense", "G16-F32-dense", "G64-F64-scatter"])
def test_padded_weight_rows_never_reach_a_result(H, case):
    """Rows of W past L (the padding of a ragged last group) are never read
    for a result: filled with NaN, they must leave the loss, logits, dW of
    the live rows and dX as the oracle has them, in every form of the dX pass
    (dense from the tiles, lean, scatter) and through the exact top-K."""
    print("case", case, flush=True)
    inp = wl.make_inputs(wl.tiny("pad", **case))
    c = inp.cfg
    assert c.L % c.G != 0
    s = 1.0 / c.B
    r = _ref(inp)
    d = Dev(inp)
    d.W[c.L:] = float("nan")
    ng = c.n_groups
    for lean in (False, True):
        dW = torch.empty_like(d.W)
        dX = torch.empty(c.B, c.D, dtype=torch.float32, device=DEV)
        b = d.bce(c.H, s)
        H.haste_tail_step(d.X, d.idx, d.W, c.L, c.G, b, dW, dX, lean=lean)
        torch.cuda.synchronize()
        check_loss(f"padded-NaN step loss (lean={lean})", b.loss.item(), r.loss_tail, "bf16")
        check(f"padded-NaN dW (lean={lean})", to_f64(dW[:c.L]), r.dWt, r.dWt_abs, "bf16", nterms=c.B)
        assert torch.all(dW[c.L:] == 0)
        check(f"padded-NaN dX (lean={lean})", to_f64(dX), r.dX_tail, r.dX_tail_abs, "bf16",
              nterms=ng * c.G)
    Z = torch.empty(c.B, c.L, dtype=torch.bfloat16, device=DEV)
    b = d.bce(c.H, s)
    b.topk_val = torch.empty(c.B, 5, dtype=torch.float32, device=DEV)
    b.topk_idx = torch.empty(c.B, 5, dtype=torch.int32, device=DEV)
    H.haste_tail_fwd(d.X, d.idx, d.W, c.L, c.G, Z=Z, bce=b)
    torch.cuda.synchronize()
    check("padded-NaN Z", to_f64(Z), r.Zt, r.Zt_abs, "bf16", nterms=c.F)
    assert torch.all(torch.isfinite(b.topk_val))
    assert int(b.topk_idx.min()) >= c.H and int(b.topk_idx.max()) < c.H + c.L
