"""Parity at the workloads' full sizes, in the calls that bench.py times
(haste_head_step, haste_tail_prepare, haste_tail_step_dw and
haste_tail_step_dx, head and tail accumulating into one dX), made one after
another on one stream; test_overlapped_steps then checks that the
arrangement bench.py times, the head on a second stream beside the tail,
gives the same outputs on every call.  The oracle cannot evaluate these
steps whole in test time, so the checks are on outputs it computes one by
one:

  - dW of sampled tail groups (all rows), including the ragged last group;
  - dWh of sampled head labels (all rows);
  - dX of sampled rows (all head and tail labels);
  - the total loss, streamed over chunks of groups.

The 8.6M-label workload also asks for the per-row top-5 over all labels
(head and tail lists merged); its oracle is streamed over the same chunks
of groups as the loss, and so is the two-stage oracle of the inference form
(stage 1 inside the logits pass, one bucket per label group, K' = 1).  The 3M-label workload runs the lean form (dz
recomputed in the dX pass, nothing of size B x L stored); the others keep
the dz tiles."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from _gpu import DEV, Dev, check, check_loss, check_topk_lists, rank_tol, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def H():
    from sparse_output_layer_amd import haste
    haste.lib()
    return haste


def _sample(n, fixed, extra, rng):
    pick = [i for i in fixed if 0 <= i < n] + list(rng.integers(0, n, size=extra))
    return np.array(sorted(set(int(i) for i in pick)), dtype=np.int32)


@pytest.mark.parametrize("name", ["c2", "c3", "c4", "c5"])
def test_full_size_step(H, name):
    print("full-size step", name, flush=True)
    cfg = wl.CONFIGS[name]
    K = cfg.topk
    inp = wl.make_inputs(cfg)
    c = inp.cfg
    B, D, L, G, Hn = c.B, c.D, c.L, c.G, c.H
    ng = c.n_groups
    s = 1.0 / B
    d = Dev(inp)
    lean = name == "c4"

    # the benchmark's step
    loss = torch.zeros(1, dtype=torch.float32, device=DEV)
    bh = H.Bce(d.row_ptr, d.labels, 0, s, loss)
    bt = H.Bce(d.row_ptr, d.labels, Hn, s, loss)
    if K:
        bh.topk_val = torch.empty(B, K, dtype=torch.float32, device=DEV)
        bh.topk_idx = torch.empty(B, K, dtype=torch.int32, device=DEV)
        bt.topk_val = torch.empty_like(bh.topk_val)
        bt.topk_idx = torch.empty_like(bh.topk_idx)
    dX = torch.empty(B, D, dtype=torch.float32, device=DEV)
    dWh = torch.empty_like(d.Wh)
    dW = torch.empty_like(d.W)
    ws_t = torch.empty(H.haste_tail_workspace_bytes(d.X, d.idx, L, G, bt, lean=lean),
                       dtype=torch.uint8, device=DEV)
    ws_h = torch.empty(max(256, H.haste_head_workspace_bytes(d.X, d.Wh, bh)), dtype=torch.uint8,
                       device=DEV)
    H.haste_head_step(d.X, d.Wh, bh, dWh, dX, workspace=ws_h)
    H.haste_tail_prepare(d.X, d.idx, L, G, bt, ws_t, lean=lean)
    H.haste_tail_step_dw(d.X, d.idx, d.W, L, G, bt, dW, ws_t, lean=lean)
    H.haste_tail_step_dx(d.X, d.idx, d.W, L, G, bt, dX, ws_t, accumulate_dX=True, lean=lean)
    if K:
        mv, mi = H.haste_topk_merge(bh.topk_val, bh.topk_idx, bt.topk_val, bt.topk_idx)
        # the inference form: top-K stage 1 inside the logits pass (one bucket
        # per label group, K' = 1), merged with the head's exact lists
        bf = H.Bce(d.row_ptr, d.labels, Hn, s, topk_kprime=1, topk_buckets=ng)
        bf.topk_val = torch.empty_like(bh.topk_val)
        bf.topk_idx = torch.empty_like(bh.topk_idx)
        H.haste_tail_fwd(d.X, d.idx, d.W, L, G, bce=bf)
        fv, fi = H.haste_topk_merge(bh.topk_val, bh.topk_idx, bf.topk_val, bf.topk_idx)
    torch.cuda.synchronize()
    print("  GPU step done", flush=True)

    X = inp.X_f64()
    Wt = inp.W_f64()
    Wh = inp.Wh_f64()
    rng = np.random.default_rng(12345)
    gp, _ = oracle.group_positives(inp.row_ptr, inp.labels, Hn, L, G)
    with_pos = np.nonzero(np.diff(gp) > 0)[0]

    # dW of sampled groups (all rows); padded label rows must be zero
    groups = _sample(ng, [0, 1, ng // 2, ng - 1] + list(with_pos[:3]), 3, rng)
    dW_h = dW.view(torch.int16).cpu().numpy().view(np.uint16)
    for g in groups:
        g = int(g)
        Z, _ = oracle.tail_logits(X, inp.idx, Wt, L, G, g0=g, g1=g + 1, want_abs=False)
        nl = Z.shape[1]
        Y = oracle.positive_mask(inp.row_ptr, inp.labels, Hn + g * G, nl)
        dz, _ = oracle.bce(Z, Y, s)
        rW, rWa = oracle.tail_dW(X, inp.idx, dz, L, G, g0=g, g1=g + 1)
        got = wl.f64_from_bf16_bits(dW_h[g * G:g * G + nl])
        check(f"dW group {g}", got, rW, rWa, "bf16", nterms=B)
        assert np.all(dW_h[g * G + nl:(g + 1) * G] == 0), f"padded rows of group {g}"

    # head: logits of all rows (small), dWh of sampled labels
    Zh, _ = oracle.head_logits(X, Wh, want_abs=False)
    Yh = oracle.positive_mask(inp.row_ptr, inp.labels, 0, Hn)
    dzh, lth = oracle.bce(Zh, Yh, s)
    labs = _sample(Hn, [0, 1, Hn // 2, Hn - 1], 4, rng)
    rWh, rWha = oracle.head_dW(X, dzh[:, labs])
    got = to_f64(dWh[torch.from_numpy(labs).long().to(DEV)])
    check("dWh sampled labels", got, rWh, rWha, "bf16", nterms=B)

    # dX of sampled rows over every head and tail label
    rows = _sample(B, [0, 1, B // 2, B - 1], 2, rng)
    Zr, _ = oracle.tail_logits(X, inp.idx, Wt, L, G, rows=rows, want_abs=False)
    Yr = oracle.positive_mask(inp.row_ptr, inp.labels, Hn, L, rows=rows)
    dzr, _ = oracle.bce(Zr, Yr, s)
    rXt, rXta = oracle.tail_dX(inp.idx, Wt, dzr, D, L, G)
    rXh, rXha = oracle.head_dX(Wh, dzh[rows])
    got = to_f64(dX[torch.from_numpy(rows).long().to(DEV)])
    check("dX sampled rows", got, rXt + rXh, rXta + rXha, "bf16", nterms=ng * G + Hn)
    print("  sampled outputs match", flush=True)

    # total loss: head from the full head logits, tail streamed over groups;
    # with a top-K, the running top-(K+1) of every row rides along, each entry
    # with its rank tolerance (reading C17); for the two-stage form (buckets =
    # label groups, K' = 1) each group's representative also records whether
    # its group's second logit lies within the two tolerances of it
    ref_loss = float(lth.sum())
    if K:
        Zh_full, Zha_full = oracle.head_logits(X, Wh, want_abs=True)
        rth = rank_tol(Zha_full, D)
        tv_, ti_ = oracle.topk(Zh_full, K + 1, id_offset=0)
        tt_ = np.take_along_axis(rth, ti_, axis=1)
        tf_, tfi_, tft_ = tv_.copy(), ti_.copy(), tt_.copy()
        tfa_ = np.zeros(tv_.shape, bool)
    chunk = max(1, (1 << 24) // (B * G))
    for g0 in range(0, ng, chunk):
        g1 = min(ng, g0 + chunk)
        Z, Za = oracle.tail_logits(X, inp.idx, Wt, L, G, g0=g0, g1=g1, want_abs=bool(K))
        Y = oracle.positive_mask(inp.row_ptr, inp.labels, Hn + g0 * G, Z.shape[1])
        _, lt = oracle.bce(Z, Y, s)
        ref_loss += float(lt.sum())
        if K:
            off = Hn + g0 * G
            rt = rank_tol(Za, c.F)
            cv, ci = oracle.topk(Z, min(K + 1, Z.shape[1]), id_offset=off)
            ct = np.take_along_axis(rt, ci - off, axis=1)
            tv_, ti_, tt_, _ = _merge_lists(tv_, ti_, tt_, None, cv, ci, ct, None, K + 1)
            # two-stage lists of the chunk's whole groups (buckets of G labels)
            sv, si = oracle.topk_two_stage(Z, K, 1, G, id_offset=off)
            st = np.take_along_axis(rt, np.maximum(si - off, 0), axis=1)
            sa = np.zeros(sv.shape, bool)
            for b_ in range(B):
                for k_ in range(sv.shape[1]):
                    if si[b_, k_] < 0:
                        continue
                    c0 = (si[b_, k_] - off) // G * G
                    c1 = min(c0 + G, Z.shape[1])
                    if c1 - c0 > 1:
                        zz = Z[b_, c0:c1]
                        o2 = np.argsort(-zz, kind="stable")[:2]
                        sa[b_, k_] = zz[o2[0]] - zz[o2[1]] <= rt[b_, c0 + o2[0]] + rt[b_, c0 + o2[1]]
            tf_, tfi_, tft_, tfa_ = _merge_lists(tf_, tfi_, tft_, tfa_, sv, si, st, sa, K + 1)
    check_loss("step loss", loss.item(), ref_loss, "bf16")
    if K:
        def zfun(b, gid):
            if gid < Hn:
                z, za = oracle.head_logits(X, Wh, rows=np.array([b], np.int32), h0=gid, h1=gid + 1)
                return float(z[0, 0]), float(rank_tol(za[0, 0], D))
            t = gid - Hn
            g = t // G
            Zg, Zga = oracle.tail_logits(X, inp.idx, Wt, L, G, rows=np.array([b], np.int32),
                                         g0=g, g1=g + 1)
            return float(Zg[0, t - g * G]), float(rank_tol(Zga[0, t - g * G], c.F))
        rows_ok, pos = check_topk_lists("merged top-K", mv.cpu().numpy(), mi.cpu().numpy(), tv_, ti_,
                                        tt_, zfun, K, Hn + L)
        print(f"  exact top-{K}: tie-free rows {rows_ok} of {B}, positions compared by id {pos} "
              f"of {B * K}", flush=True)
        assert rows_ok >= (90 * B) // 128, rows_ok
        rows_f, pos_f = check_topk_lists("merged top-K, stage 1 fused", fv.cpu().numpy(), fi.cpu().numpy(),
                                         tf_, tfi_, tft_, zfun, K, Hn + L, oamb=tfa_)
        print(f"  fused stage 1: tie-free rows {rows_f} of {B}, positions compared by id {pos_f} "
              f"of {B * K}", flush=True)
        print("  top-K matches (exact and fused stage 1)", flush=True)


def _merge_lists(av, ai, at, aa, bv, bi, bt, ba, n):
    """First n of the union of two per-row lists (value desc, ties to the
    smaller id), by the oracle's own selection over the concatenation; the
    per-entry tolerances (and ambiguity flags, when given) follow their ids."""
    v = np.concatenate([av, bv], axis=1)
    i = np.concatenate([ai, bi], axis=1)
    t = np.concatenate([at, bt], axis=1)
    am = np.concatenate([aa, ba], axis=1) if aa is not None else None
    out_v = np.empty((v.shape[0], n))
    out_i = np.empty((v.shape[0], n), np.int64)
    out_t = np.zeros((v.shape[0], n))
    out_a = np.zeros((v.shape[0], n), bool) if am is not None else None
    for r in range(v.shape[0]):
        ov, oi = oracle.topk(v[r:r + 1], n, ids=i[r])
        out_v[r], out_i[r] = ov[0], oi[0]
        pos = {int(x): p for p, x in reversed(list(enumerate(i[r])))}
        for k in range(n):
            if oi[0, k] >= 0:
                out_t[r, k] = t[r, pos[int(oi[0, k])]]
                if am is not None:
                    out_a[r, k] = am[r, pos[int(oi[0, k])]]
    return out_v, out_i, out_t, out_a


@pytest.mark.parametrize("name", ["c2", "c5"])
def test_overlapped_steps(H, name):
    """The head's step on a second stream beside the tail's calls, repeated:
    every call's dW and dWh equal those of the calls made in order on one
    stream, bit for bit, and dX (fp32 atomics from both sides, in an order
    that varies) agrees to a small multiple of fp32 rounding.  Two
    arrangements: the head launched once the tail's prep is done, and at the
    very start of the step (as bench.py times it), beside the prep kernels,
    whose LDS traffic slows the head GEMM's LDS reads; a GEMM barrier that
    did not wait for those reads gave a wrong dX tile in about one call in
    thirty there.  The 8.6M-label workload adds its per-row top-5 lists
    (head and tail merged after both streams meet), compared bit for bit."""
    print("overlapped steps", name, flush=True)
    inp = wl.make_inputs(wl.CONFIGS[name])
    c = inp.cfg
    B, D, L, G, Hn = c.B, c.D, c.L, c.G, c.H
    s = 1.0 / B
    d = Dev(inp)
    loss = torch.zeros(1, dtype=torch.float32, device=DEV)
    bh = H.Bce(d.row_ptr, d.labels, 0, s, loss)
    bt = H.Bce(d.row_ptr, d.labels, Hn, s, loss)
    K = c.topk
    if K:
        for b_ in (bh, bt):
            b_.topk_val = torch.empty(B, K, dtype=torch.float32, device=DEV)
            b_.topk_idx = torch.empty(B, K, dtype=torch.int32, device=DEV)
    dX = torch.empty(B, D, dtype=torch.float32, device=DEV)
    dWh = torch.empty_like(d.Wh)
    dW = torch.empty_like(d.W)
    ws_t = torch.empty(H.haste_tail_workspace_bytes(d.X, d.idx, L, G, bt), dtype=torch.uint8,
                       device=DEV)
    ws_h = torch.empty(max(256, H.haste_head_workspace_bytes(d.X, d.Wh, bh)), dtype=torch.uint8,
                       device=DEV)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()

    def tail_prep():
        H.haste_tail_prepare(d.X, d.idx, L, G, bt, ws_t)

    def tail_rest():
        H.haste_tail_step_dw(d.X, d.idx, d.W, L, G, bt, dW, ws_t)
        H.haste_tail_step_dx(d.X, d.idx, d.W, L, G, bt, dX, ws_t, accumulate_dX=True)

    def head_on_side():
        with torch.cuda.stream(side):
            H.haste_head_step(d.X, d.Wh, bh, dWh, dX, accumulate_dX=True, workspace=ws_h)

    def merged():
        return H.haste_topk_merge(bh.topk_val, bh.topk_idx, bt.topk_val, bt.topk_idx) if K else None

    def in_order():
        loss.zero_()
        H.haste_head_step(d.X, d.Wh, bh, dWh, dX, workspace=ws_h)
        tail_prep()
        tail_rest()
        return merged()

    def after_prep():
        loss.zero_()
        dX.zero_()
        tail_prep()
        ev = torch.cuda.Event()
        ev.record(main)
        side.wait_event(ev)
        head_on_side()
        tail_rest()
        main.wait_stream(side)
        return merged()

    def at_start():
        loss.zero_()
        dX.zero_()
        side.wait_stream(main)
        head_on_side()
        tail_prep()
        tail_rest()
        main.wait_stream(side)
        return merged()

    ref_tk = in_order()
    torch.cuda.synchronize()
    ref_dx, ref_dw, ref_dwh = dX.clone(), dW.view(torch.int16).clone(), dWh.view(torch.int16).clone()
    tol = 1e-5 * float(ref_dx.abs().max())
    for name, f in (("after prep", after_prep), ("at start", at_start)):
        bad = []
        for it in range(120):
            tk = f()
            torch.cuda.synchronize()
            err = float((dX - ref_dx).abs().max())
            same_w = torch.equal(dW.view(torch.int16), ref_dw)
            same_wh = torch.equal(dWh.view(torch.int16), ref_dwh)
            same_tk = not K or (torch.equal(tk[0], ref_tk[0]) and torch.equal(tk[1], ref_tk[1]))
            if err > tol or not same_w or not same_wh or not same_tk:
                bad.append((it, err, same_w, same_wh, same_tk))
        print(f"  head {name}: 120 calls, {len(bad)} differ (dX tol {tol:.2e})", flush=True)
        assert not bad, f"head {name}: (call, dX max diff, dW, dWh, top-K equal) {bad[:5]}"
