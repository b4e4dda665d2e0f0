"""Pins for the fp64 oracle: each test checks it against something other than
itself -- a special case that reduces to a library routine, a closed form,
exact integer arithmetic, finite differences, or brute force on tiny inputs.
A plausible mistake anywhere in the oracle (dropped term, wrong sign, wrong
index, transposed operand, ragged-group slip) fails at least one of them.

Method source: HASTE summary page (gist.science), section "Method":
item 1 (group-shared fixed fan-in; indices stored once per group), item 2
(dense head classifier); section "Results" (group sizes 16 and 64).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _f64(inp):
    return inp.X_f64(), inp.Wh_f64(), inp.W_f64()


# --------------------------------------------------------------------- P1
def test_p1_group_size_one_is_fixed_fan_in():
    """Method item 1: standard fixed fan-in gives every label its own index
    set; with G=1 the group-shared layer must be exactly that layer.  The
    fixed fan-in reference below is written per label, accumulating in f
    order like the oracle, so the fp64 results agree bit for bit."""
    cfg = wl.tiny("p1", B=7, D=50, L=37, G=1, F=9, dtype="f32", H=4)
    inp = wl.make_inputs(cfg)
    X, _, W = _f64(inp)
    Z, _ = oracle.tail_logits(X, inp.idx, W, cfg.L, cfg.G)
    ref = np.zeros((cfg.B, cfg.L))
    for t in range(cfg.L):                 # label t owns index row t
        cols = inp.idx[t]
        acc = np.zeros(cfg.B)
        for f in range(cfg.F):
            acc = acc + X[:, cols[f]] * W[t, f]
        ref[:, t] = acc
    assert np.array_equal(Z, ref)
    # gradient of the fixed fan-in layer, per label, in b order
    dZ = np.random.default_rng(1).standard_normal((cfg.B, cfg.L))
    dW, _ = oracle.tail_dW(X, inp.idx, dZ, cfg.L, cfg.G)
    ref_dW = np.zeros((cfg.L, cfg.F))
    for t in range(cfg.L):
        for f in range(cfg.F):
            acc = 0.0
            for b in range(cfg.B):
                acc += X[b, inp.idx[t, f]] * dZ[b, t]
            ref_dW[t, f] = acc
    assert np.array_equal(dW, ref_dW)


# --------------------------------------------------------------------- P2
@pytest.mark.parametrize("G", [1, 4, 16])
def test_p2_full_fan_in_is_dense_matmul(G):
    """Gather-once + dense MMA (Method item 1, 'hardware alignment'): with
    F = D and the identity index set the layer is a plain dense classifier,
    i.e. numpy's matmul, for logits and both gradients."""
    B, D, L = 9, 24, 8 * G + (3 if G > 1 else 0)
    rng = np.random.default_rng(G)
    X = rng.standard_normal((B, D))
    ng = (L + G - 1) // G
    idx = np.tile(np.arange(D, dtype=np.int32), (ng, 1))
    Wt = rng.standard_normal((ng * G, D))
    Z, Za = oracle.tail_logits(X, idx, Wt, L, G)
    ref = X @ Wt[:L].T
    assert np.allclose(Z, ref, rtol=0, atol=1e-12 * Za.max())
    dZ = rng.standard_normal((B, L))
    dW, dWa = oracle.tail_dW(X, idx, dZ, L, G)
    assert np.allclose(dW, dZ.T @ X, rtol=0, atol=1e-12 * dWa.max())
    dX, dXa = oracle.tail_dX(idx, Wt, dZ, D, L, G)
    assert np.allclose(dX, dZ @ Wt[:L], rtol=0, atol=1e-12 * dXa.max())
    # the head is the same dense layer
    Zh, Zha = oracle.head_logits(X, Wt[:L])
    assert np.allclose(Zh, ref, rtol=0, atol=1e-12 * Zha.max())
    dWh, _ = oracle.head_dW(X, dZ)
    assert np.allclose(dWh, dZ.T @ X, rtol=0, atol=1e-12 * dWa.max())
    dXh, _ = oracle.head_dX(Wt[:L], dZ)
    assert np.allclose(dXh, dZ @ Wt[:L], rtol=0, atol=1e-12 * dXa.max())


# --------------------------------------------------------------------- P3
def _masked_dense_step(X, Wh, idx, Wt, row_ptr, labels, L, G, s):
    """The same layer written as a dense masked-weight model in torch fp64,
    differentiated by autograd; BCE from torch's library routine."""
    B, D = X.shape
    H = Wh.shape[0]
    ng = idx.shape[0]
    Wd = torch.zeros(L, D, dtype=torch.float64)
    M = torch.zeros(L, D, dtype=torch.float64)
    for t in range(L):
        Wd[t, idx[t // G]] = torch.from_numpy(Wt[t])
        M[t, idx[t // G]] = 1.0
    Wd.requires_grad_(True)
    Xt = torch.from_numpy(X).clone().requires_grad_(True)
    Wht = torch.from_numpy(Wh).clone().requires_grad_(True)
    zt = Xt @ (Wd * M).T
    zh = Xt @ Wht.T
    y = torch.zeros(B, H + L, dtype=torch.float64)
    for b in range(B):
        for k in range(row_ptr[b], row_ptr[b + 1]):
            y[b, labels[k]] = 1.0
    z = torch.cat([zh, zt], dim=1)
    loss = s * torch.nn.functional.binary_cross_entropy_with_logits(
        z, y, reduction="sum")
    loss.backward()
    dWt = np.zeros((L, idx.shape[1]))
    for t in range(L):
        dWt[t] = Wd.grad[t, idx[t // G]].numpy()
    _ = ng
    return (loss.item(), zh.detach().numpy(), zt.detach().numpy(),
            Xt.grad.numpy(), Wht.grad.numpy(), dWt)


@pytest.mark.parametrize("cfgname,over", [
    ("c1", {}),
    ("c1", {"L": 1000, "G": 16}),           # ragged last group (8 live)
    ("c1", {"G": 4, "F": 7, "L": 203}),
    ("c1", {"G": 1, "F": 5, "L": 91}),
])
def test_p3_equals_masked_dense_layer_with_autograd(cfgname, over):
    """Method item 1, 'structure': labels of a group share the fan-in set but
    keep independent weights -- the layer is a dense layer whose weight
    matrix is masked by the group pattern.  torch autograd on that masked
    dense model gives loss, logits and every gradient."""
    inp = wl.make_inputs(cfgname, **over)
    cfg = inp.cfg
    X, Wh, Wt = _f64(inp)
    s = 1.0 / cfg.B
    r = oracle.step(X, Wh, inp.idx, Wt, inp.row_ptr, inp.labels, cfg.L, cfg.G, s)
    loss, zh, zt, dX, dWh, dWt = _masked_dense_step(
        X, Wh, inp.idx, Wt, inp.row_ptr, inp.labels, cfg.L, cfg.G, s)
    assert math.isclose(r.loss, loss, rel_tol=1e-12)
    assert np.allclose(r.Zh, zh, rtol=1e-12, atol=1e-13)
    assert np.allclose(r.Zt, zt, rtol=1e-12, atol=1e-13)
    assert np.allclose(r.dX, dX, rtol=1e-10, atol=1e-14)
    assert np.allclose(r.dWh, dWh, rtol=1e-10, atol=1e-14)
    assert np.allclose(r.dWt, dWt, rtol=1e-10, atol=1e-14)


def test_p3_finite_differences():
    """Central differences of the oracle's own loss (h = 1e-6) against its
    analytic gradients, on sampled coordinates of X, the tail weights and the
    head weights."""
    inp = wl.make_inputs("c1", L=203, G=16)
    cfg = inp.cfg
    X, Wh, Wt = _f64(inp)
    s = 1.0 / cfg.B

    def L_of(X_, Wh_, Wt_):
        return oracle.step(X_, Wh_, inp.idx, Wt_, inp.row_ptr, inp.labels,
                           cfg.L, cfg.G, s).loss

    r = oracle.step(X, Wh, inp.idx, Wt, inp.row_ptr, inp.labels, cfg.L, cfg.G, s)
    rng = np.random.default_rng(5)
    h = 1e-6
    for _ in range(6):
        b, d = rng.integers(cfg.B), rng.integers(cfg.D)
        Xp, Xm = X.copy(), X.copy()
        Xp[b, d] += h
        Xm[b, d] -= h
        fd = (L_of(Xp, Wh, Wt) - L_of(Xm, Wh, Wt)) / (2 * h)
        assert abs(fd - r.dX[b, d]) <= 1e-6 * max(1.0, abs(fd))
        t, f = rng.integers(cfg.L), rng.integers(cfg.F)
        Wp, Wm = Wt.copy(), Wt.copy()
        Wp[t, f] += h
        Wm[t, f] -= h
        fd = (L_of(X, Wh, Wp) - L_of(X, Wh, Wm)) / (2 * h)
        assert abs(fd - r.dWt[t, f]) <= 1e-6 * max(1.0, abs(fd))
        hh = rng.integers(cfg.H)
        Hp, Hm = Wh.copy(), Wh.copy()
        Hp[hh, d] += h
        Hm[hh, d] -= h
        fd = (L_of(X, Hp, Wt) - L_of(X, Hm, Wt)) / (2 * h)
        assert abs(fd - r.dWh[hh, d]) <= 1e-6 * max(1.0, abs(fd))
    # padded (non-existent) labels get no weight gradient row at all
    assert r.dWt.shape == (cfg.L, cfg.F)


def test_exact_integer_arithmetic():
    """Small-integer inputs make every product and sum exact in fp64, so the
    oracle must equal exact integer arithmetic on the masked dense matrix
    (Python ints via numpy int64), for logits and both gradients."""
    rng = np.random.default_rng(11)
    B, D, L, G, F = 6, 30, 45, 8, 5
    ng = (L + G - 1) // G
    X = rng.integers(-4, 5, (B, D))
    Wt = rng.integers(-4, 5, (ng * G, F))
    idx = np.stack([np.sort(rng.choice(D, F, replace=False)) for _ in range(ng)]
                   ).astype(np.int32)
    Md = np.zeros((L, D), np.int64)
    for t in range(L):
        Md[t, idx[t // G]] = Wt[t]
    Z, _ = oracle.tail_logits(X.astype(float), idx, Wt.astype(float), L, G)
    assert np.array_equal(Z, (X @ Md.T).astype(float))
    dZ = rng.integers(-3, 4, (B, L))
    dW, _ = oracle.tail_dW(X.astype(float), idx, dZ.astype(float), L, G)
    full = dZ.T @ X                         # L x D
    ref = np.stack([full[t, idx[t // G]] for t in range(L)])
    assert np.array_equal(dW, ref.astype(float))
    dX, _ = oracle.tail_dX(idx, Wt.astype(float), dZ.astype(float), D, L, G)
    assert np.array_equal(dX, (dZ @ Md).astype(float))


# --------------------------------------------------------------------- P4
def test_p4_index_storage_per_group():
    """Method item 1, 'memory efficiency': indices are stored once per group,
    so the count is ceil(L/G)*F and the saving over per-label fan-in is G."""
    gold = json.load(open(os.path.join(GOLD, "index_storage.json")))
    for c in gold["cases"]:
        lay = oracle.layout(c["L"], c["G"], c["F"])
        assert lay["n_groups"] == c["n_groups"]
        assert lay["index_count"] == c["index_count"]
        if c["L"] % c["G"] == 0:
            assert c["per_label_count"] == lay["index_count"] * c["G"]
        if "last_group_live" in c:
            assert lay["last_group_live"] == c["last_group_live"]
        cfg = wl.CONFIGS[c["name"]]
        assert (cfg.L, cfg.G, cfg.F) == (c["L"], c["G"], c["F"])


# --------------------------------------------------------------------- P5
def test_p5_bce_closed_forms():
    gold = json.load(open(os.path.join(GOLD, "bce_values.json")))
    z = np.array([c["z"] for c in gold["cases"]])
    y = np.array([c["y"] for c in gold["cases"]], dtype=float)
    for s in (1.0, 0.125):
        dz, lt = oracle.bce(z, y, s)
        for i, c in enumerate(gold["cases"]):
            assert math.isclose(lt[i], s * c["loss"], rel_tol=1e-14,
                                abs_tol=1e-40), c
            assert math.isclose(dz[i], s * c["dz"], rel_tol=1e-14,
                                abs_tol=1e-40), c
    # large |z| stays finite; matches the textbook logistic loss elsewhere
    zz = np.linspace(-700, 700, 4001)
    for yy in (0.0, 1.0):
        dz, lt = oracle.bce(zz, np.full_like(zz, yy), 1.0)
        assert np.all(np.isfinite(lt)) and np.all(np.isfinite(dz))
        mid = np.abs(zz) < 30
        # textbook forms: y=0 -> log(1+e^z); y=1 -> log(1+e^-z)
        ref_l = np.log1p(np.exp(zz[mid] if yy == 0 else -zz[mid]))
        ref_d = 1.0 / (1.0 + np.exp(-zz[mid])) - yy
        assert np.allclose(lt[mid], ref_l, rtol=1e-13, atol=1e-300)
        assert np.allclose(dz[mid], ref_d, rtol=1e-12, atol=1e-15)


# --------------------------------------------------------------------- P6
def test_p6_topk_brute_force_and_two_stage_merge():
    """Exact top-K equals a full sort by (value desc, id asc).  The two-stage
    scheme of the top-K page (gist.science 'A Faster Generalized Two-Stage
    Approximate Top-K', section on the method: top-K' per bucket, then merge
    the survivors) is exact when K' = K, on any bucketing."""
    rng = np.random.default_rng(3)
    z = np.round(rng.standard_normal((7, 500)) * 4) / 4      # many ties
    K = 5
    val, ids = oracle.topk(z, K, id_offset=100)
    for r in range(z.shape[0]):
        order = np.lexsort((np.arange(500) + 100, -z[r]))[:K]
        assert np.array_equal(ids[r], order + 100)
        assert np.array_equal(val[r], z[r, order])
    for _ in range(5):
        perm = rng.permutation(500)
        buckets = np.array_split(perm, rng.integers(2, 40))
        cand_v, cand_i = [], []
        for bk in buckets:
            v, i = oracle.topk(z[:, bk], min(K, bk.size), ids=bk + 100)
            cand_v.append(v)
            cand_i.append(i)
        cv, ci = np.concatenate(cand_v, 1), np.concatenate(cand_i, 1)
        for r in range(z.shape[0]):
            v2, i2 = oracle.topk(cv[r:r + 1], K, ids=ci[r])
            assert np.array_equal(i2[0], ids[r])


def test_p6_two_stage_approximate_topk_brute_force():
    """The approximate two-stage top-K (top-K page, section "Method": top-K'
    per bucket of consecutive ids, K' < K, then the top-K of the survivors)
    equals the top-K, found by a full lexicographic sort, of the set of items
    whose rank inside their own bucket is below K'.  A hand case: the top
    five all in the first of two buckets with K' = 2 keeps two of them, the
    other bucket gives its two, and the fifth place stays empty."""
    rng = np.random.default_rng(5)
    z = np.round(rng.standard_normal((6, 300)) * 3) / 3      # ties
    for K, kp, seg in ((5, 2, 37), (8, 1, 16), (4, 4, 300), (6, 3, 1000), (3, 1, 1)):
        val, ids = oracle.topk_two_stage(z, K, kp, seg, id_offset=7)
        for r in range(z.shape[0]):
            keep = []
            for c0 in range(0, 300, seg):
                cols = np.arange(c0, min(c0 + seg, 300))
                order = cols[np.lexsort((cols, -z[r, cols]))]
                keep.extend(order[:kp].tolist())
            keep = np.array(keep)
            best = keep[np.lexsort((keep, -z[r, keep]))][:K]
            n = best.size
            assert np.array_equal(ids[r, :n], best + 7), (K, kp, seg, r)
            assert np.array_equal(val[r, :n], z[r, best])
            assert np.all(ids[r, n:K] == -1) and np.all(np.isneginf(val[r, n:K]))
    z = np.array([[9.0, 8.0, 7.0, 6.0, 5.0, 1.0, 0.5, 0.4, 0.3, 0.2]])
    val, ids = oracle.topk_two_stage(z, 5, 2, 5)
    assert ids[0, :5].tolist() == [0, 1, 5, 6, -1]
    assert val[0, :4].tolist() == [9.0, 8.0, 1.0, 0.5] and np.isneginf(val[0, 4])


def test_p6_exact_topk_lies_in_the_k_best_groups():
    """Reading C28: a row's exact top-K lies among the labels of its K best
    groups, the groups ranked by their largest logit (value descending, ties
    to the smaller id); so the top-K over those K * G labels is the exact
    top-K.  Checked against the brute-force sort on random rows, on rows with
    many exact ties, and with a ragged last group."""
    rng = np.random.default_rng(17)
    for trial in range(40):
        G = int(rng.choice([1, 2, 4, 16]))
        n = int(rng.integers(1, 200))
        K = int(rng.integers(1, 9))
        rows = 6
        z = rng.standard_normal((rows, n))
        if trial % 3 == 0:
            z = np.round(z * 2) / 2          # many exact ties
        want_v, want_i = oracle.topk(z, K, id_offset=11)
        ng = -(-n // G)
        for r in range(rows):
            maxv = np.array([z[r, g * G:(g + 1) * G].max() for g in range(ng)])
            maxi = np.array([g * G + int(np.argmax(z[r, g * G:(g + 1) * G])) for g in range(ng)])
            order = np.lexsort((maxi, -maxv))[:K]
            labs = np.concatenate([np.arange(g * G, min(n, (g + 1) * G)) for g in order])
            v, i = oracle.topk(z[r:r + 1, labs], K, ids=labs + 11)
            assert np.array_equal(i[0], want_i[r]) and np.array_equal(v[0], want_v[r]), (trial, r)


def test_p6_expected_recall_exhaustive_and_closed_forms():
    """Expected recall of the two-stage top-K (top-K page, section
    "Theoretical analysis": hypergeometric placement of the top-K in the
    buckets) equals, exactly, the average over every placement of the K
    largest items on n positions, found by enumeration; K' = K and buckets
    of one item give 1, one bucket gives K'/K; a Monte Carlo estimate at a
    larger n agrees within four standard errors."""
    from fractions import Fraction
    from itertools import combinations
    for n, K, kp, seg in ((9, 3, 1, 3), (9, 3, 2, 4), (10, 4, 1, 3), (8, 5, 2, 3), (7, 2, 1, 7), (6, 8, 2, 4)):
        Kt = min(K, n)
        tot, cnt = Fraction(0), 0
        for pos in combinations(range(n), Kt):
            per = {}
            for p_ in pos:
                per[p_ // seg] = per.get(p_ // seg, 0) + 1
            tot += Fraction(sum(min(c, kp) for c in per.values()), Kt)
            cnt += 1
        assert oracle.topk_expected_recall(n, K, kp, seg) == tot / cnt, (n, K, kp, seg)
    for n, K in ((1000, 5), (77, 8), (33, 1)):
        assert oracle.topk_expected_recall(n, K, K, 50) == 1
        assert oracle.topk_expected_recall(n, K, 1, 1) == 1
        assert oracle.topk_expected_recall(n, K, 1, n) == Fraction(1, K)
        assert oracle.topk_expected_recall(n, K, min(2, K), n) == Fraction(min(2, K), K)
    rng = np.random.default_rng(9)
    n, K, kp, seg, trials = 2000, 6, 2, 128, 20000
    rec = np.empty(trials)
    for i in range(trials):
        pos = rng.choice(n, K, replace=False)
        cnt = np.bincount(pos // seg)
        rec[i] = np.minimum(cnt, kp).sum() / K
    exact = float(oracle.topk_expected_recall(n, K, kp, seg))
    assert abs(rec.mean() - exact) < 4 * rec.std() / np.sqrt(trials) + 1e-12, (rec.mean(), exact)


def test_p6_plan_is_the_cheapest_pair_by_enumeration():
    """The automatic (K', buckets) choice (reading C24: fewest stage-2
    candidates buckets * K' among the pairs whose expected recall reaches the
    target, ties to the smaller K', at least min_buckets buckets) equals a
    brute-force search over every pair in which the recall of each pair is
    found by enumerating every placement of the K largest items on the n
    positions (buckets of ceil(n / b) consecutive positions), not by the
    hypergeometric formula."""
    from fractions import Fraction
    from itertools import combinations

    def recall_enum(n, K, kp, b):
        seg = -(-n // b)
        Kt = min(K, n)
        tot, cnt = Fraction(0), 0
        for pos in combinations(range(n), Kt):
            per = {}
            for p_ in pos:
                per[p_ // seg] = per.get(p_ // seg, 0) + 1
            tot += Fraction(sum(min(c, kp) for c in per.values()), Kt)
            cnt += 1
        return tot / cnt

    for n, K in ((6, 2), (8, 3), (9, 4), (10, 3)):
        rec = {(kp, b): recall_enum(n, K, kp, b) for kp in range(1, K + 1) for b in range(1, n + 1)}
        for target in (Fraction(1, 2), Fraction(7, 10), Fraction(9, 10), Fraction(19, 20), Fraction(1)):
            for bmin in (1, 2, 3):
                ok = [(b * kp, kp, b) for (kp, b), r in rec.items() if b >= bmin and r >= target]
                want = None if not ok else min(ok)[1:]
                got = oracle.topk_plan(n, K, target, bmin)
                assert got == want, (n, K, target, bmin, got, want)


def test_sgd_step_descends_at_first_order_rate():
    """The update W - lr * dW with the oracle's tail gradient lowers the
    oracle's loss, and (L(W - lr g) - L(W)) / lr tends to -|g|^2 as lr -> 0
    (first-order Taylor): pins the update's sign and scale together with the
    gradient it uses."""
    inp = wl.make_inputs(wl.tiny("sgd", B=6, D=40, H=8, L=60, G=4, F=8, dtype="f32"))
    c = inp.cfg
    X, Wh, Wt = _f64(inp)
    r0 = oracle.step(X, Wh, inp.idx, Wt, inp.row_ptr, inp.labels, c.L, c.G)
    g2 = float((r0.dWt ** 2).sum())
    assert g2 > 0
    prev = None
    for lr in (1e-1, 1e-2, 1e-3):
        W1 = oracle.sgd(Wt, r0.dWt, lr)
        r1 = oracle.step(X, Wh, inp.idx, W1, inp.row_ptr, inp.labels, c.L, c.G)
        slope = (r1.loss - r0.loss) / lr
        assert r1.loss < r0.loss
        err = abs(slope + g2)
        if prev is not None:
            assert err < 0.2 * prev + 1e-12, (lr, slope, -g2)   # error shrinks with lr
        prev = err
    assert prev < 1e-2 * g2


# --------------------------------------------------------------------- P7
def test_p7_group_positives_brute_force():
    inp = wl.make_inputs("c1", L=203, G=16, pos_per_row=9)
    cfg = inp.cfg
    grp_ptr, ent = oracle.group_positives(inp.row_ptr, inp.labels, cfg.H,
                                          cfg.L, cfg.G)
    keys = []
    for b in range(cfg.B):
        for k in range(inp.row_ptr[b], inp.row_ptr[b + 1]):
            t = inp.labels[k] - cfg.H
            if 0 <= t < cfg.L:
                keys.append((t // cfg.G, b, t % cfg.G))
    keys.sort()
    ng = (cfg.L + cfg.G - 1) // cfg.G
    assert grp_ptr[0] == 0 and grp_ptr[-1] == len(keys) and grp_ptr.size == ng + 1
    for g in range(ng):
        sl = [(b, j) for (gg, b, j) in keys if gg == g]
        got = [(e // cfg.G, e % cfg.G) for e in ent[grp_ptr[g]:grp_ptr[g + 1]]]
        assert got == sl


# ------------------------------------------------------- streaming step pin
def test_streaming_tail_step_matches_composition():
    """The streaming per-group step (used for timing and large checks) equals
    the composed full step on the tail, for any group sub-range."""
    inp = wl.make_inputs("c1", L=1000, G=16)
    cfg = inp.cfg
    X, Wh, Wt = _f64(inp)
    s = 1.0 / cfg.B
    r = oracle.step(X, Wh, inp.idx, Wt, inp.row_ptr, inp.labels, cfg.L, cfg.G, s)
    loss, dW, dX = oracle.tail_step(X, inp.idx, Wt, inp.row_ptr, inp.labels,
                                    cfg.H, cfg.L, cfg.G, s)
    assert math.isclose(loss, r.loss_tail, rel_tol=1e-12)
    assert np.allclose(dW, r.dWt, rtol=1e-12, atol=1e-15)
    assert np.allclose(dX, r.dX_tail, rtol=1e-11, atol=1e-15)
    l1, dW1, _ = oracle.tail_step(X, inp.idx, Wt, inp.row_ptr, inp.labels,
                                  cfg.H, cfg.L, cfg.G, s, g0=10, g1=63,
                                  want_dX=False)
    assert np.allclose(dW1, r.dWt[10 * 16:], rtol=1e-12, atol=1e-15)


def test_generator_is_deterministic_and_shaped():
    a = wl.make_inputs("c1")
    b = wl.make_inputs("c1")
    for k in ("X", "Wh", "idx", "W", "row_ptr", "labels"):
        assert np.array_equal(getattr(a, k), getattr(b, k))
    cfg = a.cfg
    assert a.idx.shape == (cfg.n_groups, cfg.F)
    assert np.all(np.diff(a.idx, axis=1) > 0)
    assert a.idx.min() >= 0 and a.idx.max() < cfg.D
    for r in range(cfg.B):
        row = a.labels[a.row_ptr[r]:a.row_ptr[r + 1]]
        assert row.size == cfg.pos_per_row and np.all(np.diff(row) > 0)
    bits = wl.bf16_bits_from_f32(np.array([1.0, 1.00390625, 1.005859375,
                                           -2.5], np.float32))
    assert list(wl.f64_from_bf16_bits(bits)) == [1.0, 1.0, 1.0078125, -2.5]


# ------------------------------------------------------- F4: rewiring
def test_rewire_golden_example():
    """Hand-derived worked example (tests/golden/rewire_example.json): two
    groups, a ragged last group whose padded row must not count towards the
    scores, a tie between two columns, candidates that are out of range,
    kept, repeated or pruned a moment ago, and a group whose candidates run
    out."""
    ex = json.load(open(os.path.join(GOLD, "rewire_example.json")))
    i2, W2 = oracle.tail_rewire(np.array(ex["idx"]), np.array(ex["W"], np.float32),
                                ex["L"], ex["G"], ex["D"], ex["k"], np.array(ex["cand"]))
    assert i2.tolist() == ex["expected_idx"]
    assert np.array_equal(W2, np.array(ex["expected_W"], np.float32))


def _grid_weights(rng, rows, F, zero_cols=0):
    # multiples of 1/16 in [-0.5, 0.5]: every float32 sum of up to 64 of them
    # is exact, so the float64 column sums below order the positions exactly
    W = (rng.integers(-8, 9, size=(rows, F)) / 16.0).astype(np.float32)
    if zero_cols:
        W[:, rng.choice(F, zero_cols, replace=False)] = 0.0
    return W


@pytest.mark.parametrize("G,F,D,L,k", [(16, 32, 96, 200, 8), (1, 16, 40, 30, 5),
                                       (64, 16, 16, 100, 6), (32, 64, 300, 90, 64),
                                       (16, 128, 768, 48, 0)])
def test_rewire_invariants_and_function(G, F, D, L, k):
    """Checks the rewiring step against properties that fix it, each by a
    route of its own: (a) every pruned position comes before every kept one
    in (score, feature) order, with scores summed in float64 over the live
    rows (exact on this weight grid); (b) the regrown set is the first k
    distinct admissible candidates in list order (found with np.unique), then
    the smallest features left (np.setdiff1d); (c) the layer's function: the
    rewired layer's logits equal those of the old layer with the pruned
    columns zeroed (the pinned tail_logits oracle); (d) k = 0 changes nothing."""
    rng = np.random.default_rng(G * 1000 + F + k)
    ng = (L + G - 1) // G
    idx = np.sort(np.stack([rng.choice(D, F, replace=False) for _ in range(ng)]), axis=1)
    W = _grid_weights(rng, ng * G, F, zero_cols=min(3, F // 4))
    R = 12
    cand = rng.integers(-3, D + 3, size=(ng, R))
    cand[:, 1] = idx[:, 0]                      # a kept-or-pruned feature
    cand[:, 3] = cand[:, 2]                     # a repeat
    i2, W2 = oracle.tail_rewire(idx, W, L, G, D, k, cand)
    assert np.all(np.diff(i2, axis=1) > 0) and i2.min() >= 0 and i2.max() < D
    for g in range(ng):
        live = min(G, L - g * G)
        rows = slice(g * G, (g + 1) * G)
        s64 = np.abs(W[g * G:g * G + live].astype(np.float64)).sum(axis=0)
        keys = sorted((s64[f], idx[g, f], f) for f in range(F))
        pruned = {f for _, _, f in keys[:k]}
        kept = [f for f in range(F) if f not in pruned]
        kept_feats = set(idx[g, kept].tolist())
        # (a) the oracle kept exactly these features
        assert kept_feats <= set(i2[g].tolist())
        # (b) regrown features
        c = cand[g]
        ok = (c >= 0) & (c < D) & ~np.isin(c, list(kept_feats))
        vals, first = np.unique(c[ok], return_index=True)
        taken = vals[np.argsort(first)][:k].tolist()
        if len(taken) < k:
            rest = np.setdiff1d(np.arange(D), list(kept_feats) + taken)
            taken += rest[:k - len(taken)].tolist()
        assert set(i2[g].tolist()) == kept_feats | set(taken)
        # regrown columns are zero, kept ones carry their weights unchanged
        for p, feat in enumerate(i2[g]):
            if feat in kept_feats:
                f = int(np.nonzero(idx[g] == feat)[0][0])
                assert np.array_equal(W2[rows, p], W[rows, f])
            else:
                assert np.all(W2[rows, p] == 0.0)
    # (c) function
    X = rng.standard_normal((5, D))
    Wz = W.astype(np.float64).copy()
    for g in range(ng):
        live = min(G, L - g * G)
        s64 = np.abs(W[g * G:g * G + live].astype(np.float64)).sum(axis=0)
        keys = sorted((s64[f], idx[g, f], f) for f in range(F))
        for _, _, f in keys[:k]:
            Wz[g * G:(g + 1) * G, f] = 0.0
    Z_old, A = oracle.tail_logits(X, idx, Wz, L, G)
    Z_new, _ = oracle.tail_logits(X, i2, W2.astype(np.float64), L, G)
    assert np.all(np.abs(Z_new - Z_old) <= 1e-12 * A + 1e-300)
    # (d) identity at k = 0
    i0, W0 = oracle.tail_rewire(idx, W, L, G, D, 0, cand)
    assert np.array_equal(i0, idx) and np.array_equal(W0, W)


def test_rewire_prune_all_takes_the_candidates():
    """k = F: every position goes, the new set is the first F distinct
    admissible candidates (here all of them, already distinct), sorted, and
    every weight is zero."""
    rng = np.random.default_rng(5)
    G, F, D, L = 4, 8, 50, 8
    idx = np.sort(np.stack([rng.choice(D, F, replace=False) for _ in range(2)]), axis=1)
    W = _grid_weights(rng, 2 * G, F)
    cand = np.stack([rng.choice(D, F, replace=False) for _ in range(2)])
    i2, W2 = oracle.tail_rewire(idx, W, L, G, D, F, cand)
    assert np.array_equal(i2, np.sort(cand, axis=1))
    assert np.all(W2 == 0.0)
