"""GPU parity of the rewiring step (haste_tail_rewire, through the C ABI):
the new index sets and weight columns must equal the oracle's bit for bit.
Inputs are seeded; the weights sit on a coarse grid with zero columns so that
scores tie, and the candidate lists hold out-of-range values, kept features,
repeats and (with R > 64) more than one batch of 64."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests._gpu import DEV, dev_array

pytestmark = pytest.mark.gpu


def _case(G, F, D, L, k, R, dtype, seed):
    rng = np.random.default_rng(seed)
    ng = (L + G - 1) // G
    idx = np.sort(np.stack([rng.choice(D, F, replace=False) for _ in range(ng)]), axis=1)
    idx = idx.astype(np.int32)
    W32 = (rng.integers(-8, 9, size=(ng * G, F)) / 16.0).astype(np.float32)
    W32[:, rng.choice(F, max(1, F // 8), replace=False)] = 0.0
    if dtype == "f32":   # some values off the grid, exact in fp32 only
        W32[::3] += (rng.standard_normal((W32[::3].shape)) * 1e-3).astype(np.float32)
    cand = rng.integers(-2, D + 2, size=(ng, R)).astype(np.int32)
    if R >= 4:
        cand[:, 0] = idx[:, rng.integers(0, F)]
        cand[:, 3] = cand[:, 2]
    return idx, W32, cand


def _run(idx, W32, cand, D, L, G, k, dtype, inplace=False):
    from sparse_output_layer_amd import haste as H
    Wd = dev_array(wl.bf16_bits_from_f32(W32) if dtype == "bf16" else W32, dtype)
    idd = torch.from_numpy(idx).to(DEV)
    cd = torch.from_numpy(cand).to(DEV) if cand.shape[1] > 0 else None
    if inplace:
        H.haste_tail_rewire(idd, Wd, D, L, G, k, cd, idx_out=idd, W_out=Wd)
        io, Wo = idd, Wd
    else:
        io, Wo = H.haste_tail_rewire(idd, Wd, D, L, G, k, cd)
    torch.cuda.synchronize()
    return io.cpu().numpy(), Wo.float().cpu().numpy()


@pytest.mark.parametrize("G,F,D,L,k,R,dtype", [
    (16, 32, 96, 200, 8, 12, "bf16"),      # ragged last group (8 live labels)
    (16, 128, 768, 500, 32, 64, "bf16"),
    (64, 64, 1024, 300, 16, 130, "bf16"),  # three candidate batches
    (32, 128, 128, 70, 40, 8, "bf16"),     # D = F: every feature in the set
    (1, 16, 40, 33, 5, 6, "bf16"),         # per-label fan-in
    (16, 256, 3000, 40, 200, 0, "bf16"),   # no candidates: smallest features left
    (64, 32, 200, 130, 32, 10, "f32"),     # prune everything
    (3, 20, 50, 17, 0, 5, "f32"),          # k = 0: unchanged
    (16, 48, 70000 // 1000, 64, 7, 70, "f32"),
    (3, 20, 50, 17, 4, 9, "bf16"),         # rows of 40 bytes: weights moved element by element
])
def test_rewire_matches_oracle_bit_exact(G, F, D, L, k, R, dtype):
    idx, W32, cand = _case(G, F, D, L, k, R, dtype, seed=G + F + k)
    print(f"rewire G={G} F={F} D={D} L={L} k={k} R={R} {dtype}", flush=True)
    Wq = wl.f32_from_bf16_bits(wl.bf16_bits_from_f32(W32)) if dtype == "bf16" else W32
    ri, rW = oracle.tail_rewire(idx, Wq, L, G, D, k, cand)
    gi, gW = _run(idx, W32, cand, D, L, G, k, dtype)
    assert np.array_equal(gi, ri)
    assert np.array_equal(gW.view(np.uint32), rW.view(np.uint32))   # bit for bit (+0 for regrown)
    ii, iW = _run(idx, W32, cand, D, L, G, k, dtype, inplace=True)
    assert np.array_equal(ii, ri) and np.array_equal(iW.view(np.uint32), rW.view(np.uint32))


def test_rewire_full_size_670k():
    """The 670K-label workload (41,375 groups of 16, F = 128, D = 768) with 64
    uniform candidates per group and a quarter of each set pruned: sampled
    groups (the first, the last and random ones) against the oracle bit for
    bit; every group's new set valid (haste_tail_validate) and holding at
    least F - k of its old features."""
    from sparse_output_layer_amd import haste as H
    cfg = wl.CONFIGS["c2"]
    inp = wl.make_inputs(cfg)
    k, R = 32, 64
    cand = wl.rewire_candidates(cfg, R)
    print(f"rewire c2 k={k} R={R}", flush=True)
    Wd = dev_array(inp.W, "bf16")
    idd = torch.from_numpy(inp.idx).to(DEV)
    io, Wo = H.haste_tail_rewire(idd, Wd, cfg.D, cfg.L, cfg.G, k, torch.from_numpy(cand).to(DEV))
    bad = H.haste_tail_validate(io, cfg.D, cfg.L, cfg.G)
    pos = torch.searchsorted(idd.long(), io.long()).clamp_max(cfg.F - 1)
    kept = (torch.gather(idd, 1, pos) == io).sum(dim=1)
    torch.cuda.synchronize()
    assert int(bad.item()) == -1
    assert int(kept.min()) >= cfg.F - k
    rng = np.random.default_rng(7)
    ng = cfg.n_groups
    gs = np.unique(np.concatenate([[0, ng - 1], rng.integers(0, ng, 300)]))
    gi = io.cpu().numpy()
    gW = Wo.view(torch.int16).cpu().numpy().view(np.uint16)
    Wf = wl.f32_from_bf16_bits(inp.W)
    for g in gs:
        rows = slice(g * cfg.G, (g + 1) * cfg.G)
        ri, rW = oracle.tail_rewire(inp.idx[g:g + 1], Wf[rows], cfg.L - g * cfg.G, cfg.G, cfg.D, k,
                                    cand[g:g + 1])
        assert np.array_equal(gi[g], ri[0]), g
        assert np.array_equal(wl.f32_from_bf16_bits(gW[rows]).view(np.uint32), rW.view(np.uint32)), g
