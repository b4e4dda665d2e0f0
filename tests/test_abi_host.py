"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point include/haste.h declares, reports the storage layout the
oracle defines, sizes workspaces, and rejects bad arguments before anything
is enqueued (no compute call runs here)."""
import ctypes

import pytest

import oracle
from sparse_output_layer_amd import haste as H


@pytest.fixture(scope="module")
def L():
    return H.lib()


def test_exports_every_declared_symbol(L):
    names = H.header_functions()
    assert "haste_tail_fwd" in names and "haste_tail_step" in names
    missing = [n for n in names if not hasattr(L, n)]
    assert missing == []
    assert L.haste_abi_version() == 5
    for s in range(5):
        assert L.haste_status_string(s)


@pytest.mark.parametrize("Lb,G,F", [(1024, 16, 16), (662000, 16, 128), (662000, 64, 128),
                                    (2984000, 32, 128), (8600000, 64, 64), (7, 3, 5),
                                    (1, 64, 32)])
def test_layout_matches_oracle_bit_exact(Lb, G, F):
    got = H.haste_tail_layout(Lb, G, F)
    assert got == oracle.layout(Lb, G, F)


def _desc(**kw):
    d = dict(B=8, D=64, L=1024, G=16, F=32, dtype=H.HASTE_BF16)
    d.update(kw)
    return H.TailDesc(**d)


def test_workspace_sizes(L):
    d = _desc()
    lean = _desc(flags=H.HASTE_TAIL_LEAN)
    # the default form keeps dz tiles, B_pad x N_g*G bf16 (with or without bce:
    # the backward from a given dZ forms them too); the lean form has none
    n0 = L.haste_tail_workspace_bytes(ctypes.byref(d), None)
    n0l = L.haste_tail_workspace_bytes(ctypes.byref(lean), None)
    assert n0l > 0 and n0 - n0l >= 64 * 1024 * 2
    b = H.BceStruct(nnz=10000)
    n1 = L.haste_tail_workspace_bytes(ctypes.byref(d), ctypes.byref(b))
    assert n1 >= n0 + 10000 * 4 - 256
    nl = L.haste_tail_workspace_bytes(ctypes.byref(lean), ctypes.byref(b))
    assert n1 - nl >= 64 * 1024 * 2 and nl >= n0l + 10000 * 4 - 256
    # unknown flags -> 0
    assert L.haste_tail_workspace_bytes(ctypes.byref(_desc(flags=4)), None) == 0
    # the forward needs no dz tiles: its workspace is the training calls' less them
    nf = L.haste_tail_fwd_workspace_bytes(ctypes.byref(d), ctypes.byref(b))
    assert nf > 0 and n1 - nf >= 64 * 1024 * 2
    assert nf == L.haste_tail_fwd_workspace_bytes(ctypes.byref(lean), ctypes.byref(b))
    # the feature order sits at offset 0 for every BCE setup: a workspace that
    # holds it once serves every later call (HASTE_TAIL_LAYOUT_READY)
    rd = _desc(flags=H.HASTE_TAIL_LAYOUT_READY)
    assert L.haste_tail_workspace_bytes(ctypes.byref(rd), None) == n0
    # unsupported shape -> 0
    assert L.haste_tail_workspace_bytes(ctypes.byref(_desc(G=8)), None) == 0
    h = H.HeadDesc(B=8, D=64, H=128, dtype=H.HASTE_BF16)
    assert L.haste_head_workspace_bytes(ctypes.byref(h), None) >= 8 * 128 * 2


def _status(L, d, X=0x1000, idx=0x1000, W=0x1000, Z=0x1000, bce=None, ws=None, nb=0):
    return L.haste_tail_fwd(ctypes.byref(d) if d is not None else None, X, idx, W, Z, bce,
                            ws, nb, None)


def test_argument_errors_fail_before_launch(L):
    assert _status(L, None) == H.HASTE_ERR_INVALID
    assert b"NULL" in L.haste_last_error()
    assert _status(L, _desc(B=0)) == H.HASTE_ERR_INVALID
    assert _status(L, _desc(F=128, D=64)) == H.HASTE_ERR_INVALID      # F > D
    assert _status(L, _desc(dtype=7)) == H.HASTE_ERR_INVALID
    assert _status(L, _desc(flags=4)) == H.HASTE_ERR_INVALID
    assert _status(L, _desc(G=8)) == H.HASTE_ERR_UNSUPPORTED
    assert _status(L, _desc(F=48)) == H.HASTE_ERR_UNSUPPORTED
    assert _status(L, _desc(D=4096, F=128)) == H.HASTE_ERR_UNSUPPORTED
    assert _status(L, _desc(), X=0) == H.HASTE_ERR_INVALID
    assert _status(L, _desc(), X=0x1002) == H.HASTE_ERR_INVALID      # misaligned bf16
    assert _status(L, _desc(), Z=0, bce=None) == H.HASTE_ERR_INVALID  # nothing to do
    # workspace: needed but missing / too small / misaligned
    assert _status(L, _desc()) == H.HASTE_ERR_WORKSPACE
    assert _status(L, _desc(), ws=0x1000, nb=16) == H.HASTE_ERR_WORKSPACE
    assert _status(L, _desc(), ws=0x1010, nb=1 << 30) == H.HASTE_ERR_WORKSPACE
    # bce checks
    b = H.BceStruct(nnz=-1, row_ptr=0x1000)
    assert _status(L, _desc(), bce=ctypes.byref(b)) == H.HASTE_ERR_INVALID
    b = H.BceStruct(nnz=5, row_ptr=0x1000, labels=None)
    assert _status(L, _desc(), bce=ctypes.byref(b)) == H.HASTE_ERR_INVALID
    # top-K: K in [0, 8], output buffers required; the backward rejects it
    b = H.BceStruct(nnz=5, row_ptr=0x1000, labels=0x1000, topk=9, topk_val=0x1000, topk_idx=0x1000)
    assert _status(L, _desc(), bce=ctypes.byref(b)) == H.HASTE_ERR_INVALID
    b = H.BceStruct(nnz=5, row_ptr=0x1000, labels=0x1000, topk=5)
    assert _status(L, _desc(), bce=ctypes.byref(b)) == H.HASTE_ERR_INVALID
    b = H.BceStruct(nnz=5, row_ptr=0x1000, labels=0x1000, topk=5, topk_val=0x1000, topk_idx=0x1000)
    assert _status(L, _desc(), bce=ctypes.byref(b)) == H.HASTE_ERR_WORKSPACE
    assert L.haste_tail_bwd(ctypes.byref(_desc()), 0x1000, 0x1000, 0x1000, None, ctypes.byref(b),
                            0x1000, 0x1000, 0, 0x1000, 1 << 30, None) == H.HASTE_ERR_UNSUPPORTED
    # the top-K adds the fp32 logits (B x L x 4 bytes) to the workspace
    n0 = L.haste_tail_workspace_bytes(ctypes.byref(_desc()), ctypes.byref(H.BceStruct(nnz=5)))
    n1 = L.haste_tail_workspace_bytes(ctypes.byref(_desc()), ctypes.byref(b))
    assert n1 - n0 >= 8 * 1024 * 4
    # fp32 accepts any G / F
    d = _desc(dtype=H.HASTE_F32, G=3, F=7)
    assert _status(L, d) == H.HASTE_ERR_WORKSPACE
    # top-K ids are int32: the last label's global id must fit
    big = _desc(L=2 ** 31 - 100)
    for off, want in ((100, H.HASTE_ERR_WORKSPACE), (101, H.HASTE_ERR_UNSUPPORTED)):
        b = H.BceStruct(nnz=5, row_ptr=0x1000, labels=0x1000, topk=5, topk_val=0x1000,
                        topk_idx=0x1000, label_offset=off)
        assert _status(L, big, bce=ctypes.byref(b)) == want, off
    h = H.HeadDesc(B=8, D=64, H=1 << 20, dtype=H.HASTE_BF16)
    b = H.BceStruct(nnz=5, row_ptr=0x1000, labels=0x1000, topk=5, topk_val=0x1000,
                    topk_idx=0x1000, label_offset=2 ** 31 - (1 << 20) + 1)
    assert L.haste_head_fwd(ctypes.byref(h), 0x1000, 0x1000, None, ctypes.byref(b), None, 0, None) == \
        H.HASTE_ERR_UNSUPPORTED
    # the layout call: checks as the compute calls, then the workspace
    assert L.haste_tail_prepare_layout(ctypes.byref(_desc()), 0x1000, None, 0, None) == H.HASTE_ERR_WORKSPACE
    assert L.haste_tail_prepare_layout(ctypes.byref(_desc()), 0, 0x1000, 1 << 30, None) == H.HASTE_ERR_INVALID
    assert L.haste_tail_prepare_layout(ctypes.byref(_desc(G=8)), 0x1000, 0x1000, 1 << 30, None) == \
        H.HASTE_ERR_UNSUPPORTED


def test_head_and_step_argument_errors(L):
    h = H.HeadDesc(B=8, D=60, H=128, dtype=H.HASTE_BF16)       # D % 8 != 0
    assert L.haste_head_fwd(ctypes.byref(h), 0x1000, 0x1000, 0x1000, None, None, 0, None) == \
        H.HASTE_ERR_UNSUPPORTED
    h = H.HeadDesc(B=0, D=64, H=128, dtype=H.HASTE_BF16)
    assert L.haste_head_fwd(ctypes.byref(h), 0x1000, 0x1000, 0x1000, None, None, 0, None) == \
        H.HASTE_ERR_INVALID
    d = _desc()
    assert L.haste_tail_step(ctypes.byref(d), 0x1000, 0x1000, 0x1000, None, 0x1000, 0x1000, 0,
                             None, 0, None) == H.HASTE_ERR_INVALID       # bce required
    # bf16 with G = 1 (per-label fan-in): the forward and the one-call step
    # (it keeps dz: no lean form; no top-K; D <= 960); the split calls are not taken
    g1 = _desc(G=1)
    b = H.BceStruct(nnz=5, row_ptr=0x1000, labels=0x1000)
    assert _status(L, g1) == H.HASTE_ERR_WORKSPACE                       # forward: accepted

    def g1_step(d, bce, nb=0):
        return L.haste_tail_step(ctypes.byref(d), 0x1000, 0x1000, 0x1000, ctypes.byref(bce), 0x1000,
                                 0x1000, 0, 0x1000 if nb else None, nb, None)
    assert g1_step(g1, b) == H.HASTE_ERR_WORKSPACE                        # step: accepted
    assert L.haste_tail_workspace_bytes(ctypes.byref(g1), ctypes.byref(b)) >= 1024 * 64 * 2
    assert g1_step(_desc(G=1, flags=H.HASTE_TAIL_LEAN), b, 1 << 30) == H.HASTE_ERR_UNSUPPORTED
    assert g1_step(_desc(G=1, D=1024), b, 1 << 30) == H.HASTE_ERR_UNSUPPORTED
    bk = H.BceStruct(nnz=5, row_ptr=0x1000, labels=0x1000, topk=5, topk_val=0x1000, topk_idx=0x1000)
    assert g1_step(g1, bk, 1 << 30) == H.HASTE_ERR_UNSUPPORTED
    assert L.haste_tail_prepare(ctypes.byref(g1), 0x1000, ctypes.byref(b), 0x1000, 1 << 30,
                                None) == H.HASTE_ERR_UNSUPPORTED
    assert L.haste_topk_merge(4, 0, 1, 1, 1, 1, 1, 1, None) == H.HASTE_ERR_INVALID
    # approximate top-K: K' in [0, K], buckets in [0, 2^24]
    for kp, nbk in ((6, 0), (-1, 0), (2, -1), (2, (1 << 24) + 1), (2, 0)):
        b = H.BceStruct(nnz=5, row_ptr=0x1000, labels=0x1000, topk=5, topk_val=0x1000,
                        topk_idx=0x1000, topk_kprime=kp, topk_buckets=nbk)
        assert _status(L, _desc(), bce=ctypes.byref(b)) == H.HASTE_ERR_INVALID, (kp, nbk)
    b = H.BceStruct(nnz=5, row_ptr=0x1000, labels=0x1000, topk=5, topk_val=0x1000,
                    topk_idx=0x1000, topk_kprime=2, topk_buckets=64)
    assert _status(L, _desc(), bce=ctypes.byref(b)) == H.HASTE_ERR_WORKSPACE
    assert L.haste_tail_validate(None, 0x1000, 0x1000, None) == H.HASTE_ERR_INVALID


def test_noalloc_head_step_rejects_a_step_beyond_its_scratch(L):
    """The allocation-free head step checks its need against the static
    scratch before it touches the device."""
    h = H.HeadDesc(B=4096, D=64, H=16384, dtype=H.HASTE_BF16)   # dZh alone: 128 MiB
    b = H.BceStruct(nnz=5, row_ptr=0x1000, labels=0x1000)
    assert L.haste_head_step_noalloc(ctypes.byref(h), 0x1000, 0x1000, ctypes.byref(b), 0x1000,
                                     0x1000, 0, None) == H.HASTE_ERR_WORKSPACE
    assert b"scratch" in L.haste_last_error()
    assert L.haste_head_step_noalloc(ctypes.byref(h), 0x1000, 0x1000, None, 0x1000, 0x1000, 0,
                                     None) == H.HASTE_ERR_INVALID          # bce required

def test_topk_recall_and_plan_match_the_oracle(L):
    """The library's expected recall and parameter choice (host code) against
    the oracle's exact-fraction formula and plain search."""
    import oracle
    from sparse_output_layer_amd import haste as Hp
    for n, K, kp, nb in ((1000, 5, 1, 50), (3000, 8, 3, 7), (70000, 5, 2, 1), (40, 6, 2, 13),
                         (5, 8, 2, 2), (123457, 4, 1, 999)):
        got = Hp.haste_topk_expected_recall(n, K, kp, nb)
        want = float(oracle.topk_expected_recall(n, K, kp, oracle.topk_seg_len(n, nb)))
        assert abs(got - want) <= 1e-12 * max(1.0, want), (n, K, kp, nb, got, want)
    for n, K, target, bmin in ((500, 5, 0.9, 10), (800, 4, 0.97, 30), (300, 8, 0.8, 1), (2000, 5, 0.99, 64)):
        assert Hp.haste_topk_plan(n, K, target, bmin) == oracle.topk_plan(n, K, target, bmin), \
            (n, K, target, bmin)
    assert L.haste_topk_expected_recall(10, 9, 1, 0) < 0
    assert L.haste_topk_expected_recall(10, 5, 6, 1) < 0
    assert L.haste_topk_expected_recall(10, 5, 2, 0) < 0
    out = (ctypes.c_int32 * 2)()
    assert L.haste_topk_plan(100, 5, 1.5, 1, out) == H.HASTE_ERR_INVALID
    assert L.haste_topk_plan(100, 5, 0.9, 0, out) == H.HASTE_ERR_INVALID
    assert L.haste_topk_plan(100, 5, 0.9, 101, out) == H.HASTE_ERR_INVALID


def test_sgd_entry_points_reject_bad_arguments(L):
    """Argument checks of the fused SGD step and the SGD update (all return
    before any GPU work)."""
    d = _desc()
    b = H.BceStruct(nnz=5, row_ptr=0x1000, labels=0x1000)
    f, vp = ctypes.c_float, ctypes.c_void_p
    # W_out missing, overlapping W, or the fp32 dtype
    assert L.haste_tail_step_sgd(ctypes.byref(d), vp(0x1000), vp(0x1000), vp(0x2000), ctypes.byref(b),
                                 f(0.1), None, vp(0x1000), 0, vp(0x1000), 1 << 30, None) == H.HASTE_ERR_INVALID
    assert L.haste_tail_step_sgd(ctypes.byref(d), vp(0x1000), vp(0x1000), vp(0x2000), ctypes.byref(b),
                                 f(0.1), vp(0x2010), vp(0x1000), 0, vp(0x1000), 1 << 30, None) == H.HASTE_ERR_INVALID
    d32 = _desc(dtype=H.HASTE_F32)
    assert L.haste_tail_step_sgd(ctypes.byref(d32), vp(0x1000), vp(0x1000), vp(0x2000), ctypes.byref(b),
                                 f(0.1), vp(1 << 40), vp(0x1000), 0, vp(0x1000), 1 << 30, None) == \
        H.HASTE_ERR_UNSUPPORTED
    assert L.haste_tail_step_sgd(ctypes.byref(d), vp(0x1000), vp(0x1000), vp(0x2000), None,
                                 f(0.1), vp(1 << 40), vp(0x1000), 0, vp(0x1000), 1 << 30, None) == H.HASTE_ERR_INVALID
    assert L.haste_sgd_update(-1, H.HASTE_BF16, vp(0x1000), vp(0x1000), f(0.1), vp(0x1000), None) == \
        H.HASTE_ERR_INVALID
    assert L.haste_sgd_update(8, 7, vp(0x1000), vp(0x1000), f(0.1), vp(0x1000), None) == H.HASTE_ERR_INVALID
    assert L.haste_sgd_update(8, H.HASTE_F32, vp(0x1001), vp(0x1000), f(0.1), vp(0x1000), None) == \
        H.HASTE_ERR_INVALID
    assert L.haste_sgd_update(0, H.HASTE_BF16, None, None, f(0.1), None, None) == H.HASTE_OK


def test_probe_argument_checks(L):
    """The MFMA-rate probe rejects empty launches and a missing sink before any launch."""
    L.haste_probe_mfma.restype = ctypes.c_int
    L.haste_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert L.haste_probe_mfma(0, 10, 0x1000, None) == H.HASTE_ERR_INVALID
    assert L.haste_probe_mfma(4, 0, 0x1000, None) == H.HASTE_ERR_INVALID
    assert L.haste_probe_mfma(4, 10, None, None) == H.HASTE_ERR_INVALID
    assert L.haste_probe_mfma(4, 10, 0x1002, None) == H.HASTE_ERR_INVALID



def test_rewire_argument_errors_fail_before_launch(L):
    """haste_tail_rewire rejects bad arguments before it enqueues anything."""
    def rw(d, k=2, cand=0x1000, R=4, idx=0x1000, W=0x2000, io=0x100000, Wo=0x200000):
        return L.haste_tail_rewire(ctypes.byref(d) if d is not None else None, idx, W, k, cand, R,
                                   io, Wo, None)
    d = _desc(D=64, L=1024, G=16, F=32)
    assert rw(None) == H.HASTE_ERR_INVALID
    assert rw(d, k=-1) == H.HASTE_ERR_INVALID
    assert rw(d, k=33) == H.HASTE_ERR_INVALID                  # k > F
    assert rw(d, R=-1) == H.HASTE_ERR_INVALID
    assert rw(d, cand=0) == H.HASTE_ERR_INVALID                # n_cand > 0 needs a list
    assert rw(d, idx=0) == H.HASTE_ERR_INVALID
    assert rw(d, W=0x2001) == H.HASTE_ERR_INVALID              # misaligned bf16
    assert rw(_desc(D=64, F=128)) == H.HASTE_ERR_INVALID        # F > D
    assert rw(_desc(D=70000, F=32)) == H.HASTE_ERR_UNSUPPORTED
    assert rw(_desc(D=1024, F=512)) == H.HASTE_ERR_UNSUPPORTED
    assert rw(_desc(D=1024, F=32, G=65, dtype=H.HASTE_F32)) == H.HASTE_ERR_UNSUPPORTED
    # partial overlaps (in place, the same pointer, is allowed)
    assert rw(d, io=0x1000 + 64) == H.HASTE_ERR_INVALID
    assert rw(d, Wo=0x2000 + 64) == H.HASTE_ERR_INVALID
    assert b"overlaps" in L.haste_last_error()
