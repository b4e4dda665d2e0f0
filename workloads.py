"""Seeded synthetic inputs for the group-shared fixed fan-in output layer.

This module only *generates data*: it holds no step of the layer's arithmetic
(no logits, no loss, no gradients).  Both the CPU oracle's tests and the HIP
path's tests / bench draw their inputs from here, so the two sides always see
the same arrays.

Shapes follow the workloads described for HASTE (gist.science summary of
"HASTE: Hardware-Aware Dynamic Sparse Training for Large Output Spaces",
section "Results": Amazon-670K, Amazon-3M and LF-Paper2Keywords-8.6M output
spaces, groups of 16 vs 64).  The datasets themselves are not used: every
array is drawn from a fixed distribution with the stated shape.

Recipe (one numpy ``SeedSequence(seed).spawn(5)`` stream per array family):
  * X    ~ N(0, 1), shape B x D
  * W_h  ~ N(0, w_std), shape H x D            (head, dense classifier)
  * idx  : per group, F distinct feature ids in [0, D), sorted ascending;
           "uniform" = uniform without replacement, "skew10" = without
           replacement with P(j) proportional to 1/(j+10)
  * W    ~ N(0, w_std), shape (N_g*G) x F      (label-major tail weights;
           rows of padded labels in a ragged last group are drawn too)
  * positives: per row, exactly ``pos_per_row`` distinct labels drawn from a
           bounded Zipf law over ranks 1..H+L (P(r) ~ r^-s); rank r is global
           label id r-1, so head ids are [0, H) and tail id t has global id
           H + t.
bf16 configs round every float array once, fp32 -> bf16 round-to-nearest-even.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Config", "CONFIGS", "Inputs", "make_inputs", "bf16_bits_from_f32",
    "f64_from_bf16_bits", "n_groups",
]


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    D: int
    H: int
    L: int
    G: int
    F: int
    dtype: str            # "f32" or "bf16"
    w_std: float
    pos_per_row: int
    zipf_s: float
    idx_dist: str = "uniform"
    topk: int = 0
    lean: bool = False        # the step keeps no B x L array (the dX pass recomputes dz)
    seed: int = 0
    note: str = ""

    @property
    def n_groups(self) -> int:
        return n_groups(self.L, self.G)

    def replace(self, **kw) -> "Config":
        d = dict(self.__dict__)
        d.update(kw)
        return Config(**d)


def n_groups(L: int, G: int) -> int:
    return (L + G - 1) // G


# The five workloads.  c2 is the 670K-label training step the bench times.
CONFIGS = {
    "c1": Config("c1", B=8, D=64, H=64, L=1024, G=16, F=16, dtype="f32",
                 w_std=0.05, pos_per_row=3, zipf_s=1.1,
                 note="tiny CPU-checkable, fp32"),
    "c2": Config("c2", B=512, D=768, H=8192, L=662_000, G=16, F=128,
                 dtype="bf16", w_std=0.02, pos_per_row=5, zipf_s=1.1,
                 note="670K-shaped, G=16"),
    "c3": Config("c3", B=512, D=768, H=8192, L=662_000, G=64, F=128,
                 dtype="bf16", w_std=0.02, pos_per_row=5, zipf_s=1.1,
                 note="670K-shaped, G=64 (ragged last group: 48 live labels)"),
    "c4": Config("c4", B=256, D=768, H=16_384, L=2_984_000, G=32, F=128,
                 dtype="bf16", w_std=0.02, pos_per_row=6, zipf_s=1.05, lean=True,
                 note="3M-shaped, fused step, no B x L array"),
    "c5": Config("c5", B=128, D=1024, H=32_768, L=8_600_000, G=64, F=64,
                 dtype="bf16", w_std=0.02, pos_per_row=4, zipf_s=1.0,
                 idx_dist="skew10", topk=5,
                 note="8.6M-shaped, skewed fan-in, top-5"),
}


# ----------------------------------------------------------------- bf16 bits
def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round-to-nearest-even.  NaN-free
    inputs only (the generators draw finite normals)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def f64_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact float64 values."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32)


# ------------------------------------------------------------------- inputs
@dataclass
class Inputs:
    """One workload's arrays.  Float arrays are stored as the values the
    kernels consume: ``*_bits`` (uint16 bf16 patterns) for bf16 configs,
    float32 for f32 configs.  ``*_f64()`` gives the exact values."""
    cfg: Config
    X: np.ndarray            # B x D   (uint16 bits or float32)
    Wh: np.ndarray           # H x D
    idx: np.ndarray          # N_g x F int32
    W: np.ndarray            # (N_g*G) x F
    row_ptr: np.ndarray      # B+1 int32
    labels: np.ndarray       # nnz int32, global ids, ascending within a row
    extra: dict = field(default_factory=dict)

    def _f64(self, a):
        if self.cfg.dtype == "bf16":
            return f64_from_bf16_bits(a)
        return a.astype(np.float64)

    def X_f64(self):
        return self._f64(self.X)

    def Wh_f64(self):
        return self._f64(self.Wh)

    def W_f64(self):
        return self._f64(self.W)


def _round(cfg: Config, a32: np.ndarray) -> np.ndarray:
    if cfg.dtype == "bf16":
        return bf16_bits_from_f32(a32)
    return np.ascontiguousarray(a32, dtype=np.float32)


def _draw_idx(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    Ng, D, F = cfg.n_groups, cfg.D, cfg.F
    out = np.empty((Ng, F), dtype=np.int32)
    if cfg.idx_dist == "uniform":
        logw = None
    elif cfg.idx_dist == "skew10":
        logw = -np.log(np.arange(D, dtype=np.float64) + 10.0)
    else:
        raise ValueError(cfg.idx_dist)
    chunk = max(1, (1 << 23) // D)
    for g0 in range(0, Ng, chunk):
        g1 = min(Ng, g0 + chunk)
        u = rng.random((g1 - g0, D))
        if logw is None:
            keys = u
        else:
            # Weighted sampling without replacement (Efraimidis-Spirakis):
            # keep the F largest u^(1/w_j), i.e. the F largest log(u)/w_j.
            keys = np.log(u) * np.exp(-logw)[None, :]
        top = np.argpartition(-keys, F - 1, axis=1)[:, :F]
        top.sort(axis=1)
        out[g0:g1] = top.astype(np.int32)
    return out


def _draw_positives(cfg: Config, rng: np.random.Generator):
    B, P, n = cfg.B, cfg.pos_per_row, cfg.H + cfg.L
    ranks = np.arange(1, n + 1, dtype=np.float64)
    cdf = np.cumsum(ranks ** (-cfg.zipf_s))
    cdf /= cdf[-1]
    labels = np.empty((B, P), dtype=np.int64)
    for b in range(B):
        got: list[int] = []
        while len(got) < P:
            r = int(np.searchsorted(cdf, rng.random(), side="right"))
            r = min(r, n - 1)
            if r not in got:
                got.append(r)
        labels[b] = sorted(got)
    row_ptr = np.arange(B + 1, dtype=np.int32) * P
    return row_ptr, labels.reshape(-1).astype(np.int32)


def make_inputs(cfg: Config | str, **overrides) -> Inputs:
    """Draw one workload's arrays, deterministically from ``cfg.seed``."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if overrides:
        cfg = cfg.replace(**overrides)
    ss = np.random.SeedSequence(cfg.seed)
    s_x, s_wh, s_idx, s_w, s_pos = ss.spawn(5)
    rx, rwh, ridx, rw, rpos = (np.random.default_rng(s) for s in
                               (s_x, s_wh, s_idx, s_w, s_pos))
    X = _round(cfg, rx.standard_normal((cfg.B, cfg.D), dtype=np.float32))
    Wh = _round(cfg, (rwh.standard_normal((cfg.H, cfg.D), dtype=np.float32)
                      * np.float32(cfg.w_std)))
    idx = _draw_idx(cfg, ridx)
    rows = cfg.n_groups * cfg.G
    W = np.empty((rows, cfg.F), dtype=np.uint16 if cfg.dtype == "bf16"
                 else np.float32)
    step = max(1, (1 << 24) // cfg.F)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        W[r0:r1] = _round(cfg, rw.standard_normal((r1 - r0, cfg.F),
                                                  dtype=np.float32)
                          * np.float32(cfg.w_std))
    row_ptr, labels = _draw_positives(cfg, rpos)
    return Inputs(cfg, X, Wh, idx, W, row_ptr, labels)


def rewire_candidates(cfg: Config, n_cand: int, seed: int = 1) -> np.ndarray:
    """Regrowth candidates for the rewiring step: N_g x n_cand features drawn
    uniformly from [0, D) with repeats (the random draws a training loop
    makes and passes to the layer), deterministically from ``seed``."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, cfg.seed]))
    return rng.integers(0, cfg.D, size=(cfg.n_groups, n_cand), dtype=np.int32)


def tiny(name="t", **kw) -> Config:
    """Small configs for parity tests (several tiles plus ragged tails)."""
    base = dict(name=name, B=40, D=96, H=48, L=200, G=16, F=32, dtype="bf16",
                w_std=0.05, pos_per_row=3, zipf_s=1.1)
    base.update(kw)
    return Config(**base)


def positives_per_branch(inp: Inputs) -> dict:
    """Counts of head / tail positives (for reporting only)."""
    H = inp.cfg.H
    head = int(np.sum(inp.labels < H))
    return {"head": head, "tail": int(inp.labels.size - head)}


if __name__ == "__main__":  # pragma: no cover - quick look at a config
    import sys
    name = sys.argv[1] if len(sys.argv) > 1 else "c1"
    inp = make_inputs(name)
    print(inp.cfg, inp.X.shape, inp.W.shape, inp.idx.shape,
          positives_per_branch(inp), math.prod(inp.W.shape))
