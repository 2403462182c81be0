"""Comparison rules between the HIP path and the CPU oracle.

Selection (256-bin histogram top-p):
  * the top cell A must match; it may differ by one only when the oracle's largest
    logit lies within 1e-5 (relative, at least 1e-5 absolute) of a bin edge;
  * the threshold bin b* must match, or differ by one on a mass tie: the oracle's
    cumulative mass at the disputed bin lies within 1e-5 Z of p Z;
  * the selected set must equal the oracle rule's set under the GPU's (A, b*), except
    for tokens whose logit lies within 1e-5 relative of a bin edge.
Selection (fixed top-k through the same histogram): counts are exact, so b* must match
unless tokens in the edge band could move the cumulative count across k ("count tie").
Outputs: max |O_gpu - O_oracle| <= 2e-3 (fp16 or bf16 K/V) or 1e-5 (fp32 K/V).
"""
from __future__ import annotations

import numpy as np

import oracle

EDGE_REL = 1e-5
TIE_REL = 1e-5


def out_tol(dtype: str) -> float:
    # 16-bit K/V (fp16, bf16): 2e-3; fp32: 1e-5
    return 1e-5 if dtype == "f32" else 2e-3


def edge_ambiguous(z, w: float) -> np.ndarray:
    z64 = np.asarray(z, dtype=np.float32).astype(np.float64)
    edge = np.round(z64 / w) * w
    return np.abs(z64 - edge) <= EDGE_REL * np.maximum(1.0, np.abs(edge))


def mass_tie(sel: oracle.Selection, b_gpu: int, p: float) -> bool:
    C = np.cumsum(sel.hist)
    Z = C[-1]
    b = sel.bstar
    if b_gpu == b + 1:
        return abs(C[b] - p * Z) <= TIE_REL * Z
    if b_gpu == b - 1 and b >= 1:
        return abs(C[b - 1] - p * Z) <= TIE_REL * Z
    return False


def count_tie(z, sel: oracle.Selection, b_gpu: int, k: int, w: float) -> bool:
    """A different b* under top-k is explained only by edge-band tokens: the oracle's
    cumulative count at the lower of the two bins lies within that many tokens of k."""
    n_amb = int(edge_ambiguous(z, w).sum())
    if n_amb == 0:
        return False
    C = np.cumsum(sel.hist)
    lo = min(b_gpu, sel.bstar)
    return abs(C[lo] - k) <= n_amb


class SelCheck:
    def __init__(self):
        self.mass_ties = 0
        self.edge_tokens = 0
        self.rows = 0


def expected_set(z, sel: oracle.Selection, A_gpu: int, b_gpu: int, p: float, w: float,
                 stats: SelCheck, where: str, topk: int = 0) -> np.ndarray:
    """Validate (A, b*) from the GPU and return the oracle rule's set under them
    (top-p with p, or the fixed top-k rule when topk > 0)."""
    stats.rows += 1
    if A_gpu != sel.A:
        zmax_edge = edge_ambiguous(np.array([np.max(z)]), w)[0]
        assert abs(A_gpu - sel.A) == 1 and zmax_edge, \
            "%s: top cell %d != oracle %d" % (where, A_gpu, sel.A)
    if b_gpu != sel.bstar:
        ok = count_tie(z, sel, b_gpu, topk, w) if topk > 0 else mass_tie(sel, b_gpu, p)
        assert ok, "%s: b* %d != oracle %d (no %s tie)" % (where, b_gpu, sel.bstar,
                                                          "count" if topk > 0 else "mass")
        stats.mass_ties += 1
    if A_gpu == sel.A and b_gpu == sel.bstar:
        return sel.idx
    return oracle.select_with_bstar(z, A_gpu, b_gpu, w)


def compare_sets(gpu_idx: np.ndarray, exp_idx: np.ndarray, z, w: float, stats: SelCheck,
                 where: str):
    g = set(np.asarray(gpu_idx).tolist())
    e = set(np.asarray(exp_idx).tolist())
    if g == e:
        return
    diff = np.array(sorted(g ^ e), dtype=np.int64)
    amb = edge_ambiguous(np.asarray(z)[diff], w)
    assert amb.all(), "%s: %d tokens differ, %d not near a bin edge (first %s)" % (
        where, len(diff), int((~amb).sum()), diff[~amb][:8].tolist())
    stats.edge_tokens += len(diff)


def compare_count(gpu_count: int, exp_idx: np.ndarray, z, w: float, A: int, b: int,
                  stats: SelCheck, where: str):
    """Set sizes must agree up to tokens in the edge band of the threshold cell."""
    if gpu_count == len(exp_idx):
        return
    T = A - b
    zz = np.asarray(z, dtype=np.float32).astype(np.float64)
    near = np.abs(zz - T * w) <= EDGE_REL * max(1.0, abs(T * w))
    assert abs(gpu_count - len(exp_idx)) <= int(near.sum()), "%s: count %d != oracle %d" % (
        where, gpu_count, len(exp_idx))
    stats.edge_tokens += abs(gpu_count - len(exp_idx))


def max_err(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))))
