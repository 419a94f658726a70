"""Comparison rules between the GPU path and the fp64 oracle (test helpers).

Tolerances:
  * fp32 mode: max abs error 1e-4 on attention outputs and entries.
  * quantised mode: max abs error 2e-2 on attention outputs (BF16 output; the
    oracle consumes the stored FP8/BF16/MXFP4 codes decoded exactly).
  * storage codes (FP8, BF16, MXFP4): equal, except where the oracle's fp64
    value x lies within REL_CODE * max(|x|, 1) of a rounding midpoint of the
    two candidate codes (or of a power-of-two MXFP4 scale boundary).  The
    entries are O(1) (unit RMS after RMSNorm; pooled N(0,1) rows for the
    indexer), and the GPU computes them in fp32: a 2^-24 rounding per step over
    the pooling (exp2, <= 2m multiply-adds), RMSNorm (a 512-term sum of
    squares) and rotation stays below 1e-5 absolute, so 1e-4 leaves a 10x
    margin; the max(|x|, 1) floor covers entries that cancel to near zero.
  * top-k: both sets have the same size and every index in their symmetric
    difference scores within 1e-3 * |s_k| of the oracle's k-th score s_k.
"""
from __future__ import annotations

import numpy as np

from oracle import formats as F

REL_CODE = 1e-4
TOL_F32 = 1e-4
TOL_QUANT = 2e-2
TIE_REL = 1e-3


def _near_midpoint(exact, a, b, rel=REL_CODE):
    mid = (a + b) / 2
    return np.abs(exact - mid) <= rel * np.maximum(np.abs(exact), 1.0)


def check_fp8_codes(gpu_codes, exact, rel=REL_CODE):
    """GPU E4M3FN codes against the oracle's unrounded values."""
    want = F.encode_e4m3fn(exact)
    g = F.decode_e4m3fn(gpu_codes)
    w = F.decode_e4m3fn(want)
    bad = (g != w) & ~_near_midpoint(exact, g, w, rel)
    assert not bad.any(), f"{bad.sum()} FP8 codes differ away from a rounding midpoint"
    return int((g != w).sum())


def check_bf16_codes(gpu_codes, exact, rel=REL_CODE):
    want = F.encode_bf16(exact)
    g = F.decode_bf16(gpu_codes)
    w = F.decode_bf16(want)
    bad = (g != w) & ~_near_midpoint(exact, g, w, rel)
    assert not bad.any(), f"{bad.sum()} BF16 codes differ away from a rounding midpoint"
    return int((g != w).sum())


def check_mxfp4_codes(gpu_codes, gpu_scales, exact, rel=REL_CODE):
    """Blocks must share the scale unless the block max sits on a power of two;
    elements must agree unless the scaled exact value sits on a midpoint."""
    exact = np.asarray(exact, dtype=np.float64)
    want_c, want_s = F.encode_mxfp4(exact)
    D = exact.shape[-1]
    blocks = exact.reshape(exact.shape[:-1] + (D // 32, 32))
    amax = np.abs(blocks).max(-1)
    scale_diff = gpu_scales != want_s
    if scale_diff.any():
        am = amax[scale_diff]
        edge = np.exp2(np.round(np.log2(np.maximum(am, 1e-300))))
        assert np.all(np.abs(am - edge) <= rel * np.maximum(am, 1.0)), "MXFP4 scale differs off a boundary"
    g = F.decode_mxfp4(gpu_codes, gpu_scales)
    w = F.decode_mxfp4(want_c, want_s)
    same_scale = np.repeat(~scale_diff, 32, axis=-1).reshape(exact.shape)
    diff = (g != w) & same_scale
    bad = diff & ~_near_midpoint(exact, g, w, rel)
    assert not bad.any(), f"{bad.sum()} E2M1 elements differ away from a midpoint"
    return int(diff.sum())


def check_topk(gpu_idx, oracle_scores, k, tie_rel=None):
    """The top-k rule for a GPU selection against the oracle's fp64 scores: tie
    window tie_rel, by default 1e-3 of the k-th score."""
    tie = TIE_REL if tie_rel is None else tie_rel
    gpu_idx = np.asarray(gpu_idx)
    n = oracle_scores.shape[0]
    G = set(int(i) for i in gpu_idx if i >= 0)
    if n <= k:
        assert G == set(range(n)), "every visible entry must be selected"
        assert np.all(gpu_idx[n:] == -1), "padding must be -1"
        return 0
    assert len(G) == k and (gpu_idx >= 0).all()
    assert np.all(np.diff(gpu_idx) > 0), "indices must be ascending"
    order = np.lexsort((np.arange(n), -oracle_scores))
    O = set(int(i) for i in order[:k])
    s_k = oracle_scores[order[k - 1]]
    sym = G ^ O
    for i in sym:
        assert abs(oracle_scores[i] - s_k) <= tie * abs(s_k), \
            f"index {i} (score {oracle_scores[i]}) differs from the oracle away from the k-th score {s_k}"
    return len(sym)


def bf16_to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)
