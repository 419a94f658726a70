"""Whole-layer steps of the oracle over generator inputs (NumPy, per sequence).

Test infrastructure only.  Each function composes oracle.csa in the order the
pages give: compress (W2 compression equation; W3 section 一) -> indexer score
-> top-k (W2 Fig. 2 caption) -> shared-KV attention over the selected entries,
the raw window and the sink (W2 stability paragraph); HCA skips the indexer
(W2 HCA section).  Storage rounding happens where the layer stores: main
entries and window tokens to FP8/BF16, indexer keys to MXFP4 (W3 section 二).
"""
from __future__ import annotations

import numpy as np

from . import csa as C
from . import formats as F


def _np(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu()
        if str(x.dtype) == "torch.bfloat16":
            import torch
            return x.float().numpy().astype(np.float64)  # bf16 -> f32 is exact
        return x.numpy()
    return np.asarray(x)


# ------------------------------------------------------------------ fp32 (tiny) pipeline


def tiny_step(shape, inp, b=0):
    """fp32 workload, every stage from raw tokens; nothing is quantised.

    Returns a dict with entries, (keys, scores, sel) for CSA, window rows, and
    the attention output / log-sum-exp of each query.
    """
    main = {k: _np(v) for k, v in inp["main"].items()}
    L, m = shape.L, shape.m
    cb = main["cb"][b] if shape.overlap else None
    zb = main["zb"][b] if shape.overlap else None
    bb = main["bb"] if shape.overlap else None
    first, ent = C.main_entries(main["ca"][b], main["za"][b], main["ba"], m, 0, shape.theta,
                                shape.d_r, cb, zb, bb)
    assert first == 0
    win = C.window_tokens(_np(inp["win_raw"])[b], 0, shape.theta, shape.d_r)
    res = {"entries": ent, "window": win, "out": [], "lse": []}
    q = _np(inp["q"])[b]
    sink = _np(inp["sink"])
    qpos = _np(inp["q_pos"])[b]
    if shape.csa:
        ix = {k: _np(v) for k, v in inp["idx"].items()}
        _, keys = C.indexer_keys(ix["ca"][b], ix["za"][b], ix["ba"], m, 0, ix["cb"][b],
                                 ix["zb"][b], ix["bb"])
        res["keys"] = keys
        res["scores"], res["sel"] = [], []
    for r, t in enumerate(qpos):
        t = int(t)
        if shape.csa:
            n_vis = C.visible_entries(t, m, ent.shape[0])
            sc = C.index_scores(_np(inp["q_idx"])[b, r], _np(inp["w"])[b, r], keys, n_vis)
            sel = C.topk(sc, shape.top_k)
            res["scores"].append(sc)
            res["sel"].append(sel)
            o, lse = C.csa_attend(q[r], t, ent, sel, win, 0, shape.n_win, sink, shape.theta,
                                  shape.d_r, m)
        else:
            o, lse = C.hca_attend(q[r], t, ent, win, 0, shape.n_win, sink, shape.theta,
                                  shape.d_r, m)
        res["out"].append(o)
        res["lse"].append(lse)
    return res


# ------------------------------------------------------------------ quantised decode


def stored_main(nope_codes, rope_codes):
    return C.dequantise_main(nope_codes, rope_codes)


def split_entry_bytes(rows_u8, d_nope):
    """[.., 576] bytes -> (fp8 codes [.., d_nope], bf16 codes [.., d_r])."""
    rows_u8 = np.asarray(rows_u8, dtype=np.uint8)
    nope = rows_u8[..., :d_nope]
    rope = np.ascontiguousarray(rows_u8[..., d_nope:]).view(np.uint16)
    return nope, rope


def decode_entry_bytes(rows_u8, d_nope):
    n, r = split_entry_bytes(rows_u8, d_nope)
    return C.dequantise_main(n, r)


def compress_main_codes(shape, streams, b, pos0):
    """Pooled, normalised, rotated and stored main entries of one sequence.
    Returns (i_first, fp8 codes, bf16 codes, fp64 value before storage)."""
    s = {k: _np(v) for k, v in streams.items()}
    ov = shape.overlap
    first, ent = C.main_entries(s["ca"][b], s["za"][b], s["ba"], shape.m, pos0, shape.theta,
                                shape.d_r, s["cb"][b] if ov else None,
                                s["zb"][b] if ov else None, s["bb"] if ov else None)
    nope, rope = C.quantise_main(ent, shape.d_r)
    return first, nope, rope, ent


def compress_index_codes(shape, streams, b, pos0):
    s = {k: _np(v) for k, v in streams.items()}
    first, keys = C.indexer_keys(s["ca"][b], s["za"][b], s["ba"], shape.m, pos0, s["cb"][b],
                                 s["zb"][b], s["bb"])
    codes, scales = F.encode_mxfp4(keys)
    return first, codes, scales, keys


def window_codes(shape, raw_rows, pos0):
    x = C.window_tokens(_np(raw_rows), pos0, shape.theta, shape.d_r)
    nope, rope = C.quantise_main(x, shape.d_r)
    return nope, rope, x


def _take(t, b, ids):
    """Rows ids of sequence b of a [B, n, ...] array or tensor (host copy)."""
    ids = np.asarray(ids, dtype=np.int64)
    if hasattr(t, "detach"):
        import torch
        return _np(t[b][torch.as_tensor(ids, device=t.device)])
    return np.asarray(t)[b][ids]


def decode_step(shape, inp, b, sfx="", sel=None):
    """One decode step of sequence b at t = L (the quantised workloads).

    The step compresses the newest block(s) (entry L/m - 1 from rows
    [L - m*(1+overlap), L)), stores the new token in the window, scores and
    selects (CSA), then attends.  Caches are read as the stored codes, decoded
    exactly.  `sel` replaces the oracle's own top-k set in the attention (to
    score the GPU's output on the GPU's legal tie choice).  Returns a dict of
    every intermediate.
    """
    L, m = shape.L, shape.m
    d_nope = shape.d_nope
    t = L
    n_e = L // m
    rows_c = m * (2 if shape.overlap else 1)
    first, nope, rope, exact = compress_main_codes(shape, inp["main"], b, L - rows_c)
    assert first == n_e - 1 and nope.shape[0] == 1
    newest = C.dequantise_main(nope[0], rope[0])

    def cache_rows(ids):
        ids = np.asarray(ids, dtype=np.int64)
        vals = decode_entry_bytes(_take(inp["cache" + sfx], b, ids), d_nope)
        vals[ids == first] = newest
        return vals

    wn, wr, wexact = window_codes(shape, _np(inp["win_raw"])[b], L)
    win = decode_entry_bytes(_np(inp["win"])[b], d_nope)
    win[-1] = C.dequantise_main(wn[0], wr[0])
    win_pos0 = L - shape.n_win + 1
    q = _np(inp["q"])[b, 0]
    sink = _np(inp["sink"])
    n_vis = C.visible_entries(t, m, n_e)
    res = {"entry_codes": (nope[0], rope[0]), "entry_exact": exact[0], "entry_index": first,
           "win_codes": (wn[0], wr[0]), "win_exact": wexact[0], "n_vis": n_vis}
    if shape.csa:
        kf, kc, ks, kexact = compress_index_codes(shape, inp["idx"], b, L - rows_c)
        codes = _np(inp["keys_codes" + sfx][b]).copy()
        scales = _np(inp["keys_scales" + sfx][b]).copy()
        codes[kf] = kc[0]
        scales[kf] = ks[0]
        keys = F.decode_mxfp4(codes, scales)
        qI = F.decode_mxfp4(_np(inp["q_idx_codes"])[b, 0], _np(inp["q_idx_scales"])[b, 0])
        sc = C.index_scores(qI, _np(inp["w"])[b, 0], keys, n_vis)
        own = C.topk(sc, shape.top_k)
        use = own if sel is None else np.asarray(sel)
        ids = use[(use >= 0) & (use < n_vis)]
        res.update(key_codes=(kc[0], ks[0]), key_exact=kexact[0], key_index=kf, scores=sc, sel=own)
    else:
        ids = np.arange(n_vis)
    rows = C.window_rows(t, shape.n_win, win_pos0, shape.n_win)
    kv = np.concatenate([cache_rows(ids), win[rows]], axis=0)
    o, lse = C.attend_core(q, t, kv, sink, shape.theta, shape.d_r)
    res.update(out=o, lse=lse, window=win)
    return res


# ------------------------------------------------------------------ quantised prefill


def prefill_prepare(shape, inp, b):
    """Everything the chunk itself adds to the caches of sequence b: the new
    main entries (stored codes), indexer keys (stored codes) and window rows."""
    L, m = shape.L, shape.m
    tail = m if shape.overlap else 0
    first, nope, rope, exact = compress_main_codes(shape, inp["main"], b, L - tail)
    assert first == L // m
    out = {"first": first, "nope": nope, "rope": rope, "exact": exact}
    wn, wr, wexact = window_codes(shape, _np(inp["win_raw"])[b], L)
    out.update(win_nope=wn, win_rope=wr, win_exact=wexact)
    if shape.csa:
        kf, kc, ks, kexact = compress_index_codes(shape, inp["idx"], b, L - tail)
        assert kf == first
        out.update(key_codes=kc, key_scales=ks, key_exact=kexact)
    return out


def prefill_query(shape, inp, prep, b, r, sel=None):
    """Oracle result of query r (position L + r) of sequence b in a prefill chunk."""
    L, m = shape.L, shape.m
    t = L + r
    n_old = L // m
    n_all = n_old + prep["nope"].shape[0]
    n_vis = C.visible_entries(t, m, n_all)
    d_nope = shape.d_nope

    def cache_rows(ids):
        ids = np.asarray(ids, dtype=np.int64)
        old = ids[ids < n_old]
        new = ids[ids >= n_old] - n_old
        v = np.empty((ids.shape[0], shape.d))
        v[ids < n_old] = decode_entry_bytes(_take(inp["cache_old"], b, old), d_nope)
        v[ids >= n_old] = C.dequantise_main(prep["nope"][new], prep["rope"][new])
        return v

    res = {"t": t, "n_vis": n_vis}
    if shape.csa:
        n_o = min(n_vis, n_old)
        keys = np.concatenate([
            F.decode_mxfp4(_take(inp["keys_codes_old"], b, np.arange(n_o)),
                           _take(inp["keys_scales_old"], b, np.arange(n_o))),
            F.decode_mxfp4(prep["key_codes"][:max(0, n_vis - n_old)],
                           prep["key_scales"][:max(0, n_vis - n_old)])], axis=0)
        qI = F.decode_mxfp4(_take(inp["q_idx_codes"], b, [r])[0], _take(inp["q_idx_scales"], b, [r])[0])
        sc = C.index_scores(qI, _take(inp["w"], b, [r])[0], keys, n_vis)
        own = C.topk(sc, shape.top_k)
        use = own if sel is None else np.asarray(sel)
        ids = use[(use >= 0) & (use < n_vis)]
        res.update(scores=sc, sel=own)
    else:
        ids = np.arange(n_vis)
    # window buffer: rows 0 .. n_win-2 hold positions L-n_win+1 .. L-1, then the chunk
    win_pos0 = L - shape.n_win + 1
    rows = C.window_rows(t, shape.n_win, win_pos0, shape.n_win - 1 + inp["q"].shape[1])
    old_w = rows[rows < shape.n_win - 1]
    new_w = rows[rows >= shape.n_win - 1] - (shape.n_win - 1)
    wv = np.concatenate([decode_entry_bytes(_take(inp["win_old"], b, old_w), d_nope),
                         C.dequantise_main(prep["win_nope"][new_w], prep["win_rope"][new_w])], axis=0)
    kv = np.concatenate([cache_rows(ids), wv], axis=0)
    q = _take(inp["q"], b, [r])[0]
    o, lse = C.attend_core(q, t, kv, _np(inp["sink"]), shape.theta, shape.d_r)
    res.update(out=o, lse=lse)
    return res


def attend_with_selection(shape, q, t, cache, sel, win, win_pos0, sink):
    """CSA attention with a given selection (used to score the GPU output against
    the GPU's own legal tie choice)."""
    return C.csa_attend(q, t, cache, sel, win, win_pos0, shape.n_win, sink, shape.theta,
                        shape.d_r, shape.m)
