"""Plain fp64 NumPy statement of one CSA / HCA attention layer (decode and prefill).

Test infrastructure only: the product path never imports, links or runs this
package; tests, the smoke check and the benchmark's CPU baseline do.

Sources (web pages summarising the DeepSeek-V4 technical report):
  [W1] "DeepSeek-V4: Towards Highly Efficient Million-Token Context Intelligence"
       (awesome-system-papers.pages.dev), sections "核心方法 / Hybrid CSA + HCA
       Attention" and "关键观察" (observation 1).
  [W2] "DeepSeek-V4 深读：百万 Token 不是窗口数字，而是一整套系统契约"
       (ricardokevins.github.io), sections "模型全貌" (spec table), "CSA：4× 压缩
       之后再 top-k" (compression equation), "HCA：128× 压缩后保留 dense 全局视野",
       and the stability-details paragraph that closes the CSA/HCA section.
  [W3] "AI深一度 第15期|DeepSeek V4" (yeyulingfeng.com), sections 一 and 二.
  [W4] "DeepSeek-V4 论文解读" (researchpapers.dev), section "注意力栈".
  [W5] "拆解 DeepSeekv4" (daixd5520.github.io), sections CSA, HCA and 细节.

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
  * one shared vector per entry serves as key and value (W2 CSA/HCA intro);
  * gate logits are per (token, channel), biases per (offset in window, channel);
  * entry i = 0 has no b-branch candidates;
  * only complete blocks become entries;
  * RMSNorm has weight 1 and eps 1e-6, on main entries and on queries;
  * RoPE rotates interleaved pairs (x[2u], x[2u+1]) of the last d_r dims with
    inverse frequency theta**(-2u/d_r); entry i sits at position m*i;
  * softmax scale 1/sqrt(d); indexer scores carry no scale;
  * a decode query at position t sees entries i < floor(t/m) and raw window
    tokens max(0, t-n_win+1) .. t; window and compressed entries are not deduplicated;
  * top-k ties go to the lower index, the output is ascending, padded with -1.
"""
from __future__ import annotations

import math

import numpy as np

from . import formats as F

RMS_EPS = 1e-6

# --------------------------------------------------------------------- compression


def entry_range(pos0: int, n_rows: int, m: int, overlap: bool):
    """Absolute indices [i_first, i_end) of the entries a block of rows completes.

    Row r holds the token at absolute position pos0 + r (pos0 a multiple of m).
    Entry i needs its own block [m*i, m*i+m) and, with overlap and i >= 1, the
    previous block [m*(i-1), m*i) (W2 compression equation: the b-branch sums
    over j = m(i-1) .. mi-1).  Incomplete trailing blocks stay raw.
    """
    assert pos0 % m == 0
    first = pos0 // m + (1 if (overlap and pos0 > 0) else 0)
    end = (pos0 + n_rows) // m
    return first, max(first, end)


def pool(ca, za, ba, m, pos0=0, cb=None, zb=None, bb=None):
    """Softmax-gated, position-biased pooling of every m tokens into one entry.

    W2 compression equation (CSA section): for entry i,
        C_i = sum_{j=mi}^{m(i+1)-1} S^a_j * C^a_j + sum_{j=m(i-1)}^{mi-1} S^b_j * C^b_j
    where S is a softmax taken separately for every channel over all the
    candidates (W2: each channel has its own softmax; W3 section 一 and W4: the
    weights come from gates plus a learned position bias).  The logit of token j
    in the a-branch is Z^a_j + B^a_{j-mi}; in the b-branch Z^b_j + B^b_{j-m(i-1)}.
    Without cb (HCA, W2 HCA section: no overlap) only the a-branch exists.

    ca, za, cb, zb: [n_rows, D] rows at absolute positions pos0 ...; za/zb None
    means logit 0; ba/bb: [m, D] or None.
    Returns (i_first, entries [n, D], weights list) with weights[k] the
    [n_cand, D] softmax of entry i_first + k.
    """
    ca = np.asarray(ca, dtype=np.float64)
    n_rows, D = ca.shape
    overlap = cb is not None
    first, end = entry_range(pos0, n_rows, m, overlap)
    za = np.zeros_like(ca) if za is None else np.asarray(za, dtype=np.float64)
    ba = np.zeros((m, D)) if ba is None else np.asarray(ba, dtype=np.float64)
    if overlap:
        cb = np.asarray(cb, dtype=np.float64)
        zb = np.zeros_like(cb) if zb is None else np.asarray(zb, dtype=np.float64)
        bb = np.zeros((m, D)) if bb is None else np.asarray(bb, dtype=np.float64)
    out = np.zeros((end - first, D))
    weights = []
    for k, i in enumerate(range(first, end)):
        ra = m * i - pos0
        logits = [za[ra:ra + m] + ba]
        values = [ca[ra:ra + m]]
        if overlap and i >= 1:
            rb = m * (i - 1) - pos0
            logits.append(zb[rb:rb + m] + bb)
            values.append(cb[rb:rb + m])
        logits = np.concatenate(logits, axis=0)
        values = np.concatenate(values, axis=0)
        top = logits.max(axis=0)
        e = np.exp(logits - top)
        s = e / e.sum(axis=0)
        weights.append(s)
        out[k] = (s * values).sum(axis=0)
    return first, out, weights


def rmsnorm(x, eps: float = RMS_EPS):
    """x / sqrt(mean(x^2) + eps) over the last axis, weight 1 (W2 stability
    paragraph, W5 细节: queries and the compressed KV are RMS-normalised)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rope(x, pos, theta: float, d_r: int):
    """Rotate the last d_r dims of x at position pos (partial RoPE, W1 and W2:
    the last 64 dims; W2 spec table: theta 160000 on the compressed branch).

    Pairs are (x[2u], x[2u+1]) inside the last d_r dims, angle pos * theta**(-2u/d_r).
    pos may be an array broadcasting against x[..., 0].
    """
    x = np.array(x, dtype=np.float64, copy=True)
    if d_r == 0:
        return x
    d = x.shape[-1]
    u = np.arange(d_r // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * u / d_r)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    xe = x[..., d - d_r::2].copy()
    xo = x[..., d - d_r + 1::2].copy()
    x[..., d - d_r::2] = xe * c - xo * s
    x[..., d - d_r + 1::2] = xe * s + xo * c
    return x


def quantise_main(x, d_r: int):
    """Main KV entry storage (W2 stability paragraph, W3 section 二): dims
    [0, d-d_r) in FP8 E4M3FN, the RoPE dims in BF16.  Returns (fp8 codes, bf16 codes)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    return F.encode_e4m3fn(x[..., :d - d_r]), F.encode_bf16(x[..., d - d_r:])


def dequantise_main(nope_codes, rope_codes):
    return np.concatenate([F.decode_e4m3fn(nope_codes), F.decode_bf16(rope_codes)], axis=-1)


def main_entries(ca, za, ba, m, pos0, theta, d_r, cb=None, zb=None, bb=None, norm=True):
    """Pooled main-KV entries after RMSNorm and RoPE at their positions (fp64,
    before storage).  Entry i sits at position m*i."""
    first, e, _ = pool(ca, za, ba, m, pos0, cb, zb, bb)
    if norm:
        e = rmsnorm(e)
    pos = m * np.arange(first, first + e.shape[0])
    return first, rope(e, pos, theta, d_r)


def window_tokens(kv, pos0, theta, d_r, norm=True):
    """Raw window tokens (m = 1, no gate): RMSNorm then RoPE at the token's own position."""
    kv = np.asarray(kv, dtype=np.float64)
    x = rmsnorm(kv) if norm else kv
    return rope(x, pos0 + np.arange(kv.shape[0]), theta, d_r)


def indexer_keys(ca, za, ba, m, pos0, cb=None, zb=None, bb=None):
    """Indexer keys: the same overlapped pooling on the indexer's own inputs
    (W2 Fig. 2 caption: the indexer compresses history separately), with no
    norm and no RoPE; stored as MXFP4 (W2 FP4 QAT section)."""
    return pool(ca, za, ba, m, pos0, cb, zb, bb)[:2]


# --------------------------------------------------------------------- indexer


def visible_entries(t: int, m: int, n_entries: int) -> int:
    """A query cannot select the block that contains it (W1 observation 1,
    W5 细节): entries i < floor(t/m) are visible, bounded by those present."""
    return max(0, min(t // m, n_entries))


def index_scores(q_idx, w, keys, n_vis: int):
    """Lightning indexer (W2 CSA section, W5 CSA step 2):
    I_i = sum_h w_h * ReLU(q_h . k_i) over the visible entries.

    q_idx [H_I, d_I], w [H_I], keys [>= n_vis, d_I] -> [n_vis] fp64.
    """
    q = np.asarray(q_idx, dtype=np.float64)
    k = np.asarray(keys, dtype=np.float64)[:n_vis]
    dots = k @ q.T
    return (np.maximum(dots, 0.0) * np.asarray(w, dtype=np.float64)).sum(axis=1)


def topk(scores, k: int):
    """The k best entries (W2 spec table: top-k 512 Flash / 1024 Pro): highest
    score first, ties to the lower index; returned ascending, padded with -1."""
    scores = np.asarray(scores, dtype=np.float64)
    n = scores.shape[0]
    if n <= k:
        sel = np.arange(n)
    else:
        order = np.lexsort((np.arange(n), -scores))  # primary: score desc, then index asc
        sel = np.sort(order[:k])
    out = np.full(k, -1, dtype=np.int64)
    out[:sel.shape[0]] = sel
    return out


# --------------------------------------------------------------------- attention


def attend_core(q, t, kv, sink, theta, d_r, scale=None, norm_q=True, inv_rope=True):
    """Shared-KV multi-query attention with a per-head sink for one query.

    q [H, d] un-rotated query heads; kv [N, d] rows that serve as both key and
    value (W2: one 512-d shared KV entry read by all heads); sink [H].
    s_hj = (R_t q_h) . kv_j * scale (scale 1/sqrt(d));
    o_h  = sum_j e^{s_hj} kv_j / (e^{z_h} + sum_j e^{s_hj})  (W2 stability
    paragraph, W5 细节: exp(z_h) joins the denominator, so the weights may sum to
    less than 1); then the last d_r dims of o_h are rotated back by -t (W2: the
    output receives the inverse position rotation).
    Returns (o [H, d], lse [H]) with lse = log sum_j e^{s_hj} (-inf when N = 0).
    """
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    sink = np.asarray(sink, dtype=np.float64)
    H, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if norm_q:
        q = rmsnorm(q)
    qr = rope(q, t, theta, d_r)
    if kv.shape[0] == 0:
        return np.zeros((H, d)), np.full(H, -np.inf)
    s = (qr @ kv.T) * scale
    top = np.maximum(s.max(axis=1), sink)
    p = np.exp(s - top[:, None])
    den = np.exp(sink - top) + p.sum(axis=1)
    o = (p @ kv) / den[:, None]
    lse = top + np.log(p.sum(axis=1))
    if inv_rope:
        o = rope(o, -t, theta, d_r)
    return o, lse


def window_rows(t: int, n_win: int, win_pos0: int, win_len: int):
    """Buffer rows of the raw window of query t: positions max(0, t-n_win+1) .. t
    (W1: sliding window of 128 raw tokens), restricted to what the buffer holds."""
    lo = max(0, t - n_win + 1, win_pos0)
    hi = min(t, win_pos0 + win_len - 1)
    return np.arange(lo - win_pos0, hi - win_pos0 + 1) if hi >= lo else np.arange(0)


def csa_attend(q, t, entries, idx, window, win_pos0, n_win, sink, theta, d_r, m,
               n_entries=None, **kw):
    """CSA main attention for one query: the selected compressed entries
    concatenated with the raw window (W2 Fig. 2 caption; W1 CSA bullet).
    Indices < 0 or outside the visible range are ignored."""
    entries = np.asarray(entries, dtype=np.float64)
    n_entries = entries.shape[0] if n_entries is None else n_entries
    n_vis = visible_entries(t, m, n_entries)
    idx = np.asarray(idx)
    sel = idx[(idx >= 0) & (idx < n_vis)]
    rows = window_rows(t, n_win, win_pos0, np.asarray(window).shape[0])
    kv = np.concatenate([entries[sel], np.asarray(window, dtype=np.float64)[rows]], axis=0)
    return attend_core(q, t, kv, sink, theta, d_r, **kw)


def hca_attend(q, t, entries, window, win_pos0, n_win, sink, theta, d_r, m,
               n_entries=None, **kw):
    """HCA: dense attention over every visible compressed entry plus the raw
    window (W2 HCA section; W5 HCA step 2)."""
    entries = np.asarray(entries, dtype=np.float64)
    n_entries = entries.shape[0] if n_entries is None else n_entries
    n_vis = visible_entries(t, m, n_entries)
    rows = window_rows(t, n_win, win_pos0, np.asarray(window).shape[0])
    kv = np.concatenate([entries[:n_vis], np.asarray(window, dtype=np.float64)[rows]], axis=0)
    return attend_core(q, t, kv, sink, theta, d_r, **kw)
