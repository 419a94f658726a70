"""Seeded synthetic inputs for the CSA / HCA layer, shared by the GPU path's tests,
the benchmark and the oracle's tests.

This module draws random numbers and lays them out; it holds none of the
layer's arithmetic (no pooling, normalisation, rotation, scoring or
quantisation of its own).  Values that must already be stored in a cache
format are produced either by torch's own casts (float8_e4m3fn, bfloat16) or,
for MXFP4 where torch has no cast, drawn directly as codes from a fixed
categorical distribution.

Shapes follow the workloads on the pages (W2 spec table: Flash 64 heads /
top-k 512, Pro 128 heads / top-k 1024, head dim 512, one KV head, RoPE 64,
window 128, CSA m = 4, HCA m' = 128, theta 160000; indexer 64 heads x 128).
"""
from __future__ import annotations

import dataclasses
import hashlib

import torch

# ------------------------------------------------------------------ shapes


@dataclasses.dataclass(frozen=True)
class Shape:
    name: str
    B: int            # sequences
    L: int            # tokens already in context (positions 0 .. L-1)
    n_q: int          # new query tokens per sequence (1 = decode)
    H: int            # query heads
    d: int            # head dim (shared KV width)
    d_r: int          # RoPE dims (the last d_r)
    m: int            # compression of this layer (4 CSA, 128 HCA)
    overlap: bool     # CSA pools the previous block too
    top_k: int        # CSA only
    H_I: int          # indexer heads (CSA only)
    d_I: int          # indexer dim (CSA only)
    n_win: int        # raw sliding window
    theta: float = 160000.0
    fp32: bool = False
    planted: float = 0.0   # fraction of indexer keys carrying a query-aligned direction
    seed: int = 0
    signed_w: bool = False  # indexer head weights N(0,1)/sqrt(H_I) instead of |N(0,1)|/sqrt(H_I)
    mx_exp: tuple = ()      # (lo, hi): MXFP4 block exponents uniform on lo..hi instead of -2..0

    @property
    def csa(self) -> bool:
        return self.overlap

    @property
    def d_nope(self) -> int:
        return self.d - self.d_r

    def replace(self, **kw) -> "Shape":
        return dataclasses.replace(self, **kw)


# The five workloads.  The tiny one runs the whole pipeline from raw tokens in
# fp32; the others are quantised (FP8/BF16 main KV, MXFP4 indexer).
TINY_CSA = Shape("tiny-csa", B=1, L=2048, n_q=1, H=8, d=64, d_r=16, m=4, overlap=True,
                 top_k=32, H_I=4, d_I=32, n_win=16, fp32=True, seed=0)
TINY_HCA = Shape("tiny-hca", B=1, L=2048, n_q=1, H=8, d=64, d_r=16, m=32, overlap=False,
                 top_k=0, H_I=0, d_I=0, n_win=16, fp32=True, seed=0)
FLASH_CSA_DECODE = Shape("flash-csa-decode-128k", B=16, L=131072, n_q=1, H=64, d=512, d_r=64,
                         m=4, overlap=True, top_k=512, H_I=64, d_I=128, n_win=128, seed=2)
FLASH_HCA_DECODE = Shape("flash-hca-decode-1m", B=32, L=1 << 20, n_q=1, H=64, d=512, d_r=64,
                         m=128, overlap=False, top_k=0, H_I=0, d_I=0, n_win=128, seed=3)
PRO_CSA_DECODE = Shape("pro-csa-decode-1m", B=8, L=1 << 20, n_q=1, H=128, d=512, d_r=64,
                       m=4, overlap=True, top_k=1024, H_I=64, d_I=128, n_win=128,
                       planted=0.01, seed=4)
PRO_CSA_PREFILL = Shape("pro-csa-prefill-8k-after-1m", B=1, L=1 << 20, n_q=8192, H=128, d=512,
                        d_r=64, m=4, overlap=True, top_k=1024, H_I=64, d_I=128, n_win=128,
                        seed=5)
PRO_HCA_PREFILL = Shape("pro-hca-prefill-8k-after-1m", B=1, L=1 << 20, n_q=8192, H=128, d=512,
                        d_r=64, m=128, overlap=False, top_k=0, H_I=0, d_I=0, n_win=128, seed=5)

ENTRY_BYTES = 576     # 448 FP8 + 64 x BF16
IDX_BYTES = 68        # 64 B of E2M1 + 4 E8M0 scales

# ------------------------------------------------------------------ RNG


def _gen(shape: Shape, tag: str, device) -> torch.Generator:
    h = hashlib.sha256(f"{shape.name}|{shape.seed}|{tag}".encode()).digest()
    g = torch.Generator(device=device)
    g.manual_seed(int.from_bytes(h[:8], "little") & ((1 << 63) - 1))
    return g


def normal(shape: Shape, tag: str, size, device="cpu", std=1.0) -> torch.Tensor:
    g = _gen(shape, tag, device)
    return torch.randn(size, generator=g, device=device, dtype=torch.float32) * std


# Magnitude-code probabilities of E2M1 elements that mimic 2*|N(0,1)| rounded to
# the E2M1 grid {0, .5, 1, 1.5, 2, 3, 4, 6} (bin edges at the midpoints); the
# block scale is drawn around 2**-1 so the decoded values look like N(0,1).
_E2M1_MAG_P = [0.10, 0.19, 0.175, 0.15, 0.17, 0.13, 0.07, 0.015]
_E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
_SCALE_EXP_P = {-2: 0.25, -1: 0.5, 0: 0.25}


def mxfp4_codes(shape: Shape, tag: str, rows: int, D: int, device="cpu"):
    """Random MXFP4 rows: (codes [rows, D/2] uint8, scales [rows, D/32] uint8)."""
    g = _gen(shape, tag, device)
    p = torch.tensor(_E2M1_MAG_P, device=device)
    mag = torch.multinomial(p, rows * D, replacement=True, generator=g).reshape(rows, D)
    sign = torch.randint(0, 2, (rows, D), generator=g, device=device)
    nib = (mag | (sign << 3)).to(torch.uint8)
    if shape.mx_exp:
        lo, hi = shape.mx_exp
        se = torch.randint(lo, hi + 1, (rows * (D // 32),), generator=g, device=device)
    else:
        ex = torch.tensor(list(_SCALE_EXP_P.keys()), device=device)
        pe = torch.tensor(list(_SCALE_EXP_P.values()), device=device)
        se = ex[torch.multinomial(pe, rows * (D // 32), replacement=True, generator=g)]
    scales = (se + 127).to(torch.uint8).reshape(rows, D // 32)
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).to(torch.uint8)
    return codes, scales


def _mxfp4_values_local(codes, scales):
    """Decoded values, used only to aim the planted direction at the query."""
    tab = torch.tensor(_E2M1_TABLE, device=codes.device)
    nib = torch.stack([codes & 0xF, codes >> 4], dim=-1).reshape(*codes.shape[:-1], -1).long()
    v = tab[nib & 7] * torch.where((nib >> 3) & 1 == 1, -1.0, 1.0)
    sc = torch.exp2(scales.float() - 127.0)
    return (v.reshape(*v.shape[:-1], -1, 32) * sc[..., None]).reshape(v.shape)


def plant(shape: Shape, tag: str, codes, scales, q_codes, q_scales, w, device="cpu"):
    """Give a fraction shape.planted of the key rows the direction u = sum_h w_h q_h:
    their element signs follow sign(u) and their magnitudes come from the upper
    half of the E2M1 grid (2 .. 6), which lifts their indexer score by several
    standard deviations.  Returns the planted row indices (sorted)."""
    rows = codes.shape[0]
    n_pl = int(rows * shape.planted)
    if n_pl == 0:
        return torch.zeros(0, dtype=torch.long, device=device)
    g = _gen(shape, tag + "/plant", device)
    which = torch.randperm(rows, generator=g, device=device)[:n_pl].sort().values
    u = (w[:, None] * _mxfp4_values_local(q_codes, q_scales)).sum(0)     # [D]
    D = u.shape[0]
    pm = torch.tensor([0.4, 0.35, 0.2, 0.05], device=device)
    mag = 4 + torch.multinomial(pm, n_pl * D, replacement=True, generator=g).reshape(n_pl, D)
    sign = (u < 0).long().expand(n_pl, D)
    nib = (mag | (sign << 3)).to(torch.uint8)
    codes[which] = (nib[:, 0::2] | (nib[:, 1::2] << 4)).to(torch.uint8)
    scales[which] = 126
    return which


def head_weights(shape: Shape, size, device="cpu"):
    """Indexer head weights: |N(0,1)|/sqrt(H_I), or N(0,1)/sqrt(H_I) with signed_w."""
    w = normal(shape, "w", size, device)
    return (w if shape.signed_w else w.abs()) / shape.H_I ** 0.5


def fp8_bf16_rows(shape: Shape, tag: str, rows: int, device="cpu"):
    """Main-KV rows already in storage form: N(0,1) values cast by torch to
    E4M3FN (dims < d-d_r) and BF16 (last d_r dims), packed as [rows, 576] bytes."""
    x = normal(shape, tag, (rows, shape.d), device)
    nope = x[:, :shape.d_nope].to(torch.float8_e4m3fn).view(torch.uint8)
    rope = x[:, shape.d_nope:].to(torch.bfloat16).contiguous().view(torch.uint8)
    return torch.cat([nope, rope], dim=1).contiguous()


# ------------------------------------------------------------------ layer inputs


def raw_streams(shape: Shape, prefix: str, rows: int, D: int, device, dtype, overlap: bool):
    """Compressor inputs: C^a, Z^a (and C^b, Z^b with overlap) as [B, rows, D];
    biases B^a (B^b) [m, D] ~ N(0, 0.1^2)."""
    out = {}
    names = ["ca", "za"] + (["cb", "zb"] if overlap else [])
    for n in names:
        out[n] = normal(shape, f"{prefix}/{n}", (shape.B, rows, D), device).to(dtype)
    out["ba"] = normal(shape, f"{prefix}/ba", (shape.m, D), device, std=0.1)
    if overlap:
        out["bb"] = normal(shape, f"{prefix}/bb", (shape.m, D), device, std=0.1)
    return out


def tiny_inputs(shape: Shape, device="cpu"):
    """Raw-token inputs of the tiny fp32 workload: the whole context is compressed
    from scratch; the decode query sits at t = L and its own token joins the window."""
    T = shape.L
    f32 = torch.float32
    inp = {"main": raw_streams(shape, "main", T, shape.d, device, f32, shape.overlap),
           "win_raw": normal(shape, "win", (shape.B, T + shape.n_q, shape.d), device),
           "q": normal(shape, "q", (shape.B, shape.n_q, shape.H, shape.d), device),
           "sink": normal(shape, "sink", (shape.H,), device),
           "q_pos": torch.full((shape.B, shape.n_q), shape.L, dtype=torch.int64, device=device)
           + torch.arange(shape.n_q, device=device)}
    if shape.csa:
        inp["idx"] = raw_streams(shape, "idx", T, shape.d_I, device, f32, True)
        inp["q_idx"] = normal(shape, "q_idx", (shape.B, shape.n_q, shape.H_I, shape.d_I), device)
        inp["w"] = normal(shape, "w", (shape.B, shape.n_q, shape.H_I), device).abs() / shape.H_I ** 0.5
    return inp


def quant_decode_inputs(shape: Shape, device="cpu", copies: int = 1):
    """Inputs of one quantised decode step at t = L (config shapes; caches already
    in storage form).  The step's own compress calls read the raw rows of the
    last complete block(s) and of the new token.

    Keys: 'cache' [B, L/m, 576] u8, 'win' [B, n_win, 576] u8 (rows for positions
    t-n_win+1 .. t; the last row is rewritten by the step), raw streams, q, sink
    and, for CSA, indexer keys/queries/weights.  With copies > 1 the caches are
    replicated (cache_1, ...) so consecutive steps can rotate between them.
    """
    B, L = shape.B, shape.L
    n_e = L // shape.m
    bf = torch.bfloat16
    inp = {"q_pos": torch.full((B, 1), L, dtype=torch.int64, device=device),
           "win_pos0": torch.full((B,), L - shape.n_win + 1, dtype=torch.int64, device=device),
           "sink": normal(shape, "sink", (shape.H,), device),
           "q": normal(shape, "q", (B, 1, shape.H, shape.d), device).to(bf)}
    rows_c = shape.m * (2 if shape.overlap else 1)       # rows behind the newest entry
    inp["main"] = raw_streams(shape, "main", rows_c, shape.d, device, bf, shape.overlap)
    inp["win_raw"] = normal(shape, "win_raw", (B, 1, shape.d), device).to(bf)
    inp["win"] = fp8_bf16_rows(shape, "win", B * shape.n_win, device).reshape(B, shape.n_win, -1)
    for c in range(copies):
        sfx = "" if c == 0 else f"_{c}"
        inp["cache" + sfx] = fp8_bf16_rows(shape, f"cache{sfx}", B * n_e, device).reshape(B, n_e, -1)
    if shape.csa:
        inp["idx"] = raw_streams(shape, "idx", rows_c, shape.d_I, device, bf, True)
        qc, qs = mxfp4_codes(shape, "q_idx", B * shape.H_I, shape.d_I, device)
        inp["q_idx_codes"] = qc.reshape(B, 1, shape.H_I, -1)
        inp["q_idx_scales"] = qs.reshape(B, 1, shape.H_I, -1)
        inp["w"] = head_weights(shape, (B, 1, shape.H_I), device)
        for c in range(copies):
            sfx = "" if c == 0 else f"_{c}"
            kc, ks = mxfp4_codes(shape, f"keys{sfx}", B * n_e, shape.d_I, device)
            kc = kc.reshape(B, n_e, -1)
            ks = ks.reshape(B, n_e, -1)
            planted = []
            for b in range(B):
                planted.append(plant(shape, f"keys{sfx}/{b}", kc[b], ks[b],
                                     inp["q_idx_codes"][b, 0], inp["q_idx_scales"][b, 0],
                                     inp["w"][b, 0], device))
            inp["keys_codes" + sfx] = kc
            inp["keys_scales" + sfx] = ks
            inp["planted" + sfx] = planted
    return inp


def quant_prefill_inputs(shape: Shape, device="cpu"):
    """Inputs of one quantised prefill chunk: n_q new tokens at positions L .. L+n_q-1
    after an L-token context whose caches are already in storage form.

    The chunk's raw rows start one block early with overlap (the 4-token tail of
    the context feeds the b-branch of the chunk's first entry).  The window
    buffer holds positions L-n_win+1 .. L+n_q-1; its first n_win-1 rows are in
    storage form, the rest are written by the chunk's window-store compress.
    """
    B, L, n_q = shape.B, shape.L, shape.n_q
    n_e = L // shape.m
    bf = torch.bfloat16
    tail = shape.m if shape.overlap else 0
    inp = {"q_pos": (L + torch.arange(n_q, device=device, dtype=torch.int64)).expand(B, n_q).contiguous(),
           "win_pos0": torch.full((B,), L - shape.n_win + 1, dtype=torch.int64, device=device),
           "sink": normal(shape, "sink", (shape.H,), device),
           "q": normal(shape, "q", (B, n_q, shape.H, shape.d), device).to(bf),
           "main": raw_streams(shape, "main", tail + n_q, shape.d, device, bf, shape.overlap),
           "win_raw": normal(shape, "win_raw", (B, n_q, shape.d), device).to(bf),
           "win_old": fp8_bf16_rows(shape, "win", B * (shape.n_win - 1), device).reshape(B, shape.n_win - 1, -1),
           "cache_old": fp8_bf16_rows(shape, "cache", B * n_e, device).reshape(B, n_e, -1)}
    if shape.csa:
        inp["idx"] = raw_streams(shape, "idx", tail + n_q, shape.d_I, device, bf, True)
        qc, qs = mxfp4_codes(shape, "q_idx", B * n_q * shape.H_I, shape.d_I, device)
        inp["q_idx_codes"] = qc.reshape(B, n_q, shape.H_I, -1)
        inp["q_idx_scales"] = qs.reshape(B, n_q, shape.H_I, -1)
        inp["w"] = head_weights(shape, (B, n_q, shape.H_I), device)
        kc, ks = mxfp4_codes(shape, "keys", B * n_e, shape.d_I, device)
        inp["keys_codes_old"] = kc.reshape(B, n_e, -1)
        inp["keys_scales_old"] = ks.reshape(B, n_e, -1)
    return inp
