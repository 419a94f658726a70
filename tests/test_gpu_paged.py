"""Heterogeneous paged KV cache ("DeepSeek-V4: Towards Highly Efficient
Million-Token Context Intelligence", observation 3; "DeepSeek-V4 深读",
heterogeneous KV cache section and Fig. 5): compressed entries in blocks of
128 raw tokens named by block tables, window rows and compressor tails in
per-request rings, one entry compressed per completed block at decode.

Requests at different positions (held back by different delays, so blocks
complete at different steps) advance token by token through the paged decode
path, with physical blocks handed out in a shuffled order.  At checkpoints
(one request still at position 0) the paged state and results must equal,
bitwise, a contiguous recomputation of each request from its whole token
stream (one-shot compression, linear window buffer, one request per call),
and the newest request's results must match the fp64 oracle.
"""
from __future__ import annotations

import ctypes as C

import numpy as np
import pytest
import torch

import synth
from oracle import csa as OC
from oracle import formats as F
from oracle import pipeline as P

from parity_util import TOL_QUANT, bf16_to_np, check_bf16_codes, check_fp8_codes, check_mxfp4_codes, check_topk

pytestmark = pytest.mark.gpu

CSA = synth.Shape("paged-csa", B=3, L=0, n_q=1, H=64, d=512, d_r=64, m=4, overlap=True, top_k=128,
                  H_I=64, d_I=128, n_win=128, signed_w=True, seed=21)
HCA = synth.Shape("paged-hca", B=2, L=0, n_q=1, H=64, d=512, d_r=64, m=128, overlap=False, top_k=0,
                  H_I=0, d_I=0, n_win=128, seed=22)


def _K():
    import long_context_attention_09_amd._lib as K
    K.load()
    return K


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


def _inputs(S, T):
    bf = torch.bfloat16
    inp = {"main": synth.raw_streams(S, "main", T, S.d, "cpu", bf, S.overlap),
           "win_raw": synth.normal(S, "win_raw", (S.B, T, S.d)).to(bf),
           "q": synth.normal(S, "q", (S.B, 1, S.H, S.d)).to(bf),
           "sink": synth.normal(S, "sink", (S.H,))}
    if S.csa:
        inp["idx"] = synth.raw_streams(S, "idx", T, S.d_I, "cpu", bf, True)
        qc, qs = synth.mxfp4_codes(S, "q_idx", S.B * S.H_I, S.d_I)
        inp["q_idx_codes"] = qc.reshape(S.B, 1, S.H_I, -1)
        inp["q_idx_scales"] = qs.reshape(S.B, 1, S.H_I, -1)
        inp["w"] = synth.head_weights(S, (S.B, 1, S.H_I))
    return inp


def _dev(x):
    if isinstance(x, dict):
        return {k: _dev(v) for k, v in x.items()}
    return x.cuda() if isinstance(x, torch.Tensor) else x


def _contiguous(K, S, d, b, t, flags_a, flags_i):
    """Request b at query position t recomputed from its whole token stream:
    entries and keys of tokens [0, t] by one-shot compression into contiguous
    caches, window rows of positions max(0, t-127) .. t into a linear buffer,
    then index + attend for that request alone."""
    n_rows = t + 1
    n_cap = max(n_rows // S.m, 1)
    mn = {k: (v[b:b + 1, :n_rows] if v.dim() == 3 else v) for k, v in d["main"].items()}
    cache = torch.zeros(1, n_cap, 576, dtype=torch.uint8, device="cuda")
    nope, rope = K.split_main(cache)
    jobs = [K.compress_args(mn["ca"], gate_a=mn["za"], bias_a=mn["ba"], kv_b=mn.get("cb"), gate_b=mn.get("zb"),
                            bias_b=mn.get("bb"), m=S.m, pos0=0, out0=nope, out1=rope, d_rope=S.d_r,
                            rope_theta=S.theta, do_norm=True, out_fmt=K.FMT_FP8_BF16)]
    if S.csa:
        ix = {k: (v[b:b + 1, :n_rows] if v.dim() == 3 else v) for k, v in d["idx"].items()}
        kc = torch.zeros(1, n_cap, 64, dtype=torch.uint8, device="cuda")
        ks = torch.zeros(1, n_cap, 4, dtype=torch.uint8, device="cuda")
        jobs.append(K.compress_args(ix["ca"], gate_a=ix["za"], bias_a=ix["ba"], kv_b=ix["cb"], gate_b=ix["zb"],
                                    bias_b=ix["bb"], m=S.m, pos0=0, out0=kc, out1=ks, d_rope=0, do_norm=False,
                                    out_fmt=K.FMT_MXFP4))
    lo = max(0, t - S.n_win + 1)
    win = torch.zeros(1, S.n_win, 576, dtype=torch.uint8, device="cuda")
    wn, wr = K.split_main(win)
    jobs.append(K.compress_args(d["win_raw"][b:b + 1, lo:t + 1], m=1, pos0=lo, out0=wn, out1=wr, d_rope=S.d_r,
                                rope_theta=S.theta, do_norm=True, out_fmt=K.FMT_FP8_BF16, out_row0=lo))
    K.compress_batch(jobs)
    q_pos = torch.full((1, 1), t, dtype=torch.int64, device="cuda")
    win_pos0 = torch.full((1,), lo, dtype=torch.int64, device="cuda")
    res = {"cache": cache, "win": win}
    idx = None
    if S.csa:
        idx = torch.empty(1, 1, S.top_k, dtype=torch.int32, device="cuda")
        sc = torch.empty(1, 1, n_cap, device="cuda")
        K.index_topk(d["q_idx_codes"][b:b + 1], d["w"][b:b + 1], kc, q_pos, m=S.m, top_k=S.top_k, out_idx=idx,
                     q1=d["q_idx_scales"][b:b + 1], k1=ks, fmt=K.FMT_MXFP4, flags=flags_i, out_score=sc)
        res.update(kc=kc, ks=ks, idx=idx, score=sc)
    out = torch.empty(1, 1, S.H, S.d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(1, 1, S.H, device="cuda")
    fn = K.attend if S.csa else K.hca_attend
    fn(d["q"][b:b + 1], q_pos, nope, wn, win_pos0, d["sink"], out, m=S.m, n_win=S.n_win, kv1=rope, win1=wr,
       out_lse=lse, flags=flags_a, **({"idx": idx} if S.csa else {}))
    torch.cuda.synchronize()
    res.update(out=out, lse=lse)
    return res


def _oracle_check(S, inp, b, t, pool_rows, win_rows, keys, sel, out):
    """Request b's paged state and result against the fp64 oracle."""
    n_rows = t + 1
    first, nope, rope, exact = P.compress_main_codes(S, {k: (v[:, :n_rows] if v.dim() == 3 else v)
                                                        for k, v in inp["main"].items()}, b, 0)
    n_e = nope.shape[0]
    if n_e:
        got = pool_rows[:n_e]
        check_fp8_codes(got[:, :S.d_nope], exact[:, :S.d_nope])
        check_bf16_codes(np.ascontiguousarray(got[:, S.d_nope:]).view(np.uint16), exact[:, S.d_nope:])
    lo = max(0, t - S.n_win + 1)
    wn, wr, wexact = P.window_codes(S, inp["win_raw"][b, lo:t + 1].float().numpy(), lo)
    check_fp8_codes(win_rows[:, :S.d_nope], wexact[:, :S.d_nope])
    entries = P.decode_entry_bytes(pool_rows[:n_e], S.d_nope) if n_e else np.zeros((0, S.d))
    window = P.decode_entry_bytes(win_rows, S.d_nope)
    q = bf16_to_np(inp["q"][b, 0])
    sink = inp["sink"].double().numpy()
    n_vis = OC.visible_entries(t, S.m, n_e)
    if S.csa:
        _, kc, ks, kexact = P.compress_index_codes(S, {k: (v[:, :n_rows] if v.dim() == 3 else v)
                                                       for k, v in inp["idx"].items()}, b, 0)
        if n_e:
            check_mxfp4_codes(keys[0][:n_e], keys[1][:n_e], kexact)
        qI = F.decode_mxfp4(inp["q_idx_codes"][b, 0].numpy(), inp["q_idx_scales"][b, 0].numpy())
        kv = F.decode_mxfp4(keys[0][:n_e], keys[1][:n_e]) if n_e else np.zeros((0, S.d_I))
        sc = OC.index_scores(qI, inp["w"][b, 0].double().numpy(), kv, n_vis)
        check_topk(sel, sc, S.top_k)
        o, _ = OC.csa_attend(q, t, entries, sel, window, lo, S.n_win, sink, S.theta, S.d_r, S.m, n_entries=n_e)
    else:
        o, _ = OC.hca_attend(q, t, entries, window, lo, S.n_win, sink, S.theta, S.d_r, S.m, n_entries=n_e)
    err = np.abs(bf16_to_np(out) - o).max()
    assert err <= TOL_QUANT, err
    return err


@pytest.mark.parametrize("S,T,delays,checks", [
    (CSA, 900, (0, 37, 170), (130, 501, 899)),
    (HCA, 1300, (0, 300), (200, 1299)),
], ids=["csa", "hca"])
def test_paged_incremental_decode(S, T, delays, checks):
    K = _K()
    from long_context_attention_09_amd import paged
    _say(f"paged decode {S.name} B={S.B} steps={T} delays={delays}")
    inp = _inputs(S, T)
    d = _dev(inp)
    rng = np.random.default_rng(S.seed)
    blocks_per_req = -(-T // paged.TOKENS_PER_BLOCK)
    n_blocks = S.B * blocks_per_req + 5
    alloc = paged.BlockAllocator(n_blocks, order=rng.permutation(n_blocks))
    cache = paged.PagedCache(S.B, T, alloc, "cuda")
    bias = {"main": (d["main"]["ba"], d["main"].get("bb"))}
    if S.csa:
        bias["idx"] = (d["idx"]["ba"], d["idx"]["bb"])
    layer = paged.PagedLayer(cache, S, bias, "cuda")
    seq_pos = torch.zeros(S.B, dtype=torch.int64, device="cuda")
    flags_a = K.ATTEND_NORM_Q | K.ATTEND_BATCH_INVARIANT
    flags_i = K.INDEX_BATCH_INVARIANT
    step = paged.PagedDecodeStep(layer, seq_pos, d["q"], d["sink"], d.get("q_idx_codes"), d.get("q_idx_scales"),
                                 d.get("w"), attend_flags=flags_a, index_flags=flags_i)
    ar = torch.arange(S.B, device="cuda")
    for k in range(T):
        pos = [max(0, k - dl) for dl in delays]
        for b in range(S.B):
            cache.reserve(b, pos[b] + 1)
        seq_pos.copy_(torch.tensor(pos, dtype=torch.int64))
        layer.write_token(seq_pos, {n: d["main"][n][ar, seq_pos] for n in layer.main_ring},
                          {n: d["idx"][n][ar, seq_pos] for n in layer.idx_ring} if S.csa else None,
                          d["win_raw"][ar, seq_pos])
        if k not in checks:
            step.compress()
            continue
        # the whole step at these positions: the completed entries compressed on
        # a second stream while the window row, index and attention run
        step.run()
        sc = None
        if S.csa:
            n_cap = cache.max_blocks * layer.per_block
            sc = torch.empty(S.B, 1, n_cap, device="cuda")
            idx2 = torch.empty_like(step.idx)
            K.index_topk(d["q_idx_codes"], d["w"], layer.key_codes, step.q_pos, m=S.m, top_k=S.top_k,
                         out_idx=idx2, q1=d["q_idx_scales"], k1=layer.key_scales, fmt=K.FMT_MXFP4,
                         flags=flags_i, block_table=cache.block_table, out_score=sc)
            torch.cuda.synchronize()
            assert torch.equal(idx2, step.idx)
        torch.cuda.synchronize()
        for b in range(S.B):
            t = pos[b]
            ref = _contiguous(K, S, d, b, t, flags_a, flags_i)
            n_e = (t + 1) // S.m
            rows = cache.entry_rows(b, n_e, layer.per_block)
            pool = layer.pool.view(-1, 576)[torch.as_tensor(rows, device="cuda")] if n_e else None
            if n_e:
                assert torch.equal(pool, ref["cache"][0, :n_e]), f"entries of request {b} at t={t}"
            lo = max(0, t - S.n_win + 1)
            ring_rows = torch.as_tensor([p % S.n_win for p in range(lo, t + 1)], device="cuda")
            win_rows = layer.win_ring[b][ring_rows]
            assert torch.equal(win_rows, ref["win"][0, :t + 1 - lo]), f"window of request {b} at t={t}"
            keys = None
            if S.csa:
                rr = torch.as_tensor(rows, device="cuda")
                kc = layer.key_codes.view(-1, 64)[rr] if n_e else None
                ks = layer.key_scales.view(-1, 4)[rr] if n_e else None
                if n_e:
                    assert torch.equal(kc, ref["kc"][0, :n_e]) and torch.equal(ks, ref["ks"][0, :n_e])
                n_vis = t // S.m
                assert torch.equal(sc[b, 0, :n_vis].view(torch.int32), ref["score"][0, 0, :n_vis].view(torch.int32))
                assert torch.equal(step.idx[b], ref["idx"][0]), f"selection of request {b} at t={t}"
                keys = (kc.cpu().numpy() if n_e else np.zeros((0, 64), np.uint8),
                        ks.cpu().numpy() if n_e else np.zeros((0, 4), np.uint8))
            assert torch.equal(step.out[b].view(torch.int16), ref["out"][0].view(torch.int16)), \
                f"attention of request {b} at t={t}"
            assert torch.equal(step.lse[b].view(torch.int32), ref["lse"][0].view(torch.int32))
            if b == 0 and k == checks[-1]:
                err = _oracle_check(S, inp, b, t, pool.cpu().numpy() if n_e else np.zeros((0, 576), np.uint8),
                                    win_rows.cpu().numpy(), keys,
                                    step.idx[b, 0].cpu().numpy() if S.csa else None, step.out[b, 0])
                _say(f"  oracle t={t}: max |out error| {err:.2e}")
        _say(f"  step {k}: positions {pos} bitwise equal to the contiguous recomputation")
    # a finished request returns its blocks
    free0 = alloc.n_free
    cache.release(0)
    assert alloc.n_free == free0 + blocks_per_req
    assert (cache.block_table[0] == -1).all()


@pytest.mark.parametrize("name", ["pro-csa-decode-1m", "flash-hca-decode-1m"])
def test_paged_full_size_matches_contiguous(name):
    """At the benchmark shapes (8 x 2^20 tokens CSA, 32 x 2^20 HCA) the paged
    decode step over shuffled blocks gives the contiguous step's selection,
    scores, output and LSE bitwise (the step at t = L stores the window row
    only: token L completes no block)."""
    K = _K()
    from long_context_attention_09_amd import paged
    from long_context_attention_09_amd.layer import LayerStep
    S = {s.name: s for s in (synth.PRO_CSA_DECODE, synth.FLASH_HCA_DECODE)}[name]
    _say(f"paged full size {S.name} B={S.B} L={S.L}")
    inp = synth.quant_decode_inputs(S, device="cuda")
    ref = LayerStep(S, inp)
    n_cap = S.L // S.m
    sc_ref = None
    if S.csa:
        sc_ref = torch.empty(S.B, 1, n_cap, device="cuda")
        K.index_topk(inp["q_idx_codes"], inp["w"], inp["keys_codes"], inp["q_pos"], m=S.m, top_k=S.top_k,
                     out_idx=torch.empty_like(ref.idx), q1=inp["q_idx_scales"], k1=inp["keys_scales"],
                     fmt=K.FMT_MXFP4, out_score=sc_ref)
    ref.run(entries=False)
    torch.cuda.synchronize()
    per_req = -(-S.L // paged.TOKENS_PER_BLOCK) + 1
    n_blocks = S.B * per_req
    alloc = paged.BlockAllocator(n_blocks, order=np.random.default_rng(S.seed).permutation(n_blocks))
    cache = paged.PagedCache(S.B, S.L + paged.TOKENS_PER_BLOCK, alloc, "cuda")
    for b in range(S.B):
        cache.reserve(b, S.L + 1)
    mn = inp["main"]
    bias = {"main": (mn["ba"], mn.get("bb"))}
    if S.csa:
        bias["idx"] = (inp["idx"]["ba"], inp["idx"]["bb"])
    layer = paged.PagedLayer(cache, S, bias, "cuda")
    layer.import_contiguous(inp["cache"], inp.get("keys_codes"), inp.get("keys_scales"), inp["win"],
                            inp["win_pos0"].tolist())
    layer.win_raw.copy_(inp["win_raw"])
    seq_pos = inp["q_pos"].view(-1).clone()
    step = paged.PagedDecodeStep(layer, seq_pos, inp["q"], inp["sink"], inp.get("q_idx_codes"),
                                 inp.get("q_idx_scales"), inp.get("w"))
    step.run()
    torch.cuda.synchronize()
    if S.csa:
        sc = torch.empty(S.B, 1, cache.max_blocks * layer.per_block, device="cuda")
        K.index_topk(inp["q_idx_codes"], inp["w"], layer.key_codes, step.q_pos, m=S.m, top_k=S.top_k,
                     out_idx=torch.empty_like(step.idx), q1=inp["q_idx_scales"], k1=layer.key_scales,
                     fmt=K.FMT_MXFP4, block_table=cache.block_table, out_score=sc)
        torch.cuda.synchronize()
        assert torch.equal(sc[:, :, :n_cap].view(torch.int32), sc_ref.view(torch.int32))
        assert torch.equal(step.idx, ref.idx)
    assert torch.equal(step.out.view(torch.int16), ref.out.view(torch.int16))
    assert torch.equal(step.lse.view(torch.int32), ref.lse.view(torch.int32))


@pytest.mark.parametrize("name", ["pro-csa-prefill-8k-after-1m", "pro-hca-prefill-8k-after-1m"])
def test_paged_prefill_matches_contiguous(name):
    """A prefill chunk (300 queries after 4096 cached tokens) through the paged
    layout: the chunk's entries and keys compressed into shuffled blocks, the
    query-block indexer and the attention reading through the block table (the
    chunk's window in a linear buffer), bitwise equal to the contiguous chunk.
    Both sides run in the batch-invariant mode, whose splits depend on each
    query's list alone (the paged capacity is a whole number of blocks)."""
    K = _K()
    from long_context_attention_09_amd import paged
    from long_context_attention_09_amd.layer import LayerStep
    S = {s.name: s for s in (synth.PRO_CSA_PREFILL, synth.PRO_HCA_PREFILL)}[name].replace(L=4096, n_q=300)
    _say(f"paged prefill {S.name} L={S.L} n_q={S.n_q}")
    d = _dev(synth.quant_prefill_inputs(S))
    ref = LayerStep(S, d, prefill=True, batch_invariant=True)
    ref.run()
    torch.cuda.synchronize()
    T = S.L + S.n_q
    per_req = -(-T // paged.TOKENS_PER_BLOCK) + 1
    n_blocks = S.B * per_req + 3
    alloc = paged.BlockAllocator(n_blocks, order=np.random.default_rng(S.seed).permutation(n_blocks))
    cache = paged.PagedCache(S.B, T + paged.TOKENS_PER_BLOCK, alloc, "cuda")
    for b in range(S.B):
        cache.reserve(b, T)
    bias = {"main": (d["main"]["ba"], d["main"].get("bb"))}
    if S.csa:
        bias["idx"] = (d["idx"]["ba"], d["idx"]["bb"])
    layer = paged.PagedLayer(cache, S, bias, "cuda")
    layer.import_contiguous(d["cache_old"], d.get("keys_codes_old"), d.get("keys_scales_old"))
    tail = S.m if S.overlap else 0
    jobs = layer.chunk_jobs(d["main"], d.get("idx"), S.L - tail)
    win = torch.zeros(S.B, S.n_win - 1 + S.n_q, 576, dtype=torch.uint8, device="cuda")
    win[:, :S.n_win - 1] = d["win_old"]
    wn, wr = K.split_main(win)
    jobs.append(K.compress_args(d["win_raw"], m=1, pos0=S.L, out0=wn, out1=wr, d_rope=S.d_r, rope_theta=S.theta,
                                do_norm=True, out_fmt=K.FMT_FP8_BF16, out_row0=S.L - S.n_win + 1))
    K.compress_batch(jobs)
    idx = None
    if S.csa:
        idx = torch.empty(S.B, S.n_q, S.top_k, dtype=torch.int32, device="cuda")
        K.index_topk(d["q_idx_codes"], d["w"], layer.key_codes, d["q_pos"], m=S.m, top_k=S.top_k, out_idx=idx,
                     q1=d["q_idx_scales"], k1=layer.key_scales, fmt=K.FMT_MXFP4, flags=K.INDEX_BATCH_INVARIANT,
                     block_table=cache.block_table)
    out = torch.empty_like(ref.out)
    a = layer.attend_args(d["q"], d["q_pos"], d["sink"], out, idx=idx,
                          flags=K.ATTEND_NORM_Q | K.ATTEND_BATCH_INVARIANT, window=win, win_pos0=d["win_pos0"])
    ws, n = K._workspace(K.OP_ATTEND if S.csa else K.OP_HCA_ATTEND, a, None)
    fn = K.load().csa_attend if S.csa else K.load().hca_attend
    K._check(fn(C.byref(a), K._ptr(ws), n, K._stream()), "attend")
    torch.cuda.synchronize()
    n_e = T // S.m
    rows = torch.as_tensor(cache.entry_rows(0, n_e, layer.per_block), device="cuda")
    assert torch.equal(layer.pool.view(-1, 576)[rows], ref.caches[0][0, :n_e]), "chunk entries"
    if S.csa:
        assert torch.equal(idx, ref.idx), "selection"
    assert torch.equal(out.view(torch.int16), ref.out.view(torch.int16)), "attention"


def _attend_oracle(S, q, t, entries_u8, sel, win_u8, win_pos0, sink, dense):
    entries = P.decode_entry_bytes(entries_u8, S.d_nope)
    window = P.decode_entry_bytes(win_u8, S.d_nope)
    args = (q, t, entries) + (() if dense else (sel,)) + (window, win_pos0, S.n_win, sink, S.theta, S.d_r, S.m)
    return (OC.hca_attend if dense else OC.csa_attend)(*args)[0]


@pytest.mark.parametrize("H_I", [32, 64])
def test_paged_query_blocks_match_contiguous(H_I):
    """The query-block indexer (several queries per call) reading its keys
    through shuffled 32-key blocks gives, bitwise, the scores and selection of
    the contiguous layout, with fp32 scores and with BF16 scores, for 32 and 64
    indexer heads; the BF16 scores are the fp32 ones rounded, and every
    selection is the exact top-k of the scores it was made from (ties to the
    lower index)."""
    K = _K()
    B, n_q, max_blocks, top_k = 2, 9, 96, 256
    n_cap = max_blocks * 32
    S = CSA.replace(name=f"paged-qblocks-{H_I}", H_I=H_I)
    _say(f"paged query blocks H_I={H_I} B={B} n_q={n_q} n_cap={n_cap}")
    kc, ks = synth.mxfp4_codes(S, "k", B * n_cap, 128)
    kc, ks = kc.view(B, n_cap, 64), ks.view(B, n_cap, 4)
    qc, qs = synth.mxfp4_codes(S, "q", B * n_q * H_I, 128)
    qc, qs = qc.view(B, n_q, H_I, 64), qs.view(B, n_q, H_I, 4)
    w = synth.head_weights(S, (B, n_q, H_I))
    # block j of sequence b sits at a shuffled pool slot; some slots stay unused
    n_pool = B * max_blocks + 7
    slots = np.random.default_rng(5).permutation(n_pool)[:B * max_blocks].astype(np.int32)
    bt = torch.from_numpy(slots).view(B, max_blocks)
    pool_c = torch.zeros(n_pool, 32, 64, dtype=torch.uint8)
    pool_s = torch.full((n_pool, 32, 4), 127, dtype=torch.uint8)
    pool_c[bt.reshape(-1).long()] = kc.reshape(B * max_blocks, 32, 64)
    pool_s[bt.reshape(-1).long()] = ks.reshape(B * max_blocks, 32, 4)
    # visible entries from n_cap - 1 down to about 2,700, different per sequence
    q_pos = torch.stack([4 * n_cap - 1 - 5 * b - 41 * torch.arange(n_q) for b in range(B)]).contiguous()

    def run(paged, flags):
        g = _dev
        k0, k1 = (g(pool_c), g(pool_s)) if paged else (g(kc), g(ks))
        extra = {"block_table": g(bt)} if paged else {}
        idx = torch.empty(B, n_q, top_k, dtype=torch.int32, device="cuda")
        dt = torch.bfloat16 if flags else torch.float32
        sc = torch.empty(B, n_q, n_cap, dtype=dt, device="cuda")
        K.index_topk(g(qc), g(w), k0, g(q_pos), m=4, top_k=top_k, out_idx=idx, q1=g(qs), k1=k1, out_score=sc,
                     fmt=K.FMT_MXFP4, flags=flags, **extra)
        idx2 = torch.empty_like(idx)                 # the same call without caller-kept scores
        K.index_topk(g(qc), g(w), k0, g(q_pos), m=4, top_k=top_k, out_idx=idx2, q1=g(qs), k1=k1,
                     fmt=K.FMT_MXFP4, flags=flags, **extra)
        torch.cuda.synchronize()
        assert torch.equal(idx, idx2)
        return idx.cpu().numpy(), sc.float().cpu().numpy().astype(np.float64)

    got = {(paged, bf): run(paged, K.INDEX_BF16_SCORES if bf else 0) for paged in (False, True) for bf in (False, True)}
    for bf in (False, True):
        assert np.array_equal(got[(True, bf)][0], got[(False, bf)][0]), f"selection, bf16={bf}"
        assert np.array_equal(got[(True, bf)][1], got[(False, bf)][1]), f"scores, bf16={bf}"
    sc32, sc16 = got[(False, False)][1], got[(False, True)][1]
    for b in range(B):
        for r in range(n_q):
            n_vis = OC.visible_entries(int(q_pos[b, r]), 4, n_cap)
            r32 = torch.from_numpy(sc32[b, r, :n_vis].astype(np.float32)).to(torch.bfloat16).double().numpy()
            assert np.array_equal(sc16[b, r, :n_vis], r32), (b, r)
            for bf, sc in ((False, sc32), (True, sc16)):
                want = OC.topk(sc[b, r, :n_vis], top_k)
                assert np.array_equal(got[(False, bf)][0][b, r], want), (b, r, bf)


def test_attend_long_lists_split_by_the_stage():
    """Lists longer than the 2048 rows a split stages: a CSA selection of 6000
    indices (with -1 and out-of-range ones mixed in) and paged HCA lists at
    B = 256 (one split per query would hold 68 tiles, over the 64-tile stage,
    so the paged plan splits them): both against the oracle."""
    K = _K()
    from long_context_attention_09_amd import paged
    # CSA, top-k 6000 over 16384 entries
    S = synth.PRO_CSA_DECODE.replace(name="long-csa", B=2, L=1 << 16, top_k=6000, H=64)
    _say(f"long CSA selection top_k={S.top_k}")
    d = synth.quant_decode_inputs(S, device="cuda")
    n_e = S.L // S.m
    g = torch.Generator(device="cuda").manual_seed(11)
    idx = torch.stack([torch.randperm(n_e, generator=g, device="cuda")[:S.top_k].sort().values
                       for _ in range(S.B)]).to(torch.int32).view(S.B, 1, S.top_k)
    idx[0, 0, 5:40] = -1
    idx[1, 0, -30:] = n_e + 7                     # outside the visible range: skipped
    out = torch.empty_like(d["q"])
    nope, rope = K.split_main(d["cache"])
    wn, wr = K.split_main(d["win"])
    K.attend(d["q"], d["q_pos"], nope, wn, d["win_pos0"], d["sink"], out, m=S.m, n_win=S.n_win, kv1=rope,
             win1=wr, idx=idx)
    torch.cuda.synchronize()
    for b in range(S.B):
        o = _attend_oracle(S, bf16_to_np(d["q"][b, 0]), S.L, d["cache"][b].cpu().numpy(),
                           idx[b, 0].cpu().numpy(), d["win"][b].cpu().numpy(), S.L - S.n_win + 1,
                           d["sink"].double().cpu().numpy(), dense=False)
        err = np.abs(bf16_to_np(out[b, 0]) - o).max()
        assert err <= TOL_QUANT, (b, err)
    # paged HCA at B = 256
    S = synth.FLASH_HCA_DECODE.replace(name="long-hca", B=256, L=1 << 18)
    _say(f"paged HCA B={S.B} L={S.L}")
    d = synth.quant_decode_inputs(S, device="cuda")
    per_req = -(-S.L // paged.TOKENS_PER_BLOCK) + 1
    n_blocks = S.B * per_req
    alloc = paged.BlockAllocator(n_blocks, order=np.random.default_rng(5).permutation(n_blocks))
    cache = paged.PagedCache(S.B, S.L + paged.TOKENS_PER_BLOCK, alloc, "cuda")
    for b in range(S.B):
        cache.reserve(b, S.L + 1)
    layer = paged.PagedLayer(cache, S, {"main": (d["main"]["ba"], None)}, "cuda")
    layer.import_contiguous(d["cache"])
    out = torch.empty_like(d["q"])
    a = layer.attend_args(d["q"], d["q_pos"], d["sink"], out, window=d["win"], win_pos0=d["win_pos0"])
    ws, n = K._workspace(K.OP_HCA_ATTEND, a, None)
    assert n >= S.B * 2 * 64 * 512 * 2           # more than one split per query
    K._check(K.load().hca_attend(C.byref(a), K._ptr(ws), n, K._stream()), "hca_attend")
    torch.cuda.synchronize()
    for b in (0, 131, 255):
        o = _attend_oracle(S, bf16_to_np(d["q"][b, 0]), S.L, d["cache"][b].cpu().numpy(), None,
                           d["win"][b].cpu().numpy(), S.L - S.n_win + 1, d["sink"].double().cpu().numpy(),
                           dense=True)
        err = np.abs(bf16_to_np(out[b, 0]) - o).max()
        assert err <= TOL_QUANT, (b, err)
