"""Heterogeneous paged KV cache of one layer and its decode step.

The layers of a hybrid model keep caches that grow at different rates: one
CSA main entry and one indexer key per 4 tokens, one HCA entry per 128 tokens,
and raw window rows per token ("DeepSeek-V4: Towards Highly Efficient
Million-Token Context Intelligence", observation 3 and the inference
infrastructure list; "DeepSeek-V4 深读", section on the heterogeneous KV cache
and Fig. 5).  One block size in tokens cannot serve them all, so:

  * block cache: physical blocks that each cover lcm(4, 128) = 128 raw tokens
    of a request, handed out by one BlockAllocator and named in one block
    table per request row, shared by every layer.  A CSA layer's pools hold
    32 main entries ([P, 32, 576] bytes) and 32 indexer keys ([P, 32, 64]
    E2M1 codes + [P, 32, 4] E8M0 scales) per block; an HCA layer's pool holds
    one entry per block ([P, 1, 576]);
  * state cache: fixed-size rings per request row, the newest n_win window
    rows in storage form ([B, n_win, 576]) and the raw compressor inputs of
    the newest 2m (CSA, overlapped pooling) or m' (HCA) tokens.

A decode step at per-request positions seq_pos [B] (each request's newest
token, whose raw rows the model has written into the rings) is three library
calls: one batched csa_compress in the per-sequence decode mode (the entry
that token completes, if any, into the pools through the block table, and the
token's window row into the window ring), csa_index_topk over the paged keys
(CSA), and csa_attend / hca_attend over the paged entries and the window ring.
The block tables and allocator are host bookkeeping; every step of the layer
runs in the library's kernels.
"""
from __future__ import annotations

import ctypes as C
import math

import numpy as np
import torch

from . import _lib as K

TOKENS_PER_BLOCK = 128          # lcm(4, 128): one block of every layer's cache
ENTRY_BYTES = 576               # 448 E4M3FN + 64 BF16


class BlockAllocator:
    """Free list of physical block ids [0, n_blocks); `order` (a permutation)
    sets the order in which ids are handed out (tests scatter them)."""

    def __init__(self, n_blocks: int, order=None):
        ids = list(range(n_blocks)) if order is None else [int(i) for i in order]
        if sorted(ids) != list(range(n_blocks)):
            raise ValueError("order must be a permutation of the block ids")
        self.n_blocks = n_blocks
        self._free = ids[::-1]          # pop() hands out ids in `order`

    @property
    def n_free(self) -> int:
        return len(self._free)

    def alloc(self) -> int:
        if not self._free:
            raise MemoryError("block cache exhausted")
        return self._free.pop()

    def free(self, ids):
        for i in ids:
            if not 0 <= i < self.n_blocks:
                raise ValueError(f"block id {i} out of range")
        self._free.extend(int(i) for i in ids)


class PagedCache:
    """Block tables of B request rows over one allocator (shared by the layers).

    Block j of row b covers tokens [128 j, 128 j + 128); block_table[b, j] is
    its physical id, -1 while unallocated."""

    def __init__(self, B: int, max_tokens: int, allocator: BlockAllocator, device):
        self.B = B
        self.max_blocks = math.ceil(max_tokens / TOKENS_PER_BLOCK)
        self.alloc = allocator
        self.n_blocks = allocator.n_blocks
        self.table = np.full((B, self.max_blocks), -1, dtype=np.int32)
        self.block_table = torch.full((B, self.max_blocks), -1, dtype=torch.int32, device=device)
        self.device = device

    def reserve(self, b: int, n_tokens: int):
        """Allocate the blocks that tokens [0, n_tokens) of row b need and
        publish the new table entries (a small host-to-device copy)."""
        need = math.ceil(n_tokens / TOKENS_PER_BLOCK)
        if need > self.max_blocks:
            raise ValueError(f"row {b}: {n_tokens} tokens exceed the table")
        row = self.table[b]
        first = int(np.argmax(row < 0)) if (row < 0).any() else self.max_blocks
        if need <= first:
            return
        for j in range(first, need):
            row[j] = self.alloc.alloc()
        self.block_table[b, first:need] = torch.from_numpy(row[first:need].copy()).to(self.device)

    def release(self, b: int):
        """Return row b's blocks to the allocator (the request ended)."""
        row = self.table[b]
        self.alloc.free(row[row >= 0].tolist())
        row[:] = -1
        self.block_table[b].fill_(-1)

    def entry_rows(self, b: int, n_entries: int, per_block: int) -> np.ndarray:
        """Pool rows (block id * per_block + offset) of entries [0, n_entries) of row b."""
        e = np.arange(n_entries)
        blk = self.table[b, e // per_block]
        if (blk < 0).any():
            raise ValueError("entry in an unallocated block")
        return blk.astype(np.int64) * per_block + e % per_block


class PagedLayer:
    """Pools (block cache) and rings (state cache) of one CSA or HCA layer.

    shape: a synth.Shape-like object (B, H, d, d_r, m, overlap, top_k, H_I,
    d_I, n_win, theta).  bias: the compressor biases {'main': (ba, bb),
    'idx': (ba, bb)} (bb None without overlap)."""

    def __init__(self, cache: PagedCache, shape, bias, device):
        s = shape
        if TOKENS_PER_BLOCK % s.m:
            raise ValueError("m must divide the block's 128 tokens")
        self.cache, self.s, self.bias = cache, s, bias
        P, B = cache.n_blocks, cache.B
        self.per_block = TOKENS_PER_BLOCK // s.m
        bf = torch.bfloat16
        self.pool = torch.zeros(P, self.per_block, ENTRY_BYTES, dtype=torch.uint8, device=device)
        self.ring_rows = s.m * (2 if s.overlap else 1)
        names = ["ca", "za"] + (["cb", "zb"] if s.overlap else [])
        self.main_ring = {n: torch.zeros(B, self.ring_rows, s.d, dtype=bf, device=device) for n in names}
        if s.csa:
            self.key_codes = torch.zeros(P, self.per_block, s.d_I // 2, dtype=torch.uint8, device=device)
            self.key_scales = torch.zeros(P, self.per_block, s.d_I // 32, dtype=torch.uint8, device=device)
            self.idx_ring = {n: torch.zeros(B, self.ring_rows, s.d_I, dtype=bf, device=device)
                             for n in ["ca", "za", "cb", "zb"]}
        self.win_raw = torch.zeros(B, 1, s.d, dtype=bf, device=device)      # the newest token's raw row
        self.win_ring = torch.zeros(B, s.n_win, ENTRY_BYTES, dtype=torch.uint8, device=device)

    # ------------------------------------------------------------ raw token input

    def write_token(self, seq_pos: torch.Tensor, main_rows: dict, idx_rows: dict | None, win_row: torch.Tensor):
        """Put the newest token's raw rows ([B, D] each) into ring slot
        seq_pos[b] % ring: what the model's projections write before the step."""
        B = self.cache.B
        ar = torch.arange(B, device=seq_pos.device)
        slot = seq_pos % self.ring_rows
        for n, t in self.main_ring.items():
            t[ar, slot] = main_rows[n]
        if self.s.csa:
            for n, t in self.idx_ring.items():
                t[ar, slot] = idx_rows[n]
        self.win_raw[:, 0] = win_row

    def import_contiguous(self, entries, key_codes=None, key_scales=None, window=None, win_pos0=None):
        """Copy caches in the contiguous layout into this layer: entries
        [B, n, 576] (and indexer keys [B, n, 64] / [B, n, 4]) into the pools
        through the block table (blocks must be reserved), window rows
        [B, W, 576] holding positions win_pos0[b] .. + W - 1 into the ring."""
        B, n = entries.shape[:2]
        for b in range(B):
            rows = torch.as_tensor(self.cache.entry_rows(b, n, self.per_block), device=entries.device)
            self.pool.view(-1, ENTRY_BYTES)[rows] = entries[b]
            if key_codes is not None:
                self.key_codes.view(-1, key_codes.shape[-1])[rows] = key_codes[b]
                self.key_scales.view(-1, key_scales.shape[-1])[rows] = key_scales[b]
        if window is not None:
            W = window.shape[1]
            for b in range(B):
                pos = int(win_pos0[b]) + torch.arange(W, device=window.device)
                self.win_ring[b, pos % self.s.n_win] = window[b]

    # ------------------------------------------------------------ the step's calls

    def compress_jobs(self, seq_pos: torch.Tensor):
        """csa_compress jobs of a decode step: the entry (and indexer key) the
        newest token completes, into the pools; its window row, into the ring."""
        s = self.s
        bt = self.cache.block_table
        nope, rope = K.split_main(self.pool)
        mr = self.main_ring
        ba, bb = self.bias["main"]
        jobs = [K.compress_args(mr["ca"], gate_a=mr["za"], bias_a=ba, kv_b=mr.get("cb"), gate_b=mr.get("zb"),
                                bias_b=bb, m=s.m, pos0=0, out0=nope, out1=rope, d_rope=s.d_r,
                                rope_theta=s.theta, do_norm=True, out_fmt=K.FMT_FP8_BF16,
                                in_ring=self.ring_rows, block_table=bt, seq_pos=seq_pos)]
        if s.csa:
            ir = self.idx_ring
            ia, ib = self.bias["idx"]
            jobs.append(K.compress_args(ir["ca"], gate_a=ir["za"], bias_a=ia, kv_b=ir["cb"], gate_b=ir["zb"],
                                        bias_b=ib, m=s.m, pos0=0, out0=self.key_codes, out1=self.key_scales,
                                        d_rope=0, do_norm=False, out_fmt=K.FMT_MXFP4, in_ring=self.ring_rows,
                                        block_table=bt, seq_pos=seq_pos))
        wn, wr = K.split_main(self.win_ring)
        jobs.append(K.compress_args(self.win_raw, m=1, pos0=0, out0=wn, out1=wr, d_rope=s.d_r,
                                    rope_theta=s.theta, do_norm=True, out_fmt=K.FMT_FP8_BF16, in_ring=1,
                                    out_ring=s.n_win, seq_pos=seq_pos))
        return jobs

    def chunk_jobs(self, main_streams, idx_streams, pos0):
        """csa_compress jobs of a prefill chunk: every entry (and indexer key)
        that rows pos0 .. of the given linear streams ([B, rows, D]; with
        overlap the first m rows are the previous block's tail) complete, into
        the pools through the block table (the blocks must be reserved)."""
        s = self.s
        bt = self.cache.block_table
        nope, rope = K.split_main(self.pool)
        mn = main_streams
        ba, bb = self.bias["main"]
        jobs = [K.compress_args(mn["ca"], gate_a=mn["za"], bias_a=ba, kv_b=mn.get("cb"), gate_b=mn.get("zb"),
                                bias_b=bb, m=s.m, pos0=pos0, out0=nope, out1=rope, d_rope=s.d_r,
                                rope_theta=s.theta, do_norm=True, out_fmt=K.FMT_FP8_BF16, block_table=bt)]
        if s.csa:
            ix = idx_streams
            ia, ib = self.bias["idx"]
            jobs.append(K.compress_args(ix["ca"], gate_a=ix["za"], bias_a=ia, kv_b=ix["cb"], gate_b=ix["zb"],
                                        bias_b=ib, m=s.m, pos0=pos0, out0=self.key_codes, out1=self.key_scales,
                                        d_rope=0, do_norm=False, out_fmt=K.FMT_MXFP4, block_table=bt))
        return jobs

    def index_args(self, q_pos, q_codes, q_scales, w, out_idx, out_score=None, flags=0):
        s = self.s
        return K.index_args(q_codes, w, self.key_codes, q_pos, m=s.m, top_k=s.top_k, out_idx=out_idx,
                            q1=q_scales, k1=self.key_scales, fmt=K.FMT_MXFP4, flags=flags,
                            block_table=self.cache.block_table, out_score=out_score)

    def attend_args(self, q, q_pos, sink, out, idx=None, out_lse=None, flags=K.ATTEND_NORM_Q, window=None,
                    win_pos0=None):
        """Attention over the paged entries and the window ring, or (prefill:
        the chunk's queries see more window rows than the ring holds) over a
        linear window buffer [B, W, 576] whose row 0 holds position win_pos0[b]."""
        s = self.s
        nope, rope = K.split_main(self.pool)
        if window is None:
            wn, wr = K.split_main(self.win_ring)
            flags |= K.ATTEND_WIN_RING
        else:
            wn, wr = K.split_main(window)
        return K.attend_args(q, q_pos, nope, wn, win_pos0, sink, out, m=s.m, n_win=s.n_win, kv1=rope, win1=wr,
                             idx=idx, out_lse=out_lse, d_rope=s.d_r, rope_theta=s.theta,
                             fmt=K.FMT_FP8_BF16, flags=flags, block_table=self.cache.block_table)


class PagedDecodeStep:
    """One decode step of a paged layer with prepared argument structs (the
    pointers they hold stay valid while this object holds the tensors).

    q [B, 1, H, d] bf16, sink [H] fp32, seq_pos [B] int64 (each row's newest
    token = its query position); CSA also q_codes [B, 1, H_I, d_I/2],
    q_scales [B, 1, H_I, d_I/32] and w [B, 1, H_I]."""

    def __init__(self, layer: PagedLayer, seq_pos, q, sink, q_codes=None, q_scales=None, w=None,
                 attend_flags=K.ATTEND_NORM_Q, index_flags=0):
        s = layer.s
        self.layer, self.seq_pos = layer, seq_pos
        B = layer.cache.B
        dev = q.device
        self.q_pos = seq_pos.view(B, 1)
        self.out = torch.empty(B, 1, s.H, s.d, dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty(B, 1, s.H, dtype=torch.float32, device=dev)
        self.idx = torch.empty(B, 1, max(s.top_k, 1), dtype=torch.int32, device=dev)
        self._keep = (q, sink, q_codes, q_scales, w)
        jobs = layer.compress_jobs(seq_pos)
        self.jobs = (K.CompressArgs * len(jobs))(*jobs)
        n = K.compress_workspace_bytes(jobs)
        self.ws_c = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
        self.index_a = None
        if s.csa:
            self.index_a = layer.index_args(self.q_pos, q_codes, q_scales, w, self.idx, flags=index_flags)
            n = K.workspace_bytes(K.OP_INDEX_TOPK, self.index_a)
            self.ws_i = torch.zeros(max(n, 256), dtype=torch.uint8, device=dev)   # zero once: ops keep it so
        self.attend_a = layer.attend_args(q, self.q_pos, sink, self.out, idx=self.idx if s.csa else None,
                                          out_lse=self.lse, flags=attend_flags)
        n = K.workspace_bytes(K.OP_HCA_ATTEND if not s.csa else K.OP_ATTEND, self.attend_a)
        self.ws_a = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
        lib = K.load()
        self._lib = lib

    def compress(self, stream=None):
        st = K._stream() if stream is None else stream
        K._check(self._lib.csa_compress_batch_ws(self.jobs, len(self.jobs), K._ptr(self.ws_c), self.ws_c.numel(),
                                                 st), "csa_compress_batch_ws")

    def index(self, events=(None, None), stream=None):
        a = self.index_a
        a.ev_start, a.ev_stop = events
        st = K._stream() if stream is None else stream
        K._check(self._lib.csa_index_topk(C.byref(a), K._ptr(self.ws_i), self.ws_i.numel(), st), "csa_index_topk")

    def attend(self, events=(None, None), stream=None):
        a = self.attend_a
        a.ev_start, a.ev_stop = events
        st = K._stream() if stream is None else stream
        fn = self._lib.csa_attend if self.layer.s.csa else self._lib.hca_attend
        K._check(fn(C.byref(a), K._ptr(self.ws_a), self.ws_a.numel(), st), "attend")

    def run(self, stream=None):
        self.compress(stream)
        if self.layer.s.csa:
            self.index(stream=stream)
        self.attend(stream=stream)
