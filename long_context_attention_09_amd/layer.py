"""One CSA or HCA layer step driven through the C ABI (decode and prefill).

Sequencing only: every step is one library call; this module owns the output
and workspace buffers so repeated steps allocate nothing.

Decode step of a layer at query position t = L (all L tokens before t are in
the caches):
  CSA: compress the newest main-KV entry (m = 4, overlapped pooling of rows
       [L-8, L)), the newest indexer key (same rows, MXFP4) and the new
       token's raw window row (m = 1), then index + top-k, then attend.
  HCA: compress the newest entry (m' = 128, rows [L-128, L)), store the new
       window row, then dense attend.
The newest entry of a real decode completes once every m steps; compressing
it on every step is the pessimistic bound.

Prefill chunk of n_q tokens at positions L .. L+n_q-1: compress every entry
the chunk completes (with the m-token context tail feeding the b-branch), store
the chunk's raw window rows, then index + top-k and attend per query.
"""
from __future__ import annotations

import ctypes as C

import torch

from . import _lib as K


class LayerStep:
    """Buffers and calls of one layer step over device-resident inputs.

    shape: a synth.Shape-like object (B, L, n_q, H, d, d_r, m, overlap, top_k,
    H_I, d_I, n_win, theta); inp: dict of device tensors laid out as the
    seeded generator lays them out (decode: quant_decode_inputs, prefill:
    quant_prefill_inputs)."""

    def __init__(self, shape, inp, prefill: bool = False, copies: int = 1, batch_invariant: bool = False,
                 bf16_scores: bool = False):
        self.s = shape
        # batch-invariant mode: fixed attention splits and the exact indexer form;
        # bf16_scores: index scores rounded to BF16 before they are stored and selected on
        self.attend_flags = K.ATTEND_NORM_Q | (K.ATTEND_BATCH_INVARIANT if batch_invariant else 0)
        self.index_flags = ((K.INDEX_BATCH_INVARIANT if batch_invariant else 0) |
                            (K.INDEX_BF16_SCORES if bf16_scores else 0))
        self.inp = inp
        self.prefill = prefill
        s = shape
        dev = inp["q"].device
        B = s.B
        self.caches = []
        self.keys = []
        if prefill:
            n_old = s.L // s.m
            n_cap = (s.L + s.n_q) // s.m
            cache = torch.zeros(B, n_cap, 576, dtype=torch.uint8, device=dev)
            cache[:, :n_old] = inp["cache_old"]
            self.caches.append(cache)
            win = torch.zeros(B, s.n_win - 1 + s.n_q, 576, dtype=torch.uint8, device=dev)
            win[:, :s.n_win - 1] = inp["win_old"]
            self.win = win
            self.win_pos0 = inp["win_pos0"]
            if s.csa:
                kc = torch.zeros(B, n_cap, 64, dtype=torch.uint8, device=dev)
                ks = torch.zeros(B, n_cap, 4, dtype=torch.uint8, device=dev)
                kc[:, :n_old] = inp["keys_codes_old"]
                ks[:, :n_old] = inp["keys_scales_old"]
                self.keys.append((kc, ks))
        else:
            for c in range(copies):
                sfx = "" if c == 0 else f"_{c}"
                self.caches.append(inp["cache" + sfx])
                if s.csa:
                    self.keys.append((inp["keys_codes" + sfx], inp["keys_scales" + sfx]))
            self.win = inp["win"]
            self.win_pos0 = inp["win_pos0"]
        self.out = torch.empty(B, s.n_q, s.H, s.d, dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty(B, s.n_q, s.H, dtype=torch.float32, device=dev)
        self.idx = torch.empty(B, s.n_q, max(s.top_k, 1), dtype=torch.int32, device=dev)
        self.ws_index = None
        self.ws_attend = None
        self._prep = {}
        self._alloc_workspaces()

    # ------------------------------------------------------------ pieces

    def _main_streams(self):
        mn = self.inp["main"]
        return dict(kv_a=mn["ca"], gate_a=mn["za"], bias_a=mn["ba"],
                    kv_b=mn.get("cb"), gate_b=mn.get("zb"), bias_b=mn.get("bb"))

    def _rows_pos0(self):
        s = self.s
        if self.prefill:
            return s.L - (s.m if s.overlap else 0)
        return s.L - s.m * (2 if s.overlap else 1)

    def _main_job(self, c=0):
        s = self.s
        nope, rope = K.split_main(self.caches[c])
        return K.compress_args(**self._main_streams(), m=s.m, pos0=self._rows_pos0(), out0=nope,
                               out1=rope, d_rope=s.d_r, rope_theta=s.theta, do_norm=True,
                               out_fmt=K.FMT_FP8_BF16)

    def _index_job(self, c=0):
        s = self.s
        ix = self.inp["idx"]
        kc, ks = self.keys[c]
        return K.compress_args(ix["ca"], gate_a=ix["za"], bias_a=ix["ba"], kv_b=ix["cb"],
                               gate_b=ix["zb"], bias_b=ix["bb"], m=s.m, pos0=self._rows_pos0(),
                               out0=kc, out1=ks, d_rope=0, do_norm=False, out_fmt=K.FMT_MXFP4)

    def _window_job(self):
        """Raw window rows (m = 1, no gate): RMSNorm, RoPE at the token's own
        position, FP8/BF16 storage into the window buffer, whose row 0 holds
        position L - n_win + 1."""
        s = self.s
        nope, rope = K.split_main(self.win)
        return K.compress_args(self.inp["win_raw"], m=1, pos0=s.L, out0=nope, out1=rope,
                               d_rope=s.d_r, rope_theta=s.theta, do_norm=True,
                               out_fmt=K.FMT_FP8_BF16, out_row0=s.L - s.n_win + 1)

    def compress_main(self, c=0):
        K.compress_batch([self._main_job(c)])

    def compress_index(self, c=0):
        K.compress_batch([self._index_job(c)])

    def store_window(self):
        K.compress_batch([self._window_job()])

    def _all_jobs(self, c=0):
        jobs = [self._main_job(c)]
        if self.s.csa:
            jobs.append(self._index_job(c))
        jobs.append(self._window_job())
        return jobs

    def _prepared(self, c):
        """The argument structs of copy c's step, built once: every pointer
        they hold stays valid while this object holds the tensors."""
        p = self._prep.get(c)
        if p is None:
            s = self.s
            jobs = self._all_jobs(c)
            arr = (K.CompressArgs * len(jobs))(*jobs)
            p = {"jobs": arr, "n_jobs": len(jobs)}
            if s.csa:
                kc, ks = self.keys[c]
                p["index"] = K.index_args(self.inp["q_idx_codes"], self.inp["w"], kc, self.inp["q_pos"], m=s.m,
                                          top_k=s.top_k, out_idx=self.idx, q1=self.inp["q_idx_scales"], k1=ks,
                                          fmt=K.FMT_MXFP4, flags=self.index_flags)
            nope, rope = K.split_main(self.caches[c])
            wn, wr = K.split_main(self.win)
            p["attend"] = K.attend_args(self.inp["q"], self.inp["q_pos"], nope, wn, self.win_pos0,
                                        self.inp["sink"], self.out, m=s.m, n_win=s.n_win, kv1=rope, win1=wr,
                                        idx=self.idx if s.csa else None, out_lse=self.lse, d_rope=s.d_r,
                                        rope_theta=s.theta, fmt=K.FMT_FP8_BF16, flags=self.attend_flags)
            self._prep[c] = p
        return p

    def compress_all(self, c=0, stream=None, entries=True):
        """Every store of the step in one batched call: the newest entry (and,
        for CSA, the newest indexer key) and the raw window rows; long blocks
        are pooled over many workgroups through the step's workspace.  With
        entries=False only the window row is stored (a decode step whose
        position completes no block: m - 1 of every m steps)."""
        p = self._prepared(c)
        st = K._stream() if stream is None else stream
        if entries:
            jobs, n = p["jobs"], p["n_jobs"]
        else:
            if "win_only" not in p:
                p["win_only"] = (K.CompressArgs * 1)(self._window_job())
            jobs, n = p["win_only"], 1
        K._check(self._fn_compress(jobs, n, self._ws_c[0], self._ws_c[1], st), "csa_compress_batch_ws")

    def index(self, c=0, events=(None, None), stream=None):
        """csa_index_topk; `events` = optional HIP event handles recorded around
        the scoring kernel."""
        a = self._prepared(c)["index"]
        a.ev_start, a.ev_stop = events
        st = K._stream() if stream is None else stream
        K._check(self._fn_index(C.byref(a), self._ws_i[0], self._ws_i[1], st), "csa_index_topk")

    def attend(self, c=0, events=(None, None), stream=None):
        """csa_attend / hca_attend; `events` as for index()."""
        a = self._prepared(c)["attend"]
        a.ev_start, a.ev_stop = events
        st = K._stream() if stream is None else stream
        K._check(self._fn_attend(C.byref(a), self._ws_a[0], self._ws_a[1], st), "attend")

    def _alloc_workspaces(self):
        s = self.s
        dev = self.out.device
        n = K.compress_workspace_bytes(self._all_jobs(0))
        self.ws_compress = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
        if s.csa:
            kc, ks = self.keys[0]
            a = K.index_args(self.inp["q_idx_codes"], self.inp["w"], kc, self.inp["q_pos"], m=s.m,
                             top_k=s.top_k, out_idx=self.idx, q1=self.inp["q_idx_scales"], k1=ks,
                             fmt=K.FMT_MXFP4, flags=self.index_flags)
            n = K.workspace_bytes(K.OP_INDEX_TOPK, a)
            self.ws_index = (torch.zeros(max(n, 256), dtype=torch.uint8, device=dev), n)
        nope, rope = K.split_main(self.caches[0])
        wn, wr = K.split_main(self.win)
        a = K.attend_args(self.inp["q"], self.inp["q_pos"], nope, wn, self.win_pos0, self.inp["sink"],
                          self.out, m=s.m, n_win=s.n_win, kv1=rope, win1=wr,
                          idx=self.idx if s.csa else None, d_rope=s.d_r, rope_theta=s.theta,
                          fmt=K.FMT_FP8_BF16, flags=self.attend_flags)
        n = K.workspace_bytes(K.OP_ATTEND if s.csa else K.OP_HCA_ATTEND, a)
        self.ws_attend = (torch.zeros(max(n, 256), dtype=torch.uint8, device=dev) if n else None, n)
        # the library entry points and workspace (pointer, bytes) pairs, bound once
        lib = K.load()
        self._fn_compress = lib.csa_compress_batch_ws
        self._fn_index = lib.csa_index_topk
        self._fn_attend = lib.csa_attend if s.csa else lib.hca_attend
        self._ws_c = (K._ptr(self.ws_compress), self.ws_compress.numel())
        self._ws_i = (K._ptr(self.ws_index[0]), self.ws_index[1]) if self.ws_index else (None, 0)
        self._ws_a = (K._ptr(self.ws_attend[0]), self.ws_attend[1])

    # ------------------------------------------------------------ whole step

    def run(self, c=0, events=None, stream=None, entries=True):
        """One full step on the current stream (or `stream`, a HIP stream
        handle), no synchronisation.  `events` optionally maps 'index' /
        'attend' to (start, stop) HIP event handles recorded around the scoring
        and attention kernels.  entries=False: a step that completes no block
        (only the window row is stored)."""
        ev = events or {}
        st = K._stream() if stream is None else stream
        self.compress_all(c, stream=st, entries=entries)
        if self.s.csa:
            self.index(c, events=ev.get("index", (None, None)), stream=st)
        self.attend(c, events=ev.get("attend", (None, None)), stream=st)
