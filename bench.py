"""Decode throughput of one CSA + HCA layer pair at 1M context on one MI355X.

Workload (synthetic, seeded, generated on the device):
  CSA layer: Pro-shaped decode, 8 sequences at 2^20 tokens of context
             (262144 compressed entries each, 128 heads, head dim 512, indexer
             64 heads x 128 in MXFP4, top-k 1024, window 128, sink).
  HCA layer: Flash-shaped decode, 32 sequences at 2^20 tokens (8192 entries
             each, 64 heads, window 128, sink).
One step = one full decode step of each layer (compress of the newest
blocks, window store, index + top-k for CSA, attention).  Per-token cost of
the pair is t_csa / 8 + t_hca / 32, so the reported value is
1 / (t_csa / 8 + t_hca / 32) decode tokens per second per layer pair.

Caches are kept in four copies that consecutive steps rotate through, so the
256 MB Infinity Cache cannot serve a step from the previous step's reads (each
layer of a real model has caches of its own).  All inputs are resident in HBM
before the timed region.

The same line also carries a prefill measurement (config.prefill): one
Pro-shaped 8192-token chunk appended to 2^20 cached tokens, for a CSA and an
HCA layer (compress of the chunk, window store, index + top-k for CSA,
attention), as tokens/s and as the achieved fraction of the MFMA peaks
(MXFP4 for the indexer's scoring, BF16 for the attention), next to the fp64
oracle timed on sampled query rows.
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/s per layer at 1M ctx (CSA+HCA) and % of HBM roofline"
HBM_PEAK_GBS = 8000.0
MXFP4_PEAK_TFLOPS = 10100.0     # dense MFMA, published
BF16_PEAK_TFLOPS = 2500.0       # dense MFMA, published
COPIES = 4
EVENT_DISABLE_SYSTEM_FENCE = 0x20000000     # hipEventDisableSystemFence
CSRC = os.path.join(ROOT, "long_context_attention_09_amd", "csrc")

# HBM traffic per launch from rocprofv3 --pmc runs of this script (FETCH_SIZE
# in one run, WRITE_SIZE in another; KiB per dispatch, averaged over the timed
# dispatches), scaled by what the same counters read for a plain elementwise
# copy of known size (python bench.py --copy-calibration).  Each entry records
# the SHA-256 of the kernel's source file when the counters were taken; once
# the source differs, the figure no longer describes the kernel and traffic is
# reported as null.
FETCH_FACTOR = 2.0    # true bytes read / (FETCH_SIZE KiB * 1024) on the copy
WRITE_FACTOR = 1.0    # true bytes written / (WRITE_SIZE KiB * 1024) on the copy
TRAFFIC = {
    "attend_fp8_kernel(hca)": {
        "source": "attend.hip",
        "sha256": "f0cc14f98ffa7f86e21d0069cfff0b89cebd7c3d37000985ba398b2794dd716b",
        "fetch_kib": 83406.6, "write_kib": 16512.0},
    "index_mxfp4_kernel": {
        "source": "index_topk.hip",
        "sha256": "74a377de10592a718226ca83c67691ed054afc4f302426dfdff911c3aaa33eff",
        "fetch_kib": 69843.4, "write_kib": 8356.8},
}


class HipEvents:
    """HIP events through the runtime's C API, for the library's timing hook."""

    def __init__(self):
        self.h = C.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.h.hipEventSynchronize.argtypes = [C.c_void_p]

    def create(self):
        # timing events without the system-scope fence at each record (nothing
        # on the host reads memory through them)
        e = C.c_void_p()
        if self.h.hipEventCreateWithFlags(C.byref(e), C.c_uint(EVENT_DISABLE_SYSTEM_FENCE)) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return e.value

    def elapsed_ms(self, a, b):
        self.h.hipEventSynchronize(C.c_void_p(b))
        ms = C.c_float()
        if self.h.hipEventElapsedTime(C.byref(ms), C.c_void_p(a), C.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value


def algorithmic_bytes(shape, kind):
    """Bytes the method must move per launch (inputs it reads, outputs it writes).

    index: every visible key (64 B E2M1 + 4 B E8M0) plus the query heads
           (MXFP4) and head weights, per sequence.
    attend: every KV row attended (576 B: 448 FP8 + 64 BF16), the BF16 query
            and the BF16 output, per sequence.
    """
    B, L = shape.B, shape.L
    n_vis = L // shape.m
    if kind == "index":
        return B * (n_vis * 68 + shape.H_I * 68 + shape.H_I * 4)
    rows = (shape.top_k if shape.csa else n_vis) + shape.n_win
    return B * (rows * 576 + 2 * shape.H * shape.d * 2)


def prefill_flops(shape):
    """Algorithmic flops of one prefill chunk (queries t = L .. L + n_q - 1).

    index:  every visible key (t // m entries, capped by the entries that
            exist) against every indexer head: H_I * d_I multiply-adds.
    attend: every attended row (CSA: min(top_k, visible) selected entries;
            HCA: every visible entry; both plus the n_win window rows) against
            every head: d multiply-adds for the score and d for the output.
    """
    import numpy as np
    t = shape.L + np.arange(shape.n_q, dtype=np.int64)
    n_all = (shape.L + shape.n_q) // shape.m
    n_vis = np.minimum(t // shape.m, n_all)
    out = {}
    if shape.csa:
        out["index"] = float(n_vis.sum()) * shape.H_I * shape.d_I * 2
        rows = np.minimum(n_vis, shape.top_k) + shape.n_win
    else:
        rows = n_vis + shape.n_win
    out["attend"] = float(rows.sum()) * shape.H * shape.d * 4
    return out


def traffic_bytes(label):
    t = TRAFFIC.get(label)
    if t is None or FETCH_FACTOR is None or WRITE_FACTOR is None:
        return None
    with open(os.path.join(CSRC, t["source"]), "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != t["sha256"]:
            return None
    return t["fetch_kib"] * 1024 * FETCH_FACTOR + t["write_kib"] * 1024 * WRITE_FACTOR


def copy_calibration():
    """A plain elementwise copy of 1 GiB (read 1 GiB, write 1 GiB), three
    times, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4,
                      "launches": 3}), flush=True)


def copy_bandwidth():
    """Measured device bandwidth of a plain elementwise copy (1 GiB read +
    1 GiB written, best of five), the practical ceiling next to the
    published 8 TB/s."""
    import torch
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    best = None
    for _ in range(6):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None or ms < best else best
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n * 4 / (best * 1e-3) / 1e9


def time_steps(ev, st, steps, warmup, fn):
    """Average ms of fn(k) over `steps` calls after `warmup`, HIP events on st."""
    import torch
    record = ev.h.hipEventRecord
    for k in range(warmup):
        fn(k)
    marks = [(ev.create(), ev.create()) for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        record(C.c_void_p(marks[k][0]), st)
        fn(warmup + k)
        record(C.c_void_p(marks[k][1]), st)
    torch.cuda.synchronize()
    return sum(ev.elapsed_ms(a, b) for a, b in marks) / steps


def cpu_baseline(csa_shape, hca_shape, csa_inp, hca_inp, budget_s=15.0):
    """The fp64 oracle on this host's cores, on a bounded sample of the same
    workload: whole decode steps of single sequences (CSA and HCA alternately)
    until about budget_s seconds of CPU work; scaled to the pair rate."""
    from oracle import pipeline as P
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1

    def host_inputs(inp, b):
        out = {}
        for k, v in inp.items():
            if isinstance(v, dict):
                out[k] = {kk: vv[b:b + 1].cpu() if vv.dim() == 3 else vv.cpu() for kk, vv in v.items()}
            elif isinstance(v, list):
                continue
            elif k.endswith(("_1", "_2")):
                continue
            elif v.dim() >= 1 and v.shape[0] == inp["q"].shape[0] and k not in ("sink",):
                out[k] = v[b:b + 1].cpu()
            else:
                out[k] = v.cpu()
        return out

    t_csa, n_csa, t_hca, n_hca = 0.0, 0, 0.0, 0
    n_seq = min(csa_shape.B, hca_shape.B)
    hosts = {}
    k = 0
    while t_csa + t_hca < budget_s:
        b = k % n_seq               # sequences are revisited once all have been timed
        if b not in hosts:
            hosts[b] = (host_inputs(csa_inp, b), host_inputs(hca_inp, b))
        hc, hh = hosts[b]
        t0 = time.perf_counter()
        P.decode_step(csa_shape.replace(B=1), hc, 0)
        t_csa += time.perf_counter() - t0
        n_csa += 1
        t0 = time.perf_counter()
        P.decode_step(hca_shape.replace(B=1), hh, 0)
        t_hca += time.perf_counter() - t0
        n_hca += 1
        k += 1
    per_tok = t_csa / n_csa + t_hca / n_hca
    return {"value": 1.0 / per_tok, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n_csa} CSA + {n_hca} HCA single-sequence decode steps (sequences 0..."
                      f"{min(k, n_seq) - 1} of the same workload, revisited in turn; fp64 NumPy "
                      f"oracle), {t_csa + t_hca:.1f} s; rate = 1 / (t_csa_seq + t_hca_seq)"}


def prefill_oracle(shapes, inps, rows_per_layer):
    """The fp64 oracle on a sample of each prefill chunk: the chunk's own
    stores once, then rows_per_layer query rows (first, last and evenly
    spaced between); the chunk time is extrapolated as
    t_stores + n_q * t_row."""
    from oracle import pipeline as P
    per = {}
    total = 0.0
    for name, shape, inp in zip(("csa", "hca"), shapes, inps):
        t0 = time.perf_counter()
        prep = P.prefill_prepare(shape, inp, 0)
        t_prep = time.perf_counter() - t0
        rows = sorted(set(int(round(i * (shape.n_q - 1) / max(rows_per_layer - 1, 1)))
                          for i in range(rows_per_layer)))
        t0 = time.perf_counter()
        for r in rows:
            P.prefill_query(shape, inp, prep, 0, r)
        t_row = (time.perf_counter() - t0) / len(rows)
        t_chunk = t_prep + shape.n_q * t_row
        total += t_chunk
        per[name] = {"rows_timed": len(rows), "s_stores": round(t_prep, 3), "s_per_row": round(t_row, 4),
                     "tokens_per_s": round(shape.n_q / t_chunk, 2)}
    per["tokens_per_s"] = round(shapes[0].n_q / total, 2)
    per["sample"] = (f"the chunk's stores plus {rows_per_layer} query rows per layer, fp64 NumPy oracle; "
                     "chunk time extrapolated as t_stores + 8192 t_row; rate over the CSA+HCA pair")
    return per


def bf16_scores_leg(ev, st, step, shape, steps):
    """The CSA index op with fp32 and with BF16 scores over the same caches:
    selector time (the op minus its scoring kernel, HIP events on the bench
    stream) and the fraction of the fp32 selection the BF16 one keeps."""
    import torch
    from long_context_attention_09_amd import _lib as K
    res = {}
    sel = {}
    for name, flags in (("fp32", 0), ("bf16", K.INDEX_BF16_SCORES)):
        kc, ks = step.keys[0]
        idx = torch.empty_like(step.idx)
        a = K.index_args(step.inp["q_idx_codes"], step.inp["w"], kc, step.inp["q_pos"], m=shape.m,
                         top_k=shape.top_k, out_idx=idx, q1=step.inp["q_idx_scales"], k1=ks, fmt=K.FMT_MXFP4,
                         flags=flags)
        n = K.workspace_bytes(K.OP_INDEX_TOPK, a)
        ws = torch.zeros(max(n, 256), dtype=torch.uint8, device="cuda")
        lib = K.load()
        e_sc = [(ev.create(), ev.create()) for _ in range(steps + 2)]
        e_op = [(ev.create(), ev.create()) for _ in range(steps + 2)]
        torch.cuda.synchronize()
        for k in range(steps + 2):
            a.ev_start, a.ev_stop = e_sc[k]
            ev.h.hipEventRecord(C.c_void_p(e_op[k][0]), st)
            K._check(lib.csa_index_topk(C.byref(a), K._ptr(ws), ws.numel(), st), "csa_index_topk")
            ev.h.hipEventRecord(C.c_void_p(e_op[k][1]), st)
        torch.cuda.synchronize()
        t_op = sum(ev.elapsed_ms(*e_op[k]) for k in range(2, steps + 2)) / steps
        t_sc = sum(ev.elapsed_ms(*e_sc[k]) for k in range(2, steps + 2)) / steps
        res[name] = {"op_us": round(t_op * 1e3, 2), "scoring_us": round(t_sc * 1e3, 2),
                     "selector_us": round((t_op - t_sc) * 1e3, 2)}
        sel[name] = idx.clone()
        del ws
    kept = torch.isin(sel["bf16"].view(-1, shape.top_k)[0], sel["fp32"].view(-1, shape.top_k)[0])
    rec = []
    for r in range(sel["fp32"].shape[0] * sel["fp32"].shape[1]):
        a32 = sel["fp32"].view(-1, shape.top_k)[r]
        a16 = sel["bf16"].view(-1, shape.top_k)[r]
        rec.append(float(torch.isin(a16, a32).float().mean()))
    res["recall_of_fp32_selection"] = {"min": round(min(rec), 5), "mean": round(sum(rec) / len(rec), 5)}
    res["selector_speedup"] = round(res["fp32"]["selector_us"] / max(res["bf16"]["selector_us"], 1e-9), 3)
    del kept
    return res


def flash_leg(ev, st, steps):
    """Flash-shaped CSA decode (B=16, 131072 tokens of context, 64 heads,
    top-k 512): the step time, tokens/s and its fraction of the HBM roofline
    (algorithmic bytes of the index and attention per step over 8 TB/s)."""
    import torch
    import synth
    from long_context_attention_09_amd.layer import LayerStep
    shape = synth.FLASH_CSA_DECODE
    print("[bench] flash csa 128k: generating inputs", file=sys.stderr, flush=True)
    inp = synth.quant_decode_inputs(shape, device="cuda", copies=COPIES)
    step = LayerStep(shape, inp, copies=COPIES)
    torch.cuda.synchronize()
    t = time_steps(ev, st, steps, 3, lambda k: step.run(k % COPIES, stream=st))
    byts = algorithmic_bytes(shape, "index") + algorithmic_bytes(shape, "attend")
    out = {"workload": "Flash-shaped CSA decode: B=16, context 131072 (32768 entries), H=64, top-k 512, "
                       "indexer 64x128 MXFP4, window 128, sink",
           "ms_per_step": round(t, 4), "tokens_per_s": round(shape.B / (t * 1e-3), 1),
           "algorithmic_bytes": byts, "hbm_frac": round(byts / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del step, inp
    torch.cuda.empty_cache()
    return out


def paged_leg(ev, st, steps, shapes, inps, contiguous_ms):
    """The decode step over the heterogeneous paged cache: entries in shuffled
    128-token blocks through block tables, window and compressor tails in
    per-request rings, compression in the per-sequence decode mode.  Timed at
    t = L (the step stores the window row only) and at t = L + m - 1 (that
    token completes a block: the entry is compressed as well, the pessimistic
    form the headline value uses), with COPIES pool copies rotated like the
    contiguous caches."""
    import numpy as np
    import torch
    from long_context_attention_09_amd import paged
    out = {}
    for shape, inp in zip(shapes, inps):
        kind = "csa" if shape.csa else "hca"
        print(f"[bench] paged {kind}: building pools", file=sys.stderr, flush=True)
        per_req = -(-shape.L // paged.TOKENS_PER_BLOCK) + 1
        n_blocks = shape.B * per_req
        alloc = paged.BlockAllocator(n_blocks, order=np.random.default_rng(shape.seed).permutation(n_blocks))
        cache = paged.PagedCache(shape.B, shape.L + paged.TOKENS_PER_BLOCK, alloc, "cuda")
        for b in range(shape.B):
            cache.reserve(b, shape.L + paged.TOKENS_PER_BLOCK)
        mn = inp["main"]
        bias = {"main": (mn["ba"], mn.get("bb"))}
        if shape.csa:
            bias["idx"] = (inp["idx"]["ba"], inp["idx"]["bb"])
        done = shape.m - 1                               # t = L + m - 1 completes entry L / m
        steps_at = {0: [], done: []}
        layers = []
        for c in range(COPIES):
            sfx = "" if c == 0 else f"_{c}"
            layer = paged.PagedLayer(cache, shape, bias, "cuda")
            layer.import_contiguous(inp["cache" + sfx], inp.get("keys_codes" + sfx), inp.get("keys_scales" + sfx),
                                    inp["win"], inp["win_pos0"].tolist())
            for n, t in layer.main_ring.items():       # raw rows of the newest tokens (synthetic)
                t.copy_(mn[n][:, :layer.ring_rows])
            if shape.csa:
                for n, t in layer.idx_ring.items():
                    t.copy_(inp["idx"][n][:, :layer.ring_rows])
            layer.win_raw.copy_(inp["win_raw"])
            layers.append(layer)
            for dt in (0, done):
                seq_pos = inp["q_pos"].view(-1) + dt
                steps_at[dt].append(paged.PagedDecodeStep(layer, seq_pos, inp["q"], inp["sink"], inp.get("q_idx_codes"),
                                                          inp.get("q_idx_scales"), inp.get("w")))
        torch.cuda.synchronize()
        t_w = time_steps(ev, st, steps, 2, lambda k: steps_at[0][k % COPIES].run(stream=st))
        t_b = time_steps(ev, st, steps, 2, lambda k: steps_at[done][k % COPIES].run(stream=st))
        out[kind] = {"ms_window_only": round(t_w, 4), "ms_block_completes": round(t_b, 4),
                     "vs_contiguous": round(contiguous_ms[kind] / t_b, 4),
                     "blocks": n_blocks, "entries_per_block": paged.TOKENS_PER_BLOCK // shape.m}
        del steps_at, layers, cache
        torch.cuda.empty_cache()
    out["tokens_per_s"] = round(1.0 / (out["csa"]["ms_block_completes"] / shapes[0].B
                                       + out["hca"]["ms_block_completes"] / shapes[1].B) * 1e3, 1)
    out["note"] = ("blocks of 128 raw tokens (32 CSA entries / indexer keys, 1 HCA entry) in shuffled physical "
                   "order; vs_contiguous = contiguous step time / paged step time, both compressing an entry")
    return out


def selection_recall(ref, got):
    """Per row, the fraction of ref's selected indices (ascending, -1 padded)
    that got also selects; rows of [..., k] int32 tensors on the device."""
    import torch
    k = ref.shape[-1]
    r = ref.reshape(-1, k).long()
    g = got.reshape(-1, k).long()
    both = torch.cat([r, g], dim=1).sort(dim=1).values
    common = ((both[:, 1:] == both[:, :-1]) & (both[:, 1:] >= 0)).sum(dim=1)
    n_ref = (r >= 0).sum(dim=1).clamp(min=1)
    return (common.float() / n_ref.float())


def prefill_bf16_leg(ev, st, steps, csa, shape, inp):
    """The prefill chunk's CSA index op with fp32 and with BF16 scores, timed
    alternately in one loop (HIP events on the bench stream, same clocks and
    caches for both), and the recall of the fp32 selection."""
    import torch
    from long_context_attention_09_amd.layer import LayerStep
    b16 = LayerStep(shape, inp, prefill=True, bf16_scores=True)
    b16.compress_all(stream=st)
    record = ev.h.hipEventRecord
    marks = {n: [(ev.create(), ev.create()) for _ in range(steps + 1)] for n in ("fp32", "bf16")}
    for k in range(steps + 1):
        for n, step in (("fp32", csa), ("bf16", b16)):
            e0, e1 = marks[n][k]
            record(C.c_void_p(e0), st)
            step.index(stream=st)
            record(C.c_void_p(e1), st)
    torch.cuda.synchronize()
    t = {n: sum(ev.elapsed_ms(e0, e1) for e0, e1 in m[1:]) / steps for n, m in marks.items()}
    rec = selection_recall(csa.idx, b16.idx)
    res = {"fp32_index_op_ms": round(t["fp32"], 3), "bf16_index_op_ms": round(t["bf16"], 3),
           "speedup": round(t["fp32"] / t["bf16"], 3),
           "recall_of_fp32_selection": {"min": round(float(rec.min()), 5), "mean": round(float(rec.mean()), 5)}}
    del b16
    torch.cuda.empty_cache()
    return res


def prefill_leg(ev, st, steps, warmup, oracle_rows):
    """One 8192-token chunk after 2^20 cached tokens through a CSA and an HCA
    layer, timed with HIP events per operation on the bench stream."""
    import torch
    import synth
    from long_context_attention_09_amd.layer import LayerStep

    csa_shape, hca_shape = synth.PRO_CSA_PREFILL, synth.PRO_HCA_PREFILL
    print("[bench] prefill: generating inputs", file=sys.stderr, flush=True)
    csa_inp = synth.quant_prefill_inputs(csa_shape, device="cuda")
    hca_inp = synth.quant_prefill_inputs(hca_shape, device="cuda")
    csa = LayerStep(csa_shape, csa_inp, prefill=True)
    hca = LayerStep(hca_shape, hca_inp, prefill=True)
    torch.cuda.synchronize()
    record = ev.h.hipEventRecord
    n = warmup + steps
    marks = [[ev.create() for _ in range(7)] for _ in range(n)]

    def step(m):
        record(C.c_void_p(m[0]), st)
        csa.compress_all(stream=st)
        record(C.c_void_p(m[1]), st)
        csa.index(stream=st)
        record(C.c_void_p(m[2]), st)
        csa.attend(stream=st)
        record(C.c_void_p(m[3]), st)
        hca.compress_all(stream=st)
        record(C.c_void_p(m[4]), st)
        hca.attend(stream=st)
        record(C.c_void_p(m[5]), st)

    print("[bench] prefill: warmup", file=sys.stderr, flush=True)
    for k in range(warmup):
        step(marks[k])
    torch.cuda.synchronize()
    print("[bench] prefill: timed", file=sys.stderr, flush=True)
    for k in range(warmup, n):
        step(marks[k])
    torch.cuda.synchronize()
    timed = marks[warmup:]

    def avg(i, j):
        return sum(ev.elapsed_ms(m[i], m[j]) for m in timed) / steps

    t = {"csa_compress": avg(0, 1), "csa_index_topk": avg(1, 2), "csa_attend": avg(2, 3),
         "hca_compress": avg(3, 4), "hca_attend": avg(4, 5)}
    t_csa = avg(0, 3)
    t_hca = avg(3, 5)
    f_csa, f_hca = prefill_flops(csa_shape), prefill_flops(hca_shape)

    def mfma(flops, ms, peak):
        tf = flops / (ms * 1e-3) / 1e12
        return {"ms": round(ms, 3), "tflop": round(flops / 1e12, 3), "achieved_tflops": round(tf, 1),
                "peak_tflops": peak, "frac": round(tf / peak, 4)}

    out = {
        "workload": "Pro-shaped prefill chunk: 8192 new tokens after 2^20 cached tokens, B=1, H=128, "
                    "CSA (m=4 overlap, indexer 64x128 MXFP4, top-k 1024) and HCA (m=128), window 128, sink",
        "steps": steps, "warmup": warmup,
        "csa": {"ms_per_chunk": round(t_csa, 3), "tokens_per_s": round(csa_shape.n_q / (t_csa * 1e-3), 1)},
        "hca": {"ms_per_chunk": round(t_hca, 3), "tokens_per_s": round(hca_shape.n_q / (t_hca * 1e-3), 1)},
        "tokens_per_s": round(csa_shape.n_q / ((t_csa + t_hca) * 1e-3), 1),
        "ops_ms": {k: round(v, 3) for k, v in t.items()},
        # the index op is the scoring kernel plus the top-k passes of every
        # query block; its fraction counts the scoring flops only.  The
        # attention's score product runs its FP8-stored dims as scaled FP8
        # products against a two-component query (the matrix time of BF16
        # products) and the rest in BF16, so its fraction is against the
        # BF16 peak.
        "mfma": {"csa_index_topk(mxfp4)": mfma(f_csa["index"], t["csa_index_topk"], MXFP4_PEAK_TFLOPS),
                 "csa_attend(fp8+bf16)": mfma(f_csa["attend"], t["csa_attend"], BF16_PEAK_TFLOPS),
                 "hca_attend(fp8+bf16)": mfma(f_hca["attend"], t["hca_attend"], BF16_PEAK_TFLOPS)},
    }
    # BF16 index scores at prefill, where the top-k passes stream every
    # query's scores: the CSA index op against the fp32 one, and the recall
    # of the fp32 selection over every query of the chunk
    print("[bench] prefill: bf16 index scores", file=sys.stderr, flush=True)
    del hca
    torch.cuda.empty_cache()
    out["bf16_index_scores"] = prefill_bf16_leg(ev, st, steps, csa, csa_shape, csa_inp)
    if oracle_rows > 0:
        print("[bench] prefill: oracle sample", file=sys.stderr, flush=True)
        out["oracle"] = prefill_oracle((csa_shape, hca_shape), (csa_inp, hca_inp), oracle_rows)
    del csa, csa_inp, hca_inp
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--flash-steps", type=int, default=20,
                    help="timed steps of the Flash-shaped CSA decode at 128K (0: none)")
    ap.add_argument("--prefill-steps", type=int, default=3,
                    help="timed prefill chunks (0: no prefill measurement)")
    ap.add_argument("--prefill-oracle-rows", type=int, default=16,
                    help="query rows per layer the oracle is timed on (0: none)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only the 1 GiB elementwise copy used to scale HBM counters")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline decode steps (no side measurements): for profilers")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the prefill chunk and print its measurement: for profilers")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the layer's decode is "
              "measured on one GPU's share; see the design notes for how it would shard.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    from long_context_attention_09_amd import _lib as K
    from long_context_attention_09_amd.layer import LayerStep

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    K.load()
    if args.prefill_only:
        ev = HipEvents()
        st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
        print(json.dumps({"prefill": prefill_leg(ev, st, max(args.prefill_steps, 1), 1, 0)}), flush=True)
        return
    dev = "cuda"
    csa_shape, hca_shape = synth.PRO_CSA_DECODE, synth.FLASH_HCA_DECODE
    print("[bench] generating inputs", file=sys.stderr, flush=True)
    csa_inp = synth.quant_decode_inputs(csa_shape, device=dev, copies=COPIES)
    hca_inp = synth.quant_decode_inputs(hca_shape, device=dev, copies=COPIES)
    csa = LayerStep(csa_shape, csa_inp, copies=COPIES)
    hca = LayerStep(hca_shape, hca_inp, copies=COPIES)
    torch.cuda.synchronize()

    ev = HipEvents()
    stream = torch.cuda.current_stream()
    n = args.warmup + args.steps
    marks = [[ev.create() for _ in range(8)] for _ in range(n)]

    st = C.c_void_p(stream.cuda_stream)
    record = ev.h.hipEventRecord

    def step(k, m):
        c = k % COPIES
        # layer-level marks on the same stream only: the kernels' own times
        # (indexer, HCA attention) are taken after the timed region, so no
        # kernel-level marks sit inside the timed steps
        record(C.c_void_p(m[0]), st)
        csa.run(c, stream=st)
        record(C.c_void_p(m[1]), st)
        hca.run(c, stream=st)
        record(C.c_void_p(m[4]), st)

    ev.h.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
    print("[bench] warmup", file=sys.stderr, flush=True)
    for k in range(args.warmup):
        step(k, marks[k])
    torch.cuda.synchronize()
    print("[bench] timed", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for k in range(args.warmup, n):
        step(k, marks[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / args.steps * 1e3

    timed = marks[args.warmup:]
    t_csa = sum(ev.elapsed_ms(m[0], m[1]) for m in timed) / args.steps
    t_hca = sum(ev.elapsed_ms(m[1], m[4]) for m in timed) / args.steps
    # the indexer's kernel time: its own short run after the timed region
    # (whole CSA steps, marks around the scoring kernel only)
    idx_marks = [(ev.create(), ev.create()) for _ in range(10)]
    for k, (e0, e1) in enumerate(idx_marks):
        csa.run(k % COPIES, events={"index": (e0, e1)}, stream=st)
    torch.cuda.synchronize()
    k_idx = sum(ev.elapsed_ms(e0, e1) for e0, e1 in idx_marks) / len(idx_marks)
    # the HCA attention kernel's time the same way: whole HCA steps, marks
    # through the library hook around the attention kernel only
    att_marks = [(ev.create(), ev.create()) for _ in range(args.steps)]
    for k, (e0, e1) in enumerate(att_marks):
        hca.run(k % COPIES, events={"attend": (e0, e1)}, stream=st)
    torch.cuda.synchronize()
    k_hca = sum(ev.elapsed_ms(e0, e1) for e0, e1 in att_marks) / len(att_marks)
    rate_csa = csa_shape.B / (t_csa * 1e-3)
    rate_hca = hca_shape.B / (t_hca * 1e-3)
    value = 1.0 / (1.0 / rate_csa + 1.0 / rate_hca)

    b_idx = algorithmic_bytes(csa_shape, "index")
    b_hca = algorithmic_bytes(hca_shape, "attend")
    kernels = {
        "index_mxfp4_kernel": {"ms": k_idx, "bytes": b_idx, "GB/s": b_idx / (k_idx * 1e-3) / 1e9},
        "attend_fp8_kernel(hca)": {"ms": k_hca, "bytes": b_hca, "GB/s": b_hca / (k_hca * 1e-3) / 1e9},
    }
    dom_name = max(kernels, key=lambda k: kernels[k]["ms"])
    dom = kernels[dom_name]
    traffic = traffic_bytes(dom_name)
    roofline = {"bound": "hbm", "kernel": dom_name, "achieved": round(dom["GB/s"], 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dom["GB/s"] / HBM_PEAK_GBS, 4),
                "traffic": None if traffic is None else round(traffic),
                "algorithmic_bytes": dom["bytes"]}
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8/bf16 kv, mxfp4 indexer, bf16 mfma fp32 acc", "data": "synthetic",
        "config": {
            "workload": "CSA+HCA layer-pair decode at 1M context: Pro CSA (B=8, H=128, top-k 1024, "
                        "262144 entries) + Flash HCA (B=32, H=64, 8192 entries), window 128, sink",
            "csa": {"B": csa_shape.B, "ctx": csa_shape.L, "ms_per_step": round(t_csa, 4),
                    "tokens_per_s": round(rate_csa, 1)},
            "hca": {"B": hca_shape.B, "ctx": hca_shape.L, "ms_per_step": round(t_hca, 4),
                    "tokens_per_s": round(rate_hca, 1)},
            "kernels": {k: {kk: round(vv, 4) for kk, vv in v.items()} for k, v in kernels.items()},
            "cache_copies_rotated": COPIES,
        },
        "roofline": roofline,
    }
    if args.headline_only:
        print(json.dumps(line), flush=True)
        return
    # the same decode step with the newest entries' compression amortised over
    # the m (CSA) and m' (HCA) tokens a block takes to complete: steps that
    # only store the window row, plus 1/m of the entry compression
    print("[bench] amortised compression", file=sys.stderr, flush=True)
    t_csa_w = time_steps(ev, st, args.steps, 2, lambda k: csa.run(k % COPIES, stream=st, entries=False))
    t_hca_w = time_steps(ev, st, args.steps, 2, lambda k: hca.run(k % COPIES, stream=st, entries=False))
    a_csa = t_csa_w + (t_csa - t_csa_w) / csa_shape.m
    a_hca = t_hca_w + (t_hca - t_hca_w) / hca_shape.m
    line["config"]["amortised_compress"] = {
        "csa_ms_per_step": round(a_csa, 4), "hca_ms_per_step": round(a_hca, 4),
        "tokens_per_s": round(1.0 / (a_csa / csa_shape.B + a_hca / hca_shape.B) * 1e3, 1),
        "window_only_ms": {"csa": round(t_csa_w, 4), "hca": round(t_hca_w, 4)},
        "note": "value above compresses the newest entries on every step (the pessimistic form); here "
                "1/m of that work per token (m = 4 CSA, 128 HCA)"}
    # BF16 index scores: selector time against fp32 scores and recall of the
    # fp32 selection, on this workload
    print("[bench] bf16 index scores", file=sys.stderr, flush=True)
    line["config"]["bf16_index_scores"] = bf16_scores_leg(ev, st, csa, csa_shape, args.steps)
    # batch-invariant mode (fixed attention splits, exact indexer form): cost
    print("[bench] batch-invariant mode", file=sys.stderr, flush=True)
    csa_i = LayerStep(csa_shape, csa_inp, copies=COPIES, batch_invariant=True)
    hca_i = LayerStep(hca_shape, hca_inp, copies=COPIES, batch_invariant=True)
    t_csa_i = time_steps(ev, st, args.steps, 2, lambda k: csa_i.run(k % COPIES, stream=st))
    t_hca_i = time_steps(ev, st, args.steps, 2, lambda k: hca_i.run(k % COPIES, stream=st))
    v_inv = 1.0 / (t_csa_i / csa_shape.B + t_hca_i / hca_shape.B) * 1e3
    line["config"]["batch_invariant"] = {
        "csa_ms_per_step": round(t_csa_i, 4), "hca_ms_per_step": round(t_hca_i, 4),
        "tokens_per_s": round(v_inv, 1), "vs_default": round(v_inv / value, 4)}
    del csa_i, hca_i
    # the same decode over the heterogeneous paged cache (block tables + state rings)
    line["config"]["paged_kv"] = paged_leg(ev, st, args.steps, (csa_shape, hca_shape), (csa_inp, hca_inp),
                                           {"csa": t_csa, "hca": t_hca})
    # copy bandwidth measured on this GPU: the roofline against it as well
    bw = copy_bandwidth()
    roofline["measured_copy_GBps"] = round(bw, 1)
    roofline["frac_vs_copy"] = round(dom["GB/s"] / bw, 4)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(csa_shape, hca_shape, csa_inp, hca_inp, args.cpu_budget)
    if args.flash_steps > 0:
        del csa, hca, csa_inp, hca_inp
        torch.cuda.empty_cache()
        line["config"]["flash_csa_decode_128k"] = flash_leg(ev, st, args.flash_steps)
    if args.prefill_steps > 0:
        if args.flash_steps <= 0:
            del csa, hca, csa_inp, hca_inp
            torch.cuda.empty_cache()
        line["config"]["prefill"] = prefill_leg(ev, st, args.prefill_steps, 1,
                                                0 if args.no_cpu_baseline else args.prefill_oracle_rows)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
