"""ctypes binding of libcsa.so: argument marshalling only.

Every step of the layer runs in the library's gfx950 kernels.  Tensors are
torch tensors on the GPU (PyTorch provides device memory and the stream); the
binding checks dtypes, devices, shapes and contiguity, fills the C argument
structs of include/csa.h and calls the entry point on torch's current stream.
There is no fallback: a missing library or a failing call raises.
"""
from __future__ import annotations

import ctypes as C
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa.so")

CSA_OK, CSA_EINVAL, CSA_EUNSUPPORTED, CSA_EHIP, CSA_EWORKSPACE, CSA_ESCRATCH = 0, -1, -2, -3, -4, -5
NOALLOC_SCRATCH_BYTES = 64 << 20
FMT_F32, FMT_FP8_BF16, FMT_MXFP4 = 0, 1, 2
DT_F32, DT_BF16 = 0, 1
OP_COMPRESS, OP_INDEX_TOPK, OP_ATTEND, OP_HCA_ATTEND = 0, 1, 2, 3
ATTEND_NORM_Q, ATTEND_NO_INV_ROPE, ATTEND_BATCH_INVARIANT, ATTEND_WIN_RING = 1, 2, 4, 8
INDEX_BATCH_INVARIANT, INDEX_BF16_SCORES = 1, 2
INVARIANT_SPLIT_ROWS = 1024
ABI_VERSION = 3

_vp = C.c_void_p


class CompressArgs(C.Structure):
    _fields_ = [("B", C.c_int32), ("n_rows", C.c_int32), ("pos0", C.c_int64), ("m", C.c_int32),
                ("overlap", C.c_int32), ("d", C.c_int32), ("d_rope", C.c_int32),
                ("in_dtype", C.c_int32), ("out_fmt", C.c_int32), ("do_norm", C.c_int32),
                ("rms_eps", C.c_float), ("rope_theta", C.c_double),
                ("kv_a", _vp), ("gate_a", _vp), ("kv_b", _vp), ("gate_b", _vp),
                ("in_row_stride", C.c_int64), ("in_seq_stride", C.c_int64),
                ("bias_a", _vp), ("bias_b", _vp), ("out0", _vp), ("out1", _vp),
                ("out_row0", C.c_int64), ("out0_stride", C.c_int64), ("out0_seq_stride", C.c_int64),
                ("out1_stride", C.c_int64), ("out1_seq_stride", C.c_int64),
                ("in_ring", C.c_int32), ("out_block_rows", C.c_int32), ("out_block_table", _vp),
                ("out_bt_stride", C.c_int64), ("out_pool_blocks", C.c_int32), ("out_ring", C.c_int32),
                ("seq_pos", _vp)]


class IndexArgs(C.Structure):
    _fields_ = [("B", C.c_int32), ("n_q", C.c_int32), ("m", C.c_int32), ("n_cap", C.c_int32),
                ("H_I", C.c_int32), ("d_I", C.c_int32), ("fmt", C.c_int32), ("top_k", C.c_int32),
                ("flags", C.c_int32), ("_pad0", C.c_int32), ("q_pos", _vp), ("n_entries", _vp), ("q0", _vp), ("q1", _vp), ("w", _vp),
                ("k0", _vp), ("k1", _vp), ("out_idx", _vp), ("out_score", _vp),
                ("ev_start", _vp), ("ev_stop", _vp),
                ("block_table", _vp), ("bt_stride", C.c_int32), ("block_rows", C.c_int32),
                ("pool_blocks", C.c_int32), ("_pad1", C.c_int32)]


class AttendArgs(C.Structure):
    _fields_ = [("B", C.c_int32), ("n_q", C.c_int32), ("H", C.c_int32), ("d", C.c_int32),
                ("d_rope", C.c_int32), ("m", C.c_int32), ("fmt", C.c_int32), ("flags", C.c_int32),
                ("rope_theta", C.c_double), ("softmax_scale", C.c_float), ("top_k", C.c_int32),
                ("n_cap", C.c_int32), ("n_win", C.c_int32), ("win_len", C.c_int32), ("_pad0", C.c_int32),
                ("q_pos", _vp), ("q", _vp), ("kv0", _vp), ("kv1", _vp),
                ("kv_stride", C.c_int64), ("kv_seq_stride", C.c_int64),
                ("n_entries", _vp), ("idx", _vp), ("win0", _vp), ("win1", _vp),
                ("win_stride", C.c_int64), ("win_seq_stride", C.c_int64),
                ("win_pos0", _vp), ("sink", _vp), ("out", _vp), ("out_lse", _vp),
                ("ev_start", _vp), ("ev_stop", _vp),
                ("block_table", _vp), ("bt_stride", C.c_int32), ("block_rows", C.c_int32),
                ("pool_blocks", C.c_int32), ("_pad1", C.c_int32)]


_lib = None


def load(path: str = LIB_PATH):
    """Load the library (once) and check the ABI and struct layouts."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with long_context_attention_09_amd.build")
    lib = C.CDLL(path)
    lib.csa_abi_version.restype = C.c_int
    lib.csa_strerror.restype = C.c_char_p
    lib.csa_strerror.argtypes = [C.c_int]
    lib.csa_args_size.restype = C.c_size_t
    lib.csa_args_size.argtypes = [C.c_int]
    lib.csa_workspace_bytes.restype = C.c_size_t
    lib.csa_workspace_bytes.argtypes = [C.c_int, _vp]
    lib.csa_compress.argtypes = [C.POINTER(CompressArgs), _vp]
    lib.csa_compress_batch.argtypes = [C.POINTER(CompressArgs), C.c_int, _vp]
    lib.csa_compress_workspace_bytes.restype = C.c_size_t
    lib.csa_compress_workspace_bytes.argtypes = [C.POINTER(CompressArgs), C.c_int]
    lib.csa_compress_batch_ws.argtypes = [C.POINTER(CompressArgs), C.c_int, _vp, C.c_size_t, _vp]
    lib.csa_index_topk.argtypes = [C.POINTER(IndexArgs), _vp, C.c_size_t, _vp]
    lib.csa_index_topk_noalloc.argtypes = [C.POINTER(IndexArgs), _vp]
    lib.csa_index_topk_noalloc.restype = C.c_int
    lib.csa_index_query_block.argtypes = [C.POINTER(IndexArgs)]
    lib.csa_index_query_block.restype = C.c_int
    lib.csa_attend.argtypes = [C.POINTER(AttendArgs), _vp, C.c_size_t, _vp]
    lib.hca_attend.argtypes = [C.POINTER(AttendArgs), _vp, C.c_size_t, _vp]
    for fn in ("csa_compress", "csa_compress_batch", "csa_compress_batch_ws", "csa_index_topk", "csa_attend",
               "hca_attend"):
        getattr(lib, fn).restype = C.c_int
    if lib.csa_abi_version() != ABI_VERSION:
        raise RuntimeError("libcsa.so ABI version mismatch")
    for op, st in ((OP_COMPRESS, CompressArgs), (OP_INDEX_TOPK, IndexArgs), (OP_ATTEND, AttendArgs)):
        if lib.csa_args_size(op) != C.sizeof(st):
            raise RuntimeError(f"argument struct layout mismatch for op {op}")
    _lib = lib
    return lib


class CsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({load().csa_strerror(status).decode()})")


def _check(status: int, where: str):
    if status != CSA_OK:
        raise CsaError(status, where)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _on_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("every tensor must live on the GPU")


def _bytes_stride(t, dim):
    return t.stride(dim) * t.element_size()


def _block_table(bt, B):
    """(pointer, per-sequence stride) of an int32 [B, max_blocks] block table."""
    if bt is None:
        return None, 0
    _on_gpu(bt)
    if bt.dtype != torch.int32 or bt.dim() != 2 or bt.shape[0] != B or not bt.is_contiguous():
        raise ValueError("block_table must be a contiguous int32 [B, max_blocks] tensor")
    return _ptr(bt), bt.shape[1]


def workspace_bytes(op: int, args) -> int:
    n = load().csa_workspace_bytes(op, C.cast(C.pointer(args), C.c_void_p))
    if n == (1 << 64) - 1:
        raise CsaError(CSA_EINVAL, "csa_workspace_bytes")
    return n


def _workspace(op, args, ws):
    need = workspace_bytes(op, args)
    if need == 0:
        return None, 0
    if ws is None or ws.numel() < need:
        # zero-filled once: the ops keep their counters zeroed from call to call
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    return ws, ws.numel()


# ---------------------------------------------------------------- compress


def compress_args(kv_a, *, m, pos0, out0, out1=None, gate_a=None, bias_a=None, kv_b=None,
                  gate_b=None, bias_b=None, d_rope=0, rope_theta=160000.0, do_norm=True,
                  rms_eps=1e-6, out_fmt=FMT_FP8_BF16, out_row0=0, in_ring=0, n_rows=None,
                  block_table=None, out_ring=0, seq_pos=None):
    """CompressArgs over inputs [B, n_rows, d] (fp32 or bf16, last dim contiguous).

    out0/out1 are [B, n_cap, ...] tensors whose row i - out_row0 receives pooled
    entry i (see include/csa.h for the formats).  State cache: in_ring > 0 makes
    the inputs rings [B, in_ring, d] holding positions pos0 .. pos0 + n_rows - 1
    at rows p % in_ring.  Paged outputs: with block_table (int32 [B, max_blocks])
    out0/out1 are pools [n_blocks, rows_per_block, ...]; out_ring > 0 stores entry i
    at row i % out_ring.  seq_pos (int64 [B]): per-sequence decode mode, the entry
    that token seq_pos[b] completes (pos0 / n_rows ignored)."""
    _on_gpu(kv_a, gate_a, kv_b, gate_b, bias_a, bias_b, out0, out1, seq_pos)
    if seq_pos is not None and (seq_pos.dtype != torch.int64 or not seq_pos.is_contiguous()):
        raise ValueError("seq_pos must be contiguous int64 [B]")
    if kv_a.dim() != 3 or kv_a.stride(2) != 1:
        raise ValueError("kv_a must be [B, n_rows, d] with a contiguous last dim")
    dt = {torch.float32: DT_F32, torch.bfloat16: DT_BF16}[kv_a.dtype]
    for t in (gate_a, kv_b, gate_b):
        if t is not None and (t.shape != kv_a.shape or t.dtype != kv_a.dtype or t.stride() != kv_a.stride()):
            raise ValueError("kv/gate inputs must share shape, dtype and strides")
    for t in (bias_a, bias_b):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("biases are contiguous fp32 [m, d]")
    B, rows, d = kv_a.shape
    if in_ring and rows != in_ring:
        raise ValueError("ring inputs must be [B, in_ring, d]")
    n_rows = rows if n_rows is None else n_rows
    bt, bt_stride = _block_table(block_table, B)
    return CompressArgs(B=B, n_rows=n_rows, pos0=pos0, m=m, overlap=1 if kv_b is not None else 0, d=d,
                        d_rope=d_rope, in_dtype=dt, out_fmt=out_fmt, do_norm=1 if do_norm else 0,
                        rms_eps=rms_eps, rope_theta=rope_theta,
                        kv_a=_ptr(kv_a), gate_a=_ptr(gate_a), kv_b=_ptr(kv_b), gate_b=_ptr(gate_b),
                        in_row_stride=_bytes_stride(kv_a, 1), in_seq_stride=_bytes_stride(kv_a, 0),
                        bias_a=_ptr(bias_a), bias_b=_ptr(bias_b), out0=_ptr(out0), out1=_ptr(out1),
                        out_row0=out_row0, out0_stride=_bytes_stride(out0, 1),
                        out0_seq_stride=_bytes_stride(out0, 0),
                        out1_stride=_bytes_stride(out1, 1) if out1 is not None else 0,
                        out1_seq_stride=_bytes_stride(out1, 0) if out1 is not None else 0,
                        in_ring=in_ring, out_block_rows=out0.shape[1] if bt is not None else 0,
                        out_block_table=bt, out_bt_stride=bt_stride,
                        out_pool_blocks=out0.shape[0] if bt is not None else 0, out_ring=out_ring,
                        seq_pos=_ptr(seq_pos))


def compress(kv_a, **kw):
    """csa_compress (arguments as compress_args)."""
    a = compress_args(kv_a, **kw)
    _check(load().csa_compress(C.byref(a), _stream()), "csa_compress")


def compress_batch(jobs, workspace=True):
    """Compress a list of CompressArgs in one call: csa_compress_batch_ws with a
    workspace of csa_compress_workspace_bytes (workspace=True: a fresh torch
    buffer; a uint8 CUDA tensor: that buffer), or csa_compress_batch
    (workspace=None: every long block pooled by one workgroup)."""
    arr = (CompressArgs * len(jobs))(*jobs)
    lib = load()
    if workspace is None:
        _check(lib.csa_compress_batch(arr, len(jobs), _stream()), "csa_compress_batch")
        return
    n = lib.csa_compress_workspace_bytes(arr, len(jobs))
    if n == C.c_size_t(-1).value:
        raise ValueError("csa_compress_workspace_bytes: invalid job")
    if workspace is True:
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda") if n else None
    else:
        ws = workspace
        if n and (ws.numel() < n or ws.device.type != "cuda"):
            raise ValueError(f"compress workspace needs {n} device bytes")
    _check(lib.csa_compress_batch_ws(arr, len(jobs), _ptr(ws), n if ws is None else ws.numel(), _stream()),
           "csa_compress_batch_ws")


def compress_workspace_bytes(jobs):
    """csa_compress_workspace_bytes of a list of CompressArgs."""
    arr = (CompressArgs * len(jobs))(*jobs)
    return load().csa_compress_workspace_bytes(arr, len(jobs))


# ---------------------------------------------------------------- index + top-k


def index_args(q0, w, k0, q_pos, *, m, top_k, out_idx, q1=None, k1=None, n_entries=None,
               out_score=None, fmt=FMT_MXFP4, flags=0, block_table=None):
    """Fill IndexArgs.  MXFP4: q0 [B, n_q, H_I, d_I/2] u8, q1 [B, n_q, H_I, d_I/32] u8,
    k0 [B, n_cap, d_I/2] u8, k1 [B, n_cap, d_I/32] u8.  F32: q0 [B, n_q, H_I, d_I],
    k0 [B, n_cap, d_I].  w [B, n_q, H_I] fp32, q_pos [B, n_q] int64, out_idx
    [B, n_q, top_k] int32.  Paged keys: with block_table (int32 [B, max_blocks]) k0 and
    k1 are pools [n_blocks, keys_per_block, ...] and n_cap = max_blocks * keys_per_block."""
    _on_gpu(q0, q1, w, k0, k1, q_pos, n_entries, out_idx, out_score)
    for t in (q0, q1, w, k0, k1, q_pos, n_entries, out_idx, out_score):
        if t is not None and not t.is_contiguous():
            raise ValueError("index_topk tensors must be contiguous")
    B, n_q, H_I = w.shape
    bt, bt_stride = _block_table(block_table, B)
    n_cap = k0.shape[1] * (bt_stride if bt is not None else 1)
    d_I = q0.shape[-1] * (2 if fmt == FMT_MXFP4 else 1)
    if q_pos.dtype != torch.int64 or out_idx.dtype != torch.int32 or w.dtype != torch.float32:
        raise ValueError("q_pos int64, out_idx int32, w fp32")
    if tuple(out_idx.shape) != (B, n_q, top_k) or tuple(q_pos.shape) != (B, n_q):
        raise ValueError("out_idx must be [B, n_q, top_k] and q_pos [B, n_q]")
    if out_score is not None and tuple(out_score.shape) != (B, n_q, n_cap):
        raise ValueError("out_score must be [B, n_q, n_cap]")
    want = torch.bfloat16 if flags & INDEX_BF16_SCORES else torch.float32
    if out_score is not None and out_score.dtype != want:
        raise ValueError(f"out_score must be {want} with these flags")
    return IndexArgs(B=B, n_q=n_q, m=m, n_cap=n_cap, H_I=H_I, d_I=d_I, fmt=fmt, top_k=top_k,
                     flags=flags, _pad0=0, q_pos=_ptr(q_pos), n_entries=_ptr(n_entries), q0=_ptr(q0), q1=_ptr(q1),
                     w=_ptr(w), k0=_ptr(k0), k1=_ptr(k1), out_idx=_ptr(out_idx),
                     out_score=_ptr(out_score), block_table=bt, bt_stride=bt_stride,
                     block_rows=k0.shape[1] if bt is not None else 0,
                     pool_blocks=k0.shape[0] if bt is not None else 0, _pad1=0)


def index_query_block(*args, **kw):
    """csa_index_query_block: queries per sequence in each internal block of a
    csa_index_topk call with these arguments."""
    n = load().csa_index_query_block(C.byref(index_args(*args, **kw)))
    if n < 1:
        raise CsaError(n if n < 0 else CSA_EWORKSPACE, "csa_index_query_block")
    return n


def index_topk(*args, workspace=None, **kw):
    a = index_args(*args, **kw)
    ws, n = _workspace(OP_INDEX_TOPK, a, workspace)
    _check(load().csa_index_topk(C.byref(a), _ptr(ws), n, _stream()), "csa_index_topk")
    return ws


def index_topk_noalloc(*args, **kw):
    """csa_index_topk_noalloc: the same selection through the library's
    per-GPU scratch array (no workspace, no allocation)."""
    a = index_args(*args, **kw)
    _check(load().csa_index_topk_noalloc(C.byref(a), _stream()), "csa_index_topk_noalloc")


# ---------------------------------------------------------------- attention


def attend_args(q, q_pos, kv0, win0, win_pos0, sink, out, *, m, n_win, kv1=None, win1=None,
                idx=None, n_entries=None, out_lse=None, d_rope=64, rope_theta=160000.0,
                softmax_scale=0.0, flags=ATTEND_NORM_Q, fmt=FMT_FP8_BF16, top_k=None,
                block_table=None):
    """Fill AttendArgs.  q/out [B, n_q, H, d]; kv0/kv1 [B, n_cap, row] (row bytes
    with a 2-D byte stride); win0/win1 [B, win_len, row]; idx [B, n_q, top_k].
    Paged entries: with block_table (int32 [B, max_blocks]) kv0/kv1 are pools
    [n_blocks, entries_per_block, row] and n_cap = max_blocks * entries_per_block.
    A window ring (the state cache) takes flags | ATTEND_WIN_RING."""
    _on_gpu(q, q_pos, kv0, kv1, win0, win1, win_pos0, sink, out, idx, n_entries, out_lse)
    for t in (q, out, q_pos, win_pos0, sink, idx, n_entries, out_lse):
        if t is not None and not t.is_contiguous():
            raise ValueError("q, out, positions, sink, idx and lse must be contiguous")
    B, n_q, H, d = q.shape
    if tuple(out.shape) != (B, n_q, H, d) or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if q_pos.dtype != torch.int64 or (win_pos0 is not None and win_pos0.dtype != torch.int64) \
            or sink.dtype != torch.float32:
        raise ValueError("q_pos / win_pos0 int64, sink fp32")
    want = torch.float32 if fmt == FMT_F32 else torch.bfloat16
    if q.dtype != want:
        raise ValueError(f"q must be {want} for this format")
    if idx is not None and (idx.dtype != torch.int32 or idx.shape[:2] != (B, n_q)):
        raise ValueError("idx must be int32 [B, n_q, top_k]")
    bt, bt_stride = _block_table(block_table, B)
    return AttendArgs(B=B, n_q=n_q, H=H, d=d, d_rope=d_rope, m=m, fmt=fmt, flags=flags,
                      rope_theta=rope_theta, softmax_scale=softmax_scale,
                      top_k=idx.shape[2] if idx is not None else 0,
                      n_cap=kv0.shape[1] * (bt_stride if bt is not None else 1), n_win=n_win,
                      win_len=win0.shape[1], _pad0=0,
                      q_pos=_ptr(q_pos), q=_ptr(q), kv0=_ptr(kv0), kv1=_ptr(kv1),
                      kv_stride=_bytes_stride(kv0, 1), kv_seq_stride=_bytes_stride(kv0, 0),
                      n_entries=_ptr(n_entries), idx=_ptr(idx), win0=_ptr(win0), win1=_ptr(win1),
                      win_stride=_bytes_stride(win0, 1), win_seq_stride=_bytes_stride(win0, 0),
                      win_pos0=_ptr(win_pos0), sink=_ptr(sink), out=_ptr(out), out_lse=_ptr(out_lse),
                      block_table=bt, bt_stride=bt_stride, block_rows=kv0.shape[1] if bt is not None else 0,
                      pool_blocks=kv0.shape[0] if bt is not None else 0, _pad1=0)


def attend(*args, workspace=None, **kw):
    a = attend_args(*args, **kw)
    ws, n = _workspace(OP_ATTEND, a, workspace)
    _check(load().csa_attend(C.byref(a), _ptr(ws), n, _stream()), "csa_attend")
    return ws


def hca_attend(*args, workspace=None, **kw):
    if kw.get("idx") is not None:
        raise ValueError("hca_attend takes no index list")
    a = attend_args(*args, **kw)
    ws, n = _workspace(OP_HCA_ATTEND, a, workspace)
    _check(load().hca_attend(C.byref(a), _ptr(ws), n, _stream()), "hca_attend")
    return ws


def split_main(cache):
    """A packed [.., n, 576] byte cache as (nope view, rope view) for the C ABI:
    the E4M3FN bytes at offset 0 and the BF16 dims at offset 448, same strides."""
    return cache[..., :448], cache[..., 448:]
