"""ctypes binding of ``libdfv.so`` (C ABI in ``include/dfv.h``).

Argument marshalling only: every step of the attention runs in the HIP
library.  torch tensors supply device memory and the current stream.  If the
library has not been built, :func:`lib` raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdfv.so")

DFV_OK = 0
STATUS = {0: "DFV_OK", -1: "DFV_ERR_NULL", -2: "DFV_ERR_UNSUPPORTED", -3: "DFV_ERR_ALIGN",
          -4: "DFV_ERR_ARG", -5: "DFV_ERR_LAUNCH", -7: "DFV_ERR_SCRATCH"}
ENTRY_POINTS = ("dfv_status_string", "dfv_attn_check", "dfv_attn_scratch_bytes", "dfv_attn_workspace_bytes",
                "dfv_attn_chunks", "dfv_attn_split_chunks", "dfv_attn_combine_chunks", "dfv_attn_split",
                "dfv_attn_combine", "dfv_attn", "dfv_attn_noalloc", "dfv_qk_scores", "dfv_kv_append")


class DfvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


class Desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("num_splits", ctypes.c_int32), ("split_tokens", ctypes.c_int32),
                ("max_context_len", ctypes.c_int32), ("softmax_scale", ctypes.c_float)]


_LIB = None
_P = ctypes.c_void_p


def lib():
    """Load the library (once).  Raises FileNotFoundError if it was never built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(f"{LIB_PATH} is missing: build it with "
                                    "`python -m long_context_split_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.dfv_status_string.argtypes = [ctypes.c_int]
        L.dfv_status_string.restype = ctypes.c_char_p
        L.dfv_attn_check.argtypes = [ctypes.POINTER(Desc)]
        L.dfv_attn_check.restype = ctypes.c_int
        L.dfv_attn_scratch_bytes.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(ctypes.c_size_t)]
        L.dfv_attn_scratch_bytes.restype = ctypes.c_int
        L.dfv_attn_workspace_bytes.argtypes = [ctypes.POINTER(Desc)]
        L.dfv_attn_workspace_bytes.restype = ctypes.c_size_t
        L.dfv_attn_combine_chunks.argtypes = [ctypes.POINTER(Desc)] + [_P] * 7 + [_P]
        L.dfv_attn_combine_chunks.restype = ctypes.c_int
        L.dfv_attn_chunks.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(ctypes.c_int32)]
        L.dfv_attn_chunks.restype = ctypes.c_int
        L.dfv_attn_split_chunks.argtypes = [ctypes.POINTER(Desc)] + [_P] * 10 + [_P]
        L.dfv_attn_split_chunks.restype = ctypes.c_int
        L.dfv_attn_split.argtypes = [ctypes.POINTER(Desc)] + [_P] * 10 + [_P, ctypes.c_size_t, _P]
        L.dfv_attn_split.restype = ctypes.c_int
        L.dfv_attn_combine.argtypes = [ctypes.POINTER(Desc), _P, _P, _P, _P, _P]
        L.dfv_attn_combine.restype = ctypes.c_int
        L.dfv_attn.argtypes = [ctypes.POINTER(Desc)] + [_P] * 10 + [_P, ctypes.c_size_t, _P, _P]
        L.dfv_attn.restype = ctypes.c_int
        L.dfv_attn_noalloc.argtypes = [ctypes.POINTER(Desc)] + [_P] * 10 + [_P, _P]
        L.dfv_attn_noalloc.restype = ctypes.c_int
        L.dfv_qk_scores.argtypes = [ctypes.POINTER(Desc)] + [_P] * 6 + [ctypes.c_int64, _P]
        L.dfv_qk_scores.restype = ctypes.c_int
        L.dfv_kv_append.argtypes = [_P, _P, _P, ctypes.c_int32, _P, _P, _P, _P, ctypes.c_int64, _P]
        L.dfv_kv_append.restype = ctypes.c_int
        _LIB = L
    return _LIB


def make_desc(batch: int, num_q: int, max_blocks: int, max_context_len: int, *, num_splits: int = 80,
              split_tokens: int = 0, softmax_scale: float = 1.0 / 16.0, num_q_heads: int = 6,
              num_kv_heads: int = 1, head_dim: int = 256, block_size: int = 16) -> Desc:
    return Desc(batch, num_q, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks, num_splits,
                split_tokens, max_context_len, softmax_scale)


def check(desc: Desc) -> int:
    return lib().dfv_attn_check(ctypes.byref(desc))


def scratch_bytes(desc: Desc) -> int:
    n = ctypes.c_size_t(0)
    _raise(lib().dfv_attn_scratch_bytes(ctypes.byref(desc), ctypes.byref(n)), "dfv_attn_scratch_bytes")
    return int(n.value)


def workspace_bytes(desc: Desc) -> int:
    """dfv_attn_workspace_bytes: workspace (max, sum, numerator) plus scratch bytes; 0 if not admitted."""
    return int(lib().dfv_attn_workspace_bytes(ctypes.byref(desc)))


def chunks(desc: Desc) -> int:
    n = ctypes.c_int32(0)
    _raise(lib().dfv_attn_chunks(ctypes.byref(desc), ctypes.byref(n)), "dfv_attn_chunks")
    return int(n.value)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _raise(status: int, where: str):
    if status != DFV_OK:
        raise DfvError(status, where)


@dataclass
class Workspace:
    """Caller-owned outputs and scratch for one descriptor (torch device tensors)."""
    ws_max: object
    ws_sum: object
    ws_num: object
    scratch: object
    out: object

    @staticmethod
    def allocate(desc: Desc, device="cuda"):
        import torch
        rows = (desc.batch, desc.num_q, desc.num_q_heads)
        nbytes = scratch_bytes(desc)
        return Workspace(
            ws_max=torch.empty(*rows, desc.num_splits, dtype=torch.float32, device=device),
            ws_sum=torch.empty(*rows, desc.num_splits, dtype=torch.float32, device=device),
            ws_num=torch.empty(*rows, desc.num_splits, desc.head_dim, dtype=torch.float32, device=device),
            scratch=torch.empty(nbytes, dtype=torch.uint8, device=device) if nbytes else None,
            out=torch.empty(*rows, desc.head_dim, dtype=torch.float16, device=device))


def attn_split(desc: Desc, q, k_cache, v_cache, block_table, context_lens, k_scale, v_scale,
               ws_max, ws_sum, ws_num, scratch, stream=None):
    st = lib().dfv_attn_split(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                              _ptr(context_lens), _ptr(k_scale), _ptr(v_scale), _ptr(ws_max), _ptr(ws_sum),
                              _ptr(ws_num), _ptr(scratch),
                              0 if scratch is None else scratch.numel() * scratch.element_size(),
                              _stream(stream))
    _raise(st, "dfv_attn_split")


def attn_split_chunks(desc: Desc, q, k_cache, v_cache, block_table, context_lens, k_scale, v_scale,
                      chunk_max, chunk_sum, chunk_num, stream=None):
    st = lib().dfv_attn_split_chunks(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(block_table), _ptr(context_lens), _ptr(k_scale), _ptr(v_scale),
                                     _ptr(chunk_max), _ptr(chunk_sum), _ptr(chunk_num), _stream(stream))
    _raise(st, "dfv_attn_split_chunks")


def chunk_buffers(desc: Desc, device="cuda"):
    """(chunk_max, chunk_sum, chunk_num) torch tensors for dfv_attn_split_chunks."""
    import torch
    c = chunks(desc)
    rows = (desc.batch, desc.num_q, desc.num_q_heads, desc.num_splits, c)
    return (torch.empty(*rows, dtype=torch.float32, device=device),
            torch.empty(*rows, dtype=torch.float32, device=device),
            torch.empty(*rows, desc.head_dim, dtype=torch.float32, device=device))


def attn_combine_chunks(desc: Desc, chunk_max, chunk_sum, chunk_num, ws_max, ws_sum, ws_num, out,
                        stream=None):
    """dfv_attn_combine_chunks: chunk states -> workspace (and the FP16 output unless out is None)."""
    st = lib().dfv_attn_combine_chunks(ctypes.byref(desc), _ptr(chunk_max), _ptr(chunk_sum), _ptr(chunk_num),
                                       _ptr(ws_max), _ptr(ws_sum), _ptr(ws_num), _ptr(out), _stream(stream))
    _raise(st, "dfv_attn_combine_chunks")


def attn_combine(desc: Desc, ws_max, ws_sum, ws_num, out, stream=None):
    st = lib().dfv_attn_combine(ctypes.byref(desc), _ptr(ws_max), _ptr(ws_sum), _ptr(ws_num), _ptr(out),
                                _stream(stream))
    _raise(st, "dfv_attn_combine")


def attn(desc: Desc, q, k_cache, v_cache, block_table, context_lens, k_scale, v_scale,
         ws_max, ws_sum, ws_num, scratch, out, stream=None):
    st = lib().dfv_attn(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                        _ptr(context_lens), _ptr(k_scale), _ptr(v_scale), _ptr(ws_max), _ptr(ws_sum),
                        _ptr(ws_num), _ptr(scratch),
                        0 if scratch is None else scratch.numel() * scratch.element_size(),
                        _ptr(out), _stream(stream))
    _raise(st, "dfv_attn")


def attn_noalloc(desc: Desc, q, k_cache, v_cache, block_table, context_lens, k_scale, v_scale,
                 ws_max, ws_sum, ws_num, out, stream=None):
    """dfv_attn_noalloc: dfv_attn with the library's static scratch (allocates nothing)."""
    st = lib().dfv_attn_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                _ptr(context_lens), _ptr(k_scale), _ptr(v_scale), _ptr(ws_max), _ptr(ws_sum),
                                _ptr(ws_num), _ptr(out), _stream(stream))
    _raise(st, "dfv_attn_noalloc")


def qk_tiles(desc: Desc) -> int:
    """Smallest admitted tile capacity of the QK-stage scores: ceil(max_context_len / 32)."""
    return -(-desc.max_context_len // 32)


def qk_scores(desc: Desc, q, k_cache, block_table, context_lens, k_scale, scores, tiles_per_seq: int,
              stream=None):
    """dfv_qk_scores: FP32 scores, tile-major [B][tiles_per_seq][6q][32]; guard tiles untouched."""
    st = lib().dfv_qk_scores(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(block_table),
                             _ptr(context_lens), _ptr(k_scale), _ptr(scores), int(tiles_per_seq),
                             _stream(stream))
    _raise(st, "dfv_qk_scores")


def kv_append(k_new, v_new, slot_mapping, k_scale, v_scale, k_cache, v_cache, stream=None):
    """dfv_kv_append: quantize new FP16 K/V rows to E4M3 and write them by slot (int64 slots)."""
    st = lib().dfv_kv_append(_ptr(k_new), _ptr(v_new), _ptr(slot_mapping), int(slot_mapping.numel()),
                             _ptr(k_scale), _ptr(v_scale), _ptr(k_cache), _ptr(v_cache),
                             int(k_cache.shape[0]), _stream(stream))
    _raise(st, "dfv_kv_append")


def run_layer(inp, ws: Workspace, desc: Desc, stream=None):
    """dfv_attn on a ``synth.LayerInputs``; returns the workspace (outputs filled)."""
    attn(desc, inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.context_lens, inp.k_scale,
         inp.v_scale, ws.ws_max, ws.ws_sum, ws.ws_num, ws.scratch, ws.out, stream)
    return ws


def desc_for(inp, *, num_splits: int = 80, split_tokens: int = 0) -> Desc:
    """Descriptor matching a ``synth.LayerInputs``."""
    B, nq, hq, d = inp.q.shape
    lens = [int(x) for x in inp.context_lens.cpu().tolist()]
    return make_desc(B, nq, inp.block_table.shape[1], max(lens), num_splits=num_splits,
                     split_tokens=split_tokens, softmax_scale=inp.softmax_scale, num_q_heads=hq,
                     head_dim=d)
