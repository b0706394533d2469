"""Python binding of libdsa.so: argument marshalling only.

Each function has the name of the C entry point it calls (see include/dsa.h)
and takes torch tensors that already live on the GPU.  Every step of the path
runs in the library's HIP kernels; there is no fallback of any kind: if
libdsa.so is missing or fails to load, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_OK = 0
STATUS_NAMES = {0: "DSA_OK", 1: "DSA_ERR_NULL", 2: "DSA_ERR_SHAPE", 3: "DSA_ERR_UNSUPPORTED",
                4: "DSA_ERR_WORKSPACE", 5: "DSA_ERR_HIP", 6: "DSA_ERR_ALIGN"}
DSA_F32, DSA_BF16, DSA_FP8_E4M3_B128, DSA_INT8_AFFINE_B128 = 0, 1, 2, 3
DSA_BF16_TO_FP8 = 4  # indexer queries: bf16 in memory, contracted as fp8 (fp8 keys)

ENTRY_POINTS = ("dsa_version", "dsa_status_string", "dsa_indexer_prepare", "dsa_index_scores",
                "dsa_index_topk", "dsa_index_topk_workspace_bytes", "dsa_topk_workspace_bytes",
                "dsa_topk", "dsa_sparse_mla_workspace_bytes", "dsa_sparse_mla_decode",
                "dsa_sparse_mla_decode_static", "dsa_sparse_mla_prefill")
DSA_MLA_SCRATCH_BYTES = 64 << 20


class DSAError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__("%s returned %s (%s)" % (fn, STATUS_NAMES.get(status, status),
                                                  status_string(status)))


class dsa_batch(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_rows", ctypes.c_int32),
                ("max_q_len", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("cu_q_lens", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p), ("pt_stride", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32)]


class dsa_pool(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("format", ctypes.c_int32), ("dim", ctypes.c_int32),
                ("page_stride_bytes", ctypes.c_int64), ("row_stride_bytes", ctypes.c_int64)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libdsa.so not found at %s: build it with __graft_entry__.build() "
                          "(hipcc, gfx950) before using the DSA path" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    bp, pp = ctypes.POINTER(dsa_batch), ctypes.POINTER(dsa_pool)
    lib.dsa_version.restype = i32
    lib.dsa_status_string.argtypes = [i32]
    lib.dsa_status_string.restype = ctypes.c_char_p
    lib.dsa_index_scores.argtypes = [bp, vp, i32, vp, pp, i32, i32, vp, i64, vp]
    lib.dsa_indexer_prepare.argtypes = [bp, vp, vp, vp, i32, vp, vp, ctypes.c_float, vp, vp, i32, i32,
                                        i32, pp, i32, i32, vp]
    lib.dsa_indexer_prepare.restype = i32
    lib.dsa_index_topk.argtypes = [bp, vp, i32, vp, pp, i32, i32, i32, vp, vp, sz, vp]
    lib.dsa_index_topk.restype = i32
    lib.dsa_index_topk_workspace_bytes.argtypes = [i32, i32, i32, i64]
    lib.dsa_index_topk_workspace_bytes.restype = sz
    lib.dsa_topk_workspace_bytes.argtypes = [i32, i32, i32]
    lib.dsa_topk_workspace_bytes.restype = sz
    lib.dsa_topk.argtypes = [bp, vp, i64, i32, vp, vp, sz, vp]
    lib.dsa_sparse_mla_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.dsa_sparse_mla_workspace_bytes.restype = sz
    mla = [bp, vp, i32, pp, vp, i32, i32, i32, i32, ctypes.c_float, vp, vp, vp, sz, vp]
    lib.dsa_sparse_mla_decode.argtypes = mla
    lib.dsa_sparse_mla_prefill.argtypes = mla
    lib.dsa_sparse_mla_decode_static.argtypes = mla[:12] + [vp]
    for f in (lib.dsa_index_scores, lib.dsa_topk, lib.dsa_sparse_mla_decode, lib.dsa_sparse_mla_prefill,
              lib.dsa_sparse_mla_decode_static):
        f.restype = i32
    return lib


_lib = _load()


def lib():
    return _lib


def status_string(status: int) -> str:
    return _lib.dsa_status_string(status).decode()


def dsa_version() -> int:
    return _lib.dsa_version()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(stream)


def _check(fn, st):
    if st != DSA_OK:
        raise DSAError(fn, st)


def make_batch(cu_q_lens, seq_lens, page_table, num_q_rows, max_q_len, max_seq_len, page_size,
               num_pages) -> dsa_batch:
    """dsa_batch from device int32 tensors plus the host bounds."""
    b = dsa_batch(cu_q_lens.numel() - 1, num_q_rows, max_q_len, max_seq_len, cu_q_lens.data_ptr(),
                  seq_lens.data_ptr(), page_table.data_ptr(), page_table.shape[1], page_size,
                  num_pages)
    b._keep = (cu_q_lens, seq_lens, page_table)
    return b


def make_pool(pool: torch.Tensor, fmt: int, dim: int) -> dsa_pool:
    """dsa_pool viewing a [num_pages, page_size, row] tensor in place."""
    es = pool.element_size()
    p = dsa_pool(pool.data_ptr(), fmt, dim, pool.stride(0) * es, pool.stride(1) * es)
    p._keep = pool
    return p


def make_key_pool(sb) -> dsa_pool:
    """dsa_pool of a synth.Batch's indexer keys: [num_pages, P, di] in idx_fmt,
    or page-blocked fp8 pages ([num_pages, page_bytes]: P rows of 128 codes,
    then P f32 scales, page_bytes >= P*132 and a multiple of 16)."""
    cfg = sb.cfg
    if cfg.key_fmt == DSA_FP8_E4M3_B128:
        pool = sb.k_pool
        p = dsa_pool(pool.data_ptr(), DSA_FP8_E4M3_B128, cfg.di, pool.stride(0), 128)
        p._keep = pool
        return p
    return make_pool(sb.k_pool, cfg.idx_fmt, cfg.di)


def batch_from(sb) -> dsa_batch:
    """dsa_batch of a synth.Batch whose tensors are on the GPU."""
    return make_batch(sb.cu_q, sb.seq_lens_t, sb.page_table, sb.T, sb.max_q_len, sb.max_seq_len,
                      sb.cfg.page_size, sb.num_pages)


def dsa_index_scores(batch, q_idx, q_format, w, k_pool: dsa_pool, n_heads, head_dim, scores, ld,
                     stream=None):
    _check("dsa_index_scores", _lib.dsa_index_scores(
        ctypes.byref(batch), _ptr(q_idx), q_format, _ptr(w), ctypes.byref(k_pool), n_heads,
        head_dim, _ptr(scores), ld, _stream(stream)))


def dsa_indexer_prepare(batch, q_in, q_out, k_in, fmt, ln_weight, ln_bias, ln_eps, rope_cos, rope_sin,
                        rope_rows, rope_dim, rope_interleaved, k_pool: dsa_pool, n_heads, head_dim,
                        stream=None):
    _check("dsa_indexer_prepare", _lib.dsa_indexer_prepare(
        ctypes.byref(batch), _ptr(q_in), _ptr(q_out), _ptr(k_in), fmt, _ptr(ln_weight), _ptr(ln_bias),
        ln_eps, _ptr(rope_cos), _ptr(rope_sin), rope_rows, rope_dim, 1 if rope_interleaved else 0,
        ctypes.byref(k_pool), n_heads, head_dim, _stream(stream)))


def dsa_index_topk_workspace_bytes(num_q_rows, max_seq_len, k, budget_bytes) -> int:
    return _lib.dsa_index_topk_workspace_bytes(num_q_rows, max_seq_len, k, budget_bytes)


def dsa_index_topk(batch, q_idx, q_format, w, k_pool: dsa_pool, n_heads, head_dim, k, idx, ws, ws_bytes,
                   stream=None):
    _check("dsa_index_topk", _lib.dsa_index_topk(
        ctypes.byref(batch), _ptr(q_idx), q_format, _ptr(w), ctypes.byref(k_pool), n_heads, head_dim, k,
        _ptr(idx), _ptr(ws), ws_bytes, _stream(stream)))


def dsa_topk_workspace_bytes(num_q_rows, max_seq_len, k) -> int:
    return _lib.dsa_topk_workspace_bytes(num_q_rows, max_seq_len, k)


def dsa_topk(batch, scores, ld, k, idx, ws=None, ws_bytes=0, stream=None):
    _check("dsa_topk", _lib.dsa_topk(ctypes.byref(batch), _ptr(scores), ld, k, _ptr(idx), _ptr(ws),
                                     ws_bytes, _stream(stream)))


def dsa_sparse_mla_workspace_bytes(num_q_rows, n_heads, k, dc, prefill=False) -> int:
    return _lib.dsa_sparse_mla_workspace_bytes(num_q_rows, n_heads, k, dc, 1 if prefill else 0)


def _mla(fn, batch, q, q_format, kv: dsa_pool, idx, k, n_heads, dc, dr, sm_scale, out, lse, ws,
         ws_bytes, stream):
    _check(fn, getattr(_lib, fn)(ctypes.byref(batch), _ptr(q), q_format, ctypes.byref(kv), _ptr(idx),
                                 k, n_heads, dc, dr, sm_scale, _ptr(out), _ptr(lse), _ptr(ws),
                                 ws_bytes, _stream(stream)))


def dsa_sparse_mla_decode(batch, q, q_format, kv, idx, k, n_heads, dc, dr, sm_scale, out, lse=None,
                          ws=None, ws_bytes=0, stream=None):
    _mla("dsa_sparse_mla_decode", batch, q, q_format, kv, idx, k, n_heads, dc, dr, sm_scale, out,
         lse, ws, ws_bytes, stream)


def dsa_sparse_mla_prefill(batch, q, q_format, kv, idx, k, n_heads, dc, dr, sm_scale, out,
                           lse=None, ws=None, ws_bytes=0, stream=None):
    _mla("dsa_sparse_mla_prefill", batch, q, q_format, kv, idx, k, n_heads, dc, dr, sm_scale, out,
         lse, ws, ws_bytes, stream)


def dsa_sparse_mla_decode_static(batch, q, q_format, kv, idx, k, n_heads, dc, dr, sm_scale, out, lse=None,
                                 stream=None):
    _check("dsa_sparse_mla_decode_static", _lib.dsa_sparse_mla_decode_static(
        ctypes.byref(batch), _ptr(q), q_format, ctypes.byref(kv), _ptr(idx), k, n_heads, dc, dr, sm_scale,
        _ptr(out), _ptr(lse), _stream(stream)))
