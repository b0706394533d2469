"""CPU oracle for the DSA hot path -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package.  The arithmetic lives in ``dsa_oracle.c`` (plain C, double
precision, explicit loops); this module compiles it with gcc, converts the
seeded inputs to float64 (exact for bf16 and f32) and marshals arguments.

For sampled rows of large workloads the inputs are cut down to the requests
that own those rows: their pages are copied into a compact pool under a
re-numbered page table.  That copy moves values only; the oracle still reads
every token through a page table.

Parity status of each function (what pins it; see tests/test_oracle_pins.py):
  index_scores  pinned: closed forms, ReLU/sign/head-pairing cases, causal
                boundary, paging invariance, brute force on tiny inputs
  topk          pinned: hand-derived tie fixtures, identity below K, dominance
                property, numpy lexsort selection, batched == per row
  sparse_mla    pinned: dense invariant below K vs torch SDPA, absorption
                identity, mask equivalence, closed forms (K=1, q=0), re-masking
  e4m3 decode   pinned: all 256 codes against torch.float8_e4m3fn
  e4m3 encode   pinned: round trip of every finite code; every tie, its two
                float32 neighbours and random values against torch's
                float32 -> float8_e4m3fn conversion
  fp8 queries (quantize_q_fp8, index_scores(q_fp8=True)) pinned: the scale
                rule as a property over random and edge magnitudes; a head
                quantised by hand; exact on parity draws; e4m3's rounding
                bound on random queries
  fp8 index keys (page-blocked codes + per-token scales) pinned: a hand-built
                page decoded against values written out by hand
  int8 latent rows (affine codes, per-128 scale and bias) pinned: a hand-built
                row decoded against values written out by hand; sparse_mla over
                int8 rows equals sparse_mla over the decoded rows
  indexer_prepare  pinned: LayerNorm against torch's layer_norm; RoPE against
                complex multiplication by unit phasors (interleaved) and the
                dims permutation that maps one pair layout onto the other;
                a hand-worked rotation; identity at angle 0; norm
                preservation; keys found at their slots through the page table
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

FMT_F32, FMT_BF16, FMT_FP8, FMT_INT8 = 0, 1, 2, 3


def build(force: bool = True) -> str:
    """Compile dsa_oracle.c into liboracle.so next to it (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        i32p = ctypes.POINTER(ctypes.c_int32)
        f64p = ctypes.POINTER(ctypes.c_double)
        c_int, c_i64 = ctypes.c_int, ctypes.c_int64
        lib.oracle_index_scores.argtypes = [c_int, i32p, i32p, i32p, c_int, c_int, c_int,
                                            f64p, f64p, f64p, c_int, c_int, i32p, c_int,
                                            f64p, c_i64]
        lib.oracle_topk.argtypes = [c_int, i32p, i32p, f64p, c_i64, c_int, i32p, c_int, i32p]
        lib.oracle_sparse_mla.argtypes = [c_int, i32p, i32p, i32p, c_int, c_int, c_int,
                                          f64p, c_int, ctypes.c_void_p, i32p, c_int,
                                          c_int, c_int, c_int, ctypes.c_double, i32p, c_int,
                                          f64p, f64p]
        lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_to_double.restype = ctypes.c_double
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_decode_fp8_rows.argtypes = [ctypes.c_void_p, c_i64, c_int, c_int, f64p]
        lib.oracle_decode_int8_rows.argtypes = [ctypes.c_void_p, c_i64, c_int, c_int, f64p]
        lib.oracle_decode_fp8_keys.argtypes = [ctypes.c_void_p, c_i64, c_int, c_int, c_i64, c_i64, f64p]
        i64p = ctypes.POINTER(ctypes.c_int64)
        lib.oracle_indexer_prepare.argtypes = [c_int, i32p, i32p, i32p, c_int, c_int, c_int, c_int,
                                               f64p, f64p, f64p, f64p, ctypes.c_double, f64p, f64p,
                                               c_i64, c_int, c_int, c_int, c_int, f64p, f64p, f64p,
                                               i64p]
        lib.oracle_indexer_prepare.restype = c_int
        for f in (lib.oracle_index_scores, lib.oracle_topk, lib.oracle_sparse_mla):
            f.restype = c_int
        lib.oracle_threads.restype = c_int
        lib.oracle_set_threads.argtypes = [c_int]
        lib.oracle_set_threads.restype = None
        _lib = lib
    return _lib


def _p(a, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


def _i32(x):
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _f64(x):
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


class _View:
    """A batch restricted to the requests that own `rows`, pages compacted."""

    def __init__(self, batch, rows):
        self.batch = batch
        cu = [0]
        for ql in batch.q_lens:
            cu.append(cu[-1] + ql)
        T = cu[-1]
        self.rows = np.arange(T, dtype=np.int32) if rows is None else _i32(rows)
        owners = sorted({int(np.searchsorted(cu, int(t), side="right") - 1) for t in self.rows})
        self.owners = owners
        P = batch.cfg.page_size
        pt_old = batch.page_table.detach().cpu()
        self.pt_stride = pt_old.shape[1]
        pt_new = torch.full_like(pt_old, -1)
        src_pages = []
        for b in owners:
            n = min((batch.seq_lens[b] + P - 1) // P, self.pt_stride)
            ids = pt_old[b, :n]
            pt_new[b, :n] = torch.arange(len(src_pages), len(src_pages) + n, dtype=torch.int32)
            src_pages.extend(ids.tolist())
        self.src_pages = torch.tensor(src_pages, dtype=torch.long)
        self.num_pages = len(src_pages)
        self.page_table = _i32(pt_new)
        self.cu_q = _i32(cu)
        self.seq_lens = _i32(batch.seq_lens)
        self.n = len(self.rows)
        self.rows_t = torch.from_numpy(self.rows.astype(np.int64))

    def pool(self, pool):
        """Compact copy of a [num_pages, P, ...] pool (on any device) to host."""
        idx = self.src_pages.to(pool.device)
        return pool.index_select(0, idx).cpu()

    def per_row(self, x):
        return x.index_select(0, self.rows_t.to(x.device)).cpu()


def index_scores(batch, rows=None, ld=None, q_fp8=False):
    """Scores [n_rows, ld] (float64, NaN beyond each row's pos).

    q_fp8: the queries are first quantised per (row, head) as
    quantize_q_fp8 describes and the formula is applied to the values the
    codes stand for."""
    lib = _load()
    v = _View(batch, rows)
    cfg = batch.cfg
    ld = ld or max(batch.max_seq_len, 1)
    q = _f64(v.per_row(batch.q_idx))
    if q_fp8:
        codes, e = quantize_q_fp8(q)
        q = dequantize_q_fp8(codes, e)
    w = _f64(v.per_row(batch.w))
    if cfg.key_fmt == FMT_FP8:  # page-blocked fp8 keys: decoded to doubles first
        k = decode_fp8_keys(v.pool(batch.k_pool), cfg.page_size, cfg.di)
    else:
        k = _f64(v.pool(batch.k_pool))
    out = np.full((v.n, ld), np.nan, dtype=np.float64)
    st = lib.oracle_index_scores(batch.B, _p(v.cu_q, ctypes.c_int32), _p(v.seq_lens, ctypes.c_int32),
                                 _p(v.page_table, ctypes.c_int32), v.pt_stride, cfg.page_size,
                                 v.num_pages, _p(q, ctypes.c_double), _p(w, ctypes.c_double),
                                 _p(k, ctypes.c_double), cfg.hi, cfg.di,
                                 _p(v.rows, ctypes.c_int32), v.n, _p(out, ctypes.c_double), ld)
    if st != 0:
        raise RuntimeError("oracle_index_scores failed with status %d" % st)
    return out


def topk(batch, scores, k=None, rows=None):
    """Selected positions [n_rows, k] (int32, ascending, -1 padded).

    `scores` holds the listed rows' scores ([n_rows, ld], any float type).
    """
    lib = _load()
    v = _View(batch, rows)
    k = k or batch.cfg.topk
    s = _f64(scores)
    assert s.shape[0] == v.n
    out = np.empty((v.n, k), dtype=np.int32)
    st = lib.oracle_topk(batch.B, _p(v.cu_q, ctypes.c_int32), _p(v.seq_lens, ctypes.c_int32),
                         _p(s, ctypes.c_double), s.shape[1], k, _p(v.rows, ctypes.c_int32), v.n,
                         _p(out, ctypes.c_int32))
    if st != 0:
        raise RuntimeError("oracle_topk failed with status %d" % st)
    return out


def sparse_mla(batch, layer, idx, rows=None, k=None):
    """(out [n_rows, H, Dc], lse [n_rows, H]) in float64.

    idx holds the listed rows' selected positions ([n_rows, k]).
    """
    lib = _load()
    v = _View(batch, rows)
    cfg = batch.cfg
    idx = _i32(idx)
    k = k or idx.shape[1]
    assert idx.shape == (v.n, k)
    q = _f64(v.per_row(batch.q[layer]))
    pool = v.pool(batch.kv_pool[layer])
    if cfg.kv_fmt in (FMT_FP8, FMT_INT8):   # raw rows, decoded by the oracle
        kv = np.ascontiguousarray(pool.numpy())
        kv_fmt = 1 if cfg.kv_fmt == FMT_FP8 else 2
    else:
        kv = _f64(pool)
        kv_fmt = 0
    out = np.zeros((v.n, cfg.heads, cfg.dc), dtype=np.float64)
    lse = np.zeros((v.n, cfg.heads), dtype=np.float64)
    st = lib.oracle_sparse_mla(batch.B, _p(v.cu_q, ctypes.c_int32), _p(v.seq_lens, ctypes.c_int32),
                               _p(v.page_table, ctypes.c_int32), v.pt_stride, cfg.page_size,
                               v.num_pages, _p(q, ctypes.c_double), kv_fmt,
                               kv.ctypes.data_as(ctypes.c_void_p), _p(idx, ctypes.c_int32), k,
                               cfg.heads, cfg.dc, cfg.dr, cfg.sm_scale,
                               _p(v.rows, ctypes.c_int32), v.n, _p(out, ctypes.c_double),
                               _p(lse, ctypes.c_double))
    if st != 0:
        raise RuntimeError("oracle_sparse_mla failed with status %d" % st)
    return out, lse


def threads() -> int:
    """OpenMP threads the oracle's row loops run on."""
    return _load().oracle_threads()


def set_threads(n: int) -> None:
    """Run the oracle's row loops on n OpenMP threads from now on."""
    _load().oracle_set_threads(int(n))


def e4m3_encode(x: float) -> int:
    """The e4m3fn code nearest to x (ties to the even code, |x| > 448 gives 448)."""
    return int(_load().oracle_e4m3_encode(float(x)))


def q_fp8_exponent(amax: float) -> int:
    """The smallest integer e with amax <= 448 * 2^e (0 when amax is 0).

    With amax = m * 2^k, m in [0.5, 1): 448 * 2^(k-9) = 0.875 * 2^k covers
    amax when m <= 0.875, else 448 * 2^(k-8) = 1.75 * 2^k does; 448 * 2^(k-10)
    = 0.4375 * 2^k never does."""
    if amax == 0.0:
        return 0
    m, k = math.frexp(amax)
    return k - 9 if m <= 0.875 else k - 8


def quantize_q_fp8(q):
    """Per-(row, head) fp8 queries: q [..., D] float64 -> (codes uint8 [..., D],
    exponents int [...]).  Each head's D values are scaled by 2^-e, e from its
    largest magnitude (q_fp8_exponent: the scaled values stay within 448), and
    rounded to e4m3fn codes; the head stands for code * 2^e."""
    q = np.asarray(q, dtype=np.float64)
    lead = q.shape[:-1]
    flat = q.reshape(-1, q.shape[-1])
    codes = np.zeros(flat.shape, dtype=np.uint8)
    e = np.zeros(flat.shape[0], dtype=np.int64)
    for i in range(flat.shape[0]):
        e[i] = q_fp8_exponent(float(np.max(np.abs(flat[i]))))
        for d in range(flat.shape[1]):
            codes[i, d] = e4m3_encode(math.ldexp(float(flat[i, d]), -int(e[i])))
    return codes.reshape(q.shape), e.reshape(lead)


def dequantize_q_fp8(codes, e):
    """The values fp8 queries stand for: e4m3(code) * 2^e."""
    table = np.array([e4m3_to_double(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes)] * np.ldexp(1.0, np.asarray(e))[..., None]


def e4m3_to_double(byte: int) -> float:
    return _load().oracle_e4m3_to_double(byte)


def decode_fp8_rows(rows_u8, dc=512, dr=64):
    """Decode [n, 656] fp8 rows into float64 [n, dc+dr] with the oracle's decoder."""
    lib = _load()
    if isinstance(rows_u8, torch.Tensor):
        rows_u8 = rows_u8.detach().cpu().numpy()
    a = np.ascontiguousarray(rows_u8, dtype=np.uint8)
    a = a.reshape(-1, 656)
    out = np.empty((a.shape[0], dc + dr), dtype=np.float64)
    lib.oracle_decode_fp8_rows(a.ctypes.data_as(ctypes.c_void_p), a.shape[0], dc, dr,
                               _p(out, ctypes.c_double))
    return out


def decode_int8_rows(rows_u8, dc=512, dr=64):
    """Decode [n, 672] affine int8 rows into float64 [n, dc+dr] with the oracle's decoder."""
    lib = _load()
    if isinstance(rows_u8, torch.Tensor):
        rows_u8 = rows_u8.detach().cpu().numpy()
    a = np.ascontiguousarray(rows_u8, dtype=np.uint8)
    a = a.reshape(-1, dc + 8 * (dc // 128) + 2 * dr)
    out = np.empty((a.shape[0], dc + dr), dtype=np.float64)
    lib.oracle_decode_int8_rows(a.ctypes.data_as(ctypes.c_void_p), a.shape[0], dc, dr,
                                _p(out, ctypes.c_double))
    return out


def decode_fp8_keys(pages_u8, page_size, di=128, row_stride=128):
    """Decode page-blocked fp8 index keys ([num_pages, page_size*(row_stride+4)]
    bytes) into float64 [num_pages * page_size, di] with the oracle's decoder."""
    lib = _load()
    if isinstance(pages_u8, torch.Tensor):
        pages_u8 = pages_u8.detach().cpu().numpy()
    a = np.ascontiguousarray(pages_u8, dtype=np.uint8)
    n = a.shape[0]
    a = a.reshape(n, -1)
    out = np.empty((n * page_size, di), dtype=np.float64)
    lib.oracle_decode_fp8_keys(a.ctypes.data_as(ctypes.c_void_p), n, page_size, di, row_stride, a.shape[1],
                               _p(out, ctypes.c_double))
    return out


def indexer_prepare(batch, prep, with_pool=True):
    """Rotated queries, normalised and rotated keys, and the key pool after the
    keys are written (float64).

    `prep` carries q_in [T,H,D], k_in [T,D], gamma/beta [D], eps, cos/sin
    tables [rows, R/2], rope_dim R and interleaved.  Returns dict(q [T,H,D],
    k [T,D], pos [T], pool [num_pages*P, D] or None).  The pool image starts
    as the batch's key pool (bf16 / f32 values) and only the rows' slots
    change.
    """
    lib = _load()
    cfg = batch.cfg
    T, H, D = prep.q_in.shape
    q_in, k_in = _f64(prep.q_in), _f64(prep.k_in)
    gamma, beta = _f64(prep.gamma), _f64(prep.beta)
    cos, sin = _f64(prep.cos), _f64(prep.sin)
    cu = [0]
    for ql in batch.q_lens:
        cu.append(cu[-1] + ql)
    cu_q, seq_lens, pt = _i32(cu), _i32(batch.seq_lens), _i32(batch.page_table)
    pool = None
    num_pages = batch.k_pool.shape[0]
    if with_pool:
        pool = _f64(batch.k_pool).reshape(num_pages * cfg.page_size, D).copy()
    q_out = np.empty((T, H, D), dtype=np.float64)
    k_out = np.empty((T, D), dtype=np.float64)
    pos = np.empty(T, dtype=np.int64)
    st = lib.oracle_indexer_prepare(batch.B, _p(cu_q, ctypes.c_int32), _p(seq_lens, ctypes.c_int32),
                                    _p(pt, ctypes.c_int32), pt.shape[1], cfg.page_size, num_pages, T,
                                    _p(q_in, ctypes.c_double), _p(k_in, ctypes.c_double),
                                    _p(gamma, ctypes.c_double), _p(beta, ctypes.c_double),
                                    float(prep.eps), _p(cos, ctypes.c_double), _p(sin, ctypes.c_double),
                                    cos.shape[0], prep.rope_dim, int(prep.interleaved), H, D,
                                    _p(q_out, ctypes.c_double), _p(k_out, ctypes.c_double),
                                    _p(pool, ctypes.c_double) if pool is not None else None,
                                    _p(pos, ctypes.c_int64))
    if st != 0:
        raise RuntimeError("oracle_indexer_prepare failed with status %d" % st)
    return {"q": q_out, "k": k_out, "pos": pos, "pool": pool}


def run_path(batch, rows=None):
    """Scores -> top-k -> sparse MLA on every layer, for the listed rows.

    Layer 0 is the full layer; later layers reuse its indices (IndexShare).
    Returns dict(scores, idx, out=[per layer], lse=[per layer]).
    """
    sc = index_scores(batch, rows)
    idx = topk(batch, sc, rows=rows)
    outs, lses = [], []
    for layer in range(len(batch.q)):
        o, l = sparse_mla(batch, layer, idx, rows=rows)
        outs.append(o)
        lses.append(l)
    return dict(scores=sc, idx=idx, out=outs, lse=lses)
