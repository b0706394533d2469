"""Hand-built batches for the small pin and edge-case tests.

Builds a synth.Batch from token-major per-request arrays, laying the tokens
into pages (identity order or a seeded permutation).  Layout only; no method
arithmetic.
"""
import math

import torch

from sparse_attention_07_amd import synth


def paginate(per_request, page_size, permute_seed=None):
    """per_request: list of [seq_len_b, ...] tensors -> (pool, page_table)."""
    pages_per = [(x.shape[0] + page_size - 1) // page_size for x in per_request]
    num_pages = sum(pages_per)
    tail = tuple(per_request[0].shape[1:])
    if permute_seed is None:
        perm = torch.arange(num_pages, dtype=torch.int32)
    else:
        g = torch.Generator().manual_seed(permute_seed)
        perm = torch.randperm(num_pages, generator=g).to(torch.int32)
    pool = torch.zeros((num_pages, page_size) + tail, dtype=per_request[0].dtype)
    pt = torch.full((len(per_request), max(pages_per)), -1, dtype=torch.int32)
    o = 0
    for b, x in enumerate(per_request):
        n = pages_per[b]
        pt[b, :n] = perm[o:o + n]
        s = torch.arange(x.shape[0])
        pool[pt[b, s // page_size].long(), s % page_size] = x
        o += n
    return pool, pt, num_pages


def make(q_lens, seq_lens, keys, q_idx, w, page_size=4, q_layers=(), latent_layers=(),
         heads=None, dc=None, dr=None, topk=64, sm_scale=None, permute_seed=None,
         kv_fmt=synth.FMT_F32, idx_fmt=synth.FMT_F32, q_fmt=synth.FMT_F32):
    """keys / latent_layers[l]: lists of per-request token-major tensors."""
    k_pool, pt, num_pages = paginate(keys, page_size, permute_seed)
    kv_pools = []
    for lat in latent_layers:
        p, pt2, _ = paginate(lat, page_size, permute_seed)
        assert torch.equal(pt, pt2)
        kv_pools.append(p)
    hi, di = q_idx.shape[1], q_idx.shape[2]
    if q_layers:
        heads = q_layers[0].shape[1]
        D = q_layers[0].shape[2]
        dr = dr if dr is not None else 0
        dc = D - dr
    cfg = synth.Config("custom", len(q_lens), max(q_lens), min(seq_lens), max(seq_lens), topk,
                       hi, di, heads or 1, dc or 1, dr or 0, page_size, kv_fmt, idx_fmt, q_fmt,
                       sm_scale if sm_scale is not None else 1.0 / math.sqrt(max(dc or 1, 1)),
                       layers=len(q_layers))
    cu = [0]
    for ql in q_lens:
        cu.append(cu[-1] + ql)
    return synth.Batch(cfg=cfg, q_lens=list(q_lens), seq_lens=list(seq_lens),
                       cu_q=torch.tensor(cu, dtype=torch.int32),
                       seq_lens_t=torch.tensor(seq_lens, dtype=torch.int32),
                       page_table=pt, num_pages=num_pages, q_idx=q_idx, w=w, k_pool=k_pool,
                       q=list(q_layers), kv_pool=kv_pools)


def dummy_index(q_lens, seq_lens, hi=1, di=1):
    """Indexer inputs of the right shape when only the MLA part is under test."""
    T = sum(q_lens)
    keys = [torch.zeros(s, di) for s in seq_lens]
    return keys, torch.zeros(T, hi, di), torch.zeros(T, hi)
