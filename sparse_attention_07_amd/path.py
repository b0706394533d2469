"""The DSA hot path over one batch: indexer scores -> top-k -> sparse MLA per layer.

Allocates the outputs once (torch, on the batch's device) and enqueues the
library calls on the current stream.  Layer 0 is a full layer; layers 1..L-1
are IndexShare layers that reuse its indices (mlx-lm PR 1419, description:
shared layers reuse the previous full layer's top-k).
"""
from __future__ import annotations

import torch

from . import dsa
from .synth import torch_dtype


class DSAPath:
    def __init__(self, sb, prefill: bool | None = None, prep=None, score_budget: int | None = None,
                 q_fp8: bool = False):
        cfg = sb.cfg
        self.sb = sb
        # q_fp8: the indexer contracts its queries as fp8 codes (fp8 keys only)
        self.idx_q_fmt = dsa.DSA_BF16_TO_FP8 if q_fp8 else cfg.idx_fmt
        # optional indexer preparation inputs (synth.Prep): when given, each step
        # first rotates them into sb.q_idx and stores the keys into the key pool
        self.prep = prep
        self.cfg = cfg
        dev = sb.q_idx.device
        self.batch = dsa.batch_from(sb)
        self.k_pool = dsa.make_key_pool(sb)
        self.kv = [dsa.make_pool(p, cfg.kv_fmt, cfg.dc + cfg.dr) for p in sb.kv_pool]
        T = sb.T
        # score rows padded to a multiple of 64 entries (256 B)
        self.ld = max(64, (sb.max_seq_len + 63) // 64 * 64)
        self.scores = torch.empty((T, self.ld), dtype=torch.float32, device=dev)
        self.idx = torch.empty((T, cfg.topk), dtype=torch.int32, device=dev)
        odt = torch_dtype(cfg.q_fmt)
        self.out = [torch.empty((T, cfg.heads, cfg.dc), dtype=odt, device=dev) for _ in sb.q]
        self.lse = [torch.empty((T, cfg.heads), dtype=torch.float32, device=dev) for _ in sb.q]
        self.prefill = (sb.max_q_len > 64) if prefill is None else prefill
        self.ws_bytes = dsa.dsa_sparse_mla_workspace_bytes(T, cfg.heads, cfg.topk, cfg.dc, self.prefill)
        # zero-filled once: the split-merge counters in it start at 0 and every call
        # leaves them at 0
        self.ws = torch.zeros((max(self.ws_bytes, 16),), dtype=torch.uint8, device=dev)
        self.topk_ws_bytes = dsa.dsa_topk_workspace_bytes(T, sb.max_seq_len, cfg.topk)
        self.topk_ws = (torch.empty((self.topk_ws_bytes,), dtype=torch.uint8, device=dev)
                        if self.topk_ws_bytes else None)
        # bounded scoring: with a budget (bytes), scores + top-k run through
        # dsa_index_topk over a workspace of whole score rows instead of [T, ld]
        self.itk_ws_bytes = 0
        if score_budget is not None:
            self.itk_ws_bytes = dsa.dsa_index_topk_workspace_bytes(T, sb.max_seq_len, cfg.topk, score_budget)
            if self.itk_ws_bytes == 0 and T > 0:
                raise ValueError("score budget %d B is below one score row" % score_budget)
            self.itk_ws = torch.empty((max(self.itk_ws_bytes, 16) // 4,), dtype=torch.float32, device=dev)

    def indexer_prepare(self, stream=None):
        c, pr = self.cfg, self.prep
        dsa.dsa_indexer_prepare(self.batch, pr.q_in, self.sb.q_idx, pr.k_in, c.idx_fmt, pr.gamma, pr.beta,
                                pr.eps, pr.cos, pr.sin, pr.cos.shape[0], pr.rope_dim, pr.interleaved,
                                self.k_pool, c.hi, c.di, stream)

    def index_scores(self, stream=None):
        c = self.cfg
        dsa.dsa_index_scores(self.batch, self.sb.q_idx, self.idx_q_fmt, self.sb.w, self.k_pool, c.hi, c.di,
                             self.scores, self.ld, stream)

    def topk(self, stream=None):
        dsa.dsa_topk(self.batch, self.scores, self.ld, self.cfg.topk, self.idx, self.topk_ws,
                     self.topk_ws_bytes, stream)

    def index_topk(self, stream=None):
        c = self.cfg
        dsa.dsa_index_topk(self.batch, self.sb.q_idx, self.idx_q_fmt, self.sb.w, self.k_pool, c.hi, c.di, c.topk,
                           self.idx, self.itk_ws, self.itk_ws_bytes, stream)

    def mla(self, layer: int, idx=None, stream=None):
        c = self.cfg
        fn = dsa.dsa_sparse_mla_prefill if self.prefill else dsa.dsa_sparse_mla_decode
        fn(self.batch, self.sb.q[layer], c.q_fmt, self.kv[layer], self.idx if idx is None else idx,
           c.topk, c.heads, c.dc, c.dr, c.sm_scale, self.out[layer], self.lse[layer], self.ws,
           self.ws_bytes, stream)

    def step(self, stream=None):
        """One pass of the whole path: full layer, then the IndexShare layers."""
        if self.prep is not None:
            self.indexer_prepare(stream)
        if self.itk_ws_bytes:
            self.index_topk(stream)
        else:
            self.index_scores(stream)
            self.topk(stream)
        for layer in range(len(self.kv)):
            self.mla(layer, stream=stream)
