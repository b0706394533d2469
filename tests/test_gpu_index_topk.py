"""Bounded-workspace scores + top-k (dsa_index_topk) on the GPU.

The selected indices must equal the oracle's bit for bit (integer draws make
every score exact) and equal the unbounded path (dsa_index_scores then
dsa_topk) whatever the chunking: one row per chunk, a chunk size that splits
drafts and eight-row prefill units, and the whole batch at once.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_07_amd import synth
from tests import _parity

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(*a):
    print("[gpu-test]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_07_amd import dsa  # noqa: F401  (raises if libdsa.so is missing)
    yield


def _bounded(sb, rows_per_chunk):
    from sparse_attention_07_amd import dsa
    cfg = sb.cfg
    b = dsa.batch_from(sb)
    W = dsa.dsa_index_topk_workspace_bytes
    row = W(1, sb.max_seq_len, cfg.topk, 1 << 40)   # one row: scores (and two-level candidates)
    ws_bytes = W(sb.T, sb.max_seq_len, cfg.topk, rows_per_chunk * row)
    assert ws_bytes == W(min(rows_per_chunk, sb.T), sb.max_seq_len, cfg.topk, 1 << 40)
    ws = torch.full((ws_bytes // 4,), float("nan"), device=DEV)   # stale contents must not matter
    idx = torch.full((sb.T, cfg.topk), 12345, dtype=torch.int32, device=DEV)
    dsa.dsa_index_topk(b, sb.q_idx, cfg.idx_fmt, sb.w, dsa.make_key_pool(sb), cfg.hi, cfg.di, cfg.topk, idx,
                       ws, ws_bytes)
    torch.cuda.synchronize()
    return idx


CASES = {
    "decode16": dict(cfg=1, batch=6, ctx=(100, 3000), topk=512),
    "mtp_drafts": dict(cfg=4, batch=3, ctx=(3000, 9000), topk=512),
    "ragged_empty": dict(cfg=4, q_lens=[5, 0, 3, 1, 0, 5, 2], ctx=(600, 3000), topk=512),
    "prefill_rows": dict(cfg=3, q_len=130, ctx=(700, 700), topk=512),
    "fp8_keys": dict(cfg=4, batch=2, ctx=(2000, 5000), topk=512, key_fmt=synth.FMT_FP8_E4M3_B128),
    "page5": dict(cfg=1, batch=4, ctx=(300, 1300), topk=256, page_size=5),
    "tiny_f32": dict(cfg=0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_bounded_matches_oracle_and_unbounded(name):
    from sparse_attention_07_amd.path import DSAPath
    kw = dict(CASES[name])
    cfg = kw.pop("cfg")
    sb = synth.make_batch(cfg, device=DEV, layers=0, **kw)
    ref = oracle.topk(sb, oracle.index_scores(sb))
    p = DSAPath(sb)
    p.index_scores()
    p.topk()
    torch.cuda.synchronize()
    _parity.check_idx_exact(p.idx, ref, what="unbounded idx")
    for per in sorted({1, 3, 7, 8, 9, sb.T}):
        _say(name, "T=%d rows per chunk %d" % (sb.T, per))
        idx = _bounded(sb, per)
        _parity.check_idx_exact(idx, ref, what="idx, %d rows per chunk" % per)
        assert torch.equal(idx, p.idx)


@pytest.mark.parametrize("per", [1, 2, 5])
def test_long_context_rows_per_chunk(per):
    # 5 draft rows over a 300K-token context: each chunk row holds a 1.2 MB
    # score row and its two-level top-k candidates (10 segments of 32768)
    sb = synth.make_batch(4, device=DEV, layers=0, batch=1, ctx=(300000, 300000), topk=2048)
    _say("long context T=%d max_seq=%d, %d rows per chunk" % (sb.T, sb.max_seq_len, per))
    idx = _bounded(sb, per)
    ref = oracle.topk(sb, oracle.index_scores(sb))
    _parity.check_idx_exact(idx, ref)
    assert np.all((idx.cpu().numpy() >= 0).sum(1) == 2048)


@pytest.mark.parametrize("key_fmt", [None, synth.FMT_FP8_E4M3_B128])
def test_scores_skip_unmapped_and_out_of_range_pages(key_fmt):
    # Page ids are loaded without a branch and checked when the offsets are
    # formed: a page id of -1 or past the pool leaves its tokens' scores
    # unwritten, and every other score equals the oracle's (computed on the
    # intact table).
    from sparse_attention_07_amd.path import DSAPath
    kw = dict(batch=5, ctx=(700, 3000), topk=512)
    if key_fmt is not None:
        kw["key_fmt"] = key_fmt
    sb = synth.make_batch(1 if key_fmt is None else 4, device=DEV, layers=0, **kw)
    ref = oracle.index_scores(sb)
    P = sb.cfg.page_size
    bad = {(0, 1): -1, (2, 3): sb.num_pages + 7, (4, 0): -5}   # (request, logical page) -> page id
    pt = sb.page_table.clone()
    for (b, lp), pid in bad.items():
        assert lp * P < sb.seq_lens[b]
        sb.page_table[b, lp] = pid
    p = DSAPath(sb)
    p.scores.fill_(float("nan"))
    p.index_scores()
    torch.cuda.synchronize()
    got = p.scores.cpu().numpy().astype(np.float64)
    cu = sb.cu_q.tolist()
    for b in range(len(cu) - 1):
        for t in range(cu[b], cu[b + 1]):
            pos = sb.seq_lens[b] - (cu[b + 1] - cu[b]) + (t - cu[b])
            skipped = np.zeros(got.shape[1], dtype=bool)
            for (bb, lp), _ in bad.items():
                if bb == b:
                    skipped[lp * P:(lp + 1) * P] = True
            s = np.arange(pos + 1)
            keep = s[~skipped[:pos + 1]]
            assert np.all(np.isnan(got[t, s[skipped[:pos + 1]]])), "row %d: a skipped page was written" % t
            np.testing.assert_array_equal(got[t, keep], ref[t, keep].astype(np.float32).astype(np.float64))
    sb.page_table.copy_(pt)
