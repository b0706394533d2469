"""Indexer scores held back in LDS and written after the keys (needs an MI355X).

A workgroup whose share of the key blocks has at least 64 blocks, and whose
scores fit in the staged-row slots its units leave unused, keeps its scores
in LDS and writes them in one burst once every key of its share is read.
These cases give every workgroup such a share (tens of thousands of blocks
over the CUs), with single rows, units of two and three draft rows (where
some rows of a unit's last blocks have no token), partial pages, fp8 keys
and fp8 queries.  The score buffer starts as NaN: scores must equal the
oracle's exactly (integer draws) on sampled rows, entries past each row's
position must stay NaN, tokens on unmapped pages must stay NaN, and the
selections must be the oracle's and the bounded path's.
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
FP8 = synth.FMT_FP8_E4M3_B128


def _say(*a):
    print("[gpu-test]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_07_amd import dsa  # noqa: F401  (raises if libdsa.so is missing)
    yield


LONG = (17000, 30000)
CASES = {
    "decode_bf16": dict(cfg=1, batch=64, ctx=LONG, topk=512),
    "decode_fp8_keys": dict(cfg=1, batch=64, ctx=LONG, topk=512, key_fmt=FP8),
    "decode_fp8_queries": dict(cfg=1, batch=64, ctx=LONG, topk=512, key_fmt=FP8, q_fp8=True),
    "drafts_of_2": dict(cfg=4, batch=64, q_len=2, ctx=LONG, topk=512),
    "drafts_of_3": dict(cfg=4, batch=64, q_len=3, ctx=LONG, topk=512),
    "page_size_5": dict(cfg=1, batch=64, ctx=LONG, topk=512, page_size=5),
}


def _rows(sb, n=6, seed=0):
    g = np.random.default_rng(seed)
    rows = {0, sb.T - 1, sb.T // 2}
    while len(rows) < min(n, sb.T):
        rows.add(int(g.integers(0, sb.T)))
    return sorted(rows)


def _make(name):
    from sparse_attention_07_amd.path import DSAPath
    kw = dict(CASES[name])
    cfg = kw.pop("cfg")
    q_fp8 = kw.pop("q_fp8", False)
    sb = synth.make_batch(cfg, device=DEV, layers=0, **kw)
    return sb, DSAPath(sb, q_fp8=q_fp8), q_fp8


def _check_rows(sb, p, rows, ref, skipped=None):
    """Exact scores on s <= pos (except skipped tokens, left NaN), NaN past pos."""
    got = p.scores.cpu().numpy().astype(np.float64)
    pos = sb.positions()
    for i, t in enumerate(rows):
        n = pos[t] + 1
        skip = np.zeros(n, dtype=bool) if skipped is None else skipped(t, n)
        assert np.all(np.isnan(got[t, n:])), "row %d: an entry past its position was written" % t
        assert np.all(np.isnan(got[t, :n][skip])), "row %d: a token on an unmapped page was written" % t
        np.testing.assert_array_equal(got[t, :n][~skip], ref[i, :n][~skip].astype(np.float32).astype(np.float64),
                                      err_msg="row %d scores" % t)


@pytest.mark.parametrize("name", list(CASES))
def test_held_back_scores_match_the_oracle(name):
    sb, p, q_fp8 = _make(name)
    blocks = sum((s + 63) // 64 for s in sb.seq_lens)
    _say("held-back scores", name, "T=%d B=%d key blocks %d" % (sb.T, sb.B, blocks))
    p.scores.fill_(float("nan"))
    p.index_scores()
    p.topk()
    torch.cuda.synchronize()
    rows = _rows(sb, seed=len(name))
    ref = oracle.index_scores(sb, rows, ld=p.ld, q_fp8=q_fp8)
    _check_rows(sb, p, rows, ref)
    _parity.check_idx_exact(p.idx.cpu().numpy()[rows], oracle.topk(sb, ref, rows=rows))


def test_held_back_scores_skip_unmapped_pages():
    from sparse_attention_07_amd.path import DSAPath
    kw = dict(CASES["decode_bf16"])
    kw.pop("cfg")
    sb = synth.make_batch(1, device=DEV, layers=0, **kw)
    rows = [0, 17, 31, 63]
    ref = oracle.index_scores(sb, rows, ld=max(64, (sb.max_seq_len + 63) // 64 * 64))   # the intact table
    P = sb.cfg.page_size
    # (request, logical page) -> a page id that maps nothing: -1 or past the pool
    bad = {(0, 3): -1, (0, 200): sb.num_pages + 9, (31, 0): -2, (63, 100): sb.num_pages}
    pt = sb.page_table.clone()
    for (b, lp), pid in bad.items():
        assert lp * P < sb.seq_lens[b]
        sb.page_table[b, lp] = pid
    try:
        p = DSAPath(sb)
        p.scores.fill_(float("nan"))
        _say("held-back scores, unmapped pages")
        p.index_scores()
        torch.cuda.synchronize()
        req = sb.row_request()

        def skipped(t, n):
            m = np.zeros(n, dtype=bool)
            for (b, lp), _ in bad.items():
                if b == req[t]:
                    m[lp * P:min(n, (lp + 1) * P)] = True
            return m

        _check_rows(sb, p, rows, ref, skipped)
    finally:
        sb.page_table.copy_(pt)


def test_held_back_scores_bounded_path_selects_the_same():
    # dsa_index_topk over chunks of rows (smaller shares per launch) against
    # the unbounded launch, whose shares hold their scores back
    from sparse_attention_07_amd import dsa
    sb, p, _ = _make("drafts_of_2")
    p.index_scores()
    p.topk()
    cfg = sb.cfg
    b = dsa.batch_from(sb)
    W = dsa.dsa_index_topk_workspace_bytes
    row = W(1, sb.max_seq_len, cfg.topk, 1 << 40)
    for per in (16, sb.T):
        ws_bytes = W(sb.T, sb.max_seq_len, cfg.topk, per * row)
        ws = torch.full((ws_bytes // 4,), float("nan"), device=DEV)
        idx = torch.full((sb.T, cfg.topk), 12345, dtype=torch.int32, device=DEV)
        dsa.dsa_index_topk(b, sb.q_idx, cfg.idx_fmt, sb.w, dsa.make_key_pool(sb), cfg.hi, cfg.di, cfg.topk,
                           idx, ws, ws_bytes)
        torch.cuda.synchronize()
        _say("bounded, %d rows per chunk" % per)
        assert torch.equal(idx, p.idx), "rows per chunk %d" % per
