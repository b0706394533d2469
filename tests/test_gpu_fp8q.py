"""fp8 indexer queries (DSA_BF16_TO_FP8) on the fp8 matrix cores vs the oracle.

The kernel quantises each (row, head) of the bf16 queries to e4m3 codes at a
power-of-two scale and contracts them with the fp8 key codes.  Parity draws
(n/8, |n| <= 8) scale to exact e4m3 values, so there the scores equal the
oracle's exactly and the indices bit for bit.  Gaussian queries and keys at
their quantisers' scales exercise the rounding: the codes must be the
oracle's (its encoder rounds to nearest, ties to even, like the hardware
conversion), so the scores agree to f32 accumulation and the selections
overlap almost entirely.
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


CASES = {
    "decode16": dict(cfg=1, batch=6, ctx=(100, 3000), topk=512),
    "decode16_p5": dict(cfg=1, batch=4, ctx=(300, 1300), topk=256, page_size=5),
    "mtp_drafts": dict(cfg=4, batch=3, ctx=(3000, 9000), topk=512),
    "ragged": dict(cfg=4, q_lens=[5, 0, 3, 1, 0, 5, 2], ctx=(600, 3000), topk=512),
    "prefill_units_of_8": dict(cfg=3, q_len=130, ctx=(700, 700), topk=512),
    "many_requests": dict(cfg=1, batch=300, ctx=(40, 700), topk=256),
}


def _path(name, mode):
    from sparse_attention_07_amd.path import DSAPath
    kw = dict(CASES[name])
    cfg = kw.pop("cfg")
    sb = synth.make_batch(cfg, device=DEV, mode=mode, layers=0, key_fmt=FP8, **kw)
    p = DSAPath(sb, q_fp8=True)
    return sb, p


@pytest.mark.parametrize("name", list(CASES))
def test_fp8_queries_parity_draws(name):
    sb, p = _path(name, "parity")
    _say("fp8 queries, parity draws", name, "T=%d B=%d" % (sb.T, sb.B))
    p.index_scores()
    p.topk()
    torch.cuda.synchronize()
    rows = list(range(sb.T))
    ref = oracle.index_scores(sb, rows, ld=p.ld, q_fp8=True)
    _parity.check_scores_exact(p.scores, ref, sb.positions())
    _parity.check_idx_exact(p.idx, oracle.topk(sb, ref, rows=rows))


@pytest.mark.parametrize("name", ["decode16", "mtp_drafts", "prefill_units_of_8"])
def test_fp8_queries_at_real_scales(name):
    sb, p = _path(name, "perf")
    _say("fp8 queries, gaussian draws", name, "T=%d" % sb.T)
    p.index_scores()
    p.topk()
    torch.cuda.synchronize()
    g = np.random.default_rng(9)
    rows = sorted(set([0, sb.T - 1] + g.integers(0, sb.T, 6).tolist()))
    ref = oracle.index_scores(sb, rows, ld=p.ld, q_fp8=True)
    ref_idx = oracle.topk(sb, ref, rows=rows)
    g_idx = p.idx.cpu().numpy()[rows]
    pos = sb.positions()
    for i, t in enumerate(rows):
        n = pos[t] + 1
        gs = p.scores[t, :n].double().cpu().numpy()
        r = ref[i, :n]
        # exact products of codes summed in f32 against an f64 sum
        assert np.max(np.abs(gs - r)) <= 1e-4 * max(1.0, np.max(np.abs(r))), "row %d scores" % t
        a = set(g_idx[i][g_idx[i] >= 0].tolist())
        b = set(ref_idx[i][ref_idx[i] >= 0].tolist())
        assert len(a) == len(b) == min(n, sb.cfg.topk)
        assert len(a & b) >= 0.99 * len(b), "row %d overlap %d of %d" % (t, len(a & b), len(b))


def test_fp8_queries_bounded_path_matches_unbounded():
    # dsa_index_topk over a small score budget (chunks of rows) selects what
    # dsa_index_scores + dsa_topk select, with fp8 queries too
    from sparse_attention_07_amd.path import DSAPath
    sb = synth.make_batch(3, device=DEV, mode="perf", layers=0, key_fmt=FP8, q_len=130, ctx=(700, 700), topk=512)
    _say("fp8 queries, bounded path T=%d" % sb.T)
    a = DSAPath(sb, q_fp8=True)
    a.index_scores()
    a.topk()
    b = DSAPath(sb, q_fp8=True, score_budget=64 * 1024)
    b.index_topk()
    torch.cuda.synchronize()
    _parity.check_idx_exact(b.idx, a.idx.cpu().numpy(), what="bounded idx")
