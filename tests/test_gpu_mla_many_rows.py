"""The 64-head sparse MLA over more (query row, 64-head group) items than CUs,
unsplit, against the oracle (needs an MI355X).

With one split and more items than CUs the workgroups run in several rounds;
draft rows, 8-bit caches, more than 256 requests (a request search past the
first lookup round), a partial last tile, requests without rows and 64-head
groups each get a case.  Integer draws make the index path exact, so the
selections the MLA attends are the oracle's; its outputs must be within the
bf16 / 8-bit tolerances on sampled rows (the first and last rows, rows of the
second round and random ones), finite everywhere, and every lse written.
"""
import sys

import numpy as np
import pytest
import torch

from sparse_attention_07_amd import synth
from tests import _parity

pytestmark = pytest.mark.gpu

DEV = "cuda"
FP8 = synth.FMT_FP8_E4M3_B128
INT8 = synth.FMT_INT8_AFFINE_B128


def _say(*a):
    print("[gpu-test]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_07_amd import dsa  # noqa: F401  (raises if libdsa.so is missing)
    yield


CASES = {
    # 400 items: a second, partial round of workgroups; 16 tiles per item
    "decode_bf16": dict(cfg=2, batch=200, ctx=(600, 3000), topk=512),
    "decode_fp8": dict(cfg=2, batch=200, ctx=(600, 3000), topk=512, kv_fmt=FP8),
    "decode_int8": dict(cfg=2, batch=200, ctx=(600, 3000), topk=512, kv_fmt=INT8),
    # draft rows (causal inside the draft), fp8 rows, 32 tiles per item
    "drafts_fp8": dict(cfg=4, batch=40, ctx=(1100, 4000), topk=1024),
    # more than 256 requests, a partial last tile, contexts shorter than K (-1 tails)
    "300_requests_k600": dict(cfg=2, batch=300, ctx=(200, 1400), topk=600),
    # requests without rows and mixed draft lengths
    "ragged": dict(cfg=4, q_lens=[5, 0, 3, 1, 0, 5, 2, 4] * 26, ctx=(700, 2500), topk=512),
    # 64 heads: one head group per row (400 rows: one split at 64 heads)
    "h64_decode": dict(cfg=2, batch=400, ctx=(600, 2000), topk=512, heads=64),
}


def _sample(T, n_items_per_row, n=24, seed=0):
    g = np.random.default_rng(seed)
    picks = {0, T - 1}
    # rows of the second round of workgroups
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    first_second = (cus // n_items_per_row) if n_items_per_row else 0
    for t in (first_second, first_second + 1, T // 2):
        if 0 <= t < T:
            picks.add(int(t))
    while len(picks) < min(n, T):
        picks.add(int(g.integers(0, T)))
    return sorted(picks)


@pytest.mark.parametrize("name", list(CASES))
def test_many_rows_mla_matches_the_oracle(name):
    from sparse_attention_07_amd.path import DSAPath
    kw = dict(CASES[name])
    cfg = kw.pop("cfg")
    sb = synth.make_batch(cfg, device=DEV, layers=1, **kw)
    n_groups = sb.cfg.heads // 64
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert sb.T * n_groups > cus, "the case must have more items than CUs"
    _say("mla, many rows", name, "T=%d B=%d heads=%d K=%d fmt=%d" % (sb.T, sb.B, sb.cfg.heads, sb.cfg.topk,
                                                                       sb.cfg.kv_fmt))
    p = DSAPath(sb)
    p.out[0].fill_(7.0)
    p.lse[0].fill_(7.0)
    p.index_scores()
    p.topk()
    p.mla(0)
    torch.cuda.synchronize()
    rows = _sample(sb.T, n_groups, seed=len(name))
    _parity.check_path(sb, p, rows=rows)
    assert torch.isfinite(p.out[0].float()).all()
    lse = p.lse[0]
    assert not (lse == 7.0).any(), "some lse entries were not written"
