"""dsa_sparse_mla_decode_static (the entry point that allocates nothing) against
dsa_sparse_mla_decode with a caller-owned workspace (needs an MI355X).

Both run the same kernels on the same split plan, so their outputs must be
equal bit for bit; each call is also checked against the oracle on sampled
rows at the output tolerance.  Consecutive calls share the library's device
array: a call is followed by a smaller one (fewer rows, so another partial
layout over the same array), and 16-head calls by 64-head ones, in both cache
formats; then the call is captured in a HIP graph and replayed.
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


def _case(cfg, **kw):
    from sparse_attention_07_amd import dsa
    from sparse_attention_07_amd.path import DSAPath
    sb = synth.make_batch(cfg, device=DEV, layers=1, **kw)
    p = DSAPath(sb, prefill=False)
    p.index_scores()
    p.topk()
    torch.cuda.synchronize()
    c = sb.cfg
    need = dsa.dsa_sparse_mla_workspace_bytes(sb.T, c.heads, c.topk, c.dc, False)
    assert 0 < need <= dsa.DSA_MLA_SCRATCH_BYTES      # a split plan, within the library's array
    return sb, p


def _static_call(sb, p, out, lse):
    from sparse_attention_07_amd import dsa
    c = sb.cfg
    dsa.dsa_sparse_mla_decode_static(p.batch, sb.q[0], c.q_fmt, p.kv[0], p.idx, c.topk, c.heads, c.dc, c.dr,
                                     c.sm_scale, out, lse)


SEQUENCE = [
    ("h16 bf16, 100 rows", 1, dict(batch=100, ctx=(1100, 3000), topk=1024)),
    ("h16 bf16, 40 rows (smaller)", 1, dict(batch=40, ctx=(1100, 3000), topk=1024)),
    ("h128 fp8, 25 rows", 4, dict(batch=5, ctx=(1100, 3000), topk=1024)),
    ("h128 fp8, 10 rows (smaller)", 4, dict(batch=2, ctx=(1100, 3000), topk=1024)),
    ("h128 bf16, 64 rows", 2, dict(batch=64, ctx=(1100, 3000), topk=1024)),
    ("h16 int8, 12 rows (smaller)", 1, dict(batch=12, ctx=(1100, 3000), topk=1024,
                                            kv_fmt=synth.FMT_INT8_AFFINE_B128)),
]


def test_static_entry_matches_the_workspace_entry():
    for name, cfg, kw in SEQUENCE:
        sb, p = _case(cfg, **kw)
        _say("no-alloc decode:", name, "T=%d" % sb.T)
        p.mla(0)                                            # caller workspace
        out = torch.full_like(p.out[0], 7.0)
        lse = torch.full_like(p.lse[0], 7.0)
        _static_call(sb, p, out, lse)                       # the library's array
        torch.cuda.synchronize()
        assert torch.equal(out, p.out[0]) and torch.equal(lse, p.lse[0]), name
        rows = sorted({0, sb.T - 1, sb.T // 2, 1})
        ref_out, ref_lse = oracle.sparse_mla(sb, 0, p.idx.cpu().numpy()[rows], rows=rows)
        atol = _parity.atol_for(sb.cfg)
        _parity.assert_within(out.float().cpu().numpy()[rows], ref_out, atol, what=name + " out")
        _parity.assert_within(lse.cpu().numpy()[rows], ref_lse, atol, what=name + " lse")


def test_static_entry_replays_from_a_graph():
    sb, p = _case(1, batch=30, ctx=(1100, 3000), topk=1024)
    p.mla(0)
    out = torch.full_like(p.out[0], 7.0)
    lse = torch.full_like(p.lse[0], 7.0)
    _static_call(sb, p, out, lse)                           # eager first (set-up done outside capture)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _static_call(sb, p, out, lse)
    for rep in range(3):
        out.fill_(7.0)
        lse.fill_(7.0)
        torch.cuda.synchronize()
        _say("no-alloc graph replay", rep)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, p.out[0]) and torch.equal(lse, p.lse[0]), "replay %d" % rep
    assert np.isfinite(lse.cpu().numpy()).all()
