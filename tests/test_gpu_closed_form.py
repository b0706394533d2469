"""Closed forms of sparse MLA through every kernel variant (needs an MI355X).

With q = 0 every logit is 0, so the softmax is uniform over the usable
selected rows: out[t,h] = the mean of those rows' latent parts and
lse[t,h] = log(n_usable(t)), for every head.  Both are checked far tighter
than the oracle tolerance, so a row dropped or counted twice by a split, a
tile mask or a merge fails the test:
- lse within 1e-4 (one row lost out of 2048 moves it by 4.9e-4);
- out, per (row, head), in L2 over the 512 columns: losing one of n rows
  moves the mean by (x_j - mean) / (n - 1), about sqrt(512) / n in norm for
  rows of N(0, 1) values (0.011 at n = 2048), while the bf16 roundings (of
  the output and of split partials) stay near 1e-3.  The bound is
  2^-8 |mean| + 0.2 sqrt(512) / n (4.2e-3 at n = 2048), with an elementwise
  guard of 2^-7 |mean| + 8e-4.  The selections
mix usable indices with -1, negative, past-pos and huge entries, and include
rows with a single usable index and rows with none (out = 0, lse = -inf).

The variants: 16-head groups split and unsplit, with draft rows, over bf16,
fp8 and int8 caches; 64-head groups (64 and 128 heads) split and unsplit in
decode, and prefill; unsplit 64-head launches with more row x head-group
items than CUs over int8 and fp8 caches, with draft rows, more than 256
requests and a partial last tile.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_07_amd import synth

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


def _decoded_rows(sb, layer):
    """All token slots of a layer's latent pool as float64 [pages, P, dc], with
    the values the kernels attend: bf16 rows as stored; 8-bit rows decoded by
    the oracle and rounded to bf16 once (the kernels round each decoded
    element to bf16 before the MFMAs)."""
    cfg = sb.cfg
    pool = sb.kv_pool[layer].cpu()
    if cfg.kv_fmt == synth.FMT_BF16:
        return pool[..., :cfg.dc].double().numpy()
    n, P = pool.shape[0], pool.shape[1]
    dec = (oracle.decode_fp8_rows(pool.reshape(n * P, -1)) if cfg.kv_fmt == synth.FMT_FP8_E4M3_B128
           else oracle.decode_int8_rows(pool.reshape(n * P, -1)))
    lat = torch.from_numpy(dec[:, :cfg.dc]).float().to(torch.bfloat16).double().numpy()
    return lat.reshape(n, P, cfg.dc)


def _selection(sb, seed):
    """Index rows mixing usable positions with entries that must be skipped;
    row 0 has no usable entry and row 1 exactly one."""
    K = sb.cfg.topk
    pos = sb.positions()
    g = torch.Generator().manual_seed(seed)
    idx = torch.full((sb.T, K), -1, dtype=torch.int32)
    for t in range(sb.T):
        if t == 0:
            idx[t, :4] = torch.tensor([-1, -3, pos[t] + 1, 2 ** 30], dtype=torch.int32)
            continue
        n = min(pos[t] + 1, K - 6)
        sel = torch.randperm(pos[t] + 1, generator=g)[:n].to(torch.int32)
        if t == 1:
            sel = sel[:1]
        junk = torch.tensor([-1, -7, pos[t] + 1, pos[t] + 100, 2 ** 30, -1], dtype=torch.int32)
        row = torch.cat([sel, junk])
        row = row[torch.randperm(len(row), generator=g)]       # usable and junk entries interleaved
        idx[t, :len(row)] = row
    return idx


def _closed_form(sb, idx, lat):
    """Mean latent of each row's usable selected tokens, and log of their count."""
    P = sb.cfg.page_size
    pt = sb.page_table.cpu().numpy()
    pos = sb.positions()
    req = sb.row_request()
    mean = np.zeros((sb.T, sb.cfg.dc))
    lse = np.full(sb.T, -np.inf)
    for t in range(sb.T):
        s = idx[t]
        s = s[(s >= 0) & (s <= pos[t])]
        if len(s) == 0:
            continue
        pages = pt[req[t], s // P]
        mean[t] = lat[pages, s % P].mean(axis=0)
        lse[t] = np.log(len(s))
    return mean, lse


VARIANTS = {
    # 16-head groups
    "h16_split": dict(cfg=1, batch=4, ctx=(2100, 4000), topk=2048),
    "h16_split_drafts_fp8": dict(cfg=1, batch=3, q_len=5, ctx=(1500, 4000), topk=1024,
                                 kv_fmt=synth.FMT_FP8_E4M3_B128),
    "h16_split_int8": dict(cfg=1, batch=4, ctx=(2100, 4000), topk=2048, kv_fmt=synth.FMT_INT8_AFFINE_B128),
    "h16_unsplit": dict(cfg=1, batch=300, ctx=(100, 700), topk=256),
    "h32_split_p5": dict(cfg=1, batch=3, ctx=(1000, 3000), topk=1024, heads=32, page_size=5),
    "h16_prefill": dict(cfg=3, q_len=100, ctx=(1200, 1200), topk=1024, heads=16, prefill=True),
    # 64-head groups
    "h128_split": dict(cfg=2, batch=3, ctx=(2100, 4000), topk=2048, layers=1),
    "h128_split_drafts_fp8": dict(cfg=4, batch=2, ctx=(1500, 4000), topk=1024),
    "h64_split_int8": dict(cfg=2, batch=3, ctx=(2100, 4000), topk=2048, heads=64, layers=1,
                           kv_fmt=synth.FMT_INT8_AFFINE_B128),
    "h128_unsplit": dict(cfg=2, batch=200, ctx=(300, 900), topk=512, layers=1),
    "h128_prefill": dict(cfg=3, q_len=130, ctx=(1500, 1500), topk=1024, prefill=True),
    "h128_prefill_fp8": dict(cfg=3, q_len=70, ctx=(1500, 1500), topk=1024, prefill=True,
                             kv_fmt=synth.FMT_FP8_E4M3_B128),
    # 64-head groups, unsplit, more row x head-group items than CUs (several rounds)
    "h128_rounds_int8": dict(cfg=2, batch=200, ctx=(300, 900), topk=512, layers=1,
                                 kv_fmt=synth.FMT_INT8_AFFINE_B128),
    "h128_rounds_drafts_fp8": dict(cfg=4, batch=40, ctx=(1100, 3000), topk=1024),
    "h128_rounds_300_requests": dict(cfg=2, batch=300, ctx=(300, 1400), topk=600, layers=1),
    "h128_rounds_prefill_fp8": dict(cfg=3, q_len=200, ctx=(1500, 1500), topk=1024, prefill=True,
                                        kv_fmt=synth.FMT_FP8_E4M3_B128),
}


@pytest.mark.parametrize("name", list(VARIANTS))
def test_q_zero_gives_the_mean_and_log_count(name):
    from sparse_attention_07_amd.path import DSAPath
    kw = dict(VARIANTS[name])
    cfg = kw.pop("cfg")
    prefill = kw.pop("prefill", False)
    kw.setdefault("layers", 1)
    sb = synth.make_batch(cfg, device=DEV, **kw)
    sb.q[0].zero_()
    p = DSAPath(sb, prefill=prefill)
    idx = _selection(sb, seed=len(name))
    _say(name, "T=%d heads=%d K=%d prefill=%s" % (sb.T, sb.cfg.heads, sb.cfg.topk, prefill))
    p.out[0].fill_(7.0)
    p.lse[0].fill_(7.0)
    p.mla(0, idx=idx.to(DEV))
    torch.cuda.synchronize()
    mean, lse = _closed_form(sb, idx.numpy(), _decoded_rows(sb, 0))
    g_lse = p.lse[0].cpu().double().numpy()                      # [T, H]
    g_out = p.out[0].float().cpu().double().numpy()               # [T, H, dc]
    # rows with nothing usable: out = 0, lse = -inf
    assert np.all(np.isneginf(g_lse[0])) and np.all(g_out[0] == 0)
    err_lse = np.abs(g_lse[1:] - lse[1:, None])
    assert err_lse.max() <= 1e-4, "lse off by %.3g (row %s)" % (err_lse.max(), np.unravel_index(err_lse.argmax(), err_lse.shape))
    ref = mean[:, None, :]
    err = np.abs(g_out - ref)
    bound = 2.0 ** -7 * np.abs(ref) + 8e-4                        # elementwise guard
    bad = err > bound
    assert not bad.any(), "out: %d elements off, worst %.3g at %s" % (
        int(bad.sum()), float((err - bound).max()), np.unravel_index(np.argmax(err - bound), err.shape))
    n_use = np.exp(lse[1:])                                        # usable rows per query row
    l2 = np.sqrt((err[1:] ** 2).sum(-1))                           # [T-1, H]
    l2_bound = (2.0 ** -8 * np.sqrt((ref[1:] ** 2).sum(-1))
                + 0.2 * np.sqrt(sb.cfg.dc) / np.round(n_use)[:, None])
    worst = np.unravel_index(np.argmax(l2 - l2_bound), l2.shape)
    assert np.all(l2 <= l2_bound), "out: L2 error %.3g over bound %.3g at (row, head) %s" % (
        l2[worst], l2_bound[worst], (worst[0] + 1, worst[1]))
