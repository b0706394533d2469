"""GPU path vs the CPU oracle, through the C ABI (needs an MI355X).

Indices must match bit-exactly (indexer tensors are drawn as small
power-of-two-scaled integers, so every fp32 score is exact); scores must equal
the oracle's exactly; attention outputs and lse within
|g - r| <= atol + 1e-2 |r| (atol 2e-2 bf16, 6e-2 fp8 or int8 cache, 1e-4 f32).
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


def _run(sb, prefill=None):
    from sparse_attention_07_amd.path import DSAPath
    p = DSAPath(sb, prefill=prefill)
    p.step()
    torch.cuda.synchronize()
    return p


def test_tiny_full_path():
    sb = synth.make_batch(0, device=DEV)
    _say("tiny config, all rows")
    p = _run(sb)
    _parity.check_path(sb, p)


REDUCED = {
    "decode16": dict(cfg=1, batch=6, ctx=(100, 3000), topk=512),
    "decode16_p16": dict(cfg=1, batch=5, ctx=(1, 2100), topk=256, page_size=16),
    "decode16_p5": dict(cfg=1, batch=4, ctx=(300, 1300), topk=256, page_size=5),
    "decode128_share": dict(cfg=2, batch=5, ctx=(600, 5000), topk=512, layers=3),
    "prefill": dict(cfg=3, q_len=300, ctx=(2000, 2000), topk=512),
    "prefill_short": dict(cfg=3, q_len=130, ctx=(700, 700), topk=512),
    "mtp_fp8": dict(cfg=4, batch=3, ctx=(3000, 9000), topk=512),
    "mtp_fp8_near_k": dict(cfg=4, batch=4, ctx=(509, 516), topk=512),
    # head counts and cache formats outside the five workloads (kernel dispatch coverage)
    "decode16_fp8": dict(cfg=1, batch=5, ctx=(300, 3000), topk=512, kv_fmt=synth.FMT_FP8_E4M3_B128),
    "decode_h32": dict(cfg=1, batch=3, ctx=(500, 2500), topk=256, heads=32),
    "decode_h48": dict(cfg=1, batch=3, ctx=(500, 2500), topk=256, heads=48),
    "decode_h64_fp8": dict(cfg=2, batch=3, ctx=(900, 3000), topk=512, heads=64, layers=1,
                           kv_fmt=synth.FMT_FP8_E4M3_B128),
    "decode_h16_split_ragged": dict(cfg=1, batch=7, ctx=(1, 700), topk=640),
    # requests with no rows and mixed draft lengths; more than 256 requests
    "ragged_q_lens_empty": dict(cfg=4, q_lens=[5, 0, 3, 1, 0, 5, 2], ctx=(600, 3000), topk=512),
    "many_requests": dict(cfg=1, batch=300, ctx=(40, 700), topk=256),
    # affine int8 latent cache: 16-head groups, 64-head groups, drafts, prefill, page size 5
    "decode16_int8": dict(cfg=1, batch=5, ctx=(300, 3000), topk=512, kv_fmt=synth.FMT_INT8_AFFINE_B128),
    "decode16_p5_int8": dict(cfg=1, batch=4, ctx=(300, 1300), topk=256, page_size=5,
                             kv_fmt=synth.FMT_INT8_AFFINE_B128),
    "decode_h64_int8": dict(cfg=2, batch=3, ctx=(900, 3000), topk=512, heads=64, layers=1,
                            kv_fmt=synth.FMT_INT8_AFFINE_B128),
    "mtp_int8": dict(cfg=4, batch=3, ctx=(3000, 9000), topk=512, kv_fmt=synth.FMT_INT8_AFFINE_B128),
    "prefill_int8": dict(cfg=3, q_len=130, ctx=(700, 700), topk=512, kv_fmt=synth.FMT_INT8_AFFINE_B128),
    # fp8 index keys (one scale per token) under bf16 queries: decode, drafts, prefill rows
    "decode16_fp8_keys": dict(cfg=1, batch=6, ctx=(100, 3000), topk=512, key_fmt=synth.FMT_FP8_E4M3_B128),
    "decode16_p5_fp8_keys": dict(cfg=1, batch=4, ctx=(300, 1300), topk=256, page_size=5,
                                 key_fmt=synth.FMT_FP8_E4M3_B128),
    "mtp_fp8_keys": dict(cfg=4, batch=3, ctx=(3000, 9000), topk=512, key_fmt=synth.FMT_FP8_E4M3_B128),
    "ragged_fp8_keys": dict(cfg=4, q_lens=[5, 0, 3, 1, 0, 5, 2], ctx=(600, 3000), topk=512,
                            key_fmt=synth.FMT_FP8_E4M3_B128),
    "prefill_fp8_keys": dict(cfg=3, q_len=130, ctx=(700, 700), topk=512, key_fmt=synth.FMT_FP8_E4M3_B128),
    # 16-head groups with draft rows (causal inside the draft), over each cache format, and 16-head prefill
    "decode16_drafts": dict(cfg=1, batch=4, q_len=5, ctx=(300, 3000), topk=512),
    "decode16_drafts_fp8": dict(cfg=1, batch=3, q_len=5, ctx=(300, 3000), topk=512,
                                kv_fmt=synth.FMT_FP8_E4M3_B128),
    "decode16_drafts_int8": dict(cfg=1, batch=3, q_len=5, ctx=(509, 516), topk=512,
                                 kv_fmt=synth.FMT_INT8_AFFINE_B128),
    "prefill_h16": dict(cfg=3, q_len=100, ctx=(700, 700), topk=512, heads=16),
}


@pytest.mark.parametrize("name", list(REDUCED))
def test_reduced_configs_all_rows(name):
    kw = dict(REDUCED[name])
    cfg = kw.pop("cfg")
    sb = synth.make_batch(cfg, device=DEV, **kw)
    _say(name, "T=%d B=%d max_seq=%d" % (sb.T, sb.B, sb.max_seq_len))
    p = _run(sb)
    _parity.check_path(sb, p)


def _sample_rows(sb, n=6):
    pos = sb.positions()
    T = sb.T
    picks = {0, T - 1, int(np.argmax(pos)), int(np.argmin(pos))}
    g = np.random.default_rng(123)
    while len(picks) < min(n, T):
        picks.add(int(g.integers(0, T)))
    return sorted(picks)


@pytest.mark.slow
@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_full_size_sampled_rows(cfg):
    sb = synth.make_batch(cfg, device=DEV)
    _say("full config", cfg, synth.CONFIGS[cfg].name, "T=%d B=%d max_seq=%d" % (sb.T, sb.B, sb.max_seq_len))
    p = _run(sb)
    rows = _sample_rows(sb)
    _parity.check_path(sb, p, rows=rows)
    # every row: indices ascending, valid count = min(K, pos+1), all within [0, pos]
    idx = p.idx.cpu().numpy()
    pos = np.array(sb.positions())
    K = sb.cfg.topk
    nvalid = (idx >= 0).sum(1)
    assert np.array_equal(nvalid, np.minimum(K, pos + 1))
    for t in range(0, sb.T, max(1, sb.T // 64)):
        v = idx[t, :nvalid[t]]
        assert np.all(np.diff(v) > 0) and v[0] >= 0 and v[-1] <= pos[t]
        assert np.all(idx[t, nvalid[t]:] == -1)
    for out in p.out:
        assert torch.isfinite(out.float()).all()


def _row_batch(scores_rows, K):
    """One request per score row, q_len 1, seq_len = row length."""
    n = [len(r) for r in scores_rows]
    sb = synth.make_batch(1, batch=len(n), ctx=(1, 1), topk=K, layers=0)
    sb.seq_lens = n
    sb.q_lens = [1] * len(n)
    sb.seq_lens_t = torch.tensor(n, dtype=torch.int32)
    sb.cu_q = torch.arange(len(n) + 1, dtype=torch.int32)
    sb.page_table = torch.zeros((len(n), 1), dtype=torch.int32)
    return sb


@pytest.mark.parametrize("K", [1, 7, 64, 2048])
def test_topk_ties_and_lengths(K):
    from sparse_attention_07_amd import dsa
    g = torch.Generator().manual_seed(K)
    lens = [1, K - 1 if K > 1 else 1, K, K + 1, 3 * K + 5, 1000, 32768, 32769, 70001]
    rows = []
    for i, n in enumerate(lens):
        if i % 3 == 0:
            r = torch.randint(-3, 4, (n,), generator=g).float() / 2       # heavy ties
        elif i % 3 == 1:
            r = torch.randint(-1000, 1000, (n,), generator=g).float() / 64
        else:
            r = torch.zeros(n)                                              # all equal
        r[::13] = -0.0
        rows.append(r)
    sb = _row_batch(rows, K)
    ld = max(lens)
    scores = torch.full((len(rows), ld), float("nan"))
    for i, r in enumerate(rows):
        scores[i, :len(r)] = r
    ref = oracle.topk(sb, scores.double().numpy(), k=K)
    _say("topk ties K=%d" % K)
    b = dsa.make_batch(sb.cu_q.to(DEV), sb.seq_lens_t.to(DEV), sb.page_table.to(DEV), len(rows), 1,
                       ld, 16, 1)
    sd = scores.to(DEV)
    idx = torch.full((len(rows), K), 12345, dtype=torch.int32, device=DEV)
    # rows past 32768 entries take the two-level selection (segments, then candidates)
    ws_bytes = dsa.dsa_topk_workspace_bytes(len(rows), ld, K)
    assert ws_bytes > 0
    ws = torch.full((ws_bytes,), 0xAB, dtype=torch.uint8, device=DEV)   # stale contents must not matter
    dsa.dsa_topk(b, sd, ld, K, idx, ws, ws_bytes)
    torch.cuda.synchronize()
    _parity.check_idx_exact(idx, ref)


@pytest.mark.parametrize("K", [5, 2048])
def test_topk_rows_read_before_their_length_is_known(K):
    # ld <= 32768: each row's whole storage is read before its length is known;
    # entries past the length hold NaN and +-inf here and must not matter.
    from sparse_attention_07_amd import dsa
    g = torch.Generator().manual_seed(100 + K)
    lens = [1, K, K + 1, 3 * K + 5, 1000, 4097, 20000, 32767, 32768]
    ld = 32768
    scores = torch.full((len(lens), ld), float("nan"))
    scores[:, 1::7] = float("inf")
    scores[:, 2::7] = -float("inf")
    rows = []
    for i, n in enumerate(lens):
        r = (torch.randint(-3, 4, (n,), generator=g).float() / 2 if i % 2 else
             torch.randint(-1000, 1000, (n,), generator=g).float() / 64)
        scores[i, :n] = r
        rows.append(r)
    sb = _row_batch(rows, K)
    ref = oracle.topk(sb, np.where(np.isfinite(scores.numpy()), scores.numpy(), 0.0).astype(np.float64), k=K)
    _say("topk early read K=%d" % K)
    b = dsa.make_batch(sb.cu_q.to(DEV), sb.seq_lens_t.to(DEV), sb.page_table.to(DEV), len(rows), 1,
                       ld, 16, 1)
    idx = torch.full((len(rows), K), 12345, dtype=torch.int32, device=DEV)
    assert dsa.dsa_topk_workspace_bytes(len(rows), ld, K) == 0   # single level
    dsa.dsa_topk(b, scores.to(DEV), ld, K, idx, None, 0)
    torch.cuda.synchronize()
    _parity.check_idx_exact(idx, ref)


@pytest.mark.parametrize("K", [7, 2048])
def test_topk_persistent_rows(K):
    # More rows than CUs: workgroups walk several rows each and read the next
    # row ahead.  Rows of mixed lengths (some with n <= K), ties, NaN and
    # +-inf past each length; each row its own request, so the lookup also
    # goes past its first round of 64 requests.
    from sparse_attention_07_amd import dsa
    g = torch.Generator().manual_seed(300 + K)
    cycle = [1, K - 1, K, K + 1, 3 * K + 5, 1000, 4097, 20000, 32767, 32768]
    lens = [max(1, cycle[i % len(cycle)]) for i in range(600)]
    ld = 32768
    scores = torch.full((len(lens), ld), float("nan"))
    scores[:, 1::7] = float("inf")
    scores[:, 2::7] = -float("inf")
    rows = []
    for i, n in enumerate(lens):
        if i % 3 == 0:
            r = torch.randint(-3, 4, (n,), generator=g).float() / 2
        elif i % 3 == 1:
            r = torch.randint(-1000, 1000, (n,), generator=g).float() / 64
        else:
            r = torch.randn(n, generator=g)
        r[::13] = -0.0
        scores[i, :n] = r
        rows.append(r)
    sb = _row_batch(rows, K)
    ref = oracle.topk(sb, np.where(np.isfinite(scores.numpy()), scores.numpy(), 0.0).astype(np.float64), k=K)
    _say("topk persistent rows K=%d" % K)
    b = dsa.make_batch(sb.cu_q.to(DEV), sb.seq_lens_t.to(DEV), sb.page_table.to(DEV), len(rows), 1,
                       ld, 16, 1)
    idx = torch.full((len(rows), K), 12345, dtype=torch.int32, device=DEV)
    dsa.dsa_topk(b, scores.to(DEV), ld, K, idx, None, 0)
    torch.cuda.synchronize()
    _parity.check_idx_exact(idx, ref)


@pytest.mark.parametrize("K", [64, 2048])
def test_topk_many_segments(K):
    # Rows longer than the LDS cache in more (row, segment) items than CUs,
    # short rows and rows ending inside a segment included, stale workspace.
    from sparse_attention_07_amd import dsa
    g = torch.Generator().manual_seed(400 + K)
    cycle = [70001, 32769, 65536, 40000, K + 1, 1, 69999, 32768, 50001, 3 * K + 5]
    lens = [cycle[i % len(cycle)] for i in range(100)]
    ld = 70004
    scores = torch.full((len(lens), ld), float("nan"))
    rows = []
    for i, n in enumerate(lens):
        r = (torch.randint(-3, 4, (n,), generator=g).float() / 2 if i % 2 else torch.randn(n, generator=g))
        scores[i, :n] = r
        rows.append(r)
    sb = _row_batch(rows, K)
    ref = oracle.topk(sb, np.where(np.isfinite(scores.numpy()), scores.numpy(), 0.0).astype(np.float64), k=K)
    _say("topk persistent segments K=%d" % K)
    b = dsa.make_batch(sb.cu_q.to(DEV), sb.seq_lens_t.to(DEV), sb.page_table.to(DEV), len(rows), 1,
                       ld, 16, 1)
    idx = torch.full((len(rows), K), 12345, dtype=torch.int32, device=DEV)
    ws_bytes = dsa.dsa_topk_workspace_bytes(len(rows), ld, K)
    assert ws_bytes > 0
    ws = torch.full((ws_bytes,), 0xAB, dtype=torch.uint8, device=DEV)
    dsa.dsa_topk(b, scores.to(DEV), ld, K, idx, ws, ws_bytes)
    torch.cuda.synchronize()
    _parity.check_idx_exact(idx, ref)


def test_mla_invalid_entries_and_closed_forms():
    from sparse_attention_07_amd import dsa
    from sparse_attention_07_amd.path import DSAPath
    sb = synth.make_batch(1, batch=4, ctx=(300, 900), topk=64, device=DEV)
    p = DSAPath(sb)
    K = sb.cfg.topk
    pos = sb.positions()
    g = torch.Generator().manual_seed(3)
    idx = torch.full((sb.T, K), -1, dtype=torch.int32)
    for t in range(sb.T):
        if t == 0:
            continue                                       # no usable entry at all
        sel = torch.randperm(pos[t] + 1, generator=g)[:K - 8].to(torch.int32)
        if t == 1:
            sel = sel[:1]                                  # a single row: out = that latent
        junk = torch.tensor([-1, -7, pos[t] + 1, pos[t] + 100, 2 ** 30, -1, -1, -1], dtype=torch.int32)
        idx[t, :len(sel)] = sel
        idx[t, len(sel):len(sel) + 8] = junk
    idx_d = idx.to(DEV)
    _say("mla with invalid entries")
    p.mla(0, idx=idx_d)
    torch.cuda.synchronize()
    out, lse = oracle.sparse_mla(sb, 0, idx.numpy())
    _parity.assert_within(p.out[0].float().cpu().numpy(), out, _parity.ATOL_BF16, what="out")
    _parity.assert_within(p.lse[0].cpu().numpy(), lse, _parity.ATOL_BF16, what="lse")
    assert torch.all(p.out[0][0] == 0) and torch.all(torch.isneginf(p.lse[0][0]))


def test_empty_batch_is_a_no_op():
    from sparse_attention_07_amd import dsa
    sb = synth.make_batch(1, batch=2, ctx=(100, 200), topk=64, device=DEV)
    b = dsa.batch_from(sb)
    b.num_q_rows = 0
    scores = torch.full((2, 256), 7.0, device=DEV)
    idx = torch.full((2, 64), 9, dtype=torch.int32, device=DEV)
    out = torch.full((2, 16, 512), 3.0, dtype=torch.bfloat16, device=DEV)
    kp = dsa.make_pool(sb.k_pool, sb.cfg.idx_fmt, 128)
    kv = dsa.make_pool(sb.kv_pool[0], sb.cfg.kv_fmt, 576)
    dsa.dsa_index_scores(b, sb.q_idx, 1, sb.w, kp, 64, 128, scores, 256)
    dsa.dsa_topk(b, scores, 256, 64, idx)
    dsa.dsa_sparse_mla_decode(b, sb.q[0], 1, kv, idx, 64, 16, 512, 64, 0.1, out)
    torch.cuda.synchronize()
    assert torch.all(scores == 7.0) and torch.all(idx == 9) and torch.all(out == 3.0)


def test_determinism_bitwise():
    sb = synth.make_batch(4, batch=3, ctx=(3000, 6000), topk=512, mode="perf", device=DEV)
    _say("determinism")
    a = _run(sb)
    b = _run(sb)
    for t, pos in enumerate(sb.positions()):        # entries beyond pos are never written
        assert torch.equal(a.scores[t, :pos + 1], b.scores[t, :pos + 1])
    assert torch.equal(a.idx, b.idx)
    assert torch.equal(a.out[0], b.out[0]) and torch.equal(a.lse[0], b.lse[0])


def test_perf_mode_index_overlap():
    """Real-valued draws: fp32 summation order may move boundary picks; overlap stays near 1."""
    sb = synth.make_batch(1, batch=8, ctx=(3000, 8192), mode="perf", device=DEV)
    _say("perf-mode overlap")
    p = _run(sb)
    rows = [0, 3, 7]
    ref_scores = oracle.index_scores(sb, rows, ld=p.ld)
    ref_idx = oracle.topk(sb, ref_scores, rows=rows)
    g_idx = p.idx.cpu().numpy()[rows]
    for i in range(len(rows)):
        a = set(g_idx[i][g_idx[i] >= 0].tolist())
        b = set(ref_idx[i][ref_idx[i] >= 0].tolist())
        assert len(a & b) >= 0.99 * len(b)
        n = sb.positions()[rows[i]] + 1
        g = p.scores[rows[i], :n].double().cpu().numpy()
        r = ref_scores[i, :n]
        assert np.max(np.abs(g - r)) <= 1e-3 * max(1.0, np.max(np.abs(r)))


def test_graph_replay_matches_eager():
    """A captured step replays to the eager result bitwise, replay after replay."""
    from sparse_attention_07_amd.path import DSAPath
    sb = synth.make_batch(2, batch=6, ctx=(600, 4000), topk=512, layers=2, mode="perf", device=DEV)
    p = DSAPath(sb)
    p.step()
    torch.cuda.synchronize()
    ref = [p.idx.clone()] + [o.clone() for o in p.out] + [l.clone() for l in p.lse]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        p.step()
    for rep in range(3):
        for t in [p.idx] + p.out + p.lse:
            t.fill_(7)                                    # eager work between replays
        torch.cuda.synchronize()
        _say("graph replay", rep)
        g.replay()
        torch.cuda.synchronize()
        got = [p.idx] + p.out + p.lse
        for a, b in zip(got, ref):
            assert torch.equal(a, b), "replay %d differs" % rep


@pytest.mark.parametrize("case", ["prep_fp8keys_bounded", "long_rows_int8"])
def test_graph_replay_new_paths(case):
    """The preparation (fp8 key stores), bounded scoring and the two-level top-k
    replay from a captured graph to the eager result bitwise; scratch buffers get
    junk between replays."""
    from sparse_attention_07_amd.path import DSAPath
    if case == "prep_fp8keys_bounded":
        sb = synth.make_batch(1, batch=6, ctx=(600, 4000), topk=512, layers=1, mode="perf", device=DEV,
                              key_fmt=synth.FMT_FP8_E4M3_B128)
        row_bytes = (sb.max_seq_len + 63) // 64 * 64 * 4
        p = DSAPath(sb, prep=synth.make_prep(sb), score_budget=3 * row_bytes)   # 2 chunks of 3 rows
        assert p.itk_ws_bytes == 3 * row_bytes
    else:
        sb = synth.make_batch(4, batch=2, ctx=(40000, 70000), topk=512, layers=2, mode="perf", device=DEV,
                              kv_fmt=synth.FMT_INT8_AFFINE_B128)
        p = DSAPath(sb)
        assert p.topk_ws_bytes > 0                                               # two-level selection
    p.step()
    torch.cuda.synchronize()
    outs = [p.idx, sb.q_idx, sb.k_pool] + p.out + p.lse
    ref = [t.clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        p.step()
    for rep in range(3):
        for t in [p.idx] + p.out + p.lse:
            t.fill_(7)                                    # eager work between replays
        p.scores.fill_(float("nan"))
        if p.itk_ws_bytes:
            p.itk_ws.fill_(float("nan"))
        if p.topk_ws is not None:
            p.topk_ws.fill_(0xAB)
        torch.cuda.synchronize()
        _say("graph replay", case, rep)
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), "replay %d differs" % rep


FP8_KEY_CASES = {
    "decode16": dict(cfg=1, batch=6, ctx=(100, 3000), topk=512),
    "mtp_drafts": dict(cfg=4, batch=3, ctx=(3000, 9000), topk=512),
    "prefill_rows": dict(cfg=3, q_len=130, ctx=(2000, 2000), topk=512),
}


@pytest.mark.parametrize("name", list(FP8_KEY_CASES))
def test_fp8_keys_at_quantiser_scales(name):
    """fp8 index keys with each token's own amax/448 scale (the quantiser's
    regime, not the exact power-of-two scale of the integer draws).  The kernel
    applies a token's scale to its finished score, the oracle to the key: equal
    in exact arithmetic, so scores agree to f32 rounding and the selections
    overlap almost entirely."""
    from sparse_attention_07_amd.path import DSAPath
    kw = dict(FP8_KEY_CASES[name])
    cfg = kw.pop("cfg")
    sb = synth.make_batch(cfg, device=DEV, mode="perf", layers=0, key_fmt=synth.FMT_FP8_E4M3_B128, **kw)
    _say("fp8 keys at quantiser scales", name, "T=%d" % sb.T)
    p = DSAPath(sb)
    p.index_scores()
    p.topk()
    torch.cuda.synchronize()
    rows = _sample_rows(sb, n=8)
    ref_scores = oracle.index_scores(sb, rows, ld=p.ld)
    ref_idx = oracle.topk(sb, ref_scores, rows=rows)
    g_idx = p.idx.cpu().numpy()[rows]
    pos = sb.positions()
    for i, t in enumerate(rows):
        n = pos[t] + 1
        g = p.scores[t, :n].double().cpu().numpy()
        r = ref_scores[i, :n]
        assert np.max(np.abs(g - r)) <= 1e-3 * max(1.0, np.max(np.abs(r))), "row %d scores" % t
        a = set(g_idx[i][g_idx[i] >= 0].tolist())
        b = set(ref_idx[i][ref_idx[i] >= 0].tolist())
        assert len(a) == len(b) == min(n, sb.cfg.topk)
        assert len(a & b) >= 0.99 * len(b), "row %d overlap %d of %d" % (t, len(a & b), len(b))


def _grid_form_reached(B, max_q_len):
    """The persistent indexer stages its unit tables in LDS next to at least one
    unit of query rows; batches whose tables leave no room for one unit run the
    grid-form kernel instead.  (Rule of the indexer's launcher: tables of
    4B + 5 units + 10 ints, one unit = rows of 64 x 128 bf16 plus 64 f32
    weights each.)"""
    rg = max_q_len if max_q_len <= 8 else 8
    units = B * ((max_q_len + rg - 1) // rg)
    tables = ((4 * B + 1 + 5 * units + 1 + 8) * 4 + 15) // 16 * 16
    per_unit = rg * (64 * 128 * 2 + 64 * 4)
    return tables + per_unit > 160 * 1024


@pytest.mark.parametrize("key_fmt,drafts", [(None, False), (synth.FMT_FP8_E4M3_B128, True)])
def test_grid_form_indexer(key_fmt, drafts):
    """More than ~4000 requests: the grid-form indexer kernel, bit-exact."""
    from sparse_attention_07_amd.path import DSAPath
    B = 4200
    kw = dict(ctx=(1, 64), topk=16, layers=0)
    if drafts:
        kw["q_lens"] = [1 + (b * 7) % 3 for b in range(B)]
    else:
        kw["batch"] = B
    if key_fmt is not None:
        kw["key_fmt"] = key_fmt
    sb = synth.make_batch(1, device=DEV, **kw)
    assert _grid_form_reached(sb.B, sb.max_q_len)
    _say("grid-form indexer B=%d T=%d fp8 keys=%s" % (sb.B, sb.T, key_fmt is not None))
    p = DSAPath(sb)
    p.scores.fill_(float("nan"))
    p.index_scores()
    p.topk()
    torch.cuda.synchronize()
    rows = list(range(sb.T))
    ref_scores = oracle.index_scores(sb, rows, ld=p.ld)
    _parity.check_scores_exact(p.scores, ref_scores, sb.positions())
    _parity.check_idx_exact(p.idx, oracle.topk(sb, ref_scores, rows=rows))


def test_one_workspace_serves_every_shape():
    """One zero-filled workspace, sized for the largest call, reused by decode
    calls of different row counts, head counts and cache formats in turn (each
    a different split plan and partial layout): every result matches the
    oracle, so the arrival counters never start from stale partials."""
    from sparse_attention_07_amd import dsa
    from sparse_attention_07_amd.path import DSAPath
    shapes = [
        ("h16 T=100 bf16", dict(cfg=1, batch=100, ctx=(1100, 3000), topk=1024)),
        ("h16 T=64 bf16", dict(cfg=1, batch=64, ctx=(1100, 3000), topk=1024)),
        ("h16 T=64 fp8", dict(cfg=1, batch=64, ctx=(1100, 3000), topk=1024, kv_fmt=synth.FMT_FP8_E4M3_B128)),
        ("h128 T=40 bf16", dict(cfg=2, batch=40, ctx=(1100, 3000), topk=1024, layers=1)),
        ("h16 T=100 int8", dict(cfg=1, batch=100, ctx=(1100, 3000), topk=1024, kv_fmt=synth.FMT_INT8_AFFINE_B128)),
        ("h128 T=64 bf16", dict(cfg=2, batch=64, ctx=(1100, 3000), topk=1024, layers=1)),
        ("h16 T=64 bf16 again", dict(cfg=1, batch=64, ctx=(1100, 3000), topk=1024)),
    ]
    batches = []
    for name, kw in shapes:
        kw = dict(kw)
        cfg = kw.pop("cfg")
        batches.append((name, synth.make_batch(cfg, device=DEV, **kw)))
    need = max(dsa.dsa_sparse_mla_workspace_bytes(sb.T, sb.cfg.heads, sb.cfg.topk, 512, False)
               for _, sb in batches)
    ws = torch.zeros((need,), dtype=torch.uint8, device=DEV)
    for name, sb in batches:
        p = DSAPath(sb, prefill=False)
        p.ws, p.ws_bytes = ws, need
        assert dsa.dsa_sparse_mla_workspace_bytes(sb.T, sb.cfg.heads, sb.cfg.topk, 512, False) > 0
        _say("shared workspace:", name)
        p.step()
        torch.cuda.synchronize()
        _parity.check_path(sb, p, rows=_sample_rows(sb, n=6))
    assert torch.all(ws[:4096] == 0), "arrival counters left non-zero"
