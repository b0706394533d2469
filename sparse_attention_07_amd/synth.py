"""Seeded synthetic inputs for the DSA hot path (indexer -> top-k -> sparse MLA).

This module only draws random tensors and lays them out; it holds none of the
method's arithmetic.  Both the HIP path and the CPU oracle consume what it
produces, and neither side's arithmetic lives here.

Workloads (shapes follow the decode/prefill settings of the GLM-5.2 and
DeepSeek-V3.2 serving pages: lmdeploy PR 4737 "feat: support GLM-5.2",
section "Five-layer ablations" (batch 256 decode, BF16 MLA cache); lmdeploy
PR 4968 "add glm5.3-flash support", section "Measured optimization gains"
(MTP5, 2K/8K prefill, 128K/256K contexts); mlx-lm PR 1419, description
(index_topk 2048, IndexShare, MTP verify on the gather path)):

  tiny      1 request, 256 cached tokens, 8 draft queries, top-k 64, f32
  decode16  64 requests, contexts U[1024, 8192], 1 query, 16 MLA heads
  decode128 256 requests, contexts U[2048, 32768], 1 query, 128 heads,
            one full layer followed by two IndexShare layers
  prefill   one sequence, 16384 cached + 4096 new causal rows, 128 heads
  mtp_fp8   32 requests, contexts U[65536, 131072], 5 draft queries each,
            block-scaled e4m3 latent cache, 128 heads

Value modes:
  "parity"  indexer tensors are small integers scaled by powers of two, so
            every fp32 score is exact whatever the summation order and the
            selected indices are unique; MLA tensors ~ N(0, 1).
  "perf"    q_I, k_I ~ N(0, 1), w ~ N(0, 1)/8, q and latent ~ N(0, 1).

Randomness comes from torch generators seeded with 1000 + config number,
drawn on the device the tensors live on (Philox on the GPU, mt19937 on the
CPU).  Draw order: context lengths, page permutation, q_I, k_I, w, then per
layer q and latent.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

# Row formats shared with the C ABI (values of the format enum).
FMT_F32 = 0
FMT_BF16 = 1
FMT_FP8_E4M3_B128 = 2
FMT_INT8_AFFINE_B128 = 3

FP8_ROW_BYTES = 656       # 512 e4m3 bytes + 4 f32 block scales + 64 bf16 rope
INT8_ROW_BYTES = 672      # 512 unsigned codes + 4 f32 scales + 4 f32 biases + 64 bf16 rope
FP8_BLOCK = 128
FP8_MAX = 448.0
FP8_KEY_CODES = 128       # fp8 index keys: 128 e4m3 codes per token, page-blocked with
FP8_KEY_BYTES = 132       # one f32 scale per token (P rows of codes, then P scales)


@dataclass
class Config:
    name: str
    batch: int
    q_len: int
    ctx_lo: int                 # inclusive range of seq_len (cache length incl. queries)
    ctx_hi: int
    topk: int
    hi: int                     # indexer heads
    di: int                     # indexer head dim
    heads: int                  # MLA heads
    dc: int                     # latent dim
    dr: int                     # rope dim
    page_size: int
    kv_fmt: int
    idx_fmt: int                # q_I and k_I format
    q_fmt: int                  # MLA q and output format
    sm_scale: float
    layers: int = 1             # 1 full layer + (layers-1) IndexShare layers
    identity_pages: bool = False
    seed: int = 1000
    key_fmt: int | None = None  # k_I pool format when it differs from idx_fmt (fp8 keys)


CONFIGS = {
    0: Config("tiny", 1, 8, 256, 256, 64, 4, 32, 8, 64, 16, 16,
              FMT_F32, FMT_F32, FMT_F32, 1.0 / math.sqrt(48.0),
              identity_pages=True, seed=1000),
    1: Config("decode16", 64, 1, 1024, 8192, 2048, 64, 128, 16, 512, 64, 64,
              FMT_BF16, FMT_BF16, FMT_BF16, 1.0 / math.sqrt(192.0), seed=1001),
    2: Config("decode128", 256, 1, 2048, 32768, 2048, 64, 128, 128, 512, 64, 64,
              FMT_BF16, FMT_BF16, FMT_BF16, 1.0 / math.sqrt(192.0), layers=3,
              seed=1002),
    3: Config("prefill", 1, 4096, 20480, 20480, 2048, 64, 128, 128, 512, 64, 64,
              FMT_BF16, FMT_BF16, FMT_BF16, 1.0 / math.sqrt(192.0), seed=1003),
    4: Config("mtp_fp8", 32, 5, 65536, 131072, 2048, 64, 128, 128, 512, 64, 64,
              FMT_FP8_E4M3_B128, FMT_BF16, FMT_BF16, 1.0 / math.sqrt(192.0),
              seed=1004),
}


def torch_dtype(fmt: int) -> torch.dtype:
    return {FMT_F32: torch.float32, FMT_BF16: torch.bfloat16}[fmt]


def kv_row_bytes(fmt: int, dc: int, dr: int) -> int:
    if fmt == FMT_FP8_E4M3_B128:
        assert dc == 512 and dr == 64
        return FP8_ROW_BYTES
    if fmt == FMT_INT8_AFFINE_B128:
        assert dc == 512 and dr == 64
        return INT8_ROW_BYTES
    return (dc + dr) * (4 if fmt == FMT_F32 else 2)


@dataclass
class Batch:
    """One ragged batch: host copies of the small int arrays plus device tensors."""
    cfg: Config
    q_lens: list
    seq_lens: list
    cu_q: torch.Tensor          # int32 [B+1]
    seq_lens_t: torch.Tensor    # int32 [B]
    page_table: torch.Tensor    # int32 [B, pt_stride], -1 = unused
    num_pages: int
    q_idx: torch.Tensor         # [T, hi, di]
    w: torch.Tensor             # f32 [T, hi]
    k_pool: torch.Tensor        # [num_pages, P, di]; fp8 keys: uint8 [num_pages, P*132]
    q: list = field(default_factory=list)        # per layer [T, H, dc+dr]
    kv_pool: list = field(default_factory=list)  # per layer [num_pages, P, row] (uint8 for fp8)

    @property
    def T(self) -> int:
        return int(sum(self.q_lens))

    @property
    def B(self) -> int:
        return len(self.q_lens)

    @property
    def max_seq_len(self) -> int:
        return int(max(self.seq_lens)) if self.seq_lens else 0

    @property
    def max_q_len(self) -> int:
        return int(max(self.q_lens)) if self.q_lens else 0

    def positions(self) -> list:
        """pos(t) for every query row, as plain ints (used for sizing and sampling)."""
        out = []
        for ql, sl in zip(self.q_lens, self.seq_lens):
            out.extend(range(sl - ql, sl))
        return out

    def row_request(self) -> list:
        out = []
        for b, ql in enumerate(self.q_lens):
            out.extend([b] * ql)
        return out


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _int_scaled(shape, lo, hi, scale, g, device, dtype):
    """Integers uniform in [lo, hi] times scale (exact in bf16 and f32)."""
    x = torch.randint(lo, hi + 1, shape, generator=g, device=device, dtype=torch.int32)
    return (x.to(torch.float32) * scale).to(dtype)


def quantize_fp8_rows(latent: torch.Tensor, rope: torch.Tensor) -> torch.Tensor:
    """Pack latent [..., 512] (f32) and rope [..., 64] (bf16) into 656-byte rows.

    Layout per row: 512 e4m3fn bytes, four f32 scales (one per 128-wide block,
    scale = block amax / 448), then 64 bf16 rope values.  The e4m3 rounding is
    torch's own float8_e4m3fn conversion.
    """
    lead = latent.shape[:-1]
    blocks = latent.reshape(*lead, 4, FP8_BLOCK)
    amax = blocks.abs().amax(dim=-1, keepdim=True)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    codes = (blocks / scale).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    out = torch.empty(*lead, FP8_ROW_BYTES, dtype=torch.uint8, device=latent.device)
    out[..., :512] = codes.reshape(*lead, 512).view(torch.uint8)
    out[..., 512:528] = scale.reshape(*lead, 4).to(torch.float32).contiguous().view(torch.uint8)
    out[..., 528:656] = rope.to(torch.bfloat16).contiguous().view(torch.uint8)
    return out


def quantize_int8_rows(latent: torch.Tensor, rope: torch.Tensor) -> torch.Tensor:
    """Pack latent [..., 512] (f32) and rope [..., 64] (bf16) into 672-byte rows.

    Layout per row: 512 unsigned codes, four f32 scales, four f32 biases (one
    pair per 128-wide block: bias = block min, scale = (max - min) / 255), then
    64 bf16 rope values; code = round((x - bias) / scale), clamped to [0, 255].
    """
    lead = latent.shape[:-1]
    blocks = latent.reshape(*lead, 4, 128).to(torch.float32)
    mn = blocks.amin(dim=-1, keepdim=True)
    mx = blocks.amax(dim=-1, keepdim=True)
    scale = torch.where(mx > mn, (mx - mn) / 255.0, torch.ones_like(mx))
    codes = torch.round((blocks - mn) / scale).clamp(0, 255).to(torch.uint8)
    out = torch.empty(*lead, INT8_ROW_BYTES, dtype=torch.uint8, device=latent.device)
    out[..., :512] = codes.reshape(*lead, 512)
    out[..., 512:528] = scale.reshape(*lead, 4).contiguous().view(torch.uint8)
    out[..., 528:544] = mn.reshape(*lead, 4).contiguous().view(torch.uint8)
    out[..., 544:672] = rope.to(torch.bfloat16).contiguous().view(torch.uint8)
    return out


def fp8_key_page_bytes(P: int) -> int:
    """Bytes of one page-blocked fp8 key page of P tokens, 16-byte aligned."""
    return (P * FP8_KEY_BYTES + 15) // 16 * 16


def quantize_fp8_keys(k: torch.Tensor, scale: torch.Tensor | None = None) -> torch.Tensor:
    """Pack index keys [num_pages, P, 128] (f32) into page-blocked fp8 pages.

    Page layout: P rows of 128 e4m3fn codes, then P f32 scales, one per token
    (scale = token amax / 448 unless given as [num_pages, P]), then zero bytes
    up to a multiple of 16.  The e4m3 rounding is torch's own float8_e4m3fn
    conversion.
    """
    n, P, d = k.shape
    assert d == FP8_KEY_CODES
    if scale is None:
        amax = k.abs().amax(dim=-1)
        scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    codes = (k / scale[..., None]).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    out = torch.zeros(n, fp8_key_page_bytes(P), dtype=torch.uint8, device=k.device)
    out[:, :P * FP8_KEY_CODES] = codes.reshape(n, P * FP8_KEY_CODES).view(torch.uint8)
    out[:, P * FP8_KEY_CODES:P * FP8_KEY_BYTES] = scale.to(torch.float32).contiguous().view(torch.uint8).reshape(n, P * 4)
    return out


def make_batch(cfg_id: int, mode: str = "parity", device="cpu", layers: int | None = None,
               seed_offset: int = 0, batch: int | None = None, q_len: int | None = None,
               ctx: tuple | None = None, topk: int | None = None,
               page_size: int | None = None, identity_pages: bool | None = None,
               heads: int | None = None, kv_fmt: int | None = None,
               q_lens: list | None = None, key_fmt: int | None = None) -> Batch:
    """Draw one batch of config `cfg_id`.

    The keyword overrides (batch, q_len, ctx range, top-k, page size) give
    reduced-size variants of the same recipe for tests; the defaults are the
    full workload.  q_lens gives each request its own number of query rows
    (zero allowed; its length sets the batch size).  seed_offset picks an independent input set of the same
    shape (the bench rotates several to keep the 256 MB MALL from serving
    repeat reads).
    """
    base = CONFIGS[cfg_id]
    cfg = Config(**{**base.__dict__})
    if batch is not None:
        cfg.batch = batch
    if q_len is not None:
        cfg.q_len = q_len
    if ctx is not None:
        cfg.ctx_lo, cfg.ctx_hi = ctx
    if topk is not None:
        cfg.topk = topk
    if page_size is not None:
        cfg.page_size = page_size
    if identity_pages is not None:
        cfg.identity_pages = identity_pages
    if layers is not None:
        cfg.layers = layers
    if heads is not None:
        cfg.heads = heads
    if kv_fmt is not None:
        cfg.kv_fmt = kv_fmt
    if key_fmt is not None:
        cfg.key_fmt = key_fmt
    if q_lens is not None:
        cfg.batch = len(q_lens)
        cfg.q_len = max(q_lens)
    assert mode in ("parity", "perf")
    device = torch.device(device)
    g = _gen(device, cfg.seed + 7919 * seed_offset)
    gcpu = _gen("cpu", cfg.seed + 7919 * seed_offset)

    B, P = cfg.batch, cfg.page_size
    # context lengths (always on the CPU generator so host ints match across devices)
    if cfg.ctx_lo == cfg.ctx_hi:
        seq_lens = [cfg.ctx_lo] * B
    else:
        seq_lens = torch.randint(cfg.ctx_lo, cfg.ctx_hi + 1, (B,), generator=gcpu).tolist()
    q_lens = [int(x) for x in q_lens] if q_lens is not None else [cfg.q_len] * B
    seq_lens = [max(int(s), ql, 1) for s, ql in zip(seq_lens, q_lens)]
    pages_per = [(s + P - 1) // P for s in seq_lens]
    num_pages = sum(pages_per)
    pt_stride = max(pages_per)
    if cfg.identity_pages:
        perm = torch.arange(num_pages, dtype=torch.int32)
    else:
        perm = torch.randperm(num_pages, generator=gcpu).to(torch.int32)
    page_table = torch.full((B, pt_stride), -1, dtype=torch.int32)
    o = 0
    for b, n in enumerate(pages_per):
        page_table[b, :n] = perm[o:o + n]
        o += n
    cu = [0]
    for ql in q_lens:
        cu.append(cu[-1] + ql)
    T = cu[-1]

    idt = torch_dtype(cfg.idx_fmt)
    fp8_keys = cfg.key_fmt == FMT_FP8_E4M3_B128
    if fp8_keys:
        assert cfg.idx_fmt == FMT_BF16 and cfg.di == FP8_KEY_CODES
    if mode == "parity":
        q_idx = _int_scaled((T, cfg.hi, cfg.di), -8, 8, 1.0 / 8, g, device, idt)
        k_pool = _int_scaled((num_pages, P, cfg.di), -8, 8, 1.0 / 8, g, device,
                             torch.float32 if fp8_keys else idt)
        w = _int_scaled((T, cfg.hi), -4, 4, 1.0 / 4, g, device, torch.float32)
        if fp8_keys:  # codes are the integers themselves: exact in e4m3 with scale 1/8
            k_pool = quantize_fp8_keys(k_pool, torch.full((num_pages, P), 1.0 / 8, device=device))
    else:
        q_idx = torch.randn((T, cfg.hi, cfg.di), generator=g, device=device).to(idt)
        k_pool = torch.randn((num_pages, P, cfg.di), generator=g, device=device)
        k_pool = quantize_fp8_keys(k_pool) if fp8_keys else k_pool.to(idt)
        w = torch.randn((T, cfg.hi), generator=g, device=device) / 8.0

    D = cfg.dc + cfg.dr
    qdt = torch_dtype(cfg.q_fmt)
    qs, kvs = [], []
    for _ in range(cfg.layers):
        qs.append(torch.randn((T, cfg.heads, D), generator=g, device=device).to(qdt))
        if cfg.kv_fmt in (FMT_FP8_E4M3_B128, FMT_INT8_AFFINE_B128):
            lat = torch.randn((num_pages, P, cfg.dc), generator=g, device=device)
            rope = torch.randn((num_pages, P, cfg.dr), generator=g, device=device)
            kvs.append(quantize_fp8_rows(lat, rope) if cfg.kv_fmt == FMT_FP8_E4M3_B128
                       else quantize_int8_rows(lat, rope))
            del lat, rope
        else:
            kvs.append(torch.randn((num_pages, P, D), generator=g, device=device)
                       .to(torch_dtype(cfg.kv_fmt)))

    return Batch(cfg=cfg, q_lens=q_lens, seq_lens=seq_lens,
                 cu_q=torch.tensor(cu, dtype=torch.int32, device=device),
                 seq_lens_t=torch.tensor(seq_lens, dtype=torch.int32, device=device),
                 page_table=page_table.to(device), num_pages=num_pages,
                 q_idx=q_idx, w=w, k_pool=k_pool, q=qs, kv_pool=kvs)


@dataclass
class Prep:
    """Inputs of the indexer preparation for one batch's new rows."""
    q_in: torch.Tensor      # [T, hi, di] indexer queries before RoPE (idx dtype)
    k_in: torch.Tensor      # [T, di] indexer keys before LayerNorm and RoPE (idx dtype)
    gamma: torch.Tensor     # f32 [di] LayerNorm weight
    beta: torch.Tensor      # f32 [di] LayerNorm bias
    eps: float
    cos: torch.Tensor       # f32 [rows, rope_dim/2], row p = position p
    sin: torch.Tensor
    rope_dim: int
    interleaved: bool


def rope_tables(rows: int, rope_dim: int, theta: float = 10000.0, device="cpu", dtype=torch.float32):
    """The usual rotary tables: angle(p, i) = p * theta^(-2i/rope_dim), computed
    in float64 and stored as cosines and sines [rows, rope_dim/2] (f32 unless
    another dtype is asked for)."""
    i = torch.arange(rope_dim // 2, dtype=torch.float64)
    inv = theta ** (-2.0 * i / rope_dim)
    ang = torch.arange(rows, dtype=torch.float64)[:, None] * inv[None, :]
    return (torch.cos(ang).to(dtype).to(device), torch.sin(ang).to(dtype).to(device))


def make_prep(batch: Batch, rope_dim: int | None = None, interleaved: bool = False,
              eps: float = 1e-6, seed: int = 4242, device=None) -> Prep:
    """Draw the preparation inputs for `batch`'s rows.  Defaults follow the GLM
    indexer (non-interleaved RoPE over half the head, eps 1e-6); its own seed,
    so the batch's draws do not change.  Keys get a non-zero mean and spread so
    the LayerNorm has work to do."""
    cfg = batch.cfg
    device = device or batch.q_idx.device
    g = _gen(device, seed)
    dt = torch_dtype(cfg.idx_fmt)
    R = cfg.di // 2 if rope_dim is None else rope_dim
    T = batch.T
    q_in = torch.randn((T, cfg.hi, cfg.di), generator=g, device=device).to(dt)
    k_in = (torch.randn((T, cfg.di), generator=g, device=device) * 2.0 + 0.5).to(dt)
    gamma = 1.0 + 0.25 * torch.randn((cfg.di,), generator=g, device=device)
    beta = 0.1 * torch.randn((cfg.di,), generator=g, device=device)
    cos, sin = rope_tables(max(batch.max_seq_len, 1), R, device=device)
    return Prep(q_in=q_in, k_in=k_in, gamma=gamma, beta=beta, eps=eps, cos=cos, sin=sin,
                rope_dim=R, interleaved=interleaved)


def repage(batch: Batch, new_page_size: int, identity: bool, seed: int = 77) -> Batch:
    """Same token contents under another page size / page order (paging invariance)."""
    cfg = Config(**{**batch.cfg.__dict__})
    assert cfg.key_fmt in (None, cfg.idx_fmt), "page-blocked fp8 key pools are not re-paged"
    P0, P1 = cfg.page_size, new_page_size
    cfg.page_size = P1
    B = batch.B
    pages_per = [(s + P1 - 1) // P1 for s in batch.seq_lens]
    num_pages = sum(pages_per)
    g = _gen("cpu", seed)
    perm = (torch.arange(num_pages, dtype=torch.int32) if identity
            else torch.randperm(num_pages, generator=g).to(torch.int32))
    pt = torch.full((B, max(pages_per)), -1, dtype=torch.int32)
    o = 0
    for b, n in enumerate(pages_per):
        pt[b, :n] = perm[o:o + n]
        o += n
    old_pt = batch.page_table.cpu()

    def move(pool):
        pool = pool.cpu()
        tail = pool.shape[2:]
        new = torch.zeros((num_pages, P1) + tuple(tail), dtype=pool.dtype)
        for b, sl in enumerate(batch.seq_lens):
            s = torch.arange(sl)
            src = pool[old_pt[b, s // P0].long(), s % P0]
            new[pt[b, s // P1].long(), s % P1] = src
        return new

    return Batch(cfg=cfg, q_lens=list(batch.q_lens), seq_lens=list(batch.seq_lens),
                 cu_q=batch.cu_q.cpu().clone(), seq_lens_t=batch.seq_lens_t.cpu().clone(),
                 page_table=pt, num_pages=num_pages,
                 q_idx=batch.q_idx.cpu(), w=batch.w.cpu(), k_pool=move(batch.k_pool),
                 q=[x.cpu() for x in batch.q], kv_pool=[move(x) for x in batch.kv_pool])
