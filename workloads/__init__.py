"""Seeded synthetic inputs for decode attention.

This module only draws and lays out inputs: it holds none of the attention
arithmetic, and both the GPU library's tests and the oracle read what it makes.
Two seeds drive every workload: a *data* seed for the values of q, k and v and
a *structure* seed for sequence lengths, the keys that get a score offset and
the physical page permutation. Structure is drawn on the CPU, so it is the same
whatever device the values land on.

Layouts:
  q                  [B][Hq][D], or [B][q_len][Hq][D] for a multi-token step
  contiguous k, v    [B][Hkv][cap][D]         (cap >= every L_b)
  paged pool k, v    [num_pages][Hkv][P][D]   with block_table int32 [B][max_pages]
Keys at or past L_b (and unused slots of a sequence's last page) hold NaN, so a
leak of any of them into a result shows.

fp8 (float8_e4m3fn) caches: KV head h's keys are drawn as N(0, sigma_h^2),
with sigma_h drawn from U[0.5, 2] by the structure seed, and stored as
round(k / k_scale_h) with k_scale_h = sigma_h / 64 (so that +-7 sigma stays
inside the format's +-448), the usual per-head-scale quantisation of a KV
cache; values the same way with their own sigma. Past L_b they hold the
format's NaN code (0x7f). q is bf16.

Score offsets: the workloads that ask for keys with a raised score get it
through K alone, k_j <- k_j + delta * q / (scale * |q|^2), so that
scale * <q, k_j> grows by delta before rounding K to its storage type. This
needs one query head per KV head (MHA).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass
class DecodeInputs:
    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    seq_lens: torch.Tensor            # int32 [B], on the device of q
    seq_lens_host: list
    scale: float
    max_seq_len: int
    out_dtype: torch.dtype
    page_size: int = 0
    block_table: torch.Tensor | None = None   # int32 [B][max_pages], on the device of q
    num_pages: int = 0
    num_splits: int = 0                        # 0: let the planner choose
    offset_keys: dict = field(default_factory=dict)   # (b, kv head) -> list of key indices
    data_seed: int = 0
    struct_seed: int = 0
    k_scale: torch.Tensor | None = None        # fp8: float32 [Hkv], on the device of q
    v_scale: torch.Tensor | None = None

    @property
    def batch(self) -> int:
        return self.q.shape[0]

    @property
    def q_len(self) -> int:
        return self.q.shape[1] if self.q.dim() == 4 else 1

    @property
    def num_q_heads(self) -> int:
        return self.q.shape[-2]

    @property
    def num_kv_heads(self) -> int:
        return self.k.shape[1]

    @property
    def head_dim(self) -> int:
        return self.q.shape[-1]

    @property
    def kv_bytes(self) -> int:
        """Counted K+V bytes of one decode step: valid keys only."""
        return sum(self.seq_lens_host) * self.num_kv_heads * self.head_dim * 2 * self.k.element_size()

    def describe(self) -> dict:
        return {"workload": self.name, "batch": self.batch, "num_q_heads": self.num_q_heads,
                "num_kv_heads": self.num_kv_heads, "head_dim": self.head_dim,
                "max_seq_len": self.max_seq_len, "page_size": self.page_size,
                "kv_dtype": str(self.k.dtype).replace("torch.", ""), "q_len": self.q_len,
                "sum_seq_len": sum(self.seq_lens_host), "data_seed": self.data_seed,
                "struct_seed": self.struct_seed}


def _cpu_gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def _dev_gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


FP8 = torch.float8_e4m3fn
FP8_MAX = 448.0
FP8_NAN_CODE = 0x7F


def fp8_head_sigmas(num_kv_heads: int, struct_seed: int) -> tuple:
    """Per-KV-head spreads of K and of V for an fp8 cache, U[0.5, 2]."""
    g = _cpu_gen(struct_seed + 7001)
    ks = 0.5 + 1.5 * torch.rand(num_kv_heads, generator=g)
    vs = 0.5 + 1.5 * torch.rand(num_kv_heads, generator=g)
    return ks, vs


def _store(xf: torch.Tensor, dtype, head_scale=None) -> torch.Tensor:
    """fp32 [Hkv][...][D] values in the cache's storage type. For fp8 the
    values are divided by their head's scale, clamped to the format's range
    and rounded by torch's conversion."""
    if dtype != FP8:
        return xf.to(dtype)
    shape = [-1] + [1] * (xf.dim() - 1)
    y = (xf / head_scale.to(xf.device).reshape(shape)).clamp_(-FP8_MAX, FP8_MAX)
    return y.to(FP8)


def _poison(t: torch.Tensor, index) -> None:
    """Write NaN (the fp8 NaN code for an fp8 tensor) at t[index]."""
    if t.dtype == FP8:
        t.view(torch.uint8)[index] = FP8_NAN_CODE
    else:
        t[index] = float("nan")


def uniform_lengths(batch: int, lo: int, hi: int, struct_seed: int) -> list:
    """Sequence lengths drawn uniformly from the integers lo..hi inclusive."""
    return torch.randint(lo, hi + 1, (batch,), generator=_cpu_gen(struct_seed)).tolist()


def pick_offset_keys(lens, num_kv_heads: int, count: int, struct_seed: int, tail_from=None) -> dict:
    """For every (b, kv head), `count` distinct key indices below L_b; with
    tail_from set, the last of them is drawn from [tail_from, L_b)."""
    g = _cpu_gen(struct_seed + 7919)
    chosen = {}
    for b, L in enumerate(lens):
        for h in range(num_kv_heads):
            if tail_from is None:
                idx = torch.randperm(L, generator=g)[:count].tolist()
            else:
                idx = torch.randperm(tail_from, generator=g)[:count - 1].tolist()
                idx.append(tail_from + int(torch.randint(0, L - tail_from, (1,), generator=g)))
            chosen[(b, h)] = sorted(idx)
    return chosen


def _raise_scores(kf: torch.Tensor, qf: torch.Tensor, keys: list, delta: float, scale: float) -> None:
    """kf: fp32 [tokens][D] of one (b, kv head); qf: fp32 [D] of its query head."""
    if not keys:
        return
    direction = qf / (scale * torch.dot(qf, qf))
    idx = torch.as_tensor(keys, device=kf.device, dtype=torch.long)
    kf[idx] += delta * direction


def _queries(batch, q_len, num_q_heads, head_dim, dtype, gen, device):
    shape = (batch, num_q_heads, head_dim) if q_len == 1 else (batch, q_len, num_q_heads, head_dim)
    return torch.randn(shape, generator=gen, device=device).to(torch.bfloat16 if dtype == FP8 else dtype)


def _scales(dtype, num_kv_heads, struct_seed, device):
    """(k sigmas, v sigmas, k_scale, v_scale) for fp8, else Nones and unit sigmas."""
    if dtype != FP8:
        return torch.ones(num_kv_heads), torch.ones(num_kv_heads), None, None
    ks, vs = fp8_head_sigmas(num_kv_heads, struct_seed)
    return ks, vs, (ks / 64.0).to(device), (vs / 64.0).to(device)


def contiguous(name: str, batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int, lens, *,
               dtype=torch.bfloat16, out_dtype=None, cap=None, data_seed: int, struct_seed: int,
               device="cpu", offsets=None, delta: float = 0.0, num_splits: int = 0,
               scale=None, q_len: int = 1, shared_q: bool = False) -> DecodeInputs:
    """Contiguous KV [B][Hkv][cap][D] with N(0,1) values rounded to `dtype`
    (fp8: per-head spreads and scales as described above).
    offsets: dict (b, kv head) -> key indices whose score is raised by delta.
    shared_q: every query row that reads one KV head (all its tokens and
    group heads) is the same vector, so that score offsets through K reach
    all of them; without it offsets need one query row per KV head."""
    lens = [int(x) for x in lens]
    cap = cap or max(lens)
    scale = float(scale if scale is not None else 1.0 / math.sqrt(head_dim))
    gen = _dev_gen(data_seed, device)
    q = _queries(batch, q_len, num_q_heads, head_dim, dtype, gen, device)
    k = torch.empty((batch, num_kv_heads, cap, head_dim), dtype=dtype, device=device)
    v = torch.empty_like(k)
    group = num_q_heads // num_kv_heads
    q4 = q if q_len > 1 else q.unsqueeze(1)          # [B][q_len][Hq][D] view
    if shared_q:
        lead = q4[:, :1, ::group].clone()              # token 0, first head of each group
        q4.copy_(lead.repeat_interleave(group, dim=2).expand(-1, q_len, -1, -1))
    if offsets and not shared_q and (group != 1 or q_len != 1):
        raise ValueError("score offsets through K need one query row per KV head, or shared_q")
    ksig, vsig, k_scale, v_scale = _scales(dtype, num_kv_heads, struct_seed, device)
    for b in range(batch):
        kf = torch.randn((num_kv_heads, cap, head_dim), generator=gen, device=device)
        kf *= ksig.to(device).reshape(-1, 1, 1)
        if offsets:
            for h in range(num_kv_heads):
                _raise_scores(kf[h], q4[b, 0, h * group].float(), offsets.get((b, h), []), delta, scale)
        k[b] = _store(kf, dtype, k_scale)
        del kf
        vf = torch.randn((num_kv_heads, cap, head_dim), generator=gen, device=device)
        vf *= vsig.to(device).reshape(-1, 1, 1)
        v[b] = _store(vf, dtype, v_scale)
        del vf
        if lens[b] < cap:
            _poison(k, (b, slice(None), slice(lens[b], None)))
            _poison(v, (b, slice(None), slice(lens[b], None)))
    seq = torch.tensor(lens, dtype=torch.int32, device=device)
    default_out = torch.bfloat16 if dtype == FP8 else dtype
    return DecodeInputs(name=name, q=q, k=k, v=v, seq_lens=seq, seq_lens_host=lens, scale=scale,
                        max_seq_len=max(lens), out_dtype=out_dtype or default_out, num_splits=num_splits,
                        offset_keys=dict(offsets or {}), data_seed=data_seed, struct_seed=struct_seed,
                        k_scale=k_scale, v_scale=v_scale)


def paged(name: str, batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int, lens, *,
          page_size: int = 16, max_pages=None, dtype=torch.bfloat16, out_dtype=None, data_seed: int,
          struct_seed: int, device="cpu", num_splits: int = 0, spare_pages: int = 0,
          q_len: int = 1) -> DecodeInputs:
    """Paged KV: a shared pool [num_pages][Hkv][P][D] whose physical page ids
    are a seeded permutation, handed to the sequences in logical order through
    block_table (entries past a sequence's last page are -1). spare_pages adds
    pool pages that no sequence uses."""
    lens = [int(x) for x in lens]
    need = [-(-L // page_size) for L in lens]
    max_pages = max_pages or max(need)
    num_pages = sum(need) + spare_pages
    perm = torch.randperm(num_pages, generator=_cpu_gen(struct_seed + 104729))
    table = torch.full((batch, max_pages), -1, dtype=torch.int32)
    pos = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[pos:pos + n].to(torch.int32)
        pos += n
    gen = _dev_gen(data_seed, device)
    q = _queries(batch, q_len, num_q_heads, head_dim, dtype, gen, device)
    k = torch.empty((num_pages, num_kv_heads, page_size, head_dim), dtype=dtype, device=device)
    v = torch.empty_like(k)
    ksig, vsig, k_scale, v_scale = _scales(dtype, num_kv_heads, struct_seed, device)
    # Pool pages are [page][Hkv][P][D]: move the head axis first for the per-head scales.
    chunk = 4096
    for p0 in range(0, num_pages, chunk):
        p1 = min(num_pages, p0 + chunk)
        kf = torch.randn((p1 - p0, num_kv_heads, page_size, head_dim), generator=gen, device=device)
        kf *= ksig.to(device).reshape(1, -1, 1, 1)
        k[p0:p1] = _store(kf.transpose(0, 1), dtype, k_scale).transpose(0, 1)
        vf = torch.randn((p1 - p0, num_kv_heads, page_size, head_dim), generator=gen, device=device)
        vf *= vsig.to(device).reshape(1, -1, 1, 1)
        v[p0:p1] = _store(vf.transpose(0, 1), dtype, v_scale).transpose(0, 1)
        del kf, vf
    for b, L in enumerate(lens):
        used = L % page_size
        if used:
            last = int(table[b, need[b] - 1])
            _poison(k, (last, slice(None), slice(used, None)))
            _poison(v, (last, slice(None), slice(used, None)))
    seq = torch.tensor(lens, dtype=torch.int32, device=device)
    default_out = torch.bfloat16 if dtype == FP8 else dtype
    return DecodeInputs(name=name, q=q, k=k, v=v, seq_lens=seq, seq_lens_host=lens,
                        scale=1.0 / math.sqrt(head_dim), max_seq_len=max(lens),
                        out_dtype=out_dtype or default_out, page_size=page_size, block_table=table.to(device),
                        num_pages=num_pages, num_splits=num_splits, data_seed=data_seed,
                        struct_seed=struct_seed, k_scale=k_scale, v_scale=v_scale)


def to_paged(x: DecodeInputs, page_size: int = 16, struct_seed: int = 0) -> DecodeInputs:
    """The same keys and values as a contiguous workload, scattered over a
    shuffled page pool (for the paged == contiguous check)."""
    if x.page_size:
        raise ValueError("already paged")
    lens = x.seq_lens_host
    need = [-(-L // page_size) for L in lens]
    num_pages = sum(need)
    perm = torch.randperm(num_pages, generator=_cpu_gen(struct_seed + 15485863))
    table = torch.full((x.batch, max(need)), -1, dtype=torch.int32)
    dev = x.k.device
    k = torch.empty((num_pages, x.num_kv_heads, page_size, x.head_dim), dtype=x.k.dtype, device=dev)
    v = torch.empty_like(k)
    _poison(k, (slice(None),))
    _poison(v, (slice(None),))
    pos = 0
    for b, n in enumerate(need):
        ids = perm[pos:pos + n]
        table[b, :n] = ids.to(torch.int32)
        pos += n
        for i, pid in enumerate(ids.tolist()):
            lo, hi = i * page_size, min(lens[b], (i + 1) * page_size)
            k[pid, :, :hi - lo] = x.k[b, :, lo:hi]
            v[pid, :, :hi - lo] = x.v[b, :, lo:hi]
    return DecodeInputs(name=x.name + "-paged", q=x.q, k=k, v=v, seq_lens=x.seq_lens,
                        seq_lens_host=list(lens), scale=x.scale, max_seq_len=x.max_seq_len,
                        out_dtype=x.out_dtype, page_size=page_size, block_table=table.to(dev),
                        num_pages=num_pages, num_splits=x.num_splits, data_seed=x.data_seed,
                        struct_seed=struct_seed, k_scale=x.k_scale, v_scale=x.v_scale)


# --------------------------------------------------------------------------
# The five named workloads.
# --------------------------------------------------------------------------

def c1_tiny_fp32(variant: str = "plain", device="cpu", num_splits: int = 4) -> DecodeInputs:
    """Batch 1, one head, head_dim 64, 1000 keys, fp32, chunks of 256 (a
    232-key tail), scale 1/8. Variant "outliers": +30 on the scores of 3
    random keys; variant "tail": the same with one of them in the tail chunk."""
    L, data_seed, struct_seed = 1000, 1001, 2001
    offsets, delta = None, 0.0
    if variant == "outliers":
        offsets, delta = pick_offset_keys([L], 1, 3, struct_seed), 30.0
    elif variant == "tail":
        offsets, delta = pick_offset_keys([L], 1, 3, struct_seed, tail_from=768), 30.0
    elif variant != "plain":
        raise ValueError(variant)
    x = contiguous(f"c1-tiny-fp32-{variant}", 1, 1, 1, 64, [L], dtype=torch.float32, data_seed=data_seed,
                   struct_seed=struct_seed, device=device, offsets=offsets, delta=delta,
                   num_splits=num_splits, scale=1.0 / 8.0)
    rows = x.v[0, 0, :L].cpu()
    if torch.unique(rows, dim=0).shape[0] != L:
        raise AssertionError("value rows must be pairwise distinct")
    return x


def c2_gqa_32k(device="cpu", length: int = 32768, cap: int = 32768) -> DecodeInputs:
    """Batch 1, 32 query heads over 8 KV heads, head_dim 128, bf16, 64 splits."""
    return contiguous(f"c2-gqa-bf16-L{length}", 1, 32, 8, 128, [length], cap=cap, dtype=torch.bfloat16,
                      data_seed=1002, struct_seed=2002, device=device, num_splits=64)


def c3_long_mha(device="cpu", batch: int = 4, length: int = 131072, dtype=torch.bfloat16) -> DecodeInputs:
    """Batch 4, 32 heads (MHA), head_dim 128, 131072 keys, bf16, planner
    splits; 1% of the keys of every (b, head) get +20 on their score.
    dtype=FP8 stores the same draws as an fp8 cache (q stays bf16)."""
    lens = [length] * batch
    offsets = pick_offset_keys(lens, 32, int(0.01 * length), 2003)
    tag = "fp8" if dtype == FP8 else "bf16"
    return contiguous(f"c3-long-mha-{tag}-B{batch}-L{length}", batch, 32, 32, 128, lens,
                      dtype=dtype, data_seed=1003, struct_seed=2003, device=device,
                      offsets=offsets, delta=20.0)


def c4_paged(device="cpu", batch: int = 16, lo: int = 1024, hi: int = 65536, dtype=torch.bfloat16,
             q_len: int = 1) -> DecodeInputs:
    """Batch 16, lengths uniform in [1024, 65536], 32 query / 8 KV heads,
    head_dim 128, bf16, page size 16, shuffled pool, block table width 4096.
    dtype=FP8 gives an fp8 cache; q_len > 1 a multi-token (speculative
    verification) step over the same cache."""
    lens = uniform_lengths(batch, lo, hi, 2004)
    tag = ("fp8" if dtype == FP8 else "bf16") + (f"-T{q_len}" if q_len > 1 else "")
    return paged(f"c4-paged-{tag}-B{batch}", batch, 32, 8, 128, lens, page_size=16, max_pages=hi // 16,
                 data_seed=1004, struct_seed=2004, device=device, dtype=dtype, q_len=q_len)


def c5_short_batch(device="cpu", batch: int = 128, num_splits: int = 0) -> DecodeInputs:
    """Batch 128, lengths uniform in [256, 2048], 32 query / 8 KV heads,
    head_dim 128, bf16, contiguous with capacity 2048."""
    lens = uniform_lengths(batch, 256, 2048, 2005)
    return contiguous(f"c5-short-batch-bf16-B{batch}", batch, 32, 8, 128, lens, cap=2048,
                      dtype=torch.bfloat16, data_seed=1005, struct_seed=2005, device=device,
                      num_splits=num_splits)
