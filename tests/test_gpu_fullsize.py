"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (planner defaults): the long-context MHA and paged workloads, and
bench's fp8-cache and four-token variants of them. Every output row is
checked element by element against one whole-workload oracle call on host
copies of the same bytes; a few sampled rows are also checked against the
oracle over keys gathered row by row (through the block table, in logical
order), which does not share the oracle's own paged addressing. The smaller
workloads are checked on every row in test_gpu_parity.py."""
import pytest
import torch

import decode_attention_12_amd as fd
import oracle
import workloads
from fdcheck import assert_lse_close, assert_out_close, reference, run, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _banner(name):
    print(f"\n[case] {name}", flush=True)


def _check_rows(x, out, lse, rows):
    """Each sampled (b, t, h) row (one-token workloads: t = 0) against the
    oracle over just the keys it reads (gathered through the block table for
    a paged cache, in logical order)."""
    g = x.num_q_heads // x.num_kv_heads
    refs, ref_lses, gots, got_lses = [], [], [], []
    for b, t, h in rows:
        assert t == 0
        kvh = h // g
        L = x.seq_lens_host[b]
        if x.page_size:
            npg = -(-L // x.page_size)
            pages = x.block_table[b, :npg].long()
            k = x.k[pages, kvh].reshape(1, 1, npg * x.page_size, -1)[:, :, :L].cpu().contiguous()
            v = x.v[pages, kvh].reshape(1, 1, npg * x.page_size, -1)[:, :, :L].cpu().contiguous()
        else:
            k = x.k[b:b + 1, kvh:kvh + 1, :L].cpu().contiguous()
            v = x.v[b:b + 1, kvh:kvh + 1, :L].cpu().contiguous()
        q = x.q[b:b + 1, h:h + 1].cpu().contiguous()
        o, l = oracle.attention(q, k, v, torch.tensor([L], dtype=torch.int32), scale=x.scale)
        refs.append(o[0])
        ref_lses.append(l[0])
        gots.append(out[b, h].cpu())
        got_lses.append(lse[b, h].cpu())
    ref = torch.stack(refs)
    assert_out_close(torch.stack(gots), ref, x.out_dtype)
    assert_lse_close(torch.stack(got_lses), torch.stack(ref_lses), x.k.dtype)


def _check_all_rows(x, out, lse):
    """Every output row against the oracle over the whole workload."""
    ref, ref_lse = reference(x)
    D = x.head_dim
    assert_out_close(out.reshape(-1, D), ref, x.out_dtype)
    assert_lse_close(lse.reshape(-1), ref_lse, x.k.dtype)
    print(f"[rows] {ref.shape[0]} rows checked", flush=True)


def test_long_mha_full_size():
    _banner("long-context MHA, full size, all rows + 12 sampled rows")
    x = workloads.c3_long_mha(device=DEV)
    out, lse, plan, _ = run(x)
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    _check_all_rows(x, out, lse)
    rows = sample_rows(x, 12, seed=3)
    _check_rows(x, out, lse, rows)
    del x
    torch.cuda.empty_cache()


def test_paged_full_size():
    _banner("paged batch 16, full size, all rows + 16 sampled rows")
    x = workloads.c4_paged(device=DEV)
    out, lse, plan, _ = run(x)
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    _check_all_rows(x, out, lse)
    rows = [(b, 0, int(torch.randint(0, 32, (1,), generator=torch.Generator().manual_seed(b)))) for b in range(16)]
    _check_rows(x, out, lse, rows)
    del x
    torch.cuda.empty_cache()


def test_long_mha_split_mode_full_size_sampled():
    _banner("long-context MHA, full size, 16 fixed splits, 6 sampled rows")
    x = workloads.c3_long_mha(device=DEV)
    out, lse, plan, _ = run(x, splits=16)
    rows = sample_rows(x, 6, seed=4)
    _check_rows(x, out, lse, rows)
    del x
    torch.cuda.empty_cache()


def _check_sampled(x, out, lse, n, seed):
    """n sampled output rows (any token) against the oracle on the whole
    cache, scales included."""
    from fdcheck import reference
    rows = sample_rows(x, n, seed=seed)
    ref, ref_lse = reference(x, rows=rows)
    if x.q_len == 1:
        got = torch.stack([out[b, h] for b, _, h in rows])
        got_lse = torch.stack([lse[b, h] for b, _, h in rows])
    else:
        got = torch.stack([out[b, t, h] for b, t, h in rows])
        got_lse = torch.stack([lse[b, t, h] for b, t, h in rows])
    assert_out_close(got, ref, x.out_dtype)
    assert_lse_close(got_lse, ref_lse, x.k.dtype)


def test_long_mha_fp8_full_size():
    _banner("long-context MHA, fp8 cache, full size, all rows + 12 sampled rows")
    x = workloads.c3_long_mha(device=DEV, dtype=workloads.FP8)
    out, lse, plan, _ = run(x)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    _check_all_rows(x, out, lse)
    _check_sampled(x, out, lse, 12, seed=5)
    del x
    torch.cuda.empty_cache()


def test_paged_fp8_full_size():
    _banner("paged batch 16, fp8 cache, full size, all rows + 16 sampled rows")
    x = workloads.c4_paged(device=DEV, dtype=workloads.FP8)
    out, lse, plan, _ = run(x)
    _check_all_rows(x, out, lse)
    _check_sampled(x, out, lse, 16, seed=6)
    del x
    torch.cuda.empty_cache()


def test_paged_four_tokens_full_size():
    _banner("paged batch 16, 4 query tokens, full size, all rows + 24 sampled rows")
    x = workloads.c4_paged(device=DEV, q_len=4)
    out, lse, plan, _ = run(x)
    assert plan.path == fd.FD_PATH_MFMA
    _check_all_rows(x, out, lse)
    _check_sampled(x, out, lse, 24, seed=7)
    del x
    torch.cuda.empty_cache()
