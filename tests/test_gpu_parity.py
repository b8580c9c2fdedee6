"""GPU parity: the library (through its C ABI) against the fp64 oracle on the
same seeded inputs. Sizes here finish in seconds on the oracle side and still
span several tiles, several splits and ragged tails."""
import math

import pytest
import torch

import decode_attention_12_amd as fd
import workloads
from fdcheck import (assert_lse_close, assert_out_close, assert_records_close, counters, host, reference,
                     row_records, row_rel_err, run, run_fused, weight_sums)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _banner(name):
    print(f"\n[case] {name}", flush=True)


# --------------------------------------------------------------------------
# The tiny fp32 workload: 1000 keys, chunks of 256 with a 232-key tail.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("variant", ["plain", "outliers", "tail"])
def test_tiny_fp32(variant):
    _banner(f"tiny fp32 {variant}")
    x = workloads.c1_tiny_fp32(variant, device=DEV)
    out, lse, plan, ws = run(x)
    assert (plan.num_splits, plan.chunk_len) == (4, 256)
    hx = host(x)
    ref, ref_lse = reference(x, hx=hx)
    assert_out_close(out, ref, torch.float32)
    assert_lse_close(lse, ref_lse, torch.float32)
    assert_records_close(x, plan, ws, hx)
    if variant != "plain":
        # The outlier chunks dominate: at least one chunk weighs ~1 and the
        # others are far below it (the page's point about wide LSE gaps).
        w = weight_sums(x, plan, ws)
        assert (w >= 1.0).all() and (w <= plan.num_splits).all()


def test_tiny_fp32_error_vs_split_count():
    _banner("tiny fp32 split sweep")
    x = workloads.c1_tiny_fp32("outliers", device=DEV)
    ref, ref_lse = reference(x)
    errs = {}
    for S in (1, 2, 3, 4, 8, 16, 32, 63):
        out, lse, plan, ws = run(x, splits=S)
        assert plan.num_splits == S
        errs[S] = assert_out_close(out, ref, torch.float32)
        assert_lse_close(lse, ref_lse, torch.float32)
        w = weight_sums(x, plan, ws)
        assert (w >= 1.0).all() and (w <= S).all()
    print("error by split count:", {k: f"{v:.2e}" for k, v in errs.items()})
    floor = max(errs[1], 1e-7)
    for S, e in errs.items():
        assert e <= 8 * floor, f"error grows with split count: S={S} err={e:.2e} vs S=1 {errs[1]:.2e}"


# --------------------------------------------------------------------------
# GQA, bf16, contiguous (the 32K-key workload and smaller shapes).
# --------------------------------------------------------------------------

@pytest.mark.parametrize("path", [fd.FD_PATH_MFMA, fd.FD_PATH_VALU])
@pytest.mark.parametrize("length", [32768, 32731])
def test_gqa_32k(path, length):
    _banner(f"gqa 32k L={length} path={path}")
    x = workloads.c2_gqa_32k(device=DEV, length=length)
    out, lse, plan, ws = run(x, path=path)
    assert (plan.num_splits, plan.chunk_len) == (64, 512)
    hx = host(x)
    ref, ref_lse = reference(x, hx=hx)
    assert_out_close(out, ref, torch.bfloat16)
    assert_lse_close(lse, ref_lse, torch.bfloat16)
    assert_records_close(x, plan, ws, hx)


def test_gqa_error_vs_split_count():
    _banner("gqa split sweep, fp32 output")
    x = workloads.c2_gqa_32k(device=DEV)
    ref, _ = reference(x)
    errs = {}
    for S in (1, 4, 16, 64, 128):
        out, lse, plan, ws = run(x, splits=S, out_dtype=torch.float32)
        errs[S] = row_rel_err(out.cpu(), ref).max().item()
        w = weight_sums(x, plan, ws)
        assert torch.isfinite(out).all() and (w >= 1.0).all() and (w <= S).all()
    print("error by split count:", {k: f"{v:.2e}" for k, v in errs.items()})
    for S, e in errs.items():
        assert e <= 8 * max(errs[1], 1e-7) and e <= 1e-2, f"S={S}: {e:.2e} vs S=1 {errs[1]:.2e}"


@pytest.mark.parametrize("group", [4, 8, 16])
@pytest.mark.parametrize("path", [fd.FD_PATH_MFMA, fd.FD_PATH_VALU])
def test_gqa_groups_ragged(group, path):
    """Several sequences with ragged lengths (1, 15, 16, 17, 300, 1000) and
    distinct per-KV-head value offsets, so a wrong head mapping shows."""
    _banner(f"gqa group={group} path={path}")
    lens = [1, 15, 16, 17, 300, 1000]
    x = workloads.contiguous("ragged", len(lens), 2 * group, 2, 128, lens, cap=1024, dtype=torch.bfloat16,
                             data_seed=31 + group, struct_seed=32, device=DEV)
    x.v[:, 1] += 3.0
    for splits in (0, 3, 7):
        out, lse, plan, ws = run(x, splits=splits, path=path)
        ref, ref_lse = reference(x)
        assert_out_close(out, ref, torch.bfloat16)
        assert_lse_close(lse, ref_lse, torch.bfloat16)


@pytest.mark.parametrize("dtype,D", [(torch.float32, 64), (torch.float32, 128), (torch.bfloat16, 64),
                                     (torch.bfloat16, 128)])
@pytest.mark.parametrize("group", [1, 2, 3, 4])
def test_valu_shapes(dtype, D, group):
    _banner(f"valu {dtype} D={D} g={group}")
    lens = [5, 64, 999, 130]
    x = workloads.contiguous("valu", len(lens), 2 * group, 2, D, lens, cap=1000, dtype=dtype,
                             data_seed=41 + D + group, struct_seed=42, device=DEV)
    out, lse, plan, ws = run(x, splits=5)
    assert plan.path == fd.FD_PATH_VALU or (dtype == torch.bfloat16 and D == 128 and group == 4)
    hx = host(x)
    ref, ref_lse = reference(x, hx=hx)
    assert_out_close(out, ref, dtype)
    assert_lse_close(lse, ref_lse, dtype)
    if dtype == torch.float32:
        assert_records_close(x, plan, ws, hx)


# --------------------------------------------------------------------------
# Paged KV through a block table.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,group", [(torch.bfloat16, 4), (torch.bfloat16, 1), (torch.float32, 4)])
def test_paged_matches_oracle_and_contiguous(dtype, group):
    _banner(f"paged {dtype} g={group}")
    lens = [1, 16, 17, 33, 500, 2047]
    x = workloads.contiguous("pg", len(lens), 2 * group, 2, 128, lens, cap=2048, dtype=dtype, data_seed=51,
                             struct_seed=52, device=DEV)
    p = workloads.to_paged(x, page_size=16, struct_seed=53)
    for splits in (0, 4):
        out_c, lse_c, plan_c, _ = run(x, splits=splits)
        out_p, lse_p, plan_p, ws = run(p, splits=splits)
        assert (plan_c.num_splits, plan_c.chunk_len, plan_c.path) == (plan_p.num_splits, plan_p.chunk_len,
                                                                       plan_p.path)
        # Same plan, same arithmetic order: bit-identical results.
        assert torch.equal(out_c, out_p) and torch.equal(lse_c, lse_p)
        ref, ref_lse = reference(p)
        assert_out_close(out_p, ref, dtype)
        assert_lse_close(lse_p, ref_lse, dtype)


@pytest.mark.parametrize("splits", [0, 8])
def test_paged_workload_reduced(splits):
    """The paged workload's structure at a quarter of its batch and lengths:
    shuffled shared pool, NaN in unused slots of each last page; with fixed
    splits, empty splits for the short sequences."""
    _banner(f"paged reduced splits={splits}")
    x = workloads.c4_paged(device=DEV, batch=4, lo=100, hi=3000)
    out, lse, plan, ws = run(x, splits=splits)
    hx = host(x)
    ref, ref_lse = reference(x, hx=hx)
    assert_out_close(out, ref, torch.bfloat16)
    assert_lse_close(lse, ref_lse, torch.bfloat16)
    assert_records_close(x, plan, ws, hx)
    if splits:
        assert any(torch.isinf(l).any() for _, l, _ in row_records(x, plan, ws)), "expected empty splits"


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("group,dtype", [(4, torch.bfloat16), (1, torch.bfloat16), (2, torch.float32),
                                         (4, workloads.FP8)])
def test_balanced_partitions(group, dtype, paged):
    """Balanced plans with 1 .. 1000 workers over ragged lengths, one of them
    0: runs that span several segments and sequences, segments cut into many
    pieces, workers with nothing to do. Outputs and every record checked."""
    _banner(f"balanced partitions g={group} {dtype} paged={paged}")
    lens = [300, 0, 17, 1, 1000, 64, 33]
    x = workloads.contiguous("bal", len(lens), 2 * group, 2, 128, lens, cap=1000, dtype=dtype,
                             data_seed=95 + group, struct_seed=96, device=DEV)
    if paged:
        x = workloads.to_paged(x, struct_seed=97)
    keep = [b for b, L in enumerate(lens) if L > 0]
    hx = host(x)
    ref, ref_lse = reference(x, rows=[(b, 0, h) for b in keep for h in range(2 * group)], hx=hx)
    for w in (1, 2, 3, 5, 16, 64, 1000):
        out, lse, plan, ws = run(x, splits=0, workers=w, host_lens=False)
        assert plan.mode == fd.FD_MODE_BALANCED and plan.workers == w
        assert (out[1] == 0).all() and torch.isinf(lse[1]).all() and (lse[1] < 0).all()
        assert_out_close(out[keep], ref, x.out_dtype)
        assert_lse_close(lse[keep], ref_lse, x.k.dtype)
        assert_records_close(x, plan, ws, hx)


def test_bad_block_table_entries_are_masked():
    """A block-table entry outside the pool makes its keys count as masked:
    the result equals attention over the remaining keys."""
    _banner("paged bad entries")
    x = workloads.contiguous("pgbad", 1, 4, 1, 128, [64], dtype=torch.bfloat16, data_seed=61, struct_seed=62,
                             device=DEV)
    p = workloads.to_paged(x, struct_seed=63)
    p.block_table[0, 1] = p.num_pages + 5        # keys 16..31 are now unreachable
    out, lse, plan, ws = run(p, splits=1)
    keep = torch.cat([x.k[:, :, :16], x.k[:, :, 32:64]], dim=2).contiguous()
    keepv = torch.cat([x.v[:, :, :16], x.v[:, :, 32:64]], dim=2).contiguous()
    y = workloads.DecodeInputs(name="kept", q=x.q, k=keep, v=keepv, seq_lens=torch.tensor([48], device=DEV,
                               dtype=torch.int32), seq_lens_host=[48], scale=x.scale, max_seq_len=48,
                               out_dtype=x.out_dtype)
    ref, ref_lse = reference(y)
    assert_out_close(out, ref, torch.bfloat16)
    assert_lse_close(lse, ref_lse, torch.bfloat16)


# --------------------------------------------------------------------------
# Short-context high batch.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("splits", [0, 1, 16])
def test_short_batch(splits):
    _banner(f"short batch splits={splits}")
    x = workloads.c5_short_batch(device=DEV, num_splits=splits)
    out, lse, plan, ws = run(x)
    if splits:
        assert plan.num_splits == splits
    ref, ref_lse = reference(x)
    assert_out_close(out, ref, torch.bfloat16)
    assert_lse_close(lse, ref_lse, torch.bfloat16)


# --------------------------------------------------------------------------
# Edge cases and layouts.
# --------------------------------------------------------------------------

def test_nan_past_length_and_more_splits_than_needed():
    _banner("nan past length, surplus splits")
    x = workloads.contiguous("nan", 3, 8, 2, 128, [7, 100, 513], cap=1024, dtype=torch.bfloat16, data_seed=71,
                             struct_seed=72, device=DEV)
    assert torch.isnan(x.k[0, :, 7:]).all()
    ref, ref_lse = reference(x)
    for splits in (1, 2, 40, 64):       # 64 splits of 16 keys: most are empty
        out, lse, plan, ws = run(x, splits=splits, out_dtype=torch.float32)
        err = row_rel_err(out.cpu(), ref).max().item()
        assert torch.isfinite(out).all() and err < 5e-3, (splits, err)
        assert_lse_close(lse, ref_lse, torch.bfloat16)
        w = weight_sums(x, plan, ws)
        assert (w >= 1.0).all()


def test_zero_length_on_device_gives_zero_and_minus_inf():
    """Without host-side lengths the library cannot refuse L_b = 0; the device
    path then writes out = 0 and lse = -inf (never NaN)."""
    _banner("zero length on device")
    x = workloads.contiguous("zero", 2, 4, 1, 128, [40, 40], dtype=torch.bfloat16, data_seed=81, struct_seed=82,
                             device=DEV)
    x.seq_lens[1] = 0
    problem = fd.problem_of(x.q, x.k, 40)
    plan = fd.fd_plan_splits(problem, 0, 2)
    ws = torch.empty(fd.fd_workspace_size(problem, plan), dtype=torch.uint8, device=DEV)
    out = torch.full(x.q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full(x.q.shape[:2], float("nan"), device=DEV)
    fd.fd_decode_partial(problem, plan, x.q, x.k, x.v, fd.layout_of(x.k), x.seq_lens, ws, scale=x.scale)
    fd.fd_decode_combine(problem, plan, ws, out, lse)
    torch.cuda.synchronize()
    assert (out[1] == 0).all() and torch.isinf(lse[1]).all() and (lse[1] < 0).all()
    assert torch.isfinite(out[0]).all()
    with pytest.raises(fd.FdError) as e:
        fd.fd_decode_partial(problem, plan, x.q, x.k, x.v, fd.layout_of(x.k), x.seq_lens, ws, scale=x.scale,
                             seq_lens_host=[40, 0])
    assert e.value.status == -4


def test_token_major_layout_is_bit_identical():
    """A [B][L][Hkv][D] cache through strides gives the same bits as [B][Hkv][L][D]."""
    _banner("token-major strides")
    x = workloads.contiguous("tm", 2, 8, 2, 128, [300, 45], dtype=torch.bfloat16, data_seed=91, struct_seed=92,
                             device=DEV)
    k_tm = x.k.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    v_tm = x.v.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    y = workloads.DecodeInputs(name="tm", q=x.q, k=k_tm, v=v_tm, seq_lens=x.seq_lens,
                               seq_lens_host=x.seq_lens_host, scale=x.scale, max_seq_len=x.max_seq_len,
                               out_dtype=x.out_dtype)
    a = run(x, splits=3)
    b = run(y, splits=3)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_repeat_runs_are_deterministic():
    _banner("determinism")
    x = workloads.c2_gqa_32k(device=DEV)
    a = run(x)
    b = run(x)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("lead", [(0.5, 150), (0.5, 60), (1.0, 200), (0.25, 120)])
def test_balanced_partitions_with_leading_share(lead, fp8):
    """Plans whose first workers take a larger (or smaller) share of the
    tiles: outputs and every record still match, in both launches' paths."""
    frac, pct = lead
    _banner(f"leading share {frac} x {pct}% fp8={fp8}")
    lens = [300, 0, 17, 1, 1000, 64, 33, 700, 129]
    x = workloads.contiguous("lead", len(lens), 8, 2, 128, lens, cap=1000,
                             dtype=workloads.FP8 if fp8 else torch.bfloat16, data_seed=131, struct_seed=132,
                             device=DEV)
    x = workloads.to_paged(x, struct_seed=133)
    keep = [b for b, L in enumerate(lens) if L > 0]
    hx = host(x)
    ref, ref_lse = reference(x, rows=[(b, 0, h) for b in keep for h in range(8)], hx=hx)
    for w in (5, 16, 200):
        lw = max(1, int(w * frac))
        out, lse, plan, ws = run(x, splits=0, workers=w, lead=(lw, pct), host_lens=False)
        assert (plan.workers, plan.lead_workers, plan.lead_pct) == (w, lw, pct)
        assert_out_close(out[keep], ref, x.out_dtype)
        assert_lse_close(lse[keep], ref_lse, x.k.dtype)
        assert_records_close(x, plan, ws, hx)
        fout, flse, fplan, fws = run_fused(x, splits=0, workers=w, lead=(lw, pct), host_lens=False)
        assert (counters(x, fplan, fws) == 0).all()
        assert_out_close(fout[keep], ref, x.out_dtype)
        assert_lse_close(flse[keep], ref_lse, x.k.dtype)
