"""The single-launch step (fd_decode): the same results as the two-launch
path and the oracle, the piece counters back at zero after every call, and a
second call on the same workspace as good as the first."""
import pytest
import torch

import workloads
from fdcheck import assert_lse_close, assert_out_close, counters, host, reference, run, run_fused

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _banner(name):
    print(f"\n[case] {name}", flush=True)


def _check_fused(x, splits=None, workers=None, host_lens=True, rows=None):
    ref, ref_lse = reference(x, rows=rows)
    keep = slice(None) if rows is None else [b for b, _, _ in rows[::x.num_q_heads]]
    two = run(x, splits=splits, workers=workers, host_lens=host_lens)
    ws = None
    for _ in range(2):   # the second call reuses the workspace and its counters
        out, lse, plan, ws = run_fused(x, splits=splits, workers=workers, host_lens=host_lens, workspace=ws)
        assert (counters(x, plan, ws) == 0).all(), "piece counters must be back at zero"
        assert_out_close(out[keep], ref, x.out_dtype)
        assert_lse_close(lse[keep], ref_lse, x.k.dtype)
        # Same records, merged by another kernel in another order.
        diff = (out.float() - two[0].float()).abs().max().item()
        assert diff <= 2e-2 * max(1.0, two[0].float().abs().max().item()), diff
    return out, lse


def test_fused_short_batch():
    _banner("fused short-context batch 128")
    _check_fused(workloads.c5_short_batch(device=DEV))


def test_fused_paged_reduced():
    _banner("fused paged reduced")
    _check_fused(workloads.c4_paged(device=DEV, batch=4, lo=100, hi=3000))


@pytest.mark.parametrize("splits", [4, 1, 63])
def test_fused_split_mode_fp32(splits):
    _banner(f"fused split mode, tiny fp32, S={splits}")
    _check_fused(workloads.c1_tiny_fp32("outliers", device=DEV), splits=splits)


def test_fused_gqa_split_64():
    _banner("fused gqa-32k, 64 splits")
    _check_fused(workloads.c2_gqa_32k(device=DEV, length=4096, cap=4096), splits=64)


@pytest.mark.parametrize("piece_cost", [0, 1, 3])
@pytest.mark.parametrize("workers", [1, 3, 16, 1000])
@pytest.mark.parametrize("group", [4, 1])
def test_fused_balanced_with_empty_sequence(workers, group, piece_cost):
    _banner(f"fused balanced, workers={workers}, group={group}, piece_cost={piece_cost}, one empty sequence")
    lens = [300, 0, 17, 1, 1000, 64, 33]
    x = workloads.contiguous("fz", len(lens), 2 * group, 2, 128, lens, cap=1000, dtype=torch.bfloat16,
                             data_seed=120 + group, struct_seed=121, device=DEV)
    keep = [b for b, L in enumerate(lens) if L > 0]
    rows = [(b, 0, h) for b in keep for h in range(2 * group)]
    ref, ref_lse = reference(x, rows=rows)
    ws = None
    for _ in range(2):
        out, lse, plan, ws = run_fused(x, splits=0, workers=workers, host_lens=False, workspace=ws,
                                       piece_cost=piece_cost)
        assert plan.piece_cost == piece_cost
        assert (counters(x, plan, ws) == 0).all()
        assert (out[1] == 0).all() and torch.isinf(lse[1]).all() and (lse[1] < 0).all()
        assert_out_close(out[keep].reshape(-1, 128), ref, torch.bfloat16)
        assert_lse_close(lse[keep].reshape(-1), ref_lse, torch.bfloat16)


@pytest.mark.parametrize("dtype,D", [(torch.float32, 64), (torch.float32, 128), (torch.bfloat16, 64),
                                     (workloads.FP8, 64)])
@pytest.mark.parametrize("group", [1, 2, 4])
@pytest.mark.parametrize("splits", [0, 5])
def test_fused_valu_shapes(dtype, D, group, splits):
    """The single launch on every VALU row tile (1, 2, 4 rows; fp8 tiles stop
    at 2) in both modes: the merge spreads a segment's records over copies of
    its rows' lanes when the segment has fewer rows than a wave holds."""
    _banner(f"fused VALU {dtype} D={D} group={group} splits={splits}")
    lens = [200, 31, 1, 96]
    x = workloads.contiguous("fv", len(lens), 2 * group, 2, D, lens, dtype=dtype, data_seed=130 + group + D,
                             struct_seed=131, device=DEV)
    _check_fused(x, splits=splits)
