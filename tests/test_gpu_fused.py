"""The single-launch step (fd_decode) against the oracle over several
consecutive decode steps on ONE workspace, with fresh values and fresh
sequence lengths every step: split mode (every record slot rewritten, other
splits empty from step to step) and balanced mode (record slots, piece counts
and the segments a worker merges all move with the lengths). A record left
from an earlier step, or read before its writer's stores were visible to the
merging wave, would show as a wrong output because the inputs change."""
import pytest
import torch

import workloads
from fdcheck import check_fused_steps

pytestmark = pytest.mark.gpu
DEV = "cuda"
STEPS = 3


def _banner(name):
    print(f"\n[case] {name}", flush=True)


def contiguous_steps(name, Hq, Hkv, D, lens_per_step, *, cap, dtype=torch.bfloat16, seed, q_len=1):
    """One contiguous workload per step: the same shapes, max_seq_len = cap,
    new data and structure seeds every step."""
    for i, lens in enumerate(lens_per_step):
        x = workloads.contiguous(f"{name}-step{i}", len(lens), Hq, Hkv, D, lens, cap=cap, dtype=dtype, q_len=q_len,
                                 data_seed=seed + 17 * i, struct_seed=seed + 1000 + 17 * i, device=DEV)
        x.max_seq_len = cap
        yield x


def paged_steps(name, Hq, Hkv, lens_per_step, *, cap, dtype=torch.bfloat16, seed, page_size=16):
    """One paged workload per step (a new shuffled pool each time)."""
    for i, lens in enumerate(lens_per_step):
        x = workloads.paged(f"{name}-step{i}", len(lens), Hq, Hkv, 128, lens, page_size=page_size,
                            max_pages=-(-cap // page_size), dtype=dtype, data_seed=seed + 17 * i,
                            struct_seed=seed + 1000 + 17 * i, device=DEV)
        x.max_seq_len = cap
        yield x


@pytest.mark.parametrize("splits", [63, 4, 1])
def test_fused_split_mode_tiny_fp32(splits):
    """The tiny fp32 shape (one head, head_dim 64, up to 1000 keys) in split
    mode; the lengths change which trailing splits are empty."""
    _banner(f"fused split mode, tiny fp32, S={splits}, {STEPS} steps")
    lens = [[1000], [611], [937]][:STEPS]
    assert check_fused_steps(contiguous_steps("f1", 1, 1, 64, lens, cap=1000, dtype=torch.float32, seed=3100),
                             splits=splits) == STEPS


def test_fused_gqa_split_64():
    """The GQA shape (32 query / 8 KV heads) at 4096 keys and 64 splits: the
    last workgroup of each KV head merges 64 records."""
    _banner(f"fused gqa, 64 splits, {STEPS} steps")
    lens = [[4096], [3001], [4000]][:STEPS]
    assert check_fused_steps(contiguous_steps("f2", 32, 8, 128, lens, cap=4096, seed=3200), splits=64) == STEPS


def test_fused_short_batch():
    """The short-context batch (128 sequences, lengths U[256, 2048]) with the
    planner's balanced plan; the lengths are drawn anew every step."""
    _banner(f"fused short-context batch 128, {STEPS} steps")
    lens = [workloads.uniform_lengths(128, 256, 2048, struct_seed=3300 + i) for i in range(STEPS)]
    assert check_fused_steps(contiguous_steps("f5", 32, 8, 128, lens, cap=2048, seed=3300), splits=0) == STEPS


@pytest.mark.parametrize("dtype", [torch.bfloat16, workloads.FP8])
def test_fused_paged_reduced(dtype):
    """Paged GQA batch of 4 with lengths U[100, 3000], bf16 and fp8 caches."""
    _banner(f"fused paged reduced {dtype}, {STEPS} steps")
    lens = [workloads.uniform_lengths(4, 100, 3000, struct_seed=3400 + i) for i in range(STEPS)]
    assert check_fused_steps(paged_steps("f4", 32, 8, lens, cap=3000, dtype=dtype, seed=3400), splits=0) == STEPS


@pytest.mark.parametrize("workers", [1, 3, 16, 1000])
@pytest.mark.parametrize("group", [4, 1])
def test_fused_balanced_with_empty_sequences(workers, group):
    """Balanced plans of 1 .. 1000 workers over ragged lengths with a
    sequence of no key, which moves from step to step (its rows must come
    out as 0 / -inf: the device sees the 0, the host check is off)."""
    _banner(f"fused balanced, workers={workers}, group={group}, empty sequences, {STEPS} steps")
    base = [300, 0, 17, 1, 1000, 64, 33]
    lens = [base[i:] + base[:i] for i in range(STEPS)]
    steps = contiguous_steps("fz", 2 * group, 2, 128, lens, cap=1000, seed=3500 + group)
    assert check_fused_steps(steps, splits=0, workers=workers, host_lens=False) == STEPS


@pytest.mark.parametrize("dtype,D", [(torch.float32, 64), (torch.float32, 128), (torch.bfloat16, 64),
                                     (workloads.FP8, 64)])
@pytest.mark.parametrize("group", [1, 2, 4])
@pytest.mark.parametrize("splits", [0, 5])
def test_fused_valu_shapes(dtype, D, group, splits):
    """The single launch on every VALU row tile (1, 2, 4 rows; fp8 tiles stop
    at 2) in both modes: the merge spreads a segment's records over copies of
    its rows' lanes when the segment has fewer rows than a wave holds."""
    _banner(f"fused VALU {dtype} D={D} group={group} splits={splits}, {STEPS} steps")
    lens = [[200, 31, 1, 96], [7, 200, 150, 33], [96, 64, 199, 2]][:STEPS]
    steps = contiguous_steps("fv", 2 * group, 2, D, lens, cap=200, dtype=dtype, seed=3600 + group + D)
    assert check_fused_steps(steps, splits=splits) == STEPS


def test_fused_leading_share_paged():
    """A plan whose first workers take 150 % shares, over a paged bf16 cache."""
    _banner(f"fused leading share, {STEPS} steps")
    lens = [workloads.uniform_lengths(9, 1, 1000, struct_seed=3700 + i) for i in range(STEPS)]
    assert check_fused_steps(paged_steps("fl", 8, 2, lens, cap=1000, seed=3700), splits=0, workers=16,
                             lead=(8, 150)) == STEPS


def test_two_launch_steps_under_other_plans_leave_the_counters_alone():
    """One zeroed workspace used by the two-launch step under several plans
    (forced splits, balanced plans of any worker count) and by single-launch
    steps in between, never re-zeroed: the counts section comes first in every
    plan's layout and only fd_decode writes it, so every single-launch step
    still finds its counters at zero."""
    _banner("workspace shared by two-launch plans and the single launch")
    from fdcheck import assert_lse_close, assert_out_close, counters, reference, run, run_fused
    import decode_attention_12_amd as fd
    lens = workloads.uniform_lengths(5, 50, 1200, struct_seed=3800)
    x = next(contiguous_steps("fwr", 16, 4, 128, [lens], cap=1200, seed=3800))
    ref, ref_lse = reference(x)
    problem = fd.problem_of(x.q, x.k, x.max_seq_len)
    plans = [fd.fd_plan_splits(problem, 0, s) for s in (0, 3, 40)]
    size = max(fd.fd_workspace_size(problem, p) for p in plans) + 4096
    ws = torch.zeros(size, dtype=torch.uint8, device=DEV)
    for splits, workers in ((3, None), (0, 7), (40, None), (0, 300)):
        out, lse, plan, _ = run(x, splits=splits, workers=workers, workspace=ws)
        assert_out_close(out, ref, torch.bfloat16)
        for fused_splits in (0, 3):
            fout, flse, fplan, _ = run_fused(x, splits=fused_splits, workspace=ws)
            assert (counters(x, fplan, ws) == 0).all()
            assert_out_close(fout, ref, torch.bfloat16)
            assert_lse_close(flse, ref_lse, torch.bfloat16)
