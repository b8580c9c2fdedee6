"""Seeded random decode steps against the oracle: shapes, dtypes, query
lengths, page sizes, ragged lengths, plans (the planner's, forced splits,
balanced plans with any worker count, either kernel path where it is built)
and entry points (two launches, single launch, static workspace), drawn from
one fixed seed so that every run checks the same cases. Each case is valid
by construction (the host checks would refuse anything else) and is checked
on every output row and LSE."""
import random

import pytest
import torch

import decode_attention_12_amd as fd
import workloads
from fdcheck import assert_lse_close, assert_out_close, kv_layout, reference

pytestmark = pytest.mark.gpu
DEV = "cuda"
CASES = 256


def _case(i):
    r = random.Random(9000 + i)
    dtype = r.choice([torch.float32, torch.bfloat16, torch.bfloat16, workloads.FP8])
    hkv = r.choice([1, 2, 4, 8])
    g = r.choice([1, 2, 3, 4, 8])
    D = 128 if dtype != torch.float32 and r.random() < 0.7 else r.choice([64, 128])
    q_len = r.choice([1, 1, 2, 3, 4, 7])
    B = r.randint(1, 9)
    cap = r.choice([17, 300, 2000])
    cap = max(cap, q_len)
    lens = [r.randint(q_len, cap) for _ in range(B)]
    page = r.choice([0, 0, 16, 32, 64])
    entry = r.choice(["two", "two", "fused", "static"])
    mode = r.choice(["planner", "splits", "workers"])
    splits = r.randint(1, 70) if mode == "splits" else 0
    workers = r.randint(1, 300) if mode == "workers" else None
    path = r.choice([None, None, fd.FD_PATH_VALU])
    return dict(dtype=dtype, hkv=hkv, g=g, D=D, q_len=q_len, lens=lens, cap=cap, page=page, entry=entry,
                splits=splits, workers=workers, path=path, seed=9000 + i)


@pytest.mark.parametrize("i", range(CASES))
def test_random_case(i):
    c = _case(i)
    print(f"\n[case] random {i}: {c}", flush=True)
    x = workloads.contiguous(f"rnd{i}", len(c["lens"]), c["g"] * c["hkv"], c["hkv"], c["D"], c["lens"], cap=c["cap"],
                             dtype=c["dtype"], q_len=c["q_len"], data_seed=c["seed"], struct_seed=c["seed"] + 1,
                             device=DEV)
    x.max_seq_len = c["cap"]
    if c["page"]:
        x = workloads.to_paged(x, page_size=c["page"], struct_seed=c["seed"] + 2)
        x.max_seq_len = c["cap"]
        need = -(-c["cap"] // c["page"])
        if x.block_table.shape[1] < need:   # the table must cover max_seq_len
            wide = torch.full((x.batch, need), -1, dtype=torch.int32, device=DEV)
            wide[:, :x.block_table.shape[1]] = x.block_table
            x.block_table = wide
    problem = fd.problem_of(x.q, x.k, x.max_seq_len, page_size=x.page_size, num_pages=x.num_pages)
    plan = fd.fd_plan_splits(problem, 0, c["splits"])
    if c["path"] is not None:
        plan.path = c["path"]
        if plan.mode == fd.FD_MODE_BALANCED:   # the tile follows the kernel
            plan.tile = _valu_tile(problem)
    if c["workers"] is not None and plan.mode == fd.FD_MODE_BALANCED:
        plan.workers = c["workers"]
        plan.lead_workers = c["workers"] // 2 if plan.lead_pct else 0
    need = fd.fd_workspace_size(problem, plan)
    assert need > 0, f"plan refused: {plan}"
    out = torch.empty(x.q.shape, dtype=x.out_dtype, device=DEV)
    lse = torch.empty(x.q.shape[:-1], dtype=torch.float32, device=DEV)
    lay = kv_layout(x)
    kw = dict(scale=x.scale, block_table=x.block_table, seq_lens_host=x.seq_lens_host)
    if c["entry"] == "two":
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        fd.fd_decode_partial(problem, plan, x.q, x.k, x.v, lay, x.seq_lens, ws, **kw)
        fd.fd_decode_combine(problem, plan, ws, out, lse)
    elif c["entry"] == "fused":
        ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
        fd.fd_decode(problem, plan, x.q, x.k, x.v, lay, x.seq_lens, ws, out, lse, **kw)
    else:
        if need > fd.STATIC_WORKSPACE_BYTES:
            pytest.skip("plan larger than the static workspace")
        fd.fd_decode_static(problem, plan, x.q, x.k, x.v, lay, x.seq_lens, out, lse, **kw)
    torch.cuda.synchronize()
    ref, ref_lse = reference(x)
    assert_out_close(out.reshape(-1, x.head_dim), ref, x.out_dtype)
    assert_lse_close(lse.reshape(-1), ref_lse, x.k.dtype)


def _valu_tile(problem):
    """The VALU kernel's tile for this problem: the planner's tile when it
    chooses the VALU path for a one-query-row copy of the problem."""
    p = fd.make_problem(problem.batch, problem.num_kv_heads, problem.num_kv_heads, problem.head_dim,
                        problem.max_seq_len, kv_dtype=problem.kv_dtype, q_dtype=problem.q_dtype,
                        out_dtype=problem.out_dtype, page_size=problem.page_size, num_pages=problem.num_pages)
    plan = fd.fd_plan_splits(p, 256, 0)
    assert plan.path == fd.FD_PATH_VALU
    return plan.tile
