"""Stream ordering of the workspace: the merge must see every piece record
before it reads any, and the next step's pieces must not overwrite records
that a merge still reads. Each edge is tested with the producer held back by
a long spin on its stream, over inputs that differ between steps, and each
has a negative control -- the same calls without the edge -- which must go
wrong, so the positive tests are known to overlap the two streams for real.

The races of the negative controls are plain reads of finite-range memory
(split mode only: record positions there do not depend on workspace
contents), never an access outside the workspace."""
import pytest
import torch

import decode_attention_12_amd as fd
import workloads
from fdcheck import BF16_ATOL, BF16_RTOL, assert_lse_close, assert_out_close, reference

pytestmark = pytest.mark.gpu
DEV = "cuda"
SPIN = 50_000_000   # clock cycles of torch.cuda._sleep: tens of milliseconds


def _banner(name):
    print(f"\n[case] {name}", flush=True)


_PAIR = []


def stream_pair():
    """Two streams whose work the device runs concurrently. Streams share the
    process's few hardware queues, and two streams on one queue run in
    submission order, which would make every test here vacuous; so a pair is
    taken only after a probe shows that a small kernel on the second stream
    finishes while a spin on the first is still running."""
    if _PAIR:
        return _PAIR[0]
    for _ in range(16):
        sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.stream(sa):
            torch.cuda._sleep(SPIN)
        with torch.cuda.stream(sb):
            torch.zeros(1, device=DEV)
            done = torch.cuda.Event()
            done.record(sb)
        done.synchronize()
        overlapped = not sa.query()
        torch.cuda.synchronize()
        if overlapped:
            _PAIR.append((sa, sb))
            return sa, sb
    raise AssertionError("no two streams ran concurrently: the ordering tests could show nothing")


def _gqa(seed, length=4096):
    x = workloads.contiguous(f"ord{seed}", 1, 32, 8, 128, [length], cap=4096, dtype=torch.bfloat16,
                             data_seed=seed, struct_seed=seed + 1, device=DEV)
    x.max_seq_len = 4096
    return x


def _within(out, ref):
    got = out.double().cpu().reshape(ref.shape)
    return bool(torch.isfinite(got).all()) and bool(((got - ref).abs() <= BF16_ATOL + BF16_RTOL * ref.abs()).all())


def _combine_behind_partial(x, plan, with_edge):
    problem = fd.problem_of(x.q, x.k, x.max_seq_len)
    ws = torch.full((fd.fd_workspace_size(problem, plan) // 4,), float("nan"), device=DEV)
    out = torch.empty(x.q.shape, dtype=torch.bfloat16, device=DEV)
    sa, sb = stream_pair()
    torch.cuda.synchronize()
    with torch.cuda.stream(sa):
        torch.cuda._sleep(SPIN)
        fd.fd_decode_partial(problem, plan, x.q, x.k, x.v, fd.layout_of(x.k), x.seq_lens, ws, scale=x.scale,
                             stream=sa)
    with torch.cuda.stream(sb):
        fd.fd_decode_combine(problem, plan, ws, out, None, stream=sb, partial_stream=sa if with_edge else None)
    torch.cuda.synchronize()
    return out


def test_combine_waits_for_the_partial_stream():
    """Partial on stream A behind a long spin, combine on stream B with
    partial_stream = A, over a workspace poisoned with NaN."""
    _banner("combine after partial_stream")
    x = _gqa(4100)
    plan = fd.fd_plan_splits(fd.problem_of(x.q, x.k, x.max_seq_len), 0, 8)
    out = _combine_behind_partial(x, plan, with_edge=True)
    ref, _ = reference(x)
    assert_out_close(out, ref, torch.bfloat16)


def test_combine_without_the_edge_races():
    """Negative control: the same calls without partial_stream. The combine
    runs while the partial is still held back and reads the NaN records."""
    _banner("combine without partial_stream (negative control)")
    x = _gqa(4100)
    plan = fd.fd_plan_splits(fd.problem_of(x.q, x.k, x.max_seq_len), 0, 8)
    out = _combine_behind_partial(x, plan, with_edge=False)
    ref, _ = reference(x)
    assert not _within(out, ref), "the combine did not overlap the held-back partial: the edge test shows nothing"


def _next_partial_after_combine(x1, x2, plan, with_edge):
    """Step 1: partial on A, combine on B (behind a spin). Step 2: partial on
    A over the same workspace, after_stream = B when with_edge, then its
    combine on A. Returns both steps' outputs and LSEs."""
    problem = fd.problem_of(x1.q, x1.k, x1.max_seq_len)
    ws = torch.full((fd.fd_workspace_size(problem, plan) // 4,), float("nan"), device=DEV)
    outs = [torch.empty(x1.q.shape, dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    lses = [torch.empty(x1.q.shape[:-1], dtype=torch.float32, device=DEV) for _ in range(2)]
    sa, sb = stream_pair()
    torch.cuda.synchronize()
    with torch.cuda.stream(sa):
        fd.fd_decode_partial(problem, plan, x1.q, x1.k, x1.v, fd.layout_of(x1.k), x1.seq_lens, ws,
                             scale=x1.scale, stream=sa)
    with torch.cuda.stream(sb):
        torch.cuda._sleep(SPIN)
        fd.fd_decode_combine(problem, plan, ws, outs[0], lses[0], stream=sb, partial_stream=sa)
    with torch.cuda.stream(sa):
        fd.fd_decode_partial(problem, plan, x2.q, x2.k, x2.v, fd.layout_of(x2.k), x2.seq_lens, ws,
                             scale=x2.scale, stream=sa, after_stream=sb if with_edge else None)
        fd.fd_decode_combine(problem, plan, ws, outs[1], lses[1], stream=sa)
    torch.cuda.synchronize()
    return outs, lses


@pytest.mark.parametrize("mode", ["splits", "balanced"])
def test_partial_waits_for_the_previous_combine(mode):
    """after_stream: the next step's partial must not overwrite records the
    previous combine (on another stream, held back) still reads. Both steps
    against the oracle on their own inputs. Balanced mode keeps the lengths
    between the steps (the running tile counts in the workspace then agree);
    the values differ."""
    _banner(f"partial after the previous combine ({mode})")
    x1 = _gqa(4200, length=4096)
    x2 = _gqa(4300, length=2999 if mode == "splits" else 4096)
    plan = fd.fd_plan_splits(fd.problem_of(x1.q, x1.k, x1.max_seq_len), 0, 8 if mode == "splits" else 0)
    outs, lses = _next_partial_after_combine(x1, x2, plan, with_edge=True)
    for x, out, lse in ((x1, outs[0], lses[0]), (x2, outs[1], lses[1])):
        ref, ref_lse = reference(x)
        assert_out_close(out, ref, torch.bfloat16)
        assert_lse_close(lse, ref_lse, torch.bfloat16)


def test_partial_without_after_stream_races():
    """Negative control: without after_stream the second step's partial runs
    while the first step's combine is held back, so that combine merges the
    second step's records."""
    _banner("partial without after_stream (negative control)")
    x1 = _gqa(4200, length=4096)
    x2 = _gqa(4300, length=2999)
    plan = fd.fd_plan_splits(fd.problem_of(x1.q, x1.k, x1.max_seq_len), 0, 8)
    outs, _ = _next_partial_after_combine(x1, x2, plan, with_edge=False)
    ref1, _ = reference(x1)
    assert not _within(outs[0], ref1), "no overlap: the after_stream test shows nothing"


def test_fused_decode_waits_for_the_previous_user():
    """fd_decode's after_stream: a single-launch step on stream B (behind a
    spin) and the next one on stream A over the same workspace, counters
    included; both against the oracle."""
    _banner("fd_decode after_stream")
    x1 = _gqa(4400, length=4096)
    x2 = _gqa(4500, length=3001)
    problem = fd.problem_of(x1.q, x1.k, x1.max_seq_len)
    plan = fd.fd_plan_splits(problem, 0, 16)
    ws = torch.zeros(fd.fd_workspace_size(problem, plan), dtype=torch.uint8, device=DEV)
    outs = [torch.empty(x1.q.shape, dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    sa, sb = stream_pair()
    torch.cuda.synchronize()
    with torch.cuda.stream(sb):
        torch.cuda._sleep(SPIN)
        fd.fd_decode(problem, plan, x1.q, x1.k, x1.v, fd.layout_of(x1.k), x1.seq_lens, ws, outs[0], scale=x1.scale,
                     stream=sb)
    with torch.cuda.stream(sa):
        fd.fd_decode(problem, plan, x2.q, x2.k, x2.v, fd.layout_of(x2.k), x2.seq_lens, ws, outs[1], scale=x2.scale,
                     stream=sa, after_stream=sb)
    torch.cuda.synchronize()
    for x, out in ((x1, outs[0]), (x2, outs[1])):
        ref, _ = reference(x)
        assert_out_close(out, ref, torch.bfloat16)
    n = problem.batch * 8   # B x J counters (one row tile per KV head here)
    assert (ws[:4 * n].view(torch.int32) == 0).all()
