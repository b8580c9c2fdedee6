"""The decode step captured in a HIP graph: the two-launch step, the single
launch and the step on the library's static workspace are each captured once
and replayed several times, with the inputs rewritten in place (new values,
new lengths) between replays by eager work on the same stream; every replay
must give exactly what the same call gives eagerly on those inputs, and stay
within the oracle's tolerances. The library itself records no memset into a
stream, so nothing in the graph depends on one."""
import pytest
import torch

import decode_attention_12_amd as fd
import workloads
from fdcheck import assert_lse_close, assert_out_close, kv_layout, reference

pytestmark = pytest.mark.gpu
DEV = "cuda"
REPLAYS = 3


def _banner(name):
    print(f"\n[case] {name}", flush=True)


def _inputs(i, cap=1500, paged=False):
    lens = workloads.uniform_lengths(6, 1, cap, struct_seed=5100 + i)
    x = workloads.contiguous(f"graph{i}", 6, 16, 4, 128, lens, cap=cap, data_seed=5000 + i, struct_seed=5100 + i,
                             device=DEV)
    x.max_seq_len = cap
    return x


def _launch(kind, problem, plan, x, ws, out, lse):
    lay = kv_layout(x)
    if kind == "two":
        fd.fd_decode_partial(problem, plan, x.q, x.k, x.v, lay, x.seq_lens, ws, scale=x.scale)
        fd.fd_decode_combine(problem, plan, ws, out, lse)
    elif kind == "fused":
        fd.fd_decode(problem, plan, x.q, x.k, x.v, lay, x.seq_lens, ws, out, lse, scale=x.scale)
    else:
        fd.fd_decode_static(problem, plan, x.q, x.k, x.v, lay, x.seq_lens, out, lse, scale=x.scale)


@pytest.mark.parametrize("splits", [0, 7])
@pytest.mark.parametrize("kind", ["two", "fused", "static"])
def test_graph_replays_match_eager_calls(kind, splits):
    _banner(f"graph replay: {kind}, splits={splits}")
    x = _inputs(0)
    problem = fd.problem_of(x.q, x.k, x.max_seq_len)
    plan = fd.fd_plan_splits(problem, 0, splits)
    ws = torch.zeros(fd.fd_workspace_size(problem, plan), dtype=torch.uint8, device=DEV)
    out = torch.empty(x.q.shape, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(x.q.shape[:-1], dtype=torch.float32, device=DEV)
    _launch(kind, problem, plan, x, ws, out, lse)   # eager warm-up before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _launch(kind, problem, plan, x, ws, out, lse)
    torch.cuda.synchronize()
    for r in range(1, REPLAYS + 1):
        y = _inputs(r)
        # Eager work between replays: the graph's input buffers rewritten in place.
        x.q.copy_(y.q)
        x.k.copy_(y.k)
        x.v.copy_(y.v)
        x.seq_lens.copy_(y.seq_lens)
        g.replay()
        torch.cuda.synchronize()
        got, got_lse = out.clone(), lse.clone()
        e_out = torch.empty_like(out)
        e_lse = torch.empty_like(lse)
        ews = torch.zeros_like(ws)
        _launch(kind, problem, plan, x, ews, e_out, e_lse)
        torch.cuda.synchronize()
        assert torch.equal(got, e_out) and torch.equal(got_lse, e_lse), f"replay {r} differs from the eager call"
        ref, ref_lse = reference(y)
        assert_out_close(got, ref, torch.bfloat16)
        assert_lse_close(got_lse, ref_lse, torch.bfloat16)
    del g
