"""fd_decode_static, the entry point that allocates nothing (its records live
in the library's static device workspace), against fd_decode_partial +
fd_decode_combine on a caller's workspace under the same plan: bit-identical
outputs and LSEs (the same kernels run in the same order), and both within
the oracle's tolerances, on two calls in a row whose second input is
smaller -- the static workspace keeps the first call's records, and the
second call must not read any of them. Plans whose workspace exceeds the
static one are refused before anything is launched."""
import pytest
import torch

import decode_attention_12_amd as fd
from decode_attention_12_amd import binding
import workloads
from fdcheck import assert_lse_close, assert_out_close, kv_layout, reference, run

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _banner(name):
    print(f"\n[case] {name}", flush=True)


def _static(x, splits):
    problem = fd.problem_of(x.q, x.k, x.max_seq_len, out_dtype=x.out_dtype, page_size=x.page_size,
                            num_pages=x.num_pages)
    plan = fd.fd_plan_splits(problem, 0, splits)
    out = torch.empty(x.q.shape, dtype=x.out_dtype, device=DEV)
    lse = torch.empty(x.q.shape[:-1], dtype=torch.float32, device=DEV)
    fd.fd_decode_static(problem, plan, x.q, x.k, x.v, kv_layout(x), x.seq_lens, out, lse, scale=x.scale,
                        block_table=x.block_table, seq_lens_host=x.seq_lens_host)
    torch.cuda.synchronize()
    return out, lse, plan, fd.fd_workspace_size(problem, plan)


def _pair(first, second, splits):
    for x in (first, second):
        out_s, lse_s, plan_s, need = _static(x, splits)
        assert need <= fd.STATIC_WORKSPACE_BYTES
        out_r, lse_r, plan_r, _ = run(x, splits=splits)
        assert bytes(plan_s) == bytes(plan_r)
        assert torch.equal(out_s, out_r), "static workspace and caller's workspace disagree"
        assert torch.equal(lse_s, lse_r)
        ref, ref_lse = reference(x)
        assert_out_close(out_s.reshape(-1, x.head_dim), ref, x.out_dtype)
        assert_lse_close(lse_s.reshape(-1), ref_lse, x.k.dtype)


@pytest.mark.parametrize("splits", [0, 8])
def test_static_short_batch_then_smaller(splits):
    """The short-context batch (128 sequences), then a batch of 5."""
    _banner(f"static workspace: short-context batch, then a smaller batch, splits={splits}")
    big = workloads.c5_short_batch(device=DEV)
    small = workloads.contiguous("static-small", 5, 32, 8, 128, [700, 1, 2048, 33, 512], cap=2048,
                                 data_seed=4800, struct_seed=4801, device=DEV)
    _pair(big, small, splits)


@pytest.mark.parametrize("splits", [0, 5])
def test_static_paged_fp8_then_smaller(splits):
    """A paged fp8 batch of 8, then a paged bf16 batch of 3."""
    _banner(f"static workspace: paged fp8 batch, then a smaller paged batch, splits={splits}")
    lens1 = workloads.uniform_lengths(8, 100, 5000, struct_seed=4810)
    first = workloads.paged("static-p1", 8, 32, 8, 128, lens1, dtype=workloads.FP8, data_seed=4811,
                            struct_seed=4812, device=DEV)
    second = workloads.paged("static-p2", 3, 16, 4, 128, [90, 1500, 17], data_seed=4813, struct_seed=4814,
                             device=DEV)
    _pair(first, second, splits)


def test_static_refuses_a_plan_larger_than_its_workspace():
    """The short-context batch at 16 splits needs 33.8 MB of records, over the
    32 MiB static workspace: refused on the host, nothing launched."""
    _banner("static workspace: plan too large")
    x = workloads.c5_short_batch(device=DEV)
    with pytest.raises(fd.FdError) as e:
        _static(x, 16)
    assert e.value.status == binding.FD_ERR_WORKSPACE_TOO_SMALL


def test_static_on_a_side_stream():
    """On a stream other than the current one, the call uses the array of
    that stream's GPU and gives the same bytes as on the current stream."""
    _banner("static workspace: side stream")
    x = workloads.contiguous("static-side", 3, 32, 8, 128, [1500, 64, 900], cap=2048, data_seed=4820,
                             struct_seed=4821, device=DEV)
    out_a, lse_a, plan, _ = _static(x, 0)
    problem = fd.problem_of(x.q, x.k, x.max_seq_len, out_dtype=x.out_dtype, page_size=x.page_size,
                            num_pages=x.num_pages)
    out_b = torch.full(x.q.shape, float("nan"), dtype=x.out_dtype, device=DEV)
    lse_b = torch.full(x.q.shape[:-1], float("nan"), dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    fd.fd_decode_static(problem, plan, x.q, x.k, x.v, kv_layout(x), x.seq_lens, out_b, lse_b, scale=x.scale,
                        seq_lens_host=x.seq_lens_host, stream=side)
    side.synchronize()
    assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b)
