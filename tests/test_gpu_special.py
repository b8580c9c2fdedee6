"""Special cases whose results have closed forms, through the GPU path, on
every kernel family (fp32 VALU, bf16 MFMA, fp8 MFMA) and both modes:

  q = 0          every score is 0: out = the mean of the visible value rows,
                 lse = log n (n = keys the row sees);
  one key        out = v_0, lse = s_0 = scale <q, k_0>;
  two keys       out = (1 - w) v_0 + w v_1 with the logistic weight
                 w = 1 / (1 + exp(s_0 - s_1));
  huge scale     scores spread by thousands: the softmax is one-hot at the
                 largest score (out = that key's value row), and nothing
                 overflows.

The closed forms are evaluated in float64 from the stored (rounded) bytes,
and the oracle is checked alongside, so a kernel mistake cannot hide behind
a shared misreading."""
import math

import pytest
import torch

import oracle
import workloads
from fdcheck import assert_lse_close, assert_out_close, host, reference, run

pytestmark = pytest.mark.gpu
DEV = "cuda"
KINDS = [(torch.float32, 1, 64), (torch.bfloat16, 4, 128), (workloads.FP8, 4, 128)]


def _banner(name):
    print(f"\n[case] {name}", flush=True)


def _f64(x, t, kv):
    """float64 values of a cache tensor t (fp8: decoded bytes x the head's scale)."""
    if t.dtype == workloads.FP8:
        codes = t.view(torch.uint8).cpu()
        vals = oracle.decode_e4m3(codes.reshape(-1)).reshape(codes.shape)
        return vals * kv.cpu().double().reshape(1, -1, 1, 1)
    return t.cpu().double()


@pytest.mark.parametrize("splits", [0, 3])
@pytest.mark.parametrize("dtype,group,D", KINDS)
def test_zero_query_gives_the_mean_and_log_n(dtype, group, D, splits):
    _banner(f"q = 0: {dtype} group {group} D {D} splits {splits}")
    lens = [1, 17, 300, 64]
    x = workloads.contiguous("q0", len(lens), 2 * group, 2, D, lens, dtype=dtype, data_seed=5300 + D,
                             struct_seed=5301, device=DEV)
    x.q.zero_()
    out, lse, plan, _ = run(x, splits=splits)
    v = _f64(x, x.v, x.v_scale) if x.v_scale is not None else x.v.cpu().double()
    want = torch.stack([v[b, h // group, :L].mean(dim=0) for b, L in enumerate(lens) for h in range(2 * group)])
    want_lse = torch.tensor([math.log(L) for L in lens for _ in range(2 * group)], dtype=torch.float64)
    assert_out_close(out.reshape(-1, D), want, x.out_dtype)
    assert_lse_close(lse.reshape(-1), want_lse, x.k.dtype)
    ref, ref_lse = reference(x)
    assert_out_close(out.reshape(-1, D), ref, x.out_dtype)


@pytest.mark.parametrize("dtype,group,D", KINDS)
def test_one_and_two_keys(dtype, group, D):
    _banner(f"one and two keys: {dtype} group {group} D {D}")
    lens = [1, 2, 1, 2]
    x = workloads.contiguous("k12", len(lens), 2 * group, 2, D, lens, dtype=dtype, data_seed=5400 + D,
                             struct_seed=5401, device=DEV)
    out, lse, plan, _ = run(x, splits=0)
    q = x.q.cpu().double()
    k = _f64(x, x.k, x.k_scale) if x.k_scale is not None else x.k.cpu().double()
    v = _f64(x, x.v, x.v_scale) if x.v_scale is not None else x.v.cpu().double()
    want, want_lse = [], []
    for b, L in enumerate(lens):
        for h in range(2 * group):
            s = [x.scale * float(q[b, h] @ k[b, h // group, j]) for j in range(L)]
            if L == 1:
                want.append(v[b, h // group, 0])
                want_lse.append(s[0])
            else:
                w = 1.0 / (1.0 + math.exp(s[0] - s[1]))
                want.append((1.0 - w) * v[b, h // group, 0] + w * v[b, h // group, 1])
                m = max(s)
                want_lse.append(m + math.log(sum(math.exp(t - m) for t in s)))
    assert_out_close(out.reshape(-1, D), torch.stack(want), x.out_dtype)
    assert_lse_close(lse.reshape(-1), torch.tensor(want_lse, dtype=torch.float64), x.k.dtype)


@pytest.mark.parametrize("splits", [0, 5])
@pytest.mark.parametrize("dtype,group,D", KINDS)
def test_huge_scale_is_one_hot_and_finite(dtype, group, D, splits):
    _banner(f"huge scale: {dtype} group {group} D {D} splits {splits}")
    lens = [700, 33, 1000]
    x = workloads.contiguous("big", len(lens), 2 * group, 2, D, lens, dtype=dtype, data_seed=5500 + D,
                             struct_seed=5501, device=DEV, scale=400.0 / math.sqrt(D))
    out, lse, plan, _ = run(x, splits=splits)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    ref, ref_lse = reference(x, hx=host(x))
    assert_out_close(out.reshape(-1, D), ref, x.out_dtype)
    assert_lse_close(lse.reshape(-1), ref_lse, x.k.dtype)
    # The reference itself is one-hot: its output is the top key's value row.
    q = x.q.cpu().double()
    k = _f64(x, x.k, x.k_scale) if x.k_scale is not None else x.k.cpu().double()
    v = _f64(x, x.v, x.v_scale) if x.v_scale is not None else x.v.cpu().double()
    r = 0
    for b, L in enumerate(lens):
        for h in range(2 * group):
            s = (k[b, h // group, :L] @ q[b, h]) * x.scale
            top = int(torch.argmax(s))
            gap = float(s[top] - torch.topk(s, 2).values[1])
            if gap > 40.0:   # one-hot to double precision
                assert torch.allclose(ref[r], v[b, h // group, top], rtol=0, atol=1e-12)
            r += 1
