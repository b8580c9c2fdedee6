"""GPU parity for multi-token decode (q_len query tokens per sequence under
the causal window: token t of q_len sees keys 0 .. L_b - q_len + t) and for
fp8 (E4M3) KV caches with per-KV-head scales, through the C ABI against the
fp64 oracle on the same bytes. Both paths (VALU / MFMA), both modes (fixed
splits / balanced workers), contiguous and paged caches, the two-launch and
the single-launch step; every piece record is checked as well."""
import pytest
import torch

import decode_attention_12_amd as fd
import workloads
from fdcheck import (assert_lse_close, assert_out_close, assert_records_close, check_fused_steps, host, reference,
                     run)

pytestmark = pytest.mark.gpu
DEV = "cuda"
FP8 = workloads.FP8


def _banner(name):
    print(f"\n[case] {name}", flush=True)


def _x(B, Hq, Hkv, D, lens, *, dtype=torch.bfloat16, q_len=1, seed=0, paged=False, cap=None):
    x = workloads.contiguous(f"mt{q_len}-{Hq}x{Hkv}", B, Hq, Hkv, D, lens, cap=cap, dtype=dtype, q_len=q_len,
                             data_seed=500 + seed, struct_seed=600 + seed, device=DEV)
    return workloads.to_paged(x, struct_seed=700 + seed) if paged else x


def _check(x, *, splits, workers=None, path=None, out_dtype=None, host_lens=True, records=True):
    hx = host(x)
    ref, ref_lse = reference(x, hx=hx)
    out, lse, plan, ws = run(x, splits=splits, workers=workers, path=path, out_dtype=out_dtype,
                             host_lens=host_lens)
    if path is not None:
        assert plan.path == path
    D = x.head_dim
    assert_out_close(out.reshape(-1, D), ref, out_dtype or x.out_dtype)
    assert_lse_close(lse.reshape(-1), ref_lse, x.k.dtype)
    if records:
        assert_records_close(x, plan, ws, hx)
    return out, lse, plan


# --------------------------------------------------------------------------
# Multi-token decode.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("q_len,Hq,Hkv,want", [
    (2, 8, 8, fd.FD_PATH_VALU),      # MHA, 2 rows per KV head: VALU
    (3, 8, 8, fd.FD_PATH_VALU),
    (4, 8, 8, fd.FD_PATH_MFMA),      # MHA, 4 rows: one MFMA tile
    (8, 4, 4, fd.FD_PATH_MFMA),
    (2, 8, 2, fd.FD_PATH_MFMA),      # GQA 4 x 2 tokens: 8 rows
    (5, 8, 2, fd.FD_PATH_MFMA),      # 20 rows: two tiles of 10
    (3, 16, 2, fd.FD_PATH_MFMA),     # 24 rows: two tiles of 12
    (8, 16, 2, fd.FD_PATH_MFMA),     # 64 rows: four tiles of 16
])
@pytest.mark.parametrize("splits", [0, 5])
def test_multi_token_bf16(q_len, Hq, Hkv, want, splits):
    _banner(f"multi-token bf16 q_len={q_len} Hq={Hq} Hkv={Hkv} splits={splits}")
    lens = [q_len, 300, 77, 1024, 45]
    x = _x(len(lens), Hq, Hkv, 128, lens, q_len=q_len, seed=q_len + Hq)
    _, _, plan = _check(x, splits=splits)
    assert plan.path == want


@pytest.mark.parametrize("q_len", [2, 3, 7])
@pytest.mark.parametrize("paged", [False, True])
def test_multi_token_fp32_valu(q_len, paged):
    _banner(f"multi-token fp32 D64 q_len={q_len} paged={paged}")
    lens = [40, q_len, 129, 16]
    x = _x(len(lens), 4, 2, 64, lens, dtype=torch.float32, q_len=q_len, seed=10 + q_len, paged=paged)
    for splits in (0, 3):
        _check(x, splits=splits)


@pytest.mark.parametrize("workers", [1, 3, 64, 1000])
def test_multi_token_balanced_partitions_and_short_sequences(workers):
    """Sequences shorter than q_len: the rows whose window is empty come out
    as 0 and -inf (host length check left out), the others as the oracle's."""
    _banner(f"multi-token balanced workers={workers}")
    q_len = 4
    lens = [2, 200, 4, 1, 90]
    x = _x(len(lens), 8, 2, 128, lens, q_len=q_len, seed=20)
    out, lse, plan, ws = run(x, splits=0, workers=workers, host_lens=False)
    assert plan.mode == fd.FD_MODE_BALANCED and plan.path == fd.FD_PATH_MFMA
    live = [(b, t, h) for b, L in enumerate(lens) for t in range(q_len) for h in range(8) if L - q_len + t + 1 > 0]
    dead = [(b, t) for b, L in enumerate(lens) for t in range(q_len) if L - q_len + t + 1 <= 0]
    assert dead, "the case needs rows that see no key"
    for b, t in dead:
        assert (out[b, t] == 0).all() and torch.isinf(lse[b, t]).all() and (lse[b, t] < 0).all()
    ref, ref_lse = reference(x, rows=live)
    got = torch.stack([out[b, t, h] for b, t, h in live])
    got_lse = torch.stack([lse[b, t, h] for b, t, h in live])
    assert_out_close(got, ref, torch.bfloat16)
    assert_lse_close(got_lse, ref_lse, torch.bfloat16)


@pytest.mark.parametrize("splits", [0, 6])
def test_multi_token_fused_single_launch(splits):
    """Three single-launch steps of 3 query tokens on one workspace, fresh
    values and lengths each step."""
    _banner(f"multi-token fused, splits={splits}")
    q_len = 3
    lens = [[500, 3, 64, 1500], [17, 1500, 900, 4], [1499, 250, 3, 77]]
    steps = (workloads.contiguous(f"mtf-{i}", 4, 16, 2, 128, L, cap=1500, q_len=q_len, data_seed=530 + i,
                                  struct_seed=630 + i, device=DEV) for i, L in enumerate(lens))

    def tight(xs):
        for x in xs:
            x.max_seq_len = 1500
            yield x
    assert check_fused_steps(tight(steps), splits=splits) == 3


def test_multi_token_one_token_equals_plain_decode():
    """q [B][1][Hq][D] and q [B][Hq][D] give the same bytes."""
    _banner("multi-token q_len=1 layout")
    lens = [300, 77]
    x = _x(2, 8, 2, 128, lens, seed=40)
    out1, lse1, _, _ = run(x, splits=0)
    x.q = x.q.unsqueeze(1).contiguous()
    out2, lse2, _, _ = run(x, splits=0)
    assert torch.equal(out1, out2.squeeze(1)) and torch.equal(lse1, lse2.squeeze(1))


# --------------------------------------------------------------------------
# fp8 (E4M3) KV cache with per-head scales.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("Hq,Hkv,D,want", [
    (8, 8, 128, fd.FD_PATH_VALU),     # MHA
    (8, 2, 128, fd.FD_PATH_MFMA),     # GQA 4
    (16, 2, 128, fd.FD_PATH_MFMA),    # GQA 8
    (8, 4, 64, fd.FD_PATH_VALU),      # head_dim 64, 2-row VALU tiles
    (3, 3, 64, fd.FD_PATH_VALU),
])
@pytest.mark.parametrize("splits", [0, 4])
@pytest.mark.parametrize("paged", [False, True])
def test_fp8_cache(Hq, Hkv, D, want, splits, paged):
    _banner(f"fp8 Hq={Hq} Hkv={Hkv} D={D} splits={splits} paged={paged}")
    lens = [700, 33, 256, 1]
    x = _x(len(lens), Hq, Hkv, D, lens, dtype=FP8, seed=50 + Hq + D, paged=paged)
    assert x.k.dtype == FP8 and x.q.dtype == torch.bfloat16
    _, _, plan = _check(x, splits=splits)
    assert plan.path == want


@pytest.mark.parametrize("path", [fd.FD_PATH_MFMA, fd.FD_PATH_VALU])
def test_fp8_both_paths_and_fp32_output(path):
    _banner(f"fp8 forced path {path}, fp32 output")
    lens = [1000, 17, 333]
    x = _x(len(lens), 8, 2, 128, lens, dtype=FP8, seed=60)
    # A forced path goes with a split plan: a balanced plan's tile is the
    # planner's kernel's.
    _check(x, splits=6, path=path, out_dtype=torch.float32)


def test_fp8_scales_reach_the_result():
    """The same fp8 bytes with doubled value scales give doubled outputs; with
    doubled key scales, the result of doubled softmax scale."""
    _banner("fp8 scales")
    lens = [400, 90]
    x = _x(2, 8, 2, 128, lens, dtype=FP8, seed=61)
    out, lse, _, _ = run(x, splits=0, out_dtype=torch.float32)
    vs = x.v_scale.clone()
    x.v_scale = (2 * vs).contiguous()
    out2, lse2, _, _ = run(x, splits=0, out_dtype=torch.float32)
    torch.testing.assert_close(out2, 2 * out, rtol=1e-6, atol=1e-6)
    assert torch.equal(lse, lse2)
    x.v_scale = vs
    ref, ref_lse = reference(x)
    x.k_scale = (2 * x.k_scale).contiguous()
    out3, lse3, _, _ = run(x, splits=0, out_dtype=torch.float32)
    y_ref, y_lse = reference(x)
    assert_out_close(out3.reshape(-1, 128).to(torch.bfloat16), y_ref, torch.bfloat16)
    assert_lse_close(lse3.reshape(-1), y_lse, FP8)
    assert not torch.allclose(y_ref, ref)


@pytest.mark.parametrize("q_len", [2, 4])
def test_fp8_multi_token(q_len):
    _banner(f"fp8 multi-token q_len={q_len}")
    lens = [600, q_len, 95]
    for Hq, Hkv in ((8, 8), (8, 2)):
        x = _x(len(lens), Hq, Hkv, 128, lens, dtype=FP8, q_len=q_len, seed=70 + Hq + q_len)
        _check(x, splits=0)
        _check(x, splits=3)


def test_fp8_fused_paged():
    """Three single-launch steps over fp8 paged caches on one workspace."""
    _banner("fp8 fused paged")
    lens = [[2000, 1, 513, 64, 900], [64, 2000, 1, 1200, 33], [999, 800, 2000, 5, 1]]

    def steps():
        for i, L in enumerate(lens):
            x = workloads.paged(f"f8fp-{i}", 5, 16, 2, 128, L, page_size=16, max_pages=125, dtype=FP8,
                                data_seed=580 + i, struct_seed=680 + i, device=DEV)
            x.max_seq_len = 2000
            yield x
    assert check_fused_steps(steps(), splits=0) == 3


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("splits", [0, 4])
def test_fp8_mfma_second_half_keys_dominate(splits, paged):
    """The fp8 MFMA kernel copies K into LDS and waits for each 16-key half of
    a 32-key tile by counting the loads issued after it. Here some keys in
    the second half of tiles (key % 32 >= 16; splits of 384 keys keep tiles
    aligned) carry a +12 score offset, reaching every row of the group
    through one shared query vector, so they dominate the softmax: scoring
    them with stale K (an LDS read before the copy landed) would move the
    outputs far outside tolerance."""
    _banner(f"fp8 MFMA second-half keys dominate, splits={splits}, paged={paged}")
    lens = [1024, 777, 1500]
    g = torch.Generator().manual_seed(4711)
    offsets = {}
    for b, L in enumerate(lens):
        cand = torch.tensor([j for j in range(L) if j % 32 >= 16])
        for h in range(2):
            offsets[(b, h)] = sorted(cand[torch.randperm(len(cand), generator=g)[:len(cand) // 12]].tolist())
    x = workloads.contiguous("lds-late", len(lens), 16, 2, 128, lens, dtype=FP8, shared_q=True, offsets=offsets,
                             delta=12.0, data_seed=590, struct_seed=690, device=DEV)
    if paged:
        x = workloads.to_paged(x, struct_seed=691)
    ref, ref_lse = reference(x)
    lnL = torch.tensor([float(L) for L in lens]).log().repeat_interleave(16).double()
    assert (ref_lse - lnL).min().item() > 4.0, "the offset keys should dominate every row"
    out, lse, plan, _ = run(x, splits=splits)
    assert plan.path == fd.FD_PATH_MFMA
    if splits:
        assert plan.chunk_len % 32 == 0
    assert_out_close(out.reshape(-1, 128), ref, torch.bfloat16)
    assert_lse_close(lse.reshape(-1), ref_lse, FP8)
