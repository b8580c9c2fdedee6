"""GPU parity at the edges of the supported shapes: a million-key sequence,
thousands of tiny sequences, the largest q_len, an fp8 cache seen through
token-major strides, and a max_seq_len far above the real lengths."""
import pytest
import torch

import decode_attention_12_amd as fd
import workloads
from fdcheck import assert_lse_close, assert_out_close, host, reference, run

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _banner(name):
    print(f"\n[case] {name}", flush=True)


def test_one_million_keys_sampled_rows():
    """B1, 32/8 heads, 2^20 keys: 8 segments of 32768 tiles cut over the
    balanced workers; 8 sampled rows against the oracle."""
    _banner("one sequence of 2^20 keys")
    L = 1 << 20
    x = workloads.contiguous("1m", 1, 32, 8, 128, [L], dtype=torch.bfloat16, data_seed=901, struct_seed=902,
                             device=DEV)
    out, lse, plan, _ = run(x, splits=0)
    assert plan.mode == fd.FD_MODE_BALANCED
    rows = [(0, 0, h) for h in (0, 5, 9, 14, 18, 23, 27, 31)]
    ref, ref_lse = reference(x, rows=rows)
    got = torch.stack([out[0, h] for _, _, h in rows])
    assert_out_close(got, ref, torch.bfloat16)
    assert_lse_close(torch.stack([lse[0, h] for _, _, h in rows]), ref_lse, torch.bfloat16)
    del x
    torch.cuda.empty_cache()


@pytest.mark.parametrize("Hq,Hkv,dtype", [(8, 2, torch.bfloat16), (4, 4, torch.bfloat16), (2, 1, torch.float32)])
def test_thousands_of_tiny_sequences(Hq, Hkv, dtype):
    _banner(f"2048 sequences of 1..24 keys, Hq={Hq} Hkv={Hkv} {dtype}")
    lens = workloads.uniform_lengths(2048, 1, 24, struct_seed=903)
    x = workloads.contiguous("tiny-many", 2048, Hq, Hkv, 128, lens, cap=32, dtype=dtype, data_seed=904,
                             struct_seed=903, device=DEV)
    hx = host(x)
    ref, ref_lse = reference(x, hx=hx)
    for splits in (0, 2):
        out, lse, plan, _ = run(x, splits=splits)
        assert_out_close(out.reshape(-1, 128), ref, x.out_dtype)
        assert_lse_close(lse.reshape(-1), ref_lse, dtype)


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (16, 2)])
def test_largest_q_len(Hq, Hkv):
    """q_len 16: 16 rows per KV head for MHA (one full MFMA tile), 128 for
    group 8 (eight tiles of 16)."""
    _banner(f"q_len 16 Hq={Hq} Hkv={Hkv}")
    lens = [16, 700, 33]
    x = workloads.contiguous("t16", 3, Hq, Hkv, 128, lens, dtype=torch.bfloat16, q_len=16, data_seed=905,
                             struct_seed=906, device=DEV)
    ref, ref_lse = reference(x)
    for splits in (0, 3):
        out, lse, plan, _ = run(x, splits=splits)
        assert plan.path == fd.FD_PATH_MFMA
        assert_out_close(out.reshape(-1, 128), ref, torch.bfloat16)
        assert_lse_close(lse.reshape(-1), ref_lse, torch.bfloat16)


def test_fp8_token_major_strides_match_head_major():
    _banner("fp8 token-major strides")
    lens = [300, 45]
    x = workloads.contiguous("f8tm", 2, 8, 2, 128, lens, dtype=workloads.FP8, data_seed=907, struct_seed=908,
                             device=DEV)
    out1, lse1, _, _ = run(x, splits=0)
    tm_k = x.k.permute(0, 2, 1, 3).contiguous()       # [B][L][Hkv][D] storage
    tm_v = x.v.permute(0, 2, 1, 3).contiguous()
    x.k, x.v = tm_k.permute(0, 2, 1, 3), tm_v.permute(0, 2, 1, 3)
    out2, lse2, _, _ = run(x, splits=0)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_max_seq_len_far_above_the_lengths():
    """The plan covers 2^16 keys while the sequences hold at most 300: the
    result is the same as with a tight max_seq_len."""
    _banner("loose max_seq_len")
    lens = [300, 5, 128]
    x = workloads.contiguous("loose", 3, 8, 2, 128, lens, cap=1 << 16, dtype=torch.bfloat16, data_seed=909,
                             struct_seed=910, device=DEV)
    ref, ref_lse = reference(x)
    x.max_seq_len = 1 << 16
    for splits in (0, 64):
        out, lse, plan, _ = run(x, splits=splits, host_lens=False)
        assert_out_close(out, ref, torch.bfloat16)
        assert_lse_close(lse, ref_lse, torch.bfloat16)


@pytest.mark.parametrize("page", [32, 64, 256])
@pytest.mark.parametrize("Hq,Hkv,dtype", [(8, 2, torch.bfloat16), (4, 4, torch.bfloat16), (8, 2, workloads.FP8),
                                          (2, 2, torch.float32)])
def test_larger_pages(page, Hq, Hkv, dtype):
    """Pages of 32 .. 256 keys: a 16-key group is found inside its page by
    the key's offset in the page; shuffled pool, ragged lengths."""
    _banner(f"page {page} Hq={Hq} Hkv={Hkv} {dtype}")
    lens = [700, 17, 256, 1000]
    x = workloads.contiguous("pg", len(lens), Hq, Hkv, 128, lens, dtype=dtype, data_seed=920 + page,
                             struct_seed=921, device=DEV)
    p = workloads.to_paged(x, page_size=page, struct_seed=922)
    hx = host(p)
    ref, ref_lse = reference(p, hx=hx)
    for splits in (0, 3):
        out, lse, plan, _ = run(p, splits=splits)
        assert_out_close(out.reshape(-1, 128), ref, p.out_dtype)
        assert_lse_close(lse.reshape(-1), ref_lse, dtype)
    ref_c, _ = reference(x)
    torch.testing.assert_close(ref, ref_c, rtol=0, atol=0)


def test_shared_prefix_pages():
    """Two sequences whose block tables share their first pages (a common
    prefix kept once in the pool) read them as their own keys."""
    _banner("shared prefix pages")
    lens = [96, 96]
    x = workloads.contiguous("pfx", 2, 8, 2, 128, lens, dtype=torch.bfloat16, data_seed=930, struct_seed=931,
                             device=DEV)
    x.k[1, :, :64] = x.k[0, :, :64]
    x.v[1, :, :64] = x.v[0, :, :64]
    p = workloads.to_paged(x, page_size=32, struct_seed=932)
    table = p.block_table.clone()
    table[1, :2] = table[0, :2]            # sequence 1 reads sequence 0's first two pages
    p.block_table = table
    ref, ref_lse = reference(p)
    ref_x, _ = reference(x)
    torch.testing.assert_close(ref, ref_x, rtol=0, atol=0)
    out, lse, plan, _ = run(p, splits=0)
    assert_out_close(out.reshape(-1, 128), ref, torch.bfloat16)
