"""Pins for the fp64 oracle: facts fixed by the pages, by closed forms, by
library routines and by brute force, none of them the oracle's own code.

Mistakes each group would catch:
  golden example   -> wrong merge weights (e.g. exp(m_i - M) on normalised outputs),
                      averaging, wrong LSE definition
  SDPA / logsumexp -> dropped or wrong scale, transposed operands, wrong GQA index,
                      wrong LSE
  closed forms     -> max-shift errors, sign errors in the exponent
  brute force      -> any chunk-boundary or empty-chunk slip in the merge
  layout checks    -> paged index, stride and bf16-decode mistakes
"""
import json
import math
import os

import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page2_counterexample.json")


def _scalar_problem(scores, values):
    """One head, D = 1, q = 1, scale = 1: key j's score is k_j itself."""
    n = len(scores)
    q = torch.ones((1, 1, 1), dtype=torch.float32)
    k = torch.tensor(scores, dtype=torch.float32).reshape(1, 1, n, 1)
    v = torch.tensor(values, dtype=torch.float32).reshape(1, 1, n, 1)
    return q, k, v, torch.tensor([n], dtype=torch.int32)


# --------------------------------------------------------------------------
# The worked counterexample of the www.2kiu.com/news/6053916 article.
# --------------------------------------------------------------------------

def test_page_counterexample_through_the_oracle():
    """The article's example -- scores [0, 0, 10], values [0, 0, 9], chunks
    2 | 1 -- through the oracle's plain and chunked forms: the chunk outputs
    and log-sum-exps the definitions fix, the merged result equal to the
    unsplit one (the page's 1e-12), both equal to the closed form
    9 / (1 + 2 e^-10), and the plain mean of the chunk outputs (4.5) off by
    more than 1."""
    g = json.load(open(GOLDEN))["what_the_page_fixes"]
    scores, values = g["scores"], g["values"]
    closed = 9.0 / (1.0 + 2.0 * math.exp(-10.0))
    q, k, v, lens = _scalar_problem(scores, values)
    out, lse = oracle.attention(q, k, v, lens, scale=1.0)
    assert math.isclose(out[0, 0].item(), closed, rel_tol=1e-14)
    assert math.isclose(lse[0].item(), 10.0 + math.log1p(2.0 * math.exp(-10.0)), rel_tol=1e-14)
    cuts = [0, g["chunks"][0][1], g["chunks"][1][1]]
    out_c, lse_c, po, pl = oracle.attention_chunked(q, k, v, lens, cuts, scale=1.0)
    assert po[0, :, 0].tolist() == g["chunk_outputs"]
    assert pl[0, 0].item() == pytest.approx(math.log(2), rel=1e-15)
    assert pl[0, 1].item() == 10.0
    assert math.isclose(out_c[0, 0].item(), out[0, 0].item(), rel_tol=g["merged_vs_global_rel_tol"])
    assert math.isclose(out_c[0, 0].item(), closed, rel_tol=1e-14)
    assert math.isclose(lse_c[0].item(), lse[0].item(), rel_tol=1e-14)
    naive = po[0, :, 0].mean().item()
    assert naive == g["naive_average"]
    assert abs(naive - out_c[0, 0].item()) > g["naive_average_min_abs_error"]


def test_oracle_refuses_what_the_page_refuses():
    """The article's example refuses a merge with no valid block: a row that
    sees no key is an error for the oracle too."""
    q, k, v, _ = _scalar_problem([1.0, 2.0], [3.0, 4.0])
    with pytest.raises(ValueError, match="empty"):
        oracle.attention(q, k, v, torch.tensor([0], dtype=torch.int32), scale=1.0)
    with pytest.raises(ValueError, match="empty"):
        oracle.attention_chunked(q, k, v, torch.tensor([0], dtype=torch.int32), [0, 1, 2], scale=1.0)


# --------------------------------------------------------------------------
# Library routines: SDPA in float64 and logsumexp.
# --------------------------------------------------------------------------

def _sdpa_rows(q, k, v, lens, scale):
    """torch SDPA (float64, CPU, GQA by repeat-interleave) per sequence."""
    outs, lses = [], []
    for b, L in enumerate(lens):
        qb = q[b:b + 1].double().unsqueeze(2)                    # [1][Hq][1][D]
        kb = k[b:b + 1, :, :L].double()
        vb = v[b:b + 1, :, :L].double()
        o = torch.nn.functional.scaled_dot_product_attention(qb, kb, vb, scale=scale, enable_gqa=True)
        outs.append(o[0, :, 0])
        g = q.shape[1] // k.shape[1]
        kr = kb[0].repeat_interleave(g, dim=0)                   # [Hq][L][D]
        logits = torch.matmul(kr, qb[0, :, 0].unsqueeze(-1)).squeeze(-1) * scale
        lses.append(torch.logsumexp(logits, dim=-1))
    return torch.cat(outs), torch.cat(lses)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("B,Hq,Hkv,D", [(2, 8, 2, 16), (3, 4, 4, 64), (1, 6, 1, 8)])
def test_matches_sdpa_float64(dtype, B, Hq, Hkv, D):
    lens = workloads.uniform_lengths(B, 1, 53, struct_seed=11 + D)
    x = workloads.contiguous("sdpa", B, Hq, Hkv, D, lens, dtype=dtype, cap=60, data_seed=5 + B,
                             struct_seed=6, scale=0.37)
    out, lse = oracle.attention(x.q, x.k, x.v, x.seq_lens, scale=x.scale)
    ref, ref_lse = _sdpa_rows(x.q, x.k, x.v, lens, x.scale)
    torch.testing.assert_close(out, ref, rtol=1e-12, atol=1e-13)
    torch.testing.assert_close(lse, ref_lse, rtol=1e-12, atol=1e-13)


def test_gqa_mapping_distinct_kv_heads():
    """Each KV head's values carry a distinct offset, so a wrong query-head to
    KV-head mapping moves the output by whole units."""
    x = workloads.contiguous("gqa", 1, 8, 4, 16, [40], dtype=torch.float32, data_seed=3, struct_seed=4)
    x.v += torch.arange(4, dtype=torch.float32).reshape(1, 4, 1, 1) * 10.0
    out, _ = oracle.attention(x.q, x.k, x.v, x.seq_lens, scale=x.scale)
    ref, _ = _sdpa_rows(x.q, x.k, x.v, [40], x.scale)
    torch.testing.assert_close(out, ref, rtol=1e-12, atol=1e-12)
    heads = (out.mean(dim=1) / 10.0).round()
    assert heads.tolist() == [0, 0, 1, 1, 2, 2, 3, 3]


# --------------------------------------------------------------------------
# Closed forms.
# --------------------------------------------------------------------------

def test_zero_query_gives_mean_and_log_length():
    x = workloads.contiguous("q0", 2, 2, 2, 8, [7, 13], dtype=torch.float32, data_seed=9, struct_seed=9)
    x.q.zero_()
    out, lse = oracle.attention(x.q, x.k, x.v, x.seq_lens, scale=x.scale)
    for b, L in enumerate([7, 13]):
        for h in range(2):
            mean = x.v[b, h, :L].double().mean(dim=0)
            torch.testing.assert_close(out[b * 2 + h], mean, rtol=1e-14, atol=1e-15)
            assert lse[b * 2 + h].item() == pytest.approx(math.log(L), rel=1e-15)


def test_single_key_and_two_keys():
    # One key: the output is that key's value and lse is its score.
    q = torch.tensor([[[1.0, 2.0]]])
    k = torch.tensor([[[[3.0, 4.0]]]])
    v = torch.tensor([[[[-1.5, 2.25]]]])
    out, lse = oracle.attention(q, k, v, torch.tensor([1]), scale=0.5)
    assert out[0].tolist() == [-1.5, 2.25]
    assert lse[0].item() == 5.5
    # Two keys with scores 1 and 4: the second weighs sigma(3).
    k2 = torch.tensor([[[[1.0], [4.0]]]])
    v2 = torch.tensor([[[[2.0], [-6.0]]]])
    out2, lse2 = oracle.attention(torch.ones((1, 1, 1)), k2, v2, torch.tensor([2]), scale=1.0)
    sig = 1.0 / (1.0 + math.exp(-3.0))
    assert out2[0, 0].item() == pytest.approx(2.0 + sig * (-8.0), rel=1e-15)
    assert lse2[0].item() == pytest.approx(4.0 + math.log1p(math.exp(-3.0)), rel=1e-15)


def test_shift_invariance_through_an_extra_dimension():
    """Appending a dimension with q = 1 and k = c/scale adds exactly c to every
    score: the output must not move and lse must grow by c."""
    x = workloads.contiguous("shift", 1, 2, 2, 8, [31], dtype=torch.float32, data_seed=21, struct_seed=21)
    out, lse = oracle.attention(x.q, x.k, x.v, x.seq_lens, scale=0.25)
    c = 37.5
    q2 = torch.cat([x.q, torch.ones((1, 2, 1))], dim=2).contiguous()
    k2 = torch.cat([x.k, torch.full((1, 2, 31, 1), c / 0.25)], dim=3).contiguous()
    v2 = torch.cat([x.v, torch.zeros((1, 2, 31, 1))], dim=3).contiguous()
    out2, lse2 = oracle.attention(q2, k2, v2, x.seq_lens, scale=0.25)
    torch.testing.assert_close(out2[:, :8], out, rtol=1e-13, atol=1e-14)
    torch.testing.assert_close(lse2, lse + c, rtol=1e-14, atol=1e-13)


def test_dominant_keys_bound():
    """Three keys raised by +30: the output sits within the tail bound of the
    softmax over those three keys alone."""
    x = workloads.c1_tiny_fp32("outliers")
    out, _ = oracle.attention(x.q, x.k, x.v, x.seq_lens, scale=x.scale)
    top = x.offset_keys[(0, 0)]
    s = torch.matmul(x.k[0, 0].double(), x.q[0, 0].double()) * x.scale
    rest = [j for j in range(1000) if j not in top]
    wt = torch.softmax(s[top], dim=0)
    out_top = (wt.unsqueeze(1) * x.v[0, 0, top].double()).sum(dim=0)
    ratio = torch.exp(s[rest] - s[top].max()).sum() / torch.exp(s[top] - s[top].max()).sum()
    bound = ratio.item() * 2 * x.v[0, 0].abs().max().item()
    assert bound < 1e-6
    assert (out[0] - out_top).abs().max().item() <= bound


# --------------------------------------------------------------------------
# Brute force: every partition of small key ranges merges to the same result.
# --------------------------------------------------------------------------

def _compositions(n):
    for mask in range(1 << (n - 1)):
        cuts = [0] + [i + 1 for i in range(n - 1) if mask >> i & 1] + [n]
        yield cuts


@pytest.mark.parametrize("L", [1, 2, 5, 9])
def test_every_partition_merges_to_the_full_result(L):
    x = workloads.contiguous("brute", 1, 2, 1, 8, [L], dtype=torch.float32, data_seed=100 + L, struct_seed=1)
    x.k[0, 0, L // 2] += 30.0 * x.q[0, 0] / (x.scale * torch.dot(x.q[0, 0], x.q[0, 0]))
    out, lse = oracle.attention(x.q, x.k, x.v, x.seq_lens, scale=x.scale)
    count = 0
    for cuts in _compositions(L):
        out_c, lse_c, _, pl = oracle.attention_chunked(x.q, x.k, x.v, x.seq_lens, cuts, scale=x.scale)
        torch.testing.assert_close(out_c, out, rtol=1e-12, atol=1e-13)
        torch.testing.assert_close(lse_c, lse, rtol=1e-12, atol=1e-13)
        assert torch.isfinite(pl).all()
        count += 1
    assert count == 2 ** (L - 1)


def test_empty_chunks_weigh_nothing():
    x = workloads.contiguous("empty", 2, 2, 2, 8, [5, 17], dtype=torch.float32, data_seed=8, struct_seed=8)
    out, lse = oracle.attention(x.q, x.k, x.v, x.seq_lens, scale=x.scale)
    cuts = oracle.equal_chunk_cuts(17, 4, 8)          # chunks past L_b are empty
    out_c, lse_c, po, pl = oracle.attention_chunked(x.q, x.k, x.v, x.seq_lens, cuts, scale=x.scale)
    torch.testing.assert_close(out_c, out, rtol=1e-12, atol=1e-13)
    torch.testing.assert_close(lse_c, lse, rtol=1e-12, atol=1e-13)
    # Sequence 0 (5 keys) fills chunks 0-1; chunks 2.. are empty.
    assert torch.isinf(pl[0:2, 2:]).all() and (pl[0:2, 2:] < 0).all()
    assert (po[0:2, 2:] == 0).all()
    assert torch.isfinite(pl[2:4, :5]).all() and torch.isinf(pl[2:4, 5:]).all()


# --------------------------------------------------------------------------
# Layouts and decoding.
# --------------------------------------------------------------------------

def test_nan_past_length_is_never_read():
    x = workloads.contiguous("mask", 2, 4, 2, 16, [9, 23], cap=32, dtype=torch.float32, data_seed=2,
                             struct_seed=2)
    assert torch.isnan(x.k[0, :, 9:]).all()
    out, lse = oracle.attention(x.q, x.k, x.v, x.seq_lens, scale=x.scale)
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    for b, L in enumerate([9, 23]):
        qb = x.q[b:b + 1].contiguous()
        kb = x.k[b:b + 1, :, :L].contiguous()
        vb = x.v[b:b + 1, :, :L].contiguous()
        o1, l1 = oracle.attention(qb, kb, vb, torch.tensor([L]), scale=x.scale)
        assert torch.equal(o1, out[b * 4:(b + 1) * 4]) and torch.equal(l1, lse[b * 4:(b + 1) * 4])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_paged_equals_contiguous(dtype):
    x = workloads.contiguous("pg", 3, 4, 2, 16, [40, 16, 33], dtype=dtype, data_seed=12, struct_seed=12)
    p = workloads.to_paged(x, page_size=16, struct_seed=5)
    assert p.block_table[0].tolist()[:3] != [0, 1, 2] or p.block_table[1].tolist()[:1] != [3]
    out, lse = oracle.attention(x.q, x.k, x.v, x.seq_lens, scale=x.scale)
    out_p, lse_p = oracle.attention(p.q, p.k, p.v, p.seq_lens, scale=p.scale, block_table=p.block_table,
                                    page_size=16)
    assert torch.equal(out, out_p) and torch.equal(lse, lse_p)


def test_strided_token_major_layout():
    """A [B][L][Hkv][D] cache seen through a permuted view gives the same result."""
    x = workloads.contiguous("str", 2, 4, 2, 8, [11, 6], dtype=torch.float32, data_seed=13, struct_seed=13)
    k_tm = x.k.permute(0, 2, 1, 3).contiguous()      # [B][L][Hkv][D] storage
    v_tm = x.v.permute(0, 2, 1, 3).contiguous()
    out, lse = oracle.attention(x.q, x.k, x.v, x.seq_lens, scale=x.scale)
    out2, lse2 = oracle.attention(x.q, k_tm.permute(0, 2, 1, 3), v_tm.permute(0, 2, 1, 3), x.seq_lens,
                                  scale=x.scale)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_bf16_decoding_matches_torch_conversion():
    x = workloads.contiguous("bf", 2, 4, 2, 32, [19, 7], dtype=torch.bfloat16, data_seed=14, struct_seed=14)
    out, lse = oracle.attention(x.q, x.k, x.v, x.seq_lens, scale=x.scale)
    out_f, lse_f = oracle.attention(x.q.float(), x.k.float(), x.v.float(), x.seq_lens, scale=x.scale)
    assert torch.equal(out, out_f) and torch.equal(lse, lse_f)


def test_selected_rows_match_full_run():
    x = workloads.contiguous("rows", 3, 4, 2, 8, [5, 9, 3], dtype=torch.float32, data_seed=15, struct_seed=15)
    out, lse = oracle.attention(x.q, x.k, x.v, x.seq_lens, scale=x.scale)
    rows = [(2, 3), (0, 1), (1, 0)]
    o2, l2 = oracle.attention(x.q, x.k, x.v, x.seq_lens, scale=x.scale, rows=rows)
    for i, (b, h) in enumerate(rows):
        assert torch.equal(o2[i], out[b * 4 + h]) and l2[i] == lse[b * 4 + h]


def test_refusals():
    x = workloads.contiguous("bad", 1, 4, 2, 8, [4], dtype=torch.float32, data_seed=1, struct_seed=1)
    with pytest.raises(ValueError, match="empty"):
        oracle.attention(x.q, x.k, x.v, torch.tensor([0]), scale=1.0)
    with pytest.raises(ValueError, match="invalid"):
        oracle.attention(x.q[:, :3].contiguous(), x.k, x.v, x.seq_lens, scale=1.0)
    with pytest.raises(ValueError):
        oracle.attention_chunked(x.q, x.k, x.v, x.seq_lens, [0, 2], scale=1.0)   # does not cover L


def test_workload_generators_are_deterministic():
    a = workloads.c1_tiny_fp32("tail")
    b = workloads.c1_tiny_fp32("tail")
    assert torch.equal(a.k, b.k) and torch.equal(a.v, b.v) and a.offset_keys == b.offset_keys
    keys = a.offset_keys[(0, 0)]
    assert len(keys) == 3 and max(keys) >= 768
    lens = workloads.uniform_lengths(128, 256, 2048, 2005)
    assert min(lens) >= 256 and max(lens) <= 2048
    assert lens == workloads.uniform_lengths(128, 256, 2048, 2005)


def test_large_scores_do_not_overflow():
    """AI Infra page, section 2.3: a logit of 1000 overflows exp unless the
    maximum is subtracted first. Scores -1000, 1000, 999 have the closed-form
    weights 0, 1/(1+e^-1), e^-1/(1+e^-1)."""
    q, k, v, lens = _scalar_problem([-1000.0, 1000.0, 999.0], [5.0, 1.0, -2.0])
    w1 = 1.0 / (1.0 + math.exp(-1.0))
    expect = w1 * 1.0 + (1.0 - w1) * -2.0
    out, lse = oracle.attention(q, k, v, lens, scale=1.0)
    assert out[0, 0].item() == pytest.approx(expect, rel=1e-14)
    assert lse[0].item() == pytest.approx(1000.0 + math.log1p(math.exp(-1.0)), rel=1e-15)
    for cuts in ([0, 1, 3], [0, 2, 3], [0, 1, 2, 3]):
        out_c, lse_c, _, _ = oracle.attention_chunked(q, k, v, lens, cuts, scale=1.0)
        assert out_c[0, 0].item() == pytest.approx(expect, rel=1e-14)
        assert lse_c[0].item() == pytest.approx(lse[0].item(), rel=1e-15)


def test_very_negative_scores_do_not_underflow():
    """Every score near -1000: exp of the raw chunk lse underflows to zero, so
    the merge has to shift by the largest chunk lse, not by a fixed value."""
    q, k, v, lens = _scalar_problem([-1000.0, -1001.0, -999.0], [3.0, -1.0, 0.5])
    w = [math.exp(-1.0), math.exp(-2.0), 1.0]
    expect = (w[0] * 3.0 + w[1] * -1.0 + w[2] * 0.5) / sum(w)
    for cuts in ([0, 3], [0, 1, 3], [0, 1, 2, 3]):
        out_c, lse_c, _, _ = oracle.attention_chunked(q, k, v, lens, cuts, scale=1.0)
        assert out_c[0, 0].item() == pytest.approx(expect, rel=1e-14)
        assert lse_c[0].item() == pytest.approx(-999.0 + math.log(sum(w)), rel=1e-15)


# --------------------------------------------------------------------------
# Multi-token decode: the last q_len positions under the causal rule of the
# AI Infra page, section 2.5 (the speculative-verification exception).
# --------------------------------------------------------------------------

def _sdpa_window(q, k, v, lens, scale):
    """torch SDPA in float64 with an explicit boolean mask that lets the query
    at position p see key j iff j <= p, for the positions L-T .. L-1."""
    B, T, Hq, D = q.shape
    g = Hq // k.shape[1]
    outs = []
    for b, L in enumerate(lens):
        qb = q[b].double().permute(1, 0, 2).unsqueeze(0)                       # [1][Hq][T][D]
        kb = k[b:b + 1, :, :L].double().repeat_interleave(g, dim=1)            # [1][Hq][L][D]
        vb = v[b:b + 1, :, :L].double().repeat_interleave(g, dim=1)
        pos = torch.arange(L - T, L).reshape(T, 1)
        mask = torch.arange(L).reshape(1, L) <= pos                            # [T][L]
        o = torch.nn.functional.scaled_dot_product_attention(qb, kb, vb, attn_mask=mask, scale=scale)
        outs.append(o[0].permute(1, 0, 2).reshape(T * Hq, D))                  # rows (t, h)
    return torch.cat(outs)


@pytest.mark.parametrize("T,B,Hq,Hkv", [(2, 2, 4, 2), (4, 3, 2, 1), (8, 1, 8, 8), (3, 2, 6, 2)])
def test_multi_token_matches_sdpa_with_window_mask(T, B, Hq, Hkv):
    lens = workloads.uniform_lengths(B, T, 40, struct_seed=31 + T)
    x = workloads.contiguous("mt", B, Hq, Hkv, 16, lens, dtype=torch.float32, cap=48, data_seed=30 + T,
                             struct_seed=31, q_len=T)
    out, lse = oracle.attention(x.q, x.k, x.v, x.seq_lens, scale=x.scale)
    ref = _sdpa_window(x.q, x.k, x.v, lens, x.scale)
    torch.testing.assert_close(out, ref, rtol=1e-12, atol=1e-13)
    # Row (b, t, h)'s lse over exactly the keys 0 .. L_b - T + t.
    for b, L in enumerate(lens):
        for t in range(T):
            for h in range(Hq):
                n = L - T + t + 1
                s = (x.k[b, h // (Hq // Hkv), :n].double() @ x.q[b, t, h].double()) * x.scale
                r = (b * T + t) * Hq + h
                assert lse[r].item() == pytest.approx(torch.logsumexp(s, 0).item(), rel=1e-13, abs=1e-13)


def test_multi_token_square_case_is_torch_causal():
    """With L_b == q_len the window is the whole sequence: torch's own causal
    flag (query i sees keys <= i) gives the same result."""
    T = 6
    x = workloads.contiguous("sq", 1, 2, 2, 8, [T], dtype=torch.float32, data_seed=41, struct_seed=41, q_len=T)
    out, _ = oracle.attention(x.q, x.k, x.v, x.seq_lens, scale=x.scale)
    qb = x.q[0].double().permute(1, 0, 2).unsqueeze(0)
    o = torch.nn.functional.scaled_dot_product_attention(qb, x.k[:, :, :T].double(), x.v[:, :, :T].double(),
                                                         is_causal=True, scale=x.scale)
    torch.testing.assert_close(out, o[0].permute(1, 0, 2).reshape(T * 2, 8), rtol=1e-12, atol=1e-13)
    # The first token sees one key: its output is that key's value, lse its score.
    torch.testing.assert_close(out[0], x.v[0, 0, 0].double(), rtol=0, atol=0)


def test_multi_token_one_token_is_plain_decode():
    x = workloads.contiguous("mt1", 2, 4, 2, 16, [9, 30], dtype=torch.bfloat16, data_seed=42, struct_seed=42)
    q4 = x.q.unsqueeze(1)                                   # [B][1][Hq][D]
    a = oracle.attention(x.q, x.k, x.v, x.seq_lens, scale=x.scale)
    b = oracle.attention(q4, x.k, x.v, x.seq_lens, scale=x.scale)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_multi_token_chunked_merges_to_plain_and_refuses_short_sequence():
    T = 4
    x = workloads.contiguous("mtc", 2, 4, 2, 8, [13, 7], dtype=torch.float32, data_seed=43, struct_seed=43, q_len=T)
    out, lse = oracle.attention(x.q, x.k, x.v, x.seq_lens, scale=x.scale)
    for cuts in ([0, 13], [0, 4, 8, 12, 16], [0, 10, 11, 12, 13]):
        out_c, lse_c, _, pl = oracle.attention_chunked(x.q, x.k, x.v, x.seq_lens, cuts, scale=x.scale)
        torch.testing.assert_close(out_c, out, rtol=1e-12, atol=1e-13)
        torch.testing.assert_close(lse_c, lse, rtol=1e-12, atol=1e-13)
    # Sequence 0 (13 keys), cut at 10, 11, 12: token 0 sees keys 0..9 only, so
    # its chunks [10, 11), [11, 12), [12, 13) are empty; token 3 sees all.
    _, _, _, pl = oracle.attention_chunked(x.q, x.k, x.v, x.seq_lens, [0, 10, 11, 12, 13], scale=x.scale)
    row = lambda b, t, h: (b * T + t) * 4 + h
    assert torch.isinf(pl[row(0, 0, 0), 1:]).all()
    assert torch.isfinite(pl[row(0, 1, 3), :2]).all() and torch.isinf(pl[row(0, 1, 3), 2:]).all()
    assert torch.isfinite(pl[row(0, 3, 0)]).all()
    with pytest.raises(ValueError, match="empty"):
        oracle.attention(x.q, x.k, x.v, torch.tensor([13, 3]), scale=x.scale)


# --------------------------------------------------------------------------
# fp8 (E4M3) KV cache with per-head scales: the "KV Quant" of the AI Infra
# page's closing summary.
# --------------------------------------------------------------------------

def test_e4m3_decoding_fixed_points():
    """Values fixed by the format: 1 sign, 4 exponent bits (bias 7), 3 mantissa
    bits, no infinities, S.1111.111 is NaN."""
    d = oracle.decode_e4m3
    assert d([0x38]).item() == 1.0                # exponent 7, mantissa 0
    assert d([0x7E]).item() == 448.0              # largest finite: 1.75 * 2^8
    assert d([0x08]).item() == 2.0 ** -6          # smallest normal
    assert d([0x01]).item() == 2.0 ** -9          # smallest subnormal
    assert d([0x07]).item() == 7 * 2.0 ** -9      # largest subnormal
    assert d([0x3C]).item() == 1.5
    assert d([0xB8]).item() == -1.0
    z = d([0x80]).item()
    assert z == 0.0 and math.copysign(1.0, z) < 0
    assert math.isnan(d([0x7F]).item()) and math.isnan(d([0xFF]).item())
    assert d([0x78]).item() == 256.0              # exponent 15 is finite in this format


def test_e4m3_decoding_matches_torch_for_every_code():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    mine = oracle.decode_e4m3(codes)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64)
    nan = torch.isnan(ref)
    assert nan.sum().item() == 2 and torch.equal(torch.isnan(mine), nan)
    assert torch.equal(mine[~nan], ref[~nan])


@pytest.mark.parametrize("paged", [False, True])
def test_fp8_attention_is_attention_of_the_dequantised_cache(paged):
    """fp8 K/V with per-head scales give the attention of the float64 cache
    decode(x) * scale[head] (torch's conversion), through SDPA."""
    lens = [21, 5, 34]
    x = workloads.contiguous("f8", 3, 4, 2, 16, lens, dtype=workloads.FP8, data_seed=44, struct_seed=44, cap=40)
    assert x.k.dtype == torch.float8_e4m3fn and x.q.dtype == torch.bfloat16
    assert not torch.equal(x.k_scale, x.v_scale) and x.k_scale[0] != x.k_scale[1]
    if paged:
        x = workloads.to_paged(x, page_size=16, struct_seed=3)
        out, lse = oracle.attention(x.q, x.k, x.v, x.seq_lens, scale=x.scale, block_table=x.block_table,
                                    page_size=16, k_scale=x.k_scale, v_scale=x.v_scale)
        x = workloads.contiguous("f8", 3, 4, 2, 16, lens, dtype=workloads.FP8, data_seed=44, struct_seed=44,
                                 cap=40)
    else:
        out, lse = oracle.attention(x.q, x.k, x.v, x.seq_lens, scale=x.scale, k_scale=x.k_scale,
                                    v_scale=x.v_scale)
    kd = x.k.to(torch.float64) * x.k_scale.double().reshape(1, -1, 1, 1)
    vd = x.v.to(torch.float64) * x.v_scale.double().reshape(1, -1, 1, 1)
    ref, ref_lse = _sdpa_rows(x.q, kd, vd, lens, x.scale)
    torch.testing.assert_close(out, ref, rtol=1e-12, atol=1e-13)
    torch.testing.assert_close(lse, ref_lse, rtol=1e-12, atol=1e-13)


def test_fp8_scales_enter_scores_and_values_separately():
    """Doubling k_scale doubles every score; doubling v_scale doubles the output."""
    x = workloads.contiguous("f8s", 1, 2, 1, 8, [12], dtype=workloads.FP8, data_seed=45, struct_seed=45)
    ks, vs = x.k_scale.clone(), x.v_scale.clone()
    out, lse = oracle.attention(x.q, x.k, x.v, x.seq_lens, scale=x.scale, k_scale=ks, v_scale=vs)
    out2, _ = oracle.attention(x.q, x.k, x.v, x.seq_lens, scale=x.scale, k_scale=ks, v_scale=2 * vs)
    torch.testing.assert_close(out2, 2 * out, rtol=1e-14, atol=0)
    out3, lse3 = oracle.attention(x.q, x.k, x.v, x.seq_lens, scale=2 * x.scale, k_scale=ks, v_scale=vs)
    out4, lse4 = oracle.attention(x.q, x.k, x.v, x.seq_lens, scale=x.scale, k_scale=2 * ks, v_scale=vs)
    torch.testing.assert_close(out4, out3, rtol=1e-14, atol=1e-15)
    torch.testing.assert_close(lse4, lse3, rtol=1e-14, atol=1e-15)
    assert not torch.allclose(out3, out)


def test_fp8_workload_layout():
    x = workloads.contiguous("f8l", 2, 2, 2, 16, [3, 9], dtype=workloads.FP8, data_seed=46, struct_seed=46)
    raw = x.k.view(torch.uint8)
    assert (raw[0, :, 3:] == workloads.FP8_NAN_CODE).all() and (raw[1, :, 9:] == 0x7F).sum() == 0
    deq = x.k[1].to(torch.float32) * x.k_scale.reshape(-1, 1, 1)
    sig, _ = workloads.fp8_head_sigmas(2, 46)
    # The per-head spread survives quantisation (within sampling error of 9 * 16 draws).
    ratio = deq.std(dim=(1, 2)) / sig
    assert ((ratio > 0.75) & (ratio < 1.3)).all()
