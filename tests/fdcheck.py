"""Shared helpers of the GPU tests: run the library through its C ABI, run the
oracle on host copies of the same bytes, and compare them to the stated
tolerances.

Tolerances (written here once, used by every parity test):
  fp32 path (fp32 q/K/V/out):   per output row (b, t, h),
                                max|gpu - ref| / max|ref| <= 1e-5
  bf16 output:                  element-wise |gpu - ref| <= 2e-3 + 1e-2 |ref|
  LSE:                          |gpu - ref| <= LSE_TOL[dtype] * max(1, |ref|)
The LSE bounds come from fp32 arithmetic on exact inputs: the score q.k of
D = 128 terms carries a relative rounding error of a few 1e-7 and the
exponent sum another few 1e-7, so 1e-5 (fp32) and 2e-5 (bf16 inputs, whose
products are exact in fp32) leave a wide margin. fp8 caches take the bf16
bounds: their bytes become bf16 exactly, and the per-head scales add one
fp32 rounding to the score multiplier and one to the output.

Rows are output rows in (b, t, h) order, t < q_len; the oracle's row ids are
(b, i) with i = t * Hq + h.
"""
from __future__ import annotations

import bisect
import math

import torch

import decode_attention_12_amd as fd
import oracle

FP32_ROW_TOL = 1e-5
BF16_ATOL, BF16_RTOL = 2e-3, 1e-2
LSE_TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-5, torch.float8_e4m3fn: 2e-5}


def _override(plan, workers, lead):
    """Worker count and leading-worker share of a balanced plan, as a test
    asks."""
    if workers is not None:
        plan.workers = workers
        plan.lead_workers = workers // 2 if plan.lead_pct else 0
    if lead is not None:
        plan.lead_workers, plan.lead_pct = lead


def partition(plan, T):
    """Tile range [first, first + size) of every balanced worker, from the
    formula fd.h states: the first lead_workers workers take q1 tiles, the
    others q2, q2 = ceil(100 T / (lead_workers lead_pct + (W - lead_workers)
    100)), q1 = ceil(q2 lead_pct / 100); q1 = q2 = ceil(T / W) when lead_pct
    is 0."""
    W = plan.workers
    pct = plan.lead_pct or 100
    w1 = min(plan.lead_workers, W) if plan.lead_pct else 0
    q2 = max(1, -(-100 * T // (w1 * pct + (W - w1) * 100)))
    q1 = max(1, -(-q2 * pct // 100))
    firsts = [w * q1 if w < w1 else w1 * q1 + (w - w1) * q2 for w in range(W)]
    sizes = [q1 if w < w1 else q2 for w in range(W)]
    return firsts, sizes


def run(x, *, splits=None, path=None, out_dtype=None, lse=True, workspace=None, num_cus=0, workers=None,
        host_lens=True, lead=None):
    """One decode step of workload x through the library. Returns (out, lse, plan, workspace).
    workers overrides the worker count of a balanced plan, lead its
    (lead_workers, lead_pct); host_lens=False leaves the host-side length
    check out (so L_b = 0 reaches the device)."""
    out_dtype = out_dtype or x.out_dtype
    problem = fd.problem_of(x.q, x.k, x.max_seq_len, out_dtype=out_dtype, page_size=x.page_size,
                            num_pages=x.num_pages)
    plan = fd.fd_plan_splits(problem, num_cus, x.num_splits if splits is None else splits)
    if path is not None:
        plan.path = path
    _override(plan, workers, lead)
    need = fd.fd_workspace_size(problem, plan)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.q.device)
    out = torch.empty(x.q.shape, dtype=out_dtype, device=x.q.device)
    lse_t = torch.empty(x.q.shape[:-1], dtype=torch.float32, device=x.q.device) if lse else None
    fd.fd_decode_partial(problem, plan, x.q, x.k, x.v, kv_layout(x), x.seq_lens, workspace, scale=x.scale,
                         block_table=x.block_table, seq_lens_host=x.seq_lens_host if host_lens else None)
    fd.fd_decode_combine(problem, plan, workspace, out, lse_t)
    torch.cuda.synchronize()
    return out, lse_t, plan, workspace


def kv_layout(x):
    return fd.layout_of(x.k, x.k_scale, x.v_scale)


def _align(n):
    return -(-n // 256) * 256


def rows_per_seg(x, plan):
    """Query rows per segment, as the header states: of the q_len * g rows
    of a KV head, MFMA takes the largest divisor <= 16, the VALU kernel 4, 2
    or 1 (2 or 1 for an fp8 cache)."""
    n = x.q_len * (x.num_q_heads // x.num_kv_heads)
    if plan.path == fd.FD_PATH_MFMA:
        return max(r for r in range(1, 17) if n % r == 0)
    if x.k.dtype != torch.float8_e4m3fn and n % 4 == 0:
        return 4
    return 2 if n % 2 == 0 else 1


def num_rows(x):
    return x.batch * x.q_len * x.num_q_heads


def row_ids(x):
    """(b, t, h) of every output row, in order."""
    return [(b, t, h) for b in range(x.batch) for t in range(x.q_len) for h in range(x.num_q_heads)]


def row_records(x, plan, workspace):
    """Every output row's piece records, read from the workspace as the header
    lays it out: a list of (o [n][D], lse [n], key ranges [(lo, hi)] * n),
    the ranges before the row's own window is applied.

    Split mode: split s covers [s C, min((s+1) C, L_b)).
    Balanced mode: segment j of sequence b (KV head x row tile) has
    T_b = ceil(L_b / tile) tiles; segments are laid end to end in (b, j)
    order; worker p runs the tiles in its range of the partition (see
    partition); the piece of segment s run by worker p sits in slot s + p.

    Both modes: the counts section (int32 [B * J]) comes first, then the
    records' outputs and LSEs."""
    B, D = x.batch, x.head_dim
    Hq = x.num_q_heads
    lens = [min(max(int(L), 0), x.max_seq_len) for L in x.seq_lens_host]
    ws = workspace.cpu()
    out = []
    rows = num_rows(x)
    base = _align(B * segments_per_seq(x, plan) * 4)
    if plan.mode == fd.FD_MODE_SPLITS:
        S, C = plan.num_splits, plan.chunk_len
        n = rows * S
        o = ws[base:base + n * D * 4].view(torch.float32).reshape(rows, S, D)
        off = base + _align(n * D * 4)
        lse = ws[off:off + n * 4].view(torch.float32).reshape(rows, S)
        for r, (b, t, h) in enumerate(row_ids(x)):
            rng = [(s * C, max(s * C, min((s + 1) * C, lens[b]))) for s in range(S)]
            out.append((o[r], lse[r], rng))
        return out
    g = Hq // x.num_kv_heads
    hps = rows_per_seg(x, plan)
    tiles_h = x.q_len * g // hps
    J = x.num_kv_heads * tiles_h
    tile = plan.tile
    tb = [-(-L // tile) for L in lens]
    pre = [0]
    for t in tb:
        pre.append(pre[-1] + t)
    T = J * pre[-1]
    firsts, sizes = partition(plan, T)
    owner = lambda t: bisect.bisect_right(firsts, t) - 1
    slots = B * J + plan.workers - 1
    o = ws[base:base + slots * hps * D * 4].view(torch.float32).reshape(slots, hps, D)
    off = base + _align(slots * hps * D * 4)
    lse = ws[off:off + slots * hps * 4].view(torch.float32).reshape(slots, hps)
    poff = off + _align(slots * hps * 4)
    prefix = ws[poff:poff + (B + 1) * 4].view(torch.int32).tolist()
    assert prefix == pre, f"tile prefix table {prefix} != {pre}"
    for b, t, h in row_ids(x):
            kvh, hl = divmod(h, g)
            ti, hs = divmod(t * g + hl, hps)
            j = kvh * tiles_h + ti
            s = b * J + j
            if tb[b] == 0:
                out.append((o[:0, hs], lse[:0, hs], []))
                continue
            first = J * pre[b] + j * tb[b]   # the segment's first tile
            p0, p1 = owner(first), owner(first + tb[b] - 1)
            rng = []
            for p in range(p0, p1 + 1):
                t0 = max(first, firsts[p]) - first
                t1 = min(first + tb[b], firsts[p] + sizes[p]) - first
                rng.append((t0 * tile, min(lens[b], t1 * tile)))
            out.append((o[s + p0:s + p1 + 1, hs], lse[s + p0:s + p1 + 1, hs], rng))
    return out


def host(x):
    """Host copies of the inputs (same bytes the GPU reads)."""
    bt = x.block_table.cpu() if x.block_table is not None else None
    return x.q.cpu(), x.k.cpu(), x.v.cpu(), x.seq_lens.cpu(), bt


def _scales(x):
    if x.k_scale is None:
        return {}
    return {"k_scale": x.k_scale.cpu(), "v_scale": x.v_scale.cpu()}


def oracle_rows(x, rows):
    """Oracle row ids (b, i = t * Hq + h) of (b, t, h) triples."""
    return [(b, t * x.num_q_heads + h) for b, t, h in rows]


def reference(x, rows=None, hx=None):
    """Oracle outputs of the given (b, t, h) rows (default: all, in order)."""
    q, k, v, lens, bt = hx or host(x)
    return oracle.attention(q, k, v, lens, scale=x.scale, block_table=bt, page_size=x.page_size,
                            rows=None if rows is None else oracle_rows(x, rows), **_scales(x))


def reference_chunked(x, plan, hx=None):
    q, k, v, lens, bt = hx or host(x)
    cuts = [i * plan.chunk_len for i in range(plan.num_splits + 1)]
    return oracle.attention_chunked(q, k, v, lens, cuts, scale=x.scale, block_table=bt, page_size=x.page_size,
                                    **_scales(x))


def row_rel_err(got, ref):
    """Per-row max-norm relative error of [rows][D] tensors (float64)."""
    got = got.double().reshape(ref.shape)
    return ((got - ref).abs().amax(dim=-1) / ref.abs().amax(dim=-1).clamp_min(1e-300))


def assert_out_close(got, ref, out_dtype):
    got = got.double().cpu().reshape(ref.shape)
    assert torch.isfinite(got).all(), "non-finite output"
    if out_dtype == torch.float32:
        err = row_rel_err(got, ref).max().item()
        assert err <= FP32_ROW_TOL, f"max row relative error {err:.3e} > {FP32_ROW_TOL}"
        return err
    bad = (got - ref).abs() > BF16_ATOL + BF16_RTOL * ref.abs()
    if bad.any():
        i = bad.nonzero()[0].tolist()
        raise AssertionError(f"{int(bad.sum())} bf16 outputs out of tolerance, first at {i}: "
                             f"gpu {got[tuple(i)].item()} ref {ref[tuple(i)].item()}")
    return ((got - ref).abs() / (BF16_ATOL + BF16_RTOL * ref.abs())).max().item()


def assert_lse_close(got, ref, kv_dtype):
    got = got.double().cpu().reshape(ref.shape)
    tol = LSE_TOL[kv_dtype] * ref.abs().clamp_min(1.0)
    err = (got - ref).abs()
    assert torch.isfinite(got).all(), "non-finite lse"
    assert (err <= tol).all(), f"lse error {err.max().item():.3e} over tolerance"
    return (err / tol).max().item()


def assert_records_close(x, plan, workspace, hx=None):
    """Every chunk record of fd_decode_partial against the oracle's chunk
    partials for the same key ranges (fp32 bound on both halves; bf16 inputs
    with P rounded to bf16 on the MFMA path: 4e-3 on the outputs)."""
    q, k, v, lens, bt = hx or host(x)
    recs = row_records(x, plan, workspace)
    tol = FP32_ROW_TOL if x.k.dtype == torch.float32 else 4e-3
    ids = row_ids(x)
    for r, (o, lse, rng) in enumerate(recs):
        if not rng:
            continue
        b, t, h = ids[r]
        cuts = [rng[0][0]] + [hi for _, hi in rng]
        lead = [0] if cuts[0] > 0 else []
        _, _, po, pl = oracle.attention_chunked(q, k, v, lens, lead + cuts if lead else cuts, scale=x.scale,
                                                block_table=bt, page_size=x.page_size,
                                                rows=oracle_rows(x, [(b, t, h)]), **_scales(x))
        po, pl = po[0, len(lead):], pl[0, len(lead):]
        assert pl.shape[0] == len(rng)
        empty = torch.isinf(pl)
        assert torch.equal(torch.isinf(lse), empty), f"row {r}: empty-piece pattern differs"
        assert (lse[empty] < 0).all() and (o[empty] == 0).all(), "empty pieces must be (0, -inf)"
        full = ~empty
        if full.any():
            rel = row_rel_err(o[full], po[full])
            assert rel.max().item() <= tol, f"row {r}: piece output error {rel.max().item():.3e}"
            lerr = (lse[full].double() - pl[full]).abs() / pl[full].abs().clamp_min(1.0)
            assert lerr.max().item() <= LSE_TOL[x.k.dtype], f"row {r}: piece lse error {lerr.max().item():.3e}"


def weight_sums(x, plan, workspace):
    """sum_s exp(LSE_s - max LSE) per row, from the workspace records."""
    sums = []
    for o, lse, rng in row_records(x, plan, workspace):
        if lse.numel() == 0:
            sums.append(0.0)
            continue
        m = lse.max().double()
        sums.append(torch.exp(lse.double() - m).sum().item())
    return torch.tensor(sums, dtype=torch.float64)


def sample_rows(x, n, seed):
    """n distinct (b, t, h) rows, drawn with a seeded generator."""
    g = torch.Generator().manual_seed(seed)
    ids = row_ids(x)
    idx = torch.randperm(len(ids), generator=g)[:n].tolist()
    return sorted(ids[i] for i in idx)


def isclose_scalar(a, b, rel):
    return math.isclose(a, b, rel_tol=rel)


def segments_per_seq(x, plan):
    """J: KV heads x row tiles per KV head."""
    g = x.num_q_heads // x.num_kv_heads
    return x.num_kv_heads * (x.q_len * g // rows_per_seg(x, plan))


def counters(x, plan, workspace):
    """The workspace's per-segment piece counters (fd_decode only): the
    first B * J int32 of the workspace in every mode."""
    n = x.batch * segments_per_seq(x, plan)
    return workspace[:n * 4].view(torch.int32).cpu()


def run_fused(x, *, splits=None, out_dtype=None, workspace=None, workers=None, host_lens=True, lse=True,
              lead=None):
    """One decode step through fd_decode (single launch). Returns (out, lse, plan, workspace)."""
    out_dtype = out_dtype or x.out_dtype
    problem = fd.problem_of(x.q, x.k, x.max_seq_len, out_dtype=out_dtype, page_size=x.page_size,
                            num_pages=x.num_pages)
    plan = fd.fd_plan_splits(problem, 0, x.num_splits if splits is None else splits)
    _override(plan, workers, lead)
    if workspace is None:
        workspace = torch.zeros(fd.fd_workspace_size(problem, plan), dtype=torch.uint8, device=x.q.device)
    out = torch.empty(x.q.shape, dtype=out_dtype, device=x.q.device)
    lse_t = torch.empty(x.q.shape[:-1], dtype=torch.float32, device=x.q.device) if lse else None
    fd.fd_decode(problem, plan, x.q, x.k, x.v, kv_layout(x), x.seq_lens, workspace, out, lse_t, scale=x.scale,
                 block_table=x.block_table, seq_lens_host=x.seq_lens_host if host_lens else None)
    torch.cuda.synchronize()
    return out, lse_t, plan, workspace


def check_fused_steps(steps, *, splits=None, workers=None, lead=None, host_lens=True, out_dtype=None):
    """fd_decode over one workspace for each workload of `steps` in turn (the
    same shapes and plan, fresh values and lengths every step). Each step's
    outputs are checked against the oracle on that step's own inputs, rows
    that see no key must come out as 0 / -inf, and the piece counters must be
    back at zero after every call. Because the inputs change from step to
    step, a record left over from an earlier step -- or one read before its
    writer's stores were visible -- gives a wrong output here. Returns the
    number of steps run."""
    ws = None
    plan0 = None
    n = 0
    for x in steps:
        lens = [min(max(int(L), 0), x.max_seq_len) for L in x.seq_lens_host]
        rows = row_ids(x)
        live = [(b, t, h) for b, t, h in rows if lens[b] - x.q_len + 1 + t > 0]
        dead = [(b, t, h) for b, t, h in rows if lens[b] - x.q_len + 1 + t <= 0]
        ref, ref_lse = reference(x, rows=live)
        out, lse, plan, ws = run_fused(x, splits=splits, workers=workers, lead=lead, host_lens=host_lens,
                                       workspace=ws, out_dtype=out_dtype)
        if plan0 is None:
            plan0 = plan
        assert bytes(plan) == bytes(plan0), "every step must run the same plan on the same workspace"
        assert (counters(x, plan, ws) == 0).all(), "piece counters must be back at zero"
        o = out.float().cpu().reshape(x.batch, x.q_len, x.num_q_heads, x.head_dim)
        l = lse.cpu().reshape(x.batch, x.q_len, x.num_q_heads)
        if live:
            bs, ts, hs = (list(c) for c in zip(*live))
            assert_out_close(o[bs, ts, hs], ref, out_dtype or x.out_dtype)
            assert_lse_close(l[bs, ts, hs], ref_lse, x.k.dtype)
        if dead:
            bs, ts, hs = (list(c) for c in zip(*dead))
            assert (o[bs, ts, hs] == 0).all() and torch.isinf(l[bs, ts, hs]).all() and (l[bs, ts, hs] < 0).all()
        n += 1
    return n
