"""Cooperative splits: a host plan with at most half as many work items as CUs runs each
split on several workgroups, every one over a run of whole 64-token steps of the split,
and folds their partial states into the split's partial. Checked against the same split
plan with one workgroup per split (num_cus 1 fills every grid): the split partials (the
integer maxima m exactly, l, l~ and O to fp32 rounding), the fp32 outputs to 1e-5, and
the outputs against the oracle."""
import sys

import numpy as np
import pytest
import torch

import oracle
from decode_attention_gather_amd import inputs

pytestmark = pytest.mark.gpu

F32 = np.float32


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mla():
    from decode_attention_gather_amd import mla as m
    return m


def _partials(mla, plan, dc, kvb, q_lens):
    ws = plan.alloc_workspace()
    ws.zero_()
    mla.partial_ex(plan, dc.q, dc.kv, dc.block_table, dc.kv_lens, dc.softmax_scale, ws,
                   q_lens=q_lens, kv_bounds=kvb)
    info = plan.info()[0]
    rows = info.rows_per_request
    n = info.total_splits * rows
    o_bytes = (n * 512 * 4 + 255) // 256 * 256
    raw = ws.cpu().numpy()
    O = raw[:n * 2048].view(np.float32).reshape(n, 512)
    st = raw[o_bytes:o_bytes + n * 16].view(np.float32).reshape(n, 4)
    return O, st, ws


CASES = [
    # lens, heads, q_len, split_kv, kv dtype, key windows, ragged q_lens
    ([131072, 100, 33], 12, 1, 2, "e4m3", False, False),  # short requests: empty runs
    ([20000, 3000], 16, 2, 1, "e4m3", False, False),       # narrow kernel, two row tiles
    ([20000, 3000, 777], 12, 8, 1, "e4m3", False, False),  # wide kernel, causal rows
    ([9000, 20000], 12, 8, 2, "e4m3", False, True),        # wide kernel, ragged queries
    ([70000], 96, 8, 2, "e4m3", False, False),             # wide kernel, 12 row blocks
    ([20000, 5000], 12, 1, 2, "e4m3", True, False),        # key windows
    ([20000, 3000], 12, 1, 1, "bf16", False, False),       # BF16 narrow kernel
    ([20000, 3000], 12, 8, 1, "bf16", False, False),       # BF16 wide kernel
]


@pytest.mark.parametrize("lens,heads,q_len,split,dt,bounded,ragged", CASES)
def test_cooperative_splits(mla, lens, heads, q_len, split, dt, bounded, ragged):
    case = inputs.make_case(lens, num_heads=heads, q_len=q_len, seed=51, split_kv=split,
                            kv_dtype=dt)
    dc = mla.to_device(case)
    kvb = q_lens = None
    kb_host = None
    if bounded:
        kb_host = np.array([[min(1000, n // 3), n - 7] for n in lens], dtype=np.int32)
        kvb = torch.from_numpy(kb_host).cuda()
    if ragged:
        q_lens = torch.tensor([q_len - 3, q_len], dtype=torch.int32, device="cuda")
    coop = mla.Plan(dc.kv_lens_host, q_len=q_len, num_heads=heads, split_kv=split,
                    num_cus=256, kv_dtype=dt)
    whole = mla.Plan(dc.kv_lens_host, q_len=q_len, num_heads=heads, split_kv=split,
                     num_cus=1, kv_dtype=dt)
    subs = coop.info()[0].split_workgroups
    _say(f"[gpu] cooperative splits lens={lens} H={heads} q={q_len} split={split} {dt} "
         f"bounded={bounded} ragged={ragged}: {subs} workgroups per split")
    assert subs > 1
    assert whole.info()[0].split_workgroups == 1
    assert coop.info()[0].total_splits == whole.info()[0].total_splits

    Oa, sa, wa = _partials(mla, coop, dc, kvb, q_lens)
    Ob, sb, _ = _partials(mla, whole, dc, kvb, q_lens)
    torch.cuda.synchronize()
    assert np.array_equal(sa[:, 0], sb[:, 0]), "split maxima m differ"
    live = np.isfinite(sb[:, 0])
    for name, x, y in (("l", sa[:, 1], sb[:, 1]), ("l~", sa[:, 2], sb[:, 2])):
        rel = np.abs(x - y) / np.maximum(np.abs(y), 1e-30)
        assert float(rel[live].max(initial=0.0)) <= 1e-5, (name, float(rel[live].max()))
        assert np.all(x[~live] == 0) and np.all(y[~live] == 0), name
    scale = np.maximum(np.abs(Ob).max(axis=1, keepdims=True), 1e-30)
    assert float((np.abs(Oa - Ob) / scale).max()) <= 1e-5

    # fp32 outputs of both plans, and the cooperative plan's against the oracle
    rows = len(lens) * q_len * heads
    outs = []
    for plan, ws in ((coop, wa), (whole, None)):
        if ws is None:
            ws = plan.alloc_workspace()
            mla.partial_ex(plan, dc.q, dc.kv, dc.block_table, dc.kv_lens, dc.softmax_scale, ws,
                           q_lens=q_lens, kv_bounds=kvb)
        o = torch.empty((rows, 512), dtype=torch.float32, device="cuda")
        lse = torch.empty((rows,), dtype=torch.float32, device="cuda")
        mla.merge(plan, ws, dc.output_scale, o, lse)
        torch.cuda.synchronize()
        outs.append((o.cpu().numpy(), lse.cpu().numpy()))
    (oa, la), (ob, lb) = outs
    fin = np.isfinite(lb)
    assert np.array_equal(np.isfinite(la), fin)
    d = float(np.abs(oa[fin] - ob[fin]).max(initial=0.0))
    dl = float(np.abs(la[fin] - lb[fin]).max(initial=0.0))
    _say(f"  coop vs whole: max |dO| = {d:.3e}, max |dLSE| = {dl:.3e}")
    assert d <= 1e-5
    assert dl <= 1e-5 * max(1.0, float(np.abs(lb[fin]).max(initial=0.0)))

    if ragged:  # rows past a request's query count: nothing (their parity: test_gpu_varq)
        for b, qb in enumerate(q_lens.cpu().tolist()):
            dead = slice((b * q_len + qb) * heads, (b + 1) * q_len * heads)
            assert (oa[dead] == 0).all() and np.isneginf(la[dead]).all()
        return
    # oracle on sampled rows (every request, first and last query, a few heads)
    sample = sorted({(b * q_len + j) * heads + h for b in range(len(lens))
                     for j in (0, q_len - 1) for h in (0, heads // 2, heads - 1)})
    o_ref, lse_ref = oracle.mla_decode(
        case.q, case.kv, case.block_table, case.kv_lens, q_len=q_len, num_heads=heads,
        softmax_scale=F32(case.softmax_scale), output_scale=F32(case.output_scale),
        rows=sample, kv_dtype=dt, kv_bounds=kb_host)
    for i, r in enumerate(sample):
        if not np.isfinite(lse_ref[i]):
            assert not np.isfinite(la[r])
            continue
        err = np.abs(oa[r] - o_ref[i])
        assert (err <= 1e-2 + 1e-2 * np.abs(o_ref[i])).all(), (r, float(err.max()))
        assert abs(la[r] - lse_ref[i]) <= 1e-4 * max(1.0, abs(lse_ref[i])), r


def test_cooperative_splits_in_a_hip_graph(mla):
    """A host plan with shared splits enqueues three kernels (partial, fold, merge) and no
    memset, so a captured call replays: every replay, with the cache changed in between,
    equals the eager call on the same inputs."""
    case = inputs.make_case([20000, 3000], num_heads=12, q_len=1, seed=53, split_kv=2)
    dc = mla.to_device(case)
    plan = mla.Plan(dc.kv_lens_host, q_len=1, num_heads=12, split_kv=2, num_cus=256)
    assert plan.info()[0].split_workgroups > 1
    ws = plan.alloc_workspace()
    rows = 2 * 12
    o = torch.empty((rows, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((rows,), dtype=torch.float32, device="cuda")
    mla.decode(plan, dc.q, dc.kv, dc.block_table, dc.kv_lens, dc.softmax_scale,
               dc.output_scale, ws, o, lse)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        mla.decode(plan, dc.q, dc.kv, dc.block_table, dc.kv_lens, dc.softmax_scale,
                   dc.output_scale, ws, o, lse, stream=s)
    torch.cuda.synchronize()
    q0 = dc.q.clone()
    gen = torch.Generator(device="cpu").manual_seed(7)
    for i in range(4):
        _say(f"[gpu] shared splits in a HIP graph: replay {i}")
        if i:  # new queries (the heads' rows permuted) between replays
            perm = torch.randperm(12, generator=gen).to("cuda")
            dc.q.copy_(q0.view(2, 1, 12, -1)[:, :, perm].reshape(q0.shape))
            torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_g, lse_g = o.clone(), lse.clone()
        o_e = torch.empty_like(o)
        lse_e = torch.empty_like(lse)
        mla.decode(plan, dc.q, dc.kv, dc.block_table, dc.kv_lens, dc.softmax_scale,
                   dc.output_scale, plan.alloc_workspace(), o_e, lse_e)
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e) and torch.equal(lse_g, lse_e), f"replay {i}"
