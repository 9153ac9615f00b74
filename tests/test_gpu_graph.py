"""The graph path (device planner + partial + merge with device lengths and scales).

Checks, through the C ABI:
  * parity with the fp64 oracle (same bar as tests/test_gpu_parity.py) for skewed
    batches, q = 8 and 96-head shapes, and device lengths below the plan's bound;
  * the device planner reproduces the host planner: for the same lengths the graph path
    and the host-planned path give bitwise identical outputs (same splits, same kernels);
  * a request of length 0 yields O = 0 and LSE = -inf;
  * capture in a HIP graph: one captured call replayed several times while the device
    lengths and scales change between replays (eager copies and synchronisations in
    between), every replay equal to the eager call on the same inputs.
"""
import numpy as np
import pytest
import torch

from decode_attention_gather_amd import inputs
from test_gpu_parity import F32, _say, assert_parity, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    from decode_attention_gather_amd import mla as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def graph_call(mla, plan, dc, lens_dev, ss, os_, ws):
    rows = len(dc.kv_lens_host) * dc.q_len * dc.num_heads
    o = torch.empty((rows, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((rows,), dtype=torch.float32, device="cuda")
    mla.decode_graph(plan, dc.q, dc.kv, dc.block_table, lens_dev, ss, os_, ws, o, lse)
    return o, lse


def scal(x):
    return torch.tensor([x], dtype=torch.float32, device="cuda")


GRAPH_CASES = [
    # name, kv_lens (plan bound = max), device lengths, heads, q_len, split_kv
    ("skewed_q1", [40000, 100, 5000, 33], None, 12, 1, 0),
    ("shorter_on_device", [3000, 3000, 3000], [2999, 64, 1], 12, 1, 0),
    ("q8_uniform", [3000, 777], None, 12, 8, 4),
    ("q8_planner", [4096, 700, 65], None, 12, 8, 0),
    ("h96_q1", [2000, 300], None, 96, 1, 0),
    ("q2_h16", [1500, 40, 2], None, 16, 2, 0),
    ("shared_uniform", [40000, 30000], None, 12, 1, 2),         # 8 workgroups per split
    ("shared_shorter", [40000, 40000], [39000, 5000], 12, 1, 2),
    ("shared_q8", [20000, 9000], None, 12, 8, 1),
]


@pytest.mark.parametrize("name,lens,dev_lens,heads,q_len,split", GRAPH_CASES,
                         ids=[c[0] for c in GRAPH_CASES])
def test_graph_parity_and_host_equivalence(mla, name, lens, dev_lens, heads, q_len, split):
    case = inputs.make_case(lens, num_heads=heads, q_len=q_len, seed=777, split_kv=split)
    dc = mla.to_device(case)
    max_len = max(lens)
    plan = mla.Plan.graph(len(lens), q_len=q_len, num_heads=heads, max_kv_len=max_len,
                          split_kv=split)
    ws = plan.alloc_workspace()
    lens_now = dev_lens or lens
    lens_dev = torch.tensor(lens_now, dtype=torch.int32, device="cuda")
    _say(f"[gpu] graph {name}: lens={lens_now} H={heads} q={q_len} split={split}")
    o, lse = graph_call(mla, plan, dc, lens_dev, scal(case.softmax_scale), scal(case.output_scale),
                        ws)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    # the oracle on the device lengths (same cache and block table)
    ref_case = inputs.Case(q=case.q, kv=case.kv, block_table=case.block_table,
                           kv_lens=torch.tensor(lens_now, dtype=torch.int32), q_len=q_len,
                           num_heads=heads, softmax_scale=case.softmax_scale,
                           output_scale=case.output_scale)
    o_ref, lse_ref = run_oracle(ref_case)
    assert_parity(o, lse, o_ref, lse_ref, name)
    # host planner on the same lengths: identical plan, identical bits
    hplan = mla.Plan(lens_now, q_len=q_len, num_heads=heads, split_kv=split)
    dc.kv_lens.copy_(lens_dev)
    dc.kv_lens_host = list(lens_now)
    o_h, lse_h = mla.run_decode(dc, hplan)
    torch.cuda.synchronize()
    assert np.array_equal(o, o_h.float().cpu().numpy()), "graph path differs from host plan"
    assert np.array_equal(lse, lse_h.cpu().numpy())


def test_graph_zero_length_request(mla):
    case = inputs.make_case([500, 64], num_heads=12, q_len=1, seed=31, split_kv=0)
    dc = mla.to_device(case)
    plan = mla.Plan.graph(2, q_len=1, num_heads=12, max_kv_len=500)
    ws = plan.alloc_workspace()
    lens_dev = torch.tensor([0, 64], dtype=torch.int32, device="cuda")
    _say("[gpu] graph zero-length request")
    o, lse = graph_call(mla, plan, dc, lens_dev, scal(case.softmax_scale), scal(1.0), ws)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    assert (o[:12] == 0).all() and np.isneginf(lse[:12]).all()
    ref_case = inputs.Case(q=case.q[1:], kv=case.kv, block_table=case.block_table[1:],
                           kv_lens=torch.tensor([64], dtype=torch.int32), q_len=1, num_heads=12,
                           softmax_scale=case.softmax_scale)
    o_ref, lse_ref = run_oracle(ref_case)
    assert_parity(o[12:], lse[12:], o_ref, lse_ref, "zero-length neighbour")


@pytest.mark.parametrize("split", [0, 2], ids=["planner", "uniform_shared"])
def test_graph_capture_replay(mla, split):
    """One captured call, replayed while the device lengths and scales change (with a
    uniform split_kv of 2 each split is shared by several workgroups and folded)."""
    # the cache holds 6000 valid tokens for every request; the device lengths vary below
    case = inputs.make_case([6000] * 4, num_heads=12, q_len=2, seed=99, split_kv=split)
    dc = mla.to_device(case)
    plan = mla.Plan.graph(4, q_len=2, num_heads=12, max_kv_len=6000, split_kv=split)
    assert (plan.info()[0].split_workgroups > 1) == (split > 0)
    ws = plan.alloc_workspace()
    lens = [6000, 900, 33, 2500]
    lens_dev = torch.tensor(lens, dtype=torch.int32, device="cuda")
    ss, os_ = scal(case.softmax_scale), scal(1.0)
    rows = case.rows
    o = torch.empty((rows, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((rows,), dtype=torch.float32, device="cuda")
    # warm up eagerly, then capture one call on a side stream
    mla.decode_graph(plan, dc.q, dc.kv, dc.block_table, lens_dev, ss, os_, ws, o, lse)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        mla.decode_graph(plan, dc.q, dc.kv, dc.block_table, lens_dev, ss, os_, ws, o, lse, s)
    torch.cuda.synchronize()
    settings = [([6000, 900, 33, 2500], 0.0722, 1.0), ([17, 4000, 2, 2500], 0.0722, 0.5),
                ([6000, 6000, 6000, 6000], 0.05, 1.0), ([3, 5, 2, 2], 0.1, 2.0),
                ([6000, 900, 33, 2500], 0.0722, 1.0)]
    for i, (ln, sm, om) in enumerate(settings):
        lens_dev.copy_(torch.tensor(ln, dtype=torch.int32))
        ss.fill_(sm)
        os_.fill_(om)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_g, lse_g = o.clone(), lse.clone()
        # eager call on the same inputs
        o_e = torch.empty_like(o)
        lse_e = torch.empty_like(lse)
        mla.decode_graph(plan, dc.q, dc.kv, dc.block_table, lens_dev, ss, os_, ws, o_e, lse_e)
        torch.cuda.synchronize()
        _say(f"[gpu] graph replay {i}: lens={ln} scale={sm} out_scale={om}")
        ref_case = inputs.Case(q=case.q, kv=case.kv, block_table=case.block_table,
                               kv_lens=torch.tensor(ln, dtype=torch.int32), q_len=2,
                               num_heads=12, softmax_scale=sm, output_scale=om)
        o_ref, lse_ref = run_oracle(ref_case)
        assert_parity(o_g.float().cpu().numpy(), lse_g.cpu().numpy(), o_ref, lse_ref,
                      f"replay {i}")
        assert torch.equal(o_g, o_e) and torch.equal(lse_g, lse_e), f"replay {i} != eager"


# The device planner searches one wave per request set up to 64 requests and across
# waves beyond: both sides of that line, against the host planner, bit for bit.
@pytest.mark.parametrize("batch", [63, 64, 65, 100, 256])
def test_graph_equals_host_across_batch_sizes(mla, batch):
    g = torch.Generator().manual_seed(9000 + batch)
    lens = torch.randint(33, 1500, (batch,), generator=g).tolist()
    _say(f"[gpu] graph vs host: batch={batch} lens {min(lens)}..{max(lens)}")
    case = inputs.make_case(lens, num_heads=12, q_len=1, seed=900 + batch, split_kv=0)
    dc = mla.to_device(case)
    plan = mla.Plan.graph(batch, q_len=1, num_heads=12, max_kv_len=max(lens))
    ws = plan.alloc_workspace()
    o, lse = graph_call(mla, plan, dc, dc.kv_lens, scal(case.softmax_scale),
                        scal(case.output_scale), ws)
    hplan = mla.Plan(lens, q_len=1, num_heads=12, split_kv=0)
    o_h, lse_h = mla.run_decode(dc, hplan)
    torch.cuda.synchronize()
    assert torch.equal(o, o_h), "graph path differs from host plan"
    assert torch.equal(lse, lse_h)
    rows = inputs.sample_rows(case, 8)
    o_ref, lse_ref = run_oracle(case, rows)
    assert_parity(o.float().cpu().numpy()[rows], lse.cpu().numpy()[rows], o_ref, lse_ref,
                  f"graph batch={batch}")
