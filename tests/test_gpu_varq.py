"""Ragged query batches (per-request query counts), through the C ABI.

Expected values come from the fp64 oracle applied to each request on its own, with
q_len = that request's count (the causal MTP rule of the oracle then uses that count);
rows j >= q_lens[b] must come out as O = 0 and LSE = -inf. Also checked: q_lens equal
to q_len everywhere reproduces the uniform path bit for bit, and the graph path with
device q_lens reproduces the host-planned ragged call bit for bit.
"""
import numpy as np
import pytest
import torch

from decode_attention_gather_amd import inputs
from test_gpu_parity import _say, assert_parity, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    from decode_attention_gather_amd import mla as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def expected(case, q_lens):
    H, Q = case.num_heads, case.q_len
    B = case.batch
    o = np.zeros((B, Q, H, 512))
    lse = np.full((B, Q, H), -np.inf)
    for b in range(B):
        qb = q_lens[b]
        if qb == 0:
            continue
        sub = inputs.Case(q=case.q[b:b + 1, :qb].contiguous(), kv=case.kv,
                          block_table=case.block_table[b:b + 1].contiguous(),
                          kv_lens=case.kv_lens[b:b + 1].clone(), q_len=qb, num_heads=H,
                          softmax_scale=case.softmax_scale, output_scale=case.output_scale)
        ob, lb = run_oracle(sub)
        o[b, :qb] = ob.reshape(qb, H, 512)
        lse[b, :qb] = lb.reshape(qb, H)
    return o.reshape(B * Q * H, 512), lse.reshape(B * Q * H)


def run_varq(mla, case, q_lens, split_kv=0):
    dc = mla.to_device(case)
    plan = mla.Plan(dc.kv_lens_host, q_len=case.q_len, num_heads=case.num_heads,
                    split_kv=split_kv)
    ws = plan.alloc_workspace()
    rows = case.rows
    o = torch.empty((rows, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((rows,), dtype=torch.float32, device="cuda")
    ql = torch.tensor(q_lens, dtype=torch.int32, device="cuda")
    mla.decode(plan, dc.q, dc.kv, dc.block_table, dc.kv_lens, dc.softmax_scale, dc.output_scale,
               ws, o, lse, q_lens=ql)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy(), dc


def check_ragged(o, lse, o_ref, lse_ref, tag):
    dead = np.isneginf(lse_ref)
    assert (o[dead] == 0).all() and np.isneginf(lse[dead]).all(), f"{tag}: rows past q_lens"
    assert_parity(o[~dead], lse[~dead], o_ref[~dead], lse_ref[~dead], tag)


VARQ = [
    # name, kv_lens, heads, q_max, q_lens, split_kv
    ("h12_q8_wide", [3000, 777, 64, 2000], 12, 8, [8, 3, 1, 5], 0),
    ("h12_q8_split3", [3000, 777], 12, 8, [2, 7], 3),
    ("h12_q4_rows48", [900, 1500, 40], 12, 4, [4, 1, 3], 0),
    ("h16_q2_narrow", [500, 64, 300], 16, 2, [1, 2, 0], 2),
    ("h12_q2_h_rows24", [129, 2048], 12, 2, [2, 1], 0),
    ("h96_q2", [400, 900], 96, 2, [1, 2], 0),
]


@pytest.mark.parametrize("name,lens,heads,q_max,q_lens,split", VARQ, ids=[v[0] for v in VARQ])
def test_varq_parity(mla, name, lens, heads, q_max, q_lens, split):
    case = inputs.make_case(lens, num_heads=heads, q_len=q_max, seed=4321, split_kv=split)
    _say(f"[gpu] varq {name}: lens={lens} H={heads} q_max={q_max} q_lens={q_lens}")
    o, lse, _ = run_varq(mla, case, q_lens, split)
    o_ref, lse_ref = expected(case, q_lens)
    check_ragged(o, lse, o_ref, lse_ref, name)


def test_varq_full_equals_uniform(mla):
    case = inputs.make_case([3000, 777], num_heads=12, q_len=8, seed=11, split_kv=0)
    _say("[gpu] varq with every q_len = q_max vs the uniform path")
    o, lse, dc = run_varq(mla, case, [8, 8])
    plan = mla.Plan(dc.kv_lens_host, q_len=8, num_heads=12, split_kv=0)
    o_u, lse_u = mla.run_decode(dc, plan)
    torch.cuda.synchronize()
    assert np.array_equal(o, o_u.float().cpu().numpy()) and np.array_equal(lse, lse_u.cpu().numpy())


def test_varq_graph_equals_host(mla):
    case = inputs.make_case([3000, 777, 2000], num_heads=12, q_len=8, seed=12, split_kv=0)
    q_lens = [5, 8, 2]
    _say(f"[gpu] varq graph path, q_lens={q_lens}")
    o, lse, dc = run_varq(mla, case, q_lens)
    plan = mla.Plan.graph(3, q_len=8, num_heads=12, max_kv_len=3000)
    ws = plan.alloc_workspace()
    og = torch.empty((case.rows, 512), dtype=torch.bfloat16, device="cuda")
    lg = torch.empty((case.rows,), dtype=torch.float32, device="cuda")
    mla.decode_graph(plan, dc.q, dc.kv, dc.block_table, dc.kv_lens,
                     torch.tensor([case.softmax_scale], dtype=torch.float32, device="cuda"),
                     torch.tensor([1.0], dtype=torch.float32, device="cuda"), ws, og, lg,
                     q_lens=torch.tensor(q_lens, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert np.array_equal(o, og.float().cpu().numpy()) and np.array_equal(lse, lg.cpu().numpy())
