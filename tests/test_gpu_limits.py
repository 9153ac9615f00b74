"""The C ABI at its documented limits, against the fp64 oracle (same bar as
tests/test_gpu_parity.py):
  * MLA_MAX_BATCH requests in one plan (every row checked);
  * MLA_MAX_ROWS_PER_REQUEST query rows in one request (H 128, q 32: 43 wide row blocks);
  * one request longer than 2^21 tokens with split_kv = 1: a split may hold at most
    65535 pages, so the planner must cut it in two (sampled rows);
  * the BF16 cache at the batch limit.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_gather_amd import inputs
from test_gpu_parity import F32, _say, assert_parity, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    from decode_attention_gather_amd import mla as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def test_max_batch(mla):
    g = torch.Generator().manual_seed(3)
    lens = (torch.randint(1, 400, (256,), generator=g)).tolist()
    case = inputs.make_case(lens, num_heads=12, q_len=1, seed=601, split_kv=0)
    _say(f"[gpu] limits: 256 requests, lengths 1..399")
    o, lse, plan = run_gpu(mla, case, split_kv=0)
    assert plan.info()[0].batch == 256
    o_ref, lse_ref = run_oracle(case)
    assert_parity(o, lse, o_ref, lse_ref, "max batch")


def test_max_rows_per_request(mla):
    # 128 heads x 32 query tokens = 4096 rows, causal over the last 32 keys
    case = inputs.make_case([96, 200], num_heads=128, q_len=32, seed=602, split_kv=2)
    _say("[gpu] limits: 4096 rows per request (H 128, q 32)")
    o, lse, plan = run_gpu(mla, case, split_kv=2)
    info = plan.info()[0]
    # 4 splits leave CUs idle: 64 blocks of 64 rows
    assert info.rows_per_request == 4096 and info.row_tiles == 64
    rows = inputs.sample_rows(case, 600, seed=5)
    o_ref, lse_ref = run_oracle(case, rows)
    assert_parity(o[rows], lse[rows], o_ref, lse_ref, "4096 rows")
    # planned for 8 CUs the same splits fill the chip: 43 blocks of 96 rows, the last
    # one of 64 rows and 32 padding rows; a row's bits do not depend on its block
    _say("[gpu] limits: 4096 rows in 96-row blocks")
    dc = mla.to_device(case)
    p96 = mla.Plan(dc.kv_lens_host, q_len=32, num_heads=128, split_kv=2, num_cus=8)
    assert p96.info()[0].row_tiles == 43
    assert p96.info()[0].merge_groups == info.merge_groups  # the same merge order
    o96, lse96 = mla.run_decode(dc, p96)
    torch.cuda.synchronize()
    assert np.array_equal(o96.float().cpu().numpy(), o)
    assert np.array_equal(lse96.cpu().numpy(), lse)


def test_split_longer_than_chunk_limit(mla):
    L = (1 << 21) + 100  # 65539 pages: one split may hold at most 65535
    case = inputs.make_case([L], num_heads=12, q_len=1, seed=603, split_kv=1)
    _say(f"[gpu] limits: one request of {L} tokens with split_kv = 1")
    o, lse, plan = run_gpu(mla, case, split_kv=1)
    info, splits, chunks = plan.info()
    assert splits == [2] and chunks[0] <= 65535 * 32
    rows = list(range(12))
    o_ref, lse_ref = run_oracle(case, rows)
    assert_parity(o[rows], lse[rows], o_ref, lse_ref, "split > 2^21 tokens")


def test_bf16_max_batch(mla):
    g = torch.Generator().manual_seed(4)
    lens = (torch.randint(8, 300, (256,), generator=g)).tolist()
    case = inputs.make_case(lens, num_heads=12, q_len=2, seed=604, split_kv=0, kv_dtype="bf16")
    _say("[gpu] limits: 256 requests, BF16 cache, q 2")
    dc = mla.to_device(case)
    plan = mla.Plan(dc.kv_lens_host, q_len=2, num_heads=12, split_kv=0, kv_dtype="bf16")
    o, lse = mla.run_decode(dc, plan)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.mla_decode(case.q, case.kv, case.block_table, case.kv_lens, q_len=2,
                                       num_heads=12, softmax_scale=F32(case.softmax_scale),
                                       output_scale=1.0, kv_dtype="bf16")
    assert_parity(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "bf16 max batch")
