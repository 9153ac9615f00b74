"""Host-side checks of libmla_decode.so that need no GPU: the exported symbols match the
header, the planner's splits, and argument validation (every rejected call returns
before anything is launched)."""
import ctypes
import math
import os
import re

import pytest
import torch

from decode_attention_gather_amd import mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_decode\w*)\s*\(", text)))


def test_exports_match_header():
    declared = header_functions()
    assert set(declared) == set(mla.EXPORTS), declared
    lib = mla.lib_handle()
    for name in declared:
        assert hasattr(lib, name), name


def plan(lens, q_len=1, heads=12, split=0, cap=128, cus=256):
    return mla.Plan(lens, q_len=q_len, num_heads=heads, split_kv=split, max_split_kv=cap,
                    num_cus=cus)


@pytest.mark.parametrize("lens,q,h,split,exp_splits,exp_chunk", [
    ([2048], 1, 12, 4, [4], [512]),
    ([131072] * 4, 1, 12, 25, [25] * 4, [5248] * 4),
    ([131072] * 16, 8, 12, 6, [6] * 16, [21856] * 16),
    ([1048576], 1, 12, 100, [100], [10496]),
    ([1], 1, 12, 4, [1], [32]),          # one token: one split of one page
    ([65], 8, 12, 3, [3], [32]),         # last split holds a single token
    ([100], 1, 12, 0, [4], [32]),        # planner, short: limited by pages
])
def test_uniform_and_short_plans(lens, q, h, split, exp_splits, exp_chunk):
    p = plan(lens, q, h, split)
    info, splits, chunk = p.info()
    assert splits == exp_splits and chunk == exp_chunk
    assert info.rows_per_request == q * h
    steps = max_steps_of(chunk)
    assert info.row_tiles == expected_row_blocks(q * h, sum(splits), max_steps=steps)
    assert info.total_splits == sum(splits)
    assert info.work_items == sum(splits) * info.row_tiles
    assert info.split_workgroups == expected_subs(info.work_items, steps)


def split_budget(cus, tiles):
    per_xcd = (cus // 8) // tiles
    return per_xcd * 8 if per_xcd >= 1 else max(1, cus // tiles)


def max_steps_of(chunk_tokens):
    """2-page steps of the longest split."""
    return max(math.ceil(c // 32 / 2) for c in chunk_tokens)


def expected_subs(items, max_steps, cus=256):
    """Workgroups per split: as many as idle CUs allow (cus // items), each with at least
    2 steps of the longest split, at most 8, at least 1."""
    return max(1, min(cus // items, max_steps // 2, 8))


def expected_row_blocks(rows, total_splits=None, cus=256, max_steps=0):
    """Row blocks of 16-row tiles: one block of <= 2 tiles up to 32 rows, otherwise as
    few blocks of <= 6 tiles as cover the rows, each rounded up to 4 or 6 tiles. A plan
    whose splits leave CUs idle and cannot be shared by several workgroups takes blocks
    of 4 tiles instead of 6 when the larger grid still fits one wave of the chip
    (total_splits given)."""
    tiles16 = math.ceil(rows / 16)
    if tiles16 <= 2:
        return 1
    blocks = math.ceil(tiles16 / 6)
    nt = 4 if math.ceil(tiles16 / blocks) <= 4 else 6
    if nt == 6 and total_splits is not None:
        tiles4 = math.ceil(tiles16 / 4)
        shared = expected_subs(total_splits * blocks, max_steps, cus) >= 2
        if not shared and total_splits <= split_budget(cus, tiles4):
            return tiles4
    return math.ceil(tiles16 / nt)


@pytest.mark.parametrize("rows, blocks", [(12, 1), (24, 1), (32, 1), (33, 1), (48, 1), (64, 1),
                                          (65, 1), (96, 1), (97, 2), (128, 2), (192, 2),
                                          (768, 8), (4096, 43)])
def test_row_blocks(rows, blocks):
    """The minimal blocking, on a plan that fills the chip (cus = 2 leaves no idle CU)."""
    assert expected_row_blocks(rows) == blocks
    info, _, _ = plan([4096], 1, rows, 2, cus=2).info()
    assert info.row_tiles == blocks


@pytest.mark.parametrize("lens,q,h,split,cus,tiles,subs", [
    ([131072] * 16, 8, 12, 6, 256, 1, 2),  # 96 splits of 96 rows, two workgroups each
    ([512] * 16, 8, 12, 6, 256, 2, 1),     # splits of 2 steps: 192 blocks of 64 rows
    ([131072] * 16, 8, 12, 0, 256, 1, 1),  # the planner fills the chip with 96-row blocks
    ([131072] * 16, 8, 12, 6, 128, 1, 1),  # 192 items would not fit 128 CUs
    ([4096] * 8, 8, 96, 2, 256, 8, 2),     # H96: 16 splits x 8 blocks, shared by two
    ([256] * 8, 8, 96, 2, 256, 12, 1),     # short splits: 16 x 12 blocks of 64 rows
    ([4096] * 8, 8, 96, 4, 256, 8, 1),     # 32 splits x 8 blocks fill the chip
    ([131072] * 16, 1, 12, 6, 256, 1, 2),  # the headline at split 6: 192 workgroups
    ([1048576], 1, 12, 100, 256, 1, 2),
    ([131072], 1, 12, 1, 256, 1, 8),       # at most 8 workgroups per split
    ([2048], 1, 12, 4, 256, 1, 4),         # splits of 8 steps: 4 runs of 2 steps
    ([96], 1, 12, 3, 256, 1, 1),           # one-step splits stay whole
])
def test_underfilled_plans(lens, q, h, split, cus, tiles, subs):
    """Idle CUs: splits shared by several workgroups where they are long enough, else
    64-row blocks for the wide kernel where the larger grid fits one wave."""
    p = plan(lens, q, h, split, cap=256, cus=cus)
    info, splits, chunk = p.info()
    steps = max_steps_of(chunk)
    assert info.row_tiles == tiles == expected_row_blocks(q * h, sum(splits), cus, steps)
    assert info.work_items == sum(splits) * tiles
    assert info.split_workgroups == subs == expected_subs(info.work_items, steps, cus)
    # the workspace holds the split partials and, when shared, one state per workgroup
    rows = q * h
    per = (512 + 4) * 4 * rows * sum(splits)
    assert p.workspace_size() >= per * (1 + (subs if subs > 1 else 0))


def test_graph_plans_share_uniform_splits():
    """Graph plans decide shared splits on the host from the capacity and the length
    bound (uniform split_kv only); here they match the host plan of those lengths."""
    for B, L, split in ((16, 131072, 6), (2, 40000, 2), (1, 1 << 20, 100), (2, 3000, 4)):
        g = mla.Plan.graph(B, q_len=1, num_heads=12, max_kv_len=L, split_kv=split, num_cus=256)
        h = plan([L] * B, 1, 12, split, cap=256)
        assert g.info()[0].split_workgroups == h.info()[0].split_workgroups
    g = mla.Plan.graph(16, q_len=1, num_heads=12, max_kv_len=131072, split_kv=6, num_cus=256)
    assert g.info()[0].split_workgroups == 2
    g = mla.Plan.graph(16, q_len=1, num_heads=12, max_kv_len=131072, split_kv=0, num_cus=256)
    assert g.info()[0].split_workgroups == 1


def check_cover(lens, splits, chunk):
    for L, s, c in zip(lens, splits, chunk):
        assert c % 32 == 0 and c > 0
        assert (s - 1) * c < L <= s * c, (L, s, c)  # no empty split, full coverage


@pytest.mark.parametrize("lens", [[131072] * 16, [131072] * 4, [1048576], [4096, 131072, 70000, 5000],
                                  [32] * 200, [7, 1000, 123456, 99]])
def test_planner_one_wave(lens):
    p = plan(lens, 1, 12, 0, 128, 256)
    info, splits, chunk = p.info()
    check_cover(lens, splits, chunk)
    assert max(splits) <= 128
    # at most one wave unless every request is already at one split
    assert info.work_items <= 256 or max(splits) == 1
    if len(lens) == 16 and len(set(lens)) == 1:
        assert splits == [16] * 16


def test_planner_proportional_and_cap():
    lens = [4096, 131072, 65536, 8192]
    p = plan(lens, 1, 12, 0, 128, 256)
    _, splits, chunk = p.info()
    check_cover(lens, splits, chunk)
    assert splits[1] >= splits[2] >= splits[3] >= splits[0]
    p = plan([1048576], 1, 12, 0, 128, 256)
    assert p.info()[1] == [128]
    p = plan([1048576], 1, 12, 0, 256, 256)
    assert p.info()[1] == [256]


def test_merge_slices_rule():
    """Workgroups per row in the merge: 8 only when the rows of the requests holding the
    most splits number at most num_cus / 16 and those splits exceed 16 x 8; else 1."""
    assert plan([1048576], 1, 12, 0, cap=256).info()[0].merge_slices == 8   # 12 rows x 256
    assert plan([1048576], 1, 12, 100).info()[0].merge_slices == 1          # 100 splits
    assert plan([1048576], 2, 12, 0, cap=256).info()[0].merge_slices == 1   # 24 rows
    assert plan([131072] * 16, 1, 12, 0).info()[0].merge_slices == 1
    assert plan([1 << 20] + [4096] * 7, 8, 12, 0, cap=256).info()[0].merge_slices == 1
    # graph plans: as for a batch of equal requests at the largest split count
    g = mla.Plan.graph(1, q_len=1, num_heads=12, max_kv_len=1 << 20, num_cus=256)
    assert g.info()[0].merge_slices == 8
    g = mla.Plan.graph(16, q_len=1, num_heads=12, max_kv_len=131072, num_cus=256)
    assert g.info()[0].merge_slices == 1


def test_merge_groups_rule():
    assert plan([1048576], 1, 12, 100).info()[0].merge_groups == 16
    assert plan([2048], 1, 12, 4).info()[0].merge_groups == 4
    assert plan([131072] * 16, 8, 12, 6).info()[0].merge_groups == 4  # 1536 rows x 4 <= 32 x 256
    assert plan([131072] * 64, 8, 12, 6).info()[0].merge_groups == 1  # 6144 rows fill the GPU
    # the skewed batch: 96 rows of the long request fold 249 partials with 16 groups;
    # the 672 rows of one-split requests use one group each (2208 waves <= 8192)
    assert plan([1 << 20] + [4096] * 7, 8, 12, 0, cap=256).info()[0].merge_groups == 16
    # but 64 requests of 16 splits each at q8 H12: 6144 rows x 16 > 8192 -> 1
    assert plan([131072] * 64, 8, 12, 16).info()[0].merge_groups == 1
    assert plan([100], 1, 12, 1).info()[0].merge_groups == 1


def test_workspace_size():
    # 96 splits x 96 rows of fp32 (O, m, l, l~, 0), whole splits (cus 128)
    p = plan([131072] * 16, 8, 12, 6, cus=128)
    assert p.info()[0].split_workgroups == 1
    assert p.workspace_size() == 96 * 96 * 512 * 4 + 96 * 96 * 4 * 4
    # two workgroups per split: their states too
    p = plan([131072] * 16, 8, 12, 6)
    assert p.info()[0].split_workgroups == 2
    assert p.workspace_size() == 3 * (96 * 96 * 512 * 4 + 96 * 96 * 4 * 4)


@pytest.mark.parametrize("kw,status", [
    (dict(lens=[8], q_len=9), mla.MLA_ERR_INVALID_ARG),          # L < q_len
    (dict(lens=[8], q_len=0), mla.MLA_ERR_INVALID_ARG),
    (dict(lens=[8], heads=0), mla.MLA_ERR_INVALID_ARG),
    (dict(lens=[8], split=-1), mla.MLA_ERR_INVALID_ARG),
    (dict(lens=[8], cap=0), mla.MLA_ERR_INVALID_ARG),
    (dict(lens=[8], cap=2000), mla.MLA_ERR_UNSUPPORTED_SHAPE),
    (dict(lens=[8] * 257), mla.MLA_ERR_UNSUPPORTED_SHAPE),
    (dict(lens=[8], q_len=8, heads=600), mla.MLA_ERR_UNSUPPORTED_SHAPE),
])
def test_plan_rejects(kw, status):
    args = dict(lens=[8], q_len=1, heads=12, split=0, cap=128, cus=256)
    args.update(kw)
    with pytest.raises(mla.MlaError) as ei:
        plan(args["lens"], args["q_len"], args["heads"], args["split"], args["cap"], args["cus"])
    assert ei.value.status == status


def test_call_validation_before_launch():
    """Bad arguments are rejected on the host; these calls never reach a launch."""
    lib = mla.lib_handle()
    p = plan([100, 50], 1, 12, 2)
    ws_need = p.workspace_size()
    fake = ctypes.c_void_p(0x10000)  # aligned, never dereferenced on these paths
    nul = None
    # null q
    assert lib.mla_decode_partial(p.handle, nul, fake, fake, 4, fake, 0.07, fake, ws_need,
                                  nul) == mla.MLA_ERR_INVALID_ARG
    # block-table row too short for 100 tokens (needs 4 pages)
    assert lib.mla_decode_partial(p.handle, fake, fake, fake, 3, fake, 0.07, fake, ws_need,
                                  nul) == mla.MLA_ERR_INVALID_ARG
    # misaligned q
    assert lib.mla_decode_partial(p.handle, ctypes.c_void_p(0x10001), fake, fake, 4, fake, 0.07,
                                  fake, ws_need, nul) == mla.MLA_ERR_INVALID_ARG
    # non-finite scale
    assert lib.mla_decode_partial(p.handle, fake, fake, fake, 4, fake, float("nan"), fake,
                                  ws_need, nul) == mla.MLA_ERR_INVALID_ARG
    # workspace too small / misaligned / null
    assert lib.mla_decode_partial(p.handle, fake, fake, fake, 4, fake, 0.07, fake, ws_need - 1,
                                  nul) == mla.MLA_ERR_WORKSPACE
    assert lib.mla_decode_partial(p.handle, fake, fake, fake, 4, fake, 0.07,
                                  ctypes.c_void_p(0x10010), ws_need, nul) == mla.MLA_ERR_WORKSPACE
    assert lib.mla_decode_merge(p.handle, nul, ws_need, 1.0, fake, nul, nul) == mla.MLA_ERR_WORKSPACE
    assert lib.mla_decode_merge(p.handle, fake, ws_need, 1.0, nul, nul, nul) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_decode_merge_f32(p.handle, fake, ws_need, float("inf"), fake, nul,
                                    nul) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_decode(None, fake, fake, fake, 4, fake, 0.07, 1.0, fake, ws_need, fake, nul,
                          nul) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_decode_workspace_size(None) == 0


def test_strerror():
    for s in (0, -1, -2, -3, -4, -1001, 7):
        assert isinstance(mla.strerror(s), str) and mla.strerror(s)


# ---- graph plans (device lengths) -----------------------------------------------------

def gplan(batch, max_len, q_len=1, heads=12, split=0, cap=128, cus=256):
    return mla.Plan.graph(batch, q_len=q_len, num_heads=heads, max_kv_len=max_len,
                          split_kv=split, max_split_kv=cap, num_cus=cus)


@pytest.mark.parametrize("batch,max_len,q,h,split,cap_parts", [
    (16, 131072, 1, 12, 0, 16 * 2 + 256),        # min(B cap, 2 B + CUs / row blocks)
    (1, 2048, 1, 12, 0, 64),                      # bounded by the pages: 2048 / 32
    (16, 131072, 8, 12, 6, 96),                   # uniform: B * split
    (4, 131072, 1, 12, 25, 100),
    (8, 131072, 8, 96, 0, 8 * 2 + 256 // 8),      # 8 row blocks per split
    (2, 100, 1, 12, 0, 8),                        # 4 pages per request at most
    (1, 3 * 2 ** 21, 1, 12, 0, 128 + 4),          # > 2^21 tokens: + B ceil(pages / 65535)
])
def test_graph_plan_capacity(batch, max_len, q, h, split, cap_parts):
    info, splits, chunk = gplan(batch, max_len, q, h, split).info()
    assert info.total_splits == cap_parts
    assert info.work_items == cap_parts * info.row_tiles
    assert splits == [0] * batch and chunk == [0] * batch  # decided on the device
    p = gplan(batch, max_len, q, h, split)
    rows = q * h
    head = 3840  # the device plan (PlanDev, 3616 bytes) at the workspace head, 256-aligned
    o = (cap_parts * rows * 2048 + 255) // 256 * 256
    st = (cap_parts * rows * 16 + 255) // 256 * 256
    subs = info.split_workgroups  # shared splits keep one state per workgroup too
    assert (subs > 1) == (split > 0 and cap_parts * info.row_tiles * 2 <= 256)
    extra = 0
    if subs > 1:
        extra = ((cap_parts * subs * rows * 2048 + 255) // 256 * 256
                 + (cap_parts * subs * rows * 16 + 255) // 256 * 256)
    assert p.workspace_size() == head + o + st + extra


def test_graph_plan_capacity_covers_device_plans():
    """Upper bound of the device planner's split counts (its rules restated here): for
    random lengths up to the bound, sum_b S_b never exceeds the capacity."""
    import random
    rnd = random.Random(5)
    for _ in range(300):
        B = rnd.randint(1, 32)
        max_len = rnd.choice([1, 31, 32, 100, 4096, 131072, 1 << 20])
        split = rnd.choice([0, 0, 1, 3, 128])
        cap = rnd.choice([1, 16, 128])
        cus = rnd.choice([8, 80, 256])
        heads = rnd.choice([1, 12, 96])
        info = gplan(B, max_len, 1, heads, split, cap, cus).info()[0]
        lens = [rnd.randint(0, max_len) for _ in range(B)]
        hp = None
        if min(lens) >= 1:
            hp = mla.Plan(lens, q_len=1, num_heads=heads, split_kv=split, max_split_kv=cap,
                          num_cus=cus).info()[0]
            assert hp.total_splits <= info.total_splits, (B, max_len, split, cap, cus, lens)
            assert hp.merge_groups <= info.merge_groups


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), mla.MLA_ERR_INVALID_ARG),
    (dict(max_len=0), mla.MLA_ERR_INVALID_ARG),
    (dict(q=0), mla.MLA_ERR_INVALID_ARG),
    (dict(split=-1), mla.MLA_ERR_INVALID_ARG),
    (dict(batch=257), mla.MLA_ERR_UNSUPPORTED_SHAPE),
    (dict(cap=2000), mla.MLA_ERR_UNSUPPORTED_SHAPE),
])
def test_graph_plan_rejects(kw, status):
    args = dict(batch=2, max_len=100, q=1, heads=12, split=0, cap=128, cus=256)
    args.update(kw)
    with pytest.raises(mla.MlaError) as ei:
        gplan(args["batch"], args["max_len"], args["q"], args["heads"], args["split"],
              args["cap"], args["cus"])
    assert ei.value.status == status


def test_graph_and_host_plans_not_interchangeable():
    lib = mla.lib_handle()
    g = gplan(2, 100)
    h = plan([100, 50], 1, 12, 2)
    fake = ctypes.c_void_p(0x10000)
    nul = None
    need = g.workspace_size()
    # a graph plan through the host-plan entry points
    assert lib.mla_decode(g.handle, fake, fake, fake, 4, fake, 0.07, 1.0, fake, need, fake, nul,
                          nul) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_decode_partial(g.handle, fake, fake, fake, 4, fake, 0.07, fake, need,
                                  nul) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_decode_merge(g.handle, fake, need, 1.0, fake, nul, nul) == mla.MLA_ERR_INVALID_ARG
    # a host plan through the graph entry point
    assert lib.mla_decode_graph(h.handle, fake, fake, fake, 4, fake, nul, fake, fake, fake,
                                h.workspace_size(), fake, nul, nul) == mla.MLA_ERR_INVALID_ARG
    # graph call validation: null scale pointers, short block-table rows, workspace,
    # misaligned q_lens
    assert lib.mla_decode_graph(g.handle, fake, fake, fake, 4, fake, nul, nul, fake, fake, need,
                                fake, nul, nul) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_decode_graph(g.handle, fake, fake, fake, 3, fake, nul, fake, fake, fake, need,
                                fake, nul, nul) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_decode_graph(g.handle, fake, fake, fake, 4, fake, nul, fake, fake, fake,
                                need - 1, fake, nul, nul) == mla.MLA_ERR_WORKSPACE
    assert lib.mla_decode_graph(g.handle, fake, fake, fake, 4, fake, ctypes.c_void_p(0x10002),
                                fake, fake, fake, need, fake, nul, nul) == mla.MLA_ERR_INVALID_ARG
    # ragged-query entry point: needs q_lens, refuses graph plans
    assert lib.mla_decode_varq(h.handle, fake, fake, fake, 4, fake, nul, 0.07, 1.0, fake,
                               h.workspace_size(), fake, nul, nul) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_decode_varq(g.handle, fake, fake, fake, 4, fake, fake, 0.07, 1.0, fake, need,
                               fake, nul, nul) == mla.MLA_ERR_INVALID_ARG


def test_epilogue_validation_before_launch():
    """The epilogue variants reject bad pointer combinations on the host."""
    lib = mla.lib_handle()
    p = plan([100, 50], 1, 12, 2)
    ws = p.workspace_size()
    fake = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10004)  # 4-byte aligned only
    nul = None
    merge = lib.mla_decode_merge_ex
    # codes without scales, and the reverse
    assert merge(p.handle, fake, ws, 1.0, nul, fake, nul, fake, nul, nul) == mla.MLA_ERR_INVALID_ARG
    assert merge(p.handle, fake, ws, 1.0, nul, fake, nul, nul, fake, nul) == mla.MLA_ERR_INVALID_ARG
    # neither BF16 O nor MXFP8 O
    assert merge(p.handle, fake, ws, 1.0, nul, nul, nul, nul, nul, nul) == mla.MLA_ERR_INVALID_ARG
    # MXFP8 codes need 8-byte alignment; BF16 O written next to them needs 16
    assert merge(p.handle, fake, ws, 1.0, nul, fake, nul, odd, fake, nul) == mla.MLA_ERR_INVALID_ARG
    assert merge(p.handle, fake, ws, 1.0, nul, odd, nul, fake, fake, nul) == mla.MLA_ERR_INVALID_ARG
    # misaligned sinks
    assert merge(p.handle, fake, ws, 1.0, ctypes.c_void_p(0x10002), fake, nul, nul, nul,
                 nul) == mla.MLA_ERR_INVALID_ARG
    # short workspace
    assert merge(p.handle, fake, ws - 1, 1.0, nul, nul, nul, fake, fake, nul) == mla.MLA_ERR_WORKSPACE
    dec = lib.mla_decode_ex
    assert dec(p.handle, fake, fake, fake, 4, fake, ctypes.c_void_p(0x10002), 0.07, 1.0, nul,
               fake, ws, fake, nul, nul, nul, nul) == mla.MLA_ERR_INVALID_ARG
    assert dec(p.handle, fake, fake, fake, 4, fake, nul, 0.07, 1.0, nul, fake, ws, fake, nul,
               fake, nul, nul) == mla.MLA_ERR_INVALID_ARG
    # plans and entry points do not mix
    g = gplan(2, 100)
    gws = g.workspace_size()
    assert dec(g.handle, fake, fake, fake, 4, fake, nul, 0.07, 1.0, nul, fake, gws, fake, nul,
               nul, nul, nul) == mla.MLA_ERR_INVALID_ARG
    assert merge(g.handle, fake, gws, 1.0, nul, fake, nul, nul, nul, nul) == mla.MLA_ERR_INVALID_ARG
    gex = lib.mla_decode_graph_ex
    assert gex(p.handle, fake, fake, fake, 4, fake, nul, fake, fake, nul, fake, ws, fake, nul,
               nul, nul, nul) == mla.MLA_ERR_INVALID_ARG
    assert gex(g.handle, fake, fake, fake, 4, fake, nul, fake, fake, nul, fake, gws, fake, nul,
               fake, nul, nul) == mla.MLA_ERR_INVALID_ARG
    assert gex(g.handle, fake, fake, fake, 4, fake, nul, nul, fake, nul, fake, gws, fake, nul,
               nul, nul, nul) == mla.MLA_ERR_INVALID_ARG


@pytest.mark.parametrize("rows_q,heads,exp_tiles", [
    (1, 12, 1), (2, 16, 1), (8, 12, 1), (3, 12, 1), (8, 96, 8), (1, 5, 1), (7, 16, 2),
])
def test_bf16_plans_share_the_row_block_rule(rows_q, heads, exp_tiles):
    """BF16 plans block rows as E4M3 plans do: up to 32 rows in one block, more in as
    few blocks of at most 96 rows as cover them (graph plans; and host plans that fill
    the chip), and 64-row blocks where a host plan leaves CUs idle."""
    for cus in (256, 2):
        p = mla.Plan([4096, 100], q_len=rows_q, num_heads=heads, split_kv=2, num_cus=cus,
                     kv_dtype="bf16")
        e = mla.Plan([4096, 100], q_len=rows_q, num_heads=heads, split_kv=2, num_cus=cus)
        info = p.info()[0]
        assert info.row_tiles == e.info()[0].row_tiles
        steps = max_steps_of(p.info()[2])
        assert info.row_tiles == expected_row_blocks(rows_q * heads, info.total_splits, cus,
                                                     steps)
        assert info.work_items == info.total_splits * info.row_tiles
        if cus == 2:
            assert info.row_tiles == exp_tiles
    g = mla.Plan.graph(2, q_len=rows_q, num_heads=heads, max_kv_len=4096, num_cus=256,
                       kv_dtype="bf16")
    assert g.info()[0].row_tiles == exp_tiles


def test_kv_dtype_validation():
    lib = mla.lib_handle()
    lens = (ctypes.c_int32 * 1)(100)
    h = ctypes.c_void_p()
    assert lib.mla_decode_plan_ex(lens, 1, 1, 12, 0, 128, 256, 2, ctypes.byref(h)) == \
        mla.MLA_ERR_INVALID_ARG
    assert lib.mla_decode_plan_graph_ex(1, 1, 12, 100, 0, 128, 256, -1, ctypes.byref(h)) == \
        mla.MLA_ERR_INVALID_ARG
    with pytest.raises(ValueError):
        mla.Plan([100], q_len=1, num_heads=12, num_cus=256, kv_dtype="fp16")
    # the binding refuses tensors of the other element type before any launch
    p = mla.Plan([100], q_len=1, num_heads=12, num_cus=256, kv_dtype="bf16")
    q8 = torch.zeros((1, 1, 12, 576), dtype=torch.uint8)
    kv8 = torch.zeros((5, 32, 576), dtype=torch.uint8)
    with pytest.raises(TypeError):
        mla.partial(p, q8, kv8, torch.zeros((1, 4), dtype=torch.int32),
                    torch.tensor([100], dtype=torch.int32), 0.07, torch.zeros(256, dtype=torch.uint8))
    pe = mla.Plan([100], q_len=1, num_heads=12, num_cus=256)
    with pytest.raises(TypeError):
        mla.partial(pe, q8.to(torch.int16), kv8.to(torch.int16),
                    torch.zeros((1, 4), dtype=torch.int32), torch.tensor([100], dtype=torch.int32),
                    0.07, torch.zeros(256, dtype=torch.uint8))


@pytest.mark.parametrize("lens,q_len,heads,kv_dtype", [
    ([1 << 20], 8, 12, "bf16"),          # one 96-row block
    ([1 << 20], 1, 12, "e4m3"),          # one row block: the cap (256) fills the chip
    ([131072] * 16, 8, 12, "bf16"),
    ([1 << 20] + [4096] * 7, 8, 12, "e4m3"),
    ([50000, 3000, 7], 4, 16, "bf16"),
    ([131072] * 8, 8, 96, "e4m3"),       # 8 row blocks of 96 rows
])
def test_planner_wave_fits_every_xcd(lens, q_len, heads, kv_dtype):
    """Workgroup i runs on XCD i mod 8 with the row blocks of a split on one XCD: the
    planner's one-wave plan must not put more workgroups on an XCD than it has CUs."""
    p = mla.Plan(lens, q_len=q_len, num_heads=heads, split_kv=0, max_split_kv=256,
                 num_cus=256, kv_dtype=kv_dtype)
    info = p.info()[0]
    per_xcd = -(-info.total_splits // 8) * info.row_tiles
    assert per_xcd <= 32, (info.total_splits, info.row_tiles)
    # and it is not far below one wave: at least 7/8 of the CUs get work
    assert info.work_items >= 0.85 * (32 // info.row_tiles) * 8 * info.row_tiles, info.work_items


@pytest.mark.parametrize("lens,q,h,split", [([131072] * 2, 1, 12, 64), ([200000], 1, 12, 200),
                                            ([131072] * 16, 8, 12, 6), ([5000, 90], 2, 3, 7)])
def test_merge_bound_copies(lens, q, h, split):
    """PR #20380 (Description): the merge width is an upper bound of 1, 2, 4, 8 or 16 that
    the host halves until it fits; the copy keeps every split and only narrows the width."""
    p = plan(lens, q, h, split, cap=256)
    info, splits, chunk = p.info()
    for bound in (1, 2, 4, 8, 16):
        c = p.with_merge_bound(bound)
        ci, cs, cc = c.info()
        assert ci.merge_groups == min(bound, info.merge_groups)
        assert (cs, cc) == (splits, chunk)
        assert ci.merge_slices == info.merge_slices and ci.total_splits == info.total_splits
        assert c.workspace_size() == p.workspace_size()
    for bad in (0, 3, 32, -1):
        with pytest.raises(mla.MlaError):
            p.with_merge_bound(bad)
    g = mla.Plan.graph(len(lens), q_len=q, num_heads=h, max_kv_len=max(lens), split_kv=split,
                       num_cus=256)
    gi = g.info()[0]
    assert g.with_merge_bound(2).info()[0].merge_groups == min(2, gi.merge_groups)


def test_bounded_calls_validate_before_launch():
    """The key-window entry points reject bad arguments on the host (no launch)."""
    lib = mla.lib_handle()
    h = plan([100, 50], 1, 12, 2)
    g = gplan(2, 100)
    fake = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10002)
    nul = None
    need = h.workspace_size()
    # kv_bounds is required by the bounded calls, and must be 4-byte aligned
    assert lib.mla_decode_bounded(h.handle, fake, fake, fake, 4, fake, nul, nul, 0.07, 1.0, nul,
                                  fake, need, fake, nul, nul, nul, nul) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_decode_bounded(h.handle, fake, fake, fake, 4, fake, nul, odd, 0.07, 1.0, nul,
                                  fake, need, fake, nul, nul, nul, nul) == mla.MLA_ERR_INVALID_ARG
    # workspace and plan kind checks as for the unbounded calls
    assert lib.mla_decode_bounded(h.handle, fake, fake, fake, 4, fake, nul, fake, 0.07, 1.0, nul,
                                  fake, need - 1, fake, nul, nul, nul, nul) == mla.MLA_ERR_WORKSPACE
    assert lib.mla_decode_bounded(g.handle, fake, fake, fake, 4, fake, nul, fake, 0.07, 1.0, nul,
                                  fake, g.workspace_size(), fake, nul, nul, nul,
                                  nul) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_decode_graph_bounded(h.handle, fake, fake, fake, 4, fake, nul, fake, fake, fake,
                                        nul, fake, need, fake, nul, nul, nul,
                                        nul) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_decode_graph_bounded(g.handle, fake, fake, fake, 4, fake, nul, nul, fake, fake,
                                        nul, fake, g.workspace_size(), fake, nul, nul, nul,
                                        nul) == mla.MLA_ERR_INVALID_ARG
    # the partial pass: windows optional but aligned; short block-table rows refused
    assert lib.mla_decode_partial_ex(h.handle, fake, fake, fake, 4, fake, nul, odd, 0.07, fake,
                                     need, nul) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_decode_partial_ex(h.handle, fake, fake, fake, 3, fake, nul, fake, 0.07, fake,
                                     need, nul) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_decode_partial_ex(g.handle, fake, fake, fake, 4, fake, nul, fake, 0.07, fake,
                                     need, nul) == mla.MLA_ERR_INVALID_ARG


def test_noalloc_validates_before_launch():
    lib = mla.lib_handle()
    fake = ctypes.c_void_p(0x10000)
    g = gplan(2, 100)
    assert lib.mla_decode_noalloc(None, fake, fake, fake, 4, fake, 0.07, 1.0, fake, None,
                                  None) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_decode_noalloc(g.handle, fake, fake, fake, 4, fake, 0.07, 1.0, fake, None,
                                  None) == mla.MLA_ERR_INVALID_ARG
    big = plan([1 << 20] * 4, 8, 128, 1024, cap=1024)
    assert big.workspace_size() > mla.NOALLOC_SCRATCH_BYTES
    assert lib.mla_decode_noalloc(big.handle, fake, fake, fake, 32768, fake, 0.07, 1.0, fake, None,
                                  None) == mla.MLA_ERR_WORKSPACE
