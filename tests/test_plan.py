"""The launch planner on the host, through attn_decode_plan (no GPU): the
plans the measured rules pick for the five workloads and at the edge of each
rule, and, over a seeded sweep of sizes and calls, the invariants the
kernels rely on -- every partial softmax state a split launch writes has a
slot in the workspace attn_decode_workspace_bytes sizes, the chunks cover
the positions streamed, and a call that finishes in one launch writes no
partial states."""
import ctypes

import numpy as np
import pytest

import decode_attention_kv_seq_amd as ad
from decode_attention_kv_seq_amd import PLAN_DEVICE_POS, PLAN_FROM_SCORES, PLAN_PAGED, PLAN_STEP

ATTN_ERR_NULL, ATTN_ERR_DIM = 1, 2


def plan(B, H, D, S, cp=0, flags=0):
    return ad.plan(B, H, D, S, cp, flags)


@pytest.mark.parametrize("args,expect", [
    # 4 heads x 101 positions: one chunk per head block, the split writes out
    ((1, 4, 64, 128, 100), dict(balanced=0, workgroups=1, chunks=1, launches=1)),
    # 4096 positions, head_dim 128: one head per workgroup, 512 workgroups
    ((1, 32, 128, 4096, 4095), dict(balanced=0, heads_per_workgroup=1, workgroups=512, launches=2)),
    # 20001 of 32768 positions: 256 workgroups of two heads (16 head blocks)
    ((1, 32, 128, 32768, 20000), dict(balanced=0, heads_per_workgroup=2, workgroups=256, launches=2)),
    # 131072 positions, head_dim 64: 1024 workgroups of four heads (512-byte rows)
    ((1, 64, 64, 131072, 131071), dict(balanced=0, heads_per_workgroup=4, workgroups=1024, launches=2)),
])
def test_single_sequence_workload_plans(args, expect):
    p = plan(*args)
    assert {k: p[k] for k in expect} == expect, p


@pytest.mark.parametrize("H,D,S,flags", [
    (40, 128, 32768, 0), (40, 128, 8192, 0), (20, 128, 65536, 0), (96, 128, 4096, 0),
    (24, 128, 65536, PLAN_STEP), (40, 128, 32768, PLAN_STEP), (40, 192, 32768, 0), (12, 128, 32768, 0),
])
def test_two_per_cu_plans_stay_within_their_target(H, D, S, flags):
    """Single sequences whose target is at most 512 workgroups (two per CU,
    head_dim > 64) never plan more than the target, and stay close to it: a
    few past a multiple of the 256 CUs would give some CUs a third chunk."""
    p = plan(1, H, D, S, S - 1, flags)
    target = 256 if flags & PLAN_STEP and D <= 128 else 512
    assert p["workgroups"] <= target, p
    assert p["workgroups"] >= 0.85 * target, p


@pytest.mark.parametrize("H,D,S,expect", [(12, 64, 65536, 1026), (20, 64, 65536, 1025)])
def test_four_per_cu_plans_round_up(H, D, S, expect):
    """With four workgroups per CU (head_dim 64, 1024 workgroups) the chunk
    count rounds up: one or two workgroups past the target cost less than
    the longer chunks of fewer workgroups."""
    assert plan(1, H, D, S, S - 1)["workgroups"] == expect


def test_ragged_batch_workload_takes_the_balanced_grid():
    # 256 workgroups of eight heads
    for flags in (PLAN_DEVICE_POS, PLAN_PAGED):
        p = plan(64, 32, 128, 8192, flags=flags)
        assert (p["balanced"], p["workgroups"], p["heads_per_workgroup"], p["launches"]) == (1, 256, 8, 2)


@pytest.mark.parametrize("H,D,flags,hpb", [
    (16, 128, PLAN_DEVICE_POS, 4),   # four head blocks of four heads
    (16, 128, PLAN_PAGED, 8),
    (16, 64, PLAN_DEVICE_POS, 8),
    (8, 128, PLAN_DEVICE_POS, 8),    # four per workgroup would still give two blocks
    (32, 128, PLAN_DEVICE_POS, 8),
    (64, 128, PLAN_DEVICE_POS, 8),
])
def test_balanced_head_blocks(H, D, flags, hpb):
    p = plan(32, H, D, 16384, flags=flags)
    assert (p["balanced"], p["heads_per_workgroup"]) == (1, hpb), p


def kind_of(p):
    if p["balanced"]:
        return "balanced"
    return "one" if p["launches"] == 1 and p["chunks"] == 1 else "chunked"


@pytest.mark.parametrize("B,H,D,S,flags,kind", [
    # <= 256 KiB of K+V per 256-byte head block: one chunk, any workgroup count
    (64, 32, 128, 128, PLAN_DEVICE_POS, "one"),
    (2, 8, 128, 512, PLAN_DEVICE_POS, "one"),
    (2, 8, 128, 512, PLAN_PAGED, "one"),
    (64, 16, 256, 128, PLAN_DEVICE_POS, "one"),
    # 512 KiB per workgroup: one chunk from 256 workgroups on (paged: more
    # than 256); with fewer, a cache of <= 128 MiB takes the chunked grid
    (8, 32, 128, 1024, PLAN_DEVICE_POS, "one"),
    (4, 32, 128, 1024, PLAN_DEVICE_POS, "chunked"),
    (8, 64, 64, 1024, PLAN_DEVICE_POS, "one"),
    (8, 64, 64, 1024, PLAN_PAGED, "chunked"),
    (300, 2, 64, 608, PLAN_PAGED, "one"),
    (16, 32, 128, 1024, PLAN_PAGED, "one"),
    # head_dim 256 past 256 KiB: 268 MB of K+V, the balanced grid
    (64, 8, 256, 512, PLAN_DEVICE_POS, "balanced"),
    # 1 MiB per workgroup: 537 MB, balanced
    (64, 8, 128, 2048, PLAN_DEVICE_POS, "balanced"),
    # caches of <= 128 MiB of K+V outside the one-chunk rules: chunked grid
    (16, 8, 128, 1024, PLAN_DEVICE_POS, "chunked"),
    (16, 16, 64, 2048, PLAN_PAGED, "chunked"),
    (4, 8, 128, 4096, PLAN_DEVICE_POS | PLAN_STEP, "chunked"),
    # 268 MB: balanced
    (32, 8, 128, 2048, PLAN_DEVICE_POS, "balanced"),
    (8, 8, 128, 8192, PLAN_PAGED, "balanced"),
])
def test_batch_plan_rules(B, H, D, S, flags, kind):
    p = plan(B, H, D, S, flags=flags)
    assert kind_of(p) == kind, p
    if kind == "chunked" and not flags & PLAN_STEP and B * H <= 512:
        assert 256 < p["workgroups"] <= 1024, p   # aimed at 512


def test_many_head_blocks_are_widened():
    """1024 x 32 heads x 32 positions: one head per workgroup would launch
    32768 workgroups; head blocks are doubled until at most 8192 remain."""
    p = plan(1024, 32, 128, 32, flags=PLAN_DEVICE_POS)
    assert (p["heads_per_workgroup"], p["workgroups"], p["launches"]) == (4, 8192, 1)


DP, PG, ST = PLAN_DEVICE_POS, PLAN_PAGED, PLAN_STEP


@pytest.mark.parametrize("args,unroll,waves", [
    # single sequences: the knobs' unroll, never bounded
    ((1, 64, 64, 131072, 131071, 0), 8, 8),
    ((1, 32, 128, 32768, 20000, 0), 2, 2),   # head_dim 128, 16 head blocks: bounded
    ((1, 12, 128, 32768, 32767, 0), 2, 8),   # six head blocks: unbounded
    ((1, 32, 128, 32768, 20000, ST), 2, 8),
    ((1, 4, 64, 128, 100, 0), 8, 8),
    ((1, 16, 128, 512, 511, 0), 2, 2),       # one chunk per head, head_dim 128: bounded
    ((1, 16, 128, 512, 511, ST), 2, 8),
    ((1, 32, 128, 32768, 20000, PLAN_FROM_SCORES), 2, 8),
    # layouts other than the 16-byte ones for head_dim 64 / 128 run U = 4
    ((1, 40, 100, 32768, 32767, 0), 4, 8),
    ((64, 32, 100, 8192, 0, DP), 4, 8),
    # balanced grid, dense, >= 16 sequences of >= 4 head blocks: U = 2 bounded,
    # decodes and steps; paged keeps U = 4 unbounded
    ((64, 32, 128, 8192, 0, DP), 2, 2),
    ((64, 32, 128, 8192, 0, DP | ST), 2, 2),
    ((64, 32, 128, 8192, 0, PG), 4, 8),
    ((64, 32, 128, 8192, 0, PG | ST), 4, 8),
    ((32, 32, 64, 16384, 0, DP), 2, 2),
    ((8, 32, 128, 32768, 0, DP), 4, 8),      # fewer than 16 sequences
    ((32, 16, 64, 16384, 0, DP), 4, 8),      # two head blocks (eight heads of 64)
    ((32, 16, 128, 16384, 0, DP), 2, 2),     # four head blocks (four heads of 128)
    ((32, 8, 128, 16384, 0, DP), 4, 8),      # two head blocks
    # one chunk per (sequence, head block), 128-256 workgroups: U = 8, bounded
    # for dense decodes whose capacity holds four blocks (128 positions each)
    ((8, 32, 128, 1024, 0, DP), 8, 2),
    ((4, 32, 128, 512, 0, DP), 8, 2),
    ((64, 4, 128, 256, 0, DP), 8, 8),        # two blocks
    ((4, 32, 128, 512, 0, PG), 8, 8),
    ((4, 32, 128, 512, 0, DP | ST), 8, 8),
    ((8, 32, 128, 1024, 0, PG), 2, 2),       # paged: the 512 KiB band needs > 256 workgroups
    # mid-size batches: U = 2, bounded for dense and paged decodes, not steps
    ((8, 8, 128, 4096, 0, DP), 2, 2),
    ((8, 8, 128, 4096, 0, PG), 2, 2),
    ((8, 8, 128, 4096, 0, DP | ST), 2, 8),
    # past 1024 sequences: U = 8, bounded for every call whose chunk holds four blocks
    ((1100, 8, 128, 4096, 0, DP), 8, 2),
    ((1100, 8, 128, 4096, 0, PG), 8, 2),
    ((1100, 8, 128, 2048, 0, DP | ST), 8, 2),
    ((1100, 8, 128, 2048, 0, PG | ST), 8, 2),
])
def test_unroll_and_wave_bound(args, unroll, waves):
    """Which split kernel each measured rule selects: positions per row group
    and block, and whether it is the instantiation compiled for at most two
    waves per SIMD."""
    p = plan(*args)
    assert (p["unroll"], p["max_waves"]) == (unroll, waves), p


def test_batches_past_the_balanced_limit_take_the_chunked_grid():
    for S in (24, 4200, 100000):
        p = plan(1100, 2, 16, S, flags=PLAN_DEVICE_POS)
        assert p["balanced"] == 0, (S, p)
        assert p["chunks"] * p["chunk"] >= S


def test_decode_steps_take_one_launch_with_one_chunk_per_head_block():
    """A decode step whose plan gives each head block one chunk merges the new
    token and appends its rows in the split launch; with several chunks it
    merges in a second launch."""
    one = [((1, 4, 64, 128, 100), PLAN_STEP), ((1, 4, 64, 128, 0), PLAN_STEP),
           ((64, 32, 128, 128, 0), PLAN_STEP | PLAN_DEVICE_POS),
           ((1024, 32, 128, 32, 0), PLAN_STEP | PLAN_DEVICE_POS),
           ((300, 8, 64, 608, 0), PLAN_STEP | PLAN_PAGED), ((2, 8, 64, 64, 0), PLAN_STEP | PLAN_PAGED)]
    for args, flags in one:
        p = plan(*args, flags=flags)
        assert p["chunks"] == 1 and p["launches"] == 1 and p["partial_slots"] == 0, (args, p)
    two = [((1, 32, 128, 32768, 20000), PLAN_STEP), ((64, 32, 128, 8192, 0), PLAN_STEP | PLAN_DEVICE_POS),
           ((64, 32, 128, 8192, 0), PLAN_STEP | PLAN_PAGED), ((4, 8, 128, 4096, 0), PLAN_STEP | PLAN_DEVICE_POS)]
    for args, flags in two:
        p = plan(*args, flags=flags)
        assert p["launches"] == 2, (args, p)


def test_a_batch_with_one_host_position_is_the_split_pair():
    """flags 0 with batch > 1 exists only as attn_decode_f16_split + combine:
    two launches, partial states written, even when one chunk covers it."""
    p1 = plan(1, 4, 64, 128, 100)
    p3 = plan(3, 4, 64, 128, 100)
    assert p1["launches"] == 1 and p1["partial_slots"] == 0
    assert p3["launches"] == 2 and p3["chunks"] == 1
    # one partial per (sequence, head) at least, every one with its slot
    assert 3 * 4 <= p3["partial_slots"] <= p3["workspace_slots"]


def span_of(S, cp, flags):
    if flags & (PLAN_DEVICE_POS | PLAN_PAGED):
        return S
    L = min(cp, S - 1) + 1 - (1 if flags & PLAN_STEP else 0)
    return max(L, 1)


FLAG_SETS = [0, PLAN_STEP, PLAN_FROM_SCORES, PLAN_DEVICE_POS, PLAN_PAGED, PLAN_DEVICE_POS | PLAN_STEP,
             PLAN_PAGED | PLAN_STEP]


def test_partial_states_fit_the_workspace():
    rng = np.random.default_rng(4242)
    dims = [1, 2, 3, 7, 8, 16, 24, 40, 48, 64, 72, 80, 96, 100, 112, 128, 136, 192, 250, 256]
    n = 0
    for _ in range(4000):
        flags = int(rng.choice(FLAG_SETS))
        D = int(rng.choice(dims))
        H = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16, 32, 40, 64, 128]))
        S = int(np.exp(rng.uniform(0, np.log(1 << 21))))
        S = max(S, 2 if flags == PLAN_STEP else 1)
        single = not flags & (PLAN_DEVICE_POS | PLAN_PAGED)
        B = 1 if flags & PLAN_FROM_SCORES else int(rng.choice([1, 2, 5, 64, 300, 1024, 1025, 4096]))
        if single and flags & PLAN_STEP:
            B = 1
        cp = int(rng.integers(0, S - 1 if flags == PLAN_STEP else S + 3)) if S > 1 else 0
        p = plan(B, H, D, S, cp, flags)
        what = (B, H, D, S, cp, flags, p)
        hpb = p["heads_per_workgroup"]
        assert hpb >= 1 and hpb & (hpb - 1) == 0 and H % hpb == 0, what
        assert p["workgroups"] >= 1, what
        assert p["launches"] in (1, 2), what
        assert p["partial_slots"] <= p["workspace_slots"], what
        need = 256 + p["workspace_slots"] * (D + 2) * 4
        assert ad.workspace_bytes(B, H, D, S) >= need, what
        if p["balanced"]:
            assert p["chunk"] == 0 and p["chunks"] == 0 and p["launches"] == 2, what
        else:
            assert p["chunk"] % 16 == 0 and p["chunks"] >= 1, what
            assert p["chunks"] * p["chunk"] >= span_of(S, cp, flags), what
            assert (p["chunks"] - 1) * p["chunk"] < span_of(S, cp, flags), what
            assert p["workgroups"] == (H // hpb) * p["chunks"] * B, what
        if p["launches"] == 1:
            assert not p["balanced"] and p["chunks"] == 1 and p["partial_slots"] == 0, what
        elif not p["balanced"] and p["chunks"] == 1 and (B == 1 or not single):
            assert False, ("one chunk per head block in two launches", what)
        # the kernel: U in {2, 4, 8}, U = 4 off the 16-byte layouts of head_dim
        # 64 and 128; the two-wave instantiation only at U = 2 or 8, never for
        # softmax.V from stored scores, and on the balanced grid only for dense
        # calls at U = 2
        assert p["unroll"] in (2, 4, 8) and p["max_waves"] in (2, 8), what
        if D not in (64, 128):
            assert (p["unroll"], p["max_waves"]) == (4, 8), what
        if p["max_waves"] == 2:
            assert p["unroll"] in (2, 8) and not flags & PLAN_FROM_SCORES, what
            if p["balanced"]:
                assert p["unroll"] == 2 and not flags & PLAN_PAGED, what
        n += 1
    assert n == 4000


def test_plan_errors():
    lib = ad.load_library()
    info = ad.PlanInfo()
    assert lib.attn_decode_plan(1, 4, 64, 128, 0, 0, None) == ATTN_ERR_NULL
    for args in [(0, 4, 64, 128, 0, 0), (1, 4, 257, 128, 0, 0), (1, 4, 64, 0, 0, 0),
                 (1, 4, 64, 128, 0, 16), (2, 4, 64, 128, 0, PLAN_FROM_SCORES),
                 (1, 4, 64, 128, 0, PLAN_FROM_SCORES | PLAN_DEVICE_POS),
                 (1, 4, 64, 128, 128, PLAN_STEP)]:
        assert lib.attn_decode_plan(*args, ctypes.byref(info)) == ATTN_ERR_DIM, args
        assert lib.attn_last_error()
    with pytest.raises(ad.AttnError):
        ad.plan(1, 4, 64, 128, 128, PLAN_STEP)
