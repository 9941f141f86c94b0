"""GPU path against the CPU oracle, through the C-ABI library.

Bar (single-query decode attention, fp16 output): for every element
    |gpu - oracle| <= 2e-3 + 4e-3 * |oracle|
and for the fp32 score dump
    |s_gpu - s_oracle| <= 1e-4 * max(|s_oracle|, sum_i |q_i k_i| / sqrt(D)),
with every position after current_pos exactly -inf (page "Developing Apple
Metal Kernels in Rust - A Deep Dive Through Attention", section "Testing").

Oracle inputs are generated on the host by the seeded generator; the GPU
inputs come from the same generator on the device (bit-identical, checked
in test_device_generator_matches_host).  The full-size cases also run on
normal draws made on the GPU (torch.randn), the oracle taking host copies.
"""
import os

import numpy as np
import pytest
import torch

import decode_attention_kv_seq_amd as ad
from decode_attention_kv_seq_amd import workloads as wl
import oracle
import oracle_pins

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
ATOL, RTOL = 2e-3, 4e-3
DUMP_RTOL = 1e-4


def assert_close(got_f16, ref, what=""):
    got = got_f16.detach().float().cpu().numpy().astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite output" % what
    err = np.abs(got - ref)
    bound = ATOL + RTOL * np.abs(ref)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), "%s: err %.3g > bound %.3g at %s (got %r ref %r)" % (
        what, err[worst], bound[worst], worst, got[worst], ref[worst])
    return float(err.max())


def assert_dump_close(dump, ref_scores, q, k, cp, what=""):
    """dump [H, S] fp32 (GPU); ref_scores [H, S]; q [H, D], k [S, H, D] host fp16."""
    d = dump.detach().cpu().numpy().astype(np.float64)
    H, S = ref_scores.shape
    L = min(cp, S - 1) + 1
    assert np.all(d[:, L:] == -np.inf), "%s: masked slots not -inf" % what
    D = q.shape[-1]
    qf = q.astype(np.float64).reshape(H, D)
    kf = k[:L].astype(np.float64)
    floor = np.einsum("hd,phd->hp", np.abs(qf), np.abs(kf)) / np.sqrt(D)
    ref = ref_scores[:, :L]
    err = np.abs(d[:, :L] - ref)
    bound = DUMP_RTOL * np.maximum(np.abs(ref), floor)
    assert np.all(err <= bound), "%s: dump err %.3g" % (what, (err - bound).max())


def to_dev(a):
    t = torch.from_numpy(np.ascontiguousarray(a)) if isinstance(a, np.ndarray) else a
    return t.to(DEV)


def run_single(q, k, v, cp, dump=False):
    """q [H,D], k/v [S,H,D] host fp16 numpy -> GPU output (and dump)."""
    r = ad.decode(to_dev(q), to_dev(k), to_dev(v), cp, dump=dump)
    torch.cuda.synchronize()
    return r


def randn16(rng, shape, sigma=1.0, mean=0.0):
    return (rng.standard_normal(shape) * sigma + mean).astype(np.float16)


# ------------------------------------------------------------ workloads


def test_device_generator_matches_host():
    for name in ("h32_d128_s32768_cp20000_garbage", "h64_d64_s131072_spikes"):
        w = wl.WORKLOADS[name]
        k, v = wl.make_kv(w, DEV)
        for h in (0, w.n_heads - 1):
            qs, ks, vs = wl.head_slice(w, 0, h, n_rows=w.seq_len)
            assert torch.equal(ks.view(w.seq_len, -1), k[0, :, h].cpu())
            assert torch.equal(vs.view(w.seq_len, -1), v[0, :, h].cpu())
            assert torch.equal(qs.view(-1), wl.make_q(w, DEV)[0, h].cpu())
        del k, v
        torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["h4_d64_s128_cp100", "h32_d128_s4096_full",
                                  "h32_d128_s32768_cp20000_garbage"])
def test_workload_full_parity(name):
    """Every output element and every score against the oracle."""
    w = wl.WORKLOADS[name]
    print("case", name, flush=True)
    q_h = wl.make_q(w)[0]
    k_h, v_h = wl.make_kv(w)
    ref, ref_s, _ = oracle.decode(q_h, k_h[0], v_h[0], w.cur_pos, want_scores=True, threads=8)
    q, k, v = q_h.to(DEV), k_h[0].to(DEV), v_h[0].to(DEV)
    out = ad.decode(q, k, v, w.cur_pos)
    out_d, dump = ad.decode(q, k, v, w.cur_pos, dump=True)
    torch.cuda.synchronize()
    assert_close(out, ref, name)
    assert torch.equal(out, out_d), "dump variant differs from the timed kernel"
    assert_dump_close(dump, ref_s, q_h.numpy(), k_h[0].numpy(), w.cur_pos, name)


def _inputs(w, source):
    """The workload's q, k, v on the GPU: the counter-based generator
    (bounded at +-3.46 sigma) or normal draws (torch.randn)."""
    if source == "generator":
        q = wl.make_q(w, DEV)
        k, v = wl.make_kv(w, DEV)
        return q, k, v
    return wl.make_normal(w, DEV)


@pytest.mark.parametrize("source", ["normal"])
@pytest.mark.parametrize("name", ["h4_d64_s128_cp100", "h32_d128_s4096_full",
                                  "h32_d128_s32768_cp20000_garbage"])
def test_workload_full_parity_normal(name, source):
    """The same, with normal inputs drawn on the GPU (the peaked softmax of
    q with sigma 2 and the garbage with sigma 10 have their normal tails);
    the oracle takes host copies of the device tensors."""
    w = wl.WORKLOADS[name]
    print("case", name, source, flush=True)
    q, k, v = _inputs(w, source)
    out = ad.decode(q[0], k[0], v[0], w.cur_pos)
    out_d, dump = ad.decode(q[0], k[0], v[0], w.cur_pos, dump=True)
    torch.cuda.synchronize()
    qh, kh, vh = q[0].cpu(), k[0].cpu(), v[0].cpu()
    ref, ref_s, _ = oracle.decode(qh, kh, vh, w.cur_pos, want_scores=True, threads=16)
    assert_close(out, ref, name)
    assert torch.equal(out, out_d), "dump variant differs from the timed kernel"
    assert_dump_close(dump, ref_s, qh.numpy(), kh.numpy(), w.cur_pos, name)


def test_workload_peaked_query_full():
    """The seq-32768 cache with q of sigma 4 instead of 2 (the more peaked
    reading of its query distribution): scores of sigma about 4, so a few
    positions carry most of each head's weight; every output element and
    every dumped score against the oracle, normal inputs."""
    w = wl.WORKLOADS["h32_d128_s32768_cp20000_garbage"]
    q, k, v = wl.make_normal(w, DEV)
    q = (q.float() * 2.0).half()
    out = ad.decode(q[0], k[0], v[0], w.cur_pos)
    out_d, dump = ad.decode(q[0], k[0], v[0], w.cur_pos, dump=True)
    torch.cuda.synchronize()
    qh, kh, vh = q[0].cpu(), k[0].cpu(), v[0].cpu()
    ref, ref_s, _ = oracle.decode(qh, kh, vh, w.cur_pos, want_scores=True, threads=16)
    assert_close(out, ref, "q sigma 4")
    assert torch.equal(out, out_d), "dump variant differs from the timed kernel"
    assert_dump_close(dump, ref_s, qh.numpy(), kh.numpy(), w.cur_pos, "q sigma 4")


@pytest.mark.parametrize("source", ["generator", "normal"])
def test_workload_ragged_batch_full(source):
    """64 sequences x 32 heads, capacity 8192 (the full-size launch the bench
    times): every output element of every (sequence, head) and every dumped
    score against the oracle, on host copies of the device caches; every
    sequence's masked dump slots exactly -inf."""
    w = wl.WORKLOADS["b64_h32_d128_cap8192_ragged"]
    print("case", w.name, source, flush=True)
    q, k, v = _inputs(w, source)
    cp = w.positions().to(torch.int32).to(DEV)
    out = ad.decode_batched(q, k, v, cp)
    out_d, dump = ad.decode_batched(q, k, v, cp, dump=True)
    torch.cuda.synchronize()
    assert torch.equal(out, out_d)
    pos = w.positions()
    qh, kh, vh = q.cpu(), k.cpu(), v.cpu()
    del k, v
    ref, ref_s = oracle.decode_batched(qh, kh, vh, pos, want_scores=True, threads=16)
    assert_close(out, ref, "ragged batch")
    dump_h = dump.cpu()
    for b in range(w.batch):
        L = w.valid_len(b)
        assert_dump_close(dump_h[b], ref_s[b], qh[b].numpy(), kh[b].numpy(), L - 1, "b=%d" % b)


@pytest.mark.parametrize("source", ["generator", "normal"])
def test_workload_long_context_full(source):
    """seq_len 131072, 64 heads, 1% of K rows x8 (the bench's workload):
    every output element and every dumped score of all 64 heads against the
    oracle, on host copies of the device caches."""
    w = wl.WORKLOADS["h64_d64_s131072_spikes"]
    print("case", w.name, source, flush=True)
    q, k, v = _inputs(w, source)
    out = ad.decode(q[0], k[0], v[0], w.cur_pos)
    out_d, dump = ad.decode(q[0], k[0], v[0], w.cur_pos, dump=True)
    torch.cuda.synchronize()
    assert torch.equal(out, out_d)
    qh, kh, vh = q[0].cpu(), k[0].cpu(), v[0].cpu()
    del k, v
    ref, ref_s, _ = oracle.decode(qh, kh, vh, w.cur_pos, want_scores=True, threads=16)
    assert_close(out, ref, "131072 positions")
    assert_dump_close(dump, ref_s, qh.numpy(), kh.numpy(), w.cur_pos, "131072 positions")


@pytest.mark.parametrize("H,D,S,cp", [(40, 128, 32768, 32767), (20, 128, 65536, 40000),
                                      (96, 128, 4096, 4095), (40, 192, 8192, 8191), (12, 64, 65536, 65535)])
def test_head_counts_off_a_power_of_two(H, D, S, cp):
    """Single sequences with head counts that are not powers of two (the
    chunk count planned from the workgroup target rounds down for two
    workgroups per CU, up for four): every output element and every dumped
    score against the oracle, normal inputs."""
    print("case", H, D, S, cp, flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(H * 1000 + D)
    q = torch.randn((H, D), generator=g, device=DEV).half()
    k = torch.randn((S, H, D), generator=g, device=DEV).half()
    v = torch.randn((S, H, D), generator=g, device=DEV).half()
    out = ad.decode(q, k, v, cp)
    out_d, dump = ad.decode(q, k, v, cp, dump=True)
    torch.cuda.synchronize()
    assert torch.equal(out, out_d)
    qh, kh, vh = q.cpu(), k.cpu(), v.cpu()
    ref, ref_s, _ = oracle.decode(qh, kh, vh, cp, want_scores=True, threads=16)
    assert_close(out, ref, "H=%d D=%d" % (H, D))
    assert_dump_close(dump, ref_s, qh.numpy(), kh.numpy(), cp, "H=%d D=%d" % (H, D))


def test_paged_table_check_counts_entries_past_the_pool():
    """attn_paged_table_check counts the entries a paged call reads (blocks
    up to each sequence's current_pos, clamped to the capacity) that name
    no page of the pool, and names the first sequence holding one; entries
    past current_pos do not count.  Expected values from the table itself."""
    B, P, MB, NB = 5, 16, 8, 40
    rng = np.random.default_rng(31)
    table = rng.integers(0, NB, (B, MB)).astype(np.int64)
    cp = np.array([0, 16, 127, 130, 50])     # blocks read: 1, 2, 8, 8 (clamped), 4
    n_read = np.minimum(cp, P * MB - 1) // P + 1
    res = ad.paged_table_check(to_dev(table.astype(np.int32)), to_dev(cp.astype(np.int32)), P, NB)
    torch.cuda.synchronize()
    assert res.cpu().tolist() == [0, -1]
    bad = table.copy()
    bad[1, 1] = NB              # read (block 1 <= 16 // 16)
    bad[1, 2] = NB + 7          # not read
    bad[3, 7] = 2 ** 31 - 1     # read: position 130 clamps to 127
    bad[4, 3] = NB              # read
    bad[4, 4] = NB              # not read
    bad[0, 1] = NB              # not read (sequence 0 reads block 0 only)
    expect = sum(int(bad[b, j] >= NB) for b in range(B) for j in range(n_read[b]))
    res = ad.paged_table_check(to_dev(bad.astype(np.int32)), to_dev(cp.astype(np.int32)), P, NB)
    torch.cuda.synchronize()
    assert expect == 3
    assert res.cpu().tolist() == [3, 1]


def test_long_context_values_near_one_relative():
    """The 131072-position shape with V ~ N(1, 1), so outputs are mostly of
    size 1 and the bar 1e-3 |ref| + 1e-4 (tighter than the 2e-3 floor of the
    general bar) holds them to about two fp16 steps of the exact value.  (A
    head whose softmax one x8 spike row dominates returns about that row's
    V, which can be near 0: there the 1e-4 floor applies.)"""
    w = wl.WORKLOADS["h64_d64_s131072_spikes"]
    q, k, _ = wl.make_normal(w, DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(77)
    v = (torch.randn(w.kv_shape, generator=g, device=DEV) + 1.0).half()
    out = ad.decode(q[0], k[0], v[0], w.cur_pos)
    torch.cuda.synchronize()
    ref, _, _ = oracle.decode(q[0].cpu(), k[0].cpu(), v[0].cpu(), w.cur_pos, threads=16)
    got = out.float().cpu().numpy()
    err = np.abs(got - ref)
    assert np.all(err <= 1e-3 * np.abs(ref) + 1e-4), float((err - 1e-3 * np.abs(ref)).max())
    assert float(np.median(np.abs(ref))) > 0.5


# ------------------------------------------------------------ page cases


@pytest.mark.parametrize("case", oracle_pins.page_cases()["cases"], ids=lambda c: c["name"])
def test_page_cases(case):
    H, D, S, cp = case["n_heads"], case["head_dim"], case["seq_len"], case["current_pos"]
    q = oracle_pins._page_fill(H * D).reshape(H, D)
    k = oracle_pins._page_fill(S * H * D).reshape(S, H, D)
    v = k[::-1].copy()
    ref, ref_s, _ = oracle.decode(q, k, v, cp, want_scores=True)
    out, dump = run_single(q, k, v, cp, dump=True)
    assert_close(out, ref, case["name"])
    assert_dump_close(dump, ref_s, q, k, cp, case["name"])
    assert float((dump[:, : cp + 1].cpu().double() - torch.from_numpy(ref_s[:, : cp + 1])).abs().max()) < 0.5


# ------------------------------------------------------------ shapes


SHAPES = [  # (S, H, D, cp)
    (1, 1, 64, 0), (2, 3, 128, 1), (65, 2, 64, 64), (129, 32, 128, 128), (1000, 8, 128, 999),
    (4097, 32, 128, 4096), (5000, 4, 64, 3333), (300, 7, 48, 299), (77, 5, 1, 76), (90, 3, 7, 50),
    (200, 2, 8, 199), (150, 4, 16, 149), (123, 6, 40, 100), (64, 2, 72, 63), (500, 3, 96, 499),
    (100, 2, 100, 99), (70, 2, 130, 69), (60, 3, 200, 59), (50, 2, 250, 49), (40, 2, 255, 39),
    (333, 9, 256, 332), (2049, 1, 128, 2048), (20000, 2, 64, 19999), (70000, 1, 32, 69999),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "S%d_H%d_D%d_cp%d" % s)
def test_shapes_parity(shape):
    S, H, D, cp = shape
    rng = np.random.default_rng(S * 131 + H * 7 + D)
    q = randn16(rng, (H, D), 2.0)
    k = randn16(rng, (S, H, D))
    v = randn16(rng, (S, H, D))
    ref, ref_s, _ = oracle.decode(q, k, v, cp, want_scores=True, threads=4)
    out, dump = run_single(q, k, v, cp, dump=True)
    assert_close(out, ref, str(shape))
    assert_dump_close(dump, ref_s, q, k, cp, str(shape))


@pytest.mark.parametrize("offset", [1, 2, 4], ids=lambda o: "elem_offset%d" % o)
@pytest.mark.parametrize("D", [64, 128, 48])
def test_unaligned_tensors(offset, D):
    """Tensors starting 2, 4 or 8 bytes past an aligned address take the
    narrower-load paths; results still match the oracle."""
    S, H, cp = 700, 3, 650
    rng = np.random.default_rng(offset * 1000 + D)
    q = randn16(rng, (H, D))
    k = randn16(rng, (S, H, D))
    v = randn16(rng, (S, H, D))
    ref, _, _ = oracle.decode(q, k, v, cp)

    def shifted(a):
        buf = torch.zeros(a.size + 16, dtype=torch.float16, device=DEV)
        t = buf[offset:offset + a.size].view(a.shape)
        t.copy_(torch.from_numpy(a))
        return t

    qt, kt, vt = shifted(q), shifted(k), shifted(v)
    assert kt.data_ptr() % 16 != 0
    out = ad.decode(qt, kt, vt, cp)
    torch.cuda.synchronize()
    assert_close(out, ref, "offset %d" % offset)


# ------------------------------------------------------------ special cases


@pytest.mark.parametrize("D", [64, 128, 48, 7])
def test_first_position_only_is_exact(D):
    rng = np.random.default_rng(D)
    S, H = 50, 4
    q = randn16(rng, (H, D), 3.0)
    k = randn16(rng, (S, H, D), 3.0)
    v = randn16(rng, (S, H, D))
    out = run_single(q, k, v, 0)
    assert np.array_equal(out.cpu().numpy(), v[0])


@pytest.mark.parametrize("S", [100, 5000, 40000])
def test_values_all_one_give_one(S):
    rng = np.random.default_rng(S)
    H, D = 8, 128
    q = randn16(rng, (H, D), 2.0)
    k = randn16(rng, (S, H, D))
    v = np.ones((S, H, D), np.float16)
    out = run_single(q, k, v, S - 1)
    assert bool(torch.all(out == 1.0))


def test_values_near_one_relative():
    """V ~ N(1, 1): outputs near 1, where the 4e-3 relative term dominates."""
    rng = np.random.default_rng(5)
    S, H, D = 30000, 16, 64
    q = randn16(rng, (H, D))
    k = randn16(rng, (S, H, D))
    v = randn16(rng, (S, H, D), 1.0, 1.0)
    ref, _, _ = oracle.decode(q, k, v, S - 1, threads=8)
    out = run_single(q, k, v, S - 1)
    got = out.float().cpu().numpy()
    assert np.all(np.abs(got - ref) <= 1e-3 * np.abs(ref) + 1e-4)


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(6)
    S, H, D, cp = 3000, 4, 128, 2500
    q = randn16(rng, (H, D), 2.0)
    k = np.broadcast_to(randn16(rng, (1, H, D)), (S, H, D)).copy()
    v = randn16(rng, (S, H, D))
    out = run_single(q, k, v, cp)
    assert_close(out, v[: cp + 1].astype(np.float64).mean(axis=0), "mean of V")


def test_dominant_score_returns_its_row():
    rng = np.random.default_rng(7)
    S, H, D = 5000, 4, 64
    q = (3.0 * rng.choice([-1.0, 1.0], (H, D))).astype(np.float16)
    k = np.zeros((S, H, D), np.float16)
    stars = [0, 1234, 4000, 4999]
    for h, p in enumerate(stars):
        k[p, h] = q[h]
    v = randn16(rng, (S, H, D))
    out = run_single(q, k, v, S - 1).cpu().numpy()
    for h, p in enumerate(stars):
        assert np.array_equal(out[h], v[p, h]), h


@pytest.mark.parametrize("fill", [65504.0, np.inf, -np.inf, np.nan, "noise"])
def test_masked_garbage_leaves_output_bitwise_unchanged(fill):
    rng = np.random.default_rng(8)
    S, H, D, cp = 9000, 8, 128, 5000
    q = randn16(rng, (H, D))
    k = randn16(rng, (S, H, D))
    v = randn16(rng, (S, H, D))
    clean = run_single(q, k, v, cp)
    k2, v2 = k.copy(), v.copy()
    if fill == "noise":
        k2[cp + 1:] = randn16(rng, (S - cp - 1, H, D), 10.0)
        v2[cp + 1:] = randn16(rng, (S - cp - 1, H, D), 10.0)
    else:
        k2[cp + 1:] = fill
        v2[cp + 1:] = -np.float16(fill)
    out, dump = run_single(q, k2, v2, cp, dump=True)
    assert torch.equal(out, clean)
    assert bool(torch.all(torch.isfinite(dump[:, : cp + 1])))
    assert bool(torch.all(dump[:, cp + 1:] == -torch.inf))


@pytest.mark.parametrize("H", [1, 2, 4, 8, 16, 32, 64, 12])
def test_single_sequences_head_dim_128_head_counts(H):
    """Single sequences of head_dim 128 past the short-span plan: with a
    power-of-two number of head blocks, 256 workgroups in the instantiation
    compiled for two waves per SIMD; 12 heads (six blocks) keep the
    unbounded grid of two workgroups per CU.  Every output against the
    oracle, the dump against its scores, the dump variant's output bitwise
    equal to the timed kernel's."""
    S, D = 20000, 128
    cp = S - 1 - 7 * H
    p = ad.plan(1, H, D, S, cp, 0)
    bounded = H != 12
    assert p["max_waves"] == (2 if bounded else 8), p
    assert p["workgroups"] <= (256 if bounded else 512), p
    rng = np.random.default_rng(900 + H)
    q, k, v = randn16(rng, (H, D)), randn16(rng, (S, H, D)), randn16(rng, (S, H, D))
    out = run_single(q, k, v, cp)
    out_d, dump = run_single(q, k, v, cp, dump=True)
    assert torch.equal(out, out_d), "dump variant differs from the timed kernel"
    ref, ref_s, _ = oracle.decode(q, k, v, cp, want_scores=True, threads=8)
    assert_close(out, ref, "%d heads" % H)
    assert_dump_close(dump, ref_s, q, k, cp, "%d heads" % H)


def test_current_pos_beyond_cache_masks_nothing():
    rng = np.random.default_rng(9)
    S, H, D = 1500, 4, 128
    q, k, v = randn16(rng, (H, D)), randn16(rng, (S, H, D)), randn16(rng, (S, H, D))
    a = run_single(q, k, v, S - 1)
    for cp in (S, S + 100, 2 ** 32 - 1):
        assert torch.equal(run_single(q, k, v, cp), a)


def test_repeat_runs_are_bitwise_identical():
    rng = np.random.default_rng(10)
    S, H, D = 50000, 32, 128
    q, k, v = to_dev(randn16(rng, (H, D))), to_dev(randn16(rng, (S, H, D))), to_dev(randn16(rng, (S, H, D)))
    outs = [ad.decode(q, k, v, S - 1) for _ in range(5)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


# ------------------------------------------------------------ batched, phases, streams


def test_batched_matches_single_calls():
    rng = np.random.default_rng(11)
    B, S, H, D = 6, 3000, 8, 128
    q = randn16(rng, (B, H, D))
    k = randn16(rng, (B, S, H, D))
    v = randn16(rng, (B, S, H, D))
    pos = np.array([0, 63, 64, 1999, 2999, 10 ** 6], dtype=np.int64)
    cp = torch.from_numpy(np.minimum(pos, 2 ** 31 - 1).astype(np.int32)).to(DEV)
    out = ad.decode_batched(to_dev(q), to_dev(k), to_dev(v), cp)
    torch.cuda.synchronize()
    for b in range(B):
        ref, _, _ = oracle.decode(q[b], k[b], v[b], int(pos[b]))
        assert_close(out[b], ref, "b=%d" % b)
        single = run_single(q[b], k[b], v[b], int(pos[b]))
        assert_close(out[b], single.float().cpu().numpy(), "batched vs single b=%d" % b)


@pytest.mark.parametrize("S", [40, 600, 1100])
def test_many_short_sequences(S):
    """300 sequences of at most 45 positions.  Capacities of 40 and 600 take
    one chunk per sequence and head block (600: 300 KiB of K+V per workgroup,
    over 256 workgroups); one of 1100 the balanced grid, whose workgroups then
    walk many short pieces each."""
    rng = np.random.default_rng(12)
    B, H, D = 300, 2, 64
    q, k, v = randn16(rng, (B, H, D)), randn16(rng, (B, S, H, D)), randn16(rng, (B, S, H, D))
    pos = rng.integers(0, 45, B)
    cp = torch.from_numpy(pos.astype(np.int32)).to(DEV)
    out = ad.decode_batched(to_dev(q), to_dev(k), to_dev(v), cp)
    out_d, dump = ad.decode_batched(to_dev(q), to_dev(k), to_dev(v), cp, dump=True)
    torch.cuda.synchronize()
    assert torch.equal(out, out_d), "dump variant differs"
    ref, ref_s = oracle.decode_batched(q, k, v, pos, want_scores=True)
    assert_close(out, ref, "300 sequences")
    for b in (0, 1, 150, 299):
        assert_dump_close(dump[b], ref_s[b], q[b], k[b], int(pos[b]), "b=%d" % b)


@pytest.mark.parametrize("D", [64, 128])
def test_split_then_combine_matches_single_call(D):
    """The two-launch form (split kernel, then combine kernel) gives the
    single call's result bit for bit, and both match the oracle."""
    rng = np.random.default_rng(13)
    S, H, cp = 40000, 16, 33333
    qh, kh, vh = randn16(rng, (H, D)), randn16(rng, (S, H, D)), randn16(rng, (S, H, D))
    q, k, v = to_dev(qh), to_dev(kh), to_dev(vh)
    one = ad.decode(q, k, v, cp)
    ws = ad.alloc_workspace(1, H, D, S, DEV)
    out = torch.empty_like(one)
    ad.split(q, k, v, cp, ws)
    ad.combine(out, cp, 1, H, D, S, ws)
    torch.cuda.synchronize()
    ref, _, _ = oracle.decode(qh, kh, vh, cp, threads=8)
    assert_close(one, ref, "single call")
    assert_close(out, ref, "split + combine")
    assert torch.equal(one, out)


@pytest.mark.parametrize("S,H,D,cp", [(128, 4, 64, 100), (4096, 8, 128, 4095), (40000, 4, 64, 33333)],
                         ids=["tiny", "short", "long"])
def test_split_with_one_host_position_for_a_batch(S, H, D, cp):
    """attn_decode_f16_split with a batch and one host current_pos for all of
    it (the single-sequence plans, tiny, short and long, on a grid with a row
    per sequence), then the combine: each sequence against the oracle."""
    rng = np.random.default_rng(S + H)
    B = 3
    q, k, v = randn16(rng, (B, H, D), 2.0), randn16(rng, (B, S, H, D)), randn16(rng, (B, S, H, D))
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    ws = ad.alloc_workspace(B, H, D, S, DEV)
    out = torch.empty((B, H, D), dtype=torch.float16, device=DEV)
    ad.split(qd, kd, vd, cp, ws)
    ad.combine(out, cp, B, H, D, S, ws)
    torch.cuda.synchronize()
    for b in range(B):
        ref, _, _ = oracle.decode(q[b], k[b], v[b], cp)
        assert_close(out[b], ref, "b=%d" % b)


def test_workspace_reuse_across_sizes_and_repeats():
    """One workspace reused by 72 calls of changing sizes and positions: every
    output matches its first run bit for bit."""
    rng = np.random.default_rng(21)
    S, H, D = 30000, 32, 128
    k, v = to_dev(randn16(rng, (S, H, D))), to_dev(randn16(rng, (S, H, D)))
    q = to_dev(randn16(rng, (H, D)))
    ws = ad.alloc_workspace(4, H, D, S, DEV)
    cases = [20000, 29999, 777, 12345, 3]
    first = {}
    for rep in range(12):
        for cp in cases:
            out = ad.decode(q, k, v, cp, workspace=ws)
            if rep == 0:
                first[cp] = out.clone()
            else:
                assert torch.equal(out, first[cp]), (rep, cp)
        # a batched call of another shape on the same workspace
        kb = k[: 4 * 7000].view(4, 7000, H, D)
        vb = v[: 4 * 7000].view(4, 7000, H, D)
        qb = q.unsqueeze(0).expand(4, H, D).contiguous()
        cpb = torch.tensor([6999, 100, 5000, 0], dtype=torch.int32, device=DEV)
        ob = ad.decode_batched(qb, kb, vb, cpb, workspace=ws)
        torch.cuda.synchronize()
    ref, _, _ = oracle.decode(q.cpu(), k.cpu(), v.cpu(), 20000, threads=8)
    assert_close(first[20000], ref, "cp=20000")
    refb, _ = oracle.decode_batched(qb.cpu(), kb.cpu(), vb.cpu(), [6999, 100, 5000, 0], threads=8)
    assert_close(ob, refb, "batched on a shared workspace")


def test_side_stream():
    rng = np.random.default_rng(14)
    S, H, D = 8000, 8, 64
    q, k, v = to_dev(randn16(rng, (H, D))), to_dev(randn16(rng, (S, H, D))), to_dev(randn16(rng, (S, H, D)))
    ref = ad.decode(q, k, v, S - 1)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = ad.decode(q, k, v, S - 1)
    s.synchronize()
    assert torch.equal(out, ref)


def test_stream_argument_not_current():
    """stream= a side stream that is not the current one, while the current
    stream still has work queued: the wrappers' own allocations (workspace,
    out, dump) are recorded on the side stream, so the caching allocator
    does not hand their memory to the current stream's next allocations
    while the side stream's kernels still use it.  Every output equals the
    plain call's bitwise."""
    rng = np.random.default_rng(15)
    S, H, D = 30000, 16, 128
    q, k, v = to_dev(randn16(rng, (H, D))), to_dev(randn16(rng, (S, H, D))), to_dev(randn16(rng, (S, H, D)))
    ref = ad.decode(q, k, v, S - 1)
    ref_d = ad.decode(q, k, v, 20000, dump=True)
    x = torch.randn(4096, 4096, device=DEV)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for i in range(6):
        for _ in range(3):
            x = x @ x * 1e-3          # keeps the current stream busy
        outs.append(ad.decode(q, k, v, S - 1, stream=side))
        outs.append(ad.decode(q, k, v, 20000, dump=True, stream=side))
        # the current stream's allocations of the same sizes, written at once
        junk = [torch.full((ad.workspace_bytes(1, H, D, S),), 255, dtype=torch.uint8, device=DEV)
                for _ in range(2)]
        junk += [torch.full((H, D), -7.0, dtype=torch.float16, device=DEV),
                 torch.full((H, S), 3.0, dtype=torch.float32, device=DEV)]
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    for i in range(0, len(outs), 2):
        assert torch.equal(outs[i], ref), i
        assert torch.equal(outs[i + 1][0], ref_d[0]) and torch.equal(outs[i + 1][1], ref_d[1]), i


def test_binding_rejects_host_and_misshaped_buffers():
    """The library takes raw device pointers, so the binding refuses, before
    any launch, caller buffers that are on the host, of the wrong dtype or
    shape, or tensors of the wrong rank."""
    rng = np.random.default_rng(16)
    S, H, D = 300, 4, 64
    q, k, v = to_dev(randn16(rng, (H, D))), to_dev(randn16(rng, (S, H, D))), to_dev(randn16(rng, (S, H, D)))
    n = ad.workspace_bytes(1, H, D, S)
    host_ws = torch.empty(n, dtype=torch.uint8)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError, match="workspace"):
        ad.decode(q, k, v, S - 1, workspace=host_ws)
    with pytest.raises(ValueError, match="workspace"):
        ad.split(q, k, v, S - 1, host_ws)
    with pytest.raises(TypeError, match="dump"):
        ad.split(q, k, v, S - 1, ws, dump=torch.empty((1, H, S), dtype=torch.float16, device=DEV))
    with pytest.raises(ValueError, match="dump"):
        ad.split(q, k, v, S - 1, ws, dump=torch.empty((1, H, S - 1), dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError, match="workspace"):
        ad.combine(torch.empty((H, D), dtype=torch.float16, device=DEV), S - 1, 1, H, D, S, host_ws)
    with pytest.raises(ValueError, match="v must be"):
        ad.pv(torch.empty((H, S), dtype=torch.float16, device=DEV), v.unsqueeze(0), S - 1)
    with pytest.raises(ValueError, match="k must be"):
        ad.qk(q, k.unsqueeze(0), S - 1)
    x = torch.zeros((3, 5), dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError, match="workspace"):
        ad.softmax(x, workspace=torch.empty(ad.softmax_workspace_bytes(3, 5) + 1, dtype=torch.uint8))
    bt = torch.zeros((1, 2), dtype=torch.int32, device=DEV)
    cp = torch.zeros(1, dtype=torch.int32, device=DEV)
    pool = to_dev(randn16(rng, (2, 16, H, D)))
    with pytest.raises(ValueError, match="out must be"):
        ad.decode_paged(q.unsqueeze(0), pool, pool, bt, cp,
                        out=torch.empty((1, H, D + 1), dtype=torch.float16, device=DEV))
    torch.cuda.synchronize()


def test_workspace_errors_on_gpu():
    rng = np.random.default_rng(15)
    S, H, D = 1000, 4, 64
    q, k, v = to_dev(randn16(rng, (H, D))), to_dev(randn16(rng, (S, H, D))), to_dev(randn16(rng, (S, H, D)))
    small = torch.empty(64, dtype=torch.uint8, device=DEV)
    with pytest.raises(ad.AttnError) as e:
        ad.decode(q, k, v, S - 1, workspace=small)
    assert e.value.status == 4


@pytest.mark.parametrize("S,D", [(60000, 64), (30000, 128), (9000, 256)])
def test_combine_with_many_chunks(S, D):
    """One head and one sequence through the batched path: the workspace holds
    more chunk partials than the combine keeps in registers (its tiled loop)."""
    rng = np.random.default_rng(S + D)
    q = randn16(rng, (1, 1, D), 2.0)
    k = randn16(rng, (1, S, 1, D))
    v = randn16(rng, (1, S, 1, D))
    cp = torch.tensor([S - 3], dtype=torch.int32, device=DEV)
    out = ad.decode_batched(to_dev(q), to_dev(k), to_dev(v), cp)
    torch.cuda.synchronize()
    ref, _, _ = oracle.decode(q[0], k[0], v[0], S - 3)
    assert_close(out[0], ref, "S=%d D=%d" % (S, D))


@pytest.mark.parametrize("B,S,H,D,offset", [(64, 2048, 4, 100, 0), (40, 8192, 2, 72, 1), (48, 2048, 8, 48, 2),
                                             (48, 2048, 4, 136, 4), (24, 4096, 4, 250, 0)],
                         ids=["d100_8B", "d72_off2B", "d48_off4B", "d136_off8B", "d250_4B"])
def test_balanced_grid_with_narrow_loads(B, S, H, D, offset):
    """The balanced grid on the lane layouts below 16-byte loads: head_dims
    that are not multiples of 8 and tensors offset by 2, 4 or 8 bytes.  The
    caches (150-400 MB of K+V) are past the chunked plans, which the plan
    query confirms; every output against the oracle, and the score dump of
    four sequences."""
    assert ad.plan(B, H, D, S, 0, ad.PLAN_DEVICE_POS)["balanced"] == 1
    rng = np.random.default_rng(B * S + D)
    q, k, v = randn16(rng, (B, H, D), 2.0), randn16(rng, (B, S, H, D)), randn16(rng, (B, S, H, D))
    pos = rng.integers(0, S + 2, B)
    pos[::7] = 0
    cp = torch.from_numpy(pos.astype(np.int32)).to(DEV)

    def place(a):
        flat = torch.empty(a.size + offset, dtype=torch.float16, device=DEV)
        t = flat[offset:].view(a.shape)
        t.copy_(torch.from_numpy(a))
        return t

    out, dump = ad.decode_batched(place(q), place(k), place(v), cp, dump=True)
    torch.cuda.synchronize()
    ref, _ = oracle.decode_batched(q, k, v, pos, threads=8)
    assert_close(out, ref, "D=%d offset=%d" % (D, offset))
    for b in (0, 1, B // 2, B - 1):
        _, ref_s, _ = oracle.decode(q[b], k[b], v[b], int(pos[b]), want_scores=True)
        assert_dump_close(dump[b], ref_s, q[b], k[b], int(pos[b]), "b=%d" % b)


def test_batched_extreme_ragged_lengths():
    """One long sequence among many of length 1 and a few in between: the
    balanced grid splits the long one across many workgroups."""
    rng = np.random.default_rng(31)
    B, S, H, D = 40, 5000, 8, 128
    q, k, v = randn16(rng, (B, H, D), 2.0), randn16(rng, (B, S, H, D)), randn16(rng, (B, S, H, D))
    pos = np.zeros(B, dtype=np.int64)
    pos[3], pos[17], pos[39] = 4999, 2500, 63
    cp = torch.from_numpy(pos.astype(np.int32)).to(DEV)
    out, dump = ad.decode_batched(to_dev(q), to_dev(k), to_dev(v), cp, dump=True)
    torch.cuda.synchronize()
    ref, ref_s = oracle.decode_batched(q, k, v, pos, want_scores=True)
    assert_close(out, ref, "extreme ragged")
    for b in (0, 3, 17, 39):
        assert_dump_close(dump[b], ref_s[b], q[b], k[b], int(pos[b]), "b=%d" % b)


@pytest.mark.parametrize("S", [24, 4200])
def test_batched_more_sequences_than_balanced_grid_handles(S):
    """1100 short sequences: past the balanced grid's batch limit the chunked
    grid serves the call (a capacity of 24 with the short-capacity plan, one
    of 4200 with the plain chunked plan)."""
    rng = np.random.default_rng(32)
    B, H, D = 1100, 2, 16
    q, k, v = randn16(rng, (B, H, D)), randn16(rng, (B, S, H, D)), randn16(rng, (B, S, H, D))
    pos = rng.integers(0, 30, B)
    cp = torch.from_numpy(pos.astype(np.int32)).to(DEV)
    out = ad.decode_batched(to_dev(q), to_dev(k), to_dev(v), cp)
    torch.cuda.synchronize()
    ref, _ = oracle.decode_batched(q, k, v, pos)
    assert_close(out, ref, "1100 sequences")


def test_short_capacity_batch_with_many_head_blocks():
    """512 sequences x 32 heads of head_dim 128 with a 16-position capacity:
    one chunk per sequence and head block, and head blocks widened so that
    the launch stays within its workgroup budget.  Every output row against
    the oracle, with zero-length and past-capacity sequences among them."""
    rng = np.random.default_rng(33)
    B, S, H, D = 512, 16, 32, 128
    q, k, v = randn16(rng, (B, H, D), 2.0), randn16(rng, (B, S, H, D)), randn16(rng, (B, S, H, D))
    pos = rng.integers(0, S, B)
    pos[::5] = 0
    pos[1::9] = S + 100
    cp = torch.from_numpy(pos.astype(np.int32)).to(DEV)
    out = ad.decode_batched(to_dev(q), to_dev(k), to_dev(v), cp)
    torch.cuda.synchronize()
    ref, _ = oracle.decode_batched(q, k, v, pos, threads=8)
    assert_close(out, ref, "512 x 32 heads, capacity 16")


# ------------------------------------------------------------ paged cache


def page_dense_cache(k, v, page_size, rng, extra_pages=3):
    """Scatter dense [B, S, H, D] caches into a shuffled page pool.
    Returns k_pool, v_pool [NB, P, H, D] and the block table [B, S/P] (int32)."""
    B, S, H, D = k.shape
    mb = S // page_size
    nb = B * mb + extra_pages
    perm = rng.permutation(nb)[: B * mb].reshape(B, mb)
    kp = np.zeros((nb, page_size, H, D), np.float16)
    vp = np.zeros((nb, page_size, H, D), np.float16)
    for b in range(B):
        for j in range(mb):
            kp[perm[b, j]] = k[b, j * page_size:(j + 1) * page_size]
            vp[perm[b, j]] = v[b, j * page_size:(j + 1) * page_size]
    return kp, vp, perm.astype(np.int32)


@pytest.mark.parametrize("page_size", [1, 2, 16, 64, 512, 2048])
def test_paged_equals_dense_batched(page_size):
    """The same caches, dense or cut into shuffled pages: identical bits, and
    both match the oracle."""
    rng = np.random.default_rng(40 + page_size)
    B, S, H, D = 5, 2048, 8, 128
    q, k, v = randn16(rng, (B, H, D)), randn16(rng, (B, S, H, D)), randn16(rng, (B, S, H, D))
    pos = np.array([2047, 0, 1000, 15, 1536], dtype=np.int64)
    cp = torch.from_numpy(pos.astype(np.int32)).to(DEV)
    dense = ad.decode_batched(to_dev(q), to_dev(k), to_dev(v), cp)
    kp, vp, bt = page_dense_cache(k, v, page_size, rng)
    paged, dump = ad.decode_paged(to_dev(q), to_dev(kp), to_dev(vp), to_dev(bt), cp, dump=True)
    torch.cuda.synchronize()
    ref, ref_s = oracle.decode_batched(q, k, v, pos, want_scores=True)
    assert_close(paged, ref, "page %d" % page_size)
    assert torch.equal(paged, dense)
    for b in range(B):
        assert_dump_close(dump[b], ref_s[b], q[b], k[b], int(pos[b]), "page %d b=%d" % (page_size, b))


@pytest.mark.parametrize("B,S,H,D", [(64, 256, 4, 128), (16, 256, 16, 64), (8, 1024, 32, 128)],
                         ids=["b64_h4_d128", "b16_h16_d64", "b8_h32_d128_paged_two_launches"])
def test_one_chunk_batches_with_long_blocks(B, S, H, D):
    """One-chunk batches of 128-256 workgroups take 8 positions per block:
    dense and paged (shuffled 16-position pages) give the same bits where
    they take the same plan, the dump variant gives the timed kernel's bits,
    and every output matches the oracle."""
    print("case", B, S, H, D, flush=True)
    dense_plan = ad.plan(B, H, D, S, flags=ad.PLAN_DEVICE_POS)
    paged_plan = ad.plan(B, H, D, S, flags=ad.PLAN_PAGED)
    assert dense_plan["launches"] == 1 and 128 <= dense_plan["workgroups"] <= 256, dense_plan
    rng = np.random.default_rng(B * 100 + H)
    q, k, v = randn16(rng, (B, H, D)), randn16(rng, (B, S, H, D)), randn16(rng, (B, S, H, D))
    pos = rng.integers(0, S + 2, B)
    pos[0] = S - 1
    cp = torch.from_numpy(pos.astype(np.int32)).to(DEV)
    dense = ad.decode_batched(to_dev(q), to_dev(k), to_dev(v), cp)
    dense_d, _ = ad.decode_batched(to_dev(q), to_dev(k), to_dev(v), cp, dump=True)
    kp, vp, bt = page_dense_cache(k, v, 16, rng)
    paged = ad.decode_paged(to_dev(q), to_dev(kp), to_dev(vp), to_dev(bt), cp)
    torch.cuda.synchronize()
    ref, _ = oracle.decode_batched(q, k, v, pos, threads=8)
    assert_close(dense, ref, "dense")
    assert_close(paged, ref, "paged")
    assert torch.equal(dense, dense_d), "dump variant differs from the timed kernel"
    if all(paged_plan[f] == dense_plan[f] for f in ("launches", "workgroups", "unroll")):
        assert torch.equal(paged, dense)


@pytest.mark.parametrize("B,S,H,D", [(64, 2048, 4, 100), (24, 4096, 4, 250)], ids=["d100", "d250"])
def test_paged_balanced_grid_with_narrow_loads(B, S, H, D):
    """A paged pool (16-position pages, shuffled) on the balanced grid with
    head_dims that take 8- and 4-byte loads: every output against the
    oracle and bitwise equal to the dense call on the same values."""
    assert ad.plan(B, H, D, S, 0, ad.PLAN_PAGED)["balanced"] == 1
    rng = np.random.default_rng(S + D)
    q, k, v = randn16(rng, (B, H, D), 2.0), randn16(rng, (B, S, H, D)), randn16(rng, (B, S, H, D))
    pos = rng.integers(0, S + 2, B)
    cp = torch.from_numpy(pos.astype(np.int32)).to(DEV)
    kp, vp, bt = page_dense_cache(k, v, 16, rng)
    paged = ad.decode_paged(to_dev(q), to_dev(kp), to_dev(vp), to_dev(bt), cp)
    dense = ad.decode_batched(to_dev(q), to_dev(k), to_dev(v), cp)
    torch.cuda.synchronize()
    ref, _ = oracle.decode_batched(q, k, v, pos, threads=8)
    assert_close(paged, ref, "paged D=%d" % D)
    assert torch.equal(paged, dense)


@pytest.mark.parametrize("page_size", [1, 2, 64, 2048])
def test_paged_balanced_grid_page_sizes(page_size):
    """Page sizes from one position to 2048 on the balanced grid (24
    sequences x 4 heads x 8192 positions, 403 MB of K+V): bitwise equal to
    the same caches cut into 16-position pages and, since both stream the
    same block length here, to the dense call; both against the oracle on
    every sequence."""
    B, S, H, D = 24, 8192, 4, 128
    paged_plan = ad.plan(B, H, D, S, 0, ad.PLAN_PAGED)
    dense_plan = ad.plan(B, H, D, S, 0, ad.PLAN_DEVICE_POS)
    assert paged_plan["balanced"] == 1 and dense_plan["balanced"] == 1
    assert all(paged_plan[f] == dense_plan[f] for f in ("unroll", "heads_per_workgroup", "workgroups"))
    rng = np.random.default_rng(60 + page_size)
    q, k, v = randn16(rng, (B, H, D)), randn16(rng, (B, S, H, D)), randn16(rng, (B, S, H, D))
    pos = rng.integers(0, S + 2, B)
    pos[3] = 0
    cp = torch.from_numpy(pos.astype(np.int32)).to(DEV)
    kp, vp, bt = page_dense_cache(k, v, page_size, rng)
    paged = ad.decode_paged(to_dev(q), to_dev(kp), to_dev(vp), to_dev(bt), cp)
    kp16, vp16, bt16 = page_dense_cache(k, v, 16, rng)
    paged16 = ad.decode_paged(to_dev(q), to_dev(kp16), to_dev(vp16), to_dev(bt16), cp)
    dense = ad.decode_batched(to_dev(q), to_dev(k), to_dev(v), cp)
    torch.cuda.synchronize()
    assert torch.equal(paged, paged16)
    assert torch.equal(paged, dense)
    ref, _ = oracle.decode_batched(q, k, v, pos, threads=8)
    assert_close(paged, ref, "page %d" % page_size)
    assert_close(dense, ref, "dense")


def test_paged_workload_sampled():
    """64 ragged sequences in 16-position pages scattered through one pool:
    16 sampled (sequence, head) pairs against the oracle."""
    w = wl.WORKLOADS["b64_h32_d128_cap8192_ragged_paged16"]
    q = wl.make_q(w, DEV)
    kp, vp = wl.make_kv_paged(w, DEV)
    bt_h = w.block_table()
    bt = bt_h.to(torch.int32).to(DEV)
    pos = w.positions()
    cp = pos.to(torch.int32).to(DEV)
    out = ad.decode_paged(q, kp, vp, bt, cp)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    picks = [(int(b), int(rng.integers(0, w.n_heads))) for b in rng.choice(w.batch, 16, replace=False)]
    picks[0] = (int(torch.argmax(pos)), 5)
    for b, h in picks:
        qs, ks, vs = wl.head_slice_paged(w, b, h, bt_h)
        ref, _, _ = oracle.decode(qs[0], ks, vs, int(pos[b]))
        assert_close(out[b, h:h + 1], ref, "b=%d h=%d" % (b, h))


def test_paged_shared_pages_and_unused_table_entries():
    """Two sequences share their first pages (a common prefix); table entries
    past each sequence's last position hold 0xFFFFFFFF and are never used."""
    rng = np.random.default_rng(43)
    P, H, D, mb = 16, 4, 64, 64
    q = randn16(rng, (3, H, D))
    prefix_k, prefix_v = randn16(rng, (10 * P, H, D)), randn16(rng, (10 * P, H, D))
    k = randn16(rng, (3, mb * P, H, D))
    v = randn16(rng, (3, mb * P, H, D))
    k[0, :10 * P], v[0, :10 * P] = prefix_k, prefix_v
    k[1, :10 * P], v[1, :10 * P] = prefix_k, prefix_v
    kp, vp, bt = page_dense_cache(k, v, P, rng)
    bt[1, :10] = bt[0, :10]          # sequence 1 reads sequence 0's prefix pages
    pos = np.array([300, 10 * P + 40, 17], dtype=np.int64)
    for b in range(3):
        bt[b, pos[b] // P + 1:] = -1     # 0xFFFFFFFF as uint32
    cp = torch.from_numpy(pos.astype(np.int32)).to(DEV)
    out = ad.decode_paged(to_dev(q), to_dev(kp), to_dev(vp), to_dev(bt), cp)
    torch.cuda.synchronize()
    ref, _ = oracle.decode_batched(q, k, v, pos)
    assert_close(out, ref, "shared pages")


@pytest.mark.parametrize("S", [32, 600, 1104])
def test_paged_split_then_combine_and_many_sequences(S):
    """1030 sequences, past the balanced grid's batch limit: capacities of 32
    and 600 take the short-capacity plan, one of 1104 the plain chunked plan."""
    rng = np.random.default_rng(44)
    B, H, D, P = 1030, 2, 64, 8
    q, k, v = randn16(rng, (B, H, D)), randn16(rng, (B, S, H, D)), randn16(rng, (B, S, H, D))
    pos = rng.integers(0, 40, B)
    cp = torch.from_numpy(pos.astype(np.int32)).to(DEV)
    kp, vp, bt = page_dense_cache(k, v, P, rng)
    qd, kpd, vpd, btd = to_dev(q), to_dev(kp), to_dev(vp), to_dev(bt)
    one = ad.decode_paged(qd, kpd, vpd, btd, cp)
    ws = ad.alloc_workspace(B, H, D, S, DEV)
    two = torch.empty_like(one)
    ad.split_paged(qd, kpd, vpd, btd, cp, ws)
    ad.combine(two, cp, B, H, D, S, ws)
    torch.cuda.synchronize()
    assert torch.equal(one, two)
    ref, _ = oracle.decode_batched(q, k, v, pos)
    assert_close(one, ref, "1030 paged sequences")


@pytest.mark.parametrize("H,D", [(2, 128), (4, 64)], ids=["d128_two_heads", "d64_four_heads"])
def test_chunked_grid_long_ragged_sequences(H, D):
    """1030 sequences with a 1104-position capacity and ragged lengths up to
    the capacity: the chunked grid, one workgroup per sequence and head block
    (two heads of 128, four of 64) streaming eight positions per block, so
    most sequences end in a partial block.  Dense and paged caches (pages of
    16) give the same bits, the score dump matches the oracle's scores, the
    outputs the oracle."""
    rng = np.random.default_rng(47 + D)
    B, S, P = 1030, 1104, 16
    q = randn16(rng, (B, H, D))
    k, v = (rng.standard_normal((B, S, H, D), dtype=np.float32).astype(np.float16) for _ in range(2))
    pos = rng.integers(0, S, B)
    pos[:6] = [0, 1, 7, 8, S - 2, S - 1]
    cp = torch.from_numpy(pos.astype(np.int32)).to(DEV)
    assert ad.plan(B, H, D, S, flags=ad.PLAN_DEVICE_POS)["workgroups"] == B
    out, dump = ad.decode_batched(to_dev(q), to_dev(k), to_dev(v), cp, dump=True)
    kp, vp, bt = page_dense_cache(k, v, P, rng)
    paged = ad.decode_paged(to_dev(q), to_dev(kp), to_dev(vp), to_dev(bt), cp)
    torch.cuda.synchronize()
    assert torch.equal(out, paged), "paged differs from dense"
    ref, ref_s = oracle.decode_batched(q, k, v, pos, want_scores=True)
    assert_close(out, ref, "1030 long ragged sequences")
    for b in (0, 3, 4, 5, 500, B - 1):
        assert_dump_close(dump[b], ref_s[b], q[b], k[b], int(pos[b]), "b=%d" % b)


def test_wave_bound_changes_no_bits(tmp_path):
    """The split kernel compiled for at most two waves per SIMD gives the
    unbounded kernel's bits: every kind of plan that takes the bound (the
    balanced grid, one-chunk batches at U = 8, mid-size and chunked batches,
    dense, paged and steps) run here, and again in one child process with
    the bound switched off through the tuning variable."""
    import subprocess
    import sys
    import wave_cases as wc
    plans = wc.plans()
    assert all(p["max_waves"] == 2 for p in plans.values()), plans
    ref = wc.run_all(DEV)
    path = tmp_path / "unbounded.pt"
    env = dict(os.environ, ATTN_DECODE_TUNE="waves=8")
    print("child process with the bound off", flush=True)
    r = subprocess.run([sys.executable, wc.__file__, str(path)], env=env, capture_output=True,
                       text=True, timeout=240)
    assert r.returncode == 0, r.stdout + r.stderr
    seen = {ln.split()[0]: ln.split()[1:] for ln in r.stdout.splitlines() if ln.split()[0] in plans}
    for name, p in plans.items():
        assert seen[name] == [str(p["unroll"]), "8"], (name, seen[name])
    got = torch.load(path, weights_only=True)
    for name in ref:
        assert torch.equal(ref[name], got[name]), name


# ------------------------------------------------------------ two dispatches


def f16_ulp(x):
    """Spacing of fp16 values at |x| (subnormal spacing near zero)."""
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


@pytest.mark.parametrize("shape", [(64, 12, 64, 63), (64, 12, 64, 31), (35, 8, 48, 34),
                                   (5000, 8, 128, 3333), (700, 3, 7, 699), (2049, 4, 256, 100)],
                         ids=lambda s: "S%d_H%d_D%d_cp%d" % s)
def test_qk_scores_round_the_exact_score(shape):
    """First dispatch: every stored score is an fp16 neighbour of the exact
    scaled dot product, up to fp32 accumulation error (at most D * 2^-24 of
    sum_i |q_i k_i| / sqrt(D)); every masked one is exactly -inf."""
    S, H, D, cp = shape
    rng = np.random.default_rng(S + D)
    q, k = randn16(rng, (H, D), 2.0), randn16(rng, (S, H, D))
    _, s_ref, _ = oracle.decode(q, k, k, cp, want_scores=True)
    sc = ad.qk(to_dev(q), to_dev(k), cp)
    torch.cuda.synchronize()
    got = sc.cpu().numpy().astype(np.float64)
    L = min(cp, S - 1) + 1
    assert np.all(got[:, L:] == -np.inf)
    err = np.abs(got[:, :L] - s_ref[:, :L])
    cond = np.einsum("hd,phd->hp", np.abs(q.astype(np.float64)),
                     np.abs(k[:L].astype(np.float64))) / np.sqrt(D)
    assert np.all(err < f16_ulp(s_ref[:, :L]) + D * 2.0 ** -24 * cond), err.max()


@pytest.mark.parametrize("shape", [(64, 12, 64, 63), (5000, 8, 128, 4999), (300, 7, 48, 150),
                                   (20000, 2, 64, 19999), (90, 3, 7, 50)],
                         ids=lambda s: "S%d_H%d_D%d_cp%d" % s)
def test_pv_from_stored_scores(shape):
    """Second dispatch on seeded fp16 score rows (some -inf, with NaN V there)."""
    S, H, D, cp = shape
    rng = np.random.default_rng(S * 3 + D)
    sc = randn16(rng, (H, S), 2.0)
    v = randn16(rng, (S, H, D))
    holes = rng.choice(min(cp, S - 1) + 1, size=min(5, cp), replace=False)
    holes = holes[holes != 0]
    sc[:, holes] = -np.inf
    v[holes] = np.nan
    ref = oracle.pv_from_scores(sc, v, cp)
    out = ad.pv(to_dev(sc), to_dev(v), cp)
    torch.cuda.synchronize()
    assert_close(out, ref, str(shape))


@pytest.mark.parametrize("S,H,D,lo,hi", [(20000, 4, 64, 0, 12000), (20001, 8, 128, 3000, 19000),
                                         (5000, 3, 48, 0, 4990), (70000, 2, 64, 10, 65000)],
                         ids=lambda x: str(x))
def test_pv_with_long_masked_stretch(S, H, D, lo, hi):
    """Second dispatch on score rows that are -inf over [lo, hi), a stretch
    far longer than a chunk (a sliding-window mask, say), with NaN V there:
    chunks made only of -inf scores must weigh nothing."""
    rng = np.random.default_rng(S + lo + hi)
    sc = randn16(rng, (H, S), 2.0)
    sc[:, lo:hi] = -np.inf
    v = randn16(rng, (S, H, D))
    v[lo:hi] = np.nan
    ref = oracle.pv_from_scores(sc, v, S - 1)
    out = ad.pv(to_dev(sc), to_dev(v), S - 1)
    torch.cuda.synchronize()
    assert_close(out, ref, "masked [%d, %d) of %d" % (lo, hi, S))


def test_two_dispatches_against_fp16_score_reading():
    """QK then PV on the GPU equals softmax.V of the oracle's scores rounded to
    fp16 (the page's two-dispatch design stores fp16 scores), within the bar."""
    w = wl.WORKLOADS["h32_d128_s32768_cp20000_garbage"]
    q_h = wl.make_q(w)[0]
    k_h, v_h = wl.make_kv(w)
    k_h, v_h = k_h[0], v_h[0]
    _, s_ref, _ = oracle.decode(q_h, k_h, v_h, w.cur_pos, want_scores=True, threads=8)
    ref = oracle.pv_from_scores(s_ref.astype(np.float16), v_h, w.cur_pos)
    q, k, v = q_h.to(DEV), k_h.to(DEV), v_h.to(DEV)
    sc = ad.qk(q, k, w.cur_pos)
    out = ad.pv(sc, v, w.cur_pos)
    fused = ad.decode(q, k, v, w.cur_pos)
    torch.cuda.synchronize()
    assert_close(out, ref, "two dispatches")
    print("two dispatches vs one pass: max |diff| %.3g" % float((out.float() - fused.float()).abs().max()))


def test_batch_at_the_size_limit():
    """batch = 65535 (the largest the header allows), ragged lengths including
    the capacity bound; 40 sampled sequences against the oracle."""
    rng = np.random.default_rng(65535)
    B, S, H, D = 65535, 4, 1, 8
    q = randn16(rng, (B, H, D))
    k = randn16(rng, (B, S, H, D))
    v = randn16(rng, (B, S, H, D))
    cp = rng.integers(0, S + 2, B)
    out = ad.decode_batched(to_dev(q), to_dev(k), to_dev(v), to_dev(cp.astype(np.int32)))
    torch.cuda.synchronize()
    pick = np.concatenate([[0, B - 1], rng.choice(B, 38, replace=False)])
    ref, _ = oracle.decode_batched(q[pick], k[pick], v[pick], cp[pick])
    assert_close(out[torch.from_numpy(pick)], ref, "batch 65535")


# A cache row offset is (position * n_heads + head) * head_dim elements: the
# caches below put rows past element 2^31 and 2^32, where 32-bit offset
# arithmetic, signed or unsigned, would wrap.
BIG_S = (1 << 23) + 4096   # x 64 heads x head_dim 8: 4.3e9 elements per tensor


def test_cache_past_2_32_elements():
    """One cache of 8 Mi + 4096 positions x 64 heads x head_dim 8 (8 GiB per
    tensor), the newest position near the end, so the rows read run past
    element 2^32.  Four heads, the last among them, against the oracle:
    output and score dump."""
    w = wl.Workload("h64_d8_s8392704", n_heads=64, head_dim=8, seq_len=BIG_S,
                    cur_pos=BIG_S - 3, seed=9)
    assert (w.cur_pos * 64 + 63) * 8 > 1 << 32
    q = wl.make_q(w, DEV)[0]
    k, v = wl.make_kv(w, DEV)
    out, dump = ad.decode(q, k[0], v[0], w.cur_pos, dump=True)
    torch.cuda.synchronize()
    del k, v
    for h in (0, 31, 62, 63):
        qs, ks, vs = wl.head_slice(w, 0, h)
        ref, ref_s, _ = oracle.decode(qs[0], ks, vs, w.cur_pos, want_scores=True)
        assert_close(out[h:h + 1], ref, "h=%d" % h)
        assert_dump_close(dump[h:h + 1], ref_s, qs[0].numpy(), ks.numpy(), w.cur_pos, "h=%d" % h)
    del dump
    torch.cuda.empty_cache()


def test_two_dispatches_past_2_32_elements():
    """The page's two dispatches on the same 8 GiB-per-tensor cache: the
    scores pass reads K rows past element 2^32, softmax.V reads V rows there.
    Two heads: every stored score an fp16 neighbour of the oracle's, the
    output against softmax.V of the oracle's scores rounded to fp16."""
    w = wl.Workload("h64_d8_s8392704", n_heads=64, head_dim=8, seq_len=BIG_S,
                    cur_pos=BIG_S - 3, seed=9)
    q = wl.make_q(w, DEV)[0]
    k, v = wl.make_kv(w, DEV)
    sc = ad.qk(q, k[0], w.cur_pos)
    out = ad.pv(sc, v[0], w.cur_pos)
    torch.cuda.synchronize()
    del k, v
    for h in (0, 63):
        qh, kh, vh = wl.head_slice(w, 0, h)
        _, s_ref, _ = oracle.decode(qh[0], kh, vh, w.cur_pos, want_scores=True)
        L = w.cur_pos + 1
        got = sc[h].cpu().numpy().astype(np.float64)
        assert np.all(got[L:] == -np.inf)
        err = np.abs(got[:L] - s_ref[0, :L])
        cond = np.abs(kh[:, 0].numpy().astype(np.float64)) @ np.abs(qh[0, 0].numpy().astype(np.float64)) / np.sqrt(8.0)
        assert np.all(err < f16_ulp(s_ref[0, :L]) + 8 * 2.0 ** -24 * cond), h
        ref = oracle.pv_from_scores(s_ref.astype(np.float16), vh, w.cur_pos)
        assert_close(out[h:h + 1], ref, "two dispatches head %d" % h)
    del sc
    torch.cuda.empty_cache()


@pytest.mark.parametrize("page_size", [0, 256], ids=["dense", "paged256"])
def test_batch_past_2_32_elements(page_size):
    """Ten sequences of capacity 2^20 x 64 heads x head_dim 8 (5 x 2^30
    elements per cache tensor, dense or as a page pool): sequence 4 starts at
    element 2^31 and sequences 8 and 9 past 2^32 (in the pool, the pages are
    scattered through all of it).  Ragged lengths; two heads of sequences 4
    and 9 against the oracle."""
    w = wl.Workload("b10_h64_d8_cap1048576", n_heads=64, head_dim=8, seq_len=1 << 20,
                    cur_pos=None, seed=10, batch=10, page_size=page_size)
    q = wl.make_q(w, DEV)
    cp = w.positions().to(torch.int32).to(DEV)
    if page_size:
        kp, vp = wl.make_kv_paged(w, DEV)
        bt = w.block_table()
        out = ad.decode_paged(q, kp, vp, bt.to(torch.int32).to(DEV), cp)
        torch.cuda.synchronize()
        del kp, vp
    else:
        k, v = wl.make_kv(w, DEV)
        out = ad.decode_batched(q, k, v, cp)
        torch.cuda.synchronize()
        del k, v
    pos = w.positions()
    for b in (4, 9):
        for h in (1, 63):
            qs, ks, vs = wl.head_slice_paged(w, b, h, bt) if page_size else wl.head_slice(w, b, h)
            ref, _, _ = oracle.decode(qs[0], ks, vs, int(pos[b]))
            assert_close(out[b, h:h + 1], ref, "b=%d h=%d" % (b, h))
    torch.cuda.empty_cache()


def test_two_dispatches_full_size_sampled():
    """The page's two dispatches on the 131072-position cache (the bench's
    --path two_dispatch launch): every stored score of 4 sampled heads is an
    fp16 neighbour of the oracle's score, and the output of those heads
    matches softmax.V of the oracle's scores rounded to fp16."""
    w = wl.WORKLOADS["h64_d64_s131072_spikes"]
    q = wl.make_q(w, DEV)[0]
    k, v = wl.make_kv(w, DEV)
    sc = ad.qk(q, k[0], w.cur_pos)
    out = ad.pv(sc, v[0], w.cur_pos)
    torch.cuda.synchronize()
    for h in (0, 21, 42, 63):
        qh, kh, vh = wl.head_slice(w, 0, h)
        _, s_ref, _ = oracle.decode(qh[0], kh, vh, w.cur_pos, want_scores=True)
        got = sc[h].cpu().numpy().astype(np.float64)
        err = np.abs(got - s_ref[0])
        cond = np.abs(kh[:, 0].numpy().astype(np.float64)) @ np.abs(qh[0, 0].numpy().astype(np.float64)) / 8.0
        assert np.all(err < f16_ulp(s_ref[0]) + 64 * 2.0 ** -24 * cond), h
        ref = oracle.pv_from_scores(s_ref.astype(np.float16), vh, w.cur_pos)
        assert_close(out[h:h + 1], ref, "two dispatches head %d" % h)
    del k, v
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B,H", [(40, 8), (100, 8), (300, 8)], ids=["pairs320", "pairs800", "pairs2400"])
def test_combine_tiers(B, H):
    """The combine takes 1024 threads per (sequence, head) below 512 pairs,
    256 threads up to 2048, one wave per pair beyond: each tier against the
    oracle on a ragged batch (some sequences shorter than one chunk)."""
    rng = np.random.default_rng(B * H)
    S, D = 1536, 64
    q, k, v = randn16(rng, (B, H, D)), randn16(rng, (B, S, H, D)), randn16(rng, (B, S, H, D))
    pos = rng.integers(0, S, B)
    pos[::5] = rng.integers(0, 8, len(pos[::5]))
    out = ad.decode_batched(to_dev(q), to_dev(k), to_dev(v), to_dev(pos.astype(np.int32)))
    torch.cuda.synchronize()
    pick = np.concatenate([[0, B - 1], rng.choice(B, 14, replace=False)])
    ref, _ = oracle.decode_batched(q[pick], k[pick], v[pick], pos[pick])
    assert_close(out[torch.from_numpy(pick)], ref, "B=%d H=%d" % (B, H))
