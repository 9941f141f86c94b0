"""GPU decode step (rotate, append, attend) and the standalone rotation
against the CPU oracle, through the C-ABI library.

Rotation (page "Tutorial 16: Writing Custom Metal Kernels", section "5.
Example: Fused RoPE Kernel").  The kernel forms the angle and reduces it in
fp64, evaluates cos/sin in fp32 (error e_t below 2^-21) and rotates in fp32,
so before the fp16 store a rotated value is within
    E = (|a| + |b|) * 2^-20
of the exact rotation of its pair (a, b) (a 2x margin over e_t plus the two
fp32 roundings).  The stored fp16 value is then within half an fp16 step of
that, so the bar is
    |gpu - exact| <= E + 0.5 * ulp16(|exact| + E),
values past rope_dims bit-exact, and (a sanity check of the same fact) fp16
words differing from the oracle's own rounding in at most 1% of the rotated
values, by one step.

Attention output: the decode bar, |gpu - oracle| <= 2e-3 + 4e-3 |oracle|, with
the oracle attending with its own fp16 rounding of the rotated q and key.
Cache: the new token's value row bit-exact, its key row to the rotation bar,
every other row untouched.
"""
import numpy as np
import pytest
import torch

import decode_attention_kv_seq_amd as ad
from decode_attention_kv_seq_amd import workloads as wl
import oracle

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
ATOL, RTOL = 2e-3, 4e-3


def randn16(rng, shape, sigma=1.0):
    return (rng.standard_normal(shape) * sigma).astype(np.float16)


def f16_ulp(x):
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def pair_magnitude(x, dims, traditional):
    """|a| + |b| of the pair each element belongs to ([..., D] float64)."""
    ax = np.abs(np.asarray(x, np.float64))
    D = ax.shape[-1]
    idx = np.arange(D)
    if traditional:
        partner = np.where(idx < dims, idx ^ 1, idx)
    else:
        h = dims // 2
        partner = np.where(idx < h, idx + h, np.where(idx < dims, idx - h, idx))
    return ax + ax[..., partner]


def assert_rotation(got_bits, x, exact, oracle_bits, dims, traditional, what=""):
    """got_bits: uint16 [..., D] from the GPU; x: fp16 input; exact: fp64."""
    got = got_bits.view(np.float16).astype(np.float64)
    D = x.shape[-1]
    rot = np.arange(D) < dims
    assert np.array_equal(got_bits[..., ~rot], x.view(np.uint16)[..., ~rot]), \
        "%s: values past rope_dims changed" % what
    E = pair_magnitude(x, dims, traditional) * 2.0 ** -20
    bound = E + 0.5 * f16_ulp(np.abs(exact) + E)
    err = np.abs(got - exact)
    bad = (err > bound) & rot
    assert not bad.any(), "%s: rotation err %.3g > %.3g at %s" % (
        what, err[bad].max(), bound[bad][np.argmax(err[bad])], np.argwhere(bad)[0])
    diff = (got_bits != oracle_bits) & rot
    n_rot = max(int(rot.sum()) * (got_bits.size // D), 1)
    assert diff.sum() <= max(2, n_rot // 100), "%s: %d of %d fp16 words differ" % (
        what, int(diff.sum()), n_rot)
    if diff.any():
        # fp16 steps apart on the ordered line (+0 and -0 equal), against one
        # step of rounding, or the width of the bound in steps where it spans
        # more: a rotation that cancels (|exact| far below |a|+|b|) keeps the
        # fp32 rotation's error, which is of the inputs' size
        def ordered(bits):
            b = bits.astype(np.int64)
            return np.where(b & 0x8000, -(b & 0x7FFF), b)
        steps = np.abs(ordered(got_bits[diff]) - ordered(oracle_bits[diff]))
        allowed = np.maximum(1.0, np.ceil(bound / f16_ulp(np.abs(exact))))[diff]
        assert np.all(steps <= allowed), "%s: rounding differs by more steps than the bound spans" % what


def assert_close(got_f16, ref, what=""):
    got = got_f16.detach().float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    bound = ATOL + RTOL * np.abs(ref)
    assert np.all(np.isfinite(got)), "%s: non-finite output" % what
    assert np.all(err <= bound), "%s: err %.3g" % (what, (err - bound).max())


# ------------------------------------------------------------- rotation


@pytest.mark.parametrize("D,dims", [(64, 64), (128, 128), (128, 64), (80, 64), (6, 4), (256, 256)])
@pytest.mark.parametrize("traditional", [False, True])
@pytest.mark.parametrize("base", [10000.0, 500000.0])
def test_rope_matches_oracle(D, dims, traditional, base):
    rng = np.random.default_rng(D * 7 + dims + int(traditional))
    positions = np.array([0, 1, 7, 4095, 20000, 131071, 1 << 20, (1 << 31) - 1, (1 << 32) - 1],
                         dtype=np.uint32)
    B, H = positions.size, 5
    x = randn16(rng, (B, H, D), 2.0)
    print("rope D=%d dims=%d trad=%s base=%g" % (D, dims, traditional, base), flush=True)
    got = ad.rope(torch.from_numpy(x).to(DEV),
                  torch.from_numpy(positions.view(np.int32)).to(DEV),
                  rope_dims=dims, rope_base=base, traditional=traditional)
    torch.cuda.synchronize()
    exact = oracle.rope(x, positions[:, None].astype(np.int64), dims=dims, base=base,
                        traditional=traditional)
    assert_rotation(got.cpu().numpy().view(np.uint16), x, exact, oracle.double_to_half(exact),
                    dims, traditional, "D%d dims%d" % (D, dims))


def test_rope_position_zero_is_identity_bitwise():
    """Page test test_rope_position_zero_is_identity, on the GPU: exact."""
    rng = np.random.default_rng(3)
    x = randn16(rng, (4, 8, 128), 3.0)
    pos = torch.zeros(4, dtype=torch.int32, device=DEV)
    for trad in (False, True):
        got = ad.rope(torch.from_numpy(x).to(DEV), pos, traditional=trad)
        assert torch.equal(got.cpu(), torch.from_numpy(x))


# ------------------------------------------------------------ decode step


def run_step_single(q, kn, vn, kc, vc, cp, dims, trad=False, base=10000.0):
    """GPU step on copies of host arrays; returns (out, k_cache, v_cache) on the host."""
    kc_d, vc_d = torch.from_numpy(kc).to(DEV), torch.from_numpy(vc).to(DEV)
    out = ad.decode_step(torch.from_numpy(q).to(DEV), torch.from_numpy(kn).to(DEV),
                         torch.from_numpy(vn).to(DEV), kc_d, vc_d, cp, rope_dims=dims,
                         rope_base=base, traditional=trad)
    torch.cuda.synchronize()
    return out, kc_d.cpu().numpy(), vc_d.cpu().numpy()


def check_step(out, kc_gpu, vc_gpu, kc0, vc0, q, kn, vn, cp, dims, trad, base=10000.0,
               threads=8, what=""):
    """Oracle step on host copies; compare output, the appended rows and the rest."""
    kc_o, vc_o = kc0.view(np.uint16).copy(), vc0.view(np.uint16).copy()
    r = oracle.decode_step(q, kn, vn, kc_o, vc_o, cp, dims=dims, base=base, traditional=trad,
                           threads=threads)
    pos = r["pos"]
    assert_close(out, r["out"], what)
    assert np.array_equal(vc_gpu.view(np.uint16)[pos], vn.view(np.uint16)), "%s: v row" % what
    assert_rotation(kc_gpu.view(np.uint16)[pos], kn, r["k_rot"], r["k16"], dims, trad,
                    what + " k row")
    others = np.ones(kc0.shape[0], bool)
    others[pos] = False
    assert np.array_equal(kc_gpu.view(np.uint16)[others], kc0.view(np.uint16)[others])
    assert np.array_equal(vc_gpu.view(np.uint16)[others], vc0.view(np.uint16)[others])


@pytest.mark.parametrize("name", ["h4_d64_s128_cp100", "h32_d128_s4096_full",
                                  "h32_d128_s32768_cp20000_garbage"])
def test_step_workloads_full_parity(name):
    w = wl.WORKLOADS[name]
    print("case", name, flush=True)
    rng = np.random.default_rng(w.seed + 100)
    q = wl.make_q(w)[0].numpy()
    k, v = wl.make_kv(w)
    kc, vc = k[0].numpy(), v[0].numpy()
    kn, vn = randn16(rng, q.shape), randn16(rng, q.shape)
    cp = min(w.cur_pos, w.seq_len - 1)
    out, kg, vg = run_step_single(q, kn, vn, kc, vc, cp, w.head_dim)
    check_step(out, kg, vg, kc, vc, q, kn, vn, cp, w.head_dim, False, what=name)


STEP_SHAPES = [  # (S, H, D, cp, dims, traditional)
    (64, 12, 64, 63, 64, False), (64, 12, 64, 0, 64, True), (33, 4, 128, 17, 96, False),
    (1000, 8, 128, 999, 128, True), (300, 7, 48, 150, 48, False), (90, 3, 6, 50, 4, True),
    (257, 5, 7, 256, 6, False), (2049, 4, 256, 2000, 128, False), (40, 2, 80, 39, 64, True),
    (5000, 1, 64, 4321, 0, False),
]


@pytest.mark.parametrize("shape", STEP_SHAPES, ids=lambda s: "S%d_H%d_D%d_cp%d_r%d_t%d" % s)
def test_step_shapes(shape):
    S, H, D, cp, dims, trad = shape
    print("step shape", shape, flush=True)
    rng = np.random.default_rng(S * 31 + D)
    q, kn, vn = randn16(rng, (H, D), 1.5), randn16(rng, (H, D)), randn16(rng, (H, D))
    kc, vc = randn16(rng, (S, H, D)), randn16(rng, (S, H, D))
    out, kg, vg = run_step_single(q, kn, vn, kc, vc, cp, dims, trad)
    check_step(out, kg, vg, kc, vc, q, kn, vn, cp, dims, trad, what=str(shape))


@pytest.mark.parametrize("shape", [(8192, 40, 128, 8191), (32768, 24, 128, 30000)],
                         ids=lambda s: "S%d_H%d_D%d_cp%d" % s)
def test_step_head_counts_off_a_power_of_two(shape):
    """Head counts that are not powers of two, on the plans that keep the
    workgroup count within the target (two per CU)."""
    S, H, D, cp = shape
    print("step shape", shape, flush=True)
    rng = np.random.default_rng(S + H)
    q, kn, vn = randn16(rng, (H, D), 1.5), randn16(rng, (H, D)), randn16(rng, (H, D))
    kc, vc = randn16(rng, (S, H, D)), randn16(rng, (S, H, D))
    out, kg, vg = run_step_single(q, kn, vn, kc, vc, cp, D, False)
    check_step(out, kg, vg, kc, vc, q, kn, vn, cp, D, False, threads=16, what=str(shape))


def test_step_at_position_zero_returns_new_value_exactly():
    rng = np.random.default_rng(5)
    for D in (64, 128, 7):
        q, kn, vn = randn16(rng, (4, D)), randn16(rng, (4, D)), randn16(rng, (4, D))
        kc, vc = randn16(rng, (50, 4, D)), randn16(rng, (50, 4, D))
        out, kg, _ = run_step_single(q, kn, vn, kc, vc, 0, D - D % 2)
        assert np.array_equal(out.cpu().numpy().view(np.uint16), vn.view(np.uint16))
        assert np.array_equal(kg[0].view(np.uint16), kn.view(np.uint16))   # angle 0


def test_step_without_rotation_appends_the_rows_bitwise():
    """rope_dims = 0: the appended key is k_new itself."""
    rng = np.random.default_rng(6)
    q, kn, vn = randn16(rng, (8, 128)), randn16(rng, (8, 128)), randn16(rng, (8, 128))
    kc, vc = randn16(rng, (600, 8, 128)), randn16(rng, (600, 8, 128))
    out, kg, vg = run_step_single(q, kn, vn, kc, vc, 432, 0)
    assert np.array_equal(kg[432].view(np.uint16), kn.view(np.uint16))
    check_step(out, kg, vg, kc, vc, q, kn, vn, 432, 0, False, what="dims 0")


def test_step_agrees_with_rope_then_decode():
    """The step's output against the GPU's own two-stage route: the standalone
    rotation of q, then a plain decode over the cache the step appended to."""
    rng = np.random.default_rng(7)
    S, H, D, cp = 20000, 16, 128, 19000
    q, kn, vn = randn16(rng, (H, D)), randn16(rng, (H, D)), randn16(rng, (H, D))
    kc, vc = randn16(rng, (S, H, D)), randn16(rng, (S, H, D))
    kc_d, vc_d = torch.from_numpy(kc).to(DEV), torch.from_numpy(vc).to(DEV)
    qd = torch.from_numpy(q).to(DEV)
    out = ad.decode_step(qd, torch.from_numpy(kn).to(DEV), torch.from_numpy(vn).to(DEV), kc_d,
                         vc_d, cp)
    q_rot = ad.rope(qd[None], torch.full((1,), cp, dtype=torch.int32, device=DEV))[0]
    two_stage = ad.decode(q_rot, kc_d, vc_d, cp)
    torch.cuda.synchronize()
    d = (out.float() - two_stage.float()).abs().max().item()
    assert d <= 2e-3, d


def _offset_view(x_host, off):
    """A contiguous GPU copy of x_host that starts `off` fp16 elements into
    its own buffer (so not 16-byte aligned for odd `off`)."""
    flat = torch.from_numpy(np.ascontiguousarray(x_host)).reshape(-1)
    base = torch.zeros(flat.numel() + off, dtype=torch.float16, device=DEV)
    base[off:] = flat.to(DEV)
    return base[off:].view(x_host.shape)


@pytest.mark.parametrize("off", [1, 3])
@pytest.mark.parametrize("S,H,D,cp", [(120, 4, 64, 100), (5000, 8, 128, 4000), (300, 6, 48, 299)],
                         ids=["one_launch_d64", "two_launches_d128", "one_launch_d48"])
def test_step_unaligned_tensors(S, H, D, cp, off):
    """q, k_new, v_new and both caches offset by `off` elements (narrower
    loads): the step, in one launch or two, against the oracle, with the
    appended rows and every other row checked."""
    print("step unaligned", S, H, D, cp, off, flush=True)
    rng = np.random.default_rng(S + off)
    q, kn, vn = randn16(rng, (H, D)), randn16(rng, (H, D)), randn16(rng, (H, D))
    kc, vc = randn16(rng, (S, H, D)), randn16(rng, (S, H, D))
    kc_d, vc_d = _offset_view(kc, off), _offset_view(vc, off)
    out = ad.decode_step(_offset_view(q, off), _offset_view(kn, off), _offset_view(vn, off), kc_d, vc_d,
                         cp, rope_dims=D, traditional=bool(off & 2))
    torch.cuda.synchronize()
    check_step(out, kc_d.cpu().numpy(), vc_d.cpu().numpy(), kc, vc, q, kn, vn, cp, D, bool(off & 2),
               what="offset %d" % off)


def test_consecutive_steps_grow_the_cache():
    """Five steps in a row at positions 40..44 (the decode loop), each
    checked against the oracle run on its own copy of the cache."""
    rng = np.random.default_rng(8)
    S, H, D = 64, 6, 64
    kc, vc = randn16(rng, (S, H, D)), randn16(rng, (S, H, D))
    kc_d, vc_d = torch.from_numpy(kc).to(DEV), torch.from_numpy(vc).to(DEV)
    kc_o, vc_o = kc.view(np.uint16).copy(), vc.view(np.uint16).copy()
    for pos in range(40, 45):
        q, kn, vn = randn16(rng, (H, D)), randn16(rng, (H, D)), randn16(rng, (H, D))
        out = ad.decode_step(torch.from_numpy(q).to(DEV), torch.from_numpy(kn).to(DEV),
                             torch.from_numpy(vn).to(DEV), kc_d, vc_d, pos, traditional=True)
        torch.cuda.synchronize()
        r = oracle.decode_step(q, kn, vn, kc_o, vc_o, pos, dims=D, traditional=True)
        assert_close(out, r["out"], "step at %d" % pos)
    kg = kc_d.cpu().numpy().view(np.uint16)
    assert np.array_equal(vc_d.cpu().numpy().view(np.uint16), vc_o)
    assert np.abs(kg.astype(np.int64) - kc_o.astype(np.int64)).max() <= 1   # fp16 rounding steps


def batched_inputs(rng, B, S, H, D, cps):
    q, kn, vn = (randn16(rng, (B, H, D)) for _ in range(3))
    kc, vc = randn16(rng, (B, S, H, D)), randn16(rng, (B, S, H, D))
    return q, kn, vn, kc, vc, np.asarray(cps, dtype=np.int64)


def run_step_batched(q, kn, vn, kc, vc, cps, dims, trad=False):
    kc_d, vc_d = torch.from_numpy(kc).to(DEV), torch.from_numpy(vc).to(DEV)
    cp = torch.from_numpy(cps.astype(np.int32)).to(DEV)
    out = ad.decode_step(torch.from_numpy(q).to(DEV), torch.from_numpy(kn).to(DEV),
                         torch.from_numpy(vn).to(DEV), kc_d, vc_d, cp, rope_dims=dims,
                         traditional=trad)
    torch.cuda.synchronize()
    return out.cpu(), kc_d.cpu().numpy(), vc_d.cpu().numpy()


@pytest.mark.parametrize("D,dims,trad", [(128, 128, False), (64, 32, True), (48, 48, False)])
def test_step_batched_ragged(D, dims, trad):
    rng = np.random.default_rng(D + dims)
    B, S, H = 9, 2048, 8
    cps = [0, 1, 2047, 3000, 5, 1024, 77, 2046, 400]   # 3000: past the cache, slot 2047
    q, kn, vn, kc, vc, cps = batched_inputs(rng, B, S, H, D, cps)
    print("batched step D=%d dims=%d" % (D, dims), flush=True)
    out, kg, vg = run_step_batched(q, kn, vn, kc, vc, cps, dims, trad)
    for b in range(B):
        check_step(out[b], kg[b], vg[b], kc[b], vc[b], q[b], kn[b], vn[b], int(cps[b]), dims,
                   trad, what="sequence %d" % b)


@pytest.mark.parametrize("D,dims,trad", [(48, 48, False), (64, 32, True)])
def test_step_batched_on_the_balanced_grid(D, dims, trad):
    """The batched step with caches past the chunked plans (9 sequences x 8
    heads x 16384 positions, 226-302 MB of K+V: the balanced grid, as the
    plan query confirms), head_dim 48 taking 8-byte loads: every sequence
    against the oracle's step."""
    rng = np.random.default_rng(D + dims + 1)
    B, S, H = 9, 16384, 8
    assert ad.plan(B, H, D, S, 0, ad.PLAN_DEVICE_POS | ad.PLAN_STEP)["balanced"] == 1
    cps = [0, 1, 16383, 20000, 5, 8192, 77, 16382, 4000]
    q, kn, vn, kc, vc, cps = batched_inputs(rng, B, S, H, D, cps)
    out, kg, vg = run_step_batched(q, kn, vn, kc, vc, cps, dims, trad)
    for b in range(B):
        check_step(out[b], kg[b], vg[b], kc[b], vc[b], q[b], kn[b], vn[b], int(cps[b]), dims,
                   trad, what="sequence %d" % b)


def test_step_batched_every_sequence_at_position_zero():
    """No earlier positions anywhere: the split launch streams nothing."""
    rng = np.random.default_rng(9)
    q, kn, vn, kc, vc, cps = batched_inputs(rng, 5, 32, 4, 64, [0] * 5)
    out, kg, _ = run_step_batched(q, kn, vn, kc, vc, cps, 64)
    assert np.array_equal(out.numpy().view(np.uint16), vn.view(np.uint16))
    assert np.array_equal(kg[:, 0].view(np.uint16), kn.view(np.uint16))


@pytest.mark.parametrize("S,D", [(24, 64), (600, 64), (1100, 64), (1100, 128)])
def test_step_batched_more_sequences_than_balanced_grid_handles(S, D):
    """1030 sequences take the chunked grid with per-sequence lengths, some 0
    (capacities of 24 and 600: the short-capacity plan; 1100: the plain
    chunked one, eight positions per block)."""
    rng = np.random.default_rng(10)
    B, H = 1030, 2
    cps = rng.integers(0, S, B)
    cps[::7] = 0
    q, kn, vn, kc, vc, cps = batched_inputs(rng, B, S, H, D, cps)
    out, kg, vg = run_step_batched(q, kn, vn, kc, vc, cps, D)
    for b in list(range(0, B, 97)) + [B - 1, 7, 14]:
        check_step(out[b], kg[b], vg[b], kc[b], vc[b], q[b], kn[b], vn[b], int(cps[b]), D,
                   False, threads=1, what="sequence %d" % b)


def sampled_heads_step(w, heads, cp, trad=False):
    """Full-size single-sequence step on the GPU; the oracle on sampled heads."""
    rng = np.random.default_rng(w.seed + 200)
    q = wl.make_q(w)[0].numpy()
    kn, vn = randn16(rng, q.shape), randn16(rng, q.shape)
    kc_d, vc_d = wl.make_kv(w, DEV)
    kc_d, vc_d = kc_d[0], vc_d[0]
    out = ad.decode_step(torch.from_numpy(q).to(DEV), torch.from_numpy(kn).to(DEV),
                         torch.from_numpy(vn).to(DEV), kc_d, vc_d, cp, traditional=trad)
    torch.cuda.synchronize()
    out = out.cpu()
    for h in heads:
        # host inputs from the generator (rows 0..cp; the oracle writes row cp)
        _, kt, vt = wl.head_slice(w, 0, h, n_rows=cp + 1)
        kh = kt.numpy().view(np.uint16).copy()
        vh = vt.numpy().view(np.uint16).copy()
        new_k = kc_d[cp, h:h + 1].cpu().numpy().view(np.uint16)
        assert np.array_equal(vc_d[cp, h:h + 1].cpu().numpy().view(np.uint16),
                              vn[h:h + 1].view(np.uint16))
        r = oracle.decode_step(q[h:h + 1], kn[h:h + 1], vn[h:h + 1], kh, vh, cp, dims=w.head_dim,
                               traditional=trad)
        assert_close(out[h:h + 1], r["out"], "%s head %d" % (w.name, h))
        assert_rotation(new_k, kn[h:h + 1], r["k_rot"], r["k16"], w.head_dim, trad,
                        "%s head %d k row" % (w.name, h))
    del kc_d, vc_d
    torch.cuda.empty_cache()


def test_step_long_context_sampled():
    """131072 positions x 64 heads (the streaming workload at full size), the
    new token in the last slot: 4 sampled heads against the oracle."""
    w = wl.WORKLOADS["h64_d64_s131072_spikes"]
    sampled_heads_step(w, [0, 21, 42, 63], w.seq_len - 1)


def test_step_past_2_32_elements():
    """The step on a cache of 8 Mi + 4096 positions x 64 heads x head_dim 8
    (8 GiB per tensor): the rows read and the new token's appended rows lie
    past element 2^32."""
    S = (1 << 23) + 4096
    w = wl.Workload("h64_d8_s8392704", n_heads=64, head_dim=8, seq_len=S, cur_pos=S - 3, seed=9)
    assert w.cur_pos * 64 * 8 > 1 << 32
    sampled_heads_step(w, [0, 63], w.cur_pos)


def test_step_masked_garbage_sampled():
    w = wl.WORKLOADS["h32_d128_s32768_cp20000_garbage"]
    sampled_heads_step(w, [0, 31], w.cur_pos, trad=True)


# ------------------------------------------------------ paged decode step


def scatter_pages(kc, vc, page_size, rng, extra=3):
    """Dense [B, S, H, D] caches -> shuffled page pools and a block table."""
    B, S, H, D = kc.shape
    mb = S // page_size
    nb = B * mb + extra
    perm = rng.permutation(nb)[: B * mb].reshape(B, mb)
    kp = np.zeros((nb, page_size, H, D), np.float16)
    vp = np.zeros((nb, page_size, H, D), np.float16)
    for b in range(B):
        for j in range(mb):
            kp[perm[b, j]] = kc[b, j * page_size:(j + 1) * page_size]
            vp[perm[b, j]] = vc[b, j * page_size:(j + 1) * page_size]
    return kp, vp, perm.astype(np.int32)


@pytest.mark.parametrize("page_size", [1, 16, 256])
def test_paged_step_equals_dense_step(page_size):
    """The same caches dense or in shuffled pages: the paged step gives the
    dense step's output bits, writes the same rows into the right pages,
    leaves every other pool row alone, and matches the oracle."""
    rng = np.random.default_rng(300 + page_size)
    B, S, H, D = 6, 1024, 8, 128
    cps = [1023, 0, 500, 15, 16, 2000]      # 2000: past the capacity, slot 1023
    q, kn, vn, kc, vc, cps = batched_inputs(rng, B, S, H, D, cps)
    print("paged step, page %d" % page_size, flush=True)
    dense_out, dense_k, dense_v = run_step_batched(q, kn, vn, kc, vc, cps, D, True)
    kp, vp, bt = scatter_pages(kc, vc, page_size, rng)
    kp_d, vp_d = torch.from_numpy(kp).to(DEV), torch.from_numpy(vp).to(DEV)
    cp = torch.from_numpy(cps.astype(np.int32)).to(DEV)
    out = ad.decode_step_paged(torch.from_numpy(q).to(DEV), torch.from_numpy(kn).to(DEV),
                               torch.from_numpy(vn).to(DEV), kp_d, vp_d,
                               torch.from_numpy(bt).to(DEV), cp, traditional=True)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), dense_out)
    kp_g, vp_g = kp_d.cpu().numpy(), vp_d.cpu().numpy()
    want_k, want_v = kp.copy(), vp.copy()
    for b in range(B):
        pos = min(int(cps[b]), S - 1)
        page, r = bt[b, pos // page_size], pos % page_size
        want_k[page, r] = dense_k[b, pos]
        want_v[page, r] = dense_v[b, pos]
    assert np.array_equal(kp_g.view(np.uint16), want_k.view(np.uint16))
    assert np.array_equal(vp_g.view(np.uint16), want_v.view(np.uint16))
    for b in (0, 2, 5):
        check_step(out[b], dense_k[b], dense_v[b], kc[b], vc[b], q[b], kn[b], vn[b],
                   int(cps[b]), D, True, what="paged sequence %d" % b)


@pytest.mark.parametrize("D", [64, 128])
def test_paged_step_past_the_balanced_grid(D):
    """1030 sequences with a 1104-position capacity: the paged step takes the
    chunked grid like the dense step (eight positions per block, in the
    instantiation compiled for two waves per SIMD), gives the dense step's
    output bits, writes the new rows into the right pages and nothing else,
    and matches the oracle's step on sampled sequences."""
    rng = np.random.default_rng(310 + D)
    B, S, H, P = 1030, 1104, 2, 16
    cps = rng.integers(0, S, B)
    cps[:4] = [0, 1, S - 1, S + 5]
    dense_plan = ad.plan(B, H, D, S, 0, ad.PLAN_DEVICE_POS | ad.PLAN_STEP)
    paged_plan = ad.plan(B, H, D, S, 0, ad.PLAN_PAGED | ad.PLAN_STEP)
    assert dense_plan == paged_plan, (dense_plan, paged_plan)
    assert (dense_plan["unroll"], dense_plan["max_waves"]) == (8, 2), dense_plan
    q, kn, vn, kc, vc, cps = batched_inputs(rng, B, S, H, D, cps)
    print("paged step, 1030 sequences, D %d" % D, flush=True)
    dense_out, dense_k, dense_v = run_step_batched(q, kn, vn, kc, vc, cps, D, True)
    kp, vp, bt = scatter_pages(kc, vc, P, rng)
    kp_d, vp_d = torch.from_numpy(kp).to(DEV), torch.from_numpy(vp).to(DEV)
    cp = torch.from_numpy(cps.astype(np.int32)).to(DEV)
    out = ad.decode_step_paged(torch.from_numpy(q).to(DEV), torch.from_numpy(kn).to(DEV),
                               torch.from_numpy(vn).to(DEV), kp_d, vp_d,
                               torch.from_numpy(bt).to(DEV), cp, traditional=True)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), dense_out)
    kp_g, vp_g = kp_d.cpu().numpy(), vp_d.cpu().numpy()
    want_k, want_v = kp.copy(), vp.copy()
    for b in range(B):
        pos = min(int(cps[b]), S - 1)
        page, r = bt[b, pos // P], pos % P
        want_k[page, r] = dense_k[b, pos]
        want_v[page, r] = dense_v[b, pos]
    assert np.array_equal(kp_g.view(np.uint16), want_k.view(np.uint16))
    assert np.array_equal(vp_g.view(np.uint16), want_v.view(np.uint16))
    for b in (0, 1, 2, 3, 700):
        check_step(out[b], dense_k[b], dense_v[b], kc[b], vc[b], q[b], kn[b], vn[b],
                   int(cps[b]), D, True, threads=1, what="paged sequence %d" % b)


def test_paged_step_out_of_range_entry_writes_nothing():
    """A block-table entry past the pool for the new slot: no row is written
    (the output is unspecified but the call stays in bounds)."""
    rng = np.random.default_rng(77)
    B, S, H, D, P = 2, 64, 2, 64, 16
    q, kn, vn, kc, vc, cps = batched_inputs(rng, B, S, H, D, [40, 63])
    kp, vp, bt = scatter_pages(kc, vc, P, rng)
    bt[1, 63 // P] = kp.shape[0] + 5
    kp_d, vp_d = torch.from_numpy(kp).to(DEV), torch.from_numpy(vp).to(DEV)
    ad.decode_step_paged(torch.from_numpy(q).to(DEV), torch.from_numpy(kn).to(DEV),
                         torch.from_numpy(vn).to(DEV), kp_d, vp_d, torch.from_numpy(bt).to(DEV),
                         torch.from_numpy(cps.astype(np.int32)).to(DEV))
    torch.cuda.synchronize()
    kp_g = kp_d.cpu().numpy().view(np.uint16)
    changed = np.argwhere(np.any(kp_g != kp.view(np.uint16), axis=(2, 3)))
    assert changed.tolist() == [[bt[0, 40 // P], 40 % P]]


def _full_batch_step_sampled(name, pairs):
    """The decode step on a whole 64-sequence workload (the bench's --path
    step launch), (sequence, head) pairs against the oracle on host copies
    regenerated from the seeded generator."""
    w = wl.WORKLOADS[name]
    rng = np.random.default_rng(w.seed + 300)
    q = wl.make_q(w, DEV)
    kn = torch.from_numpy(randn16(rng, w.q_shape)).to(DEV)
    vn = torch.from_numpy(randn16(rng, w.q_shape)).to(DEV)
    cp = w.positions().to(torch.int32).to(DEV)
    if w.paged:
        kp, vp = wl.make_kv_paged(w, DEV)
        bt = w.block_table()
        out = ad.decode_step_paged(q, kn, vn, kp, vp, bt.to(torch.int32).to(DEV), cp)
    else:
        kc, vc = wl.make_kv(w, DEV)
        out = ad.decode_step(q, kn, vn, kc, vc, cp)
    torch.cuda.synchronize()
    pos_all = w.positions()
    for b, h in pairs:
        pos = min(int(pos_all[b]), w.seq_len - 1)
        if w.paged:
            qh, kh, vh = wl.head_slice_paged(w, b, h, bt)
            new_k = kp[bt[b, pos // w.page_size], pos % w.page_size, h].cpu().numpy()
        else:
            qh, kh, vh = wl.head_slice(w, b, h)
            new_k = kc[b, pos, h].cpu().numpy()
        kh = kh.numpy().view(np.uint16).copy()   # rows 0..pos; the oracle rewrites row pos
        vh = vh.numpy().view(np.uint16).copy()
        knh = kn[b, h:h + 1].cpu().numpy()
        vnh = vn[b, h:h + 1].cpu().numpy()
        r = oracle.decode_step(qh[0].numpy(), knh, vnh, kh, vh, pos, dims=w.head_dim)
        assert_close(out[b, h:h + 1], r["out"], "%s b=%d h=%d" % (name, b, h))
        assert_rotation(new_k.view(np.uint16)[None], knh, r["k_rot"], r["k16"], w.head_dim, False,
                        "%s b=%d h=%d k row" % (name, b, h))


def test_step_full_ragged_batch_sampled():
    w = wl.WORKLOADS["b64_h32_d128_cap8192_ragged"]
    lens = w.positions()
    longest, shortest = int(torch.argmax(lens)), int(torch.argmin(lens))
    _full_batch_step_sampled(w.name, [(0, 0), (longest, 31), (shortest, 5), (17, 12), (63, 30)])
    torch.cuda.empty_cache()


def test_step_full_paged_batch_sampled():
    w = wl.WORKLOADS["b64_h32_d128_cap8192_ragged_paged16"]
    lens = w.positions()
    longest, shortest = int(torch.argmax(lens)), int(torch.argmin(lens))
    _full_batch_step_sampled(w.name, [(1, 3), (longest, 0), (shortest, 31), (40, 17)])
    torch.cuda.empty_cache()
