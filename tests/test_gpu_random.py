"""Seeded random configurations through every entry point, against the
oracle: head_dim 1..256 (every lane layout), odd head counts, ragged and
out-of-range lengths, page sizes, rotation settings, unaligned tensors,
stored score rows with -inf stretches.
Each case prints its parameters before it runs.  Bars as in the other GPU
tests: |gpu - oracle| <= 2e-3 + 4e-3 |oracle| for fp16 outputs; the rotation
and softmax bars of test_gpu_decode_step.py and test_gpu_softmax.py."""
import numpy as np
import pytest
import torch

import decode_attention_kv_seq_amd as ad
import oracle
from test_gpu_decode_step import (assert_rotation, batched_inputs, check_step, run_step_batched,
                                  scatter_pages)
from test_gpu_softmax import check as softmax_check

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
ATOL, RTOL = 2e-3, 4e-3
N_CASES = 40


def close(got, ref, what):
    g = got.detach().float().cpu().numpy().astype(np.float64)
    err = np.abs(g - ref)
    assert np.all(np.isfinite(g)), what
    assert np.all(err <= ATOL + RTOL * np.abs(ref)), "%s: err %.3g" % (what, err.max())


def randn16(rng, shape, sigma=1.0):
    return (rng.standard_normal(shape) * sigma).astype(np.float16)


def dev_unaligned(a, offset):
    """Copy a host fp16 array to the GPU at an element offset inside a larger
    buffer (offset 0: 256-byte aligned)."""
    flat = torch.empty(a.size + offset, dtype=torch.float16, device=DEV)
    t = flat[offset:].view(a.shape)
    t.copy_(torch.from_numpy(a))
    return t


def shape_draw(rng):
    D = int(rng.choice([1, 2, 3, 6, 8, 16, 24, 40, 48, 64, 72, 96, 100, 128, 136, 192, 250, 256]))
    H = int(rng.integers(1, 9))
    S = int(rng.choice([1, 2, 15, 16, 17, 100, 257, 1000, 3000]))
    return D, H, S


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_single_and_batched(case):
    rng = np.random.default_rng(1000 + case)
    D, H, S = shape_draw(rng)
    B = int(rng.integers(1, 6))
    offset = int(rng.choice([0, 0, 1, 2, 4]))
    pos = rng.integers(0, S + 3, B)
    print("case", case, dict(B=B, S=S, H=H, D=D, offset=offset, pos=pos.tolist()), flush=True)
    q = randn16(rng, (B, H, D), float(rng.choice([0.5, 1.0, 3.0])))
    k = randn16(rng, (B, S, H, D))
    v = randn16(rng, (B, S, H, D))
    ref, _ = oracle.decode_batched(q, k, v, pos)
    out = ad.decode_batched(dev_unaligned(q, offset), dev_unaligned(k, offset),
                            dev_unaligned(v, offset), torch.from_numpy(pos.astype(np.int32)).to(DEV))
    one = ad.decode(dev_unaligned(q[0], offset), dev_unaligned(k[0], offset),
                    dev_unaligned(v[0], offset), int(pos[0]))
    torch.cuda.synchronize()
    close(out, ref, "batched case %d" % case)
    close(one, ref[0], "single case %d" % case)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_paged(case):
    rng = np.random.default_rng(2000 + case)
    D, H, _ = shape_draw(rng)
    P = int(rng.choice([1, 2, 4, 16, 64]))
    MB = int(rng.integers(1, 12))
    B = int(rng.integers(1, 5))
    S = P * MB
    NB = B * MB + int(rng.integers(0, 4))
    pos = rng.integers(0, S + 2, B)
    print("case", case, dict(B=B, P=P, MB=MB, NB=NB, H=H, D=D, pos=pos.tolist()), flush=True)
    q = randn16(rng, (B, H, D))
    kp = randn16(rng, (NB, P, H, D))
    vp = randn16(rng, (NB, P, H, D))
    bt = rng.permutation(NB)[: B * MB].reshape(B, MB).astype(np.int32)
    dense_k = np.stack([kp[bt[b]].reshape(S, H, D) for b in range(B)])
    dense_v = np.stack([vp[bt[b]].reshape(S, H, D) for b in range(B)])
    ref, _ = oracle.decode_batched(q, dense_k, dense_v, pos)
    out = ad.decode_paged(torch.from_numpy(q).to(DEV), torch.from_numpy(kp).to(DEV),
                          torch.from_numpy(vp).to(DEV), torch.from_numpy(bt).to(DEV),
                          torch.from_numpy(pos.astype(np.int32)).to(DEV))
    torch.cuda.synchronize()
    close(out, ref, "paged case %d" % case)


# case 74 adds a rotation that cancels (-2.0e-4 from inputs near 1.8), where
# the fp32 rotation's error spans many fp16 steps of the result
@pytest.mark.parametrize("case", list(range(N_CASES)) + [74])
def test_random_decode_step(case):
    rng = np.random.default_rng(3000 + case)
    D, H, S = shape_draw(rng)
    dims = int(rng.choice([0, D - D % 2, (D // 4) * 2]))
    trad = bool(rng.integers(0, 2))
    base = float(rng.choice([10000.0, 500000.0, 17.5]))
    B = int(rng.integers(1, 5))
    pos = rng.integers(0, S + 2, B)
    print("case", case, dict(B=B, S=S, H=H, D=D, dims=dims, trad=trad, base=base,
                             pos=pos.tolist()), flush=True)
    q, kn, vn = (randn16(rng, (B, H, D)) for _ in range(3))
    kc, vc = randn16(rng, (B, S, H, D)), randn16(rng, (B, S, H, D))
    kc_d, vc_d = torch.from_numpy(kc).to(DEV), torch.from_numpy(vc).to(DEV)
    out = ad.decode_step(torch.from_numpy(q).to(DEV), torch.from_numpy(kn).to(DEV),
                         torch.from_numpy(vn).to(DEV), kc_d, vc_d,
                         torch.from_numpy(pos.astype(np.int32)).to(DEV), rope_dims=dims,
                         rope_base=base, traditional=trad)
    torch.cuda.synchronize()
    kg = kc_d.cpu().numpy()
    for b in range(B):
        kco, vco = kc[b].view(np.uint16).copy(), vc[b].view(np.uint16).copy()
        r = oracle.decode_step(q[b], kn[b], vn[b], kco, vco, int(pos[b]), dims=dims, base=base,
                               traditional=trad)
        close(out[b], r["out"], "step case %d b=%d" % (case, b))
        assert_rotation(kg[b, r["pos"]].view(np.uint16), kn[b], r["k_rot"], r["k16"], dims, trad,
                        "step case %d b=%d" % (case, b))


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_two_dispatch(case):
    rng = np.random.default_rng(4000 + case)
    D, H, S = shape_draw(rng)
    cp = int(rng.integers(0, S + 2))
    print("case", case, dict(S=S, H=H, D=D, cp=cp), flush=True)
    q, k, v = randn16(rng, (H, D)), randn16(rng, (S, H, D)), randn16(rng, (S, H, D))
    _, s_ref, _ = oracle.decode(q, k, v, cp, want_scores=True)
    sc = ad.qk(torch.from_numpy(q).to(DEV), torch.from_numpy(k).to(DEV), cp)
    torch.cuda.synchronize()
    L = min(cp, S - 1) + 1
    got = sc.cpu().numpy().astype(np.float64)
    assert np.all(got[:, L:] == -np.inf)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(s_ref[:, :L]), 2.0 ** -14))) - 10)
    cond = np.einsum("hd,phd->hp", np.abs(q.astype(np.float64)),
                     np.abs(k[:L].astype(np.float64))) / np.sqrt(D)
    assert np.all(np.abs(got[:, :L] - s_ref[:, :L]) < ulp + D * 2.0 ** -24 * cond)
    # the second dispatch on the oracle's scores rounded to fp16 (an input
    # both sides take; nothing of the GPU's feeds the oracle)
    s16 = s_ref.astype(np.float16)
    ref = oracle.pv_from_scores(s16, v, cp)
    out = ad.pv(torch.from_numpy(s16).to(DEV), torch.from_numpy(v).to(DEV), cp)
    torch.cuda.synchronize()
    close(out, ref, "two dispatches case %d" % case)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_masked_score_rows(case):
    """Second dispatch on fp16 score rows with random -inf stretches (some far
    longer than a chunk) and holes, NaN V under them; at least one finite
    score per head."""
    rng = np.random.default_rng(6000 + case)
    D, H, _ = shape_draw(rng)
    S = int(rng.choice([50, 1000, 5000, 20000, 40001]))
    cp = int(rng.integers(0, S + 2))
    L = min(cp, S - 1) + 1
    print("case", case, dict(S=S, H=H, D=D, cp=cp), flush=True)
    sc = randn16(rng, (H, S), float(rng.choice([1.0, 3.0])))
    v = randn16(rng, (S, H, D))
    masked = np.zeros((H, S), dtype=bool)
    for _ in range(int(rng.integers(1, 4))):
        lo = int(rng.integers(0, L))
        hi = int(rng.integers(lo, L + 1))
        masked[:, lo:hi] = True
    masked[:, rng.integers(0, L, size=int(rng.integers(0, 6)))] = True
    for h in range(H):                        # keep one finite score per head
        if masked[h, :L].all():
            masked[h, int(rng.integers(0, L))] = False
    sc[masked] = -np.inf
    v[masked.T] = np.nan                      # V of (position, head) pairs never weighed
    ref = oracle.pv_from_scores(sc, v, cp)
    out = ad.pv(torch.from_numpy(sc).to(DEV), torch.from_numpy(v).to(DEV), cp)
    torch.cuda.synchronize()
    close(out, ref, "masked score rows case %d" % case)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_softmax_and_rope(case):
    rng = np.random.default_rng(5000 + case)
    rows = int(rng.choice([1, 3, 17, 300]))
    cols = int(rng.choice([1, 5, 64, 1000, 1025, 4096, 5000, 33000, 70000]))
    print("case", case, dict(rows=rows, cols=cols), flush=True)
    x = (rng.standard_normal((rows, cols)) * float(rng.choice([1, 5, 30]))).astype(np.float32)
    if rng.integers(0, 2):
        x[:, int(rng.integers(0, cols)):] = -np.inf
        x[:, 0] = 0.0
    got = ad.softmax(torch.from_numpy(x).to(DEV))
    torch.cuda.synchronize()
    softmax_check(got, x, "softmax case %d" % case, threads=4)
    D = int(rng.choice([2, 6, 64, 128, 256]))
    dims = int(rng.choice([0, D, D // 2 - (D // 2) % 2]))
    trad = bool(rng.integers(0, 2))
    B, H = int(rng.integers(1, 4)), int(rng.integers(1, 5))
    xr = randn16(rng, (B, H, D), 2.0)
    pos = rng.integers(0, 1 << 31, B).astype(np.uint32)
    got = ad.rope(torch.from_numpy(xr).to(DEV), torch.from_numpy(pos.view(np.int32)).to(DEV),
                  rope_dims=dims, traditional=trad)
    torch.cuda.synchronize()
    exact = oracle.rope(xr, pos[:, None].astype(np.int64), dims=dims, traditional=trad)
    assert_rotation(got.cpu().numpy().view(np.uint16), xr, exact, oracle.double_to_half(exact),
                    dims, trad, "rope case %d" % case)


N_BATCH_CASES = 30


def large_batch_draw(case, rng):
    """Sizes for test_random_large_batches; the case number picks the region:
    0 <= 256 KiB of K+V per 256-byte head block, 1 the 512 KiB band with just
    enough sequences x heads for 256 workgroups (paged: one more), 2 longer
    capacities with few sequences."""
    paged = bool(case % 2)
    region = case % 3
    if region == 0:
        D = int(rng.choice([8, 16, 32, 48, 64, 96, 128]))
        H = int(rng.choice([1, 2, 4, 8, 16, 32]))
        B = int(rng.choice([16, 64, 200, 700]))
        S = int(rng.choice([1, 16, 100, 300, 512]))
        while B * S * H * D > 24 << 20:
            S = max(1, S // 2)
    elif region == 1:
        D = int(rng.choice([64, 128]))
        H = int(rng.choice([8, 16, 32]))
        S = int(rng.choice([520, 600, 1000, 1024]))
        heads_per_group = 2 if D == 64 else 1
        B = -(-256 * heads_per_group // H) + int(rng.integers(0, 12)) + (1 if paged else 0)
    else:
        D = int(rng.choice([32, 64, 128]))
        H = int(rng.choice([2, 4, 8]))
        B = int(rng.choice([4, 16, 64]))
        S = int(rng.choice([1100, 2048, 3000]))
    if paged:   # whole pages
        S = max(16, S // 16 * 16) if S >= 16 else S
    return paged, B, S, H, D


@pytest.mark.parametrize("case", range(N_BATCH_CASES))
def test_random_large_batches(case):
    """Batches of 4-700 sequences, dense or paged, drawn on both sides of the
    one-chunk plans' edges (256 and 512 KiB of K+V per workgroup, 256
    workgroups, head blocks widened past 8192 workgroups) and on the balanced
    grid: every output against the oracle."""
    rng = np.random.default_rng(5000 + case)
    paged, B, S, H, D = large_batch_draw(case, rng)
    pos = rng.integers(0, S + 2, B)
    flags = ad.PLAN_PAGED if paged else ad.PLAN_DEVICE_POS
    print("case", case, dict(B=B, S=S, H=H, D=D, paged=paged), ad.plan(B, H, D, S, 0, flags), flush=True)
    q = randn16(rng, (B, H, D))
    k = randn16(rng, (B, S, H, D))
    v = randn16(rng, (B, S, H, D))
    ref, _ = oracle.decode_batched(q, k, v, pos, threads=8)
    cp = torch.from_numpy(pos.astype(np.int32)).to(DEV)
    if paged:
        P = int(rng.choice([p for p in (1, 4, 16) if S % p == 0]))
        MB = S // P
        perm = rng.permutation(B * MB)
        kp = np.empty((B * MB, P, H, D), np.float16)
        vp = np.empty((B * MB, P, H, D), np.float16)
        kp[perm] = k.reshape(B * MB, P, H, D)
        vp[perm] = v.reshape(B * MB, P, H, D)
        bt = perm.reshape(B, MB).astype(np.int32)
        out = ad.decode_paged(torch.from_numpy(q).to(DEV), torch.from_numpy(kp).to(DEV),
                              torch.from_numpy(vp).to(DEV), torch.from_numpy(bt).to(DEV), cp)
    else:
        out = ad.decode_batched(torch.from_numpy(q).to(DEV), torch.from_numpy(k).to(DEV),
                                torch.from_numpy(v).to(DEV), cp)
    torch.cuda.synchronize()
    close(out, ref, "large batch case %d" % case)


@pytest.mark.parametrize("case", range(18))
def test_random_large_batch_steps(case):
    """The decode step on batches drawn like test_random_large_batches (the
    one-chunk, mid-size and balanced plans), dense caches: six sampled
    sequences, the first and last among them, against the oracle's step --
    output, the appended rows, every other row unchanged."""
    rng = np.random.default_rng(7000 + case)
    _, B, S, H, D = large_batch_draw(case * 2, rng)   # the dense draws
    cps = rng.integers(0, S + 2, B)
    print("case", case, dict(B=B, S=S, H=H, D=D), ad.plan(B, H, D, S, 0, ad.PLAN_DEVICE_POS | ad.PLAN_STEP),
          flush=True)
    q, kn, vn = (randn16(rng, (B, H, D)) for _ in range(3))
    kc, vc = randn16(rng, (B, S, H, D)), randn16(rng, (B, S, H, D))
    out, kg, vg = run_step_batched(q, kn, vn, kc, vc, cps, D)
    for b in sorted({0, B - 1, *rng.choice(B, 4, replace=False).tolist()}):
        check_step(out[b], kg[b], vg[b], kc[b], vc[b], q[b], kn[b], vn[b], int(cps[b]), D, False,
                   what="case %d sequence %d" % (case, b))


@pytest.mark.parametrize("case", range(20))
def test_random_paged_step(case):
    """The decode step on shuffled page pools (pages of 1-64 positions),
    random batches: the dense step's output bits where both take the same
    plan, the new rows in the right pages and nothing else written, and
    three sequences against the oracle's step."""
    rng = np.random.default_rng(11000 + case)
    P = int(rng.choice([1, 2, 4, 16, 64]))
    MB = int(rng.choice([1, 2, 5, 16, 64]))
    S = P * MB
    D = int(rng.choice([8, 16, 48, 64, 96, 128]))
    H = int(rng.choice([1, 2, 4, 8]))
    B = int(rng.choice([1, 3, 8, 40, 300]))
    while B * S * H * D > 8 << 20:
        B = max(1, B // 2)
    trad = bool(rng.integers(0, 2))
    cps = rng.integers(0, S + 2, B)
    print("case", case, dict(B=B, S=S, H=H, D=D, P=P, trad=trad), flush=True)
    q, kn, vn, kc, vc, cps = batched_inputs(rng, B, S, H, D, cps)
    dense_out, dense_k, dense_v = run_step_batched(q, kn, vn, kc, vc, cps, D, trad)
    kp, vp, bt = scatter_pages(kc, vc, P, rng)
    kp_d, vp_d = torch.from_numpy(kp).to(DEV), torch.from_numpy(vp).to(DEV)
    out = ad.decode_step_paged(torch.from_numpy(q).to(DEV), torch.from_numpy(kn).to(DEV),
                               torch.from_numpy(vn).to(DEV), kp_d, vp_d, torch.from_numpy(bt).to(DEV),
                               torch.from_numpy(cps.astype(np.int32)).to(DEV), traditional=trad).cpu()
    torch.cuda.synchronize()
    if ad.plan(B, H, D, S, 0, ad.PLAN_PAGED | ad.PLAN_STEP) == ad.plan(B, H, D, S, 0, ad.PLAN_DEVICE_POS | ad.PLAN_STEP):
        assert torch.equal(out, dense_out)
    want_k, want_v = kp.copy(), vp.copy()
    for b in range(B):
        pos = min(int(cps[b]), S - 1)
        want_k[bt[b, pos // P], pos % P] = dense_k[b, pos]
        want_v[bt[b, pos // P], pos % P] = dense_v[b, pos]
    assert np.array_equal(kp_d.cpu().numpy().view(np.uint16), want_k.view(np.uint16))
    assert np.array_equal(vp_d.cpu().numpy().view(np.uint16), want_v.view(np.uint16))
    for b in sorted({0, B - 1, B // 2}):
        check_step(out[b], dense_k[b], dense_v[b], kc[b], vc[b], q[b], kn[b], vn[b], int(cps[b]), D, trad,
                   what="case %d sequence %d" % (case, b))
