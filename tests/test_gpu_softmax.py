"""GPU row softmax (the Foundry notes' fm_softmax, max-shifted as the page
"Developing Apple Metal Kernels in Rust - A Deep Dive Through Attention"
does in attention_pv_f16) against the CPU oracle, through the C-ABI library.

Bar, derived from the kernel's fp32 arithmetic.  With t_i = x_i - max (exact,
fp64) and T = sum_j w_j |t_j| (the weight-averaged distance from the max):
  - the exponent argument (x - m) * log2(e) carries at most 3 fp32 roundings,
    so e_i is off by at most 3 * 2^-24 * |t_i| relative, plus 2^-22 for the
    hardware 2^x;
  - the row sum inherits 3 * 2^-24 * T + 2^-22 from its terms and at most
    96 * 2^-24 from its own fp32 additions (32 per thread, the wave and
    workgroup trees, the chunk merge);
  - the scaling by 1/sum adds two roundings.
So |gpu - oracle| <= w_i * (3 * 2^-24 * (|t_i| + T) + 2 * 2^-22 + 98 * 2^-24)
+ 2^-125 (results below the smallest normal fp32 may flush to zero).
-inf entries must be exactly 0; a row of -inf only, or holding a NaN, NaN.
"""
import numpy as np
import pytest
import torch

import decode_attention_kv_seq_amd as ad
from decode_attention_kv_seq_amd import workloads as wl
import oracle

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def softmax_bound(x, ref):
    x64 = np.asarray(x, np.float64)
    with np.errstate(invalid="ignore"):
        m = np.max(np.where(np.isfinite(x64), x64, -np.inf), axis=1, keepdims=True)
        t = np.abs(np.where(np.isfinite(x64), x64 - m, 0.0))
    T = np.sum(ref * t, axis=1, keepdims=True)
    rel = 3 * 2.0 ** -24 * (t + T) + 2 * 2.0 ** -22 + 98 * 2.0 ** -24
    return ref * rel + 2.0 ** -125


def check(got, x, what="", threads=8):
    """got: GPU tensor; x: host fp32 numpy [rows, cols]."""
    ref = oracle.softmax_rows(x, threads=threads)
    g = got.cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape
    nan_rows = np.isnan(ref).any(axis=1)
    assert np.all(np.isnan(g[nan_rows])), "%s: NaN rows" % what
    g, ref, xx = g[~nan_rows], ref[~nan_rows], x[~nan_rows]
    masked = np.isneginf(xx)
    assert np.all(g[masked] == 0.0), "%s: -inf entries must give exactly 0" % what
    err = np.abs(g - ref)
    bound = softmax_bound(xx, ref)
    bad = err > bound
    assert not bad.any(), "%s: err %.3g > %.3g at %s (got %r ref %r)" % (
        what, err[bad].max(), bound[bad][np.argmax(err[bad])], np.argwhere(bad)[0],
        g[bad][0], ref[bad][0])
    return float((err / np.maximum(ref, 1e-300)).max()) if ref.size else 0.0


SHAPES = [  # rows, cols: the plan takes a wave per row up to 1024 columns, a
            # workgroup per row up to 32768 with enough rows or little data,
            # else the split path in 4096-column chunks
    (1, 1), (1, 2), (3, 7), (5, 64), (7, 1000), (4, 1024), (4, 1025), (300, 4096), (2, 8192),
    (3, 8193), (2, 16385), (2, 32768), (300, 1030), (2, 32769), (64, 40000), (100, 30000),
    (1, 300001), (3, 4097), (260, 20000),
    # long rows, 64-100 of them (split path; odd widths take scalar loads)
    (64, 262143), (64, 262144), (64, 131072), (70, 65536), (100, 32769), (64, 40001),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "r%d_c%d" % s)
def test_softmax_shapes(shape):
    rows, cols = shape
    print("softmax", shape, flush=True)
    rng = np.random.default_rng(rows * 7919 + cols)
    x = (rng.standard_normal((rows, cols)) * 3.0).astype(np.float32)
    got = ad.softmax(torch.from_numpy(x).to(DEV))
    torch.cuda.synchronize()
    check(got, x, str(shape))


@pytest.mark.parametrize("offset,cols,rows", [(1, 64, 5), (1, 5000, 5), (2, 1024, 5), (3, 40000, 5),
                                              (1, 70000, 64)])
def test_softmax_unaligned(offset, cols, rows):
    """Rows not 16-byte aligned (scalar loads): a view offset by whole floats."""
    rng = np.random.default_rng(offset + cols)
    base = torch.from_numpy(rng.standard_normal(rows * cols + offset).astype(np.float32)).to(DEV)
    x = base[offset:].view(rows, cols)
    out_base = torch.empty(rows * cols + offset, dtype=torch.float32, device=DEV)
    out = out_base[offset:].view(rows, cols)
    ad.softmax(x, out=out)
    torch.cuda.synchronize()
    check(out, x.cpu().numpy(), "offset %d" % offset)


@pytest.mark.parametrize("rows", [8, 64])
@pytest.mark.parametrize("cols", [100, 5000, 40000, 100000])
def test_softmax_masked_rows(cols, rows):
    """-inf tails (whole -inf chunks on the split path), a row of -inf only, a
    row with a NaN, a row with +inf, a single finite entry; 8 or 64 rows."""
    rng = np.random.default_rng(cols + rows)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x[0, cols // 3:] = -np.inf
    x[1, :] = -np.inf
    x[2, cols // 2] = np.nan
    x[3, 1:] = -np.inf                  # one entry: weight exactly 1
    x[4, cols - 1] = np.inf
    x[5, : cols - 1] = -np.inf
    got = ad.softmax(torch.from_numpy(x).to(DEV))
    torch.cuda.synchronize()
    g = got.cpu().numpy()
    assert np.all(np.isnan(g[1])) and np.all(np.isnan(g[2])) and np.all(np.isnan(g[4]))
    assert g[3, 0] == 1.0 and np.all(g[3, 1:] == 0.0)
    assert g[5, -1] == 1.0 and np.all(g[5, :-1] == 0.0)
    keep = [0, 3, 5] + list(range(6, rows))
    check(got[keep], np.ascontiguousarray(x[keep]), "masked cols=%d" % cols)


@pytest.mark.parametrize("name", sorted(wl.SOFTMAX_WORKLOADS))
def test_softmax_workloads_full(name):
    """The decode workloads' score matrices, every element."""
    w = wl.SOFTMAX_WORKLOADS[name]
    print("case", name, flush=True)
    x = wl.make_scores(w, DEV)
    got = ad.softmax(x)
    torch.cuda.synchronize()
    worst = check(got, x.cpu().numpy(), name)
    print("%s: worst relative error %.3g" % (name, worst))


def test_softmax_in_place_and_repeatable():
    rng = np.random.default_rng(11)
    for shape in [(300, 4096), (4, 100000), (50, 700), (64, 100000)]:
        x_h = (rng.standard_normal(shape) * 2).astype(np.float32)
        x = torch.from_numpy(x_h).to(DEV)
        a = ad.softmax(x)
        b = ad.softmax(x)
        y = x.clone()
        ad.softmax(y, out=y)
        torch.cuda.synchronize()
        assert torch.equal(a, b), shape
        assert torch.equal(a, y), shape


def test_softmax_of_decode_scores():
    """The fp32 score dump of a decode, put through the row softmax, gives
    the oracle's attention weights to the dump's own accuracy
    (|ds| <= 1e-4 of the score scale, so about 1e-4 * |s| relative)."""
    w = wl.WORKLOADS["h32_d128_s32768_cp20000_garbage"]
    q_h = wl.make_q(w)[0]
    k_d, v_d = wl.make_kv(w, DEV)
    _, dump = ad.decode(q_h.to(DEV), k_d[0], v_d[0], w.cur_pos, dump=True)
    weights = ad.softmax(dump)
    torch.cuda.synchronize()
    heads = [0, 17, 31]
    for h in heads:
        _, kh, vh = wl.head_slice(w, 0, h, n_rows=w.seq_len)
        _, _, ref_w = oracle.decode(q_h[h:h + 1], kh, vh, w.cur_pos, want_weights=True)
        g = weights[h].cpu().numpy().astype(np.float64)
        L = w.cur_pos + 1
        assert np.all(g[L:] == 0.0)
        assert np.allclose(g[:L], ref_w[0, :L], rtol=1e-3, atol=1e-12), h
    del k_d, v_d
    torch.cuda.empty_cache()


def test_softmax_million_short_rows():
    """2^20 rows of 24 columns (the wave-per-row path at scale), sampled rows."""
    rng = np.random.default_rng(20)
    rows, cols = 1 << 20, 24
    x = (rng.standard_normal((rows, cols)) * 4).astype(np.float32)
    got = ad.softmax(torch.from_numpy(x).to(DEV))
    torch.cuda.synchronize()
    pick = np.concatenate([[0, rows - 1], rng.choice(rows, 2000, replace=False)])
    check(got[torch.from_numpy(pick).to(DEV)], np.ascontiguousarray(x[pick]), "2^20 rows")


@pytest.mark.parametrize("rows,cols,check_rows", [
    ((1 << 17) + 1, 32768, (0, 1 << 16, 1 << 17)),   # a workgroup per row
    (64, (1 << 26) + 64, (32, 63)),                  # split path, 4096-column chunks
], ids=["row_path", "split_path"])
def test_softmax_past_2_32_elements(rows, cols, check_rows):
    """Inputs of just over 2^32 fp32 elements (17 GB in, 17 GB out), filled on
    the device by the shared generator: the checked rows start at or cross
    elements 2^31 and 2^32, where 32-bit offsets would wrap.  The oracle
    regenerates only those rows on the host."""
    assert rows * cols > 1 << 32
    print("softmax past 2^32", rows, cols, flush=True)
    x = torch.empty((rows, cols), dtype=torch.float32, device=DEV)
    flat = x.view(-1)
    step = 1 << 26
    for lo in range(0, flat.numel(), step):
        hi = min(flat.numel(), lo + step)
        flat[lo:hi] = wl.normal_f32(77, 0, torch.arange(lo, hi, dtype=torch.int64, device=DEV), 3.0)
    got = ad.softmax(x)
    torch.cuda.synchronize()
    del x
    for r in check_rows:
        xr = wl.normal_f32(77, 0, torch.arange(r * cols, (r + 1) * cols, dtype=torch.int64), 3.0)
        check(got[r:r + 1], xr.numpy().reshape(1, cols), "row %d" % r)
    del got
    torch.cuda.empty_cache()
