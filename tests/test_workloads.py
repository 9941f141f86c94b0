"""The seeded input generator (no GPU): definition, determinism, head slices."""
import numpy as np
import pytest
import torch

from decode_attention_kv_seq_amd import workloads as wl


def _np_words(seed, stream, idx):
    """SplitMix64 written directly with numpy uint64 arithmetic."""
    key = np.uint64(wl.stream_key(seed, stream) % (1 << 64))
    with np.errstate(over="ignore"):
        z = (idx.astype(np.uint64) + np.uint64(1)) * np.uint64(wl.GAMMA) + key
        z = (z ^ (z >> np.uint64(30))) * np.uint64(wl.M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(wl.M2)
    return z ^ (z >> np.uint64(31))


def test_splitmix64_known_value():
    # SplitMix64 seeded with 0: the first output of the reference generator
    # (state += GAMMA, then mix) is 0xE220A8397B1DCDAF.
    z = torch.tensor([wl._s64(wl.GAMMA)], dtype=torch.int64)
    assert int(wl.mix64(z)[0]) % (1 << 64) == 0xE220A8397B1DCDAF


def test_words_match_uint64_definition():
    idx = np.arange(0, 100000, 7)
    for seed, stream in [(1, 0), (5, 1), (4, 3)]:
        got = wl.words(seed, stream, torch.from_numpy(idx.astype(np.int64))).numpy().view(np.uint64)
        assert np.array_equal(got, _np_words(seed, stream, idx))


def test_normal_values_definition_and_moments():
    idx = torch.arange(1 << 18, dtype=torch.int64)
    x = wl.normal_f16(3, 2, idx, 2.0)
    w = _np_words(3, 2, idx.numpy())
    tot = sum(((w >> np.uint64(s)) & np.uint64(0xFFFF)).astype(np.int64) for s in (0, 16, 32, 48))
    c = (tot - wl.IRWIN_HALL_CENTRE).astype(np.float32)
    ref = (c * np.float32(2.0 / wl.IRWIN_HALL_SD)).astype(np.float16)
    assert np.array_equal(x.numpy(), ref)
    xf = x.double()
    assert abs(float(xf.mean())) < 0.02 and abs(float(xf.std()) - 2.0) < 0.02
    assert float(xf.abs().max()) <= 2.0 * 3.47


def test_chunking_does_not_change_values():
    idx = torch.arange(300000, dtype=torch.int64)
    a = wl.normal_f16(9, 1, idx, 1.0)
    b = torch.cat([wl._normal_f16(9, 1, idx[i:i + 1000], 1.0) for i in range(0, 300000, 1000)])
    assert torch.equal(a, b)


@pytest.mark.parametrize("seed", [11, 12])
def test_head_slice_matches_full_tensors(seed):
    w = wl.Workload("t", n_heads=3, head_dim=16, seq_len=40, cur_pos=25, seed=seed,
                    sigma_q=2.0, garbage_sigma=10.0, spike_fraction=0.1)
    q = wl.make_q(w)
    k, v = wl.make_kv(w)
    for h in range(3):
        qs, ks, vs = wl.head_slice(w, 0, h, n_rows=40)
        assert torch.equal(qs.view(-1), q[0, h])
        assert torch.equal(ks.view(40, 16), k[0, :, h])
        assert torch.equal(vs.view(40, 16), v[0, :, h])
    assert float(k[0, 26:].double().std()) > 5.0
    rows = w.spike_rows()
    assert len(rows) == 4 and len(set(rows.tolist())) == 4


def test_batched_positions_and_bytes():
    w = wl.WORKLOADS["b64_h32_d128_cap8192_ragged"]
    cp = w.positions()
    assert cp.shape == (64,) and int(cp.min()) >= 0 and int(cp.max()) <= 8191
    assert torch.equal(cp, w.positions())
    assert w.kv_bytes_read() == int((cp + 1).sum()) * 32 * 128 * 4
    w5 = wl.WORKLOADS["h64_d64_s131072_spikes"]
    assert w5.kv_bytes_read() == 2 * 131072 * 64 * 64 * 2
    assert len(w5.spike_rows()) == 1311


def test_softmax_workloads_follow_their_decode_workloads():
    """Score-matrix inputs: shape from the decode workload, -inf exactly after
    each row's valid length, spike columns scaled, rows regenerated alike."""
    from decode_attention_kv_seq_amd import workloads as wl
    for name, w in wl.SOFTMAX_WORKLOADS.items():
        d = w.decode
        x = wl.make_scores(w)
        assert tuple(x.shape) == (d.batch * d.n_heads, d.seq_len), name
        lens = w.row_lengths()
        cols = torch.arange(w.cols)[None, :]
        assert torch.equal(torch.isinf(x), cols >= lens[:, None]), name
        assert not torch.isnan(x).any()
        some = torch.tensor([0, w.rows // 2, w.rows - 1])
        assert torch.equal(wl.score_rows(w, some), x[some]), name
        if d.spike_fraction > 0:
            sp = d.spike_rows()
            assert x[:, sp].abs().mean() > 4 * x.abs().mean() / 2
    assert wl.SOFTMAX_WORKLOADS["sm_h32_s32768_masked"].row_lengths().unique().tolist() == [20001]
