"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph): the
header promises no call allocates or synchronises, so capture must work and
every replay must give the eager call's bits.  Each replay is separated by
eager work and a synchronisation, and every replay is checked, since graph
nodes have been seen to misbehave only on replays after the first."""
import numpy as np
import pytest
import torch

import decode_attention_kv_seq_amd as ad
from decode_attention_kv_seq_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def replay_and_check(g, outs, expected, disturb):
    for i in range(4):
        for o in outs:
            o.fill_(float("nan")) if o.dtype.is_floating_point else o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, expected):
            assert torch.equal(o, e), "replay %d differs" % i
        disturb()
        torch.cuda.synchronize()


def test_graph_decode_single_and_batched():
    rng = np.random.default_rng(1)
    S, H, D, cp = 5000, 8, 128, 4321
    q = torch.from_numpy(rng.standard_normal((H, D)).astype(np.float16)).to(DEV)
    k = torch.from_numpy(rng.standard_normal((S, H, D)).astype(np.float16)).to(DEV)
    v = torch.from_numpy(rng.standard_normal((S, H, D)).astype(np.float16)).to(DEV)
    w = wl.WORKLOADS["b64_h32_d128_cap8192_ragged"]
    qb = wl.make_q(w, DEV)
    kb, vb = wl.make_kv(w, DEV)
    cpb = w.positions().to(torch.int32).to(DEV)
    ws1 = ad.alloc_workspace(1, H, D, S, DEV)
    wsb = ad.alloc_workspace(w.batch, w.n_heads, w.head_dim, w.seq_len, DEV)
    out1 = torch.empty((H, D), dtype=torch.float16, device=DEV)
    outb = torch.empty(w.q_shape, dtype=torch.float16, device=DEV)
    e1 = ad.decode(q, k, v, cp, workspace=ws1).clone()
    eb = ad.decode_batched(qb, kb, vb, cpb, workspace=wsb).clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm the side stream before capture
        ad.decode(q, k, v, cp, out=out1, workspace=ws1)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ad.decode(q, k, v, cp, out=out1, workspace=ws1)
        ad.decode_batched(qb, kb, vb, cpb, out=outb, workspace=wsb)
    scratch = torch.empty(1 << 22, device=DEV)

    def disturb():   # eager work between replays, reusing the same workspaces
        ad.decode(q, k, v, 17, workspace=ws1)
        ad.decode_batched(qb, kb, vb, torch.zeros_like(cpb), workspace=wsb)
        scratch.uniform_()

    replay_and_check(g, [out1, outb], [e1, eb], disturb)


def test_graph_decode_step_and_softmax():
    rng = np.random.default_rng(2)
    S, H, D, cp = 3000, 4, 64, 2500
    q, kn, vn = (torch.from_numpy(rng.standard_normal((H, D)).astype(np.float16)).to(DEV)
                 for _ in range(3))
    k0 = torch.from_numpy(rng.standard_normal((S, H, D)).astype(np.float16)).to(DEV)
    v0 = torch.from_numpy(rng.standard_normal((S, H, D)).astype(np.float16)).to(DEV)
    kc, vc = k0.clone(), v0.clone()
    ws = ad.alloc_workspace(1, H, D, S, DEV)
    e_out = ad.decode_step(q, kn, vn, kc, vc, cp, workspace=ws).clone()
    e_k, e_v = kc.clone(), vc.clone()
    x = torch.from_numpy((rng.standard_normal((64, 40000)) * 3).astype(np.float32)).to(DEV)
    sws = torch.empty(ad.softmax_workspace_bytes(64, 40000), dtype=torch.uint8, device=DEV)
    e_sm = ad.softmax(x, workspace=sws).clone()
    out = torch.empty((H, D), dtype=torch.float16, device=DEV)
    sm = torch.empty_like(x)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ad.decode_step(q, kn, vn, kc, vc, cp, out=out, workspace=ws)
        ad.softmax(x, out=sm, workspace=sws)

    def disturb():
        kc.copy_(k0)
        vc.copy_(v0)
        ad.softmax(x[:3].contiguous(), workspace=sws)

    disturb()
    torch.cuda.synchronize()
    replay_and_check(g, [out, sm], [e_out, e_sm], disturb)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(kc, e_k) and torch.equal(vc, e_v)


def test_graph_paged_and_two_dispatches():
    rng = np.random.default_rng(3)
    B, P, MB, H, D = 3, 16, 8, 8, 64
    NB = B * MB + 5
    q = torch.from_numpy(rng.standard_normal((B, H, D)).astype(np.float16)).to(DEV)
    kp = torch.from_numpy(rng.standard_normal((NB, P, H, D)).astype(np.float16)).to(DEV)
    vp = torch.from_numpy(rng.standard_normal((NB, P, H, D)).astype(np.float16)).to(DEV)
    bt = torch.from_numpy(rng.permutation(NB)[: B * MB].reshape(B, MB).astype(np.int32)).to(DEV)
    cp = torch.tensor([5, P * MB - 1, 77], dtype=torch.int32, device=DEV)
    wsp = ad.alloc_workspace(B, H, D, P * MB, DEV)
    S, cp1 = 4000, 3210
    q1 = torch.from_numpy(rng.standard_normal((H, D)).astype(np.float16)).to(DEV)
    k1 = torch.from_numpy(rng.standard_normal((S, H, D)).astype(np.float16)).to(DEV)
    v1 = torch.from_numpy(rng.standard_normal((S, H, D)).astype(np.float16)).to(DEV)
    ws1 = ad.alloc_workspace(1, H, D, S, DEV)
    e_p = ad.decode_paged(q, kp, vp, bt, cp, workspace=wsp).clone()
    e_sc = ad.qk(q1, k1, cp1).clone()
    e_o = ad.pv(e_sc, v1, cp1, workspace=ws1).clone()
    out_p = torch.empty((B, H, D), dtype=torch.float16, device=DEV)
    sc = torch.empty((H, S), dtype=torch.float16, device=DEV)
    out1 = torch.empty((H, D), dtype=torch.float16, device=DEV)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ad.decode_paged(q, kp, vp, bt, cp, out=out_p, workspace=wsp)
        ad.qk(q1, k1, cp1, scores=sc)
        ad.pv(sc, v1, cp1, out=out1, workspace=ws1)

    def disturb():
        ad.decode_paged(q, kp, vp, bt, torch.zeros_like(cp), workspace=wsp)
        ad.pv(torch.zeros_like(e_sc), v1, 10, workspace=ws1)

    replay_and_check(g, [out_p, sc, out1], [e_p, e_sc, e_o], disturb)


def test_graph_one_launch_plans():
    """The plans that finish in the split launch alone, captured together: a
    tiny single sequence (one chunk per head block), a dense batch of short
    capacity (one chunk per sequence and head block), and a decode step on a
    short-capacity batch (its combine appends the new rows)."""
    rng = np.random.default_rng(5)

    def t16(shape):
        return torch.from_numpy(rng.standard_normal(shape).astype(np.float16)).to(DEV)

    q1, k1, v1 = t16((4, 64)), t16((128, 4, 64)), t16((128, 4, 64))
    ws1 = ad.alloc_workspace(1, 4, 64, 128, DEV)
    B, S, H, D = 16, 256, 8, 128
    qb, kb, vb = t16((B, H, D)), t16((B, S, H, D)), t16((B, S, H, D))
    cpb = torch.from_numpy(rng.integers(0, S + 3, B).astype(np.int32)).to(DEV)
    wsb = ad.alloc_workspace(B, H, D, S, DEV)
    Bs, Ss, Hs, Ds = 8, 64, 4, 64
    qs, kn, vn = t16((Bs, Hs, Ds)), t16((Bs, Hs, Ds)), t16((Bs, Hs, Ds))
    k0, v0 = t16((Bs, Ss, Hs, Ds)), t16((Bs, Ss, Hs, Ds))
    kc, vc = k0.clone(), v0.clone()
    cps = torch.from_numpy(rng.integers(0, Ss, Bs).astype(np.int32)).to(DEV)
    wss = ad.alloc_workspace(Bs, Hs, Ds, Ss, DEV)
    e1 = ad.decode(q1, k1, v1, 100, workspace=ws1).clone()
    eb = ad.decode_batched(qb, kb, vb, cpb, workspace=wsb).clone()
    es = ad.decode_step(qs, kn, vn, kc, vc, cps, workspace=wss).clone()
    e_k, e_v = kc.clone(), vc.clone()
    out1 = torch.empty_like(e1)
    outb = torch.empty_like(eb)
    outs = torch.empty_like(es)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ad.decode(q1, k1, v1, 100, out=out1, workspace=ws1)
        ad.decode_batched(qb, kb, vb, cpb, out=outb, workspace=wsb)
        ad.decode_step(qs, kn, vn, kc, vc, cps, out=outs, workspace=wss)

    def disturb():   # eager calls on the same workspaces, caches restored
        ad.decode(q1, k1, v1, 3, workspace=ws1)
        ad.decode_batched(qb, kb, vb, torch.zeros_like(cpb), workspace=wsb)
        kc.copy_(k0)
        vc.copy_(v0)

    disturb()
    torch.cuda.synchronize()
    replay_and_check(g, [out1, outb, outs], [e1, eb, es], disturb)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(kc, e_k) and torch.equal(vc, e_v)


def test_two_streams_at_once():
    """Calls enqueued on two streams at once, each stream with its own
    workspace, give the bits of the same calls run one after another: the
    library keeps no state across calls."""
    rng = np.random.default_rng(4)
    S, H, D, cp = 20000, 8, 128, 19000
    q = torch.from_numpy(rng.standard_normal((H, D)).astype(np.float16)).to(DEV)
    k = torch.from_numpy(rng.standard_normal((S, H, D)).astype(np.float16)).to(DEV)
    v = torch.from_numpy(rng.standard_normal((S, H, D)).astype(np.float16)).to(DEV)
    B, Sb, Hb, Db = 6, 3000, 4, 64
    qb = torch.from_numpy(rng.standard_normal((B, Hb, Db)).astype(np.float16)).to(DEV)
    kb = torch.from_numpy(rng.standard_normal((B, Sb, Hb, Db)).astype(np.float16)).to(DEV)
    vb = torch.from_numpy(rng.standard_normal((B, Sb, Hb, Db)).astype(np.float16)).to(DEV)
    cpb = torch.from_numpy(rng.integers(0, Sb, B).astype(np.int32)).to(DEV)
    ws1 = ad.alloc_workspace(1, H, D, S, DEV)
    ws2 = ad.alloc_workspace(B, Hb, Db, Sb, DEV)
    e1 = ad.decode(q, k, v, cp, workspace=ws1).clone()
    e2 = ad.decode_batched(qb, kb, vb, cpb, workspace=ws2).clone()
    n = 12
    outs1 = [torch.empty((H, D), dtype=torch.float16, device=DEV) for _ in range(n)]
    outs2 = [torch.empty((B, Hb, Db), dtype=torch.float16, device=DEV) for _ in range(n)]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for i in range(n):
        with torch.cuda.stream(s1):
            ad.decode(q, k, v, cp, out=outs1[i], workspace=ws1)
        with torch.cuda.stream(s2):
            ad.decode_batched(qb, kb, vb, cpb, out=outs2[i], workspace=ws2)
    torch.cuda.synchronize()
    for i in range(n):
        assert torch.equal(outs1[i], e1), "stream 1 call %d" % i
        assert torch.equal(outs2[i], e2), "stream 2 call %d" % i
