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
