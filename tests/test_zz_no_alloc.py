"""attn_decode_f16_batched_noalloc through the C ABI: its output equals that
of attn_decode_f16_batched (its own workspace) bitwise, on two calls in a
row, the second with a smaller batch and cache, and is within the oracle bar
(page "Developing Apple Metal Kernels in Rust - A Deep Dive Through
Attention", section "The MSL, briefly", for each sequence)."""
import numpy as np
import pytest
import torch

import decode_attention_kv_seq_amd as ad
import oracle

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _inputs(B, S, H, D, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    q = torch.randn((B, H, D), generator=g, device=DEV).half()
    k = torch.randn((B, S, H, D), generator=g, device=DEV).half()
    v = torch.randn((B, S, H, D), generator=g, device=DEV).half()
    cp = torch.randint(0, S + 3, (B,), generator=g, device=DEV, dtype=torch.int32)
    cp[0] = S - 1
    return q, k, v, cp


def test_noalloc_matches_batched_call_twice():
    lib = ad.load_library()
    # the second call is smaller: fewer sequences, shorter caches, another head_dim
    for (B, S, H, D, seed) in [(9, 3000, 16, 128, 1), (3, 700, 8, 64, 2)]:
        print("case B=%d S=%d H=%d D=%d" % (B, S, H, D), flush=True)
        q, k, v, cp = _inputs(B, S, H, D, seed)
        ref = ad.decode_batched(q, k, v, cp)
        out = torch.full_like(ref, float("nan"))
        ad.decode_batched_noalloc(q, k, v, cp, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "allocation-free call differs from the batched call"
        # and within the oracle bar, on every head of three sequences
        pos = cp.cpu().numpy()
        for b in (0, 1, B - 1):
            o, _, _ = oracle.decode(q[b].cpu(), k[b].cpu(), v[b].cpu(), int(pos[b]), threads=4)
            got = out[b].float().cpu().numpy()
            assert np.all(np.abs(got - o) <= 2e-3 + 4e-3 * np.abs(o)), (B, b)



FIRST_CALL_CAPTURED = """
import sys, torch
sys.path.insert(0, sys.argv[1])
import decode_attention_kv_seq_amd as ad
dev = torch.device("cuda:0")
g = torch.Generator(device=dev)
g.manual_seed(3)
B, S, H, D = 4, 500, 8, 64
q = torch.randn((B, H, D), generator=g, device=dev).half()
k = torch.randn((B, S, H, D), generator=g, device=dev).half()
v = torch.randn((B, S, H, D), generator=g, device=dev).half()
cp = torch.tensor([499, 0, 250, 700], dtype=torch.int32, device=dev)
out = torch.empty_like(q)
torch.cuda.synchronize()
graph = torch.cuda.CUDAGraph()
with torch.cuda.graph(graph):          # the process's first allocation-free call
    ad.decode_batched_noalloc(q, k, v, cp, out=out)
graph.replay()
torch.cuda.synchronize()
ref = ad.decode_batched(q, k, v, cp)
torch.cuda.synchronize()
assert torch.equal(out, ref)
print("first call under capture: ok", flush=True)
"""


def test_noalloc_under_graph_capture():
    """The callers this entry point is for capture it in a graph: a captured
    call, replayed four times with eager calls of other sizes on the same
    array in between, gives the batched call's output bitwise each time;
    and the process's very first call (which looks up the array's address)
    may itself be made under capture (child process)."""
    import os
    import subprocess
    import sys
    q, k, v, cp = _inputs(6, 1200, 8, 128, 11)
    ref = ad.decode_batched(q, k, v, cp)
    out = torch.full_like(ref, float("nan"))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ad.decode_batched_noalloc(q, k, v, cp, out=out)
    q2, k2, v2, cp2 = _inputs(3, 400, 4, 64, 12)
    ref2 = ad.decode_batched(q2, k2, v2, cp2)
    for i in range(4):
        out.fill_(float("nan"))
        out2 = torch.empty_like(ref2)
        ad.decode_batched_noalloc(q2, k2, v2, cp2, out=out2)   # eager, same array
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out2, ref2), i
        assert torch.equal(out, ref), "replay %d differs from the batched call" % i
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", FIRST_CALL_CAPTURED, root], capture_output=True, text=True,
                       timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
