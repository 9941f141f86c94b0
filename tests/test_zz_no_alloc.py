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

