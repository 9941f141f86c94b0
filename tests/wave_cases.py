"""Calls whose plans take the split kernel compiled for at most two waves per
SIMD, on seeded device inputs, for the test that runs them again in a child
process with that bound switched off (ATTN_DECODE_TUNE=waves=8) and compares
the bits.  Run as a script: python wave_cases.py OUT_PATH writes the outputs
with torch.save."""
import os
import sys

import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import decode_attention_kv_seq_amd as ad  # noqa: E402

DP, PG, ST = ad.PLAN_DEVICE_POS, ad.PLAN_PAGED, ad.PLAN_STEP

# name, batch, heads, head_dim, capacity, call
CASES = [
    ("balanced", 16, 32, 128, 8192, "dense"),
    ("balanced_step", 16, 32, 128, 8192, "step"),
    ("one_chunk_u8", 8, 32, 128, 1024, "dense"),
    ("mid", 8, 8, 128, 4096, "dense"),
    ("mid_paged", 8, 8, 128, 4096, "paged"),
    ("chunked", 1030, 2, 128, 1104, "dense"),
    ("chunked_paged", 1030, 2, 128, 1104, "paged"),
    ("chunked_step", 1030, 2, 128, 1104, "step"),
]
PAGE = 16


def plan_flags(call):
    return {"dense": DP, "paged": PG, "step": DP | ST}[call]


def run_case(name, B, H, D, S, call, dev):
    g = torch.Generator(device=dev)
    g.manual_seed(sum(map(ord, name)))   # the same in every process
    q = torch.randn((B, H, D), generator=g, device=dev).half()
    k = torch.randn((B, S, H, D), generator=g, device=dev).half()
    v = torch.randn((B, S, H, D), generator=g, device=dev).half()
    cp = torch.randint(0, S, (B,), generator=g, device=dev, dtype=torch.int32)
    cp[0] = 0
    cp[1] = S - 1
    if call == "dense":
        return ad.decode_batched(q, k, v, cp)
    if call == "paged":
        nb = B * (S // PAGE)
        perm = torch.randperm(nb, generator=g, device=dev)
        kp = torch.empty((nb, PAGE, H, D), dtype=torch.float16, device=dev)
        vp = torch.empty_like(kp)
        kp[perm] = k.view(nb, PAGE, H, D)
        vp[perm] = v.view(nb, PAGE, H, D)
        bt = perm.to(torch.int32).view(B, S // PAGE).contiguous()
        return ad.decode_paged(q, kp, vp, bt, cp)
    kn = torch.randn((B, H, D), generator=g, device=dev).half()
    vn = torch.randn((B, H, D), generator=g, device=dev).half()
    return ad.decode_step(q, kn, vn, k, v, cp)


def run_all(dev):
    out = {}
    for name, B, H, D, S, call in CASES:
        out[name] = run_case(name, B, H, D, S, call, dev).cpu()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def plans():
    return {name: ad.plan(B, H, D, S, 0, plan_flags(call)) for name, B, H, D, S, call in CASES}


if __name__ == "__main__":
    dev = torch.device("cuda:0")
    for name, p in plans().items():
        print(name, p["unroll"], p["max_waves"], flush=True)
    torch.save(run_all(dev), sys.argv[1])
    print("saved", flush=True)
