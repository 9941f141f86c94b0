"""A host without a GPU: calls whose arguments are valid reach the HIP
runtime, which has no device to run them on.  Each returns ATTN_ERR_HIP with
the runtime's reason in attn_last_error(), and nothing aborts (errors are
values, as the page "Developing Apple Metal Kernels in Rust - A Deep Dive
Through Attention" has its launcher return them, section "The Launcher:
where the real work is").  Run in a child process, so an abort would fail
the test rather than end the run; host-only, since the calls pass stand-in
device addresses."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import decode_attention_kv_seq_amd as ad
lib = ad.load_library()
FAKE = 0x100000
big = 1 << 30
calls = {
    "attn_decode_f16": lambda: lib.attn_decode_f16(FAKE, FAKE, FAKE, FAKE, 4, 64, 128, 100, None,
                                                   FAKE, big, None),
    "attn_decode_f16_batched": lambda: lib.attn_decode_f16_batched(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4,
                                                                   64, 128, None, FAKE, big, None),
    "attn_decode_f16_batched_noalloc": lambda: lib.attn_decode_f16_batched_noalloc(
        FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 64, 128, None, None),
    "attn_qk_f16": lambda: lib.attn_qk_f16(FAKE, FAKE, FAKE, 4, 64, 128, 100, None),
    "attn_softmax_f32": lambda: lib.attn_softmax_f32(FAKE, FAKE, 8, 5000, FAKE, big, None),
    "attn_rope_f16": lambda: lib.attn_rope_f16(FAKE, FAKE, FAKE, 2, 4, 64, 64, 1e4, 0, None),
}
for name, call in calls.items():
    rc = call()
    print(name, rc, lib.attn_last_error().decode().replace(" ", "_") or "-")
print("done")
"""


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="needs a host without a GPU")
def test_valid_calls_without_a_device_return_hip_errors():
    r = subprocess.run([sys.executable, "-c", CHILD], capture_output=True, text=True, timeout=300,
                       cwd=ROOT)
    assert r.returncode == 0, r.stdout + r.stderr
    lines = [l.split() for l in r.stdout.splitlines()]
    assert lines[-1] == ["done"]
    results = {l[0]: (int(l[1]), l[2]) for l in lines[:-1]}
    assert len(results) == 6
    for name, (rc, detail) in results.items():
        assert rc == 5, (name, rc, detail)          # ATTN_ERR_HIP
        assert detail != "-" and len(detail) > 8, (name, detail)
