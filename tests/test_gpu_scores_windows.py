"""First dispatch (scores alone) with chunks longer than the kernel's LDS
score window, so each workgroup writes several windows, the last one
partial.  The default plan cuts these sequences into chunks no longer than
one window, and the planner's knobs are read once per process, so the GPU
call runs in a child process planned with one or two target workgroups
(ATTN_DECODE_TUNE): chunks of 8192 positions, that is two to four windows
each.  The child writes the scores to a file; this process checks them
against the oracle with the bar of test_qk_scores_round_the_exact_score:
every stored score an fp16 neighbour of the exact scaled dot product up to
the fp32 accumulation error, every masked one exactly -inf."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# seq_len, heads, head_dim, current_pos, planner override.  Windows are
# 8192/hpb positions: 2048 at 4 heads per workgroup, 4096 at 2.  20001 is
# odd, so most score rows are not 16-byte aligned (element-wise writes).
CASES = [
    (20000, 4, 64, 19999, "wgs=1"),
    (20001, 4, 64, 17000, "wgs=1,unroll=8,pf=0"),
    (9000, 8, 128, 8999, "wgs=1"),
    (12345, 2, 64, 12000, "wgs=2,unroll=4"),
]


def make_inputs(S, H, D, seed):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((H, D)) * 2.0).astype(np.float16)
    k = rng.standard_normal((S, H, D)).astype(np.float16)
    return q, k


def f16_ulp(x):
    a = np.abs(np.asarray(x, np.float64))
    return 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -14))) - 10)


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=lambda c: "S%d_H%d_D%d_cp%d_%s" % c)
def test_scores_over_several_windows(case, tmp_path):
    import oracle

    S, H, D, cp, tune = case
    seed = S + 7 * D
    path = str(tmp_path / "scores.npy")
    print("case", case, flush=True)
    env = dict(os.environ, ATTN_DECODE_TUNE=tune, PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, os.path.abspath(__file__), path, str(S), str(H), str(D),
                        str(cp), str(seed)], env=env, cwd=ROOT, capture_output=True, text=True,
                       timeout=180)
    assert r.returncode == 0, r.stdout + r.stderr
    got = np.load(path).astype(np.float64)
    q, k = make_inputs(S, H, D, seed)
    L = min(cp, S - 1) + 1
    _, s_ref, _ = oracle.decode(q, k[:L], k[:L], L - 1, want_scores=True, threads=8)
    assert got.shape == (H, S)
    assert np.all(got[:, L:] == -np.inf)
    cond = np.einsum("hd,phd->hp", np.abs(q.astype(np.float64)),
                     np.abs(k[:L].astype(np.float64))) / np.sqrt(D)
    err = np.abs(got[:, :L] - s_ref[:, :L])
    bad = err >= f16_ulp(s_ref[:, :L]) + D * 2.0 ** -24 * cond
    assert not bad.any(), "first bad (head, position): %s" % (np.argwhere(bad)[0],)


def _child(path, S, H, D, cp, seed):
    """GPU side, in its own process so the planner override takes effect."""
    import torch

    import decode_attention_kv_seq_amd as ad

    print("child: qk S=%d H=%d D=%d cp=%d (%s)" % (S, H, D, cp, os.environ.get("ATTN_DECODE_TUNE")),
          flush=True)
    q, k = make_inputs(S, H, D, seed)
    dev = torch.device("cuda:0")
    sc = ad.qk(torch.from_numpy(q).to(dev), torch.from_numpy(k).to(dev), cp)
    torch.cuda.synchronize()
    np.save(path, sc.cpu().numpy())


if __name__ == "__main__":
    _child(sys.argv[1], *(int(x) for x in sys.argv[2:7]))
