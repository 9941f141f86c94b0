"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The CPU oracle (oracle/attn_oracle.c) built with gcc
  -fsanitize=address,undefined runs every pin; a copy with a planted
  one-past-the-end read, and one with a planted undefined shift, must be
  reported by the sanitizers, so a silent pass means something.
* The library's host code (argument checks, launch planner, workspace
  layout, status text) built with the same sanitizers on the host side
  (-Xarch_host; the gfx950 code is built as usual) runs the ABI and planner
  tests.  None of these calls reaches a GPU.

Each run is a child process with the sanitizer runtime preloaded; any
report aborts it."""
import hashlib
import os
import subprocess
import sys

import pytest

import oracle
from oracle import _build as oracle_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_kv_seq_amd", "csrc")
SAN_DIR = os.path.join(ROOT, "_build", "sanitized")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _gcc_runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return path


def _clang_runtime():
    """The sanitizer runtime of the compiler hipcc drives (AddressSanitizer
    with the UndefinedBehaviorSanitizer handlers)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    r = subprocess.run([hipcc, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True)
    path = r.stdout.strip().splitlines()[-1] if r.stdout.strip() else ""
    if not os.path.isabs(path) or not os.path.exists(path):
        import glob
        found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
        if not found:
            pytest.skip("the HIP compiler's AddressSanitizer runtime is not installed")
        path = found[-1]
    return path


def _child(code, timeout=600, runtime=None):
    env = dict(os.environ, LD_PRELOAD=runtime or _gcc_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=87")
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                          timeout=timeout, env=env, cwd=ROOT)


def _build_oracle(src, lib):
    cmd = ["gcc", "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-Wall", "-fno-fast-math",
           "-ffp-contract=off"] + SAN_FLAGS + [src, "-o", lib, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return lib


RUN_PINS = """
import sys
sys.path.insert(0, 'tests')
import oracle, oracle_pins
orc = oracle.OracleLib(%r)
for pin in oracle_pins.ALL_PINS:
    pin(orc)
# wider shapes than the pins: every head split, the scores and weights rows
import numpy as np
rng = np.random.default_rng(3)
for (S, H, D, cp) in [(1, 1, 1, 0), (257, 7, 200, 300), (33, 16, 256, 5)]:
    q = rng.standard_normal((H, D)).astype(np.float16)
    k = rng.standard_normal((S, H, D)).astype(np.float16)
    orc.decode(q, k, k, cp, want_scores=True, want_weights=True, threads=3)
    orc.pv_from_scores(orc.double_to_half(rng.standard_normal((H, S))), k, cp)
    orc.rope(k, np.arange(S)[:, None], dims=D - D %% 2)
orc.softmax_rows(rng.standard_normal((5, 300)).astype(np.float32), threads=2)
print('pins ok', len(oracle_pins.ALL_PINS))
"""


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = _build_oracle(oracle_build.SRC, str(tmp_path / "liboracle_san.so"))
    r = _child(RUN_PINS % lib)
    assert r.returncode == 0 and "pins ok" in r.stdout, r.stdout + r.stderr[-4000:]


@pytest.mark.parametrize("name,old,new,report", [
    ("read_one_past_the_weights",
     "            for (size_t p = 0; p < L; ++p)\n                acc += (e[p] / z)",
     "            for (size_t p = 0; p <= L; ++p)\n                acc += (e[p] / z)",
     "AddressSanitizer"),
    ("signed_shift_overflow",
     "    const double scale = 1.0 / sqrt((double)D);\n",
     "    const double scale = 1.0 / sqrt((double)D);\n"
     "    volatile int planted = (int)H + 1;\n    planted = planted << 31;\n",
     "runtime error"),
])
def test_sanitizers_report_planted_faults(tmp_path, name, old, new, report):
    """Controls: a planted heap over-read and a planted undefined shift in
    copies of the oracle are reported (the run fails, naming the sanitizer)."""
    src = open(oracle_build.SRC).read()
    assert src.count(old) == 1, name
    path = tmp_path / "planted.c"
    path.write_text(src.replace(old, new))
    lib = _build_oracle(str(path), str(tmp_path / "libplanted.so"))
    r = _child(RUN_PINS % lib)
    assert r.returncode != 0 and report in r.stderr, (name, r.returncode, r.stderr[-2000:])


def _sanitized_library():
    """The library with host-side sanitizers, built once per source state
    into _build/sanitized (git-ignored); the device code is built as usual,
    so the library loads exactly like the product one."""
    from decode_attention_kv_seq_amd import _build as lib_build
    units = list(lib_build.SOURCES)
    sources = units + [os.path.join(CSRC, "attn_internal.h"), os.path.join(ROOT, "include", "attn_decode.h")]
    h = hashlib.sha256()
    for p in sources:
        h.update(open(p, "rb").read())
    lib = os.path.join(SAN_DIR, "libattn_decode_san_%s.so" % h.hexdigest()[:16])
    if os.path.exists(lib):
        return lib
    os.makedirs(SAN_DIR, exist_ok=True)
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    host_san = []
    for f in SAN_FLAGS:
        host_san += ["-Xarch_host", f]
    objs, procs = [], []
    for src in units:
        obj = os.path.join(SAN_DIR, os.path.basename(src) + ".o")
        cmd = ([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + host_san +
               ["-x", "hip", "-c", "-I", os.path.join(ROOT, "include"), "-I", CSRC, src, "-o", obj])
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
        objs.append(obj)
    for p in procs:
        _, err = p.communicate()
        assert p.returncode == 0, err[-3000:]
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC"] + host_san + objs + ["-o", lib + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    for o in objs:
        os.remove(o)
    os.replace(lib + ".tmp", lib)
    return lib


@pytest.mark.skipif(__import__("torch").cuda.device_count() > 0,
                    reason="the ABI tests use stand-in device addresses: host-only")
def test_library_host_code_under_sanitizers():
    lib = _sanitized_library()
    code = ("import sys\nimport decode_attention_kv_seq_amd as ad\nad.load_library(%r)\n"
            "import pytest\nsys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', "
            "'tests/test_abi.py', 'tests/test_plan.py', 'tests/test_no_device.py']))\n" % lib)
    r = _child(code, timeout=900, runtime=_clang_runtime())
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout
