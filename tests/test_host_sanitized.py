"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

`api.cpp` and `codebook.cpp` (argument checks, workspace carving, launch shapes, the exact
fold of the double-quantization mean, the codebook tables) are built with g++
`-fsanitize=address,undefined` together with `tests/host_san/`: a host-only stand-in for
the HIP runtime and a driver that calls every entry point.  The kernel sources are built for
the host side only (their launchers), without instrumentation.  No kernel runs: the stand-in
records each launch and checks it against the hardware's launch limits.

Checks:
- the driver's own: every entry point returns QLORA_OK at shapes that reach each launch
  path, on exact-size buffers and workspaces of exactly the size asked for; every error case
  returns its status and launches nothing;
- the fold: the exact sum of a quantize exponent histogram, rounded once to double, equals
  the correctly rounded value computed here with integer arithmetic (Fraction), on edge
  histograms (empty, one bin, every bin full, ties to even, subnormal-only) and random ones;
- no sanitizer report.
"""

import concurrent.futures as cf
import os
import random
import shutil
import subprocess
from fractions import Fraction

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_nf4_quantized_dq_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_san")
OUT = os.path.join(ROOT, "_build", "host_san")
KERNEL_SOURCES = ["quantize", "dequant", "lora", "gemv", "gemv_stream", "gemm", "gemm_nt", "merge", "adamw", "mlp",
                  "noalloc", "gemv_rows"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
INC = ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", HERE]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(" ".join(cmd) + "\n" + r.stdout + r.stderr)


def _host_side(src):
    """The launcher half of a kernel source: host code only, no device code, no sanitizer."""
    obj = os.path.join(OUT, src + ".o")
    _run(["/opt/rocm/bin/hipcc", "-O1", "-fPIC", "-std=c++17", "-ffp-contract=off", *INC, "-x", "hip",
          "--offload-arch=gfx950", "--offload-host-only", "-c", os.path.join(CSRC, src + ".hip"), "-o", obj])
    return obj


def _sanitized(path):
    obj = os.path.join(OUT, os.path.splitext(os.path.basename(path))[0] + ".san.o")
    _run(["g++", "-O1", "-g", "-std=c++17", "-w", "-ffp-contract=off", "-D__HIP_PLATFORM_AMD__", "-I",
          "/opt/rocm/include", *INC, *SAN, "-c", path, "-o", obj])
    return obj


def _fatbin_stubs(objs):
    """Host-only objects refer to the device-code image of their source by a per-source
    symbol; the stand-in registers no images, so each symbol is given a dummy definition."""
    names = set()
    for o in objs:
        r = subprocess.run(["nm", "-u", o], capture_output=True, text=True, check=True)
        names.update(ln.split()[-1] for ln in r.stdout.splitlines() if "__hip_fatbin_" in ln)
    path = os.path.join(OUT, "fatbin_stubs.c")
    with open(path, "w") as f:
        for n in sorted(names):
            f.write(f"unsigned char {n}[16];\n")
    obj = os.path.join(OUT, "fatbin_stubs.o")
    _run(["gcc", "-c", path, "-o", obj])
    return obj


@pytest.fixture(scope="module")
def host_check():
    if not (shutil.which("g++") and os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("needs g++ and hipcc")
    os.makedirs(OUT, exist_ok=True)
    san_src = [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "codebook.cpp"),
               os.path.join(HERE, "sim_runtime.cpp"), os.path.join(HERE, "host_check.cpp")]
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 2)) as ex:
        kern = list(ex.map(_host_side, KERNEL_SOURCES))
        san = list(ex.map(_sanitized, san_src))
    exe = os.path.join(OUT, "host_check")
    _run(["g++", *SAN, "-o", exe, *san, *kern, _fatbin_stubs(kern), "-lpthread"])
    return exe


def _exact_double(hist):
    """sum_e hist[e] * 2^(e - 150) for e >= 1, rounded to the nearest double (ties to even)."""
    return float(Fraction(sum(h << (e - 1) for e, h in enumerate(hist) if e >= 1), 1 << 149))


def _histograms():
    rng = random.Random(20240531)
    top = (1 << 64) - 1
    H = [[0] * 256]
    for e in (1, 2, 126, 127, 150, 254, 255):
        h = [0] * 256
        h[e] = rng.randrange(1, 1 << 24)
        H.append(h)
    H.append([0] + [top] * 255)                    # every bin full
    H.append([0, top] + [0] * 254)                 # subnormal constants only
    # halfway cases: 2^53 + 1 units of one bin (ties to even, down) and 2^53 + 3 (up)
    for odd in (1, 3):
        h = [0] * 256
        h[100] = (1 << 53) + odd
        H.append(h)
    # a halfway pattern that a sticky bit far below breaks
    h = [0] * 256
    h[200] = (1 << 53) + 1
    h[1] = 1
    H.append(h)
    # typical tensors: block constants around 2^-5 .. 2^-3, counts up to 2^26 blocks
    for _ in range(40):
        h = [0] * 256
        for e in range(118, 126):
            h[e] = rng.randrange(0, 1 << 26) * rng.randrange(1 << 23, 1 << 24)
        H.append(h)
    for _ in range(40):
        H.append([0] + [rng.randrange(0, 1 << rng.randrange(1, 65)) for _ in range(255)])
    return H


def test_host_code_under_sanitizers(host_check, tmp_path):
    H = _histograms()
    path = tmp_path / "hist.txt"
    path.write_text("\n".join(" ".join(str(v) for v in h) for h in H) + "\n")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([host_check, str(path)], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout.splitlines()
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-8000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-8000:]
    assert out[-1].startswith("OK ") and int(out[-1].split()[1]) > 500, out[-3:]
    folds = [float.fromhex(ln.split()[1]) for ln in out if ln.startswith("FOLD ")]
    assert len(folds) == len(H)
    for i, (h, got) in enumerate(zip(H, folds)):
        assert got == _exact_double(h), (i, got, _exact_double(h))
