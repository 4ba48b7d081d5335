"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

oracle/oracle.c is compiled together with tests/oracle_sanitized_driver.c
with ``-fsanitize=address,undefined -fno-sanitize-recover=all``, and the
driver runs every oracle routine on small seeded cases whose buffers are
allocated to the exact sizes the routines' contracts give: ragged column
counts (padding columns in the packed layout), a ragged last k-tile, group
size equal to K, both weight widths, both half formats, and a shape the
packed layout rejects.  Any out-of-bounds access, leak or undefined behaviour
ends the run with a sanitizer report; the driver's own round-trip checks end
it with a FAIL line.  The numeric outputs must equal the ordinary build's bit
for bit, so the instrumented build checks the same code the other tests use.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from synth import make_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER_SRC = os.path.join(ROOT, "tests", "oracle_sanitized_driver.c")
ORACLE_SRC = os.path.join(ROOT, "oracle", "oracle.c")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1",
             "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-Wall"]

# (bits, M, K, N, G, dtype)
CASES = [
    (4, 3, 256, 40, 32, "bf16"),   # 40 columns: the last 16-column block is half padding
    (4, 1, 384, 24, 128, "f16"),
    (4, 4, 96, 8, 96, "bf16"),     # one k-tile shorter than 128 rows, G = K, a single 8-column word
    (8, 2, 160, 24, 32, "bf16"),   # ragged last k-tile (160 = 128 + 32)
    (8, 5, 96, 16, 96, "f16"),
    (8, 2, 64, 10, 16, "bf16"),    # G = 16: dequant and linear only, the packed layout rejects it
]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not installed")
    exe = str(tmp_path_factory.mktemp("asan") / "oracle_sanitized_driver")
    subprocess.check_call(["gcc", *SAN_FLAGS, DRIVER_SRC, ORACLE_SRC, "-o", exe, "-lm"])
    return exe


def _write(d, name, a):
    np.ascontiguousarray(a).tofile(os.path.join(d, name))


def _read(d, name, dtype):
    return np.fromfile(os.path.join(d, name), dtype=dtype)


@pytest.mark.parametrize("bits,M,K,N,G,dtype", CASES)
def test_oracle_clean_under_sanitizers(driver, tmp_path, bits, M, K, N, G, dtype):
    case = make_inputs(bits, M, K, N, G, seed=(77, bits, K, N, G), dtype=dtype)
    cols = np.array(sorted({0, N - 1, N // 2, (5 * N) // 7}), dtype=np.int64)
    d = str(tmp_path)
    with open(os.path.join(d, "spec.txt"), "w") as f:
        f.write(f"{bits} {M} {K} {N} {G} {oracle.FORMATS[dtype]} {cols.size}\n")
    _write(d, "qweight.bin", case.qweight)
    _write(d, "qzeros.bin", case.qzeros)
    _write(d, "scales.bin", case.scales)
    _write(d, "x.bin", case.x)
    _write(d, "cols.bin", cols)
    env = dict(os.environ, OMP_NUM_THREADS="4", ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([driver, d], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "OK", r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr

    # the instrumented build computes what the ordinary build computes
    w = oracle.dequant(bits, case.qweight, case.qzeros, case.scales, K, N, G, dtype=dtype)
    y = oracle.linear(case.x, w, dtype=dtype)
    assert np.array_equal(_read(d, "y.bin", np.float64).view(np.uint64), y.reshape(-1).view(np.uint64))
    rounded = oracle.f64_to_f16(y) if dtype == "f16" else oracle.f64_to_bf16(y)
    assert np.array_equal(_read(d, "out.bin", np.uint16), rounded.reshape(-1))
    if N % 2 == 0:
        s = oracle.silu_mul(y[0, : N // 2], y[0, N // 2 :])
        assert np.array_equal(_read(d, "silu.bin", np.float64).view(np.uint64), s.view(np.uint64))
    if oracle.packed_bytes(bits, K, N, G):
        ref = oracle.repack(bits, case.qweight, case.qzeros, case.scales, K, N, G)
        assert np.array_equal(_read(d, "packed.bin", np.uint8), ref)
    else:
        assert not os.path.exists(os.path.join(d, "packed.bin"))
