"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Two CPU-only builds with gcc / g++ and -fsanitize=address,undefined (no GPU
code is involved): the oracle (oracle/oracle.c) and the library's host
packers (binary_bit_weight_amd/csrc/formats.cpp with status.cpp, the code
behind ll_packed_size, ll_pack_* / ll_unpack_*, ll_tq2_split,
ll_w1_from_dense and ll_validate).  Each runs in a child process with the
sanitizer runtimes preloaded and every report fatal:

  - the oracle's pin tests (tests/test_oracle_pins.py) against the
    sanitized oracle;
  - a driver that takes every packer through round trips, ragged and
    single-row shapes, the largest codes, invalid codes and the error paths
    (bad shapes, NULL pointers), checking each result.
"""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fPIC", "-shared"]


def _runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _env(extra):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan or shutil.which("g++") is None:
        pytest.skip("gcc sanitizer runtimes not available")
    env = dict(os.environ)
    env.update(extra)
    env["LD_PRELOAD"] = asan + ":" + ubsan
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["PYTHONPATH"] = os.pathsep.join([ROOT, os.path.join(ROOT, "tests")])
    return env


@pytest.fixture(scope="module")
def san_libs(tmp_path_factory):
    d = tmp_path_factory.mktemp("san")
    orc = d / "liboracle_san.so"
    subprocess.check_call(["gcc", *SAN, "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-o", str(orc),
                           os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    fmt = d / "libformats_san.so"
    csrc = os.path.join(ROOT, "binary_bit_weight_amd", "csrc")
    subprocess.check_call(["g++", *SAN, "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", csrc, "-o", str(fmt),
                           os.path.join(csrc, "formats.cpp"), os.path.join(csrc, "status.cpp")])
    return str(orc), str(fmt)


def test_oracle_pins_under_sanitizers(san_libs):
    orc, _ = san_libs
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       env=_env({"ORACLE_LIB_OVERRIDE": orc}), capture_output=True, text=True, cwd=ROOT, timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout


DRIVER = textwrap.dedent(r'''
    import ctypes as C, sys
    import numpy as np
    L = C.CDLL(sys.argv[1])
    P, I64, I32 = C.c_void_p, C.c_int64, C.c_int32
    L.ll_packed_size.restype = C.c_size_t
    L.ll_packed_size.argtypes = [I32, I64, I64, I32, P]
    for f, a in {"ll_pack_i2s": [P, I64, I64, C.c_float, P], "ll_unpack_i2s": [P, I64, I64, P, P],
                 "ll_pack_tq2": [P, P, I64, I64, P], "ll_unpack_tq2": [P, I64, I64, P, P],
                 "ll_tq2_split": [P, I64, I64, P, P], "ll_pack_w1": [P, I64, I64, P],
                 "ll_unpack_w1": [P, I64, I64, P], "ll_w1_from_dense": [P, I64, I64, I32, P, P],
                 "ll_validate": [I32, P, I64, I64, P]}.items():
        getattr(L, f).restype = C.c_int
        getattr(L, f).argtypes = a
    ptr = lambda a: a.ctypes.data_as(P)
    rng = np.random.default_rng(7)
    sizes = C.c_size_t()
    for N, K in [(1, 128), (3, 256), (5, 512), (17, 1280), (64, 768)]:
        # i2_s: exact buffer sizes, round trip, scale tail, invalid code
        n = L.ll_packed_size(1, N, K, 0, C.byref(sizes))
        assert n == N * K // 4 + 4 and sizes.value == 0
        w = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
        out = np.empty(n, np.uint8)
        assert L.ll_pack_i2s(ptr(w), N, K, 0.375, ptr(out)) == 0
        back, sc = np.empty((N, K), np.int8), C.c_float()
        assert L.ll_unpack_i2s(ptr(out), N, K, ptr(back), C.byref(sc)) == 0
        assert np.array_equal(back, w) and sc.value == 0.375
        bad = C.c_int64()
        assert L.ll_validate(1, ptr(out), N, K, C.byref(bad)) == 0 and bad.value == -1
        out[N * K // 4 - 1] |= 0x03
        assert L.ll_validate(1, ptr(out), N, K, C.byref(bad)) == -4 and 0 <= bad.value < N * K
        w2 = w.copy(); w2[N - 1, K - 1] = 2
        assert L.ll_pack_i2s(ptr(w2), N, K, 1.0, ptr(out)) == -4
        if K % 256 == 0:
            # TQ2_0: blocks, split layout, round trip, invalid code
            nb = L.ll_packed_size(2, N, K, 0, C.byref(sizes))
            assert nb == 66 * N * K // 256 and sizes.value == 2 * N * K // 256
            s16 = rng.integers(0, 0x7C00, size=N * K // 256).astype(np.uint16)
            blocks = np.empty(nb, np.uint8)
            assert L.ll_pack_tq2(ptr(w), ptr(s16), N, K, ptr(blocks)) == 0
            s_back = np.empty_like(s16)
            assert L.ll_unpack_tq2(ptr(blocks), N, K, ptr(back), ptr(s_back)) == 0
            assert np.array_equal(back, w) and np.array_equal(s_back, s16)
            codes, s_split = np.empty(N * K // 4, np.uint8), np.empty_like(s16)
            assert L.ll_tq2_split(ptr(blocks), N, K, ptr(codes), ptr(s_split)) == 0
            assert np.array_equal(s_split, s16)
            assert L.ll_validate(2, ptr(codes), N, K, C.byref(bad)) == 0 and bad.value == -1
            codes[-1] = 0xAA
            assert L.ll_validate(2, ptr(codes), N, K, C.byref(bad)) == -4
        else:
            assert L.ll_pack_tq2(ptr(w), None, N, K, None) != 0
        # W1: signs, round trip, from dense with every group size dividing K
        wb = np.where(rng.integers(0, 2, size=(N, K)) == 1, 1, -1).astype(np.int8)
        bits = np.empty((N, K // 32), np.uint32)
        assert L.ll_pack_w1(ptr(wb), N, K, ptr(bits)) == 0
        assert L.ll_unpack_w1(ptr(bits), N, K, ptr(back)) == 0 and np.array_equal(back, wb)
        assert L.ll_validate(3, ptr(bits), N, K, C.byref(bad)) == 0
        for G in (32, 64, 128, 256):
            if K % G:
                continue
            assert L.ll_packed_size(3, N, K, G, C.byref(sizes)) == N * K // 8 and sizes.value == 2 * N * K // G
            W = rng.standard_normal((N, K)).astype(np.float32)
            W[0, :] = 0.0
            s1 = np.empty((N, K // G), np.uint16)
            assert L.ll_w1_from_dense(ptr(W), N, K, G, ptr(bits), ptr(s1)) == 0
            assert L.ll_unpack_w1(ptr(bits), N, K, ptr(back)) == 0
            assert np.array_equal(back, np.where(W > 0, 1, -1).astype(np.int8))
            assert (s1[0] == 0).all()
    # error paths: shapes, NULL pointers, unknown formats
    one = np.zeros(4096, np.uint8)
    assert L.ll_packed_size(1, 4, 100, 0, None) == 0
    assert L.ll_packed_size(9, 4, 128, 0, None) == 0
    assert L.ll_pack_i2s(ptr(one), 1, 100, 1.0, ptr(one)) == -2
    assert L.ll_pack_i2s(None, 1, 128, 1.0, ptr(one)) == -1
    assert L.ll_unpack_i2s(ptr(one), 1, 128, None, None) == -1
    assert L.ll_pack_tq2(ptr(one), ptr(one), 1, 128, ptr(one)) == -2
    assert L.ll_pack_w1(ptr(one), 1, 40, ptr(one)) == -2
    assert L.ll_w1_from_dense(ptr(one), 1, 128, 96, ptr(one), ptr(one)) == -2
    assert L.ll_w1_from_dense(ptr(one), 1, 128, 0, ptr(one), ptr(one)) == -2
    assert L.ll_validate(7, ptr(one), 1, 128, None) == -1
    assert L.ll_validate(1, ptr(one), 1, 128, None) == 0
    print("packers ok")
''')


def test_host_packers_under_sanitizers(san_libs):
    _, fmt = san_libs
    r = subprocess.run([sys.executable, "-c", DRIVER, fmt], env=_env({}), capture_output=True, text=True, cwd=ROOT,
                       timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "packers ok" in r.stdout
