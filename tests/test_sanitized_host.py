"""The host-side C and C++ under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

The oracle (oracle/oracle.c) and the weight-image packer (block_format_gemv_amd/csrc/pack.cpp)
are built with gcc/g++ and -fsanitize=address,undefined, every finding fatal.  Then, in a child
process with libasan preloaded: every oracle pin (its mutant tests aside, which build unsanitized
variants) runs against the sanitized oracle, and the sanitized packer packs Q4_K-, Q6_K-, Q8_0-
and Q4_0-style fields of ragged shapes, checked byte for byte by the independent unpackers, and
meets each refusal (null pointers, out-of-range fields, inf/NaN scales, bad shapes).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_format_gemv_amd", "csrc")
ROCM_INCLUDE = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")

# the packer's only outside needs: the library's reason string and its setter
STUBS = r"""
#include <stdarg.h>
#include <stdio.h>
namespace qg {
static thread_local char reason[512];
int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(reason, sizeof reason, fmt, ap);
    va_end(ap);
    return status;
}
}  // namespace qg
extern "C" const char *qg_last_error(void) { return qg::reason; }
"""

PACK_CHECK = r"""
import ctypes, sys
import numpy as np
from workloads import gen
from image_layout import unpack_b32, unpack_q4k, unpack_q6k

L = ctypes.CDLL(sys.argv[1])
L.qg_image_bytes.restype = ctypes.c_size_t
L.qg_image_bytes.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64]
L.qg_last_error.restype = ctypes.c_char_p
vp = ctypes.c_void_p
i64 = ctypes.c_int64
L.qg_pack_q4k.argtypes = [i64, i64, vp, vp, vp, vp, vp, vp]
L.qg_pack_q6k.argtypes = [i64, i64, vp, vp, vp, vp]
L.qg_pack_b32.argtypes = [ctypes.c_int, i64, i64, vp, vp, vp]
Q4K, Q6K, Q8_0, Q4_0 = 1, 2, 3, 4
OK, E_INVALID, E_SHAPE, E_UNSUPPORTED, E_UNREADABLE = 0, 1, 2, 3, 4

def p(a):
    return None if a is None else a.ctypes.data_as(vp)

def pack(f):
    fmt = {"q4k": Q4K, "q6k": Q6K, "q8_0": Q8_0, "q4_0": Q4_0}[f["fmt"]]
    rows, cols = f["rows"], f["cols"]
    img = np.full(L.qg_image_bytes(fmt, rows, cols), 0xA5, np.uint8)   # padding must be written
    c = {k: np.ascontiguousarray(v) for k, v in f.items() if isinstance(v, np.ndarray)}
    if fmt == Q4K:
        st = L.qg_pack_q4k(rows, cols, p(c["q"].astype(np.uint8)), p(c["sc"].astype(np.uint8)),
                           p(c["mn"].astype(np.uint8)), p(c["d"].astype(np.uint16)), p(c["dmin"].astype(np.uint16)), p(img))
    elif fmt == Q6K:
        st = L.qg_pack_q6k(rows, cols, p(c["q"].astype(np.uint8)), p(c["sc"].astype(np.int8)),
                           p(c["d"].astype(np.uint16)), p(img))
    else:
        q = c["q"].astype(np.int8 if fmt == Q8_0 else np.uint8)
        st = L.qg_pack_b32(fmt, rows, cols, p(q), p(c["d"].astype(np.uint16)), p(img))
    return st, img

checked = 0
for rows, cols in [(1, 256), (5, 768), (64, 1024), (70, 512), (130, 1280), (3, 4096)]:
    f = gen.q4k_fields(rows, cols, rows + cols)
    st, img = pack(f)
    assert st == OK, L.qg_last_error()
    u = unpack_q4k(img, rows, cols)
    assert all(np.array_equal(u[k], f[k]) for k in ("q", "sc", "mn", "d", "dmin")), (rows, cols)
    f = gen.q6k_fields(rows, cols, rows + 2 * cols)
    st, img = pack(f)
    assert st == OK, L.qg_last_error()
    u = unpack_q6k(img, rows, cols)
    assert all(np.array_equal(u[k], f[k]) for k in ("q", "sc", "d")), (rows, cols)
    for fmt in ("q8_0", "q4_0"):
        f = (gen.q8_0_fields if fmt == "q8_0" else gen.q4_0_fields)(rows, cols, rows + 3 * cols)
        st, img = pack(f)
        assert st == OK, L.qg_last_error()
        u = unpack_b32(img, fmt == "q8_0", rows, cols)
        assert np.array_equal(u["q"], f["q"]) and np.array_equal(u["d"], f["d"]), (fmt, rows, cols)
    checked += 4

# refusals: each returns its status with a reason, writing nothing out of bounds
f = gen.q4k_fields(3, 512, 9)
f["q"][1, 7] = 16
assert pack(f)[0] == E_INVALID
f = gen.q4k_fields(3, 512, 9)
f["sc"][2, 3] = 64
assert pack(f)[0] == E_INVALID
f = gen.q4k_fields(3, 512, 9)
f["dmin"][0, 1] = 0x7E00
assert pack(f)[0] == E_UNREADABLE and b"row 0" in L.qg_last_error()
f = gen.q6k_fields(2, 256, 9)
f["q"][0, 0] = 64
assert pack(f)[0] == E_INVALID
f = gen.q6k_fields(2, 256, 9)
f["d"][1, 0] = 0xFC00
assert pack(f)[0] == E_UNREADABLE
f = gen.q8_0_fields(2, 256, 9)
f["d"][0, 3] = 0x7C00
assert pack(f)[0] == E_UNREADABLE
f = gen.q4_0_fields(2, 256, 9)
f["q"][1, 9] = 16
assert pack(f)[0] == E_INVALID
img = np.zeros(9216, np.uint8)
assert L.qg_pack_q4k(2, 300, None, None, None, None, None, p(img)) == E_SHAPE
assert L.qg_pack_q4k(2, 256, None, None, None, None, None, p(img)) == E_INVALID
assert L.qg_pack_q6k(2, 256, None, None, None, p(img)) == E_INVALID
assert L.qg_pack_b32(Q4K, 2, 256, None, None, p(img)) == E_INVALID
assert L.qg_pack_b32(Q8_0, 2, 0, None, None, p(img)) == E_SHAPE
assert L.qg_image_bytes(9, 64, 256) == 0 and L.qg_image_bytes(Q4K, 64, 100) == 0
print("packer checked on", checked, "shapes x formats")
"""


def _tool(name):
    path = shutil.which(name)
    if path is None:
        pytest.skip(f"{name} is not installed")
    return path


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    gcc, gxx = _tool("gcc"), _tool("g++")
    libasan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(libasan) or not os.path.exists(libasan):
        pytest.skip("gcc has no AddressSanitizer runtime")
    d = tmp_path_factory.mktemp("sanitized")
    sys.path.insert(0, ROOT)
    from oracle import build as obuild

    oracle_lib = obuild.build_sanitized(str(d / "liboracle_san.so"))
    stubs = d / "stubs.cpp"
    stubs.write_text(STUBS)
    pack_lib = str(d / "libqgpack_san.so")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-Wall", "-Werror", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
           "-I" + ROCM_INCLUDE, "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, os.path.join(CSRC, "pack.cpp"),
           str(stubs), "-o", pack_lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ)
    env.update({"LD_PRELOAD": libasan, "QG_ORACLE_LIB": oracle_lib,
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:detect_odr_violation=0",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
                "PYTHONPATH": os.pathsep.join([ROOT, os.path.join(ROOT, "tests")]), "OMP_NUM_THREADS": "4"})
    return {"oracle": oracle_lib, "pack": pack_lib, "env": env}


def test_oracle_pins_under_sanitizers(sanitized):
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_kv.py"), "-k", "not mutant"],
                       capture_output=True, text=True, env=sanitized["env"], cwd=ROOT, timeout=900)
    out = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
    assert " passed" in r.stdout


def test_packer_under_sanitizers(sanitized):
    r = subprocess.run([sys.executable, "-c", PACK_CHECK, sanitized["pack"]], capture_output=True, text=True,
                       env=sanitized["env"], cwd=ROOT, timeout=600)
    out = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
    assert "packer checked on 24" in r.stdout, out
