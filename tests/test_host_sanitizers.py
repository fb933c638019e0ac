"""Host AddressSanitizer / UndefinedBehaviorSanitizer builds of the CPU oracle and of the C-ABI
layer (CPU only: no GPU code is instrumented and no kernel is launched).

* The oracle (oracle/convrot_oracle.c) is compiled with gcc -fsanitize=address,undefined together
  with tests/sanitize/oracle_driver.c, which calls every oracle function on exactly-sized heap
  buffers, on its error paths and at its edge cases.
* The C-ABI layer (csrc/convrot_abi.hip) is compiled with its host side instrumented
  (hipcc -Xarch_host -fsanitize=...) and linked with the library's other objects into a C driver
  generated from the host-side ABI cases of test_abi_host.py: every precondition violation (fake,
  never-dereferenced pointers), the empty-input no-ops, the size queries at their edges (huge
  M, N and K included, where a signed overflow would be reported), the status strings, and one
  call that passes every check and stops at the missing device.

Any sanitizer report makes the driver exit non-zero (-fno-sanitize-recover=all).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_SRC = os.path.join(ROOT, "oracle", "convrot_oracle.c")
ORACLE_DRIVER = os.path.join(HERE, "sanitize", "oracle_driver.c")
ABI_SRC = os.path.join(ROOT, "int4_quantized_linear_amd", "csrc", "convrot_abi.hip")
INCLUDE = os.path.join(ROOT, "include")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")

SAN_ENV = dict(os.environ, UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\nexit %d\n%s\n%s" % (" ".join(cmd), r.returncode, r.stdout[-4000:], r.stderr[-4000:])
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_asan")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-ffp-contract=off", "-fopenmp", "-o", exe, ORACLE_SRC, ORACLE_DRIVER, "-lm"])
    r = _run([exe], env=dict(SAN_ENV, ASAN_OPTIONS="detect_leaks=1"))
    assert "all checks held" in r.stdout


# ---------------------------------------------------------------------------------------- ABI

def _c_arg(value, ctype) -> str:
    import ctypes
    if ctype in (ctypes.c_void_p, ctypes.c_char_p):
        return "NULL" if value is None else "(void *)(uintptr_t)0x%xull" % value
    if value is None:
        return "0"
    if ctype in (ctypes.c_int64, ctypes.c_longlong):
        return "(int64_t)%dll" % value
    if ctype in (ctypes.c_size_t, ctypes.c_uint64, ctypes.c_ulonglong):
        return "(size_t)%dull" % value
    return "%d" % value


def _abi_driver_source() -> str:
    from tests import test_abi_host as T
    cr = T.cr
    lines = ['#include <stdint.h>', '#include <stdio.h>', '#include <string.h>', '#include "convrot.h"', '',
             'static int failures = 0;',
             'static void expect(const char *what, int rc, int want, const char *name) {',
             '    const char *msg = convrot_last_error();',
             '    if (rc != want) { fprintf(stderr, "%s: rc %d, expected %d (%s)\\n", what, rc, want, msg); ++failures; }',
             '    else if (name && want != 0 && !strstr(msg, name)) {',
             '        fprintf(stderr, "%s: message does not name %s: %s\\n", what, name, msg); ++failures; }',
             '}', '', 'int main(void) {']
    for i, (name, args, status) in enumerate(T.CASES):
        argt, _ = cr.SIGNATURES[name]
        cargs = ", ".join(_c_arg(a, t) for a, t in zip(args, argt))
        lines.append('    expect("case %d %s", %s(%s), %d, "%s");' % (i, name, name, cargs, T.ERR[status], name))
    # empty inputs: OK without pointers or a device
    empties = [
        ("convrot_quantize_act", (None, 1, 0, 512, 256, 8, None, None, None)),
        ("convrot_linear", (None, 1, None, None, 0, 256, 512, 256, None, None, None, None, None, 0, None)),
        ("convrot_linear", (None, 1, None, None, 16, 0, 512, 256, None, None, None, None, None, 0, None)),
        ("convrot_linear_noalloc", (None, 1, None, None, 0, 256, 512, 256, None, None, None, None, None)),
        ("convrot_linear_w4a4", (None, 1, None, None, 0, 256, 512, 256, None, None, None, None, None, 0, None)),
        ("convrot_linear_w4a8", (None, 1, None, None, 0, 256, 512, 256, None, 0, None, None, None, 0, None)),
        ("convrot_pack_weight_w4a8", (None, None, 0, 512, None, None)),
        ("convrot_pack_weight_w4a4", (None, 0, 512, None, None)),
        ("convrot_gemm_i8_i32", (None, None, 0, 256, 512, None, None, 0, None)),
    ]
    for name, args in empties:
        argt, _ = cr.SIGNATURES[name]
        lines.append('    expect("empty %s", %s(%s), 0, NULL);' % (name, name, ", ".join(_c_arg(a, t) for a, t in zip(args, argt))))
    # a call that passes every host check and stops at the missing device
    M, N, K = 64, 1024, 512
    lines.append('    { size_t ws = convrot_workspace_bytes(%d, 0, %d, 4);' % (M, K))
    lines.append('      expect("packed w4a4 reaches the device", convrot_linear_w4a4_packed((void *)0x100000, 1, NULL, NULL, '
                 '%d, %d, %d, 256, (void *)0x200000, (void *)0x300000, NULL, (void *)0x400000, (void *)0x500000, ws, NULL), '
                 '%d, "hipGetDevice"); }' % (M, N, K, T.ERR["CONVROT_ERR_HIP"]))
    # size queries and pure helpers at their edges (results are checked by test_abi_host; here only
    # that no undefined behaviour or out-of-bounds access happens on the way)
    big = [(1 << 62), (1 << 40), (1 << 31), (1 << 31) - 1, 131072, 133144, -1, 0, 1, 17]
    lines.append('    volatile size_t sink = 0;')
    lines.append('    const int64_t v[] = {%s};' % ", ".join("(int64_t)%dll" % b for b in big))
    lines.append('    const int nv = (int)(sizeof v / sizeof v[0]);')
    lines.append('    for (int a = 0; a < nv; ++a) for (int b = 0; b < nv; ++b) for (int c = 0; c < nv; ++c) {')
    lines.append('        sink += convrot_workspace_bytes(v[a], v[b], v[c], 8) + convrot_workspace_bytes(v[a], v[b], v[c], 4);')
    lines.append('        sink += convrot_workspace_bytes_w4a8(v[a], v[b], v[c]);')
    lines.append('        sink += convrot_packed_bytes_w4a8(v[a], v[b]) + convrot_packed_bytes_w4a4(v[a], v[b]);')
    lines.append('        sink += convrot_packed_bytes_w4a8_group(v[a], v[b], 128) + convrot_packed_bytes_w4a8_group(v[a], v[b], 256);')
    lines.append('        sink += (size_t)convrot_dynamic_group(v[a], (int)(v[b] & 0x7fffffff));')
    lines.append('    }')
    lines.append('    for (int s = -3; s < 40; ++s) sink += strlen(convrot_status_string(s));')
    lines.append('    (void)sink;')
    lines.append('    if (failures) fprintf(stderr, "%d ABI checks failed\\n", failures);')
    lines.append('    else printf("ABI sanitizer driver: all checks held\\n");')
    lines.append('    return failures ? 1 : 0;')
    lines.append('}')
    return "\n".join(lines) + "\n"


def test_abi_host_code_under_asan_ubsan(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm toolchain not available")
    if os.path.exists("/dev/kfd"):
        pytest.skip("host-only check (fake device pointers)")
    pytest.importorskip("int4_quantized_linear_amd.convrot")
    from int4_quantized_linear_amd import build as B
    objs = [os.path.join(B.HERE, "_build", s.replace(".hip", ".o")) for s in B.SOURCES if s != "convrot_abi.hip"]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    abi_obj = str(tmp_path / "convrot_abi_asan.o")
    _run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=" + B.ARCH, *B.DEVICE_FLAGS,
          "-Wno-unused-command-line-argument", *san, "-c", ABI_SRC, "-o", abi_obj])
    drv_c = tmp_path / "abi_driver.c"
    drv_c.write_text(_abi_driver_source())
    drv_obj = str(tmp_path / "abi_driver.o")
    _run([CLANG, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE, "-I", os.path.join(ROCM, "include"),
          "-c", str(drv_c), "-o", drv_obj])
    exe = str(tmp_path / "abi_asan")
    _run([HIPCC, "--offload-arch=" + B.ARCH, *san, "-o", exe, drv_obj, abi_obj, *objs])
    # the HIP runtime keeps allocations until exit: leak checking would report those
    r = _run([exe], env=dict(SAN_ENV, ASAN_OPTIONS="detect_leaks=0"))
    assert "all checks held" in r.stdout
