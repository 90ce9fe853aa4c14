"""Host-side sanitizer runs (CPU only).

* The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer runs
  the pins that need no torch.
* The library's host code (argument validation, workspace layout, path
  choice) built with AddressSanitizer on the host side only runs every
  validation case of the C-ABI; none reaches a HIP call, so no GPU is needed.
"""
import glob
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mxfp4_routed_expert_router_amd")


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd[:3])}...\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    so = str(tmp_path / "liboracle_asan.so")
    _run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
          "-o", so, os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True).stdout.strip()
    script = textwrap.dedent(f"""
        import sys
        sys.path.insert(0, {ROOT!r}); sys.path.insert(0, {os.path.join(ROOT, 'tests')!r})
        import oracle, pins
        o = oracle.Oracle({so!r})
        skip = {{"pin_ue8m0", "pin_e4m3_table"}}   # these import torch
        for pin in pins.ALL_PINS:
            if pin.__name__ not in skip:
                pin(o)
        print("pins ok under asan+ubsan")
    """)
    env = dict(os.environ, LD_PRELOAD=libasan, OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = _run([sys.executable, "-c", script], env=env, timeout=900)
    assert "pins ok" in r.stdout


def test_host_validation_under_asan(tmp_path):
    objs = sorted(glob.glob(os.path.join(PKG, "_build", "*.o")))
    api_o = os.path.join(PKG, "_build", "api.o")
    if api_o not in objs:
        pytest.skip("the library is not built (run the package build first)")
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rt:
        pytest.skip("no clang AddressSanitizer runtime")
    asan_api = str(tmp_path / "api_asan.o")
    hipcc = "/opt/rocm/bin/hipcc"
    _run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-c", os.path.join(PKG, "csrc", "api.hip"), "-o", asan_api])
    so = str(tmp_path / "libmoe_fp4_asan.so")
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", so, asan_api,
          *[o for o in objs if o != api_o]])
    script = textwrap.dedent(f"""
        import ctypes
        lib = ctypes.CDLL({so!r})
        FAKE = 0x7F0000000000
        class Dims(ctypes.Structure):
            _fields_ = [(n, ctypes.c_int32) for n in ("T", "H", "I", "E", "k")]
        class W(ctypes.Structure):
            _fields_ = [(n, ctypes.c_void_p) for n in ("w1", "s1", "w3", "s3", "w2", "s2")] + \\
                       [("expert_stride", ctypes.c_int64 * 6)]
        class R(ctypes.Structure):
            _fields_ = [(n, ctypes.c_void_p) for n in
                        ("topk_idx", "gates", "counts", "offsets", "sorted_pairs", "pair_slot")]
        P, SZ = ctypes.c_void_p, ctypes.c_size_t
        lib.moe_fp4_forward.argtypes = [ctypes.POINTER(Dims), P, P, ctypes.POINTER(W), P,
                                        ctypes.c_int, ctypes.c_int, P, SZ, P]
        lib.moe_fp4_route.argtypes = [ctypes.POINTER(Dims), P, ctypes.POINTER(R), P, SZ, P]
        lib.moe_fp4_workspace_size.argtypes = [ctypes.POINTER(Dims), ctypes.c_int, ctypes.POINTER(SZ)]
        lib.moe_fp4_route_workspace_size.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(SZ)]
        lib.moe_fp4_plan.argtypes = [ctypes.POINTER(Dims), ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
        lib.moe_fp4_status_string.restype = ctypes.c_char_p
        w = W(*([FAKE] * 6))
        n = SZ()
        calls = 0
        for T, H, I, E, k in ((1, 5120, 2304, 384, 6), (2048, 5120, 2304, 384, 6), (0, 64, 32, 4, 2),
                              (3, 48, 32, 4, 2), (4, 64, 32, 2000, 2), (4, 64, 32, 4, 5),
                              (65536, 64, 32, 4, 2), (16, 256, 128, 16, 2)):
            d = Dims(T, H, I, E, k)
            for mode in range(-1, 5):
                lib.moe_fp4_workspace_size(ctypes.byref(d), mode, ctypes.byref(n))
                path = ctypes.c_int()
                lib.moe_fp4_plan(ctypes.byref(d), mode, ctypes.byref(path))
                # workspace too small, misaligned or null pointers: refused before any HIP call
                for ws, nb, x in ((FAKE, 0, FAKE), (FAKE + 8, 1 << 40, FAKE), (FAKE, 1 << 40, None),
                                  (None, 1 << 40, FAKE), (FAKE, 1 << 40, FAKE + 2)):
                    rc = lib.moe_fp4_forward(ctypes.byref(d), x, FAKE, ctypes.byref(w), FAKE, mode, 0,
                                             ws, nb, None)
                    assert rc != 0, (T, H, I, E, k, mode, rc)
                    calls += 1
            lib.moe_fp4_route_workspace_size(ctypes.byref(d), ctypes.byref(n))
            r = R(*([FAKE] * 6))
            assert lib.moe_fp4_route(ctypes.byref(d), FAKE + 2, ctypes.byref(r), None, 0, None) != 0
        for s in range(-2, 8):
            lib.moe_fp4_status_string(s)
        print("validation ok under asan", calls)
    """)
    env = dict(os.environ, LD_PRELOAD=rt[0], ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               HIP_VISIBLE_DEVICES="")
    r = _run([sys.executable, "-c", script], env=env)
    assert "validation ok" in r.stdout
