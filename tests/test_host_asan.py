"""AddressSanitizer run of the library's host code: argument validation,
workspace sizing, split planning and the status strings.

The library's sources are compiled with -fsanitize=address on the host side
only (the device code is built without it) into a separate shared object,
which a child Python
process loads under the ASan runtime and drives through every entry point's
host-side paths: valid and invalid configurations (fuzzed fields, extreme
sizes, NaN / infinite limits, unknown modes and layouts), NULL pointers,
misaligned pointers, short workspaces and oversized batches.  Every such call returns before
anything would be launched, so no GPU is needed.  ASan aborts the child on
any out-of-bounds access or use of freed memory.  Host only: this test never
runs on a GPU machine's test pass.
"""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mxfp4_quantized_weights_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"

DRIVER = textwrap.dedent(r'''
    import ctypes, math, random, sys
    lib = ctypes.CDLL(sys.argv[1])
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t

    class Pad(ctypes.Structure):
        _fields_ = [("hidden", I32), ("hidden_padded", I32), ("inter", I32), ("inter_padded", I32)]

    class Cfg(ctypes.Structure):
        _fields_ = [("num_experts", I32), ("top_k", I32), ("quant_mode", I32), ("gate_mode", I32),
                    ("weight_layout", I32), ("block_m", I32), ("swiglu_limit", ctypes.c_float), ("pad", Pad)]

    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_workspace_bytes.restype = SZ
    lib.moe_splitk_bytes.restype = SZ
    for s in list(range(-3, 12)) + [2**31 - 1, -2**31]:
        assert lib.moe_status_string(s)
    TILED = 0x4D310002
    FAKE = P(1 << 40)      # never dereferenced: every call below is refused first
    rng = random.Random(7)
    vals = [-(2**31), -129, -1, 0, 1, 2, 7, 8, 16, 17, 32, 64, 100, 128, 129, 255, 256, 288, 1000, 1023,
            1024, 1025, 4000, 4096, 65536, 65537, 2**30, 2**31 - 1]
    limits = [float("nan"), float("inf"), -1.0, 0.0, 1e-30, 10.0, 3.4e38]
    ok = 0
    for it in range(20000):
        h = rng.choice(vals); hp = rng.choice([h, (h + 127) // 128 * 128 if 0 < h < 2**30 else h, rng.choice(vals)])
        i = rng.choice(vals); ip = rng.choice([i, (i + 127) // 128 * 128 if 0 < i < 2**30 else i, rng.choice(vals)])
        c = Cfg(rng.choice(vals), rng.choice([-1, 0, 1, 2, 8, 16, 17, 1024]), rng.choice([-1, 0, 1, 2, 3, 4]),
                rng.choice([0, 0, 0, 1, 7]), rng.choice([TILED, TILED, 0, 12345]), rng.choice([0, 8, 16, 32, 64, 128, 256]),
                rng.choice(limits), Pad(h, hp, i, ip))
        T = rng.choice([-1, 0, 1, 7, 64, 4096, 2**21, 2**24, 2**31 - 1])
        st = lib.moe_validate_cfg(ctypes.byref(c))
        ok += st == 0
        lib.moe_workspace_bytes(ctypes.byref(c), T)
        for which in (13, 2, 7):
            lib.moe_plan_ksplit(ctypes.byref(c), T, which)
            for ks in (-16, -8, -3, -2, 1, 2, 3, 4, 8, 16):
                lib.moe_splitk_bytes(ctypes.byref(c), T, which, ks)
            a, b = SZ(), SZ()
            lib.moe_preshuffled_bytes(ctypes.byref(c), which, ctypes.byref(a), ctypes.byref(b))
        a, b = SZ(), SZ()
        lib.moe_intermediate_bytes(ctypes.byref(c), T, ctypes.byref(a), ctypes.byref(b))
        lib.moe_max_blocks(T if T < 2**31 else -1, c.num_experts, c.block_m)
        # the layer entry points, refused before any launch: NULL x / NULL
        # workspace / a 1-byte workspace / the no-allocation entry point with a
        # NULL argument
        lib.moe_forward(ctypes.byref(c), T, None, I64(h), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, I64(h), FAKE, SZ(1 << 40), None)
        lib.moe_forward(ctypes.byref(c), T, FAKE, I64(h), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, I64(h), None, SZ(0), None)
        if T > 0 and st == 0:
            assert lib.moe_forward(ctypes.byref(c), T, FAKE, I64(h), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, I64(h), FAKE,
                                   SZ(1), None) != 0
        lib.moe_forward_noalloc(ctypes.byref(c), T, FAKE, I64(h), None, FAKE, FAKE, FAKE, FAKE, FAKE, I64(h), None)
        lib.moe_grouped_gemm1_swiglu(ctypes.byref(c), T, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
        lib.moe_grouped_gemm1_swiglu_splitk(ctypes.byref(c), T, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                            rng.choice([-8, -2, 2, 3, 8]), None, SZ(0), None)
        lib.moe_grouped_gemm2_combine(ctypes.byref(c), T, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      I64(h), FAKE, SZ(0), None)
        lib.moe_grouped_gemm2_combine_splitk(ctypes.byref(c), T, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                             I64(h), rng.choice([1, 2, 4]), FAKE, SZ(0), None)
        lib.moe_route_permute_quant(ctypes.byref(c), T, None, FAKE, I64(h), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    FAKE, None)
        lib.moe_preshuffle_weights(ctypes.byref(c), rng.choice([13, 2, 0]), None, FAKE, FAKE, FAKE, None)
        lib.moe_decode_supported(ctypes.byref(c), T)
        lib.moe_decode_gemm1_swiglu(ctypes.byref(c), T, FAKE, FAKE, None, FAKE, FAKE, FAKE, None)
        lib.moe_decode_gemm1_swiglu(ctypes.byref(c), T, P((1 << 40) + 8), FAKE, FAKE, FAKE, FAKE, FAKE, None)
        lib.moe_decode_gemm2_combine(ctypes.byref(c), T, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, I64(h), None, FAKE,
                                     None)
        lib.moe_decode_gemm2_combine(ctypes.byref(c), T, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, I64(h), FAKE, FAKE,
                                     None) if T == 0 or lib.moe_decode_supported(ctypes.byref(c), T) == 0 else None
        E, k = c.num_experts, c.top_k
        lib.moe_route_topk(None, T, E, k, FAKE, FAKE, None)
        lib.moe_permute_align(FAKE, T, k, E, c.block_m, FAKE, FAKE, None, FAKE, None)
        lib.moe_quant_act(None, rng.choice([0, 1, 2, 3]), T, h, I64(hp), hp, c.quant_mode, FAKE, FAKE, None)
        lib.moe_quant_weights(c.quant_mode, None, E, i, h, FAKE, FAKE, None)
    for kind in (-1, 0, 1, 2):
        lib.moe_diag_mfma_tile(kind, None, FAKE, FAKE, None)
    lib.moe_diag_mfma_tile(0, P((1 << 40) + 4), FAKE, FAKE, None)
    lib.moe_validate_cfg(None)
    lib.moe_workspace_bytes(None, 1)
    print("valid configurations seen:", ok)
''')


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not found")
def test_host_code_under_asan(tmp_path):
    flags = ["--offload-arch=gfx950", "-O1", "-std=c++20", "-fPIC", "-Xarch_host", "-g",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    objs = [str(tmp_path / f"{src}.o") for src in ("api", "route", "quant", "gemm", "diag", "decode")]
    procs = [subprocess.Popen([HIPCC, *flags, "-c", os.path.join(CSRC, os.path.basename(o)[:-2] + ".hip"), "-o", o],
                              stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True) for o in objs]
    for p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, out
    so = tmp_path / "libmoe_asan.so"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address", *objs,
                        "-o", str(so)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    syms = subprocess.run(["/opt/rocm/llvm/bin/llvm-objdump", "-T", str(so)], capture_output=True,
                          text=True).stdout
    assert "__asan_report_load" in syms, "the host code is not instrumented"
    rt = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    assert os.path.exists(rt)
    drv = tmp_path / "drive.py"
    drv.write_text(DRIVER)
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, str(drv), str(so)], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0 and "AddressSanitizer" not in r.stderr, r.stdout[-3000:] + r.stderr[-6000:]
    assert "valid configurations seen:" in r.stdout
