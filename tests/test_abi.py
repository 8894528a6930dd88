"""Host-side tests of the C ABI (no GPU needed).

- libmoe.so loads and exports every function include/moe.h declares;
- every rejected configuration returns its status code before anything is
  enqueued (sglang PR #38546 "[AMD] [GLM-5.3-Flash Day 0] Enable FP8 and Quark
  MXFP4 MoE on gfx950", contract table: unsupported configurations fail at
  construction; gate mode explicit; limit forwarded; layout owned by the
  runner; padding metadata).  These calls return before any HIP call, so
  they are safe without a GPU; the pointer arguments are never dereferenced.
- workspace / block-count / buffer-size arithmetic.
"""
import ctypes
import math
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
LIB = os.path.join(ROOT, "mxfp4_quantized_weights_amd", "libmoe.so")

if not os.path.exists(LIB):  # CPU host without a prior build: build here (cross-compile)
    import importlib.util  # noqa: E402
    _spec = importlib.util.spec_from_file_location("_moe_build", os.path.join(ROOT, "mxfp4_quantized_weights_amd",
                                                                            "build.py"))
    _build = importlib.util.module_from_spec(_spec)
    _spec.loader.exec_module(_build)  # the package itself needs the library to import
    _build.build()

import mxfp4_quantized_weights_amd as M  # noqa: E402

FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
OK, NULL, SHAPE, ALIGN, UNSUP, LAYOUT, WS = 0, 1, 2, 3, 4, 5, 6


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_abi():
    names = _declared_functions()
    for must in ("moe_route_topk", "moe_permute_align", "moe_quant_act", "moe_grouped_gemm1_swiglu",
                 "moe_grouped_gemm2_combine", "moe_forward", "moe_workspace_bytes",
                 "moe_preshuffle_weights", "moe_status_string"):
        assert must in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], stdout=subprocess.PIPE, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)", out))
    declared = set(_declared_functions())
    assert declared <= exported, declared - exported
    assert declared == set(M.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(M.lib(), name)


def cfg(**kw):
    base = dict(num_experts=288, top_k=8, quant="fp8", hidden=4096, inter=1024, block_m=16)
    base.update(kw)
    return M.make_cfg(validate=False, **base)


def status(c):
    return M.validate_cfg(c)


def test_valid_configs():
    assert status(cfg()) == OK
    assert status(cfg(quant="mxfp4")) == OK
    assert status(cfg(quant="fp8_ue8m0")) == OK
    assert status(cfg(hidden=4000, inter=1000, hidden_padded=4096, inter_padded=1024)) == OK
    assert status(cfg(swiglu_limit=math.inf)) == OK
    for bm in (16, 32, 64, 128):
        assert status(cfg(block_m=bm)) == OK
    assert status(cfg(num_experts=1, top_k=1)) == OK
    assert status(cfg(num_experts=16, top_k=16)) == OK


@pytest.mark.parametrize("kw,code", [
    (dict(gate_mode=M.MOE_GATE_INTERLEAVED), UNSUP),
    (dict(gate_mode=7), UNSUP),
    (dict(quant=4), UNSUP),
    (dict(quant=0), UNSUP),
    (dict(block_m=48), UNSUP),
    (dict(block_m=256), UNSUP),
    (dict(swiglu_limit=0.0), UNSUP),
    (dict(swiglu_limit=-10.0), UNSUP),
    (dict(swiglu_limit=math.nan), UNSUP),
    (dict(hidden=4000, hidden_padded=4000), ALIGN),
    (dict(inter_padded=1000, inter=1000), ALIGN),
    (dict(hidden=4100, hidden_padded=4096), SHAPE),
    (dict(top_k=9, num_experts=8), SHAPE),
    (dict(top_k=17, num_experts=64), SHAPE),
    (dict(top_k=0), SHAPE),
    (dict(num_experts=0), SHAPE),
    (dict(num_experts=1025), SHAPE),
    (dict(hidden=0), SHAPE),
])
def test_rejected_configs(kw, code):
    assert status(cfg(**kw)) == code
    # the same rejection through every entry point that takes a cfg
    c = cfg(**kw)
    assert M.workspace_bytes(c, 64) == 0
    lib = M.lib()
    r = lib.moe_forward(ctypes.byref(c), 64, FAKE, 4096, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, FAKE, 1 << 40,
                        None)
    assert r == code


def test_null_cfg():
    assert M.lib().moe_validate_cfg(None) == NULL
    assert M.lib().moe_workspace_bytes(None, 4) == 0


def test_layout_tag_is_owned_by_the_runner():
    c = cfg(weight_layout=M.MOE_LAYOUT_CANONICAL)
    assert status(c) == OK  # a valid cfg ...
    lib = M.lib()
    r = lib.moe_forward(ctypes.byref(c), 64, FAKE, 4096, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, FAKE, 1 << 40, None)
    assert r == LAYOUT      # ... whose weights were not preshuffled by this library
    r = lib.moe_grouped_gemm1_swiglu(ctypes.byref(c), 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert r == LAYOUT
    c2 = cfg(weight_layout=0x1234)
    r = lib.moe_grouped_gemm2_combine(ctypes.byref(c2), 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      4096, FAKE, 1 << 40, None)
    assert r == LAYOUT


def test_short_workspace_and_bad_strides():
    c = cfg()
    need = M.workspace_bytes(c, 64)
    assert need > 0
    lib = M.lib()
    args = lambda ws, ldx=4096, ldo=4096: (ctypes.byref(c), 64, FAKE, ldx, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ldo,
                                            FAKE, ws, None)
    assert lib.moe_forward(*args(need - 1)) == WS
    assert lib.moe_forward(*args(need, ldx=4095)) == SHAPE
    assert lib.moe_forward(*args(need, ldo=100)) == SHAPE
    # null pointers are reported before the workspace is looked at
    assert lib.moe_forward(ctypes.byref(c), 64, None, 4096, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, FAKE, need,
                           None) == NULL
    # T = 0 is a valid no-op
    assert lib.moe_forward(ctypes.byref(c), 0, None, 4096, None, None, None, None, None, None, 4096, None, 0,
                           None) == OK
    assert lib.moe_forward(ctypes.byref(c), -1, FAKE, 4096, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, FAKE, need,
                           None) == SHAPE


def test_stage_entry_points_validate_before_launch():
    lib = M.lib()
    assert lib.moe_route_topk(FAKE, 4, 8, 9, FAKE, FAKE, None) == SHAPE
    assert lib.moe_route_topk(FAKE, 4, 8, 17, FAKE, FAKE, None) == SHAPE
    assert lib.moe_route_topk(None, 0, 8, 2, None, None, None) == OK
    assert lib.moe_route_topk(None, 4, 8, 2, FAKE, FAKE, None) == NULL
    assert lib.moe_permute_align(FAKE, 4, 2, 8, 8, FAKE, FAKE, FAKE, FAKE, None) == UNSUP
    assert lib.moe_permute_align(FAKE, 4, 2, 2000, 16, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
    assert lib.moe_quant_act(FAKE, 9, 4, 128, 128, 128, 1, FAKE, FAKE, None) == UNSUP
    assert lib.moe_quant_act(FAKE, 1, 4, 128, 128, 128, 5, FAKE, FAKE, None) == UNSUP
    assert lib.moe_quant_act(FAKE, 1, 4, 100, 100, 100, 1, FAKE, FAKE, None) == ALIGN
    assert lib.moe_quant_act(FAKE, 1, 4, 200, 200, 128, 1, FAKE, FAKE, None) == SHAPE
    assert lib.moe_quant_act(FAKE, 1, 4, 128, 64, 128, 1, FAKE, FAKE, None) == SHAPE
    assert lib.moe_quant_act(None, 1, 0, 128, 128, 128, 1, None, None, None) == OK
    assert lib.moe_quant_weights(1, FAKE, 2, 100, 128, FAKE, FAKE, None) == ALIGN
    assert lib.moe_quant_weights(2, FAKE, 2, 100, 96, FAKE, FAKE, None) == ALIGN
    assert lib.moe_quant_weights(7, FAKE, 2, 128, 128, FAKE, FAKE, None) == UNSUP
    assert lib.moe_quant_weights(3, FAKE, 2, 128, 96, FAKE, FAKE, None) == ALIGN
    assert lib.moe_quant_act(FAKE, 1, 4, 100, 100, 100, 3, FAKE, FAKE, None) == ALIGN
    c = cfg()
    assert lib.moe_preshuffle_weights(ctypes.byref(c), 3, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
    assert lib.moe_preshuffle_weights(ctypes.byref(c), 13, None, FAKE, FAKE, FAKE, None) == NULL


def test_status_strings():
    for code in range(8):
        s = M.lib().moe_status_string(code).decode()
        assert s.startswith(M.STATUS_NAMES[code])


def test_block_and_buffer_sizes():
    import oracle as O
    for P, E, BM in [(512, 288, 16), (32768, 288, 128), (8, 288, 16), (0, 8, 16), (16384, 288, 64), (5, 1, 128)]:
        assert M.max_blocks(P, E, BM) == O.max_blocks(P, E, BM)
    c = cfg(quant="fp8", block_m=128)
    aq, as_ = M.intermediate_bytes(c, 4096)
    rows = O.max_blocks(4096 * 8, 288, 128) * 128
    assert (aq, as_) == (rows * 1024, rows * 8 * 4)
    c = cfg(quant="mxfp4", block_m=128)
    assert M.intermediate_bytes(c, 4096) == (rows * 512, rows * 32)
    # UE8M0: one scale byte per 128 columns, rows rounded up to whole dwords
    c = cfg(quant="fp8_ue8m0", block_m=128)
    assert M.intermediate_bytes(c, 4096) == (rows * 1024, rows * 8)
    c = cfg(quant="fp8_ue8m0", block_m=128, inter=128)
    assert M.intermediate_bytes(c, 4096) == (rows * 128, rows * 4)
    assert M.e8_scale_ld(128) == 4 and M.e8_scale_ld(4096) == 32 and M.e8_scale_ld(4224) == 36
    # TILED_V2 keeps UE8M0 block scales as fp32 values
    assert M.preshuffled_bytes(cfg(quant="fp8_ue8m0"), 13) == M.preshuffled_bytes(cfg(), 13)
    assert M.preshuffled_bytes(cfg(), 13) == (288 * 2048 * 4096, 288 * 16 * 32 * 4)
    assert M.preshuffled_bytes(cfg(), 2) == (288 * 4096 * 1024, 288 * 32 * 8 * 4)
    assert M.preshuffled_bytes(cfg(quant="mxfp4"), 13) == (288 * 2048 * 2048, 288 * 128 * 8 * 64 * 4)
    assert M.preshuffled_bytes(cfg(quant="mxfp4"), 2) == (288 * 4096 * 512, 288 * 256 * 2 * 64 * 4)
    # whole N tiles of 256 rows: a half last N tile of w2 (Hp = 384) is padded
    # to 512 rows; w13's N tiles (128 gate + 128 up rows) are always whole
    c = cfg(hidden=384, inter=640)
    assert M.preshuffled_bytes(c, 2) == (288 * 512 * 640, 288 * 3 * 5 * 4)
    assert M.preshuffled_bytes(c, 13) == (288 * 1280 * 384, 288 * 10 * 3 * 4)
    c = cfg(quant="mxfp4", hidden=384, inter=640)
    assert M.preshuffled_bytes(c, 2) == (288 * 512 * 320, 288 * 2 * 2 * 16 * 64 * 4)
    assert M.preshuffled_bytes(c, 13) == (288 * 1280 * 192, 288 * 5 * 1 * 16 * 64 * 4)
    # workspace grows with T and covers the GEMM2 rows for gemm2_combine
    assert M.workspace_bytes(cfg(), 1) < M.workspace_bytes(cfg(), 64) < M.workspace_bytes(cfg(), 4096)
    assert M.workspace_bytes(cfg(), 64) >= 64 * 8 * 4096 * 4
    # ... never shrinks as T grows (a workspace for T_max serves every T <= T_max),
    # and large batches keep the per-pair rows in column chunks of a capped buffer
    for q in ("fp8", "mxfp4", "fp8_ue8m0"):
        c = cfg(quant=q, block_m=128)
        sizes = [M.workspace_bytes(c, T) for T in range(1, 40000, 97)]
        assert all(b >= a for a, b in zip(sizes, sizes[1:]))
    assert M.workspace_bytes(cfg(block_m=128), 16384) < 16384 * 8 * 4096 * 4


def test_pick_block_m():
    assert M.pick_block_m(1, 288, 8) == 16
    assert M.pick_block_m(64, 288, 8) == 16
    assert M.pick_block_m(4096, 288, 8) == 128
    assert M.pick_block_m(600, 288, 8) == 32
    assert M.pick_block_m(2048, 288, 8) == 128


def test_ksplit_plan_and_scratch():
    """The K split of small batches: usable splits, the planned split (from
    the expected number of active experts; this host has no GPU, so the
    library assumes 256 compute units), and scratch sizes within the layer
    workspace."""
    c = cfg()  # 288 experts, top-8, H=4096, I=1024, block_m 16
    # decode, one token: 8 experts x 8 N tiles = 64 GEMM1 items -> 4 pieces
    # (256 pieces for 256 workgroups); GEMM2: 128 items -> 2 pieces
    assert M.plan_ksplit(c, 1, 13) == 4 and M.plan_ksplit(c, 1, 2) == 2
    # two tokens: ~15.8 experts, 126 GEMM1 items -> 2 pieces; GEMM2 none
    assert M.plan_ksplit(c, 2, 13) == 2 and M.plan_ksplit(c, 2, 2) == 1
    # 64 tokens: ~240 active experts, every workgroup has items: GEMM1 takes
    # the tail split (whole rounds unsplit, the rest in 8 pieces), GEMM2 none
    assert M.plan_ksplit(c, 64, 13) == -8 and M.plan_ksplit(c, 64, 2) == 1
    # a shared expert (E = 1, top-1): 8 GEMM1 items -> 8 pieces
    assert M.plan_ksplit(cfg(num_experts=1, top_k=1, block_m=128), 64, 13) == 8
    # above 1024 pairs: no split of every item; GEMM1 keeps the tail split (it
    # needs no per-pair scratch) where the last round is expected to be mostly
    # idle: 100 experts at block_m 32 or 64 and 400 tokens give ~800 items, 32
    # past 3 rounds of 256 (at most 4 pieces at block_m 64 and 128); at 129
    # tokens ~2240 items leave 0.75 of a round (the kernel would not split
    # it), and 8 tokens ~470 items 0.84
    assert M.plan_ksplit(c, 129, 13) == 1 and M.plan_ksplit(c, 4096, 2) == 1 and M.plan_ksplit(c, 8, 13) == 1
    assert M.plan_ksplit(cfg(num_experts=100, block_m=64), 400, 13) == -4
    assert M.plan_ksplit(cfg(num_experts=100, block_m=32), 400, 13) == -8
    # one GPU's share of the prefill layer under 8-way tensor parallelism
    # (I = 128: one N tile per block): ~290 items, one round and a few left
    assert M.plan_ksplit(cfg(inter=128, block_m=128), 4096, 13) == -4
    # the prefill layer itself: ~2300-2500 items, most of a round left
    assert M.plan_ksplit(cfg(block_m=128), 4096, 13) == 1
    assert M.plan_ksplit(c, 16, 13) == -8 and M.plan_ksplit(c, 32, 13) == -8
    assert M.plan_ksplit(cfg(inter=256), 64, 13) == 1   # 2 N tiles: ~480 items, 0.875 of a round left
    assert M.plan_ksplit(c, 1, 7) == -1
    P = 64 * 8
    for ks in (1, 2, 4, 8):
        assert M.splitk_bytes(c, 64, 13, ks) == (0 if ks == 1 else ks * P * 2048 * 4 + P * 4)
    # a tail split: the pieces of at most one leftover item per workgroup (256
    # compute units assumed here), block_m rows of 256 fp32 partial sums each
    for ks in (2, 4, 8):
        assert M.splitk_bytes(c, 64, 13, -ks) == ks * 256 * 16 * 256 * 4
        assert M.splitk_bytes(cfg(block_m=32), 64, 13, -ks) == ks * 256 * 32 * 256 * 4
        assert M.splitk_bytes(cfg(block_m=64), 64, 13, -ks) == (ks * 256 * 64 * 256 * 4 if ks <= 4 else 0)
        assert M.splitk_bytes(c, 64, 2, -ks) == 0                  # GEMM1 only
    assert M.splitk_bytes(c, 64, 13, -3) == 0 and M.splitk_bytes(c, 64, 13, -16) == 0
    # GEMM2's y plane: int16 values [P, Hp] and one exponent byte per 64 columns
    plane = P * 4096 * 2 + P * 4096 // 64
    assert M.splitk_bytes(c, 64, 2, 2) == 2 * plane
    assert M.splitk_bytes(c, 64, 2, 1) == plane
    # unusable: not a power of two up to 8, pieces under 4 K blocks, or (MX,
    # UE8M0) not whole dwords of 4 scale bytes, or too many pairs
    assert M.splitk_bytes(c, 64, 13, 3) == 0 and M.splitk_bytes(c, 64, 13, 16) == 0
    assert M.splitk_bytes(c, 64, 2, 4) == 0          # 2 K blocks per piece
    assert M.splitk_bytes(c, 129, 13, 2) == 0        # 1032 pairs
    c24 = cfg(hidden=3072)                           # 24 K blocks
    assert M.splitk_bytes(c24, 4, 13, 4) > 0         # FP8: 6 K blocks per piece
    assert M.splitk_bytes(c24, 4, 13, -8) == 0 and M.plan_ksplit(c24, 64, 13) == -4
    for q in ("mxfp4", "fp8_ue8m0"):
        assert M.splitk_bytes(cfg(quant=q, hidden=3072), 4, 13, 4) == 0
        assert M.splitk_bytes(cfg(quant=q, hidden=3072), 4, 13, 2) > 0
        assert M.plan_ksplit(cfg(quant=q, hidden=3072), 1, 13) == 2
        assert M.plan_ksplit(cfg(quant=q, hidden=3072), 64, 13) == -2
    # every planned split fits the layer workspace, which stays monotone
    for q in ("fp8", "mxfp4", "fp8_ue8m0"):
        for E, k, bm in ((288, 8, 16), (1, 1, 128), (16, 4, 32)):
            cc = cfg(quant=q, num_experts=E, top_k=k, block_m=bm)
            for T in (1, 2, 5, 16, 64, 128, 300):
                need = max(M.splitk_bytes(cc, T, 2, M.plan_ksplit(cc, T, 2)),
                           M.splitk_bytes(cc, T, 13, M.plan_ksplit(cc, T, 13)))
                assert 0 < need <= M.workspace_bytes(cc, T)
    # unsplit GEMM2 of a batch whose y rows are column-chunked (P * Hp * 2 > 1 GiB)
    cc = cfg(num_experts=8, hidden=4100, inter=256, block_m=64)
    assert 0 < M.splitk_bytes(cc, 16384, 2, 1) <= M.workspace_bytes(cc, 16384)
    assert M.splitk_bytes(cc, 16384, 2, 1) < 16384 * 8 * 4224 * 2


def test_ksplit_entry_points_validate_before_launch():
    lib = M.lib()
    c = cfg()
    big = 1 << 40
    args1 = [ctypes.byref(c), 4] + [FAKE] * 9
    assert lib.moe_grouped_gemm1_swiglu_splitk(*args1, 3, FAKE, big, None) == UNSUP
    assert lib.moe_grouped_gemm1_swiglu_splitk(*args1, 16, FAKE, big, None) == UNSUP
    assert lib.moe_grouped_gemm1_swiglu_splitk(*args1, 2, FAKE, 1024, None) == WS
    assert lib.moe_grouped_gemm1_swiglu_splitk(*args1, 2, None, big, None) == NULL
    assert lib.moe_grouped_gemm1_swiglu_splitk(*args1, -3, FAKE, big, None) == UNSUP
    assert lib.moe_grouped_gemm1_swiglu_splitk(*args1, -8, FAKE, 1024, None) == WS
    assert lib.moe_grouped_gemm1_swiglu_splitk(*args1, -8, None, big, None) == NULL
    c64 = cfg(block_m=64)
    assert lib.moe_grouped_gemm1_swiglu_splitk(ctypes.byref(c64), 4, *([FAKE] * 9), -8, FAKE, big, None) == UNSUP
    args2 = [ctypes.byref(c), 4] + [FAKE] * 9 + [4096]
    assert lib.moe_grouped_gemm2_combine_splitk(*args2, 4, FAKE, big, None) == UNSUP
    assert lib.moe_grouped_gemm2_combine_splitk(*args2, -2, FAKE, big, None) == UNSUP
    assert lib.moe_grouped_gemm2_combine_splitk(*args2, 2, FAKE, 1024, None) == WS
    assert lib.moe_grouped_gemm2_combine_splitk(*args2[:-1], 100, 2, FAKE, big, None) == SHAPE
    assert lib.moe_grouped_gemm2_combine(*args2, FAKE, 1024, None) == WS


def test_no_kernel_uses_scratch_memory(tmp_path):
    """Every kernel of the built gfx950 code objects keeps its state in
    registers and LDS: a kernel with private (scratch) memory has lost an
    inlined helper or spilled, which once made a GEMM launch 4x slower.  Read
    from the kernels' own metadata in a copy of libmoe.so."""
    import shutil
    import subprocess
    llvm = "/opt/rocm/llvm/bin"
    objdump, readelf = os.path.join(llvm, "llvm-objdump"), os.path.join(llvm, "llvm-readelf")
    if not (os.path.exists(objdump) and os.path.exists(readelf)):
        pytest.skip("LLVM tools of the ROCm install not found")
    lib = tmp_path / "libmoe.so"
    shutil.copy(M.LIB_PATH, lib)
    subprocess.run([objdump, "--offloading", str(lib)], cwd=tmp_path, check=True, capture_output=True)
    objs = sorted(p for p in tmp_path.iterdir() if "gfx950" in p.name)
    assert objs, "no gfx950 code object in libmoe.so"
    kernels = {}
    for o in objs:
        notes = subprocess.run([readelf, "--notes", str(o)], check=True, capture_output=True, text=True).stdout
        name = None
        for line in notes.splitlines():
            line = line.strip()
            if line.startswith(".name:"):
                name = line.split(":", 1)[1].strip()
            elif line.startswith(".private_segment_fixed_size:") and name:
                kernels[name] = int(line.split(":", 1)[1])
    assert len(kernels) > 50
    assert any("moe_gemm_stream_kernel" in k for k in kernels)
    assert {k: v for k, v in kernels.items() if v} == {}


def test_m0_written_only_by_the_direct_lds_loads(tmp_path):
    """The GEMMs' direct global->LDS loads are inline assembly that sets M0
    (the LDS destination base) right before each load.  The compiler keeps M0
    for itself and cannot see those writes, so this holds only while no
    compiler-generated code in the library uses M0.  Checked on the
    disassembly of the built gfx950 code objects: every instruction that
    names m0 is `s_mov_b32 m0, <sgpr>` followed by `s_nop 0` and a
    global_load_lds_dword{,x4}; every such load comes right after one; and no
    instruction that uses M0 implicitly (register-indexed moves, messages,
    GWS/append/consume, buffer loads to LDS) appears."""
    import re
    import shutil
    import subprocess
    objdump = "/opt/rocm/llvm/bin/llvm-objdump"
    if not os.path.exists(objdump):
        pytest.skip("LLVM tools of the ROCm install not found")
    lib = tmp_path / "libmoe.so"
    shutil.copy(M.LIB_PATH, lib)
    subprocess.run([objdump, "--offloading", str(lib)], cwd=tmp_path, check=True, capture_output=True)
    objs = sorted(p for p in tmp_path.iterdir() if "gfx950" in p.name)
    assert objs
    insts = []
    for o in objs:
        dis = subprocess.run([objdump, "-d", "--mcpu=gfx950", str(o)], check=True, capture_output=True,
                             text=True).stdout
        for line in dis.splitlines():
            line = line.split("//")[0].strip()
            if line and not line.endswith(":") and not line.startswith(("Disassembly", "file format")):
                insts.append(line)
    writes = loads = 0
    implicit = re.compile(r"movrel|s_sendmsg|ds_gws|ds_append|ds_consume|set_gpr_idx|buffer_load\S*\s.*\blds\b")
    for i, ins in enumerate(insts):
        op = ins.split()[0]
        assert not implicit.search(ins), f"instruction with an implicit M0 use: {ins}"
        if re.search(r"\bm0\b", ins):
            assert re.fullmatch(r"s_mov_b32 m0, s\d+", ins), f"M0 used outside the direct loads: {ins}"
            assert insts[i + 1] == "s_nop 0" and insts[i + 2].startswith("global_load_lds_dword"), insts[i:i + 3]
            writes += 1
        if op.startswith("global_load_lds"):
            assert insts[i - 1] == "s_nop 0" and insts[i - 2].startswith("s_mov_b32 m0,"), insts[i - 2:i + 1]
            loads += 1
    assert writes == loads > 1000


def test_mfma_results_read_after_their_wait_states(tmp_path):
    """The compiler inserts the wait states between an MFMA and a VALU read of
    its result (the hardware does not interlock them).  Across a branch it
    once counted too few after the FP8 16x16x128 instruction, and the first
    result register was read stale.  Checked on the disassembly of the built
    code objects, in linear order across branches (the fall-through path):
    every read of a register written by an FP8 (8-pass) 16x16x128 scaled MFMA
    comes at least 12 wait states later, or after another MFMA, and every read
    after an FP4 (4-pass) one at least 8 wait states later.  Reads by MFMAs of
    their own accumulator chain are interlocked by the hardware and exempt."""
    import re
    import shutil
    import subprocess
    objdump = "/opt/rocm/llvm/bin/llvm-objdump"
    if not os.path.exists(objdump):
        pytest.skip("LLVM tools of the ROCm install not found")
    lib = tmp_path / "libmoe.so"
    shutil.copy(M.LIB_PATH, lib)
    subprocess.run([objdump, "--offloading", str(lib)], cwd=tmp_path, check=True, capture_output=True)
    objs = sorted(p for p in tmp_path.iterdir() if "gfx950" in p.name)
    assert objs

    def regs(spec):
        m = re.match(r"([av])\[(\d+):(\d+)\]", spec)
        if m:
            return {f"{m.group(1)}{k}" for k in range(int(m.group(2)), int(m.group(3)) + 1)}
        return {spec} if re.match(r"[av]\d+$", spec) else set()

    checked = 0
    for o in objs:
        dis = subprocess.run([objdump, "-d", "--mcpu=gfx950", str(o)], check=True, capture_output=True,
                             text=True).stdout
        funcs = re.split(r"\n[0-9a-f]+ <[^>]+>:\n", dis)
        for body in funcs[1:]:
            insts = [l.split("//")[0].strip() for l in body.splitlines()]
            insts = [x for x in insts if x and not x.endswith(":")]
            for j, t in enumerate(insts):
                if not t.startswith("v_mfma_scale_f32_16x16x128_f8f6f4"):
                    continue
                need = 8 if "cbsz:4" in t else 12
                ops = t.replace(",", " ").split()
                dst = regs(ops[1])
                ws = 0
                for t2 in insts[j + 1:j + 400]:
                    f2 = t2.replace(",", " ").split()
                    if f2[0] == "s_nop":
                        ws += int(f2[1]) + 1
                        continue
                    if f2[0] == "s_endpgm":
                        break
                    reads = set().union(*[regs(x) for x in f2[2:]]) if len(f2) > 2 else set()
                    if dst & reads:
                        if f2[0].startswith("v_mfma") and f2[1] == ops[1]:
                            break                     # the same accumulator chain
                        assert ws >= need, f"{t} read after {ws} wait states by {t2}"
                        checked += 1
                        break
                    if f2[0].startswith("v_mfma"):
                        if dst & regs(f2[1]):
                            break                     # overwritten first
                        break                         # an MFMA in between outlasts the wait
                    ws += 1
    assert checked > 100


def test_mfma_rate_diagnostic_rejects_bad_arguments_before_any_launch():
    lib = M.lib()
    sink = ctypes.c_void_p(16)  # never dereferenced: the checks come first
    assert lib.moe_diag_mfma_rate(3, 1, sink, None) == UNSUP
    assert lib.moe_diag_mfma_rate(-1, 1, sink, None) == UNSUP
    assert lib.moe_diag_mfma_rate(0, 0, sink, None) == UNSUP
    assert lib.moe_diag_mfma_rate(0, 1, None, None) == NULL


def test_stream_diagnostic_rejects_bad_arguments_before_any_launch():
    lib = M.lib()
    p16 = ctypes.c_void_p(256)  # never dereferenced: the checks come first
    assert lib.moe_diag_stream_read(None, 16, p16, None) == NULL
    assert lib.moe_diag_stream_read(p16, 16, None, None) == NULL
    assert lib.moe_diag_stream_read(p16, -16, p16, None) == SHAPE
    assert lib.moe_diag_stream_read(ctypes.c_void_p(264), 16, p16, None) == ALIGN
    assert lib.moe_diag_stream_read(p16, 24, p16, None) == ALIGN


def test_noalloc_scratch_covers_the_documented_decode_batches():
    # the header's figures: 793 tokens at block_m 16 and 731 at block_m 32 of
    # the 288-expert top-8 H = 4096, I = 1024 block-FP8 layer fit the static
    # scratch, one more token does not
    lim = 128 << 20
    for bm, T in ((16, 793), (32, 731)):
        c = M.make_cfg(288, 8, "fp8", 4096, 1024, block_m=bm)
        assert M.workspace_bytes(c, T) <= lim < M.workspace_bytes(c, T + 1)
