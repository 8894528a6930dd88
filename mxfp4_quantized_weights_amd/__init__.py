"""Python binding of libmoe.so, the routed-expert MoE layer for MI355X (gfx950).

Argument marshalling only: every function here checks tensor devices, dtypes
and shapes, allocates outputs with torch, and calls the C ABI declared in
include/moe.h with raw device pointers and torch's current HIP stream.  All
computation runs in the library's HIP kernels; there is no fallback.  If
libmoe.so has not been built, importing this package raises ImportError.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

# ---- constants mirrored from include/moe.h ---------------------------------
MOE_OK = 0
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_ALIGN",
                4: "MOE_ERR_UNSUPPORTED", 5: "MOE_ERR_LAYOUT", 6: "MOE_ERR_WORKSPACE", 7: "MOE_ERR_HIP"}
MOE_QUANT_FP8_BLOCK = 1
MOE_QUANT_MXFP4 = 2
MOE_QUANT_FP8_UE8M0 = 3
MOE_GATE_SEPARATED = 0
MOE_GATE_INTERLEAVED = 1
MOE_LAYOUT_CANONICAL = 0
MOE_LAYOUT_TILED_V2 = 0x4D310002
MOE_DTYPE_BF16 = 1
MOE_DTYPE_F32 = 2
MOE_NOALLOC_SCRATCH_BYTES = 128 << 20
QUANT_MODES = {"fp8": MOE_QUANT_FP8_BLOCK, "mxfp4": MOE_QUANT_MXFP4, "fp8_ue8m0": MOE_QUANT_FP8_UE8M0}


def e8_scale_ld(cols_padded: int) -> int:
    """Row stride in bytes of UE8M0 activation scales: one byte per 128
    columns, rounded up to whole dwords."""
    return (cols_padded // 128 + 3) // 4 * 4


class MoePad(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("hidden_padded", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("inter_padded", ctypes.c_int32)]


class MoeCfg(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("quant_mode", ctypes.c_int32), ("gate_mode", ctypes.c_int32),
                ("weight_layout", ctypes.c_int32), ("block_m", ctypes.c_int32),
                ("swiglu_limit", ctypes.c_float), ("pad", MoePad)]

    @property
    def fp8(self) -> bool:
        """e4m3 codes, one byte per element (block FP8 with fp32 or UE8M0 scales)."""
        return self.quant_mode in (MOE_QUANT_FP8_BLOCK, MOE_QUANT_FP8_UE8M0)


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_status_string(status)} ({STATUS_NAMES.get(status, status)})")


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m mxfp4_quantized_weights_amd.build` "
                      "(there is no non-HIP fallback)")
_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_CFGP = ctypes.POINTER(MoeCfg)

_SIGS = {
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_validate_cfg": (ctypes.c_int, [_CFGP]),
    "moe_max_blocks": (_I32, [_I32, _I32, _I32]),
    "moe_workspace_bytes": (_SZ, [_CFGP, _I32]),
    "moe_intermediate_bytes": (ctypes.c_int, [_CFGP, _I32, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)]),
    "moe_route_topk": (ctypes.c_int, [_P, _I32, _I32, _I32, _P, _P, _P]),
    "moe_permute_align": (ctypes.c_int, [_P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P]),
    "moe_quant_act": (ctypes.c_int, [_P, _I32, _I32, _I32, _I64, _I32, _I32, _P, _P, _P]),
    "moe_quant_weights": (ctypes.c_int, [_I32, _P, _I32, _I32, _I32, _P, _P, _P]),
    "moe_route_permute_quant": (ctypes.c_int, [_CFGP, _I32, _P, _P, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_preshuffled_bytes": (ctypes.c_int, [_CFGP, _I32, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)]),
    "moe_preshuffle_weights": (ctypes.c_int, [_CFGP, _I32, _P, _P, _P, _P, _P]),
    "moe_grouped_gemm1_swiglu": (ctypes.c_int, [_CFGP, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_grouped_gemm2_combine": (ctypes.c_int, [_CFGP, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I64,
                                                 _P, _SZ, _P]),
    "moe_forward": (ctypes.c_int, [_CFGP, _I32, _P, _I64, _P, _P, _P, _P, _P, _P, _I64, _P, _SZ, _P]),
    "moe_plan_ksplit": (_I32, [_CFGP, _I32, _I32]),
    "moe_splitk_bytes": (_SZ, [_CFGP, _I32, _I32, _I32]),
    "moe_grouped_gemm1_swiglu_splitk": (ctypes.c_int, [_CFGP, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P,
                                                       _SZ, _P]),
    "moe_grouped_gemm2_combine_splitk": (ctypes.c_int, [_CFGP, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I64,
                                                        _I32, _P, _SZ, _P]),
    "moe_forward_noalloc": (ctypes.c_int, [_CFGP, _I32, _P, _I64, _P, _P, _P, _P, _P, _P, _I64, _P]),
    "moe_diag_mfma_tile": (ctypes.c_int, [_I32, _P, _P, _P, _P]),
    "moe_diag_mfma_rate": (ctypes.c_int, [_I32, _I32, _P, _P]),
    "moe_diag_stream_read": (ctypes.c_int, [_P, _I64, _P, _P]),
    "moe_decode_supported": (_I32, [_CFGP, _I32]),
    "moe_decode_gemm1_swiglu": (ctypes.c_int, [_CFGP, _I32, _P, _P, _P, _P, _P, _P, _P]),
    "moe_decode_gemm2_combine": (ctypes.c_int, [_CFGP, _I32, _P, _P, _P, _P, _P, _P, _I64, _P, _P, _P]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED_SYMBOLS = tuple(_SIGS)


def _status_string(status: int) -> str:
    return _lib.moe_status_string(status).decode()


def _check(status: int, what: str):
    if status != MOE_OK:
        raise MoeError(status, what)


def lib() -> ctypes.CDLL:
    return _lib


# ---- configuration ---------------------------------------------------------

def make_cfg(num_experts: int, top_k: int, quant: str | int, hidden: int, inter: int,
             hidden_padded: int | None = None, inter_padded: int | None = None, block_m: int = 16,
             swiglu_limit: float = 10.0, gate_mode: int = MOE_GATE_SEPARATED,
             weight_layout: int = MOE_LAYOUT_TILED_V2, validate: bool = True) -> MoeCfg:
    """Builds (and by default validates) a moe_cfg_t."""
    qm = QUANT_MODES[quant] if isinstance(quant, str) else int(quant)
    hp = hidden_padded if hidden_padded is not None else -(-hidden // 128) * 128
    ip = inter_padded if inter_padded is not None else -(-inter // 128) * 128
    cfg = MoeCfg(num_experts, top_k, qm, gate_mode, weight_layout, block_m, swiglu_limit,
                 MoePad(hidden, hp, inter, ip))
    if validate:
        _check(_lib.moe_validate_cfg(ctypes.byref(cfg)), "moe_validate_cfg")
    return cfg


def pick_block_m(T: int, num_experts: int, top_k: int) -> int:
    """Rows per expert block for T tokens: 16 or 32 when experts see few
    tokens (decode), else 128 (a 128-row block uses each streamed weight tile
    for twice the rows of a 64-row one; measured faster on the T=2048 skewed
    and T=4096 uniform workloads).  A launch choice; any valid value gives the
    same results up to fp32 summation order."""
    per_expert = T * top_k / max(num_experts, 1)
    if per_expert <= 16:
        return 16
    if per_expert <= 32:
        return 32
    return 128


def validate_cfg(cfg: MoeCfg) -> int:
    return _lib.moe_validate_cfg(ctypes.byref(cfg))


def max_blocks(num_pairs: int, num_experts: int, block_m: int) -> int:
    return _lib.moe_max_blocks(num_pairs, num_experts, block_m)


def workspace_bytes(cfg: MoeCfg, T_max: int) -> int:
    return _lib.moe_workspace_bytes(ctypes.byref(cfg), T_max)


def intermediate_bytes(cfg: MoeCfg, T: int):
    a, s = _SZ(), _SZ()
    _check(_lib.moe_intermediate_bytes(ctypes.byref(cfg), T, ctypes.byref(a), ctypes.byref(s)),
           "moe_intermediate_bytes")
    return a.value, s.value


def preshuffled_bytes(cfg: MoeCfg, which: int):
    w, s = _SZ(), _SZ()
    _check(_lib.moe_preshuffled_bytes(ctypes.byref(cfg), which, ctypes.byref(w), ctypes.byref(s)),
           "moe_preshuffled_bytes")
    return w.value, s.value


# ---- helpers ---------------------------------------------------------------

def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, dtype, name: str, contiguous: bool = True):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _empty_bytes(n: int, device) -> torch.Tensor:
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


# ---- entry points ------------------------------------------------------------

def moe_route_topk(logits: torch.Tensor, top_k: int, stream=None):
    """-> ids int32 [T, k], weights float32 [T, k]."""
    T, E = logits.shape
    ids = torch.empty(T, top_k, dtype=torch.int32, device=logits.device)
    w = torch.empty(T, top_k, dtype=torch.float32, device=logits.device)
    _check(_lib.moe_route_topk(_dev(logits, torch.float32, "logits"), T, E, top_k, ids.data_ptr(),
                               w.data_ptr(), _stream(stream)), "moe_route_topk")
    return ids, w


def moe_permute_align(ids: torch.Tensor, num_experts: int, block_m: int, stream=None):
    """-> sorted_ids [nb*BM], block_expert [nb], expert_offsets [E+1], num_post_padded [1] (int32)."""
    T, k = ids.shape
    nb = max_blocks(T * k, num_experts, block_m)
    dev = ids.device
    sorted_ids = torch.empty(max(nb * block_m, 1), dtype=torch.int32, device=dev)
    block_expert = torch.empty(max(nb, 1), dtype=torch.int32, device=dev)
    offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
    npp = torch.empty(1, dtype=torch.int32, device=dev)
    _check(_lib.moe_permute_align(_dev(ids, torch.int32, "ids"), T, k, num_experts, block_m,
                                  sorted_ids.data_ptr(), block_expert.data_ptr(), offsets.data_ptr(),
                                  npp.data_ptr(), _stream(stream)), "moe_permute_align")
    return sorted_ids[:nb * block_m], block_expert[:nb], offsets, npp


def moe_quant_act(x: torch.Tensor, cols_padded: int, quant: str | int, stream=None):
    """Row quantisation of bf16/f32 [rows, cols] (row stride taken from x).
    -> FP8: (q uint8 [rows, cols_padded], s float32 [rows, cols_padded/128]);
       MXFP4: (q uint8 [rows, cols_padded/2], s uint8 [rows, cols_padded/32]);
       FP8_UE8M0: (q uint8 [rows, cols_padded], s uint8 [rows, e8_scale_ld(cols_padded)]),
       the scale bytes of group g in s[:, g], zeros past cols_padded/128."""
    qm = QUANT_MODES[quant] if isinstance(quant, str) else int(quant)
    rows, cols = x.shape
    if x.stride(1) != 1:
        raise ValueError("x must have unit column stride")
    dt = {torch.bfloat16: MOE_DTYPE_BF16, torch.float32: MOE_DTYPE_F32}.get(x.dtype)
    if dt is None:
        raise ValueError("x must be bf16 or f32")
    q, s = _act_buffers(qm, rows, cols_padded, x.device)
    _check(_lib.moe_quant_act(_dev(x, None, "x", contiguous=False), dt, rows, cols, x.stride(0), cols_padded,
                              qm, q.data_ptr(), s.data_ptr(), _stream(stream)), "moe_quant_act")
    return q, s


def _act_buffers(qm: int, rows: int, cols_padded: int, device):
    """Quantised-activation outputs of moe_quant_act's layout."""
    if qm == MOE_QUANT_FP8_BLOCK:
        return (torch.empty(rows, cols_padded, dtype=torch.uint8, device=device),
                torch.empty(rows, cols_padded // 128, dtype=torch.float32, device=device))
    if qm == MOE_QUANT_FP8_UE8M0:
        return (torch.empty(rows, cols_padded, dtype=torch.uint8, device=device),
                torch.empty(rows, e8_scale_ld(cols_padded), dtype=torch.uint8, device=device))
    return (torch.empty(rows, cols_padded // 2, dtype=torch.uint8, device=device),
            torch.empty(rows, cols_padded // 32, dtype=torch.uint8, device=device))


def moe_route_permute_quant(cfg: MoeCfg, x: torch.Tensor, logits: torch.Tensor, stream=None):
    """Routing + permutation + quantisation of bf16 x [T, H] in as few launches
    as the batch allows.  -> (ids, weights, sorted_ids, block_expert,
    expert_offsets, num_post_padded, xq, xs), as the three stage calls."""
    T = x.shape[0]
    if x.stride(1) != 1:
        raise ValueError("x must have unit column stride")
    E, k, bm = cfg.num_experts, cfg.top_k, cfg.block_m
    dev = x.device
    nb = max_blocks(T * k, E, bm)
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    w = torch.empty(T, k, dtype=torch.float32, device=dev)
    sorted_ids = torch.empty(max(nb * bm, 1), dtype=torch.int32, device=dev)
    block_expert = torch.empty(max(nb, 1), dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    npp = torch.empty(1, dtype=torch.int32, device=dev)
    xq, xs = _act_buffers(cfg.quant_mode, T, cfg.pad.hidden_padded, dev)
    _check(_lib.moe_route_permute_quant(ctypes.byref(cfg), T, _dev(logits, torch.float32, "router_logits"),
                                        _dev(x, torch.bfloat16, "x", contiguous=False), x.stride(0),
                                        ids.data_ptr(), w.data_ptr(), sorted_ids.data_ptr(), block_expert.data_ptr(),
                                        offsets.data_ptr(), npp.data_ptr(), xq.data_ptr(), xs.data_ptr(),
                                        _stream(stream)), "moe_route_permute_quant")
    return ids, w, sorted_ids[:nb * bm], block_expert[:nb], offsets, npp, xq, xs


def moe_quant_weights(w: torch.Tensor, quant: str | int, stream=None):
    """Canonical quantisation of float32 [E, N, K] (already padded)."""
    qm = QUANT_MODES[quant] if isinstance(quant, str) else int(quant)
    E, N, K = w.shape
    if qm in (MOE_QUANT_FP8_BLOCK, MOE_QUANT_FP8_UE8M0):
        q = torch.empty(E, N, K, dtype=torch.uint8, device=w.device)
        s = torch.empty(E, N // 128, K // 128, device=w.device,
                        dtype=torch.float32 if qm == MOE_QUANT_FP8_BLOCK else torch.uint8)
    else:
        q = torch.empty(E, N, K // 2, dtype=torch.uint8, device=w.device)
        s = torch.empty(E, N, K // 32, dtype=torch.uint8, device=w.device)
    _check(_lib.moe_quant_weights(qm, _dev(w, torch.float32, "w"), E, N, K, q.data_ptr(), s.data_ptr(),
                                  _stream(stream)), "moe_quant_weights")
    return q, s


def moe_preshuffle_weights(cfg: MoeCfg, which: int, q: torch.Tensor, s: torch.Tensor, stream=None):
    """CANONICAL -> TILED_V2 for w13 (which=13) or w2 (which=2); flat uint8 outputs."""
    wb, sb = preshuffled_bytes(cfg, which)
    qo = torch.empty(wb, dtype=torch.uint8, device=q.device)
    so = torch.empty(sb, dtype=torch.uint8, device=q.device)
    _check(_lib.moe_preshuffle_weights(ctypes.byref(cfg), which, _dev(q, torch.uint8, "w"),
                                       _dev(s, None, "scales"), qo.data_ptr(), so.data_ptr(),
                                       _stream(stream)), "moe_preshuffle_weights")
    return qo, so


def plan_ksplit(cfg: MoeCfg, T: int, which: int) -> int:
    """K split the library uses for GEMM `which` (13 or 2) at T tokens."""
    return _lib.moe_plan_ksplit(ctypes.byref(cfg), T, which)


def splitk_bytes(cfg: MoeCfg, T: int, which: int, ksplit: int) -> int:
    return _lib.moe_splitk_bytes(ctypes.byref(cfg), T, which, ksplit)


def moe_grouped_gemm1_swiglu(cfg: MoeCfg, T: int, xq, xs, sorted_ids, block_expert, npp, w13, s13,
                             ksplit: int = 1, stream=None):
    """-> (aq, as) flat uint8 buffers, rows indexed by sorted position.
    ksplit > 1: the K-split launch pair (fp32 partials in a scratch buffer)."""
    ab, sb = intermediate_bytes(cfg, T)
    dev = xq.device
    aq = _empty_bytes(ab, dev)
    as_ = _empty_bytes(sb, dev)
    args = [ctypes.byref(cfg), T, _dev(xq, None, "xq"), _dev(xs, None, "xs"),
            _dev(sorted_ids, torch.int32, "sorted_ids"), _dev(block_expert, torch.int32, "block_expert"),
            _dev(npp, torch.int32, "num_post_padded"), _dev(w13, None, "w13"), _dev(s13, None, "w13_scale"),
            aq.data_ptr(), as_.data_ptr()]
    if ksplit == 1:
        _check(_lib.moe_grouped_gemm1_swiglu(*args, _stream(stream)), "moe_grouped_gemm1_swiglu")
    else:
        nbytes = splitk_bytes(cfg, T, 13, ksplit)
        ws = _empty_bytes(max(nbytes, 1), dev)
        _check(_lib.moe_grouped_gemm1_swiglu_splitk(*args, ksplit, ws.data_ptr(), nbytes, _stream(stream)),
               "moe_grouped_gemm1_swiglu_splitk")
    return aq[:ab], as_[:sb]


def moe_grouped_gemm2_combine(cfg: MoeCfg, T: int, aq, as_, sorted_ids, block_expert, npp, w2, s2, topk_w,
                              out: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                              ksplit: int | None = None, stream=None):
    """ksplit None: the library's own split (moe_plan_ksplit); else that split."""
    dev = aq.device
    if out is None:
        out = torch.empty(T, cfg.pad.hidden, dtype=torch.bfloat16, device=dev)
    if ws is None:
        ws = _empty_bytes(workspace_bytes(cfg, T) if ksplit is None else splitk_bytes(cfg, T, 2, ksplit), dev)
    args = [ctypes.byref(cfg), T, _dev(aq, None, "aq"), _dev(as_, None, "as"),
            _dev(sorted_ids, torch.int32, "sorted_ids"), _dev(block_expert, torch.int32, "block_expert"),
            _dev(npp, torch.int32, "num_post_padded"), _dev(w2, None, "w2"), _dev(s2, None, "w2_scale"),
            _dev(topk_w, torch.float32, "topk_w"), _dev(out, torch.bfloat16, "out", contiguous=False),
            out.stride(0)]
    wsb = ws.numel() * ws.element_size()
    if ksplit is None:
        _check(_lib.moe_grouped_gemm2_combine(*args, ws.data_ptr(), wsb, _stream(stream)),
               "moe_grouped_gemm2_combine")
    else:
        _check(_lib.moe_grouped_gemm2_combine_splitk(*args, ksplit, ws.data_ptr(), wsb, _stream(stream)),
               "moe_grouped_gemm2_combine_splitk")
    return out


def decode_intermediate_bytes(cfg: MoeCfg, T: int):
    """Sizes in bytes of the decode path's intermediate codes and scales
    (pair order: T*k rows of Ip codes; fp32 per 128 or UE8M0 bytes in rows of
    whole dwords)."""
    rows, ip = T * cfg.top_k, cfg.pad.inter_padded
    if cfg.quant_mode == MOE_QUANT_FP8_UE8M0:
        return rows * ip, rows * ((ip // 128 + 3) // 4 * 4)
    return rows * ip, rows * (ip // 128) * 4


def decode_supported(cfg: MoeCfg, T: int) -> bool:
    """Whether moe_forward runs the decode (M-tiled GEMV) kernels for T tokens."""
    return bool(_lib.moe_decode_supported(ctypes.byref(cfg), T))


def moe_decode_gemm1_swiglu(cfg: MoeCfg, xq, xs, topk_ids, w13, s13, a: torch.Tensor | None = None, stream=None):
    """Decode GEMM1 + clamped SwiGLU -> a float32 [T*k, Ip] (pair order)."""
    T = topk_ids.shape[0]
    if a is None:
        a = torch.zeros(T * cfg.top_k, cfg.pad.inter_padded, dtype=torch.float32, device=topk_ids.device)
    _check(_lib.moe_decode_gemm1_swiglu(ctypes.byref(cfg), T, _dev(xq, None, "xq"), _dev(xs, None, "xs"),
                                        _dev(topk_ids, torch.int32, "topk_ids"), _dev(w13, None, "w13"),
                                        _dev(s13, None, "w13_scale"), _dev(a, torch.float32, "a"),
                                        _stream(stream)), "moe_decode_gemm1_swiglu")
    return a


def moe_decode_gemm2_combine(cfg: MoeCfg, a, topk_ids, topk_w, w2, s2, out: torch.Tensor | None = None,
                             aq: torch.Tensor | None = None, as_: torch.Tensor | None = None, stream=None):
    """Decode re-quantisation + GEMM2 + combine -> out bf16 [T, H]; aq / as_
    (pair order; allocated when not given) receive the intermediate codes
    and scales."""
    T = topk_ids.shape[0]
    if out is None:
        out = torch.empty(T, cfg.pad.hidden, dtype=torch.bfloat16, device=a.device)
    if aq is None or as_ is None:
        aq_b, as_b = decode_intermediate_bytes(cfg, T)
        aq = torch.empty(aq_b, dtype=torch.uint8, device=a.device)
        as_ = torch.empty(as_b, dtype=torch.uint8, device=a.device)
    _check(_lib.moe_decode_gemm2_combine(ctypes.byref(cfg), T, _dev(a, torch.float32, "a"),
                                         _dev(topk_ids, torch.int32, "topk_ids"),
                                         _dev(topk_w, torch.float32, "topk_w"), _dev(w2, None, "w2"),
                                         _dev(s2, None, "w2_scale"), _dev(out, torch.bfloat16, "out", contiguous=False),
                                         out.stride(0), aq.data_ptr(), as_.data_ptr(), _stream(stream)),
           "moe_decode_gemm2_combine")
    return out


def moe_forward(cfg: MoeCfg, x: torch.Tensor, logits: torch.Tensor, w13, s13, w2, s2,
                out: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None):
    """The whole layer.  x bf16 [T, H] (unit column stride), logits f32 [T, E]."""
    T = x.shape[0]
    if x.stride(1) != 1:
        raise ValueError("x must have unit column stride")
    if out is None:
        out = torch.empty(T, cfg.pad.hidden, dtype=torch.bfloat16, device=x.device)
    if ws is None:
        ws = _empty_bytes(workspace_bytes(cfg, T), x.device)
    _check(_lib.moe_forward(ctypes.byref(cfg), T, _dev(x, torch.bfloat16, "x", contiguous=False), x.stride(0),
                            _dev(logits, torch.float32, "router_logits"), _dev(w13, None, "w13"),
                            _dev(s13, None, "w13_scale"), _dev(w2, None, "w2"), _dev(s2, None, "w2_scale"),
                            _dev(out, torch.bfloat16, "out", contiguous=False), out.stride(0), ws.data_ptr(),
                            ws.numel() * ws.element_size(), _stream(stream)), "moe_forward")
    return out


def moe_forward_noalloc(cfg: MoeCfg, x: torch.Tensor, logits: torch.Tensor, w13, s13, w2, s2,
                        out: torch.Tensor | None = None, stream=None):
    """moe_forward with the library's static scratch (no workspace argument;
    the library allocates nothing).  Raises MoeError(MOE_ERR_WORKSPACE) when
    the batch needs more than MOE_NOALLOC_SCRATCH_BYTES."""
    T = x.shape[0]
    if x.stride(1) != 1:
        raise ValueError("x must have unit column stride")
    if out is None:
        out = torch.empty(T, cfg.pad.hidden, dtype=torch.bfloat16, device=x.device)
    _check(_lib.moe_forward_noalloc(ctypes.byref(cfg), T, _dev(x, torch.bfloat16, "x", contiguous=False),
                                    x.stride(0), _dev(logits, torch.float32, "router_logits"), _dev(w13, None, "w13"),
                                    _dev(s13, None, "w13_scale"), _dev(w2, None, "w2"), _dev(s2, None, "w2_scale"),
                                    _dev(out, torch.bfloat16, "out", contiguous=False), out.stride(0),
                                    _stream(stream)), "moe_forward_noalloc")
    return out


def moe_diag_mfma_tile(kind: int, a: torch.Tensor, b: torch.Tensor, stream=None) -> torch.Tensor:
    """Diagnostic: C = A . B^T (f32 [16, 16]) from e4m3 codes a, b (u8 [16, 128])
    with one FP8 MFMA (kind 0) or four f16 MFMAs on exactly widened operands
    (kind 1), as the grouped GEMMs compute one K block."""
    out = torch.empty(16, 16, dtype=torch.float32, device=a.device)
    _check(_lib.moe_diag_mfma_tile(kind, _dev(a, torch.uint8, "a"), _dev(b, torch.uint8, "b"), out.data_ptr(),
                                   _stream(stream)), "moe_diag_mfma_tile")
    return out


# moe_diag_mfma_rate: workgroups of 4 waves per launch (MOE_DIAG_MFMA_RATE_WORKGROUPS)
# and FLOP per instruction of each kind (f16 16x16x32, FP8 and FP4 16x16x128)
DIAG_MFMA_RATE_WORKGROUPS = 1024
DIAG_MFMA_RATE_FLOP = (16384, 65536, 65536)


def moe_diag_mfma_rate(kind: int, iters: int, sink: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Diagnostic: one launch of the matrix-core rate loop (kind 0 f16, 1 FP8,
    2 FP4; ``iters`` rounds of 8 MFMAs per wave) on ``stream``; the caller times
    it.  FLOPs per launch: DIAG_MFMA_RATE_WORKGROUPS * 4 * iters * 8 *
    DIAG_MFMA_RATE_FLOP[kind].  -> the f32 sink the kernel writes."""
    if sink is None:
        sink = torch.empty(DIAG_MFMA_RATE_WORKGROUPS * 256, dtype=torch.float32, device="cuda")
    _check(_lib.moe_diag_mfma_rate(kind, iters, sink.data_ptr(), _stream(stream)), "moe_diag_mfma_rate")
    return sink


DIAG_STREAM_WORKGROUPS = 256    # of 512 threads


def moe_diag_stream_read(src: torch.Tensor, sink: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Diagnostic: one launch that reads every byte of ``src`` (contiguous device
    memory, 16-byte aligned, a multiple of 16 bytes) with the GEMMs' kind of
    load, on ``stream``; the caller times it.  -> the u32 checksum sink (int32)."""
    if sink is None:
        sink = torch.empty(DIAG_STREAM_WORKGROUPS * 512, dtype=torch.int32, device=src.device)
    _check(_lib.moe_diag_stream_read(_dev(src, None, "src"), src.numel() * src.element_size(), sink.data_ptr(),
                                     _stream(stream)), "moe_diag_stream_read")
    return sink


class ExpertWeights:
    """Quantised, preshuffled expert weights of one layer (device memory).

    Built from padded float32 weights w13 [E, 2Ip, Hp] / w2 [E, Hp, Ip]
    with the library's own quantiser and preshuffle, optionally a few experts
    at a time (``add_experts``) so the fp32 copies never coexist in full.
    """

    def __init__(self, cfg: MoeCfg, device="cuda"):
        self.cfg = cfg
        E, Hp, Ip = cfg.num_experts, cfg.pad.hidden_padded, cfg.pad.inter_padded
        fp8 = cfg.fp8
        sdt = torch.float32 if cfg.quant_mode == MOE_QUANT_FP8_BLOCK else torch.uint8
        self.device = device
        self.q13 = torch.empty(E, 2 * Ip, Hp if fp8 else Hp // 2, dtype=torch.uint8, device=device)
        self.s13 = (torch.empty(E, 2 * Ip // 128, Hp // 128, dtype=sdt, device=device) if fp8
                    else torch.empty(E, 2 * Ip, Hp // 32, dtype=torch.uint8, device=device))
        self.q2 = torch.empty(E, Hp, Ip if fp8 else Ip // 2, dtype=torch.uint8, device=device)
        self.s2 = (torch.empty(E, Hp // 128, Ip // 128, dtype=sdt, device=device) if fp8
                   else torch.empty(E, Hp, Ip // 32, dtype=torch.uint8, device=device))
        self.w13 = self.w13_scale = self.w2 = self.w2_scale = None

    def add_experts(self, first: int, w13: torch.Tensor, w2: torch.Tensor):
        """Quantises experts [first, first + len(w13)) into the canonical buffers."""
        n = w13.shape[0]
        q, s = moe_quant_weights(w13.contiguous(), self.cfg.quant_mode)
        self.q13[first:first + n] = q
        self.s13[first:first + n] = s
        q, s = moe_quant_weights(w2.contiguous(), self.cfg.quant_mode)
        self.q2[first:first + n] = q
        self.s2[first:first + n] = s

    def finalize(self):
        """Preshuffles the canonical buffers into TILED_V2 (and keeps both)."""
        self.w13, self.w13_scale = moe_preshuffle_weights(self.cfg, 13, self.q13, self.s13)
        self.w2, self.w2_scale = moe_preshuffle_weights(self.cfg, 2, self.q2, self.s2)
        return self

    def tiled(self):
        return self.w13, self.w13_scale, self.w2, self.w2_scale

    def tiled_bytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.tiled())


__all__ = [n for n in dir() if n.startswith(("moe_", "MOE_", "Moe"))] + [
    "make_cfg", "pick_block_m", "e8_scale_ld", "QUANT_MODES", "validate_cfg", "max_blocks", "workspace_bytes", "intermediate_bytes",
    "plan_ksplit", "splitk_bytes",
    "preshuffled_bytes", "ExpertWeights", "EXPORTED_SYMBOLS", "LIB_PATH", "lib"]
