"""Python binding of libnv4moe.so, the NVFP4 W4A4 mixture-of-experts expert path
for AMD Instinct MI355X (gfx950).

The binding only marshals arguments: torch provides device memory and the
current HIP stream, every step of the path runs in the library's HIP kernels.
The entry points carry the names of the C ABI (include/nv4moe.h):

    nvfp4_quantize      NVFP4 quantisation (rows, columns, batched columns)
    nvfp4_quantize_sr   the same with stochastic rounding of the elements
    moe_permute         top-k routing and stable permutation by expert (+ row gather)
    nvfp4_grouped_gemm  grouped NVFP4 x NVFP4 GEMM (GROUP_M with optional SwiGLU, GROUP_K)
    moe_combine         top-k weighted combine back to token order
    nv4_to_bf16         BF16 operands: BF16-dequantised NVFP4 or BF16, rows / columns
    bf16_grouped_gemm   the same grouped GEMM on BF16 operands

``moe_forward`` and ``moe_backward`` compose these calls into the expert layer's
forward (route, quantise, permute, GEMM + SwiGLU, quantise, GEMM, combine) and
its four backward grouped GEMMs.  ``moe_forward_bf16`` is the unquantised layer
and ``moe_backward_bf16`` the backward on BF16 operands: the forward's NVFP4
tensors dequantised (the dequantized backward) or the BF16 tensors themselves.
There is no fallback: if the library is not built, every call raises.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnv4moe.so")

# constants (mirror include/nv4moe.h)
NV4_BF16, NV4_F32 = 0, 1
NV4_ROWS, NV4_COLS, NV4_COLS_BATCHED, NV4_ROWS_AND_COLS = 1, 2, 3, 4
NV4_SCALE_TENSOR, NV4_SCALE_SEGMENT, NV4_SCALE_ROW, NV4_SCALE_SEGMENT_HALVES = 0, 1, 2, 3
NV4_GROUP_M, NV4_GROUP_K = 0, 1
NV4_EPI_NONE, NV4_EPI_SWIGLU = 0, 1
NV4_RENORM = 1
NV4_DS_NONFINITE, NV4_DS_BAD_EXPERT, NV4_DS_NAN_LOGIT = 1, 2, 4
STATUS = {0: "NV4_OK", -1: "NV4_EINVAL", -2: "NV4_EALIGN", -3: "NV4_EUNSUPPORTED", -4: "NV4_EWORKSPACE",
          -5: "NV4_EHIP"}


class NV4Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class NV4Tensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("tscale", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("K", ctypes.c_int64), ("scale_mode", ctypes.c_int32),
                ("nseg", ctypes.c_int32), ("f16", ctypes.c_void_p)]


_lib = None
_P, _I64, _I, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t

_SIGS = {
    "nv4_version": (ctypes.c_int, []),
    "nv4_status_string": (ctypes.c_char_p, [_I]),
    "nv4_last_error": (ctypes.c_char_p, []),
    "nvfp4_quantize_workspace": (_SZ, [_I64, _I64, _I, _I, _I]),
    "nvfp4_quantize": (_I, [_P, _I, _I64, _I64, _I64, _P, _I, _I, _I, _P, _P, _P, _P, ctypes.POINTER(NV4Tensor),
                            ctypes.POINTER(NV4Tensor), _P, _SZ, _P, _P]),
    "nvfp4_quantize_sr": (_I, [_P, _I, _I64, _I64, _I64, _P, _I, _I, _I, _P, _P, _P, _P, ctypes.POINTER(NV4Tensor),
                               ctypes.POINTER(NV4Tensor), _P, _SZ, _P, ctypes.c_uint64, _P]),
    "nv4_amax": (_I, [_P, _I64, _P, _P, _P]),
    "moe_permute_workspace": (_SZ, [_I64, _I, _I]),
    "moe_permute": (_I, [_P, _I64, _I, _I, _I, _P, _P, _P, _P, _P, _P, ctypes.POINTER(NV4Tensor),
                         ctypes.POINTER(NV4Tensor), _P, _SZ, _P, _P]),
    "moe_permute_noalloc_max_workspace": (_SZ, []),
    "moe_permute_noalloc": (_I, [_P, _I64, _I, _I, _I, _P, _P, _P, _P, _P, _P, ctypes.POINTER(NV4Tensor),
                                 ctypes.POINTER(NV4Tensor), _P, _P]),
    "nvfp4_grouped_gemm_workspace": (_SZ, [ctypes.POINTER(NV4Tensor), ctypes.POINTER(NV4Tensor), _I]),
    "nvfp4_grouped_gemm": (_I, [ctypes.POINTER(NV4Tensor), ctypes.POINTER(NV4Tensor), _P, _I, _I64, _I64, _P,
                                _I, _I, _P, _I, _I64, _P, _P, _SZ, _P]),
    "moe_combine": (_I, [_P, _I, _I64, _P, _P, _I64, _I, _I64, _P, _I, _P]),
    "nvfp4_decode_f16": (_I, [ctypes.POINTER(NV4Tensor), _P, _I64, _P]),
    "nv4_to_bf16": (_I, [_P, _I64, _I64, ctypes.POINTER(NV4Tensor), _I64, _I64, _P, _I, _I, _P, _P, _P, _I64, _I64,
                         _P]),
    "bf16_grouped_gemm": (_I, [_P, _I64, _P, _I64, _I64, _P, _I, _I64, _I64, _P, _I, _I, _P, _I, _I64, _P, _P, _SZ,
                               _P]),
    # measurement kernels (include/nv4moe_bench.h)
    "nv4_bench_copy": (_I, [_P, _P, _SZ, _P]),
    "nv4_bench_read": (_I, [_P, _SZ, ctypes.c_uint32, _P, _P]),
    "nv4_bench_mix": (_I, [_P, _SZ, _P, _P]),
    "nv4_bench_write": (_I, [_P, _SZ, _P]),
    "nv4_bench_lds_out_words": (_SZ, []),
    "nv4_bench_lds": (_I, [_P, _I, _P]),
    "nv4_bench_mfma_out_floats": (_SZ, [_I]),
    "nv4_bench_mfma": (_I, [_P, _I, _I, _P]),
}


def load() -> ctypes.CDLL:
    """Load libnv4moe.so (built in-tree by ``nvfp4_w4a4_moe_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m nvfp4_w4a4_moe_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status: int):
    if status != 0:
        raise NV4Error(status, load().nv4_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return NV4_BF16
    if t.dtype == torch.float32:
        return NV4_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


@dataclass
class NVFP4:
    """Device NVFP4 tensor: codes [rows, K/2] u8, scales [rows, K/16] u8 (E4M3),
    tscale FP32 decode scales (1, nseg or rows of them)."""
    codes: torch.Tensor
    scales: torch.Tensor
    tscale: torch.Tensor
    rows: int
    K: int
    scale_mode: int = NV4_SCALE_TENSOR
    nseg: int = 1
    f16: torch.Tensor | None = None  # exact FP16 values without the decode scale (nvfp4_decode_f16), or None

    @staticmethod
    def empty(rows: int, K: int, ngroups: int = 1, device="cuda") -> "NVFP4":
        return NVFP4(torch.empty((rows, K // 2), dtype=torch.uint8, device=device),
                     torch.empty((rows, K // 16), dtype=torch.uint8, device=device),
                     torch.empty((max(ngroups, 1),), dtype=torch.float32, device=device), rows, K)

    def c(self) -> NV4Tensor:
        return NV4Tensor(self.codes.data_ptr(), self.scales.data_ptr(), self.tscale.data_ptr(),
                         self.rows, self.K, self.scale_mode, self.nseg,
                         None if self.f16 is None else self.f16.data_ptr())


def _ngroups(rows, scale_mode, nseg):
    if scale_mode == NV4_SCALE_TENSOR:
        return 1
    if scale_mode == NV4_SCALE_SEGMENT:
        return nseg
    if scale_mode == NV4_SCALE_SEGMENT_HALVES:
        return 2 * nseg
    return rows


def nvfp4_quantize(x: torch.Tensor, layout: int = NV4_ROWS, scale_mode: int = NV4_SCALE_TENSOR, nseg: int = 1,
                   seg_offsets: torch.Tensor | None = None, seg_padded_offsets: torch.Tensor | None = None,
                   amax_in: torch.Tensor | None = None, amax_out: torch.Tensor | None = None,
                   out: NVFP4 | None = None, out_K: int | None = None, ws: torch.Tensor | None = None,
                   dev_status: torch.Tensor | None = None, row_index: torch.Tensor | None = None,
                   out_rows: NVFP4 | None = None, sr_seed: int | None = None, stream=None) -> NVFP4:
    """NVFP4-quantise a 2-D BF16/FP32 tensor (row stride x.stride(0)).  With row_index
    (int32 [rows]), logical row r is x row row_index[r] (rows = row_index.numel()).
    NV4_ROWS_AND_COLS returns the column output and fills `out_rows` (allocated when
    None and then reachable as the result's `rows_out` attribute).  With sr_seed the
    elements round stochastically (nvfp4_quantize_sr)."""
    lib = load()
    assert x.dim() == 2 and x.stride(1) == 1
    rows, K = x.shape
    if row_index is not None:
        assert row_index.dtype == torch.int32 and row_index.is_contiguous()
        rows = row_index.numel()
    if layout == NV4_ROWS:
        orows, oK = rows, K
    elif layout == NV4_COLS_BATCHED:
        orows, oK = nseg * K, rows // nseg
    else:
        orows = K
        oK = out_K if out_K is not None else ((rows + 15 * nseg + 63) // 64) * 64
    if layout == NV4_ROWS_AND_COLS and out_rows is None:
        out_rows = NVFP4.empty(rows, K, 1, device=x.device)
    ng = _ngroups(rows, scale_mode, nseg)
    if out is None:
        out = NVFP4.empty(orows, oK, ng, device=x.device)
    if ws is None and amax_out is None and amax_in is None:
        ws = torch.empty(lib.nvfp4_quantize_workspace(rows, K, layout, scale_mode, nseg), dtype=torch.uint8,
                         device=x.device)
    d = out.c()
    d2 = out_rows.c() if out_rows is not None else None
    args = (_ptr(x), _dtype(x), rows, K, x.stride(0), _ptr(row_index), layout, scale_mode, nseg,
            _ptr(seg_offsets), _ptr(seg_padded_offsets), _ptr(amax_in), _ptr(amax_out),
            ctypes.byref(d), None if d2 is None else ctypes.byref(d2), _ptr(ws),
            0 if ws is None else ws.numel(), _ptr(dev_status))
    if sr_seed is None:
        _check(lib.nvfp4_quantize(*args, _stream(stream)))
    else:
        _check(lib.nvfp4_quantize_sr(*args, ctypes.c_uint64(sr_seed & (2 ** 64 - 1)), _stream(stream)))
    out.scale_mode, out.nseg = d.scale_mode, d.nseg
    if out.f16 is not None:  # keep an attached FP16 copy in step with the new codes
        nvfp4_decode_f16(out, out=out.f16, stream=stream)
    if d2 is not None:
        out_rows.scale_mode, out_rows.nseg = d2.scale_mode, d2.nseg
        out.rows_out = out_rows
    return out


def nvfp4_decode_f16(q: NVFP4, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Exact FP16 values e2m1 * e4m3 of q's elements, [rows, K] (the decode scale G
    not applied)."""
    if out is None:
        out = torch.empty((q.rows, q.K), dtype=torch.float16, device=q.codes.device)
    assert out.dtype == torch.float16 and out.dim() == 2 and out.stride(1) == 1
    d = q.c()
    _check(load().nvfp4_decode_f16(ctypes.byref(d), _ptr(out), out.stride(0), _stream(stream)))
    return out


def with_f16(q: NVFP4, stream=None) -> NVFP4:
    """q with its decoded FP16 values attached (the grouped GEMM then reads a GROUP_M
    B operand from them instead of decoding it)."""
    q.f16 = nvfp4_decode_f16(q, stream=stream)
    return q


def nv4_amax(x: torch.Tensor, amax: torch.Tensor | None = None, dev_status: torch.Tensor | None = None,
             stream=None) -> torch.Tensor:
    """max |x| of an FP32 tensor into a one-element FP32 tensor (e.g. the tensor amax
    from the per-row amaxes a per-token quantisation recorded)."""
    assert x.dtype == torch.float32 and x.is_contiguous()
    if amax is None:
        amax = torch.empty(1, dtype=torch.float32, device=x.device)
    _check(load().nv4_amax(_ptr(x), x.numel(), _ptr(amax), _ptr(dev_status), _stream(stream)))
    return amax


@dataclass
class Routing:
    topk_ids: torch.Tensor      # [T, k] int32
    topk_w: torch.Tensor        # [T, k] fp32
    offsets: torch.Tensor       # [E+1] int32
    padded_offsets: torch.Tensor  # [E+1] int32
    row_token: torch.Tensor     # [T*k] int32
    token_row: torch.Tensor     # [T, k] int32


def moe_permute(logits: torch.Tensor | None, E: int, k: int, T: int | None = None, flags: int = 0,
                topk_ids: torch.Tensor | None = None, topk_w: torch.Tensor | None = None,
                gather_src: NVFP4 | None = None, gather_dst: NVFP4 | None = None,
                ws: torch.Tensor | None = None, dev_status: torch.Tensor | None = None,
                stream=None, device="cuda", out: Routing | None = None) -> Routing:
    """Route (when logits are given) and permute.  With `out`, its buffers are reused."""
    lib = load()
    if logits is not None:
        assert logits.dtype == torch.float32 and logits.is_contiguous() and logits.shape[1] == E
        T = logits.shape[0]
        device = logits.device
    elif topk_ids is not None:
        T = topk_ids.shape[0]
        device = topk_ids.device
    if out is not None:
        if topk_ids is None:
            topk_ids = out.topk_ids
        if topk_w is None and logits is not None:
            topk_w = out.topk_w
        offsets, padded, row_token, token_row = out.offsets, out.padded_offsets, out.row_token, out.token_row
    else:
        offsets = torch.empty((E + 1,), dtype=torch.int32, device=device)
        padded = torch.empty((E + 1,), dtype=torch.int32, device=device)
        row_token = torch.empty((T * k,), dtype=torch.int32, device=device)
        token_row = torch.empty((T, k), dtype=torch.int32, device=device)
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=device)
    if topk_w is None and logits is not None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=device)
    if ws is None:
        ws = torch.empty(lib.moe_permute_workspace(T, E, k), dtype=torch.uint8, device=device)
    gs = ctypes.byref(gather_src.c()) if gather_src is not None else None
    gd = ctypes.byref(gather_dst.c()) if gather_dst is not None else None
    _check(lib.moe_permute(_ptr(logits), T, E, k, flags, _ptr(topk_ids), _ptr(topk_w), _ptr(offsets),
                           _ptr(padded), _ptr(row_token), _ptr(token_row), gs, gd, _ptr(ws), ws.numel(),
                           _ptr(dev_status), _stream(stream)))
    return Routing(topk_ids, topk_w, offsets, padded, row_token, token_row)


def moe_permute_noalloc(logits: torch.Tensor | None, E: int, k: int, out: Routing, T: int | None = None,
                        flags: int = 0, topk_ids: torch.Tensor | None = None,
                        gather_src: NVFP4 | None = None, gather_dst: NVFP4 | None = None,
                        dev_status: torch.Tensor | None = None, stream=None) -> Routing:
    """moe_permute without a workspace (the library's static one) into the caller's
    preallocated Routing buffers `out`: nothing is allocated, by the binding or the
    library, so the call can run under HIP graph capture or in a serving loop."""
    lib = load()
    if logits is not None:
        assert logits.dtype == torch.float32 and logits.is_contiguous() and logits.shape[1] == E
        T = logits.shape[0]
    elif topk_ids is not None:
        T = topk_ids.shape[0]
    ids = topk_ids if topk_ids is not None else out.topk_ids
    gs = ctypes.byref(gather_src.c()) if gather_src is not None else None
    gd = ctypes.byref(gather_dst.c()) if gather_dst is not None else None
    _check(lib.moe_permute_noalloc(_ptr(logits), T, E, k, flags, _ptr(ids),
                                   _ptr(out.topk_w) if logits is not None else None, _ptr(out.offsets),
                                   _ptr(out.padded_offsets), _ptr(out.row_token), _ptr(out.token_row), gs, gd,
                                   _ptr(dev_status), _stream(stream)))
    return Routing(ids, out.topk_w, out.offsets, out.padded_offsets, out.row_token, out.token_row)


def _gemm_ws(ws, group_mode, device, A: "NVFP4 | None" = None, B: "NVFP4 | None" = None):
    """The grouped GEMM's workspace (GROUP_K tile counter; repacked operands when K % 64
    != 0): the caller's when it is large enough, else a new one."""
    need = 256 if group_mode == NV4_GROUP_K else 0
    if A is not None and B is not None:
        a, b = A.c(), B.c()
        need = load().nvfp4_grouped_gemm_workspace(ctypes.byref(a), ctypes.byref(b), group_mode)
    if need == 0:
        return ws
    if ws is not None and ws.numel() >= need:
        return ws
    return torch.empty(need, dtype=torch.uint8, device=device)


def nvfp4_grouped_gemm(A: NVFP4, B: NVFP4, offsets: torch.Tensor, E: int, N: int, M_cap: int | None = None,
                       a_rows: torch.Tensor | None = None, group_mode: int = NV4_GROUP_M,
                       epilogue: int = NV4_EPI_NONE, out_dtype=torch.float32, C: torch.Tensor | None = None,
                       amax_out: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                       stream=None) -> torch.Tensor:
    """GROUP_M: C [M_cap, N] = per-expert A_e . B_e^T (SwiGLU: N output columns from 2N
    rows of B per expert).  GROUP_K: C [E, N=A.rows, M=B.rows] over per-expert K ranges,
    tiles balanced through the workspace `ws` (allocated when not given)."""
    lib = load()
    if group_mode == NV4_GROUP_M:
        if M_cap is None:
            M_cap = A.rows
        if C is None:
            C = torch.empty((M_cap, N), dtype=out_dtype, device=A.codes.device)
        ldc = C.stride(0)
    else:
        N = A.rows
        if C is None:
            C = torch.empty((E, A.rows, B.rows), dtype=out_dtype, device=A.codes.device)
        ldc = C.stride(1)
        M_cap = 0
    a, b = A.c(), B.c()
    ws = _gemm_ws(ws, group_mode, A.codes.device, A, B)
    _check(lib.nvfp4_grouped_gemm(ctypes.byref(a), ctypes.byref(b), _ptr(offsets), E, M_cap, N, _ptr(a_rows),
                                  group_mode, epilogue, _ptr(C), _dtype(C), ldc, _ptr(amax_out), _ptr(ws),
                                  0 if ws is None else ws.numel(), _stream(stream)))
    return C


def moe_combine(Y: torch.Tensor, token_row: torch.Tensor, topk_w: torch.Tensor, out_dtype=torch.float32,
                out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    lib = load()
    T, k = token_row.shape
    H = Y.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=Y.device)
    _check(lib.moe_combine(_ptr(Y), _dtype(Y), Y.stride(0), _ptr(token_row), _ptr(topk_w), T, k, H, _ptr(out),
                           _dtype(out), _stream(stream)))
    return out


# ----------------------------------------------------------------------------- layer composition

@dataclass
class ExpertWeights:
    """Quantised expert weights: W13 [E*2I, H] (rows gate_e then up_e; 2E scale
    segments, gate_e with tscale[2e] and up_e with tscale[2e+1]) and W2 [E*H, I]
    (one scale per expert): one tensor scale per expert and projection."""
    w13: NVFP4
    w2: NVFP4
    E: int
    H: int
    I: int


def quantize_expert_weights(W13: torch.Tensor, W2: torch.Tensor, f16: bool = False, stream=None) -> ExpertWeights:
    """W13 [E, 2I, H] and W2 [E, H, I] (BF16) -> NVFP4 with one scale per expert and
    projection (gate, up and down).  f16: also keep each tensor's exact decoded FP16
    values, which the grouped GEMMs then read instead of decoding the weights."""
    E, I2, H = W13.shape
    w13 = nvfp4_quantize(W13.reshape(E * I2, H), scale_mode=NV4_SCALE_SEGMENT, nseg=2 * E, stream=stream)
    w2 = nvfp4_quantize(W2.reshape(E * H, I2 // 2), scale_mode=NV4_SCALE_SEGMENT, nseg=E, stream=stream)
    if f16:
        with_f16(w13, stream)
        with_f16(w2, stream)
    return ExpertWeights(w13, w2, E, H, I2 // 2)


@dataclass
class ForwardBuffers:
    """Every intermediate of one forward, preallocated so that a timed forward
    enqueues kernels only."""
    xq: NVFP4
    xamax: torch.Tensor
    xg: NVFP4
    hact: torch.Tensor
    hamax: torch.Tensor
    hq: NVFP4
    y: torch.Tensor
    out: torch.Tensor
    pws: torch.Tensor
    hq_ws: torch.Tensor
    routing: Routing | None = None
    token_scale: bool = False   # per-token FP32 scales for X and the SwiGLU output
    hamax_rows: torch.Tensor | None = None  # per-row amax of the SwiGLU output (per-token mode)
    hc: NVFP4 | None = None     # [I, Kcap] the SwiGLU output's column form, filled with hq when allocated


def alloc_forward(T: int, H: int, E: int, k: int, I: int, out_dtype=torch.bfloat16, hact_dtype=torch.bfloat16,
                  device="cuda", token_scale: bool = False, hact_cols: bool = False) -> ForwardBuffers:
    """token_scale: X and the SwiGLU output carry one FP32 scale per row (the
    per-token recipe) instead of one per tensor.  hact_cols (a backward follows;
    tensor scales, BF16 SwiGLU output, I % 64 == 0): the forward also produces the
    SwiGLU output's column (token-direction) quantisation, reading it once for both
    its row and its column form; moe_backward then takes it from here."""
    lib = load()
    R = T * k
    if hact_cols and (token_scale or hact_dtype != torch.bfloat16 or I % 64):
        raise ValueError("hact_cols needs tensor scales, a BF16 SwiGLU output and I % 64 == 0")
    return ForwardBuffers(
        hc=NVFP4.empty(I, cols_capacity(R, E), 1, device) if hact_cols else None,
        xq=NVFP4.empty(T, H, T if token_scale else 1, device),
        xamax=torch.zeros((T if token_scale else 1,), dtype=torch.float32, device=device),
        xg=NVFP4.empty(R, H, 1, device),
        hact=torch.empty((R, I), dtype=hact_dtype, device=device),
        hamax=torch.zeros((1,), dtype=torch.float32, device=device),
        hq=NVFP4.empty(R, I, R if token_scale else 1, device),
        token_scale=token_scale,
        hamax_rows=torch.zeros((R,), dtype=torch.float32, device=device) if token_scale else None,
        y=torch.empty((R, H), dtype=torch.float32, device=device),
        out=torch.empty((T, H), dtype=out_dtype, device=device),
        pws=torch.empty(lib.moe_permute_workspace(T, E, k), dtype=torch.uint8, device=device),
        hq_ws=torch.empty(256, dtype=torch.uint8, device=device))


class StageEvents(list):
    """A list for ``stage_events`` that also runs ``before()`` (for example a cache
    eviction) on the launch stream ahead of every stage, outside the stage's events."""

    def __init__(self, before=None):
        super().__init__()
        self.before = before


class _Stage:
    """Optional per-stage timing: HIP events recorded on the launch stream."""

    def __init__(self, events, name, stream):
        self.events, self.name, self.stream = events, name, stream

    def __enter__(self):
        if self.events is not None:
            before = getattr(self.events, "before", None)
            if before is not None:
                with torch.cuda.stream(self.stream):
                    before()
            self.t0 = torch.cuda.Event(enable_timing=True)
            self.t0.record(self.stream)

    def __exit__(self, *exc):
        if self.events is not None:
            t1 = torch.cuda.Event(enable_timing=True)
            t1.record(self.stream)
            self.events.append((self.name, self.t0, t1))


def moe_forward(x: torch.Tensor, logits: torch.Tensor, w: ExpertWeights, k: int, bufs: ForwardBuffers | None = None,
                fuse_gather: bool = True, stream=None, stage_events: list | None = None) -> ForwardBuffers:
    """One expert-layer forward on device: returns the buffers (out holds the result).
    With stage_events (a list), (name, start_event, end_event) is appended per stage."""
    T, H = x.shape
    if bufs is None:
        bufs = alloc_forward(T, H, w.E, k, w.I, device=x.device)
    R = T * k
    mode = NV4_SCALE_ROW if bufs.token_scale else NV4_SCALE_TENSOR
    if bufs.token_scale and not fuse_gather:
        raise ValueError("per-token scales are used with the fused gather")
    st = stream if stream is not None else torch.cuda.current_stream()
    with _Stage(stage_events, "quantize_x", st):
        nvfp4_quantize(x, scale_mode=mode, out=bufs.xq, amax_out=bufs.xamax, stream=stream)
    with _Stage(stage_events, "route_permute", st):
        if fuse_gather:
            bufs.routing = moe_permute(logits, w.E, k, ws=bufs.pws, stream=stream, out=bufs.routing)
            a, a_rows = bufs.xq, bufs.routing.row_token
        else:
            bufs.routing = moe_permute(logits, w.E, k, gather_src=bufs.xq, gather_dst=bufs.xg, ws=bufs.pws,
                                       stream=stream, out=bufs.routing)
            bufs.xg.tscale = bufs.xq.tscale
            a, a_rows = bufs.xg, None
    with _Stage(stage_events, "gemm1_swiglu", st):
        bufs.hamax.zero_()
        nvfp4_grouped_gemm(a, w.w13, bufs.routing.offsets, w.E, w.I, M_cap=R, a_rows=a_rows,
                           epilogue=NV4_EPI_SWIGLU, C=bufs.hact, amax_out=bufs.hamax, stream=stream)
    with _Stage(stage_events, "quantize_hact", st):
        if bufs.token_scale:
            nvfp4_quantize(bufs.hact, scale_mode=NV4_SCALE_ROW, out=bufs.hq, amax_out=bufs.hamax_rows, stream=stream)
        elif bufs.hc is not None:
            rt = bufs.routing
            nvfp4_quantize(bufs.hact, layout=NV4_ROWS_AND_COLS, nseg=w.E, seg_offsets=rt.offsets,
                           seg_padded_offsets=rt.padded_offsets, amax_in=bufs.hamax, out=bufs.hc, out_rows=bufs.hq,
                           stream=stream)
        else:
            nvfp4_quantize(bufs.hact, amax_in=bufs.hamax, out=bufs.hq, stream=stream)
    with _Stage(stage_events, "gemm2", st):
        nvfp4_grouped_gemm(bufs.hq, w.w2, bufs.routing.offsets, w.E, H, M_cap=R, C=bufs.y, stream=stream)
    with _Stage(stage_events, "combine", st):
        moe_combine(bufs.y, bufs.routing.token_row, bufs.routing.topk_w, out=bufs.out, stream=stream)
    return bufs


# ----------------------------------------------------------------------------- backward

@dataclass
class TransposedWeights:
    """Expert weights transposed and re-quantised along their new contraction
    dimension (the operands of the data gradients): W2^T [E*I, H] (one scale per
    expert) and W13^T [E*H, 2I] (per expert, the gate scale on K [0, I) and the up
    scale on [I, 2I)): one tensor scale per expert and projection."""
    w2t: NVFP4
    w13t: NVFP4


def quantize_expert_weights_t(W13: torch.Tensor, W2: torch.Tensor, f16: bool = False,
                              stream=None) -> TransposedWeights:
    """W13 [E, 2I, H] and W2 [E, H, I] (BF16) -> per-expert transposes in NVFP4 (f16:
    with their exact decoded FP16 values, as quantize_expert_weights)."""
    E, I2, H = W13.shape
    w2t = nvfp4_quantize(W2.reshape(E * H, I2 // 2), layout=NV4_COLS_BATCHED, scale_mode=NV4_SCALE_SEGMENT,
                         nseg=E, stream=stream)
    w13t = nvfp4_quantize(W13.reshape(E * I2, H), layout=NV4_COLS_BATCHED, scale_mode=NV4_SCALE_SEGMENT_HALVES,
                          nseg=E, stream=stream)
    if f16:
        with_f16(w2t, stream)
        with_f16(w13t, stream)
    return TransposedWeights(w2t, w13t)


def cols_capacity(R: int, E: int) -> int:
    """Column capacity of a segment-transposed operand: R rows, each of E segments
    padded to 16, rounded up to 64."""
    return ((R + 15 * E + 63) // 64) * 64


@dataclass
class BackwardBuffers:
    """Every intermediate and result of one backward (preallocated)."""
    dy2q: NVFP4
    dy13q: NVFP4
    dy2_amax: torch.Tensor
    dy13_amax: torch.Tensor
    dhact: torch.Tensor     # [R, I]
    dxperm: torch.Tensor    # [R, H]
    dy2c: NVFP4             # [H, Kcap]
    hc: NVFP4               # [I, Kcap]
    dy13c: NVFP4            # [2I, Kcap]
    xc: NVFP4               # [H, Kcap]
    dw2: torch.Tensor       # [E, H, I]
    dw13: torch.Tensor      # [E, 2I, H]
    x_amax: torch.Tensor | None = None  # tensor amax of X when the forward scaled per token
    gemm_ws: torch.Tensor | None = None  # the weight-gradient GEMMs' tile-schedule workspace


def alloc_backward(T: int, H: int, E: int, k: int, I: int, dgrad_dtype=torch.bfloat16, wgrad_dtype=torch.float32,
                   device="cuda") -> BackwardBuffers:
    R = T * k
    kc = cols_capacity(R, E)
    f1 = lambda: torch.zeros((1,), dtype=torch.float32, device=device)
    return BackwardBuffers(
        dy2q=NVFP4.empty(R, H, 1, device), dy13q=NVFP4.empty(R, 2 * I, 1, device), dy2_amax=f1(), dy13_amax=f1(),
        dhact=torch.empty((R, I), dtype=dgrad_dtype, device=device),
        dxperm=torch.empty((R, H), dtype=dgrad_dtype, device=device),
        dy2c=NVFP4.empty(H, kc, 1, device), hc=NVFP4.empty(I, kc, 1, device),
        dy13c=NVFP4.empty(2 * I, kc, 1, device), xc=NVFP4.empty(H, kc, 1, device),
        dw2=torch.empty((E, H, I), dtype=wgrad_dtype, device=device),
        dw13=torch.empty((E, 2 * I, H), dtype=wgrad_dtype, device=device),
        x_amax=torch.zeros((1,), dtype=torch.float32, device=device),
        gemm_ws=torch.empty(256, dtype=torch.uint8, device=device))


def moe_backward(x: torch.Tensor, fwd: ForwardBuffers, wt: TransposedWeights, dY2: torch.Tensor,
                 dY13: torch.Tensor, bufs: BackwardBuffers | None = None, stream=None,
                 stage_events: list | None = None, dual: bool = True, sr_seed: int | None = None) -> BackwardBuffers:
    """The four backward grouped GEMMs of the expert layer, every operand re-quantised
    to NVFP4 along its new contraction dimension.

    dY2 [R, H] is the gradient of the down projection's output rows and dY13 [R, 2I]
    that of the gate/up output rows, both in expert (permuted) row order.
      dHact  = dY2_e . W2_e            (GROUP_M over H)
      dXperm = dY13_e . W13_e          (GROUP_M over 2I)
      dW2[e]  = dY2_e^T . Hact_e       (GROUP_K over expert e's tokens)
      dW13[e] = dY13_e^T . Xperm_e     (GROUP_K; Xperm = X rows in expert order)
    The tensor scale of each activation and gradient operand is the same for its
    row and column quantisation (one amax per tensor): the row pass of dY records
    it, the forward recorded those of X and of the SwiGLU output.  With `dual`, each
    upstream gradient is read once for both its row and its column quantisation
    (NV4_ROWS_AND_COLS); otherwise the two are separate passes.  With sr_seed the
    upstream gradients' elements round stochastically (the pretraining recipe's
    gradient rounding): dY2 with seed sr_seed, dY13 with sr_seed + 1."""
    T, H = x.shape
    rt = fwd.routing
    E = rt.offsets.numel() - 1
    R = rt.row_token.numel()
    k = R // T
    I = fwd.hact.shape[1]
    if bufs is None:
        bufs = alloc_backward(T, H, E, k, I, device=x.device)
    st = stream if stream is not None else torch.cuda.current_stream()
    seg = dict(layout=NV4_COLS, nseg=E, seg_offsets=rt.offsets, seg_padded_offsets=rt.padded_offsets, stream=stream)
    sr2 = None if sr_seed is None else sr_seed
    sr13 = None if sr_seed is None else sr_seed + 1
    if dual:
        both = dict(layout=NV4_ROWS_AND_COLS, nseg=E, seg_offsets=rt.offsets, seg_padded_offsets=rt.padded_offsets,
                    stream=stream)
        with _Stage(stage_events, "quantize_dy2", st):
            nvfp4_quantize(dY2, out=bufs.dy2c, out_rows=bufs.dy2q, amax_out=bufs.dy2_amax, sr_seed=sr2, **both)
        with _Stage(stage_events, "quantize_dy13", st):
            nvfp4_quantize(dY13, out=bufs.dy13c, out_rows=bufs.dy13q, amax_out=bufs.dy13_amax, sr_seed=sr13, **both)
    else:
        with _Stage(stage_events, "quantize_dy2", st):
            nvfp4_quantize(dY2, out=bufs.dy2q, amax_out=bufs.dy2_amax, sr_seed=sr2, stream=stream)
        with _Stage(stage_events, "quantize_dy13", st):
            nvfp4_quantize(dY13, out=bufs.dy13q, amax_out=bufs.dy13_amax, sr_seed=sr13, stream=stream)
    with _Stage(stage_events, "dgrad_hact", st):
        nvfp4_grouped_gemm(bufs.dy2q, wt.w2t, rt.offsets, E, I, M_cap=R, C=bufs.dhact, stream=stream)
    with _Stage(stage_events, "dgrad_x", st):
        nvfp4_grouped_gemm(bufs.dy13q, wt.w13t, rt.offsets, E, H, M_cap=R, C=bufs.dxperm, stream=stream)
    if not dual:
        with _Stage(stage_events, "quantize_cols_dy2", st):
            nvfp4_quantize(dY2, amax_in=bufs.dy2_amax, out=bufs.dy2c, sr_seed=sr2, **seg)
    hc = fwd.hc
    if hc is None:  # the forward did not produce the SwiGLU output's column form
        hc = bufs.hc
        with _Stage(stage_events, "quantize_cols_hact", st):
            nvfp4_quantize(fwd.hact, amax_in=fwd.hamax, out=hc, **seg)
    with _Stage(stage_events, "wgrad_w2", st):
        nvfp4_grouped_gemm(bufs.dy2c, hc, rt.padded_offsets, E, H, group_mode=NV4_GROUP_K, C=bufs.dw2,
                           ws=bufs.gemm_ws, stream=stream)
    if not dual:
        with _Stage(stage_events, "quantize_cols_dy13", st):
            nvfp4_quantize(dY13, amax_in=bufs.dy13_amax, out=bufs.dy13c, sr_seed=sr13, **seg)
    with _Stage(stage_events, "quantize_cols_x", st):
        if fwd.token_scale:
            # the forward recorded every token's amax: their maximum is the tensor amax
            nv4_amax(fwd.xamax, bufs.x_amax, stream=stream)
            nvfp4_quantize(x, amax_in=bufs.x_amax, out=bufs.xc, row_index=rt.row_token, **seg)
        else:
            nvfp4_quantize(x, amax_in=fwd.xamax, out=bufs.xc, row_index=rt.row_token, **seg)
    with _Stage(stage_events, "wgrad_w13", st):
        nvfp4_grouped_gemm(bufs.dy13c, bufs.xc, rt.padded_offsets, E, 2 * I, group_mode=NV4_GROUP_K, C=bufs.dw13,
                           ws=bufs.gemm_ws, stream=stream)
    return bufs


# ----------------------------------------------------------------------------- BF16 operands

def cols_capacity_bf16(R: int, E: int) -> int:
    """Column capacity of a BF16 column operand (a multiple of 32, the BF16 GEMM's stage)."""
    return cols_capacity(R, E)


def nv4_to_bf16(src, layout: int = NV4_ROWS, nseg: int = 1, seg_offsets: torch.Tensor | None = None,
                seg_padded_offsets: torch.Tensor | None = None, row_index: torch.Tensor | None = None,
                out: torch.Tensor | None = None, out_cols: int | None = None, stream=None) -> torch.Tensor:
    """A BF16 operand from `src`: a 2-D BF16 tensor, or an NVFP4 tensor whose
    BF16-dequantised values are taken.  NV4_ROWS gives [rows, K]; NV4_COLS the
    segment transpose [K, cap] (segments zero-padded to 16); NV4_COLS_BATCHED the
    per-matrix transposes [nseg*K, rows/nseg].  With row_index, logical row r is
    source row row_index[r]."""
    lib = load()
    if isinstance(src, NVFP4):
        q, x, x_rows, ldx = src.c(), None, 0, 0
        src_rows, K, device = src.rows, src.K, src.codes.device
    else:
        assert src.dim() == 2 and src.stride(1) == 1 and src.dtype == torch.bfloat16
        q, x, x_rows, ldx = None, src, src.shape[0], src.stride(0)
        src_rows, K, device = src.shape[0], src.shape[1], src.device
    rows = row_index.numel() if row_index is not None else src_rows
    if layout == NV4_ROWS:
        shape = (rows, K)
    elif layout == NV4_COLS:
        shape = (K, out_cols if out_cols is not None else cols_capacity_bf16(rows, nseg))
    else:
        shape = (nseg * K, rows // nseg)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    assert out.dtype == torch.bfloat16 and out.is_contiguous()
    _check(lib.nv4_to_bf16(_ptr(x), x_rows, ldx, None if q is None else ctypes.byref(q), rows, K, _ptr(row_index),
                           layout, nseg, _ptr(seg_offsets), _ptr(seg_padded_offsets), _ptr(out), out.shape[0],
                           out.shape[1], _stream(stream)))
    return out


def bf16_grouped_gemm(A: torch.Tensor, B: torch.Tensor, offsets: torch.Tensor, E: int, N: int,
                      M_cap: int | None = None, a_rows: torch.Tensor | None = None, group_mode: int = NV4_GROUP_M,
                      epilogue: int = NV4_EPI_NONE, out_dtype=torch.float32, C: torch.Tensor | None = None,
                      amax_out: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                      stream=None) -> torch.Tensor:
    """nvfp4_grouped_gemm on BF16 operands A [a_rows, K] and B [b_rows, K] (K contiguous)."""
    lib = load()
    for t in (A, B):
        assert t.dtype == torch.bfloat16 and t.dim() == 2 and t.is_contiguous()
    K = A.shape[1]
    assert B.shape[1] == K
    if group_mode == NV4_GROUP_M:
        if M_cap is None:
            M_cap = A.shape[0]
        if C is None:
            C = torch.empty((M_cap, N), dtype=out_dtype, device=A.device)
        ldc = C.stride(0)
    else:
        N = A.shape[0]
        if C is None:
            C = torch.empty((E, A.shape[0], B.shape[0]), dtype=out_dtype, device=A.device)
        ldc = C.stride(1)
        M_cap = 0
    ws = _gemm_ws(ws, group_mode, A.device)
    _check(lib.bf16_grouped_gemm(_ptr(A), A.shape[0], _ptr(B), B.shape[0], K, _ptr(offsets), E, M_cap, N,
                                 _ptr(a_rows), group_mode, epilogue, _ptr(C), _dtype(C), ldc, _ptr(amax_out),
                                 _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    return C


# ----------------------------------------------------------------------------- BF16 layer and backward

@dataclass
class BF16TransposedWeights:
    """BF16 expert weights transposed for the data gradients: W2^T [E*I, H] and
    W13^T [E*H, 2I] (either the BF16 weights or the BF16 values of their NVFP4
    forward form)."""
    w2t: torch.Tensor
    w13t: torch.Tensor


def bf16_expert_weights_t(W13: torch.Tensor, W2: torch.Tensor, stream=None) -> BF16TransposedWeights:
    """Transposes of the BF16 weights W13 [E, 2I, H] and W2 [E, H, I]."""
    E, I2, H = W13.shape
    w2t = nv4_to_bf16(W2.reshape(E * H, I2 // 2), layout=NV4_COLS_BATCHED, nseg=E, stream=stream)
    w13t = nv4_to_bf16(W13.reshape(E * I2, H), layout=NV4_COLS_BATCHED, nseg=E, stream=stream)
    return BF16TransposedWeights(w2t, w13t)


def dequantize_expert_weights_t(w: ExpertWeights, stream=None) -> BF16TransposedWeights:
    """Transposes of the BF16-dequantised NVFP4 weights of the forward (DQ(Q(W)))."""
    w2t = nv4_to_bf16(w.w2, layout=NV4_COLS_BATCHED, nseg=w.E, stream=stream)
    w13t = nv4_to_bf16(w.w13, layout=NV4_COLS_BATCHED, nseg=w.E, stream=stream)
    return BF16TransposedWeights(w2t, w13t)


@dataclass
class BF16ForwardBuffers:
    hact: torch.Tensor      # [R, I] BF16
    y: torch.Tensor         # [R, H] FP32
    out: torch.Tensor       # [T, H]
    pws: torch.Tensor
    routing: Routing | None = None


def alloc_forward_bf16(T: int, H: int, E: int, k: int, I: int, out_dtype=torch.bfloat16,
                       device="cuda") -> BF16ForwardBuffers:
    lib = load()
    R = T * k
    return BF16ForwardBuffers(hact=torch.empty((R, I), dtype=torch.bfloat16, device=device),
                              y=torch.empty((R, H), dtype=torch.float32, device=device),
                              out=torch.empty((T, H), dtype=out_dtype, device=device),
                              pws=torch.empty(lib.moe_permute_workspace(T, E, k), dtype=torch.uint8, device=device))


def moe_forward_bf16(x: torch.Tensor, logits: torch.Tensor, W13: torch.Tensor, W2: torch.Tensor, k: int,
                     bufs: BF16ForwardBuffers | None = None, stream=None,
                     stage_events: list | None = None) -> BF16ForwardBuffers:
    """The unquantised expert layer: W13 [E, 2I, H], W2 [E, H, I] in BF16; the same
    routing, permutation, SwiGLU and combine as ``moe_forward``."""
    T, H = x.shape
    E, I2, _ = W13.shape
    I = I2 // 2
    if bufs is None:
        bufs = alloc_forward_bf16(T, H, E, k, I, device=x.device)
    R = T * k
    st = stream if stream is not None else torch.cuda.current_stream()
    with _Stage(stage_events, "route_permute", st):
        bufs.routing = moe_permute(logits, E, k, ws=bufs.pws, stream=stream, out=bufs.routing)
    with _Stage(stage_events, "gemm1_swiglu", st):
        bf16_grouped_gemm(x, W13.reshape(E * I2, H), bufs.routing.offsets, E, I, M_cap=R,
                          a_rows=bufs.routing.row_token, epilogue=NV4_EPI_SWIGLU, C=bufs.hact, stream=stream)
    with _Stage(stage_events, "gemm2", st):
        bf16_grouped_gemm(bufs.hact, W2.reshape(E * H, I), bufs.routing.offsets, E, H, M_cap=R, C=bufs.y,
                          stream=stream)
    with _Stage(stage_events, "combine", st):
        moe_combine(bufs.y, bufs.routing.token_row, bufs.routing.topk_w, out=bufs.out, stream=stream)
    return bufs


@dataclass
class BF16BackwardBuffers:
    dhact: torch.Tensor     # [R, I]
    dxperm: torch.Tensor    # [R, H]
    dy2c: torch.Tensor      # [H, Kcap] BF16
    hc: torch.Tensor        # [I, Kcap]
    dy13c: torch.Tensor     # [2I, Kcap]
    xc: torch.Tensor        # [H, Kcap]
    dw2: torch.Tensor       # [E, H, I]
    dw13: torch.Tensor      # [E, 2I, H]
    gemm_ws: torch.Tensor | None = None  # the weight-gradient GEMMs' tile-schedule workspace


def alloc_backward_bf16(T: int, H: int, E: int, k: int, I: int, dgrad_dtype=torch.bfloat16,
                        wgrad_dtype=torch.float32, device="cuda") -> BF16BackwardBuffers:
    R = T * k
    kc = cols_capacity_bf16(R, E)
    b = lambda r: torch.empty((r, kc), dtype=torch.bfloat16, device=device)
    return BF16BackwardBuffers(
        dhact=torch.empty((R, I), dtype=dgrad_dtype, device=device),
        dxperm=torch.empty((R, H), dtype=dgrad_dtype, device=device),
        dy2c=b(H), hc=b(I), dy13c=b(2 * I), xc=b(H),
        dw2=torch.empty((E, H, I), dtype=wgrad_dtype, device=device),
        dw13=torch.empty((E, 2 * I, H), dtype=wgrad_dtype, device=device),
        gemm_ws=torch.empty(256, dtype=torch.uint8, device=device))


def moe_backward_bf16(x_op, hact_op, wt: BF16TransposedWeights, dY2: torch.Tensor, dY13: torch.Tensor,
                      routing: Routing, bufs: BF16BackwardBuffers | None = None, stream=None,
                      stage_events: list | None = None) -> BF16BackwardBuffers:
    """The four backward grouped GEMMs of ``moe_backward`` on BF16 operands, with
    the upstream gradients dY2 [R, H] and dY13 [R, 2I] (expert row order) in BF16.

    x_op is X [T, H] in BF16 or the forward's NVFP4 X; hact_op is the SwiGLU output
    [R, I] in BF16 or the forward's NVFP4 form of it.  An NVFP4 operand enters as
    its BF16-dequantised values: with the forward's NVFP4 tensors and
    ``dequantize_expert_weights_t`` this is the dequantized backward; with the
    BF16 tensors and ``bf16_expert_weights_t`` the BF16 backward."""
    rt = routing
    E = rt.offsets.numel() - 1
    R = rt.row_token.numel()
    H = dY2.shape[1]
    I = dY13.shape[1] // 2
    T = x_op.rows if isinstance(x_op, NVFP4) else x_op.shape[0]
    if bufs is None:
        bufs = alloc_backward_bf16(T, H, E, R // T, I, device=dY2.device)
    st = stream if stream is not None else torch.cuda.current_stream()
    seg = dict(layout=NV4_COLS, nseg=E, seg_offsets=rt.offsets, seg_padded_offsets=rt.padded_offsets, stream=stream)
    with _Stage(stage_events, "dgrad_hact", st):
        bf16_grouped_gemm(dY2, wt.w2t, rt.offsets, E, I, M_cap=R, C=bufs.dhact, stream=stream)
    with _Stage(stage_events, "dgrad_x", st):
        bf16_grouped_gemm(dY13, wt.w13t, rt.offsets, E, H, M_cap=R, C=bufs.dxperm, stream=stream)
    with _Stage(stage_events, "cols_dy2_hact", st):
        nv4_to_bf16(dY2, out=bufs.dy2c, **seg)
        nv4_to_bf16(hact_op, out=bufs.hc, **seg)
    with _Stage(stage_events, "wgrad_w2", st):
        bf16_grouped_gemm(bufs.dy2c, bufs.hc, rt.padded_offsets, E, H, group_mode=NV4_GROUP_K, C=bufs.dw2,
                          ws=bufs.gemm_ws, stream=stream)
    with _Stage(stage_events, "cols_dy13_x", st):
        nv4_to_bf16(dY13, out=bufs.dy13c, **seg)
        nv4_to_bf16(x_op, out=bufs.xc, row_index=rt.row_token, **seg)
    with _Stage(stage_events, "wgrad_w13", st):
        bf16_grouped_gemm(bufs.dy13c, bufs.xc, rt.padded_offsets, E, 2 * I, group_mode=NV4_GROUP_K, C=bufs.dw13,
                          ws=bufs.gemm_ws, stream=stream)
    return bufs


# ----------------------------------------------------------------------------- measurement kernels

def nv4_bench_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """Stream-copy src into dst (same byte size, a multiple of 16): 2x the bytes of HBM traffic."""
    nb = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() == nb
    _check(load().nv4_bench_copy(_ptr(src), _ptr(dst), nb, _stream(stream)))


def nv4_bench_read(src: torch.Tensor, sink: torch.Tensor, never: int = 0xDEADBEEF, stream=None) -> None:
    """Stream-read src (a pure read stream unless the XOR of its words equals `never`)."""
    _check(load().nv4_bench_read(_ptr(src), src.numel() * src.element_size(), ctypes.c_uint32(never), _ptr(sink),
                                 _stream(stream)))


def nv4_bench_mix(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """Read all of src and write a quarter of its bytes to dst (a quantiser's traffic mix)."""
    nb = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() >= nb // 4
    _check(load().nv4_bench_mix(_ptr(src), nb, _ptr(dst), _stream(stream)))


def nv4_bench_mfma(out: torch.Tensor | None, iters: int, waves_per_simd: int = 2, stream=None) -> tuple:
    """A loop of FP16 MFMAs on every SIMD; returns (out, FLOPs of the call)."""
    lib = load()
    n = lib.nv4_bench_mfma_out_floats(waves_per_simd)
    if out is None or out.numel() < n:
        out = torch.empty(n, dtype=torch.float32, device="cuda")
    _check(lib.nv4_bench_mfma(_ptr(out), iters, waves_per_simd, _stream(stream)))
    return out, (n // 64) * iters * 8 * 32768


def nv4_bench_write(dst: torch.Tensor, stream=None) -> None:
    """Fill dst (16-byte multiple) with 16-byte stores."""
    _check(load().nv4_bench_write(_ptr(dst), dst.numel() * dst.element_size(), _stream(stream)))


def nv4_bench_lds(out: torch.Tensor | None, iters: int, stream=None) -> tuple:
    """16-byte LDS reads on every compute unit; returns (out, LDS bytes read by the call)."""
    lib = load()
    n = lib.nv4_bench_lds_out_words()
    if out is None or out.numel() < n:
        out = torch.empty(n, dtype=torch.int32, device="cuda")
    _check(lib.nv4_bench_lds(_ptr(out), iters, _stream(stream)))
    return out, n * iters * 8 * 16
