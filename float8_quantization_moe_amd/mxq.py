"""Python binding of libmxq (ctypes): argument marshalling only.

Every function has the name of the C entry point it calls (see include/mxq.h)
and takes torch tensors for the device buffers; torch is used for device memory
and streams only.  All arithmetic runs in the HIP kernels of libmxq.so.  There
is no fallback: if the library is missing or a call fails, an exception is
raised.

Sources of the operations: "[mxfp8 MoE training] Support mxfp8 all to all in
expert parallel" (Summary) for the MXFP8 codec, "[moe training] fix
uncoalesced global accesses in per group rowwise scaling kernel" (Summary) for
the group scaling and the layout transform, and "[float8] add float8 rowwise
MoE prototype" (Summary) for the scaled grouped GEMM.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmxq.so")

MXQ_LAYOUT_ROW = 0
MXQ_LAYOUT_COL = 1
MXQ_OK = 0
MXQ_ERR_NULL, MXQ_ERR_SHAPE, MXQ_ERR_ALIGN, MXQ_ERR_LAYOUT, MXQ_ERR_WORKSPACE, MXQ_ERR_HIP = 1, 2, 3, 4, 5, 6
MXQ_ERR_DTYPE = 8
MXQ_ERR_RULE = 9
MXQ_OUT_BF16 = 0
MXQ_OUT_F32 = 1
MXQ_SCALE_FLOOR = 0
MXQ_SCALE_RCEIL = 1
MXQ_GROUP_POW2_SCALE = 1
MXQ_GROUP_INVERSE_SCALE = 2

EXPORTED = ("mxq_abi_version", "mxq_status_string", "mxq_last_hip_error", "mxq_quantize_mx",
            "mxq_dequantize_mx", "mxq_group_scale_workspace_bytes", "mxq_group_scale_fp8",
            "mxq_transpose_u8", "mxq_grouped_mm_workspace_bytes", "mxq_scaled_grouped_mm",
            "mxq_quantize_mx_ex", "mxq_dequantize_mx_ex", "mxq_group_scale_fp8_ex",
            "mxq_dispatch_pack_workspace_bytes", "mxq_dispatch_pack_mx", "mxq_scaled_grouped_mm_packed",
            "mxq_set_group_scale_knobs", "mxq_group_scale_fp8_noalloc", "mxq_group_scale_route_counters")

GROUP_METHODS = {"auto": 0, "hold": 1, "twopass": 2, "split": 3}


class MxqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().mxq_status_string(status).decode()
        if status == MXQ_ERR_HIP:
            msg += f" (hipError {lib().mxq_last_hip_error()})"
        super().__init__(f"{where}: {msg}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmxq.so.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libmxq.so not found at {LIB_PATH}; build it with "
                              "`python -m float8_quantization_moe_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, P, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
        L.mxq_abi_version.restype = ctypes.c_int
        L.mxq_abi_version.argtypes = []
        L.mxq_status_string.restype = ctypes.c_char_p
        L.mxq_status_string.argtypes = [ctypes.c_int]
        L.mxq_last_hip_error.restype = ctypes.c_int
        L.mxq_last_hip_error.argtypes = []
        L.mxq_quantize_mx.restype = ctypes.c_int
        L.mxq_quantize_mx.argtypes = [P, i64, i64, P, P, P]
        L.mxq_dequantize_mx.restype = ctypes.c_int
        L.mxq_dequantize_mx.argtypes = [P, P, i64, i64, P, P]
        L.mxq_quantize_mx_ex.restype = ctypes.c_int
        L.mxq_quantize_mx_ex.argtypes = [P, i64, i64, ctypes.c_int, ctypes.c_int, P, P, P]
        L.mxq_dequantize_mx_ex.restype = ctypes.c_int
        L.mxq_dequantize_mx_ex.argtypes = [P, P, i64, i64, ctypes.c_int, P, P]
        L.mxq_group_scale_workspace_bytes.restype = sz
        L.mxq_group_scale_workspace_bytes.argtypes = [i64, i64, i32]
        L.mxq_group_scale_fp8.restype = ctypes.c_int
        L.mxq_group_scale_fp8.argtypes = [P, i64, i64, P, i32, ctypes.c_int, P, P, P, sz, P]
        L.mxq_group_scale_fp8_ex.restype = ctypes.c_int
        L.mxq_group_scale_fp8_ex.argtypes = [P, i64, i64, P, i32, ctypes.c_int, ctypes.c_int, P, P, P, sz, P]
        L.mxq_transpose_u8.restype = ctypes.c_int
        L.mxq_transpose_u8.argtypes = [P, i64, i64, P, P]
        L.mxq_grouped_mm_workspace_bytes.restype = sz
        L.mxq_grouped_mm_workspace_bytes.argtypes = [i64, i64, i64, i32]
        L.mxq_dispatch_pack_workspace_bytes.restype = sz
        L.mxq_dispatch_pack_workspace_bytes.argtypes = [i64, i64, i32, i32]
        L.mxq_dispatch_pack_mx.restype = ctypes.c_int
        L.mxq_dispatch_pack_mx.argtypes = [P, i64, i64, P, i32, i32, P, P, P, P, sz, P]
        L.mxq_scaled_grouped_mm_packed.restype = ctypes.c_int
        L.mxq_scaled_grouped_mm_packed.argtypes = [P, P, P, P, i64, i64, i64, i32, ctypes.c_int, P, P, sz, P]
        L.mxq_group_scale_fp8_noalloc.restype = ctypes.c_int
        L.mxq_group_scale_fp8_noalloc.argtypes = [P, i64, i64, P, i32, ctypes.c_int, ctypes.c_int, P, P, P]
        L.mxq_set_group_scale_knobs.restype = ctypes.c_int
        L.mxq_set_group_scale_knobs.argtypes = [ctypes.c_int, ctypes.c_int, i64, ctypes.c_int]
        L.mxq_group_scale_route_counters.restype = ctypes.c_int
        L.mxq_group_scale_route_counters.argtypes = [P, sz, i64, i64, i32, ctypes.c_int, P, P]
        L.mxq_scaled_grouped_mm.restype = ctypes.c_int
        L.mxq_scaled_grouped_mm.argtypes = [P, P, P, P, P, i64, i64, i64, i32, ctypes.c_int, P, P, sz, P]
        _lib = L
    return _lib


def mxq_set_group_scale_knobs(method: str = "auto", hold_tiles: int = -1, wait_us: int = -1,
                              strip_block: int = 0) -> None:
    """Test hook: force the group-scaling route (see include/mxq.h).  Defaults restore the automatic choice."""
    _check(lib().mxq_set_group_scale_knobs(GROUP_METHODS[method], int(hold_tiles), int(wait_us), int(strip_block)),
           "mxq_set_group_scale_knobs")


def mxq_group_scale_route_counters(workspace: torch.Tensor, M: int, K: int, G: int, out_layout: int,
                                   stream=None) -> tuple:
    """Test hook: the hold method's (timed-out tiles, strips re-read from X) of the
    last call that used `workspace` (see include/mxq.h).  Synchronises the stream."""
    out = (ctypes.c_uint32 * 2)()
    pw = _dev(workspace, "workspace")
    wbytes = workspace.numel() * workspace.element_size()
    _check(lib().mxq_group_scale_route_counters(pw, wbytes, int(M), int(K), int(G), int(out_layout), out,
                                                _stream(stream)), "mxq_group_scale_route_counters")
    return int(out[0]), int(out[1])


@contextlib.contextmanager
def group_scale_knobs(**kw):
    """Context manager around mxq_set_group_scale_knobs that restores the defaults on exit."""
    mxq_set_group_scale_knobs(**kw)
    try:
        yield
    finally:
        mxq_set_group_scale_knobs()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(t: torch.Tensor, name: str, dtype=None, numel=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()}")
    return t.data_ptr()


def _check(status: int, where: str) -> None:
    if status != MXQ_OK:
        raise MxqError(status, where)


def mxq_abi_version() -> int:
    return lib().mxq_abi_version()


def mxq_quantize_mx(x: torch.Tensor, q: torch.Tensor, s: torch.Tensor, stream=None) -> None:
    """x (M, K) bf16 -> q (M, K) uint8 E4M3 codes, s (M, K/32) uint8 E8M0 codes."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D (M, K)")
    M, K = x.shape
    px = _dev(x, "x", torch.bfloat16)
    pq = _dev(q, "q", torch.uint8, M * K)
    ps = _dev(s, "s", torch.uint8, M * (K // 32) if K % 32 == 0 else None)
    _check(lib().mxq_quantize_mx(px, M, K, pq, ps, _stream(stream)), "mxq_quantize_mx")


def mxq_dequantize_mx(q: torch.Tensor, s: torch.Tensor, y: torch.Tensor, stream=None) -> None:
    """q (M, K) uint8 E4M3 + s (M, K/32) uint8 E8M0 -> y (M, K) bf16."""
    if y.dim() != 2:
        raise ValueError("y must be 2-D (M, K)")
    M, K = y.shape
    pq = _dev(q, "q", torch.uint8, M * K)
    ps = _dev(s, "s", torch.uint8, M * (K // 32) if K % 32 == 0 else None)
    py = _dev(y, "y", torch.bfloat16)
    _check(lib().mxq_dequantize_mx(pq, ps, M, K, py, _stream(stream)), "mxq_dequantize_mx")


def _mx_scale_numel(M: int, K: int, axis: int):
    if axis == 1:
        return M * (K // 32) if K % 32 == 0 else None
    if axis == 0:
        return (M // 32) * K if M % 32 == 0 else None
    return None


def mxq_quantize_mx_ex(x: torch.Tensor, axis: int, rule: int, q: torch.Tensor, s: torch.Tensor,
                       stream=None) -> None:
    """MX variants: x (M, K) bf16 -> q (M, K) uint8 E4M3 and s E8M0 codes, (M, K/32) for
    axis 1 or (M/32, K) for axis 0; rule MXQ_SCALE_FLOOR or MXQ_SCALE_RCEIL."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D (M, K)")
    M, K = x.shape
    px = _dev(x, "x", torch.bfloat16)
    pq = _dev(q, "q", torch.uint8, M * K)
    ps = _dev(s, "s", torch.uint8, _mx_scale_numel(M, K, axis))
    _check(lib().mxq_quantize_mx_ex(px, M, K, int(axis), int(rule), pq, ps, _stream(stream)), "mxq_quantize_mx_ex")


def mxq_dequantize_mx_ex(q: torch.Tensor, s: torch.Tensor, axis: int, y: torch.Tensor, stream=None) -> None:
    """Inverse of mxq_quantize_mx_ex for either axis -> y (M, K) bf16."""
    if y.dim() != 2:
        raise ValueError("y must be 2-D (M, K)")
    M, K = y.shape
    pq = _dev(q, "q", torch.uint8, M * K)
    ps = _dev(s, "s", torch.uint8, _mx_scale_numel(M, K, axis))
    py = _dev(y, "y", torch.bfloat16)
    _check(lib().mxq_dequantize_mx_ex(pq, ps, M, K, int(axis), py, _stream(stream)), "mxq_dequantize_mx_ex")


def mxq_group_scale_workspace_bytes(M: int, K: int, G: int) -> int:
    return int(lib().mxq_group_scale_workspace_bytes(int(M), int(K), int(G)))


def mxq_group_scale_fp8(x: torch.Tensor, group_end_offs: torch.Tensor, out_layout: int,
                        q: torch.Tensor, scales: torch.Tensor, workspace: torch.Tensor,
                        stream=None) -> None:
    """x (M, K) bf16, group_end_offs int32[G] (device) -> q uint8 ((M, K) for ROW,
    (K, M) for COL) and scales float32 (G, K)."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D (M, K)")
    M, K = x.shape
    G = group_end_offs.numel()
    px = _dev(x, "x", torch.bfloat16)
    po = _dev(group_end_offs, "group_end_offs", torch.int32)
    pq = _dev(q, "q", torch.uint8, M * K)
    ps = _dev(scales, "scales", torch.float32, G * K)
    pw = _dev(workspace, "workspace")
    wbytes = workspace.numel() * workspace.element_size()
    _check(lib().mxq_group_scale_fp8(px, M, K, po, G, int(out_layout), pq, ps, pw, wbytes, _stream(stream)),
           "mxq_group_scale_fp8")


def mxq_group_scale_fp8_ex(x: torch.Tensor, group_end_offs: torch.Tensor, out_layout: int, flags: int,
                           q: torch.Tensor, scales: torch.Tensor, workspace: torch.Tensor,
                           stream=None) -> None:
    """mxq_group_scale_fp8 with flags MXQ_GROUP_POW2_SCALE / MXQ_GROUP_INVERSE_SCALE."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D (M, K)")
    M, K = x.shape
    G = group_end_offs.numel()
    px = _dev(x, "x", torch.bfloat16)
    po = _dev(group_end_offs, "group_end_offs", torch.int32)
    pq = _dev(q, "q", torch.uint8, M * K)
    ps = _dev(scales, "scales", torch.float32, G * K)
    pw = _dev(workspace, "workspace")
    wbytes = workspace.numel() * workspace.element_size()
    _check(lib().mxq_group_scale_fp8_ex(px, M, K, po, G, int(out_layout), int(flags), pq, ps, pw, wbytes,
                                        _stream(stream)), "mxq_group_scale_fp8_ex")


def mxq_group_scale_fp8_noalloc(x: torch.Tensor, group_end_offs: torch.Tensor, out_layout: int, flags: int,
                                q: torch.Tensor, scales: torch.Tensor, stream=None) -> None:
    """mxq_group_scale_fp8_ex with the library's static per-GPU scratch instead of a workspace."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D (M, K)")
    M, K = x.shape
    G = group_end_offs.numel()
    px = _dev(x, "x", torch.bfloat16)
    po = _dev(group_end_offs, "group_end_offs", torch.int32)
    pq = _dev(q, "q", torch.uint8, M * K)
    ps = _dev(scales, "scales", torch.float32, G * K)
    _check(lib().mxq_group_scale_fp8_noalloc(px, M, K, po, G, int(out_layout), int(flags), pq, ps,
                                             _stream(stream)), "mxq_group_scale_fp8_noalloc")


def mxq_transpose_u8(inp: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    """out (C, R) = inp (R, C)^T for uint8 tensors."""
    if inp.dim() != 2:
        raise ValueError("inp must be 2-D")
    R, C = inp.shape
    pi = _dev(inp, "inp", torch.uint8)
    po = _dev(out, "out", torch.uint8, R * C)
    _check(lib().mxq_transpose_u8(pi, R, C, po, _stream(stream)), "mxq_transpose_u8")


def mxq_grouped_mm_workspace_bytes(M: int, N: int, K: int, G: int) -> int:
    return int(lib().mxq_grouped_mm_workspace_bytes(int(M), int(N), int(K), int(G)))


def mxq_scaled_grouped_mm(xq: torch.Tensor, xs: torch.Tensor, wq: torch.Tensor, ws: torch.Tensor,
                          group_end_offs: torch.Tensor, y: torch.Tensor, workspace: torch.Tensor,
                          stream=None) -> None:
    """xq (M, K) / xs (M, K/32) and wq (G, N, K) / ws (G, N, K/32) uint8 MXFP8
    operands, group_end_offs int32[G] (device) -> y (M, N) bf16 or float32."""
    if xq.dim() != 2 or wq.dim() != 3 or y.dim() != 2:
        raise ValueError("xq must be (M, K), wq (G, N, K) and y (M, N)")
    M, K = xq.shape
    G, N, Kw = wq.shape
    if Kw != K or tuple(y.shape) != (M, N):
        raise ValueError("operand shapes do not match")
    if group_end_offs.numel() != G:
        raise ValueError("need one end offset per group")
    if y.dtype == torch.bfloat16:
        out_dtype = MXQ_OUT_BF16
    elif y.dtype == torch.float32:
        out_dtype = MXQ_OUT_F32
    else:
        raise TypeError("y must be bfloat16 or float32")
    kb = K // 32 if K % 32 == 0 else None
    pxq = _dev(xq, "xq", torch.uint8)
    pxs = _dev(xs, "xs", torch.uint8, M * kb if kb is not None else None)
    pwq = _dev(wq, "wq", torch.uint8)
    pws = _dev(ws, "ws", torch.uint8, G * N * kb if kb is not None else None)
    po = _dev(group_end_offs, "group_end_offs", torch.int32)
    py = _dev(y, "y")
    pw = _dev(workspace, "workspace")
    wbytes = workspace.numel() * workspace.element_size()
    _check(lib().mxq_scaled_grouped_mm(pxq, pxs, pwq, pws, po, M, N, K, G, out_dtype, py, pw, wbytes,
                                       _stream(stream)), "mxq_scaled_grouped_mm")


# ---------------------------------------------------------------- helpers ---
# Allocate outputs with torch and call the entry points above.

def quantize_mx(x: torch.Tensor, stream=None):
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    s = torch.empty((M, K // 32), dtype=torch.uint8, device=x.device)
    mxq_quantize_mx(x, q, s, stream)
    return q, s


def dequantize_mx(q: torch.Tensor, s: torch.Tensor, stream=None) -> torch.Tensor:
    y = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    mxq_dequantize_mx(q, s, y, stream)
    return y


def group_scale_fp8(x: torch.Tensor, group_end_offs: torch.Tensor, out_layout: int = MXQ_LAYOUT_ROW,
                    stream=None):
    M, K = x.shape
    G = group_end_offs.numel()
    q = torch.empty((M, K) if out_layout == MXQ_LAYOUT_ROW else (K, M), dtype=torch.uint8, device=x.device)
    scales = torch.empty((G, K), dtype=torch.float32, device=x.device)
    ws = torch.empty(max(mxq_group_scale_workspace_bytes(M, K, G), 16), dtype=torch.uint8, device=x.device)
    mxq_group_scale_fp8(x, group_end_offs, out_layout, q, scales, ws, stream)
    return q, scales


def transpose_u8(inp: torch.Tensor, stream=None) -> torch.Tensor:
    R, C = inp.shape
    out = torch.empty((C, R), dtype=torch.uint8, device=inp.device)
    mxq_transpose_u8(inp, out, stream)
    return out


def scaled_grouped_mm(xq: torch.Tensor, xs: torch.Tensor, wq: torch.Tensor, ws: torch.Tensor,
                      group_end_offs: torch.Tensor, out_dtype=torch.bfloat16, stream=None) -> torch.Tensor:
    M, K = xq.shape
    G, N, _ = wq.shape
    y = torch.empty((M, N), dtype=out_dtype, device=xq.device)
    wsp = torch.empty(max(mxq_grouped_mm_workspace_bytes(M, N, K, G), 16), dtype=torch.uint8,
                      device=xq.device)
    mxq_scaled_grouped_mm(xq, xs, wq, ws, group_end_offs, y, wsp, stream)
    return y


def mxq_dispatch_pack_workspace_bytes(M: int, K: int, topk: int, E: int) -> int:
    return int(lib().mxq_dispatch_pack_workspace_bytes(int(M), int(K), int(topk), int(E)))


def mxq_dispatch_pack_mx(x: torch.Tensor, expert_ids: torch.Tensor, E: int, packed: torch.Tensor,
                         group_end_offs: torch.Tensor, src_pair: torch.Tensor, workspace: torch.Tensor,
                         stream=None) -> None:
    """x (M, K) bf16, expert_ids (M, topk) int32 -> packed (M*topk, K + K/32) uint8 rows
    [e4m3 | e8m0] sorted stably by expert, group_end_offs int32[E], src_pair int32[M*topk]."""
    if x.dim() != 2 or expert_ids.dim() != 2 or expert_ids.shape[0] != x.shape[0]:
        raise ValueError("x must be (M, K) and expert_ids (M, topk)")
    M, K = x.shape
    topk = expert_ids.shape[1]
    px = _dev(x, "x", torch.bfloat16)
    pi = _dev(expert_ids, "expert_ids", torch.int32)
    pp = _dev(packed, "packed", torch.uint8, M * topk * (K + K // 32))
    pe = _dev(group_end_offs, "group_end_offs", torch.int32, int(E))
    ps = _dev(src_pair, "src_pair", torch.int32, M * topk)
    pw = _dev(workspace, "workspace")
    wbytes = workspace.numel() * workspace.element_size()
    _check(lib().mxq_dispatch_pack_mx(px, M, K, pi, topk, int(E), pp, pe, ps, pw, wbytes, _stream(stream)),
           "mxq_dispatch_pack_mx")


def mxq_scaled_grouped_mm_packed(packed: torch.Tensor, wq: torch.Tensor, ws: torch.Tensor,
                                 group_end_offs: torch.Tensor, y: torch.Tensor, workspace: torch.Tensor,
                                 stream=None) -> None:
    """packed (M, K + K/32) uint8 token rows [e4m3 | e8m0], wq (G, N, K) / ws (G, N, K/32) ->
    y (M, N), bf16 or float32 by y's dtype."""
    if packed.dim() != 2 or wq.dim() != 3 or y.dim() != 2:
        raise ValueError("packed must be 2-D, wq 3-D (G, N, K), y 2-D (M, N)")
    G, N, K = wq.shape
    M = packed.shape[0]
    if packed.shape[1] != K + K // 32 or tuple(y.shape) != (M, N):
        raise ValueError("shapes do not match")
    dt = {torch.bfloat16: MXQ_OUT_BF16, torch.float32: MXQ_OUT_F32}.get(y.dtype)
    if dt is None:
        raise TypeError("y must be bfloat16 or float32")
    pp = _dev(packed, "packed", torch.uint8)
    pwq = _dev(wq, "wq", torch.uint8)
    pws = _dev(ws, "ws", torch.uint8, G * N * (K // 32))
    po = _dev(group_end_offs, "group_end_offs", torch.int32, G)
    py = _dev(y, "y")
    pw = _dev(workspace, "workspace")
    wbytes = workspace.numel() * workspace.element_size()
    _check(lib().mxq_scaled_grouped_mm_packed(pp, pwq, pws, po, M, N, K, G, dt, py, pw, wbytes, _stream(stream)),
           "mxq_scaled_grouped_mm_packed")
