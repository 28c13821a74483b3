"""CPU oracle for the float8 MoE quantization path -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never does, and this package imports nothing from it.

The arithmetic lives in ``oracle.c`` (plain scalar C, compiled here with gcc);
this module only marshals numpy arrays.  bf16 tensors travel as ``uint16`` bit
patterns, E4M3 / E8M0 codes as ``uint8``.

Pages followed (see the header of ``oracle.c`` for the readings):
  "[mxfp8 MoE training] Support mxfp8 all to all in expert parallel", Summary;
  "[moe training] fix uncoalesced global accesses in per group rowwise scaling
  kernel", Summary.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra"]

LAYOUT_ROW = 0
LAYOUT_COL = 1
RULE_FLOOR = 0
RULE_RCEIL = 1
GROUP_POW2_SCALE = 1
GROUP_INVERSE_SCALE = 2


def compile_source(src: str, out: str) -> str:
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build() -> str:
    """Compile oracle.c into liboracle.so next to it (always recompiles)."""
    return compile_source(SOURCE, LIB_PATH)


_u8, _u16, _i32, _i64, _f32, _f64 = (ctypes.c_uint8, ctypes.c_uint16, ctypes.c_int32,
                                     ctypes.c_int64, ctypes.c_float, ctypes.c_double)
_P = ctypes.c_void_p
_SIGS = {
    "oracle_abi_version": (ctypes.c_int, []),
    "oracle_bf16_value": (_f64, [_u16]),
    "oracle_bf16_round": (_u16, [_f64]),
    "oracle_e4m3_decode": (_f64, [_u8]),
    "oracle_e4m3_encode": (_u8, [_f64]),
    "oracle_e8m0_decode": (_f64, [_u8]),
    "oracle_mx_encode_element": (_u8, [_u16, _u8]),
    "oracle_mx_decode_element": (_u16, [_u8, _u8]),
    "oracle_mx_quantize": (None, [_P, _i64, _i64, _P, _P]),
    "oracle_mx_dequantize": (None, [_P, _P, _i64, _i64, _P]),
    "oracle_mx_quantize_ex": (None, [_P, _i64, _i64, ctypes.c_int, ctypes.c_int, _P, _P]),
    "oracle_mx_dequantize_ex": (None, [_P, _P, _i64, _i64, ctypes.c_int, _P]),
    "oracle_group_scale_value": (_f32, [_f32]),
    "oracle_group_encode_element": (_u8, [_u16, _f32]),
    "oracle_group_scale": (None, [_P, _i64, _i64, _P, _i32, ctypes.c_int, _P, _P]),
    "oracle_group_scale_ex": (None, [_P, _i64, _i64, _P, _i32, ctypes.c_int, ctypes.c_int, _P, _P]),
    "oracle_transpose_u8": (None, [_P, _i64, _i64, _P]),
    "oracle_dispatch_pack": (None, [_P, _i64, _i64, _P, _i32, _i32, _P, _P, _P]),
    "oracle_mx_encode_elements": (None, [_P, _P, _i64, _P]),
    "oracle_mx_decode_elements": (None, [_P, _P, _i64, _P]),
    "oracle_e4m3_encode_f32_array": (None, [_P, _i64, _P]),
    "oracle_bf16_round_f64_array": (None, [_P, _i64, _P]),
    "oracle_group_encode_elements": (None, [_P, _P, _i64, _P]),
    "oracle_mx_grouped_mm": (None, [_P, _P, _P, _P, _P, _i64, _i64, _i64, _i32,
                                    _P, _i64, _P, _i64, _P]),
}


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _as_u16(x) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError(f"expected uint16 bf16 bit patterns, got {x.dtype}")
    return x


class Oracle:
    """numpy front end of one compiled copy of oracle.c."""

    def __init__(self, path: str):
        L = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        self._L = L
        self.path = path

    # ------------------------------------------------------------ scalars --
    def bf16_value(self, bits: int) -> float:
        return self._L.oracle_bf16_value(int(bits))

    def bf16_round(self, v: float) -> int:
        return self._L.oracle_bf16_round(float(v))

    def e4m3_decode(self, code: int) -> float:
        return self._L.oracle_e4m3_decode(int(code))

    def e4m3_encode(self, y: float) -> int:
        return self._L.oracle_e4m3_encode(float(y))

    def e8m0_decode(self, code: int) -> float:
        return self._L.oracle_e8m0_decode(int(code))

    def mx_encode_element(self, xbits: int, scale_code: int) -> int:
        return self._L.oracle_mx_encode_element(int(xbits), int(scale_code))

    def mx_decode_element(self, q: int, scale_code: int) -> int:
        return self._L.oracle_mx_decode_element(int(q), int(scale_code))

    def group_scale_value(self, amax: float) -> float:
        return self._L.oracle_group_scale_value(float(amax))

    def group_encode_element(self, xbits: int, s: float) -> int:
        return self._L.oracle_group_encode_element(int(xbits), float(s))

    # ------------------------------------------------------------- arrays --
    def mx_quantize(self, x_bits):
        """(M, K) uint16 bf16 bits -> (q (M, K) uint8 E4M3, s (M, K/32) uint8 E8M0)."""
        x = _as_u16(x_bits)
        M, K = x.shape
        if K % 32:
            raise ValueError("K must be a multiple of 32")
        q = np.empty((M, K), np.uint8)
        s = np.empty((M, K // 32), np.uint8)
        if M and K:
            self._L.oracle_mx_quantize(_ptr(x), M, K, _ptr(q), _ptr(s))
        return q, s

    def mx_dequantize(self, q, s):
        """E4M3 (M, K) + E8M0 (M, K/32) -> (M, K) uint16 bf16 bits."""
        q = np.ascontiguousarray(q, dtype=np.uint8)
        s = np.ascontiguousarray(s, dtype=np.uint8)
        M, K = q.shape
        if K % 32 or s.shape != (M, K // 32):
            raise ValueError("scale shape must be (M, K/32)")
        y = np.empty((M, K), np.uint16)
        if M and K:
            self._L.oracle_mx_dequantize(_ptr(q), _ptr(s), M, K, _ptr(y))
        return y

    def mx_quantize_ex(self, x_bits, axis: int = 1, rule: int = RULE_FLOOR):
        """MX variants: axis 1 = blocks of 32 along a row (scales (M, K/32)), axis 0 =
        blocks of 32 rows of a column (scales (M/32, K)); rule RULE_FLOOR or RULE_RCEIL.
        Returns (q (M, K) uint8 E4M3 in X's layout, s uint8 E8M0)."""
        x = _as_u16(x_bits)
        M, K = x.shape
        if axis not in (0, 1) or rule not in (RULE_FLOOR, RULE_RCEIL):
            raise ValueError("axis must be 0 or 1, rule RULE_FLOOR or RULE_RCEIL")
        if (axis == 1 and K % 32) or (axis == 0 and M % 32):
            raise ValueError("the blocked dimension must be a multiple of 32")
        q = np.empty((M, K), np.uint8)
        s = np.empty((M, K // 32) if axis == 1 else (M // 32, K), np.uint8)
        if M and K:
            self._L.oracle_mx_quantize_ex(_ptr(x), M, K, int(axis), int(rule), _ptr(q), _ptr(s))
        return q, s

    def mx_dequantize_ex(self, q, s, axis: int = 1):
        """Inverse of mx_quantize_ex for either axis -> (M, K) uint16 bf16 bits."""
        q = np.ascontiguousarray(q, dtype=np.uint8)
        s = np.ascontiguousarray(s, dtype=np.uint8)
        M, K = q.shape
        want = (M, K // 32) if axis == 1 else (M // 32, K)
        if axis not in (0, 1) or (axis == 1 and K % 32) or (axis == 0 and M % 32) or s.shape != want:
            raise ValueError("scale shape does not match the axis")
        y = np.empty((M, K), np.uint16)
        if M and K:
            self._L.oracle_mx_dequantize_ex(_ptr(q), _ptr(s), M, K, int(axis), _ptr(y))
        return y

    def group_scale(self, x_bits, group_end, layout: int = LAYOUT_ROW):
        """Per-(group, column) float8 scaling.

        Returns (q, scales): q is (M, K) for LAYOUT_ROW or (K, M) for LAYOUT_COL;
        scales is (G, K) float32, the multiplier applied before the cast."""
        x = _as_u16(x_bits)
        M, K = x.shape
        ends = np.ascontiguousarray(np.asarray(group_end, dtype=np.int32))
        G = int(ends.shape[0])
        if G < 1:
            raise ValueError("need at least one group")
        q = np.empty((M, K) if layout == LAYOUT_ROW else (K, M), np.uint8)
        scales = np.empty((G, K), np.float32)
        self._L.oracle_group_scale(_ptr(x), M, K, _ptr(ends), G, int(layout), _ptr(q), _ptr(scales))
        return q, scales

    def group_scale_ex(self, x_bits, group_end, layout: int = LAYOUT_ROW, flags: int = 0):
        """Group scaling with the variant flags GROUP_POW2_SCALE (multiplier rounded down
        to a power of two) and GROUP_INVERSE_SCALE (1/s stored instead of s)."""
        x = _as_u16(x_bits)
        M, K = x.shape
        ends = np.ascontiguousarray(np.asarray(group_end, dtype=np.int32))
        G = int(ends.shape[0])
        if G < 1:
            raise ValueError("need at least one group")
        if flags & ~(GROUP_POW2_SCALE | GROUP_INVERSE_SCALE):
            raise ValueError("unknown flag")
        q = np.empty((M, K) if layout == LAYOUT_ROW else (K, M), np.uint8)
        scales = np.empty((G, K), np.float32)
        self._L.oracle_group_scale_ex(_ptr(x), M, K, _ptr(ends), G, int(layout), int(flags), _ptr(q), _ptr(scales))
        return q, scales

    def dispatch_pack(self, x_bits, expert_ids, E: int):
        """Dispatch pack: x (M, K) bf16 bits, expert_ids (M, topk) int32 -> (packed
        (M*topk, K + K/32) uint8 rows [e4m3 codes | e8m0 scales] ordered stably by
        expert, src_pair (M*topk,) int32 pair index t*topk + j of each row (-1 past
        the last end), group_end (E,) int32).  Rows past the last end are zero here
        (the oracle writes nothing there)."""
        x = _as_u16(x_bits)
        M, K = x.shape
        ids = np.ascontiguousarray(np.asarray(expert_ids, dtype=np.int32))
        if ids.ndim != 2 or ids.shape[0] != M or K % 32 or E < 1:
            raise ValueError("expert_ids must be (M, topk), K a multiple of 32, E >= 1")
        topk = ids.shape[1]
        P = M * topk
        packed = np.zeros((P, K + K // 32), np.uint8)
        src = np.empty(P, np.int32)
        ends = np.empty(E, np.int32)
        self._L.oracle_dispatch_pack(_ptr(x), M, K, _ptr(ids), topk, E, _ptr(packed), _ptr(src), _ptr(ends))
        return packed, src, ends

    def transpose_u8(self, a):
        a = np.ascontiguousarray(a, dtype=np.uint8)
        R, C = a.shape
        out = np.empty((C, R), np.uint8)
        if R and C:
            self._L.oracle_transpose_u8(_ptr(a), R, C, _ptr(out))
        return out

    def mx_grouped_mm(self, xq, xs, wq, ws, group_end, rows=None, cols=None):
        """Y[rows][:, cols] of the grouped product of MXFP8 operands, float64.

        xq (M, K) / xs (M, K/32): tokens; wq (G, N, K) / ws (G, N, K/32): one
        weight per group; Y[m, n] = sum_k x(m, k) w_g(n, k) for m in group g,
        0 for rows past the last (clamped) end.  rows / cols default to all."""
        xq = np.ascontiguousarray(xq, dtype=np.uint8)
        xs = np.ascontiguousarray(xs, dtype=np.uint8)
        wq = np.ascontiguousarray(wq, dtype=np.uint8)
        ws = np.ascontiguousarray(ws, dtype=np.uint8)
        M, K = xq.shape
        G, N, Kw = wq.shape
        if Kw != K or K % 32 or xs.shape != (M, K // 32) or ws.shape != (G, N, K // 32):
            raise ValueError("operand shapes do not match")
        ends = np.ascontiguousarray(np.asarray(group_end, dtype=np.int32))
        if ends.shape != (G,):
            raise ValueError("need one end offset per group")
        rows = np.arange(M, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
        cols = np.arange(N, dtype=np.int64) if cols is None else np.ascontiguousarray(cols, np.int64)
        if rows.size and (rows.min() < 0 or rows.max() >= M):
            raise ValueError("row index out of range")
        if cols.size and (cols.min() < 0 or cols.max() >= N):
            raise ValueError("column index out of range")
        y = np.zeros((rows.size, cols.size), np.float64)
        if rows.size and cols.size:
            self._L.oracle_mx_grouped_mm(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), _ptr(ends),
                                         M, N, K, G, _ptr(rows), rows.size, _ptr(cols),
                                         cols.size, _ptr(y))
        return y

    # ----------------------------------------------- element-wise arrays --
    def mx_encode_elements(self, x_bits, scale_codes):
        """E4M3 code of each bf16 x under the E8M0 scale code beside it (finite blocks)."""
        x = _as_u16(x_bits).ravel()
        c = np.ascontiguousarray(scale_codes, dtype=np.uint8).ravel()
        if x.shape != c.shape:
            raise ValueError("shape mismatch")
        out = np.empty(x.shape, np.uint8)
        self._L.oracle_mx_encode_elements(_ptr(x), _ptr(c), x.size, _ptr(out))
        return out

    def mx_decode_elements(self, q, scale_codes):
        q = np.ascontiguousarray(q, dtype=np.uint8).ravel()
        c = np.ascontiguousarray(scale_codes, dtype=np.uint8).ravel()
        if q.shape != c.shape:
            raise ValueError("shape mismatch")
        out = np.empty(q.shape, np.uint16)
        self._L.oracle_mx_decode_elements(_ptr(q), _ptr(c), q.size, _ptr(out))
        return out

    def e4m3_encode_f32(self, y):
        y = np.ascontiguousarray(y, dtype=np.float32).ravel()
        out = np.empty(y.shape, np.uint8)
        self._L.oracle_e4m3_encode_f32_array(_ptr(y), y.size, _ptr(out))
        return out

    def bf16_round_f64(self, v):
        v = np.ascontiguousarray(v, dtype=np.float64).ravel()
        out = np.empty(v.shape, np.uint16)
        self._L.oracle_bf16_round_f64_array(_ptr(v), v.size, _ptr(out))
        return out

    def group_encode_elements(self, x_bits, s):
        x = _as_u16(x_bits).ravel()
        s = np.ascontiguousarray(s, dtype=np.float32).ravel()
        if x.shape != s.shape:
            raise ValueError("shape mismatch")
        out = np.empty(x.shape, np.uint8)
        self._L.oracle_group_encode_elements(_ptr(x), _ptr(s), x.size, _ptr(out))
        return out


_default = None


def default() -> Oracle:
    """The oracle compiled from oracle.c (built on first use if missing)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            build()
        _default = Oracle(LIB_PATH)
    return _default


def __getattr__(name):
    # module-level access to the default instance's methods: oracle.mx_quantize(...)
    if not name.startswith("_") and hasattr(Oracle, name):
        return getattr(default(), name)
    raise AttributeError(name)
