"""The C-ABI library without a GPU: it loads, exports every entry point the
header declares, and rejects bad arguments on the host before touching a device
(no kernel is ever launched here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxq.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mxq_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    from float8_quantization_moe_amd import mxq
    if not os.path.exists(mxq.LIB_PATH):
        pytest.fail("libmxq.so is not built (run `python -m float8_quantization_moe_amd.build`)")
    return mxq.lib()


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("mxq_quantize_mx", "mxq_dequantize_mx", "mxq_group_scale_fp8",
              "mxq_group_scale_workspace_bytes", "mxq_transpose_u8", "mxq_abi_version",
              "mxq_grouped_mm_workspace_bytes", "mxq_scaled_grouped_mm", "mxq_quantize_mx_ex",
              "mxq_dequantize_mx_ex", "mxq_group_scale_fp8_ex", "mxq_dispatch_pack_workspace_bytes",
              "mxq_dispatch_pack_mx", "mxq_scaled_grouped_mm_packed"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    from float8_quantization_moe_amd import mxq
    raw = ctypes.CDLL(mxq.LIB_PATH)
    for name in _declared():
        assert hasattr(raw, name), f"{name} is declared in mxq.h but not exported"
    assert sorted(mxq.EXPORTED) == _declared()


def test_abi_version_and_status_strings(L):
    assert L.mxq_abi_version() == 1
    for code in range(0, 10):
        assert L.mxq_status_string(code).startswith(b"MXQ_")
    assert L.mxq_status_string(99) == b"unknown mxq_status"
    assert L.mxq_last_hip_error() == 0


A = 1 << 20   # a fake, 16-byte aligned "device" address.  Every call below either fails
              # validation or is a no-op, so nothing is ever enqueued with it.


def test_quantize_mx_argument_errors(L):
    S = 0
    assert L.mxq_quantize_mx(A, 4, 31, A, A, S) == 2          # K % 32
    assert L.mxq_quantize_mx(A, -1, 32, A, A, S) == 2         # negative
    assert L.mxq_quantize_mx(A, 1 << 30, 1 << 30, A, A, S) == 2  # too large
    assert L.mxq_quantize_mx(0, 4, 32, A, A, S) == 1          # null
    assert L.mxq_quantize_mx(A, 4, 32, 0, A, S) == 1
    assert L.mxq_quantize_mx(A, 4, 32, A, 0, S) == 1
    assert L.mxq_quantize_mx(A + 8, 4, 32, A, A, S) == 3      # misaligned
    assert L.mxq_quantize_mx(A, 4, 32, A + 1, A, S) == 3
    assert L.mxq_quantize_mx(0, 0, 32, 0, 0, S) == 0          # empty: no-op
    assert L.mxq_quantize_mx(0, 7, 0, 0, 0, S) == 0


def test_dequantize_mx_argument_errors(L):
    S = 0
    assert L.mxq_dequantize_mx(A, A, 4, 48, A, S) == 2
    assert L.mxq_dequantize_mx(0, A, 4, 32, A, S) == 1
    assert L.mxq_dequantize_mx(A, 0, 4, 32, A, S) == 1
    assert L.mxq_dequantize_mx(A, A, 4, 32, 0, S) == 1
    assert L.mxq_dequantize_mx(A, A + 4, 4, 32, A, S) == 3
    assert L.mxq_dequantize_mx(0, 0, 0, 64, 0, S) == 0


def test_mx_variant_argument_errors(L):
    S = 0
    q, d = L.mxq_quantize_mx_ex, L.mxq_dequantize_mx_ex
    assert q(A, 64, 64, 2, 0, A, A, S) == 4                    # unknown axis
    assert q(A, 64, 64, -1, 0, A, A, S) == 4
    assert q(A, 64, 64, 1, 2, A, A, S) == 9                    # unknown rule
    assert q(A, 64, 64, 0, -1, A, A, S) == 9
    assert q(A, 4, 48, 1, 1, A, A, S) == 2                     # axis 1: K % 32
    assert q(A, 48, 64, 0, 1, A, A, S) == 2                    # axis 0: M % 32
    assert q(A, 64, 6, 0, 0, A, A, S) == 2                     # axis 0: K % 4
    assert q(A, 32, (1 << 24) + 4, 0, 0, A, A, S) == 2         # axis 0: K too large
    assert q(A, 1 << 36, 1024, 0, 0, A, A, S) == 2             # axis 0: grid too large
    assert q(0, 64, 64, 0, 1, A, A, S) == 1                    # null
    assert q(A, 64, 64, 0, 1, A, 0, S) == 1
    assert q(A, 64, 64, 0, 1, A + 4, A, S) == 3                # misaligned
    assert q(0, 0, 64, 0, 1, 0, 0, S) == 0                     # empty: no-op
    assert d(A, A, 64, 64, 3, A, S) == 4
    assert d(A, A, 40, 64, 0, A, S) == 2
    assert d(A, A, 64, 64, 0, 0, S) == 1
    assert d(A, A + 8, 64, 64, 0, A, S) == 3
    assert d(0, 0, 64, 0, 0, 0, S) == 0


def test_group_scale_argument_errors(L):
    S = 0
    ws = L.mxq_group_scale_workspace_bytes(512, 256, 4)
    assert ws > 0 and ws % 256 == 0
    assert L.mxq_group_scale_workspace_bytes(512, 250, 4) == 0   # K % 8
    assert L.mxq_group_scale_workspace_bytes(512, 256, 0) == 0   # G < 1
    assert L.mxq_group_scale_workspace_bytes(-1, 256, 4) == 0
    f = L.mxq_group_scale_fp8
    assert f(A, 512, 252, A, 4, 0, A, A, A, ws, S) == 2           # K % 8
    assert f(A, 512, 256, A, 0, 0, A, A, A, ws, S) == 2           # G < 1
    assert f(A, 1 << 31, 256, A, 4, 0, A, A, A, ws, S) == 2       # rows beyond int32 offsets
    assert f(A, 512, 256, A, 4, 2, A, A, A, ws, S) == 4           # layout
    assert f(A, 512, 256, A, 4, -1, A, A, A, ws, S) == 4
    assert f(0, 512, 256, A, 4, 0, A, A, A, ws, S) == 1           # null x
    assert f(A, 512, 256, 0, 4, 0, A, A, A, ws, S) == 1           # null offsets
    assert f(A, 512, 256, A, 4, 0, 0, A, A, ws, S) == 1           # null q
    assert f(A, 512, 256, A, 4, 0, A, 0, A, ws, S) == 1           # null scales
    assert f(A, 512, 256, A, 4, 0, A, A, 0, ws, S) == 5           # no workspace
    assert f(A, 512, 256, A, 4, 0, A, A, A, ws - 1, S) == 5       # workspace too small
    assert f(A + 2, 512, 256, A, 4, 0, A, A, A, ws, S) == 3       # misaligned x
    assert f(A, 512, 256, A + 2, 4, 0, A, A, A, ws, S) == 3       # misaligned offsets
    assert f(A, 512, 256, A, 4, 0, A, A + 4, A, ws, S) == 3       # misaligned scales
    assert f(A, 512, 0, A, 4, 0, A, A, A, ws, S) == 0             # K == 0: no-op
    fx = L.mxq_group_scale_fp8_ex
    assert fx(A, 512, 256, A, 4, 0, 4, A, A, A, ws, S) == 9      # unknown flag bit
    na = L.mxq_group_scale_fp8_noalloc                           # allocation-free variant: host checks first
    assert na(A, 512, 252, A, 4, 0, 0, A, A, S) == 2              # K % 8
    assert na(A, 512, 256, A, 4, 2, 0, A, A, S) == 4              # layout
    assert na(A, 512, 256, A, 4, 0, 4, A, A, S) == 9              # flag
    assert na(A, 512, 256, A, 4, 0, 0, 0, A, S) == 1              # null q
    assert na(A, 512, 256, A + 2, 4, 0, 0, A, A, S) == 3          # misaligned offsets
    assert L.mxq_group_scale_workspace_bytes(262144, 8192, 16) > (16 << 20)
    assert na(A, 262144, 8192, A, 16, 0, 0, A, A, S) == 5         # needs more than the 16 MiB scratch
    assert na(A, 512, 0, A, 4, 0, 0, A, A, S) == 0                # K == 0: no-op
    k = L.mxq_set_group_scale_knobs                              # the route hook: method 0..2 only
    assert k(4, -1, -1, 0) == 9 and k(-1, -1, -1, 0) == 9
    assert k(2, 5, 0, 2) == 0 and k(0, -1, -1, 0) == 0
    assert fx(A, 512, 256, A, 4, 0, -1, A, A, A, ws, S) == 9
    assert fx(A, 512, 256, A, 4, 2, 1, A, A, A, ws, S) == 4      # layout before flags
    assert fx(A, 512, 252, A, 4, 0, 3, A, A, A, ws, S) == 2
    assert fx(A, 512, 256, A, 4, 0, 3, A, A, A, ws - 1, S) == 5
    assert fx(A, 512, 0, A, 4, 0, 3, A, A, A, ws, S) == 0


def test_dispatch_pack_argument_errors(L):
    S = 0
    wb = L.mxq_dispatch_pack_workspace_bytes
    ws = wb(1000, 5120, 1, 16)
    assert ws == 4 * 16 * 4                                   # 4 blocks of 256 pairs x 16 experts
    assert wb(1000, 5120, 2, 16) == 8 * 16 * 4
    assert wb(1000, 5000, 1, 16) == 0                         # K % 256
    assert wb(1000, 0, 1, 16) == 0                            # K == 0
    assert wb(1000, 5120, 0, 16) == 0 and wb(1000, 5120, 65, 16) == 0   # topk
    assert wb(1000, 5120, 1, 0) == 0 and wb(1000, 5120, 1, 1025) == 0   # experts
    assert wb(1 << 31, 256, 1, 4) == 0                        # pairs beyond int32
    f = L.mxq_dispatch_pack_mx
    assert f(A, 1000, 5000, A, 1, 16, A, A, A, A, ws, S) == 2
    assert f(A, 1000, 5120, A, 1, 2000, A, A, A, A, ws, S) == 2
    assert f(A, 1000, 5120, A, 1, 16, A, 0, A, A, ws, S) == 1      # null group ends
    assert f(0, 1000, 5120, A, 1, 16, A, A, A, A, ws, S) == 1      # null x
    assert f(A, 1000, 5120, 0, 1, 16, A, A, A, A, ws, S) == 1      # null ids
    assert f(A, 1000, 5120, A, 1, 16, 0, A, A, A, ws, S) == 1      # null packed
    assert f(A, 1000, 5120, A, 1, 16, A, A, 0, A, ws, S) == 1      # null src_pair
    assert f(A, 1000, 5120, A, 1, 16, A, A, A, 0, ws, S) == 5      # no workspace
    assert f(A, 1000, 5120, A, 1, 16, A, A, A, A, ws - 1, S) == 5
    assert f(A + 4, 1000, 5120, A, 1, 16, A, A, A, A, ws, S) == 3  # misaligned x
    assert f(A, 1000, 5120, A + 2, 1, 16, A, A, A, A, ws, S) == 3  # misaligned ids
    assert f(A, 1000, 5120, A, 1, 16, A + 8, A, A, A, ws, S) == 3  # misaligned packed
    assert f(A, 1000, 5120, A, 1, 16, A, A + 1, A, A, ws, S) == 3  # misaligned group ends


def test_grouped_mm_packed_argument_errors(L):
    S = 0
    need = L.mxq_grouped_mm_workspace_bytes(300, 256, 5120, 4)
    g = L.mxq_scaled_grouped_mm_packed
    assert g(A, A, A, A, 300, 256, 5120 - 128, 4, 0, A, A, need, S) == 2    # K % 512
    assert g(A, A, A, A, 300, 250, 5120, 4, 0, A, A, need, S) == 2          # N % 8
    assert g(A, A, A, A, 300, 256, 5120, 4, 2, A, A, need, S) == 8          # dtype
    assert g(0, A, A, A, 300, 256, 5120, 4, 0, A, A, need, S) == 1
    assert g(A + 4, A, A, A, 300, 256, 5120, 4, 0, A, A, need, S) == 3
    assert g(A, A, A, A, 300, 256, 5120, 4, 0, A, A, need - 1, S) == 5
    assert g(0, 0, 0, 0, 0, 256, 5120, 4, 0, 0, 0, 0, S) == 0               # M == 0: no-op


def test_transpose_argument_errors(L):
    S = 0
    assert L.mxq_transpose_u8(A, -3, 4, A, S) == 2
    assert L.mxq_transpose_u8(0, 3, 4, A, S) == 1
    assert L.mxq_transpose_u8(A, 3, 4, 0, S) == 1
    assert L.mxq_transpose_u8(A + 1, 3, 4, A, S) == 3
    assert L.mxq_transpose_u8(0, 0, 4, 0, S) == 0


def test_grouped_mm_argument_errors(L):
    S = 0
    M, N, K, G = 700, 264, 384, 5
    ws = L.mxq_grouped_mm_workspace_bytes(M, N, K, G)
    assert ws >= 16 + 16 * ((M + 255) // 256 + G + 1) * ((N + 255) // 256)
    assert L.mxq_grouped_mm_workspace_bytes(M, N, 320, G) == 0        # K % 128
    assert L.mxq_grouped_mm_workspace_bytes(M, N, 0, G) == 0          # K == 0
    assert L.mxq_grouped_mm_workspace_bytes(M, 260, K, G) == 0        # N % 8
    assert L.mxq_grouped_mm_workspace_bytes(M, N, K, 0) == 0          # G < 1
    assert L.mxq_grouped_mm_workspace_bytes(M, N, K, 4096) == 0       # G > 4095
    assert L.mxq_grouped_mm_workspace_bytes(M, N, K, 4095) > 0
    assert L.mxq_grouped_mm_workspace_bytes(M, N, 1 << 24, G) == 0    # K too large
    f = L.mxq_scaled_grouped_mm
    args = lambda **kw: [kw.get(k, d) for k, d in (
        ("xq", A), ("xs", A), ("wq", A), ("wsc", A), ("offs", A), ("M", M), ("N", N), ("K", K),
        ("G", G), ("dt", 0), ("y", A), ("ws", A), ("wb", ws), ("s", S))]
    assert f(*args(K=320)) == 2
    assert f(*args(N=12)) == 2
    assert f(*args(G=0)) == 2
    assert f(*args(M=-1)) == 2
    assert f(*args(dt=2)) == 8                                          # unknown output type
    assert f(*args(xq=0)) == 1
    assert f(*args(xs=0)) == 1
    assert f(*args(wq=0)) == 1
    assert f(*args(wsc=0)) == 1
    assert f(*args(offs=0)) == 1
    assert f(*args(y=0)) == 1
    assert f(*args(xq=A + 8)) == 3
    assert f(*args(wsc=A + 4)) == 3
    assert f(*args(y=A + 8)) == 3
    assert f(*args(offs=A + 2)) == 3
    assert f(*args(ws=0)) == 5
    assert f(*args(wb=ws - 1)) == 5
    assert f(*args(M=0, xq=0, y=0)) == 0                                # empty: no-op
    assert f(*args(N=0, wq=0, y=0)) == 0


def test_binding_refuses_host_tensors():
    import torch
    from float8_quantization_moe_amd import mxq
    x = torch.zeros((4, 32), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mxq.mxq_quantize_mx(x, torch.zeros(128, dtype=torch.uint8), torch.zeros(4, dtype=torch.uint8))


def test_product_path_does_not_import_the_oracle():
    """The HIP binding and package never reference the oracle."""
    pkg = os.path.join(ROOT, "float8_quantization_moe_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "oracle" not in text.lower(), f"{fn} mentions the oracle"


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built library every entry point raises: there is no fallback path."""
    import torch
    from float8_quantization_moe_amd import mxq
    monkeypatch.setattr(mxq, "LIB_PATH", str(tmp_path / "libmxq.so"))
    monkeypatch.setattr(mxq, "_lib", None)
    with pytest.raises(ImportError, match="libmxq.so not found"):
        mxq.lib()
    with pytest.raises(ImportError):
        mxq.mxq_abi_version()
