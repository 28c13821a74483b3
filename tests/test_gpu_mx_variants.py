"""MXFP8 variants on the GPU -- the RCEIL scale rule and blocks along dim 0 --
bit-exact against the CPU oracle.

"[mxfp8 MoE training] Support mxfp8 all to all in expert parallel", Summary:
the e4m3 + e8m0 encoding of the payload; the scale rule and the blocking axis
are the two choices the format leaves to its user (readings of this
repository).  Every byte of codes, scales and the bf16 round trip is compared.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import gpu_util as U
import oracle
import workloads as W
from float8_quantization_moe_amd import mxq

pytestmark = pytest.mark.gpu

FLOOR, RCEIL = mxq.MXQ_SCALE_FLOOR, mxq.MXQ_SCALE_RCEIL
VARIANTS = [(1, FLOOR), (1, RCEIL), (0, FLOOR), (0, RCEIL)]
VIDS = ["rows-floor", "rows-rceil", "cols-floor", "cols-rceil"]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "these tests need an MI355X"
    mxq.lib()
    yield


def _scale_shape(M, K, axis):
    return (M, K // 32) if axis == 1 else (M // 32, K)


def oracle_quantize(x_bits, axis, rule):
    """The oracle's variant quantizer, rows (axis 1) or columns (axis 0) split across threads."""
    M, K = x_bits.shape
    q = np.empty((M, K), np.uint8)
    s = np.empty(_scale_shape(M, K, axis), np.uint8)
    if axis == 1:
        parts = U._row_slices(M, U.THREADS * 2)
    else:
        step = max(4, -(-K // (U.THREADS * 2)))
        parts = [(a, min(K, a + step)) for a in range(0, K, step)]

    def run(sl):
        a, b = sl
        if axis == 1:
            q[a:b], s[a:b] = oracle.mx_quantize_ex(np.ascontiguousarray(x_bits[a:b]), 1, rule)
        else:
            q[:, a:b], s[:, a:b] = oracle.mx_quantize_ex(np.ascontiguousarray(x_bits[:, a:b]), 0, rule)

    with ThreadPoolExecutor(U.THREADS) as ex:
        list(ex.map(run, parts))
    return q, s


def oracle_dequantize(q, s, axis):
    M, K = q.shape
    y = np.empty((M, K), np.uint16)
    if axis == 1:
        parts = U._row_slices(M, U.THREADS * 2)
    else:
        step = max(4, -(-K // (U.THREADS * 2)))
        parts = [(a, min(K, a + step)) for a in range(0, K, step)]

    def run(sl):
        a, b = sl
        if axis == 1:
            y[a:b] = oracle.mx_dequantize_ex(np.ascontiguousarray(q[a:b]), np.ascontiguousarray(s[a:b]), 1)
        else:
            y[:, a:b] = oracle.mx_dequantize_ex(np.ascontiguousarray(q[:, a:b]), np.ascontiguousarray(s[:, a:b]), 0)

    with ThreadPoolExecutor(U.THREADS) as ex:
        list(ex.map(run, parts))
    return y


def _roundtrip(x_bits, axis, rule, name):
    M, K = x_bits.shape
    sshape = _scale_shape(M, K, axis)
    print(f"case {name} M={M} K={K} axis={axis} rule={rule}", flush=True)
    x = U.dev_bf16(x_bits)
    qg = U.Guarded(M * K, torch.uint8, (M, K))
    sg = U.Guarded(sshape[0] * sshape[1], torch.uint8, sshape)
    mxq.mxq_quantize_mx_ex(x, axis, rule, qg.t, sg.t)
    yg = U.Guarded(M * K, torch.bfloat16, (M, K))
    mxq.mxq_dequantize_mx_ex(qg.t, sg.t, axis, yg.t)
    torch.cuda.synchronize()
    q, s = oracle_quantize(x_bits, axis, rule)
    gq, gs = U.host_u8(qg.t), U.host_u8(sg.t)
    assert np.array_equal(gs, s), f"{name} scales: {U.first_mismatch(gs, s)}"
    assert np.array_equal(gq, q), f"{name} codes: {U.first_mismatch(gq, q)}"
    y = oracle_dequantize(q, s, axis)
    gy = U.host_u16(yg.t)
    assert np.array_equal(gy, y), f"{name} dequant: {U.first_mismatch(gy, y)}"
    assert qg.guard_intact() and sg.guard_intact() and yg.guard_intact(), f"{name}: wrote past the end"
    return gq, gs


@pytest.mark.parametrize("axis,rule", VARIANTS, ids=VIDS)
def test_tiny(axis, rule):
    _roundtrip(W.bf16_bits(W.tiny_x(0)), axis, rule, "tiny (512, 256)")


@pytest.mark.parametrize("axis,rule", VARIANTS, ids=VIDS)
def test_every_element_under_every_scale(axis, rule):
    """The exhaustive blocks of the plain codec's test (every finite element with
    every block maximum, subnormal maxima, Inf/NaN blocks), as rows for axis 1
    and as columns for axis 0."""
    blocks = U.exhaustive_mx_blocks()
    nb = blocks.shape[0]
    if axis == 1:
        nb8 = -(-nb // 8) * 8
        x_bits = np.concatenate([blocks, np.zeros((nb8 - nb, 32), np.uint16)]).reshape(-1, 256)
    else:
        nb4 = -(-nb // 4) * 4
        x_bits = np.ascontiguousarray(np.concatenate([blocks, np.zeros((nb4 - nb, 32), np.uint16)]).T)
    _roundtrip(x_bits, axis, rule, "exhaustive blocks")


def test_rceil_every_block_maximum():
    """Under RCEIL every finite |bf16| pattern as a block maximum, with and without
    the mantissa past 1.75 that moves the scale up: the maximum plus 31 random
    smaller elements of either sign, as rows and as columns."""
    rng = np.random.default_rng(3)
    amax = np.arange(0, 0x7F80, dtype=np.uint32)
    others = (rng.random((amax.size, 31)) * (amax[:, None] + 1)).astype(np.uint32)
    blocks = np.concatenate([amax[:, None], others], axis=1).astype(np.uint16)
    blocks |= (rng.integers(0, 2, blocks.shape) << 15).astype(np.uint16)
    for i in range(blocks.shape[0]):
        rng.shuffle(blocks[i])
    _roundtrip(blocks.reshape(-1, 256), 1, RCEIL, "every maximum, rows")
    _roundtrip(np.ascontiguousarray(blocks.T), 0, RCEIL, "every maximum, columns")


def test_dequantize_dim0_every_code_under_every_scale():
    """Column k carries scale code k in all 8 of its blocks and rows run through
    the 256 codes: every (E4M3 code, E8M0 code) pair along dim 0."""
    q = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 256, axis=1)
    s = np.tile(np.arange(256, dtype=np.uint8), (8, 1))
    yg = U.Guarded(q.size, torch.bfloat16, q.shape)
    mxq.mxq_dequantize_mx_ex(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda(), 0, yg.t)
    torch.cuda.synchronize()
    want = oracle_dequantize(q, s, 0)
    got = U.host_u16(yg.t)
    assert np.array_equal(got, want), U.first_mismatch(got, want)
    assert yg.guard_intact()


@pytest.mark.parametrize("M,K", [(32, 4), (32, 1028), (64, 2052), (96, 8), (4096, 12), (256, 5120)])
@pytest.mark.parametrize("rule", [FLOOR, RCEIL], ids=["floor", "rceil"])
def test_dim0_edge_shapes(M, K, rule):
    """Partial 1024-column workgroups, single blocks, narrow and tall shapes."""
    x = W.lognormal_rows(M, K, seed=M * 3 + K).to(torch.bfloat16)
    _roundtrip(W.bf16_bits(x), 0, rule, f"({M}, {K})")


@pytest.mark.parametrize("M,K", [(1, 32), (37, 1056), (4097, 32)])
def test_rceil_rows_edge_shapes(M, K):
    x = W.lognormal_rows(M, K, seed=M * 5 + K).to(torch.bfloat16)
    _roundtrip(W.bf16_bits(x), 1, RCEIL, f"({M}, {K})")


def test_rows_floor_is_the_plain_codec():
    """mxq_quantize_mx_ex(axis 1, floor) writes the same bytes as mxq_quantize_mx."""
    x = U.dev_bf16(W.bf16_bits(W.lognormal_rows(300, 1024, seed=11).to(torch.bfloat16)))
    q1 = torch.empty((300, 1024), dtype=torch.uint8, device="cuda")
    s1 = torch.empty((300, 32), dtype=torch.uint8, device="cuda")
    q2, s2 = torch.empty_like(q1), torch.empty_like(s1)
    mxq.mxq_quantize_mx(x, q1, s1)
    mxq.mxq_quantize_mx_ex(x, 1, FLOOR, q2, s2)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1, s2)


@pytest.fixture(scope="module")
def dispatch_bits():
    return W.bf16_bits(W.dispatch_payload())


@pytest.mark.parametrize("axis", [1, 0], ids=["rows", "cols"])
def test_dispatch_payload_full_size_rceil(dispatch_bits, axis):
    """(65536, 5120) dispatch payload under RCEIL, both axes: every byte."""
    _roundtrip(dispatch_bits, axis, RCEIL, "dispatch (65536, 5120)")


def test_dispatch_payload_full_size_dim0_floor(dispatch_bits):
    _roundtrip(dispatch_bits, 0, FLOOR, "dispatch (65536, 5120)")
