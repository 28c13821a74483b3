"""Seeded random shapes on the GPU, each compared with the CPU oracle: row and
column tails of every size, group structures with empty and one-row groups,
every flag of the group scaling under both of its methods, random transposes,
dispatch packs and grouped products.  Valid inputs only; the seeds are fixed,
so every run checks the same cases.

Sources as in the per-call test files: "[mxfp8 MoE training] Support mxfp8 all
to all in expert parallel", Summary (the MXFP8 codec and the dispatch payload);
"[moe training] fix uncoalesced global accesses in per group rowwise scaling
kernel", Summary (per-group scaling, both layouts, the transform).
"""
import numpy as np
import pytest
import torch

import gpu_util as U
import oracle
import test_gpu_grouped_mm as GM
import workloads as W
from float8_quantization_moe_amd import mxq

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "these tests need an MI355X"
    mxq.lib()
    yield


def _bits(rng, M, K):
    x = (rng.standard_normal((M, K)) * np.exp(2.0 * rng.standard_normal((M, 1)))).astype(np.float32)
    b = (x.view(np.uint32) >> 16).astype(np.uint16)
    if M and K and rng.random() < 0.3:                    # an occasional non-finite element
        b[rng.integers(0, M), rng.integers(0, K)] = rng.choice([0x7F80, 0xFF80, 0x7FC1])
    return b


def _sizes(rng, M, G):
    """G group sizes summing to M (or less: rows past the last end), with empty
    and one-row groups mixed in."""
    cuts = np.sort(rng.integers(0, M + 1, G - 1)) if G > 1 else np.array([], np.int64)
    sizes = np.diff(np.concatenate([[0], cuts, [M]]))
    if rng.random() < 0.3:
        sizes[rng.integers(0, G)] = 0
    tail = int(rng.integers(0, max(1, M // 10))) if rng.random() < 0.3 else 0
    sizes[-1] = max(0, sizes[-1] - tail)
    return np.cumsum(sizes).astype(np.int32)


@pytest.mark.parametrize("seed", range(8))
def test_mx_codec_random(seed):
    rng = np.random.default_rng(1000 + seed)
    M = int(rng.integers(1, 3000))
    K = 32 * int(rng.integers(1, 200))
    rule = int(rng.integers(0, 2))
    print(f"mx seed={seed} M={M} K={K} rule={rule}", flush=True)
    x_bits = _bits(rng, M, K)
    x = U.dev_bf16(x_bits)
    qg, sg = U.Guarded(M * K, torch.uint8, (M, K)), U.Guarded(M * K // 32, torch.uint8, (M, K // 32))
    mxq.mxq_quantize_mx_ex(x, 1, rule, qg.t, sg.t)
    yg = U.Guarded(M * K, torch.bfloat16, (M, K))
    mxq.mxq_dequantize_mx(qg.t, sg.t, yg.t)
    torch.cuda.synchronize()
    assert qg.guard_intact() and sg.guard_intact() and yg.guard_intact()
    wq, ws = oracle.mx_quantize_ex(x_bits, 1, rule)
    assert np.array_equal(U.host_u8(sg.t), ws) and np.array_equal(U.host_u8(qg.t), wq)
    assert np.array_equal(U.host_u16(yg.t), oracle.mx_dequantize(wq, ws))


@pytest.mark.parametrize("seed", range(6))
def test_mx_dim0_random(seed):
    rng = np.random.default_rng(2000 + seed)
    M = 32 * int(rng.integers(1, 80))
    K = 4 * int(rng.integers(1, 1200))
    rule = int(rng.integers(0, 2))
    print(f"mx dim0 seed={seed} M={M} K={K} rule={rule}", flush=True)
    x_bits = _bits(rng, M, K)
    qg, sg = U.Guarded(M * K, torch.uint8, (M, K)), U.Guarded(M * K // 32, torch.uint8, (M // 32, K))
    mxq.mxq_quantize_mx_ex(U.dev_bf16(x_bits), 0, rule, qg.t, sg.t)
    yg = U.Guarded(M * K, torch.bfloat16, (M, K))
    mxq.mxq_dequantize_mx_ex(qg.t, sg.t, 0, yg.t)
    torch.cuda.synchronize()
    assert qg.guard_intact() and sg.guard_intact() and yg.guard_intact()
    wq, ws = oracle.mx_quantize_ex(x_bits, 0, rule)
    assert np.array_equal(U.host_u8(sg.t), ws) and np.array_equal(U.host_u8(qg.t), wq)
    assert np.array_equal(U.host_u16(yg.t), oracle.mx_dequantize_ex(wq, ws, 0))


@pytest.mark.parametrize("mode", ["hold", "twopass", "split"])
@pytest.mark.parametrize("seed", range(8))
def test_group_scaling_random(seed, mode, group_knobs):
    group_knobs(method=mode)
    rng = np.random.default_rng(3000 + seed)
    M = int(rng.integers(1, 5000))
    K = 8 * int(rng.integers(1, 300))
    G = int(rng.integers(1, 200))
    flags = int(rng.integers(0, 4))
    ends = _sizes(rng, M, G)
    print(f"group seed={seed} mode={mode} M={M} K={K} G={G} flags={flags}", flush=True)
    x_bits = _bits(rng, M, K)
    x = U.dev_bf16(x_bits)
    offs = torch.from_numpy(ends).cuda()
    ws = torch.empty(max(16, mxq.mxq_group_scale_workspace_bytes(M, K, G)), dtype=torch.uint8, device="cuda")
    ws.fill_(0x5A)
    for layout in (mxq.MXQ_LAYOUT_ROW, mxq.MXQ_LAYOUT_COL):
        qg = U.Guarded(M * K, torch.uint8, (M, K) if layout == mxq.MXQ_LAYOUT_ROW else (K, M))
        sg = U.Guarded(G * K, torch.float32, (G, K))
        mxq.mxq_group_scale_fp8_ex(x, offs, layout, flags, qg.t, sg.t, ws)
        torch.cuda.synchronize()
        assert qg.guard_intact() and sg.guard_intact(), "wrote past the end"
        wq, wscale = oracle.group_scale_ex(x_bits, ends, layout, flags)
        got_s, want_s = U.host_f32_bits(sg.t), wscale.view(np.uint32)
        assert np.array_equal(got_s, want_s), f"layout {layout} scales: {U.first_mismatch(got_s, want_s)}"
        got_q = U.host_u8(qg.t)
        assert np.array_equal(got_q, wq), f"layout {layout} codes: {U.first_mismatch(got_q, wq)}"


@pytest.mark.parametrize("seed", range(6))
def test_transpose_random(seed):
    rng = np.random.default_rng(4000 + seed)
    R, C = int(rng.integers(1, 3000)), int(rng.integers(1, 3000))
    a = rng.integers(0, 256, (R, C)).astype(np.uint8)
    og = U.Guarded(R * C, torch.uint8, (C, R))
    mxq.mxq_transpose_u8(torch.from_numpy(a).cuda(), og.t)
    torch.cuda.synchronize()
    assert og.guard_intact() and np.array_equal(U.host_u8(og.t), oracle.transpose_u8(a))


@pytest.mark.parametrize("seed", range(6))
def test_dispatch_pack_random(seed):
    rng = np.random.default_rng(5000 + seed)
    M = int(rng.integers(1, 2500))
    K = 256 * int(rng.integers(1, 12))
    topk = int(rng.integers(1, 9))
    E = int(rng.integers(1, 300))
    ids = rng.integers(-1, E + 1, (M, topk)).astype(np.int32)     # -1 and E are dropped
    print(f"dispatch seed={seed} M={M} K={K} topk={topk} E={E}", flush=True)
    x_bits = _bits(rng, M, K)
    P = M * topk
    pk = U.Guarded(P * (K + K // 32), torch.uint8, (P, K + K // 32))
    pk.t.fill_(0)
    eg = U.Guarded(E, torch.int32, (E,))
    sp = U.Guarded(P, torch.int32, (P,))
    ws = torch.empty(mxq.mxq_dispatch_pack_workspace_bytes(M, K, topk, E), dtype=torch.uint8, device="cuda")
    mxq.mxq_dispatch_pack_mx(U.dev_bf16(x_bits), torch.from_numpy(ids).cuda(), E, pk.t, eg.t, sp.t, ws)
    torch.cuda.synchronize()
    assert pk.guard_intact() and eg.guard_intact() and sp.guard_intact()
    wp, wsrc, we = oracle.dispatch_pack(x_bits, ids, E)
    assert np.array_equal(eg.t.cpu().numpy(), we)
    assert np.array_equal(sp.t.cpu().numpy(), wsrc)
    n = int(we[-1])
    got = U.host_u8(pk.t)
    assert np.array_equal(got[:n], wp[:n]) and not got[n:].any()


@pytest.mark.parametrize("seed", range(4))
def test_grouped_mm_random(seed):
    rng = np.random.default_rng(6000 + seed)
    M = int(rng.integers(1, 800))
    N = 8 * int(rng.integers(1, 41))
    K = 128 * int(rng.integers(1, 5))
    G = int(rng.integers(1, 12))
    ends = _sizes(rng, M, G)
    out = torch.bfloat16 if rng.random() < 0.5 else torch.float32
    print(f"gemm seed={seed} M={M} N={N} K={K} G={G} {out}", flush=True)
    xq, xs, wq, ws = GM.make_operands(M, N, K, G, seed=7000 + seed)
    y, _ = GM.run_gpu(xq, xs, wq, ws, ends, out, guarded=True)
    rows, cols = np.arange(M), np.arange(N)
    ref, mag, ref_bf16 = GM.oracle_ref(xq, xs, wq, ws, ends, rows, cols)
    GM.check(y, ref, mag, rows, ends, M, K, out == torch.bfloat16, ref_bf16, what=f"seed {seed}")
