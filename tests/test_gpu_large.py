"""Sizes past 2^31 elements on the GPU: every 32-bit element offset overflows
here, so the kernels' 64-bit indexing is what keeps the bytes right.

"[mxfp8 MoE training] Support mxfp8 all to all in expert parallel", Summary
(the MXFP8 codec) and "[moe training] fix uncoalesced global accesses in per
group rowwise scaling kernel", Summary (per-group scaling, both layouts, the
transform): the same calls at (266240, 8192) bf16, 2.18e9 elements, whose
element offset 2^31 falls on row 262144.  The oracle checks sampled rows of the
MX codec (row blocks are independent) and whole sampled columns of the group
scaling (columns are independent); the transform is checked in full against
the row-major output.  The grouped product writes a (266240, 8192) output, also
past 2^31 elements, checked at sampled rows and columns against the
double-precision oracle with the bounds of test_gpu_grouped_mm.
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

M, K = 266240, 8192                 # M * K = 2,181,038,080 > 2^31
BOUNDARY_ROW = (1 << 31) // K       # 262144
ROW, COL = mxq.MXQ_LAYOUT_ROW, mxq.MXQ_LAYOUT_COL


@pytest.fixture(scope="module")
def x():
    assert torch.cuda.is_available(), "these tests need an MI355X"
    mxq.lib()
    t = W.device_tokens(M, K, seed=21)
    torch.cuda.synchronize()
    yield t
    del t
    torch.cuda.empty_cache()


def _rows():
    rng = np.random.default_rng(5)
    fixed = [0, 1, BOUNDARY_ROW - 1, BOUNDARY_ROW, BOUNDARY_ROW + 1, M - 2, M - 1]
    return np.array(sorted(set(fixed + rng.integers(0, M, 9).tolist())), np.int64)


def _cols():
    rng = np.random.default_rng(6)
    fixed = list(range(0, 8)) + list(range(K - 8, K)) + list(range(4096, 4104))
    return np.array(sorted(set(fixed + rng.integers(0, K, 8).tolist())), np.int64)


def _host_bits(t):
    return U.host_u16(t)


def test_mx_round_trip_past_2_31_elements(x):
    print(f"MX round trip M={M} K={K}", flush=True)
    qg = U.Guarded(M * K, torch.uint8, (M, K))
    sg = U.Guarded(M * K // 32, torch.uint8, (M, K // 32))
    mxq.mxq_quantize_mx(x, qg.t, sg.t)
    yg = U.Guarded(M * K, torch.bfloat16, (M, K))
    mxq.mxq_dequantize_mx(qg.t, sg.t, yg.t)
    torch.cuda.synchronize()
    assert qg.guard_intact() and sg.guard_intact() and yg.guard_intact(), "wrote past the end"
    rows = torch.from_numpy(_rows()).cuda()
    xb = _host_bits(x.index_select(0, rows))
    wq, ws = U.oracle_mx_quantize(xb)
    gq, gs = U.host_u8(qg.t.index_select(0, rows)), U.host_u8(sg.t.index_select(0, rows))
    assert np.array_equal(gs, ws), U.first_mismatch(gs, ws)
    assert np.array_equal(gq, wq), U.first_mismatch(gq, wq)
    wy = U.oracle_mx_dequantize(wq, ws)
    gy = U.host_u16(yg.t.index_select(0, rows))
    assert np.array_equal(gy, wy), U.first_mismatch(gy, wy)


def test_mx_dim0_past_2_31_elements(x):
    """Blocks of 32 rows along dim 0 (RCEIL): whole sampled columns."""
    print(f"MX dim 0 M={M} K={K}", flush=True)
    qg = U.Guarded(M * K, torch.uint8, (M, K))
    sg = U.Guarded(M * K // 32, torch.uint8, (M // 32, K))
    mxq.mxq_quantize_mx_ex(x, 0, mxq.MXQ_SCALE_RCEIL, qg.t, sg.t)
    torch.cuda.synchronize()
    assert qg.guard_intact() and sg.guard_intact(), "wrote past the end"
    cols = torch.from_numpy(_cols()).cuda()
    xb = np.ascontiguousarray(_host_bits(x.index_select(1, cols)))
    wq, ws = oracle.mx_quantize_ex(xb, 0, oracle.RULE_RCEIL)
    gq, gs = U.host_u8(qg.t.index_select(1, cols)), U.host_u8(sg.t.index_select(1, cols))
    assert np.array_equal(gs, ws), U.first_mismatch(gs, ws)
    assert np.array_equal(gq, wq), U.first_mismatch(gq, wq)


@pytest.mark.parametrize("mode", ["hold", "twopass", "split"])
def test_group_scaling_and_transform_past_2_31_elements(x, mode, group_knobs):
    """16 Zipf groups (the largest far beyond what one launch can hold, so the
    hold method streams it through its deferred pass), row-major and
    column-major, and the transform of the column-major codes."""
    group_knobs(method=mode)
    G = 16
    ends = W.zipf_group_ends(M, G)
    print(f"group scaling M={M} K={K} G={G} mode={mode}", flush=True)
    offs = torch.from_numpy(ends).cuda()
    ws = torch.empty(mxq.mxq_group_scale_workspace_bytes(M, K, G), dtype=torch.uint8, device="cuda")
    qr = U.Guarded(M * K, torch.uint8, (M, K))
    sr = U.Guarded(G * K, torch.float32, (G, K))
    mxq.mxq_group_scale_fp8(x, offs, ROW, qr.t, sr.t, ws)
    qc = U.Guarded(M * K, torch.uint8, (K, M))
    sc = U.Guarded(G * K, torch.float32, (G, K))
    mxq.mxq_group_scale_fp8(x, offs, COL, qc.t, sc.t, ws)
    torch.cuda.synchronize()
    assert all(b.guard_intact() for b in (qr, sr, qc, sc)), "wrote past the end"

    cols_np = _cols()
    cols = torch.from_numpy(cols_np).cuda()
    xb = np.ascontiguousarray(_host_bits(x.index_select(1, cols)))
    wq, wscale = oracle.group_scale(xb, ends, oracle.LAYOUT_ROW)
    want_s = wscale.view(np.uint32)
    for name, s in (("row", sr), ("col", sc)):
        got_s = U.host_f32_bits(s.t.index_select(1, cols))
        assert np.array_equal(got_s, want_s), f"{name} scales: {U.first_mismatch(got_s, want_s)}"
    got_r = U.host_u8(qr.t.index_select(1, cols))
    assert np.array_equal(got_r, wq), f"row codes: {U.first_mismatch(got_r, wq)}"
    got_c = U.host_u8(qc.t.index_select(0, cols)).T
    assert np.array_equal(got_c, wq), f"col codes: {U.first_mismatch(got_c, wq)}"

    # the transform of the column-major codes is the row-major output, every byte
    del sr, sc
    tg = U.Guarded(M * K, torch.uint8, (M, K))
    mxq.mxq_transpose_u8(qc.t, tg.t)
    torch.cuda.synchronize()
    assert tg.guard_intact()
    assert torch.equal(tg.t, qr.t), "transform of the column-major codes differs from the row-major codes"


def test_grouped_mm_output_past_2_31_elements():
    """Tokens (266240, 256) in 16 Zipf groups times 16 experts' (8192, 256)
    weights: the bf16 output's element offset 2^31 falls on row 262144."""
    Mx, N, Kx, G = M, 8192, 256, 16
    assert torch.cuda.is_available(), "these tests need an MI355X"
    print(f"grouped mm M={Mx} N={N} K={Kx} G={G}", flush=True)
    ends = W.zipf_group_ends(Mx, G)
    xq, xs = U.oracle_mx_quantize(W.bf16_bits(W.moe_tokens(Mx, Kx, seed=22)))
    wq, ws = U.oracle_mx_quantize(W.bf16_bits(W.expert_weights(G, N, Kx, seed=23)).reshape(G * N, Kx))
    wq, ws = wq.reshape(G, N, Kx), ws.reshape(G, N, Kx // 32)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    wsp = torch.empty(mxq.mxq_grouped_mm_workspace_bytes(Mx, N, Kx, G), dtype=torch.uint8, device="cuda")
    yg = U.Guarded(Mx * N, torch.bfloat16, (Mx, N))
    mxq.mxq_scaled_grouped_mm(d(xq), d(xs), d(wq), d(ws), d(ends), yg.t, wsp)
    torch.cuda.synchronize()
    assert yg.guard_intact(), "wrote past the end of y"
    rng = np.random.default_rng(24)
    boundary = (1 << 31) // N
    rows = np.array(sorted(set(GM._sample_rows(ends, Mx, rng).tolist() + [boundary - 1, boundary, Mx - 1])), np.int64)
    cols = np.array(sorted(set([0, 1, 255, 256, 4095, 4096, N - 1] + rng.integers(0, N, 24).tolist())), np.int64)
    ys = yg.t.index_select(0, torch.from_numpy(rows).cuda()).index_select(1, torch.from_numpy(cols).cuda())
    ys = ys.float().cpu().numpy().astype(np.float64)
    ref, mag, ref_bf16 = GM.oracle_ref(xq, xs, wq, ws, ends, rows, cols)
    worst = GM.check(ys, ref, mag, rows, ends, Mx, Kx, True, ref_bf16, what="output past 2^31 elements")
    print(f"  worst group relative Frobenius error {worst:.3e} over {rows.size} x {cols.size} samples")
