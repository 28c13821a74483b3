"""Parity of mxq_scaled_grouped_mm (HIP, gfx950 scaled-fp8 MFMA) with the CPU
oracle's double-precision grouped product of the same MXFP8 operands.

Operands are drawn on the CPU (workloads.py) and quantized to MXFP8 by the
oracle, so that no input of either side comes from the HIP path.

Accuracy bars (the oracle's value ``ref`` is the exact sum of exact products,
rounded once to double):
  * fp32 output: |y - ref| <= 2^-10 * sum_k |x w| elementwise, and the relative
    Frobenius error of every group <= 1e-3.  The elementwise bound comes from the
    matrix core's arithmetic as measured on gfx950: it sums the 32 products of
    one E8M0 block in a fixed-point window about 14 bits below the block's
    largest product (a 2^-6 product beside a 448 one is dropped, 2^-3 is kept),
    then accumulates blocks in fp32; over full-range random codes the worst
    error seen was 2^-12 of sum |x w|, so the bound leaves a factor 4;
  * bf16 output: the fp32 result above rounded once, so |y - ref| <= 2^-8 |ref|
    plus the fp32 bound; the relative Frobenius error of every group against the
    oracle's correctly rounded bf16 of ref <= 1e-3 (against the unrounded ref the
    output rounding alone is about 1.5e-3 for normally distributed outputs);
  * the bf16 output is bit-identical to the fp32 output rounded to nearest even.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gpu_util as U
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

FRO_BAR = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def mxq():
    from float8_quantization_moe_amd import mxq as m
    return m


def make_operands(M, N, K, G, seed):
    """MXFP8 codes of token rows and expert weights, quantized by the oracle."""
    x = W.bf16_bits(W.moe_tokens(M, K, seed=seed))
    w = W.bf16_bits(W.expert_weights(G, N, K, seed=seed + 1)).reshape(G * N, K)
    xq, xs = U.oracle_mx_quantize(x)
    wq, ws = U.oracle_mx_quantize(w)
    return xq, xs, wq.reshape(G, N, K), ws.reshape(G, N, K // 32)


def run_gpu(xq, xs, wq, ws, ends, out_dtype, guarded=False):
    m = mxq()
    M, K = xq.shape
    G, N, _ = wq.shape
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    offs = d(np.asarray(ends, np.int32))
    wsp = torch.empty(max(m.mxq_grouped_mm_workspace_bytes(M, N, K, G), 16), dtype=torch.uint8, device="cuda")
    if guarded:
        g = U.Guarded(M * N, out_dtype, (M, N))
        y = g.t
    else:
        g = None
        y = torch.empty((M, N), dtype=out_dtype, device="cuda")
    m.mxq_scaled_grouped_mm(d(xq), d(xs), d(wq), d(ws), offs, y, wsp)
    torch.cuda.synchronize()
    if g is not None:
        assert g.guard_intact(), "write past the end of y"
    return y.float().cpu().numpy().astype(np.float64), y


def clamped_ends(ends, M):
    out, run = [], 0
    for e in ends:
        run = min(max(run, int(e)), M)
        out.append(run)
    return out


def abs_operand(q):
    return (q & 0x7F).astype(np.uint8)


def check(y, ref, mag, rows, ends, M, K, bf16, ref_bf16=None, what=""):
    """Elementwise bound and per-group relative Frobenius error over the given rows."""
    acc_bound = 2.0 ** -10 * mag
    err = np.abs(y - ref)
    if bf16:
        bound = 2.0 ** -8 * np.abs(ref) + acc_bound
    else:
        bound = acc_bound
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} outputs off, worst {np.max(err - bound):.3e}"
    ce = clamped_ends(ends, M)
    starts = [0] + ce[:-1]
    rows = np.asarray(rows)
    worst = 0.0
    for g, (a, b) in enumerate(zip(starts, ce)):
        sel = (rows >= a) & (rows < b)
        if not sel.any():
            continue
        target = ref_bf16[sel] if bf16 else ref[sel]
        den = np.linalg.norm(ref[sel])
        num = np.linalg.norm(y[sel] - target)
        rel = num / den if den > 0 else num
        worst = max(worst, rel)
        assert rel <= FRO_BAR, f"{what}: group {g} relative Frobenius error {rel:.3e}"
    tail = rows >= (ce[-1] if ce else 0)
    assert np.all(y[tail] == 0.0), f"{what}: rows past the last end must be zero"
    return worst


def oracle_ref(xq, xs, wq, ws, ends, rows, cols):
    ref = U.oracle_mx_grouped_mm(xq, xs, wq, ws, ends, rows, cols)
    mag = U.oracle_mx_grouped_mm(abs_operand(xq), xs, abs_operand(wq), ws, ends, rows, cols)
    rb = oracle.bf16_round_f64(ref.ravel()).reshape(ref.shape)
    ref_bf16 = (rb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return ref, mag, ref_bf16


CASES = {
    # name: (M, N, K, group sizes or explicit ends, seed)
    "ragged": (700, 264, 384, {"sizes": [300, 0, 257, 1, 100]}, 3),        # 42 tail rows, N tail
    "single_group": (300, 256, 128, {"sizes": [300]}, 5),
    "exact_tiles": (768, 512, 256, {"sizes": [256, 512]}, 7),
    "one_row_groups": (40, 64, 256, {"sizes": [1] * 24}, 9),               # 16 tail rows
    "all_rows_in_no_group": (90, 72, 128, {"ends": [0, 0]}, 11),
    "decreasing_offsets": (600, 136, 256, {"ends": [300, 100, 500, 2000]}, 13),
    "min_n": (64, 8, 128, {"sizes": [10, 54]}, 15),
    # K past one 1024-byte scale chunk: the two-slot scale ring wraps (K > 1024),
    # including scale rows K/32 that are not a multiple of 16 (K = 640, 1152)
    "k640_ragged": (520, 200, 640, {"sizes": [200, 0, 171, 9, 100]}, 17),       # 40 tail rows, N tail
    "k1152_ragged": (390, 136, 1152, {"sizes": [1, 128, 250]}, 19),             # 11 tail rows
    "k1536_two_groups": (300, 264, 1536, {"sizes": [129, 171]}, 21),
    "k2048_ragged": (700, 264, 2048, {"sizes": [300, 0, 257, 1, 100]}, 23),     # 42 tail rows
    "k5120_moe_width": (300, 200, 5120, {"sizes": [150, 0, 140]}, 25),          # the MoE hidden size, 10 tail rows
}


def _ends(spec):
    if "ends" in spec:
        return np.asarray(spec["ends"], np.int32)
    return W.ends_from_sizes(spec["sizes"])


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_full_matrix(name, out_dtype):
    M, N, K, spec, seed = CASES[name]
    ends = _ends(spec)
    G = len(ends)
    print(f"case {name} M={M} N={N} K={K} G={G} {out_dtype}", flush=True)
    xq, xs, wq, ws = make_operands(M, N, K, G, seed)
    y, _ = run_gpu(xq, xs, wq, ws, ends, out_dtype, guarded=True)
    rows = np.arange(M)
    ref, mag, ref_bf16 = oracle_ref(xq, xs, wq, ws, ends, rows, np.arange(N))
    bf16 = out_dtype == torch.bfloat16
    worst = check(y, ref, mag, rows, ends, M, K, bf16, ref_bf16, what=name)
    print(f"  worst group relative Frobenius error {worst:.3e}")


def test_bf16_output_is_rounded_f32_output():
    M, N, K, spec, seed = CASES["ragged"]
    ends = _ends(spec)
    xq, xs, wq, ws = make_operands(M, N, K, len(ends), seed)
    _, y32 = run_gpu(xq, xs, wq, ws, ends, torch.float32)
    _, y16 = run_gpu(xq, xs, wq, ws, ends, torch.bfloat16)
    assert torch.equal(y32.cpu().to(torch.bfloat16).view(torch.int16), y16.cpu().view(torch.int16))


def test_repeated_calls_are_bitwise_identical():
    M, N, K, spec, seed = CASES["exact_tiles"]
    ends = _ends(spec)
    xq, xs, wq, ws = make_operands(M, N, K, len(ends), seed)
    _, a = run_gpu(xq, xs, wq, ws, ends, torch.bfloat16)
    _, b = run_gpu(xq, xs, wq, ws, ends, torch.bfloat16)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def _sample_rows(ends, M, rng, per_group=2):
    ce = clamped_ends(ends, M)
    starts = [0] + ce[:-1]
    rows = set()
    for a, b in zip(starts, ce):
        if b > a:
            rows.update([a, b - 1])
            rows.update(rng.integers(a, b, per_group).tolist())
    if ce[-1] < M:
        rows.update([ce[-1], M - 1])
    return np.array(sorted(rows), np.int64)


@pytest.mark.slow
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_moe_config_sampled(out_dtype):
    """X (16640, 5120) routed to 16 experts (Zipf 1.1), W (16, 8192, 5120) ~ N(0, 0.02^2),
    in the launch configuration the benchmark times; outputs checked at sampled rows
    (each group's first and last row plus random ones) and columns (tile edges plus
    random ones)."""
    M, K = W.TOKENS_SHAPE
    G, N, _ = W.EXPERTS_SHAPE
    print(f"moe config M={M} N={N} K={K} G={G} {out_dtype}", flush=True)
    ends = W.zipf_group_ends(M, G)
    xq, xs = U.oracle_mx_quantize(W.bf16_bits(W.moe_tokens(M, K)))
    wq, ws = U.oracle_mx_quantize(W.bf16_bits(W.expert_weights()).reshape(G * N, K))
    wq = wq.reshape(G, N, K)
    ws = ws.reshape(G, N, K // 32)
    y, _ = run_gpu(xq, xs, wq, ws, ends, out_dtype)
    rng = np.random.default_rng(21)
    rows = _sample_rows(ends, M, rng)
    cols = np.array(sorted(set([0, 1, 255, 256, 4095, 4096, N - 1] + rng.integers(0, N, 40).tolist())), np.int64)
    ref, mag, ref_bf16 = oracle_ref(xq, xs, wq, ws, ends, rows, cols)
    ys = y[np.ix_(rows, cols)]
    bf16 = out_dtype == torch.bfloat16
    worst = check(ys, ref, mag, rows, ends, M, K, bf16, ref_bf16, what="moe config")
    print(f"  worst group relative Frobenius error {worst:.3e} over {rows.size} x {cols.size} samples")
