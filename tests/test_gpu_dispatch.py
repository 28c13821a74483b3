"""Fused dispatch pack and the grouped GEMM on the packed payload, on the GPU,
against the CPU oracle.

"[mxfp8 MoE training] Support mxfp8 all to all in expert parallel", Summary:
the routed tokens travel as mxfp8 (e4m3 data + e8m0 scales).  The dispatch pack
sorts the token-expert pairs by expert and writes each row as [codes | scales];
its bytes, the source index of every row and the experts' end offsets are
compared exactly.  The grouped GEMM reading that buffer directly is compared
with the double-precision oracle product (the bounds of test_gpu_grouped_mm)
and bit for bit with the GEMM on the same operands unpacked.
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


def zipf_ids(M, E, seed, topk=1):
    return W.routed_expert_ids(M, E, topk=topk, seed=seed)


def run_pack(x_bits, ids, E):
    M, K = x_bits.shape
    topk = ids.shape[1]
    P = M * topk
    x = U.dev_bf16(x_bits)
    pk = U.Guarded(P * (K + K // 32), torch.uint8, (P, K + K // 32))
    pk.t.fill_(0)
    eg = U.Guarded(E, torch.int32, (E,))
    sg = U.Guarded(max(P, 1), torch.int32, (max(P, 1),))
    ws = torch.empty(mxq.mxq_dispatch_pack_workspace_bytes(M, K, topk, E), dtype=torch.uint8, device="cuda")
    ws.fill_(0xCD)
    mxq.mxq_dispatch_pack_mx(x, torch.from_numpy(ids).cuda(), E, pk.t, eg.t, sg.t[:P] if P else sg.t[:0], ws)
    torch.cuda.synchronize()
    assert pk.guard_intact() and eg.guard_intact() and sg.guard_intact(), "wrote past the end"
    return pk.t.cpu().numpy(), eg.t.cpu().numpy(), sg.t[:P].cpu().numpy()


def check_pack(x_bits, ids, E, name):
    M, K = x_bits.shape
    print(f"case {name} M={M} K={K} topk={ids.shape[1]} E={E}", flush=True)
    gp, ge, gs = run_pack(x_bits, ids, E)
    wp, ws_, we = oracle.dispatch_pack(x_bits, ids, E)
    assert np.array_equal(ge, we), f"{name} ends: {U.first_mismatch(ge, we)}"
    assert np.array_equal(gs, ws_), f"{name} src_pair: {U.first_mismatch(gs, ws_)}"
    n = int(we[-1])
    assert np.array_equal(gp[:n], wp[:n]), f"{name} rows: {U.first_mismatch(gp[:n], wp[:n])}"
    assert not gp[n:].any(), f"{name}: rows past the last end were written"
    return gp, ge


CASES = {
    # name: (M, K, topk, E, dropped fraction)
    "tiny_one_expert": (40, 256, 1, 1, 0.0),
    "ragged_blocks": (1000, 512, 1, 7, 0.0),            # 1000 pairs: a partial 256-pair block
    "top2_with_drops": (777, 768, 2, 16, 0.1),           # ids -1 and E dropped
    "many_experts": (3000, 256, 1, 1024, 0.0),           # the largest E: one column per thread in the scan
    "top8_small": (64, 1024, 8, 128, 0.05),
    "empty_experts": (500, 256, 1, 64, 0.0),             # most experts receive nothing
}


@pytest.mark.parametrize("case", list(CASES), ids=list(CASES))
def test_dispatch_pack_cases(case):
    M, K, topk, E, drop = CASES[case]
    rng = np.random.default_rng(M + K + E)
    x_bits = W.bf16_bits(W.lognormal_rows(M, K, seed=M + topk).to(torch.bfloat16))
    if case == "empty_experts":
        ids = rng.choice([3, 17, 60], size=(M, topk)).astype(np.int32)
    else:
        ids = zipf_ids(M, E, seed=M, topk=topk)
    if drop:
        sel = rng.random(ids.shape) < drop
        ids[sel] = np.where(rng.random(sel.sum()) < 0.5, -1, E)
    check_pack(x_bits, ids, E, case)


def test_dispatch_pack_no_tokens():
    E = 5
    eg = torch.full((E,), 77, dtype=torch.int32, device="cuda")
    ws = torch.empty(mxq.mxq_dispatch_pack_workspace_bytes(0, 512, 1, E), dtype=torch.uint8, device="cuda")
    x = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((0, 1), dtype=torch.int32, device="cuda")
    pk = torch.empty((0, 528), dtype=torch.uint8, device="cuda")
    sp = torch.empty((0,), dtype=torch.int32, device="cuda")
    mxq.mxq_dispatch_pack_mx(x, ids, E, pk, eg, sp, ws)
    torch.cuda.synchronize()
    assert eg.cpu().tolist() == [0] * E


def test_dispatch_pack_full_size():
    """The (65536, 5120) dispatch payload routed top-1 over 16 Zipf experts."""
    M, K = W.DISPATCH_SHAPE
    x_bits = W.bf16_bits(W.dispatch_payload(M, K, seed=0))
    ids = zipf_ids(M, 16, seed=1)
    gp, ge = check_pack(x_bits, ids, 16, "dispatch (65536, 5120)")
    assert np.array_equal(ge, W.zipf_group_ends(M, 16, seed=1))


def test_dispatch_pack_is_deterministic():
    M, K, E = 2048, 512, 8
    x_bits = W.bf16_bits(W.lognormal_rows(M, K, seed=3).to(torch.bfloat16))
    ids = zipf_ids(M, E, seed=4, topk=2)
    a = run_pack(x_bits, ids, E)
    b = run_pack(x_bits, ids, E)
    assert all(np.array_equal(u, v) for u, v in zip(a, b))


def _packed_from_oracle(M, K, G, seed):
    """Tokens routed top-1 to G experts, packed by the oracle; weights quantized by the oracle."""
    x_bits = W.bf16_bits(W.moe_tokens(M, K, seed=seed))
    ids = zipf_ids(M, G, seed=seed + 1)
    packed, _, ends = oracle.dispatch_pack(x_bits, ids, G)
    return packed, ends


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_grouped_mm_on_packed_payload(out_dtype):
    """Y_g = X_g W_g^T straight from the packed rows: within the oracle bounds, and
    bit-identical to mxq_scaled_grouped_mm on the unpacked codes and scales."""
    M, N, K, G = 900, 264, 1024, 5
    packed, ends = _packed_from_oracle(M, K, G, seed=9)
    w = W.bf16_bits(W.expert_weights(G, N, K, seed=10)).reshape(G * N, K)
    wq, wsc = U.oracle_mx_quantize(w)
    wq, wsc = wq.reshape(G, N, K), wsc.reshape(G, N, K // 32)
    xq, xs = np.ascontiguousarray(packed[:, :K]), np.ascontiguousarray(packed[:, K:])
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    offs = d(ends)
    wsp = torch.empty(mxq.mxq_grouped_mm_workspace_bytes(M, N, K, G), dtype=torch.uint8, device="cuda")
    yg = U.Guarded(M * N, out_dtype, (M, N))
    mxq.mxq_scaled_grouped_mm_packed(d(packed), d(wq), d(wsc), offs, yg.t, wsp)
    y2 = torch.empty((M, N), dtype=out_dtype, device="cuda")
    mxq.mxq_scaled_grouped_mm(d(xq), d(xs), d(wq), d(wsc), offs, y2, wsp)
    torch.cuda.synchronize()
    assert yg.guard_intact()
    bits = torch.int32 if out_dtype == torch.float32 else torch.int16
    assert torch.equal(yg.t.view(bits), y2.view(bits)), "packed and unpacked products differ"
    y = yg.t.float().cpu().numpy().astype(np.float64)
    rows, cols = np.arange(M), np.arange(N)
    ref, mag, ref_bf16 = GM.oracle_ref(xq, xs, wq, wsc, ends, rows, cols)
    GM.check(y, ref, mag, rows, ends, M, K, out_dtype == torch.bfloat16, ref_bf16, what="packed")


def test_dispatch_then_grouped_mm_end_to_end():
    """GPU dispatch pack, then the GPU product on its output, against the oracle's
    product of the oracle's pack of the same tokens (sampled rows)."""
    M, N, K, G = 4096, 512, 2048, 8
    x_bits = W.bf16_bits(W.moe_tokens(M, K, seed=12))
    ids = zipf_ids(M, G, seed=13)
    gp, ge, gs = run_pack(x_bits, ids, G)
    wp, wsrc, we = oracle.dispatch_pack(x_bits, ids, G)
    assert np.array_equal(ge, we) and np.array_equal(gs, wsrc)
    w = W.bf16_bits(W.expert_weights(G, N, K, seed=14)).reshape(G * N, K)
    wq, wsc = U.oracle_mx_quantize(w)
    wq, wsc = wq.reshape(G, N, K), wsc.reshape(G, N, K // 32)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    wsp = torch.empty(mxq.mxq_grouped_mm_workspace_bytes(M, N, K, G), dtype=torch.uint8, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mxq.mxq_scaled_grouped_mm_packed(d(gp), d(wq), d(wsc), d(ge), y, wsp)
    torch.cuda.synchronize()
    rng = np.random.default_rng(15)
    rows = GM._sample_rows(we, M, rng)
    cols = np.array(sorted(set([0, N - 1] + rng.integers(0, N, 30).tolist())), np.int64)
    xq, xs = np.ascontiguousarray(wp[:, :K]), np.ascontiguousarray(wp[:, K:])
    ref, mag, ref_bf16 = GM.oracle_ref(xq, xs, wq, wsc, we, rows, cols)
    ys = y.float().cpu().numpy().astype(np.float64)[np.ix_(rows, cols)]
    GM.check(ys, ref, mag, rows, we, M, K, True, ref_bf16, what="dispatch + product")
