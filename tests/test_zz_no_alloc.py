"""The allocation-free group scaling entry point (mxq_group_scale_fp8_noalloc),
called through the C ABI, against the workspace entry point
(mxq_group_scale_fp8_ex): bit-identical codes and scales, on two calls in a row
(the second with a smaller input), in both layouts and with the scale flags.
The scratch array keeps the previous call's contents, so the second call checks
that nothing left in it changes a result.

"[moe training] fix uncoalesced global accesses in per group rowwise scaling
kernel", Summary: per-group float8 scaling of the grouped GEMM's left operand.
"""
import numpy as np
import pytest
import torch

import gpu_util as U
import oracle
import workloads as W
from float8_quantization_moe_amd import mxq

pytestmark = pytest.mark.gpu

ROW, COL = mxq.MXQ_LAYOUT_ROW, mxq.MXQ_LAYOUT_COL


def _run(x, ends, layout, flags, noalloc):
    M, K = x.shape
    G = len(ends)
    offs = torch.from_numpy(np.asarray(ends, np.int32)).cuda()
    q = U.Guarded(M * K, torch.uint8, (M, K) if layout == ROW else (K, M))
    s = U.Guarded(G * K, torch.float32, (G, K))
    if noalloc:
        mxq.mxq_group_scale_fp8_noalloc(x, offs, layout, flags, q.t, s.t)
    else:
        ws = torch.empty(mxq.mxq_group_scale_workspace_bytes(M, K, G), dtype=torch.uint8, device="cuda")
        mxq.mxq_group_scale_fp8_ex(x, offs, layout, flags, q.t, s.t, ws)
    torch.cuda.synchronize()
    assert q.guard_intact() and s.guard_intact()
    return U.host_u8(q.t), U.host_f32_bits(s.t)


@pytest.mark.parametrize("layout", [ROW, COL], ids=["row", "col"])
@pytest.mark.parametrize("flags", [0, mxq.MXQ_GROUP_POW2_SCALE | mxq.MXQ_GROUP_INVERSE_SCALE], ids=["plain", "pow2_inv"])
def test_noalloc_matches_workspace_entry_point_twice(layout, flags):
    assert torch.cuda.is_available()
    # first call: (16640, 5120) with 128 Zipf groups (the largest scratch use here)
    x1 = W.moe_tokens(16640, 5120, seed=0).cuda()
    e1 = W.zipf_group_ends(16640, 128, seed=1)
    a = _run(x1, e1, layout, flags, True)
    b = _run(x1, e1, layout, flags, False)
    assert np.array_equal(a[1], b[1]), "scales differ"
    assert np.array_equal(a[0], b[0]), U.first_mismatch(a[0], b[0])
    # second call, smaller: (3000, 1040), uneven groups with an empty one and tail rows
    rng = np.random.default_rng(7)
    xs = (rng.standard_normal((3000, 1040)) * np.exp(rng.standard_normal((3000, 1)))).astype(np.float32)
    xb = (xs.view(np.uint32) >> 16).astype(np.uint16)
    e2 = np.cumsum([1200, 0, 500, 7, 893]).astype(np.int32)      # 2600 of 3000 rows in groups
    x2 = U.dev_bf16(xb)
    a2 = _run(x2, e2, layout, flags, True)
    b2 = _run(x2, e2, layout, flags, False)
    assert np.array_equal(a2[1], b2[1]), "scales differ"
    assert np.array_equal(a2[0], b2[0]), U.first_mismatch(a2[0], b2[0])
    # and the workspace entry point's bytes are the oracle's
    if flags == 0:
        want_q, want_s = oracle.group_scale(xb, e2, oracle.LAYOUT_ROW if layout == ROW else oracle.LAYOUT_COL)
        assert np.array_equal(a2[0], want_q) and np.array_equal(a2[1], want_s.view(np.uint32))


def test_noalloc_rejects_sizes_past_its_scratch():
    """(262144, 8192) with 16 groups needs about 34 MB of scratch: rejected on the
    host before anything is enqueued (so small real buffers are safe to pass)."""
    L = mxq.lib()
    assert L.mxq_group_scale_workspace_bytes(262144, 8192, 16) > (16 << 20)
    buf = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    p = buf.data_ptr()
    st = torch.cuda.current_stream().cuda_stream
    assert L.mxq_group_scale_fp8_noalloc(p, 262144, 8192, p, 16, ROW, 0, p, p, st) == mxq.MXQ_ERR_WORKSPACE
    torch.cuda.synchronize()
