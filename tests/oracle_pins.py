"""Pins for the CPU oracle: checks against what the definitions and independent
libraries fix, never against the oracle's own formulas.

Every check takes an ``oracle.Oracle`` instance so that the same battery can be
run against deliberately broken copies of the oracle (see
test_oracle_mutations.py): a plausible mistake anywhere in the oracle must make
at least one of these fail.

Kinds of pin used here:
  * library routines: torch's CPU float8_e4m3fn / float8_e8m0fnu decoders, its
    float32 -> bfloat16 cast, its float32 -> float8_e4m3fn cast (made saturating
    by clamping first), numpy's binary32 division and multiplication;
  * brute force: the nearest-even E4M3 value found by comparing against every
    grid midpoint (exact in binary64), over all bf16 patterns x all scale codes;
  * closed facts of the formats (code counts, extreme codes);
  * hand-worked fixtures in tests/golden/;
  * torch float64 matmuls of operands dequantized by torch's decoders (the
    grouped product), and closed forms of constant operands;
  * invariants: exact dequantization for scale codes >= 3, idempotence,
    the per-block maximum landing in [256, 448], slicing and permutation
    invariance of group scaling, the two layouts being transposes.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch

import _golden

ALL_BF16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _f32_of_bf16(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def e4m3_grid():
    """Non-negative finite E4M3 values in code order 0x00..0x7E (from torch's decoder)."""
    codes = torch.arange(0, 0x7F, dtype=torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def nearest_even_e4m3_codes(y: np.ndarray) -> np.ndarray:
    """Brute-force E4M3 encoding of exact binary64 values y (finite):
    nearest grid value, ties to the even code, saturating at 448, sign kept.
    Comparisons against the grid midpoints are exact in binary64."""
    grid = e4m3_grid()                       # 127 increasing magnitudes
    mids = (grid[:-1] + grid[1:]) / 2.0      # exact: 5 significant bits at most
    a = np.abs(y)
    # index of the first midpoint >= a: a is nearest to grid[i] if mids[i-1] < a < mids[i]
    i = np.searchsorted(mids, a, side="left")
    i = np.minimum(i, len(grid) - 1)
    tie = (i < len(mids)) & (mids[np.minimum(i, len(mids) - 1)] == a)
    # on a tie between grid[i] and grid[i+1] keep the even code
    code = np.where(tie & (i % 2 == 1), i + 1, i)
    code = np.minimum(code, 0x7E)            # saturation
    sign = np.signbit(y).astype(np.uint8) << 7
    return code.astype(np.uint8) | sign


# --------------------------------------------------------------- formats ---
def check_e4m3_decode_vs_torch(o):
    codes = np.arange(256, dtype=np.uint8)
    mine = np.array([o.e4m3_decode(int(c)) for c in codes])
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(mine) & np.isnan(ref)
    assert np.all(both_nan | (mine == ref)), "E4M3 decode differs from torch"
    assert np.array_equal(np.signbit(mine[~np.isnan(mine)]), np.signbit(ref[~np.isnan(ref)]))


def check_e4m3_code_facts(o):
    vals = np.array([o.e4m3_decode(c) for c in range(256)])
    nan = np.isnan(vals)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    fin = vals[~nan]
    assert fin.size == 254 and np.unique(fin).size == 253       # +0 and -0 compare equal
    assert vals[0x7E] == 448.0 and np.nanmax(vals) == 448.0 and np.nanmin(vals) == -448.0
    assert vals[0x08] == 2.0 ** -6 and vals[0x01] == 2.0 ** -9
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0), "codes 0x00..0x7E must increase"
    assert np.array_equal(vals[0x80:0xFF], -vals[0x00:0x7F])


def check_e4m3_encode_roundtrip(o):
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        assert o.e4m3_encode(o.e4m3_decode(c)) == c, hex(c)


def check_e8m0_decode_vs_torch(o):
    codes = np.arange(256, dtype=np.uint8)
    mine = np.array([o.e8m0_decode(int(c)) for c in codes])
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(mine[255]) and np.isnan(ref[255])
    assert np.array_equal(mine[:255], ref[:255])


def check_bf16_round_vs_torch(o, n_random=200_000, seed=5):
    # every bf16 pattern with several low halves (ties, sticky bits), plus random binary32
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    hi = ALL_BF16.astype(np.uint32) << 16
    w = (hi[None, :] | lows[:, None]).ravel()
    rng = np.random.default_rng(seed)
    w = np.concatenate([w, rng.integers(0, 1 << 32, n_random, dtype=np.uint64).astype(np.uint32)])
    f = w.view(np.float32)
    f = f[~np.isnan(f)]
    mine = o.bf16_round_f64(f.astype(np.float64))
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref), "bf16 rounding differs from torch's float32 -> bfloat16 cast"


def check_e4m3_encode_vs_torch_saturating(o, n_random=300_000, seed=6):
    rng = np.random.default_rng(seed)
    # binary32 values spanning the whole E4M3 range and beyond, with full 24-bit mantissas
    e = rng.integers(-30, 12, n_random)
    m = rng.random(n_random) + 1.0
    y = (m * np.exp2(e) * np.where(rng.random(n_random) < 0.5, -1, 1)).astype(np.float32)
    extra = np.array([0.0, -0.0, 448.0, 464.0, 480.0, 1e30, -1e30, 2.0 ** -10, 3 * 2.0 ** -10,
                      2.0 ** -9 * 1.5, 447.99, 448.01, 463.99, 464.01], np.float32)
    y = np.concatenate([y, extra, _f32_of_bf16(ALL_BF16)])
    y = y[np.isfinite(y)]
    mine = o.e4m3_encode_f32(y)
    ref = torch.from_numpy(y.copy()).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref), "E4M3 encoding differs from torch's clamped cast"


def check_mx_encode_exhaustive(o, codes=None):
    """All 65,536 bf16 patterns x every finite scale code (or a given subset),
    against the midpoint brute force."""
    xs = ALL_BF16[(ALL_BF16 & 0x7F80) != 0x7F80]          # finite patterns
    xv = _f32_of_bf16(xs).astype(np.float64)
    codes = range(255) if codes is None else codes
    for c in codes:
        y = xv / np.ldexp(1.0, int(c) - 127)               # exact
        ref = nearest_even_e4m3_codes(y)
        mine = o.mx_encode_elements(xs, np.full(xs.shape, c, np.uint8))
        if not np.array_equal(mine, ref):
            bad = np.nonzero(mine != ref)[0][0]
            raise AssertionError(f"scale code {c}: x=0x{int(xs[bad]):04x} oracle 0x{int(mine[bad]):02x} "
                                 f"brute force 0x{int(ref[bad]):02x}")


def check_mx_encode_fraction_sample(o, n=400, seed=7):
    """Exact-rational nearest-even search over the whole grid on a small sample."""
    grid = [Fraction(v) for v in e4m3_grid()]
    rng = np.random.default_rng(seed)
    xs = rng.integers(0, 1 << 16, n).astype(np.uint16)
    xs = xs[(xs & 0x7F80) != 0x7F80]
    cs = rng.integers(0, 255, xs.size).astype(np.uint8)
    mine = o.mx_encode_elements(xs, cs)
    for x, c, got in zip(xs, cs, mine):
        v = Fraction(float(_f32_of_bf16(np.array([x]))[0])) / Fraction(2) ** (int(c) - 127)
        a = abs(v)
        best = min(range(len(grid)), key=lambda i: (abs(grid[i] - a), i % 2))
        if a > 448:
            best = 0x7E
        want = best | (0x80 if (x & 0x8000) else 0)
        assert got == want, (hex(int(x)), int(c), hex(int(got)), hex(want))


# ------------------------------------------------------------ MX blocks ---
def check_mx_worked_blocks(o):
    blocks, decodes = _golden.load_mx_cases()
    for b in blocks:
        x = np.array([b["x"]], dtype=np.uint16)
        q, s = o.mx_quantize(x)
        assert s[0, 0] == b["s"], (b["name"], hex(int(s[0, 0])), hex(b["s"]))
        assert list(q[0]) == b["q"], (b["name"], [hex(int(v)) for v in q[0]])
        y = o.mx_dequantize(q, s)
        assert list(y[0]) == b["y"], (b["name"], [hex(int(v)) for v in y[0]])
    for d in decodes:
        got = o.mx_decode_element(d["q"], d["s"])
        assert got == d["y"], (d["name"], hex(got), hex(d["y"]))


def _random_blocks(rng, nblocks):
    """Blocks of 32 finite bf16 with mixed magnitudes, zeros and sign patterns."""
    base = rng.standard_normal((nblocks, 32)) * np.exp2(rng.integers(-130, 127, (nblocks, 1)))
    base *= np.where(rng.random((nblocks, 32)) < 0.1, 0.0, 1.0)
    f = base.astype(np.float32)
    f[~np.isfinite(f)] = 0.0
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)    # truncate to bf16 (any bf16 will do)
    bits[(bits & 0x7F80) == 0x7F80] = 0
    return bits


def check_mx_invariants(o, nblocks=20000, seed=8):
    rng = np.random.default_rng(seed)
    x = _random_blocks(rng, nblocks)
    q, s = o.mx_quantize(x)
    y = o.mx_dequantize(q, s)
    codes = s[:, 0]
    dec = torch.from_numpy(q.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    # (1) exactness: for scale code >= 3 the bf16 output equals e4m3(q) * 2^(s-127)
    sel = codes >= 3
    exact = dec[sel] * np.exp2(codes[sel].astype(np.float64) - 127)[:, None]
    yv = _f32_of_bf16(y[sel]).astype(np.float64)
    assert np.array_equal(yv, exact)
    assert np.array_equal(np.signbit(yv), np.signbit(exact))
    # (2) the block maximum lands in [256, 448] whenever the block's amax is a normal bf16
    amax_bits = (x & 0x7FFF).max(axis=1)
    normal = (amax_bits >= 0x0080) & (codes > 0)
    bmax = np.abs(dec[normal]).max(axis=1)
    assert np.all((bmax >= 256) & (bmax <= 448))
    # (3) scale code = floor(log2 amax) - 8 + 127 for normal amax (from numpy's frexp)
    amax = np.abs(_f32_of_bf16(x).astype(np.float64)).max(axis=1)
    _, e = np.frexp(amax[normal])
    want = np.clip(e - 1 - 8 + 127, 0, 254)
    assert np.array_equal(codes[normal].astype(np.int64), want)
    # (4) idempotence on blocks whose code is >= 3 or that are all zero
    keep = (codes >= 3) | (amax == 0)
    q2, s2 = o.mx_quantize(y[keep])
    assert np.array_equal(q2, q[keep]) and np.array_equal(s2, s[keep])
    # (5) the sign of every code follows the sign of its input
    assert np.array_equal(q >> 7, (x >> 15).astype(np.uint8))


def check_mx_row_block_layout(o, seed=9):
    """A (M, K) call equals the same rows and blocks quantized one block at a time
    (catches block/row index mix-ups)."""
    rng = np.random.default_rng(seed)
    M, K = 5, 96
    x = _random_blocks(rng, M * K // 32).reshape(M, K)
    q, s = o.mx_quantize(x)
    for m in range(M):
        for b in range(K // 32):
            qb, sb = o.mx_quantize(np.ascontiguousarray(x[m:m + 1, 32 * b:32 * b + 32]))
            assert sb[0, 0] == s[m, b] and np.array_equal(qb[0], q[m, 32 * b:32 * b + 32])
    y = o.mx_dequantize(q, s)
    for m in range(M):
        for b in range(K // 32):
            yb = o.mx_dequantize(q[m:m + 1, 32 * b:32 * b + 32], s[m:m + 1, b:b + 1])
            assert np.array_equal(yb[0], y[m, 32 * b:32 * b + 32])


# ---------------------------------------------------------- MX variants ---
RULE_RCEIL = 1


def check_mx_rceil_worked_blocks(o):
    """Hand-worked RCEIL blocks (tests/golden/mx_rceil_blocks.txt), as rows and as columns."""
    blocks, _ = _golden.load_mx_cases("mx_rceil_blocks.txt")
    for b in blocks:
        x = np.array([b["x"]], dtype=np.uint16)
        q, s = o.mx_quantize_ex(x, axis=1, rule=RULE_RCEIL)
        assert s[0, 0] == b["s"], (b["name"], hex(int(s[0, 0])), hex(b["s"]))
        assert list(q[0]) == b["q"], (b["name"], [hex(int(v)) for v in q[0]])
        assert list(o.mx_dequantize_ex(q, s, axis=1)[0]) == b["y"], b["name"]
        q0, s0 = o.mx_quantize_ex(np.ascontiguousarray(x.T), axis=0, rule=RULE_RCEIL)
        assert s0.shape == (1, 1) and s0[0, 0] == b["s"] and list(q0[:, 0]) == b["q"], b["name"]
        assert list(o.mx_dequantize_ex(q0, s0, axis=0)[:, 0]) == b["y"], b["name"]


def check_mx_rceil_vs_division(o, nblocks=20000, seed=15):
    """RCEIL code = ceil(log2(amax / 448)) + 127 with the quotient from numpy's binary64
    division and the ceiling read off frexp (a quotient of bf16 amax by 448 is either an
    exact power of two or at least 2^-9 away from one in relative terms); the codes are
    the element-wise MX encoder's under that scale; nothing saturates."""
    rng = np.random.default_rng(seed)
    x = _random_blocks(rng, nblocks)
    q, s = o.mx_quantize_ex(x, axis=1, rule=RULE_RCEIL)
    codes = s[:, 0].astype(np.int64)
    amax = np.abs(_f32_of_bf16(x).astype(np.float64)).max(axis=1)
    nz = amax > 0
    f, e = np.frexp(amax[nz] / 448.0)
    ceil_log2 = np.where(f == 0.5, e - 1, e)
    want = np.zeros(amax.shape, np.int64)
    want[nz] = np.clip(ceil_log2 + 127, 0, 254)
    assert np.array_equal(codes, want)
    assert np.array_equal(q.ravel(), o.mx_encode_elements(x.ravel(), np.repeat(s[:, 0], 32)))
    dec = np.abs(torch.from_numpy(q.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy())
    assert dec.max() <= 448.0
    # for blocks whose code is not clamped, the scaled maximum lies in (224, 448] and encodes in [224, 448]
    free = nz & (want > 0)
    bmax = dec[free].max(axis=1)
    assert np.all((bmax >= 224) & (bmax <= 448))
    # against the floor rule: the same code, or one more exactly when amax's bf16 mantissa
    # exceeds 0x60 (1.75) -- read off the bit patterns, for blocks neither rule clamps
    _, sf = o.mx_quantize(x)
    amax_bits = (x & 0x7FFF).max(axis=1).astype(np.int64)
    unclamped = (sf[:, 0] > 0) & (amax_bits < 0x7F80)
    inc = ((amax_bits & 0x7F) > 0x60).astype(np.int64)
    assert np.array_equal(codes[unclamped], sf[unclamped, 0].astype(np.int64) + inc[unclamped])


def check_mx_axis0_is_transpose(o, seed=16):
    """Blocks along dim 0 are the row blocks of the transpose, for both rules; the
    floor rule along dim 1 is the MX quantizer pinned above; one 32 x 1 block at a
    time gives the same bytes as the whole call."""
    rng = np.random.default_rng(seed)
    M, K = 64, 96
    x = _random_blocks(rng, M * K // 32).reshape(M, K)
    for rule in (0, RULE_RCEIL):
        q0, s0 = o.mx_quantize_ex(x, axis=0, rule=rule)
        q1, s1 = o.mx_quantize_ex(np.ascontiguousarray(x.T), axis=1, rule=rule)
        assert s0.shape == (M // 32, K)
        assert np.array_equal(q0, q1.T) and np.array_equal(s0, s1.T)
        y0 = o.mx_dequantize_ex(q0, s0, axis=0)
        y1 = o.mx_dequantize_ex(q1, s1, axis=1)
        assert np.array_equal(y0, y1.T)
    qf, sf = o.mx_quantize_ex(x, axis=1, rule=0)
    qr, sr = o.mx_quantize(x)
    assert np.array_equal(qf, qr) and np.array_equal(sf, sr)
    assert np.array_equal(o.mx_dequantize_ex(qr, sr, axis=1), o.mx_dequantize(qr, sr))
    q0, s0 = o.mx_quantize_ex(x, axis=0, rule=RULE_RCEIL)
    for a in (0, 1):
        for k in (0, 5, K - 1):
            qb, sb = o.mx_quantize_ex(np.ascontiguousarray(x[32 * a:32 * a + 32, k:k + 1]), axis=0, rule=RULE_RCEIL)
            assert sb[0, 0] == s0[a, k] and np.array_equal(qb[:, 0], q0[32 * a:32 * a + 32, k])


# -------------------------------------------------------- group scaling ---
def check_group_worked(o):
    for c in _golden.load_group_cases():
        x = np.array(c["x"], dtype=np.uint16)
        for layout in (0, 1):
            q, scales = o.group_scale(x, c["ends"], layout)
            got_s = scales.view(np.uint32)
            assert np.array_equal(got_s, np.array(c["scales"], np.uint32)), (c["name"], got_s)
            qr = q if layout == 0 else q.T
            assert np.array_equal(qr, np.array(c["q"], np.uint8)), (c["name"], layout, qr)


def group_reference_by_libraries(x_bits, ends):
    """Row-layout group scaling rebuilt from numpy / torch primitives:
    numpy max of |x|, numpy binary32 division and product, torch's E4M3 cast."""
    M, K = x_bits.shape
    xf = _f32_of_bf16(x_bits)
    q = np.zeros((M, K), np.uint8)
    scales = np.empty((len(ends), K), np.float32)
    start = 0
    for g, e in enumerate(ends):
        end = min(max(int(e), start), M)
        seg = xf[start:end]
        amax = np.abs(seg).max(axis=0) if end > start else np.zeros(K, np.float32)
        s = np.float32(448.0) / np.maximum(amax, np.float32(1e-12))
        bad = ~np.isfinite(amax)
        s[bad] = np.float32("nan")
        scales[g] = s
        p = (seg * s[None, :]).astype(np.float32)
        qq = torch.from_numpy(np.nan_to_num(p, nan=0.0)).clamp(-448, 448).to(torch.float8_e4m3fn)
        qq = qq.view(torch.uint8).numpy().copy()
        qq[:, bad] = 0x7F
        q[start:end] = qq
        start = end
    return q, scales


def _token_matrix(rng, M, K):
    f = (rng.standard_normal((M, K)) * np.exp(rng.standard_normal((M, 1)))).astype(np.float32)
    f *= (rng.random((M, K)) > 0.02)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def check_group_vs_libraries(o, seed=10):
    rng = np.random.default_rng(seed)
    for (M, K, sizes) in [(257, 40, [100, 0, 57, 1, 99]), (64, 16, [64]), (50, 8, [0, 0, 50]),
                          (90, 24, [10, 20, 30, 29])]:   # last: one row in no group
        x = _token_matrix(rng, M, K)
        ends = np.cumsum(sizes).astype(np.int32)
        q, scales = o.group_scale(x, ends, 0)
        qr, sr = group_reference_by_libraries(x, ends)
        assert np.array_equal(scales.view(np.uint32), sr.view(np.uint32)), (M, K, sizes)
        assert np.array_equal(q, qr), (M, K, sizes)


GROUP_POW2, GROUP_INVERSE = 1, 2


def _row_multipliers(scales, ends, M):
    """Per-element multiplier of every row (its group's row of `scales`), NaN for rows in no group."""
    K = scales.shape[1]
    out = np.full((M, K), np.nan, np.float32)
    start = 0
    for g, e in enumerate(ends):
        end = min(max(int(e), start), M)
        out[start:end] = scales[g]
        start = end
    return out


def check_group_variants(o, seed=17):
    """Power-of-two and inverse scales against what fixes them: the plain variant is
    the group scaling pinned above; power-of-two multipliers have a zero significand
    and lie in (s/2, s]; their codes are the element encoder's (pinned exhaustively)
    under that multiplier; the column maximum still encodes in [224, 448]; inverse
    scales are numpy's binary32 1/s and leave the codes unchanged; COL is ROW
    transposed."""
    rng = np.random.default_rng(seed)
    M, K = 257, 40
    x = _token_matrix(rng, M, K)
    x[:, 3] = 0                                     # an all-zero column
    x[7, 5] = 0x7FC0                                # a NaN column in group 0
    sizes = [100, 0, 57, 1, 99]
    ends = np.cumsum(sizes).astype(np.int32)
    q0, s0 = o.group_scale_ex(x, ends, 0, 0)
    qp, sp = o.group_scale(x, ends, 0)
    assert np.array_equal(q0, qp) and np.array_equal(s0.view(np.uint32), sp.view(np.uint32))
    q1, s1 = o.group_scale_ex(x, ends, 0, GROUP_POW2)
    nan0 = np.isnan(s0)
    assert np.array_equal(np.isnan(s1), nan0)
    fin = ~nan0
    m, _ = np.frexp(s1[fin])
    assert np.all(m == 0.5), "power-of-two multipliers"
    assert np.all((s1[fin].astype(np.float64) <= s0[fin]) & (2.0 * s1[fin].astype(np.float64) > s0[fin]))
    mult = _row_multipliers(s1, ends, M)
    in_group = ~np.isnan(mult[:, 0])
    col_nan = np.isnan(mult)
    ok = in_group[:, None] & ~col_nan
    enc = o.group_encode_elements(x[ok], mult[ok])
    assert np.array_equal(q1[ok], enc)
    assert np.all(q1[in_group[:, None] & col_nan] == 0x7F) and np.all(q1[~in_group] == 0)
    dec = np.abs(torch.from_numpy(q1.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy())
    start = 0
    for g, e in enumerate(ends):
        end = min(max(int(e), start), M)
        if end > start:
            for k in range(K):
                if fin[g, k] and np.any(x[start:end, k] & 0x7FFF):
                    assert 224.0 <= dec[start:end, k].max() <= 448.0, (g, k)
        start = end
    q2, s2 = o.group_scale_ex(x, ends, 0, GROUP_INVERSE)
    assert np.array_equal(q2, q0)
    want = np.float32(1.0) / s0
    assert np.array_equal(np.isnan(s2), nan0) and np.array_equal(s2[fin].view(np.uint32), want[fin].view(np.uint32))
    q3, s3 = o.group_scale_ex(x, ends, 0, GROUP_POW2 | GROUP_INVERSE)
    assert np.array_equal(q3, q1)
    assert np.array_equal(s3[fin].astype(np.float64) * s1[fin].astype(np.float64), np.ones(fin.sum()))
    qc, sc = o.group_scale_ex(x, ends, 1, GROUP_POW2 | GROUP_INVERSE)
    assert np.array_equal(qc, q3.T) and np.array_equal(sc.view(np.uint32), s3.view(np.uint32))


def check_dispatch_pack(o, seed=18):
    """Dispatch pack against numpy's stable argsort and bincount, and every packed
    row against the MX quantizer pinned above (codes in front, scales behind)."""
    rng = np.random.default_rng(seed)
    for (M, K, topk, E) in [(50, 64, 1, 4), (37, 96, 2, 5), (20, 32, 3, 1)]:
        x = _random_blocks(rng, M * K // 32).reshape(M, K)
        ids = rng.integers(-1, E + 1, (M, topk)).astype(np.int32)   # -1 and E are dropped
        packed, src, ends = o.dispatch_pack(x, ids, E)
        flat = ids.ravel()
        keep = np.nonzero((flat >= 0) & (flat < E))[0]
        order = keep[np.argsort(flat[keep], kind="stable")]
        n = order.size
        assert np.array_equal(src[:n], order) and np.all(src[n:] == -1)
        assert np.array_equal(ends, np.cumsum(np.bincount(flat[keep], minlength=E)))
        q, s = o.mx_quantize(np.ascontiguousarray(x[order // topk]))
        assert packed.shape == (M * topk, K + K // 32)
        assert np.array_equal(packed[:n, :K], q) and np.array_equal(packed[:n, K:], s)


def check_group_invariants(o, seed=11):
    rng = np.random.default_rng(seed)
    M, K = 300, 48
    x = _token_matrix(rng, M, K)
    sizes = [120, 0, 75, 105]
    ends = np.cumsum(sizes).astype(np.int32)
    q, scales = o.group_scale(x, ends, 0)
    qc, scales_c = o.group_scale(x, ends, 1)
    # the two layouts hold the same bytes
    assert np.array_equal(qc, q.T) and np.array_equal(scales, scales_c)
    dec = torch.from_numpy(q.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    start = 0
    for g, e in enumerate(ends):
        rows = slice(start, int(e))
        if e > start:
            # every column with a non-zero amax reaches 448 exactly
            nz = (x[rows] & 0x7FFF).max(axis=0) > 0
            assert np.all(np.abs(dec[rows]).max(axis=0)[nz] == 448.0)
            # slicing: the group on its own gives the same bytes and scales
            qg, sg = o.group_scale(np.ascontiguousarray(x[rows]), [int(e) - start], 0)
            assert np.array_equal(qg, q[rows]) and np.array_equal(sg[0], scales[g])
            # permuting rows inside the group permutes the output rows
            perm = rng.permutation(int(e) - start)
            xp = x.copy()
            xp[rows] = x[rows][perm]
            qp, sp = o.group_scale(xp, ends, 0)
            assert np.array_equal(qp[rows], q[rows][perm]) and np.array_equal(sp, scales)
        start = int(e)
    # G = 1 equals per-column scaling of the whole tensor with the library rebuild
    q1, s1 = o.group_scale(x, [M], 0)
    qr, sr = group_reference_by_libraries(x, [M])
    assert np.array_equal(q1, qr) and np.array_equal(s1, sr)


def check_group_offsets_clamped(o, seed=12):
    """Out-of-contract end offsets: decreasing ends behave as the running maximum,
    ends past M are cut at M, rows past the last end get zero bytes."""
    rng = np.random.default_rng(seed)
    M, K = 40, 8
    x = _token_matrix(rng, M, K)
    q, s = o.group_scale(x, [10, 5, 60], 0)        # -> [10, 10, 40]
    q2, s2 = o.group_scale(x, [10, 10, 40], 0)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    q3, _ = o.group_scale(x, [10, 25], 0)
    assert np.all(q3[25:] == 0)


# ------------------------------------------------------------ transpose ---
def check_transpose(o, seed=13):
    rng = np.random.default_rng(seed)
    for R, C in [(1, 1), (3, 7), (64, 48), (129, 31)]:
        a = rng.integers(0, 256, (R, C)).astype(np.uint8)
        t = o.transpose_u8(a)
        assert np.array_equal(t, a.T)
        assert np.array_equal(o.transpose_u8(t), a)


# ------------------------------------------------ scaled grouped GEMM ---
def _random_mx_operand(rng, shape, scale_lo=112, scale_hi=142):
    """Random finite E4M3 codes (never 0x7F / 0xFF) and E8M0 codes in a range."""
    q = rng.integers(0, 256, size=shape).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] ^= 0x01
    s = rng.integers(scale_lo, scale_hi, size=shape[:-1] + (shape[-1] // 32,)).astype(np.uint8)
    return q, s


def mx_values_by_torch(q, s):
    """Dequantized MXFP8 values from torch's own E4M3 and E8M0 decoders, float64."""
    v = torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64)
    sc = torch.from_numpy(np.ascontiguousarray(s)).view(torch.float8_e8m0fnu).to(torch.float64)
    return (v * sc.repeat_interleave(32, dim=-1)).numpy()


def grouped_mm_by_torch(xq, xs, wq, ws, ends):
    """Y (M, N) float64 from torch matmuls of torch-dequantized operands, and the
    matching sum of |products| (the scale of the rounding in any summation order)."""
    X = mx_values_by_torch(xq, xs)
    W = mx_values_by_torch(wq, ws)
    M = X.shape[0]
    N = W.shape[1]
    Y = np.zeros((M, N))
    A = np.zeros((M, N))
    start = 0
    for g, e in enumerate(ends):
        end = min(max(int(e), start), M)
        Xg = torch.from_numpy(X[start:end])
        Wg = torch.from_numpy(W[g])
        Y[start:end] = (Xg @ Wg.T).numpy()
        A[start:end] = (Xg.abs() @ Wg.abs().T).numpy()
        start = end
    return Y, A


def check_grouped_mm_vs_torch(o, seed=14):
    """Ragged groups (one empty, one cut tail row range) against torch's decoders
    and float64 matmul; only the summation order differs."""
    rng = np.random.default_rng(seed)
    M, N, K = 150, 40, 192
    for ends in ([40, 40, 97, 130], [150], [0, 10, 150, 150]):
        G = len(ends)
        xq, xs = _random_mx_operand(rng, (M, K))
        wq, ws = _random_mx_operand(rng, (G, N, K))
        y = o.mx_grouped_mm(xq, xs, wq, ws, ends)
        ref, mag = grouped_mm_by_torch(xq, xs, wq, ws, ends)
        assert y.shape == (M, N)
        assert np.all(np.abs(y - ref) <= 1e-13 * mag), ends
        # sampled rows and columns are the same numbers
        rows = np.array([0, 39, 40, 96, 97, 129, 130, 149])
        cols = np.array([0, 7, 39])
        assert np.array_equal(o.mx_grouped_mm(xq, xs, wq, ws, ends, rows, cols), y[np.ix_(rows, cols)])


def check_grouped_mm_closed_form(o):
    """All operand values 1 with weight scale 2^g: Y = K * 2^g on group g's rows,
    0 past the last end; decreasing ends act as their running maximum."""
    M, N, K, G = 30, 8, 96, 4
    xq = np.full((M, K), 0x38, np.uint8)          # E4M3 1.0
    xs = np.full((M, K // 32), 127, np.uint8)     # 2^0
    wq = np.full((G, N, K), 0x38, np.uint8)
    ws = np.empty((G, N, K // 32), np.uint8)
    for g in range(G):
        ws[g] = 127 + g
    y = o.mx_grouped_mm(xq, xs, wq, ws, [6, 2, 11, 25])     # -> [6, 6, 11, 25]
    expect = np.zeros((M, N))
    expect[0:6] = K * 1.0
    expect[6:11] = K * 4.0
    expect[11:25] = K * 8.0
    assert np.array_equal(y, expect)
    # one E4M3 code in one weight row changes exactly that output column's sum
    wq2 = wq.copy()
    wq2[3, 5, 70] = 0xC0                          # -2.0 instead of 1.0
    y2 = o.mx_grouped_mm(xq, xs, wq2, ws, [6, 2, 11, 25])
    expect[11:25, 5] -= 3.0 * 8.0
    assert np.array_equal(y2, expect)


def check_grouped_mm_block_scales(o):
    """Each E8M0 scale covers its own 32 consecutive k: doubling one block's
    scale adds exactly that block's partial sum."""
    rng = np.random.default_rng(15)
    M, N, K = 6, 5, 128
    xq, xs = _random_mx_operand(rng, (M, K), 120, 130)
    wq, ws = _random_mx_operand(rng, (1, N, K), 120, 130)
    y = o.mx_grouped_mm(xq, xs, wq, ws, [M])
    X = mx_values_by_torch(xq, xs)
    W = mx_values_by_torch(wq, ws)[0]
    for b in range(K // 32):
        xs2 = xs.copy()
        xs2[2, b] += 1
        y2 = o.mx_grouped_mm(xq, xs2, wq, ws, [M])
        part = X[2, 32 * b:32 * b + 32] @ W[:, 32 * b:32 * b + 32].T
        mag = np.abs(X[2]) @ np.abs(W).T
        assert np.all(np.abs(y2[2] - (y[2] + part)) <= 1e-13 * 2 * mag)
        assert np.array_equal(np.delete(y2, 2, 0), np.delete(y, 2, 0))


def check_grouped_mm_nan(o):
    """A NaN scale code (0xFF) or a NaN E4M3 code poisons exactly the outputs it
    enters."""
    M, N, K = 4, 3, 64
    xq = np.full((M, K), 0x38, np.uint8)
    xs = np.full((M, K // 32), 127, np.uint8)
    wq = np.full((1, N, K), 0x38, np.uint8)
    ws = np.full((1, N, K // 32), 127, np.uint8)
    ws[0, 1, 1] = 0xFF
    xq[2, 5] = 0x7F
    y = o.mx_grouped_mm(xq, xs, wq, ws, [M])
    nan = np.isnan(y)
    assert nan[:, 1].all() and nan[2, :].all()
    assert nan.sum() == M + N - 1


FAST_CHECKS = [
    check_e4m3_decode_vs_torch, check_e4m3_code_facts, check_e4m3_encode_roundtrip,
    check_e8m0_decode_vs_torch, check_bf16_round_vs_torch, check_e4m3_encode_vs_torch_saturating,
    check_mx_worked_blocks, check_mx_invariants, check_mx_row_block_layout,
    check_group_worked, check_group_vs_libraries, check_group_invariants,
    check_group_offsets_clamped, check_transpose,
    check_grouped_mm_vs_torch, check_grouped_mm_closed_form, check_grouped_mm_block_scales,
    check_grouped_mm_nan,
    check_mx_rceil_worked_blocks, check_mx_rceil_vs_division, check_mx_axis0_is_transpose,
    check_group_variants, check_dispatch_pack,
]


def run_battery(o, checks=None, exhaustive_codes=(0, 1, 2, 3, 100, 119, 127, 130, 200, 246, 254)):
    """Run the checks; return the names of those that failed."""
    failed = []
    for chk in (checks or FAST_CHECKS):
        try:
            chk(o)
        except AssertionError:
            failed.append(chk.__name__)
    try:
        check_mx_encode_exhaustive(o, exhaustive_codes)
    except AssertionError:
        failed.append("check_mx_encode_exhaustive")
    return failed
