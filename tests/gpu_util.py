"""Helpers for the GPU parity tests: moving bit patterns to and from the device,
guarded output buffers, and the CPU oracle run over independent slices in
parallel threads (the oracle itself is unchanged; row blocks of the MX codec and
column blocks of group scaling are independent by definition)."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle

THREADS = max(1, min(16, os.cpu_count() or 1))
CANARY = 0xCD
GUARD = 256


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy()


def host_f32_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy().view(np.uint32)


class Guarded:
    """A device buffer of n elements followed by a guard band, all filled with a
    canary byte pattern, to catch unwritten and out-of-bounds bytes."""

    def __init__(self, n: int, dtype: torch.dtype, shape):
        esz = torch.tensor([], dtype=dtype).element_size()
        self.raw = torch.full((n * esz + GUARD,), CANARY, dtype=torch.uint8, device="cuda")
        self.t = self.raw[: n * esz].view(dtype).view(shape)
        self.n_bytes = n * esz

    def guard_intact(self) -> bool:
        return bool((self.raw[self.n_bytes:] == CANARY).all().item())


def _row_slices(M: int, parts: int):
    step = max(1, -(-M // parts))
    return [(a, min(M, a + step)) for a in range(0, M, step)]


def oracle_mx_quantize(x_bits: np.ndarray):
    M, K = x_bits.shape
    q = np.empty((M, K), np.uint8)
    s = np.empty((M, K // 32), np.uint8)

    def run(sl):
        a, b = sl
        q[a:b], s[a:b] = oracle.mx_quantize(np.ascontiguousarray(x_bits[a:b]))

    with ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(run, _row_slices(M, THREADS * 2)))
    return q, s


def oracle_mx_dequantize(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    M, K = q.shape
    y = np.empty((M, K), np.uint16)

    def run(sl):
        a, b = sl
        y[a:b] = oracle.mx_dequantize(np.ascontiguousarray(q[a:b]), np.ascontiguousarray(s[a:b]))

    with ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(run, _row_slices(M, THREADS * 2)))
    return y


def oracle_group_scale_row(x_bits: np.ndarray, ends) -> tuple:
    """Row-layout output and (G, K) scales, columns split across threads."""
    M, K = x_bits.shape
    G = len(ends)
    q = np.empty((M, K), np.uint8)
    scales = np.empty((G, K), np.float32)
    step = max(8, -(-K // (THREADS * 2)))
    cols = [(a, min(K, a + step)) for a in range(0, K, step)]

    def run(sl):
        a, b = sl
        qq, ss = oracle.group_scale(np.ascontiguousarray(x_bits[:, a:b]), ends, oracle.LAYOUT_ROW)
        q[:, a:b] = qq
        scales[:, a:b] = ss

    with ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(run, cols))
    return q, scales


def first_mismatch(a: np.ndarray, b: np.ndarray) -> str:
    if a.shape != b.shape:
        return f"shape {a.shape} vs {b.shape}"
    idx = np.argwhere(a != b)
    if idx.size == 0:
        return "equal"
    i = tuple(idx[0])
    return f"{len(idx)} mismatches, first at {i}: got {a[i]!r} want {b[i]!r}"


def exhaustive_mx_blocks(seed: int = 0) -> np.ndarray:
    """Blocks of 32 bf16 covering every (finite element, scale code) pair the
    quantizer can meet: for each code c = 0..246 an anchor of biased exponent
    c + 8 (mantissa all ones) fixes the block maximum, and the other 31 slots
    take every finite pattern of magnitude at most the anchor.  Each block is
    shuffled so the maximum sits anywhere in the block.  Also: blocks whose
    maximum is subnormal or below 2^-119, and blocks holding Inf or NaN."""
    rng = np.random.default_rng(seed)
    allp = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    fin = allp[(allp & 0x7F80) != 0x7F80]
    mag = fin & 0x7FFF
    blocks = []
    for c in range(247):
        anchor = np.uint16(((c + 8) << 7) | 0x7F)
        pool = fin[mag <= anchor]
        pool = np.concatenate([pool, np.zeros((-len(pool)) % 31, np.uint16)])
        b = pool.reshape(-1, 31)
        blocks.append(np.concatenate([np.full((b.shape[0], 1), anchor, np.uint16), b], axis=1))
    for E in range(0, 9):                       # block maxima with biased exponent 0..8
        for _ in range(16):
            v = (rng.integers(0, 1 << 7, 32) | (rng.integers(0, E + 1, 32) << 7)).astype(np.uint16)
            v |= (rng.integers(0, 2, 32) << 15).astype(np.uint16)
            blocks.append(v[None, :])
    nonfinite = rng.integers(0, 1 << 16, (512, 32)).astype(np.uint16)
    nonfinite[(nonfinite & 0x7F80) == 0x7F80] = 0
    specials = np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x7F81], np.uint16)
    nonfinite[np.arange(512), rng.integers(0, 32, 512)] = specials[rng.integers(0, 5, 512)]
    blocks.append(nonfinite)
    allb = np.concatenate(blocks, axis=0)
    for i in range(allb.shape[0]):
        rng.shuffle(allb[i])
    return allb


def exhaustive_mx_codes():
    """(q, s) covering every (E4M3 code, E8M0 code) pair: row r has scale code r
    on all 8 of its blocks and the 256 codes in order."""
    q = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
    s = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 8, axis=1)
    return q, s


def oracle_mx_grouped_mm(xq, xs, wq, ws, ends, rows, cols) -> np.ndarray:
    """The oracle's grouped product at the given rows and columns, row blocks in
    parallel threads (rows are independent by definition)."""
    rows = np.asarray(rows, dtype=np.int64)
    y = np.empty((rows.size, len(cols)), np.float64)

    def run(sl):
        a, b = sl
        y[a:b] = oracle.mx_grouped_mm(xq, xs, wq, ws, ends, rows[a:b], cols)

    with ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(run, _row_slices(rows.size, THREADS * 2)))
    return y
