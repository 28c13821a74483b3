"""Seeded synthetic inputs for the float8 MoE quantization path.

This module holds no arithmetic of the method: it only draws random tensors
with the shapes and value distributions of the MoE workloads (token payloads
and expert routing) and hands out the same bytes to the HIP library and to the
CPU oracle.  Everything is drawn on the CPU with ``torch.Generator`` so that a
seed always gives the same bytes, whatever device the consumer runs on.

Workloads (shapes from the pages' MoE setting: hidden dim 5120, 16 experts,
sequence 8192 x local batch 8 tokens per rank -- "[mxfp8 MoE training] Support
mxfp8 all to all in expert parallel", Performance / Additional context; and the
(16640, 5120) kernel shape of "[moe training] fix uncoalesced global accesses in
per group rowwise scaling kernel", Performance tables):

  tiny       X (512, 256) ~ N(0, 1); four token groups of sizes 100, 37, 0, 375.
  dispatch   X (65536, 5120): N(0, 1) times a per-row lognormal(0, 1) factor,
             0.1 % of the elements (drawn with replacement) multiplied by 100,
             1 % of the rows set to zero -- one rank's dispatch payload.
  tokens     X (16640, 5120): N(0, 1) times a per-row lognormal(0, 1) factor.
  routing    16640 tokens drawn to G experts with probabilities proportional
             to (g + 1) ** -1.1 (Zipf 1.1, expert 0 hottest); group g's size is
             the count of tokens drawn to it; end offsets are the running sums.
  experts    W (16, 8192, 5120): one (N, K) weight per expert, N(0, 0.02^2) --
             the right operand of the grouped product Y_g = X_g W_g^T over the
             tokens routed to expert g.
"""
from __future__ import annotations

import numpy as np
import torch

TINY_SHAPE = (512, 256)
TINY_GROUP_SIZES = (100, 37, 0, 375)
DISPATCH_SHAPE = (65536, 5120)
TOKENS_SHAPE = (16640, 5120)
EXPERTS_SHAPE = (16, 8192, 5120)
EXPERT_WEIGHT_STD = 0.02
ZIPF_ALPHA = 1.1


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(int(seed))
    return g


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    """uint16 view of a CPU bf16 tensor (bit patterns, no conversion)."""
    if x.dtype != torch.bfloat16:
        raise TypeError("expected a bfloat16 tensor")
    return x.contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bf16_bits(bits: np.ndarray) -> torch.Tensor:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)


def ends_from_sizes(sizes) -> np.ndarray:
    return np.cumsum(np.asarray(sizes, dtype=np.int64)).astype(np.int32)


def tiny_x(seed: int = 0) -> torch.Tensor:
    return torch.randn(TINY_SHAPE, generator=_gen(seed)).to(torch.bfloat16)


def tiny_group_ends() -> np.ndarray:
    return ends_from_sizes(TINY_GROUP_SIZES)


def lognormal_rows(M: int, K: int, seed: int = 0) -> torch.Tensor:
    """N(0, 1) times a per-row lognormal(0, 1) factor, in float32."""
    g = _gen(seed)
    x = torch.randn((M, K), generator=g)
    x *= torch.exp(torch.randn((M, 1), generator=g))
    return x


def device_tokens(M: int, K: int, seed: int = 0, chunk_rows: int = 32768) -> torch.Tensor:
    """As lognormal_rows (N(0, 1) times a per-row lognormal(0, 1) factor), but drawn
    on the current GPU in row chunks and cast to bf16 there: for sizes too large to
    draw and copy from the host.  Both sides read the same device bytes."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    for a in range(0, M, chunk_rows):
        b = min(M, a + chunk_rows)
        c = torch.randn((b - a, K), generator=g, device="cuda")
        c *= torch.exp(torch.randn((b - a, 1), generator=g, device="cuda"))
        x[a:b] = c.to(torch.bfloat16)
    return x


def dispatch_payload(M: int = DISPATCH_SHAPE[0], K: int = DISPATCH_SHAPE[1], seed: int = 0,
                     outlier_frac: float = 0.001, outlier_mult: float = 100.0,
                     zero_row_frac: float = 0.01) -> torch.Tensor:
    g = _gen(seed)
    x = torch.randn((M, K), generator=g)
    x *= torch.exp(torch.randn((M, 1), generator=g))
    flat = x.view(-1)
    n_out = int(outlier_frac * M * K)
    if n_out:
        idx = torch.randint(0, M * K, (n_out,), generator=g)
        flat[idx] = flat[idx] * outlier_mult
    n_zero = int(zero_row_frac * M)
    if n_zero:
        rows = torch.randperm(M, generator=g)[:n_zero]
        x[rows] = 0.0
    return x.to(torch.bfloat16)


def moe_tokens(M: int = TOKENS_SHAPE[0], K: int = TOKENS_SHAPE[1], seed: int = 0) -> torch.Tensor:
    return lognormal_rows(M, K, seed).to(torch.bfloat16)


def zipf_group_sizes(M: int, G: int, alpha: float = ZIPF_ALPHA, seed: int = 1) -> np.ndarray:
    p = torch.arange(1, G + 1, dtype=torch.float64) ** (-alpha)
    p = p / p.sum()
    assign = torch.multinomial(p, M, replacement=True, generator=_gen(seed))
    return torch.bincount(assign, minlength=G).numpy().astype(np.int64)


def zipf_group_ends(M: int, G: int, alpha: float = ZIPF_ALPHA, seed: int = 1) -> np.ndarray:
    return ends_from_sizes(zipf_group_sizes(M, G, alpha, seed))


def routed_expert_ids(M: int, E: int, topk: int = 1, alpha: float = ZIPF_ALPHA, seed: int = 1) -> np.ndarray:
    """(M, topk) int32 expert ids, Zipf(alpha) over E experts (expert 0 hottest): the
    same draw as zipf_group_sizes, so for topk = 1 the ids' bincount is exactly those
    group sizes (the dispatch pack of these ids yields zipf_group_ends)."""
    p = torch.arange(1, E + 1, dtype=torch.float64) ** (-alpha)
    p = p / p.sum()
    assign = torch.multinomial(p, M * topk, replacement=True, generator=_gen(seed))
    return assign.numpy().astype(np.int32).reshape(M, topk)


def random_bf16_bits(shape, seed: int, finite_only: bool = True) -> np.ndarray:
    """Uniformly random bf16 bit patterns (all exponents), optionally finite only."""
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 1 << 16, size=shape, dtype=np.uint32).astype(np.uint16)
    if finite_only:
        bad = (bits & 0x7F80) == 0x7F80
        bits[bad] &= 0xBFFF  # clear the top exponent bit: now finite
    return bits


def expert_weights(G: int = EXPERTS_SHAPE[0], N: int = EXPERTS_SHAPE[1], K: int = EXPERTS_SHAPE[2],
                   seed: int = 2) -> torch.Tensor:
    """(G, N, K) bf16 expert weights ~ N(0, 0.02^2), drawn in fp32 and cast once."""
    w = torch.randn((G, N, K), generator=_gen(seed), dtype=torch.float32)
    w.mul_(EXPERT_WEIGHT_STD)
    return w.to(torch.bfloat16)
