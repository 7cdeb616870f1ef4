"""Seeded synthetic workloads: shapes and random draws only.

This module holds none of the NF4 arithmetic.  It is the one place both the
oracle-side tests and the GPU-side tests/benchmark take their inputs from, so
the two sides see identical bytes.  Every draw comes from
numpy.random.default_rng(SeedSequence([base, workload, layer, proj, kind])).

Shapes are those of the models the pages measure on (Llama-3.1-8B streaming in
Soup issue #842 "Why"; Qwen2.5-32B in bitsandbytes #2034 "The evidence,
briefly"; OLMoE-1B-7B experts in the Experts PR "Measurements").  No
checkpoint or dataset is used: weights are 0.02 * N(0, 1) fp32, activations
and output gradients are N(0, 1) rounded to bf16 by torch.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

BASE_SEED = 20251202

# workload ids inside the seed sequence
W_TINY, W_LLAMA, W_DECODE, W_QWEN, W_OLMOE = 0, 1, 2, 3, 4
# tensor kinds inside the seed sequence
K_WEIGHT, K_X, K_GY, K_ROUTE = 0, 1, 2, 3


@dataclass(frozen=True)
class Proj:
    name: str
    N: int   # out features (rows of W)
    K: int   # in features


# Llama-3.1-8B projections, W in the F.linear [out, in] layout.
LLAMA_8B = (
    Proj("q", 4096, 4096), Proj("k", 1024, 4096), Proj("v", 1024, 4096),
    Proj("o", 4096, 4096), Proj("gate", 14336, 4096), Proj("up", 14336, 4096),
    Proj("down", 4096, 14336),
)
LLAMA_LAYERS = 32
LLAMA_M = 512            # batch 1, S = 512
DECODE_MS = (1, 8, 32)

# Qwen-32B-shaped projections at M = 2048.
QWEN_32B = (
    Proj("q", 5120, 5120), Proj("k", 1024, 5120), Proj("v", 1024, 5120),
    Proj("o", 5120, 5120), Proj("gate", 27648, 5120), Proj("up", 27648, 5120),
    Proj("down", 5120, 27648),
)
QWEN_M = 2048

# OLMoE-1B-7B experts: 64 experts, hidden 2048, intermediate 1024, top-8, 512 tokens.
OLMOE_E, OLMOE_HIDDEN, OLMOE_INTER, OLMOE_TOPK, OLMOE_TOKENS = 64, 2048, 1024, 8, 512

# Tiny NF4 linear (non-nested): M = 64, N = 128, K = 256.
TINY_M, TINY_N, TINY_K = 64, 128, 256


# Call arguments, not arithmetic: the 16 NF4 levels (4-decimal NormalFloat-4
# values) and the 256-entry nested table (2j - 255) / 255 that every call of
# the codec and the matmuls receives as input.
NF4_LEVELS = (
    -1.0, -0.6962, -0.5251, -0.3949, -0.2844, -0.1848, -0.0911, 0.0,
    0.0796, 0.1609, 0.2461, 0.3379, 0.4407, 0.5626, 0.7230, 1.0,
)
NESTED_UNIFORM = tuple((2.0 * j - 255.0) / 255.0 for j in range(256))
# The 4-bit float alternative (fp4, a code-table swap on the same kernels):
# the 16 values of a 1-sign / 2-exponent / 1-mantissa float, magnitudes
# {0, 0.5, 1, 1.5, 2, 3, 4, 6}, divided by 6 so the largest is 1, in
# ascending order with -0 before +0.  The stored 4-bit index is the rank in
# this table, not the float's bit pattern.
FP4_LEVELS = (
    -1.0, -4 / 6, -3 / 6, -2 / 6, -1.5 / 6, -1 / 6, -0.5 / 6, -0.0,
    0.0, 0.5 / 6, 1 / 6, 1.5 / 6, 2 / 6, 3 / 6, 4 / 6, 1.0,
)


def int8_code_np() -> np.ndarray:
    """The 8-bit integer map (a call argument): index j stands for the signed
    integer j - 128 scaled by 1/127, so |t| <= 1 uses indices 1 .. 255 and
    the block's absmax element maps to +-127 exactly."""
    j = np.arange(256, dtype=np.float64)
    return ((j - 128.0) / 127.0).astype(np.float32)


def fp8_e4m3_code_np() -> np.ndarray:
    """The fp8 e4m3 codebook (a call argument): the values of all 256 bit
    patterns of a float with 1 sign, 4 exponent (bias 7) and 3 mantissa bits,
    exponent field 0 subnormal, every pattern finite (largest 1.875 * 2^8 =
    480), divided by 480 so the largest is 1, in ascending order with -0
    before +0.  The stored byte is the rank in this table."""
    vals = []
    for bits in range(256):
        sign = -1.0 if bits & 0x80 else 1.0
        e, m = (bits >> 3) & 15, bits & 7
        mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
        vals.append((sign * mag, 0 if bits & 0x80 else 1))
    vals.sort()
    return np.array([v / 480.0 for v, _ in vals], dtype=np.float64).astype(np.float32)


def nf4_code_np() -> np.ndarray:
    return np.array(NF4_LEVELS, dtype=np.float64).astype(np.float32)


def fp4_code_np() -> np.ndarray:
    return np.array(FP4_LEVELS, dtype=np.float64).astype(np.float32)


def nested_code_np() -> np.ndarray:
    return np.array(NESTED_UNIFORM, dtype=np.float64).astype(np.float32)


def rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([BASE_SEED, *key]))


def weight_f32(N: int, K: int, *key: int, std: float = 0.02) -> np.ndarray:
    """W [N, K] fp32 ~ std * N(0, 1)."""
    g = rng(*key, K_WEIGHT)
    return (g.standard_normal((N, K), dtype=np.float32) * np.float32(std)).astype(np.float32)


def normal_bf16(M: int, C: int, *key: int) -> torch.Tensor:
    """[M, C] bf16 CPU tensor of N(0, 1) draws (torch rounds to bf16)."""
    g = rng(*key)
    a = g.standard_normal((M, C), dtype=np.float32)
    return torch.from_numpy(a).to(torch.bfloat16)


def x_bf16(M: int, K: int, *key: int) -> torch.Tensor:
    return normal_bf16(M, K, *key, K_X)


def grad_y_bf16(M: int, N: int, *key: int) -> torch.Tensor:
    return normal_bf16(M, N, *key, K_GY)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bf16 bit patterns of a CPU bf16 tensor, as uint16 (no arithmetic)."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def olmoe_routing(tokens: int = OLMOE_TOKENS, experts: int = OLMOE_E, topk: int = OLMOE_TOPK,
                  *key: int):
    """Top-k distinct experts per token, uniform without replacement.

    Returns (order, expert_of_row, offsets): `order` maps each sorted row to
    its token, rows are stably sorted by expert, offsets[e] is the first row
    of expert e (length experts + 1).
    """
    g = rng(W_OLMOE, *key, K_ROUTE)
    choice = np.argsort(g.random((tokens, experts)), axis=1)[:, :topk]   # distinct per token
    tok = np.repeat(np.arange(tokens), topk)
    exp = choice.reshape(-1)
    perm = np.argsort(exp, kind="stable")
    counts = np.bincount(exp, minlength=experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return tok[perm], exp[perm], offsets


# Seeds of the 32-layer stacks the benchmark draws on the device: the weight
# of projection i in layer l, the layer's inputs (q/k/v read one input,
# gate/up another; X_SLOT maps a projection to its input) and one grad_y per
# projection.
LLAMA_STACK_W_SEED, LLAMA_STACK_IN_SEED = 10_000, 20_000
X_SLOT = (0, 0, 0, 1, 2, 2, 3)


def stack_weight_seed(seed0: int, layer: int, i: int) -> int:
    return seed0 + 16 * layer + i


def stack_x_seed(seed0: int, layer: int, slot: int) -> int:
    return seed0 + 4 * layer + slot


def stack_gy_seed(seed0: int, layer: int, i: int) -> int:
    return seed0 + 10_000 + 16 * layer + i


def gpu_weight_f32(N: int, K: int, seed: int, device="cuda", std: float = 0.02) -> torch.Tensor:
    """W [N, K] fp32 ~ std * N(0, 1) drawn on the device by torch's seeded
    Philox generator (used where host draws would be too slow: the 32-layer
    benchmark stack)."""
    g = torch.Generator(device=device)
    g.manual_seed(BASE_SEED * 1000 + seed)
    return torch.randn((N, K), generator=g, device=device, dtype=torch.float32).mul_(std)


def gpu_normal_bf16(M: int, C: int, seed: int, device="cuda") -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(BASE_SEED * 1000 + seed)
    return torch.randn((M, C), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
