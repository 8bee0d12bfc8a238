"""Seeded generators for the five synthetic workloads.

Every tensor is drawn from its own ``numpy.random.Generator`` seeded by
``(seed, crc32(name))``, so a tensor's bytes do not depend on which other tensors were
drawn first. Storage formats:

* activations and dense weights: bf16 bit patterns (``uint16``), rounded from fp32 draws
  with round-to-nearest-even;
* expert weight banks: packed int4 bytes ``[E][N][K/2]`` -- int4 values uniform over
  -8..7 are exactly uniform nibbles, so the bank is drawn directly as uniform random
  bytes (no packing code is needed or present here);
* expert weight scales: fp32 ``[E][N][K/128]`` uniform in [0.005, 0.02);
* router logits: fp32 ``[T][E]``.

The shapes and value distributions follow the workloads of the FP8 grouped-expert prefill
note (octopusresearch.org, "FP8 grouped-expert prefill with on-chip int4-to-e4m3 dequant",
section 1) and the W8A8 dense projection PR (FreeToken PR #389, "What this adds" and
"Limits"), fixed to concrete sizes below.
"""

from __future__ import annotations

import zlib
from dataclasses import dataclass

import numpy as np

GROUP = 128


def rng_for(seed: int, name: str) -> np.random.Generator:
    """Independent stream per (seed, tensor name)."""
    return np.random.default_rng([int(seed), zlib.crc32(name.encode())])


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest, ties to even (finite inputs)."""
    b = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    lsb = (b >> 16) & 1
    b += np.uint32(0x7FFF)  # no overflow for finite fp32 bit patterns
    b += lsb
    b >>= 16
    return b.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> the fp32 value it denotes (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------------
# Workload presets
# ----------------------------------------------------------------------------------


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int  # tokens
    H: int  # hidden size (K of the gate|up GEMM, N of the down GEMM)
    E: int  # experts
    k: int  # experts per token
    I: int  # expert intermediate size
    zipf_s: float = 0.0  # >0: router logits biased by -s*ln(e+1)
    seed: int = 0

    @property
    def R(self) -> int:
        return self.T * self.k


@dataclass(frozen=True)
class DenseConfig:
    name: str
    M: int
    K: int
    N_qkv: int
    N_o: int
    outlier_frac: float = 0.01
    outlier_mul: float = 20.0
    seed: int = 0


@dataclass(frozen=True)
class StackConfig:
    name: str
    L: int
    T: int
    H: int
    n_q: int
    n_kv: int
    head_dim: int
    E: int
    k: int
    I: int
    V: int
    seed: int = 0


CONFIGS = {
    # Tiny single MoE FFN layer; the size the oracle finishes in well under a second.
    "moe_tiny": MoEConfig("moe_tiny", T=64, H=256, E=8, k=2, I=512),
    # Dense W8A8 projections: fused qkv (N=6144) and o_proj (N=4096), K=4096, M=2048.
    "dense_w8a8": DenseConfig("dense_w8a8", M=2048, K=4096, N_qkv=6144, N_o=4096),
    # One MoE prefill layer: 4096 tokens, hidden 2048, 64 experts, top-8, I=768.
    "moe_prefill": MoEConfig("moe_prefill", T=4096, H=2048, E=64, k=8, I=768),
    # Skewed large layer: 16384 tokens, hidden 4096, 128 experts, top-8, I=1536, Zipf 1.2.
    "moe_skewed": MoEConfig("moe_skewed", T=16384, H=4096, E=128, k=8, I=1536, zipf_s=1.2),
    # Depth stacks of 8 and 12 layers at T=2048.
    "stack_L8": StackConfig("stack_L8", L=8, T=2048, H=2048, n_q=16, n_kv=4, head_dim=128,
                            E=64, k=8, I=768, V=32000),
    "stack_L12": StackConfig("stack_L12", L=12, T=2048, H=2048, n_q=16, n_kv=4, head_dim=128,
                             E=64, k=8, I=768, V=32000),
}


# ----------------------------------------------------------------------------------
# Draws
# ----------------------------------------------------------------------------------


def _normal_bf16(seed: int, name: str, shape, std: float = 1.0) -> np.ndarray:
    x = rng_for(seed, name).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return bf16_bits_from_f32(x)


def _bank(seed: int, name: str, E: int, N: int, K: int):
    """Packed int4 bank [E][N][K/2] (uniform nibbles) and fp32 scales [E][N][K/128]."""
    assert K % GROUP == 0
    nbytes = E * N * (K // 2)
    words = rng_for(seed, name + ".q").bit_generator.random_raw((nbytes + 7) // 8)
    w = np.asarray(words, dtype=np.uint64).view(np.uint8)[:nbytes].reshape(E, N, K // 2)
    s = rng_for(seed, name + ".s").uniform(0.005, 0.02, size=(E, N, K // GROUP))
    return w, s.astype(np.float32)


def router_logits(seed: int, name: str, T: int, E: int, zipf_s: float = 0.0) -> np.ndarray:
    z = rng_for(seed, name).standard_normal((T, E), dtype=np.float32)
    if zipf_s > 0.0:
        # log of a Zipf(s) popularity weight by expert rank: -s * ln(e + 1)
        bias = (-zipf_s * np.log(np.arange(E, dtype=np.float64) + 1.0)).astype(np.float32)
        z = z + bias[None, :]
    return z


def moe_inputs(cfg: MoEConfig, seed: int | None = None, T: int | None = None) -> dict:
    """Inputs of one MoE layer. ``T`` may shrink the token count (same weights)."""
    seed = cfg.seed if seed is None else seed
    T = cfg.T if T is None else T
    x = _normal_bf16(seed, f"{cfg.name}.x", (cfg.T, cfg.H))[:T]
    logits = router_logits(seed, f"{cfg.name}.logits", cfg.T, cfg.E, cfg.zipf_s)[:T]
    w_gu, s_gu = _bank(seed, f"{cfg.name}.w_gu", cfg.E, 2 * cfg.I, cfg.H)
    w_dn, s_dn = _bank(seed, f"{cfg.name}.w_dn", cfg.E, cfg.H, cfg.I)
    return dict(x=np.ascontiguousarray(x), logits=np.ascontiguousarray(logits),
                w_gu=w_gu, s_gu=s_gu, w_dn=w_dn, s_dn=s_dn)


def outlier_columns(seed: int, name: str, K: int, frac: float) -> np.ndarray:
    n = max(1, int(round(frac * K)))
    return np.sort(rng_for(seed, name).choice(K, size=n, replace=False))


def _act_with_outliers(seed: int, name: str, M: int, K: int, frac: float, mul: float):
    x = rng_for(seed, name).standard_normal((M, K), dtype=np.float32)
    cols = outlier_columns(seed, name + ".cols", K, frac)
    x[:, cols] *= np.float32(mul)
    return bf16_bits_from_f32(x), cols


def dense_inputs(cfg: DenseConfig, seed: int | None = None, M: int | None = None) -> dict:
    """bf16 activations (1% outlier channels x20) and bf16 N(0, 0.02) weights."""
    seed = cfg.seed if seed is None else seed
    M = cfg.M if M is None else M
    x, cols = _act_with_outliers(seed, f"{cfg.name}.x", cfg.M, cfg.K, cfg.outlier_frac,
                                 cfg.outlier_mul)
    xo, _ = _act_with_outliers(seed, f"{cfg.name}.x_o", cfg.M, cfg.K, cfg.outlier_frac,
                               cfg.outlier_mul)
    w_qkv = _normal_bf16(seed, f"{cfg.name}.w_qkv", (cfg.N_qkv, cfg.K), std=0.02)
    w_o = _normal_bf16(seed, f"{cfg.name}.w_o", (cfg.N_o, cfg.K), std=0.02)
    return dict(x=np.ascontiguousarray(x[:M]), x_o=np.ascontiguousarray(xo[:M]),
                outlier_cols=cols, w_qkv=w_qkv, w_o=w_o)


def stack_inputs(cfg: StackConfig, seed: int | None = None, T: int | None = None,
                 L: int | None = None) -> dict:
    """Random-init depth stack: per layer W8A8 q/k/v/o (bf16 source weights), a bf16
    router, int4 expert banks; a bf16 LM head. RMSNorm gains are 1."""
    seed = cfg.seed if seed is None else seed
    T = cfg.T if T is None else T
    L = cfg.L if L is None else L
    H, hd = cfg.H, cfg.head_dim
    nqkv = (cfg.n_q + 2 * cfg.n_kv) * hd
    layers = []
    for li in range(L):
        p = f"stack.layer{li}"
        w_gu, s_gu = _bank(seed, f"{p}.w_gu", cfg.E, 2 * cfg.I, H)
        w_dn, s_dn = _bank(seed, f"{p}.w_dn", cfg.E, H, cfg.I)
        layers.append(dict(
            w_qkv=_normal_bf16(seed, f"{p}.w_qkv", (nqkv, H), std=0.02),
            w_o=_normal_bf16(seed, f"{p}.w_o", (H, cfg.n_q * hd), std=0.02),
            w_router=_normal_bf16(seed, f"{p}.w_router", (cfg.E, H), std=0.02),
            w_gu=w_gu, s_gu=s_gu, w_dn=w_dn, s_dn=s_dn))
    x0 = _normal_bf16(seed, "stack.x0", (cfg.T, H))[:T]
    w_lm = _normal_bf16(seed, "stack.w_lm", (cfg.V, H), std=0.02)
    return dict(x0=np.ascontiguousarray(x0), layers=layers, w_lm=w_lm)
