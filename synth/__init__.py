"""Seeded synthetic inputs for the FP4 weight-only MoE expert path.

This module is shared by the CPU oracle and the GPU path.  It only draws
random bytes and numbers and lays them out; it holds none of the method's
arithmetic (no code decoding, no scale decoding, no matmul, no routing).

Layouts (one MoE layer):
  logits  float32 [T][E]
  x       bfloat16 bits (uint16) [T][H]
  w1      uint8 [E][H][I]       FC1 packed E2M1, K=H, N=2I; byte (e,k,j): low nibble = column 2j
  s1      uint8 [E][H/B][2I]    FC1 block scales (E4M3 bytes for NVFP4, E8M0 bytes for MXFP4)
  g1      float32 [E] or None   FC1 per-expert global scale (NVFP4; MXFP4 when mx_global)
  w2      uint8 [E][I][H/2]     FC2 packed E2M1, K=I, N=H
  s2      uint8 [E][I/B][H]
  g2      float32 [E] or None
FP8 (W8A16) layers instead hold w1 uint8 [E][2I][H] and w2 uint8 [E][H][I]
(E4M3FN bytes, each output column's K weights contiguous), s1 = s2 = None,
and global scales g1, g2.

Random streams: one numpy PCG64 generator per (seed, tensor id), so every
tensor is reproducible on its own.  Tensor ids: 0 logits, 1 x, 2 w1, 3 s1,
4 g1, 5 w2, 6 s2, 7 g2, 8 hot/popularity permutation, 9 router weights.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

NVFP4 = "nvfp4"
MXFP4 = "mxfp4"
FP8 = "fp8"          # W8A16: E4M3FN weight bytes [E][N][K], per-expert global scale, no block scales
BLOCK = {NVFP4: 16, MXFP4: 32, FP8: 1}

# E4M3 scale bytes whose magnitude lies in [2^-4, 2^2]: exponent field 3..8
# with any mantissa field, plus exponent field 9 with mantissa field 0, both
# signs.  Chosen by bit fields only.
_E4M3_ELIGIBLE = np.array(
    [(s << 7) | (e << 3) | m for s in (0, 1) for e in range(3, 9) for m in range(8)]
    + [(s << 7) | (9 << 3) for s in (0, 1)],
    dtype=np.uint8,
)
_E4M3_ELIGIBLE_POS = _E4M3_ELIGIBLE[_E4M3_ELIGIBLE < 0x80]
# E8M0 bytes for the exponents -8..+2 (bias 127).
_E8M0_LO, _E8M0_HI = 127 - 8, 127 + 2


def stream(seed: int, tid: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(tid)])))


def normal_f32(g: np.random.Generator, shape) -> np.ndarray:
    return g.standard_normal(size=shape, dtype=np.float64).astype(np.float32)


def to_bf16_bits(a_f32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (torch's round-to-nearest-even cast)."""
    t = torch.from_numpy(np.ascontiguousarray(a_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def packed_codes(g: np.random.Generator, shape) -> np.ndarray:
    """Uniform random bytes: both nibbles are independent uniform 4-bit codes."""
    n = int(np.prod(shape))
    raw = g.bit_generator.random_raw((n + 7) // 8).view(np.uint8)
    return raw[:n].reshape(shape)


def e4m3_scales(g: np.random.Generator, shape, positive_only: bool = False) -> np.ndarray:
    pool = _E4M3_ELIGIBLE_POS if positive_only else _E4M3_ELIGIBLE
    return pool[g.integers(0, len(pool), size=shape)]


def e8m0_scales(g: np.random.Generator, shape) -> np.ndarray:
    return g.integers(_E8M0_LO, _E8M0_HI + 1, size=shape, dtype=np.uint8)


# E4M3FN weight bytes with magnitude in [2^-3, 2^3): exponent field 4..9, any
# mantissa, both signs (never the NaN bytes).  Chosen by bit fields only.
_FP8_WEIGHT_BYTES = np.array([(s << 7) | (e << 3) | m for s in (0, 1) for e in range(4, 10) for m in range(8)],
                             dtype=np.uint8)


def fp8_weight_bytes(g: np.random.Generator, shape) -> np.ndarray:
    # uint8 table indices keep a prefill layer's 6.4 GB draw at one byte per weight
    return _FP8_WEIGHT_BYTES[g.integers(0, len(_FP8_WEIGHT_BYTES), size=shape, dtype=np.uint8)]


def global_scales(g: np.random.Generator, n: int) -> np.ndarray:
    return (0.5 + 1.5 * g.random(n)).astype(np.float32)


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    fmt: str
    T: int
    E: int
    k: int
    H: int
    I: int
    routing: str = "normal"       # "normal" | "hot3" | "zipf"
    seed: int = 0
    positive_scales: bool = False
    mx_global: bool = False       # MXFP4 with a per-expert global scale too

    @property
    def B(self) -> int:
        return BLOCK[self.fmt]

    @property
    def rows(self) -> int:
        return self.T * self.k


@dataclasses.dataclass(frozen=True)
class DequantConfig:
    name: str
    fmt: str
    E: int
    K: int
    N: int
    seed: int = 0

    @property
    def B(self) -> int:
        return BLOCK[self.fmt]


# The workloads: shapes and value distributions of the decode, MTP-verify,
# dequant and prefill cases the pages measure.
TINY = LayerConfig("tiny_nvfp4_T1_E8_top2_H256_I128", NVFP4, T=1, E=8, k=2, H=256, I=128)
DEQUANT = DequantConfig("dequant_mxfp4_E32_K2048_N1536", MXFP4, E=32, K=2048, N=1536)
DECODE = LayerConfig("decode_nvfp4_T1_E256_top8_H2048_I768", NVFP4, T=1, E=256, k=8, H=2048, I=768)
MTP4 = LayerConfig("mtp_nvfp4_T4_E256_top8_H2048_I768_hot3", NVFP4, T=4, E=256, k=8, H=2048, I=768, routing="hot3")
MTP8 = LayerConfig("mtp_nvfp4_T8_E256_top8_H2048_I768_hot3", NVFP4, T=8, E=256, k=8, H=2048, I=768, routing="hot3")
# the same layer at 2 tokens (16 rows): the middle of the decode GEMV's 4-64 row range
MTP2 = LayerConfig("mtp_nvfp4_T2_E256_top8_H2048_I768_hot3", NVFP4, T=2, E=256, k=8, H=2048, I=768, routing="hot3")
MX_DECODE = LayerConfig("decode_mxfp4_T8_E256_top8_H4096_I2048", MXFP4, T=8, E=256, k=8, H=4096, I=2048)
MX_PREFILL = LayerConfig("prefill_mxfp4_T512_E256_top8_H4096_I2048_zipf", MXFP4, T=512, E=256, k=8, H=4096, I=2048, routing="zipf")

# W8A16 decode at the NVFP4 MTP-verify shape (the pages' FP8 path, sections 6.4 and 10).
FP8_MTP4 = LayerConfig("mtp_fp8_T4_E256_top8_H2048_I768_hot3", FP8, T=4, E=256, k=8, H=2048, I=768, routing="hot3")
FP8_PREFILL = LayerConfig("prefill_fp8_T512_E256_top8_H4096_I2048_zipf", FP8, T=512, E=256, k=8, H=4096, I=2048,
                          routing="zipf")

LAYER_CONFIGS = {c.name: c for c in (TINY, DECODE, MTP2, MTP4, MTP8, MX_DECODE, MX_PREFILL, FP8_MTP4, FP8_PREFILL)}

HOT_BOOST = 6.0


def logits(cfg: LayerConfig) -> np.ndarray:
    g = stream(cfg.seed, 0)
    if cfg.routing == "zipf":
        # Popularity rank pi(e) from a seeded shuffle; logit = ln(1/(pi+1)) + Gumbel.
        # Top-k over these draws k experts without replacement with probability
        # proportional to 1/(pi+1) (Zipf exponent 1).
        pi = stream(cfg.seed, 8).permutation(cfg.E)
        gum = g.gumbel(size=(cfg.T, cfg.E))
        return (-np.log(pi + 1.0)[None, :] + gum).astype(np.float32)
    lg = g.standard_normal(size=(cfg.T, cfg.E), dtype=np.float64)
    if cfg.routing == "hot3":
        hot = stream(cfg.seed, 8).permutation(cfg.E)[:3]
        lg[:, hot] += HOT_BOOST
    return lg.astype(np.float32)


def activations(cfg: LayerConfig) -> np.ndarray:
    return to_bf16_bits(normal_f32(stream(cfg.seed, 1), (cfg.T, cfg.H)))


def fc_weights(cfg: LayerConfig, which: int):
    """which=1: FC1 (K=H, N=2I); which=2: FC2 (K=I, N=H). Returns (w, s, g)."""
    K, N = (cfg.H, 2 * cfg.I) if which == 1 else (cfg.I, cfg.H)
    base = 2 if which == 1 else 5
    if cfg.fmt == FP8:
        w = fp8_weight_bytes(stream(cfg.seed, base), (cfg.E, N, K))
        return w, None, global_scales(stream(cfg.seed, base + 2), cfg.E)
    w = packed_codes(stream(cfg.seed, base), (cfg.E, K, N // 2))
    if cfg.fmt == NVFP4:
        s = e4m3_scales(stream(cfg.seed, base + 1), (cfg.E, K // cfg.B, N), cfg.positive_scales)
        gs = global_scales(stream(cfg.seed, base + 2), cfg.E)
    else:
        s = e8m0_scales(stream(cfg.seed, base + 1), (cfg.E, K // cfg.B, N))
        gs = global_scales(stream(cfg.seed, base + 2), cfg.E) if cfg.mx_global else None
    return w, s, gs


def router_weights(cfg: LayerConfig) -> np.ndarray:
    """float32 [T][E] mixing weights for DeepSeek-style routing: sigmoid
    scores of their own normal draws, in (0, 1)."""
    z = stream(cfg.seed, 9).standard_normal(size=(cfg.T, cfg.E))
    return (1.0 / (1.0 + np.exp(-z))).astype(np.float32)


@dataclasses.dataclass
class LayerInputs:
    cfg: LayerConfig
    logits: np.ndarray
    x: np.ndarray
    w1: np.ndarray
    s1: np.ndarray
    g1: np.ndarray | None
    w2: np.ndarray
    s2: np.ndarray
    g2: np.ndarray | None


def layer_inputs(cfg: LayerConfig) -> LayerInputs:
    w1, s1, g1 = fc_weights(cfg, 1)
    w2, s2, g2 = fc_weights(cfg, 2)
    return LayerInputs(cfg, logits(cfg), activations(cfg), w1, s1, g1, w2, s2, g2)


def dequant_inputs(cfg: DequantConfig):
    w = packed_codes(stream(cfg.seed, 2), (cfg.E, cfg.K, cfg.N // 2))
    if cfg.fmt == MXFP4:
        s = e8m0_scales(stream(cfg.seed, 3), (cfg.E, cfg.K // cfg.B, cfg.N))
        gs = None
    else:
        s = e4m3_scales(stream(cfg.seed, 3), (cfg.E, cfg.K // cfg.B, cfg.N))
        gs = global_scales(stream(cfg.seed, 4), cfg.E)
    return w, s, gs


def with_rows(cfg: LayerConfig, T: int, name: str | None = None) -> LayerConfig:
    return dataclasses.replace(cfg, T=T, name=name or f"{cfg.name}_T{T}")


def shrink(cfg: LayerConfig, E: int | None = None, H: int | None = None, I: int | None = None,
           T: int | None = None, k: int | None = None, seed: int | None = None) -> LayerConfig:
    """A smaller layer with the same codec and value distributions."""
    c = dataclasses.replace(
        cfg, E=E or cfg.E, H=H or cfg.H, I=I or cfg.I, T=T or cfg.T, k=k or cfg.k,
        seed=cfg.seed if seed is None else seed)
    g = "_g" if c.mx_global else ""
    return dataclasses.replace(c, name=f"{cfg.fmt}{g}_T{c.T}_E{c.E}_top{c.k}_H{c.H}_I{c.I}_{c.routing}_s{c.seed}")

