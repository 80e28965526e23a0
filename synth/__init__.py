"""Seeded synthetic inputs of the verify-window MoE layer.

This module only draws random numbers and encodes them in the documented storage
formats (binary16, bfloat16, packed codes). It holds none of the layer's arithmetic,
and both the HIP path's tests/benchmark and the CPU oracle take their inputs from it.

The pages measure whole models whose weights and prompts are not available (Strata
docs/BATCHING.md, "Measured": UD-Q4_K_XL, Q2_0, IQ3_S models and the benchmark's own
prompts). These generators stand in for them with the shapes of five workloads:

  name                 hidden  ffn   experts  top_k  bits  rows        activations
  small_f32            256     128   16       2      4     2           float32, independent
  two_slots_mtp        2048    768   128      8      4     4           bf16, independent, uniform routing
  four_slots_mtp_zipf  2048    768   128      8      4     8           bf16, 4 (token, proposal) pairs with
                                                                       cosine ~0.9, Zipf(1.1) router prior
  stack24_head         24 layers of two_slots_mtp's shape, 8 rows, then an 8-bit head of vocab 151936
  e256_2bit            4096    1024  256      8      2     1, 2, 4, 8  bf16, independent, uniform routing

Each workload's `seed` keys its random streams.

Value recipe (not from the pages; chosen so activations stay O(1) through 24 layers and
the dequantised weights are exact in float32):
  codes:  uniform over all codes (random bytes for 2/4-bit; int8 uniform in [-127, 127])
  scale:  binary16( g * U(0.75, 1.25) / (sigma_q * sqrt(cols)) ), sigma_q = std of the code,
          g = 1, except g = 1/4 for the down projections of the 24-layer stack: every
          matrix then has unit gain, and the layer's output grows with the square of its
          input (silu(gate x) * up x), so with g = 1 a stack whose x_next feeds the next
          layer overflows float32 by layer 10; with 1/4 the stream's rms goes 1.0 -> 1.6
          over 24 layers (the models on the pages normalise each layer's input; that
          dense part is outside this layer)
  min:    binary16( -scale * (2^bits - 1) / 2 )      (affine formats only)
  router: float32 N(0, 0.02);  bias (Zipf workloads): -1.1 * ln(rank_e), rank a random permutation
  x:      N(0, 1); paired workloads' rows (2s, 2s+1): x_p = 0.9 x_t + sqrt(0.19) z; then bf16 (RNE)
"""
from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Config:
    name: str
    seed: int
    hidden: int
    ffn: int
    experts: int
    top_k: int
    bits: int
    rows: int
    x_dtype: str          # "f32" or "bf16"
    zipf: bool = False
    pairs: bool = False
    layers: int = 1
    vocab: int = 0
    head_bits: int = 8


CONFIGS = {c.name: c for c in (
    Config("small_f32", 0, 256, 128, 16, 2, 4, 2, "f32"),
    Config("two_slots_mtp", 1, 2048, 768, 128, 8, 4, 4, "bf16"),
    Config("four_slots_mtp_zipf", 2, 2048, 768, 128, 8, 4, 8, "bf16", zipf=True, pairs=True),
    Config("stack24_head", 3, 2048, 768, 128, 8, 4, 8, "bf16", layers=24, vocab=151936),
    Config("e256_2bit", 4, 4096, 1024, 256, 8, 2, 8, "bf16"),
)}
E256_ROWS = (1, 2, 4, 8)


def config(name, **over):
    c = CONFIGS[name]
    return replace(c, **over) if over else c


def _rng(*key):
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def f32_to_bf16_bits(a):
    """bfloat16 bit patterns of float32 values, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _code_std(bits):
    if bits == 8:      # uniform integers in [-127, 127]
        return float(np.sqrt(127 * 128 / 3.0))
    n = 1 << bits      # uniform integers in [0, n)
    return float(np.sqrt((n * n - 1) / 12.0))


def qmatrix(rng, n_mat, rows, cols, bits, gain=1.0):
    """Random quantized matrices: codes uint8 [n_mat, rows*cols*bits/8] and meta
    ([n_mat, rows*cols/32], uint32 scale|min<<16 for 2/4-bit, uint16 scale for 8-bit).
    Every code and every block's (scale, min) is drawn independently, so the arrays do
    not depend on where the layout puts each weight. gain multiplies every scale."""
    assert rows % 16 == 0 and cols % (512 // bits) == 0
    nbytes = rows * cols * bits // 8
    nblk = rows * cols // 32
    codes = rng.integers(0, 256, size=(n_mat, nbytes), dtype=np.uint8)
    if bits == 8:  # int8 uniform over [-127, 127]: redraw every -128
        bad = np.flatnonzero(codes == 0x80)
        while bad.size:
            codes.flat[bad] = rng.integers(0, 256, size=bad.size, dtype=np.uint8)
            bad = bad[codes.flat[bad] == 0x80]
    scale = (gain * rng.uniform(0.75, 1.25, size=(n_mat, nblk)) / (_code_std(bits) * np.sqrt(cols))).astype(np.float16)
    if bits == 8:
        return codes, scale.view(np.uint16)
    mn = (-scale.astype(np.float64) * ((1 << bits) - 1) / 2.0).astype(np.float16)
    meta = scale.view(np.uint16).astype(np.uint32) | (mn.view(np.uint16).astype(np.uint32) << 16)
    return codes, meta


@dataclass
class Layer:
    gate_w: np.ndarray        # [E, H] float32
    bias: object              # [E] float32 or None
    gate: tuple               # (codes [E, ...], meta [E, ...]) of [F, H] matrices
    up: tuple
    down: tuple               # [H, F] matrices
    sh_gate: tuple            # (codes [1, ...], meta [1, ...])
    sh_up: tuple
    sh_down: tuple


def make_router(cfg, layer=0):
    """Router of layer instance `layer`: (gate_w [E, H] float32, bias [E] float32 or None)."""
    E, H = cfg.experts, cfg.hidden
    gate_w = _rng(cfg.seed, 1, layer, 0).normal(0.0, 0.02, size=(E, H)).astype(np.float32)
    bias = None
    if cfg.zipf:
        rank = _rng(cfg.seed, 1, layer, 3).permutation(E) + 1
        bias = (-1.1 * np.log(rank)).astype(np.float32)
    return gate_w, bias


def make_layer(cfg, layer=0):
    """Weights of MoE layer instance `layer` of configuration `cfg`."""
    E, H, F, b = cfg.experts, cfg.hidden, cfg.ffn, cfg.bits
    gate_w, bias = make_router(cfg, layer)
    r_exp, r_sh = _rng(cfg.seed, 1, layer, 1), _rng(cfg.seed, 1, layer, 2)
    g_down = 0.25 if cfg.layers > 1 else 1.0   # the stack's down gain (module docstring)
    gate = qmatrix(r_exp, E, F, H, b)
    up = qmatrix(r_exp, E, F, H, b)
    down = qmatrix(r_exp, E, H, F, b, g_down)
    sh_gate = qmatrix(r_sh, 1, F, H, b)
    sh_up = qmatrix(r_sh, 1, F, H, b)
    sh_down = qmatrix(r_sh, 1, H, F, b, g_down)
    return Layer(gate_w, bias, gate, up, down, sh_gate, sh_up, sh_down)


def make_head(cfg):
    """8-bit head [vocab, hidden]: (codes [1, ...], meta [1, ...])."""
    return qmatrix(_rng(cfg.seed, 2), 1, cfg.vocab, cfg.hidden, cfg.head_bits)


def make_window(cfg, window=0, rows=None):
    """Activations of one window: float32 [R, H] (x_dtype f32) or bf16 bits uint16."""
    R = cfg.rows if rows is None else rows
    rng = _rng(cfg.seed, 3, window)
    x = rng.standard_normal((R, cfg.hidden))
    if cfg.pairs:
        for s in range(R // 2):
            z = rng.standard_normal(cfg.hidden)
            x[2 * s + 1] = 0.9 * x[2 * s] + np.sqrt(0.19) * z
    x = x.astype(np.float32)
    return x if cfg.x_dtype == "f32" else f32_to_bf16_bits(x)
