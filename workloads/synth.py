"""Seeded generators and workload shapes (no method arithmetic here).

Every array is drawn from ``numpy.random.default_rng``.  Small single-matrix
cases draw from one stream in a fixed order; multi-matrix fields give each
purpose (codes, scales, activations, coordinates, lenses, scores) and each
matrix its own stream, keyed ``default_rng([seed, tag, index])``, so any one
matrix can be regenerated without drawing the others.

Distributions (the workloads' stated recipe):
  * int8 codes uniform in [-127, 127]            ``integers(-127, 128)``
  * per-row fp32 scales ~ U(0.001, 0.02)          ``uniform``
  * activations fp32 ~ N(0, 1)                     ``standard_normal``
  * block coordinates fp64 on the unit square, uniform or clustered
    (8 Gaussian clusters, sigma 0.05, not clipped)
  * lens centres at the coordinates of distinct, uniformly chosen blocks;
    lens sizes r uniform in a stated range
  * escalation uncertainty scores ~ Beta(2, 5)
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np

ROWS_PER_BLOCK = 64

# stream tags for multi-matrix workloads
TAG_CODES, TAG_SCALES, TAG_X, TAG_COORDS, TAG_LENSES, TAG_SCORES, TAG_REQ_LENSES, TAG_EMBED = range(1, 9)


def stream(seed: int, tag: int, index: int = 0) -> np.random.Generator:
    """Independent generator for one purpose / one matrix."""
    return np.random.default_rng([int(seed), int(tag), int(index)])


# --------------------------------------------------------------------------
# elementary draws
# --------------------------------------------------------------------------

def int8_codes(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    return rng.integers(-127, 128, size=(N, K), dtype=np.int8)


def row_scales(rng: np.random.Generator, N: int) -> np.ndarray:
    return rng.uniform(0.001, 0.02, size=N).astype(np.float32)


def activations(rng: np.random.Generator, B: int, K: int) -> np.ndarray:
    return rng.standard_normal((B, K)).astype(np.float32)


def uniform_coords(rng: np.random.Generator, n_blocks: int) -> np.ndarray:
    return rng.uniform(0.0, 1.0, size=(n_blocks, 2))


def clustered_coords(rng: np.random.Generator, n_blocks: int, n_clusters: int = 8,
                     sigma: float = 0.05) -> np.ndarray:
    centres = rng.uniform(0.0, 1.0, size=(n_clusters, 2))
    label = rng.integers(0, n_clusters, size=n_blocks)
    return centres[label] + rng.normal(0.0, sigma, size=(n_blocks, 2))


def lens_set(rng: np.random.Generator, coords: np.ndarray, n_lenses: int,
             r_lo: float, r_hi: float) -> Tuple[np.ndarray, np.ndarray]:
    """Lens centres at distinct random blocks, sizes r ~ U[r_lo, r_hi]."""
    idx = rng.choice(coords.shape[0], size=n_lenses, replace=False)
    centres = coords[idx].copy()
    if r_lo == r_hi:
        radii = np.full(n_lenses, float(r_lo))
    else:
        radii = rng.uniform(r_lo, r_hi, size=n_lenses)
    return centres, radii


def escalation_scores(seed: int, n_steps: int) -> np.ndarray:
    return stream(seed, TAG_SCORES).beta(2.0, 5.0, size=n_steps)


# --------------------------------------------------------------------------
# workload descriptions
# --------------------------------------------------------------------------

@dataclass
class LensParams:
    """The three controls plus the lens list (plain data)."""
    centres: np.ndarray            # [n_lenses, 2] fp64
    radii: np.ndarray              # [n_lenses] fp64
    f: float = 0.5                 # focus_area
    g: float = 0.75                # focus_strength
    combine: str = "sum"           # 'sum' or 'max'
    glass: int = 1                 # rung index of the glass (1 = D2)
    n_rungs: int = 5               # ZERO, D2, D4, D6, D8
    stops: object = None          # None = default spacing


@dataclass
class Matrix:
    name: str
    N: int
    K: int
    index: int                     # position in the field (stream index)

    @property
    def n_blocks(self) -> int:
        return self.N // ROWS_PER_BLOCK


@dataclass
class Field:
    """A set of matrices with one global block order (matrix order, then
    row block) and one 2-D coordinate per block."""
    name: str
    seed: int
    matrices: List[Matrix]
    coords: np.ndarray = field(default=None)

    @property
    def n_blocks(self) -> int:
        return sum(m.n_blocks for m in self.matrices)

    @property
    def n_weights(self) -> int:
        return sum(m.N * m.K for m in self.matrices)

    def block_offsets(self) -> List[int]:
        out, o = [], 0
        for m in self.matrices:
            out.append(o)
            o += m.n_blocks
        return out

    def block_weights(self) -> np.ndarray:
        """w_b = 64 * K_b for every block, in field order (int64)."""
        return np.concatenate([np.full(m.n_blocks, ROWS_PER_BLOCK * m.K, dtype=np.int64)
                               for m in self.matrices])

    def codes(self, i: int) -> np.ndarray:
        m = self.matrices[i]
        return int8_codes(stream(self.seed, TAG_CODES, m.index), m.N, m.K)

    def scales(self, i: int) -> np.ndarray:
        m = self.matrices[i]
        return row_scales(stream(self.seed, TAG_SCALES, m.index), m.N)

    def x(self, i: int, B: int = 1) -> np.ndarray:
        m = self.matrices[i]
        return activations(stream(self.seed, TAG_X, m.index), B, m.K)


# ---- workload 1: single 512x256 layer, 8 blocks -------------------------

def single_layer_512x256(seed: int = 0):
    """W int8 512x256 (8 blocks of 64 rows), codes U[-127,127], scales
    U(0.001, 0.02), x ~ N(0,1) batch 1, block coords U[0,1]^2, 2 lenses
    (r = 0.2, f = 0.5, g = 0.75, sum), glass D2, ladder ZERO..D8.
    One stream, drawn in this order: codes, scales, x, coords, lens centres."""
    rng = np.random.default_rng(seed)
    W = int8_codes(rng, 512, 256)
    scales = row_scales(rng, 512)
    x = activations(rng, 1, 256)
    coords = uniform_coords(rng, 8)
    centres, radii = lens_set(rng, coords, 2, 0.2, 0.2)
    lp = LensParams(centres=centres, radii=radii, f=0.5, g=0.75, combine="sum", glass=1)
    return dict(W=W, scales=scales, x=x, coords=coords, lens=lp)


# ---- workload 2: Gemma-E2B-scale weight field ---------------------------

E2B_LAYER = (("q", 1536, 1536), ("k", 1536, 1536), ("v", 1536, 1536), ("o", 1536, 1536),
             ("gate", 6144, 1536), ("up", 6144, 1536), ("down", 1536, 6144))


def e2b_field(seed: int = 0, n_layers: int = 30) -> Field:
    """30 synthetic decoder layers (q/k/v/o 1536x1536, gate/up 6144x1536,
    down 1536x6144), int8 with per-row scales; block coords clustered
    (8 Gaussian clusters, sigma = 0.05); independent x per matrix."""
    mats, i = [], 0
    for layer in range(n_layers):
        for name, N, K in E2B_LAYER:
            mats.append(Matrix(f"L{layer}.{name}", N, K, i))
            i += 1
    fld = Field("e2b_field", seed, mats)
    fld.coords = clustered_coords(stream(seed, TAG_COORDS), fld.n_blocks)
    return fld


def e2b_lenses(fld: Field, n_lenses: int = 5, f: float = 0.5, g: float = 0.75) -> LensParams:
    centres, radii = lens_set(stream(fld.seed, TAG_LENSES), fld.coords, n_lenses, 0.05, 0.3)
    return LensParams(centres=centres, radii=radii, f=f, g=g, combine="sum", glass=1)


# ---- workload 3: Qwen3-0.6B-shaped decode -------------------------------

QWEN_HIDDEN = 1024
QWEN_LAYER = (("q", 2048, 1024), ("k", 1024, 1024), ("v", 1024, 1024), ("o", 1024, 2048),
              ("gate", 3072, 1024), ("up", 3072, 1024), ("down", 1024, 3072))
QWEN_VOCAB = 151936


def decoder_field(seed: int, n_layers: int, hidden: int, q_dim: int, kv_dim: int, ffn: int, vocab: int,
                  name: str = "decoder") -> Field:
    """Matrices of a decoder-only model, per layer q [q_dim, hidden],
    k and v [kv_dim, hidden], o [hidden, q_dim], gate and up [ffn, hidden],
    down [hidden, ffn], then a [vocab, hidden] head; int8 codes."""
    shapes = (("q", q_dim, hidden), ("k", kv_dim, hidden), ("v", kv_dim, hidden), ("o", hidden, q_dim),
              ("gate", ffn, hidden), ("up", ffn, hidden), ("down", hidden, ffn))
    mats, i = [], 0
    for layer in range(n_layers):
        for nm, N, K in shapes:
            mats.append(Matrix(f"L{layer}.{nm}", N, K, i))
            i += 1
    mats.append(Matrix("lm_head", vocab, hidden, i))
    return Field(name, seed, mats)


def qwen_decode_field(seed: int = 0, n_layers: int = 28) -> Field:
    """28 layers (hidden 1024; 16 Q heads / 8 KV heads of dim 128; FFN 3072)
    plus the tied 151936x1024 head, int8 weights."""
    return decoder_field(seed, n_layers, QWEN_HIDDEN, 2048, 1024, 3072, QWEN_VOCAB, "qwen_decode")


def embedding_table(seed: int, vocab: int, hidden: int) -> np.ndarray:
    """Token-feedback stand-in: one N(0, 1) fp32 row per token, [vocab, hidden]."""
    return stream(seed, TAG_EMBED).standard_normal((vocab, hidden), dtype=np.float32)


def decode_inputs(seed: int, n_steps: int, hidden: int = QWEN_HIDDEN) -> np.ndarray:
    """x0 ~ N(0, 1) per step, [n_steps, hidden] fp32."""
    return activations(stream(seed, TAG_X, 10_000), n_steps, hidden)


# ---- workload 4: batched per-request GEMM -------------------------------

def batched_layer(seed: int = 0) -> Field:
    """One layer: 4096x4096, 14336x4096 and 4096x14336 int8; coords U[0,1]^2."""
    mats = [Matrix("attn", 4096, 4096, 0), Matrix("up", 14336, 4096, 1),
            Matrix("down", 4096, 14336, 2)]
    fld = Field("batched_layer", seed, mats)
    fld.coords = uniform_coords(stream(seed, TAG_COORDS), fld.n_blocks)
    return fld


def request_lenses(fld: Field, B: int, n_lenses: int = 3):
    """Per request: 3 lenses, r ~ U[0.05, 0.3], centres at random blocks."""
    return [lens_set(stream(fld.seed, TAG_REQ_LENSES, r), fld.coords, n_lenses, 0.05, 0.3)
            for r in range(B)]


# ---- workload 5: large streaming layer stack ----------------------------

def streaming_stack(seed: int = 0, n_layers: int = 8) -> Field:
    """8 layers of 8192x28672 and 28672x8192 int8 (~3.8 GB at 8 bits);
    coords U[0,1]^2."""
    mats, i = [], 0
    for layer in range(n_layers):
        mats.append(Matrix(f"L{layer}.down", 8192, 28672, i))
        mats.append(Matrix(f"L{layer}.up", 28672, 8192, i + 1))
        i += 2
    fld = Field("streaming_stack", seed, mats)
    fld.coords = uniform_coords(stream(seed, TAG_COORDS), fld.n_blocks)
    return fld


def stack_lenses(fld: Field, n_lenses: int = 4) -> Tuple[np.ndarray, np.ndarray]:
    return lens_set(stream(fld.seed, TAG_LENSES), fld.coords, n_lenses, 0.05, 0.3)
