"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module only draws and packs bytes; it holds none of the Q2_K decode or
product arithmetic, so the oracle and the HIP path stay independent.

Two families of inputs:

* The fixtures of the docs.rs source page of mlx-native 0.10.8,
  tests/deepseek_q2_k.rs: ``page_block(seed)`` restates fn block (scale byte
  per 16-weight group, code bytes from an affine sequence, d = 1/8 and
  dmin = 1/16 as f16) and ``page_input(rows)`` restates fn input (values
  ((17 i + 11) mod 97) / 48 - 1 in f32).
* The five synthetic workloads (``CONFIGS``): random blocks whose scale nibble
  is uniform on 1..15, min nibble uniform on 0..15, code bytes uniform, d = f16
  of U[0.01, 0.2] and dmin = f16 of U[0, 0.1]; f32 activations; u32 token ids.
  Each workload draws from numpy's PCG64 with seed 1000 + its index, in the
  fixed order scale nibbles, min nibbles, code bytes, d, dmin, activations, ids.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

QK_K = 256
BLOCK_BYTES = 84


def page_block(seed: int) -> np.ndarray:
    """fn block(seed): one 84-byte block of the page's fixture (u8 wrapping arithmetic)."""
    seed &= 0xFF
    out = np.empty(BLOCK_BYTES, dtype=np.uint8)
    for group in range(16):
        scale = ((group + seed) & 0xFF) % 15 + 1
        mn = 15 - ((((group * 3) & 0xFF) + seed) & 0xFF) % 16
        out[group] = (mn << 4) | scale
    for index in range(64):
        out[16 + index] = (((index * 73) & 0xFF) + ((seed * 19) & 0xFF)) & 0xFF
    out[80:82] = np.frombuffer(np.float16(0.125).tobytes(), dtype=np.uint8)
    out[82:84] = np.frombuffer(np.float16(0.0625).tobytes(), dtype=np.uint8)
    return out


def page_input(rows: int) -> np.ndarray:
    """fn input(rows): rows*256 f32 values ((17 i + 11) mod 97) / 48 - 1, computed in f32."""
    i = np.arange(rows * QK_K, dtype=np.int64)
    num = ((i * 17 + 11) % 97).astype(np.float32)
    return (num / np.float32(48.0) - np.float32(1.0)).astype(np.float32)


def pack_blocks(lo: np.ndarray, hi: np.ndarray, qs: np.ndarray, d: np.ndarray, dmin: np.ndarray) -> np.ndarray:
    """Pack per-block fields into 84-byte records: scales, codes, d (f16 LE), dmin (f16 LE)."""
    nb = lo.shape[0]
    out = np.empty((nb, BLOCK_BYTES), dtype=np.uint8)
    out[:, 0:16] = (hi.astype(np.uint8) << 4) | lo.astype(np.uint8)
    out[:, 16:80] = qs
    out[:, 80:82] = np.ascontiguousarray(d.astype("<f2")).view(np.uint8).reshape(nb, 2)
    out[:, 82:84] = np.ascontiguousarray(dmin.astype("<f2")).view(np.uint8).reshape(nb, 2)
    return out.reshape(-1)


def random_blocks(rng: np.random.Generator, nb: int) -> np.ndarray:
    """nb random blocks in the workload distribution, drawn in the fixed field order."""
    lo = rng.integers(1, 16, size=(nb, 16), dtype=np.uint8)
    hi = rng.integers(0, 16, size=(nb, 16), dtype=np.uint8)
    qs = rng.integers(0, 256, size=(nb, 64), dtype=np.uint8)
    d = rng.uniform(0.01, 0.2, nb).astype(np.float16)
    dmin = rng.uniform(0.0, 0.1, nb).astype(np.float16)
    return pack_blocks(lo, hi, qs, d, dmin)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    kind: str          # "matmul" or "gather"
    M: int = 0
    N: int = 0
    K: int = 0
    vocab: int = 0
    embed_dim: int = 0
    n_tokens: int = 0
    x_dist: str = "normal"   # "uniform" (U[-1,1]) or "normal" (N(0,1))
    bad_id_pos: int = -1     # gather: position of the out-of-range id in the bad-id run
    notes: str = ""

    @property
    def seed(self) -> int:
        return 1000 + self.index


CONFIGS = [
    Config(0, "tiny Q2_K matmul M=4 N=8 K=256 + dequant of its 8 blocks", "matmul",
           M=4, N=8, K=256, x_dist="uniform"),
    Config(1, "decode GEMV M=1 N=4096 K=4096", "matmul", M=1, N=4096, K=4096),
    Config(2, "Q2_K embedding gather vocab=262144 embed_dim=4096, 512 ids", "gather",
           vocab=262144, embed_dim=4096, n_tokens=512, bad_id_pos=257),
    Config(3, "batched mat-vec M=8 N=14336 K=4096", "matmul", M=8, N=14336, K=4096),
    Config(4, "prefill matmul M=512 N=14336 K=4096", "matmul", M=512, N=14336, K=4096),
]


@dataclass
class Inputs:
    config: Config
    blocks: np.ndarray                  # u8, whole weight matrix or table
    x: np.ndarray | None = None         # f32 [M, K]
    ids: np.ndarray | None = None       # u32 [n_tokens]
    hashes: dict = field(default_factory=dict)


def make_inputs(cfg: Config | int) -> Inputs:
    """Draw a workload's inputs from PCG64(1000 + index) in the fixed order."""
    if isinstance(cfg, int):
        cfg = CONFIGS[cfg]
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    if cfg.kind == "matmul":
        nb = cfg.N * (cfg.K // QK_K)
        blocks = random_blocks(rng, nb)
        if cfg.x_dist == "uniform":
            x = rng.uniform(-1.0, 1.0, (cfg.M, cfg.K)).astype(np.float32)
        else:
            x = rng.standard_normal((cfg.M, cfg.K), dtype=np.float32)
        inp = Inputs(cfg, blocks, x=x)
    else:
        nb = cfg.vocab * (cfg.embed_dim // QK_K)
        blocks = random_blocks(rng, nb)
        ids = rng.integers(0, cfg.vocab, cfg.n_tokens).astype(np.uint32)
        inp = Inputs(cfg, blocks, ids=ids)
    inp.hashes = {k: sha256(v) for k, v in (("blocks", inp.blocks), ("x", inp.x), ("ids", inp.ids))
                  if v is not None}
    return inp


def bad_ids(inp: Inputs) -> np.ndarray:
    """The gather workload's ids with one entry set to vocab (must be rejected)."""
    ids = inp.ids.copy()
    ids[inp.config.bad_id_pos] = inp.config.vocab
    return ids


def rows_of(blocks: np.ndarray, K: int, rows) -> np.ndarray:
    """Bytes of the selected weight rows (rows of K/256 consecutive blocks)."""
    rb = (K // QK_K) * BLOCK_BYTES
    b = blocks.reshape(-1, rb)
    return np.ascontiguousarray(b[np.asarray(rows)]).reshape(-1)


# --- Expert-routed (mm_id) inputs ------------------------------------------

def page_expert_weights(experts: int, n: int) -> np.ndarray:
    """fn run_expert's weights: row r of expert e is fn block(e * n + r + 1) (K = 256, one block per row)."""
    return np.concatenate([page_block(e * n + r + 1) for e in range(experts) for r in range(n)])


def page_routes(tokens: int, top_k: int, experts: int) -> np.ndarray:
    """fn run_expert's routing: route (token t, slot s) takes expert (3 t + s) mod experts; u32 [tokens*top_k]."""
    t = np.arange(tokens, dtype=np.int64)[:, None]
    s = np.arange(top_k, dtype=np.int64)[None, :]
    return ((3 * t + s) % experts).astype(np.uint32).reshape(-1)


def random_routes(rng: np.random.Generator, tokens: int, top_k: int, experts: int) -> np.ndarray:
    """Router-like ids: per token, top_k distinct experts drawn uniformly; u32 [tokens*top_k]."""
    if top_k > experts:
        return rng.integers(0, experts, tokens * top_k).astype(np.uint32)
    keys = rng.random((tokens, experts))
    return np.argsort(keys, axis=1)[:, :top_k].astype(np.uint32).reshape(-1)


@dataclass(frozen=True)
class MoeConfig:
    index: int
    name: str
    tokens: int
    top_k: int
    experts: int
    n: int
    K: int

    @property
    def seed(self) -> int:
        return 2000 + self.index

    @property
    def routes(self) -> int:
        return self.tokens * self.top_k


# The page's expert count and top_k (8 experts, top_k 6), with each expert the
# size of the dense workloads' weight matrix (14336 x 4096).
MOE_CONFIGS = [
    MoeConfig(0, "expert-routed decode: 1 token, top_k 6 of 8 experts, N=14336 K=4096", 1, 6, 8, 14336, 4096),
    MoeConfig(1, "expert-routed prefill: 512 tokens, top_k 6 of 8 experts, N=14336 K=4096", 512, 6, 8, 14336, 4096),
]


@dataclass
class MoeInputs:
    config: MoeConfig
    blocks: np.ndarray   # u8, experts x n rows x K/256 blocks, expert stride n * K/256 * 84
    x: np.ndarray        # f32 [tokens, K]
    ids: np.ndarray      # u32 [tokens * top_k]


def make_moe_inputs(cfg: MoeConfig | int) -> MoeInputs:
    """Draw an expert-routed workload from PCG64(2000 + index): blocks, activations N(0,1), routes."""
    if isinstance(cfg, int):
        cfg = MOE_CONFIGS[cfg]
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    blocks = random_blocks(rng, cfg.experts * cfg.n * (cfg.K // QK_K))
    x = rng.standard_normal((cfg.tokens, cfg.K), dtype=np.float32)
    ids = random_routes(rng, cfg.tokens, cfg.top_k, cfg.experts)
    return MoeInputs(cfg, blocks, x, ids)
