"""Counter-based seeded generators (no attention arithmetic here).

Every value is a pure function of (seed, tensor_id, index), so a tensor is the
same whatever chunking, thread count or machine produced it.

* ``uniform_u64``: the splitmix64 output function (Steele, Lea and Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014) applied to a
  Weyl sequence keyed by (seed, tensor_id).
* ``normal_bf16``: the Box-Muller transform (Box and Muller, 1958) on two such
  uniforms per element (cosine branch only), in float64, rounded to float32 and
  then to bfloat16 with round-to-nearest-even.

Tensor ids: Q = 1, K = 2, V = 3, outlier channels = 4, policies = 5, decode q = 6.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

TID_Q, TID_K, TID_V, TID_OUTLIER, TID_POLICY, TID_DECODE_Q = 1, 2, 3, 4, 5, 6
TID_BLOCK_MAG, TID_GAMMA = 7, 8


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _key(seed: int, tid: int) -> np.uint64:
    with np.errstate(over="ignore"):
        base = np.array([(seed * GOLDEN + tid) & MASK64], dtype=np.uint64)
        return _mix64(base)[0]


def uniform_u64(seed: int, tid: int, start: int, count: int) -> np.ndarray:
    """64-bit outputs number start .. start+count-1 of stream (seed, tid)."""
    key = _key(seed, tid)
    ctr = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64(key + ctr * np.uint64(GOLDEN))


def _open_unit(u: np.ndarray) -> np.ndarray:
    # 53-bit mantissa, shifted half a step off zero so log() is finite
    return ((u >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def float32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); finite inputs only."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return b.astype(np.uint16)


def bf16_bits_to_float32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(seed: int, tid: int, count: int, chunk: int = 1 << 22,
                scale_channels: Optional[np.ndarray] = None, row_len: int = 0,
                channel_factor: float = 8.0) -> np.ndarray:
    """``count`` N(0,1) samples as bf16 bit patterns (uint16).

    If ``scale_channels`` is given, elements whose index modulo ``row_len`` is in
    it are multiplied by ``channel_factor`` in float32 before the bf16 rounding
    (the outlier key channels of the Llama-shaped workloads).
    """
    out = np.empty(count, dtype=np.uint16)

    def one(s: int) -> None:
        c = min(chunk, count - s)
        u = uniform_u64(seed, tid, 2 * s, 2 * c)
        u1 = _open_unit(u[0::2])
        u2 = _open_unit(u[1::2])
        z = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
        f = z.astype(np.float32)
        if scale_channels is not None and len(scale_channels):
            col = (np.arange(s, s + c, dtype=np.int64) % row_len)
            sel = np.isin(col, scale_channels)
            f[sel] *= np.float32(channel_factor)
        out[s:s + c] = float32_to_bf16_bits(f)

    starts = list(range(0, count, chunk))
    if len(starts) <= 1:
        for s in starts:
            one(s)
    else:
        # numpy ufuncs release the GIL; chunks are independent (counter-based)
        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(one, starts))
    return out


def outlier_channels(seed: int, d: int, count: int = 4) -> np.ndarray:
    """``count`` distinct channel indices in [0, d), drawn in order from stream 4."""
    chosen: list[int] = []
    i = 0
    while len(chosen) < count:
        c = int(uniform_u64(seed, TID_OUTLIER, i, 1)[0] % np.uint64(d))
        i += 1
        if c not in chosen:
            chosen.append(c)
    return np.array(chosen, dtype=np.int64)


def _uint(seed: int, tid: int, i: int, lo: int, hi: int) -> int:
    """Integer uniform on [lo, hi] inclusive (modulo reduction; bias < 2^-50)."""
    u = int(uniform_u64(seed, tid, i, 1)[0])
    return lo + u % (hi - lo + 1)


def policy_draws(seed: int, n_heads: int, hi_range: tuple[int, int], keep_max: int) -> tuple[np.ndarray, np.ndarray]:
    """Per-head (hi, keep): hi ~ U[hi_range], then keep ~ U[hi, keep_max]."""
    hi = np.zeros(n_heads, dtype=np.int32)
    keep = np.zeros(n_heads, dtype=np.int32)
    for h in range(n_heads):
        hi[h] = _uint(seed, TID_POLICY, 2 * h, hi_range[0], hi_range[1])
        keep[h] = _uint(seed, TID_POLICY, 2 * h + 1, int(hi[h]), keep_max)
    return hi, keep


@dataclass
class Config:
    """One synthetic workload: shapes, the policy recipe and the seed."""
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seq_len: int
    block: int
    seed: int
    outliers: bool = False
    hi_range: tuple[int, int] = (0, 0)
    keep_max: int = 0
    fixed: dict = field(default_factory=dict)   # head -> (hi, keep) overrides
    decode: bool = False                        # policies per KV head, one query token

    @property
    def nb(self) -> int:
        return (self.seq_len + self.block - 1) // self.block

    def policy(self) -> tuple[np.ndarray, np.ndarray]:
        n = self.n_kv_heads if self.decode else self.n_q_heads
        hi, keep = policy_draws(self.seed, n, self.hi_range, self.keep_max)
        for h, (a, b) in self.fixed.items():
            hi[h], keep[h] = a, b
        return hi, keep

    def scaled(self, **kw) -> "Config":
        d = dict(self.__dict__)
        d.update(kw)
        return Config(**d)


# The five synthetic workloads by name: shapes, policy recipes and seeds.
CONFIGS = {
    "tiny": Config("tiny-prefill b1 h2/1 d64 n512 B64", 1, 2, 1, 64, 512, 64, seed=1,
              hi_range=(2, 2), keep_max=4, fixed={0: (2, 4), 1: (2, 4)}),
    "llama3_8b_layer": Config("llama3-8b-layer-prefill b1 h32/8 d128 n8192 B128", 1, 32, 8, 128, 8192, 128, seed=2,
              outliers=True, hi_range=(1, 8), keep_max=64),
    "long_prefill": Config("long-prefill b1 h32/8 d128 n65536 B128", 1, 32, 8, 128, 65536, 128, seed=3,
              outliers=True, hi_range=(2, 16), keep_max=128),
    "decode_b16": Config("decode b16 h32/8 d128 ctx32768 B128", 16, 32, 8, 128, 32768, 128, seed=4,
              hi_range=(2, 16), keep_max=128, decode=True),
    "batched_mixed": Config("batched-mixed-prefill b4 h28/4 d128 n16384 B128", 4, 28, 4, 128, 16384, 128, seed=5,
              hi_range=(0, 127), keep_max=127, fixed={0: (127, 127), 1: (0, 0), 2: (0, 127)}),
}


def make_prefill_inputs(cfg: Config):
    """Q [b][Hq][n][d], K, V [b][Hkv][n][d] as bf16 bit arrays (uint16), BHSD."""
    b, hq, hk, d, n = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.seq_len
    ch = outlier_channels(cfg.seed, d) if cfg.outliers else None
    q = normal_bf16(cfg.seed, TID_Q, b * hq * n * d).reshape(b, hq, n, d)
    k = normal_bf16(cfg.seed, TID_K, b * hk * n * d, scale_channels=ch, row_len=d).reshape(b, hk, n, d)
    v = normal_bf16(cfg.seed, TID_V, b * hk * n * d).reshape(b, hk, n, d)
    return q, k, v


def make_decode_inputs(cfg: Config):
    """K, V [b][Hkv][ctx][d] and the query q [b][Hq][d], bf16 bits."""
    b, hq, hk, d, n = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.seq_len
    ch = outlier_channels(cfg.seed, d) if cfg.outliers else None
    k = normal_bf16(cfg.seed, TID_K, b * hk * n * d, scale_channels=ch, row_len=d).reshape(b, hk, n, d)
    v = normal_bf16(cfg.seed, TID_V, b * hk * n * d).reshape(b, hk, n, d)
    q = normal_bf16(cfg.seed, TID_DECODE_Q, b * hq * d).reshape(b, hq, d)
    return k, v, q


def make_skip_decode_inputs(cfg: Config, mag_range: tuple[float, float] = (0.1, 1.0),
                            gamma_range: tuple[float, float] = (0.6, 0.9)):
    """Decode inputs with block structure, for dynamic block skipping.

    K [b][Hkv][ctx][d]: N(0,1) rows times one magnitude per (b, KV head, block),
    uniform on mag_range (stream 7); V and q as make_decode_inputs.  thresholds
    [b][Hq] (fp32, logit units): gamma * ||q_bh||_2 with gamma uniform on
    gamma_range per (b, h) (stream 8) -- with sm_scale = 1/sqrt(d) a block of
    magnitude m has scores of order m * ||q|| * |cos|, so gamma sets how many blocks
    a head keeps (a stand-in for a learned per-head, per-query threshold).
    Returns k, v, q (bf16 bits) and thresholds.
    """
    k, v, q = make_decode_inputs(cfg)
    k, thresholds = apply_block_structure(cfg, k, q, mag_range, gamma_range)
    return k, v, q, thresholds


def apply_block_structure(cfg: Config, k: np.ndarray, q: np.ndarray, mag_range: tuple[float, float] = (0.1, 1.0),
                          gamma_range: tuple[float, float] = (0.6, 0.9)):
    """The block magnitudes and thresholds of make_skip_decode_inputs, applied to
    existing decode inputs k [b][Hkv][ctx][d] and q [b][Hq][d] (bf16 bits)."""
    b, hq, hk, d, n, blk = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.seq_len, cfg.block
    nb = (n + blk - 1) // blk
    u = _open_unit(uniform_u64(cfg.seed, TID_BLOCK_MAG, 0, b * hk * nb)).reshape(b, hk, nb)
    mag = (mag_range[0] + (mag_range[1] - mag_range[0]) * u).astype(np.float32)
    kf = bf16_bits_to_float32(k).reshape(b, hk, n, d)
    scale = np.repeat(mag, blk, axis=2)[:, :, :n, None]
    k = float32_to_bf16_bits(kf * scale).reshape(b, hk, n, d)
    g = _open_unit(uniform_u64(cfg.seed, TID_GAMMA, 0, b * hq)).reshape(b, hq)
    gamma = gamma_range[0] + (gamma_range[1] - gamma_range[0]) * g
    qn = np.sqrt((bf16_bits_to_float32(q).astype(np.float64) ** 2).sum(axis=-1))
    thresholds = (gamma * qn).astype(np.float32)
    return k, thresholds
