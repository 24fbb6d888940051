"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module holds no attention arithmetic. It draws the workloads'
tensors (iid standard-normal Q, K, V), rounds them to bfloat16 when a
workload is bf16, and draws the 128x128 block masks of the block-sparse
workload. Both sides receive exactly the same values: the HIP path gets
the raw bf16 bit patterns (or fp32 values), the oracle gets the same
numbers as float32 arrays (every bf16 value is exactly representable in
float32).

The workloads stand in for the pages' own, which are not available here:
the HCMS page (HCMS: Head-Chunked Multi-Stream Pipeline ..., Abstract)
measures video-generation sequences of 31K-56K tokens on Wan2.2, and the
db-SP page (db-SP: Accelerating Sparse Attention for Visual Generative
Models ..., Abstract) uses block-sparse DiT attention masks. Neither the
model activations nor the masks exist in this repository, so seeded iid
N(0,1) tensors of the same shapes and seeded masks with per-head density
drawn from U[0.1, 0.6) are used instead.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# Fixed root of every seed sequence; recorded in bench output.
ROOT_SEED = 0x15A7_2026

# Stream ids inside one workload's seed sequence.
_STREAM_Q, _STREAM_K, _STREAM_V, _STREAM_MASK, _STREAM_DO = 0, 1, 2, 3, 4

MASK_BLOCK = 128  # block edge of the block-sparse mask, in tokens


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one workload. All tensors are [B, S, H, D], D contiguous."""
    wid: int
    name: str
    dtype: str          # "f32" or "bf16"
    B: int
    Sq: int
    Skv: int
    H: int
    D: int
    kv_blocks: int = 1            # ring partials: number of equal KV blocks
    head_chunks: tuple = ()       # head-chunked pipeline: chunk sizes
    sparse: bool = False          # block-sparse mask
    density: tuple = (0.1, 0.6)   # per-head mask density range

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


# The workloads measured and checked by this repository (1-5: forward;
# 6: the backward of the dense forward at the chunked workload's shape).
WORKLOADS = {
    1: Workload(1, "dense_f32_B4_S128_H32_D128", "f32", 4, 128, 128, 32, 128),
    2: Workload(2, "ring_partials_bf16_Sq4096_Skv32768_H8_D128", "bf16",
                1, 4096, 32768, 8, 128, kv_blocks=8),
    3: Workload(3, "chunked_bf16_S32760_H40_D128_chunks16_12_12", "bf16",
                1, 32760, 32760, 40, 128, head_chunks=(16, 12, 12)),
    4: Workload(4, "dense_bf16_S56160_H40_D128", "bf16",
                1, 56160, 56160, 40, 128),
    5: Workload(5, "blocksparse_bf16_S32768_H40_D128_mask128", "bf16",
                1, 32768, 32768, 40, 128, sparse=True),
    6: Workload(6, "attn_bwd_bf16_S32760_H40_D128", "bf16", 1, 32760, 32760, 40, 128),
}


def rng_for(wid: int, stream: int, seed: int = 0) -> np.random.Generator:
    """Independent generator per (workload id, tensor stream, user seed)."""
    return np.random.default_rng(
        np.random.SeedSequence([ROOT_SEED, int(wid), int(stream), int(seed)]))


def standard_normal_f32(shape, wid: int, stream: int, seed: int = 0) -> np.ndarray:
    return rng_for(wid, stream, seed).standard_normal(shape, dtype=np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, ties to even; returns uint16 bits.

    Inputs must be finite (the generators only produce finite values).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 values of bfloat16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Tensor:
    """One input tensor: exact values (float32) plus what the GPU receives."""
    values: np.ndarray            # float32, exact values the GPU computes on
    bits: np.ndarray | None       # uint16 bf16 bits, or None for fp32 tensors

    @property
    def device_array(self) -> np.ndarray:
        return self.bits if self.bits is not None else self.values


def make_tensor(shape, dtype: str, wid: int, stream: int, seed: int = 0) -> Tensor:
    x = standard_normal_f32(shape, wid, stream, seed)
    if dtype == "f32":
        return Tensor(x, None)
    if dtype != "bf16":
        raise ValueError(f"unknown dtype {dtype!r}")
    b = bf16_bits(x)
    del x
    return Tensor(bf16_bits_to_f32(b), b)


def make_qkv(w: Workload, seed: int = 0, Sq: int | None = None, Skv: int | None = None):
    """Q [B,Sq,H,D], K and V [B,Skv,H,D] for workload ``w``.

    ``Sq``/``Skv`` override the workload's lengths (used by small parity
    cases that keep a workload's dtype and head shape).
    """
    Sq = w.Sq if Sq is None else Sq
    Skv = w.Skv if Skv is None else Skv
    q = make_tensor((w.B, Sq, w.H, w.D), w.dtype, w.wid, _STREAM_Q, seed)
    k = make_tensor((w.B, Skv, w.H, w.D), w.dtype, w.wid, _STREAM_K, seed)
    v = make_tensor((w.B, Skv, w.H, w.D), w.dtype, w.wid, _STREAM_V, seed)
    return q, k, v


def make_dout(w: Workload, seed: int = 0, Sq: int | None = None) -> Tensor:
    """Upstream gradient dO [B, Sq, H, D] of workload ``w`` (iid N(0, 1),
    rounded to the workload's dtype), from its own seed stream."""
    Sq = w.Sq if Sq is None else Sq
    return make_tensor((w.B, Sq, w.H, w.D), w.dtype, w.wid, _STREAM_DO, seed)


def make_custom_dout(shape_q, dtype: str, seed: int, wid: int = 99) -> Tensor:
    """dO for the arbitrary-shape cases of make_custom."""
    return make_tensor(shape_q, dtype, wid, _STREAM_DO, seed)


def make_custom(shape_q, shape_kv, dtype: str, seed: int, wid: int = 99):
    """Q, K, V with arbitrary shapes (small and odd-shape cases)."""
    q = make_tensor(shape_q, dtype, wid, _STREAM_Q, seed)
    k = make_tensor(shape_kv, dtype, wid, _STREAM_K, seed)
    v = make_tensor(shape_kv, dtype, wid, _STREAM_V, seed)
    return q, k, v


def make_block_mask(B: int, H: int, n_qb: int, n_kb: int, wid: int = 5,
                    seed: int = 0, lo: float = 0.1, hi: float = 0.6):
    """Block mask uint8 [B, H, n_qb, n_kb] and the per-head densities.

    Per head: a density rho ~ U[lo, hi) is drawn; the head keeps
    n = max(n_diag, round(rho * n_qb * n_kb)) blocks, always including the
    n_diag = min(n_qb, n_kb) diagonal blocks; the remaining n - n_diag kept
    blocks are drawn uniformly without replacement from the off-diagonal
    blocks. Every batch entry gets the same mask (the workloads use B=1).
    Returns (mask, densities) with densities[h] = n_h / (n_qb * n_kb).
    """
    rng = rng_for(wid, _STREAM_MASK, seed)
    nb = n_qb * n_kb
    nd = min(n_qb, n_kb)
    diag = np.arange(nd, dtype=np.int64) * n_kb + np.arange(nd, dtype=np.int64)
    is_diag = np.zeros(nb, dtype=bool)
    is_diag[diag] = True
    off = np.flatnonzero(~is_diag)
    mask = np.zeros((B, H, n_qb, n_kb), dtype=np.uint8)
    dens = np.zeros(H, dtype=np.float64)
    for h in range(H):
        rho = rng.uniform(lo, hi)
        n = max(nd, int(round(rho * nb)))
        n = min(n, nb)
        pick = rng.choice(off, size=n - nd, replace=False)
        flat = np.zeros(nb, dtype=np.uint8)
        flat[diag] = 1
        flat[pick] = 1
        mask[:, h] = flat.reshape(n_qb, n_kb)
        dens[h] = n / nb
    return mask, dens


def sample_rows(S: int, n: int, seed: int, tile: int = 128) -> np.ndarray:
    """Seeded subset of query rows that always includes the first row and
    every row of the last (possibly partial) ``tile``-row tile."""
    rng = np.random.default_rng(np.random.SeedSequence([ROOT_SEED, 7777, S, seed]))
    last0 = ((S - 1) // tile) * tile
    fixed = np.concatenate([[0], np.arange(last0, S)])
    pool = np.setdiff1d(np.arange(S), fixed)
    k = max(0, min(n - fixed.size, pool.size))
    extra = rng.choice(pool, size=k, replace=False) if k else np.empty(0, np.int64)
    return np.unique(np.concatenate([fixed, extra])).astype(np.int64)
