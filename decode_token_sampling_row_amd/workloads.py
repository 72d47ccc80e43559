"""Seeded synthetic workloads for the batched logits sampler.

This module only draws random inputs and casts them to the storage dtype; it
holds none of the sampler's arithmetic, so the HIP path and the CPU oracle can
both be fed from it without sharing any of the method.

Every array comes from ``numpy.random.default_rng(SeedSequence([cfg, stream,
seed]))`` -- [B, V] arrays from one generator per block of 16 rows,
``SeedSequence([cfg, stream, seed, block])``, filled on several host threads
(the values do not depend on the thread count) -- with fixed streams:

    0 logits   1 q   2 top_k   3 top_p   4 history ids   5 spike positions
    6 spike sizes   7 row choice (rows whose k is zeroed)

bf16 logits are drawn in float32 and rounded to bf16 with round-to-nearest-even
(torch's ``to(torch.bfloat16)``); the workload keeps the 16-bit patterns as a
``uint16`` array.  ``q`` is float32 Exp(1).

The five configurations follow the batch/vocabulary shapes and value
distributions of the decode-time sampling workloads the pages describe:
default sampling parameters T = 0.85, top_k = 50, top_p = 0.85 of the MiniMind
generation chapter (defaults table), the 1 <= k <= 1024 top-k range and the
eight stage combinations of the Ascend top-k/top-p/sample operator page, and
vocabularies of common decoder LLMs (32000, 151936, 128256, 6400, 262144).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

ROW_TOPK, ROW_TOPP, ROW_SAMPLE = 1, 2, 4
ALL_STAGES = ROW_TOPK | ROW_TOPP | ROW_SAMPLE

F32, BF16 = "f32", "bf16"

# stream ids
S_LOGITS, S_Q, S_TOPK, S_TOPP, S_IDS, S_POS, S_SIZE, S_ROWS = range(8)


ROW_BLOCK = 16


def _rng(cfg: int, stream: int, seed: int, *extra: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg, stream, seed, *extra]))


def _rows(cfg: int, stream: int, seed: int, B: int, V: int, draw) -> np.ndarray:
    """[B, V] float32 filled block by block: draw(generator, rows, V)."""
    from concurrent.futures import ThreadPoolExecutor
    import os

    out = np.empty((B, V), np.float32)

    def fill(blk):
        r0, r1 = blk * ROW_BLOCK, min(B, (blk + 1) * ROW_BLOCK)
        out[r0:r1] = draw(_rng(cfg, stream, seed, blk), r1 - r0, V)

    nblk = (B + ROW_BLOCK - 1) // ROW_BLOCK
    workers = max(1, min(16, os.cpu_count() or 1, nblk))
    if workers == 1:
        for i in range(nblk):
            fill(i)
    else:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact widening)."""
    return (h.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Workload:
    name: str
    B: int
    V: int
    dtype: str                       # "f32" or "bf16"
    logits: np.ndarray               # [B, V] float32, or uint16 bf16 bits
    q: Optional[np.ndarray]          # [B, V] float32 or None
    top_k: Optional[np.ndarray]      # [B] int32 or None
    top_p: Optional[np.ndarray]      # [B] float32 or None
    row_flags: Optional[np.ndarray]  # [B] uint8 or None (= all stages on)
    eps: float = 1e-20
    temperature: float = 1.0
    penalty: float = 1.0
    ids: Optional[np.ndarray] = None      # [nnz] int32
    offsets: Optional[np.ndarray] = None  # [B+1] int64
    need_logits: bool = False
    need_probs: bool = False
    meta: dict = field(default_factory=dict)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == BF16 else 4

    def logits_f32(self) -> np.ndarray:
        if self.dtype == BF16:
            return bf16_bits_to_f32(self.logits)
        return self.logits


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return to_bf16_bits(x32) if dtype == BF16 else np.ascontiguousarray(x32, np.float32)


def _q(cfg: int, B: int, V: int, seed: int) -> np.ndarray:
    return _rows(cfg, S_Q, seed, B, V,
                 lambda g, n, v: g.standard_exponential((n, v), dtype=np.float32))


def _normal(cfg: int, B: int, V: int, seed: int, scale: float) -> np.ndarray:
    return _rows(cfg, S_LOGITS, seed, B, V,
                 lambda g, n, v: g.standard_normal((n, v), dtype=np.float32) * np.float32(scale))


def config1(B: int = 4, V: int = 32000, seed: int = 0) -> Workload:
    """B=4, V=32000, fp32 N(0, 2^2); T=0.85, k=50, p=0.85 on every row; all
    three stages on; dense filtered logits requested."""
    x = _normal(1, B, V, seed, 2.0)
    return Workload("cfg1_topk_topp_sample_dense", B, V, F32, _store(x, F32), _q(1, B, V, seed),
                    np.full(B, 50, np.int32), np.full(B, 0.85, np.float32),
                    np.full(B, ALL_STAGES, np.uint8), eps=1e-20, temperature=0.85,
                    need_logits=True)


def config2(B: int = 64, V: int = 151936, seed: int = 0) -> Workload:
    """B=64, V=151936, bf16 of N(0,1) plus 8 spikes of +U[6,10] per row;
    k ~ U{1..1024} with round(10%) of rows set to 0 (stage skipped);
    p ~ U[0.5, 1); sampling on; no dense output."""
    x = _normal(2, B, V, seed, 1.0)
    pos_rng, size_rng = _rng(2, S_POS, seed), _rng(2, S_SIZE, seed)
    n_spk = min(8, V)
    for b in range(B):
        pos = pos_rng.choice(V, size=n_spk, replace=False)
        x[b, pos] += size_rng.uniform(6.0, 10.0, size=n_spk).astype(np.float32)
    k = _rng(2, S_TOPK, seed).integers(1, 1025, size=B).astype(np.int32)
    n0 = int(round(0.1 * B))
    zero_rows = _rng(2, S_ROWS, seed).permutation(B)[:n0]
    k[zero_rows] = 0
    p = _rng(2, S_TOPP, seed).uniform(0.5, 1.0, size=B).astype(np.float32)
    return Workload("cfg2_bf16_spiky_mixed_k", B, V, BF16, _store(x, BF16), _q(2, B, V, seed),
                    k, p, np.full(B, ALL_STAGES, np.uint8), eps=1e-20,
                    meta={"k_zero_rows": np.sort(zero_rows)})


def config3(B: int = 128, V: int = 128256, seed: int = 0) -> Workload:
    """Top-p only (k = 0 on every row): B=128, V=128256, fp32.  Even rows are
    peaked (N(0,1) with 20 entries +12), odd rows flat (N(0, 0.05)).
    p = 0.9 when (row // 2) is even, else 0.99.  Sampling on."""
    x = _normal(3, B, V, seed, 1.0)
    x[1::2] *= np.float32(0.05)  # flat rows
    pos_rng = _rng(3, S_POS, seed)
    n_spk = min(20, V)
    for b in range(0, B, 2):     # peaked rows
        x[b, pos_rng.choice(V, size=n_spk, replace=False)] += np.float32(12.0)
    p = np.where((np.arange(B) // 2) % 2 == 0, 0.9, 0.99).astype(np.float32)
    return Workload("cfg3_topp_only_peaked_flat", B, V, F32, _store(x, F32), _q(3, B, V, seed),
                    np.zeros(B, np.int32), p, np.full(B, ALL_STAGES, np.uint8), eps=1e-20)


def config4(B: int = 256, V: int = 6400, seed: int = 0, hist: int = 512) -> Workload:
    """Penalty + temperature: B=256, V=6400, fp32 N(0, 3^2); each row has a
    history of 512 ids uniform in [0, V) (duplicates allowed); rho=1.1,
    T=0.85, k=50 (k=1 on rows r % 32 == 0), p=0.85; all stages on."""
    x = _normal(4, B, V, seed, 3.0)
    ids = _rng(4, S_IDS, seed).integers(0, V, size=B * hist).astype(np.int32)
    offsets = (np.arange(B + 1, dtype=np.int64) * hist)
    k = np.full(B, 50, np.int32)
    k[np.arange(B) % 32 == 0] = 1
    return Workload("cfg4_penalty_temperature", B, V, F32, _store(x, F32), _q(4, B, V, seed),
                    k, np.full(B, 0.85, np.float32), np.full(B, ALL_STAGES, np.uint8),
                    eps=1e-20, temperature=0.85, penalty=1.1, ids=ids, offsets=offsets)


def config5(B: int = 1024, V: int = 262144, seed: int = 0) -> Workload:
    """Large batch: B=1024, V=262144, bf16 of 4 * Gumbel(0,1); row r runs
    stage combination r % 8 (bit0 top-k with k=1024, bit1 top-p with
    p=0.95, bit2 sample); dense filtered logits on every row."""
    x = _rows(5, S_LOGITS, seed, B, V,
              lambda g, n, v: (4.0 * g.gumbel(0.0, 1.0, size=(n, v))).astype(np.float32))
    flags = (np.arange(B) % 8).astype(np.uint8)
    return Workload("cfg5_large_batch_8_combos", B, V, BF16, _store(x, BF16), _q(5, B, V, seed),
                    np.full(B, 1024, np.int32), np.full(B, 0.95, np.float32), flags,
                    eps=1e-20, need_logits=True)


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}


def make(cfg: int, B: Optional[int] = None, V: Optional[int] = None, seed: int = 0,
         **kw) -> Workload:
    """Workload ``cfg`` (1..5), optionally at a reduced (B, V)."""
    fn = CONFIGS[cfg]
    args = {}
    if B is not None:
        args["B"] = B
    if V is not None:
        args["V"] = V
    args.update(kw)
    return fn(seed=seed, **args)


@dataclass
class DecodeLoop:
    """Inputs of several decode steps over one batch (the MiniMind generation
    loop's shape: one logits row per sequence and step, a history that grows
    by one id per step).  Per step, logits[s] is [B, V] in the storage dtype
    and q[s] / u[s] are fresh random numbers; the history is a CSR of slots
    (prompt ids first, then filler ids that are not history), with per-row
    capacities, a few rows already finished, and an EOS logit that rises
    over the steps at a row-dependent rate so that rows end at different
    steps."""
    B: int
    V: int
    dtype: str
    eos: int
    logits: list
    q: list
    u: list
    top_k: np.ndarray
    top_p: np.ndarray
    row_flags: np.ndarray
    ids: np.ndarray
    offsets: np.ndarray
    lens: np.ndarray
    finished: np.ndarray


def decode_loop(B: int, V: int, dtype: str = F32, steps: int = 8, prompt: int = 6,
                eos: int = 2, seed: int = 0) -> DecodeLoop:
    """Seeded decode-loop inputs: per-row base logits N(0, 2^2) plus N(0, 0.3^2)
    step noise (so that a row's likely tokens recur and the penalty matters),
    EOS logit -4 + 2.5 s (b mod 7 + 1) / 7 at step s, k in [0, min(V, 1024)],
    p in [0.5, 1), every stage combination; every fifth row's slot holds only
    prompt + 3 ids, every seventh row starts finished."""
    g = _rng(99, S_LOGITS, seed)
    base = g.standard_normal((B, V)).astype(np.float32) * 2
    rate = ((np.arange(B) % 7) + 1) / 7.0
    logits, q, u = [], [], []
    for s in range(steps):
        x = base + g.standard_normal((B, V)).astype(np.float32) * np.float32(0.3)
        x[:, eos] = np.float32(-4.0) + (2.5 * s * rate).astype(np.float32)
        logits.append(_store(x, dtype))
        q.append(g.standard_exponential((B, V)).astype(np.float32))
        u.append(g.random(B).astype(np.float32))
    top_k = g.integers(0, min(V, 1024) + 1, size=B).astype(np.int32)
    top_p = g.uniform(0.5, 1.0, size=B).astype(np.float32)
    row_flags = (np.arange(B) % 8).astype(np.uint8)
    cap = np.where(np.arange(B) % 5 == 4, prompt + 3, prompt + steps).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(cap)]).astype(np.int64)
    ids = g.integers(0, V, size=int(offsets[-1])).astype(np.int32)  # prompt + filler
    lens = np.full(B, prompt, np.int32)
    finished = np.where(np.arange(B) % 7 == 6, 1 + (np.arange(B) % 3), 0).astype(np.uint8)
    return DecodeLoop(B, V, dtype, eos, logits, q, u, top_k, top_p, row_flags, ids, offsets,
                      lens, finished)
