"""ctypes wrapper of the plain CPU oracle (``sampler_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``.  The product library never loads
it, and it imports nothing from the product package.

``run`` takes numpy arrays shaped like the library's arguments and returns the
oracle outputs plus per-row diagnostics (kept-set size, top-p decision margin,
sampling ratio gap).  ``decode_epilogue`` is the decode-step epilogue (EOS
forcing, finished flags, history append), written in plain Python.  Rows can be processed on several host threads; ctypes
drops the GIL while the C code runs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sampler_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1
ROW_TOPK, ROW_TOPP, ROW_SAMPLE = 1, 2, 4
NEED_LOGITS, NEED_PROBS, TOPK_TIES = 1, 2, 4

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle into ``oracle/liboracle.so`` with gcc."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-Wextra", "-o", _LIB, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.oracle_run.restype = ctypes.c_int
        lib.oracle_run.argtypes = [
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, ctypes.c_int64,
            P, P, P, P, ctypes.c_float, ctypes.c_float, ctypes.c_float, P, P, P,
            ctypes.c_uint32, P, P, P, P, P, P, ctypes.c_int32, ctypes.c_int32]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _arr(a, dtype):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


def run(logits, dtype, vocab=None, top_k=None, top_p=None, q=None, eps=1e-20,
        temperature=1.0, penalty=1.0, ids=None, offsets=None, row_flags=None,
        need_logits=True, need_probs=False, rows=None, threads=1, u=None, topk_ties=False,
        lens=None):
    """Run the oracle.

    logits: [B, ld] float32 (dtype F32) or uint16 bf16 bit patterns (BF16);
    vocab: V <= ld (default ld).
    rows: optional iterable of row indices to compute (others are left as
    zeros / -1); used to sample rows of large workloads.
    u: optional [B] uniforms; sampling rows then draw by inverse CDF (and
    ``gap`` holds that decision's margin) instead of racing with q.
    topk_ties: top-k keeps every element equal to the k-th value too.
    lens: optional [B] history lengths: row b's history is then the first
    clamp(lens[b], 0, slot size) ids of its CSR slot instead of the whole slot.
    Returns a dict with idx [B] int64, logits [B, V] float32 or None,
    probs [B, V] float32 or None, nkept [B] int32, margin [B], gap [B].
    """
    lib = _load()
    B, ld = logits.shape
    logits = np.ascontiguousarray(logits)
    if dtype == F32:
        assert logits.dtype == np.float32
    else:
        assert logits.dtype == np.uint16
    V = int(ld if vocab is None else vocab)
    if q is not None:
        assert q.shape == (B, V)
    top_k = _arr(top_k, np.int32)
    top_p = _arr(top_p, np.float32)
    q = _arr(q, np.float32)
    u = _arr(u, np.float32)
    if u is not None:
        assert u.shape == (B,)
    ids = _arr(ids, np.int32)
    offsets = _arr(offsets, np.int64)
    if lens is not None and ids is not None:
        # the filled part of every slot, as a CSR of its own
        parts, offs = [], [0]
        for b in range(B):
            n = min(max(int(lens[b]), 0), max(int(offsets[b + 1] - offsets[b]), 0))
            parts.append(ids[offsets[b]:offsets[b] + n])
            offs.append(offs[-1] + n)
        ids = np.ascontiguousarray(np.concatenate(parts) if parts else ids[:0], dtype=np.int32)
        offsets = np.asarray(offs, dtype=np.int64)
    row_flags = _arr(row_flags, np.uint8)
    flags = ((NEED_LOGITS if need_logits else 0) | (NEED_PROBS if need_probs else 0)
             | (TOPK_TIES if topk_ties else 0))

    out_idx = np.full(B, -1, dtype=np.int64)
    out_logits = np.zeros((B, V), dtype=np.float32) if need_logits else None
    out_probs = np.zeros((B, V), dtype=np.float32) if need_probs else None
    nkept = np.zeros(B, dtype=np.int32)
    margin = np.full(B, np.inf)
    gap = np.full(B, np.inf)

    def call(r0, r1):
        rc = lib.oracle_run(B, V, dtype, _ptr(logits), ld, _ptr(top_k), _ptr(top_p),
                            _ptr(q), _ptr(u), eps, temperature, penalty, _ptr(ids),
                            _ptr(offsets), _ptr(row_flags), flags, _ptr(out_idx),
                            _ptr(out_logits), _ptr(out_probs), _ptr(nkept),
                            _ptr(margin), _ptr(gap), r0, r1)
        if rc != 0:
            raise RuntimeError(f"oracle_run failed ({rc})")

    if B == 0:
        return {"idx": out_idx, "logits": out_logits, "probs": out_probs,
                "nkept": nkept, "margin": margin, "gap": gap}
    if rows is None:
        ranges = []
        n = max(1, int(threads))
        step = (B + n - 1) // n
        for r0 in range(0, B, step):
            ranges.append((r0, min(B, r0 + step)))
    else:
        ranges = [(int(r), int(r) + 1) for r in rows]
    if threads > 1 and len(ranges) > 1:
        with ThreadPoolExecutor(max_workers=int(threads)) as ex:
            list(ex.map(lambda rr: call(*rr), ranges))
    else:
        for rr in ranges:
            call(*rr)
    return {"idx": out_idx, "logits": out_logits, "probs": out_probs,
            "nkept": nkept, "margin": margin, "gap": gap}


def decode_epilogue(idx, finished=None, eos_id=None, ids=None, offsets=None, lens=None,
                    append=False):
    """The decode-step epilogue of the MiniMind generation loop, row by row.

    MiniMind generation chapter, sec. 10.9 (EOS batch handling), in its order:
      1. a row already finished outputs EOS instead of its draw;
      2. a row whose output is EOS becomes finished (a nonzero flag stays);
      3. the output is concatenated onto the row's sequence -- here written
         at position lens[b] of its history slot ids[offsets[b]:offsets[b+1]]
         (sec. 10.7 penalises every id of that sequence), unless the slot is
         full;
      4. the rows not yet finished are counted (the loop ends at zero).
    Returns new arrays (inputs untouched): idx, finished, ids, lens and
    counts = [unfinished rows, appends that found a full slot].
    """
    idx = np.array(idx, dtype=np.int64)
    B = idx.shape[0]
    fin = None if finished is None else np.array(finished, dtype=np.uint8)
    ids = None if ids is None else np.array(ids, dtype=np.int32)
    lens = None if lens is None else np.array(lens, dtype=np.int32)
    unfinished, full = 0, 0
    for b in range(B):
        if fin is not None:
            if fin[b] != 0:
                idx[b] = eos_id
            elif idx[b] == eos_id:
                fin[b] = 1
            if fin[b] == 0:
                unfinished += 1
        else:
            unfinished += 1
        if append:
            start, cap = int(offsets[b]), int(offsets[b + 1] - offsets[b])
            n = max(int(lens[b]), 0)
            if n < cap:
                ids[start + n] = idx[b]
                lens[b] = n + 1
            else:
                full += 1
    return {"idx": idx, "finished": fin, "ids": ids, "lens": lens,
            "counts": np.array([unfinished, full], dtype=np.int32)}
