"""Thin ctypes binding of the C ABI in ``include/sampler.h``.

Same entry points, same names; this module only marshals arguments (torch
tensors -> device pointers, the current HIP stream) and turns return codes
into exceptions.  Every step of the sampling runs in the HIP kernels of
``libsampler.so``; there is no other implementation behind these calls, and a
missing library is an error.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsampler.so")

SAMPLER_OK, SAMPLER_EINVAL, SAMPLER_ENOMEM, SAMPLER_EHIP = 0, -1, -2, -3
SAMPLER_F32, SAMPLER_BF16 = 0, 1
SAMPLER_ROW_TOPK, SAMPLER_ROW_TOPP, SAMPLER_ROW_SAMPLE, SAMPLER_ROW_ALL = 1, 2, 4, 7
SAMPLER_NEED_LOGITS, SAMPLER_NEED_PROBS, SAMPLER_TOPK_TIES = 1, 2, 4
SAMPLER_APPEND_HISTORY, SAMPLER_PROFILE = 8, 256
SAMPLER_TOPK_MAX = 1024
SAMPLER_VOCAB_MAX = 1 << 21

EXPORTS = ("sampler_create", "sampler_check", "sampler_run", "sampler_profile",
           "sampler_destroy", "sampler_strerror", "sampler_run_static")
SAMPLER_STATIC_SCRATCH_BYTES = 32 << 20
SAMPLER_PROFILE_SLOTS = 6


class SamplerError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {sampler_strerror(code)} ({code})")
        self.code = code


class sampler_opts(ctypes.Structure):
    _fields_ = [("topk_guess", ctypes.c_int32), ("segment_len", ctypes.c_int32),
                ("rows_per_launch", ctypes.c_int32)]


class sampler_args(ctypes.Structure):
    _fields_ = [
        ("logits", ctypes.c_void_p),
        ("ld", ctypes.c_int64),
        ("top_k", ctypes.c_void_p),
        ("top_p", ctypes.c_void_p),
        ("q", ctypes.c_void_p),
        ("eps", ctypes.c_float),
        ("temperature", ctypes.c_float),
        ("repetition_penalty", ctypes.c_float),
        ("penalty_ids", ctypes.c_void_p),
        ("penalty_offsets", ctypes.c_void_p),
        ("row_flags", ctypes.c_void_p),
        ("flags", ctypes.c_uint32),
        ("out_idx", ctypes.c_void_p),
        ("out_logits", ctypes.c_void_p),
        ("out_probs", ctypes.c_void_p),
        ("u", ctypes.c_void_p),
        ("penalty_len", ctypes.c_void_p),
        ("finished", ctypes.c_void_p),
        ("eos_id", ctypes.c_int64),
        ("counts", ctypes.c_void_p),
    ]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libsampler.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP sampler library not found at {path}; build it with "
            "`python -m decode_token_sampling_row_amd.build` (hipcc, gfx950)")
    # torch's HIP runtime must be the one in the process: the library then
    # binds to it (same soname) and accepts torch's streams and allocations.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.sampler_create.argtypes = [ctypes.POINTER(P), ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.POINTER(sampler_opts)]
    lib.sampler_create.restype = ctypes.c_int
    lib.sampler_check.argtypes = [P, ctypes.c_int32, ctypes.POINTER(sampler_args)]
    lib.sampler_check.restype = ctypes.c_int
    lib.sampler_run.argtypes = [P, ctypes.c_int32, ctypes.POINTER(sampler_args), P]
    lib.sampler_run.restype = ctypes.c_int
    lib.sampler_profile.argtypes = [P, ctypes.POINTER(ctypes.c_float), ctypes.c_int32]
    lib.sampler_profile.restype = ctypes.c_int
    lib.sampler_destroy.argtypes = [P]
    lib.sampler_destroy.restype = ctypes.c_int
    lib.sampler_strerror.argtypes = [ctypes.c_int]
    lib.sampler_strerror.restype = ctypes.c_char_p
    lib.sampler_run_static.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.POINTER(sampler_opts),
                                       ctypes.POINTER(sampler_args), P]
    lib.sampler_run_static.restype = ctypes.c_int
    _lib = lib
    return lib


def sampler_strerror(code: int) -> str:
    return load_library().sampler_strerror(int(code)).decode()


def sampler_create(max_batch: int, vocab: int, dtype: int, topk_guess: int = 0,
                   segment_len: int = 0, rows_per_launch: int = 0) -> ctypes.c_void_p:
    """sampler_create on the current HIP device; returns the handle."""
    lib = load_library()
    h = ctypes.c_void_p()
    opts = sampler_opts(int(topk_guess), int(segment_len), int(rows_per_launch))
    rc = lib.sampler_create(ctypes.byref(h), int(max_batch), int(vocab), int(dtype),
                            ctypes.byref(opts))
    if rc != SAMPLER_OK:
        raise SamplerError(rc, "sampler_create")
    return h


def sampler_destroy(h) -> None:
    rc = load_library().sampler_destroy(h)
    if rc != SAMPLER_OK:
        raise SamplerError(rc, "sampler_destroy")


def _ptr(t, dtype=None, what=""):
    if t is None:
        return None
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{what}: must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what}: expected {dtype}, got {t.dtype}")
    return t.data_ptr()


def make_args(logits, out_idx, *, top_k=None, top_p=None, q=None, eps=1e-20,
              temperature=1.0, repetition_penalty=1.0, penalty_ids=None,
              penalty_offsets=None, row_flags=None, out_logits=None, out_probs=None,
              profile=False, u=None, topk_ties=False, penalty_len=None, finished=None,
              eos_id=None, counts=None, append_history=False) -> sampler_args:
    """Marshal torch tensors into a sampler_args struct.

    The decode-step epilogue: ``finished`` (uint8 [B], updated in place) with
    ``eos_id``; ``append_history`` appends the output ids to the history
    slots ``penalty_ids`` / ``penalty_offsets`` filled up to ``penalty_len``
    (int32 [B], advanced in place); ``counts`` (int32 [2]) receives the
    unfinished rows and the appends that found a full slot.
    """
    import torch

    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be [B, ld] with unit column stride")
    if logits.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("logits must be float32 or bfloat16")
    for name, t in (("q", q), ("out_logits", out_logits), ("out_probs", out_probs)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [B, V]")
    flags = 0
    if out_logits is not None:
        flags |= SAMPLER_NEED_LOGITS
    if out_probs is not None:
        flags |= SAMPLER_NEED_PROBS
    if profile:
        flags |= SAMPLER_PROFILE
    if topk_ties:
        flags |= SAMPLER_TOPK_TIES
    if append_history:
        flags |= SAMPLER_APPEND_HISTORY
    if finished is not None and eos_id is None:
        raise ValueError("finished needs eos_id")
    a = sampler_args()
    a.logits = _ptr(logits, None, "logits")
    a.ld = logits.stride(0)
    a.top_k = _ptr(top_k, torch.int32, "top_k")
    a.top_p = _ptr(top_p, torch.float32, "top_p")
    a.q = _ptr(q, torch.float32, "q")
    a.eps = float(eps)
    a.temperature = float(temperature)
    a.repetition_penalty = float(repetition_penalty)
    a.penalty_ids = _ptr(penalty_ids, torch.int32, "penalty_ids")
    a.penalty_offsets = _ptr(penalty_offsets, torch.int64, "penalty_offsets")
    a.row_flags = _ptr(row_flags, torch.uint8, "row_flags")
    a.flags = flags
    a.out_idx = _ptr(out_idx, torch.int64, "out_idx")
    a.out_logits = _ptr(out_logits, torch.float32, "out_logits")
    a.out_probs = _ptr(out_probs, torch.float32, "out_probs")
    a.u = _ptr(u, torch.float32, "u")
    a.penalty_len = _ptr(penalty_len, torch.int32, "penalty_len")
    a.finished = _ptr(finished, torch.uint8, "finished")
    a.eos_id = int(eos_id) if eos_id is not None else 0
    a.counts = _ptr(counts, torch.int32, "counts")
    return a


def sampler_check(h, batch: int, args: sampler_args) -> int:
    return load_library().sampler_check(h, int(batch), ctypes.byref(args))


def sampler_run(h, batch: int, args: sampler_args, stream: Optional[int] = None) -> None:
    """sampler_run on `stream` (raw hipStream_t; default torch's current stream)."""
    if stream is None:
        import torch

        stream = torch.cuda.current_stream().cuda_stream
    rc = load_library().sampler_run(h, int(batch), ctypes.byref(args), ctypes.c_void_p(stream))
    if rc != SAMPLER_OK:
        raise SamplerError(rc, "sampler_run")


def sampler_run_static(batch: int, vocab: int, dtype: int, args: sampler_args,
                       stream: Optional[int] = None, topk_guess: int = 0, segment_len: int = 0,
                       rows_per_launch: int = 0) -> int:
    """sampler_run_static: the call without a handle, on the library's static
    per-GPU workspace (nothing is allocated).  Returns the C return code."""
    if stream is None:
        import torch

        stream = torch.cuda.current_stream().cuda_stream
    opts = sampler_opts(int(topk_guess), int(segment_len), int(rows_per_launch))
    return load_library().sampler_run_static(int(batch), int(vocab), int(dtype),
                                             ctypes.byref(opts), ctypes.byref(args),
                                             ctypes.c_void_p(stream))


def run_static(logits, out_idx, stream=None, topk_guess=0, segment_len=0, rows_per_launch=0,
               **kw) -> None:
    """Check and marshal torch tensors, then sampler_run_static (raises on a
    nonzero return code)."""
    import torch

    dt = SAMPLER_BF16 if logits.dtype == torch.bfloat16 else SAMPLER_F32
    check_tensors(logits.shape[1], dt, logits.shape[0], logits, out_idx, **kw)
    args = make_args(logits, out_idx, **kw)
    rc = sampler_run_static(logits.shape[0], logits.shape[1], dt, args, stream, topk_guess,
                            segment_len, rows_per_launch)
    if rc != SAMPLER_OK:
        raise SamplerError(rc, "sampler_run_static")


def sampler_profile(h, n: int = SAMPLER_PROFILE_SLOTS):
    """Per-kernel milliseconds averaged over the profiled calls since the last read."""
    buf = (ctypes.c_float * n)()
    rc = load_library().sampler_profile(h, buf, int(n))
    if rc < 0:
        raise SamplerError(rc, "sampler_profile")
    return [float(buf[i]) for i in range(rc)]


def check_tensors(vocab: int, dtype: int, max_batch: int, logits, out_idx, *, top_k=None,
                  top_p=None, q=None, penalty_ids=None, penalty_offsets=None, row_flags=None,
                  out_logits=None, out_probs=None, u=None, penalty_len=None, finished=None,
                  counts=None, **_):
    """Reject, before any device access, tensors whose dtype or shape does not
    match a handle of `vocab` and storage `dtype` (SAMPLER_F32 / _BF16): the
    C side sees only pointers, so a wrong element type or a short buffer
    would otherwise be read or written past its end.  Raises TypeError or
    ValueError.  (The history ids cannot be checked against the offsets
    without reading them; the caller keeps offsets[B] <= len(penalty_ids).)"""
    import torch

    want = torch.bfloat16 if dtype == SAMPLER_BF16 else torch.float32
    if logits.dtype != want:
        raise TypeError(f"logits: the handle was created for {want}, got {logits.dtype}")
    if logits.dim() != 2 or logits.shape[1] != vocab:
        raise ValueError(f"logits: expected [B, {vocab}], got {list(logits.shape)}")
    B = logits.shape[0]
    if B > max_batch:
        raise ValueError(f"logits: batch {B} exceeds the handle's max_batch {max_batch}")

    def vec(name, t, dt, n):
        if t is None:
            return
        if t.dtype != dt:
            raise TypeError(f"{name}: expected {dt}, got {t.dtype}")
        if t.dim() != 1 or t.shape[0] != n or not t.is_contiguous():
            raise ValueError(f"{name}: expected a contiguous [{n}] tensor, got {list(t.shape)}")

    def mat(name, t):
        if t is None:
            return
        if t.dtype != torch.float32:
            raise TypeError(f"{name}: expected torch.float32, got {t.dtype}")
        if list(t.shape) != [B, vocab] or not t.is_contiguous():
            raise ValueError(f"{name}: expected a contiguous [{B}, {vocab}] tensor, "
                             f"got {list(t.shape)}")

    vec("out_idx", out_idx, torch.int64, B)
    vec("top_k", top_k, torch.int32, B)
    vec("top_p", top_p, torch.float32, B)
    vec("u", u, torch.float32, B)
    vec("row_flags", row_flags, torch.uint8, B)
    vec("penalty_len", penalty_len, torch.int32, B)
    vec("finished", finished, torch.uint8, B)
    vec("penalty_offsets", penalty_offsets, torch.int64, B + 1)
    if penalty_ids is not None:
        if penalty_ids.dtype != torch.int32:
            raise TypeError(f"penalty_ids: expected torch.int32, got {penalty_ids.dtype}")
        if penalty_ids.dim() != 1 or not penalty_ids.is_contiguous():
            raise ValueError("penalty_ids: expected a contiguous 1-D tensor")
    if counts is not None:
        if counts.dtype != torch.int32:
            raise TypeError(f"counts: expected torch.int32, got {counts.dtype}")
        if counts.numel() < 2 or not counts.is_contiguous():
            raise ValueError("counts: expected a contiguous tensor of at least 2 elements")
    mat("q", q)
    mat("out_logits", out_logits)
    mat("out_probs", out_probs)


class Sampler:
    """Owns one handle; ``run`` checks and marshals tensors and calls sampler_run."""

    def __init__(self, max_batch: int, vocab: int, dtype, topk_guess: int = 0,
                 segment_len: int = 0, rows_per_launch: int = 0):
        import torch

        dt = SAMPLER_BF16 if dtype in (torch.bfloat16, SAMPLER_BF16, "bf16") else SAMPLER_F32
        self.vocab = int(vocab)
        self.dtype = dt
        self.max_batch = int(max_batch)
        self.handle = sampler_create(max_batch, vocab, dt, topk_guess, segment_len,
                                     rows_per_launch)

    def run(self, logits, out_idx, stream=None, **kw) -> None:
        check_tensors(self.vocab, self.dtype, self.max_batch, logits, out_idx, **kw)
        args = make_args(logits, out_idx, **kw)
        sampler_run(self.handle, logits.shape[0], args, stream)

    def profile(self):
        return sampler_profile(self.handle)

    def close(self):
        if self.handle is not None:
            sampler_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
