"""Host-side checks of the C-ABI library that need no GPU: it builds, loads,
exports every entry point the header declares, the Python argument structs
match the C layout, and argument validation that runs before any HIP call."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from decode_token_sampling_row_amd import sampler as smp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sampler.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(smp.LIB_PATH):
        from decode_token_sampling_row_amd import build

        build.build()
    return smp.load_library()


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(sampler_\w+)\s*\(", txt, re.M)))


def test_header_declares_the_binding_names():
    assert _declared() == sorted(smp.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", smp.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    for name in _declared():
        assert re.search(rf"\bT {name}$", out, re.M), name


def test_args_struct_layout_matches_header():
    src = r"""
    #include <stddef.h>
    #include <stdio.h>
    #include "sampler.h"
    #define O(f) printf("%zu ", offsetof(sampler_args, f))
    int main(void) {
      printf("%zu %zu ", sizeof(sampler_args), sizeof(sampler_opts));
      printf("%zu %zu %zu ", offsetof(sampler_opts, topk_guess), offsetof(sampler_opts, segment_len),
             offsetof(sampler_opts, rows_per_launch));
      O(logits); O(ld); O(top_k); O(top_p); O(q); O(eps); O(temperature);
      O(repetition_penalty); O(penalty_ids); O(penalty_offsets); O(row_flags);
      O(flags); O(out_idx); O(out_logits); O(out_probs); O(u); O(penalty_len);
      O(finished); O(eos_id); O(counts);
      return 0;
    }
    """
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        exe = os.path.join(d, "t")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-I", os.path.dirname(HEADER), c, "-o", exe], check=True)
        got = [int(v) for v in subprocess.run([exe], capture_output=True, text=True,
                                              check=True).stdout.split()]
    A = smp.sampler_args
    O = smp.sampler_opts
    want = ([ctypes.sizeof(A), ctypes.sizeof(O)] + [getattr(O, f).offset for f, _ in O._fields_]
            + [getattr(A, f).offset for f, _ in A._fields_])
    assert got == want


def test_constants_match_header():
    txt = open(HEADER).read()

    def val(name):
        m = re.search(rf"#define {name} \(?(-?[0-9u]+)", txt)
        return int(m.group(1).rstrip("u"))

    for name in ["SAMPLER_OK", "SAMPLER_EINVAL", "SAMPLER_ENOMEM", "SAMPLER_EHIP",
                 "SAMPLER_F32", "SAMPLER_BF16", "SAMPLER_ROW_TOPK", "SAMPLER_ROW_TOPP",
                 "SAMPLER_ROW_SAMPLE", "SAMPLER_ROW_ALL", "SAMPLER_NEED_LOGITS",
                 "SAMPLER_NEED_PROBS", "SAMPLER_TOPK_TIES", "SAMPLER_APPEND_HISTORY",
                 "SAMPLER_PROFILE",
                 "SAMPLER_PROFILE_SLOTS",
                 "SAMPLER_TOPK_MAX"]:
        assert getattr(smp, name) == val(name), name


def test_create_rejects_bad_arguments_before_touching_the_gpu(lib):
    h = ctypes.c_void_p()
    bad = [(0, 10, 0), (-1, 10, 0), (4, 0, 0), (4, (1 << 21) + 1, 0), (4, 10, 2), (4, 10, -1)]
    for mb, v, dt in bad:
        assert lib.sampler_create(ctypes.byref(h), mb, v, dt, None) == smp.SAMPLER_EINVAL
    for g, c, r in [(-1, 0, 0), (1025, 0, 0), (0, 512, 0), (0, -1024, 0), (0, 1500, 0),
                    (0, 33792, 0), (0, 0, -1)]:
        o = smp.sampler_opts(g, c, r)
        assert lib.sampler_create(ctypes.byref(h), 4, 100, 0, ctypes.byref(o)) == smp.SAMPLER_EINVAL
    assert lib.sampler_create(None, 4, 100, 0, None) == smp.SAMPLER_EINVAL


def test_null_handle_paths(lib):
    a = smp.sampler_args()
    assert lib.sampler_check(None, 1, ctypes.byref(a)) == smp.SAMPLER_EINVAL
    assert lib.sampler_run(None, 1, ctypes.byref(a), None) == smp.SAMPLER_EINVAL
    assert lib.sampler_destroy(None) == smp.SAMPLER_OK
    buf = (ctypes.c_float * 4)()
    assert lib.sampler_profile(None, buf, 4) == smp.SAMPLER_EINVAL


def test_strerror(lib):
    assert smp.sampler_strerror(0) == "ok"
    assert "invalid" in smp.sampler_strerror(-1)
    assert smp.sampler_strerror(12345) == "unknown error"


def test_create_without_gpu_reports_hip_error(lib):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    h = ctypes.c_void_p()
    assert lib.sampler_create(ctypes.byref(h), 4, 100, 0, None) == smp.SAMPLER_EHIP


def _good(B=3, V=10, bf16=False):
    import torch

    return dict(logits=torch.zeros((B, V), dtype=torch.bfloat16 if bf16 else torch.float32),
                out_idx=torch.zeros(B, dtype=torch.int64),
                top_k=torch.zeros(B, dtype=torch.int32), top_p=torch.ones(B),
                q=torch.ones((B, V)), penalty_ids=torch.zeros(6, dtype=torch.int32),
                penalty_offsets=torch.arange(B + 1, dtype=torch.int64) * 2,
                row_flags=torch.zeros(B, dtype=torch.uint8), out_logits=torch.zeros((B, V)),
                out_probs=torch.zeros((B, V)), u=torch.zeros(B),
                penalty_len=torch.zeros(B, dtype=torch.int32),
                finished=torch.zeros(B, dtype=torch.uint8),
                counts=torch.zeros(2, dtype=torch.int32))


def test_binding_rejects_mismatched_tensors_before_any_device_access():
    """The binding checks dtypes and shapes against the handle before the C
    call sees bare pointers (CPU tensors: no device is touched)."""
    import torch

    V, B = 10, 3
    kw = _good(B, V)
    smp.check_tensors(V, smp.SAMPLER_F32, 4, **kw)  # consistent: accepted
    smp.check_tensors(V, smp.SAMPLER_BF16, 4, **_good(B, V, bf16=True))
    with pytest.raises(TypeError):  # bf16 logits to an f32 handle: twice the bytes read
        smp.check_tensors(V, smp.SAMPLER_F32, 4, **_good(B, V, bf16=True))
    with pytest.raises(TypeError):
        smp.check_tensors(V, smp.SAMPLER_BF16, 4, **kw)
    with pytest.raises(ValueError):  # vocab mismatch
        smp.check_tensors(V + 1, smp.SAMPLER_F32, 4, **kw)
    with pytest.raises(ValueError):  # batch beyond the handle
        smp.check_tensors(V, smp.SAMPLER_F32, 2, **kw)
    bad = [("q", torch.ones((B, V - 1))), ("q", torch.ones((B - 1, V))),
           ("out_logits", torch.zeros((B, V + 1))), ("out_probs", torch.zeros((B, V)).t()),
           ("top_k", torch.zeros(B + 1, dtype=torch.int32)), ("top_p", torch.ones(B - 1)),
           ("u", torch.zeros(B + 2)), ("row_flags", torch.zeros(B - 1, dtype=torch.uint8)),
           ("penalty_offsets", torch.zeros(B, dtype=torch.int64)),
           ("penalty_len", torch.zeros(B + 1, dtype=torch.int32)),
           ("finished", torch.zeros(1, dtype=torch.uint8)),
           ("counts", torch.zeros(1, dtype=torch.int32)),
           ("out_idx", torch.zeros(B - 1, dtype=torch.int64))]
    for name, t in bad:
        with pytest.raises(ValueError):
            smp.check_tensors(V, smp.SAMPLER_F32, 4, **dict(kw, **{name: t}))
    wrong_type = [("q", torch.ones((B, V), dtype=torch.float64)),
                  ("top_k", torch.zeros(B, dtype=torch.int64)),
                  ("top_p", torch.ones(B, dtype=torch.float16)),
                  ("row_flags", torch.zeros(B, dtype=torch.int32)),
                  ("penalty_ids", torch.zeros(6, dtype=torch.int64)),
                  ("penalty_offsets", torch.zeros(B + 1, dtype=torch.int32)),
                  ("out_idx", torch.zeros(B, dtype=torch.int32)),
                  ("counts", torch.zeros(2, dtype=torch.int64))]
    for name, t in wrong_type:
        with pytest.raises(TypeError):
            smp.check_tensors(V, smp.SAMPLER_F32, 4, **dict(kw, **{name: t}))
