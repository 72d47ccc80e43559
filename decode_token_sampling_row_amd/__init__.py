"""MI355X (gfx950) batched logits sampler: repetition penalty, temperature,
rolling top-k, top-p, exponential-race sampling and dense filtered outputs,
in hand-written HIP kernels behind the C ABI of ``include/sampler.h``.

``sampler``   thin ctypes binding (same entry-point names as the C ABI)
``build``     in-tree hipcc build of ``libsampler.so``
``workloads`` seeded synthetic inputs
"""
