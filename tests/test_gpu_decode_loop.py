"""Parity of the decode-step epilogue through the C ABI: several decode steps
in a row, each one a sampler call that also forces EOS on finished rows,
updates the finished flags, appends its output to the history slots (which
the next step's repetition penalty reads) and counts the unfinished rows,
against the oracle's run + decode_epilogue on the same inputs.

Rows where several outputs are correct (sampling near-ties, top-p boundary
ties; counted by the oracle's diagnostics) may differ in their draw: the
oracle then continues from the HIP draw, so that both sides keep one history.
Everything else -- the output ids after the epilogue, the finished flags,
the history slots and lengths, the counts, the dense filtered logits -- is
compared exactly at every step.
"""
import numpy as np
import pytest

from decode_token_sampling_row_amd import workloads as wl
from gpu_util import GAP_TIE, MARGIN_TIE, U_TIE, compare
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

CASES = [
    # label, B, V, dtype, draw, rows per launch
    ("greedy_f32", 48, 3000, wl.F32, "greedy", 0),
    ("race_bf16", 40, 20011, wl.BF16, "race", 0),
    ("inverse_f32", 64, 9000, wl.F32, "inverse", 0),
    ("race_f32_1500rows_chunks", 1500, 700, wl.F32, "race", 256),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    from decode_token_sampling_row_amd import sampler

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sampler.load_library()
    yield


@pytest.mark.parametrize("label,B,V,dtype,draw,rpl", CASES, ids=[c[0] for c in CASES])
def test_decode_loop_parity(label, B, V, dtype, draw, rpl):
    import torch

    from decode_token_sampling_row_amd.sampler import Sampler

    D = wl.decode_loop(B, V, dtype, steps=8, seed=len(label))
    print(f"[case] decode loop {label} B={B} V={V} {dtype} {draw}", flush=True)
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    s = Sampler(B, V, torch.bfloat16 if dtype == wl.BF16 else torch.float32, rows_per_launch=rpl)
    flags = D.row_flags if draw != "greedy" else D.row_flags & 3
    d_ids, d_off, d_len, d_fin = t(D.ids), t(D.offsets), t(D.lens), t(D.finished)
    d_tk, d_tp, d_fl = t(D.top_k), t(D.top_p), t(flags)
    counts = torch.full((2,), -1, dtype=torch.int32, device=dev)
    out_idx = torch.empty(B, dtype=torch.int64, device=dev)
    out_l = torch.empty((B, V), dtype=torch.float32, device=dev)
    ids, lens, fin = D.ids.copy(), D.lens.copy(), D.finished.copy()
    temp, rho = 0.8, 1.25
    for step in range(len(D.logits)):
        x = D.logits[step]
        xs = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16) if dtype == wl.BF16 \
            else torch.from_numpy(x)
        u = D.u[step] if draw == "inverse" else None
        q = D.q[step] if draw == "race" else None
        s.run(xs.to(dev), out_idx, top_k=d_tk, top_p=d_tp, q=None if q is None else t(q),
              u=None if u is None else t(u), temperature=temp, repetition_penalty=rho,
              penalty_ids=d_ids, penalty_offsets=d_off, penalty_len=d_len, row_flags=d_fl,
              out_logits=out_l, finished=d_fin, eos_id=D.eos, counts=counts,
              append_history=True)
        torch.cuda.synchronize()
        ref = orc.run(x, orc.BF16 if dtype == wl.BF16 else orc.F32, top_k=D.top_k, top_p=D.top_p,
                      q=q, u=u, temperature=temp, penalty=rho, ids=ids, offsets=D.offsets,
                      lens=lens, row_flags=flags, need_logits=True, threads=8)
        W = wl.Workload("decode", B, V, dtype, x, q, D.top_k, D.top_p, flags,
                        temperature=temp, penalty=rho)
        # dense outputs: the draw itself is checked after the epilogue below
        compare(W, {"idx": ref["idx"], "logits": out_l.cpu().numpy(), "probs": None}, ref,
                label=f"{label} step {step}", inverse=draw == "inverse")
        hip_idx = out_idx.cpu().numpy()
        sampling = (flags & 4) != 0
        tie = (ref["margin"] < MARGIN_TIE) | (sampling & (ref["gap"] <= (U_TIE if u is not None
                                                                           else GAP_TIE)))
        raw = ref["idx"].copy()
        free_choice = tie & (fin == 0)
        raw[free_choice] = hip_idx[free_choice]
        e = orc.decode_epilogue(raw, fin, D.eos, ids, D.offsets, lens, append=True)
        np.testing.assert_array_equal(hip_idx, e["idx"], err_msg=f"{label} step {step} idx")
        np.testing.assert_array_equal(d_fin.cpu().numpy(), e["finished"])
        np.testing.assert_array_equal(d_len.cpu().numpy(), e["lens"])
        np.testing.assert_array_equal(d_ids.cpu().numpy(), e["ids"])
        np.testing.assert_array_equal(counts.cpu().numpy(), e["counts"])
        ids, lens, fin = e["ids"], e["lens"], e["finished"]
        print(f"[parity] {label} step {step}: unfinished {e['counts'][0]} full {e['counts'][1]} "
              f"ties {int(tie.sum())}", flush=True)
    assert ((fin != 0) & (D.finished == 0)).any() and not fin.all()
    assert (lens == D.lens + len(D.logits)).any() and (lens < D.lens + len(D.logits)).any()
    s.close()


def test_epilogue_without_history_and_counts_only():
    """finished without append, and counts alone (every row unfinished)."""
    import torch

    from decode_token_sampling_row_amd.sampler import Sampler

    B, V = 30, 500
    rng = np.random.default_rng(5)
    x = rng.standard_normal((B, V)).astype(np.float32)
    dev = torch.device("cuda:0")
    s = Sampler(B, V, torch.float32)
    out_idx = torch.empty(B, dtype=torch.int64, device=dev)
    counts = torch.full((2,), -1, dtype=torch.int32, device=dev)
    fl = torch.zeros(B, dtype=torch.uint8, device=dev)
    s.run(torch.from_numpy(x).to(dev), out_idx, row_flags=fl, counts=counts)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [B, 0]
    np.testing.assert_array_equal(out_idx.cpu().numpy(), np.argmax(x, axis=1))
    fin0 = (np.arange(B) % 4 == 1).astype(np.uint8) * 3
    eos = int(np.argmax(x[0]))
    fin = torch.from_numpy(fin0).to(dev)
    s.run(torch.from_numpy(x).to(dev), out_idx, row_flags=fl, finished=fin, eos_id=eos,
          counts=counts)
    torch.cuda.synchronize()
    e = orc.decode_epilogue(np.argmax(x, axis=1), fin0, eos)
    np.testing.assert_array_equal(out_idx.cpu().numpy(), e["idx"])
    np.testing.assert_array_equal(fin.cpu().numpy(), e["finished"])
    assert counts.cpu().tolist() == e["counts"].tolist()
    s.close()
