"""Helpers of the GPU parity tests: run a workload through the C ABI (HIP
path) and through the CPU oracle, and compare them with the parity rules:

* the output id is bit-exact on every row except sampling rows whose two
  largest ratios pi/(q+eps) are within 1e-5 (relative) of each other, and
  top-p boundary ties (a prefix mass within 1e-9 of p); those are counted;
* the dense filtered logits are bit-exact (so the kept sets are too) on every
  row that is not a top-p boundary tie;
* probabilities agree within 1e-5 absolute;
* with inverse-CDF sampling (uniforms u) the output id is bit-exact except
  where u lies within 1e-9 of a cumulative-probability boundary (counted).
"""
import numpy as np

from decode_token_sampling_row_amd import workloads as wl
from oracle import oracle as orc

GAP_TIE = 1e-5
MARGIN_TIE = 1e-9
U_TIE = 1e-9
PROB_ATOL = 1e-5


def device_inputs(W, ld_pad=0):
    import torch

    dev = torch.device("cuda:0")
    B, V = W.B, W.V
    if W.dtype == wl.BF16:
        x = torch.from_numpy(W.logits.view(np.int16)).view(torch.bfloat16)
    else:
        x = torch.from_numpy(W.logits)
    if ld_pad:
        buf = torch.zeros((B, V + ld_pad), dtype=x.dtype)
        buf[:, :V] = x
        x = buf.to(dev)[:, :V]
    else:
        x = x.to(dev)
    t = lambda a, dt: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return {
        "logits": x,
        "q": t(W.q, None),
        "top_k": t(W.top_k, None),
        "top_p": t(W.top_p, None),
        "row_flags": t(W.row_flags, None),
        "penalty_ids": t(W.ids, None),
        "penalty_offsets": t(W.offsets, None),
    }


def run_hip(W, need_logits=True, need_probs=False, guess=0, seg=0, ld_pad=0, sampler=None,
            inputs=None, rpl=0, u=None, drop_q=False, ties=False):
    import torch

    from decode_token_sampling_row_amd.sampler import Sampler

    d = inputs if inputs is not None else device_inputs(W, ld_pad)
    dev = d["logits"].device
    B, V = W.B, W.V
    out_idx = torch.full((B,), -7, dtype=torch.int64, device=dev)
    out_l = torch.full((B, V), 12345.0, dtype=torch.float32, device=dev) if need_logits else None
    out_p = torch.full((B, V), -1.0, dtype=torch.float32, device=dev) if need_probs else None
    s = sampler or Sampler(max(B, 1), V, torch.bfloat16 if W.dtype == wl.BF16 else torch.float32,
                           topk_guess=guess, segment_len=seg, rows_per_launch=rpl)
    ud = None if u is None else torch.from_numpy(np.ascontiguousarray(u, np.float32)).to(dev)
    s.run(d["logits"], out_idx, top_k=d["top_k"], top_p=d["top_p"],
          q=None if drop_q else d["q"], u=ud, eps=W.eps,
          temperature=W.temperature, repetition_penalty=W.penalty,
          penalty_ids=d["penalty_ids"], penalty_offsets=d["penalty_offsets"],
          row_flags=d["row_flags"], out_logits=out_l, out_probs=out_p, topk_ties=ties)
    torch.cuda.synchronize()
    res = {"idx": out_idx.cpu().numpy(),
           "logits": out_l.cpu().numpy() if need_logits else None,
           "probs": out_p.cpu().numpy() if need_probs else None}
    return res


def run_oracle(W, need_logits=True, need_probs=False, rows=None, threads=8, u=None,
               ties=False):
    return orc.run(W.logits, orc.BF16 if W.dtype == wl.BF16 else orc.F32, vocab=W.V,
                   top_k=W.top_k, top_p=W.top_p, q=W.q, eps=W.eps, temperature=W.temperature,
                   penalty=W.penalty, ids=W.ids, offsets=W.offsets, row_flags=W.row_flags,
                   need_logits=need_logits, need_probs=need_probs, rows=rows, threads=threads,
                   u=u, topk_ties=ties)


def compare(W, hip, ref, rows=None, label="", inverse=False, max_exempt=None):
    """Assert the parity rules on `rows` (default all); returns tie counts.
    inverse: the runs sampled by inverse CDF (ref["gap"] is then the u
    margin).  The rows exempted from the id check (near ties and top-p
    boundary ties, both decided by the oracle alone) may not exceed
    max_exempt, by default 1 % of the compared rows rounded down (so none on
    fewer than 100 rows): an exemption count above that would make the id
    check vacuous."""
    rows = np.arange(W.B) if rows is None else np.asarray(rows)
    flags = W.row_flags if W.row_flags is not None else np.full(W.B, 7, np.uint8)
    sampling = ((flags & 4) != 0) & (inverse or W.q is not None)
    margin_tie = ref["margin"] < MARGIN_TIE
    near = sampling & (ref["gap"] <= (U_TIE if inverse else GAP_TIE))
    n_margin = int(margin_tie[rows].sum())
    n_near = int(near[rows].sum())
    allowed = int(0.01 * rows.size) if max_exempt is None else int(max_exempt)
    exempt = int((margin_tie[rows] | near[rows]).sum())
    assert exempt <= allowed, (
        f"{label}: {exempt} of {rows.size} rows exempted from the id check "
        f"({n_near} near ties, {n_margin} top-p boundary ties), more than {allowed}")
    check_idx = rows[~margin_tie[rows] & ~near[rows]]
    bad = check_idx[hip["idx"][check_idx] != ref["idx"][check_idx]]
    assert bad.size == 0, (
        f"{label}: idx mismatch on rows {bad[:10].tolist()} hip={hip['idx'][bad[:10]].tolist()} "
        f"ref={ref['idx'][bad[:10]].tolist()} flags={flags[bad[:10]].tolist()}")
    exact_rows = rows[~margin_tie[rows]]
    if hip["logits"] is not None and ref["logits"] is not None:
        h = hip["logits"][exact_rows].view(np.uint32)
        r = ref["logits"][exact_rows].view(np.uint32)
        neq = np.nonzero((h != r).any(axis=1))[0]
        if neq.size:
            b = exact_rows[neq[0]]
            cols = np.nonzero(hip["logits"][b].view(np.uint32) != ref["logits"][b].view(np.uint32))[0]
            raise AssertionError(
                f"{label}: dense logits differ on {neq.size} rows, first row {b} "
                f"(flags {flags[b]}) at {cols.size} cols, e.g. col {cols[0]}: "
                f"hip={hip['logits'][b, cols[0]]} ref={ref['logits'][b, cols[0]]} "
                f"kept hip={np.isfinite(hip['logits'][b]).sum()} ref={np.isfinite(ref['logits'][b]).sum()}")
    if hip["probs"] is not None and ref["probs"] is not None:
        err = np.abs(hip["probs"][exact_rows] - ref["probs"][exact_rows]).max() if exact_rows.size else 0
        assert err <= PROB_ATOL, f"{label}: probs differ by {err}"
    return {"near_ties": n_near, "boundary_ties": n_margin, "rows": int(rows.size)}
