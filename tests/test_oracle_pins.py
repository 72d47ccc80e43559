"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a worked
example printed on a page (fixtures under tests/golden/, each with its
source), a closed form, brute-force enumeration on tiny inputs, an
independent statement of the same rule from another page, a library routine
the step reduces to, or a distributional law.  A plausible slip in the oracle
(a dropped term, a wrong sign or comparison, an off-by-one in the prefix, q
paired with the wrong candidate) fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TOPK, TOPP, SAMPLE = orc.ROW_TOPK, orc.ROW_TOPP, orc.ROW_SAMPLE


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def run_f32(x, flags, top_k=None, top_p=None, q=None, **kw):
    x = np.atleast_2d(np.asarray(x, np.float32))
    B = x.shape[0]
    flags = np.broadcast_to(np.asarray(flags, np.uint8), (B,)).copy()
    if top_k is not None:
        top_k = np.broadcast_to(np.asarray(top_k, np.int32), (B,)).copy()
    if top_p is not None:
        top_p = np.broadcast_to(np.asarray(top_p, np.float32), (B,)).copy()
    return orc.run(x, orc.F32, top_k=top_k, top_p=top_p, q=q, row_flags=flags, **kw)


def kept_set(out_logits_row):
    return set(np.nonzero(np.isfinite(out_logits_row))[0].tolist())


def precedes(x, i, j):
    """Total order of the row: larger value first, then smaller vocab id."""
    return x[i] > x[j] or (x[i] == x[j] and i < j)


# ---------------------------------------------------------------- worked examples

def test_topk_worked_example():
    g = _golden("minimind_topk_example.json")
    r = run_f32(g["logits"], TOPK, top_k=g["top_k"])
    want = np.array([-np.inf if v == "-inf" else v for v in g["filtered"]], np.float32)
    np.testing.assert_array_equal(r["logits"][0], want)
    assert r["nkept"][0] == g["top_k"]
    assert r["idx"][0] == int(np.argmax(g["logits"]))  # sample off -> greedy


def test_topp_worked_example():
    g = _golden("minimind_topp_example.json")
    x = np.log(np.array(g["sorted_probs"], np.float64)).astype(np.float32)
    r = run_f32(x, TOPP, top_p=g["top_p"], need_probs=True)
    assert r["nkept"][0] == g["kept"]
    assert kept_set(r["logits"][0]) == set(range(g["kept"]))
    # renormalised over the 3 kept tokens: 0.5/0.95, 0.3/0.95, 0.15/0.95
    kept_mass = sum(g["sorted_probs"][: g["kept"]])
    want = [p / kept_mass for p in g["sorted_probs"][: g["kept"]]] + [0.0, 0.0]
    np.testing.assert_allclose(r["probs"][0], want, atol=1e-6)
    # the printed cumulative column crosses 0.85 exactly at position 3
    cum = g["cumulative"]
    assert cum[g["kept"] - 2] < g["top_p"] <= cum[g["kept"] - 1]


def test_penalty_worked_example_and_dedup():
    g = _golden("minimind_penalty_example.json")
    x = [c[0] for c in g["cases"]]
    ids = np.array([0, 1, 0, 1, 0], np.int32)  # duplicates: penalised once
    r = run_f32(x, 0, penalty=g["penalty"], ids=ids, offsets=np.array([0, 5], np.int64))
    tol = 0.5 * 10 ** (-g["printed_decimals"])
    for j, (_, want) in enumerate(g["cases"]):
        assert abs(float(r["logits"][0][j]) - want) <= tol


def test_penalty_ignores_out_of_range_and_zero():
    x = [0.0, 3.0, -1.0, 2.0]
    ids = np.array([-1, 4, 100, 0, 1], np.int32)
    r = run_f32(x, 0, penalty=2.0, ids=ids, offsets=np.array([0, 5], np.int64))
    # id 0 (value 0) stays 0, id 1 halves, ids 2 and 3 are untouched
    np.testing.assert_array_equal(r["logits"][0], np.array([0.0, 1.5, -1.0, 2.0], np.float32))


def test_temperature_worked_example():
    g = _golden("minimind_temperature_example.json")
    for t_str, want in g["scaled"].items():
        r = run_f32(g["logits"], 0, temperature=float(t_str), need_probs=True)
        np.testing.assert_array_equal(r["logits"][0], np.array(want, np.float32))
        np.testing.assert_allclose(r["probs"][0], g["closed_form_probs"][t_str], atol=1e-4)
        printed = g["printed_probs_not_used"][t_str]
        assert abs(sum(printed) - 1.0) > 0.04  # the page's column is not a distribution


def test_negative_zero_is_canonical():
    r = run_f32([-0.0, 1.0, -0.0], 0)
    assert not np.signbit(r["logits"][0][0]) and not np.signbit(r["logits"][0][2])


def test_bf16_widening_matches_torch():
    import torch

    rng = np.random.default_rng(7)
    x = rng.standard_normal((3, 257)).astype(np.float32) * 5
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    r = orc.run(bits, orc.BF16, row_flags=np.zeros(3, np.uint8))
    np.testing.assert_array_equal(r["logits"], ref)


# ---------------------------------------------------------------- brute force

def _brute_topk(x, k):
    """The unique k-subset whose every member precedes every non-member."""
    V = len(x)
    found = []
    for S in itertools.combinations(range(V), k):
        Sset = set(S)
        if all(precedes(x, s, t) for s in S for t in range(V) if t not in Sset):
            found.append(Sset)
    assert len(found) == 1
    return found[0]


def _brute_nucleus(x, cand, p):
    """Smallest subset of ``cand`` that is closed upward under the order and
    whose softmax mass (renormalised over ``cand``) reaches p."""
    cand = sorted(cand)
    m = max(x[i] for i in cand)
    w = {i: math.exp(float(x[i]) - float(m)) for i in cand}
    Z = sum(w.values())
    best = None
    global _last_brute_dist
    _last_brute_dist = min(abs(sum(w[s] for s in S) / Z - p)
                           for r in range(1, len(cand) + 1)
                           for S in itertools.combinations(cand, r)
                           if all(s in set(S) for t in S for s in cand if precedes(x, s, t)))
    for r in range(1, len(cand) + 1):
        for S in itertools.combinations(cand, r):
            Sset = set(S)
            closed = all(s in Sset for t in S for s in cand if precedes(x, s, t))
            if not closed:
                continue
            mass = sum(w[s] for s in S) / Z
            if mass >= p:
                best = Sset
                break
        if best is not None:
            break
    return best


@pytest.mark.parametrize("seed", range(12))
def test_topk_brute_force_with_ties(seed):
    rng = np.random.default_rng(100 + seed)
    V = int(rng.integers(3, 9))
    x = rng.integers(-2, 3, size=V).astype(np.float32)  # many exact ties
    for k in range(1, V + 1):
        r = run_f32(x, TOPK, top_k=k)
        assert kept_set(r["logits"][0]) == _brute_topk(x, k)
        assert r["nkept"][0] == k


@pytest.mark.parametrize("seed", range(12))
def test_topk_keeping_ties_matches_minimind_topk(seed):
    """TOPK_TIES reading: the MiniMind chapter's own top-k line (mask the
    logits below the k-th value of torch.topk) gives the kept set, ties at
    the k-th value included."""
    rng = np.random.default_rng(150 + seed)
    B, V = 6, int(rng.integers(5, 60))
    x = rng.integers(-3, 4, size=(B, V)).astype(np.float32)  # many exact ties
    for k in sorted({1, 2, V // 3 + 1, V // 2 + 1, V}):
        r = run_f32(x, TOPK, top_k=k, topk_ties=True)
        for b in range(B):
            mm = _minimind_chain(x[b], k, 1.0)
            assert kept_set(r["logits"][b]) == set(np.nonzero(np.isfinite(mm))[0].tolist())
            kth = np.sort(x[b])[::-1][k - 1]
            assert r["nkept"][b] == int(np.sum(x[b] >= kth))
    # without the flag exactly k survive
    r = run_f32(x, TOPK, top_k=3)
    assert np.all(r["nkept"] == 3)


@pytest.mark.parametrize("seed", range(12))
def test_topp_brute_force(seed):
    rng = np.random.default_rng(200 + seed)
    V = int(rng.integers(2, 10))
    x = (rng.integers(-3, 4, size=V) * 0.7).astype(np.float32)  # ties again
    for p in [0.05, 0.3, 0.5, 0.77, 0.9, 0.99]:
        r = run_f32(x, TOPP, top_p=p)
        want = _brute_nucleus(x, range(V), p)
        if _last_brute_dist < 1e-9:
            continue
        assert kept_set(r["logits"][0]) == want
    # top-k then top-p: the nucleus is taken within the k survivors
    for k in range(1, V + 1):
        for p in [0.4, 0.8]:
            r = run_f32(x, TOPK | TOPP, top_k=k, top_p=p)
            want = _brute_nucleus(x, _brute_topk(x, k), p)
            if _last_brute_dist < 1e-9:
                continue
            assert kept_set(r["logits"][0]) == want


# ---------------------------------------------------------------- independent statements

_last_brute_dist = None


def _near_boundary(probs_sorted, p, tol=1e-9):
    """True when some prefix mass of the sorted probabilities is within tol
    of p (a top-p boundary tie, excluded from exact comparisons)."""
    cum = np.cumsum(np.asarray(probs_sorted, np.float64))
    return bool(np.min(np.abs(cum - p)) < tol)


def _quickselect_nucleus_size(probs, p):
    """Nucleus size by repeated partitioning around a pivot, the idea the C++
    post-processing blog describes for top_p (expected linear time): split the
    live range into entries above the pivot and the rest; if the upper part
    already holds mass p, recurse into it, otherwise take it whole, subtract
    its mass and the pivot's, and continue below."""
    vals = list(probs)
    lo_taken = 0
    target = p
    live = vals
    while True:
        if len(live) == 1:
            return lo_taken + 1
        pivot = live[-1]
        upper = [v for v in live[:-1] if v > pivot]
        lower = [v for v in live[:-1] if v <= pivot]
        s_up = sum(upper)
        if s_up >= target:
            live = upper
        elif s_up + pivot < target:
            lo_taken += len(upper) + 1
            target -= s_up + pivot
            live = lower
            if not live:
                return lo_taken
        else:
            return lo_taken + len(upper) + 1


@pytest.mark.parametrize("seed", range(6))
def test_topp_matches_quickselect_partition(seed):
    rng = np.random.default_rng(300 + seed)
    V = int(rng.integers(50, 2000))
    x = (rng.standard_normal(V) * rng.uniform(0.2, 3.0)).astype(np.float32)
    e = np.exp(x.astype(np.float64) - x.max())
    probs = e / e.sum()
    for p in [0.1, 0.5, 0.85, 0.95]:
        r = run_f32(x, TOPP, top_p=p)
        if _near_boundary(np.sort(probs)[::-1], p):
            continue
        assert r["nkept"][0] == _quickselect_nucleus_size(probs.tolist(), p)


@pytest.mark.parametrize("seed", range(6))
def test_topp_matches_ascend_fallback_mask(seed):
    """Ascend page, top-p fallback: sort descending, cumsum, and drop entry v
    when (cumsum - sorted)[v] > top_p.  On rows where no exclusive prefix sits
    exactly at p this keeps the same prefix as the shortest-prefix rule."""
    rng = np.random.default_rng(400 + seed)
    V = int(rng.integers(50, 3000))
    x = (rng.standard_normal(V) * 2).astype(np.float32)
    srt = np.sort(x.astype(np.float64))[::-1]
    pr = np.exp(srt - srt[0])
    pr /= pr.sum()
    excl = np.cumsum(pr) - pr
    for p in [0.2, 0.6, 0.9]:
        keep = int(np.sum(~(excl > p)))
        r = run_f32(x, TOPP, top_p=p)
        if _near_boundary(pr, p):
            continue
        assert r["nkept"][0] == keep


def _tie_free(rng, V, scale):
    while True:
        x = (rng.standard_normal(V) * scale).astype(np.float32)
        if len(np.unique(x)) == V:
            return x


def _minimind_chain(x, k, p):
    """top-k then top-p as the MiniMind chapter states them with torch ops:
    mask below the k-th largest value, then sort, softmax, cumsum, remove
    where the cumulative mass before an entry already exceeds p."""
    import torch

    t = torch.from_numpy(np.asarray(x, np.float32)).clone().unsqueeze(0)
    if k > 0:
        kth = torch.topk(t, k).values[..., -1:]
        t = t.masked_fill(t < kth, float("-inf"))
    if p < 1.0:
        vals, order = torch.sort(t, descending=True)
        cum = torch.cumsum(torch.softmax(vals.double(), dim=-1), dim=-1)
        drop = torch.zeros_like(cum, dtype=torch.bool)
        drop[..., 1:] = cum[..., :-1] > p
        mask = torch.zeros_like(drop).scatter(1, order, drop)
        t = t.masked_fill(mask, float("-inf"))
    return t[0].numpy()


@pytest.mark.parametrize("seed", range(8))
def test_matches_minimind_chain_on_tie_free_rows(seed):
    rng = np.random.default_rng(500 + seed)
    V = int(rng.integers(100, 5000))
    x = _tie_free(rng, V, 2.0)
    for k, p in [(0, 0.9), (50, 1.0), (50, 0.85), (7, 0.3), (min(V, 1024), 0.97)]:
        flags = (TOPK if k > 0 else 0) | (TOPP if p < 1 else 0)
        r = run_f32(x, flags, top_k=k, top_p=p)
        srt = np.sort(x.astype(np.float64))[::-1][: (k if k > 0 else V)]
        w = np.exp(srt - srt[0])
        if p < 1 and _near_boundary(w / w.sum(), p):
            continue
        np.testing.assert_array_equal(r["logits"][0], _minimind_chain(x, k, p))


# ---------------------------------------------------------------- sampling law

def _chi2_ok(counts, probs, n):
    from scipy.stats import chi2

    exp = probs * n
    stat = float(np.sum((counts - exp) ** 2 / exp))
    return chi2.sf(stat, len(probs) - 1) > 1e-4, stat


@pytest.mark.parametrize("k,p", [(0, 1.0), (3, 1.0), (0, 0.8), (4, 0.7)])
def test_exponential_race_law(k, p):
    """For iid q ~ Exp(1), argmax pi_i / q_i picks i with probability pi_i
    (the exponential race; equivalent to Gumbel-max sampling)."""
    x = np.array([1.0, 0.5, 0.0, -0.5, 2.0, 0.25], np.float32)
    n = 60000
    rng = np.random.default_rng(600)
    X = np.tile(x, (n, 1))
    q = rng.standard_exponential((n, x.size)).astype(np.float32)
    flags = SAMPLE | (TOPK if k else 0) | (TOPP if p < 1 else 0)
    r = run_f32(X, flags, top_k=k, top_p=p, q=q, eps=1e-20, need_logits=False, threads=4)
    # expected law: softmax over the kept set, worked out independently
    order = sorted(range(x.size), key=lambda i: (-x[i], i))
    cand = order[:k] if k else order
    w = np.exp(x[cand].astype(np.float64) - x[cand[0]])
    mass = np.cumsum(w) / w.sum()
    nk = len(cand) if p >= 1 else int(np.argmax(mass >= p)) + 1
    keep = cand[:nk]
    pk = w[:nk] / w[:nk].sum()
    counts = np.array([np.sum(r["idx"] == i) for i in keep], np.float64)
    assert counts.sum() == n  # never outside the kept set
    ok, stat = _chi2_ok(counts, pk, n)
    assert ok, (stat, counts, pk * n)


@pytest.mark.parametrize("k,p", [(0, 1.0), (3, 1.0), (4, 0.7)])
def test_inverse_cdf_law(k, p):
    """With u ~ U(0, 1), the inverse-CDF draw picks i with probability pi_i
    (MiniMind sec. 10.8: a multinomial draw from the filtered softmax)."""
    x = np.array([1.0, 0.5, 0.0, -0.5, 2.0, 0.25], np.float32)
    n = 60000
    rng = np.random.default_rng(610)
    X = np.tile(x, (n, 1))
    u = rng.random(n).astype(np.float32)
    flags = SAMPLE | (TOPK if k else 0) | (TOPP if p < 1 else 0)
    r = run_f32(X, flags, top_k=k, top_p=p, u=u, need_logits=False, threads=4)
    order = sorted(range(x.size), key=lambda i: (-x[i], i))
    cand = order[:k] if k else order
    w = np.exp(x[cand].astype(np.float64) - x[cand[0]])
    mass = np.cumsum(w) / w.sum()
    nk = len(cand) if p >= 1 else int(np.argmax(mass >= p)) + 1
    keep = cand[:nk]
    pk = w[:nk] / w[:nk].sum()
    counts = np.array([np.sum(r["idx"] == i) for i in keep], np.float64)
    assert counts.sum() == n
    ok, stat = _chi2_ok(counts, pk, n)
    assert ok, (stat, counts, pk * n)


def test_inverse_cdf_maps_u_intervals_of_length_pi():
    """Sweeping u over a fine grid, each kept element is drawn on one interval
    of u, in the row's order, whose length is its probability."""
    rng = np.random.default_rng(611)
    x = rng.normal(0.0, 1.0, 40).astype(np.float32)
    x[[3, 9, 17]] = x[5]  # ties: equal values go to the smaller id first
    g = 20001
    u = ((np.arange(g) + 0.5) / g).astype(np.float32)
    X = np.tile(x, (g, 1))
    r = run_f32(X, TOPK | SAMPLE, top_k=12, u=u, need_logits=False, need_probs=True)
    order = sorted(range(x.size), key=lambda i: (-x[i], i))
    pos = {v: n for n, v in enumerate(order)}
    drawn = np.array([pos[int(i)] for i in r["idx"]])
    assert np.all(np.diff(drawn) >= 0)  # non-decreasing position in the order
    assert drawn.max() <= 11
    probs = r["probs"][0]
    for n, i in enumerate(order[:12]):
        width = np.sum(drawn == n) / g
        assert abs(width - probs[i]) <= 2.0 / g, (n, width, probs[i])


def test_inverse_cdf_endpoints_and_greedy_cases():
    rng = np.random.default_rng(612)
    B, V = 30, 200
    x = rng.integers(-4, 5, size=(B, V)).astype(np.float32)  # heavy ties
    greedy = np.argmax(x, axis=1)
    for uv in [0.0, -0.5, float("nan")]:
        r = run_f32(x, TOPK | TOPP | SAMPLE, top_k=50, top_p=0.9,
                    u=np.full(B, uv, np.float32), need_logits=False)
        np.testing.assert_array_equal(r["idx"], greedy)
    # k = 1: the draw is the argmax whatever u is
    r = run_f32(x, TOPK | SAMPLE, top_k=1, u=rng.random(B).astype(np.float32),
                need_logits=False)
    np.testing.assert_array_equal(r["idx"], greedy)
    # u just below 1: the last element of K (here the k-th of the order)
    r = run_f32(x, TOPK | SAMPLE, top_k=7, u=np.full(B, np.nextafter(np.float32(1), 0)),
                need_logits=True)
    for b in range(B):
        order = sorted(range(V), key=lambda i: (-x[b, i], i))
        assert r["idx"][b] == order[6]
    # equal values: K is uniform, the draw for u in ((n-1)/|K|, n/|K|) is
    # the n-th smallest id of K
    xe = np.zeros((8, 50), np.float32)
    ue = ((np.arange(8) + 0.5) / 10.0).astype(np.float32)
    r = run_f32(xe, TOPK | SAMPLE, top_k=10, u=ue, need_logits=False)
    np.testing.assert_array_equal(r["idx"], np.arange(8))


def test_k1_and_constant_q_and_sample_off_are_greedy():
    rng = np.random.default_rng(700)
    B, V = 40, 300
    x = rng.integers(-5, 6, size=(B, V)).astype(np.float32)  # heavy ties
    greedy = np.argmax(x, axis=1)  # first occurrence of the max
    q = rng.standard_exponential((B, V)).astype(np.float32)
    r = run_f32(x, TOPK | SAMPLE, top_k=1, q=q)
    np.testing.assert_array_equal(r["idx"], greedy)
    qc = np.full((B, V), 0.7, np.float32)
    r = run_f32(x, TOPK | TOPP | SAMPLE, top_k=20, top_p=0.9, q=qc)
    np.testing.assert_array_equal(r["idx"], greedy)
    r = run_f32(x, TOPK | TOPP, top_k=20, top_p=0.9, q=q)
    np.testing.assert_array_equal(r["idx"], greedy)


# ---------------------------------------------------------------- invariants

def test_skipped_stage_is_identity():
    rng = np.random.default_rng(800)
    for V in [10, 700, 3000]:
        x = (rng.standard_normal((3, V)) * 2).astype(np.float32)
        q = rng.standard_exponential((3, V)).astype(np.float32)
        base = run_f32(x, TOPP | SAMPLE, top_p=0.8, q=q)
        for k in [0, -3, 1025, V + 1]:
            if 1 <= k <= min(V, 1024):
                continue
            r = run_f32(x, TOPK | TOPP | SAMPLE, top_k=k, top_p=0.8, q=q)
            np.testing.assert_array_equal(r["idx"], base["idx"])
            np.testing.assert_array_equal(r["logits"], base["logits"])
        nop = run_f32(x, SAMPLE, q=q)
        for p in [1.0, 1.5, float("nan")]:
            r = run_f32(x, TOPP | SAMPLE, top_p=p, q=q)
            np.testing.assert_array_equal(r["idx"], nop["idx"])
            np.testing.assert_array_equal(r["logits"], nop["logits"])
        np.testing.assert_array_equal(nop["logits"], x)


@pytest.mark.parametrize("seed", range(4))
def test_kept_set_is_minimal_prefix(seed):
    rng = np.random.default_rng(900 + seed)
    B, V = 16, 4000
    x = (rng.standard_normal((B, V)) * rng.uniform(0.1, 4.0, size=(B, 1))).astype(np.float32)
    k = rng.integers(1, 1025, size=B).astype(np.int32)
    p = rng.uniform(0.05, 0.999, size=B).astype(np.float32)
    r = run_f32(x, TOPK | TOPP, top_k=k, top_p=p, need_probs=True)
    for b in range(B):
        K = np.nonzero(np.isfinite(r["logits"][b]))[0]
        assert 1 <= len(K) <= k[b]
        # every kept entry precedes every dropped entry of the row
        xs = x[b]
        worst_kept = min(K, key=lambda i: (-xs[i], i))
        dropped = np.setdiff1d(np.arange(V), K)
        assert all(precedes(xs, worst_kept, t) for t in dropped[:200])
        # mass of K within the top-k set reaches p; without its last entry it does not
        order = sorted(range(V), key=lambda i: (-xs[i], i))[: k[b]]
        w = np.exp(xs[order].astype(np.float64) - xs[order[0]])
        w /= w.sum()
        if _near_boundary(w, p[b]):
            continue
        # the oracle's reported margin is the distance of the two bracketing
        # prefix masses to p
        cum = np.cumsum(w)
        n_ = len(K)
        want_margin = cum[n_ - 1] - p[b] if n_ == 1 else min(cum[n_ - 1] - p[b], p[b] - cum[n_ - 2])
        assert abs(r["margin"][b] - want_margin) < 1e-9
        n = len(K)
        assert w[:n].sum() >= p[b] - 1e-12
        assert n == 1 or w[: n - 1].sum() < p[b] + 1e-12
        np.testing.assert_allclose(r["probs"][b][order[:n]], w[:n] / w[:n].sum(), atol=1e-7)


def test_permutation_equivariance():
    """Permuting vocab columns of logits and q together permutes the output:
    q is paired with candidates by vocab id, not by sorted position."""
    rng = np.random.default_rng(1000)
    B, V = 64, 500
    x = (rng.standard_normal((B, V)) * 1.5).astype(np.float32)
    q = rng.standard_exponential((B, V)).astype(np.float32)
    perm = rng.permutation(V)
    r0 = run_f32(x, TOPK | TOPP | SAMPLE, top_k=100, top_p=0.9, q=q)
    r1 = run_f32(x[:, perm], TOPK | TOPP | SAMPLE, top_k=100, top_p=0.9, q=q[:, perm])
    ok = r0["gap"] > 1e-5
    np.testing.assert_array_equal(perm[r1["idx"][ok]], r0["idx"][ok])
    np.testing.assert_array_equal(r1["logits"], r0["logits"][:, perm])


def test_row_range_and_threads_do_not_change_results():
    rng = np.random.default_rng(1100)
    B, V = 23, 1000
    x = (rng.standard_normal((B, V)) * 2).astype(np.float32)
    q = rng.standard_exponential((B, V)).astype(np.float32)
    a = run_f32(x, 7, top_k=30, top_p=0.9, q=q, threads=1)
    b = run_f32(x, 7, top_k=30, top_p=0.9, q=q, threads=5)
    c = run_f32(x, 7, top_k=30, top_p=0.9, q=q, rows=range(B))
    for key in ["idx", "logits", "nkept", "gap", "margin"]:
        np.testing.assert_array_equal(a[key], b[key])
        np.testing.assert_array_equal(a[key], c[key])


def test_topk_range_boundary():
    """Valid range 1 <= k <= min(V, 1024) (Ascend page, topK range rule)."""
    rng = np.random.default_rng(1200)
    x = _tie_free(rng, 3000, 1.0)
    assert run_f32(x, TOPK, top_k=1024)["nkept"][0] == 1024
    assert run_f32(x, TOPK, top_k=1025)["nkept"][0] == 3000
    assert run_f32(x, TOPK, top_k=1)["nkept"][0] == 1
    y = x[:700]
    assert run_f32(y, TOPK, top_k=700)["nkept"][0] == 700
    assert run_f32(y, TOPK, top_k=699)["nkept"][0] == 699


# ---------------------------------------------------------------- decode-step epilogue

def _history(prompt, cap, junk):
    """CSR history slots: row b holds prompt[b] then junk up to cap ids."""
    B = len(prompt)
    ids = np.zeros(B * cap, np.int32)
    for b in range(B):
        ids[b * cap:(b + 1) * cap] = junk[b]
        ids[b * cap:b * cap + len(prompt[b])] = prompt[b]
    offsets = np.arange(B + 1, dtype=np.int64) * cap
    lens = np.array([len(p) for p in prompt], np.int32)
    return ids, offsets, lens


def test_eos_batch_table():
    """The batch illustration of the EOS section: greedy draws that name the
    table's tokens (a non-EOS token where the table shows a forced EOS), run
    through the oracle and its epilogue, reproduce every cell, the finished
    column, and the loop's end after step 6."""
    g = _golden("minimind_eos_batch_table.json")
    eos, V, B = g["eos_token_id"], 32, 3
    tok = {f"tok_{c}": 10 + i for i, c in enumerate("abcdefghi")}
    prompt = [[5, 6, 7]] * B
    ids, offsets, lens = _history(prompt, 3 + len(g["steps"]), [31] * B)
    fin = np.zeros(B, np.uint8)
    for st in g["steps"]:
        raw = [20 + st["step"] if st["forced"][b] else (eos if st["tokens"][b] == "EOS" else tok[st["tokens"][b]])
               for b in range(B)]
        x = np.zeros((B, V), np.float32)
        x[np.arange(B), raw] = 5.0
        r = run_f32(x, 0)
        assert r["idx"].tolist() == raw
        e = orc.decode_epilogue(r["idx"], fin, eos, ids, offsets, lens, append=True)
        want = [eos if t == "EOS" else tok[t] for t in st["tokens"]]
        assert e["idx"].tolist() == want
        assert [bool(f) for f in e["finished"]] == st["finished"]
        assert (e["counts"][0] == 0) == (st["step"] == g["loop_ends_after_step"])
        assert e["counts"][1] == 0
        fin, ids, lens = e["finished"], e["ids"], e["lens"]
    for b in range(B):
        col = [eos if s["tokens"][b] == "EOS" else tok[s["tokens"][b]] for s in g["steps"]]
        assert ids[offsets[b]:offsets[b] + lens[b]].tolist() == prompt[b] + col


def _minimind_greedy_loop(step_logits, prompt, rho, temperature, eos):
    """The MiniMind generate loop with do_sample=False, in torch: temperature,
    penalty over torch.unique of the whole sequence, argmax, EOS forcing,
    concatenation, finished update and the all-finished break."""
    import torch

    input_ids = torch.tensor(prompt, dtype=torch.int64)
    finished = torch.zeros(input_ids.shape[0], dtype=torch.bool)
    for x in step_logits:
        logits = torch.from_numpy(x.copy()) / temperature
        for i in range(input_ids.shape[0]):
            seen = torch.unique(input_ids[i])
            score = logits[i, seen]
            logits[i, seen] = torch.where(score > 0, score / rho, score * rho)
        nxt = torch.argmax(logits, dim=-1, keepdim=True)
        nxt = torch.where(finished.unsqueeze(-1), nxt.new_full((nxt.shape[0], 1), eos), nxt)
        input_ids = torch.cat([input_ids, nxt], dim=-1)
        finished |= nxt.squeeze(-1).eq(eos)
        if finished.all():
            break
    return input_ids.numpy()


@pytest.mark.parametrize("seed", range(4))
def test_greedy_decode_loop_matches_minimind_loop(seed):
    """Several decode steps of the oracle with its epilogue (penalty reads
    only the filled part of each history slot, the slot's tail holds ids
    that must not be penalised) against the MiniMind loop in torch.  The
    temperature is a power of two, so that its division commutes exactly
    with the penalty (the loop divides first, the library penalises first)."""
    rng = np.random.default_rng(1300 + seed)
    B, V, P, S, eos = 6, 40, 5, 14, 2
    base = rng.standard_normal((B, V)).astype(np.float32) * 2
    base[:, eos] = -4.0
    steps = []
    for s in range(S):
        x = base + rng.standard_normal((B, V)).astype(np.float32) * 0.3
        x[:, eos] += np.float32(0.6) * s * (1 + np.arange(B)) / B
        steps.append(x.astype(np.float32))
    prompt = rng.integers(3, V, (B, P)).tolist()
    junk = [int(np.argmax(base[b])) for b in range(B)]  # would change the draws if read
    ids, offsets, lens = _history(prompt, P + S, junk)
    want = _minimind_greedy_loop(steps, prompt, 1.3, 0.5, eos)
    fin = np.zeros(B, np.uint8)
    n = 0
    for x in steps:
        r = run_f32(x, 0, temperature=0.5, penalty=1.3, ids=ids, offsets=offsets, lens=lens)
        e = orc.decode_epilogue(r["idx"], fin, eos, ids, offsets, lens, append=True)
        fin, ids, lens = e["finished"], e["ids"], e["lens"]
        n += 1
        if e["counts"][0] == 0:
            break
    assert want.shape[1] == P + n
    assert n < S or not fin.all()
    for b in range(B):
        assert ids[offsets[b]:offsets[b] + lens[b]].tolist() == want[b].tolist()


def test_epilogue_full_slots_and_no_eos():
    """Appends to a full slot are dropped and counted; without finished
    flags every row counts as unfinished and no output is replaced."""
    idx = np.array([4, 2, 9, 2])
    ids = np.arange(8, dtype=np.int32)
    offsets = np.array([0, 2, 4, 6, 8])
    lens = np.array([2, 1, 5, -3], np.int32)  # full, room, beyond cap, negative -> 0
    e = orc.decode_epilogue(idx, None, None, ids, offsets, lens, append=True)
    assert e["idx"].tolist() == idx.tolist()
    assert e["counts"].tolist() == [4, 2]
    assert e["lens"].tolist() == [2, 2, 5, 1]
    assert e["ids"].tolist() == [0, 1, 2, 2, 4, 5, 2, 7]
    e = orc.decode_epilogue(idx, np.array([0, 0, 3, 0], np.uint8), 9)
    assert e["idx"].tolist() == [4, 2, 9, 2]
    assert e["finished"].tolist() == [0, 0, 3, 0]
    assert e["counts"].tolist() == [3, 0]


# ---------------------------------------------------------------- the gap diagnostic
#
# The GPU parity tests exempt a sampling row from the id check only when the
# oracle's `gap` says the decision is a near tie, so `gap` itself is pinned
# here against an independent numpy statement of the same quantities: the
# kept set from a lexicographic sort, the ratios pi / (q + eps) over it
# (Ascend page, Sample section), and for inverse-CDF draws the distance of u
# to the nearest cumulative-probability boundary.

def _numpy_kept(x, k, p):
    """Kept ids of one row in the order (value desc, id asc), numpy only."""
    V = x.size
    order = np.lexsort((np.arange(V), -x.astype(np.float64)))
    if 1 <= k <= min(V, 1024):
        order = order[:k]
    if p < 1.0:
        e = np.exp(x[order].astype(np.float64) - float(x[order[0]]))
        S = np.cumsum(e) / e.sum()
        n = int(np.searchsorted(S >= p, True)) + 1 if (S >= p).any() else order.size
        order = order[:n]
    return order


def _numpy_race_gap(x, q, eps, kept):
    e = np.exp(x[kept].astype(np.float64) - float(x[kept[0]]))
    den = q[kept].astype(np.float64) + float(eps)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(np.isneginf(x[kept]), 0.0,
                     np.where(den == 0.0, np.inf, (e / e.sum()) / den))
    best = int(kept[np.lexsort((kept, -r))[0]])
    if kept.size < 2:
        return best, np.inf
    r1, r2 = np.sort(r)[::-1][:2]
    if np.isinf(r1):
        return best, np.inf
    return best, (r1 - r2) / r1


@pytest.mark.parametrize("seed", range(6))
def test_gap_is_the_relative_ratio_gap(seed):
    rng = np.random.default_rng(500 + seed)
    B, V = 24, 700
    x = (rng.standard_normal((B, V)) * (0.5 + seed)).astype(np.float32)
    if seed % 2:
        x = np.round(x * 2) / 2  # many exact value ties
    q = rng.standard_exponential((B, V)).astype(np.float32)
    # a few rows with two candidates at an almost equal ratio
    q[3, :] = 1.0
    x[3, 10] = x[3].max() + 1.0
    x[3, 11] = x[3, 10]
    k = rng.integers(0, 40, size=B).astype(np.int32)
    p = rng.uniform(0.3, 1.0, size=B).astype(np.float32)
    eps = 1e-20
    r = run_f32(x, 7, top_k=k, top_p=p, q=q, eps=eps)
    for b in range(B):
        kept = _numpy_kept(x[b], int(k[b]), float(p[b]))
        assert r["nkept"][b] == kept.size
        idx, gap = _numpy_race_gap(x[b], q[b], eps, kept)
        assert r["idx"][b] == idx
        if np.isinf(gap):
            assert np.isinf(r["gap"][b])
        else:
            assert r["gap"][b] == pytest.approx(gap, rel=1e-9, abs=1e-15), b
    assert r["gap"][3] == 0.0  # exact tie: exempt on the GPU side


def test_gap_with_zero_denominators():
    """eps = 0 and exact zeros in q: a finite logit's ratio is +inf there,
    ties among them go to the lowest id and count as decided (gap +inf); a
    -inf logit never wins whatever its q."""
    rng = np.random.default_rng(77)
    B, V = 8, 300
    x = (rng.standard_normal((B, V)) * 20).astype(np.float32)
    q = rng.standard_exponential((B, V)).astype(np.float32)
    q[0, [17, 250]] = 0.0           # two zero-q tokens: the lower id wins
    q[1, 5] = 0.0                   # one, far down the order
    x[1, 5] = x[1].min() - 900.0    # its double exponential underflows
    q[2, 9] = 0.0
    x[2, 9] = -np.inf               # probability 0: never drawn
    r = run_f32(x, SAMPLE, q=q, eps=0.0)
    assert r["idx"][0] == 17 and np.isinf(r["gap"][0])
    assert r["idx"][1] == 5 and np.isinf(r["gap"][1])
    assert r["idx"][2] != 9
    for b in range(B):
        kept = np.lexsort((np.arange(V), -x[b].astype(np.float64)))
        idx, gap = _numpy_race_gap(x[b], q[b], 0.0, kept)
        assert r["idx"][b] == idx
        if np.isfinite(gap):
            assert r["gap"][b] == pytest.approx(gap, rel=1e-9)


@pytest.mark.parametrize("seed", range(4))
def test_inverse_cdf_gap_is_the_distance_to_the_nearest_boundary(seed):
    rng = np.random.default_rng(600 + seed)
    B, V = 16, 400
    x = (rng.standard_normal((B, V)) * 1.5).astype(np.float32)
    k = rng.integers(0, 60, size=B).astype(np.int32)
    p = rng.uniform(0.4, 1.0, size=B).astype(np.float32)
    u = rng.random(B).astype(np.float32)
    u[0] = 0.0
    r = run_f32(x, 7, top_k=k, top_p=p, u=u)
    for b in range(B):
        kept = _numpy_kept(x[b], int(k[b]), float(p[b]))
        e = np.exp(x[b, kept].astype(np.float64) - float(x[b, kept[0]]))
        S = np.cumsum(e / e.sum())
        uu = float(u[b])
        if uu <= 0.0:
            assert r["idx"][b] == kept[0] and np.isinf(r["gap"][b])
            continue
        hit = np.nonzero(S >= uu)[0]
        n = int(hit[0]) + 1 if hit.size else kept.size
        assert r["idx"][b] == kept[n - 1]
        below = S[n - 2] if n > 1 else None
        want = S[n - 1] - uu if below is None else min(S[n - 1] - uu, uu - below)
        assert r["gap"][b] == pytest.approx(max(want, 0.0), rel=1e-6, abs=1e-12), b
