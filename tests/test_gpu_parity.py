"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Seeded inputs from ``workloads``; reduced sizes compare every row, the full
sizes compare sampled rows in the launch configuration the benchmark uses.
Edge cases: tiny and ragged vocabularies, segment boundaries, k = V, exact
ties everywhere, signed zeros and -inf, padded row strides, every stage
combination, top-p boundary cases that need the full-row search, and the
tuning knobs (guess size, segment length), which must not change anything.
"""
import numpy as np
import pytest

from decode_token_sampling_row_amd import workloads as wl

from gpu_util import compare, device_inputs, run_hip, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    from decode_token_sampling_row_amd import sampler

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sampler.load_library()  # fails loudly when the HIP library is missing
    yield


def _log(label, stats):
    print(f"[parity] {label}: {stats}", flush=True)


SMALL = [
    ("cfg1_full", 1, None, None),
    ("cfg4_full", 4, None, None),
    ("cfg2_B24_V20008", 2, 24, 20008),
    ("cfg2_B12_V20011_unaligned", 2, 12, 20011),
    ("cfg3_B16_V30000", 3, 16, 30000),
    ("cfg5_B32_V40000", 5, 32, 40000),
    ("cfg4_B64_V6403_unaligned", 4, 64, 6403),
    ("cfg1_B8_V70000", 1, 8, 70000),
]


@pytest.mark.parametrize("label,cfg,B,V", SMALL, ids=[s[0] for s in SMALL])
def test_parity_every_row(label, cfg, B, V):
    W = wl.make(cfg, B=B, V=V, seed=1)
    print(f"[case] {label} B={W.B} V={W.V} dtype={W.dtype}", flush=True)
    hip = run_hip(W, need_logits=True, need_probs=True)
    ref = run_oracle(W, need_logits=True, need_probs=True)
    _log(label, compare(W, hip, ref, label=label))


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_parity_full_size_every_row(cfg):
    """Every row of each workload at its full size, in the launch
    configuration the benchmark times (one call over the whole batch); the
    oracle and the comparison go in chunks of rows to bound host memory."""
    import torch

    W = wl.make(cfg, seed=0)
    print(f"[case] full cfg{cfg} B={W.B} V={W.V}", flush=True)
    hip = run_hip(W, need_logits=W.need_logits)
    chunk = 64
    tot = {"near_ties": 0, "boundary_ties": 0, "rows": 0}
    for r0 in range(0, W.B, chunk):
        rows = np.arange(r0, min(W.B, r0 + chunk))
        ref = run_oracle(W, need_logits=W.need_logits, rows=rows, threads=16)
        st = compare(W, hip, ref, rows=rows, label=f"full cfg{cfg} rows {r0}..",
                     max_exempt=rows.size)  # the bound applies to the whole batch below
        for k in tot:
            tot[k] += st[k]
        del ref
    _log(f"full cfg{cfg}", tot)
    assert tot["near_ties"] + tot["boundary_ties"] <= int(0.01 * W.B)
    torch.cuda.empty_cache()


def _custom(x, top_k=None, top_p=None, flags=7, q=None, dtype=wl.F32, seed=0, **kw):
    x = np.asarray(x, np.float32)
    B, V = x.shape
    rng = np.random.default_rng(seed)
    if q is None:
        q = rng.standard_exponential((B, V)).astype(np.float32)
    logits = wl.to_bf16_bits(x) if dtype == wl.BF16 else x
    bc = lambda v, dt: None if v is None else np.broadcast_to(np.asarray(v, dt), (B,)).copy()
    return wl.Workload("custom", B, V, dtype, logits, q, bc(top_k, np.int32),
                       bc(top_p, np.float32), bc(flags, np.uint8), **kw)


def _check(W, label, need_probs=True, max_exempt=None, **kw):
    print(f"[case] {label} B={W.B} V={W.V}", flush=True)
    hip = run_hip(W, need_logits=True, need_probs=need_probs, **kw)
    ref = run_oracle(W, need_logits=True, need_probs=need_probs)
    _log(label, compare(W, hip, ref, label=label, max_exempt=max_exempt))
    return hip, ref


def _all_combos(B):
    return (np.arange(B) % 8).astype(np.uint8)


@pytest.mark.parametrize("V", [1, 2, 5, 63, 64, 65, 256, 257, 1000, 2047, 2048, 2049])
@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_tiny_and_ragged_vocab(V, dtype):
    rng = np.random.default_rng(V)
    B = 16
    x = (rng.standard_normal((B, V)) * 2).astype(np.float32)
    k = rng.integers(0, min(V, 1024) + 2, size=B)
    p = rng.uniform(0.0, 1.0, size=B)
    W = _custom(x, top_k=k, top_p=p, flags=_all_combos(B), dtype=dtype)
    _check(W, f"tiny V={V} {dtype}")


@pytest.mark.parametrize("V", [8191, 8192, 8193, 32768, 32769])
def test_segment_boundaries(V):
    rng = np.random.default_rng(V)
    B = 16
    x = (rng.standard_normal((B, V)) * 3).astype(np.float32)
    k = np.array([1, 2, 50, 1023, 1024, 1024, 0, 7] * 2)
    W = _custom(x, top_k=k, top_p=0.9, flags=_all_combos(B))
    _check(W, f"segments V={V}")


@pytest.mark.parametrize("seg", [0, 1024])
def test_largest_vocab(seg):
    """V = 2^21, the largest the library accepts; with 1024-element tiles a
    wave's sub-slot holds a single candidate, so many rows overflow and take
    the full-row search."""
    rng = np.random.default_rng(41)
    B, V = 8, 1 << 21
    x = (rng.standard_normal((B, V)) * 2).astype(np.float32)
    k = np.array([1024, 7, 1, 0, 1024, 300, 0, 1000])
    W = _custom(x, top_k=k, top_p=0.9, flags=_all_combos(B), dtype=wl.BF16)
    _check(W, f"V=2^21 seg={seg}", need_probs=False, seg=seg)


def test_k_equals_vocab_and_cap():
    rng = np.random.default_rng(3)
    for V, ks in [(700, [700, 699, 1, 701]), (1024, [1024, 1023]), (5000, [1024, 1025])]:
        x = (rng.standard_normal((len(ks), V))).astype(np.float32)
        W = _custom(x, top_k=ks, top_p=0.97, flags=[1, 3, 5, 7][: len(ks)])
        _check(W, f"k~V V={V}")


def test_exact_ties_everywhere():
    B, V = 16, 30000
    x = np.zeros((B, V), np.float32)
    x[1::2] = np.round(np.random.default_rng(5).standard_normal((B // 2, V)) * 2) / 2
    flags = _all_combos(B)
    # an all-zero row whose top-p stage is on has its cutoff exactly at p =
    # 0.5 (n / V reaches it at n = V / 2): a top-p boundary tie by
    # construction, exempt from the checks
    boundary = int(((flags & 2) != 0)[0::2].sum())
    for dt in (wl.F32, wl.BF16):
        W = _custom(x, top_k=np.array([10, 1024, 1, 0] * 4), top_p=0.5, flags=flags, dtype=dt)
        _check(W, f"ties {dt}", max_exempt=boundary)


def test_signed_zero_and_neg_inf():
    rng = np.random.default_rng(9)
    B, V = 16, 5000
    x = (rng.standard_normal((B, V))).astype(np.float32)
    x[:, ::7] = -0.0
    x[:, 3::11] = 0.0
    x[:, 5::13] = -np.inf
    W = _custom(x, top_k=np.array([100, 0] * 8), top_p=0.95, flags=_all_combos(B))
    hip, _ = _check(W, "zeros/-inf")
    assert not np.signbit(hip["logits"][np.isfinite(hip["logits"]) & (hip["logits"] == 0)]).any()


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_kept_neg_inf_entries(dtype):
    """Rows with only 30 finite logits: a top-k larger than that keeps -inf
    entries, whose dense logit stays -inf and whose probability is 0 (the
    dense writer composes listed tiles from the kept values alone)."""
    rng = np.random.default_rng(88 if dtype == wl.F32 else 89)
    B, V = 16, 4096
    x = np.full((B, V), -np.inf, np.float32)
    for r in range(B):
        x[r, rng.choice(V, size=30, replace=False)] = rng.standard_normal(30).astype(np.float32)
    k = np.array([1, 30, 31, 100, 1024, 0, 64, 500] * 2)
    p = np.array([1.0] * 8 + [0.5] * 8, np.float32)
    W = _custom(x, top_k=k, top_p=p, flags=_all_combos(B), dtype=dtype, seed=90)
    hip, ref = _check(W, f"kept -inf {dtype}")
    # some rows keep more entries than they have finite logits
    assert (ref["nkept"] > 30).any()
    assert np.array_equal(np.isneginf(hip["logits"]), np.isneginf(ref["logits"]))


def test_randomized_sweep():
    """300 seeded random calls, every row against the oracle: batch 1..100,
    vocabularies from 7 to 70001 (both sides of 256 and of the tile
    lengths), fp32 / bf16, near-flat, Gumbel, coarse-grid (tied) and spiky
    rows, any k (including 0 and past min(V, 1024)), any p, every stage
    combination, temperature and repetition penalty (history ids partly out
    of range), top-k ties kept or not, race or inverse-CDF draws, automatic
    or fixed tile lengths.  Random rows can land on near ties, so up to a
    tenth of a call's rows (at least one) may be exempted from the id check
    by the oracle's own margins."""
    rng = np.random.default_rng(20241203)
    for case in range(300):
        B = int(rng.choice([1, 3, 8, 17, 40, 100]))
        V = int(rng.choice([7, 64, 255, 256, 257, 1000, 4097, 6400, 20000, 32000, 70001]))
        dtype = wl.BF16 if rng.random() < 0.5 else wl.F32
        kind = int(rng.integers(0, 4))
        if kind == 0:
            x = rng.standard_normal((B, V)) * rng.choice([0.05, 1.0, 3.0])
        elif kind == 1:
            x = rng.gumbel(size=(B, V)) * 4.0
        elif kind == 2:
            x = np.round(rng.standard_normal((B, V)) * 4.0) / 4.0
        else:
            x = rng.standard_normal((B, V))
            for r in range(B):
                x[r, rng.choice(V, size=min(V, 10), replace=False)] += rng.uniform(5, 15)
        k = rng.integers(0, min(V, 1024) + 2, size=B)
        p = np.where(rng.random(B) < 0.3, 1.0, rng.uniform(0.05, 1.0, size=B))
        flags = rng.integers(0, 8, size=B)
        kw = dict(temperature=float(rng.choice([1.0, 0.7, 1.3])),
                  penalty=float(rng.choice([1.0, 1.2])))
        if kw["penalty"] != 1.0:
            kw["ids"] = rng.integers(-5, V + 5, size=B * 20).astype(np.int32)
            kw["offsets"] = np.arange(B + 1, dtype=np.int64) * 20
        W = _custom(x.astype(np.float32), top_k=k, top_p=p, flags=flags, dtype=dtype,
                    seed=case, **kw)
        inverse = bool(rng.random() < 0.25)
        ties = bool(rng.random() < 0.2)
        u = rng.random(B).astype(np.float32) if inverse else None
        seg = int(rng.choice([0, 0, 0, 1024, 3072]))
        label = (f"sweep {case}: B={B} V={V} {dtype} rows={kind} inverse={inverse} "
                 f"ties={ties} seg={seg} {kw.get('temperature')} {kw.get('penalty')}")
        hip = run_hip(W, need_logits=True, need_probs=True, u=u, drop_q=inverse, ties=ties,
                      seg=seg)
        ref = run_oracle(W, need_logits=True, need_probs=True, u=u, ties=ties)
        compare(W, hip, ref, label=label, inverse=inverse, max_exempt=max(1, B // 10))


@pytest.mark.parametrize("pad", [8, 3])
def test_padded_row_stride(pad):
    W = wl.make(5, B=16, V=20000, seed=2)
    _check(W, f"ld=V+{pad}", ld_pad=pad)


@pytest.mark.parametrize("guess,seg", [(1, 8192), (16, 1024), (1024, 3072), (256, 32768), (64, 5120)])
def test_knobs_do_not_change_results(guess, seg):
    W = wl.make(3, B=8, V=30000, seed=4)
    W.row_flags = np.array([2, 6, 3, 7, 2, 6, 1, 0], np.uint8)
    W.top_k = np.array([0, 0, 40, 1024, 0, 0, 77, 0], np.int32)
    base = run_hip(W, need_logits=True, need_probs=True)
    other = run_hip(W, need_logits=True, need_probs=True, guess=guess, seg=seg)
    np.testing.assert_array_equal(base["idx"], other["idx"])
    np.testing.assert_array_equal(base["logits"].view(np.uint32), other["logits"].view(np.uint32))
    # probabilities are a floating-point output: the row normaliser is summed
    # in a tile-dependent order
    np.testing.assert_allclose(base["probs"], other["probs"], rtol=1e-6, atol=1e-12)


@pytest.mark.parametrize("B", [1, 32, 33, 200])
def test_automatic_tile_length_across_batches(B):
    """With the tile length left automatic, a call's batch picks it: at
    V = 32000 on a 256-CU device, tiles of 1024 up to 32 rows, 2048 at 33
    rows, 7168 at 200 rows (a length that is not a power of two).  Every row against the
    oracle, and bit-identical to fixed 8192-element tiles."""
    rng = np.random.default_rng(300 + B)
    V = 32000
    x = (rng.standard_normal((B, V)) * 2).astype(np.float32)
    k = rng.integers(0, 1025, size=B)
    p = rng.uniform(0.3, 1.0, size=B)
    W = _custom(x, top_k=k, top_p=p, flags=_all_combos(B), seed=301)
    hip, _ = _check(W, f"automatic tiles B={B}")
    fixed = run_hip(W, need_logits=True, need_probs=True, seg=8192)
    np.testing.assert_array_equal(hip["idx"], fixed["idx"])
    np.testing.assert_array_equal(hip["logits"].view(np.uint32), fixed["logits"].view(np.uint32))


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("draw", ["race", "inverse"])
def test_small_candidate_sets_with_ties(dtype, draw):
    """Small k, where the row merge places at most 256 candidates by
    counting: values on a coarse grid put many equal values around the k-th
    and inside the nucleus, so the order among them is the vocab id's."""
    rng = np.random.default_rng(77 if dtype == wl.F32 else 78)
    ks = [1, 2, 3, 17, 50, 120]
    ps = [0.3, 0.8, 0.97, 1.0]
    B, V = len(ks) * len(ps), 12000
    x = np.round(rng.standard_normal((B, V)) * 4.0) / 4.0
    k = np.repeat(ks, len(ps))
    p = np.tile(ps, len(ks)).astype(np.float32)
    W = _custom(x.astype(np.float32), top_k=k, top_p=p, flags=7, dtype=dtype, seed=79)
    u = rng.random(B).astype(np.float32) if draw == "inverse" else None
    print(f"[case] small candidate sets with ties {dtype} {draw} B={B} V={V}", flush=True)
    hip = run_hip(W, need_logits=True, need_probs=True, u=u, drop_q=u is not None)
    ref = run_oracle(W, need_logits=True, need_probs=True, u=u)
    _log(f"small sets {dtype} {draw}", compare(W, hip, ref, label="small sets",
                                               inverse=u is not None))


@pytest.mark.parametrize("rpl", [1, 5])
def test_rows_per_launch_changes_nothing(rpl):
    # flat top-p rows (the full-row search queue fills across chunks), rows
    # whose sample overstates the row (the full-row search), greedy and
    # sample-only rows, in chunks of rpl rows
    W = wl.make(3, B=12, V=20000, seed=9)
    W.row_flags = np.array([2, 6, 3, 7, 0, 4, 1, 5, 2, 6, 2, 6], np.uint8)
    W.top_k = np.array([0, 0, 40, 1024, 0, 0, 77, 5, 0, 0, 0, 0], np.int32)
    print(f"[case] rows_per_launch={rpl} B={W.B} V={W.V}", flush=True)
    base = run_hip(W, need_logits=True, need_probs=True)
    other = run_hip(W, need_logits=True, need_probs=True, rpl=rpl)
    np.testing.assert_array_equal(base["idx"], other["idx"])
    np.testing.assert_array_equal(base["logits"].view(np.uint32), other["logits"].view(np.uint32))
    np.testing.assert_array_equal(base["probs"].view(np.uint32), other["probs"].view(np.uint32))
    compare(W, other, run_oracle(W, need_logits=True), label=f"rpl={rpl}")


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_inverse_cdf_sampling(cfg):
    # the caller's uniforms replace q: listed rows draw in k_rows, unfiltered
    # rows and rows whose guess failed draw through the full-row search
    sizes = {1: (4, 32000), 2: (16, 30000), 3: (12, 20000), 4: (64, 6400), 5: (24, 40000)}
    B, V = sizes[cfg]
    W = wl.make(cfg, B=B, V=V, seed=21)
    if W.row_flags is None:
        W.row_flags = np.full(W.B, 7, np.uint8)
    u = np.random.default_rng(77 + cfg).random(W.B).astype(np.float32)
    u[0] = 0.0  # the first kept token
    if W.B > 1:
        u[1] = np.nextafter(np.float32(1), np.float32(0))  # the last kept token
    print(f"[case] inverse CDF cfg{cfg} B={W.B} V={W.V}", flush=True)
    hip = run_hip(W, need_logits=True, u=u, drop_q=True)
    ref = run_oracle(W, need_logits=True, u=u)
    stats = compare(W, hip, ref, label=f"inverse cfg{cfg}", inverse=True)
    print(f"[case] inverse cfg{cfg}: {stats}", flush=True)


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_far_spikes_in_the_estimate_sample(dtype):
    """A few logits far above the rest (1e4 over a N(0, 2^2) bulk) put the
    estimate sample's maximum so far up that the r-th sampled key lies
    outside the fine bins below it; the estimate then finds it in two steps
    (coarse bin, then fine bin inside)."""
    rng = np.random.default_rng(41)
    B, V = 24, 100000
    x = (rng.standard_normal((B, V)) * 2).astype(np.float32)
    for r in range(B):
        x[r, rng.choice(V, size=40, replace=False)] += np.float32(1e4)
    k = np.array([1024, 300, 0, 50] * 6)
    W = _custom(x, top_k=k, top_p=0.9, flags=_all_combos(B), dtype=dtype, seed=42)
    _check(W, f"far spikes {dtype}")


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("draw", ["race", "inverse"])
def test_topp_selection_sizes(dtype, draw):
    """Top-p over selections on both sides of the row merge's size limits:
    at most 256 entries are cut by one wave (4 largest first, then a register
    sort), larger ones by maxima extraction and then the workgroup sort.
    Near-flat rows make the nuclei long enough to reach the sorts; bf16
    rows add ties inside the selection."""
    rng = np.random.default_rng(31 if dtype == wl.F32 else 32)
    ks = [3, 4, 5, 255, 256, 257, 511, 1024]
    ps = [0.2, 0.6, 0.9, 0.999]
    B, V = len(ks) * len(ps), 20000
    x = (rng.standard_normal((B, V)) * 0.3).astype(np.float32)
    k = np.repeat(ks, len(ps))
    p = np.tile(ps, len(ks)).astype(np.float32)
    W = _custom(x, top_k=k, top_p=p, flags=7, dtype=dtype, seed=33)
    u = rng.random(B).astype(np.float32) if draw == "inverse" else None
    print(f"[case] top-p selection sizes {dtype} {draw} B={B} V={V}", flush=True)
    hip = run_hip(W, need_logits=True, need_probs=True, u=u, drop_q=u is not None)
    ref = run_oracle(W, need_logits=True, need_probs=True, u=u)
    _log(f"top-p sizes {dtype} {draw}", compare(W, hip, ref, label="top-p sizes",
                                                inverse=u is not None))
    # every selection size and p produced a non-trivial cut somewhere
    assert (ref["nkept"] > 8).any() and (ref["nkept"] < k).any()


def test_repeated_runs_bit_identical():
    import torch

    from decode_token_sampling_row_amd.sampler import Sampler

    W = wl.make(5, B=64, V=50000, seed=6)
    d = device_inputs(W)
    s = Sampler(W.B, W.V, torch.bfloat16)
    first = run_hip(W, need_logits=True, sampler=s, inputs=d)
    for _ in range(4):
        again = run_hip(W, need_logits=True, sampler=s, inputs=d)
        np.testing.assert_array_equal(first["idx"], again["idx"])
        np.testing.assert_array_equal(first["logits"].view(np.uint32),
                                      again["logits"].view(np.uint32))


def test_fallback_with_huge_tie_block():
    """The top-p cutoff falls inside a block of >4096 equal logits: the kept
    members of the block are the ones with the smallest vocab ids."""
    B, V = 4, 30000
    x = np.full((B, V), -2.0, np.float32)
    x[:, :10] = 3.0
    x[:, 5000:25000] = 0.0
    W = _custom(x, top_k=0, top_p=np.array([0.5, 0.9, 0.3, 0.7]), flags=[2, 6, 2, 6])
    _check(W, "tie block")


def _sample_runs(V, b):
    """Positions of the 16 runs of 512 logits of row b that the select pass
    estimates its admission value from: run s lies in the s-th sixteenth of
    the row (bounds rounded down to multiples of 8), at one of 16 staggered
    offsets."""
    run = 512
    pos = []
    for s in range(16):
        seg0 = (s * V // 16) & ~7
        seg1 = ((s + 1) * V // 16) & ~7
        step = ((seg1 - seg0 - run) // 16) & ~7
        a = seg0 + ((s * 5 + b * 3) & 15) * step
        pos.append(np.arange(a, a + run))
    return np.concatenate(pos)


@pytest.mark.parametrize("case", ["high", "low", "chunk0_heavy"])
@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_unrepresentative_sample(case, dtype):
    """Rows on which the admission estimate is wrong, so the row merge finds
    the handed-over candidates incomplete and the full-row search selects the
    row exactly.  high: the row's largest values all sit in the sampled runs,
    so too few elements are admitted; low: the sampled runs hold the smallest
    values, so every tile overflows its buffers; chunk0_heavy: the first tile
    is full of large values outside the sample, so that tile overflows while
    the others stay within their buffers."""
    rng = np.random.default_rng(21)
    B, V = 16, 262144
    x = rng.standard_normal((B, V)).astype(np.float32)
    for b in range(B):
        pos = _sample_runs(V, b)
        if case == "high":
            x[b, pos] += 6.0
        elif case == "low":
            x[b, pos] -= 6.0
        else:
            heavy = np.zeros(V, bool)
            heavy[: V // 8] = True
            heavy[pos] = False
            x[b, heavy] += 6.0
    k = np.array([1024, 50, 1, 0, 1024, 300, 0, 1000] * 2)
    W = _custom(x, top_k=k, top_p=0.9, flags=_all_combos(B), dtype=dtype)
    _check(W, f"sample {case} {dtype}")


@pytest.mark.parametrize("case", ["ties", "ties_inverse", "redone"])
@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_topk_keeping_ties(case, dtype):
    """SAMPLER_TOPK_TIES: top-k keeps every value equal to the k-th.  Integer
    logits make large tie groups: small k stay within a list (the row merge
    extends the selection), k near 1024 exceed it and go to the full-row
    search with the k-th value as floor, as do rows selected again exactly."""
    rng = np.random.default_rng(31)
    if case == "redone":
        B, V = 16, 262144
        x = np.round(rng.standard_normal((B, V)) * 2.0).astype(np.float32)
        for b in range(B):
            x[b, _sample_runs(V, b)] += 6.0  # the sample overstates the row
        k = np.array([1024, 50, 1, 7, 1024, 300, 2, 1000] * 2)
    else:
        B, V = 32, 30000
        x = rng.integers(-20, 21, size=(B, V)).astype(np.float32)
        k = np.array([1, 5, 50, 300, 1000, 1024, 2, 0] * 4)
    W = _custom(x, top_k=k, top_p=0.9, flags=_all_combos(B), dtype=dtype)
    u = rng.random(B).astype(np.float32) if case == "ties_inverse" else None
    label = f"topk ties {case} {dtype}"
    print(f"[case] {label} B={W.B} V={W.V}", flush=True)
    hip = run_hip(W, need_logits=True, need_probs=True, ties=True, u=u, drop_q=u is not None)
    ref = run_oracle(W, need_logits=True, need_probs=True, ties=True, u=u)
    _log(label, compare(W, hip, ref, label=label, inverse=u is not None))
    # more than k survive where the k-th value is tied
    tk = (W.row_flags & 1) != 0
    assert np.any(ref["nkept"][tk & ((W.row_flags & 2) == 0)] > k[tk & ((W.row_flags & 2) == 0)])


def test_flat_rows_force_full_row_search():
    rng = np.random.default_rng(11)
    B, V = 8, 128256
    x = (rng.standard_normal((B, V)) * 0.05).astype(np.float32)
    W = _custom(x, top_k=0, top_p=np.array([0.9, 0.99, 0.5, 0.999, 0.1, 0.95, 0.75, 0.6]),
                flags=[2, 6] * 4)
    _check(W, "flat full-row search")


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_full_row_search_race_winner_penalised(dtype):
    """Flat top-p rows (the full-row search) with a repetition penalty and a
    temperature, q set so that the race winner is a penalised id near the top
    of the row (far above the cut's boundary): the search keeps each value
    bin's best race candidate and reads the winner's logit and history again,
    so its transformed value must match the pass's.  Other rows put the
    winner next to the cut (a zero of q at the ~k-th element, k from the
    cut's size) or leave q random."""
    rng = np.random.default_rng(61)
    B, V = 12, 50021
    x = (rng.standard_normal((B, V)) * 0.05).astype(np.float32)
    x[:, 0] = 0.3  # a positive top entry that the penalty divides
    q = rng.exponential(size=(B, V)).astype(np.float32)
    order = np.argsort(-x, axis=1, kind="stable")
    hist = []
    for b in range(B):
        h = rng.integers(0, V, size=400)
        h[:3] = order[b, [0, 1, 4]]  # the top entries penalised
        hist.append(h)
        if b % 3 == 0:
            q[b, order[b, 4]] = 1e-30      # a penalised top entry wins
        elif b % 3 == 1:
            q[b, order[b, int(V * 0.85)]] = 1e-30  # near the boundary of p = 0.9
    ids = np.concatenate(hist).astype(np.int32)
    offs = (np.arange(B + 1) * 400).astype(np.int64)
    for rho in (1.3, 0.8):
        W = _custom(x, top_k=0, top_p=0.9, flags=[6] * B, q=q, dtype=dtype, penalty=rho,
                    temperature=0.7, ids=ids, offsets=offs)
        _check(W, f"penalised winner rho={rho} {dtype}")


def test_top_p_nonpositive_keeps_one():
    rng = np.random.default_rng(12)
    B, V = 8, 9000
    x = (rng.standard_normal((B, V))).astype(np.float32)
    W = _custom(x, top_k=np.array([0, 0, 30, 30, 0, 0, 5, 5]), top_p=np.array(
        [0.0, -1.0, 0.0, -0.5, 1e-30, 0.0, 1.0, 2.0]), flags=[2, 6, 3, 7, 6, 2, 7, 3])
    hip, ref = _check(W, "p<=0")
    assert (np.isfinite(hip["logits"]).sum(axis=1)[:6] == 1).all()


def test_penalty_ids_out_of_range_and_duplicates():
    rng = np.random.default_rng(13)
    B, V = 8, 4000
    x = (rng.standard_normal((B, V)) * 3).astype(np.float32)
    ids = np.concatenate([rng.integers(-50, V + 50, size=300) for _ in range(B)]).astype(np.int32)
    offs = (np.arange(B + 1) * 300).astype(np.int64)
    for rho in (1.3, 0.7):
        W = _custom(x, top_k=np.array([50, 0] * 4), top_p=0.8, flags=_all_combos(B),
                    penalty=rho, temperature=0.7, ids=ids, offsets=offs)
        _check(W, f"penalty rho={rho}")


def test_empty_batch_and_argument_checks():
    import ctypes

    import torch

    from decode_token_sampling_row_amd import sampler as smp

    s = smp.Sampler(4, 100, torch.float32)
    lib = smp.load_library()
    x = torch.zeros((4, 100), device="cuda")
    idx = torch.zeros(4, dtype=torch.int64, device="cuda")
    q = torch.ones((4, 100), device="cuda")
    good = smp.make_args(x, idx, q=q)
    assert smp.sampler_check(s.handle, 4, good) == 0
    assert smp.sampler_check(s.handle, 0, smp.sampler_args()) == 0
    smp.sampler_run(s.handle, 0, smp.sampler_args())  # empty batch: no-op
    assert smp.sampler_check(s.handle, 5, good) == smp.SAMPLER_EINVAL
    for field, val in [("temperature", 0.0), ("temperature", float("inf")),
                       ("repetition_penalty", -1.0), ("eps", -1e-3), ("flags", 16),
                       ("ld", 99), ("out_idx", None), ("logits", None)]:
        a = smp.make_args(x, idx, q=q)
        setattr(a, field, val)
        assert smp.sampler_check(s.handle, 4, a) == smp.SAMPLER_EINVAL, field
    a = smp.make_args(x, idx, q=q)
    a.flags = smp.SAMPLER_NEED_LOGITS
    assert smp.sampler_check(s.handle, 4, a) == smp.SAMPLER_EINVAL
    a = smp.make_args(x, idx)  # every row samples (row_flags NULL) but no q
    assert smp.sampler_check(s.handle, 4, a) == smp.SAMPLER_EINVAL
    a = smp.make_args(x, idx, q=q)
    a.penalty_ids = a.q
    assert smp.sampler_check(s.handle, 4, a) == smp.SAMPLER_EINVAL
    with pytest.raises(smp.SamplerError):
        smp.sampler_run(s.handle, 4, a)
    hist = torch.zeros(8, dtype=torch.int32, device="cuda")
    offs = torch.arange(5, dtype=torch.int64, device="cuda") * 2
    lens = torch.zeros(4, dtype=torch.int32, device="cuda")
    fin = torch.zeros(4, dtype=torch.uint8, device="cuda")
    a = smp.make_args(x, idx, q=q, penalty_len=lens)  # lengths without a history
    assert smp.sampler_check(s.handle, 4, a) == smp.SAMPLER_EINVAL
    a = smp.make_args(x, idx, q=q, penalty_ids=hist, penalty_offsets=offs, append_history=True)
    assert smp.sampler_check(s.handle, 4, a) == smp.SAMPLER_EINVAL  # append needs lengths
    a = smp.make_args(x, idx, q=q, penalty_ids=hist, penalty_offsets=offs, penalty_len=lens,
                      append_history=True)
    assert smp.sampler_check(s.handle, 4, a) == 0
    for eos, rc in [(-1, smp.SAMPLER_EINVAL), (100, smp.SAMPLER_EINVAL), (0, 0), (99, 0)]:
        a = smp.make_args(x, idx, q=q, finished=fin, eos_id=eos)
        assert smp.sampler_check(s.handle, 4, a) == rc, eos
    s.close()
    del lib, ctypes


def test_profile_reports_kernel_times():
    import torch

    from decode_token_sampling_row_amd.sampler import SamplerError, Sampler

    W = wl.make(5, B=16, V=40000, seed=3)
    d = device_inputs(W)
    s = Sampler(W.B, W.V, torch.bfloat16)
    out_idx = torch.zeros(W.B, dtype=torch.int64, device="cuda")
    out_l = torch.empty((W.B, W.V), device="cuda")
    with pytest.raises(SamplerError):
        s.profile()  # nothing profiled yet
    for _ in range(3):
        s.run(d["logits"], out_idx, top_k=d["top_k"], top_p=d["top_p"], q=d["q"],
              row_flags=d["row_flags"], out_logits=out_l, profile=True)
    ms = s.profile()
    assert len(ms) == 6 and all(t > 0 for t in ms[:5]) and ms[5] == 0
    # without top-k / top-p, uniforms and dense outputs, neither the planning,
    # the full-row search nor the dense writer is launched
    s.run(d["logits"], out_idx, q=d["q"], row_flags=d["row_flags"], profile=True)
    ms = s.profile()
    assert ms[1] > 0 and ms[2] > 0 and ms[0] == ms[3] == ms[4] == ms[5] == 0
    counts = torch.zeros(2, dtype=torch.int32, device="cuda")
    s.run(d["logits"], out_idx, q=d["q"], row_flags=d["row_flags"], counts=counts, profile=True)
    assert s.profile()[5] > 0  # the epilogue
    with pytest.raises(SamplerError):
        s.profile()  # the averaged calls are forgotten
    s.close()


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_race_extreme_q_and_zero_eps(dtype):
    """The exponential race where fp32 arithmetic is weakest: eps = 0 with
    exact zeros in q (a finite logit over a zero denominator has an infinite
    ratio; ties among those go to the lowest id), q spread over 28 decades
    (exp of U[-60, 5]) and logits N(0, 20^2), so that the logit differences
    the race compares reach 80 and more.  Sample-only rows race in the
    streaming pass, filtered rows in the row merge, flat top-p rows in the
    full-row search."""
    rng = np.random.default_rng(51)
    B, V = 48, 40000
    x = (rng.standard_normal((B, V)) * 20.0).astype(np.float32)
    x[40:] = (rng.standard_normal((8, V)) * 0.05).astype(np.float32)  # flat: full-row search
    q = np.exp(rng.uniform(-60.0, 5.0, size=(B, V))).astype(np.float32)
    order = np.argsort(-x, axis=1, kind="stable")
    flags = np.array([4, 5, 6, 7] * 12, np.uint8)
    k = np.array([0, 50, 0, 1024] * 12, np.int32)
    p = np.array([1.0, 1.0, 0.9, 0.95] * 12, np.float32)
    flags[40:], k[40:], p[40:] = 6, 0, 0.9  # flat rows: top-p alone, the full-row search
    must_zero = []  # rows whose draw must land on a zero of q
    for b in range(B):
        if b >= 40:                     # flat rows, full-row search: two zeros inside K
            q[b, order[b, [100, 5000]]] = 0.0
            must_zero.append(b)
        elif b % 8 == 0:                # sample only: two zeros near the top, lower id wins
            q[b, order[b, [3, 7]]] = 0.0
            must_zero.append(b)
        elif b % 8 == 4:                # sample only: one zero far down the row
            q[b, order[b, V - 10]] = 0.0
            must_zero.append(b)
        elif b % 4 == 1:                # top-k 50: two zeros inside the kept set
            q[b, order[b, [10, 20]]] = 0.0
            must_zero.append(b)
        elif b % 4 == 2:                # zeros anywhere (mostly outside K)
            q[b, rng.choice(V, size=3, replace=False)] = 0.0
        else:                           # top-k 1024 + top-p: a zero at the third place
            q[b, order[b, 2]] = 0.0
    W = _custom(x, top_k=k, top_p=p, flags=flags, q=q, dtype=dtype, eps=0.0)
    hip, ref = _check(W, f"race extremes {dtype}")
    must_zero = np.array(must_zero)
    assert (q[must_zero, ref["idx"][must_zero]] == 0.0).all()
