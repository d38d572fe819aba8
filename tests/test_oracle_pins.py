"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print (the path table), published known-answer vectors (Philox), closed
forms, library routines (scipy's softmax, numpy's argmax and sort, torch's
bf16 conversion, the transformers library's repetition-penalty and min-length
processors and its top-k / top-p / min-p warpers), brute force over tiny vocabularies, and distribution tests
of the Gumbel-max draw against the categorical distribution.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def run(logits, **kw):
    kw.setdefault("want_probs", True)
    kw.setdefault("want_logprobs", True)
    return oracle.step(np.atleast_2d(np.asarray(logits, dtype=np.float32)), **kw)


# ---------------------------------------------------------------- Philox
def test_philox_known_answers():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) if l.strip() and l[0] != "#"]
    assert len(rows) == 3
    for r in rows:
        w = [int(x, 16) for x in r]
        out = oracle.philox4x32_10(w[0:4], w[4:6])
        assert [int(x) for x in out] == w[6:10]


def test_draw_word_layout():
    # entry i of a row is word (i & 3) of the block at counter (i >> 2, stream, off_lo, off_hi)
    seed, stream, off = 0x0123456789ABCDEF, 77, 0x0000000500000003
    for i in [0, 1, 2, 3, 4, 7, 1021, 151935]:
        blk = oracle.philox4x32_10([i >> 2, stream, off & 0xFFFFFFFF, off >> 32],
                                   [seed & 0xFFFFFFFF, seed >> 32])
        assert oracle.draw_word(seed, stream, off, i) == int(blk[i & 3])


def test_philox_bit_balance():
    words = np.array([oracle.draw_word(5, 3, 11, i) for i in range(40000)], dtype=np.uint64)
    bits = ((words[:, None] >> np.arange(32, dtype=np.uint64)) & 1).astype(np.float64)
    frac = bits.mean(0)
    # each bit is Bernoulli(1/2): 6 sigma at n = 40000 is 0.015
    assert np.all(np.abs(frac - 0.5) < 0.015)


# ---------------------------------------------------------------- Exp(1)
def test_exp1_extreme_words_closed_form():
    # x = 0: w = 2^-33, E = -ln(1 - 2^-33) ~= 2^-33;  x = 2^32-1: E = 33 ln 2
    assert oracle.exp1_from_word(0) == pytest.approx(2.0 ** -33, rel=1e-9)
    assert oracle.exp1_from_word(2**32 - 1) == pytest.approx(33 * math.log(2.0), rel=1e-12)
    assert oracle.exp1_from_word(2**31) == pytest.approx(-math.log(0.5 - 0.5 * 2.0**-32), rel=1e-12)


def test_exp1_moments_and_ks():
    e = oracle.exp1_draws(seed=12345, stream=0, offset=0, n=10_000_000)
    assert abs(e.mean() - 1.0) < 1e-3
    assert abs(e.var() - 1.0) < 2e-3
    ks = scipy.stats.kstest(e[:1_000_000], "expon")
    assert ks.pvalue > 1e-3


# ---------------------------------------------------------------- predicate
def test_path_table_from_page():
    spec = json.load(open(os.path.join(GOLDEN, "path_table.json")))
    for case in spec["cases"]:
        rows = case["rows"]
        got = oracle.select_path([r["temperature"] for r in rows], [r["top_k"] for r in rows],
                                 [r["top_p"] for r in rows], [r["min_p"] for r in rows],
                                 deterministic=case["deterministic"])
        assert got == case["expected"], case["name"]


def test_empty_batch_is_an_error():
    with pytest.raises(ValueError):
        oracle.select_path(np.zeros(0, np.float32))


def test_normalisation_rules():
    assert oracle.normalized_top_k(0.0, -1) == 1
    assert oracle.normalized_top_k(0.0, 50) == 1
    assert oracle.normalized_top_k(0.7, -1) == 1 << 30
    assert oracle.normalized_top_k(0.7, 50) == 50
    # a negative temperature is not greedy (0 <= T is part of the rule)
    assert oracle.normalized_top_k(-0.5, -1) == 1 << 30


def test_penalty_flag_defaults_table():
    spec = json.load(open(os.path.join(GOLDEN, "vllm_flags.json")))
    d = spec["defaults"]
    for case in spec["cases"]:
        p = dict(d, **case["change"])
        got = oracle.do_penalties([p["repetition_penalty"]], [p["presence_penalty"]], [p["frequency_penalty"]])
        assert got == case["do_penalties"], case


# ---------------------------------------------------------------- softmax / log_softmax
def test_softmax_matches_scipy_untruncated():
    rng = np.random.default_rng(0)
    x = (4 * rng.standard_normal((6, 257))).astype(np.float32)
    T = np.array([1.0, 0.5, 2.0, 0.3, 1.7, 1.0], np.float32)
    o = run(x, temperature=T)
    z = (x / T[:, None]).astype(np.float32)          # numpy's IEEE fp32 division
    ref_p = scipy.special.softmax(z.astype(np.float64), axis=1)
    ref_lp = scipy.special.log_softmax(z.astype(np.float64), axis=1)
    np.testing.assert_allclose(o["probs"], ref_p, rtol=0, atol=1e-7)
    np.testing.assert_allclose(o["logprobs"], ref_lp, rtol=2e-7, atol=1e-6)
    assert np.all(np.abs(o["probs"].astype(np.float64).sum(1) - 1.0) < 1e-5)


def test_softmax_closed_forms():
    V = 1000
    o = run(np.zeros((1, V), np.float32))
    np.testing.assert_allclose(o["probs"], 1.0 / V, rtol=1e-7)
    np.testing.assert_allclose(o["logprobs"], -math.log(V), rtol=1e-7)
    d = 1.75
    o = run(np.array([[0.0, -d]], np.float32))
    assert o["probs"][0, 0] == pytest.approx(1.0 / (1.0 + math.exp(-d)), rel=1e-7)
    assert o["logprobs"][0, 1] == pytest.approx(-d - math.log1p(math.exp(-d)), rel=1e-7)


def test_bf16_conversion_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**16, size=(1, 4096), dtype=np.uint16)
    f = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    bits[~np.isfinite(f)] = 0  # keep finite values
    f = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    f = np.clip(f, -60, 60)
    bits = workloads.f32_to_bf16_bits(f)  # values in range now round-trip exactly
    f2 = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    o = oracle.step(bits, dtype="bf16")
    ref = scipy.special.log_softmax(f2.astype(np.float64), axis=1)
    np.testing.assert_allclose(o["logprobs"], ref, rtol=2e-7, atol=1e-6)


# ---------------------------------------------------------------- greedy
def test_greedy_is_first_argmax():
    rng = np.random.default_rng(2)
    x = rng.integers(-3, 3, size=(40, 50)).astype(np.float32)   # many ties
    T = np.zeros(40, np.float32)
    o = run(x, temperature=T)
    np.testing.assert_array_equal(o["token_ids"], np.argmax(x, axis=1))
    # greedy rows: probs/logprobs untruncated at T = 1
    np.testing.assert_allclose(o["probs"], scipy.special.softmax(x.astype(np.float64), axis=1), atol=1e-7)
    # explicit top_k = 1 rows: the same token, probability shared by the tied maxima
    o1 = run(x, temperature=np.full(40, 0.8, np.float32), top_k=np.ones(40, np.int32))
    np.testing.assert_array_equal(o1["token_ids"], np.argmax(x, axis=1))
    ties = (x == x.max(1, keepdims=True))
    np.testing.assert_allclose(o1["probs"], ties / ties.sum(1, keepdims=True), atol=1e-7)


# ---------------------------------------------------------------- masks by brute force
def brute_force_kept(z, k, p, min_p):
    """Kept set from the definitions, by enumeration (V <= 10)."""
    V = len(z)
    zd = z.astype(np.float64)
    q = np.exp(zd - zd.max())
    # top-k: fewer than k values strictly above
    Kk = [i for i in range(V) if sum(zd[j] > zd[i] for j in range(V)) < k]
    # top-p: among subsets of Kk closed upward in value, the lightest one
    # whose mass reaches p * mass(Kk)
    tot = sum(q[i] for i in Kk)
    best = None
    for mask in range(1, 1 << len(Kk)):
        S = [Kk[b] for b in range(len(Kk)) if mask >> b & 1]
        closed = all((j in S) for i in S for j in Kk if zd[j] >= zd[i])
        if not closed:
            continue
        m = sum(q[i] for i in S)
        if m >= p * tot and (best is None or m < best[0]):
            best = (m, set(S))
    Kp = best[1]
    # min-p: probability at least min_p times the largest
    return {i for i in Kp if q[i] >= min_p}, tot, best[0]


@pytest.mark.parametrize("ties", [False, True])
def test_masks_brute_force(ties):
    rng = np.random.default_rng(3 + ties)
    n_checked = 0
    for trial in range(300):
        V = int(rng.integers(1, 11))
        if ties:
            x = rng.integers(-2, 3, size=V).astype(np.float32) * 0.75
        else:
            x = (2 * rng.standard_normal(V)).astype(np.float32)
        k = int(rng.choice([1, 2, 3, 5, V, V + 2, -1]))
        p = float(rng.choice([1.0, 0.9, 0.5, 0.3, 0.05]))
        mp = float(rng.choice([0.0, 0.1, 0.3, 0.6]))
        T = np.float32(rng.choice([0.5, 1.0, 1.3]))
        z = (x / T).astype(np.float32)
        kk = V if k == -1 else k
        want, tot, m = brute_force_kept(z, kk, np.float32(p), np.float32(mp))
        o = run(x, temperature=[T], top_k=[k], top_p=[p], min_p=[mp])
        if o["flags"][0] & (oracle.FLAG_TOPP_MARGIN | oracle.FLAG_MINP_MARGIN):
            # a boundary within the margin: the exact set is one the flag allows
            alts = oracle.row_alternatives(np.atleast_2d(x), 0, temperature=[T], top_k=[k], top_p=[p], min_p=[mp])
            assert any(set(np.flatnonzero(a).tolist()) == want for a in alts), (x, k, p, mp, T)
            continue
        got = set(np.flatnonzero(np.isfinite(o["logprobs"][0])).tolist())
        assert got == want, (x, k, p, mp, T)
        assert o["kept"][0] == len(want)
        # the sampled token is always kept
        assert o["token_ids"][0] in want
        n_checked += 1
    assert n_checked > 250


def test_topp_margin_flag_on_exact_crossing():
    # p equal (to fp32 precision) to the top token's share puts the crossing on the boundary
    p = _share_top_of_two()
    o = run(np.array([[1.0, 0.0]], np.float32), top_p=[p])
    assert o["flags"][0] & oracle.FLAG_TOPP_MARGIN
    assert o["topp_margin"][0] < 1e-7
    o = run(np.array([[1.0, 0.0]], np.float32), top_p=[0.6])
    assert not (o["flags"][0] & oracle.FLAG_TOPP_MARGIN)


# The diagnostic flags mark a row only where rounding at a rule's boundary
# could change what the row returns; each has a case that must flag and one
# that must not.
def _share_top_of_two():
    # the fp32 top_p nearest the exact share of the larger of two tokens
    # one nat apart: the crossing lies on the boundary (to fp32 precision)
    return np.float32(1.0 / (1.0 + math.exp(-1.0)))


def test_topp_margin_flag_only_where_top_p_decides():
    x = np.array([[1.0, 0.0]], np.float32)
    p = _share_top_of_two()
    # min-p 0.3 keeps the second token (ratio e^-1 = 0.37): the crossing's
    # side decides whether it is kept
    o = run(x, top_p=[p], min_p=[0.3])
    assert o["flags"][0] & oracle.FLAG_TOPP_MARGIN
    # min-p 0.5 drops it whatever top-p does: no flag
    o = run(x, top_p=[p], min_p=[0.5])
    assert not (o["flags"][0] & oracle.FLAG_TOPP_MARGIN)
    assert o["topp_margin"][0] < 1e-7  # the margin itself is still reported
    # top-k 1 keeps one token whatever top-p does: no flag
    o = run(x, top_p=[p], top_k=[1])
    assert not (o["flags"][0] & oracle.FLAG_TOPP_MARGIN)


def test_topp_margin_alternatives_are_the_neighbouring_groups():
    x = np.array([[1.0, 0.0, -3.0]], np.float32)
    p = _share_top_of_two() * np.float32((1 + math.exp(-1.0)) / (1 + math.exp(-1.0) + math.exp(-4.0)))
    alts = oracle.row_alternatives(x, 0, top_p=[p])
    sets = [set(np.flatnonzero(a).tolist()) for a in alts]
    own = set(np.flatnonzero(np.isfinite(run(x, top_p=[p])["logprobs"][0])).tolist())
    assert sets[0] == own
    assert sorted(map(sorted, sets)) == [[0], [0, 1]]
    # an unflagged row allows its own set alone
    assert len(oracle.row_alternatives(x, 0, top_p=[0.6])) == 1


def test_minp_margin_flag():
    # m = fl32(ln 2 + 1e-3) and z = fl32(m - ln 2) (a tiny value with a fine
    # fp32 grid): exp(z - m) = 1/2 to ~1e-12, on min_p = 1/2's boundary
    m = np.float32(math.log(2.0) + 1e-3)
    zb = np.float32(float(m) - math.log(2.0))
    assert abs(math.exp(float(zb) - float(m)) / 0.5 - 1.0) < 1e-9
    x = np.array([[m, zb, -4.0]], np.float32)
    o = run(x, min_p=[0.5])
    assert o["flags"][0] & oracle.FLAG_MINP_MARGIN
    assert len(oracle.row_alternatives(x, 0, min_p=[0.5])) == 2
    # a value 1e-6 nat away is outside the margin
    x2 = np.array([[m, np.float32(float(zb) - 1e-6), -4.0]], np.float32)
    assert not (run(x2, min_p=[0.5])["flags"][0] & oracle.FLAG_MINP_MARGIN)
    # top-k 1 drops the near-boundary value whatever min-p does: no flag
    assert not (run(x, min_p=[0.5], top_k=[1])["flags"][0] & oracle.FLAG_MINP_MARGIN)


def test_gumbel_near_tie_flag():
    # tokens 0 and 1 get equal Gumbel scores (to fp32 precision of the
    # logit): z_1 = ln(E_1 / E_0) with the row's own Exp(1) draws
    seed, stream, off = 5, 0, 9
    E = oracle.exp1_draws(seed, stream, off, 4)
    a = np.float32(math.log(E[1] / E[0]))
    x = np.array([[0.0, a, -6.0, -6.0]], np.float32)
    kw = dict(seed=seed, offset=off, row_stream=[stream])
    o = run(x, **kw)
    assert o["flags"][0] & oracle.FLAG_GUMBEL_NEAR_TIE
    assert o["gumbel_gap"][0] < 1e-6
    assert sorted([int(o["token_ids"][0]), int(o["token_alt"][0])]) == [0, 1]
    # the brute-force scores agree: the two best are tokens 0 and 1
    q = np.exp(x[0].astype(np.float64) - x[0].max())
    assert set(np.argsort(-(q / E))[:2].tolist()) == {0, 1}
    o = run(np.array([[0.0, a - np.float32(1e-3), -6.0, -6.0]], np.float32), **kw)
    assert not (o["flags"][0] & oracle.FLAG_GUMBEL_NEAR_TIE)
    assert o["token_alt"][0] == -1


def test_icdf_margin_flag():
    # u for (seed 11, stream 0, offset 1803) lies within 5e-5 of 1/3; with
    # masses (1, 1, e^z2) and e^z2 = 1/u - 2, u S falls on the step after
    # token 0
    seed, off = 11, 1803
    u = oracle.icdf_uniform(seed, 0, off)
    assert abs(u - 1.0 / 3.0) < 5e-5
    z2 = np.float32(math.log(1.0 / u - 2.0))
    x = np.array([[0.0, 0.0, z2]], np.float32)
    kw = dict(seed=seed, offset=off, row_stream=[0], inverse_cdf=True)
    o = run(x, **kw)
    assert o["flags"][0] & oracle.FLAG_ICDF_MARGIN
    assert sorted([int(o["token_ids"][0]), int(o["token_alt"][0])]) == [0, 1]
    o = run(np.array([[0.0, 0.0, z2 + np.float32(0.01)]], np.float32), **kw)
    assert not (o["flags"][0] & oracle.FLAG_ICDF_MARGIN)


def test_masks_match_transformers_warpers():
    # top-k, top-p and min-p applied in that order by the transformers
    # library's warpers, each on the previous one's output (so top-p sees
    # the top-k set renormalised and min-p compares with the largest kept
    # probability), give the reading's kept sets at vocabulary sizes brute
    # force cannot reach.  Continuous values (no ties, which the library's
    # sort would break arbitrarily); rows within 1e-4 of a top-p or 1e-5 of
    # a min-p boundary are skipped: the library decides them from fp32
    # cumulative sums and an fp32 softmax.
    transformers = pytest.importorskip("transformers")
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(91)
    n, V = 96, 2000
    scale = rng.choice([0.7, 1.5, 2.5], n)[:, None]   # flat to peaked rows
    x = (scale * rng.standard_normal((n, V))).astype(np.float32)
    k = rng.choice([-1, 1, 5, 50, 400], n).astype(np.int32)
    p = rng.choice([1.0, 0.95, 0.8, 0.5, 0.2], n).astype(np.float32)
    mp = rng.choice([0.0, 0.01, 0.1, 0.5], n).astype(np.float32)
    o = run(x, temperature=np.ones(n, np.float32), top_k=k, top_p=p, min_p=mp)
    ids = torch.zeros((1, 1), dtype=torch.long)
    checked = 0
    for r in range(n):
        q = np.exp(x[r].astype(np.float64) - float(x[r].max()))
        if p[r] < 1.0 and o["topp_margin"][r] < 1e-4:
            continue
        if mp[r] > 0 and np.min(np.abs(q / float(mp[r]) - 1.0)) < 1e-5:
            continue
        s = torch.from_numpy(x[r:r + 1].copy())
        if k[r] > 0:
            s = transformers.TopKLogitsWarper(int(k[r]))(ids, s)
        if p[r] < 1.0:
            s = transformers.TopPLogitsWarper(float(p[r]))(ids, s)
        if mp[r] > 0:
            s = transformers.MinPLogitsWarper(float(mp[r]))(ids, s)
        want = np.isfinite(s.numpy()[0])
        assert np.array_equal(np.isfinite(o["logprobs"][r]), want), (r, k[r], p[r], mp[r])
        np.testing.assert_allclose(o["probs"][r][want], scipy.special.softmax(x[r][want].astype(np.float64)),
                                   rtol=0, atol=1e-7)
        checked += 1
    assert checked >= 80


# ---------------------------------------------------------------- Gumbel-max distribution
def _draw_tokens(x, n_draws, chunk=100_000, inverse_cdf=False, **kw):
    V = x.shape[-1]
    counts = np.zeros(V, np.int64)
    for start in range(0, n_draws, chunk):
        n = min(chunk, n_draws - start)
        L = np.broadcast_to(x.astype(np.float32), (n, V))
        o = oracle.step(np.ascontiguousarray(L), want_probs=False, want_logprobs=False,
                        row_seed=np.full(n, 99, np.uint64), row_stream=np.zeros(n, np.uint32),
                        row_offset=np.arange(start, start + n, dtype=np.uint64), n_threads=8,
                        inverse_cdf=inverse_cdf,
                        **{k: np.broadcast_to(np.asarray(v), (n,)).copy() for k, v in kw.items()})
        assert np.all(o["row_status"] == 0)
        counts += np.bincount(o["token_ids"], minlength=V)
    return counts


def _chi2_pvalue(counts, probs):
    exp = probs * counts.sum()
    keep = exp >= 5
    obs = np.append(counts[keep], counts[~keep].sum())
    ex = np.append(exp[keep], exp[~keep].sum())
    if ex[-1] == 0:
        obs, ex = obs[:-1], ex[:-1]
    return scipy.stats.chisquare(obs, ex).pvalue


def test_gumbel_matches_categorical_chi2():
    rng = np.random.default_rng(5)
    x = (1.5 * rng.standard_normal(64)).astype(np.float32)
    counts = _draw_tokens(x, 1_000_000, temperature=np.float32(0.9))
    z = (x / np.float32(0.9)).astype(np.float32).astype(np.float64)
    assert _chi2_pvalue(counts, scipy.special.softmax(z)) > 1e-3


def test_gumbel_truncated_matches_renormalised_chi2():
    rng = np.random.default_rng(6)
    x = (1.5 * rng.standard_normal(48)).astype(np.float32)
    counts = _draw_tokens(x, 1_000_000, top_k=np.int32(10), top_p=np.float32(0.8))
    # kept set from numpy's sort: the top 10, then the 0.8 nucleus over them
    order = np.lexsort((np.arange(48), -x.astype(np.float64)))
    q = np.exp(x.astype(np.float64) - x.max())
    top = order[:10]
    c = np.cumsum(q[top])
    n_p = int(np.searchsorted(c, 0.8 * c[-1], side="left")) + 1
    kept = top[:n_p]
    probs = np.zeros(48)
    probs[kept] = q[kept] / q[kept].sum()
    assert counts[probs == 0].sum() == 0          # never outside the kept set
    assert _chi2_pvalue(counts, probs) > 1e-3


def test_gumbel_high_temperature_is_uniform():
    rng = np.random.default_rng(7)
    x = (2 * rng.standard_normal(32)).astype(np.float32)
    counts = _draw_tokens(x, 400_000, temperature=np.float32(1e6))
    assert _chi2_pvalue(counts, np.full(32, 1 / 32)) > 1e-3


def test_one_hot_row_always_picks_it():
    x = np.full((1, 100), -np.inf, np.float32)
    x[0, 37] = 2.0
    for off in range(50):
        o = run(x, offset=off, temperature=[1.3])
        assert o["token_ids"][0] == 37
        assert o["probs"][0, 37] == 1.0 and o["logprobs"][0, 37] == 0.0


def test_two_spellings_agree():
    b = workloads.random_small(11, 64, 4097, penalties=True)
    o = oracle.step(b.logits, temperature=b.temperature, top_k=b.top_k, top_p=b.top_p, min_p=b.min_p,
                    repetition_penalty=b.repetition_penalty, presence_penalty=b.presence_penalty,
                    frequency_penalty=b.frequency_penalty, history_ids=b.history_ids,
                    history_start=b.history_start, history_len=b.history_len, seed=b.seed, offset=b.offset)
    assert not np.any(o["flags"] & oracle.FLAG_SPELLING_MISMATCH)


# ---------------------------------------------------------------- penalties (reading, not fixed by the pages)
def test_penalty_hand_worked_example():
    # x = [2, -1, 0.5, 3], history [0, 0, 1, 3]; rep 2, freq 0.5, pres 0.25:
    # token 0 (count 2): 2/2 = 1, 1 - 1.0 = 0, 0 - 0.25 = -0.25
    # token 1 (count 1): -1*2 = -2, -2 - 0.5 = -2.5, -2.75
    # token 2 (count 0): 0.5 unchanged
    # token 3 (count 1): 3/2 = 1.5, 1.0, 0.75
    x = np.array([[2.0, -1.0, 0.5, 3.0]], np.float32)
    o = run(x, repetition_penalty=[2.0], frequency_penalty=[0.5], presence_penalty=[0.25],
            history_ids=np.array([0, 0, 1, 3], np.int32), history_start=[0], history_len=[4])
    z = np.array([-0.25, -2.75, 0.5, 0.75])
    np.testing.assert_allclose(o["logprobs"][0], scipy.special.log_softmax(z), rtol=1e-7)


def _penalised_shift(x, tok, ref, counts, rep=1.0, freq=0.0, pres=0.0):
    """Logit of token `tok` minus that of the untouched token `ref` after the
    penalties, read from the oracle's logprobs at T = 1, with `tok` seen
    `counts` times in the history."""
    hist = np.full(max(counts, 1), tok, np.int32) if counts else np.zeros(1, np.int32)
    o = run(x, temperature=[1.0], repetition_penalty=[rep], frequency_penalty=[freq], presence_penalty=[pres],
            history_ids=hist, history_start=[0], history_len=[counts])
    return float(o["logprobs"][0, tok]) - float(o["logprobs"][0, ref])


def test_frequency_and_presence_invariants():
    # The pages name the frequency and presence penalties and their defaults
    # ([C] "哪些参数会额外打开一趟全词表计算") but print no formula; these
    # invariants pin the terms: presence moves a seen token by a constant
    # whatever its count, frequency moves it linearly in the count, both
    # lower it, and the two add.  Dyadic values keep every step exact.
    x = np.array([0.5, 1.0, -0.75, 0.25, 2.0, -1.5, 0.0, 0.125], np.float32)
    tok, ref = 1, 0
    base = _penalised_shift(x, tok, ref, 0, freq=0.125, pres=0.375)
    assert base == pytest.approx(0.5, abs=1e-6)              # an unseen token does not move
    pres = [_penalised_shift(x, tok, ref, c, pres=0.375) for c in (1, 2, 7)]
    assert pres[0] == pytest.approx(0.5 - 0.375, abs=1e-6)   # lowered once ...
    assert pres[1] == pres[0] and pres[2] == pres[0]         # ... whatever the count
    freq = [_penalised_shift(x, tok, ref, c, freq=0.125) for c in (1, 2, 3, 4)]
    steps = np.diff([0.5] + freq)
    np.testing.assert_allclose(steps, -0.125, atol=1e-6)     # linear in the count, downwards
    both = [_penalised_shift(x, tok, ref, c, freq=0.125, pres=0.375) for c in (1, 3)]
    np.testing.assert_allclose(both, [0.5 - 0.375 - 0.125, 0.5 - 0.375 - 0.375], atol=1e-6)
    # with a repetition penalty the frequency and presence terms act on the
    # repetition-adjusted logit (the order of reading 4): a positive logit
    # 1.0 with rep 2 becomes 0.5, then - 2 * 0.125 - 0.375
    assert _penalised_shift(x, tok, ref, 2, rep=2.0, freq=0.125, pres=0.375) == pytest.approx(
        (1.0 / 2.0 - 0.25 - 0.375) - 0.5, abs=1e-6)


def test_repetition_penalty_matches_transformers_processor():
    # The repetition part of the reading is the CTRL rule as the transformers
    # library applies it (RepetitionPenaltyLogitsProcessor): each token seen
    # in the history has a negative logit multiplied and a positive one
    # divided by the penalty, once, whatever its count; other tokens stay.
    # Penalties above and below 1, zero logits and repeated ids included.
    transformers = pytest.importorskip("transformers")
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(77)
    n, V, H = 6, 257, 48
    x = rng.normal(0.0, 3.0, (n, V)).astype(np.float32)
    x[:, :6] = 0.0
    hist = rng.integers(0, V, (n, H)).astype(np.int32)
    hist[:, :12] = np.arange(12)                  # zeros and repeats in every history
    hist[:, 12:16] = hist[:, 16:20]
    rep = np.array([1.3, 0.7, 2.0, 1.0, 1.05, 3.5], np.float32)
    zeros = np.zeros(n, np.float32)
    o = run(x, temperature=np.ones(n, np.float32), repetition_penalty=rep, presence_penalty=zeros,
            frequency_penalty=zeros, history_ids=hist.ravel(), history_start=np.arange(n, dtype=np.int64) * H,
            history_len=np.full(n, H, np.int32))
    for r in range(n):
        proc = transformers.RepetitionPenaltyLogitsProcessor(penalty=float(rep[r]))
        z = proc(torch.from_numpy(hist[r:r + 1].astype(np.int64)), torch.from_numpy(x[r:r + 1].copy()))
        z = z.numpy()[0].astype(np.float64)
        # torch may divide by a scalar through its reciprocal: 1 fp32 ulp of a
        # logit is below 1e-6 here
        np.testing.assert_allclose(o["logprobs"][r], scipy.special.log_softmax(z), rtol=0, atol=2e-6)
    # a planted sign slip (dividing negative logits instead) is caught
    bad = np.where(x < 0, x / rep[:, None], x * rep[:, None]).astype(np.float64)
    seen = np.zeros((n, V), bool)
    seen[np.repeat(np.arange(n), H), hist.ravel()] = True
    wrong = np.where(seen, bad, x)
    assert np.abs(o["logprobs"] - scipy.special.log_softmax(wrong, axis=1)).max() > 1e-2


def test_penalty_identity_at_defaults_and_locality():
    b = workloads.random_small(12, 8, 300, penalties=True, mix="plain")
    common = dict(temperature=b.temperature, top_k=b.top_k, top_p=b.top_p, min_p=b.min_p,
                  seed=b.seed, offset=b.offset)
    base = oracle.step(b.logits, **common)
    ident = oracle.step(b.logits, repetition_penalty=np.ones(8, np.float32),
                        presence_penalty=np.zeros(8, np.float32), frequency_penalty=np.zeros(8, np.float32),
                        history_ids=b.history_ids, history_start=b.history_start, history_len=b.history_len,
                        **common)
    for key in ("token_ids", "probs", "logprobs"):
        np.testing.assert_array_equal(base[key], ident[key])
    # with penalties on, only history tokens move relative to the others:
    pen = oracle.step(b.logits, repetition_penalty=b.repetition_penalty, presence_penalty=b.presence_penalty,
                      frequency_penalty=b.frequency_penalty, history_ids=b.history_ids,
                      history_start=b.history_start, history_len=b.history_len, **common)
    for r in range(8):
        hist = set(b.history_ids[b.history_start[r]:b.history_start[r] + b.history_len[r]].tolist())
        others = np.array(sorted(set(range(300)) - hist))
        d = pen["logprobs"][r, others].astype(np.float64) - base["logprobs"][r, others]
        assert np.ptp(d) < 1e-4          # a common shift (the normaliser) only


# ---------------------------------------------------------------- outputs, status, modes
def test_output_byte_count_full_chain():
    # probs + logprobs are two fp32 [N, V] tensors: 8 * N * V bytes
    n, V = 64, 128_000
    assert 8 * n * V == 65_536_000
    b = workloads.config(4, n_rows=2, vocab=128_000)
    o = oracle.step(b.logits, temperature=b.temperature, want_probs=True, want_logprobs=True)
    assert o["probs"].nbytes + o["logprobs"].nbytes == 8 * 2 * V


def test_no_finite_logit_status():
    x = np.array([[np.nan, -np.inf, np.nan], [0.0, np.nan, 1.0]], np.float32)
    o = run(x)
    assert o["row_status"].tolist() == [1, 0]
    assert o["token_ids"][0] == -1
    assert np.all(o["probs"][0] == 0) and np.all(np.isneginf(o["logprobs"][0]))
    assert np.isneginf(o["logprobs"][1, 1])        # NaN reads as -inf


def test_deterministic_defaults_seed_42_stream_0():
    b = workloads.random_small(13, 6, 200, penalties=False, mix="plain")
    common = dict(temperature=b.temperature, top_k=b.top_k, top_p=b.top_p, min_p=b.min_p, offset=9)
    d = oracle.step(b.logits, deterministic=True, **common)
    e = oracle.step(b.logits, row_seed=np.full(6, 42, np.uint64), row_stream=np.zeros(6, np.uint32), **common)
    np.testing.assert_array_equal(d["token_ids"], e["token_ids"])
    # position independence: the same row alone gives the same token
    for r in range(6):
        s = oracle.step(b.logits[r:r + 1], deterministic=True,
                        **{k: (v[r:r + 1] if isinstance(v, np.ndarray) else v) for k, v in common.items()})
        assert s["token_ids"][0] == d["token_ids"][r]


def test_top_logprobs_match_sort():
    b = workloads.random_small(14, 16, 500, penalties=False)
    o = oracle.step(b.logits, temperature=b.temperature, top_k=b.top_k, top_p=b.top_p, min_p=b.min_p,
                    top_logprobs=5)
    for r in range(16):
        lp = o["logprobs"][r]
        kept = np.flatnonzero(np.isfinite(lp))
        # z order equals logprob order; sort by (-lp, index) with numpy
        order = kept[np.lexsort((kept, -lp[kept].astype(np.float64)))][:5]
        got = o["top_logprob_ids"][r]
        n = min(5, len(kept))
        np.testing.assert_array_equal(np.sort(got[:n]), np.sort(order[:n]))
        np.testing.assert_array_equal(o["top_logprob_vals"][r, :n], lp[got[:n]])
        assert np.all(got[n:] == -1) and np.all(np.isneginf(o["top_logprob_vals"][r, n:]))


# ---------------------------------------------------------------- logits processors
def test_grammar_mask_matches_scipy_on_allowed_set():
    # [B] "Constrained decoding": the bitmask removes tokens before sampling;
    # the kept distribution is the softmax over the allowed tokens only.
    rng = np.random.default_rng(21)
    n, V = 5, 203
    x = (3 * rng.standard_normal((n, V))).astype(np.float32)
    T = np.array([1.0, 0.7, 1.3, 1.0, 0.5], np.float32)
    allowed = rng.random((n, V)) < 0.3
    allowed[3] = False
    allowed[3, [7, 150]] = True                       # two tokens left
    words = np.zeros((n, (V + 31) // 32 + 1), np.uint32)   # one spare word of stride
    for r in range(n):
        for i in np.flatnonzero(allowed[r]):
            words[r, i >> 5] |= np.uint32(1 << (i & 31))
    o = run(x, temperature=T, vocab_mask=words)
    z = np.where(allowed, (x / T[:, None]).astype(np.float32), -np.inf).astype(np.float64)
    np.testing.assert_allclose(o["probs"], scipy.special.softmax(z, axis=1), rtol=0, atol=1e-7)
    lp = scipy.special.log_softmax(z, axis=1)
    assert np.array_equal(np.isneginf(o["logprobs"]), np.isneginf(lp))
    fin = np.isfinite(lp)
    np.testing.assert_allclose(o["logprobs"][fin], lp[fin], rtol=2e-7, atol=1e-6)
    assert np.all(allowed[np.arange(n), o["token_ids"]])
    # greedy over the allowed set is numpy's first argmax there
    g = run(x, temperature=np.zeros(n, np.float32), vocab_mask=words)
    np.testing.assert_array_equal(g["token_ids"], np.argmax(np.where(allowed, x, -np.inf), axis=1))
    # nothing allowed: no finite logit
    e = run(x[:1], vocab_mask=np.zeros((1, 7), np.uint32))
    assert e["row_status"][0] == 1 and e["token_ids"][0] == -1


def test_logit_bias_matches_numpy_float32_sums():
    # logit_bias ([B] sampler options): each token's entries are summed, then
    # added to its logit in fp32, before the temperature division.
    rng = np.random.default_rng(22)
    n, V = 3, 150
    x = (2 * rng.standard_normal((n, V))).astype(np.float32)
    T = np.array([0.8, 1.0, 1.7], np.float32)
    ids = np.array([5, 9, 5, 149, 0, 3, 3, 70, -1, 150], np.int32)   # -1 and 150 are ignored
    vals = np.array([1.5, -2.25, 0.375, 4.0, -100.0, 0.1, 0.2, 7.0, 9.0, 9.0], np.float32)
    start = np.array([0, 4, 0], np.int64)
    length = np.array([4, 6, 0], np.int32)
    o = run(x, temperature=T, bias_ids=ids, bias_vals=vals, bias_start=start, bias_len=length)
    xb = x.copy()
    for r in range(n):
        tot = {}
        for j in range(start[r], start[r] + length[r]):
            i = int(ids[j])
            if 0 <= i < V:
                tot[i] = vals[j] if i not in tot else np.float32(tot[i] + vals[j])
        for i, b in tot.items():
            xb[r, i] = np.float32(xb[r, i] + b)
    z = (xb / T[:, None]).astype(np.float32).astype(np.float64)
    np.testing.assert_allclose(o["probs"], scipy.special.softmax(z, axis=1), rtol=0, atol=1e-7)
    np.testing.assert_allclose(o["logprobs"], scipy.special.log_softmax(z, axis=1), rtol=2e-7, atol=1e-6)
    # the probability ratio of a biased token to an unbiased one moves by exp(b / T)
    r, i, j = 0, 149, 1
    ratio = (o["probs"][r, i] / o["probs"][r, j]) / math.exp((float(x[r, i]) - float(x[r, j])) / float(T[r]))
    assert ratio == pytest.approx(math.exp(4.0 / 0.8), rel=1e-5)
    # a +inf bias makes +inf (status 2); a NaN sum becomes -inf
    s = run(x[:1], bias_ids=np.array([3], np.int32), bias_vals=np.array([np.inf], np.float32),
            bias_start=[0], bias_len=[1])
    assert s["row_status"][0] == 2
    q = run(np.array([[-np.inf, 0.0, 1.0]], np.float32), bias_ids=np.array([0], np.int32),
            bias_vals=np.array([np.inf], np.float32), bias_start=[0], bias_len=[1])
    assert q["row_status"][0] == 0 and q["probs"][0, 0] == 0.0


def test_min_tokens_masks_stop_ids_only_while_active():
    # [C] step _apply_min_tokens_penalty: stop ids are -inf until the row has
    # produced min_tokens tokens.
    rng = np.random.default_rng(23)
    n, V = 4, 64
    x = (2 * rng.standard_normal((n, V))).astype(np.float32)
    x[:, 11] = 10.0                                   # a stop token that would dominate
    stops = np.array([11, 40, 11, 63], np.int32)
    kw = dict(stop_ids=stops, stop_start=[0, 0, 2, 0], stop_len=[2, 2, 2, 0],
              min_tokens=[5, 5, 1, 9], output_len=[0, 5, 0, 0])
    base = run(x)
    active = [True, False, True, False]               # row 3 has no stop ids
    for seed in range(40):
        o = run(x, seed=seed, **kw)
        b = run(x, seed=seed)
        for r in range(n):
            if active[r]:
                assert o["token_ids"][r] not in (11, 40, 63)
                assert o["probs"][r, 11] == 0.0
            else:
                assert o["token_ids"][r] == b["token_ids"][r]
    o = run(x, **kw)
    z = x.astype(np.float64).copy()
    z[0, [11, 40]] = -np.inf
    np.testing.assert_allclose(o["probs"][0], scipy.special.softmax(z[0]), rtol=0, atol=1e-7)
    np.testing.assert_array_equal(o["probs"][1], base["probs"][1])


def test_min_tokens_boundary_matches_transformers_processor():
    # The activation rule (stop ids masked while output_len < min_tokens) at
    # and around the boundary, against the transformers library's
    # min-length processor over a sequence of output_len tokens, with the
    # row's stop ids as its end-of-sequence ids.
    transformers = pytest.importorskip("transformers")
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(29)
    V = 50
    stops = np.array([3, 17, 49], np.int32)
    cases = [(m, L) for m in (0, 1, 4) for L in (0, max(m - 1, 0), m, m + 1)]
    n = len(cases)
    x = (2 * rng.standard_normal((n, V))).astype(np.float32)
    o = run(x, stop_ids=stops, stop_start=np.zeros(n, np.int64), stop_len=np.full(n, 3, np.int32),
            min_tokens=[m for m, _ in cases], output_len=[L for _, L in cases])
    for r, (m, L) in enumerate(cases):
        proc = transformers.MinLengthLogitsProcessor(m, [int(s) for s in stops])
        s = proc(torch.zeros((1, L), dtype=torch.long), torch.from_numpy(x[r:r + 1].copy())).numpy()[0]
        np.testing.assert_array_equal(np.isfinite(o["logprobs"][r]), np.isfinite(s), err_msg=str((m, L)))
        np.testing.assert_allclose(o["probs"][r], scipy.special.softmax(s.astype(np.float64)), rtol=0, atol=1e-7)


# ---------------------------------------------------------------- logprob modes
def test_logprob_modes_match_scipy():
    # [B] "Logprobs are temperature-scaled": the temperature mode is the
    # untruncated log_softmax(logits / T); the raw mode log_softmax(logits).
    rng = np.random.default_rng(24)
    n, V = 6, 300
    x = (3 * rng.standard_normal((n, V))).astype(np.float32)
    T = np.array([0.5, 1.0, 1.4, 0.0, 0.9, 2.0], np.float32)     # row 3 greedy
    kw = dict(temperature=T, top_k=[5, -1, 40, -1, -1, 3], top_p=[1.0, 0.8, 0.9, 1.0, 1.0, 1.0],
              min_p=[0.0, 0.0, 0.0, 0.0, 0.1, 0.0], top_logprobs=4)
    proc = run(x, **kw)
    tmp = run(x, logprob_mode="temperature", **kw)
    raw = run(x, logprob_mode="raw", **kw)
    Te = np.where(T < 1e-6, 1.0, T).astype(np.float32)
    z = (x / Te[:, None]).astype(np.float32).astype(np.float64)
    np.testing.assert_allclose(tmp["logprobs"], scipy.special.log_softmax(z, axis=1), rtol=2e-7, atol=1e-6)
    np.testing.assert_allclose(raw["logprobs"], scipy.special.log_softmax(x.astype(np.float64), axis=1),
                               rtol=2e-7, atol=1e-6)
    # tokens and probs do not depend on the mode; greedy rows agree in all modes
    for o in (tmp, raw):
        np.testing.assert_array_equal(o["token_ids"], proc["token_ids"])
        np.testing.assert_array_equal(o["probs"], proc["probs"])
    np.testing.assert_array_equal(tmp["logprobs"][3], proc["logprobs"][3])
    np.testing.assert_array_equal(raw["logprobs"][3], proc["logprobs"][3])
    # top logprobs list the largest values over every token (numpy sort)
    for o in (tmp, raw):
        for r in range(n):
            lp = o["logprobs"][r].astype(np.float64)
            order = np.lexsort((np.arange(V), -z[r]))[:4]
            np.testing.assert_array_equal(o["top_logprob_ids"][r], order)
            np.testing.assert_array_equal(o["top_logprob_vals"][r], lp[order].astype(np.float32))


# ---------------------------------------------------------------- inverse-CDF selection (seeded multinomial)
def test_icdf_uniform_is_uniform():
    u = np.array([oracle.icdf_uniform(3, 0, off) for off in range(200_000)])
    assert u.min() >= 0.0 and u.max() < 1.0
    assert scipy.stats.kstest(u, "uniform").pvalue > 1e-3
    # 53 bits: the Philox words 0 and 1 of block (0xFFFFFFFF, stream, off_lo, off_hi)
    w = oracle.philox4x32_10([0xFFFFFFFF, 5, 7, 0], [11, 0])
    x = (int(w[1]) << 32) | int(w[0])
    assert oracle.icdf_uniform(11, 5, 7) == (x >> 11) * 2.0 ** -53


def test_icdf_token_is_numpy_searchsorted():
    # the first kept token whose running mass exceeds u * total: numpy's
    # cumsum and searchsorted over the kept set in index order
    b = workloads.random_small(50, 24, 700, penalties=False)
    o = oracle.step(b.logits, temperature=b.temperature, top_k=b.top_k, top_p=b.top_p, min_p=b.min_p,
                    seed=b.seed, offset=b.offset, inverse_cdf=True)
    for r in range(24):
        p = o["probs"][r].astype(np.float64)
        if o["row_status"][r] != 0 or oracle.normalized_top_k(b.temperature[r], b.top_k[r]) == 1:
            continue
        kept = np.flatnonzero(p > 0)
        z = (b.logits[r] / b.temperature[r]).astype(np.float32).astype(np.float64)
        q = np.exp(z[kept] - z.max())
        c = np.cumsum(q)
        u = oracle.icdf_uniform(b.seed, r, b.offset)
        j = int(np.searchsorted(c, u * c[-1], side="right"))
        assert o["token_ids"][r] == kept[j]


def test_icdf_matches_categorical_chi2():
    rng = np.random.default_rng(51)
    x = (1.5 * rng.standard_normal(40)).astype(np.float32)
    counts = _draw_tokens(x, 400_000, inverse_cdf=True, temperature=np.float32(1.1))
    z = (x / np.float32(1.1)).astype(np.float32).astype(np.float64)
    assert _chi2_pvalue(counts, scipy.special.softmax(z)) > 1e-3
    counts = _draw_tokens(x, 400_000, inverse_cdf=True, top_k=np.int32(6))
    order = np.lexsort((np.arange(40), -x.astype(np.float64)))[:6]
    probs = np.zeros(40)
    probs[order] = scipy.special.softmax(x[order].astype(np.float64))
    assert counts[probs == 0].sum() == 0
    assert _chi2_pvalue(counts, probs) > 1e-3


def test_icdf_keeps_argmax_rows_and_outputs():
    b = workloads.random_small(52, 16, 300, penalties=True)
    kw = dict(temperature=b.temperature, top_k=b.top_k, top_p=b.top_p, min_p=b.min_p, seed=b.seed,
              offset=b.offset, repetition_penalty=b.repetition_penalty, presence_penalty=b.presence_penalty,
              frequency_penalty=b.frequency_penalty, history_ids=b.history_ids, history_start=b.history_start,
              history_len=b.history_len)
    g = oracle.step(b.logits, **kw)
    i = oracle.step(b.logits, inverse_cdf=True, **kw)
    np.testing.assert_array_equal(g["probs"], i["probs"])
    np.testing.assert_array_equal(g["logprobs"], i["logprobs"])
    top1 = np.array([oracle.normalized_top_k(t, k) == 1 for t, k in zip(b.temperature, b.top_k)])
    np.testing.assert_array_equal(g["token_ids"][top1], i["token_ids"][top1])
