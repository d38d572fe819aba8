"""The parity rules of tests/parity.py on the CPU: flagged rows are checked
against what their flag allows (an allowed kept set's outputs, or the
token on the other side of a near-tie), never skipped, and a batch may flag
only a few of its rows.  The "GPU" outputs here are oracle outputs with a
planted change."""
import math

import numpy as np

import oracle
import workloads
from parity import compare, run_oracle


def _batch(x, **params):
    x = np.atleast_2d(np.asarray(x, np.float32))
    n = x.shape[0]
    b = workloads.Batch("rules", "f32", x, temperature=np.ones(n, np.float32), top_k=np.full(n, -1, np.int32),
                        top_p=np.ones(n, np.float32), min_p=np.zeros(n, np.float32), want_probs=True,
                        want_logprobs=True, top_logprobs=2)
    for k, v in params.items():
        cur = getattr(b, k, None)
        setattr(b, k, np.asarray(v, dtype=cur.dtype) if isinstance(cur, np.ndarray) else v)
    return b


def _as_gpu(o):
    return {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in o.items() if not k.startswith("_")}


def _topp_flagged():
    # the crossing on the boundary (to fp32 precision of top_p), min-p 0.3
    # keeps the second token: kept sets {0} and {0, 1} are both allowed
    p = np.float32(1.0 / (1.0 + math.exp(-1.0) + math.exp(-4.0)))
    b = _batch([[1.0, 0.0, -3.0]] * 3, top_p=[p] * 3, min_p=[0.3] * 3)
    b.top_p[1] = np.float32(0.6)   # rows 1 and 2 unflagged
    b.top_p[2] = np.float32(0.6)
    return b


def test_flagged_row_matching_an_allowed_alternative_passes():
    b = _topp_flagged()
    o = run_oracle(b, n_threads=1)
    assert o["flags"][0] & oracle.FLAG_TOPP_MARGIN and not o["flags"][1]
    logits, kw = o["_call"]
    alts = oracle.row_alternatives(logits, 0, **kw)
    assert len(alts) == 2
    for kept in alts:
        g = _as_gpu(o)
        alt = oracle.row_with_kept(logits, 0, kept, **kw)
        for k in ("token_ids", "probs", "logprobs", "top_logprob_vals", "top_logprob_ids"):
            g[k][0] = alt[k]
        r = compare(g, o)
        assert r.ok() and r.flagged == 1 and r.flagged_by_class["topp_margin"] == 1, r


def test_flagged_row_with_a_wrong_value_fails():
    b = _topp_flagged()
    o = run_oracle(b, n_threads=1)
    g = _as_gpu(o)
    g["probs"][0, 0] += 1e-5          # a prob off by more than the tolerance
    r = compare(g, o)
    assert not r.ok() and r.flagged_failed == [0]
    g = _as_gpu(o)
    g["token_ids"][0] = 2             # a token no allowed set keeps
    assert compare(g, o).flagged_failed == [0]


def test_kept_set_outside_the_allowed_ones_fails():
    b = _topp_flagged()
    o = run_oracle(b, n_threads=1)
    logits, kw = o["_call"]
    g = _as_gpu(o)
    alt = oracle.row_with_kept(logits, 0, np.array([True, True, True]), **kw)   # all three kept
    for k in ("token_ids", "probs", "logprobs", "top_logprob_vals", "top_logprob_ids"):
        g[k][0] = alt[k]
    assert compare(g, o).flagged_failed == [0]


def test_near_tie_row_takes_either_of_the_two_best():
    seed, off = 5, 9
    E = oracle.exp1_draws(seed, 0, off, 4)
    a = np.float32(math.log(E[1] / E[0]))
    b = _batch([[0.0, a, -6.0, -6.0]], seed=seed, offset=off, row_stream=np.zeros(1, np.uint32))
    o = run_oracle(b, n_threads=1)
    assert o["flags"][0] & oracle.FLAG_GUMBEL_NEAR_TIE
    g = _as_gpu(o)
    g["token_ids"][0] = o["token_alt"][0]
    assert compare(g, o).ok()
    g["token_ids"][0] = 3
    assert not compare(g, o).ok()
    # the other outputs are still compared on a near-tie row
    g = _as_gpu(o)
    g["logprobs"][0, 1] -= 1e-4
    assert not compare(g, o).ok()


def test_unflagged_rows_are_exact():
    b = _topp_flagged()
    o = run_oracle(b, n_threads=1)
    g = _as_gpu(o)
    g["token_ids"][1] = 1 - g["token_ids"][1]
    r = compare(g, o)
    assert r.token_mismatch == [1] and not r.ok()


def test_flag_ceiling():
    # twenty flagged rows of twenty: more than 5% of the batch
    p = np.float32(1.0 / (1.0 + math.exp(-1.0) + math.exp(-4.0)))
    b = _batch([[1.0, 0.0, -3.0]] * 20, top_p=[p] * 20, min_p=[0.3] * 20)
    o = run_oracle(b, n_threads=1)
    r = compare(_as_gpu(o), o)
    assert r.flagged == 20 and not r.flagged_failed and not r.ok()
