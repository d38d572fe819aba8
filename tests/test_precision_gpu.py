"""Top-p decisions near the oracle's flag margin, on the GPU through the C
ABI: rows whose top-p crossing lies between 1e-6 and 3e-6 (relative to the
row's mass) from its target are not flagged by the oracle, so the GPU must
take the same kept set, token and outputs.  The GPU finds such a crossing
from fp32-quality window masses and must send rows it cannot decide with
certainty to its exact path."""
import numpy as np
import pytest

import workloads
from parity import compare, run_gpu, run_oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def near_margin_batch(n, V, seed):
    """Rows of Zipf-biased logits at temperature 1 with top_p placed 1e-6 to
    3e-6 (relative) beyond the end of a chosen tie group (lo side) or before
    it (hi side); crossings from a few to thousands of tokens deep."""
    rng = np.random.default_rng(seed)
    L = np.stack([workloads.zipf_row(np.random.default_rng([seed, r]), V)[0] for r in range(n)])
    L = (L * np.float32(1.6)).astype(np.float32)   # flatter rows: deeper crossings
    top_p = np.zeros(n, np.float32)
    want = []
    for r in range(n):
        z = L[r].astype(np.float64)
        order = np.lexsort((np.arange(V), -z))
        q = np.exp(z[order] - z.max())
        cum = np.cumsum(q)
        tot = cum[-1]
        while True:
            j = int(rng.integers(2, min(V - 1, 4000)))   # the crossing group ends at position j
            if z[order[j]] != z[order[j + 1]] and z[order[j - 1]] != z[order[j]] and q[j] > 1e-5 * tot:
                break
        delta = rng.uniform(1.4e-6, 2.6e-6) * tot
        side = r % 2
        target = cum[j] - delta if side == 0 else cum[j - 1] + delta
        top_p[r] = np.float32(target / tot)
        want.append((j, side))
    b = workloads.Batch("near-margin top-p", "f32", L, temperature=np.ones(n, np.float32),
                        top_k=np.full(n, -1, np.int32), top_p=top_p, min_p=np.zeros(n, np.float32),
                        seed=seed, offset=3, want_probs=True, want_logprobs=True, top_logprobs=4)
    return b


@pytest.mark.parametrize("seed,V", [(1, 128_000), (2, 151_936), (3, 40_000)])
def test_topp_crossings_near_the_flag_margin(seed, V):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_step_token_sampler_amd as dsts
    n = 32
    b = near_margin_batch(n, V, seed)
    o = run_oracle(b)
    # the construction lands every row inside [1e-6, 3e-6] and unflagged
    assert np.all((o["topp_margin"] >= 1e-6) & (o["topp_margin"] <= 3e-6)), o["topp_margin"]
    assert not np.any(o["flags"]), o["flags"]
    s = dsts.Sampler(n, V, max_history_per_row=0, max_top_logprobs=4)
    g = run_gpu(s, b)
    r = compare(g, o)
    assert r.ok() and r.flagged == 0, r
    np.testing.assert_array_equal(np.isfinite(g["logprobs"]), np.isfinite(o["logprobs"]))
    s.close()
