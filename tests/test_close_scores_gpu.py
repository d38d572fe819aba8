"""Rows whose two best Gumbel-max scores z - ln E differ by less than an
fp32 score resolves (2e-6 to 5e-4 nats) but more than the oracle's near-tie
margin: the small-row and chunked-row kernels rank candidates by an fp32
score and settle every value within 2^-10 nats of the best by the exact fp64
score, the row and streaming kernels score every value that passes their
linear-domain bound in fp64, so each must return the oracle's token on each
row.  The rows are
built from the oracle's own Exp(1) draws (seed, stream = row, offset): every
value sits far below except two tokens whose logits put their scores the
given gap apart."""
import numpy as np
import pytest

import oracle
import workloads
from parity import compare, run_gpu, run_oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GAPS = [2e-6, -3e-6, 1e-5, -4e-5, 2e-4, -5e-4, 6e-6, -1.5e-5]


def close_rows(V, pairs, seed=5, offset=9, base=-60.0, top=4.0):
    """Logits (fp32) with two close candidates per row; the exact fp64 score
    gap each row ends up with (b minus a, after fp32 rounding)."""
    n = len(pairs)
    x = np.full((n, V), base, np.float32)
    gaps = []
    for r, ((a, b), gap) in enumerate(zip(pairs, GAPS[:n])):
        lnE = np.log(oracle.exp1_draws(seed, r, offset, V))
        x[r, a] = np.float32(lnE[a] + top)
        x[r, b] = np.float32(lnE[b] + top + gap)
        gaps.append((float(x[r, b]) - lnE[b]) - (float(x[r, a]) - lnE[a]))
    return x, np.array(gaps)


def run_close(kernel, V, pairs, **handle):
    import decode_step_token_sampler_amd as dsts
    x, gaps = close_rows(V, pairs)
    n = x.shape[0]
    b = workloads.Batch("close scores", "f32", x, temperature=np.ones(n, np.float32), top_k=np.full(n, -1, np.int32),
                        top_p=np.ones(n, np.float32), min_p=np.zeros(n, np.float32), seed=5, offset=9,
                        want_probs=False, want_logprobs=False)
    s = dsts.Sampler(16, max(V, 8192), max_history_per_row=0, **handle)
    try:
        g = run_gpu(s, b)
    finally:
        s.close()
    assert g["kernel"] == kernel, g["kernel"]
    o = run_oracle(b)
    # every gap is far from fp32's reach and above the oracle's near-tie margin
    assert np.all(np.abs(gaps) > 1.5e-6) and np.all(np.abs(gaps) < 1e-3), gaps
    assert np.all((o["flags"] & oracle.FLAG_GUMBEL_NEAR_TIE) == 0), o["flags"]
    want = np.array([pb if gp > 0 else pa for (pa, pb), gp in zip(pairs, gaps)])
    assert np.array_equal(o["token_ids"], want), (o["token_ids"], want)
    assert np.array_equal(g["token_ids"], want), (g["token_ids"], want, gaps)
    r = compare(g, o)
    assert r.ok(), r


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_small_kernel_close_scores():
    _need_gpu()
    # pairs in one thread's group, in adjacent groups and far apart
    run_close("small", 1000, [(3, 900), (10, 11), (0, 999), (512, 513), (100, 101), (4, 8), (2, 700), (300, 301)])


def test_chunk_kernel_close_scores():
    _need_gpu()
    # pairs within one chunk and across chunks (1,024 values per chunk)
    run_close("chunk", 9000, [(3, 8900), (10, 11), (0, 8999), (1023, 1024), (2047, 5000), (4, 8), (2, 7000),
                              (4096, 4097)])


CHUNK_PAIRS = [(3, 8900), (10, 11), (0, 8999), (1023, 1024), (2047, 5000), (4, 8), (2, 7000), (4096, 4097)]


def test_row_kernel_close_scores():
    _need_gpu()
    run_close("row", 9000, CHUNK_PAIRS, force_path="filtered")


def test_stream_kernel_close_scores():
    _need_gpu()
    run_close("stream", 9000, CHUNK_PAIRS, stream_rows="force")
