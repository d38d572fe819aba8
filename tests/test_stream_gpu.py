"""The streaming kernel (steps that want only token ids and top logprobs of
the sampled distribution: one workgroup per row, the row read in passes)
against the CPU oracle on a real MI355X, through the C ABI, under the parity
rules of parity.py.  Every step asserts which kernel ran; the rows the
streaming kernel leaves (ranges too full, thresholds outside its window)
are sampled by the row kernel after it, and the cases below force both."""
import numpy as np
import pytest

import workloads
from parity import compare, run_gpu, run_oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def sampler_stream():
    _need_gpu()
    import decode_step_token_sampler_amd as dsts
    s = dsts.Sampler(512, 262_144, max_history_per_row=2048, max_top_logprobs=32, stream_rows="force")
    yield s
    s.close()


@pytest.fixture(scope="module")
def sampler_auto():
    _need_gpu()
    import decode_step_token_sampler_amd as dsts
    s = dsts.Sampler(512, 262_144, max_history_per_row=2048, max_top_logprobs=32)
    yield s
    s.close()


def ids_only(b, K):
    b.want_probs = False
    b.want_logprobs = False
    b.top_logprobs = K
    return b


def check(b, s, kernel="stream", **over):
    g = run_gpu(s, b, **over)
    assert g["kernel"] == kernel, g["kernel"]
    o = run_oracle(b)
    r = compare(g, o)
    print(b.name, "K=%d" % b.top_logprobs, r)
    assert r.ok(), r
    return g, o


@pytest.mark.parametrize("K", [0, 5, 20])
@pytest.mark.parametrize("seed,n,V,dtype,ties", [
    (100, 1, 1, "f32", False), (101, 3, 2, "bf16", False), (102, 17, 63, "f32", True), (103, 16, 64, "bf16", False),
    (104, 9, 65, "f32", False), (105, 11, 1000, "bf16", True), (106, 13, 4097, "f32", False),
    (107, 8, 50_001, "bf16", False), (108, 6, 131_071, "f32", True), (109, 24, 40_000, "f32", False),
])
def test_random_shapes(sampler_stream, seed, n, V, dtype, ties, K):
    check(ids_only(workloads.random_small(seed, n, V, dtype, ties=ties), min(K, 32)), sampler_stream)


def test_forks_workload_reduced(sampler_stream):
    check(workloads.config(5, n_rows=64, vocab=32_768), sampler_stream)


def test_forks_workload_full_size_automatic(sampler_auto):
    """N=512 forks at V=256,000: the handle picks the streaming kernel by itself."""
    b = workloads.config(5)
    g, _ = check(b, sampler_auto)
    tok = g["token_ids"].reshape(-1, 4)
    assert np.mean(tok[:, 0] == tok[:, 1]) < 0.9


@pytest.mark.parametrize("K", [0, 20])
def test_full_chain_ids_only(sampler_stream, K):
    check(ids_only(workloads.config(4), K), sampler_stream)


def test_plain_and_greedy_rows(sampler_stream):
    """Rows that keep every value (Gumbel-max over the whole row) and greedy
    rows, with and without a top-logprob list."""
    for K in (0, 8):
        b = ids_only(workloads.random_small(120, 12, 30_000, "bf16", mix="plain"), K)
        check(b, sampler_stream)


def test_edge_rows(sampler_stream):
    V = 300
    x = np.random.default_rng(3).standard_normal((7, V)).astype(np.float32)
    x[0, :] = -np.inf                 # no finite logit
    x[1, :] = np.nan                  # NaN reads as -inf
    x[2, 5] = np.inf                  # +inf
    x[3, :] = -np.inf
    x[3, 17] = 1.0                    # one finite value
    x[4, ::2] = np.nan                # half NaN
    b = workloads.Batch("edge rows", "f32", x, temperature=np.array([1, 1, 1, 0.5, 0.8, 1e-7, 1], np.float32),
                        top_k=np.array([-1, 5, -1, 3, 2, -1, 1], np.int32),
                        top_p=np.array([1, 1, 1, 0.5, 0.9, 1, 1], np.float32),
                        min_p=np.zeros(7, np.float32), want_probs=False, want_logprobs=False, top_logprobs=4)
    g, _ = check(b, sampler_stream)
    assert g["row_status"].tolist() == [1, 1, 2, 0, 0, 0, 0]
    assert g["token_ids"][:3].tolist() == [-1, -1, -1]
    assert g["token_ids"][3] == 17


def test_rows_left_to_the_row_kernel(sampler_stream):
    """Rows the streaming kernel cannot settle from its gathered values: a
    top-k bin holding thousands of equal values, a flat row under top-p, a
    top-k reaching below the window, a top-p crossing in crowded bins; mixed
    with ordinary rows.  Every row must still equal the oracle."""
    rng = np.random.default_rng(7)
    n, V = 10, 20_000
    x = (3.0 * rng.standard_normal((n, V))).astype(np.float32)
    x[0, :5000] = 9.0                 # 5,000 equal maxima, top_k 10
    x[1, :] = 0.25                    # a flat row, top_p 0.5
    x[2] = np.linspace(0.0, -400.0, V, dtype=np.float32)  # top_k deep below a 16-nat window
    x[3] = (0.3 * rng.standard_normal(V)).astype(np.float32)  # crowded bins at the top-p crossing
    T = np.ones(n, np.float32)
    top_k = np.array([10, -1, 15_000, -1, 50, -1, 5, -1, 20, -1], np.int32)
    top_p = np.array([1, 0.5, 1, 0.5, 0.9, 0.9, 1, 1, 0.95, 1], np.float32)
    min_p = np.array([0, 0, 0, 0, 0, 0.05, 0, 0.1, 0, 0], np.float32)
    for K in (0, 6):
        b = workloads.Batch("left rows", "f32", x, temperature=T, top_k=top_k, top_p=top_p, min_p=min_p, seed=11,
                            offset=3, want_probs=False, want_logprobs=False, top_logprobs=K)
        check(b, sampler_stream)


def test_forced_greedy_path():
    """SAMPLER_FORCE_PATH_GREEDY: every row takes the first argmax (the head
    of its top-logprob list, whose every entry still equals the oracle's)."""
    import decode_step_token_sampler_amd as dsts
    s = dsts.Sampler(64, 65_536, max_history_per_row=256, max_top_logprobs=8, stream_rows="force",
                     force_path="greedy")
    try:
        b = ids_only(workloads.random_small(130, 20, 20_000, "f32", history_len=200), 6)
        g = run_gpu(s, b)
        assert g["kernel"] == "stream"
        r = compare(g, run_oracle(b))
        assert r.toplp_mismatch == 0 and r.status_mismatch == 0, r
        ok = g["row_status"] == 0
        assert np.array_equal(g["token_ids"][ok], g["top_logprob_ids"][ok, 0])
    finally:
        s.close()


def test_row_kernel_and_streaming_kernel_agree():
    """The same ids-only batch on handles that never and always stream: both
    match the oracle, and their tokens agree on every unflagged row."""
    import decode_step_token_sampler_amd as dsts
    a = dsts.Sampler(64, 131_072, max_history_per_row=2048, max_top_logprobs=32, stream_rows="off")
    s = dsts.Sampler(64, 131_072, max_history_per_row=2048, max_top_logprobs=32, stream_rows="force")
    try:
        b = ids_only(workloads.config(4, set_id=1), 10)
        ga, o = check(b, a, kernel="row")
        gs, _ = check(b, s)
        unflagged = (o["flags"] & 0xF) == 0
        assert np.array_equal(ga["token_ids"][unflagged], gs["token_ids"][unflagged])
    finally:
        a.close()
        s.close()


def test_replay_stability(sampler_stream):
    b = ids_only(workloads.config(5, n_rows=96, vocab=50_000), 20)
    first = run_gpu(sampler_stream, b)
    for _ in range(10):
        again = run_gpu(sampler_stream, b)
        for k in ("token_ids", "top_logprob_ids", "top_logprob_vals", "row_status"):
            assert np.array_equal(first[k], again[k]), k


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unaligned_rows(sampler_stream, dtype):
    """An odd base offset and an odd row stride (scalar loads)."""
    from parity import to_device
    b = ids_only(workloads.random_small(140, 6, 1001, dtype), 5)
    L, H = to_device(b)
    wide = torch.full((b.n_rows, 1003), float("nan"), dtype=L.dtype, device=L.device)
    wide[:, 1:1002] = L
    g = run_gpu(sampler_stream, b, logits=wide[:, 1:1002], history=H)
    assert g["kernel"] == "stream"
    r = compare(g, run_oracle(b))
    assert r.ok(), r


def test_handle_too_large_for_streaming_takes_the_row_kernel():
    """A handle whose largest vocabulary and histories (2^19 values, 4,096-id
    histories) need more LDS than the streaming kernel's workgroup has never
    streams, even forced: its steps run on the row kernel and still equal
    the oracle."""
    import decode_step_token_sampler_amd as dsts
    s = dsts.Sampler(8, 1 << 19, max_history_per_row=4096, max_top_logprobs=8, stream_rows="force")
    try:
        b = ids_only(workloads.random_small(132, 6, 1 << 19, "bf16", history_len=3000), 4)
        check(b, s, kernel="row")
    finally:
        s.close()
