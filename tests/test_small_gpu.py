"""The small-row kernel (rows of at most 4096 values that keep every value:
Gumbel-max or greedy, no penalties, processors or top-logprob list) against
the CPU oracle on a real MI355X, through the C ABI, under the parity rules
of parity.py; every step asserts which kernel ran."""
import numpy as np
import pytest

import workloads
from parity import compare, run_gpu, run_oracle, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def sampler_small():
    _need_gpu()
    import decode_step_token_sampler_amd as dsts
    s = dsts.Sampler(64, 8192, max_history_per_row=64, max_top_logprobs=8)
    yield s
    s.close()


def check(b, s, kernel="small", **over):
    g = run_gpu(s, b, **over)
    assert g["kernel"] == kernel, g["kernel"]
    o = run_oracle(b, **{k: v for k, v in over.items() if k == "logprob_mode"})
    r = compare(g, o)
    print(b.name, r)
    assert r.ok(), r
    return g, o


def plain(seed, n, V, dtype, probs=True, logprobs=True):
    b = workloads.random_small(seed, n, V, dtype, penalties=False, mix="plain")
    b.want_probs, b.want_logprobs, b.top_logprobs = probs, logprobs, 0
    return b


def test_workload1_gumbel_only(sampler_small):
    check(workloads.config(1), sampler_small)


@pytest.mark.parametrize("seed,n,V,dtype", [(150, 1, 1, "f32"), (151, 3, 2, "bf16"), (152, 17, 63, "f32"),
                                            (153, 16, 64, "bf16"), (154, 9, 65, "f32"), (155, 11, 1000, "bf16"),
                                            (156, 13, 4095, "f32"), (157, 40, 4096, "bf16")])
def test_random_plain_rows(sampler_small, seed, n, V, dtype):
    check(plain(seed, n, V, dtype), sampler_small)


def test_many_rows_through_the_record_ring():
    # more rows than the kernel arguments carry (72): the records go through
    # the pinned ring to device memory
    import decode_step_token_sampler_amd as dsts
    s = dsts.Sampler(300, 4096, max_history_per_row=0)
    try:
        check(plain(158, 300, 777, "bf16"), s)
    finally:
        s.close()


@pytest.mark.parametrize("probs,logprobs", [(False, False), (True, False), (False, True)])
def test_output_subsets(sampler_small, probs, logprobs):
    check(plain(160, 12, 3000, "f32", probs, logprobs), sampler_small)


def test_temperature_logprob_mode(sampler_small):
    # untruncated rows: the temperature mode's logprobs are the processed ones
    check(plain(161, 10, 2048, "bf16"), sampler_small, logprob_mode="temperature")


def test_edge_rows(sampler_small):
    V = 300
    x = np.random.default_rng(4).standard_normal((6, V)).astype(np.float32)
    x[0, :] = -np.inf
    x[1, :] = np.nan
    x[2, 5] = np.inf
    x[3, :] = -np.inf
    x[3, 17] = 1.0
    x[4, ::2] = np.nan
    x[5, 100:140] = 9.0                 # a plateau of equal maxima
    b = workloads.Batch("edge rows", "f32", x, temperature=np.array([1, 1, 1, 0.5, 0.8, 1e-7], np.float32),
                        top_k=np.full(6, -1, np.int32), top_p=np.ones(6, np.float32), min_p=np.zeros(6, np.float32),
                        want_probs=True, want_logprobs=True)
    g, _ = check(b, sampler_small)
    assert g["row_status"].tolist() == [1, 1, 2, 0, 0, 0]
    assert g["token_ids"][3] == 17 and g["token_ids"][5] == 100


def test_unaligned_rows(sampler_small):
    b = plain(162, 6, 1001, "f32")
    L, _ = to_device(b)
    wide = torch.full((b.n_rows, 1003), float("nan"), dtype=L.dtype, device=L.device)
    wide[:, 1:1002] = L
    g = run_gpu(sampler_small, b, logits=wide[:, 1:1002])
    assert g["kernel"] == "small"
    r = compare(g, run_oracle(b))
    assert r.ok(), r


def test_agrees_with_the_row_kernel():
    import decode_step_token_sampler_amd as dsts
    row = dsts.Sampler(64, 8192, max_history_per_row=64, max_top_logprobs=8, force_path="filtered")
    small = dsts.Sampler(64, 8192, max_history_per_row=64, max_top_logprobs=8)
    try:
        b = plain(163, 32, 4096, "f32")
        ga, o = check(b, row, kernel="row")
        gs, _ = check(b, small)
        ok = (o["flags"] & 0xF) == 0
        assert np.array_equal(ga["token_ids"][ok], gs["token_ids"][ok])
    finally:
        row.close()
        small.close()


def test_forced_greedy_path():
    import decode_step_token_sampler_amd as dsts
    s = dsts.Sampler(64, 8192, max_history_per_row=64, max_top_logprobs=8, force_path="greedy")
    try:
        b = plain(164, 20, 2500, "bf16")
        g = run_gpu(s, b)
        assert g["kernel"] == "small"
        r = compare(g, run_oracle(b))
        assert r.max_prob_err <= 1e-6 and r.max_logprob_err <= 1e-5 and r.inf_mismatch == 0
        ok = np.flatnonzero(g["row_status"] == 0)
        # the first argmax of the processed logits holds the largest probability
        tok = g["token_ids"][ok]
        assert np.array_equal(g["probs"][ok, tok], g["probs"][ok].max(axis=1))
    finally:
        s.close()


def test_rows_outside_its_scope_take_the_row_kernel(sampler_small):
    b = plain(165, 4, 1000, "f32")
    b.top_k = np.full(4, 5, np.int32)
    check(b, sampler_small, kernel="row")
    b = plain(166, 4, 1000, "f32")
    b.top_logprobs = 3
    check(b, sampler_small, kernel="row")
    b = workloads.random_small(167, 4, 1000, "f32", mix="plain")  # with penalties
    check(b, sampler_small, kernel="row")
    check(plain(168, 4, 4097, "f32"), sampler_small, kernel="row")
