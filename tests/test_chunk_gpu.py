"""The chunked-row kernel (rows longer than 4096 values that keep every
value -- Gumbel-max or greedy, no penalties, processors or top-logprob list
-- in steps that want only token ids) against the CPU oracle on a real
MI355X, through the C ABI, under the parity rules of parity.py; every step
asserts which kernel ran."""
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
def sampler_chunk():
    _need_gpu()
    import decode_step_token_sampler_amd as dsts
    s = dsts.Sampler(96, 1 << 20, max_history_per_row=64, max_top_logprobs=8)
    yield s
    s.close()


def check(b, s, kernel="chunk", **over):
    g = run_gpu(s, b, **over)
    assert g["kernel"] == kernel, g["kernel"]
    o = run_oracle(b, **{k: v for k, v in over.items() if k == "logprob_mode"})
    r = compare(g, o)
    print(b.name, r)
    assert r.ok(), r
    return g, o


def ids_only(seed, n, V, dtype):
    b = workloads.random_small(seed, n, V, dtype, penalties=False, mix="plain")
    b.want_probs, b.want_logprobs, b.top_logprobs = False, False, 0
    return b


@pytest.mark.parametrize("t", [1.0, 0.0])
def test_batch1_decode(sampler_chunk, t):
    # the batch-1 decode workload at full size: Gumbel-max at T = 1, greedy at T = 0
    for step in range(3):
        check(workloads.config(2, temperature=t, step=step), sampler_chunk)


# sizes across the chunk boundaries (1024 values per chunk at one group per
# thread, which rows of up to 64 such chunks take), ragged tails, longer
# rows at two groups per thread, and batches of more than 4096 chunks at two
# (four groups per thread)
@pytest.mark.parametrize("seed,n,V,dtype", [(170, 1, 4097, "f32"), (171, 3, 5000, "bf16"), (172, 5, 8191, "f32"),
                                            (173, 7, 8192, "bf16"), (174, 2, 151_936, "bf16"),
                                            (175, 30, 151_936, "bf16"), (176, 64, 151_936, "f32"),
                                            (177, 2, 262_144, "bf16"), (178, 2, 1 << 20, "bf16")])
def test_random_rows(sampler_chunk, seed, n, V, dtype):
    check(ids_only(seed, n, V, dtype), sampler_chunk)


def test_many_long_rows(sampler_chunk):
    # 96 rows of 262,144 values: four groups per thread, 64 chunks a row,
    # 6,144 workgroups in the launch
    check(ids_only(179, 96, 262_144, "bf16"), sampler_chunk)


def test_edge_rows(sampler_chunk):
    V = 5000
    x = np.random.default_rng(5).standard_normal((8, V)).astype(np.float32)
    x[0, :] = -np.inf
    x[1, :] = np.nan
    x[2, 4100] = np.inf                 # +inf in the last chunk
    x[3, :] = -np.inf
    x[3, 4999] = 1.0                    # the only finite value, the last index
    x[4, ::2] = np.nan
    x[5, 1000:1100] = 9.0               # a plateau across a chunk boundary
    x[6, 2048:] = -np.inf               # whole chunks without a finite value
    x[7, :] = 3.0                       # every value equal
    b = workloads.Batch("edge rows", "f32", x,
                        temperature=np.array([1, 1, 1, 0.5, 0.8, 1e-7, 1.3, 0], np.float32),
                        top_k=np.full(8, -1, np.int32), top_p=np.ones(8, np.float32), min_p=np.zeros(8, np.float32),
                        want_probs=False, want_logprobs=False)
    g, _ = check(b, sampler_chunk)
    assert g["row_status"].tolist() == [1, 1, 2, 0, 0, 0, 0, 0]
    assert g["token_ids"][3] == 4999 and g["token_ids"][5] == 1000 and g["token_ids"][7] == 0
    assert g["token_ids"][6] < 2048


def test_unaligned_rows(sampler_chunk):
    b = ids_only(180, 5, 9001, "bf16")
    L, _ = to_device(b)
    wide = torch.full((b.n_rows, 9003), float("nan"), dtype=L.dtype, device=L.device)
    wide[:, 1:9002] = L
    g = run_gpu(sampler_chunk, b, logits=wide[:, 1:9002])
    assert g["kernel"] == "chunk"
    r = compare(g, run_oracle(b))
    assert r.ok(), r


def test_repeated_steps_of_other_shapes(sampler_chunk):
    # the last chunk of a row resets the row's arrival count for the next
    # launch: steps of other row counts and chunk counts in a row, each checked
    for seed, n, V in [(181, 40, 151_936), (182, 3, 20_000), (183, 40, 151_936), (184, 1, 4097)]:
        check(ids_only(seed, n, V, "bf16"), sampler_chunk)


def test_agrees_with_the_row_kernel():
    import decode_step_token_sampler_amd as dsts
    row = dsts.Sampler(64, 200_000, max_history_per_row=64, max_top_logprobs=8, force_path="filtered")
    chunk = dsts.Sampler(64, 200_000, max_history_per_row=64, max_top_logprobs=8)
    try:
        b = ids_only(185, 16, 151_936, "bf16")
        ga, o = check(b, row, kernel="row")
        gc, _ = check(b, chunk)
        ok = (o["flags"] & 0xF) == 0
        assert np.array_equal(ga["token_ids"][ok], gc["token_ids"][ok])
    finally:
        row.close()
        chunk.close()


def test_forced_greedy_path():
    import decode_step_token_sampler_amd as dsts
    s = dsts.Sampler(64, 200_000, max_history_per_row=64, max_top_logprobs=8, force_path="greedy")
    try:
        b = ids_only(186, 20, 70_000, "f32")
        g = run_gpu(s, b)
        assert g["kernel"] == "chunk"
        # the first argmax of the processed logits z = fl32(x / T) (T = 1 on
        # greedy rows; NaN never wins)
        T = np.where(b.temperature < 1e-6, 1.0, b.temperature).astype(np.float32)
        z = (b.logits.astype(np.float32) / T[:, None]).astype(np.float32)
        z[np.isnan(z)] = -np.inf
        assert np.array_equal(g["token_ids"], np.argmax(z, axis=1))
        assert np.all(g["row_status"] == 0)
    finally:
        s.close()


def test_steps_outside_its_scope(sampler_chunk):
    b = ids_only(187, 4, 9000, "f32")
    b.want_probs = True
    check(b, sampler_chunk, kernel="row")
    b = ids_only(188, 4, 9000, "f32")
    b.top_logprobs = 3
    check(b, sampler_chunk, kernel="row")
    b = ids_only(189, 4, 9000, "f32")
    b.top_k = np.full(4, 5, np.int32)
    check(b, sampler_chunk, kernel="row")
    b = workloads.random_small(190, 4, 9000, "f32", mix="plain")  # with penalties
    b.want_probs, b.want_logprobs, b.top_logprobs = False, False, 0
    check(b, sampler_chunk, kernel="row")
    check(ids_only(191, 4, 4096, "f32"), sampler_chunk, kernel="small")
