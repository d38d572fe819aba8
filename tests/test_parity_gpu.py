"""Parity of the HIP library (through the C ABI) with the CPU oracle on a
real MI355X, plus invariants: replay, run-to-run stability, path invariance,
deterministic batch invariance and the Gumbel-max distribution.

Parity rules (also in parity.py): token ids bit-exact except oracle-flagged
near-tie / boundary rows; probs within 1e-6; logprobs within 1e-5 with an
identical -inf pattern; top logprobs ids identical and values within 1e-5.
"""
import numpy as np
import pytest

import workloads
from parity import PROB_TOL, LOGPROB_TOL, compare, run_gpu, run_oracle, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def sampler():
    _need_gpu()
    import decode_step_token_sampler_amd as dsts
    s = dsts.Sampler(512, 262_144, max_history_per_row=2048, max_top_logprobs=32)
    yield s
    s.close()


def check(batch, sampler, rows=None, **over):
    g = run_gpu(sampler, batch, **over)
    sub = batch if rows is None else batch.subset(rows)
    o = run_oracle(sub, **{k: v for k, v in over.items() if k == "deterministic"})
    r = compare(g, o, rows)
    print(batch.name, r)
    assert r.ok(), r
    return g, o, r


# ------------------------------------------------------------ the five workloads
def test_workload1_gumbel_only(sampler):
    g, o, r = check(workloads.config(1), sampler)
    assert g["path"] == "gumbel"


def test_workload2_batch1_gumbel_and_greedy(sampler):
    sets = [workloads.config(2, set_id=s) for s in range(4)]
    for step in range(48):
        b = sets[step % 4]
        b.offset = step
        check(b, sampler)
    greedy = workloads.config(2, temperature=0.0)
    g, o, r = check(greedy, sampler)
    assert g["path"] == "greedy"
    x = workloads.bf16_bits_to_f32(greedy.logits)
    assert g["token_ids"][0] == int(np.argmax(x[0]))


def test_workload3_mixed_filtered(sampler):
    b = workloads.config(3)
    g, o, r = check(b, sampler)
    assert g["path"] == "filtered"   # the greedy row forces it


def test_workload4_full_chain(sampler):
    for step in range(2):
        b = workloads.config(4, set_id=step, step=step)
        g, o, r = check(b, sampler)
        assert g["path"] == "filtered"


@pytest.mark.parametrize("stage", ["defaults", "penalties", "min_p"])
def test_workload4_ablation_stages(sampler, stage):
    # the full chain with features added one at a time, at full size: without
    # truncation every row keeps every value (Gumbel path, Philox and the
    # listing cut on most of the vocabulary, exact sums for the outputs)
    b = workloads.config(4, set_id=1, step=1).ablation(stage)
    g, o, r = check(b, sampler)
    assert g["path"] == ("filtered" if stage == "min_p" else "gumbel")


def test_workload5_large_vocab_forks(sampler):
    b = workloads.config(5)
    g, o, r = check(b, sampler)
    # forks share parameters and history but draw independently
    tok = g["token_ids"].reshape(-1, 4)
    assert np.mean(tok[:, 0] == tok[:, 1]) < 0.9


# ------------------------------------------------------------ randomised shapes
@pytest.mark.parametrize("seed,n,V,dtype,ties", [
    (0, 1, 1, "f32", False), (1, 3, 2, "f32", False), (2, 5, 3, "bf16", True), (3, 17, 63, "f32", True),
    (4, 16, 64, "bf16", False), (5, 9, 65, "f32", False), (6, 11, 1000, "bf16", True), (7, 13, 4097, "f32", False),
    (8, 4, 50_001, "bf16", False), (9, 2, 131_071, "f32", True), (10, 6, 40_000, "f32", False),
])
def test_random_small(sampler, seed, n, V, dtype, ties):
    check(workloads.random_small(seed, n, V, dtype, ties=ties), sampler)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unaligned_stride_and_outputs(sampler, dtype):
    b = workloads.random_small(20, 6, 1001, dtype)
    L, H = to_device(b)
    wide = torch.full((b.n_rows, 1003), float("nan"), dtype=L.dtype, device=L.device)
    wide[:, 1:1002] = L
    view = wide[:, 1:1002]            # odd base offset and odd row stride
    g = run_gpu(sampler, b, logits=view, history=H)
    o = run_oracle(b)
    r = compare(g, o)
    assert r.ok(), r


def test_edge_rows(sampler):
    V = 300
    x = np.random.default_rng(3).standard_normal((6, V)).astype(np.float32)
    x[0, :] = -np.inf                 # no finite logit
    x[1, :] = np.nan                  # NaN reads as -inf
    x[2, 5] = np.inf                  # +inf
    x[3, :] = -np.inf
    x[3, 17] = 1.0                    # one finite value
    x[4, ::2] = np.nan                # half NaN
    b = workloads.Batch("edge rows", "f32", x, temperature=np.array([1, 1, 1, 0.5, 0.8, 1e-7], np.float32),
                        top_k=np.array([-1, 5, -1, 3, 2, -1], np.int32), top_p=np.array([1, 1, 1, 0.5, 0.9, 1], np.float32),
                        min_p=np.zeros(6, np.float32), want_probs=True, want_logprobs=True, top_logprobs=4)
    g, o, r = check(b, sampler)
    assert g["row_status"].tolist() == [1, 1, 2, 0, 0, 0]
    assert g["token_ids"][:3].tolist() == [-1, -1, -1]
    assert g["token_ids"][3] == 17


def test_exchange3_list_sizes(sampler):
    """Top-k rows whose candidate lists span one value per lane, up to four
    per lane (the single-wave form of the exact selection: boundaries at 64
    and 256) and beyond (the workgroup form); half with top-p as well."""
    V = 60_000
    ks = np.array([30, 63, 64, 65, 129, 200, 255, 256, 257, 300, 600, 900], np.int32)
    n = len(ks)
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((n, V)) * 2.0).astype(np.float32)
    x[1::3] = np.round(x[1::3] * 16.0) / 16.0  # tie groups
    top_p = np.where(np.arange(n) % 2 == 0, 1.0, 0.97).astype(np.float32)
    b = workloads.Batch("exchange-3 list sizes", "f32", x, temperature=np.full(n, 1.0, np.float32), top_k=ks,
                        top_p=top_p, min_p=np.zeros(n, np.float32), want_probs=True, want_logprobs=True, top_logprobs=20)
    check(b, sampler)


def test_history_edges(sampler):
    b = workloads.random_small(30, 8, 777, "f32", penalties=True, history_len=40)
    b.history_ids[::7] = -5           # ids outside [0, V) are ignored
    b.history_ids[3::11] = 777 + 9
    b.history_start[5] = b.history_start[2]   # aliased spans
    b.history_len[6] = 0
    check(b, sampler)


def test_max_vocab():
    _need_gpu()
    import decode_step_token_sampler_amd as dsts
    s = dsts.Sampler(4, 1 << 20, max_history_per_row=1024, max_top_logprobs=8)
    b = workloads.random_small(40, 2, 1 << 20, "bf16", history_len=1024)
    b.top_logprobs = 8
    check(b, s)
    s.close()


# ------------------------------------------------------------ logits processors
@pytest.fixture(scope="module")
def sampler_proc():
    _need_gpu()
    import decode_step_token_sampler_amd as dsts
    s = dsts.Sampler(64, 131_072, max_history_per_row=2048, max_top_logprobs=32, max_bias_per_row=512)
    yield s
    s.close()


def _processors_on_device(p):
    def dev(a):
        return torch.from_numpy(a).to("cuda:0")
    return dict(vocab_mask=dev(p.vocab_mask.view(np.int32)), bias_ids=dev(p.bias_ids), bias_vals=dev(p.bias_vals),
                stop_ids=dev(p.stop_ids), bias_start=p.bias_start, bias_len=p.bias_len, stop_start=p.stop_start,
                stop_len=p.stop_len, min_tokens=p.min_tokens, output_len=p.output_len)


@pytest.mark.parametrize("seed,n,V,dtype", [(31, 12, 4000, "f32"), (32, 10, 40_000, "bf16"), (33, 7, 129, "f32"),
                                            (34, 15, 90_001, "f32")])
def test_logits_processors(sampler_proc, seed, n, V, dtype):
    """Grammar bitmask, logit_bias (repeats, ignored ids, -inf and large
    values, tokens with and without history) and min_tokens stop lists, with
    penalties and every truncation, against the oracle."""
    b = workloads.random_small(seed, n, V, dtype, penalties=True, history_len=300)
    p = workloads.processors(seed, b)
    g = run_gpu(sampler_proc, b, **_processors_on_device(p))
    o = run_oracle(b, **p.kwargs())
    r = compare(g, o)
    print(b.name, r)
    assert r.ok(), r
    assert np.all(g["row_status"][np.arange(n) % 10 == 9] == 1)      # nothing allowed


def test_logits_processors_full_chain(sampler_proc):
    """The full-chain workload (N=64, V=128,000) with processors on every row."""
    b = workloads.config(4)
    p = workloads.processors(35, b)
    g = run_gpu(sampler_proc, b, **_processors_on_device(p))
    o = run_oracle(b, **p.kwargs())
    r = compare(g, o)
    print(b.name, r)
    assert r.ok(), r


def test_logits_processors_absent_is_identity(sampler_proc, sampler):
    """A handle with a bias table and no processor inputs gives the same
    results as one without."""
    b = workloads.random_small(36, 9, 5000, "f32", penalties=True)
    g1 = run_gpu(sampler_proc, b)
    g2 = run_gpu(sampler, b)
    for k in ("token_ids", "probs", "logprobs", "top_logprob_ids", "top_logprob_vals", "row_status"):
        np.testing.assert_array_equal(g1[k], g2[k])


# ------------------------------------------------------------ logprob modes
@pytest.mark.parametrize("seed,n,V,dtype", [(41, 12, 3000, "f32"), (42, 9, 70_000, "bf16"), (43, 16, 257, "f32")])
def test_logprob_mode_temperature(sampler, seed, n, V, dtype):
    """Untruncated logprobs at the row's temperature for every token; top
    logprobs over all tokens."""
    b = workloads.random_small(seed, n, V, dtype, penalties=True)
    b.top_logprobs = 7
    g = run_gpu(sampler, b, logprob_mode="temperature")
    o = run_oracle(b, logprob_mode="temperature")
    r = compare(g, o)
    print(b.name, r)
    assert r.ok(), r
    assert np.all(np.isfinite(g["logprobs"][g["row_status"] == 0]))


def test_logprob_mode_temperature_workloads(sampler):
    for b in (workloads.config(3), workloads.config(4)):
        g = run_gpu(sampler, b, logprob_mode="temperature")
        o = run_oracle(b, logprob_mode="temperature")
        r = compare(g, o)
        print(b.name, r)
        assert r.ok(), r


def test_logprob_mode_top_list_below_the_window(sampler):
    """Truncated rows whose top-logprob list must reach values far below the
    row max (deeper than the threshold window): the general path."""
    V = 5000
    x = np.full((3, V), -60.0, np.float32) - np.arange(V, dtype=np.float32) * 1e-3
    x[:, :3] = [0.0, -0.5, -1.0]
    b = workloads.Batch("deep top list", "f32", x, temperature=np.array([1.0, 0.8, 1.0], np.float32),
                        top_k=np.array([2, -1, 3], np.int32), top_p=np.array([1.0, 0.5, 1.0], np.float32),
                        min_p=np.array([0.0, 0.0, 0.2], np.float32), want_probs=True, want_logprobs=True,
                        top_logprobs=6)
    for mode in ("processed", "temperature"):
        g = run_gpu(sampler, b, logprob_mode=mode)
        o = run_oracle(b, logprob_mode=mode)
        r = compare(g, o)
        print(mode, r)
        assert r.ok(), r
    assert np.all(g["top_logprob_ids"] >= 0)          # six listed in the temperature mode


def test_logprob_mode_raw_at_unit_temperature(sampler):
    b = workloads.random_small(44, 10, 9000, "bf16", penalties=True)
    b.temperature = np.where(np.arange(10) % 3 == 0, 0.0, 1.0).astype(np.float32)
    g = run_gpu(sampler, b, logprob_mode="raw")
    o = run_oracle(b, logprob_mode="raw")
    r = compare(g, o)
    assert r.ok(), r


@pytest.mark.parametrize("T", [0.5, 1.3])
@pytest.mark.parametrize("seed,n,V,dtype", [(45, 10, 9000, "bf16"), (46, 7, 70_001, "f32"), (47, 13, 257, "f32")])
def test_logprob_mode_raw_at_other_temperatures(sampler, T, seed, n, V, dtype):
    # log_softmax of the processed logits (penalties, grammar mask, bias and
    # stop lists applied, no temperature) at T = 0.5 and 1.3, beside greedy
    # rows and rows at T = 1
    b = workloads.random_small(seed, n, V, dtype, penalties=True)
    b.temperature = np.where(np.arange(n) % 4 == 0, 0.0, np.where(np.arange(n) % 4 == 1, 1.0, T)).astype(np.float32)
    p = workloads.processors(seed, b, max_entries=64)
    kw = p.kwargs()
    L, H = to_device(b)
    dk = {k: (torch.from_numpy(np.ascontiguousarray(v)).to("cuda:0") if k in ("vocab_mask", "bias_ids", "bias_vals",
                                                                             "stop_ids") else v)
          for k, v in kw.items()}
    import decode_step_token_sampler_amd as dsts
    s = dsts.Sampler(16, 80_000, max_history_per_row=64, max_top_logprobs=8, max_bias_per_row=64)
    g = run_gpu(s, b, logits=L, history=H, logprob_mode="raw", **dk)
    o = run_oracle(b, logprob_mode="raw", **kw)
    r = compare(g, o)
    assert r.ok(), r
    s.close()


def test_logprob_mode_raw_workloads(sampler):
    # the mixed filtered batch and the full chain, every row's logprobs raw
    for cfg in (3, 4):
        b = workloads.config(cfg, n_rows=16, vocab=60_000, history_len=512)
        b.top_logprobs = 5
        g = run_gpu(sampler, b, logprob_mode="raw")
        o = run_oracle(b, logprob_mode="raw")
        r = compare(g, o)
        assert r.ok(), (cfg, r)


# ------------------------------------------------------------ invariants
def test_replay_and_run_to_run_stability(sampler):
    b = workloads.config(4, n_rows=16, vocab=50_000, history_len=512)
    L, H = to_device(b)
    first = run_gpu(sampler, b, logits=L, history=H)
    for _ in range(100):
        again = run_gpu(sampler, b, logits=L, history=H)
        for k in ("token_ids", "probs", "logprobs", "row_status"):
            np.testing.assert_array_equal(first[k], again[k])


def test_forced_filtered_path_is_identical():
    _need_gpu()
    import decode_step_token_sampler_amd as dsts
    a = dsts.Sampler(64, 20_000, max_history_per_row=64)
    f = dsts.Sampler(64, 20_000, max_history_per_row=64, force_filtered=True)
    plain = workloads.random_small(50, 12, 9_999, "bf16", penalties=True, mix="plain")
    plain.temperature = np.full(12, 0.9, np.float32)   # no greedy row: Gumbel path
    for b in (workloads.config(1, n_rows=9, vocab=20_000), plain):
        b.want_logprobs = True
        for T in (None, 0.0):
            if T is not None:
                b.temperature = np.zeros(b.n_rows, np.float32)
            ga = run_gpu(a, b)
            gf = run_gpu(f, b)
            assert ga["path"] in ("gumbel", "greedy")
            for k in ("token_ids", "probs", "logprobs"):
                np.testing.assert_array_equal(ga[k], gf[k])
    a.close()
    f.close()


def test_one_greedy_row_changes_path_not_results(sampler):
    # [A] worked case: a temperature-0 request moves the batch to filtered
    b = workloads.config(1, n_rows=6, vocab=30_000)
    b.want_logprobs = True
    b.row_stream = np.arange(6, dtype=np.uint32)
    plain = run_gpu(sampler, b)
    x = np.concatenate([b.logits, b.logits[:1]])
    b2 = workloads.Batch("plus greedy", "f32", x, temperature=np.append(b.temperature, 0.0).astype(np.float32),
                         top_k=np.full(7, -1, np.int32), top_p=np.ones(7, np.float32), min_p=np.zeros(7, np.float32),
                         row_stream=np.arange(7, dtype=np.uint32), want_probs=True, want_logprobs=True)
    mixed = run_gpu(sampler, b2)
    assert plain["path"] == "gumbel" and mixed["path"] == "filtered"
    for k in ("token_ids", "probs", "logprobs"):
        np.testing.assert_array_equal(plain[k], mixed[k][:6])


def test_deterministic_batch_invariance():
    _need_gpu()
    import decode_step_token_sampler_amd as dsts
    s = dsts.Sampler(32, 100_000, max_history_per_row=256, deterministic=True)
    big = workloads.random_small(60, 12, 70_000, "f32", penalties=True, history_len=256)
    big.row_seed = None
    big.row_stream = None
    ref = run_gpu(s, big)
    o = run_oracle(big, deterministic=True)
    r = compare(ref, o)
    assert r.ok(), r
    for r_ in (0, 5, 11):
        for n_before in (0, 3):
            rows = list(range(n_before)) + [r_]
            sub = big.subset(rows)
            sub.row_seed = None
            sub.row_stream = None
            sub.row_offset = None
            g = run_gpu(s, sub)
            for k in ("token_ids", "probs", "logprobs"):
                np.testing.assert_array_equal(g[k][-1], ref[k][r_])
    s.close()


# ------------------------------------------------------------ inverse-CDF selection
@pytest.fixture(scope="module")
def sampler_icdf():
    _need_gpu()
    import decode_step_token_sampler_amd as dsts
    s = dsts.Sampler(512, 262_144, max_history_per_row=2048, max_top_logprobs=32, inverse_cdf=True)
    yield s
    s.close()


@pytest.mark.parametrize("seed,n,V,dtype", [(61, 12, 3000, "f32"), (62, 9, 70_000, "bf16"), (63, 16, 257, "f32"),
                                            (64, 5, 131_071, "f32")])
def test_inverse_cdf_random(sampler_icdf, seed, n, V, dtype):
    b = workloads.random_small(seed, n, V, dtype, penalties=True)
    g = run_gpu(sampler_icdf, b)
    o = run_oracle(b, inverse_cdf=True)
    r = compare(g, o)
    print(b.name, r)
    assert r.ok(), r


def test_inverse_cdf_workloads(sampler_icdf):
    for b in (workloads.config(1), workloads.config(3), workloads.config(4), workloads.config(5)):
        g = run_gpu(sampler_icdf, b)
        o = run_oracle(b, inverse_cdf=True)
        r = compare(g, o)
        print(b.name, r)
        assert r.ok(), r


def test_inverse_cdf_exact_tokens_over_offsets(sampler_icdf):
    """10^5 draws of one V=64 row (offsets 0..), token for token against the
    oracle (whose chi-square against the categorical is pinned)."""
    import parity
    rng = np.random.default_rng(65)
    x = (1.5 * rng.standard_normal(64)).astype(np.float32)
    n = 500
    for start in range(0, 100_000, n):
        L = np.ascontiguousarray(np.broadcast_to(x, (n, 64)))
        b = workloads.Batch("icdf draws", "f32", L, temperature=np.full(n, 0.9, np.float32),
                            top_k=np.full(n, -1, np.int32), top_p=np.full(n, 1.0, np.float32),
                            min_p=np.zeros(n, np.float32), want_probs=False, want_logprobs=False, top_logprobs=0)
        b.row_seed = np.full(n, 7, np.uint64)
        b.row_stream = np.zeros(n, np.uint32)
        b.row_offset = np.arange(start, start + n, dtype=np.uint64)
        g = run_gpu(sampler_icdf, b)
        o = run_oracle(b, inverse_cdf=True)
        ok = (o["flags"] & parity.FLAG_MASK) == 0
        assert np.array_equal(g["token_ids"][ok], o["token_ids"][ok]), start


def test_inverse_cdf_deterministic_batch_invariance():
    _need_gpu()
    import decode_step_token_sampler_amd as dsts
    s = dsts.Sampler(32, 100_000, max_history_per_row=256, deterministic=True, inverse_cdf=True)
    big = workloads.random_small(66, 12, 70_000, "f32", penalties=True, history_len=256)
    big.row_seed = None
    big.row_stream = None
    ref = run_gpu(s, big)
    o = run_oracle(big, deterministic=True, inverse_cdf=True)
    r = compare(ref, o)
    assert r.ok(), r
    for r_ in (0, 5, 11):
        for n_before in (0, 3, 7):
            rows = list(range(n_before)) + [r_]
            sub = big.subset(rows)
            sub.row_seed = None
            sub.row_stream = None
            sub.row_offset = None
            g = run_gpu(s, sub)
            for k in ("token_ids", "probs", "logprobs"):
                np.testing.assert_array_equal(g[k][-1], ref[k][r_])
    s.close()


# ------------------------------------------------------------ device parameters and graph capture
def _device_params(b):
    def dev(a, dt):
        return torch.from_numpy(np.ascontiguousarray(a).view(dt)).to("cuda:0")
    p = dict(temperature=dev(b.temperature, np.float32), top_p=dev(b.top_p, np.float32),
             top_k=dev(b.top_k, np.int32), min_p=dev(b.min_p, np.float32))
    if b.repetition_penalty is not None:
        p.update(repetition_penalty=dev(b.repetition_penalty, np.float32),
                 presence_penalty=dev(b.presence_penalty, np.float32),
                 frequency_penalty=dev(b.frequency_penalty, np.float32),
                 history_start=dev(b.history_start, np.int64), history_len=dev(b.history_len, np.int32))
    n = b.n_rows
    rs = b.row_seed if b.row_seed is not None else np.full(n, b.seed, np.uint64)
    ro = b.row_offset if b.row_offset is not None else np.full(n, b.offset, np.uint64)
    rst = b.row_stream if b.row_stream is not None else np.arange(n, dtype=np.uint32)
    p.update(row_seed=dev(rs.astype(np.uint64), np.int64), row_offset=dev(ro.astype(np.uint64), np.int64),
             row_stream=dev(rst.astype(np.uint32), np.int32))
    return p


def _outputs(n, V, K):
    d = "cuda:0"
    return dict(token_ids=torch.empty(n, dtype=torch.int32, device=d), probs=torch.empty(n, V, device=d),
                logprobs=torch.empty(n, V, device=d), top_logprob_vals=torch.empty(n, K, device=d),
                top_logprob_ids=torch.empty(n, K, dtype=torch.int32, device=d),
                row_status=torch.empty(n, dtype=torch.int32, device=d))


def _host(out):
    return {k: v.cpu().numpy() for k, v in out.items()}


def test_step_graph_eager_matches_host_step(sampler):
    b = workloads.random_small(70, 14, 30_000, "bf16", penalties=True, history_len=200)
    L, H = to_device(b)
    out = _outputs(b.n_rows, b.vocab, b.top_logprobs)
    sampler.step_graph(L, _device_params(b), history_ids=H, out=out, top_logprobs=b.top_logprobs)
    torch.cuda.synchronize()
    g = _host(out)
    h = run_gpu(sampler, b, logits=L, history=H)
    for k in ("token_ids", "probs", "logprobs", "top_logprob_ids", "top_logprob_vals", "row_status"):
        np.testing.assert_array_equal(g[k], h[k])
    r = compare(g, run_oracle(b))
    assert r.ok(), r


def test_step_graph_raw_logprobs_and_replays():
    # the raw logprob mode on device-side parameters: the raw kernel follows
    # the row kernel in the captured graph, and each replay (its own pair of
    # launches) equals the host-path step and the oracle
    _need_gpu()
    import decode_step_token_sampler_amd as dsts
    s = dsts.Sampler(16, 30_000, max_history_per_row=200, max_top_logprobs=8)
    b = workloads.random_small(72, 12, 30_000, "f32", penalties=True, history_len=200)
    b.temperature = np.where(np.arange(12) % 3 == 0, 1.0, 0.6).astype(np.float32)
    L, H = to_device(b)
    params = _device_params(b)
    out = _outputs(b.n_rows, b.vocab, b.top_logprobs)
    s.step_graph(L, params, history_ids=H, out=out, top_logprobs=b.top_logprobs, logprob_mode="raw")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        s.step_graph(L, params, history_ids=H, out=out, top_logprobs=b.top_logprobs, logprob_mode="raw")
    torch.cuda.synchronize()
    o = run_oracle(b, logprob_mode="raw")
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        g = _host(out)
        r = compare(g, o)
        assert r.ok(), (rep, r)
        h = run_gpu(s, b, logits=L, history=H, logprob_mode="raw")
        for k in ("token_ids", "probs", "logprobs", "top_logprob_ids", "top_logprob_vals", "row_status"):
            np.testing.assert_array_equal(g[k], h[k], err_msg=k)
    s.close()


def test_step_graph_bad_rows_get_status_4(sampler):
    b = workloads.random_small(71, 8, 4000, "f32", penalties=True)
    b.temperature[1] = -1.0
    b.top_p[3] = 0.0
    b.top_k[5] = 0
    b.history_len[6] = 4000             # beyond max_history_per_row
    L, H = to_device(b)
    out = _outputs(b.n_rows, b.vocab, b.top_logprobs)
    sampler.step_graph(L, _device_params(b), history_ids=H, out=out, top_logprobs=b.top_logprobs)
    torch.cuda.synchronize()
    g = _host(out)
    bad = [1, 3, 5, 6]
    assert g["row_status"][bad].tolist() == [4, 4, 4, 4]
    assert np.all(g["token_ids"][bad] == -1) and np.all(g["probs"][bad] == 0)
    assert np.all(np.isneginf(g["logprobs"][bad])) and np.all(g["top_logprob_ids"][bad] == -1)
    good = [0, 2, 4, 7]
    r = compare(g, run_oracle(b.subset(good)), rows=good)
    assert r.ok(), r


def test_step_graph_capture_and_replay():
    """Capture one step into a graph, then replay it after updating the
    logits and the per-row parameters in place (a decode loop), with eager
    steps and synchronisations between the replays; every replay equals the
    eager host-path step on the same inputs and the oracle."""
    _need_gpu()
    import decode_step_token_sampler_amd as dsts
    s = dsts.Sampler(32, 70_000, max_history_per_row=256, max_top_logprobs=8)
    batches = [workloads.random_small(80 + i, 12, 60_000, "f32", penalties=True, history_len=256) for i in range(4)]
    for bb in batches[1:]:                    # one history buffer layout for all replays
        bb.history_ids = batches[0].history_ids
        bb.history_start = batches[0].history_start
    b0 = batches[0]
    L, H = to_device(b0)
    params = _device_params(b0)
    out = _outputs(b0.n_rows, b0.vocab, b0.top_logprobs)
    s.step_graph(L, params, history_ids=H, out=out, top_logprobs=b0.top_logprobs)   # warm-up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        s.step_graph(L, params, history_ids=H, out=out, top_logprobs=b0.top_logprobs)
    torch.cuda.synchronize()
    for step, b in enumerate(batches):
        b.offset = 1000 + step
        b.row_offset = None
        Ln, _ = to_device(b)
        L.copy_(Ln)
        for k, v in _device_params(b).items():
            params[k].copy_(v)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        g = _host(out)
        e = run_gpu(s, b, logits=L, history=H)    # eager host path between replays
        for k in ("token_ids", "probs", "logprobs", "top_logprob_ids", "top_logprob_vals", "row_status"):
            np.testing.assert_array_equal(g[k], e[k], err_msg=f"replay {step} {k}")
        r = compare(g, run_oracle(b))
        assert r.ok(), (step, r)
    s.close()


def test_gumbel_distribution_chi2_and_exact_tokens():
    _need_gpu()
    import scipy.special
    import scipy.stats
    import decode_step_token_sampler_amd as dsts
    n_chunk, chunks, V = 100_000, 10, 64
    s = dsts.Sampler(n_chunk, V, max_history_per_row=0, max_top_logprobs=0)
    x = (1.5 * np.random.default_rng(8).standard_normal(V)).astype(np.float32)
    for top_k, top_p in ((-1, 1.0), (10, 0.8)):
        counts = np.zeros(V, np.int64)
        for c in range(chunks):
            L = np.ascontiguousarray(np.broadcast_to(x, (n_chunk, V)))
            b = workloads.Batch("chi2", "f32", L, temperature=np.full(n_chunk, 0.9, np.float32),
                                top_k=np.full(n_chunk, top_k, np.int32), top_p=np.full(n_chunk, top_p, np.float32),
                                min_p=np.zeros(n_chunk, np.float32), row_seed=np.full(n_chunk, 99, np.uint64),
                                row_stream=np.zeros(n_chunk, np.uint32),
                                row_offset=np.arange(c * n_chunk, (c + 1) * n_chunk, dtype=np.uint64))
            g = run_gpu(s, b, want_status=True)
            if c < 2:   # exact token parity on a fifth of the draws
                o = run_oracle(b)
                r = compare(g, o)
                assert r.ok(), r
            counts += np.bincount(g["token_ids"], minlength=V)
        z = (x / np.float32(0.9)).astype(np.float64)
        if top_k == -1:
            probs = scipy.special.softmax(z)
        else:
            order = np.lexsort((np.arange(V), -z))
            top = order[:top_k]
            q = np.exp(z[top] - z.max())
            cum = np.cumsum(q)
            keep = top[:int(np.searchsorted(cum, top_p * cum[-1])) + 1]
            probs = np.zeros(V)
            probs[keep] = np.exp(z[keep] - z.max())
            probs /= probs.sum()
            assert counts[probs == 0].sum() == 0
        exp = probs * counts.sum()
        m = exp >= 5
        obs, ex = counts[m], exp[m]
        if exp[~m].sum() > 0:
            obs, ex = np.append(obs, counts[~m].sum()), np.append(ex, exp[~m].sum())
        p = scipy.stats.chisquare(obs, ex * (obs.sum() / ex.sum())).pvalue
        assert p > 1e-3, (top_k, p)
    s.close()


def test_cooperative_launch_is_identical():
    # the plain launch (default) and the cooperative one run the same kernel
    _need_gpu()
    import decode_step_token_sampler_amd as dsts
    a = dsts.Sampler(64, 128_000, max_history_per_row=2048)
    c = dsts.Sampler(64, 128_000, max_history_per_row=2048, cooperative_launch=True)
    b = workloads.config(4, n_rows=24)
    ga, gc = run_gpu(a, b), run_gpu(c, b)
    for k in ("token_ids", "probs", "logprobs", "row_status"):
        np.testing.assert_array_equal(ga[k], gc[k])
    assert np.all(ga["row_status"] == 0)
    a.close()
    c.close()


# ------------------------------------------------------------ long histories
@pytest.fixture(scope="module")
def sampler_long():
    _need_gpu()
    import decode_step_token_sampler_amd as dsts
    s = dsts.Sampler(64, 131_072, max_history_per_row=16_384, max_top_logprobs=32, max_bias_per_row=512)
    yield s
    s.close()


def test_full_chain_with_16384_id_histories(sampler_long):
    """The full-chain workload (N=64, V=128,000, fp32) with 16,384-id Zipf(1.1)
    histories: counted ahead of the row kernel, penalties as for short ones."""
    b = workloads.config(4, history_len=16_384)
    check(b, sampler_long)


@pytest.mark.parametrize("seed,n,V,dtype", [(81, 6, 30_000, "f32"), (82, 9, 70_001, "bf16")])
def test_long_uniform_histories_mixed_with_short(sampler_long, seed, n, V, dtype):
    """Uniform histories of up to 16,384 ids: slices with more than 4,096
    distinct ids (the list's second pass), in batches that mix long rows with
    rows the row kernel's own hash counts."""
    b = workloads.random_small(seed, n, V, dtype, penalties=True, history_len=16_384)
    b.history_len[0] = 16_384
    b.history_len[1] = 4096
    b.history_len[2] = 4097
    check(b, sampler_long)


def test_long_histories_with_processors_and_raw_logprobs(sampler_long):
    """Long histories with logit_bias / stop lists (bias entries on tokens with
    and without history) and a grammar mask, in the processed and the raw
    logprob modes."""
    b = workloads.random_small(83, 10, 40_000, "f32", penalties=True, history_len=12_000)
    p = workloads.processors(83, b)
    g = run_gpu(sampler_long, b, **_processors_on_device(p))
    r = compare(g, run_oracle(b, **p.kwargs()))
    assert r.ok(), r
    g = run_gpu(sampler_long, b, logprob_mode="raw", **_processors_on_device(p))
    r = compare(g, run_oracle(b, logprob_mode="raw", **p.kwargs()))
    assert r.ok(), r


def test_long_histories_on_device_params(sampler_long):
    """sampler_step_graph with long histories: the count kernel runs on every
    step of a handle planned for them; outputs equal the host-path step."""
    b = workloads.random_small(84, 12, 30_000, "bf16", penalties=True, history_len=9000)
    L, H = to_device(b)
    out = _outputs(b.n_rows, b.vocab, b.top_logprobs)
    sampler_long.step_graph(L, _device_params(b), history_ids=H, out=out, top_logprobs=b.top_logprobs)
    torch.cuda.synchronize()
    g = _host(out)
    h = run_gpu(sampler_long, b, logits=L, history=H)
    for k in ("token_ids", "probs", "logprobs", "top_logprob_ids", "top_logprob_vals", "row_status"):
        np.testing.assert_array_equal(g[k], h[k], err_msg=k)
    r = compare(g, run_oracle(b))
    assert r.ok(), r


# ------------------------------------------------------------ light launches
def test_light_launch_with_penalties_processors_and_long_histories(sampler_long):
    """A launch whose rows only meet in the final merge (ids only; rows greedy
    or keeping every token) spreads each row over up to 64 workgroups: with
    penalties over short and long histories, logit_bias, stop lists and a
    grammar mask, its tokens equal the oracle's."""
    b = workloads.random_small(85, 6, 131_000, "bf16", penalties=True, history_len=6000, mix="plain")
    b.temperature[1] = 0.0                     # a greedy row
    b.history_len[2] = 6000                    # longer than the row kernel's own hash
    b.want_probs = b.want_logprobs = False
    b.top_logprobs = 0
    p = workloads.processors(85, b)
    g = run_gpu(sampler_long, b, **_processors_on_device(p))
    o = run_oracle(b, **p.kwargs())
    r = compare(g, o)
    print(b.name, r)
    assert r.ok(), r


# ------------------------------------------------------------ extreme parameters
@pytest.mark.parametrize("V,dtype", [(100_003, "f32"), (4097, "bf16")])
def test_extreme_parameters(sampler, V, dtype):
    """Temperatures at the greedy boundary and far above 1, top-p down to
    1e-6, min-p near 1, top-k of V - 1 and 1, logits of large and tiny
    magnitude: every row against the oracle."""
    rng = np.random.default_rng(V)
    n = 12
    x = (rng.standard_normal((n, V)) * 3.0).astype(np.float32)
    x[6] *= 3000.0                                  # large magnitudes
    x[7] *= 1e-30                                   # tiny magnitudes (near-uniform row)
    x[8, rng.integers(0, V, 40)] = 25.0             # a plateau of equal maxima
    T = np.array([1e-6, 1e-5, 50.0, 1e4, 1.0, 1.0, 0.7, 1.0, 1.0, 0.3, 2.0, 1.0], np.float32)
    top_k = np.array([-1, -1, -1, -1, V - 1, 1, 20, -1, 5, -1, 3, -1], np.int32)
    top_p = np.array([1, 0.5, 0.9, 1, 1e-6, 1, 0.99, 0.5, 1, 1e-3, 0.7, 1], np.float32)
    min_p = np.array([0, 0, 0.5, 0.999, 0, 0, 0, 0.01, 0, 0.9, 0, 0.3], np.float32)
    L = workloads.f32_to_bf16_bits(x) if dtype == "bf16" else x
    b = workloads.Batch("extreme parameters V=%d %s" % (V, dtype), dtype, L, temperature=T, top_k=top_k,
                        top_p=top_p, min_p=min_p, seed=123, offset=7, want_probs=True, want_logprobs=True,
                        top_logprobs=8)
    g, o, r = check(b, sampler)
    assert np.all(g["row_status"] == 0)
