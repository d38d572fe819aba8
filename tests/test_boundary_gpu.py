"""GPU checks of the boundary's failure handling, switches and argument
checks, all through the C ABI: recovery after a step whose cross-workgroup
waits expired (eager and captured steps), a deterministic handle's cut that
depends on the vocabulary alone, the forced selection paths, rows without
exchanges in groups that walk several rows, the binding's refusal of tensors
the kernel would misread, and the 10,000-step batch-1 decode run."""
import numpy as np
import pytest

import workloads
from parity import compare, run_gpu, run_oracle, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _dsts():
    _need_gpu()
    import decode_step_token_sampler_amd as dsts
    return dsts


def test_recovery_after_expired_waits():
    # A wait bound of one poll makes waits expire (the rows of such a step
    # report status 3); the handle's next steps must be exact again.
    dsts = _dsts()
    s = dsts.Sampler(64, 50_000, max_history_per_row=512, max_top_logprobs=5)
    b = workloads.config(4, n_rows=24, vocab=40_000, history_len=512)
    b.top_logprobs = 5
    for _ in range(2):
        s.set_wait_spin_limit(1)
        g = run_gpu(s, b)
        assert set(np.unique(g["row_status"]).tolist()) <= {0, 3}
        s.set_wait_spin_limit(0)
        for _ in range(2):
            g = run_gpu(s, b)
            r = compare(g, run_oracle(b))
            assert r.ok() and np.all(g["row_status"] == 0), r
    s.close()


def _graph_inputs(b):
    from test_parity_gpu import _device_params, _outputs
    L, H = to_device(b)
    return L, H, _device_params(b), _outputs(b.n_rows, b.vocab, b.top_logprobs)


def test_graph_replays_recover_after_expired_waits():
    # A graph captured with a one-poll bound aborts when replayed; replays of
    # a graph captured with the default bound, eager steps and further
    # replays after it must all be exact (each replay is a launch of its own).
    dsts = _dsts()
    s = dsts.Sampler(32, 30_000, max_history_per_row=200, max_top_logprobs=5)
    b = workloads.random_small(90, 12, 30_000, "f32", penalties=True, history_len=200)
    L, H, params, out = _graph_inputs(b)
    K = b.top_logprobs
    s.step_graph(L, params, history_ids=H, out=out, top_logprobs=K)   # warm-up
    torch.cuda.synchronize()
    s.set_wait_spin_limit(1)
    aborting = torch.cuda.CUDAGraph()
    with torch.cuda.graph(aborting):
        s.step_graph(L, params, history_ids=H, out=out, top_logprobs=K)
    s.set_wait_spin_limit(0)
    good = torch.cuda.CUDAGraph()
    with torch.cuda.graph(good):
        s.step_graph(L, params, history_ids=H, out=out, top_logprobs=K)
    torch.cuda.synchronize()
    o = run_oracle(b)

    def check_good(what):
        g = {k: v.cpu().numpy() for k, v in out.items()}
        r = compare(g, o)
        assert r.ok() and np.all(g["row_status"] == 0), (what, r)

    for rnd in range(2):
        aborting.replay()
        torch.cuda.synchronize()
        assert set(np.unique(out["row_status"].cpu().numpy()).tolist()) <= {0, 3}
        for rep in range(2):
            good.replay()
            torch.cuda.synchronize()
            check_good(f"round {rnd} replay {rep}")
        g = run_gpu(s, b, logits=L, history=H)      # an eager step in between
        r = compare(g, o)
        assert r.ok() and np.all(g["row_status"] == 0), r
    s.close()


def test_deterministic_cut_depends_on_vocab_only():
    # two deterministic handles whose LDS plans differ (history and bias
    # limits) cut a row the same way, so their results are bit-identical
    dsts = _dsts()
    V = 131_072
    a = dsts.Sampler(16, V, max_history_per_row=4096, max_bias_per_row=512, deterministic=True)
    c = dsts.Sampler(16, V, max_history_per_row=2048, max_bias_per_row=0, deterministic=True)
    b = workloads.config(4, n_rows=6, vocab=V, history_len=2048)
    ga, gc = run_gpu(a, b), run_gpu(c, b)
    for k in ("token_ids", "probs", "logprobs", "row_status"):
        np.testing.assert_array_equal(ga[k], gc[k], err_msg=k)
    r = compare(ga, run_oracle(b, deterministic=True))
    assert r.ok(), r
    a.close()
    c.close()


def test_forced_paths():
    dsts = _dsts()
    b = workloads.config(4, n_rows=12, vocab=20_000, history_len=256)
    plain = dsts.Sampler(16, 20_000, max_history_per_row=256)
    gum = dsts.Sampler(16, 20_000, max_history_per_row=256, force_path="gumbel")
    gre = dsts.Sampler(16, 20_000, max_history_per_row=256, force_path="greedy")
    gp, gg, gr = run_gpu(plain, b), run_gpu(gum, b), run_gpu(gre, b)
    # the Gumbel label changes nothing: selection is per row
    for k in ("token_ids", "probs", "logprobs", "row_status"):
        np.testing.assert_array_equal(gp[k], gg[k], err_msg=k)
    assert gg["path"] == gp["path"] == "filtered"   # path_out reports the predicate's choice
    # the greedy path takes every row's first argmax; the distributions still
    # follow each row's parameters
    o = run_oracle(b)
    np.testing.assert_array_equal(gr["probs"], gp["probs"])
    np.testing.assert_array_equal(gr["logprobs"], gp["logprobs"])
    argmax = run_oracle(b, top_k=np.ones(b.n_rows, np.int32))["token_ids"]
    np.testing.assert_array_equal(gr["token_ids"], argmax)
    assert compare(gp, o).ok()
    for s in (plain, gum, gre):
        s.close()


def test_exchange_free_rows_in_groups_that_walk_several_rows():
    # Gumbel rows with no outputs meet their peers only at the final
    # exchange; with more rows than row groups each group walks several of
    # them, and every token must still be the oracle's
    dsts = _dsts()
    n, V = 512, 151_936
    s = dsts.Sampler(n, V, max_history_per_row=0)
    b = workloads.config(2, n_rows=n, vocab=V)
    b.row_offset = np.arange(n, dtype=np.uint64)
    b.row_stream = np.zeros(n, np.uint32)
    g = run_gpu(s, b)
    assert g["path"] == "gumbel"
    r = compare(g, run_oracle(b))
    assert r.ok(), r
    s.close()


def test_binding_rejects_tensors_the_kernel_would_misread():
    dsts = _dsts()
    s = dsts.Sampler(8, 4096, max_history_per_row=64, max_bias_per_row=8)
    b = workloads.random_small(95, 4, 4000, "f32", penalties=True, history_len=64)
    L, H = to_device(b)
    kw = dict(temperature=b.temperature, history_start=b.history_start, history_len=b.history_len,
              repetition_penalty=b.repetition_penalty)
    with pytest.raises(ValueError, match="int32"):
        s.step(L, history_ids=H.to(torch.int64), **kw)
    with pytest.raises(ValueError, match="outside"):
        s.step(L, history_ids=H[:10], **kw)
    with pytest.raises(ValueError, match="shape"):
        s.step(L, history_ids=H, want_probs=True, out={"probs": torch.empty(4, 100, device="cuda:0")}, **kw)
    with pytest.raises(ValueError, match="float32"):
        ids = torch.zeros(2, dtype=torch.int32, device="cuda:0")
        s.step(L, bias_ids=ids, bias_vals=torch.zeros(2, dtype=torch.float64, device="cuda:0"),
               bias_start=[0] * 4, bias_len=[1] * 4)
    g = s.step(L, history_ids=H, **kw)   # and the good call still runs
    torch.cuda.synchronize()
    assert g["token_ids"].shape == (4,)
    s.close()


def test_batch1_decode_10000_steps():
    # The batch-1 decode workload over 10,000 steps (offset = step) on one
    # logits row: every token equals the oracle's, and the token histogram
    # follows the softmax (G-test on the bins expecting at least 5 draws).
    dsts = _dsts()
    import scipy.stats
    steps = 10_000
    b = workloads.config(2, set_id=0)
    V = b.vocab
    s = dsts.Sampler(1, V, max_history_per_row=0)
    L, _ = to_device(b)
    tok = torch.empty(steps, dtype=torch.int32, device="cuda:0")
    for step in range(steps):
        s.step(L, temperature=b.temperature, seed=0, offset=step, want_status=False,
               out={"token_ids": tok[step:step + 1]})
    torch.cuda.synchronize()
    tok = tok.cpu().numpy()
    chunk = 500
    for c0 in range(0, steps, chunk):
        many = workloads.Batch("batch-1 steps", "bf16", np.ascontiguousarray(np.broadcast_to(b.logits, (chunk, V))),
                               temperature=np.full(chunk, 1.0, np.float32), top_k=np.full(chunk, -1, np.int32),
                               top_p=np.ones(chunk, np.float32), min_p=np.zeros(chunk, np.float32),
                               row_seed=np.zeros(chunk, np.uint64), row_stream=np.zeros(chunk, np.uint32),
                               row_offset=np.arange(c0, c0 + chunk, dtype=np.uint64))
        r = compare({"token_ids": tok[c0:c0 + chunk]}, run_oracle(many))
        assert r.ok(), (c0, r)
    x = workloads.bf16_bits_to_f32(b.logits[0]).astype(np.float64)
    p = np.exp(x - x.max())
    p /= p.sum()
    counts = np.bincount(tok, minlength=V)
    exp = p * steps
    m = exp >= 5
    obs = np.append(counts[m], counts[~m].sum())
    ex = np.append(exp[m], exp[~m].sum())
    assert scipy.stats.power_divergence(obs, ex, lambda_="log-likelihood").pvalue > 1e-3
    s.close()
