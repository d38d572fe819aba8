"""sampler_step_noalloc (no handle; the library's fixed scratch array)
against sampler_step on a handle, through the C ABI: two calls in a row, the
second with a smaller batch, each compared with the handle's step and with
the oracle under the parity rules.  (The two entry points may cut a row into
different slices, so their floating-point results agree to the parity
tolerances, and their tokens exactly.)"""
import numpy as np
import pytest

import workloads
from parity import LOGPROB_TOL, PROB_TOL, compare, run_gpu, run_oracle, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _noalloc(b, flags=0):
    import decode_step_token_sampler_amd as dsts
    L, H = to_device(b)
    out = dsts.step_noalloc(L, flags=flags, temperature=b.temperature, top_p=b.top_p, top_k=b.top_k, min_p=b.min_p,
                            repetition_penalty=b.repetition_penalty, presence_penalty=b.presence_penalty,
                            frequency_penalty=b.frequency_penalty, history_ids=H, history_start=b.history_start,
                            history_len=b.history_len, seed=b.seed, offset=b.offset, row_seed=b.row_seed,
                            row_offset=b.row_offset, row_stream=b.row_stream, want_probs=b.want_probs,
                            want_logprobs=b.want_logprobs, top_logprobs=b.top_logprobs)
    torch.cuda.synchronize()
    return {k: (v.cpu().numpy() if hasattr(v, "cpu") else v) for k, v in out.items()}


def _agree(a, h):
    np.testing.assert_array_equal(a["token_ids"], h["token_ids"])
    np.testing.assert_array_equal(a["row_status"], h["row_status"])
    for k, tol in (("probs", PROB_TOL), ("logprobs", LOGPROB_TOL), ("top_logprob_vals", LOGPROB_TOL)):
        if k in h:
            x, y = a[k].astype(np.float64), h[k].astype(np.float64)
            np.testing.assert_array_equal(np.isneginf(x), np.isneginf(y))
            fin = ~np.isneginf(y)
            assert np.all(np.abs(x[fin] - y[fin]) <= tol), k
    if "top_logprob_ids" in h:
        np.testing.assert_array_equal(a["top_logprob_ids"], h["top_logprob_ids"])


def test_noalloc_matches_handle_step_on_two_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_step_token_sampler_amd as dsts
    big = workloads.config(4, n_rows=100, vocab=50_000, history_len=1024)   # more rows than one launch carries
    big.top_logprobs = 6
    small = workloads.random_small(40, 8, 20_000, "bf16", penalties=True, history_len=300)
    h = dsts.Sampler(128, 60_000, max_history_per_row=1024, max_top_logprobs=8)
    for b in (big, small):
        a = _noalloc(b)
        g = run_gpu(h, b)
        assert a["path"] == g["path"]
        _agree(a, g)
        r = compare(a, run_oracle(b))
        assert r.ok(), r
    h.close()


def test_noalloc_deterministic_and_inverse_cdf():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_step_token_sampler_amd as dsts
    b = workloads.random_small(41, 12, 30_000, "f32", penalties=True, history_len=200)
    for flags, kw in ((dsts.FLAG_DETERMINISTIC, dict(deterministic=True)), (dsts.FLAG_INVERSE_CDF, dict(inverse_cdf=True))):
        a = _noalloc(b, flags)
        r = compare(a, run_oracle(b, **kw))
        assert r.ok(), (flags, r)


def test_noalloc_rejects_bad_arguments():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_step_token_sampler_amd as dsts
    b = workloads.random_small(42, 4, 1000, "f32", penalties=False)
    L, _ = to_device(b)
    with pytest.raises(dsts.SamplerError) as e:
        dsts.step_noalloc(L, flags=dsts.FLAG_COOPERATIVE_LAUNCH, temperature=b.temperature)
    assert e.value.status == dsts.SAMPLER_EINVAL
    with pytest.raises(dsts.SamplerError) as e:
        dsts.step_noalloc(L, temperature=b.temperature, top_logprobs=33)
    assert e.value.status == dsts.SAMPLER_ECAPACITY


def test_noalloc_raw_logprobs_only_at_unit_temperature():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_step_token_sampler_amd as dsts
    b = workloads.random_small(43, 4, 1000, "f32", penalties=False)
    L, _ = to_device(b)
    with pytest.raises(dsts.SamplerError) as e:
        dsts.step_noalloc(L, temperature=[0.5, 1.0, 1.0, 1.0], want_logprobs=True, logprob_mode="raw")
    assert e.value.status == dsts.SAMPLER_ENOTSUP
    out = dsts.step_noalloc(L, temperature=[0.0, 1.0, 1.0, 1.0], want_logprobs=True, logprob_mode="raw")
    torch.cuda.synchronize()
    assert out["token_ids"].shape == (4,)
