"""C-ABI checks that need no GPU: the library loads and exports every entry
point the header declares; the batch predicate and the host-side argument
validation behave as documented; sampler_create fails cleanly without a
device."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import decode_step_token_sampler_amd as dsts
from decode_step_token_sampler_amd import build as dbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


@pytest.fixture(scope="module")
def lib():
    dbuild.ensure_built()
    return dsts.load_library()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "sampler.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sampler_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(dsts.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    # nm agrees: defined, global, text symbols
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", dsts.LIB_PATH], capture_output=True, text=True).stdout
    defined = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for n in names:
        assert n in defined, n


def test_predicate_matches_page_table(lib):
    spec = json.load(open(os.path.join(GOLDEN, "path_table.json")))
    for case in spec["cases"]:
        rows = case["rows"]
        got = dsts.select_path([r["temperature"] for r in rows], [r["top_k"] for r in rows],
                               [r["top_p"] for r in rows], [r["min_p"] for r in rows],
                               deterministic=case["deterministic"])
        assert got == case["expected"], case["name"]


def test_predicate_agrees_with_oracle_on_random_batches(lib):
    import oracle
    rng = np.random.default_rng(0)
    for _ in range(300):
        n = int(rng.integers(1, 9))
        T = rng.choice(np.array([0.0, 5e-7, 0.5, 1.0, 1.3], np.float32), n)
        k = rng.choice(np.array([-1, -1, -1, 1, 5, 50, 1 << 30], np.int32), n)
        p = rng.choice(np.array([1.0, 1.0, 0.9], np.float32), n)
        mp = rng.choice(np.array([0.0, 0.0, 0.05], np.float32), n)
        det = bool(rng.integers(0, 2))
        assert dsts.select_path(T, k, p, mp, deterministic=det) == oracle.select_path(T, k, p, mp, det)


def test_empty_batch_rejected(lib):
    with pytest.raises(dsts.SamplerError) as e:
        dsts.select_path([], [], [], [], n_rows=0)
    assert e.value.status == dsts.SAMPLER_EINVAL


def _args(n=2, V=16, **kw):
    keep = []
    a = dsts.StepArgs()
    a.logits = 0x1000
    a.dtype = dsts.DTYPE_F32
    a.n_rows = n
    a.vocab = V
    a.row_stride = V
    a.token_ids = 0x2000
    for k, v in kw.items():
        if isinstance(v, np.ndarray):
            keep.append(v)
            setattr(a, k, v.ctypes.data)
        else:
            setattr(a, k, v)
    return a, keep


CFG = dsts.Config(max_rows=8, max_vocab=1024, max_history_per_row=64, max_top_logprobs=20, device=0, flags=0,
                  max_bias_per_row=16)


@pytest.mark.parametrize("change,status", [
    (dict(n_rows=0), dsts.SAMPLER_EINVAL),
    (dict(n_rows=9), dsts.SAMPLER_ECAPACITY),
    (dict(vocab=0), dsts.SAMPLER_EINVAL),
    (dict(vocab=2048, row_stride=2048), dsts.SAMPLER_ECAPACITY),
    (dict(row_stride=8), dsts.SAMPLER_EINVAL),
    (dict(logits=None), dsts.SAMPLER_EINVAL),
    (dict(token_ids=None), dsts.SAMPLER_EINVAL),
    (dict(dtype=7), dsts.SAMPLER_EINVAL),
    (dict(temperature=np.array([1.0, -0.5], np.float32)), dsts.SAMPLER_EINVAL),
    (dict(temperature=np.array([1.0, np.nan], np.float32)), dsts.SAMPLER_EINVAL),
    (dict(temperature=np.array([1.0, np.inf], np.float32)), dsts.SAMPLER_EINVAL),
    (dict(top_p=np.array([0.0, 1.0], np.float32)), dsts.SAMPLER_EINVAL),
    (dict(top_p=np.array([1.5, 1.0], np.float32)), dsts.SAMPLER_EINVAL),
    (dict(top_k=np.array([0, 5], np.int32)), dsts.SAMPLER_EINVAL),
    (dict(top_k=np.array([-2, 5], np.int32)), dsts.SAMPLER_EINVAL),
    (dict(min_p=np.array([-0.1, 0.0], np.float32)), dsts.SAMPLER_EINVAL),
    (dict(min_p=np.array([1.1, 0.0], np.float32)), dsts.SAMPLER_EINVAL),
    (dict(repetition_penalty=np.array([0.0, 1.0], np.float32)), dsts.SAMPLER_EINVAL),
    (dict(presence_penalty=np.array([np.inf, 0.0], np.float32)), dsts.SAMPLER_EINVAL),
    (dict(history_len=np.array([65, 0], np.int32), history_start=np.zeros(2, np.int64), history_ids=0x3000),
     dsts.SAMPLER_ECAPACITY),
    (dict(history_len=np.array([4, 0], np.int32), history_start=np.zeros(2, np.int64)), dsts.SAMPLER_EINVAL),
    (dict(history_len=np.array([4, 0], np.int32), history_ids=0x3000), dsts.SAMPLER_EINVAL),
    (dict(history_len=np.array([-1, 0], np.int32), history_start=np.zeros(2, np.int64), history_ids=0x3000),
     dsts.SAMPLER_EINVAL),
    (dict(top_logprobs=21, top_logprob_vals=0x4000, top_logprob_ids=0x5000), dsts.SAMPLER_ECAPACITY),
    (dict(top_logprobs=5), dsts.SAMPLER_EINVAL),
    # logits processors
    (dict(vocab_mask=0x6000, mask_stride=0), dsts.SAMPLER_EINVAL),          # needs ceil(16 / 32) = 1 word
    (dict(bias_len=np.array([2, 0], np.int32), bias_start=np.zeros(2, np.int64)), dsts.SAMPLER_EINVAL),
    (dict(bias_len=np.array([17, 0], np.int32), bias_start=np.zeros(2, np.int64), bias_ids=0x7000,
          bias_vals=0x8000), dsts.SAMPLER_ECAPACITY),
    (dict(bias_len=np.array([-1, 0], np.int32), bias_start=np.zeros(2, np.int64), bias_ids=0x7000,
          bias_vals=0x8000), dsts.SAMPLER_EINVAL),
    (dict(bias_len=np.array([10, 0], np.int32), bias_start=np.zeros(2, np.int64), bias_ids=0x7000,
          bias_vals=0x8000, stop_len=np.array([7, 0], np.int32), stop_start=np.zeros(2, np.int64),
          stop_ids=0x9000, min_tokens=np.array([3, 3], np.int32), output_len=np.array([0, 0], np.int32)),
     dsts.SAMPLER_ECAPACITY),                                                # 10 + 7 active stop ids > 16
    (dict(stop_len=np.array([2, 0], np.int32), stop_start=np.zeros(2, np.int64),
          min_tokens=np.array([3, 3], np.int32), output_len=np.array([0, 0], np.int32)), dsts.SAMPLER_EINVAL),
    (dict(min_tokens=np.array([3, 3], np.int32)), dsts.SAMPLER_EINVAL),      # without output_len
    # logprob modes
    (dict(logprob_mode=3), dsts.SAMPLER_EINVAL),
])
def test_validation_errors(lib, change, status):
    a, keep = _args(**change)
    st, msg = dsts.validate(CFG, a)
    assert st == status, msg
    assert msg


def test_validation_accepts_good_args(lib):
    a, keep = _args(temperature=np.array([0.0, 0.7], np.float32), top_k=np.array([-1, 20], np.int32),
                    top_p=np.array([1.0, 0.9], np.float32), min_p=np.array([0.0, 0.05], np.float32),
                    history_len=np.array([4, 0], np.int32), history_start=np.zeros(2, np.int64),
                    history_ids=0x3000, top_logprobs=20, top_logprob_vals=0x4000, top_logprob_ids=0x5000)
    st, msg = dsts.validate(CFG, a)
    assert st == dsts.SAMPLER_OK, msg


def test_validation_accepts_processors_and_modes(lib):
    # a mask of exactly ceil(V / 32) words; stop lists count only while min_tokens is active
    a, keep = _args(vocab_mask=0x6000, mask_stride=1, bias_len=np.array([10, 16], np.int32),
                    bias_start=np.array([0, 10], np.int64), bias_ids=0x7000, bias_vals=0x8000,
                    stop_len=np.array([7, 7], np.int32), stop_start=np.zeros(2, np.int64), stop_ids=0x9000,
                    min_tokens=np.array([3, 3], np.int32), output_len=np.array([3, 5], np.int32),
                    logprob_mode=1)
    st, msg = dsts.validate(CFG, a)
    assert st == dsts.SAMPLER_OK, msg
    for t in ([0.0, 1.0], [1.0, 1.0], [1e-7, 0.0]):
        a, keep = _args(logprob_mode=2, temperature=np.array(t, np.float32))
        st, msg = dsts.validate(CFG, a)
        assert st == dsts.SAMPLER_OK, msg


def test_create_without_gpu_reports_ehip(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(dsts.SamplerError) as e:
        dsts.Sampler(4, 1024)
    assert e.value.status == dsts.SAMPLER_EHIP
    assert "device" in str(e.value)


def test_create_rejects_bad_config(lib):
    h = ctypes.c_void_p()
    bad = dsts.Config(max_rows=0, max_vocab=1024, max_history_per_row=0, max_top_logprobs=0, device=0, flags=0)
    assert lib.sampler_create(ctypes.byref(bad), ctypes.byref(h)) in (dsts.SAMPLER_EINVAL, dsts.SAMPLER_EHIP)
    assert not h.value


def test_create_history_cap(lib):
    # histories up to 2^17 - 1 ids per row (longer than 4,096: counted ahead
    # of the row kernel); beyond that the config is rejected before any
    # device is touched
    h = ctypes.c_void_p()
    cfg = dsts.Config(max_rows=4, max_vocab=1024, max_history_per_row=131_072, max_top_logprobs=0, device=0)
    assert lib.sampler_create(ctypes.byref(cfg), ctypes.byref(h)) == dsts.SAMPLER_EINVAL
    lib.sampler_last_error.restype = ctypes.c_char_p
    assert b"131071" in lib.sampler_last_error(None)
    assert not h.value
    cfg = dsts.Config(max_rows=4, max_vocab=1024, max_history_per_row=131_071, max_top_logprobs=0, device=0)
    st = lib.sampler_create(ctypes.byref(cfg), ctypes.byref(h))
    if st == dsts.SAMPLER_OK:  # a GPU is present
        lib.sampler_destroy(h)
    else:
        assert st == dsts.SAMPLER_EHIP


def test_create_rejects_two_force_flags(lib):
    h = ctypes.c_void_p()
    for flags in (dsts.FLAG_FORCE_FILTERED | dsts.FLAG_FORCE_PATH_GREEDY,
                  dsts.FLAG_FORCE_PATH_GREEDY | dsts.FLAG_FORCE_PATH_GUMBEL,
                  dsts.FLAG_FORCE_STREAM | dsts.FLAG_NO_STREAM, 1 << 9):
        cfg = dsts.Config(max_rows=4, max_vocab=1024, max_history_per_row=0, max_top_logprobs=0, device=0,
                          flags=flags)
        assert lib.sampler_create(ctypes.byref(cfg), ctypes.byref(h)) == dsts.SAMPLER_EINVAL
        assert not h.value
    cfg = dsts.Config(max_rows=4, max_vocab=1024, device=0, wait_spin_limit=-1)
    assert lib.sampler_create(ctypes.byref(cfg), ctypes.byref(h)) == dsts.SAMPLER_EINVAL


def test_set_wait_spin_limit_rejects_bad_arguments(lib):
    assert lib.sampler_set_wait_spin_limit(None, 0) == dsts.SAMPLER_EINVAL


def test_binding_checks_device_tensors():
    # the binding refuses tensors the kernel would misread: wrong dtype,
    # wrong device, non-contiguous, wrong shape, spans past the buffer
    import torch
    from decode_step_token_sampler_amd import _check_spans, _check_tensor
    dev = torch.device("cuda", 0)
    with pytest.raises(ValueError, match="CUDA"):
        _check_tensor(torch.zeros(4, dtype=torch.int32), "history_ids", torch.int32, dev)
    starts, lens = np.array([0, 6], np.int64), np.array([4, 4], np.int32)
    with pytest.raises(ValueError, match="outside"):
        _check_spans("history_ids", 8, starts, lens)
    _check_spans("history_ids", 10, starts, lens)
    _check_spans("history_ids", 8, starts, np.array([4, 0], np.int32))  # empty spans may point anywhere
    with pytest.raises(ValueError, match="outside"):
        _check_spans("bias_ids", 8, np.array([-1], np.int64), np.array([1], np.int32))


def test_noalloc_without_gpu_reports_ehip(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    a = dsts.StepArgs()
    a.n_rows, a.vocab, a.row_stride = 1, 16, 16
    assert lib.sampler_step_noalloc(ctypes.byref(a), 0, 0, None) == dsts.SAMPLER_EHIP
    assert "device" in lib.sampler_noalloc_last_error().decode()
    # flags are checked before the device
    assert lib.sampler_step_noalloc(ctypes.byref(a), dsts.FLAG_COOPERATIVE_LAUNCH, 0, None) == dsts.SAMPLER_EINVAL


def test_validation_accepts_raw_logprobs_at_any_temperature(lib):
    a, keep = _args(logprob_mode=2, temperature=np.array([1.0, 0.7], np.float32))
    st, msg = dsts.validate(CFG, a)
    assert st == dsts.SAMPLER_OK, msg
