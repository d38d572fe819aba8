"""Host-side checks of the benchmark's workload table and of the full-chain
ablation stages (no GPU)."""
import os
import subprocess
import sys

import numpy as np
import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.fixture(scope="module")
def chain():
    return workloads.config(4, set_id=0, n_rows=16, vocab=512)


def _filtered(b):
    return bool(np.any((b.top_k != -1) | (b.top_p != 1.0) | (b.min_p > 0)))


def _penalised(b):
    if b.repetition_penalty is None:
        return False
    return bool(np.any((b.repetition_penalty != 1) | (b.presence_penalty != 0) | (b.frequency_penalty != 0)))


def test_ablation_stages_add_one_feature_each(chain):
    d = chain.ablation("defaults")
    assert not _filtered(d) and not _penalised(d) and d.history_ids is None
    p = chain.ablation("penalties")
    assert not _filtered(p) and _penalised(p) and p.history_ids is chain.history_ids
    m = chain.ablation("min_p")
    assert _penalised(m) and np.array_equal(m.min_p, chain.min_p)
    assert np.all(m.top_k == -1) and np.all(m.top_p == 1.0)
    assert chain.ablation("all") is chain
    for b in (d, p, m):  # logits, temperatures, outputs and keys unchanged
        assert b.logits is chain.logits and b.temperature is chain.temperature
        assert (b.want_probs, b.want_logprobs, b.seed, b.offset) == (
            chain.want_probs, chain.want_logprobs, chain.seed, chain.offset)
    # the stages differ in bytes only by the histories
    assert chain.algorithmic_bytes() - d.algorithmic_bytes() == 4 * int(chain.history_len.sum())
    with pytest.raises(ValueError):
        chain.ablation("top_k")


def test_workload_table():
    assert "full-chain" in bench.WORKLOADS
    for name, (cfg, temp, sets, desc, stage) in bench.WORKLOADS.items():
        assert cfg in (1, 2, 3, 4, 5) and sets >= 1 and desc
        assert stage is None or (cfg == 4 and stage in workloads.Batch.ABLATION_STAGES)
    stages = {w[4] for w in bench.WORKLOADS.values() if w[4] is not None}
    assert stages == set(workloads.Batch.ABLATION_STAGES) - {"all"}


def test_more_than_one_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stdout


def test_batch_record_fields():
    # the note's batch switches for the full chain, and for a Gumbel-only batch
    full = bench.batch_record(workloads.config(4, set_id=0, n_rows=64, vocab=128_000 // 100))
    assert full["do_top_p_top_k"] and full["do_min_p"] and full["do_penalties"] and full["param_mixed"]
    assert full["sampling_tensor_bytes"] == 8 * 64 * 1280
    g = bench.batch_record(workloads.config(1))
    assert not (g["do_top_p_top_k"] or g["do_min_p"] or g["do_penalties"] or g["param_mixed"])
    assert g["num_seqs"] == 4 and g["vocab_size"] == 1024


def test_host_cpu_reports_cores():
    h = bench.host_cpu()
    assert h["logical_cores"] == os.cpu_count()
