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
