"""Helpers that run one batch through the HIP library and through the CPU
oracle, and compare them under the parity rules:

  token ids     bit-exact, except rows the oracle flags (Gumbel near-tie
                below 1e-6 relative, top-p crossing within 1e-6 relative of
                the target mass, min-p boundary within 1e-9, inverse-CDF
                target within 1e-10 relative of a step of the CDF): counted
                and reported, not compared
  probs         |gpu - oracle| <= 1e-6 (absolute)
  logprobs      the -inf pattern identical; finite values within 1e-5
  top logprobs  ids identical, values within 1e-5
  row status    identical
"""
from __future__ import annotations

import dataclasses

import numpy as np

import oracle

PROB_TOL = 1e-6
LOGPROB_TOL = 1e-5
FLAG_MASK = oracle.FLAG_GUMBEL_NEAR_TIE | oracle.FLAG_TOPP_MARGIN | oracle.FLAG_MINP_MARGIN | oracle.FLAG_ICDF_MARGIN


def to_device(batch, device="cuda:0"):
    import torch
    if batch.dtype == "bf16":
        L = torch.from_numpy(batch.logits.view(np.int16)).view(torch.bfloat16).to(device)
    else:
        L = torch.from_numpy(batch.logits).to(device)
    H = None if batch.history_ids is None else torch.from_numpy(batch.history_ids).to(device)
    return L, H


def run_gpu(sampler, batch, logits=None, history=None, **over):
    if logits is None:
        logits, history = to_device(batch)
    kw = dict(temperature=batch.temperature, top_p=batch.top_p, top_k=batch.top_k, min_p=batch.min_p,
              repetition_penalty=batch.repetition_penalty, presence_penalty=batch.presence_penalty,
              frequency_penalty=batch.frequency_penalty, history_ids=history, history_start=batch.history_start,
              history_len=batch.history_len, seed=batch.seed, offset=batch.offset, row_seed=batch.row_seed,
              row_offset=batch.row_offset, row_stream=batch.row_stream, want_probs=batch.want_probs,
              want_logprobs=batch.want_logprobs, top_logprobs=batch.top_logprobs)
    kw.update(over)
    out = sampler.step(logits, **kw)
    import torch
    torch.cuda.synchronize()
    res = {k: (v.cpu().numpy() if hasattr(v, "cpu") else v) for k, v in out.items()}
    return res


def run_oracle(batch, n_threads=16, deterministic=False, **over):
    kw = dict(dtype=batch.dtype, temperature=batch.temperature, top_p=batch.top_p, top_k=batch.top_k,
              min_p=batch.min_p, repetition_penalty=batch.repetition_penalty,
              presence_penalty=batch.presence_penalty, frequency_penalty=batch.frequency_penalty,
              history_ids=batch.history_ids, history_start=batch.history_start, history_len=batch.history_len,
              seed=batch.seed, offset=batch.offset, row_seed=batch.row_seed, row_offset=batch.row_offset,
              row_stream=batch.row_stream, want_probs=batch.want_probs, want_logprobs=batch.want_logprobs,
              top_logprobs=batch.top_logprobs, n_threads=n_threads, deterministic=deterministic)
    kw.update(over)
    return oracle.step(batch.logits, **kw)


@dataclasses.dataclass
class Report:
    rows: int
    flagged: int
    token_mismatch: list
    max_prob_err: float
    max_logprob_err: float
    max_logprob_ulps: float
    inf_mismatch: int
    toplp_mismatch: int
    status_mismatch: int

    def ok(self) -> bool:
        return (not self.token_mismatch and self.max_prob_err <= PROB_TOL and self.max_logprob_err <= LOGPROB_TOL
                and self.inf_mismatch == 0 and self.toplp_mismatch == 0 and self.status_mismatch == 0)


def compare(g, o, rows=None) -> Report:
    """Compare GPU outputs g with oracle outputs o (rows: GPU row index of each oracle row)."""
    n = len(o["token_ids"])
    rows = np.arange(n) if rows is None else np.asarray(rows)
    flagged = (o["flags"] & FLAG_MASK) != 0
    tok_g = g["token_ids"][rows]
    mism = [int(r) for r in np.flatnonzero((tok_g != o["token_ids"]) & ~flagged)]
    status_mis = int(np.sum(g["row_status"][rows] != o["row_status"])) if "row_status" in g else 0
    pe = le = ulps = 0.0
    inf_mis = 0
    good = ~flagged
    if o["probs"] is not None and "probs" in g:
        d = np.abs(g["probs"][rows][good].astype(np.float64) - o["probs"][good])
        pe = float(d.max()) if d.size else 0.0
    if o["logprobs"] is not None and "logprobs" in g:
        gl = g["logprobs"][rows][good]
        ol = o["logprobs"][good]
        gi, oi = np.isneginf(gl), np.isneginf(ol)
        inf_mis = int(np.sum(gi != oi))
        fin = ~gi & ~oi
        if fin.any():
            d = np.abs(gl[fin].astype(np.float64) - ol[fin].astype(np.float64))
            le = float(d.max())
            ulp = np.spacing(np.abs(ol[fin])).astype(np.float64)
            ulps = float((d / ulp).max())
    tl_mis = 0
    if o["top_logprob_ids"] is not None and "top_logprob_ids" in g:
        gi = g["top_logprob_ids"][rows][good]
        oi = o["top_logprob_ids"][good]
        gv = g["top_logprob_vals"][rows][good].astype(np.float64)
        ov = o["top_logprob_vals"][good].astype(np.float64)
        same_inf = np.isneginf(gv) == np.isneginf(ov)
        fin = ~np.isneginf(ov)
        val_bad = np.zeros_like(same_inf)
        val_bad[fin] = np.abs(gv[fin] - ov[fin]) > LOGPROB_TOL
        tl_mis = int(np.sum((gi != oi) | ~same_inf | val_bad))
    return Report(rows=n, flagged=int(flagged.sum()), token_mismatch=mism, max_prob_err=pe, max_logprob_err=le,
                  max_logprob_ulps=ulps, inf_mismatch=inf_mis, toplp_mismatch=tl_mis, status_mismatch=status_mis)
