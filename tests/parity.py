"""Helpers that run one batch through the HIP library and through the CPU
oracle, and compare them under the parity rules:

  token ids     bit-exact
  probs         |gpu - oracle| <= 1e-6 (absolute)
  logprobs      the -inf pattern identical; finite values within 1e-5
  top logprobs  ids identical, values within 1e-5
  row status    identical

Rows the oracle flags are checked too, against what their flag allows:
  Gumbel near-tie (top two scores within 1e-6 relative) or inverse-CDF
      margin (u S within 1e-10 relative of a step): every output as above,
      and the token is the oracle's or the one on the other side of the tie
      or step;
  top-p margin (the crossing within 1e-6 of the target mass, where it
      decides the kept set) or min-p margin (a kept value within 1e-9 of
      min_p times the largest probability): the row must match, output for
      output, the oracle's outputs for one of the kept sets the margin allows
      (the crossing one tie group earlier or later, the near-boundary values
      in or out).
A row that matches none of them fails.  The flagged rows are counted by
class, and a batch may flag at most FLAG_CEILING of its rows (at least one).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

import oracle

PROB_TOL = 1e-6
LOGPROB_TOL = 1e-5
FLAG_MASK = oracle.FLAG_GUMBEL_NEAR_TIE | oracle.FLAG_TOPP_MARGIN | oracle.FLAG_MINP_MARGIN | oracle.FLAG_ICDF_MARGIN
FLAG_CLASSES = {"gumbel_near_tie": oracle.FLAG_GUMBEL_NEAR_TIE, "topp_margin": oracle.FLAG_TOPP_MARGIN,
                "minp_margin": oracle.FLAG_MINP_MARGIN, "icdf_margin": oracle.FLAG_ICDF_MARGIN}
FLAG_CEILING = 0.05


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
    o = oracle.step(batch.logits, **kw)
    o["_call"] = (batch.logits, kw)
    return o


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
    flagged_by_class: dict = dataclasses.field(default_factory=dict)
    flagged_failed: list = dataclasses.field(default_factory=list)
    flag_ceiling: int = 0

    def ok(self) -> bool:
        return (not self.token_mismatch and self.max_prob_err <= PROB_TOL and self.max_logprob_err <= LOGPROB_TOL
                and self.inf_mismatch == 0 and self.toplp_mismatch == 0 and self.status_mismatch == 0
                and not self.flagged_failed and self.flagged <= self.flag_ceiling)


def _row_errors(g, gi, ref):
    """Deviations of GPU row gi from a reference row (1-D arrays): (prob
    error, logprob error, logprob ulps, -inf mismatches, top-logprob
    mismatches)."""
    pe = le = ulps = 0.0
    inf_mis = tl_mis = 0
    if ref.get("probs") is not None and "probs" in g:
        pe = float(np.max(np.abs(g["probs"][gi].astype(np.float64) - ref["probs"]))) if ref["probs"].size else 0.0
    if ref.get("logprobs") is not None and "logprobs" in g:
        gl, ol = g["logprobs"][gi], ref["logprobs"]
        gn, on = np.isneginf(gl), np.isneginf(ol)
        inf_mis = int(np.sum(gn != on))
        fin = ~gn & ~on
        if fin.any():
            d = np.abs(gl[fin].astype(np.float64) - ol[fin].astype(np.float64))
            le = float(d.max())
            ulps = float((d / np.spacing(np.abs(ol[fin])).astype(np.float64)).max())
    if ref.get("top_logprob_ids") is not None and "top_logprob_ids" in g:
        gv = g["top_logprob_vals"][gi].astype(np.float64)
        ov = ref["top_logprob_vals"].astype(np.float64)
        fin = ~np.isneginf(ov)
        bad = (g["top_logprob_ids"][gi] != ref["top_logprob_ids"]) | (np.isneginf(gv) != np.isneginf(ov))
        bad[fin] |= np.abs(gv[fin] - ov[fin]) > LOGPROB_TOL
        tl_mis = int(np.sum(bad))
    return pe, le, ulps, inf_mis, tl_mis


def _row_ok(g, gi, ref) -> bool:
    """GPU row gi against one reference row; the token may also be the
    reference's alternative where the reference flags a near-tie or an
    inverse-CDF margin."""
    tok = int(g["token_ids"][gi])
    alt = int(ref["token_alt"]) if int(ref["flags"]) & (oracle.FLAG_GUMBEL_NEAR_TIE | oracle.FLAG_ICDF_MARGIN) else None
    if tok != int(ref["token_ids"]) and (alt is None or tok != alt):
        return False
    if "row_status" in g and int(g["row_status"][gi]) != int(ref["row_status"]):
        return False
    pe, le, _, inf_mis, tl_mis = _row_errors(g, gi, ref)
    return pe <= PROB_TOL and le <= LOGPROB_TOL and inf_mis == 0 and tl_mis == 0


def check_flagged_row(g, gi, o, r) -> bool:
    """GPU row gi against oracle row r, which the oracle flags: its own
    outputs (with the token's alternative), else the outputs of each kept
    set its margin allows."""
    own = {k: (None if v is None else v[r]) for k, v in o.items() if not k.startswith("_")}
    if _row_ok(g, gi, own):
        return True
    if not int(o["flags"][r]) & (oracle.FLAG_TOPP_MARGIN | oracle.FLAG_MINP_MARGIN):
        return False
    logits, kw = o["_call"]
    for kept in oracle.row_alternatives(logits, r, **kw)[1:]:
        if _row_ok(g, gi, oracle.row_with_kept(logits, r, kept, **kw)):
            return True
    return False


def compare(g, o, rows=None) -> Report:
    """Compare GPU outputs g with oracle outputs o (rows: GPU row index of each oracle row)."""
    n = len(o["token_ids"])
    rows = np.arange(n) if rows is None else np.asarray(rows)
    flagged = (o["flags"] & FLAG_MASK) != 0
    by_class = {name: int(np.sum((o["flags"] & bit) != 0)) for name, bit in FLAG_CLASSES.items()}
    failed = [int(r) for r in np.flatnonzero(flagged) if not check_flagged_row(g, int(rows[r]), o, int(r))]
    good = ~flagged
    tok_g = g["token_ids"][rows]
    mism = [int(r) for r in np.flatnonzero((tok_g != o["token_ids"]) & good)]
    status_mis = int(np.sum(g["row_status"][rows][good] != o["row_status"][good])) if "row_status" in g else 0
    pe = le = ulps = 0.0
    inf_mis = 0
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
                  max_logprob_ulps=ulps, inf_mismatch=inf_mis, toplp_mismatch=tl_mis, status_mismatch=status_mis,
                  flagged_by_class=by_class, flagged_failed=failed,
                  flag_ceiling=max(1, math.ceil(FLAG_CEILING * n)))
