"""Seeded synthetic inputs for the per-decode-step sampler.

This module produces inputs only.  It holds none of the sampler's arithmetic,
and the HIP library and the CPU oracle both consume what it makes.  The
pages' workloads are real decode batches: an SGLang batch at several batch
sizes over Qwen vocabularies ("SGLang's +75% sampler speedup skips Qwen3 chat
requests", section "What a free T4 can and cannot tell you"), and a vLLM
0.5.0 deployment at concurrency 64 with a ~128k vocabulary (the
xbrilliance.ai note on sampling-parameter decode cost, introduction).  No
dataset is involved.  The generators below stand in for real logits with a
Zipf-biased Gaussian:

  logit_i = 3 * N(0, 1) + bias_i,  bias_i = -1.1 * ln(rank_r(i) + 1)

where rank_r is a seeded permutation of 0..V-1 per row.  Histories draw
Zipf(1.1) ranks over 1..V by inverse CDF and map each rank back through the
same permutation, so the tokens that repeat are the high-prior ones.  bf16
inputs are the fp32 values rounded to nearest-even.  Each row has its own
numpy PCG64 stream keyed by (config, set, row).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

TOP_K_ALL = -1


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32)


def zipf_row(rng: np.random.Generator, V: int):
    """One row of Zipf-biased Gaussian logits and its rank permutation."""
    rank = rng.permutation(V).astype(np.int64)          # rank_r(i)
    bias = -1.1 * np.log(rank.astype(np.float64) + 1.0)
    x = 3.0 * rng.standard_normal(V) + bias
    return x.astype(np.float32), rank


def zipf_history(rng: np.random.Generator, rank: np.ndarray, length: int, s: float = 1.1) -> np.ndarray:
    """`length` ids whose ranks are Zipf(s) over 1..V, mapped through `rank`."""
    V = rank.shape[0]
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = rng.random(length)
    ranks = np.minimum(np.searchsorted(cdf, u, side="left"), V - 1)  # rank - 1
    inv = np.empty(V, dtype=np.int64)
    inv[rank] = np.arange(V)
    return inv[ranks].astype(np.int32)


@dataclasses.dataclass
class Batch:
    """One step's inputs, all host numpy arrays."""
    name: str
    dtype: str                       # "f32" or "bf16"
    logits: np.ndarray               # [N, V] float32, or uint16 bf16 bits
    temperature: np.ndarray
    top_k: np.ndarray
    top_p: np.ndarray
    min_p: np.ndarray
    repetition_penalty: Optional[np.ndarray] = None
    presence_penalty: Optional[np.ndarray] = None
    frequency_penalty: Optional[np.ndarray] = None
    history_ids: Optional[np.ndarray] = None
    history_start: Optional[np.ndarray] = None
    history_len: Optional[np.ndarray] = None
    seed: int = 0
    offset: int = 0
    row_seed: Optional[np.ndarray] = None
    row_offset: Optional[np.ndarray] = None
    row_stream: Optional[np.ndarray] = None
    want_probs: bool = False
    want_logprobs: bool = False
    top_logprobs: int = 0

    @property
    def n_rows(self) -> int:
        return int(self.logits.shape[0])

    @property
    def vocab(self) -> int:
        return int(self.logits.shape[1])

    def algorithmic_bytes(self) -> int:
        """Bytes the method must move once: logits read, outputs written, history read."""
        n, v = self.n_rows, self.vocab
        b = n * v * (2 if self.dtype == "bf16" else 4)
        b += 4 * n                                    # token ids
        if self.want_probs:
            b += 4 * n * v
        if self.want_logprobs:
            b += 4 * n * v
        if self.top_logprobs:
            b += 8 * n * self.top_logprobs
        if self.history_len is not None:
            # each distinct span is read once
            spans = {(int(s), int(l)) for s, l in zip(self.history_start, self.history_len)}
            b += 4 * sum(l for _, l in spans)
        return b

    def subset(self, rows) -> "Batch":
        """The same rows as an independent batch (explicit per-row RNG keys)."""
        rows = np.asarray(rows, dtype=np.int64)
        n = self.n_rows
        rs = self.row_seed if self.row_seed is not None else np.full(n, self.seed, np.uint64)
        ro = self.row_offset if self.row_offset is not None else np.full(n, self.offset, np.uint64)
        rst = self.row_stream if self.row_stream is not None else np.arange(n, dtype=np.uint32)
        pick = lambda a: None if a is None else np.ascontiguousarray(a[rows])
        return dataclasses.replace(
            self, logits=np.ascontiguousarray(self.logits[rows]),
            temperature=pick(self.temperature), top_k=pick(self.top_k), top_p=pick(self.top_p),
            min_p=pick(self.min_p), repetition_penalty=pick(self.repetition_penalty),
            presence_penalty=pick(self.presence_penalty), frequency_penalty=pick(self.frequency_penalty),
            history_start=pick(self.history_start), history_len=pick(self.history_len),
            row_seed=np.ascontiguousarray(rs[rows]), row_offset=np.ascontiguousarray(ro[rows]),
            row_stream=np.ascontiguousarray(rst[rows]))

    ABLATION_STAGES = ("defaults", "penalties", "min_p", "all")

    def ablation(self, stage: str) -> "Batch":
        """The per-feature ablation of a full-chain batch, one stage of it:
        "defaults" keeps only the temperatures (no penalties and no history,
        top_k = -1, top_p = 1, min_p = 0); "penalties" adds the batch's own
        penalties and histories; "min_p" adds its min_p; "all" adds top-k and
        top-p, which is the batch unchanged.  Logits, outputs and RNG keys
        stay the same throughout."""
        if stage not in self.ABLATION_STAGES:
            raise ValueError("unknown ablation stage %r" % stage)
        if stage == "all":
            return self
        n = self.n_rows
        b = dataclasses.replace(self, top_k=np.full(n, -1, np.int32), top_p=np.ones(n, np.float32))
        if stage != "min_p":
            b = dataclasses.replace(b, min_p=np.zeros(n, np.float32))
        if stage == "defaults":
            b = dataclasses.replace(b, repetition_penalty=None, presence_penalty=None, frequency_penalty=None,
                                    history_ids=None, history_start=None, history_len=None)
        return b


def _logits(cfg: int, set_id: int, n: int, V: int, dtype: str):
    rows, ranks = [], []
    for r in range(n):
        x, rank = zipf_row(_rng(cfg, set_id, r, 0), V)
        rows.append(x)
        ranks.append(rank)
    L = np.stack(rows)
    if dtype == "bf16":
        L = f32_to_bf16_bits(L)
    return L, ranks


def _chain_params(p: np.random.Generator, n: int):
    """Per-row parameters of the full-chain workload (N=64, V=128,000)."""
    T = p.uniform(0.3, 1.2, n).astype(np.float32)
    rep = p.uniform(1.0, 1.3, n).astype(np.float32)
    pres = p.uniform(0.0, 0.5, n).astype(np.float32)
    freq = p.uniform(0.0, 0.5, n).astype(np.float32)
    top_k = np.where(p.random(n) < 0.5, -1, 50).astype(np.int32)
    top_p = np.where(p.random(n) < 0.5, 1.0, 0.9).astype(np.float32)
    min_p = np.where(p.random(n) < 0.5, 0.0, 0.02).astype(np.float32)
    if not np.any((top_k != -1) | (top_p != 1.0) | (min_p > 0)):
        top_k[0] = 50
    return T, rep, pres, freq, top_k, top_p, min_p


def config(cfg: int, set_id: int = 0, n_rows: Optional[int] = None, vocab: Optional[int] = None,
           history_len: int = 2048, temperature: Optional[float] = None, step: int = 0) -> Batch:
    """The five workloads; n_rows / vocab shrink them for quick parity cases.

    1: Gumbel only, N=4, V=1,024, fp32, T=0.7, ids + probs.
    2: batch-1 decode, N=1, V=151,936, bf16, T=1.0 (or 0 for the greedy run),
       ids only, offset = step.
    3: mixed filtered batch, N=32, V=151,936, bf16; half top_k=20/top_p=0.95,
       a quarter min_p=0.05, a quarter plain with one greedy row; ids + probs
       + logprobs.
    4: full chain, N=64, V=128,000, fp32, penalties over 2,048-id histories,
       top_k in {-1,50}, top_p in {1,0.9}, min_p in {0,0.02}; ids + probs +
       logprobs.
    5: N=512 (128 requests x 4 forks sharing history and parameters),
       V=256,000, bf16, parameters as 4; ids + top-20 logprobs.
    """
    p = _rng(cfg, set_id, 999_983)
    if cfg == 1:
        n, V = n_rows or 4, vocab or 1024
        L, _ = _logits(1, set_id, n, V, "f32")
        return Batch("gumbel-only N=%d V=%d fp32" % (n, V), "f32", L,
                     temperature=np.full(n, 0.7, np.float32), top_k=np.full(n, -1, np.int32),
                     top_p=np.ones(n, np.float32), min_p=np.zeros(n, np.float32),
                     seed=0, offset=0, want_probs=True)
    if cfg == 2:
        n, V = n_rows or 1, vocab or 151_936
        L, _ = _logits(2, set_id, n, V, "bf16")
        t = 1.0 if temperature is None else temperature
        return Batch("batch-1 decode N=%d V=%d bf16 T=%g" % (n, V, t), "bf16", L,
                     temperature=np.full(n, t, np.float32), top_k=np.full(n, -1, np.int32),
                     top_p=np.ones(n, np.float32), min_p=np.zeros(n, np.float32),
                     seed=0, offset=step)
    if cfg == 3:
        n, V = n_rows or 32, vocab or 151_936
        L, _ = _logits(3, set_id, n, V, "bf16")
        T = p.uniform(0.5, 1.5, n).astype(np.float32)
        top_k = np.full(n, -1, np.int32)
        top_p = np.ones(n, np.float32)
        min_p = np.zeros(n, np.float32)
        perm = p.permutation(n)
        h, q = n // 2, n // 4
        top_k[perm[:h]] = 20
        top_p[perm[:h]] = 0.95
        min_p[perm[h:h + q]] = 0.05
        T[perm[-1]] = 0.0                              # the greedy row
        return Batch("mixed filtered N=%d V=%d bf16" % (n, V), "bf16", L, temperature=T, top_k=top_k,
                     top_p=top_p, min_p=min_p, seed=0, offset=step, want_probs=True, want_logprobs=True)
    if cfg == 4:
        n, V = n_rows or 64, vocab or 128_000
        L, ranks = _logits(4, set_id, n, V, "f32")
        T, rep, pres, freq, top_k, top_p, min_p = _chain_params(p, n)
        H = np.concatenate([zipf_history(_rng(4, set_id, r, 1), ranks[r], history_len) for r in range(n)])
        return Batch("full chain N=%d V=%d fp32" % (n, V), "f32", L, temperature=T, top_k=top_k,
                     top_p=top_p, min_p=min_p, repetition_penalty=rep, presence_penalty=pres,
                     frequency_penalty=freq, history_ids=H,
                     history_start=(np.arange(n, dtype=np.int64) * history_len),
                     history_len=np.full(n, history_len, np.int32), seed=0, offset=step,
                     want_probs=True, want_logprobs=True)
    if cfg == 5:
        n, V = n_rows or 512, vocab or 256_000
        forks = 4
        n_req = (n + forks - 1) // forks
        L, ranks = _logits(5, set_id, n, V, "bf16")
        T, rep, pres, freq, top_k, top_p, min_p = _chain_params(p, n_req)
        req = np.arange(n) // forks
        H = np.concatenate([zipf_history(_rng(5, set_id, j, 1), ranks[j * forks], history_len)
                            for j in range(n_req)])
        return Batch("large vocab N=%d V=%d bf16 forks=4" % (n, V), "bf16", L, temperature=T[req],
                     top_k=top_k[req], top_p=top_p[req], min_p=min_p[req], repetition_penalty=rep[req],
                     presence_penalty=pres[req], frequency_penalty=freq[req], history_ids=H,
                     history_start=(req.astype(np.int64) * history_len),
                     history_len=np.full(n, history_len, np.int32), seed=0, offset=step,
                     row_stream=np.arange(n, dtype=np.uint32), top_logprobs=20)
    raise ValueError("unknown workload %r" % cfg)


def random_small(seed: int, n: int, V: int, dtype: str = "f32", *, ties: bool = False,
                 penalties: bool = True, history_len: int = 64, mix: str = "all") -> Batch:
    """Randomised small batch for parity sweeps (odd sizes, ties, every option)."""
    r = _rng(7, seed, n, V)
    if ties:
        x = r.integers(-4, 3, size=(n, V)).astype(np.float32) * 0.5
    else:
        x = (3.0 * r.standard_normal((n, V))).astype(np.float32)
    L = f32_to_bf16_bits(x) if dtype == "bf16" else x
    T = r.uniform(0.2, 1.6, n).astype(np.float32)
    top_k = r.choice(np.array([-1, 1, 2, 5, 20, 50, max(V - 1, 1), V, V + 3], np.int32), n)
    top_p = r.choice(np.array([1.0, 0.95, 0.9, 0.5, 0.1], np.float32), n)
    min_p = r.choice(np.array([0.0, 0.0, 0.02, 0.1, 0.5], np.float32), n)
    greedy = r.random(n) < 0.15
    T[greedy] = 0.0
    if mix == "plain":
        top_k[:] = -1
        top_p[:] = 1.0
        min_p[:] = 0.0
    b = Batch("random n=%d V=%d %s" % (n, V, dtype), dtype, L, temperature=T, top_k=top_k, top_p=top_p,
              min_p=min_p, seed=int(r.integers(0, 2**63)), offset=int(r.integers(0, 2**40)),
              want_probs=True, want_logprobs=True, top_logprobs=int(min(5, V)))
    if penalties:
        b.repetition_penalty = r.uniform(1.0, 1.5, n).astype(np.float32)
        b.presence_penalty = r.uniform(0.0, 0.8, n).astype(np.float32)
        b.frequency_penalty = r.uniform(0.0, 0.8, n).astype(np.float32)
        b.history_ids = r.integers(0, V, size=n * history_len).astype(np.int32)
        b.history_start = np.arange(n, dtype=np.int64) * history_len
        b.history_len = r.integers(0, history_len + 1, size=n).astype(np.int32)
    return b


@dataclasses.dataclass
class Processors:
    """Logits-processor inputs of one batch (grammar bitmask, logit_bias,
    min_tokens stop lists), as host arrays."""
    vocab_mask: np.ndarray       # uint32 [n, words + 1] (one spare word of stride)
    bias_ids: np.ndarray         # int32
    bias_vals: np.ndarray        # float32
    bias_start: np.ndarray       # int64 [n]
    bias_len: np.ndarray         # int32 [n]
    stop_ids: np.ndarray         # int32
    stop_start: np.ndarray       # int64 [n]
    stop_len: np.ndarray         # int32 [n]
    min_tokens: np.ndarray       # int32 [n]
    output_len: np.ndarray       # int32 [n]

    def kwargs(self) -> dict:
        return dict(vocab_mask=self.vocab_mask, bias_ids=self.bias_ids, bias_vals=self.bias_vals,
                    bias_start=self.bias_start, bias_len=self.bias_len, stop_ids=self.stop_ids,
                    stop_start=self.stop_start, stop_len=self.stop_len, min_tokens=self.min_tokens,
                    output_len=self.output_len)


def processors(seed: int, batch: Batch, max_entries: int = 512) -> Processors:
    """Seeded grammar masks, logit_bias lists and stop lists for `batch`.

    Masks per row cycle through: everything allowed, ~half allowed, ~5%
    allowed, two tokens allowed, nothing allowed.  Bias lists mix ids from the
    row's history (where there is one) with random ids, a few repeated ids
    (a token's entries are summed) and out-of-range ids, with values in
    [-5, 5]; one row biases its top token by -inf (a banned word) and one by
    a large positive value.  Stop lists of 1-8 ids are active on every other
    row (output_len < min_tokens)."""
    n, V = batch.n_rows, batch.vocab
    g = _rng(9001, seed, n, V)
    words = (V + 31) // 32
    allowed = np.ones((n, V), dtype=bool)
    for r in range(n):
        kind = r % 5
        if kind == 1:
            allowed[r] = g.random(V) < 0.5
        elif kind == 2:
            allowed[r] = g.random(V) < 0.05
        elif kind == 3:
            allowed[r] = False
            allowed[r, g.choice(V, size=min(2, V), replace=False)] = True
        elif kind == 4 and r % 10 == 9:
            allowed[r] = False
    bits = np.zeros((n, words * 32), dtype=np.uint64)
    bits[:, :V] = allowed
    packed = (bits.reshape(n, words, 32) << np.arange(32, dtype=np.uint64)).sum(axis=2).astype(np.uint32)
    mask = np.zeros((n, words + 1), dtype=np.uint32)
    mask[:, :words] = packed
    ids, vals, bstart, blen = [], [], [], []
    sids, sstart, slen = [], [], []
    for r in range(n):
        nb = int(g.integers(0, max_entries // 2 + 1)) if r % 4 != 3 else 0
        row_ids = []
        if batch.history_ids is not None and batch.history_len is not None and batch.history_len[r] > 0:
            h = batch.history_ids[batch.history_start[r]:batch.history_start[r] + batch.history_len[r]]
            row_ids += list(g.choice(h, size=min(nb // 2, len(h))))
        row_ids += list(g.integers(0, V, size=nb - len(row_ids)))
        if row_ids:
            row_ids[:2] = [-1, V][:len(row_ids[:2])]               # ignored ids
            if len(row_ids) > 6:
                row_ids[3] = row_ids[4]                            # a repeated id
        rv = list(g.uniform(-5.0, 5.0, size=len(row_ids)).astype(np.float32))
        if r % 7 == 5 and len(row_ids) > 8:
            row_ids[8] = int(np.argmax(batch.logits[r].view(np.float32) if batch.dtype == "f32"
                                       else bf16_bits_to_f32(batch.logits[r])))
            rv[8] = np.float32(-np.inf)
        if r % 7 == 6 and len(row_ids) > 8:
            rv[8] = np.float32(25.0)
        bstart.append(len(ids))
        blen.append(len(row_ids))
        ids += [int(x) for x in row_ids]
        vals += rv
        ns = int(g.integers(1, 9))
        sstart.append(len(sids))
        slen.append(ns)
        sids += [int(x) for x in g.integers(0, V, size=ns)]
        # stop lists must fit beside the bias list when active
        if blen[-1] + ns > max_entries:
            blen[-1] = max_entries - ns
    min_tokens = np.full(n, 4, dtype=np.int32)
    output_len = np.array([2 if r % 2 == 0 else 6 for r in range(n)], dtype=np.int32)
    return Processors(mask, np.array(ids, np.int32), np.array(vals, np.float32), np.array(bstart, np.int64),
                      np.array(blen, np.int32), np.array(sids, np.int32), np.array(sstart, np.int64),
                      np.array(slen, np.int32), min_tokens, output_len)
