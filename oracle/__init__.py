"""CPU oracle for the per-decode-step token sampler -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never loads it and
shares no code with it: the arithmetic lives in ``sampler_oracle.c`` (plain
scalar C, fp32 steps rounded one at a time, fp64 after the temperature
division); this module only marshals numpy arrays through ctypes.

What each part follows (page titles; the C file names the sections):
  [A] "SGLang's +75% sampler speedup skips Qwen3 chat requests"
  [B] the SGLang 101 operations manual ("Logprobs are temperature-scaled",
      "What the flag switches")
  [C] "采样参数对解码开销的影响：temperature、top_p 与采样核路径"

Parity unpinned: the order of the three penalties (the pages name the three
penalties and their defaults but print no formula).  The repetition term is
pinned against the transformers library's repetition-penalty processor, the
frequency and presence terms by invariants (count-independence of presence,
linearity of frequency in the count, additivity), the whole by its identity
at the defaults, its locality and a hand-worked example.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sampler_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_sampler_oracle.so")
_lock = threading.Lock()
_lib = None

TOP_K_ALL = 1 << 30
PATH_GREEDY, PATH_GUMBEL, PATH_FILTERED, PATH_DETERMINISTIC = 0, 1, 2, 3
PATH_NAMES = {0: "greedy", 1: "gumbel", 2: "filtered", 3: "deterministic"}
FLAG_GUMBEL_NEAR_TIE, FLAG_TOPP_MARGIN, FLAG_MINP_MARGIN, FLAG_SPELLING_MISMATCH = 1, 2, 4, 8
FLAG_ICDF_MARGIN = 16

GCC_FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11", "-pthread"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (scalar, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Args(ctypes.Structure):
    _fields_ = [
        ("logits", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("n_rows", ctypes.c_int32),
        ("vocab", ctypes.c_int32),
        ("row_stride", ctypes.c_int64),
        ("temperature", ctypes.c_void_p),
        ("top_p", ctypes.c_void_p),
        ("min_p", ctypes.c_void_p),
        ("repetition_penalty", ctypes.c_void_p),
        ("presence_penalty", ctypes.c_void_p),
        ("frequency_penalty", ctypes.c_void_p),
        ("top_k", ctypes.c_void_p),
        ("history_ids", ctypes.c_void_p),
        ("history_start", ctypes.c_void_p),
        ("history_len", ctypes.c_void_p),
        ("seed", ctypes.c_uint64),
        ("offset", ctypes.c_uint64),
        ("row_seed", ctypes.c_void_p),
        ("row_offset", ctypes.c_void_p),
        ("row_stream", ctypes.c_void_p),
        ("deterministic", ctypes.c_int32),
        ("n_threads", ctypes.c_int32),
        ("token_ids", ctypes.c_void_p),
        ("probs", ctypes.c_void_p),
        ("logprobs", ctypes.c_void_p),
        ("top_logprobs", ctypes.c_int32),
        ("top_logprob_vals", ctypes.c_void_p),
        ("top_logprob_ids", ctypes.c_void_p),
        ("row_status", ctypes.c_void_p),
        ("diag_flags", ctypes.c_void_p),
        ("diag_gumbel_gap", ctypes.c_void_p),
        ("diag_topp_margin", ctypes.c_void_p),
        ("diag_kept", ctypes.c_void_p),
        ("vocab_mask", ctypes.c_void_p),
        ("mask_stride", ctypes.c_int64),
        ("bias_ids", ctypes.c_void_p),
        ("bias_vals", ctypes.c_void_p),
        ("bias_start", ctypes.c_void_p),
        ("bias_len", ctypes.c_void_p),
        ("stop_ids", ctypes.c_void_p),
        ("stop_start", ctypes.c_void_p),
        ("stop_len", ctypes.c_void_p),
        ("min_tokens", ctypes.c_void_p),
        ("output_len", ctypes.c_void_p),
        ("logprob_mode", ctypes.c_int32),
        ("inverse_cdf", ctypes.c_int32),
        ("diag_token_alt", ctypes.c_void_p),
    ]


LOGPROB_MODES = {"processed": 0, "temperature": 1, "raw": 2}


def lib():
    global _lib
    with _lock:
        if _lib is None:
            # ORACLE_LIBRARY: an oracle built elsewhere from the same source
            # (the sanitizer test builds one with address and UB checks)
            path = os.environ.get("ORACLE_LIBRARY") or build()
            L = ctypes.CDLL(path)
            L.orc_step.argtypes = [ctypes.POINTER(_Args)]
            L.orc_step.restype = ctypes.c_int
            L.orc_philox4x32_10.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
            L.orc_philox4x32_10.restype = None
            L.orc_draw_word.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int64]
            L.orc_draw_word.restype = ctypes.c_uint32
            L.orc_exp1_from_word.argtypes = [ctypes.c_uint32]
            L.orc_exp1_from_word.restype = ctypes.c_double
            L.orc_icdf_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64]
            L.orc_icdf_uniform.restype = ctypes.c_double
            L.orc_fill_exp1.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int64,
                                        ctypes.c_void_p]
            L.orc_fill_exp1.restype = None
            L.orc_select_path.argtypes = [ctypes.c_int32] + [ctypes.c_void_p] * 4 + [ctypes.c_int32, ctypes.c_void_p]
            L.orc_select_path.restype = ctypes.c_int
            L.orc_do_penalties.argtypes = [ctypes.c_int32] + [ctypes.c_void_p] * 3
            L.orc_do_penalties.restype = ctypes.c_int
            L.orc_row_is_greedy.argtypes = [ctypes.c_float]
            L.orc_row_is_greedy.restype = ctypes.c_int
            L.orc_normalized_top_k.argtypes = [ctypes.c_float, ctypes.c_int32]
            L.orc_normalized_top_k.restype = ctypes.c_int32
            L.orc_row_alternative.argtypes = [ctypes.POINTER(_Args), ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
            L.orc_row_alternative.restype = ctypes.c_int
            L.orc_row_with_kept.argtypes = [ctypes.POINTER(_Args), ctypes.c_int32, ctypes.c_void_p]
            L.orc_row_with_kept.restype = ctypes.c_int
            _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _arr(a, dtype, n=None):
    if a is None:
        return None
    out = np.ascontiguousarray(np.asarray(a, dtype=dtype))
    if n is not None and out.shape != (n,):
        raise ValueError(f"expected shape ({n},), got {out.shape}")
    return out


def philox4x32_10(counter, key):
    """Four 32-bit words of Philox4x32-10 for a 4-word counter and 2-word key."""
    c = np.ascontiguousarray(np.asarray(counter, dtype=np.uint32).reshape(4))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32).reshape(2))
    out = np.zeros(4, dtype=np.uint32)
    lib().orc_philox4x32_10(c.ctypes.data, k.ctypes.data, out.ctypes.data)
    return out


def draw_word(seed: int, stream: int, offset: int, index: int) -> int:
    return int(lib().orc_draw_word(seed, stream, offset, index))


def exp1_from_word(x: int) -> float:
    return float(lib().orc_exp1_from_word(x))


def icdf_uniform(seed: int, stream: int, offset: int) -> float:
    """The row's uniform for inverse-CDF selection."""
    return float(lib().orc_icdf_uniform(seed, stream, offset))


def exp1_draws(seed: int, stream: int, offset: int, n: int) -> np.ndarray:
    """Exp(1) variates the oracle uses for vocabulary entries 0..n-1 of a row."""
    out = np.empty(n, dtype=np.float64)
    lib().orc_fill_exp1(seed, stream, offset, n, out.ctypes.data)
    return out


def select_path(temperature, top_k=None, top_p=None, min_p=None, deterministic=False):
    """Batch predicate; returns a path name, raises ValueError on an empty batch."""
    t = _arr(temperature, np.float32)
    n = 0 if t is None else t.shape[0]
    k = _arr(top_k, np.int32, n)
    p = _arr(top_p, np.float32, n)
    mp = _arr(min_p, np.float32, n)
    out = ctypes.c_int32(-1)
    rc = lib().orc_select_path(n, _ptr(t), _ptr(k), _ptr(p), _ptr(mp), int(deterministic), ctypes.addressof(out))
    if rc != 0:
        raise ValueError("a batch needs at least one row")
    return PATH_NAMES[out.value]


def do_penalties(repetition=None, presence=None, frequency=None, n=None):
    arrs = [_arr(x, np.float32) for x in (repetition, presence, frequency)]
    if n is None:
        n = next((a.shape[0] for a in arrs if a is not None), 0)
    return bool(lib().orc_do_penalties(n, *[_ptr(a) for a in arrs]))


def normalized_top_k(temperature: float, top_k: int) -> int:
    return int(lib().orc_normalized_top_k(temperature, top_k))


def _make_args(logits, *, dtype="f32", vocab=None, temperature=None, top_p=None, top_k=None, min_p=None,
               repetition_penalty=None, presence_penalty=None, frequency_penalty=None,
               history_ids=None, history_start=None, history_len=None,
               seed=0, offset=0, row_seed=None, row_offset=None, row_stream=None, deterministic=False,
               want_probs=True, want_logprobs=True, top_logprobs=0, n_threads=1,
               vocab_mask=None, bias_ids=None, bias_vals=None, bias_start=None, bias_len=None,
               stop_ids=None, stop_start=None, stop_len=None, min_tokens=None, output_len=None,
               logprob_mode="processed", inverse_cdf=False):
    """The oracle's argument block for host arrays, the output arrays it
    writes, and the converted inputs it points at (kept alive by the caller)."""
    if dtype not in ("f32", "bf16"):
        raise ValueError("dtype must be 'f32' or 'bf16'")
    L = np.ascontiguousarray(logits, dtype=np.uint16 if dtype == "bf16" else np.float32)
    if L.ndim != 2:
        raise ValueError("logits must be 2-D")
    n, stride = L.shape
    V = stride if vocab is None else int(vocab)
    T = _arr(temperature, np.float32, n)
    P = _arr(top_p, np.float32, n)
    K = _arr(top_k, np.int32, n)
    MP = _arr(min_p, np.float32, n)
    RP = _arr(repetition_penalty, np.float32, n)
    PP = _arr(presence_penalty, np.float32, n)
    FP = _arr(frequency_penalty, np.float32, n)
    H = _arr(history_ids, np.int32)
    HS = _arr(history_start, np.int64, n)
    HL = _arr(history_len, np.int32, n)
    RS = _arr(row_seed, np.uint64, n)
    RO = _arr(row_offset, np.uint64, n)
    RST = _arr(row_stream, np.uint32, n)
    M = None if vocab_mask is None else np.ascontiguousarray(vocab_mask, dtype=np.uint32)
    if M is not None and (M.ndim != 2 or M.shape[0] != n or M.shape[1] < (V + 31) // 32):
        raise ValueError("vocab_mask must be [n_rows, >= ceil(vocab / 32)] uint32")
    BI, BV = _arr(bias_ids, np.int32), _arr(bias_vals, np.float32)
    BS, BL = _arr(bias_start, np.int64, n), _arr(bias_len, np.int32, n)
    SI = _arr(stop_ids, np.int32)
    SS, SL = _arr(stop_start, np.int64, n), _arr(stop_len, np.int32, n)
    MT, OL = _arr(min_tokens, np.int32, n), _arr(output_len, np.int32, n)
    if logprob_mode not in LOGPROB_MODES:
        raise ValueError("logprob_mode must be one of %s" % sorted(LOGPROB_MODES))
    out = {
        "token_ids": np.full(n, -7, dtype=np.int32),
        "probs": np.zeros((n, V), dtype=np.float32) if want_probs else None,
        "logprobs": np.zeros((n, V), dtype=np.float32) if want_logprobs else None,
        "top_logprob_vals": np.zeros((n, top_logprobs), dtype=np.float32) if top_logprobs else None,
        "top_logprob_ids": np.zeros((n, top_logprobs), dtype=np.int32) if top_logprobs else None,
        "row_status": np.zeros(n, dtype=np.int32),
        "flags": np.zeros(n, dtype=np.int32),
        "gumbel_gap": np.zeros(n, dtype=np.float64),
        "topp_margin": np.zeros(n, dtype=np.float64),
        "kept": np.zeros(n, dtype=np.int32),
        "token_alt": np.full(n, -1, dtype=np.int32),
    }
    a = _Args()
    a.logits = L.ctypes.data
    a.dtype = 1 if dtype == "bf16" else 0
    a.n_rows, a.vocab, a.row_stride = n, V, stride
    a.temperature, a.top_p, a.min_p = _ptr(T), _ptr(P), _ptr(MP)
    a.repetition_penalty, a.presence_penalty, a.frequency_penalty = _ptr(RP), _ptr(PP), _ptr(FP)
    a.top_k = _ptr(K)
    a.history_ids, a.history_start, a.history_len = _ptr(H), _ptr(HS), _ptr(HL)
    a.seed, a.offset = int(seed) & (2**64 - 1), int(offset) & (2**64 - 1)
    a.row_seed, a.row_offset, a.row_stream = _ptr(RS), _ptr(RO), _ptr(RST)
    a.deterministic = int(bool(deterministic))
    a.n_threads = int(n_threads)
    a.token_ids = out["token_ids"].ctypes.data
    a.probs = _ptr(out["probs"])
    a.logprobs = _ptr(out["logprobs"])
    a.top_logprobs = int(top_logprobs)
    a.top_logprob_vals = _ptr(out["top_logprob_vals"])
    a.top_logprob_ids = _ptr(out["top_logprob_ids"])
    a.row_status = out["row_status"].ctypes.data
    a.diag_flags = out["flags"].ctypes.data
    a.diag_gumbel_gap = out["gumbel_gap"].ctypes.data
    a.diag_topp_margin = out["topp_margin"].ctypes.data
    a.diag_kept = out["kept"].ctypes.data
    a.diag_token_alt = out["token_alt"].ctypes.data
    a.vocab_mask = _ptr(M)
    a.mask_stride = 0 if M is None else M.shape[1]
    a.bias_ids, a.bias_vals, a.bias_start, a.bias_len = _ptr(BI), _ptr(BV), _ptr(BS), _ptr(BL)
    a.stop_ids, a.stop_start, a.stop_len = _ptr(SI), _ptr(SS), _ptr(SL)
    a.min_tokens, a.output_len = _ptr(MT), _ptr(OL)
    a.logprob_mode = LOGPROB_MODES[logprob_mode]
    a.inverse_cdf = int(bool(inverse_cdf))
    for ids, st, ln, what in ((BI, BS, BL, "bias"), (SI, SS, SL, "stop")):
        if ids is not None and st is not None and ln is not None:
            if np.any(st < 0) or np.any(st + ln > ids.shape[0]):
                raise ValueError(f"{what} span outside the id buffer")
    if BI is not None and BV is not None and BV.shape != BI.shape:
        raise ValueError("bias_vals must match bias_ids")
    if HS is not None and H is not None and HL is not None:
        if np.any(HS < 0) or np.any(HS + HL > H.shape[0]):
            raise ValueError("history span outside the id buffer")
    keep = (L, T, P, K, MP, RP, PP, FP, H, HS, HL, RS, RO, RST, M, BI, BV, BS, BL, SI, SS, SL, MT, OL)
    return a, out, keep


def step(logits, **kw):
    """Run the oracle on host arrays.

    ``logits`` is a 2-D array: float32, or uint16 holding bf16 bits when
    ``dtype == "bf16"``; its row stride is its second dimension unless
    ``vocab`` is smaller.  ``vocab_mask`` is a 2-D uint32 array of allowed
    bits (bit i & 31 of word i >> 5; its row stride is its second
    dimension).  Keyword arguments are those of the sampler step (see
    ``_make_args``).  Returns a dict of numpy outputs and diagnostics.
    """
    a, out, keep = _make_args(logits, **kw)
    rc = lib().orc_step(ctypes.byref(a))
    if rc != 0:
        raise RuntimeError(f"oracle step failed ({rc})")
    del keep
    return out


def row_alternatives(logits, row: int, **kw):
    """The kept sets (bool [V] arrays) row ``row`` allows: the oracle's own
    first, then, where the row is flagged, each set a rounding of its top-p
    crossing (one tie group earlier or later) or of its min-p boundary could
    give.  Unflagged rows allow one set."""
    a, out, keep = _make_args(logits, **kw)
    V = a.vocab
    sets = []
    which = 0
    while True:
        k = np.zeros(V, dtype=np.uint8)
        rc = lib().orc_row_alternative(ctypes.byref(a), int(row), which, k.ctypes.data)
        if rc == -1:
            break
        if rc < 0:
            raise RuntimeError(f"oracle row alternative failed ({rc})")
        if rc == 1 and not any(np.array_equal(k, s) for s in sets):
            sets.append(k.copy())
        which += 1
    del keep
    return [s.astype(bool) for s in sets]


def row_with_kept(logits, row: int, kept, **kw):
    """Row ``row``'s outputs when ``kept`` (bool [V]) is its kept set: a
    dict like ``step``'s, for that row alone (1-D arrays)."""
    a, out, keep = _make_args(logits, **kw)
    k = np.ascontiguousarray(np.asarray(kept, dtype=np.uint8))
    if k.shape != (a.vocab,):
        raise ValueError("kept must have one entry per vocabulary token")
    rc = lib().orc_row_with_kept(ctypes.byref(a), int(row), k.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"oracle row_with_kept failed ({rc})")
    del keep
    return {name: (None if v is None else v[row]) for name, v in out.items()}
