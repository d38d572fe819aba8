"""MI355X (gfx950) per-decode-step token sampler.

A thin ctypes binding over the C ABI in ``include/sampler.h`` (built into
``libdsts_sampler.so`` next to this file).  Every step of the sampling path
runs in the library's HIP kernels; this module only marshals arguments.
PyTorch provides device memory and the current stream.  There is no CPU
fallback: a missing library raises.

Pages the behaviour follows (titles):
  [A] "SGLang's +75% sampler speedup skips Qwen3 chat requests"
  [B] the SGLang 101 operations manual
  [C] "采样参数对解码开销的影响：temperature、top_p 与采样核路径"
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# DSTS_LIBRARY: the same library built elsewhere (the sanitizer test loads
# one whose host code carries address and UB checks)
LIB_PATH = os.environ.get("DSTS_LIBRARY") or os.path.join(_PKG, "libdsts_sampler.so")

SAMPLER_OK, SAMPLER_EINVAL, SAMPLER_ECAPACITY, SAMPLER_EHIP, SAMPLER_ENOTSUP = 0, -1, -2, -3, -4
STATUS_NAMES = {0: "OK", -1: "EINVAL", -2: "ECAPACITY", -3: "EHIP", -4: "ENOTSUP"}
PATH_GREEDY, PATH_GUMBEL, PATH_FILTERED, PATH_DETERMINISTIC = 0, 1, 2, 3
PATH_NAMES = {0: "greedy", 1: "gumbel", 2: "filtered", 3: "deterministic"}
DTYPE_F32, DTYPE_BF16 = 0, 1
FLAG_DETERMINISTIC = 1 << 0
FLAG_FORCE_FILTERED = 1 << 1
FLAG_COOPERATIVE_LAUNCH = 1 << 2
FLAG_INVERSE_CDF = 1 << 3
FLAG_FORCE_PATH_GREEDY = 1 << 4
FLAG_FORCE_PATH_GUMBEL = 1 << 5
FLAG_FORCE_STREAM = 1 << 6
FLAG_NO_STREAM = 1 << 7

# symbols the header declares
EXPORTS = ("sampler_create", "sampler_step", "sampler_step_graph", "sampler_select_path", "sampler_validate",
           "sampler_destroy", "sampler_last_error", "sampler_profile_start", "sampler_profile_stop",
           "sampler_set_wait_spin_limit", "sampler_step_noalloc", "sampler_noalloc_last_error",
           "sampler_phase_stamps")


class SamplerError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [
        ("max_rows", ctypes.c_int32),
        ("max_vocab", ctypes.c_int32),
        ("max_history_per_row", ctypes.c_int32),
        ("max_top_logprobs", ctypes.c_int32),
        ("device", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("max_bias_per_row", ctypes.c_int32),
        ("wait_spin_limit", ctypes.c_int32),
    ]


class StepArgs(ctypes.Structure):
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
        ("token_ids", ctypes.c_void_p),
        ("probs", ctypes.c_void_p),
        ("logprobs", ctypes.c_void_p),
        ("top_logprobs", ctypes.c_int32),
        ("top_logprob_vals", ctypes.c_void_p),
        ("top_logprob_ids", ctypes.c_void_p),
        ("row_status", ctypes.c_void_p),
        ("path_out", ctypes.c_void_p),
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
        ("kernel_out", ctypes.c_void_p),
    ]


LOGPROB_MODES = {"processed": 0, "temperature": 1, "raw": 2}


class DeviceParams(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in (
        "temperature", "top_p", "min_p", "repetition_penalty", "presence_penalty", "frequency_penalty", "top_k",
        "history_start", "history_len", "row_seed", "row_offset", "row_stream", "bias_start", "bias_len",
        "stop_start", "stop_len", "min_tokens", "output_len")]


# dtype of each device array of DeviceParams
DEVICE_PARAM_DTYPES = dict(
    temperature="float32", top_p="float32", min_p="float32", repetition_penalty="float32",
    presence_penalty="float32", frequency_penalty="float32", top_k="int32", history_start="int64",
    history_len="int32", row_seed="int64", row_offset="int64", row_stream="int32", bias_start="int64",
    bias_len="int32", stop_start="int64", stop_len="int32", min_tokens="int32", output_len="int32")


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with __graft_entry__.build() "
                          "or python decode_step_token_sampler_amd/build.py")
    L = ctypes.CDLL(path)
    L.sampler_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(ctypes.c_void_p)]
    L.sampler_create.restype = ctypes.c_int
    L.sampler_step.argtypes = [ctypes.c_void_p, ctypes.POINTER(StepArgs), ctypes.c_void_p]
    L.sampler_step.restype = ctypes.c_int
    L.sampler_step_graph.argtypes = [ctypes.c_void_p, ctypes.POINTER(StepArgs), ctypes.POINTER(DeviceParams),
                                     ctypes.c_void_p]
    L.sampler_step_graph.restype = ctypes.c_int
    L.sampler_select_path.argtypes = [ctypes.POINTER(StepArgs), ctypes.c_uint32, ctypes.POINTER(ctypes.c_int32)]
    L.sampler_select_path.restype = ctypes.c_int
    L.sampler_validate.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(StepArgs), ctypes.c_char_p, ctypes.c_int32]
    L.sampler_validate.restype = ctypes.c_int
    L.sampler_destroy.argtypes = [ctypes.c_void_p]
    L.sampler_destroy.restype = None
    L.sampler_profile_start.argtypes = [ctypes.c_void_p, ctypes.c_int32]
    L.sampler_profile_start.restype = ctypes.c_int
    L.sampler_profile_stop.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                       ctypes.POINTER(ctypes.c_int32)]
    L.sampler_profile_stop.restype = ctypes.c_int
    L.sampler_set_wait_spin_limit.argtypes = [ctypes.c_void_p, ctypes.c_int32]
    L.sampler_set_wait_spin_limit.restype = ctypes.c_int
    L.sampler_step_noalloc.argtypes = [ctypes.POINTER(StepArgs), ctypes.c_uint32, ctypes.c_int32, ctypes.c_void_p]
    L.sampler_step_noalloc.restype = ctypes.c_int
    L.sampler_noalloc_last_error.argtypes = []
    L.sampler_noalloc_last_error.restype = ctypes.c_char_p
    L.sampler_last_error.argtypes = [ctypes.c_void_p]
    L.sampler_last_error.restype = ctypes.c_char_p
    L.sampler_phase_stamps.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                       ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    L.sampler_phase_stamps.restype = ctypes.c_int
    _lib = L
    return L


def phase_stamps():
    """The phase stamps of the last launches on the current device (a library
    built with the `stamps` option), cleared after reading: (uint64 array
    [blocks, slots], clock rate in kHz).  Raises SamplerError elsewhere."""
    L = load_library()
    blocks, slots, khz = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    st = L.sampler_phase_stamps(None, 0, ctypes.byref(blocks), ctypes.byref(slots), None)
    out = np.zeros((blocks.value, slots.value), dtype=np.uint64)
    st = L.sampler_phase_stamps(out.ctypes.data, out.size, ctypes.byref(blocks), ctypes.byref(slots),
                                ctypes.byref(khz))
    if st != SAMPLER_OK:
        raise SamplerError(st, "phase stamps need a library built with the stamps option")
    return out, khz.value


def _host(a, dtype, n):
    """Host array of n entries (or None) kept alive by the caller."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor
        a = a.detach().cpu().numpy()
    out = np.ascontiguousarray(np.asarray(a, dtype=dtype))
    if out.ndim == 0:
        out = np.full(n, out, dtype=dtype)
    if out.shape != (n,):
        raise ValueError(f"expected {n} per-row values, got shape {out.shape}")
    return out


def _p(a):
    return None if a is None else a.ctypes.data


def _check_tensor(t, name, dtype, device, shape=None):
    """A device tensor the library reads or writes: CUDA, on the logits'
    device, of the given dtype, contiguous (and of the given shape)."""
    if not getattr(t, "is_cuda", False) or t.device != device:
        raise ValueError(f"{name} must be a CUDA tensor on {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _check_spans(name, numel, start, length):
    """Every span [start, start + length) of the rows lies inside a buffer of numel entries."""
    if start is None or length is None:
        return
    live = length > 0
    if np.any(start[live] < 0) or np.any(start[live] + length[live] > numel):
        raise ValueError(f"a span of {name} lies outside its {numel} entries")


class _Marshalled:
    """Fills StepArgs from Python values and keeps the host arrays alive."""

    def __init__(self, n_rows, vocab, temperature=None, top_p=None, top_k=None, min_p=None,
                 repetition_penalty=None, presence_penalty=None, frequency_penalty=None,
                 history_start=None, history_len=None, row_seed=None, row_offset=None, row_stream=None,
                 bias_start=None, bias_len=None, stop_start=None, stop_len=None, min_tokens=None,
                 output_len=None):
        n = int(n_rows)
        self.keep = dict(
            temperature=_host(temperature, np.float32, n), top_p=_host(top_p, np.float32, n),
            min_p=_host(min_p, np.float32, n), repetition_penalty=_host(repetition_penalty, np.float32, n),
            presence_penalty=_host(presence_penalty, np.float32, n),
            frequency_penalty=_host(frequency_penalty, np.float32, n), top_k=_host(top_k, np.int32, n),
            history_start=_host(history_start, np.int64, n), history_len=_host(history_len, np.int32, n),
            row_seed=_host(row_seed, np.uint64, n), row_offset=_host(row_offset, np.uint64, n),
            row_stream=_host(row_stream, np.uint32, n),
            bias_start=_host(bias_start, np.int64, n), bias_len=_host(bias_len, np.int32, n),
            stop_start=_host(stop_start, np.int64, n), stop_len=_host(stop_len, np.int32, n),
            min_tokens=_host(min_tokens, np.int32, n), output_len=_host(output_len, np.int32, n))
        a = StepArgs()
        a.n_rows = n
        a.vocab = int(vocab)
        for k, v in self.keep.items():
            setattr(a, k, _p(v))
        self.args = a


def select_path(temperature=None, top_k=None, top_p=None, min_p=None, *, n_rows=None, deterministic=False) -> str:
    """The batch predicate through the C ABI (host only; no GPU needed)."""
    L = load_library()
    if n_rows is None:
        n_rows = next((len(x) for x in (temperature, top_k, top_p, min_p) if x is not None), 0)
    m = _Marshalled(n_rows, 1, temperature=temperature, top_p=top_p, top_k=top_k, min_p=min_p)
    out = ctypes.c_int32(-1)
    st = L.sampler_select_path(ctypes.byref(m.args), FLAG_DETERMINISTIC if deterministic else 0, ctypes.byref(out))
    if st != SAMPLER_OK:
        raise SamplerError(st, "invalid batch for the predicate")
    return PATH_NAMES[out.value]


def validate(config: Config, args: StepArgs):
    """Host-side checks of a step against a config; returns (status, message)."""
    L = load_library()
    buf = ctypes.create_string_buffer(512)
    st = L.sampler_validate(ctypes.byref(config), ctypes.byref(args), buf, 512)
    return st, buf.value.decode()


def _prepare_step(logits, *, vocab: Optional[int] = None, temperature=None, top_p=None, top_k=None,
                  min_p=None, repetition_penalty=None, presence_penalty=None, frequency_penalty=None,
                  history_ids=None, history_start=None, history_len=None, seed: int = 0, offset: int = 0,
                  row_seed=None, row_offset=None, row_stream=None, want_probs: bool = False,
                  want_logprobs: bool = False, top_logprobs: int = 0, want_status: bool = True,
                  out: Optional[dict] = None, stream=None, vocab_mask=None, bias_ids=None, bias_vals=None,
                  bias_start=None, bias_len=None, stop_ids=None, stop_start=None, stop_len=None, min_tokens=None,
                  output_len=None, logprob_mode: str = "processed"):
    """Marshal one decode step (argument checks only, no arithmetic): returns
    the filled StepArgs, the output tensors, the path word, the host arrays
    to keep alive until the call returns, and the stream handle."""
    import torch
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be 2-D with unit column stride")
    if logits.dtype == torch.float32:
        dt = DTYPE_F32
    elif logits.dtype == torch.bfloat16:
        dt = DTYPE_BF16
    else:
        raise ValueError("logits must be float32 or bfloat16")
    n = logits.shape[0]
    V = logits.shape[1] if vocab is None else int(vocab)
    dev = logits.device
    if not logits.is_cuda:
        raise ValueError("logits must be a CUDA tensor")
    o = dict(out or {})
    # caller-supplied outputs: the kernel writes exactly these shapes
    for name, dtype, shape in (("token_ids", torch.int32, (n,)), ("probs", torch.float32, (n, V)),
                               ("logprobs", torch.float32, (n, V)), ("row_status", torch.int32, (n,)),
                               ("top_logprob_vals", torch.float32, (n, top_logprobs)),
                               ("top_logprob_ids", torch.int32, (n, top_logprobs))):
        if name in o:
            _check_tensor(o[name], f"out['{name}']", dtype, dev, shape)
    if "token_ids" not in o:
        o["token_ids"] = torch.empty(n, dtype=torch.int32, device=dev)
    if want_probs and "probs" not in o:
        o["probs"] = torch.empty(n, V, dtype=torch.float32, device=dev)
    if want_logprobs and "logprobs" not in o:
        o["logprobs"] = torch.empty(n, V, dtype=torch.float32, device=dev)
    if top_logprobs and "top_logprob_vals" not in o:
        o["top_logprob_vals"] = torch.empty(n, top_logprobs, dtype=torch.float32, device=dev)
        o["top_logprob_ids"] = torch.empty(n, top_logprobs, dtype=torch.int32, device=dev)
    if want_status and "row_status" not in o:
        o["row_status"] = torch.empty(n, dtype=torch.int32, device=dev)
    m = _Marshalled(n, V, temperature=temperature, top_p=top_p, top_k=top_k, min_p=min_p,
                    repetition_penalty=repetition_penalty, presence_penalty=presence_penalty,
                    frequency_penalty=frequency_penalty, history_start=history_start,
                    history_len=history_len, row_seed=row_seed, row_offset=row_offset, row_stream=row_stream,
                    bias_start=bias_start, bias_len=bias_len, stop_start=stop_start, stop_len=stop_len,
                    min_tokens=min_tokens, output_len=output_len)
    a = m.args
    k = m.keep
    # the device id buffers: dtype, device, and every row's span inside them
    if history_ids is not None:
        _check_tensor(history_ids, "history_ids", torch.int32, dev)
        _check_spans("history_ids", history_ids.numel(), k["history_start"], k["history_len"])
    if bias_ids is not None or bias_vals is not None:
        if bias_ids is None or bias_vals is None:
            raise ValueError("bias_ids and bias_vals go together")
        _check_tensor(bias_ids, "bias_ids", torch.int32, dev)
        _check_tensor(bias_vals, "bias_vals", torch.float32, dev, tuple(bias_ids.shape))
        _check_spans("bias_ids", bias_ids.numel(), k["bias_start"], k["bias_len"])
    if stop_ids is not None:
        _check_tensor(stop_ids, "stop_ids", torch.int32, dev)
        _check_spans("stop_ids", stop_ids.numel(), k["stop_start"], k["stop_len"])
    a.logits = logits.data_ptr()
    a.dtype = dt
    a.row_stride = logits.stride(0)
    a.history_ids = None if history_ids is None else history_ids.data_ptr()
    a.bias_ids = None if bias_ids is None else bias_ids.data_ptr()
    a.bias_vals = None if bias_vals is None else bias_vals.data_ptr()
    a.stop_ids = None if stop_ids is None else stop_ids.data_ptr()
    if logprob_mode not in LOGPROB_MODES:
        raise ValueError("logprob_mode must be one of %s" % sorted(LOGPROB_MODES))
    a.logprob_mode = LOGPROB_MODES[logprob_mode]
    if vocab_mask is not None:
        if vocab_mask.dim() != 2 or vocab_mask.stride(1) != 1 or vocab_mask.element_size() != 4:
            raise ValueError("vocab_mask must be a 2-D 32-bit tensor with unit column stride")
        if not vocab_mask.is_cuda or vocab_mask.device != dev:
            raise ValueError(f"vocab_mask must be a CUDA tensor on {dev}")
        if vocab_mask.shape[0] != n or vocab_mask.shape[1] < (V + 31) // 32:
            raise ValueError(f"vocab_mask must be [{n}, >= {(V + 31) // 32}] words")
        a.vocab_mask = vocab_mask.data_ptr()
        a.mask_stride = vocab_mask.stride(0)
    a.seed = int(seed) & (2**64 - 1)
    a.offset = int(offset) & (2**64 - 1)
    a.token_ids = o["token_ids"].data_ptr()
    a.probs = o["probs"].data_ptr() if "probs" in o else None
    a.logprobs = o["logprobs"].data_ptr() if "logprobs" in o else None
    a.top_logprobs = int(top_logprobs)
    a.top_logprob_vals = o["top_logprob_vals"].data_ptr() if top_logprobs else None
    a.top_logprob_ids = o["top_logprob_ids"].data_ptr() if top_logprobs else None
    a.row_status = o["row_status"].data_ptr() if "row_status" in o else None
    path = ctypes.c_int32(-1)
    a.path_out = ctypes.addressof(path)
    kern = ctypes.c_int32(0)
    a.kernel_out = ctypes.addressof(kern)
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else int(stream)
    return a, o, path, (m, path, kern), s



def step_noalloc(logits, *, flags: int = 0, **kw) -> dict:
    """One decode step through sampler_step_noalloc (no handle; the library's
    fixed scratch array on the logits' GPU).  Keywords as for Sampler.step;
    ``flags``: FLAG_DETERMINISTIC, FLAG_INVERSE_CDF and at most one FORCE
    flag."""
    L = load_library()
    a, o, path, keep, s = _prepare_step(logits, **kw)
    st = L.sampler_step_noalloc(ctypes.byref(a), int(flags), int(logits.device.index or 0), ctypes.c_void_p(s))
    if st != SAMPLER_OK:
        raise SamplerError(st, L.sampler_noalloc_last_error().decode())
    o["path"] = PATH_NAMES[path.value]
    del keep
    return o


class Sampler:
    """One handle (device workspace + pinned staging ring) on one GPU."""

    def __init__(self, max_rows: int, max_vocab: int, *, max_history_per_row: int = 4096,
                 max_top_logprobs: int = 32, device: int = 0, deterministic: bool = False,
                 force_filtered: bool = False, cooperative_launch: bool = False, max_bias_per_row: int = 0,
                 inverse_cdf: bool = False, wait_spin_limit: int = 0, force_path: Optional[str] = None,
                 stream_rows: Optional[str] = None):
        L = load_library()
        self._L = L
        cfg = Config(max_rows=max_rows, max_vocab=max_vocab, max_history_per_row=max_history_per_row,
                     max_top_logprobs=max_top_logprobs, device=device, max_bias_per_row=max_bias_per_row,
                     wait_spin_limit=wait_spin_limit,
                     flags=(FLAG_DETERMINISTIC if deterministic else 0) | (FLAG_FORCE_FILTERED if force_filtered else 0)
                           | (FLAG_COOPERATIVE_LAUNCH if cooperative_launch else 0)
                           | (FLAG_INVERSE_CDF if inverse_cdf else 0)
                           | {None: 0, "greedy": FLAG_FORCE_PATH_GREEDY, "gumbel": FLAG_FORCE_PATH_GUMBEL,
                              "filtered": FLAG_FORCE_FILTERED}[force_path]
                           | {None: 0, "force": FLAG_FORCE_STREAM, "off": FLAG_NO_STREAM}[stream_rows])
        self.config = cfg
        h = ctypes.c_void_p()
        st = L.sampler_create(ctypes.byref(cfg), ctypes.byref(h))
        if st != SAMPLER_OK:
            raise SamplerError(st, L.sampler_last_error(None).decode())
        self._h = h
        self.device = device

    def close(self):
        if getattr(self, "_h", None):
            self._L.sampler_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def last_error(self) -> str:
        return self._L.sampler_last_error(self._h).decode()

    def set_wait_spin_limit(self, limit: int):
        """Bound of the cross-workgroup waits of later steps (0: the default)."""
        st = self._L.sampler_set_wait_spin_limit(self._h, int(limit))
        if st != SAMPLER_OK:
            raise SamplerError(st, self.last_error())

    def profile_start(self, capacity: int):
        """Record kernel durations of the next `capacity` steps (HIP events)."""
        st = self._L.sampler_profile_start(self._h, int(capacity))
        if st != SAMPLER_OK:
            raise SamplerError(st, self.last_error())

    def profile_stop(self) -> np.ndarray:
        """Kernel durations (ms) of the recorded steps, in launch order."""
        cap = 1 << 20
        buf = np.zeros(cap, dtype=np.float32)
        n = ctypes.c_int32(0)
        st = self._L.sampler_profile_stop(self._h, buf.ctypes.data, cap, ctypes.byref(n))
        if st != SAMPLER_OK:
            raise SamplerError(st, self.last_error())
        return buf[:n.value].copy()

    def step_raw(self, args: StepArgs, stream: int = 0) -> int:
        """Enqueue with a filled StepArgs (pointers already set); returns the status."""
        return self._L.sampler_step(self._h, ctypes.byref(args), ctypes.c_void_p(stream))

    def step(self, logits, **kw) -> dict:
        """Enqueue one decode step on the current torch stream; returns the output tensors.

        ``logits``: a CUDA tensor [N, row_stride] of float32 or bfloat16 with unit
        column stride.  Per-row parameters: host sequences / numpy arrays.
        ``history_ids``, ``bias_ids``, ``bias_vals``, ``stop_ids``: CUDA tensors
        (int32 / float32); ``vocab_mask``: a CUDA int32 or uint32-bits tensor
        [N, words] with unit column stride.  Outputs are allocated with torch
        on the logits' device unless ``out`` supplies them (each is checked
        for dtype, device and shape).  Keywords: those of ``_prepare_step``.
        """
        a, o, path, keep, s = _prepare_step(logits, **kw)
        st = self._L.sampler_step(self._h, ctypes.byref(a), ctypes.c_void_p(s))
        if st != SAMPLER_OK:
            raise SamplerError(st, self.last_error())
        o["path"] = PATH_NAMES[path.value]
        o["kernel"] = {0: "row", 1: "stream", 2: "small", 3: "chunk"}[keep[2].value]
        del keep
        return o

    def step_graph(self, logits, params: dict, *, vocab: Optional[int] = None, history_ids=None, seed: int = 0,
                   offset: int = 0, out: dict, top_logprobs: int = 0, vocab_mask=None, bias_ids=None,
                   bias_vals=None, stop_ids=None, logprob_mode: str = "processed", stream=None) -> None:
        """Enqueue one step whose per-row parameters are CUDA tensors (``params``:
        names of DeviceParams -> tensors of DEVICE_PARAM_DTYPES, n_rows entries
        each; missing names take the defaults).  Outputs go to the tensors of
        ``out`` (token_ids required; probs, logprobs, top_logprob_vals /
        top_logprob_ids, row_status optional), so the call can be captured
        into a graph and replayed after the parameter tensors are updated in
        place."""
        import torch
        if logits.dim() != 2 or logits.stride(1) != 1:
            raise ValueError("logits must be 2-D with unit column stride")
        dt = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}.get(logits.dtype)
        if dt is None:
            raise ValueError("logits must be float32 or bfloat16")
        n = logits.shape[0]
        dp = DeviceParams()
        for name, t in params.items():
            if name not in DEVICE_PARAM_DTYPES:
                raise ValueError(f"unknown device parameter {name}")
            want = getattr(torch, DEVICE_PARAM_DTYPES[name])
            if t.dtype != want or t.dim() != 1 or t.shape[0] != n or not t.is_contiguous() or not t.is_cuda:
                raise ValueError(f"{name} must be a contiguous CUDA {want} tensor of {n} entries")
            setattr(dp, name, t.data_ptr())
        a = StepArgs()
        a.logits = logits.data_ptr()
        a.dtype = dt
        a.n_rows = n
        a.vocab = logits.shape[1] if vocab is None else int(vocab)
        a.row_stride = logits.stride(0)
        a.history_ids = None if history_ids is None else history_ids.data_ptr()
        a.bias_ids = None if bias_ids is None else bias_ids.data_ptr()
        a.bias_vals = None if bias_vals is None else bias_vals.data_ptr()
        a.stop_ids = None if stop_ids is None else stop_ids.data_ptr()
        if vocab_mask is not None:
            a.vocab_mask = vocab_mask.data_ptr()
            a.mask_stride = vocab_mask.stride(0)
        a.seed = int(seed) & (2**64 - 1)
        a.offset = int(offset) & (2**64 - 1)
        a.token_ids = out["token_ids"].data_ptr()
        a.probs = out["probs"].data_ptr() if "probs" in out else None
        a.logprobs = out["logprobs"].data_ptr() if "logprobs" in out else None
        a.top_logprobs = int(top_logprobs)
        a.top_logprob_vals = out["top_logprob_vals"].data_ptr() if top_logprobs else None
        a.top_logprob_ids = out["top_logprob_ids"].data_ptr() if top_logprobs else None
        a.row_status = out["row_status"].data_ptr() if "row_status" in out else None
        a.logprob_mode = LOGPROB_MODES[logprob_mode]
        s = torch.cuda.current_stream(logits.device).cuda_stream if stream is None else int(stream)
        st = self._L.sampler_step_graph(self._h, ctypes.byref(a), ctypes.byref(dp), ctypes.c_void_p(s))
        if st != SAMPLER_OK:
            raise SamplerError(st, self.last_error())
