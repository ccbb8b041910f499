"""ctypes binding of libspecverify.so (declared in include/specverify.h).

Argument marshalling only: tensors are checked for device, dtype, contiguity and shape,
their device pointers and torch's current HIP stream are handed to the C ABI, and a non-OK
status becomes ``SpecVerifyError``.  Every step of the verify path runs in the library's
HIP kernels; there is no fallback, and a missing library raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

# mirrors include/specverify.h
SV_MAX_S = 64
SV_MAX_NGRAM = 8
SV_BLOCK = 32
STATE_WORDS = 80
STATE_LEN, STATE_J, STATE_NVALID, STATE_NUSED, STATE_FLAGS, STATE_ROUNDS, STATE_SUMJ, STATE_HIST = 0, 1, 2, 3, 4, 5, 6, 8
STATE_GATE_AFTER, STATE_ZERO_RUN, STATE_GATED = 72, 73, 74
FLAG_CAPACITY, FLAG_TOKEN, FLAG_ARGMAX = 1, 2, 4
STATUS = {0: "SV_OK", 1: "SV_ERR_NULL", 2: "SV_ERR_SHAPE", 3: "SV_ERR_ALIGN", 4: "SV_ERR_WORKSPACE",
          5: "SV_ERR_CAPACITY", 6: "SV_ERR_HIP", 7: "SV_ERR_DEVICE"}

EXPORTS = (
    "specverify_propose", "specverify_verify_workspace_bytes", "specverify_verify", "specverify_round",
    "specverify_round_noalloc",
    "specverify_accept", "specverify_gather_window", "specverify_gather_positions", "specverify_generate", "specverify_verify_q4b32",
    "specverify_round_q4b32", "specverify_sample_workspace_bytes", "specverify_verify_sample",
    "specverify_accept_sample", "specverify_round_sample", "specverify_propose_tree", "specverify_accept_tree",
    "specverify_round_tree", "specverify_generate_sample", "specverify_generate_tree",
    "specverify_rmsnorm", "specverify_stack_workspace_bytes", "specverify_gateup_silu_q8b32",
    "specverify_linear_q8b32", "specverify_linear_residual_rmsnorm_q8b32",
    "specverify_stack_forward_workspace_bytes", "specverify_stack", "specverify_set_tuning", "specverify_profile_next_matmul", "specverify_status_string", "specverify_last_error",
)

_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


def load():
    """Load the library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing; build it with `python -m weight_bound_verify_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "specverify_propose": (_I, [_P, _I, _P, _I, _I, _P, _P]),
        "specverify_verify_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I]),
        "specverify_verify": (_I, [_P, _P, _I, _I, _P, _I, _P, _P, _P, ctypes.c_size_t, _P]),
        "specverify_round": (_I, [_P, _P, _I, _I, _P, _I, _P, _P, _I, _P, _I, _P, _P, _P, _P, ctypes.c_size_t, _P]),
        "specverify_round_noalloc": (_I, [_P, _P, _I, _I, _P, _I, _P, _P, _I, _P, _I, _P, _P, _P, _P]),
        "specverify_accept": (_I, [_P, _P, _I, _P, _I, _P, _P]),
        "specverify_gather_window": (_I, [_P, _I, _P, _P, _I, _P, _I, _I, _P, _P]),
        "specverify_gather_positions": (_I, [_P, _I, _P, _I, _I, _I, _P, _P]),
        "specverify_verify_q4b32": (_I, [_P, _P, _I, _I, _P, _I, _P, _P, _P, ctypes.c_size_t, _P]),
        "specverify_round_q4b32": (_I, [_P, _P, _I, _I, _P, _I, _P, _P, _I, _P, _I, _P, _P, _P, _P, ctypes.c_size_t,
                                        _P]),
        "specverify_sample_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I]),
        "specverify_verify_sample": (_I, [_P, _P, _I, _I, _P, _I, _P, ctypes.c_float, ctypes.c_uint64, _P, _P, _P,
                                          _P, _P, _P, ctypes.c_size_t, _P]),
        "specverify_accept_sample": (_I, [_P, _P, _P, _P, _I, _I, ctypes.c_uint64, _P, _I, _P, _P]),
        "specverify_round_sample": (_I, [_P, _P, _I, _I, _P, _I, _P, ctypes.c_float, ctypes.c_uint64, _P, _I, _P,
                                         _I, _P, _P, _P, _P, ctypes.c_size_t, _P]),
        "specverify_propose_tree": (_I, [_P, _I, _P, _I, _I, _I, _I, _P, _P, _P]),
        "specverify_accept_tree": (_I, [_P, _P, _P, _I, _P, _I, _P, _P]),
        "specverify_round_tree": (_I, [_P, _P, _I, _I, _P, _I, _P, _P, _P, _I, _P, _I, _I, _I, _P, _P, _P, _P, _P,
                                       ctypes.c_size_t, _P]),
        "specverify_generate": (_I, [_P, _P, _I, _I, _P, _I, _I, _P, _I, _P, _I, _P, _P, _P, _P, ctypes.c_size_t,
                                     _P]),
        "specverify_generate_sample": (_I, [_P, _P, _I, _I, _P, _I, _I, ctypes.c_float, ctypes.c_uint64, _P, _I, _P,
                                            _I, _P, _P, _P, ctypes.c_size_t, _P]),
        "specverify_generate_tree": (_I, [_P, _P, _I, _I, _P, _I, _I, _P, _I, _P, _I, _I, _I, _P, _P, _P, _P, _P,
                                          ctypes.c_size_t, _P]),
        "specverify_rmsnorm": (_I, [_P, _I, _I, ctypes.c_float, _P, _P]),
        "specverify_stack_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
        "specverify_gateup_silu_q8b32": (_I, [_P, _P, _P, _P, _I, _I, _P, _I, _P, _P, ctypes.c_size_t, _P]),
        "specverify_linear_q8b32": (_I, [_P, _P, _I, _I, _P, _I, _P, _P, _P, ctypes.c_size_t, _P]),
        "specverify_linear_residual_rmsnorm_q8b32": (_I, [_P, _P, _I, _I, _P, _I, _P, _P, ctypes.c_float, _P, _P,
                                                          ctypes.c_size_t, _P]),
        "specverify_stack_forward_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I]),
        "specverify_stack": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _I, ctypes.c_float, _P, _P, _P,
                                  ctypes.c_size_t, _P]),
        "specverify_set_tuning": (None, [_I, _I, _I, _I, _I]),
        "specverify_profile_next_matmul": (_I, [_P, _P]),
        "specverify_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "specverify_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        detail = load().specverify_last_error().decode(errors="replace")
        raise SpecVerifyError(status, detail)


def _ptr(t, dtype, name, numel=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def new_state(device="cuda") -> torch.Tensor:
    return torch.zeros(STATE_WORDS, dtype=torch.int32, device=device)


def verify_workspace_bytes(V: int, H: int, S: int) -> int:
    return int(load().specverify_verify_workspace_bytes(V, H, S))


def stack_workspace_bytes(N: int, K: int, S: int, gateup: bool) -> int:
    return int(load().specverify_stack_workspace_bytes(N, K, S, int(gateup)))


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """Device scratch of at least ``nbytes`` (no initialisation needed)."""
    return torch.empty(max(16, nbytes), dtype=torch.uint8, device=device)


def set_tuning(waves_per_group: int = 0, max_groups: int = 0, depth: int = 0, head_kernel: int = 0,
               split: int = 0) -> None:
    load().specverify_set_tuning(int(waves_per_group), int(max_groups), int(depth), int(head_kernel), int(split))


def profile_next_matmul(before, after, stream=None) -> None:
    """Record two torch.cuda.Events around the next matmul kernel this thread launches."""
    if stream is None:
        stream = torch.cuda.current_stream()
    for ev in (before, after):
        if not ev.cuda_event:           # torch creates its events on first record
            ev.record(stream)
    _check(load().specverify_profile_next_matmul(ctypes.c_void_p(before.cuda_event),
                                                 ctypes.c_void_p(after.cuda_event)))


def propose(tokens, state, drafts, ngram_max: int = 3, stream=None) -> None:
    """n-gram drafts of ``tokens[:state[0]]`` into ``drafts`` (int32 [K])."""
    _check(load().specverify_propose(_ptr(tokens, torch.int32, "tokens"), tokens.numel(),
                                     _ptr(state, torch.int32, "state", STATE_WORDS), int(ngram_max),
                                     drafts.numel(), _ptr(drafts, torch.int32, "drafts"), _stream(stream)))


def verify(wq, wscale, hidden, argmax, ws, logits=None, stream=None) -> None:
    """argmax[s] of the q8b32 head over ``hidden`` rows; optional fp32 logits [S, V]."""
    V, H = wq.shape
    S = hidden.shape[0]
    if hidden.shape[1] != H or tuple(wscale.shape) != (V, H // SV_BLOCK):
        raise ValueError("shape mismatch between wq, wscale and hidden")
    _check(load().specverify_verify(
        _ptr(wq, torch.int8, "wq"), _ptr(wscale, torch.float16, "wscale"), V, H,
        _ptr(hidden, torch.float16, "hidden"), S, _ptr(argmax, torch.int32, "argmax", S),
        _ptr(logits, torch.float32, "logits", S * V), _ptr(ws, torch.uint8, "workspace"), ws.numel(),
        _stream(stream)))


def round(wq, wscale, hidden, drafts_in, tokens, state, drafts_out, argmax, ws, ngram_max: int = 3, logits=None,
          stream=None) -> None:
    """verify(hidden) -> accept(argmax, drafts_in) -> propose(next drafts into drafts_out), fused."""
    V, H = wq.shape
    S = hidden.shape[0]
    K = S - 1
    if hidden.shape[1] != H or tuple(wscale.shape) != (V, H // SV_BLOCK) or drafts_in.numel() < K:
        raise ValueError("shape mismatch")
    _check(load().specverify_round(
        _ptr(wq, torch.int8, "wq"), _ptr(wscale, torch.float16, "wscale"), V, H,
        _ptr(hidden, torch.float16, "hidden"), K, _ptr(drafts_in, torch.int32, "drafts_in", K),
        _ptr(tokens, torch.int32, "tokens"), tokens.numel(), _ptr(state, torch.int32, "state", STATE_WORDS),
        int(ngram_max), _ptr(drafts_out, torch.int32, "drafts_out", K), _ptr(argmax, torch.int32, "argmax", S),
        _ptr(logits, torch.float32, "logits", S * V), _ptr(ws, torch.uint8, "workspace"), ws.numel(),
        _stream(stream)))


def round_noalloc(wq, wscale, hidden, drafts_in, tokens, state, drafts_out, argmax, ngram_max: int = 3, logits=None,
                  stream=None) -> None:
    """``round`` with the library's own static scratch instead of a workspace (allocates nothing)."""
    V, H = wq.shape
    S = hidden.shape[0]
    K = S - 1
    if hidden.shape[1] != H or tuple(wscale.shape) != (V, H // SV_BLOCK) or drafts_in.numel() < K:
        raise ValueError("shape mismatch")
    _check(load().specverify_round_noalloc(
        _ptr(wq, torch.int8, "wq"), _ptr(wscale, torch.float16, "wscale"), V, H,
        _ptr(hidden, torch.float16, "hidden"), K, _ptr(drafts_in, torch.int32, "drafts_in", K),
        _ptr(tokens, torch.int32, "tokens"), tokens.numel(), _ptr(state, torch.int32, "state", STATE_WORDS),
        int(ngram_max), _ptr(drafts_out, torch.int32, "drafts_out", K), _ptr(argmax, torch.int32, "argmax", S),
        _ptr(logits, torch.float32, "logits", S * V), _stream(stream)))


def verify_q4(wq4, wscale, hidden, argmax, ws, logits=None, stream=None) -> None:
    """argmax[s] of the int4 per-block-32 head (codes uint8 [V, H/2]); optional fp32 logits."""
    V, half = wq4.shape
    H = 2 * half
    S = hidden.shape[0]
    if hidden.shape[1] != H or tuple(wscale.shape) != (V, H // SV_BLOCK):
        raise ValueError("shape mismatch between wq4, wscale and hidden")
    _check(load().specverify_verify_q4b32(
        _ptr(wq4, torch.uint8, "wq4"), _ptr(wscale, torch.float16, "wscale"), V, H,
        _ptr(hidden, torch.float16, "hidden"), S, _ptr(argmax, torch.int32, "argmax", S),
        _ptr(logits, torch.float32, "logits", S * V), _ptr(ws, torch.uint8, "workspace"), ws.numel(),
        _stream(stream)))


def round_q4(wq4, wscale, hidden, drafts_in, tokens, state, drafts_out, argmax, ws, ngram_max: int = 3, logits=None,
             stream=None) -> None:
    """The fused round on the int4 head."""
    V, half = wq4.shape
    H = 2 * half
    S = hidden.shape[0]
    K = S - 1
    if hidden.shape[1] != H or tuple(wscale.shape) != (V, H // SV_BLOCK) or drafts_in.numel() < K:
        raise ValueError("shape mismatch")
    _check(load().specverify_round_q4b32(
        _ptr(wq4, torch.uint8, "wq4"), _ptr(wscale, torch.float16, "wscale"), V, H,
        _ptr(hidden, torch.float16, "hidden"), K, _ptr(drafts_in, torch.int32, "drafts_in", K),
        _ptr(tokens, torch.int32, "tokens"), tokens.numel(), _ptr(state, torch.int32, "state", STATE_WORDS),
        int(ngram_max), _ptr(drafts_out, torch.int32, "drafts_out", K), _ptr(argmax, torch.int32, "argmax", S),
        _ptr(logits, torch.float32, "logits", S * V), _ptr(ws, torch.uint8, "workspace"), ws.numel(),
        _stream(stream)))


def sample_workspace_bytes(V: int, H: int, S: int) -> int:
    return int(load().specverify_sample_workspace_bytes(V, H, S))


def _seed(seed: int) -> int:
    return int(seed) & ((1 << 64) - 1)


def verify_sample(wq, wscale, hidden, drafts, temperature: float, seed: int, state, sample, lse, zd, ws, logits=None,
                  stream=None) -> None:
    """Sampling verify of the window: per-row residual draws, log-normalisers of L / T and the
    scaled logits of the drafts (see specverify_verify_sample)."""
    V, H = wq.shape
    S = hidden.shape[0]
    if hidden.shape[1] != H or tuple(wscale.shape) != (V, H // SV_BLOCK):
        raise ValueError("shape mismatch between wq, wscale and hidden")
    _check(load().specverify_verify_sample(
        _ptr(wq, torch.int8, "wq"), _ptr(wscale, torch.float16, "wscale"), V, H,
        _ptr(hidden, torch.float16, "hidden"), S, _ptr(drafts, torch.int32, "drafts", S - 1) if S > 1 else None,
        float(temperature), _seed(seed), _ptr(state, torch.int32, "state", STATE_WORDS),
        _ptr(sample, torch.int32, "sample", S), _ptr(lse, torch.float32, "lse", S), _ptr(zd, torch.float32, "zd", S),
        _ptr(logits, torch.float32, "logits", S * V), _ptr(ws, torch.uint8, "workspace"), ws.numel(),
        _stream(stream)))


def accept_sample(sample, lse, zd, drafts, V: int, seed: int, tokens, state, stream=None) -> None:
    """Sampling accept from verify_sample's outputs; ``sample`` holds K+1 draws."""
    K = sample.numel() - 1
    _check(load().specverify_accept_sample(
        _ptr(sample, torch.int32, "sample"), _ptr(lse, torch.float32, "lse", K + 1),
        _ptr(zd, torch.float32, "zd", K + 1), _ptr(drafts, torch.int32, "drafts", K) if K > 0 else None, K, int(V),
        _seed(seed), _ptr(tokens, torch.int32, "tokens"), tokens.numel(),
        _ptr(state, torch.int32, "state", STATE_WORDS), _stream(stream)))


def round_sample(wq, wscale, hidden, drafts_in, temperature: float, seed: int, tokens, state, drafts_out, ws,
                 ngram_max: int = 3, sample=None, lse=None, stream=None) -> None:
    """verify_sample -> accept_sample -> propose, fused (see specverify_round_sample)."""
    V, H = wq.shape
    S = hidden.shape[0]
    K = S - 1
    if hidden.shape[1] != H or tuple(wscale.shape) != (V, H // SV_BLOCK) or drafts_in.numel() < K:
        raise ValueError("shape mismatch")
    _check(load().specverify_round_sample(
        _ptr(wq, torch.int8, "wq"), _ptr(wscale, torch.float16, "wscale"), V, H,
        _ptr(hidden, torch.float16, "hidden"), K, _ptr(drafts_in, torch.int32, "drafts_in", K), float(temperature),
        _seed(seed), _ptr(tokens, torch.int32, "tokens"), tokens.numel(),
        _ptr(state, torch.int32, "state", STATE_WORDS), int(ngram_max), _ptr(drafts_out, torch.int32, "drafts_out", K),
        _ptr(sample, torch.int32, "sample", S), _ptr(lse, torch.float32, "lse", S), _ptr(ws, torch.uint8, "workspace"),
        ws.numel(), _stream(stream)))


def propose_tree(tokens, state, parents, drafts, ngram_max: int = 3, branches: int = 2, depth: int = 4,
                 stream=None) -> None:
    """Tree drafts of ``tokens[:state[0]]``: K = drafts.numel() nodes (parents, tokens)."""
    K = drafts.numel()
    _check(load().specverify_propose_tree(_ptr(tokens, torch.int32, "tokens"), tokens.numel(),
                                          _ptr(state, torch.int32, "state", STATE_WORDS), int(ngram_max), K,
                                          int(branches), int(depth), _ptr(parents, torch.int32, "parents", K),
                                          _ptr(drafts, torch.int32, "drafts"), _stream(stream)))


def accept_tree(argmax, parents, drafts, tokens, state, stream=None) -> None:
    """The greedy walk down the tree; ``argmax`` holds K+1 ids."""
    K = argmax.numel() - 1
    _check(load().specverify_accept_tree(_ptr(argmax, torch.int32, "argmax"), _ptr(parents, torch.int32, "parents", K),
                                         _ptr(drafts, torch.int32, "drafts", K), K, _ptr(tokens, torch.int32, "tokens"),
                                         tokens.numel(), _ptr(state, torch.int32, "state", STATE_WORDS),
                                         _stream(stream)))


def round_tree(wq, wscale, hidden, parents_in, drafts_in, tokens, state, parents_out, drafts_out, argmax, ws,
               ngram_max: int = 3, branches: int = 2, depth: int = 4, logits=None, stream=None) -> None:
    """verify(hidden, S = K+1) -> accept_tree -> propose_tree, fused."""
    V, H = wq.shape
    S = hidden.shape[0]
    K = S - 1
    if hidden.shape[1] != H or tuple(wscale.shape) != (V, H // SV_BLOCK) or drafts_in.numel() < K:
        raise ValueError("shape mismatch")
    _check(load().specverify_round_tree(
        _ptr(wq, torch.int8, "wq"), _ptr(wscale, torch.float16, "wscale"), V, H,
        _ptr(hidden, torch.float16, "hidden"), K, _ptr(parents_in, torch.int32, "parents_in", K),
        _ptr(drafts_in, torch.int32, "drafts_in", K), _ptr(tokens, torch.int32, "tokens"), tokens.numel(),
        _ptr(state, torch.int32, "state", STATE_WORDS), int(ngram_max), int(branches), int(depth),
        _ptr(parents_out, torch.int32, "parents_out", K), _ptr(drafts_out, torch.int32, "drafts_out", K),
        _ptr(argmax, torch.int32, "argmax", S), _ptr(logits, torch.float32, "logits", S * V),
        _ptr(ws, torch.uint8, "workspace"), ws.numel(), _stream(stream)))


def accept(argmax, drafts, tokens, state, stream=None) -> None:
    """Commit the accepted drafts and the next anchor; ``argmax`` holds K+1 ids."""
    K = argmax.numel() - 1
    _check(load().specverify_accept(_ptr(argmax, torch.int32, "argmax"),
                                    _ptr(drafts, torch.int32, "drafts", K) if K > 0 else None, K,
                                    _ptr(tokens, torch.int32, "tokens"), tokens.numel(),
                                    _ptr(state, torch.int32, "state", STATE_WORDS), _stream(stream)))


def gather_window(tokens, state, drafts, table, window, stream=None) -> None:
    """window[0] = table[anchor], window[i] = table[drafts[i-1]] (pads read row 0)."""
    V, H = table.shape
    K = window.shape[0] - 1
    if window.shape[1] != H:
        raise ValueError("window and table widths differ")
    _check(load().specverify_gather_window(
        _ptr(tokens, torch.int32, "tokens"), tokens.numel(), _ptr(state, torch.int32, "state", STATE_WORDS),
        _ptr(drafts, torch.int32, "drafts", K) if K > 0 else None, K, _ptr(table, torch.float16, "table"), V, H,
        _ptr(window, torch.float16, "window"), _stream(stream)))


def gather_positions(state, cap: int, rows, window, stream=None) -> None:
    """window[i] = rows[state[0] - 1 + i] (a position-indexed stand-in model); ``cap`` is the
    token buffer's capacity."""
    S, H = window.shape
    if rows.shape[1] != H:
        raise ValueError("rows and window must have the same width")
    _check(load().specverify_gather_positions(_ptr(state, torch.int32, "state", STATE_WORDS), int(cap),
                                              _ptr(rows, torch.float16, "rows"), rows.shape[0], H, S - 1,
                                              _ptr(window, torch.float16, "window"), _stream(stream)))


def generate(wq, wscale, table, tokens, state, drafts, window, argmax, ws, rounds: int, ngram_max: int = 3,
             stream=None) -> None:
    """``rounds`` device-resident rounds: gather the window from ``table``, verify, accept, draft."""
    V, H = wq.shape
    K = drafts.numel()
    if tuple(table.shape) != (V, H) or tuple(window.shape) != (K + 1, H) or tuple(wscale.shape) != (V, H // SV_BLOCK):
        raise ValueError("shape mismatch")
    _check(load().specverify_generate(
        _ptr(wq, torch.int8, "wq"), _ptr(wscale, torch.float16, "wscale"), V, H, _ptr(table, torch.float16, "table"),
        K, int(rounds), _ptr(tokens, torch.int32, "tokens"), tokens.numel(),
        _ptr(state, torch.int32, "state", STATE_WORDS), int(ngram_max), _ptr(drafts, torch.int32, "drafts", K),
        _ptr(window, torch.float16, "window"), _ptr(argmax, torch.int32, "argmax", K + 1),
        _ptr(ws, torch.uint8, "workspace"), ws.numel(), _stream(stream)))


def generate_sample(wq, wscale, table, tokens, state, drafts, window, ws, rounds: int, temperature: float,
                    seed: int, ngram_max: int = 3, stream=None) -> None:
    """``rounds`` device-resident sampling rounds: gather the window, verify_sample, accept, draft."""
    V, H = wq.shape
    K = drafts.numel()
    if tuple(table.shape) != (V, H) or tuple(window.shape) != (K + 1, H) or tuple(wscale.shape) != (V, H // SV_BLOCK):
        raise ValueError("shape mismatch")
    _check(load().specverify_generate_sample(
        _ptr(wq, torch.int8, "wq"), _ptr(wscale, torch.float16, "wscale"), V, H, _ptr(table, torch.float16, "table"),
        K, int(rounds), float(temperature), _seed(seed), _ptr(tokens, torch.int32, "tokens"), tokens.numel(),
        _ptr(state, torch.int32, "state", STATE_WORDS), int(ngram_max), _ptr(drafts, torch.int32, "drafts", K),
        _ptr(window, torch.float16, "window"), _ptr(ws, torch.uint8, "workspace"), ws.numel(), _stream(stream)))


def generate_tree(wq, wscale, table, tokens, state, parents, drafts, window, argmax, ws, rounds: int,
                  ngram_max: int = 3, branches: int = 2, depth: int = 4, stream=None) -> None:
    """``rounds`` device-resident tree rounds: gather the node rows, verify, walk, draft the next tree."""
    V, H = wq.shape
    K = drafts.numel()
    if (tuple(table.shape) != (V, H) or tuple(window.shape) != (K + 1, H) or tuple(wscale.shape) != (V, H // SV_BLOCK)
            or parents.numel() != K):
        raise ValueError("shape mismatch")
    _check(load().specverify_generate_tree(
        _ptr(wq, torch.int8, "wq"), _ptr(wscale, torch.float16, "wscale"), V, H, _ptr(table, torch.float16, "table"),
        K, int(rounds), _ptr(tokens, torch.int32, "tokens"), tokens.numel(),
        _ptr(state, torch.int32, "state", STATE_WORDS), int(ngram_max), int(branches), int(depth),
        _ptr(parents, torch.int32, "parents", K), _ptr(drafts, torch.int32, "drafts", K),
        _ptr(window, torch.float16, "window"), _ptr(argmax, torch.int32, "argmax", K + 1),
        _ptr(ws, torch.uint8, "workspace"), ws.numel(), _stream(stream)))


def rmsnorm(x, y, eps: float = 1e-6, stream=None) -> None:
    S, H = x.shape
    _check(load().specverify_rmsnorm(_ptr(x, torch.float16, "x"), S, H, float(eps),
                                     _ptr(y, torch.float16, "y", S * H), _stream(stream)))


def gateup_silu(wg, sg, wu, su, x, m, ws=None, stream=None) -> None:
    """m = fp16(silu(x Wg^T) * (x Wu^T)); ``ws`` is needed when stack_workspace_bytes(...) > 0."""
    N, K = wg.shape
    S = x.shape[0]
    if tuple(wu.shape) != (N, K) or x.shape[1] != K:
        raise ValueError("shape mismatch")
    _check(load().specverify_gateup_silu_q8b32(
        _ptr(wg, torch.int8, "wg"), _ptr(sg, torch.float16, "sg"), _ptr(wu, torch.int8, "wu"),
        _ptr(su, torch.float16, "su"), N, K, _ptr(x, torch.float16, "x"), S, _ptr(m, torch.float16, "m", S * N),
        _ptr(ws, torch.uint8, "workspace"), 0 if ws is None else ws.numel(), _stream(stream)))


def linear(w, scale, x, y, residual=None, ws=None, stream=None) -> None:
    """y = fp16(x W^T [+ residual]); ``ws`` is needed when stack_workspace_bytes(...) > 0."""
    N, K = w.shape
    S = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("shape mismatch")
    _check(load().specverify_linear_q8b32(
        _ptr(w, torch.int8, "w"), _ptr(scale, torch.float16, "scale"), N, K, _ptr(x, torch.float16, "x"), S,
        _ptr(residual, torch.float16, "residual", S * N), _ptr(y, torch.float16, "y", S * N),
        _ptr(ws, torch.uint8, "workspace"), 0 if ws is None else ws.numel(), _stream(stream)))


def linear_residual_rmsnorm(w, scale, x, y, norm_out, residual=None, eps: float = 1e-6, ws=None,
                            stream=None) -> None:
    """y = fp16(x W^T [+ residual]) and norm_out = fp16(rmsnorm(y)) in one call."""
    N, K = w.shape
    S = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("shape mismatch")
    _check(load().specverify_linear_residual_rmsnorm_q8b32(
        _ptr(w, torch.int8, "w"), _ptr(scale, torch.float16, "scale"), N, K, _ptr(x, torch.float16, "x"), S,
        _ptr(residual, torch.float16, "residual", S * N), _ptr(y, torch.float16, "y", S * N), float(eps),
        _ptr(norm_out, torch.float16, "norm_out", S * N), _ptr(ws, torch.uint8, "workspace"),
        0 if ws is None else ws.numel(), _stream(stream)))


def stack_forward_workspace_bytes(H: int, F: int, S: int) -> int:
    return int(load().specverify_stack_forward_workspace_bytes(H, F, S))


def stack(wg, sg, wu, su, wd, sd, x, norm_out, ws, eps: float = 1e-6, x_layers=None, stream=None) -> None:
    """The dense stack: L x [rmsnorm -> gate/up SiLU*mul -> down + residual], then
    norm_out = rmsnorm(x).  wg/wu [L, F, H], wd [L, H, F] int8 with fp16 block scales; x [S, H]
    is updated in place unless ``x_layers`` [L, S, H] receives every block's output."""
    L, F, H = wg.shape
    S = x.shape[0]
    if (tuple(wu.shape) != (L, F, H) or tuple(wd.shape) != (L, H, F) or tuple(sg.shape) != (L, F, H // SV_BLOCK)
            or tuple(su.shape) != (L, F, H // SV_BLOCK) or tuple(sd.shape) != (L, H, F // SV_BLOCK)
            or tuple(x.shape) != (S, H) or tuple(norm_out.shape) != (S, H)):
        raise ValueError("shape mismatch")
    if x_layers is not None and tuple(x_layers.shape) != (L, S, H):
        raise ValueError("x_layers must be [L, S, H]")
    _check(load().specverify_stack(
        _ptr(wg, torch.int8, "wg"), _ptr(sg, torch.float16, "sg"), _ptr(wu, torch.int8, "wu"),
        _ptr(su, torch.float16, "su"), _ptr(wd, torch.int8, "wd"), _ptr(sd, torch.float16, "sd"), L, H, F,
        _ptr(x, torch.float16, "x"), S, float(eps), _ptr(x_layers, torch.float16, "x_layers"),
        _ptr(norm_out, torch.float16, "norm_out"), _ptr(ws, torch.uint8, "workspace"), ws.numel(), _stream(stream)))
