"""Speculative-decoding verify step on MI355X (gfx950): Python binding.

Thin ctypes wrapper over ``libspecverify.so`` (C ABI in include/spec_verify.h).
It only marshals arguments: device pointers of torch tensors, sizes read from
their shapes, and the current HIP stream.  Every step of the verify path runs
in the library's HIP kernels; if the library is missing, every call raises.

    spec_verify_logits(hidden, w_lmhead, logits)
    spec_accept_greedy(logits, draft_tokens, accepted_len, out_tokens, workspace, rows=None)
    spec_accept_sample(logits, draft_logits, draft_tokens, temperature, seeds,
                       accepted_len, out_tokens, workspace, rows=None, probs_at_draft=None)
    spec_accept_greedy_ragged(logits, draft_tokens, row_start, K_max, accepted_len, out_tokens, workspace,
                              rows=None)
    spec_accept_sample_ragged(logits, draft_logits, draft_tokens, row_start, K_max, temperature, seeds,
                              accepted_len, out_tokens, workspace, rows=None, probs_at_draft=None)
    spec_tree_accept_greedy(logits, parents, tokens, accepted_len, out_tokens, workspace, out_nodes=None,
                            rows=None)
    spec_ngram_propose(history, hist_start, max_len, max_ngram, n_drafts, drafts, draft_count, workspace,
                       row_start=None)
    spec_verify_step(hidden, w_lmhead, logits, accepted_len, out_tokens, workspace, draft_logits=None,
                     draft_tokens=None, temperature=1.0, seeds=None, greedy_rows=None, sampled_rows=None,
                     probs_at_draft=None)
    spec_verify_step_noalloc(hidden, w_lmhead, logits, accepted_len, out_tokens, draft_logits=None,
                             draft_tokens=None, temperature=1.0, seeds=None, greedy_rows=None, sampled_rows=None,
                             probs_at_draft=None)
    spec_verify_step_ragged(hidden, w_lmhead, logits, row_start, K_max, accepted_len, out_tokens, workspace,
                            draft_logits=None, draft_tokens=None, temperature=1.0, seeds=None, greedy_rows=None,
                            sampled_rows=None, probs_at_draft=None)
    spec_tree_verify_step(hidden, w_lmhead, logits, parents, tokens, accepted_len, out_tokens, workspace,
                          out_nodes=None, rows=None)
    spec_workspace_bytes(B, K, V), spec_ngram_workspace_bytes(B, max_len), spec_verify_step_workspace_bytes(B, K, V),
    spec_verify_step_ragged_workspace_bytes(B, K_max, V)
"""
from __future__ import annotations

import ctypes
import os
import re

__all__ = [
    "SpecVerifyError", "SPEC_OK", "SPEC_ERR_ARG", "SPEC_ERR_DTYPE", "SPEC_ERR_ALIGN",
    "SPEC_ERR_WORKSPACE", "SPEC_ERR_HIP", "SPEC_BF16", "SPEC_F32", "LIB_PATH", "HEADER_PATH",
    "load_library", "declared_symbols", "spec_verify_logits", "spec_accept_greedy",
    "spec_accept_sample", "spec_accept_greedy_ragged", "spec_accept_sample_ragged", "spec_tree_accept_greedy", "spec_ngram_propose", "spec_ngram_workspace_bytes",
    "spec_verify_step", "spec_verify_step_workspace_bytes", "spec_verify_step_noalloc", "spec_tree_verify_step",
    "spec_verify_step_ragged", "spec_verify_step_ragged_workspace_bytes",
    "spec_workspace_bytes", "spec_status_string", "spec_last_error_detail", "spec_set_poll_limit",
]

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; SPECVERIFY_LIBRARY names another build of the same
# sources (the host-sanitized copy the CPU tests load)
LIB_PATH = os.environ.get("SPECVERIFY_LIBRARY") or os.path.join(PKG_DIR, "libspecverify.so")
HEADER_PATH = os.path.join(os.path.dirname(PKG_DIR), "include", "spec_verify.h")

SPEC_OK, SPEC_ERR_ARG, SPEC_ERR_DTYPE, SPEC_ERR_ALIGN, SPEC_ERR_WORKSPACE, SPEC_ERR_HIP = range(6)
SPEC_BF16, SPEC_F32 = 0, 1

_c_void_p, _c_int, _c_size_t, _c_float = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float

_SIGNATURES = {
    "spec_verify_logits": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_void_p, _c_int, _c_int, _c_int, _c_int,
                                    _c_void_p]),
    "spec_accept_greedy": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_void_p,
                                    _c_void_p, _c_void_p, _c_size_t, _c_void_p]),
    "spec_accept_sample": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_float, _c_void_p, _c_void_p, _c_int, _c_int,
                                    _c_int, _c_int, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_size_t,
                                    _c_void_p]),
    "spec_accept_greedy_ragged": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_int, _c_void_p, _c_int, _c_int, _c_int,
                                           _c_int, _c_void_p, _c_void_p, _c_void_p, _c_size_t, _c_void_p]),
    "spec_accept_sample_ragged": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_float, _c_void_p,
                                           _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_void_p, _c_void_p,
                                           _c_void_p, _c_void_p, _c_size_t, _c_void_p]),
    "spec_tree_accept_greedy": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_int,
                                         _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_size_t, _c_void_p]),
    "spec_ngram_propose": (_c_int, [_c_void_p, ctypes.c_int64, _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_void_p,
                                    _c_void_p, _c_void_p, _c_void_p, _c_size_t, _c_void_p]),
    "spec_ngram_workspace_bytes": (_c_size_t, [_c_int, _c_int]),
    "spec_verify_step": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_void_p, _c_void_p, _c_float, _c_void_p, _c_void_p,
                                  _c_int, _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_void_p, _c_void_p,
                                  _c_void_p, _c_void_p, _c_void_p, _c_size_t, _c_void_p]),
    "spec_verify_step_workspace_bytes": (_c_size_t, [_c_int, _c_int, _c_int]),
    "spec_verify_step_ragged": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_void_p, _c_void_p, _c_void_p, _c_int,
                                         _c_float, _c_void_p, _c_void_p, _c_int, _c_void_p, _c_int, _c_int, _c_int,
                                         _c_int, _c_int, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                         _c_size_t, _c_void_p]),
    "spec_verify_step_ragged_workspace_bytes": (_c_size_t, [_c_int, _c_int, _c_int]),
    "spec_tree_verify_step": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_int,
                                       _c_int, _c_int, _c_int, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                       _c_size_t, _c_void_p]),
    "spec_verify_step_noalloc": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_void_p, _c_void_p, _c_float, _c_void_p,
                                          _c_void_p, _c_int, _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                          _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "spec_workspace_bytes": (_c_size_t, [_c_int, _c_int, _c_int]),
    "spec_status_string": (ctypes.c_char_p, [_c_int]),
    "spec_last_error_detail": (ctypes.c_char_p, []),
    "spec_set_poll_limit": (_c_int, [_c_int]),
}

_lib = None


class SpecVerifyError(RuntimeError):
    """A library call returned a status other than SPEC_OK."""

    def __init__(self, fn: str, status: int):
        self.status = status
        detail = ""
        if status == SPEC_ERR_HIP:
            detail = " (" + load_library().spec_last_error_detail().decode() + ")"
        super().__init__("%s: %s%s" % (fn, spec_status_string(status), detail))


def load_library(path: str = LIB_PATH):
    """Load libspecverify.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("%s is missing: build it with `python -m speculative_decoding_verification_02_amd.build` "
                           "(or __graft_entry__.build())" % path)
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def declared_symbols(header: str = HEADER_PATH) -> list[str]:
    """Names of the functions include/spec_verify.h declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_[a-z_]+)\s*\(", text)))


# ------------------------------------------------------------ marshalling --

def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("every tensor argument must be on the GPU (got one on %s)" % t.device)
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(fn: str, status: int):
    if status != SPEC_OK:
        raise SpecVerifyError(fn, status)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return SPEC_BF16
    if t.dtype == torch.float32:
        return SPEC_F32
    raise TypeError("hidden/w_lmhead must be bfloat16 or float32, got %s" % t.dtype)


_T = None   # torch, imported on first use (importing the package does not need it)


def _torch():
    global _T
    if _T is None:
        import torch
        _T = torch
    return _T


def _arg(t, name, dtypes, shape=None, optional=False):
    """A device tensor the library reads or writes through a bare pointer:
    the kernels trust its dtype and extent, so they are checked here (shape
    entries of None match any size; _ptr checks the device).  Returns t."""
    if t is None:
        if optional:
            return None
        raise ValueError("%s is required" % name)
    try:
        dt = t.dtype
    except AttributeError:
        raise TypeError("%s must be a torch.Tensor" % name) from None
    if dt is not dtypes and (type(dtypes) is not tuple or dt not in dtypes):
        want = dtypes if type(dtypes) is tuple else (dtypes,)
        raise TypeError("%s must be %s, got %s" % (name, " or ".join(str(d) for d in want), dt))
    if shape is not None:
        ts = t.shape
        ok = len(ts) == len(shape)
        if ok:
            for d, w in zip(ts, shape):
                if w is not None and d != w:
                    ok = False
                    break
        if not ok:
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(ts),
                                                                tuple("*" if w is None else w for w in shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


_DT = {}


def _dt(key):
    """Cached dtype (or dtype tuple) by name."""
    v = _DT.get(key)
    if v is None:
        torch = _torch()
        v = {"i32": torch.int32, "f32": torch.float32, "i64": torch.int64,
             "seed": (torch.int64, torch.uint64) if hasattr(torch, "uint64") else torch.int64,
             "ws": (torch.uint8, torch.int8, torch.int32, torch.int64, torch.float32)}[key]
        _DT[key] = v
    return v


def _i32():
    return _dt("i32")


def _f32():
    return _dt("f32")


def _seed_types():
    return _dt("seed")


def _ws(workspace):
    return _arg(workspace, "workspace", _dt("ws"))


def _rows(rows):
    if rows is None:
        return None, 0
    _arg(rows, "rows", _i32(), (None,))
    return rows, int(rows.numel())


def spec_workspace_bytes(B: int, K: int, V: int) -> int:
    return int(load_library().spec_workspace_bytes(B, K, V))


def spec_status_string(status: int) -> str:
    return load_library().spec_status_string(status).decode()


def spec_last_error_detail() -> str:
    return load_library().spec_last_error_detail().decode()


def spec_set_poll_limit(rounds: int) -> int:
    """Bound the chunk-sum wait of the one-launch accept + residual draw
    (negative: the library default); returns the previous bound."""
    return int(load_library().spec_set_poll_limit(int(rounds)))


def spec_verify_logits(hidden, w_lmhead, logits, stream=None) -> None:
    """logits[B, K+1, V] (fp32) = hidden[B, K+1, H] . w_lmhead[V, H]ᵀ."""
    B, P, H = hidden.shape
    V = w_lmhead.shape[0]
    if w_lmhead.dtype != hidden.dtype:
        raise TypeError("hidden and w_lmhead must share a dtype")
    if tuple(logits.shape) != (B, P, V) or w_lmhead.shape[1] != H:
        raise ValueError("shape mismatch: hidden %s, w_lmhead %s, logits %s"
                         % (tuple(hidden.shape), tuple(w_lmhead.shape), tuple(logits.shape)))
    _dtype_code(hidden)
    for t, n in ((hidden, "hidden"), (w_lmhead, "w_lmhead")):
        _arg(t, n, hidden.dtype)
    _arg(logits, "logits", _f32(), (B, P, V))
    lib = load_library()
    _check("spec_verify_logits",
           lib.spec_verify_logits(_ptr(hidden), _ptr(w_lmhead), _dtype_code(hidden), _ptr(logits),
                                  B, P - 1, V, H, _stream(stream)))


def spec_accept_greedy(logits, draft_tokens, accepted_len, out_tokens, workspace, rows=None, stream=None) -> None:
    """Greedy acceptance of the selected rows (all rows if ``rows`` is None)."""
    B, P, V = _arg(logits, "logits", _f32(), (None, None, None)).shape
    _arg(draft_tokens, "draft_tokens", _i32(), (B, P - 1), optional=P == 1)
    _arg(accepted_len, "accepted_len", _i32(), (B,))
    _arg(out_tokens, "out_tokens", _i32(), (B, P))
    _ws(workspace)
    rows_t, n_rows = _rows(rows)
    lib = load_library()
    _check("spec_accept_greedy",
           lib.spec_accept_greedy(_ptr(logits), _ptr(draft_tokens) if P > 1 else None, _ptr(rows_t), n_rows,
                                  B, P - 1, V, _ptr(accepted_len), _ptr(out_tokens), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)))


def spec_accept_sample(logits, draft_logits, draft_tokens, temperature, seeds, accepted_len, out_tokens, workspace,
                       rows=None, probs_at_draft=None, stream=None) -> None:
    """Speculative sampling of the selected rows (all rows if ``rows`` is None)."""
    B, P, V = _arg(logits, "logits", _f32(), (None, None, None)).shape
    _arg(draft_logits, "draft_logits", _f32(), (B, P - 1, V), optional=P == 1)
    _arg(draft_tokens, "draft_tokens", _i32(), (B, P - 1), optional=P == 1)
    _arg(seeds, "seeds", _seed_types(), (B,))
    _arg(accepted_len, "accepted_len", _i32(), (B,))
    _arg(out_tokens, "out_tokens", _i32(), (B, P))
    _arg(probs_at_draft, "probs_at_draft", _f32(), (B, P - 1, 2), optional=True)
    _ws(workspace)
    rows_t, n_rows = _rows(rows)
    lib = load_library()
    _check("spec_accept_sample",
           lib.spec_accept_sample(_ptr(logits), _ptr(draft_logits) if P > 1 else None,
                                  _ptr(draft_tokens) if P > 1 else None, float(temperature), _ptr(seeds),
                                  _ptr(rows_t), n_rows, B, P - 1, V, _ptr(accepted_len), _ptr(out_tokens),
                                  _ptr(probs_at_draft), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)))


def spec_accept_greedy_ragged(logits, draft_tokens, row_start, K_max, accepted_len, out_tokens, workspace, rows=None,
                              stream=None) -> None:
    """Greedy acceptance of a ragged batch: logits [R, V] packed by row_start [B+1]."""
    R, V = _arg(logits, "logits", _f32(), (None, None)).shape
    B = _arg(row_start, "row_start", _i32(), (None,)).numel() - 1
    _arg(draft_tokens, "draft_tokens", _i32(), (R - B,), optional=R <= B)
    _arg(accepted_len, "accepted_len", _i32(), (B,))
    _arg(out_tokens, "out_tokens", _i32(), (R,))
    _ws(workspace)
    rows_t, n_rows = _rows(rows)
    lib = load_library()
    _check("spec_accept_greedy_ragged",
           lib.spec_accept_greedy_ragged(_ptr(logits), _ptr(draft_tokens) if R > B else None, _ptr(row_start), R,
                                         _ptr(rows_t), n_rows, B, int(K_max), V, _ptr(accepted_len),
                                         _ptr(out_tokens), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _stream(stream)))


def spec_accept_sample_ragged(logits, draft_logits, draft_tokens, row_start, K_max, temperature, seeds, accepted_len,
                              out_tokens, workspace, rows=None, probs_at_draft=None, stream=None) -> None:
    """Speculative sampling of a ragged batch: logits [R, V], draft_logits [R-B, V]
    packed by row_start [B+1]."""
    R, V = _arg(logits, "logits", _f32(), (None, None)).shape
    B = _arg(row_start, "row_start", _i32(), (None,)).numel() - 1
    _arg(draft_logits, "draft_logits", _f32(), (R - B, V), optional=R <= B)
    _arg(draft_tokens, "draft_tokens", _i32(), (R - B,), optional=R <= B)
    _arg(seeds, "seeds", _seed_types(), (B,))
    _arg(accepted_len, "accepted_len", _i32(), (B,))
    _arg(out_tokens, "out_tokens", _i32(), (R,))
    _arg(probs_at_draft, "probs_at_draft", _f32(), (R - B, 2), optional=True)
    _ws(workspace)
    rows_t, n_rows = _rows(rows)
    lib = load_library()
    _check("spec_accept_sample_ragged",
           lib.spec_accept_sample_ragged(_ptr(logits), _ptr(draft_logits) if R > B else None,
                                         _ptr(draft_tokens) if R > B else None, _ptr(row_start), R,
                                         float(temperature), _ptr(seeds), _ptr(rows_t), n_rows, B, int(K_max), V,
                                         _ptr(accepted_len), _ptr(out_tokens), _ptr(probs_at_draft),
                                         _ptr(workspace), workspace.numel() * workspace.element_size(),
                                         _stream(stream)))


def spec_tree_accept_greedy(logits, parents, tokens, accepted_len, out_tokens, workspace, out_nodes=None, rows=None,
                            stream=None) -> None:
    """Greedy verification of draft trees: logits [B, N+1, V], parents and
    tokens [B, N+1] (entry 0 of each row is the root and is ignored)."""
    B, P, V = _arg(logits, "logits", _f32(), (None, None, None)).shape
    _arg(parents, "parents", _i32(), (B, P), optional=P == 1)
    _arg(tokens, "tokens", _i32(), (B, P), optional=P == 1)
    _arg(accepted_len, "accepted_len", _i32(), (B,))
    _arg(out_tokens, "out_tokens", _i32(), (B, P))
    _arg(out_nodes, "out_nodes", _i32(), (B, P), optional=True)
    _ws(workspace)
    rows_t, n_rows = _rows(rows)
    lib = load_library()
    _check("spec_tree_accept_greedy",
           lib.spec_tree_accept_greedy(_ptr(logits), _ptr(parents) if P > 1 else None,
                                       _ptr(tokens) if P > 1 else None, _ptr(rows_t), n_rows, B, P - 1, V,
                                       _ptr(accepted_len), _ptr(out_tokens), _ptr(out_nodes), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(stream)))


def spec_tree_verify_step(hidden, w_lmhead, logits, parents, tokens, accepted_len, out_tokens, workspace,
                          out_nodes=None, rows=None, stream=None) -> None:
    """LM head and greedy tree verification in one call: hidden [B, N+1, H],
    w_lmhead [V, H], logits [B, N+1, V]; the rest as in
    spec_tree_accept_greedy."""
    B, P, H = hidden.shape
    V = w_lmhead.shape[0]
    if w_lmhead.dtype != hidden.dtype or w_lmhead.shape[1] != H:
        raise ValueError("shape or dtype mismatch")
    _dtype_code(hidden)
    _arg(hidden, "hidden", hidden.dtype)
    _arg(w_lmhead, "w_lmhead", hidden.dtype)
    _arg(logits, "logits", _f32(), (B, P, V))
    _arg(parents, "parents", _i32(), (B, P), optional=P == 1)
    _arg(tokens, "tokens", _i32(), (B, P), optional=P == 1)
    _arg(accepted_len, "accepted_len", _i32(), (B,))
    _arg(out_tokens, "out_tokens", _i32(), (B, P))
    _arg(out_nodes, "out_nodes", _i32(), (B, P), optional=True)
    _ws(workspace)
    rows_t, n_rows = _rows(rows)
    lib = load_library()
    _check("spec_tree_verify_step",
           lib.spec_tree_verify_step(_ptr(hidden), _ptr(w_lmhead), _dtype_code(hidden),
                                     _ptr(parents) if P > 1 else None, _ptr(tokens) if P > 1 else None,
                                     _ptr(rows_t), n_rows, B, P - 1, V, H, _ptr(logits), _ptr(accepted_len),
                                     _ptr(out_tokens), _ptr(out_nodes), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(stream)))


def spec_ngram_workspace_bytes(B: int, max_len: int) -> int:
    return int(load_library().spec_ngram_workspace_bytes(B, max_len))


def spec_ngram_propose(history, hist_start, max_len, max_ngram, n_drafts, drafts, draft_count, workspace,
                       row_start=None, stream=None) -> None:
    """Prompt-lookup drafts: history int32 (packed), hist_start int64 [B+1];
    drafts [B, n_drafts] and draft_count [B] int32 (row_start [B+1] int32
    optional)."""
    _arg(history, "history", _i32(), (None,))
    B = _arg(hist_start, "hist_start", _dt("i64"), (None,)).numel() - 1
    # drafts[b, i] lives at b * n_drafts + i: with n_drafts = 0 nothing is written
    _arg(drafts, "drafts", _i32(), (B, int(n_drafts)) if n_drafts else None, optional=not n_drafts)
    _arg(draft_count, "draft_count", _i32(), (B,))
    _arg(row_start, "row_start", _i32(), (B + 1,), optional=True)
    _ws(workspace)
    lib = load_library()
    _check("spec_ngram_propose",
           lib.spec_ngram_propose(_ptr(history) if history.numel() else None, int(history.numel()),
                                  _ptr(hist_start), B, int(max_len),
                                  int(max_ngram), int(n_drafts), _ptr(drafts) if n_drafts else None,
                                  _ptr(draft_count), _ptr(row_start), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)))


def spec_verify_step_workspace_bytes(B: int, K: int, V: int) -> int:
    return int(load_library().spec_verify_step_workspace_bytes(B, K, V))


def _row_list(rows, B):
    """(pointer, n) for the fused step: None = none, "all" = every sequence,
    else an int32 device tensor."""
    if rows is None:
        return None, 0
    if isinstance(rows, str) and rows == "all":
        return None, B
    _arg(rows, "rows", _i32(), (None,))
    return rows, int(rows.numel())


def _step_args(hidden, w_lmhead, logits, accepted_len, out_tokens, draft_logits, draft_tokens, seeds, greedy_rows,
               sampled_rows, probs_at_draft):
    """Checks of the step's tensors; returns (B, P, V, H, greedy, n_greedy, sampled, n_sampled)."""
    B, P, H = hidden.shape
    V = w_lmhead.shape[0]
    if w_lmhead.dtype != hidden.dtype or tuple(logits.shape) != (B, P, V) or w_lmhead.shape[1] != H:
        raise ValueError("shape or dtype mismatch")
    _dtype_code(hidden)
    _arg(hidden, "hidden", hidden.dtype)
    _arg(w_lmhead, "w_lmhead", hidden.dtype)
    _arg(logits, "logits", _f32(), (B, P, V))
    sampled = sampled_rows is not None and (isinstance(sampled_rows, str) or sampled_rows.numel() > 0)
    _arg(draft_logits, "draft_logits", _f32(), (B, P - 1, V), optional=P == 1 or not sampled)
    _arg(draft_tokens, "draft_tokens", _i32(), (B, P - 1), optional=P == 1)
    _arg(seeds, "seeds", _seed_types(), (B,), optional=not sampled)
    _arg(accepted_len, "accepted_len", _i32(), (B,))
    _arg(out_tokens, "out_tokens", _i32(), (B, P))
    _arg(probs_at_draft, "probs_at_draft", _f32(), (B, P - 1, 2), optional=True)
    g, ng = _row_list(greedy_rows, B)
    sm, ns = _row_list(sampled_rows, B)
    return B, P, V, H, g, ng, sm, ns


def spec_verify_step(hidden, w_lmhead, logits, accepted_len, out_tokens, workspace, draft_logits=None,
                     draft_tokens=None, temperature=1.0, seeds=None, greedy_rows=None, sampled_rows=None,
                     probs_at_draft=None, stream=None) -> None:
    """The whole verify step: logits[B, K+1, V] = hidden . w_lmheadᵀ, then greedy
    acceptance of ``greedy_rows`` and speculative sampling of ``sampled_rows``
    (each None, "all", or an int32 device tensor of sequence indices)."""
    B, P, V, H, g, ng, sm, ns = _step_args(hidden, w_lmhead, logits, accepted_len, out_tokens, draft_logits,
                                           draft_tokens, seeds, greedy_rows, sampled_rows, probs_at_draft)
    _ws(workspace)
    lib = load_library()
    _check("spec_verify_step",
           lib.spec_verify_step(_ptr(hidden), _ptr(w_lmhead), _dtype_code(hidden),
                                _ptr(draft_logits) if P > 1 else None, _ptr(draft_tokens) if P > 1 else None,
                                float(temperature), _ptr(seeds), _ptr(g), ng, _ptr(sm), ns, B, P - 1, V, H,
                                _ptr(logits), _ptr(accepted_len), _ptr(out_tokens), _ptr(probs_at_draft),
                                _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def spec_verify_step_ragged_workspace_bytes(B: int, K_max: int, V: int) -> int:
    return int(load_library().spec_verify_step_ragged_workspace_bytes(B, K_max, V))


def spec_verify_step_ragged(hidden, w_lmhead, logits, row_start, K_max, accepted_len, out_tokens, workspace,
                            draft_logits=None, draft_tokens=None, temperature=1.0, seeds=None, greedy_rows=None,
                            sampled_rows=None, probs_at_draft=None, stream=None) -> None:
    """The whole verify step of a ragged batch: hidden [R, H] packed by
    row_start [B+1], logits [R, V] = hidden . w_lmheadᵀ, then the two rules
    over ``greedy_rows`` / ``sampled_rows`` as in spec_verify_step; the
    draft and output tensors as in spec_accept_sample_ragged."""
    R, H = hidden.shape
    V = w_lmhead.shape[0]
    if w_lmhead.dtype != hidden.dtype or w_lmhead.shape[1] != H:
        raise ValueError("shape or dtype mismatch")
    _dtype_code(hidden)
    _arg(hidden, "hidden", hidden.dtype)
    _arg(w_lmhead, "w_lmhead", hidden.dtype)
    _arg(logits, "logits", _f32(), (R, V))
    B = _arg(row_start, "row_start", _i32(), (None,)).numel() - 1
    sampled = sampled_rows is not None and (isinstance(sampled_rows, str) or sampled_rows.numel() > 0)
    _arg(draft_logits, "draft_logits", _f32(), (R - B, V), optional=R <= B or not sampled)
    _arg(draft_tokens, "draft_tokens", _i32(), (R - B,), optional=R <= B)
    _arg(seeds, "seeds", _seed_types(), (B,), optional=not sampled)
    _arg(accepted_len, "accepted_len", _i32(), (B,))
    _arg(out_tokens, "out_tokens", _i32(), (R,))
    _arg(probs_at_draft, "probs_at_draft", _f32(), (R - B, 2), optional=True)
    g, ng = _row_list(greedy_rows, B)
    sm, ns = _row_list(sampled_rows, B)
    _ws(workspace)
    lib = load_library()
    _check("spec_verify_step_ragged",
           lib.spec_verify_step_ragged(_ptr(hidden), _ptr(w_lmhead), _dtype_code(hidden),
                                       _ptr(draft_logits) if R > B else None, _ptr(draft_tokens) if R > B else None,
                                       _ptr(row_start), R, float(temperature), _ptr(seeds), _ptr(g), ng, _ptr(sm), ns,
                                       B, int(K_max), V, H, _ptr(logits), _ptr(accepted_len), _ptr(out_tokens),
                                       _ptr(probs_at_draft), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(stream)))


def spec_verify_step_noalloc(hidden, w_lmhead, logits, accepted_len, out_tokens, draft_logits=None,
                             draft_tokens=None, temperature=1.0, seeds=None, greedy_rows=None, sampled_rows=None,
                             probs_at_draft=None, stream=None) -> None:
    """spec_verify_step without a workspace: the library's own per-GPU
    scratch (64 MiB) takes its place.  Calls that may overlap on one GPU race
    on that scratch."""
    B, P, V, H, g, ng, sm, ns = _step_args(hidden, w_lmhead, logits, accepted_len, out_tokens, draft_logits,
                                           draft_tokens, seeds, greedy_rows, sampled_rows, probs_at_draft)
    lib = load_library()
    _check("spec_verify_step_noalloc",
           lib.spec_verify_step_noalloc(_ptr(hidden), _ptr(w_lmhead), _dtype_code(hidden),
                                        _ptr(draft_logits) if P > 1 else None, _ptr(draft_tokens) if P > 1 else None,
                                        float(temperature), _ptr(seeds), _ptr(g), ng, _ptr(sm), ns, B, P - 1, V, H,
                                        _ptr(logits), _ptr(accepted_len), _ptr(out_tokens), _ptr(probs_at_draft),
                                        _stream(stream)))
