"""C-ABI checks that need no GPU: the library loads, exports every function
include/spec_verify.h declares, sizes its workspace, and rejects bad
arguments on the host before anything is enqueued (these calls return before
the first HIP runtime call, so they run on a machine without a GPU)."""
import ctypes
import math
import os
import re

import pytest

import speculative_decoding_verification_02_amd as sv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
P = ctypes.c_void_p
A = P(0x10000)          # a 16-byte-aligned stand-in address (never dereferenced)
MIS = P(0x10004)        # misaligned stand-in


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sv.LIB_PATH):
        pytest.fail("libspecverify.so is not built: run __graft_entry__.build()")
    return sv.load_library()


def test_exports_every_declared_symbol(lib):
    names = sv.declared_symbols()
    assert set(names) == {"spec_verify_logits", "spec_accept_greedy", "spec_accept_sample",
                          "spec_accept_greedy_ragged", "spec_accept_sample_ragged", "spec_tree_accept_greedy",
                          "spec_ngram_propose", "spec_ngram_workspace_bytes",
                          "spec_verify_step", "spec_verify_step_workspace_bytes", "spec_verify_step_noalloc",
                          "spec_tree_verify_step", "spec_verify_step_ragged",
                          "spec_verify_step_ragged_workspace_bytes",
                          "spec_workspace_bytes", "spec_status_string", "spec_last_error_detail",
                          "spec_set_poll_limit"}
    for n in names:
        assert hasattr(lib, n), n


def test_poll_limit_setter(lib):
    default = sv.spec_set_poll_limit(5)
    assert default == 65536
    assert sv.spec_set_poll_limit(0) == 5
    assert sv.spec_set_poll_limit(-1) == 0
    assert sv.spec_set_poll_limit(-1) == default


def test_status_strings(lib):
    for code in range(6):
        assert sv.spec_status_string(code).startswith("SPEC_")
    assert "unknown" in sv.spec_status_string(99)
    assert sv.spec_last_error_detail() == ""


def test_workspace_bytes(lib):
    assert sv.spec_workspace_bytes(0, 1, 10) == 0
    assert sv.spec_workspace_bytes(1, 64, 10) == 0
    assert sv.spec_workspace_bytes(1, -1, 10) == 0
    assert sv.spec_workspace_bytes(1, 1, 0) == 0
    assert sv.spec_workspace_bytes(1, 1, 4096 * 1024 + 1) == 0
    a = sv.spec_workspace_bytes(1, 5, 128256)
    b = sv.spec_workspace_bytes(64, 4, 128256)
    c = sv.spec_workspace_bytes(256, 8, 152064)
    assert 0 < a < b < c
    assert a % 256 == 0 and c % 256 == 0
    assert sv.spec_workspace_bytes(1, 0, 1) > 0
    assert sv.spec_workspace_bytes(1, 63, 4096 * 1024) > 0


def test_verify_logits_validation(lib):
    f = lib.spec_verify_logits
    assert f(None, A, 0, A, 1, 1, 16, 8, None) == sv.SPEC_ERR_ARG
    assert f(A, None, 0, A, 1, 1, 16, 8, None) == sv.SPEC_ERR_ARG
    assert f(A, A, 0, None, 1, 1, 16, 8, None) == sv.SPEC_ERR_ARG
    assert f(A, A, 7, A, 1, 1, 16, 8, None) == sv.SPEC_ERR_DTYPE
    assert f(A, A, 0, A, 0, 1, 16, 8, None) == sv.SPEC_ERR_ARG     # B = 0
    assert f(A, A, 0, A, 1, 64, 16, 8, None) == sv.SPEC_ERR_ARG    # K > 63
    assert f(A, A, 0, A, 1, -1, 16, 8, None) == sv.SPEC_ERR_ARG
    assert f(A, A, 0, A, 1, 1, 0, 8, None) == sv.SPEC_ERR_ARG      # V = 0
    assert f(A, A, 0, A, 1, 1, 16, 12, None) == sv.SPEC_ERR_ARG    # H % 8
    assert f(A, A, 0, A, 1, 1, 16, 0, None) == sv.SPEC_ERR_ARG
    assert f(MIS, A, 0, A, 1, 1, 16, 8, None) == sv.SPEC_ERR_ALIGN
    assert f(A, MIS, 1, A, 1, 1, 16, 8, None) == sv.SPEC_ERR_ALIGN
    assert f(A, A, 0, MIS, 1, 1, 16, 8, None) == sv.SPEC_ERR_ALIGN


def _greedy(lib, logits=A, drafts=A, rows=None, n_rows=0, B=2, K=3, V=100, acc=A, out=A, ws=A, wsb=None):
    if wsb is None:
        wsb = sv.spec_workspace_bytes(B, K, V) if sv.spec_workspace_bytes(B, K, V) else 1 << 20
    return lib.spec_accept_greedy(logits, drafts, rows, n_rows, B, K, V, acc, out, ws, wsb, None)


def test_accept_greedy_validation(lib):
    need = sv.spec_workspace_bytes(2, 3, 100)
    assert _greedy(lib, logits=None) == sv.SPEC_ERR_ARG
    assert _greedy(lib, drafts=None) == sv.SPEC_ERR_ARG             # K > 0 needs drafts
    assert _greedy(lib, acc=None) == sv.SPEC_ERR_ARG
    assert _greedy(lib, out=None) == sv.SPEC_ERR_ARG
    assert _greedy(lib, B=0) == sv.SPEC_ERR_ARG
    assert _greedy(lib, K=64) == sv.SPEC_ERR_ARG
    assert _greedy(lib, V=0) == sv.SPEC_ERR_ARG
    assert _greedy(lib, rows=A, n_rows=3) == sv.SPEC_ERR_ARG        # n_rows > B
    assert _greedy(lib, rows=A, n_rows=-1) == sv.SPEC_ERR_ARG
    assert _greedy(lib, logits=MIS) == sv.SPEC_ERR_ALIGN
    assert _greedy(lib, ws=None) == sv.SPEC_ERR_WORKSPACE
    assert _greedy(lib, wsb=need - 1) == sv.SPEC_ERR_WORKSPACE
    assert _greedy(lib, ws=MIS) == sv.SPEC_ERR_ALIGN


def _sample(lib, T=1.0, seeds=A, dl=A, drafts=A, logits=A, K=3, B=2, V=100, wsb=None, rows=None, n_rows=0):
    if wsb is None:
        wsb = sv.spec_workspace_bytes(B, K, V) or (1 << 20)
    return lib.spec_accept_sample(logits, dl, drafts, T, seeds, rows, n_rows, B, K, V, A, A, None, A, wsb, None)


def test_accept_sample_validation(lib):
    assert _sample(lib, T=0.0) == sv.SPEC_ERR_ARG
    assert _sample(lib, T=-1.0) == sv.SPEC_ERR_ARG
    assert _sample(lib, T=math.nan) == sv.SPEC_ERR_ARG
    assert _sample(lib, T=math.inf) == sv.SPEC_ERR_ARG
    assert _sample(lib, seeds=None) == sv.SPEC_ERR_ARG
    assert _sample(lib, dl=None) == sv.SPEC_ERR_ARG                 # K > 0 needs draft logits
    assert _sample(lib, drafts=None) == sv.SPEC_ERR_ARG
    assert _sample(lib, dl=MIS) == sv.SPEC_ERR_ALIGN
    assert _sample(lib, logits=MIS) == sv.SPEC_ERR_ALIGN
    assert _sample(lib, wsb=16) == sv.SPEC_ERR_WORKSPACE
    assert _sample(lib, B=1, rows=A, n_rows=2) == sv.SPEC_ERR_ARG


def _greedy_ragged(lib, rs=A, total=5, B=2, K=3, V=100, drafts=A, rows=None, n_rows=0, wsb=None):
    if wsb is None:
        wsb = sv.spec_workspace_bytes(B, K, V) or (1 << 20)
    return lib.spec_accept_greedy_ragged(A, drafts, rs, total, rows, n_rows, B, K, V, A, A, A, wsb, None)


def _sample_ragged(lib, rs=A, total=5, B=2, K=3, V=100, dl=A, drafts=A, T=1.0, rows=None, n_rows=0):
    wsb = sv.spec_workspace_bytes(B, K, V) or (1 << 20)
    return lib.spec_accept_sample_ragged(A, dl, drafts, rs, total, T, A, rows, n_rows, B, K, V, A, A, None, A, wsb,
                                         None)


def test_ragged_validation(lib):
    for f in (_greedy_ragged, _sample_ragged):
        assert f(lib, rs=None) == sv.SPEC_ERR_ARG
        assert f(lib, rs=P(0x10002)) == sv.SPEC_ERR_ALIGN             # int32 offsets: 4-byte aligned
        assert f(lib, total=1) == sv.SPEC_ERR_ARG                     # fewer rows than sequences
        assert f(lib, total=9) == sv.SPEC_ERR_ARG                     # more than B*(K_max+1)
        assert f(lib, K=64, total=5) == sv.SPEC_ERR_ARG
        assert f(lib, drafts=None) == sv.SPEC_ERR_ARG                 # total > B: there are drafts
        assert f(lib, rows=A, n_rows=0) == sv.SPEC_OK                 # nothing selected: no-op
        assert f(lib, total=2, drafts=None, rows=A, n_rows=0) == sv.SPEC_OK   # no drafts at all
    assert _sample_ragged(lib, dl=None) == sv.SPEC_ERR_ARG
    assert _sample_ragged(lib, dl=MIS) == sv.SPEC_ERR_ALIGN
    assert _sample_ragged(lib, T=0.0) == sv.SPEC_ERR_ARG
    assert _greedy_ragged(lib, wsb=16) == sv.SPEC_ERR_WORKSPACE


def _tree(lib, par=A, tok=A, N=5, B=2, V=100, logits=A, rows=None, n_rows=0, wsb=None):
    if wsb is None:
        wsb = sv.spec_workspace_bytes(B, N, V) or (1 << 20)
    return lib.spec_tree_accept_greedy(logits, par, tok, rows, n_rows, B, N, V, A, A, None, A, wsb, None)


def test_tree_validation(lib):
    assert _tree(lib, par=None) == sv.SPEC_ERR_ARG
    assert _tree(lib, tok=None) == sv.SPEC_ERR_ARG
    assert _tree(lib, N=64) == sv.SPEC_ERR_ARG
    assert _tree(lib, logits=MIS) == sv.SPEC_ERR_ALIGN
    assert _tree(lib, wsb=16) == sv.SPEC_ERR_WORKSPACE
    assert _tree(lib, par=None, tok=None, N=0, rows=A, n_rows=0) == sv.SPEC_OK
    assert _tree(lib, rows=A, n_rows=0) == sv.SPEC_OK


def _ngram(lib, hist=A, hl=100, hs=A, B=2, max_len=100, g=3, k=5, drafts=A, count=A, ws=A, wsb=None):
    if wsb is None:
        wsb = sv.spec_ngram_workspace_bytes(B, max_len) or 256
    return lib.spec_ngram_propose(hist, hl, hs, B, max_len, g, k, drafts, count, None, ws, wsb, None)


def test_ngram_validation(lib):
    assert sv.spec_ngram_workspace_bytes(0, 10) == 0 and sv.spec_ngram_workspace_bytes(3, 100) == 256
    assert sv.spec_ngram_workspace_bytes(3, -1) == 0
    assert sv.spec_ngram_workspace_bytes(64, 4097) == 64 * 8         # 4096 end positions: one segment
    assert sv.spec_ngram_workspace_bytes(64, 4098) == 64 * 8 * 2
    assert sv.spec_ngram_workspace_bytes(64, 8194) == 64 * 8 * 3
    assert _ngram(lib, B=0) == sv.SPEC_ERR_ARG
    assert _ngram(lib, max_len=-1) == sv.SPEC_ERR_ARG
    assert _ngram(lib, g=0) == sv.SPEC_ERR_ARG
    assert _ngram(lib, g=17) == sv.SPEC_ERR_ARG
    assert _ngram(lib, k=64) == sv.SPEC_ERR_ARG
    assert _ngram(lib, k=-1) == sv.SPEC_ERR_ARG
    assert _ngram(lib, hist=None) == sv.SPEC_ERR_ARG
    assert _ngram(lib, hl=-1) == sv.SPEC_ERR_ARG                      # negative history length
    assert _ngram(lib, hist=None, hl=1) == sv.SPEC_ERR_ARG            # entries declared behind a null pointer
    assert _ngram(lib, hs=None) == sv.SPEC_ERR_ARG
    assert _ngram(lib, drafts=None) == sv.SPEC_ERR_ARG
    assert _ngram(lib, count=None) == sv.SPEC_ERR_ARG
    assert _ngram(lib, hs=P(0x10004)) == sv.SPEC_ERR_ALIGN
    assert _ngram(lib, ws=None) == sv.SPEC_ERR_WORKSPACE
    assert _ngram(lib, wsb=8) == sv.SPEC_ERR_WORKSPACE
    assert _ngram(lib, ws=P(0x10004)) == sv.SPEC_ERR_ALIGN


def _step(lib, hid=A, w=A, dt=0, dl=A, dtok=A, T=1.0, seeds=A, g=None, ng=0, sm=None, ns=2, B=2, K=3, V=100,
          H=64, logits=A, acc=A, out=A, ws=A, wsb=None):
    if wsb is None:
        wsb = sv.spec_verify_step_workspace_bytes(B, K, V) or (1 << 20)
    return lib.spec_verify_step(hid, w, dt, dl, dtok, T, seeds, g, ng, sm, ns, B, K, V, H, logits, acc, out, None,
                                ws, wsb, None)


def test_step_validation(lib):
    # M <= 16: one record per cooperative-kernel workgroup (at most 1024) for
    # each of the M target and B*K draft rows; M > 16: one per 256 vocabulary
    # entries for each target row
    assert sv.spec_verify_step_workspace_bytes(1, 5, 128256) == sv.spec_workspace_bytes(1, 5, 128256) + 11 * 1024 * 16
    a = sv.spec_verify_step_workspace_bytes(4, 5, 128256)
    assert a >= sv.spec_workspace_bytes(4, 5, 128256) + 24 * 501 * 16 and a % 256 == 0
    assert sv.spec_verify_step_workspace_bytes(1, 64, 100) == 0
    assert _step(lib, hid=None) == sv.SPEC_ERR_ARG
    assert _step(lib, logits=None) == sv.SPEC_ERR_ARG
    assert _step(lib, acc=None) == sv.SPEC_ERR_ARG
    assert _step(lib, dt=5) == sv.SPEC_ERR_DTYPE
    assert _step(lib, K=64) == sv.SPEC_ERR_ARG
    assert _step(lib, H=12) == sv.SPEC_ERR_ARG
    assert _step(lib, ns=1) == sv.SPEC_ERR_ARG             # NULL list: 0 or B only
    assert _step(lib, sm=A, ns=3) == sv.SPEC_ERR_ARG       # more than B
    assert _step(lib, g=A, ng=-1) == sv.SPEC_ERR_ARG
    assert _step(lib, dtok=None) == sv.SPEC_ERR_ARG
    assert _step(lib, dl=None) == sv.SPEC_ERR_ARG
    assert _step(lib, seeds=None) == sv.SPEC_ERR_ARG
    assert _step(lib, T=0.0) == sv.SPEC_ERR_ARG
    assert _step(lib, T=math.nan) == sv.SPEC_ERR_ARG
    assert _step(lib, dl=MIS) == sv.SPEC_ERR_ALIGN
    assert _step(lib, hid=MIS) == sv.SPEC_ERR_ALIGN
    assert _step(lib, wsb=16) == sv.SPEC_ERR_WORKSPACE
    assert _step(lib, ws=MIS) == sv.SPEC_ERR_ALIGN
    # greedy rows only: no seeds, draft logits or temperature needed
    assert _step(lib, ns=0, seeds=None, dl=None, T=0.0, g=A, ng=0, ws=None) == sv.SPEC_ERR_WORKSPACE


def _step_ragged(lib, hid=A, w=A, dt=0, dl=A, dtok=A, rs=A, total=5, T=1.0, seeds=A, g=None, ng=0, sm=None, ns=2,
                 B=2, K=3, V=100, H=64, logits=A, acc=A, out=A, ws=A, wsb=None):
    if wsb is None:
        wsb = sv.spec_verify_step_ragged_workspace_bytes(B, K, V) or (1 << 20)
    return lib.spec_verify_step_ragged(hid, w, dt, dl, dtok, rs, total, T, seeds, g, ng, sm, ns, B, K, V, H, logits,
                                       acc, out, None, ws, wsb, None)


def test_ragged_step_workspace_bytes(lib):
    """Any R in [B, B*(K_max+1)]: R <= 16 takes the cooperative kernel's
    records (at most 1024 per row) for R target and R - B draft rows, R > 16
    one record per 256 vocabulary entries of each target row."""
    base = sv.spec_workspace_bytes
    rec = 16                                                 # bytes per record
    # B = 1, K_max = 5: R <= 6, so 2*6 - 1 = 11 rows of cooperative records,
    # as in the dense step
    assert sv.spec_verify_step_ragged_workspace_bytes(1, 5, 128256) == sv.spec_verify_step_workspace_bytes(1, 5, 128256)
    # B = 4, K_max = 7: R up to 32, but R = 16 (cooperative) needs 28 rows of
    # 1024 records, more than 32 rows of 501
    assert sv.spec_verify_step_ragged_workspace_bytes(4, 7, 128256) == base(4, 7, 128256) + 28 * 1024 * rec
    # B = 20: R >= 20 > 16, never cooperative
    assert sv.spec_verify_step_ragged_workspace_bytes(20, 3, 128256) == \
        base(20, 3, 128256) + (80 * 501 * rec + 255) // 256 * 256
    assert sv.spec_verify_step_ragged_workspace_bytes(1, 64, 100) == 0
    assert sv.spec_verify_step_ragged_workspace_bytes(0, 3, 100) == 0


def test_ragged_step_validation(lib):
    assert _step_ragged(lib, hid=None) == sv.SPEC_ERR_ARG
    assert _step_ragged(lib, logits=None) == sv.SPEC_ERR_ARG
    assert _step_ragged(lib, dt=3) == sv.SPEC_ERR_DTYPE
    assert _step_ragged(lib, K=64) == sv.SPEC_ERR_ARG
    assert _step_ragged(lib, H=12) == sv.SPEC_ERR_ARG
    assert _step_ragged(lib, rs=None) == sv.SPEC_ERR_ARG
    assert _step_ragged(lib, rs=P(0x10002)) == sv.SPEC_ERR_ALIGN
    assert _step_ragged(lib, total=1) == sv.SPEC_ERR_ARG           # fewer rows than sequences
    assert _step_ragged(lib, total=9) == sv.SPEC_ERR_ARG           # more than B*(K_max+1)
    assert _step_ragged(lib, ns=1) == sv.SPEC_ERR_ARG              # NULL list: 0 or B only
    assert _step_ragged(lib, sm=A, ns=3) == sv.SPEC_ERR_ARG
    assert _step_ragged(lib, dtok=None) == sv.SPEC_ERR_ARG         # R > B: there are drafts
    assert _step_ragged(lib, dl=None) == sv.SPEC_ERR_ARG
    assert _step_ragged(lib, seeds=None) == sv.SPEC_ERR_ARG
    assert _step_ragged(lib, T=-1.0) == sv.SPEC_ERR_ARG
    assert _step_ragged(lib, dl=MIS) == sv.SPEC_ERR_ALIGN
    assert _step_ragged(lib, hid=MIS) == sv.SPEC_ERR_ALIGN
    assert _step_ragged(lib, logits=MIS) == sv.SPEC_ERR_ALIGN
    assert _step_ragged(lib, wsb=16) == sv.SPEC_ERR_WORKSPACE
    # the dense step's size is not enough where R <= 16 can be cooperative
    assert _step_ragged(lib, B=4, K=7, total=16, ns=4,
                        wsb=sv.spec_verify_step_workspace_bytes(4, 7, 100)) == sv.SPEC_ERR_WORKSPACE
    assert _step_ragged(lib, ws=MIS) == sv.SPEC_ERR_ALIGN
    # no drafts at all (R == B): neither draft logits nor tokens needed
    assert _step_ragged(lib, total=2, dl=None, dtok=None, ws=None) == sv.SPEC_ERR_WORKSPACE


def _tree_step(lib, hid=A, w=A, dt=sv.SPEC_BF16, par=A, tok=A, rows=None, nr=0, B=2, N=7, V=1000, H=64,
               logits=A, acc=A, out=A, nodes=None, ws=A, wsb=None):
    if wsb is None:
        wsb = sv.spec_verify_step_workspace_bytes(B, N, V)
    return lib.spec_tree_verify_step(hid, w, dt, par, tok, rows, nr, B, N, V, H, logits, acc, out, nodes, ws, wsb,
                                     None)


def test_tree_step_validation(lib):
    assert _tree_step(lib, hid=None) == sv.SPEC_ERR_ARG
    assert _tree_step(lib, logits=None) == sv.SPEC_ERR_ARG
    assert _tree_step(lib, out=None) == sv.SPEC_ERR_ARG
    assert _tree_step(lib, dt=7) == sv.SPEC_ERR_DTYPE
    assert _tree_step(lib, N=64) == sv.SPEC_ERR_ARG
    assert _tree_step(lib, H=12) == sv.SPEC_ERR_ARG
    assert _tree_step(lib, par=None) == sv.SPEC_ERR_ARG
    assert _tree_step(lib, tok=None) == sv.SPEC_ERR_ARG
    assert _tree_step(lib, rows=A, nr=3) == sv.SPEC_ERR_ARG       # more than B
    assert _tree_step(lib, w=MIS) == sv.SPEC_ERR_ALIGN
    assert _tree_step(lib, logits=MIS) == sv.SPEC_ERR_ALIGN
    assert _tree_step(lib, wsb=16) == sv.SPEC_ERR_WORKSPACE
    assert _tree_step(lib, ws=MIS) == sv.SPEC_ERR_ALIGN
    # N = 0: no parents or tokens needed (the workspace check comes after)
    assert _tree_step(lib, N=0, par=None, tok=None, ws=None) == sv.SPEC_ERR_WORKSPACE


def test_zero_selected_rows_is_a_no_op(lib):
    # n_rows == 0 with a row list: valid, nothing to enqueue, no HIP call
    assert _greedy(lib, rows=A, n_rows=0) == sv.SPEC_OK
    assert _sample(lib, rows=A, n_rows=0) == sv.SPEC_OK


def test_binding_fails_loudly_without_library(tmp_path):
    import importlib
    mod = importlib.import_module("speculative_decoding_verification_02_amd")
    saved = mod._lib
    mod._lib = None
    try:
        with pytest.raises(RuntimeError, match="missing"):
            mod.load_library(str(tmp_path / "nope.so"))
    finally:
        mod._lib = saved


def test_product_never_touches_the_oracle():
    """The package (binding and kernels) neither imports nor names the oracle."""
    pkg = os.path.join(ROOT, "speculative_decoding_verification_02_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn)).read()
                assert not re.search(r"\boracle\b", text), fn


def test_binding_checks_tensors_before_any_launch():
    """The kernels trust the dtype and extent behind every pointer, so the
    binding rejects a wrong dtype, a wrong shape, a strided view or a host
    tensor before it reaches the library."""
    import torch
    B, K, V = 2, 3, 64
    z = torch.zeros((B, K + 1, V))
    d32 = torch.zeros((B, K), dtype=torch.int32)
    acc = torch.zeros((B,), dtype=torch.int32)
    out = torch.zeros((B, K + 1), dtype=torch.int32)
    ws = torch.zeros((64,), dtype=torch.uint8)
    with pytest.raises(TypeError, match="logits"):
        sv.spec_accept_greedy(z.double(), d32, acc, out, ws)
    with pytest.raises(TypeError, match="draft_tokens"):
        sv.spec_accept_greedy(z, d32.long(), acc, out, ws)                  # int64 tokens
    with pytest.raises(ValueError, match="draft_tokens has shape"):
        sv.spec_accept_greedy(z, torch.zeros((B, K + 1), dtype=torch.int32), acc, out, ws)
    with pytest.raises(ValueError, match="out_tokens has shape"):
        sv.spec_accept_greedy(z, d32, acc, out[:, :K].contiguous(), ws)
    with pytest.raises(ValueError, match="contiguous"):
        sv.spec_accept_greedy(z, torch.zeros((K, B), dtype=torch.int32).t(), acc, out, ws)
    with pytest.raises(ValueError, match="on the GPU"):
        sv.spec_accept_greedy(z, d32, acc, out, ws)
    with pytest.raises(TypeError, match="seeds"):
        sv.spec_accept_sample(z, torch.zeros((B, K, V)), d32, 1.0, torch.zeros((B,), dtype=torch.int32), acc, out,
                              ws)
    with pytest.raises(ValueError, match="draft_logits has shape"):
        sv.spec_verify_step(torch.zeros((B, K + 1, 8), dtype=torch.bfloat16),
                            torch.zeros((V, 8), dtype=torch.bfloat16), z, acc, out, ws,
                            draft_logits=torch.zeros((B, K + 1, V)), draft_tokens=d32,
                            seeds=torch.zeros((B,), dtype=torch.int64), sampled_rows="all")
    with pytest.raises(ValueError, match="row_start"):
        sv.spec_accept_greedy_ragged(torch.zeros((6, V)), torch.zeros((4,), dtype=torch.int32),
                                     torch.zeros((2, 2), dtype=torch.int32), K, acc, torch.zeros((6,), dtype=torch.int32),
                                     ws)


def test_noalloc_step_size_limit(lib):
    """spec_verify_step_noalloc refuses, before any HIP call, sizes whose
    workspace would exceed the library's 64 MiB scratch, and names the
    limit; sizes out of range are argument errors."""
    def call(B, K, V, H=64):
        return lib.spec_verify_step_noalloc(A, A, sv.SPEC_BF16, A, A, 1.0, A, None, B, None, 0, B, K, V, H,
                                            A, A, A, None, None)
    assert sv.spec_verify_step_workspace_bytes(256, 63, 262144) > 64 << 20
    assert call(256, 63, 262144) == sv.SPEC_ERR_WORKSPACE
    assert "64 MiB" in sv.spec_last_error_detail()
    assert call(0, 4, 1000) == sv.SPEC_ERR_ARG
    assert call(1, 64, 1000) == sv.SPEC_ERR_ARG
    for B, K, V in ((1, 5, 128256), (64, 4, 128256), (256, 8, 152064), (512, 3, 262144), (32, 15, 151936)):
        assert 0 < sv.spec_verify_step_workspace_bytes(B, K, V) <= 64 << 20, (B, K, V)
