"""The one-call steps under HIP graph capture.

Callers that capture their decode loop into a graph record the verify step
once and replay it with new inputs written into the captured tensors.  Every
kernel here clears what it counts on with kernels of its own (no memset
nodes), so a replay must give the same bits as an eager call.  Each case
captures the step once, then for several rounds writes the round's inputs,
runs the same call eagerly into separate outputs, synchronises, replays the
graph, synchronises again and compares every output bit for bit.

The cases cover each launch structure of the step: the cooperative LM head
with the one-launch accept + residual (B=1), the direct-to-LDS kernel with
its statistics epilogue and the one-launch draw (B=8), the grouped polled
residual of moderate batches (B=64, a separate accept launch), the two-launch
residual of large batches (B=160 sampled, 5120 chunk blocks), the ragged step
and the tree step; the dense cases through spec_verify_step and through
spec_verify_step_noalloc (the library's own scratch).
"""
import numpy as np
import pytest
import torch

import synth
import speculative_decoding_verification_02_amd as sv
from gpu_support import dev, say, seeds_tensor

pytestmark = pytest.mark.gpu

ROUNDS = 3


def _wl(B, K, H, V, modes, seed):
    return synth.Workload("g", B=B, K=K, H=H, V=V, dtype="bf16", w_std=0.03, temperature=0.9, draft="additive",
                          draft_sigma=(0.3, 0.6), modes=modes, data_seed=seed)


def _capture(call):
    """Warm up on a side stream, then capture one call."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    return g


def _replay_rounds(g, load, eager, captured_out, eager_out, what):
    for rnd in range(1, ROUNDS + 1):
        load(rnd)
        # entries the step does not write (probabilities of greedy rows)
        # hold the same marker on both sides
        for t in eager_out:
            t.fill_(-7)
        eager()
        torch.cuda.synchronize()
        for t in captured_out:
            t.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("logits", "accepted_len", "out_tokens", "probs/nodes"), captured_out, eager_out):
            assert torch.equal(torch.nan_to_num(a, nan=3.25), torch.nan_to_num(b, nan=3.25)), \
                "%s: replay %d differs in %s" % (what, rnd, name)
        say("  %s: replay %d matches the eager call" % (what, rnd))


@pytest.mark.parametrize("B,K,H,V,modes,path", [
    (1, 5, 4096, 128256, "sample", "cooperative LM head, one-launch accept + residual"),
    (8, 4, 256, 5003, "half", "direct-to-LDS epilogue, one-launch accept + residual"),
    (64, 4, 256, 128256, "half", "epilogue, grouped polled residual"),
    (160, 3, 64, 128256, "sample", "two-launch residual (5120 chunk blocks)"),
])
@pytest.mark.parametrize("entry", ["spec_verify_step", "spec_verify_step_noalloc"])
def test_step_graph_replays(B, K, H, V, modes, path, entry):
    wl = _wl(B, K, H, V, modes, seed=B + K + V)
    say("graph capture of %s, B=%d K=%d H=%d V=%d: %s" % (entry, B, K, H, V, path))
    inp = synth.round_inputs(wl, 0, device=dev())
    W = inp["W"]
    sm = inp["sampled"]
    g_rows = torch.as_tensor(np.nonzero(~sm)[0].astype(np.int32), device=dev())
    s_rows = torch.as_tensor(np.nonzero(sm)[0].astype(np.int32), device=dev())
    g_arg = g_rows if len(g_rows) else None
    s_arg = s_rows if len(s_rows) else None
    hid = inp["hidden"].clone()
    zd = inp["draft_logits"].clone()
    d = inp["drafts"].clone()
    seeds = seeds_tensor(inp["seeds"])
    P = K + 1

    def outputs():
        return (torch.empty((B, P, V), dtype=torch.float32, device=dev()),
                torch.empty((B,), dtype=torch.int32, device=dev()),
                torch.empty((B, P), dtype=torch.int32, device=dev()),
                torch.empty((B, K, 2), dtype=torch.float32, device=dev()))
    cap, eag = outputs(), outputs()
    ws = torch.empty(sv.spec_verify_step_workspace_bytes(B, K, V), dtype=torch.uint8, device=dev())

    def call(o):
        kw = dict(draft_logits=zd, draft_tokens=d, temperature=wl.temperature, seeds=seeds, greedy_rows=g_arg,
                  sampled_rows=s_arg, probs_at_draft=o[3])
        if entry == "spec_verify_step":
            sv.spec_verify_step(hid, W, o[0], o[1], o[2], ws, **kw)
        else:
            sv.spec_verify_step_noalloc(hid, W, o[0], o[1], o[2], **kw)

    def load(rnd):
        r = synth.round_inputs(wl, rnd, device=dev(), W=W)
        hid.copy_(r["hidden"])
        zd.copy_(r["draft_logits"])
        d.copy_(r["drafts"])
        seeds.copy_(seeds_tensor(r["seeds"]))

    g = _capture(lambda: call(cap))
    _replay_rounds(g, load, lambda: call(eag), cap, eag, entry)


def test_ragged_step_graph_replays():
    B, K_max, H, V = 16, 7, 256, 5003
    wl = _wl(B, K_max, H, V, "half", seed=71)
    counts = synth.draft_counts(B, K_max, 71)
    rs = torch.as_tensor(synth.row_start(counts), device=dev())
    say("graph capture of spec_verify_step_ragged, B=%d K_max=%d R=%d" % (B, K_max, int(rs[-1])))
    inp = synth.round_inputs(wl, 0, device=dev())
    W = inp["W"]
    sm = inp["sampled"]
    g_rows = torch.as_tensor(np.nonzero(~sm)[0].astype(np.int32), device=dev())
    s_rows = torch.as_tensor(np.nonzero(sm)[0].astype(np.int32), device=dev())
    hp = synth.pack_rows(inp["hidden"], counts).contiguous()
    zdp = synth.pack_rows(inp["draft_logits"], counts, True).contiguous()
    dp = synth.pack_rows(inp["drafts"], counts, True).contiguous()
    seeds = seeds_tensor(inp["seeds"])
    R = hp.shape[0]

    def outputs():
        return (torch.empty((R, V), dtype=torch.float32, device=dev()),
                torch.empty((B,), dtype=torch.int32, device=dev()),
                torch.empty((R,), dtype=torch.int32, device=dev()),
                torch.empty((R - B, 2), dtype=torch.float32, device=dev()))
    cap, eag = outputs(), outputs()
    ws = torch.empty(sv.spec_verify_step_ragged_workspace_bytes(B, K_max, V), dtype=torch.uint8, device=dev())

    def call(o):
        sv.spec_verify_step_ragged(hp, W, o[0], rs, K_max, o[1], o[2], ws, draft_logits=zdp, draft_tokens=dp,
                                   temperature=wl.temperature, seeds=seeds, greedy_rows=g_rows, sampled_rows=s_rows,
                                   probs_at_draft=o[3])

    def load(rnd):
        r = synth.round_inputs(wl, rnd, device=dev(), W=W)
        hp.copy_(synth.pack_rows(r["hidden"], counts))
        zdp.copy_(synth.pack_rows(r["draft_logits"], counts, True))
        dp.copy_(synth.pack_rows(r["drafts"], counts, True))
        seeds.copy_(seeds_tensor(r["seeds"]))

    g = _capture(lambda: call(cap))
    _replay_rounds(g, load, lambda: call(eag), cap, eag, "spec_verify_step_ragged")


@pytest.mark.parametrize("B,N,H,V,path", [(2, 7, 256, 3001, "cooperative records (M = 16)"),
                                          (4, 31, 256, 5003, "epilogue records, folded (M = 128)")])
def test_tree_step_graph_replays(B, N, H, V, path):
    wl = _wl(B, N, H, V, "greedy", seed=B * N)
    say("graph capture of spec_tree_verify_step, B=%d N=%d: %s" % (B, N, path))
    W = synth.weights(wl, dev())
    par = torch.as_tensor(synth.tree_parents(B, N, seed=5), device=dev())
    hid = synth.hidden_states(wl, dev(), 0).clone()
    tok = torch.empty((B, N + 1), dtype=torch.int32, device=dev())

    def load(rnd):
        hid.copy_(synth.hidden_states(wl, dev(), rnd))
        tok.copy_(synth.tree_tokens(synth.base_logits(hid, W), par.cpu().numpy(), seed=rnd, sigma=0.3).to(dev()))

    load(0)

    def outputs():
        return (torch.empty((B, N + 1, V), dtype=torch.float32, device=dev()),
                torch.empty((B,), dtype=torch.int32, device=dev()),
                torch.empty((B, N + 1), dtype=torch.int32, device=dev()),
                torch.empty((B, N + 1), dtype=torch.int32, device=dev()))
    cap, eag = outputs(), outputs()
    ws = torch.empty(sv.spec_verify_step_workspace_bytes(B, N, V), dtype=torch.uint8, device=dev())

    def call(o):
        sv.spec_tree_verify_step(hid, W, o[0], par, tok, o[1], o[2], ws, out_nodes=o[3])

    g = _capture(lambda: call(cap))
    _replay_rounds(g, load, lambda: call(eag), cap, eag, "spec_tree_verify_step")
