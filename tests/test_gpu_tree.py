"""GPU parity of spec_tree_accept_greedy against the oracle's tree rule.

On fp32 logits both sides see, results must agree exactly (token ids, kept
depth, node indices): random tree shapes from N = 0 to the largest tree one
wavefront holds (63 nodes), several vocabulary sizes (one chunk, many chunks,
a ragged last chunk, V not a multiple of 4), row subsets.  A chain is the
linear greedy rule of spec_accept_greedy, bit for bit.  Malformed trees and
bad rows are faults.  End to end from hidden states, decisions may differ
only where the oracle's fp64 logits of a row on the kept path have a near
tie; and the 8-sequence, 63-node workload at full size.  spec_tree_verify_step
(LM head and tree rule in one call, the argmaxes from the LM head's own
records) must give the separate calls' logits, lengths, tokens and nodes bit
for bit on every LM-head path, faults included.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import speculative_decoding_verification_02_amd as sv
from gpu_support import NEAR_TIE, dev, f64, gpu_accept_greedy, gpu_logits, say, workspace

pytestmark = pytest.mark.gpu


def _run(logits, par, tok, rows=None):
    B, P, V = logits.shape
    acc = torch.full((B,), -2, dtype=torch.int32, device=dev())
    out = torch.full((B, P), -9, dtype=torch.int32, device=dev())
    nodes = torch.full((B, P), -9, dtype=torch.int32, device=dev())
    rows_t = None if rows is None else torch.as_tensor(np.asarray(rows, np.int32), device=dev())
    sv.spec_tree_accept_greedy(logits.to(dev()), torch.as_tensor(par, device=dev()),
                               torch.as_tensor(np.asarray(tok), device=dev()), acc, out, workspace(B, P - 1, V),
                               out_nodes=nodes, rows=rows_t)
    return acc.cpu().numpy(), out.cpu().numpy(), nodes.cpu().numpy()


def _check_exact(res, acc, out, nodes, rows):
    for b in rows:
        assert acc[b] == res.accepted_len[b], (b, acc[b], res.accepted_len[b])
        np.testing.assert_array_equal(out[b], res.out_tokens[b])
        np.testing.assert_array_equal(nodes[b], res.out_nodes[b])


@pytest.mark.parametrize("N", [0, 1, 7, 31, 63])
@pytest.mark.parametrize("V", [1000, 4096 * 3 + 5])
def test_tree_exact(N, V):
    B = 48
    g = torch.Generator().manual_seed(N * 7 + V)
    z = torch.randn((B, N + 1, V), generator=g) * 2.0
    z[::9, :, 5] = z[::9].max(dim=-1).values        # argmax ties: lowest index wins
    par = synth.tree_parents(B, N, seed=N + V)
    tok = synth.tree_tokens(z, par, seed=N + 3 * V, p_random=0.2).numpy()
    # the first child of each node follows the parent's true argmax more often
    am = z.argmax(dim=-1).numpy()
    follow = np.random.default_rng(N).random((B, N + 1)) < 0.5
    for b in range(B):
        for v in range(1, N + 1):
            if follow[b, v]:
                tok[b, v] = am[b, par[b, v]]
    say("tree exact B=%d N=%d V=%d" % (B, N, V))
    for rows in (None, [3, 47, 0, 12]):
        acc, out, nodes = _run(z, par, tok, rows)
        res = oracle.tree_accept_greedy(z.double().numpy(), par, tok, rows)
        _check_exact(res, acc, out, nodes, range(B) if rows is None else rows)
        if rows is not None:
            mask = np.ones(B, bool)
            mask[rows] = False
            assert np.all(acc[mask] == -2) and np.all(out[mask] == -9)
    acc, _, _ = _run(z, par, tok)
    say("  kept depths: mean %.2f max %d" % (acc.mean(), acc.max()))


@pytest.mark.parametrize("N", [1, 5, 63])
def test_chain_matches_linear_call(N):
    B, V = 40, 5003
    g = torch.Generator().manual_seed(N)
    z = torch.randn((B, N + 1, V), generator=g)
    am = z[:, :N].argmax(dim=-1)
    d = torch.where(torch.rand((B, N), generator=g) < 0.85, am, torch.randint(0, V, (B, N), generator=g))
    par = np.tile(np.arange(-1, N, dtype=np.int32), (B, 1))
    par[:, 0] = 0
    tok = np.concatenate([np.zeros((B, 1), np.int32), d.numpy().astype(np.int32)], axis=1)
    say("tree chain == linear B=%d N=%d" % (B, N))
    acc, out, nodes = _run(z, par, tok)
    acc_l, out_l = gpu_accept_greedy(z.to(dev()), d.to(torch.int32).to(dev()))
    np.testing.assert_array_equal(acc, acc_l.cpu().numpy())
    np.testing.assert_array_equal(out, out_l.cpu().numpy())
    for b in range(B):
        assert nodes[b, :acc[b]].tolist() == list(range(1, acc[b] + 1))


def test_tree_faults():
    B, N, V = 6, 9, 2000
    g = torch.Generator().manual_seed(11)
    z = torch.randn((B, N + 1, V), generator=g)
    par = synth.tree_parents(B, N, seed=11)
    tok = synth.tree_tokens(z, par, seed=12).numpy()
    par[1, 4] = 4               # not topological
    par[2, 7] = -1              # negative parent
    tok[3, 9] = V               # token out of range
    z[4, 6, 100] = float("nan")
    z[5, 2, :] = float("-inf")  # a row with no finite entry
    say("tree faults")
    acc, out, nodes = _run(z, par, tok)
    res = oracle.tree_accept_greedy(z.double().numpy(), par, tok)
    assert acc.tolist()[1:] == [-1] * 5 and acc[0] >= 0
    assert np.all(out[1:] == -1) and np.all(nodes[1:] == -1)
    _check_exact(res, acc, out, nodes, [0])


def test_tree_end_to_end():
    B, N, H, V = 12, 31, 1024, 3001
    wl = synth.Workload("t", B=B, K=N, H=H, V=V, dtype="bf16", w_std=0.03, temperature=1.0, draft="additive",
                        data_seed=21)
    W, hid = synth.weights(wl), synth.hidden_states(wl)
    say("tree end to end B=%d N=%d H=%d V=%d" % (B, N, H, V))
    logits = gpu_logits(hid.to(dev()), W.to(dev()))
    z = oracle.lm_head_logits(f64(hid).reshape(B * (N + 1), H), f64(W)).reshape(B, N + 1, V)
    par = synth.tree_parents(B, N, seed=21)
    tok = synth.tree_tokens(torch.from_numpy(z).float(), par, seed=22, p_random=0.1, sigma=0.05).numpy()
    acc, out, nodes = _run(logits, par, tok)
    res = oracle.tree_accept_greedy(z, par, tok)
    near = 0
    for b in range(B):
        if acc[b] == res.accepted_len[b] and np.array_equal(out[b], res.out_tokens[b]):
            np.testing.assert_array_equal(nodes[b], res.out_nodes[b])
            continue
        # a differing sequence must hinge on a near tie of a row whose argmax
        # the decision read: the root or a node on either side's kept path
        rows = {0} | set(res.out_nodes[b][res.out_nodes[b] >= 0].tolist()) | set(nodes[b][nodes[b] >= 0].tolist())
        assert min(res.margin[b, r] for r in rows) < NEAR_TIE, b
        near += 1
    say("  %d sequences, %d decided by near ties, mean depth %.2f" % (B, near, res.accepted_len.mean()))


def test_full_size_tree_workload():
    wl = synth.WORKLOADS["b8_tree63_h4096_v128256"]
    say("full-size tree workload %s: generating inputs on the GPU" % wl.name)
    W, hid = synth.weights(wl, dev()), synth.hidden_states(wl, dev())
    logits = gpu_logits(hid, W)
    par = synth.tree_parents(wl.B, wl.K, seed=wl.data_seed)
    tok = synth.tree_tokens(synth.base_logits(hid, W), par, seed=wl.data_seed + 1, sigma=wl.draft_sigma[0]).numpy()
    acc, out, nodes = _run(logits, par, tok)
    res = oracle.tree_accept_greedy(logits.double().cpu().numpy(), par, tok)
    _check_exact(res, acc, out, nodes, range(wl.B))
    say("  kept depths %s" % acc.tolist())


def _tree_step(hid, W, par, tok, rows=None, separate=False):
    """spec_tree_verify_step, or (separate) spec_verify_logits followed by
    spec_tree_accept_greedy, on the same device inputs."""
    B, P, H = hid.shape
    V = W.shape[0]
    logits = torch.full((B, P, V), float("nan"), dtype=torch.float32, device=dev())
    acc = torch.full((B,), -2, dtype=torch.int32, device=dev())
    out = torch.full((B, P), -9, dtype=torch.int32, device=dev())
    nodes = torch.full((B, P), -9, dtype=torch.int32, device=dev())
    rows_t = None if rows is None else torch.as_tensor(np.asarray(rows, np.int32), device=dev())
    par_t = torch.as_tensor(par, device=dev())
    tok_t = torch.as_tensor(np.asarray(tok), device=dev())
    if separate:
        sv.spec_verify_logits(hid, W, logits)
        sv.spec_tree_accept_greedy(logits, par_t, tok_t, acc, out, workspace(B, P - 1, V), out_nodes=nodes,
                                   rows=rows_t)
    else:
        ws = torch.empty(sv.spec_verify_step_workspace_bytes(B, P - 1, V), dtype=torch.uint8, device=dev())
        sv.spec_tree_verify_step(hid, W, logits, par_t, tok_t, acc, out, ws, out_nodes=nodes, rows=rows_t)
    torch.cuda.synchronize()
    return logits.cpu(), acc.cpu().numpy(), out.cpu().numpy(), nodes.cpu().numpy()


@pytest.mark.parametrize("B,N,H,V,dtype,path", [
    (2, 7, 512, 3001, "bf16", "cooperative kernel's records (M = 16)"),
    (1, 5, 4096, 40000, "bf16", "cooperative kernel's records, H = 4096"),
    (3, 1, 256, 37, "bf16", "cooperative, V = 37 (workgroups with no tile)"),
    (8, 63, 256, 4099, "bf16", "direct-to-LDS epilogue records, folded (M = 512)"),
    (12, 31, 1024, 3001, "bf16", "direct-to-LDS, 256-row tiles in split rings (M = 384)"),
    (5, 15, 520, 2053, "bf16", "tiled kernel (H % 64 != 0): the separate calls' kernels"),
    (4, 7, 256, 1000, "f32", "fp32: the separate calls' kernels"),
])
def test_tree_step_matches_separate_calls(B, N, H, V, dtype, path):
    wl = synth.Workload("t", B=B, K=N, H=H, V=V, dtype=dtype, w_std=0.03 if dtype == "bf16" else 0.05,
                        temperature=1.0, draft="additive", data_seed=B + N + V)
    W, hid = synth.weights(wl, dev()), synth.hidden_states(wl, dev())
    par = synth.tree_parents(B, N, seed=B + N)
    tok = synth.tree_tokens(synth.base_logits(hid, W), par, seed=V, p_random=0.1, sigma=0.05).numpy()
    say("tree step B=%d N=%d H=%d V=%d %s: %s" % (B, N, H, V, dtype, path))
    for rows in (None, [B - 1] + list(range(0, B - 1, 2))):
        fused = _tree_step(hid, W, par, tok, rows=rows)
        sep = _tree_step(hid, W, par, tok, rows=rows, separate=True)
        assert torch.equal(fused[0], sep[0]), "the tree step changed the logits"
        for a, b in zip(fused[1:], sep[1:]):
            np.testing.assert_array_equal(a, b)
        sel = range(B) if rows is None else rows
        assert all(fused[1][b] >= 0 for b in sel)
    say("  kept depths %s" % fused[1].tolist())


def test_tree_step_faults():
    """A NaN in one node row faults exactly that sequence, as in the separate
    calls."""
    B, N, H, V = 6, 15, 256, 3001
    wl = synth.Workload("t", B=B, K=N, H=H, V=V, dtype="bf16", w_std=0.03, temperature=1.0, draft="additive",
                        data_seed=5)
    W, hid = synth.weights(wl, dev()), synth.hidden_states(wl, dev())
    hid[2, 4, 7] = float("nan")
    par = synth.tree_parents(B, N, seed=5)
    tok = synth.tree_tokens(synth.base_logits(hid.nan_to_num(), W), par, seed=6).numpy()
    say("tree step faults B=%d N=%d" % (B, N))
    fused = _tree_step(hid, W, par, tok)
    sep = _tree_step(hid, W, par, tok, separate=True)
    for a, b in zip(fused[1:], sep[1:]):
        np.testing.assert_array_equal(a, b)
    assert fused[1][2] == -1 and (fused[2][2] == -1).all()
    assert (np.delete(fused[1], 2) >= 0).all()


def test_full_size_tree_step():
    wl = synth.WORKLOADS["b8_tree63_h4096_v128256"]
    say("full-size tree step %s" % wl.name)
    W, hid = synth.weights(wl, dev()), synth.hidden_states(wl, dev())
    par = synth.tree_parents(wl.B, wl.K, seed=wl.data_seed)
    tok = synth.tree_tokens(synth.base_logits(hid, W), par, seed=wl.data_seed + 1, sigma=wl.draft_sigma[0]).numpy()
    fused = _tree_step(hid, W, par, tok)
    sep = _tree_step(hid, W, par, tok, separate=True)
    assert torch.equal(fused[0], sep[0])
    for a, b in zip(fused[1:], sep[1:]):
        np.testing.assert_array_equal(a, b)
    res = oracle.tree_accept_greedy(fused[0].double().numpy(), par, tok)
    _check_exact(res, fused[1], fused[2], fused[3], range(wl.B))
    say("  kept depths %s" % fused[1].tolist())
