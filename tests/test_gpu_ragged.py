"""GPU parity of the packed-batch calls (per-sequence draft counts K_b):
spec_accept_greedy_ragged and spec_accept_sample_ragged against the oracle's
packed rules, on fp32 logits both sides see (greedy exact, sampled decision
by decision), plus: a batch with every K_b = K reproduces the dense calls bit
for bit; all K_b = 0 (no draft rows at all); malformed offsets mark only their
sequences and leave their rows untouched; the LM head on packed hidden states
end to end; and the 64-sequence packed workload at full size.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import speculative_decoding_verification_02_amd as sv
from gpu_support import (ParityCounts, compare_greedy, compare_sample, dev, f64, gpu_accept_greedy,
                         gpu_accept_sample, gpu_logits, say, seeds_tensor, workspace)

pytestmark = pytest.mark.gpu


def _inputs(B, K_max, V, seed, counts=None, T=1.0):
    g = torch.Generator().manual_seed(seed)
    counts = synth.draft_counts(B, K_max, seed) if counts is None else np.asarray(counts, np.int32)
    zt = torch.randn((B, K_max + 1, V), generator=g) * 2.0
    zd = zt[:, :K_max] + torch.randn((B, K_max, V), generator=g)
    # sampled rows: drafts from softmax(zd/T) by Gumbel-max; greedy rows: the
    # target argmax, corrupted with probability 0.2
    u = torch.rand((B, K_max, V), generator=g, dtype=torch.float64).clamp_(min=1e-300)
    samp = torch.argmax(zd.double() / T - torch.log(-torch.log(u)), dim=-1)
    am = torch.argmax(zt[:, :K_max], dim=-1)
    bad = torch.rand((B, K_max), generator=g) > 0.8
    greedy = torch.where(bad, torch.randint(0, V, (B, K_max), generator=g), am)
    seeds = np.random.default_rng(seed).integers(0, 2 ** 63, B).astype(np.uint64)
    return counts, zt, zd, samp.to(torch.int32), greedy.to(torch.int32), seeds


def _pack(counts, zt, zd, d):
    rs = synth.row_start(counts)
    return (rs, synth.pack_rows(zt, counts).contiguous(), synth.pack_rows(zd, counts, True).contiguous(),
            synth.pack_rows(d, counts, True).contiguous())


def _run_greedy(rs, zp, dp, K_max, rows=None):
    R, V = zp.shape
    B = len(rs) - 1
    acc = torch.full((B,), -2, dtype=torch.int32, device=dev())
    out = torch.full((R,), -9, dtype=torch.int32, device=dev())
    rows_t = None if rows is None else torch.as_tensor(np.asarray(rows, np.int32), device=dev())
    sv.spec_accept_greedy_ragged(zp.to(dev()), dp.to(dev()) if R > B else None,
                                 torch.as_tensor(rs, device=dev()), K_max, acc, out, workspace(B, K_max, V),
                                 rows=rows_t)
    return acc.cpu().numpy(), out.cpu().numpy()


def _run_sample(rs, zp, zdp, dp, K_max, T, seeds, rows=None, probs=False):
    R, V = zp.shape
    B = len(rs) - 1
    acc = torch.full((B,), -2, dtype=torch.int32, device=dev())
    out = torch.full((R,), -9, dtype=torch.int32, device=dev())
    pad = torch.full((R - B, 2), float("nan"), dtype=torch.float32, device=dev()) if probs else None
    rows_t = None if rows is None else torch.as_tensor(np.asarray(rows, np.int32), device=dev())
    sv.spec_accept_sample_ragged(zp.to(dev()), zdp.to(dev()) if R > B else None,
                                 dp.to(dev()) if R > B else None, torch.as_tensor(rs, device=dev()), K_max, T,
                                 seeds_tensor(seeds), acc, out, workspace(B, K_max, V), rows=rows_t,
                                 probs_at_draft=pad)
    return acc.cpu().numpy(), out.cpu().numpy(), None if pad is None else pad.cpu().numpy()


def _seq_greedy(res, rs, b):
    t0, t1 = int(rs[b]), int(rs[b + 1])
    return oracle.GreedyResult(res.accepted_len[b:b + 1], res.out_tokens[None, t0:t1], res.argmax[None, t0:t1],
                               res.margin[None, t0:t1])


def _seq_sample(res, rs, b):
    t0, t1 = int(rs[b]), int(rs[b + 1])
    d0, d1 = t0 - b, t1 - 1 - b
    return oracle.SampleResult(res.accepted_len[b:b + 1], res.out_tokens[None, t0:t1],
                               res.probs_at_draft[None, d0:d1], res.ratio[None, d0:d1], res.u_accept[None, t0:t1],
                               res.u_terminal[None, t0:t1], res.accept_margin[None, d0:d1],
                               res.terminal_margin[b:b + 1], res.residual_mass[b:b + 1], res.alpha[None, d0:d1])


def _compare(kind, res, acc, out, rs, rows, exact=False):
    c = ParityCounts()
    for b in rows:
        t0, t1 = int(rs[b]), int(rs[b + 1])
        if kind == "greedy":
            c.merge(compare_greedy(_seq_greedy(res, rs, b), acc[b:b + 1], out[None, t0:t1], [0], exact=exact))
        else:
            c.merge(compare_sample(_seq_sample(res, rs, b), acc[b:b + 1], out[None, t0:t1], [0]))
    return c


@pytest.mark.parametrize("K_max,V", [(1, 1000), (7, 5003), (63, 1000), (5, 2 * 4096 + 7)])
def test_ragged_greedy_exact(K_max, V):
    B = 40
    counts, zt, _, _, dg, _ = _inputs(B, K_max, V, seed=K_max * 31 + V)
    counts[:3] = [0, K_max, 0]
    rs, zp, _, dp = _pack(counts, zt, zt[:, :K_max], dg)
    say("ragged greedy B=%d K_max=%d V=%d R=%d" % (B, K_max, V, len(zp)))
    for rows in (None, np.array([5, 0, 17, 39, 2])):
        acc, out = _run_greedy(rs, zp, dp, K_max, rows)
        res = oracle.accept_greedy_ragged(zp.double().numpy(), dp.numpy(), rs, K_max, rows)
        sel = range(B) if rows is None else rows
        c = _compare("greedy", res, acc, out, rs, sel, exact=True)
        if rows is not None:   # unselected sequences untouched
            mask = np.ones(B, bool)
            mask[rows] = False
            assert np.all(acc[mask] == -2)
        say("  " + str(c))


@pytest.mark.parametrize("K_max,V,T", [(1, 1000, 1.0), (7, 5003, 0.8), (63, 1000, 1.0), (5, 2 * 4096 + 7, 1.3)])
def test_ragged_sample(K_max, V, T):
    B = 40
    counts, zt, zd, ds, _, seeds = _inputs(B, K_max, V, seed=K_max * 17 + V, T=T)
    counts[:3] = [0, K_max, 0]
    rs, zp, zdp, dp = _pack(counts, zt, zd, ds)
    say("ragged sample B=%d K_max=%d V=%d R=%d T=%g" % (B, K_max, V, len(zp), T))
    for rows in (None, np.array([3, 1, 38, 20])):
        acc, out, pad = _run_sample(rs, zp, zdp, dp, K_max, T, seeds, rows, probs=True)
        res = oracle.accept_sample_ragged(zp.double().numpy(), zdp.double().numpy(), dp.numpy(), rs, K_max, T,
                                          seeds, rows)
        sel = range(B) if rows is None else rows
        c = _compare("sample", res, acc, out, rs, sel)
        for b in sel:
            d0, d1 = int(rs[b]) - b, int(rs[b + 1]) - 1 - b
            np.testing.assert_allclose(pad[d0:d1], res.probs_at_draft[d0:d1], atol=1e-5, rtol=0)
        say("  " + str(c))


@pytest.mark.parametrize("K", [0, 3])
def test_uniform_counts_match_dense_calls(K):
    B, V, T = 24, 3001, 0.9
    counts, zt, zd, ds, dg, seeds = _inputs(B, K, V, seed=400 + K, counts=[K] * 24, T=T)
    rs, zp, zdp, dp = _pack(counts, zt, zd, ds)
    say("ragged == dense B=%d K=%d V=%d" % (B, K, V))
    acc_d, out_d, pad_d = gpu_accept_sample(zt.to(dev()), zd.to(dev()), ds.to(dev()), T, seeds, probs=True)
    acc_r, out_r, pad_r = _run_sample(rs, zp, zdp, dp, K, T, seeds, probs=True)
    np.testing.assert_array_equal(acc_d.cpu().numpy(), acc_r)
    np.testing.assert_array_equal(out_d.cpu().numpy().reshape(-1), out_r)
    np.testing.assert_array_equal(pad_d.cpu().numpy().reshape(-1, 2), pad_r)
    _, _, _, dpg = _pack(counts, zt, zd, dg)
    acc_d, out_d = gpu_accept_greedy(zt.to(dev()), dg.to(dev()))
    acc_r, out_r = _run_greedy(rs, zp, dpg, K)
    np.testing.assert_array_equal(acc_d.cpu().numpy(), acc_r)
    np.testing.assert_array_equal(out_d.cpu().numpy().reshape(-1), out_r)


def test_all_zero_drafts():
    B, V, T = 33, 4099, 1.1
    counts, zt, zd, ds, dg, seeds = _inputs(B, 6, V, seed=77, counts=[0] * 33, T=T)
    rs, zp, _, _ = _pack(counts, zt, zd, ds)
    say("ragged, no drafts: B=%d V=%d (R = B)" % (B, V))
    acc, out = _run_greedy(rs, zp, torch.zeros(0, dtype=torch.int32), 6)
    np.testing.assert_array_equal(acc, 0)
    np.testing.assert_array_equal(out, np.argmax(zp.numpy(), axis=-1))
    acc, out, _ = _run_sample(rs, zp, torch.zeros((0, V)), torch.zeros(0, dtype=torch.int32), 6, T, seeds)
    res = oracle.accept_sample_ragged(zp.double().numpy(), None, None, rs, 6, T, seeds)
    say("  " + str(_compare("sample", res, acc, out, rs, range(B))))


def test_malformed_offsets():
    B, K_max, V, T = 5, 3, 2000, 1.0
    counts, zt, zd, ds, dg, seeds = _inputs(B, K_max, V, seed=5, counts=[1, 2, 0, 3, 1], T=T)
    rs, zp, zdp, dp = _pack(counts, zt, zd, ds)
    bad = rs.copy()
    bad[2] = bad[3] + 1          # sequence 1: K_1 = 4 > K_max; sequence 2: K_2 = -2
    say("ragged malformed offsets %s -> %s" % (rs.tolist(), bad.tolist()))
    acc, out, _ = _run_sample(bad, zp, zdp, dp, K_max, T, seeds)
    res = oracle.accept_sample_ragged(zp.double().numpy(), zdp.double().numpy(), dp.numpy(), bad, K_max, T, seeds)
    assert acc[1] == -1 and acc[2] == -1
    np.testing.assert_array_equal(out[rs[1]:rs[3]], -9)          # rows of sequences 1 and 2 never written
    _compare("sample", res, acc, out, rs, [0, 3, 4])
    acc, out = _run_greedy(bad, zp, dp, K_max)
    assert acc[1] == -1 and acc[2] == -1
    np.testing.assert_array_equal(out[rs[1]:rs[3]], -9)


def test_end_to_end_packed_hidden():
    B, K_max, H, V, T = 16, 7, 512, 3001, 0.8
    wl = synth.Workload("t", B=B, K=K_max, H=H, V=V, dtype="bf16", w_std=0.03, temperature=T,
                        draft="additive", draft_sigma=(0.5, 0.5), data_seed=9)
    counts = synth.draft_counts(B, K_max, 9)
    rs = synth.row_start(counts)
    W, hid = synth.weights(wl), synth.hidden_states(wl)
    hp = synth.pack_rows(hid, counts).contiguous()
    R = hp.shape[0]
    say("ragged end to end B=%d K_max=%d H=%d V=%d R=%d" % (B, K_max, H, V, R))
    logits = gpu_logits(hp.view(R, 1, H).to(dev()), W.to(dev())).view(R, V)
    z = oracle.lm_head_logits(f64(hp), f64(W))
    # draft rows: the target rows at each sequence's draft positions plus noise
    g = torch.Generator().manual_seed(3)
    keep = [i for b in range(B) for i in range(int(rs[b]), int(rs[b + 1]) - 1)]
    zdp = (torch.from_numpy(z[keep]).float() + 0.5 * torch.randn((len(keep), V), generator=g)).contiguous()
    u = torch.rand(zdp.shape, generator=g, dtype=torch.float64).clamp_(min=1e-300)
    dp = torch.argmax(zdp.double() / T - torch.log(-torch.log(u)), dim=-1).to(torch.int32)
    seeds = np.arange(B, dtype=np.uint64) + 1000
    acc = torch.full((B,), -2, dtype=torch.int32, device=dev())
    out = torch.full((R,), -9, dtype=torch.int32, device=dev())
    sv.spec_accept_sample_ragged(logits, zdp.to(dev()), dp.to(dev()), torch.as_tensor(rs, device=dev()), K_max, T,
                                 seeds_tensor(seeds), acc, out, workspace(B, K_max, V))
    res = oracle.accept_sample_ragged(z, zdp.double().numpy(), dp.numpy(), rs, K_max, T, seeds)
    say("  " + str(_compare("sample", res, acc.cpu().numpy(), out.cpu().numpy(), rs, range(B))))


def test_full_size_packed_workload():
    wl = synth.WORKLOADS["b64_k0to7_h4096_v128256"]
    counts = synth.draft_counts(wl.B, wl.K, wl.data_seed)
    rs = synth.row_start(counts)
    say("full-size packed workload %s, R=%d: generating inputs on the GPU" % (wl.name, int(rs[-1])))
    inp = synth.round_inputs(wl, 0, device=dev())
    hp = synth.pack_rows(inp["hidden"], counts).contiguous()
    R = hp.shape[0]
    logits = gpu_logits(hp.view(R, 1, wl.H), inp["W"]).view(R, wl.V)
    zdp = synth.pack_rows(inp["draft_logits"], counts, True).contiguous()
    dp = synth.pack_rows(inp["drafts"], counts, True).contiguous()
    sm = inp["sampled"]
    greedy_rows, sampled_rows = np.nonzero(~sm)[0], np.nonzero(sm)[0]
    acc = torch.full((wl.B,), -2, dtype=torch.int32, device=dev())
    out = torch.full((R,), -9, dtype=torch.int32, device=dev())
    ws = workspace(wl.B, wl.K, wl.V)
    rs_t = torch.as_tensor(rs, device=dev())
    sv.spec_accept_greedy_ragged(logits, dp, rs_t, wl.K, acc, out, ws,
                                 rows=torch.as_tensor(greedy_rows.astype(np.int32), device=dev()))
    sv.spec_accept_sample_ragged(logits, zdp, dp, rs_t, wl.K, wl.temperature, seeds_tensor(inp["seeds"]), acc, out,
                                 ws, rows=torch.as_tensor(sampled_rows.astype(np.int32), device=dev()))
    z = logits.double().cpu().numpy()
    acc, out = acc.cpu().numpy(), out.cpu().numpy()
    rg = oracle.accept_greedy_ragged(z, dp.cpu().numpy(), rs, wl.K, greedy_rows)
    rsmp = oracle.accept_sample_ragged(z, zdp.double().cpu().numpy(), dp.cpu().numpy(), rs, wl.K, wl.temperature,
                                       inp["seeds"], sampled_rows)
    c = _compare("greedy", rg, acc, out, rs, greedy_rows, exact=True)
    c.merge(_compare("sample", rsmp, acc, out, rs, sampled_rows))
    say("  " + str(c))


# ------------------------------------------------ the one-call ragged step --

def _step_inputs(B, K_max, H, V, dtype, seed, counts=None, T=0.9):
    wl = synth.Workload("t", B=B, K=K_max, H=H, V=V, dtype=dtype, w_std=0.03 if dtype == "bf16" else 0.05,
                        temperature=T, draft="additive", draft_sigma=(0.5, 0.5), data_seed=seed)
    inp = synth.round_inputs(wl, 0, device=dev())
    counts = synth.draft_counts(B, K_max, seed) if counts is None else np.asarray(counts, np.int32)
    rs = synth.row_start(counts)
    hp = synth.pack_rows(inp["hidden"], counts).contiguous()
    zdp = synth.pack_rows(inp["draft_logits"], counts, True).contiguous()
    dp = synth.pack_rows(inp["drafts"], counts, True).contiguous()
    return wl, inp, rs, hp, zdp, dp


def _ragged_step(hp, W, rs, K_max, zdp, dp, T, seeds, greedy_rows, sampled_rows):
    R, V = hp.shape[0], W.shape[0]
    B = len(rs) - 1
    logits = torch.full((R, V), float("nan"), dtype=torch.float32, device=dev())
    acc = torch.full((B,), -2, dtype=torch.int32, device=dev())
    out = torch.full((R,), -9, dtype=torch.int32, device=dev())
    pad = torch.full((R - B, 2), float("nan"), dtype=torch.float32, device=dev())
    ws = torch.empty(sv.spec_verify_step_ragged_workspace_bytes(B, K_max, V), dtype=torch.uint8, device=dev())

    def rl(r):
        if r is None or isinstance(r, str):
            return r
        return torch.as_tensor(np.asarray(r, np.int32), device=dev())
    sv.spec_verify_step_ragged(hp, W, logits, torch.as_tensor(rs, device=dev()), K_max, acc, out, ws,
                               draft_logits=zdp if R > B else None, draft_tokens=dp if R > B else None,
                               temperature=T, seeds=seeds_tensor(seeds), greedy_rows=rl(greedy_rows),
                               sampled_rows=rl(sampled_rows), probs_at_draft=pad)
    torch.cuda.synchronize()
    return logits, acc.cpu().numpy(), out.cpu().numpy(), pad.cpu().numpy()


def _check_step(wl, inp, rs, hp, zdp, dp, greedy_rows, sampled_rows):
    """Logits bit-identical to spec_verify_logits on the packed rows; greedy
    decisions identical to spec_accept_greedy_ragged and exact against the
    oracle; sampled decisions of the step and of spec_accept_sample_ragged
    against the oracle, probabilities within 1e-5."""
    B, K, V, T = wl.B, wl.K, wl.V, wl.temperature
    R = hp.shape[0]
    logits, acc, out, pad = _ragged_step(hp, inp["W"], rs, K, zdp, dp, T, inp["seeds"], greedy_rows, sampled_rows)
    ref = gpu_logits(hp.view(R, 1, wl.H), inp["W"]).view(R, V)
    assert torch.equal(logits, ref), "the ragged step changed the logits"
    z = ref.double().cpu().numpy()
    g_rows = np.arange(B) if isinstance(greedy_rows, str) else np.asarray(greedy_rows if greedy_rows is not None
                                                                          else [], np.int64)
    s_rows = np.arange(B) if isinstance(sampled_rows, str) else np.asarray(sampled_rows if sampled_rows is not None
                                                                           else [], np.int64)
    c = ParityCounts()
    if len(g_rows):
        acc_g, out_g = _run_greedy(rs, ref.cpu(), dp.cpu(), K, g_rows)
        np.testing.assert_array_equal(acc[g_rows], acc_g[g_rows])
        for b in g_rows:
            np.testing.assert_array_equal(out[rs[b]:rs[b + 1]], out_g[rs[b]:rs[b + 1]])
        res = oracle.accept_greedy_ragged(z, dp.cpu().numpy(), rs, K, g_rows)
        c.merge(_compare("greedy", res, acc, out, rs, g_rows, exact=True))
    if len(s_rows):
        res = oracle.accept_sample_ragged(z, zdp.double().cpu().numpy(), dp.cpu().numpy(), rs, K, T, inp["seeds"],
                                          s_rows)
        c.merge(_compare("sample", res, acc, out, rs, s_rows))
        acc_s, out_s, _ = _run_sample(rs, ref.cpu(), zdp.cpu(), dp.cpu(), K, T, inp["seeds"], s_rows)
        c.merge(_compare("sample", res, acc_s, out_s, rs, s_rows))
        for b in s_rows:
            d0, d1 = int(rs[b]) - b, int(rs[b + 1]) - 1 - b
            np.testing.assert_allclose(pad[d0:d1], res.probs_at_draft[d0:d1], atol=1e-5, rtol=0)
    say("  " + str(c))


@pytest.mark.parametrize("B,K_max,H,V,dtype,counts,path", [
    (3, 4, 512, 3001, "bf16", [4, 0, 2], "cooperative records, one-launch accept + residual (R = 9)"),
    (6, 4, 256, 2053, "bf16", [1, 0, 2, 1, 0, 1], "cooperative records, separate residual launch (R = 11)"),
    (2, 5, 4096, 40000, "bf16", [5, 3], "cooperative records, H = 4096 (R = 10)"),
    (4, 7, 256, 5003, "bf16", [0, 7, 3, 2], "cooperative at R = 16 where B*(K_max+1) = 32"),
    (8, 5, 256, 4099, "bf16", None, "direct-to-LDS epilogue records merged from memory"),
    (6, 15, 256, 5003, "bf16", None, "direct-to-LDS epilogue records folded to chunks (K_max = 15)"),
    (20, 3, 128, 1031, "bf16", [0] * 20, "direct-to-LDS, no draft rows at all (R = B)"),
    (5, 7, 520, 2053, "bf16", None, "tiled kernel (H % 64 != 0): the separate calls' kernels"),
    (4, 3, 256, 1000, "f32", None, "fp32: the separate calls' kernels"),
])
def test_ragged_step_paths(B, K_max, H, V, dtype, counts, path):
    wl, inp, rs, hp, zdp, dp = _step_inputs(B, K_max, H, V, dtype, seed=B * 7 + K_max + V, counts=counts)
    say("ragged step B=%d K_max=%d H=%d V=%d %s R=%d: %s" % (B, K_max, H, V, dtype, hp.shape[0], path))
    half = B // 2
    _check_step(wl, inp, rs, hp, zdp, dp, list(range(half)), list(range(half, B)))
    _check_step(wl, inp, rs, hp, zdp, dp, None, "all")
    _check_step(wl, inp, rs, hp, zdp, dp, "all", None)


@pytest.mark.parametrize("B,K", [(2, 5), (8, 4)])
def test_ragged_step_uniform_counts_match_dense_step(B, K):
    """Every K_b = K: the same kernels and record layouts as spec_verify_step
    on the dense batch, so every output matches bit for bit."""
    wl, inp, rs, hp, zdp, dp = _step_inputs(B, K, 256, 3001, "bf16", seed=50 + B, counts=[K] * B)
    say("ragged step, uniform counts B=%d K=%d: against the dense step" % (B, K))
    P, V = K + 1, wl.V
    sm = list(range(1, B, 2))
    gr = list(range(0, B, 2))
    logits, acc, out, pad = _ragged_step(hp, inp["W"], rs, K, zdp, dp, wl.temperature, inp["seeds"], gr, sm)
    d_logits = torch.empty((B, P, V), dtype=torch.float32, device=dev())
    d_acc = torch.full((B,), -2, dtype=torch.int32, device=dev())
    d_out = torch.full((B, P), -9, dtype=torch.int32, device=dev())
    d_pad = torch.full((B, K, 2), float("nan"), dtype=torch.float32, device=dev())
    ws = torch.empty(sv.spec_verify_step_workspace_bytes(B, K, V), dtype=torch.uint8, device=dev())
    sv.spec_verify_step(inp["hidden"], inp["W"], d_logits, d_acc, d_out, ws, draft_logits=inp["draft_logits"],
                        draft_tokens=inp["drafts"], temperature=wl.temperature, seeds=seeds_tensor(inp["seeds"]),
                        greedy_rows=torch.as_tensor(np.asarray(gr, np.int32), device=dev()),
                        sampled_rows=torch.as_tensor(np.asarray(sm, np.int32), device=dev()), probs_at_draft=d_pad)
    torch.cuda.synchronize()
    assert torch.equal(logits, d_logits.view(B * P, V))
    np.testing.assert_array_equal(acc, d_acc.cpu().numpy())
    np.testing.assert_array_equal(out, d_out.cpu().numpy().reshape(-1))
    p_r, p_d = pad.reshape(B, K, 2)[sm], d_pad.cpu().numpy()[sm]
    np.testing.assert_array_equal(p_r, p_d)


def test_ragged_step_malformed_offsets():
    B, K_max, H, V = 5, 3, 256, 2000
    wl, inp, rs, hp, zdp, dp = _step_inputs(B, K_max, H, V, "bf16", seed=5, counts=[1, 2, 0, 3, 1])
    bad = rs.copy()
    bad[2] = bad[3] + 1          # sequence 1: K_1 = 4 > K_max; sequence 2: K_2 = -2
    say("ragged step, malformed offsets %s -> %s" % (rs.tolist(), bad.tolist()))
    for gr, sm in (([0, 1, 2], [3, 4]), (None, "all")):
        _, acc, out, _ = _ragged_step(hp, inp["W"], bad, K_max, zdp, dp, wl.temperature, inp["seeds"], gr, sm)
        assert acc[1] == -1 and acc[2] == -1, acc
        np.testing.assert_array_equal(out[rs[1]:rs[3]], -9)      # rows of sequences 1 and 2 never written
        R = hp.shape[0]
        ref = gpu_logits(hp.view(R, 1, H), inp["W"]).view(R, V)
        res = oracle.accept_sample_ragged(ref.double().cpu().numpy(), zdp.double().cpu().numpy(), dp.cpu().numpy(),
                                          bad, K_max, wl.temperature, inp["seeds"], [3, 4])
        _compare("sample", res, acc, out, rs, [3, 4])


def test_full_size_ragged_step():
    wl = synth.WORKLOADS["b64_k0to7_h4096_v128256"]
    counts = synth.draft_counts(wl.B, wl.K, wl.data_seed)
    rs = synth.row_start(counts)
    say("full-size packed workload %s through the one-call step, R=%d" % (wl.name, int(rs[-1])))
    inp = synth.round_inputs(wl, 0, device=dev())
    hp = synth.pack_rows(inp["hidden"], counts).contiguous()
    zdp = synth.pack_rows(inp["draft_logits"], counts, True).contiguous()
    dp = synth.pack_rows(inp["drafts"], counts, True).contiguous()
    sm = inp["sampled"]
    _check_step(wl, inp, rs, hp, zdp, dp, np.nonzero(~sm)[0], np.nonzero(sm)[0])
