"""GPU parity of spec_verify_logits (LM-head contraction) against the oracle.

Covers the small-M kernels (M <= 16), the direct-to-LDS MFMA kernel in each
of its tile heights (M > 16, H a multiple of 64), the LDS-tiled kernel (other
H), and the fp32 kernel, on shapes that span several tiles with ragged tails
in V, M and H; integer-valued inputs that must come out bit-exact whatever the
summation order; the full-size workloads (all entries at B=1, sampled entries
at the larger ones); and run-to-run determinism.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_support import check_logits, dev, f64, gpu_logits, say

pytestmark = pytest.mark.gpu


def _case(B, K, H, V, dtype, w_std=0.05, seed=0, device="cpu"):
    wl = synth.Workload("t", B=B, K=K, H=H, V=V, dtype=dtype, w_std=w_std, temperature=1.0,
                        draft="additive", data_seed=seed)
    return synth.weights(wl, device), synth.hidden_states(wl, device)


def _check(hidden, W):
    B, P, H = hidden.shape
    say("logits case B=%d K=%d H=%d V=%d %s" % (B, P - 1, H, W.shape[0], hidden.dtype))
    g = gpu_logits(hidden.to(dev()), W.to(dev()))
    torch.cuda.synchronize()
    x, w = f64(hidden).reshape(B * P, H), f64(W)
    o = oracle.lm_head_logits(x, w)
    absdot = oracle.lm_head_logits(np.abs(x), np.abs(w))
    ratio = check_logits(g.cpu().numpy().reshape(B * P, -1).astype(np.float64), o, absdot, H)
    say("  max err / fp32 bound = %.3g" % ratio)


def test_fp32_tiny_workload():
    W, h = _case(1, 4, 256, 1000, "f32", 0.05, seed=1)
    _check(h, W)


@pytest.mark.parametrize("B,K", [(1, 0), (1, 5), (2, 2), (4, 3), (16, 0)])
@pytest.mark.parametrize("H,V", [(264, 1000), (4096, 4099), (520, 33)])
def test_bf16_small_m(B, K, H, V):
    W, h = _case(B, K, H, V, "bf16", 0.02, seed=B * 100 + K + H + V)
    _check(h, W)


@pytest.mark.parametrize("B,K", [(1, 0), (4, 3)])
def test_bf16_small_m_long_vocabulary(B, K):
    """A vocabulary range per workgroup too long for the logits to wait in LDS
    at M = 16 (the cooperative kernel stores each tile as it goes), and at
    M = 1 still short enough (it writes them out after the last tile)."""
    W, h = _case(B, K, 264, 400003, "bf16", 0.02, seed=B + 400003)
    _check(h, W)


@pytest.mark.parametrize("B,K,H,V", [(1, 0, 8192, 3001), (2, 1, 6144, 4099), (1, 3, 4104, 130), (4, 3, 8192, 128256)])
def test_bf16_small_m_wide_hidden(B, K, H, V):
    """M <= 16 with 4096 < H <= 8192: the cooperative kernel with four stages
    per tile, two of them in flight across the tile boundary."""
    W, h = _case(B, K, H, V, "bf16", 0.02, seed=H + V)
    _check(h, W)


def test_bf16_wide_hidden_long_vocabulary_sampled():
    """M = 16, H = 4160 (the four-stage cooperative configuration) and a
    vocabulary range per workgroup too long for the logits to wait in LDS:
    the tiles store as they go.  Sampled entries (the weights are 2.7 GB)."""
    B, K, H, V = 4, 3, 4160, 330011
    W, h = _case(B, K, H, V, "bf16", 0.02, seed=V + H, device=dev())
    say("wide-hidden long-vocabulary logits B=%d K=%d H=%d V=%d (sampled)" % (B, K, H, V))
    g = gpu_logits(h, W)
    torch.cuda.synchronize()
    M = B * (K + 1)
    rng = np.random.default_rng(7)
    vs = np.concatenate([rng.integers(0, V, 400), [0, 1, 15, 16, V - 17, V - 16, V - 2, V - 1]])
    ms = rng.integers(0, M, len(vs))
    x = f64(h.reshape(M, H)[torch.as_tensor(ms, device=dev())])
    w = f64(W[torch.as_tensor(vs, device=dev())])
    o = np.sum(x * w, axis=1)
    absdot = np.sum(np.abs(x * w), axis=1)
    gv = g.reshape(M, V)[torch.as_tensor(ms, device=dev()), torch.as_tensor(vs, device=dev())].cpu().numpy()
    u = 2.0 ** -24
    gam = (H + 1) * u / (1 - (H + 1) * u)
    err = np.abs(gv.astype(np.float64) - o)
    assert np.all(err <= gam * absdot), np.max(err / (gam * absdot))
    assert not torch.isnan(g).any().item()
    say("  %d entries, max err / fp32 bound = %.3g" % (len(vs), np.max(err / (gam * absdot))))


@pytest.mark.parametrize("B,K,H,V", [(1, 0, 8200, 3001), (2, 1, 12288, 1000), (1, 5, 16384, 517)])
def test_bf16_small_m_beyond_cooperative(B, K, H, V):
    """M <= 16 with H > 8192 and the hidden rows fitting in LDS: the LDS-staged
    streaming kernel."""
    W, h = _case(B, K, H, V, "bf16", 0.02, seed=H + V + 1)
    _check(h, W)


def test_bf16_small_m_tiled():
    """M = 16 with H = 8200: neither small-M kernel fits, the tiled kernel."""
    W, h = _case(4, 3, 8200, 1000, "bf16", 0.02, seed=8201)
    _check(h, W)


@pytest.mark.parametrize("B,K", [(6, 2), (130, 0), (64, 4), (3, 63)])
@pytest.mark.parametrize("H,V", [(64, 1000), (520, 2053), (1032, 257)])
def test_bf16_tiled(B, K, H, V):
    """H = 520 and 1032 are not multiples of 64: the 128 x 128 tiled kernel."""
    W, h = _case(B, K, H, V, "bf16", 0.02, seed=B * 7 + K + H + V)
    _check(h, W)


@pytest.mark.parametrize("B,K,H,V", [(128, 3, 576, 1000), (300, 3, 1024, 2053), (171, 2, 64, 513)])
def test_bf16_big_m(B, K, H, V):
    """M >= 512 with H a multiple of 64: the direct-to-LDS 256 x 256 kernel,
    including tiles cut by the ragged edges of M and V."""
    W, h = _case(B, K, H, V, "bf16", 0.02, seed=B + K + H + V)
    _check(h, W)


# M = B*(K+1) in each tile-height band of the direct-to-LDS kernel (17-64,
# 65-128, 129-160, 161-192, 193-256, 257-320 as two 160-row tiles, 321-511),
# each at a band edge or with a ragged last tile, against a ragged V.
@pytest.mark.parametrize("B,K", [(17, 0), (4, 4), (16, 3), (25, 3), (32, 3), (13, 9), (32, 4), (20, 7), (38, 4), (43, 5),
                                 (64, 3), (51, 4), (64, 4), (107, 2), (90, 4), (511, 0)])
@pytest.mark.parametrize("H,V", [(128, 1000), (448, 2053)])
def test_bf16_tile_heights(B, K, H, V):
    W, h = _case(B, K, H, V, "bf16", 0.02, seed=3 * B + K + H + V)
    _check(h, W)


@pytest.mark.parametrize("B,K,V,dtype", [(1, 5, 3001, "bf16"), (64, 4, 1031, "bf16"), (1, 4, 999, "f32"),
                                         (160, 3, 777, "bf16")])
def test_small_integers_bit_exact(B, K, V, dtype):
    """Inputs in -4..4 (exact in bf16): every partial sum is an integer below
    2^24, so the fp32 result is exact in any summation order."""
    H = 4096
    g = torch.Generator().manual_seed(V)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    h = torch.randint(-4, 5, (B, K + 1, H), generator=g).to(tdt)
    W = torch.randint(-4, 5, (V, H), generator=g).to(tdt)
    say("integer logits B=%d K=%d V=%d %s" % (B, K, V, dtype))
    out = gpu_logits(h.to(dev()), W.to(dev())).cpu().numpy().reshape(B * (K + 1), V)
    ref = oracle.lm_head_logits(f64(h).reshape(-1, H), f64(W))
    np.testing.assert_array_equal(out.astype(np.float64), ref)


def test_full_size_b1_k5_all_entries():
    wl = synth.WORKLOADS["b1_k5_h4096_v128256"]
    W, h = synth.weights(wl, dev()), synth.hidden_states(wl, dev())
    _check(h, W)


@pytest.mark.parametrize("name", ["b64_k4_h4096_v128256", "b256_k8_h8192_v152064", "b512_k3_h5120_v262144"])
def test_full_size_sampled_entries(name):
    wl = synth.WORKLOADS[name]
    say("full-size logits %s: generating inputs on the GPU" % name)
    W, h = synth.weights(wl, dev()), synth.hidden_states(wl, dev())
    g = gpu_logits(h, W)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    ms = rng.integers(0, wl.M, 512)
    vs = np.concatenate([rng.integers(0, wl.V, 500), [0, 1, wl.V - 2, wl.V - 1] * 3])
    ms = ms[: len(vs)]
    x = f64(h.reshape(wl.M, wl.H)[torch.as_tensor(ms, device=dev())])
    w = f64(W[torch.as_tensor(vs, device=dev())])
    o = np.sum(x * w, axis=1)
    absdot = np.sum(np.abs(x * w), axis=1)
    gv = g.reshape(wl.M, wl.V)[torch.as_tensor(ms, device=dev()), torch.as_tensor(vs, device=dev())]
    gv = gv.cpu().numpy().astype(np.float64)
    u = 2.0 ** -24
    gam = (wl.H + 1) * u / (1 - (wl.H + 1) * u)
    err = np.abs(gv - o)
    assert np.all(err <= gam * absdot), np.max(err / (gam * absdot))
    assert not torch.isnan(g).any().item()
    say("  %d entries, max err / fp32 bound = %.3g" % (len(vs), np.max(err / (gam * absdot))))


@pytest.mark.parametrize("B,K,H,V", [(1, 5, 4096, 128256), (40, 7, 512, 5003)])
def test_deterministic(B, K, H, V):
    W, h = _case(B, K, H, V, "bf16", 0.02, seed=3, device=dev())
    a = gpu_logits(h, W)
    b = gpu_logits(h, W)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
