"""Pins for the fp64 CPU oracle (oracle/): each oracle function is checked
against something other than itself -- a hand-worked example, exhaustive
enumeration, brute-force Python loops, numpy/scipy/torch library routines and
closed forms -- chosen so that a plausible slip (wrong shift, dropped term,
sign, transposed operand, tie order, softmax scope) fails at least one test.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import pw_synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _lut_rule(R, k):
    v = np.arange(1 << k, dtype=np.float64)
    half = float(1 << (k - 1))
    return np.stack([(r + 1) * (v - half + 0.5) / half for r in range(R)]).astype(np.float16)


def _golden_layer():
    with open(os.path.join(GOLDEN, "worked_example_tiny.json")) as f:
        G = json.load(f)
    shape = pw_synth.LayerShape(H=G["H"], I=G["I"], E=G["E"], top_k=G["top_k"])
    gu, dn = [], []
    for e in range(G["E"]):
        for mod, lst in (("gate_up", gu), ("down", dn)):
            b = G["blocks"]["%d.%s" % (e, mod)]
            code8 = np.array(b["code8"], dtype=np.uint8)
            luts = {k: _lut_rule(code8.shape[0], k) for k in range(3, 9)}
            lst.append(pw_synth.Block(code8=code8, luts=luts, q=b["q"]))
    w = pw_synth.LayerWeights(shape=shape, gate_up=gu, down=dn)
    a = pw_synth.Activations(x=np.array(G["x"], dtype=np.float16),
                             logits=np.array(G["logits"], dtype=np.float32))
    return G, w, a


# ---------------------------------------------------------------- worked example

def test_golden_decode_matches_hand_values():
    G, w, _ = _golden_layer()
    for e in range(G["E"]):
        for mod, blk in (("gate_up", w.gate_up[e]), ("down", w.down[e])):
            b = G["blocks"]["%d.%s" % (e, mod)]
            assert np.array_equal(oracle.decode_codes(blk.code8, blk.q), np.array(b["child"], np.uint8))
            assert np.array_equal(oracle.decode_block(blk), np.array(b["W"], np.float64))


def test_golden_routing_and_permutation():
    G, w, a = _golden_layer()
    idx, gw = oracle.route_topk(a.logits, G["top_k"])
    assert idx.tolist() == G["expect_idx"]
    assert np.array_equal(gw, np.array(G["expect_w"]))
    offsets, srt = oracle.permute(idx, G["E"])
    assert offsets.tolist() == G["expect_offsets"]
    assert srt.tolist() == G["expect_sorted"]


def test_golden_ffn_from_hand_intermediates():
    G, w, a = _golden_layer()
    out = oracle.moe_layer(w, a)
    H = G["H"]
    for t in range(2):
        ref = np.zeros(H)
        for j, e in enumerate(G["expect_idx"][t]):
            g, u = G["g_u"]["t%d.e%d" % (t, e)]
            h = g * u / (1.0 + math.exp(-g))
            Wd = np.array(G["blocks"]["%d.down" % e]["W"])
            ref += G["expect_w"][t][j] * Wd[:, 0] * h
        np.testing.assert_allclose(out["y"][t], ref, rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------- decode

def test_truncation_identity_exhaustive():
    """Reading the top k bit-planes (plane 0 = MSB) of every 8-bit code gives code >> (8-k)."""
    codes = np.arange(256, dtype=np.uint8)
    planes = [(codes.astype(np.int64) >> (7 - p)) & 1 for p in range(8)]
    for k in range(1, 9):
        top = np.zeros(256, dtype=np.int64)
        for p in range(k):
            top += planes[p] << (k - 1 - p)
        assert np.array_equal(oracle.decode_codes(codes, k), top.astype(np.uint8)), k


def test_q8_decode_is_direct_parent_lut():
    w, _ = pw_synth.make_small(H=64, I=32, E=1, top_k=1, T=1, q_fixed=8, seed=7)
    for blk in (w.gate_up[0], w.down[0]):
        direct = np.take_along_axis(blk.luts[8].astype(np.float64), blk.code8.astype(np.int64), axis=1)
        assert np.array_equal(oracle.decode_block(blk), direct)


@pytest.mark.parametrize("q", [3, 4, 5, 6, 7, 8])
def test_decode_brute_force_every_code(q):
    """Tiny block whose rows hold each code 0..255 once: pure-Python lookup."""
    rng = np.random.default_rng(q)
    R, K = 3, 256
    code8 = np.stack([rng.permutation(256) for _ in range(R)]).astype(np.uint8)
    luts = pw_synth.draw_luts(rng, R)
    blk = pw_synth.Block(code8=code8, luts=luts, q=q)
    W = oracle.decode_block(blk)
    for r in range(R):
        for c in range(K):
            child = int(code8[r, c]) // (2 ** (8 - q))
            assert W[r, c] == float(luts[q][r, child])


# ---------------------------------------------------------------- routing

def _route_lexsort(logits, k):
    T, E = logits.shape
    idx = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t].astype(np.float64)))
        idx[t] = order[:k]
    return idx


@pytest.mark.parametrize("E,k", [(4, 2), (8, 2), (60, 4), (7, 7), (5, 1)])
def test_route_matches_lexsort_with_ties(E, k):
    rng = np.random.default_rng(E * 10 + k)
    T = 200
    logits = rng.normal(size=(T, E)).astype(np.float32)
    logits[::3] = np.round(logits[::3] * 2) / 2  # many exact ties
    logits[5] = 0.25
    idx, w = oracle.route_topk(logits, k)
    assert np.array_equal(idx, _route_lexsort(logits, k))


def test_gate_weights_softmax_over_selected():
    from scipy.special import softmax
    rng = np.random.default_rng(3)
    logits = rng.normal(size=(50, 16)).astype(np.float32)
    idx, w = oracle.route_topk(logits, 4)
    sel = np.take_along_axis(logits.astype(np.float64), idx.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, softmax(sel, axis=1), rtol=1e-14, atol=0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-15)
    assert np.all(np.diff(w, axis=1) <= 0)  # selected in descending logit order


def test_gate_weights_special_cases():
    logits = np.array([[1.0, 3.0, -2.0]], dtype=np.float32)
    idx, w = oracle.route_topk(logits, 1)
    assert idx.tolist() == [[1]] and w.tolist() == [[1.0]]
    idx, w = oracle.route_topk(np.full((1, 6), 0.75, np.float32), 3)
    assert idx.tolist() == [[0, 1, 2]]
    np.testing.assert_allclose(w, 1.0 / 3.0, rtol=1e-15)


def test_permute_matches_stable_argsort():
    rng = np.random.default_rng(11)
    for T, E, k in [(1, 4, 2), (37, 8, 2), (64, 60, 4), (513, 5, 3)]:
        idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        offsets, srt = oracle.permute(idx, E)
        flat = idx.reshape(-1)
        assert np.array_equal(srt, np.argsort(flat, kind="stable"))
        assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
        assert offsets[-1] == T * k and np.all(np.diff(offsets) >= 0)


# ---------------------------------------------------------------- FFN

def _dense_reference(w, a):
    """Textbook dense SwiGLU MoE on materialised weights (numpy + scipy expit)."""
    from scipy.special import expit
    s = w.shape
    x = a.x.astype(np.float64)
    lg = a.logits.astype(np.float64)
    y = np.zeros((x.shape[0], s.H))
    order = np.argsort(-lg, axis=1, kind="stable")[:, :s.top_k]
    for t in range(x.shape[0]):
        sel = lg[t, order[t]]
        gw = np.exp(sel - sel.max())
        gw /= gw.sum()
        for j, e in enumerate(order[t]):
            Wg = np.take_along_axis(w.gate_up[e].luts[w.gate_up[e].q].astype(np.float64),
                                    (w.gate_up[e].code8 >> (8 - w.gate_up[e].q)).astype(np.int64), axis=1)
            Wd = np.take_along_axis(w.down[e].luts[w.down[e].q].astype(np.float64),
                                    (w.down[e].code8 >> (8 - w.down[e].q)).astype(np.int64), axis=1)
            gu = Wg @ x[t]
            g, u = gu[:s.I], gu[s.I:]
            y[t] += gw[j] * (Wd @ (g * expit(g) * u))
        if s.I_shared:
            Wg = np.take_along_axis(w.shared_gate_up.luts[8].astype(np.float64),
                                    w.shared_gate_up.code8.astype(np.int64), axis=1)
            Wd = np.take_along_axis(w.shared_down.luts[8].astype(np.float64),
                                    w.shared_down.code8.astype(np.int64), axis=1)
            gu = Wg @ x[t]
            g, u = gu[:s.I_shared], gu[s.I_shared:]
            y[t] += Wd @ (g * expit(g) * u)
    return y


@pytest.mark.parametrize("shared", [0, 96])
def test_ffn_matches_dense_numpy(shared):
    w, a = pw_synth.make_small(H=96, I=64, E=6, top_k=3, T=9, I_shared=shared, seed=21 + shared)
    out = oracle.moe_layer(w, a)
    ref = _dense_reference(w, a)
    rel = np.linalg.norm(out["y"] - ref) / np.linalg.norm(ref)
    assert rel <= 1e-12


def test_ffn_token_subset_equals_full():
    w, a = pw_synth.make_small(H=64, I=32, E=4, top_k=2, T=7, seed=5)
    full = oracle.moe_layer(w, a)["y"]
    sub = oracle.moe_layer(w, a, tokens=[6, 0, 3])["y"]
    assert np.array_equal(sub, full[[6, 0, 3]])


def test_ffn_zero_lut_gives_zero():
    w, a = pw_synth.make_small(H=64, I=32, E=3, top_k=2, T=4, seed=9)
    for b in w.gate_up + w.down:
        b.luts = {k: np.zeros_like(v) for k, v in b.luts.items()}
    assert np.all(oracle.moe_layer(w, a)["y"] == 0.0)


def test_ffn_constant_lut_closed_form():
    """Constant LUTs v (gate_up) and vd (down): g = u = v*sum(x),
    h = silu(g)*g for every i, d_o = vd*I*h, y = sum_j w_j d = vd*I*h (sum w = 1)."""
    H, I, E, k, T = 32, 16, 3, 2, 5
    w, a = pw_synth.make_small(H=H, I=I, E=E, top_k=k, T=T, seed=13)
    v, vd = 0.0625, -0.125
    for b in w.gate_up:
        b.luts = {kk: np.full_like(t, v) for kk, t in b.luts.items()}
    for b in w.down:
        b.luts = {kk: np.full_like(t, vd) for kk, t in b.luts.items()}
    y = oracle.moe_layer(w, a)["y"]
    for t in range(T):
        S = float(a.x[t].astype(np.float64).sum())
        g = v * S
        h = g * g / (1.0 + math.exp(-g))
        np.testing.assert_allclose(y[t], vd * I * h, rtol=1e-12, atol=1e-14)


def test_ffn_top1_single_expert_is_plain_swiglu_mlp():
    import torch
    w, a = pw_synth.make_small(H=48, I=40, E=1, top_k=1, T=6, seed=17)
    y = oracle.moe_layer(w, a)["y"]
    Wg = torch.from_numpy(oracle.decode_block(w.gate_up[0]))
    Wd = torch.from_numpy(oracle.decode_block(w.down[0]))
    x = torch.from_numpy(a.x.astype(np.float64))
    gu = x @ Wg.T
    ref = (torch.nn.functional.silu(gu[:, :40]) * gu[:, 40:]) @ Wd.T
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_ffn_linear_in_gate_weights():
    w, a = pw_synth.make_small(H=64, I=32, E=4, top_k=2, T=5, seed=19)
    P = oracle.PreparedLayer(w)
    idx, gw = oracle.route_topk(a.logits, 2)
    y1 = P.ffn(a.x, idx, gw)
    y3 = P.ffn(a.x, idx, 3.0 * gw)
    np.testing.assert_allclose(y3, 3.0 * y1, rtol=1e-13, atol=1e-15)
    only0 = gw.copy()
    only0[:, 1] = 0.0
    only1 = gw.copy()
    only1[:, 0] = 0.0
    np.testing.assert_allclose(P.ffn(a.x, idx, only0) + P.ffn(a.x, idx, only1), y1, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("k", [3, 4, 5, 6, 7])
def test_q_invariance_when_low_bits_are_zero(k):
    """Codes whose low (8-k) bits are zero and LUT_k[v] := LUT_8[v << (8-k)]
    decode identically at width k and width 8, so y is identical."""
    w, a = pw_synth.make_small(H=64, I=32, E=3, top_k=2, T=4, seed=23 + k)
    for b in w.gate_up + w.down:
        b.code8 = (b.code8 >> (8 - k)) << (8 - k)
        b.luts[k] = b.luts[8][:, (np.arange(1 << k) << (8 - k))].copy()
    for b in w.gate_up + w.down:
        b.q = 8
    y8 = oracle.moe_layer(w, a)["y"]
    for b in w.gate_up + w.down:
        b.q = k
    yk = oracle.moe_layer(w, a)["y"]
    assert np.array_equal(y8, yk)
