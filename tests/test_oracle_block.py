"""The oracle's block-forward functions against their pins, and planted
mistakes that the pins must catch (no GPU)."""
import numpy as np
import pytest

import oracle
from block_pins import attention_pins, rmsnorm_pins, silu_gate_pins
from oracle.dspark_oracle import bf16_to_f64


@pytest.mark.parametrize("suite,fn", [(rmsnorm_pins, oracle.rmsnorm), (silu_gate_pins, oracle.silu_gate),
                                      (attention_pins, oracle.attention_ragged)],
                         ids=["rmsnorm", "silu_gate", "attention_ragged"])
def test_block_oracle_meets_every_pin(suite, fn):
    failed = [(n, d) for n, ok, d in suite(fn) if not ok]
    assert not failed, failed


def _rms_mutant(kind):
    def f(x, gamma_bits, eps):
        x64 = np.asarray(x, np.float32).astype(np.float64)
        g = bf16_to_f64(gamma_bits)
        ms = np.sum(x64 * x64, axis=-1, keepdims=True) if kind == "sum" else np.mean(x64 * x64, axis=-1, keepdims=True)
        den = np.sqrt(ms) + eps if kind == "eps_outside" else np.sqrt(ms + eps)
        y = x64 / den
        return y if kind == "no_gamma" else y * g
    return f


@pytest.mark.parametrize("kind", ["sum", "eps_outside", "no_gamma"])
def test_rmsnorm_mutant_is_caught(kind):
    assert any(not ok for _, ok, _ in rmsnorm_pins(_rms_mutant(kind))), kind


def _silu_mutant(kind):
    def f(gu, F):
        gu64 = np.asarray(gu, np.float32).astype(np.float64)
        g, u = gu64[:, :F], gu64[:, F:2 * F]
        if kind == "swap":
            g, u = u, g
        sig = 1.0 / (1.0 + np.exp(-g))
        return sig * u if kind == "sigmoid_only" else g * sig * u if kind != "tanh" else np.tanh(g) * u
    return f


@pytest.mark.parametrize("kind", ["swap", "sigmoid_only", "tanh"])
def test_silu_gate_mutant_is_caught(kind):
    assert any(not ok for _, ok, _ in silu_gate_pins(_silu_mutant(kind))), kind


def _attn_mutant(kind):
    def f(q, k_blk, v_blk, R, B, H, Dh, k_ctx_bits, v_ctx_bits, ctx_len, block_causal=False):
        q64 = np.asarray(q, np.float32).astype(np.float64).reshape(R, B, H, Dh)
        kb = np.asarray(k_blk, np.float32).astype(np.float64).reshape(R, B, H, Dh)
        vb = np.asarray(v_blk, np.float32).astype(np.float64).reshape(R, B, H, Dh)
        kc = bf16_to_f64(k_ctx_bits)
        Lmax = kc.shape[1]
        kc = kc.reshape(R, Lmax, H, Dh)
        vc = bf16_to_f64(v_ctx_bits).reshape(R, Lmax, H, Dh)
        out = np.empty((R, B, H, Dh))
        for r in range(R):
            L = Lmax if kind == "ignore_len" else int(ctx_len[r])
            for i in range(B):
                nb = (i if kind == "causal_off_by_one" else i + 1) if block_causal else B
                if kind == "no_block":
                    nb = 0 if L > 0 else nb
                for h in range(H):
                    keys = np.concatenate([kc[r, :L, h], kb[r, :nb, h]])
                    vals = np.concatenate([vc[r, :L, h], vb[r, :nb, h]])
                    if len(keys) == 0:
                        out[r, i, h] = 0
                        continue
                    s = keys @ q64[r, i, h] / (1.0 if kind == "no_scale" else np.sqrt(Dh))
                    w = np.exp(s - s.max())
                    out[r, i, h] = (w / (1.0 if kind == "no_normalize" else w.sum())) @ vals
        return out.reshape(R * B, H * Dh)
    return f


@pytest.mark.parametrize("kind", ["ignore_len", "causal_off_by_one", "no_block", "no_scale", "no_normalize"])
def test_attention_mutant_is_caught(kind):
    assert any(not ok for _, ok, _ in attention_pins(_attn_mutant(kind))), kind


def test_block_forward_pins():
    """The composed block: with o and down zero it returns h exactly (the
    residual path); the MLP branch is linear in W_down (doubling W_down
    doubles h3 - h2, with h2 the output at W_down = 0); the attention branch
    does not see W_down."""
    from gemv_markov_argmax_amd import synth
    inp = synth.block_inputs(2, 3, 2, 16, 48, 10, [4, 10], 11)
    w = dict(inp["layers"][0])
    args = (2, 3, 2, 16, inp["k_ctx"], inp["v_ctx"], inp["ctx_len"], 1e-6)
    zero = dict(w, o=np.zeros_like(w["o"]), down=np.zeros_like(w["down"]))
    y0 = oracle.draft_block_forward(inp["h"], zero, *args)
    assert np.array_equal(y0, inp["h"].astype(np.float64))
    nodown = dict(w, down=np.zeros_like(w["down"]))
    h2 = oracle.draft_block_forward(inp["h"], nodown, *args)
    y1 = oracle.draft_block_forward(inp["h"], w, *args)
    dbl = synth.bf16_bits_rne(((w["down"].astype(np.uint32) << 16).view(np.float32) * 2).astype(np.float32))
    y2 = oracle.draft_block_forward(inp["h"], dict(w, down=dbl), *args)
    assert np.allclose(y2 - h2, 2 * (y1 - h2), rtol=1e-12, atol=1e-12)


def test_draft_forward_pins():
    """The drafter's forward: with fc the identity and no blocks it is the
    final rmsnorm of its input; a block whose o and down are zero passes its
    input through, so prepending one changes nothing, and the blocks after it
    still read their own context caches in order; the output is linear in the
    final norm's gain."""
    from gemv_markov_argmax_amd import synth
    R, B, H, Dh, F, Lmax = 2, 3, 2, 8, 24, 6
    inp = synth.draft_forward_inputs(R, B, H, Dh, F, Lmax, [6, 2], layers=2, n_fc=1, seed=21)
    d = H * Dh
    eye = synth.bf16_bits_rne(np.eye(d, dtype=np.float32))
    x = inp["x_in"]
    y = oracle.draft_forward(x, eye, [], [], [], inp["ctx_len"], inp["norm"], 1e-6, R, B, H, Dh)
    assert np.array_equal(y, oracle.rmsnorm(x, inp["norm"], 1e-6))
    w0, w1 = inp["layers"]
    ident = dict(w0, o=np.zeros_like(w0["o"]), down=np.zeros_like(w0["down"]))
    args = (inp["ctx_len"], inp["norm"], 1e-6, R, B, H, Dh)
    one = oracle.draft_forward(x, inp["fc"], [w1], [inp["k_ctx"][1]], [inp["v_ctx"][1]], *args)
    two = oracle.draft_forward(x, inp["fc"], [ident, w1], inp["k_ctx"], inp["v_ctx"], *args)
    assert np.array_equal(one, two)
    swapped = oracle.draft_forward(x, inp["fc"], [ident, w1], inp["k_ctx"][::-1], inp["v_ctx"][::-1], *args)
    assert not np.allclose(one, swapped)
    dbl = synth.bf16_bits_rne(2 * (inp["norm"].astype(np.uint32) << 16).view(np.float32))
    twice = oracle.draft_forward(x, inp["fc"], [w1], [inp["k_ctx"][1]], [inp["v_ctx"][1]], inp["ctx_len"], dbl,
                                 1e-6, R, B, H, Dh)
    assert np.array_equal(twice, 2 * one)


def test_block_forward_norm_placement():
    """Each norm gain feeds only its own branch: with W_o = 0 the block is
    h + MLP(rmsnorm(h, ln2)) and must not depend on ln1; with W_down = 0 it
    is h + attention(rmsnorm(h, ln1)) W_o and must not depend on ln2; and each
    gain does change its own branch."""
    from gemv_markov_argmax_amd import synth
    inp = synth.block_inputs(2, 3, 2, 16, 48, 10, [4, 10], 13)
    w = dict(inp["layers"][0])
    args = (2, 3, 2, 16, inp["k_ctx"], inp["v_ctx"], inp["ctx_len"], 1e-6)
    other = synth.bf16_bits_rne(np.linspace(0.5, 1.5, w["ln1"].shape[0]).astype(np.float32))
    no_o = dict(w, o=np.zeros_like(w["o"]))
    a = oracle.draft_block_forward(inp["h"], no_o, *args)
    assert np.array_equal(a, oracle.draft_block_forward(inp["h"], dict(no_o, ln1=other), *args))
    assert not np.allclose(a, oracle.draft_block_forward(inp["h"], dict(no_o, ln2=other), *args))
    no_down = dict(w, down=np.zeros_like(w["down"]))
    b = oracle.draft_block_forward(inp["h"], no_down, *args)
    assert np.array_equal(b, oracle.draft_block_forward(inp["h"], dict(no_down, ln2=other), *args))
    assert not np.allclose(b, oracle.draft_block_forward(inp["h"], dict(no_down, ln1=other), *args))
