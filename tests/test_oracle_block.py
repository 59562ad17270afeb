"""The oracle's block-forward functions against their pins, and planted
mistakes that the pins must catch (no GPU)."""
import numpy as np
import pytest

import oracle
from block_pins import attention_pins, block_forward_pins, draft_forward_pins, rmsnorm_pins, silu_gate_pins
from oracle import dspark_oracle
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


def test_block_forward_meets_every_pin():
    failed = [(n, d) for n, ok, d in block_forward_pins(oracle.draft_block_forward) if not ok]
    assert not failed, failed


def test_draft_forward_meets_every_pin():
    failed = [(n, d) for n, ok, d in draft_forward_pins(oracle.draft_forward, oracle.draft_block_forward) if not ok]
    assert not failed, failed


def _block_mutant(kind):
    """The block composed from the oracle's pinned steps with one planted
    mistake in how they are put together."""
    O = dspark_oracle

    def f(h, w, R, B, H, Dh, k_ctx, v_ctx, ctx_len, eps, block_causal=False):
        HD = H * Dh
        h64 = np.asarray(h, np.float32).astype(np.float64)
        x1 = O.rmsnorm(h64, w["ln2" if kind == "ln_swap" else "ln1"], eps)
        qkv = O.gemv(w["qkv"], x1)
        q, k, v = qkv[:, :HD], qkv[:, HD:2 * HD], qkv[:, 2 * HD:]
        if kind == "qk_swap":
            q, k = k, q
        if kind == "v_from_k":
            v = k
        causal = False if kind == "causal_ignored" else block_causal
        a = O.attention_ragged(q, k, v, R, B, H, Dh, k_ctx, v_ctx, ctx_len, causal)
        Wo = w["o"]
        if kind == "o_transposed":
            Wo = np.ascontiguousarray(np.asarray(Wo).T)
        h2 = (0 if kind == "no_res1" else h64) + O.gemv(Wo, a)
        x2 = O.rmsnorm(h64 if kind == "x2_from_h" else h2, w["ln1" if kind == "ln_swap" else "ln2"], eps)
        gu = O.gemv(w["gate_up"], x2)
        F = gu.shape[1] // 2
        if kind == "gate_up_swap":
            gu = np.concatenate([gu[:, F:], gu[:, :F]], axis=1)
        mlp = O.gemv(w["down"], O.silu_gate(gu, F))
        return (h64 if kind == "res2_from_h" else h2) + mlp
    return f


BLOCK_MUTANTS = ["qk_swap", "v_from_k", "causal_ignored", "o_transposed", "no_res1", "x2_from_h", "ln_swap",
                 "gate_up_swap", "res2_from_h"]


@pytest.mark.parametrize("kind", BLOCK_MUTANTS)
def test_block_composition_mutant_is_caught(kind):
    assert any(not ok for _, ok, _ in block_forward_pins(_block_mutant(kind))), kind


def test_block_mutant_harness_is_faithful():
    """Without a planted mistake the hand-composed block is the oracle's."""
    assert not [n for n, ok, _ in block_forward_pins(_block_mutant("none")) if not ok]


def _forward_mutant(kind):
    O = dspark_oracle

    def f(x_in, fc, layers, kcs, vcs, ctx_len, norm, eps, R, B, H, Dh, block_causal=False):
        if kind == "fc_transposed":
            fc = np.ascontiguousarray(np.asarray(fc).T)
        h = O.gemv(fc, x_in)
        order = list(zip(layers, kcs, vcs))
        if kind == "reversed":
            order = order[::-1]
        if kind == "shared_cache" and order:
            order = [(w, kcs[0], vcs[0]) for w, _, _ in order]
        for w, kc, vc in order:
            h = O.draft_block_forward(h.astype(np.float32), w, R, B, H, Dh, kc, vc, ctx_len, eps, block_causal)
        return h if kind == "no_final_norm" else O.rmsnorm(h.astype(np.float32), norm, eps)
    return f


@pytest.mark.parametrize("kind", ["fc_transposed", "reversed", "shared_cache", "no_final_norm"])
def test_forward_composition_mutant_is_caught(kind):
    assert any(not ok for _, ok, _ in draft_forward_pins(_forward_mutant(kind), oracle.draft_block_forward)), kind


def _rms_dropped_mean(x, gamma_bits, eps):
    x64 = np.asarray(x).astype(np.float64)
    return x64 / np.sqrt(np.sum(x64 * x64, axis=-1, keepdims=True) + eps) * bf16_to_f64(gamma_bits)


def _rms_eps_outside(x, gamma_bits, eps):
    x64 = np.asarray(x).astype(np.float64)
    return x64 / (np.sqrt(np.mean(x64 * x64, axis=-1, keepdims=True)) + eps) * bf16_to_f64(gamma_bits)


@pytest.mark.parametrize("name,mutant,pins", [
    ("rmsnorm", _rms_dropped_mean, rmsnorm_pins), ("rmsnorm", _rms_eps_outside, rmsnorm_pins),
    ("attention_ragged", _attn_mutant("no_scale"), attention_pins),
], ids=["rms_sum_for_mean", "rms_eps_outside_root", "attention_dropped_scale"])
def test_block_runs_through_the_pinned_steps(monkeypatch, name, mutant, pins):
    """A mistake planted in one of the pinned steps changes the block's
    output (the block has no private copy of that step), and the step's own
    pins catch it."""
    inp = __import__("gemv_markov_argmax_amd.synth", fromlist=["x"]).block_inputs(2, 3, 2, 16, 48, 10, [4, 10], 19)
    args = (inp["h"], inp["layers"][0], 2, 3, 2, 16, inp["k_ctx"], inp["v_ctx"], inp["ctx_len"], 1e-6)
    good = oracle.draft_block_forward(*args)
    monkeypatch.setattr(dspark_oracle, name, mutant)
    bad = dspark_oracle.draft_block_forward(*args)
    assert not np.allclose(good, bad, rtol=1e-9, atol=1e-12), f"block ignores {name}"
    assert any(not ok for _, ok, _ in pins(mutant)), f"{name} pins miss the mutant"
