"""Plant plausible mistakes in copies of the oracle and check that the pins
catch every one of them (no GPU). A pin set that a dropped term, a wrong sign
or index, a transposed operand or a wrong tie rule could pass would not pin
the oracle."""
import numpy as np
import pytest

import oracle
from oracle.dspark_oracle import _markov_loop, bf16_to_f64, fp16_to_f64
from oracle_pins import gemv_pins, gemv_q8_pins, markov_pins, markov_q8_pins, probe_pins


def _markov_mutant(kind):
    def sample(base, w1_bits, w2_bits, prev0, k, d2t=None):
        base = np.asarray(base, np.float32)
        R, B, V = base.shape
        W1, W2 = bf16_to_f64(w1_bits), bf16_to_f64(w2_bits)
        ids = np.empty((R, k), np.int64)
        tok = np.empty((R, k), np.int64)
        margin = np.empty((R, k))
        for q in range(R):
            prev = int(prev0[q])
            for i in range(k):
                row = base[q, 0] if kind == "base_row0" else base[q, min(i + 1, B - 1)] if kind == "row_shift" else base[q, i]
                e = W1[prev] if kind != "swap_w1_w2" else W2[prev]
                M2 = W2 if kind != "swap_w1_w2" else W1
                bias = M2 @ e
                if kind == "no_bias":
                    bias = 0.0 * bias
                s = row.astype(np.float64) + (-bias if kind == "bias_sign" else bias)
                if kind == "gather_next_row":
                    s = row.astype(np.float64) + M2 @ W1[(prev + 1) % V]
                s32 = s.astype(np.float32)
                t = int(V - 1 - np.argmax(s32[::-1])) if kind == "highest_tie" else int(np.argmax(s32))
                rest = s.copy()
                rest[t] = -np.inf
                tok[q, i], margin[q, i] = t, s[t] - rest.max()
                ids[q, i] = t if d2t is None else int(d2t[t])
                if kind == "no_prev_update":
                    continue
                prev = int(ids[q, i]) if kind == "d2t_prev" else t
        return dict(ids=ids, tok=tok, margin=margin, runner_up=tok)
    return sample


MARKOV_MUTANTS = ["no_prev_update", "highest_tie", "base_row0", "row_shift", "bias_sign",
                  "no_bias", "swap_w1_w2", "gather_next_row", "d2t_prev"]


@pytest.mark.parametrize("kind", MARKOV_MUTANTS)
def test_markov_mutant_is_caught(kind):
    results = markov_pins(_markov_mutant(kind), n_brute=40)
    assert any(not ok for _, ok, _ in results), f"mutant {kind} passed every pin"


def _gemv_mutant(kind):
    def gemv(W_bits, X):
        W = bf16_to_f64(W_bits)
        X64 = np.asarray(X, np.float32).astype(np.float64)
        if kind == "transposed":
            return X64 @ W
        if kind == "drop_last_term":
            return X64[:, :-1] @ W[:, :-1].T
        if kind == "sign":
            return -(X64 @ W.T)
        if kind == "x_rounded_to_bf16":
            from gemv_markov_argmax_amd import synth
            return bf16_to_f64(synth.bf16_bits_rne(X64.astype(np.float32))) @ W.T
        raise AssertionError(kind)
    return gemv


@pytest.mark.parametrize("kind", ["transposed", "drop_last_term", "sign", "x_rounded_to_bf16"])
def test_gemv_mutant_is_caught(kind):
    results = gemv_pins(_gemv_mutant(kind))
    assert any(not ok for _, ok, _ in results), f"mutant {kind} passed every pin"


def _probe_mutant(kind):
    def probe(x, w_bits, bias, threshold):
        x64 = np.asarray(x, np.float32).astype(np.float64)
        w = bf16_to_f64(w_bits)
        logit = x64 @ w
        if kind != "no_bias":
            logit = logit + (-bias if kind == "bias_sign" else bias)
        if kind == "ignore_w":
            logit = x64.sum(axis=1) + bias
        passed = logit > threshold if kind == "strict_gate" else logit >= threshold
        return logit, passed
    return probe


@pytest.mark.parametrize("kind", ["no_bias", "bias_sign", "ignore_w", "strict_gate"])
def test_probe_mutant_is_caught(kind):
    results = probe_pins(_probe_mutant(kind))
    assert any(not ok for _, ok, _ in results), f"mutant {kind} passed every pin"


def _q8_dequant_mutant(kind):
    def deq(q, d_bits):
        q = np.asarray(q, np.int8)
        d_bits = np.asarray(d_bits, np.uint16)
        d = fp16_to_f64(d_bits)
        qv = q.astype(np.uint8).astype(np.float64) if kind == "unsigned_q" else q.astype(np.float64)
        if kind == "scale_as_bf16":
            d = bf16_to_f64(d_bits)
        if kind == "no_scale":
            d = np.ones_like(d)
        if kind == "scale_shift":
            d = np.roll(d, 1, axis=-1)
        K = q.shape[-1]
        idx = np.arange(K) // (16 if kind == "block16" else 32)
        idx = idx % d.shape[-1]
        return qv * d[..., idx]
    return deq


Q8_MUTANTS = ["unsigned_q", "scale_as_bf16", "no_scale", "scale_shift", "block16"]


@pytest.mark.parametrize("kind", Q8_MUTANTS)
def test_gemv_q8_mutant_is_caught(kind):
    deq = _q8_dequant_mutant(kind)

    def gemv_q8(Wq, Wd, X):
        return np.asarray(X, np.float32).astype(np.float64) @ deq(Wq, Wd).T
    results = gemv_q8_pins(gemv_q8)
    assert any(not ok for _, ok, _ in results), f"mutant {kind} passed every pin"


@pytest.mark.parametrize("kind", Q8_MUTANTS)
def test_markov_q8_mutant_is_caught(kind):
    deq = _q8_dequant_mutant(kind)

    def sample(base, w1q, w1d, w2q, w2d, prev0, k, d2t=None):
        return _markov_loop(base, deq(w1q, w1d), deq(w2q, w2d), prev0, k, d2t)
    results = markov_q8_pins(sample, n_brute=30)
    assert any(not ok for _, ok, _ in results), f"mutant {kind} passed every pin"
