"""Pins of the fp64 oracle: checks against what the pages and mathematics fix,
independent of the oracle's own formulas.

Each ``*_pins`` function runs every pin for one oracle function and returns a
list of (pin name, ok, detail). The same pins are run on deliberately broken
copies of the oracle (test_oracle_mutants.py) to show that each plausible
mistake fails at least one of them.
"""
from __future__ import annotations

import json
import os

import numpy as np

from exact_bruteforce import (exact_argmax, exact_gemv, exact_gemv_q8, exact_markov, exact_markov_values,
                              exact_probe, frac_q8)
from gemv_markov_argmax_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bits(values):
    """bf16 bits of values that must be exactly representable."""
    a = np.asarray(values, dtype=np.float32)
    b = synth.bf16_bits_rne(a)
    back = (b.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(back, a), "fixture value not exact in bf16"
    return b


def _run(name, fn):
    try:
        ok, detail = fn()
    except Exception as exc:  # a crash is a failed pin
        ok, detail = False, f"raised {type(exc).__name__}: {exc}"
    return (name, bool(ok), detail)


# ---------------------------------------------------------------------------
# Markov loop
# ---------------------------------------------------------------------------

def _tiny_markov(seed, V=None, r=None, k=None, R=1):
    g = np.random.default_rng(seed)
    V = V or int(g.integers(2, 65))
    r = r or int(g.integers(1, 9))
    k = k or int(g.integers(1, 5))
    base = g.standard_normal((R, k, V)).astype(np.float32)
    w1 = synth.bf16_bits_rne((g.standard_normal((V, r)) * 0.5).astype(np.float32))
    w2 = synth.bf16_bits_rne((g.standard_normal((V, r)) * 0.5).astype(np.float32))
    prev0 = g.integers(0, V, size=R)
    return base, w1, w2, prev0, k


def markov_pins(markov_sample, n_brute=200):
    pins = []
    fx = _load("markov_hand_3tok.json")
    base = np.asarray(fx["base"], np.float32)
    w1, w2 = _bits(fx["w1"]), _bits(fx["w2"])

    def hand():
        out = markov_sample(base, w1, w2, fx["prev0"], fx["k"])
        ok = np.array_equal(out["ids"], fx["expected_ids"]) and np.allclose(out["margin"], fx["expected_margin"], atol=0)
        return ok, f"ids {out['ids'].tolist()} margin {out['margin'].tolist()}"
    pins.append(_run("hand 3-token example", hand))

    def hand_d2t():
        out = markov_sample(base, w1, w2, fx["prev0"], fx["k"], d2t=np.asarray(fx["d2t"]))
        return np.array_equal(out["ids"], fx["expected_ids_d2t"]), f"ids {out['ids'].tolist()}"
    pins.append(_run("hand example with d2t (prev stays in draft space)", hand_d2t))

    def brute():
        bad = []
        for seed in range(n_brute):
            b, a1, a2, p0, k = _tiny_markov(seed)
            out = markov_sample(b, a1, a2, p0, k)
            ex = exact_markov(b, a1, a2, p0, k)[0]
            for i, (tok, margin, s) in enumerate(ex):
                scale = max(1.0, float(max(abs(x) for x in s)))
                if float(margin) > 1e-6 * scale:
                    if int(out["tok"][0, i]) != tok:
                        bad.append((seed, i, "tok", int(out["tok"][0, i]), tok))
                        break
                elif out["tok"][0, i] not in [v for v in range(len(s)) if s[tok] - s[v] <= 1e-6 * scale]:
                    bad.append((seed, i, "near-tie tok invalid"))
                    break
                if abs(float(out["margin"][0, i]) - float(margin)) > 1e-12 * scale:
                    bad.append((seed, i, "margin", float(out["margin"][0, i]), float(margin)))
                    break
                if int(out["tok"][0, i]) != tok:
                    break  # a legitimate near-tie divergence: later steps differ in prev
        return not bad, f"{len(bad)} mismatching problems, first {bad[:1]}"
    pins.append(_run("exact rational brute force, tiny random problems", brute))

    def zero_w2():
        g = np.random.default_rng(7)
        V, r, k = 50, 4, 4
        b = g.standard_normal((2, k, V)).astype(np.float32)
        w1 = synth.bf16_bits_rne(g.standard_normal((V, r)).astype(np.float32))
        w2 = np.zeros((V, r), np.uint16)
        out = markov_sample(b, w1, w2, np.array([3, 17]), k)
        want = np.stack([[np.argmax(b[q, i]) for i in range(k)] for q in range(2)])
        return np.array_equal(out["ids"], want), f"{out['ids'].tolist()} vs {want.tolist()}"
    pins.append(_run("W2 = 0 reduces to numpy.argmax of each base row", zero_w2))

    def constant_base():
        V, r, k = 9, 3, 3
        b = np.full((1, k, V), 0.75, np.float32)
        out = markov_sample(b, np.ones((V, r), np.uint16) * 0x3F80, np.zeros((V, r), np.uint16), [5], k)
        return np.array_equal(out["ids"], [[0, 0, 0]]) and np.all(out["margin"] == 0), f"{out['ids'].tolist()}"
    pins.append(_run("constant base, W2 = 0: every draft is index 0 with margin 0", constant_base))

    def bigram_walk():
        # r = V and W2 = I: the bias is W1[prev] itself, i.e. greedy decoding
        # of a first-order chain with a full bigram score table.
        g = np.random.default_rng(11)
        V, k = 24, 4
        b = g.standard_normal((1, k, V)).astype(np.float32)
        table = g.standard_normal((V, V)).astype(np.float32)
        w1 = synth.bf16_bits_rne(table)
        eye = _bits(np.eye(V))
        out = markov_sample(b, w1, eye, [6], k)
        tb = (w1.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        prev, want = 6, []
        for i in range(k):
            sc = b[0, i].astype(np.float64) + tb[prev]
            prev = int(np.argmax(sc))
            want.append(prev)
        return np.array_equal(out["ids"][0], want), f"{out['ids'][0].tolist()} vs {want}"
    pins.append(_run("r = V, W2 = I: greedy bigram walk", bigram_walk))

    def rank_one():
        g = np.random.default_rng(13)
        V, k = 40, 3
        b = g.standard_normal((1, k, V)).astype(np.float32)
        w1 = _bits(g.integers(-4, 5, size=(V, 1)))
        w2 = synth.bf16_bits_rne(g.standard_normal((V, 1)).astype(np.float32))
        c = (w1.astype(np.uint32) << 16).view(np.float32)[:, 0].astype(np.float64)
        col = (w2.astype(np.uint32) << 16).view(np.float32)[:, 0].astype(np.float64)
        out = markov_sample(b, w1, w2, [2], k)
        prev, want = 2, []
        for i in range(k):
            prev = int(np.argmax(b[0, i].astype(np.float64) + c[prev] * col))
            want.append(prev)
        return np.array_equal(out["ids"][0], want), f"{out['ids'][0].tolist()} vs {want}"
    pins.append(_run("r = 1: argmax(base_i + c_prev * W2[:, 0])", rank_one))

    def constructed_ties():
        b, a1, a2, p0, ties = synth.markov_inputs(2, 6, 300, 16, seed=5, tie_frac=0.3)
        out = markov_sample(b, a1, a2, p0, 6)
        bad = [(q, i, a, bb, int(out["tok"][q, i])) for (q, i, a, bb) in ties
               if out["tok"][q, i] != a or out["margin"][q, i] != 0.0]
        return bool(ties) and not bad, f"{len(ties)} tie rows, bad {bad[:2]}"
    pins.append(_run("constructed exact ties pick the lower index", constructed_ties))

    def requests_independent():
        b, a1, a2, p0, _ = synth.markov_inputs(3, 4, 200, 8, seed=9)
        out = markov_sample(b, a1, a2, p0, 4)
        ok = all(np.array_equal(out["ids"][q], markov_sample(b[q:q + 1], a1, a2, p0[q:q + 1], 4)["ids"][0])
                 for q in range(3))
        return ok, "batched vs single"
    pins.append(_run("requests are independent", requests_independent))

    def permutation():
        b, a1, a2, p0, _ = synth.markov_inputs(1, 5, 150, 8, seed=21)
        out = markov_sample(b, a1, a2, p0, 5)
        perm = np.random.default_rng(3).permutation(150)
        inv = np.argsort(perm)
        # new index j holds old entry perm[j]
        outp = markov_sample(b[:, :, perm], a1[perm], a2[perm], inv[p0], 5)
        ok = np.array_equal(perm[outp["tok"]], out["tok"]) or np.any(out["margin"] < 1e-9)
        return ok, f"{out['tok'].tolist()} vs {perm[outp['tok']].tolist()}"
    pins.append(_run("vocabulary permutation equivariance", permutation))

    def base_row_of_step():
        # A huge value at a different index in each base row must be drafted
        # at that step whatever the bias.
        V, r, k = 30, 4, 5
        g = np.random.default_rng(17)
        b = g.standard_normal((1, k, V)).astype(np.float32)
        spots = [3, 29, 0, 11, 7]
        for i, v in enumerate(spots):
            b[0, i, v] = 100.0
        w1 = synth.bf16_bits_rne(g.standard_normal((V, r)).astype(np.float32))
        w2 = synth.bf16_bits_rne(g.standard_normal((V, r)).astype(np.float32))
        out = markov_sample(b, w1, w2, [1], k)
        return np.array_equal(out["ids"][0], spots), f"{out['ids'][0].tolist()}"
    pins.append(_run("step i reads base row i", base_row_of_step))
    return pins


# ---------------------------------------------------------------------------
# GEMV (projections, lm_head)
# ---------------------------------------------------------------------------

def gemv_pins(gemv):
    pins = []
    fx = _load("gemv_hand.json")

    def hand():
        y = gemv(_bits(fx["W"]), np.asarray(fx["X"], np.float32))
        return np.array_equal(y, fx["expected_Y"]), f"{np.asarray(y).tolist()}"
    pins.append(_run("hand 2x3 example", hand))

    def identity():
        g = np.random.default_rng(1)
        X = g.standard_normal((5, 33)).astype(np.float32)
        y = gemv(_bits(np.eye(33)), X)
        return np.array_equal(y, X.astype(np.float64)), "W = I gives Y = X"
    pins.append(_run("W = I returns X exactly", identity))

    def brute():
        bad = 0
        for seed in range(60):
            g = np.random.default_rng(seed)
            M, N, K = int(g.integers(1, 5)), int(g.integers(1, 9)), int(g.integers(1, 17))
            X = g.standard_normal((M, K)).astype(np.float32)
            W = synth.bf16_bits_rne((g.standard_normal((N, K)) * 0.3).astype(np.float32))
            y = np.asarray(gemv(W, X))
            ex = exact_gemv(W.tolist(), X.tolist())
            Wf = (W.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            mag = np.abs(X.astype(np.float64)) @ np.abs(Wf).T
            err = np.abs(y - np.array([[float(v) for v in row] for row in ex]))
            bad += int(np.any(err > 1e-14 * np.maximum(mag, 1e-300) + 1e-300))
        return bad == 0, f"{bad} problems off the exact value"
    pins.append(_run("exact rational brute force, tiny random problems", brute))

    def one_hot_rows():
        g = np.random.default_rng(2)
        X = g.standard_normal((3, 20)).astype(np.float32)
        W = np.zeros((4, 20), np.float32)
        cols = [0, 19, 7, 7]
        for n, c in enumerate(cols):
            W[n, c] = 1.0
        y = gemv(_bits(W), X)
        return np.array_equal(y, X[:, cols].astype(np.float64)), "one-hot weight rows select columns"
    pins.append(_run("one-hot weight rows select activation columns", one_hot_rows))
    return pins


# ---------------------------------------------------------------------------
# Probe
# ---------------------------------------------------------------------------

def probe_pins(conf_probe):
    pins = []
    fx = _load("probe_hand.json")

    def hand():
        bad = []
        for c in fx["cases"]:
            logit, ok = conf_probe(np.asarray([c["x"]], np.float32), _bits(c["w"]), c["bias"], c["threshold"])
            if float(logit[0]) != c["logit"] or bool(ok[0]) != c["pass"]:
                bad.append((c["derivation"], float(logit[0]), bool(ok[0])))
        return not bad, f"{bad}"
    pins.append(_run("hand cases incl. logit exactly at the threshold", hand))

    def one_hot():
        g = np.random.default_rng(4)
        x = g.standard_normal((6, 64)).astype(np.float32)
        w = np.zeros(64, np.float32)
        w[37] = 1.0
        logit, _ = conf_probe(x, _bits(w), 0.5, 0.0)
        return np.array_equal(logit, x[:, 37].astype(np.float64) + 0.5), "one-hot w gives x[:, j] + bias"
    pins.append(_run("one-hot weight gives x[m, j] + bias", one_hot))

    def brute():
        bad = 0
        for seed in range(40):
            g = np.random.default_rng(100 + seed)
            M, D = int(g.integers(1, 4)), int(g.integers(1, 40))
            x = g.standard_normal((M, D)).astype(np.float32)
            w = synth.bf16_bits_rne((g.standard_normal(D) * 0.1).astype(np.float32))
            bias = float(np.float32(g.standard_normal()))
            logit, ok = conf_probe(x, w, bias, 0.0)
            ex = exact_probe(x.tolist(), w.tolist(), bias)
            for m in range(M):
                if abs(float(logit[m]) - float(ex[m])) > 1e-13 * max(1.0, abs(float(ex[m]))):
                    bad += 1
                if bool(ok[m]) != (ex[m] >= 0):
                    bad += 1
        return bad == 0, f"{bad} mismatches"
    pins.append(_run("exact rational brute force", brute))
    return pins


# ---------------------------------------------------------------------------
# Q8_0 weights: the GEMV and the Markov loop
# ---------------------------------------------------------------------------

def _q8_rows(nonzero, K):
    q = np.zeros((len(nonzero), K), np.int8)
    for n, pairs in enumerate(nonzero):
        for j, v in pairs:
            q[n, j] = v
    return q


def _hex16(vals):
    return np.array([int(v, 16) for v in vals], np.uint16)


def _rand_q8(g, rows, K, d_kind="mixed"):
    q = g.integers(-128, 128, size=(rows, K)).astype(np.int8)
    nb = K // 32
    if d_kind == "one":
        d = np.full((rows, nb), 0x3C00, np.uint16)
    else:  # finite binary16 patterns of either sign, normals and subnormals
        e = g.integers(0, 31, size=(rows, nb))
        f = g.integers(0, 1024, size=(rows, nb))
        sgn = g.integers(0, 2, size=(rows, nb))
        d = ((sgn << 15) | (e << 10) | f).astype(np.uint16)
    return q, d


def gemv_q8_pins(gemv_q8, gemv_bf16=None):
    pins = []
    fx = _load("q8_hand.json")
    gx = fx["gemv"]

    def hand():
        K = gx["K"]
        Wq = _q8_rows(gx["W_q_nonzero"], K)
        Wd = np.stack([_hex16(r) for r in gx["W_d_bits"]])
        X = np.zeros((2, K), np.float32)
        for j, v in gx["X_nonzero"][0]:
            X[0, j] = v
        X[1, :] = 1.0
        y = gemv_q8(Wq, Wd, X)
        return np.array_equal(y, gx["expected_Y"]), f"{np.asarray(y).tolist()}"
    pins.append(_run("hand two-block example (scales per 32-entry block, signed quants)", hand))

    def fp16_scales():
        bad = []
        for bits, val, why in fx["fp16"]["cases"]:
            q = np.zeros((1, 32), np.int8)
            q[0, 0] = 1
            y = gemv_q8(q, _hex16([bits]).reshape(1, 1), np.ones((1, 32), np.float32))
            got = float(np.asarray(y)[0, 0])
            if got != val:  # (a zero scale gives a zero sum, whose sign the pin leaves open)
                bad.append((bits, got, val))
        return not bad, f"{bad}"
    pins.append(_run("binary16 scales decode to their IEEE 754 values", fp16_scales))

    def block_boundary():
        K = 96
        X = np.arange(1, K + 1, dtype=np.float32).reshape(1, K)
        Wd = _hex16(["0x3c00", "0x4000", "0x4400"]).reshape(1, 3)  # 1, 2, 4
        want = {0: 1.0, 31: 32.0, 32: 2 * 33.0, 63: 2 * 64.0, 64: 4 * 65.0, 95: 4 * 96.0}
        bad = []
        for j, v in want.items():
            q = np.zeros((1, K), np.int8)
            q[0, j] = 1
            got = float(np.asarray(gemv_q8(q, Wd, X))[0, 0])
            if got != v:
                bad.append((j, got, v))
        return not bad, f"{bad}"
    pins.append(_run("entries 32b..32b+31 take scale b", block_boundary))

    def brute():
        bad = 0
        for seed in range(40):
            g = np.random.default_rng(500 + seed)
            M, N, K = int(g.integers(1, 4)), int(g.integers(1, 5)), 32 * int(g.integers(1, 3))
            X = g.standard_normal((M, K)).astype(np.float32)
            q, d = _rand_q8(g, N, K)
            y = np.asarray(gemv_q8(q, d, X))
            ex = exact_gemv_q8(q.tolist(), d.tolist(), X.tolist())
            Wf = np.array([[float(v) for v in frac_q8(q[n], d[n])] for n in range(N)])
            mag = np.abs(X.astype(np.float64)) @ np.abs(Wf).T
            err = np.abs(y - np.array([[float(v) for v in row] for row in ex]))
            bad += int(np.any(err > 1e-14 * np.maximum(mag, 1e-300) + 1e-300))
        return bad == 0, f"{bad} problems off the exact value"
    pins.append(_run("exact rational brute force, tiny random Q8_0 problems", brute))

    if gemv_bf16 is not None:
        def unit_scales():
            g = np.random.default_rng(9)
            q, d = _rand_q8(g, 6, 64, "one")
            X = g.standard_normal((3, 64)).astype(np.float32)
            wb = _bits(q.astype(np.float32))  # small integers are exact in bf16
            return np.allclose(gemv_q8(q, d, X), gemv_bf16(wb, X), rtol=1e-14, atol=0), "d = 1 vs bf16 weights q"
        pins.append(_run("unit scales reduce to the bf16 GEMV on weights q", unit_scales))
    return pins


def markov_q8_pins(markov_sample_q8, markov_sample_bf16=None, n_brute=60):
    pins = []
    fx = _load("markov_hand_3tok.json")
    d_half = int(_load("q8_hand.json")["markov"]["d_bits"], 16)

    def q8_of(w):
        w = np.asarray(w, np.float64)
        q = np.zeros((w.shape[0], 32), np.int8)
        q[:, : w.shape[1]] = (2 * w).astype(np.int8)
        return q, np.full((w.shape[0], 1), d_half, np.uint16)

    def hand():
        base = np.asarray(fx["base"], np.float32)
        (q1, d1), (q2, d2) = q8_of(fx["w1"]), q8_of(fx["w2"])
        out = markov_sample_q8(base, q1, d1, q2, d2, fx["prev0"], fx["k"])
        ok = np.array_equal(out["ids"], fx["expected_ids"]) and np.array_equal(out["margin"], fx["expected_margin"])
        out2 = markov_sample_q8(base, q1, d1, q2, d2, fx["prev0"], fx["k"], d2t=np.asarray(fx["d2t"]))
        ok = ok and np.array_equal(out2["ids"], fx["expected_ids_d2t"])
        return ok, f"ids {out['ids'].tolist()} margin {out['margin'].tolist()}"
    pins.append(_run("hand 3-token example in Q8_0 form", hand))

    def brute():
        bad = []
        for seed in range(n_brute):
            g = np.random.default_rng(900 + seed)
            V, k, r = int(g.integers(2, 40)), int(g.integers(1, 4)), 32 * int(g.integers(1, 3))
            base = g.standard_normal((1, k, V)).astype(np.float32)
            q1, d1 = _rand_q8(g, V, r)
            q2, d2 = _rand_q8(g, V, r)
            # keep the scores in a modest range: scales 2^-12 .. 2^-6
            d1 = ((g.integers(3, 9, size=d1.shape) << 10) | (d1 & 0x83FF)).astype(np.uint16)
            d2 = ((g.integers(3, 9, size=d2.shape) << 10) | (d2 & 0x83FF)).astype(np.uint16)
            p0 = g.integers(0, V, size=1)
            out = markov_sample_q8(base, q1, d1, q2, d2, p0, k)
            W1f = [frac_q8(q1[v], d1[v]) for v in range(V)]
            W2f = [frac_q8(q2[v], d2[v]) for v in range(V)]
            ex = exact_markov_values(base.tolist(), W1f, W2f, p0, k)[0]
            for i, (tok, margin, sc) in enumerate(ex):
                scale = max(1.0, float(max(abs(x) for x in sc)))
                if float(margin) > 1e-6 * scale and int(out["tok"][0, i]) != tok:
                    bad.append((seed, i, int(out["tok"][0, i]), tok))
                    break
                if abs(float(out["margin"][0, i]) - float(margin)) > 1e-12 * scale:
                    bad.append((seed, i, "margin"))
                    break
                if int(out["tok"][0, i]) != tok:
                    break
        return not bad, f"{len(bad)} mismatching problems, first {bad[:1]}"
    pins.append(_run("exact rational brute force, tiny random Q8_0 problems", brute))

    def block_scales():
        # r = 64, W1[prev] = 1 everywhere with scales (1, 1); W2 row v holds a
        # single quant 1 at column c_v, scales (1, 8): the bias of row v is 1
        # when c_v < 32 and 8 otherwise, so the draft is the row with c_v in
        # the second block.
        V, r = 6, 64
        cols = [0, 31, 33, 30, 5, 12]
        q2 = np.zeros((V, r), np.int8)
        for v, c in enumerate(cols):
            q2[v, c] = 1
        d2 = np.tile(_hex16(["0x3c00", "0x4800"]), (V, 1))
        q1 = np.ones((V, r), np.int8)
        d1 = np.tile(_hex16(["0x3c00", "0x3c00"]), (V, 1))
        base = np.zeros((1, 1, V), np.float32)
        out = markov_sample_q8(base, q1, d1, q2, d2, [0], 1)
        return int(out["tok"][0, 0]) == 2 and float(out["margin"][0, 0]) == 7.0, f"{out['tok'].tolist()} {out['margin'].tolist()}"
    pins.append(_run("the second 32-entry block takes the second scale", block_scales))

    if markov_sample_bf16 is not None:
        def unit_scales():
            b, _, _, p0, _ = synth.markov_inputs(2, 4, 120, 32, seed=31)
            g = np.random.default_rng(41)
            q1, d1 = _rand_q8(g, 120, 32, "one")
            q2, d2 = _rand_q8(g, 120, 32, "one")
            q1 = (q1 // 16).astype(np.int8)  # small bias terms: scores stay comparable to the base
            q2 = (q2 // 16).astype(np.int8)
            a = markov_sample_q8(b, q1, d1, q2, d2, p0, 4)
            c = markov_sample_bf16(b, _bits(q1.astype(np.float32)), _bits(q2.astype(np.float32)), p0, 4)
            return np.array_equal(a["ids"], c["ids"]) and np.array_equal(a["margin"], c["margin"]), "d = 1 vs bf16"
        pins.append(_run("unit scales reduce to the bf16 loop on weights q", unit_scales))
    return pins


__all__ = ["markov_pins", "gemv_pins", "probe_pins", "gemv_q8_pins", "markov_q8_pins", "exact_argmax"]
