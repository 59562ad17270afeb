"""Pins of the oracle's block-forward functions (RMSNorm, SiLU gate,
attention over a ragged context): hand-worked values, closed forms,
invariants and an independent evaluation with the math module, so that a
plausible mistake fails at least one (test_oracle_block.py plants them)."""
from __future__ import annotations

import json
import math
import os

import numpy as np

from gemv_markov_argmax_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "block_hand.json")


def _fx():
    with open(GOLDEN) as f:
        return json.load(f)


def _bits(values):
    a = np.asarray(values, dtype=np.float32)
    b = synth.bf16_bits_rne(a)
    assert np.array_equal((b.astype(np.uint32) << 16).view(np.float32), a), "not exact in bf16"
    return b


def _run(name, fn):
    try:
        ok, detail = fn()
    except Exception as exc:  # a crash is a failed pin
        ok, detail = False, f"raised {type(exc).__name__}: {exc}"
    return (name, bool(ok), detail)


def rmsnorm_pins(rmsnorm):
    pins = []
    fx = _fx()["rmsnorm"]

    def hand():
        bad = []
        for c in fx:
            y = np.asarray(rmsnorm(np.asarray([c["x"]], np.float32), _bits(c["gamma"]), c["eps"]))[0]
            if not np.allclose(y, c["y"], rtol=1e-15, atol=0):
                bad.append((c["derivation"], y.tolist()))
        return not bad, f"{bad}"
    pins.append(_run("hand cases", hand))

    def scale_invariance():
        g = np.random.default_rng(3)
        x = g.standard_normal((3, 40)).astype(np.float32)
        gamma = synth.bf16_bits_rne(g.standard_normal(40).astype(np.float32))
        a = np.asarray(rmsnorm(x, gamma, 0.0))
        b = np.asarray(rmsnorm(x * np.float32(8.0), gamma, 0.0))
        return np.allclose(a, b, rtol=1e-14, atol=0), "rmsnorm(8 x) = rmsnorm(x) at eps = 0"
    pins.append(_run("scale invariance at eps = 0", scale_invariance))

    def independent():
        g = np.random.default_rng(5)
        x = g.standard_normal((2, 24)).astype(np.float32)
        gamma = synth.bf16_bits_rne(g.standard_normal(24).astype(np.float32))
        eps = 1e-5
        y = np.asarray(rmsnorm(x, gamma, eps))
        gv = (gamma.astype(np.uint32) << 16).view(np.float32)
        bad = 0
        for m in range(2):
            row = [float(v) for v in x[m]]
            inv = 1.0 / math.sqrt(math.fsum(v * v for v in row) / len(row) + float(np.float32(eps)))
            for t in range(24):
                bad += abs(y[m, t] - row[t] * inv * float(gv[t])) > 1e-14 * max(1.0, abs(y[m, t]))
        return bad == 0, f"{bad} entries off"
    pins.append(_run("math-module evaluation", independent))
    return pins


def silu_gate_pins(silu_gate):
    pins = []
    fx = _fx()["silu_gate"]

    def hand():
        bad = []
        for c in fx:
            a = float(np.asarray(silu_gate(np.asarray([[c["g"], c["u"]]], np.float32), 1))[0, 0])
            want = c["a"]
            # inputs pass through float32: compare with the definition at those inputs
            g32, u32 = float(np.float32(c["g"])), float(np.float32(c["u"]))
            exact = g32 / (1.0 + math.exp(-g32)) * u32
            if abs(a - exact) > 1e-15 * max(1.0, abs(exact)) or abs(a - want) > 1e-6 * max(1.0, abs(want)):
                bad.append((c["derivation"], a))
        return not bad, f"{bad}"
    pins.append(_run("hand cases (gate first, up second)", hand))

    def limits():
        gu = np.asarray([[60.0, -60.0, 3.0, 3.0]], np.float32)  # g = [60, -60], u = [3, 3]
        a = np.asarray(silu_gate(gu, 2))[0]
        return abs(a[0] - 180.0) < 1e-12 and abs(a[1]) < 1e-20, f"{a.tolist()}"
    pins.append(_run("silu(g) -> g for large g, -> 0 for very negative g", limits))

    def independent():
        g = np.random.default_rng(7)
        gu = (g.standard_normal((3, 20)) * 3).astype(np.float32)
        a = np.asarray(silu_gate(gu, 10))
        bad = 0
        for m in range(3):
            for j in range(10):
                gg, uu = float(gu[m, j]), float(gu[m, 10 + j])
                bad += abs(a[m, j] - gg / (1.0 + math.exp(-gg)) * uu) > 1e-15 * max(1.0, abs(a[m, j]))
        return bad == 0, f"{bad} entries off"
    pins.append(_run("math-module evaluation", independent))
    return pins


def _attn_inputs(seed, R, B, H, Dh, Lmax):
    g = np.random.default_rng(seed)
    q = g.standard_normal((R * B, H * Dh)).astype(np.float32)
    kb = g.standard_normal((R * B, H * Dh)).astype(np.float32)
    vb = g.standard_normal((R * B, H * Dh)).astype(np.float32)
    kc = synth.bf16_bits_rne(g.standard_normal((R, Lmax, H * Dh)).astype(np.float32))
    vc = synth.bf16_bits_rne(g.standard_normal((R, Lmax, H * Dh)).astype(np.float32))
    return q, kb, vb, kc, vc


def attention_pins(attn):
    pins = []
    fx = _fx()["attention"]

    def hand():
        q = np.asarray(fx["q"], np.float32).reshape(2, 1)
        k = np.asarray(fx["k"], np.float32).reshape(2, 1)
        v = np.asarray(fx["v"], np.float32).reshape(2, 1)
        empty = np.zeros((1, 1, 1), np.uint16)
        full = np.asarray(attn(q, k, v, 1, 2, 1, 1, empty, empty, [0], False))[:, 0]
        caus = np.asarray(attn(q, k, v, 1, 2, 1, 1, empty, empty, [0], True))[:, 0]
        ok = np.allclose(full, fx["out_full"], atol=1e-6) and np.allclose(caus, fx["out_causal"], atol=1e-6)
        return ok, f"full {full.tolist()} causal {caus.tolist()}"
    pins.append(_run("hand two-key example, full and causal", hand))

    def single_key():
        q, kb, vb, kc, vc = _attn_inputs(1, 2, 1, 3, 4, 5)
        out = np.asarray(attn(q, kb, vb, 2, 1, 3, 4, kc, vc, [0, 0], False))
        return np.array_equal(out, vb.astype(np.float64)), "one key: output = its value"
    pins.append(_run("a single key returns its value exactly", single_key))

    def equal_keys():
        R, B, H, Dh, L = 1, 2, 2, 4, 6
        q, kb, vb, kc, vc = _attn_inputs(2, R, B, H, Dh, L)
        kc[:] = 0
        kb[:] = 0
        out = np.asarray(attn(q, kb, vb, R, B, H, Dh, kc, vc, [L], False))
        vals = np.concatenate([((vc[0].astype(np.uint32) << 16).view(np.float32)).astype(np.float64), vb.astype(np.float64)])
        want = np.tile(vals.mean(axis=0), (B, 1))
        return np.allclose(out, want, rtol=1e-14, atol=1e-14), "equal scores: the mean of all values"
    pins.append(_run("equal scores give the mean of the values", equal_keys))

    def ragged_mask():
        R, B, H, Dh, Lmax = 2, 3, 2, 8, 10
        q, kb, vb, kc, vc = _attn_inputs(3, R, B, H, Dh, Lmax)
        lens = [4, 7]
        a = np.asarray(attn(q, kb, vb, R, B, H, Dh, kc, vc, lens, False))
        kc2, vc2 = kc.copy(), vc.copy()
        kc2[0, 4:] = synth.bf16_bits_rne(np.full((6, H * Dh), 50.0, np.float32))
        vc2[1, 7:] = synth.bf16_bits_rne(np.full((3, H * Dh), -50.0, np.float32))
        b = np.asarray(attn(q, kb, vb, R, B, H, Dh, kc2, vc2, lens, False))
        kc3 = kc.copy()
        kc3[0, 3] = synth.bf16_bits_rne(np.full(H * Dh, 50.0, np.float32))  # inside the context: must matter
        c = np.asarray(attn(q, kb, vb, R, B, H, Dh, kc3, vc, lens, False))
        return np.array_equal(a, b) and not np.allclose(a[:B], c[:B]), "positions past ctx_len ignored"
    pins.append(_run("context positions past ctx_len are ignored", ragged_mask))

    def permutation():
        R, B, H, Dh, L = 1, 3, 2, 4, 9
        q, kb, vb, kc, vc = _attn_inputs(4, R, B, H, Dh, L)
        a = np.asarray(attn(q, kb, vb, R, B, H, Dh, kc, vc, [L], False))
        perm = np.random.default_rng(0).permutation(L)
        b = np.asarray(attn(q, kb, vb, R, B, H, Dh, kc[:, perm], vc[:, perm], [L], False))
        return np.allclose(a, b, rtol=1e-13, atol=1e-13), "context order does not matter"
    pins.append(_run("context permutation invariance", permutation))

    def independent():
        R, B, H, Dh, L = 1, 3, 2, 4, 5
        q, kb, vb, kc, vc = _attn_inputs(5, R, B, H, Dh, L)
        out = np.asarray(attn(q, kb, vb, R, B, H, Dh, kc, vc, [L], True))
        kcf = (kc.astype(np.uint32) << 16).view(np.float32)
        vcf = (vc.astype(np.uint32) << 16).view(np.float32)
        bad = 0
        for i in range(B):
            for h in range(H):
                sl = slice(h * Dh, (h + 1) * Dh)
                keys = [kcf[0, j, sl] for j in range(L)] + [kb[j, sl] for j in range(i + 1)]
                vals = [vcf[0, j, sl] for j in range(L)] + [vb[j, sl] for j in range(i + 1)]
                sc = [math.fsum(float(a) * float(b) for a, b in zip(q[i, sl], kk)) / math.sqrt(Dh) for kk in keys]
                mx = max(sc)
                ws = [math.exp(x - mx) for x in sc]
                tot = math.fsum(ws)
                for d in range(Dh):
                    want = math.fsum(w * float(vv[d]) for w, vv in zip(ws, vals)) / tot
                    bad += abs(out[i, h * Dh + d] - want) > 1e-13 * max(1.0, abs(want))
        return bad == 0, f"{bad} entries off"
    pins.append(_run("math-module evaluation (causal, with context)", independent))

    def heads_independent():
        R, B, H, Dh, L = 1, 2, 3, 4, 5
        q, kb, vb, kc, vc = _attn_inputs(6, R, B, H, Dh, L)
        a = np.asarray(attn(q, kb, vb, R, B, H, Dh, kc, vc, [L], False))
        q2 = q.copy()
        q2[:, 0:Dh] *= 3  # change head 0 only
        b = np.asarray(attn(q2, kb, vb, R, B, H, Dh, kc, vc, [L], False))
        return np.array_equal(a[:, Dh:], b[:, Dh:]) and not np.allclose(a[:, :Dh], b[:, :Dh]), "heads separate"
    pins.append(_run("heads are independent", heads_independent))
    return pins
