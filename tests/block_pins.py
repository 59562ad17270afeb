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


# ---------------------------------------------------------------------------
# The composed block and the drafter's forward
# ---------------------------------------------------------------------------

def _bf_vals(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _cyclic(n):
    """bf16 bits of the permutation matrix P with P[a, (a + 1) % n] = 1: y = x P^T
    gives y[a] = x[(a + 1) % n] (its transpose shifts the other way)."""
    p = np.zeros((n, n), np.float32)
    p[np.arange(n), (np.arange(n) + 1) % n] = 1.0
    return synth.bf16_bits_rne(p)


def block_forward_pins(block):
    """Pins of the draft block as a composition (the function under test takes
    (h, w, R, B, H, Dh, k_ctx, v_ctx, ctx_len, eps, block_causal)). Each pin
    is a closed form or an invariant that the block's structure fixes:
    residual paths, which slice of the qkv projection plays which role,
    which half of gate_up is gated, where each norm sits and what the MLP
    reads."""
    pins = []
    R, B, H, Dh, F, Lmax = 2, 3, 2, 8, 24, 10
    lens = [4, 10]
    HD = H * Dh

    def fresh(seed):
        inp = synth.block_inputs(R, B, H, Dh, F, Lmax, lens, seed)
        return inp, dict(inp["layers"][0])

    def run(inp, w, causal=False):
        return np.asarray(block(inp["h"], w, R, B, H, Dh, inp["k_ctx"], inp["v_ctx"], inp["ctx_len"], 1e-6, causal))

    def zeros_like(a):
        return np.zeros_like(np.asarray(a))

    def residual():
        inp, w = fresh(11)
        y = run(inp, dict(w, o=zeros_like(w["o"]), down=zeros_like(w["down"])))
        return np.array_equal(y, inp["h"].astype(np.float64)), "o = down = 0 returns h exactly"
    pins.append(_run("residual path: o and down zero return h", residual))

    def uniform_attention():
        # q rows zero: every score is 0, so each position averages its values
        # evenly; v rows zero: the block's own values are 0, so the average is
        # the sum of the request's first ctx_len context values over the
        # number of keys (ctx_len + B, or ctx_len + i + 1 when causal). o is a
        # cyclic permutation and down is zero: y[:, a] = h[:, a] + avg[:, a + 1].
        inp, w = fresh(12)
        qkv = np.asarray(w["qkv"]).copy()
        qkv[:HD] = 0
        qkv[2 * HD:] = 0
        w2 = dict(w, qkv=qkv, o=_cyclic(HD), down=zeros_like(w["down"]))
        vc = _bf_vals(inp["v_ctx"])
        bad = []
        for causal in (False, True):
            y = run(inp, w2, causal)
            want = inp["h"].astype(np.float64).copy()
            for r in range(R):
                L = lens[r]
                for i in range(B):
                    nk = L + (i + 1 if causal else B)
                    avg = vc[r, :L].sum(axis=0) / nk
                    want[r * B + i] += np.roll(avg, -1)
            if not np.allclose(y, want, rtol=1e-13, atol=1e-13):
                bad.append((causal, float(np.abs(y - want).max())))
        return not bad, f"{bad}"
    pins.append(_run("uniform attention: ctx values averaged over all keys, o applied as W_o", uniform_attention))

    def query_rows_alone_see_keys():
        # With the q rows zero the output cannot depend on the k rows or on
        # the context keys; with them nonzero it does.
        inp, w = fresh(13)
        qkv = np.asarray(w["qkv"]).copy()
        qkv[:HD] = 0
        w0 = dict(w, qkv=qkv)
        a = run(inp, w0)
        qkv2 = qkv.copy()
        qkv2[HD:2 * HD] = synth.bf16_bits_rne(2 * _bf_vals(qkv[HD:2 * HD]).astype(np.float32))
        b = run(inp, dict(w, qkv=qkv2))
        inp2 = dict(inp, k_ctx=synth.bf16_bits_rne((-_bf_vals(inp["k_ctx"])).astype(np.float32)))
        c = run(inp2, w0)
        d_full, e_full = run(inp, w), run(inp2, w)
        return (np.allclose(a, b, rtol=1e-13, atol=1e-13) and np.allclose(a, c, rtol=1e-13, atol=1e-13)
                and not np.allclose(d_full, e_full)), "q = 0: no dependence on k rows or context keys"
    pins.append(_run("the first third of qkv is the query", query_rows_alone_see_keys))

    def up_half_is_linear():
        # With o zero the block is h + MLP(h); the MLP is linear in the up
        # rows (second half of gate_up) and not in the gate rows.
        inp, w = fresh(14)
        w0 = dict(w, o=zeros_like(w["o"]))
        gu = _bf_vals(w["gate_up"])
        base = run(inp, w0) - inp["h"].astype(np.float64)
        up2, gate2 = gu.copy(), gu.copy()
        up2[F:] *= 2
        gate2[:F] *= 2
        mu = run(inp, dict(w0, gate_up=synth.bf16_bits_rne(up2.astype(np.float32)))) - inp["h"].astype(np.float64)
        mg = run(inp, dict(w0, gate_up=synth.bf16_bits_rne(gate2.astype(np.float32)))) - inp["h"].astype(np.float64)
        return (np.allclose(mu, 2 * base, rtol=1e-12, atol=1e-12)
                and not np.allclose(mg, 2 * base, rtol=1e-6, atol=1e-9)), "up half linear, gate half not"
    pins.append(_run("gate_up: the second half is the linear (up) factor", up_half_is_linear))

    def mlp_linear_in_down():
        inp, w = fresh(15)
        h2 = run(inp, dict(w, down=zeros_like(w["down"])))
        y1 = run(inp, w)
        dbl = synth.bf16_bits_rne((_bf_vals(w["down"]) * 2).astype(np.float32))
        y2 = run(inp, dict(w, down=dbl))
        return np.allclose(y2 - h2, 2 * (y1 - h2), rtol=1e-12, atol=1e-12), "MLP branch linear in W_down"
    pins.append(_run("the MLP branch is linear in W_down", mlp_linear_in_down))

    def norm_placement():
        inp, w = fresh(16)
        other = synth.bf16_bits_rne(np.linspace(0.5, 1.5, w["ln1"].shape[0]).astype(np.float32))
        no_o = dict(w, o=zeros_like(w["o"]))
        a = run(inp, no_o)
        no_down = dict(w, down=zeros_like(w["down"]))
        b = run(inp, no_down)
        ok = (np.array_equal(a, run(inp, dict(no_o, ln1=other)))
              and not np.allclose(a, run(inp, dict(no_o, ln2=other)))
              and np.array_equal(b, run(inp, dict(no_down, ln2=other)))
              and not np.allclose(b, run(inp, dict(no_down, ln1=other))))
        return ok, "ln1 feeds only the attention branch, ln2 only the MLP"
    pins.append(_run("each norm gain feeds only its own branch", norm_placement))

    def mlp_reads_attention_output():
        # y = h + A + MLP(h + A): not the sum of the branches taken apart.
        inp, w = fresh(17)
        h = inp["h"].astype(np.float64)
        A = run(inp, dict(w, down=zeros_like(w["down"]))) - h
        M0 = run(inp, dict(w, o=zeros_like(w["o"]))) - h
        y = run(inp, w)
        return not np.allclose(y, h + A + M0, rtol=1e-9, atol=1e-12), "MLP input includes the attention output"
    pins.append(_run("the MLP reads the residual after the attention", mlp_reads_attention_output))
    return pins


def draft_forward_pins(fwd, block):
    """Pins of the drafter's forward (fc, blocks in order, final norm); the
    function under test takes (x_in, fc, layers, k_ctx_list, v_ctx_list,
    ctx_len, norm, eps, R, B, H, Dh). ``block`` is the (separately pinned)
    single-block forward, used to state that blocks apply one after the
    other."""
    pins = []
    R, B, H, Dh, F, Lmax = 2, 3, 2, 8, 24, 6
    inp = synth.draft_forward_inputs(R, B, H, Dh, F, Lmax, [6, 2], layers=2, n_fc=1, seed=21)
    d = H * Dh
    x = inp["x_in"]
    ones = synth.bf16_bits_rne(np.ones(d, np.float32))
    w0, w1 = inp["layers"]
    ident = dict(w0, o=np.zeros_like(w0["o"]), down=np.zeros_like(w0["down"]))
    tail = (inp["ctx_len"], inp["norm"], 1e-6, R, B, H, Dh)

    def f(*a, **k):
        return np.asarray(fwd(*a, **k))

    def no_blocks_is_final_norm():
        # fc = I, no blocks, unit gain: every row is scaled to unit RMS and
        # keeps its direction.
        eye = synth.bf16_bits_rne(np.eye(d, dtype=np.float32))
        y = f(x, eye, [], [], [], inp["ctx_len"], ones, 0.0, R, B, H, Dh)
        x64 = x.astype(np.float64)
        rms = np.sqrt((y * y).mean(axis=1))
        cos = (y * x64).sum(axis=1) / (np.linalg.norm(y, axis=1) * np.linalg.norm(x64, axis=1))
        return np.allclose(rms, 1.0, rtol=1e-13) and np.allclose(cos, 1.0, rtol=1e-13), "unit RMS, same direction"
    pins.append(_run("fc = I with no blocks: the final norm of the input", no_blocks_is_final_norm))

    def fc_orientation():
        # fc = cyclic P: h = x P^T, i.e. h[:, a] = x[:, a + 1]; with unit gain
        # the norm commutes with the permutation.
        eye = synth.bf16_bits_rne(np.eye(d, dtype=np.float32))
        y = f(x, _cyclic(d), [], [], [], inp["ctx_len"], ones, 1e-6, R, B, H, Dh)
        z = f(np.roll(x, -1, axis=1), eye, [], [], [], inp["ctx_len"], ones, 1e-6, R, B, H, Dh)
        return np.array_equal(y, z), "h = x fc^T"
    pins.append(_run("fc is applied as x fc^T", fc_orientation))

    def identity_block_and_cache_order():
        one = f(x, inp["fc"], [w1], [inp["k_ctx"][1]], [inp["v_ctx"][1]], *tail)
        two = f(x, inp["fc"], [ident, w1], inp["k_ctx"], inp["v_ctx"], *tail)
        swapped = f(x, inp["fc"], [ident, w1], inp["k_ctx"][::-1], inp["v_ctx"][::-1], *tail)
        return np.array_equal(one, two) and not np.allclose(one, swapped), "blocks read their own caches in order"
    pins.append(_run("an o = down = 0 block passes through; caches stay with their blocks", identity_block_and_cache_order))

    def block_order():
        # With fc = I, running [w0, w1] on x is running [w1] on the float32
        # output of block w0 on x (its own cache), and not the other order.
        eye = synth.bf16_bits_rne(np.eye(d, dtype=np.float32))
        ab = f(x, eye, [w0, w1], inp["k_ctx"], inp["v_ctx"], *tail)
        x1 = np.asarray(block(x, w0, R, B, H, Dh, inp["k_ctx"][0], inp["v_ctx"][0], inp["ctx_len"], 1e-6)).astype(np.float32)
        then = f(x1, eye, [w1], [inp["k_ctx"][1]], [inp["v_ctx"][1]], *tail)
        x2 = np.asarray(block(x, w1, R, B, H, Dh, inp["k_ctx"][1], inp["v_ctx"][1], inp["ctx_len"], 1e-6)).astype(np.float32)
        other = f(x2, eye, [w0], [inp["k_ctx"][0]], [inp["v_ctx"][0]], *tail)
        return np.array_equal(ab, then) and not np.allclose(ab, other), "first block first"
    pins.append(_run("blocks run in the given order", block_order))

    def gain_linear():
        one = f(x, inp["fc"], [w1], [inp["k_ctx"][1]], [inp["v_ctx"][1]], *tail)
        dbl = synth.bf16_bits_rne(2 * _bf_vals(inp["norm"]).astype(np.float32))
        twice = f(x, inp["fc"], [w1], [inp["k_ctx"][1]], [inp["v_ctx"][1]], inp["ctx_len"], dbl, 1e-6, R, B, H, Dh)
        return np.array_equal(twice, 2 * one), "output linear in the final gain"
    pins.append(_run("the output is linear in the final norm's gain", gain_linear))
    return pins
