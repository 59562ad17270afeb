"""Exact rational brute force for tiny inputs (test helper).

Decodes every bf16 bit pattern and float32 value to an exact Fraction through
the struct module (a route independent of the oracle's numpy decoding) and
evaluates the plain definitions with exact rational arithmetic, so the fp64
oracle can be pinned to the exact answer.
"""
from __future__ import annotations

import struct
from fractions import Fraction


def frac_bf16(bits: int) -> Fraction:
    (v,) = struct.unpack(">f", struct.pack(">I", (int(bits) & 0xFFFF) << 16))
    return Fraction(v)


def frac_f32(x) -> Fraction:
    (v,) = struct.unpack(">f", struct.pack(">f", float(x)))
    return Fraction(v)


def frac_f16(bits: int) -> Fraction:
    """Exact value of an IEEE binary16 bit pattern (struct's 'e' format)."""
    (v,) = struct.unpack("<e", struct.pack("<H", int(bits) & 0xFFFF))
    return Fraction(v)


def frac_q8(q_row, d_row):
    """Exact values of one Q8_0 row: entry j is d[j // 32] * q[j]."""
    return [Fraction(int(q_row[j])) * frac_f16(d_row[j // 32]) for j in range(len(q_row))]


def exact_gemv_q8(Wq, Wd, X):
    Wf = [frac_q8(Wq[n], Wd[n]) for n in range(len(Wq))]
    K = len(Wf[0])
    return [[sum((frac_f32(xr[t]) * Wf[n][t] for t in range(K)), Fraction(0)) for n in range(len(Wf))] for xr in X]


def exact_markov_values(base, W1f, W2f, prev0, k):
    """exact_markov over already exact weight values (lists of Fractions)."""
    out = []
    for req in range(len(base)):
        prev = int(prev0[req])
        steps = []
        for i in range(k):
            e = W1f[prev]
            s = [frac_f32(base[req][i][v]) + sum((W2f[v][j] * e[j] for j in range(len(e))), Fraction(0))
                 for v in range(len(base[req][i]))]
            tok, margin, _ = exact_argmax(s)
            steps.append((tok, margin, s))
            prev = tok
        out.append(steps)
    return out


def exact_gemv(W_bits, X):
    N, K = len(W_bits), len(W_bits[0])
    Wf = [[frac_bf16(W_bits[n][t]) for t in range(K)] for n in range(N)]
    return [[sum((frac_f32(xr[t]) * Wf[n][t] for t in range(K)), Fraction(0)) for n in range(N)] for xr in X]


def exact_scores(base_row, w1_bits, w2_bits, prev):
    r = len(w1_bits[0])
    e = [frac_bf16(w1_bits[prev][j]) for j in range(r)]
    return [frac_f32(base_row[v]) + sum((frac_bf16(w2_bits[v][j]) * e[j] for j in range(r)), Fraction(0))
            for v in range(len(base_row))]


def exact_argmax(s):
    """(lowest index of the max, exact top-2 margin, runner-up index)."""
    best = 0
    for v in range(1, len(s)):
        if s[v] > s[best]:
            best = v
    runner = None
    for v in range(len(s)):
        if v != best and (runner is None or s[v] > s[runner]):
            runner = v
    return best, s[best] - s[runner], runner


def exact_markov(base, w1_bits, w2_bits, prev0, k):
    """Per request: list of (tok, margin, scores) for the k steps."""
    out = []
    for req in range(len(base)):
        prev = int(prev0[req])
        steps = []
        for i in range(k):
            s = exact_scores(base[req][i], w1_bits, w2_bits, prev)
            tok, margin, _ = exact_argmax(s)
            steps.append((tok, margin, s))
            prev = tok
        out.append(steps)
    return out


def exact_probe(x_rows, w_bits, bias):
    wf = [frac_bf16(b) for b in w_bits]
    return [sum((frac_f32(x[t]) * wf[t] for t in range(len(wf))), Fraction(0)) + frac_f32(bias) for x in x_rows]
