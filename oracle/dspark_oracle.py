"""Plain fp64 CPU oracle for the DSpark draft-round hot path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the tests, the smoke check of the build entry point
and the benchmark's CPU-baseline leg use it. It shares no code with the HIP
path (the two meet only at the seeded input generator, which does no
arithmetic of the method).

Sources (the pages; a reader has them, not this copy):

[W7]   vllm.cpp #436, "SPEC-DSPARK W7: the sequential Markov sample loop is
       HOST-side - 28% of the draft step, 14.9 MB downloaded per step".
       Sections "Measured", "The fix", "Gate" and the "W7 LANDED" comment.
[SI441] SharpInference #441, "perf(cuda): DSpark GPU draft round runs ~3x the
       bandwidth floor - small-M (B=7) projection GEMMs -> weight-stationary
       matvec". Sections "Observation", "Hypothesis", "Proposed work".
[DS772] ds4 #772, "dspark: cut per-cycle CUDA overheads (single-draft decode,
       GPU confidence probe)". Sections "Summary", "Performance".

Every function computes its plain definition in float64 from the exact input
values (bf16 bits decode exactly; float32 inputs widen exactly). A library
matmul is used as a step; nothing is blocked, fused or reordered.

Readings taken where the pages leave a step open are listed with each
function. The argmax decision is taken on float32 scores, the precision the
pages give the scores ([W7] "W7 LANDED": base logits are f32), from the exact
fp64 score rounded once to float32.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

NEAR_TIE = 1e-3  # top-2 margin below which a drafted id is reported, not required


def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns: the bf16 is the high half of an
    IEEE binary32, so shifting the 16 bits up by 16 gives the same number."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def fp16_to_f64(bits) -> np.ndarray:
    """Exact value of IEEE 754 binary16 bit patterns (numpy's half-precision
    decode, widened exactly)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


QK8_0 = 32  # entries per Q8_0 block


def q8_0_to_f64(q, d_bits) -> np.ndarray:
    """Exact values of Q8_0 weights.

    [DS772] "Summary": the GPU confidence path takes Q8_0 markov weights
    (any other format falls back to the CPU). The pages do not spell the
    format out; the reading taken is the Q8_0 block format of the GGUF files
    that project loads: each run of 32 consecutive entries of a row shares
    one IEEE binary16 scale d, and entry j of the block is d * q[j] with q a
    signed 8-bit integer. Here the quants and the scales are passed as two
    arrays: q int8 [..., K] and d_bits uint16 [..., K / 32] (binary16 bit
    patterns); block b of a row covers entries 32b .. 32b + 31.
    """
    q = np.asarray(q, dtype=np.int8)
    d = fp16_to_f64(d_bits)
    if q.shape[-1] % QK8_0 != 0 or d.shape != q.shape[:-1] + (q.shape[-1] // QK8_0,):
        raise ValueError("Q8_0: q [..., K] with K % 32 == 0 and d [..., K / 32] required")
    _finite(d)
    return q.astype(np.float64) * np.repeat(d, QK8_0, axis=-1)


def _finite(*arrays):
    for a in arrays:
        if not np.all(np.isfinite(a)):
            raise ValueError("oracle inputs must be finite")


def _values(x) -> np.ndarray:
    """Exact float64 values of an activation input: a float64 array is taken
    as it is (a value the oracle computed itself, e.g. inside the draft
    block), anything else is read as float32 (the type the path hands
    between its steps) and widened exactly."""
    a = np.asarray(x)
    if a.dtype == np.float64:
        return a
    return np.asarray(a, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Small-M projections and the lm_head
# ---------------------------------------------------------------------------

def gemv(W_bits, X) -> np.ndarray:
    """Y[m, n] = sum_t X[m, t] * W[n, t], in float64.

    [SI441] "Observation": every draft projection and the lm_head multiplies
    the B drafted positions' activations by one weight matrix, reading the
    weight once for all B rows. W is [N, K] bf16 (row n is output n), X is
    [M, K] float32 (or float64 values, taken exactly), Y is [M, N].
    """
    W = bf16_to_f64(W_bits)
    X64 = _values(X)
    _finite(W, X64)
    if W.ndim != 2 or X64.ndim != 2 or W.shape[1] != X64.shape[1]:
        raise ValueError("gemv: W [N, K] and X [M, K] required")
    return X64 @ W.T


def gemv_rows(W_bits, X, rows) -> np.ndarray:
    """The same definition evaluated only for the output columns ``rows``
    (returns [M, len(rows)]); used to check sampled outputs at full size."""
    rows = np.asarray(rows, dtype=np.int64)
    return gemv(np.asarray(W_bits)[rows], X)


proj_smallm = gemv
lm_head = gemv


def gemv_q8(Wq, Wd_bits, X) -> np.ndarray:
    """Y[m, n] = sum_t X[m, t] * W[n, t] with W given as Q8_0 blocks.

    The same definition as gemv ([SI441] "Observation"), over weights stored
    in the quantized form whose weight-stationary matvec [SI441] "Proposed
    work" cites as the existing quantized kernels: W = q8_0_to_f64(Wq, Wd),
    Wq int8 [N, K], Wd binary16 [N, K / 32]; X float32 [M, K]; in float64.
    """
    W = q8_0_to_f64(Wq, Wd_bits)
    X64 = np.asarray(X, dtype=np.float32).astype(np.float64)
    _finite(X64)
    if W.ndim != 2 or X64.ndim != 2 or W.shape[1] != X64.shape[1]:
        raise ValueError("gemv_q8: W [N, K] and X [M, K] required")
    return X64 @ W.T


def gemv_q8_rows(Wq, Wd_bits, X, rows) -> np.ndarray:
    """gemv_q8 evaluated only for the output columns ``rows``."""
    rows = np.asarray(rows, dtype=np.int64)
    return gemv_q8(np.asarray(Wq)[rows], np.asarray(Wd_bits)[rows], X)


# ---------------------------------------------------------------------------
# Markov-biased greedy sampling loop
# ---------------------------------------------------------------------------

@dataclass
class StepResult:
    tok: int          # drafted id (draft vocabulary), float32 decision
    margin: float     # s64[tok] - max_{v != tok} s64[v]; 0 for an exact tie
    runner_up: int    # lowest index attaining that max over v != tok
    s: np.ndarray     # fp64 scores of the step


def _decoded(w) -> np.ndarray:
    return w if (isinstance(w, np.ndarray) and w.dtype == np.float64) else bf16_to_f64(w)


def markov_scores(base_row, w1_bits, w2, prev: int) -> np.ndarray:
    """Scores of one step: s[v] = base_row[v] + sum_j W2[v, j] * W1[prev, j].

    [W7] "The fix": gather the markov_w1 row of the previous token, multiply
    markov_w2 [V, r] by it, add the step's base-logit row. No scale,
    temperature or nonlinearity appears on the page, so none is applied.
    ``w1_bits`` and ``w2`` may be bf16 bits or already decoded float64
    arrays (the values of weights in any storage format).
    """
    w1 = np.asarray(w1_bits)
    V = w1.shape[0]
    if not (0 <= prev < V):
        raise ValueError(f"prev {prev} outside [0, {V})")
    e = _decoded(w1[prev])
    W2 = _decoded(w2)
    b = np.asarray(base_row, dtype=np.float32).astype(np.float64)
    _finite(b)
    return b + W2 @ e


def greedy_argmax(s64: np.ndarray) -> StepResult:
    """Greedy pick with the lowest index winning ties ([W7] "The fix": the
    device argmax and the host loop share that tie rule).

    The decision is made on the scores rounded to float32; the reported
    margin is measured on the exact fp64 scores.
    """
    s32 = s64.astype(np.float32)
    tok = int(np.argmax(s32))  # numpy returns the first (lowest) index of the max
    rest = s64.copy()
    rest[tok] = -np.inf
    runner = int(np.argmax(rest))
    return StepResult(tok=tok, margin=float(s64[tok] - rest[runner]), runner_up=runner, s=s64)


def markov_step(base_row, w1_bits, w2, prev: int) -> StepResult:
    """One step of the loop from a given previous token."""
    return greedy_argmax(markov_scores(base_row, w1_bits, w2, prev))


def markov_sample(base, w1_bits, w2_bits, prev0, k: int, d2t=None) -> dict:
    """The k-step loop for every request, in the order the pages give it.

    [W7] "Measured" (the host loop: per step i of k, add the Markov bias to
    row i and take the argmax) and "The fix" (gather -> GEMV -> add the
    step's base row -> lowest-index argmax -> d2t -> prev stays the drafted
    token). Readings:
      * step i uses base row i of the request (k <= B);
      * step 0 is biased by prev0, the request's last committed token given
        in draft-vocabulary space;
      * prev takes the draft-space token; only the emitted ids go through
        d2t (identity when d2t is None), since W1 is indexed by draft ids;
      * requests are independent and share the weights.

    base: float32 [R, B, V]; w1, w2: bf16 bits [V, r]; prev0: int [R].
    Returns dict(ids [R, k] int64, tok [R, k], margin [R, k] float64,
    runner_up [R, k]).
    """
    return _markov_loop(base, bf16_to_f64(w1_bits), bf16_to_f64(w2_bits), prev0, k, d2t)


def markov_sample_q8(base, w1q, w1d_bits, w2q, w2d_bits, prev0, k: int, d2t=None) -> dict:
    """The same loop with markov_w1 and markov_w2 given as Q8_0 blocks.

    [DS772] "Summary": the GPU path takes Q8_0 markov weights. Reading: both
    markov tensors are Q8_0 (blocks along the rank dimension, r % 32 == 0);
    the loop is unchanged and runs on their exact values (q8_0_to_f64).
    w1q, w2q int8 [V, r]; w1d_bits, w2d_bits binary16 [V, r / 32].
    """
    return _markov_loop(base, q8_0_to_f64(w1q, w1d_bits), q8_0_to_f64(w2q, w2d_bits), prev0, k, d2t)


def _markov_loop(base, W1, W2, prev0, k: int, d2t=None) -> dict:
    base = np.asarray(base, dtype=np.float32)
    R, B, V = base.shape
    if not (1 <= k <= B):
        raise ValueError("need 1 <= k <= B")
    if W1.shape != W2.shape or W1.shape[0] != V:
        raise ValueError("markov_w1 and markov_w2 must both be [V, r]")
    _finite(W1, W2)
    ids = np.empty((R, k), np.int64)
    tok = np.empty((R, k), np.int64)
    margin = np.empty((R, k), np.float64)
    runner = np.empty((R, k), np.int64)
    for req in range(R):
        prev = int(prev0[req])
        for i in range(k):
            st = markov_step(base[req, i], W1, W2, prev)
            tok[req, i] = st.tok
            margin[req, i] = st.margin
            runner[req, i] = st.runner_up
            ids[req, i] = st.tok if d2t is None else int(d2t[st.tok])
            prev = st.tok
    return dict(ids=ids, tok=tok, margin=margin, runner_up=runner)


# ---------------------------------------------------------------------------
# Confidence probe
# ---------------------------------------------------------------------------

def conf_probe(x, w_bits, bias: float, threshold: float):
    """logit[m] = sum_t w[t] * x[m, t] + bias; pass[m] = logit[m] >= threshold.

    [DS772] "Summary": the proposer's confidence probe is one wide dot product
    on the drafted row's hidden state whose single scalar result gates how
    many drafted tokens are proposed; "Performance": GPU and CPU evaluations
    differ only by summation order. Reading: the gate compares the logit
    itself with a logit-space threshold and keeps drafting when it is at
    least the threshold (the page names no squashing function).
    """
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    w = bf16_to_f64(w_bits)
    _finite(x64, w)
    logit = x64 @ w + float(np.float32(bias))
    return logit, logit >= float(np.float32(threshold))


# ---------------------------------------------------------------------------
# One draft round
# ---------------------------------------------------------------------------

def draft_round(W_lm_bits, H, w1_bits, w2_bits, prev0, num_reqs: int, B: int, k: int,
                probe_w_bits, probe_bias: float, probe_threshold: float, d2t=None) -> dict:
    """lm_head -> Markov loop -> probe on every drafted row.

    The base logits handed from the lm_head to the loop are float32 ([W7]
    "Measured": nqpr x draft_vocab floats), so the fp64 lm_head result is
    rounded once to float32 before the loop reads it.
    """
    base64 = lm_head(W_lm_bits, H)                      # [R*B, V]
    V = base64.shape[1]
    base32 = base64.astype(np.float32).reshape(num_reqs, B, V)
    mk = markov_sample(base32, w1_bits, w2_bits, prev0, k, d2t)
    logit, passed = conf_probe(H, probe_w_bits, probe_bias, probe_threshold)
    return dict(base=base64, base32=base32, logit=logit, passed=passed, **mk)


def draft_round_q8(Wq_lm, Wd_lm_bits, H, w1q, w1d_bits, w2q, w2d_bits, prev0, num_reqs: int, B: int, k: int,
                   probe_w_bits, probe_bias: float, probe_threshold: float, d2t=None) -> dict:
    """draft_round with a Q8_0 lm_head and Q8_0 markov weights ([DS772]
    "Summary"); the probe weights stay bf16."""
    base64 = gemv_q8(Wq_lm, Wd_lm_bits, H)
    V = base64.shape[1]
    base32 = base64.astype(np.float32).reshape(num_reqs, B, V)
    mk = markov_sample_q8(base32, w1q, w1d_bits, w2q, w2d_bits, prev0, k, d2t)
    logit, passed = conf_probe(H, probe_w_bits, probe_bias, probe_threshold)
    return dict(base=base64, base32=base32, logit=logit, passed=passed, **mk)


# ---------------------------------------------------------------------------
# The rest of the draft block forward at small M
# ---------------------------------------------------------------------------
#
# [SI441] "Observation" lists the draft block's operations: the fc, q/k/v/o
# and gate/up/down projections, the lm_head, and AttentionBatchedRagged over
# a short context. The pages name no norm, activation or position encoding;
# the readings taken (a pre-norm transformer layer with RMSNorm, a SiLU-gated
# MLP, multi-head attention without a position encoding, each draft position
# attending to its request's context and to its own block) are listed in the
# design notes.

def rmsnorm(x, gamma_bits, eps: float):
    """y[m, t] = x[m, t] / sqrt(mean_t x[m, t]^2 + eps) * gamma[t]; gamma bf16,
    x float32 (or float64 values, taken exactly: the block's second norm reads
    the float64 residual sum)."""
    x64 = _values(x)
    g = bf16_to_f64(gamma_bits)
    _finite(x64, g)
    ms = np.mean(x64 * x64, axis=-1, keepdims=True)
    return x64 / np.sqrt(ms + float(np.float32(eps))) * g


def silu_gate(gu, F: int):
    """a[m, j] = silu(g) * u with g = gu[m, j], u = gu[m, F + j], silu(g) = g / (1 + exp(-g)).
    gu float32 (or float64 values, taken exactly)."""
    gu64 = _values(gu)
    _finite(gu64)
    g, u = gu64[:, :F], gu64[:, F:2 * F]
    return g / (1.0 + np.exp(-g)) * u


def attention_ragged(q, k_blk, v_blk, R: int, B: int, H: int, Dh: int, k_ctx_bits, v_ctx_bits, ctx_len,
                     block_causal: bool = False):
    """Multi-head attention of the B draft positions of each request.

    Position i of request r, head h, attends to the request's first
    ctx_len[r] context positions (k_ctx, v_ctx: bf16 [R, Lmax, H * Dh]) and
    to the positions of its own block (k_blk, v_blk: fp32 [R * B, H * Dh]),
    all of them, or those j <= i when block_causal. Scores are q . k /
    sqrt(Dh); softmax over those keys; the output is the weighted sum of the
    values. q, k_blk, v_blk, out: [R * B, H * Dh], row r * B + i; q, k_blk
    and v_blk float32 (or float64 values, taken exactly).
    """
    q64 = _values(q).reshape(R, B, H, Dh)
    kb = _values(k_blk).reshape(R, B, H, Dh)
    vb = _values(v_blk).reshape(R, B, H, Dh)
    kc = bf16_to_f64(k_ctx_bits)
    vc = bf16_to_f64(v_ctx_bits)
    Lmax = kc.shape[1]
    kc = kc.reshape(R, Lmax, H, Dh)
    vc = vc.reshape(R, Lmax, H, Dh)
    _finite(q64, kb, vb, kc, vc)
    out = np.empty((R, B, H, Dh))
    for r in range(R):
        L = int(ctx_len[r])
        if not (0 <= L <= Lmax):
            raise ValueError("ctx_len outside [0, Lmax]")
        for i in range(B):
            nb = i + 1 if block_causal else B
            for h in range(H):
                keys = np.concatenate([kc[r, :L, h], kb[r, :nb, h]])
                vals = np.concatenate([vc[r, :L, h], vb[r, :nb, h]])
                s = keys @ q64[r, i, h] / np.sqrt(Dh)
                w = np.exp(s - s.max())
                out[r, i, h] = (w / w.sum()) @ vals
    return out.reshape(R * B, H * Dh)


def draft_block_forward(h, w: dict, R: int, B: int, H: int, Dh: int, k_ctx_bits, v_ctx_bits, ctx_len,
                        eps: float, block_causal: bool = False):
    """One draft block (layer) forward at small M = R * B, in float64, as
    the readings above compose it:
      x1 = rmsnorm(h, ln1); [q | k | v] = x1 W_qkv^T; a = attention(q, k, v);
      h2 = h + a W_o^T; x2 = rmsnorm(h2, ln2); gu = x2 W_gate_up^T;
      h3 = h2 + silu_gate(gu) W_down^T.
    w: bf16 bits of qkv [3 H Dh, d] (q rows, then k rows, then v rows), o
    [d, H Dh], gate_up [2 F, d] (gate rows, then up rows), down [d, F], ln1
    and ln2 [d]. Every step is the module's own function for it (gemv,
    rmsnorm, attention_ragged, silu_gate) applied to the float64 values of
    the step before; h is float32."""
    HD = H * Dh
    h64 = _values(np.asarray(h, dtype=np.float32))
    x1 = rmsnorm(h64, w["ln1"], eps)
    qkv = gemv(w["qkv"], x1)
    a = attention_ragged(qkv[:, :HD], qkv[:, HD:2 * HD], qkv[:, 2 * HD:], R, B, H, Dh, k_ctx_bits, v_ctx_bits,
                         ctx_len, block_causal)
    h2 = h64 + gemv(w["o"], a)
    x2 = rmsnorm(h2, w["ln2"], eps)
    gu = gemv(w["gate_up"], x2)
    return h2 + gemv(w["down"], silu_gate(gu, gu.shape[1] // 2))


def draft_forward(x_in, fc_bits, layers, k_ctx_list, v_ctx_list, ctx_len, norm_bits, eps: float, R: int, B: int,
                  H: int, Dh: int, block_causal: bool = False):
    """The drafter's forward at small M = R * B, up to the hidden states the
    lm_head reads: h = x_in fc^T, then each block in order (each with its own
    context cache), then a final rmsnorm.

    [SI441] "Observation" lists fc among the drafter's projections and the
    block stack around it; the final norm is the plainest reading of a
    Qwen3-derived drafter. The hidden state handed from one block to the
    next is float32 (the blocks' input type), rounded once per hand-over;
    inside a block everything stays float64."""
    h = gemv(fc_bits, x_in)
    for w, kc, vc in zip(layers, k_ctx_list, v_ctx_list):
        h = draft_block_forward(h.astype(np.float32), w, R, B, H, Dh, kc, vc, ctx_len, eps, block_causal)
    return rmsnorm(h.astype(np.float32), norm_bits, eps)
