"""A seeded sweep of shapes against the fp64 oracle on an MI355X.

The parity tests of test_gpu_parity.py pick their shapes by hand, one per
case the kernels distinguish. This sweep draws further shapes from a fixed
seed across every entry point's size range, so the boundaries between the
kernel variants (tiles per workgroup, K phases, packed or split A blocks,
the scheduled lm_head's reach, launches of more than 16 or 80 rows, the
Markov loop's grid, register and LDS tiles, request counts) are crossed at
places nobody chose. The draw is the same on every run.
"""
import numpy as np
import pytest

import oracle
from gemv_markov_argmax_amd import synth
from parity import check_markov, logits_close, probe_close, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gemv_markov_argmax_amd import ops
    ops.lib()  # fail loudly if the library is missing
    return torch.device("cuda:0")


def _ops():
    from gemv_markov_argmax_amd import ops
    return ops


def _up(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _draw(seed, n, m_range, n_range, k_range, k_step, big_n=()):
    """n shapes (M, N, K): M uniform in m_range, N log-uniform in n_range
    (plus the given large N values), K a multiple of k_step in k_range."""
    rng = np.random.default_rng(seed)
    out = []
    for j in range(n):
        M = int(rng.integers(m_range[0], m_range[1] + 1))
        if j < len(big_n):
            N = int(big_n[j])
        else:
            N = int(np.exp(rng.uniform(np.log(n_range[0]), np.log(n_range[1]))))
        K = int(rng.integers(k_range[0] // k_step, k_range[1] // k_step + 1)) * k_step
        out.append((M, N, K))
    return out


# bf16 GEMV: M from 1 to 170 (two and three launches past 80 rows), N up to
# 6000, K a multiple of 8 up to 3000.
BF16_SHAPES = _draw(20251, 24, (1, 170), (1, 6000), (8, 3000), 8)
# The scheduled lm_head: up to 8 rows, vocabularies on both sides of 16
# tiles per CU (65536 rows on 256 CUs), K up to 4096.
SCHED_SHAPES = _draw(20252, 8, (1, 8), (1, 4000), (8, 4096), 8, big_n=(65537, 70017, 131071, 99999))
# Q8_0: K a multiple of 32, M up to 40 (several 16-row launches).
Q8_SHAPES = _draw(20253, 16, (1, 40), (1, 6000), (32, 3072), 32)
# Fused RMSNorm: M up to 16.
NORM_SHAPES = _draw(20254, 12, (1, 16), (2, 6000), (8, 3000), 8)


@pytest.mark.parametrize("M,N,K", BF16_SHAPES)
def test_sweep_bf16(dev, M, N, K):
    seed = 8100 + M * 7 + N + K
    say(f"[sweep bf16] M={M} N={N} K={K} seed={seed}")
    W, X = synth.gemv_inputs(M, N, K, seed)
    ops = _ops()
    Wd, Xd = ops.bf16_from_bits(W, dev), _up(X, dev)
    y = ops.lm_head(Wd, Xd)
    torch.cuda.synchronize()
    logits_close(y.cpu().numpy(), oracle.gemv(W, X), f"lm_head M={M} N={N} K={K}")
    if M <= 16:
        y2 = ops.proj_smallm(Wd, Xd)
        torch.cuda.synchronize()
        assert torch.equal(y, y2), "proj_smallm and lm_head differ on the same shape"


@pytest.mark.parametrize("M,N,K", SCHED_SHAPES)
def test_sweep_lm_head_sched(dev, M, N, K):
    seed = 8200 + M * 7 + N + K
    say(f"[sweep sched] M={M} N={N} K={K} seed={seed}")
    W, X = synth.gemv_inputs(M, N, K, seed)
    ops = _ops()
    Wd, Xd = ops.bf16_from_bits(W, dev), _up(X, dev)
    cnt = ops.lm_head_counter(dev)
    y = ops.lm_head_sched(Wd, Xd, cnt)
    y2 = ops.lm_head_sched(Wd, Xd, cnt)
    torch.cuda.synchronize()
    assert int(cnt.item()) == 0, "the counter was not left at 0"
    assert torch.equal(y, y2), "rerun differs"
    logits_close(y.cpu().numpy(), oracle.gemv(W, X), f"lm_head_sched M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", Q8_SHAPES)
def test_sweep_q8(dev, M, N, K):
    seed = 8300 + M * 7 + N + K
    say(f"[sweep q8] M={M} N={N} K={K} seed={seed}")
    Wq, Wd, X = synth.gemv_q8_inputs(M, N, K, seed)
    ops = _ops()
    q, d = ops.q8_from_numpy(Wq, Wd, dev)
    y = ops.lm_head_q8(q, d, _up(X, dev))
    torch.cuda.synchronize()
    logits_close(y.cpu().numpy(), oracle.gemv_q8(Wq, Wd, X), f"lm_head_q8 M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", NORM_SHAPES)
def test_sweep_norm(dev, M, N, K):
    seed = 8400 + M * 7 + N + K
    say(f"[sweep norm] M={M} N={N} K={K} seed={seed}")
    ops = _ops()
    if not ops.proj_smallm_norm_fits(N, K, M):
        pytest.skip("shape outside the fused kernel (its callers take rmsnorm + proj_smallm)")
    W, X = synth.gemv_inputs(M, N, K, seed)
    gamma = synth.bf16_bits_rne(1.0 + synth.normal_f32(seed, synth.S_BASE, (K,), 0.2))
    y = ops.proj_smallm_norm(ops.bf16_from_bits(W, dev), _up(X, dev), ops.bf16_from_bits(gamma, dev), 1e-6)
    torch.cuda.synchronize()
    logits_close(y.cpu().numpy(), oracle.gemv(W, oracle.rmsnorm(X, gamma, 1e-6)), f"proj norm M={M} N={N} K={K}")


def _draw_markov(seed, n):
    """n shapes (R, B, k, V, r, tie_frac): up to 16 requests and 16 steps,
    V log-uniform up to 60000, r a multiple of 8 up to 512; every other one
    (where V leaves room for two entries per row) with exactly tied maxima in
    5% of its base rows."""
    rng = np.random.default_rng(seed)
    out = []
    for j in range(n):
        R = int(rng.integers(1, 17))
        B = int(rng.integers(1, 17))
        k = int(rng.integers(1, B + 1))
        V = int(np.exp(rng.uniform(0.0, np.log(60000))))
        r = 8 * int(rng.integers(1, 65))
        out.append((R, B, k, V, r, 0.05 if j % 2 and V >= 4 * R * B else 0.0))
    return out


MARKOV_SHAPES = _draw_markov(20255, 14)


@pytest.mark.parametrize("R,B,k,V,r,tie", MARKOV_SHAPES)
def test_sweep_markov(dev, R, B, k, V, r, tie):
    seed = 8500 + R * 7 + V + r
    say(f"[sweep markov] R={R} B={B} k={k} V={V} r={r} tie={tie} seed={seed}")
    base, w1, w2, prev0, _ = synth.markov_inputs(R, B, V, r, seed, tie_frac=tie)
    ops = _ops()
    ids = ops.markov_sample(_up(base, dev), ops.bf16_from_bits(w1, dev), ops.bf16_from_bits(w2, dev),
                            _up(prev0, dev), k)
    torch.cuda.synchronize()
    check_markov(ids.cpu().numpy(), base, w1, w2, prev0, k)


def _draw_rounds(seed, n):
    """n whole-round shapes (R, B, k, V, d, r): R * B <= 72 rows (one or
    more lm_head kernels), V log-uniform from 16 to 40000, d a multiple of 8
    up to 1024, r a multiple of 8 up to 256."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        R = int(rng.integers(1, 9))
        B = int(rng.integers(1, 10))
        k = int(rng.integers(1, B + 1))
        V = int(np.exp(rng.uniform(np.log(16), np.log(40000))))
        d = 8 * int(rng.integers(1, 129))
        r = 8 * int(rng.integers(1, 33))
        out.append((R, B, k, V, d, r))
    return out


ROUND_SHAPES = _draw_rounds(20256, 8)


@pytest.mark.parametrize("R,B,k,V,d,r", ROUND_SHAPES)
def test_sweep_draft_round(dev, R, B, k, V, d, r):
    """dspark_draft_round end to end: logits, drafted ids and probe."""
    seed = 8600 + R * 7 + V + d + r
    say(f"[sweep round] R={R} B={B} k={k} V={V} d={d} r={r} seed={seed}")
    W, H = synth.gemv_inputs(R * B, V, d, seed)
    _, w1, w2, prev0, _ = synth.markov_inputs(R, 1, V, r, seed)
    _, pw = synth.probe_inputs(1, d, seed)
    thr = 0.01
    ops = _ops()
    out = ops.draft_round(ops.bf16_from_bits(W, dev), _up(H, dev), ops.bf16_from_bits(w1, dev),
                          ops.bf16_from_bits(w2, dev), _up(prev0, dev), B, k, probe_w=ops.bf16_from_bits(pw, dev),
                          probe_bias=-0.02, probe_threshold=thr)
    torch.cuda.synchronize()
    ref = oracle.draft_round(W, H, w1, w2, prev0, R, B, k, pw, -0.02, thr)
    logits_close(out["base"].view(R * B, -1).cpu().numpy(), ref["base"], "sweep round logits")
    check_markov(out["ids"].cpu().numpy(), ref["base32"], w1, w2, prev0, k)
    probe_close(out["logit"].cpu().numpy(), out["passed"].cpu().numpy(), ref["logit"], ref["passed"], thr)
