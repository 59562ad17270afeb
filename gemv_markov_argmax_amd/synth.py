"""Seeded synthetic inputs for the DSpark draft-round hot path.

This module only draws random numbers and arranges them into the shapes the
hot path consumes. It holds none of the method's arithmetic (no products, no
argmax), so the fp64 oracle and the HIP path can both be fed from it without
sharing any computation.

Workload shapes stand in for the lanes described on the pages (none of their
models, prompts or weights exist here):

* ``tiny`` -- a small case the oracle finishes in well under a second.
* ``qwen3_8b_head`` -- Qwen3-8B block-7 drafter head: B = k = 7, d = 4096,
  V = 151936, markov rank 256 (SharpInference #441, section "Observation" and
  "Proposed work", which sizes markov_w2 at 78 MB).
* ``lane27b`` -- vllm.cpp #436 "SPEC-DSPARK W7", section "Measured": k = 15
  drafted rows over a 248320-entry draft vocabulary.
* ``reduced_vocab_batched`` -- the 35B lane's 32000-entry draft vocabulary
  (same page, same section), batched over 8 requests with B = k = 9.
* ``draft_layer`` -- one draft transformer layer's projections at M = 7
  (SharpInference #441, "Hypothesis") plus a 7424-wide confidence probe
  (ds4 #772, "Summary").
* ``qwen3_8b_head_q8``, ``lane27b_q8`` -- the two single-request heads with
  the lm_head and markov weights in Q8_0 (ds4 #772, "Summary").

Every tensor is drawn from its own PCG64 stream, keyed by (seed, stream id,
block index), so a value never depends on how many threads fill the array.
Normals are drawn in float32; bf16 tensors are rounded to bf16 by
round-to-nearest-even on the bit pattern and returned as ``uint16`` bits.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SEED_BASE = 20261200

# Stream ids: fixed, so adding a tensor never shifts another one's values.
S_W_LM, S_W1, S_W2, S_H, S_PREV0, S_PROBE_W, S_PROBE_X, S_TIES, S_D2T, S_BASE = range(10)
S_LAYER = 16  # q, k, v, o, gate, up, down and their inputs follow from here

_BLOCK = 1 << 22  # elements per independently seeded block

CONFIGS = {
    "tiny": dict(num_reqs=1, B=4, k=4, d=256, V=4096, r=32),
    "qwen3_8b_head": dict(num_reqs=1, B=7, k=7, d=4096, V=151936, r=256),
    "lane27b": dict(num_reqs=1, B=15, k=15, d=5120, V=248320, r=256, tie_frac=0.05),
    "reduced_vocab_batched": dict(num_reqs=8, B=9, k=9, d=5120, V=32000, r=256),
    "draft_layer": dict(M=7, d=4096, ffn=12288, probe_width=7424),
    # The two R = 1 heads with Q8_0 lm_head and markov weights (ds4 #772,
    # "Summary": the GPU path takes Q8_0 markov weights).
    "qwen3_8b_head_q8": dict(num_reqs=1, B=7, k=7, d=4096, V=151936, r=256, weights="q8_0"),
    "lane27b_q8": dict(num_reqs=1, B=15, k=15, d=5120, V=248320, r=256, weights="q8_0"),
}
CONFIG_SEED_INDEX = {name: i + 1 for i, name in enumerate(CONFIGS)}

W_STD = 0.02  # weights ~ N(0, 0.02)
TIE_VALUE = np.float32(32.0)  # far above any N(0, 1.3) base draw


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _gen(seed: int, stream: int, block: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, block])))


def bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits.

    Inputs must be finite. This is input preparation, not part of the method.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (r >> np.uint32(16)).astype(np.uint16)


def _fill_blocks(n: int, fn) -> None:
    nblk = (n + _BLOCK - 1) // _BLOCK
    if nblk <= 1:
        for b in range(nblk):
            fn(b, b * _BLOCK, min(n, (b + 1) * _BLOCK))
        return
    with ThreadPoolExecutor(max_workers=_threads()) as ex:
        list(ex.map(lambda b: fn(b, b * _BLOCK, min(n, (b + 1) * _BLOCK)), range(nblk)))


def normal_f32(seed: int, stream: int, shape, std: float = 1.0) -> np.ndarray:
    """float32 draws from N(0, std^2), blockwise seeded."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)

    def fill(b, lo, hi):
        v = _gen(seed, stream, b).standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[lo:hi] = v

    _fill_blocks(n, fill)
    return out.reshape(shape)


def normal_bf16(seed: int, stream: int, shape, std: float = W_STD) -> np.ndarray:
    """bf16 bits of N(0, std^2) draws (drawn in float32, rounded RNE)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)

    def fill(b, lo, hi):
        v = _gen(seed, stream, b).standard_normal(hi - lo, dtype=np.float32)
        v *= np.float32(std)
        out[lo:hi] = bf16_bits_rne(v)

    _fill_blocks(n, fill)
    return out.reshape(shape)


def q8_0_quantize(x: np.ndarray):
    """Round float32 rows to Q8_0 blocks (32 entries along the last axis):
    per block d = max|x| / 127, stored as IEEE binary16 (nearest), and
    q = x / d rounded half away from zero, in [-127, 127]; an all-zero block
    gets d = 0 and q = 0. This is how such weights are usually produced;
    here it only prepares inputs. Returns (q int8 [..., K], d bits uint16
    [..., K / 32])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    K = x.shape[-1]
    if K % 32:
        raise ValueError("Q8_0 needs K % 32 == 0")
    xb = x.reshape(x.shape[:-1] + (K // 32, 32))
    d = np.abs(xb).max(axis=-1) / np.float32(127.0)
    inv = np.where(d > 0, np.float32(1.0) / np.where(d > 0, d, np.float32(1.0)), np.float32(0.0)).astype(np.float32)
    v = xb * inv[..., None]
    q = np.clip(np.sign(v) * np.floor(np.abs(v) + np.float32(0.5)), -127, 127).astype(np.int8)
    return q.reshape(x.shape), d.astype(np.float16).view(np.uint16)


def normal_q8(seed: int, stream: int, shape, std: float = W_STD):
    """Q8_0 form (q int8, d bits uint16) of N(0, std^2) float32 draws."""
    n = int(np.prod(shape))
    x = np.empty(n, dtype=np.float32)

    def fill(b, lo, hi):
        v = _gen(seed, stream, b).standard_normal(hi - lo, dtype=np.float32)
        v *= np.float32(std)
        x[lo:hi] = v

    _fill_blocks(n, fill)
    return q8_0_quantize(x.reshape(shape))


def uniform_index(seed: int, stream: int, n: int, high: int) -> np.ndarray:
    """int64 draws uniform in [0, high)."""
    return _gen(seed, stream).integers(0, high, size=n, dtype=np.int64)


def config_seed(name: str, replica: int = 0) -> int:
    return SEED_BASE + CONFIG_SEED_INDEX[name] + 1000 * replica


# ----------------------------------------------------------------------------
# Inputs per entry point
# ----------------------------------------------------------------------------

def gemv_inputs(M: int, N: int, K: int, seed: int, w_std: float = W_STD):
    """W bf16 bits [N, K] ~ N(0, w_std^2); X float32 [M, K] ~ N(0, 1)."""
    W = normal_bf16(seed, S_W_LM, (N, K), w_std)
    X = normal_f32(seed, S_H, (M, K))
    return W, X


def probe_inputs(M: int, D: int, seed: int):
    """x float32 [M, D] ~ N(0, 1); w bf16 bits [D] ~ N(0, 0.02^2)."""
    x = normal_f32(seed, S_PROBE_X, (M, D))
    w = normal_bf16(seed, S_PROBE_W, (D,))
    return x, w


def markov_inputs(num_reqs: int, B: int, V: int, r: int, seed: int,
                  base_std: float = 1.28, tie_frac: float = 0.0,
                  tie_exact: bool = True):
    """Inputs of the Markov loop taken on their own (base drawn directly).

    base float32 [R, B, V] ~ N(0, base_std^2) -- 1.28 is what an lm_head with
    d = 4096, weights N(0, 0.02^2) and unit hidden states produces;
    w1, w2 bf16 bits [V, r] ~ N(0, 0.02^2); prev0 int64 [R] uniform in [0, V).

    tie_frac > 0 marks that fraction of the R*B base rows (at least one) as
    tie rows: two distinct vocabulary entries a < b of the row are both set to
    TIE_VALUE, well above every other draw. With tie_exact the W2 row b is
    also made a copy of row a, so the two scores are exactly equal and the
    lowest-index rule must pick a. Pairs are disjoint across rows.
    Returns (base, w1, w2, prev0, ties) where ties is a list of
    (request, row, a, b).
    """
    base = normal_f32(seed, S_BASE, (num_reqs, B, V), base_std)
    w1 = normal_bf16(seed, S_W1, (V, r))
    w2 = normal_bf16(seed, S_W2, (V, r))
    prev0 = uniform_index(seed, S_PREV0, num_reqs, V)
    ties = []
    if tie_frac > 0:
        g = _gen(seed, S_TIES)
        rows = np.flatnonzero(g.random(num_reqs * B) < tie_frac)
        if rows.size == 0:
            rows = np.array([int(g.integers(0, num_reqs * B))])
        idx = g.choice(V, size=2 * rows.size, replace=False)
        for j, row in enumerate(rows):
            a, b = sorted((int(idx[2 * j]), int(idx[2 * j + 1])))
            req, i = divmod(int(row), B)
            base[req, i, a] = TIE_VALUE
            base[req, i, b] = TIE_VALUE
            if tie_exact:
                w2[b, :] = w2[a, :]
            ties.append((req, i, a, b))
    return base, w1, w2, prev0, ties


def gemv_q8_inputs(M: int, N: int, K: int, seed: int, w_std: float = W_STD):
    """W as Q8_0 (q int8 [N, K], d bits [N, K/32]) of N(0, w_std^2) draws; X float32 [M, K] ~ N(0, 1)."""
    Wq, Wd = normal_q8(seed, S_W_LM, (N, K), w_std)
    X = normal_f32(seed, S_H, (M, K))
    return Wq, Wd, X


def markov_q8_inputs(num_reqs: int, B: int, V: int, r: int, seed: int, base_std: float = 1.28):
    """The Markov loop's inputs with markov_w1 and markov_w2 as Q8_0 of
    N(0, 0.02^2) draws (r % 32 == 0). Returns (base, w1q, w1d, w2q, w2d, prev0)."""
    base = normal_f32(seed, S_BASE, (num_reqs, B, V), base_std)
    w1q, w1d = normal_q8(seed, S_W1, (V, r))
    w2q, w2d = normal_q8(seed, S_W2, (V, r))
    prev0 = uniform_index(seed, S_PREV0, num_reqs, V)
    return base, w1q, w1d, w2q, w2d, prev0


def d2t_map(V: int, seed: int, offset: int = 1000) -> np.ndarray:
    """An injective draft->target id map (test use only): a seeded
    permutation of [offset, offset + V)."""
    return _gen(seed, S_D2T).permutation(V).astype(np.int64) + offset


def round_inputs(name: str, seed: int | None = None, with_base: bool = False):
    """All tensors of one draft round for a head configuration.

    Returns a dict: W_lm [V, d] bf16, H [R*B, d] f32, w1/w2 [V, r] bf16,
    prev0 [R] int64, probe_w [d] bf16, plus the shape fields.
    """
    cfg = dict(CONFIGS[name])
    if "V" not in cfg:
        raise ValueError(f"{name} is not a head configuration")
    seed = config_seed(name) if seed is None else seed
    R, B, d, V, r = cfg["num_reqs"], cfg["B"], cfg["d"], cfg["V"], cfg["r"]
    out = dict(cfg, seed=seed, name=name)
    if cfg.get("weights") == "q8_0":  # lm_head and markov weights as Q8_0 (q int8, d binary16 bits)
        out["Wq_lm"], out["Wd_lm"] = normal_q8(seed, S_W_LM, (V, d))
        out["w1q"], out["w1d"] = normal_q8(seed, S_W1, (V, r))
        out["w2q"], out["w2d"] = normal_q8(seed, S_W2, (V, r))
    else:
        out["W_lm"] = normal_bf16(seed, S_W_LM, (V, d))
        out["w1"] = normal_bf16(seed, S_W1, (V, r))
        out["w2"] = normal_bf16(seed, S_W2, (V, r))
    out["H"] = normal_f32(seed, S_H, (R * B, d))
    out["prev0"] = uniform_index(seed, S_PREV0, R, V)
    out["probe_w"] = normal_bf16(seed, S_PROBE_W, (d,))
    out["probe_bias"] = np.float32(0.0)
    out["probe_threshold"] = np.float32(0.0)
    return out


def layer_inputs(seed: int | None = None, copies: int = 1):
    """One draft layer at M = 7 (q/k/v/o [4096, 4096], gate/up [12288, 4096],
    down [4096, 12288], bf16 ~ N(0, 0.02^2)), inputs X [7, K] ~ N(0, 1), and
    a 7424-wide probe (w ~ N(0, 0.02^2), x ~ N(0, 1)). As in a transformer
    layer, q, k and v read the same input, and so do gate and up; o and down
    have their own.

    ``copies`` > 1 draws that many independent weight sets.
    """
    cfg = CONFIGS["draft_layer"]
    seed = config_seed("draft_layer") if seed is None else seed
    M, d, f = cfg["M"], cfg["d"], cfg["ffn"]
    shapes = dict(q=(d, d), k=(d, d), v=(d, d), o=(d, d), gate=(f, d), up=(f, d), down=(d, f))
    layers = []
    for c in range(copies):
        ws = {}
        for j, (nm, shp) in enumerate(shapes.items()):
            ws[nm] = normal_bf16(seed, S_LAYER + 16 * c + j, shp)
        layers.append(ws)
    xs = {nm: normal_f32(seed, S_LAYER + 15 * 16 + j, (M, shp[1])) for j, (nm, shp) in enumerate(shapes.items())
          if nm in ("q", "o", "gate", "down")}
    xs["k"] = xs["v"] = xs["q"]
    xs["up"] = xs["gate"]
    px, pw = probe_inputs(M, cfg["probe_width"], seed)
    return dict(cfg, seed=seed, layers=layers, X=xs, probe_x=px, probe_w=pw,
                probe_bias=np.float32(0.0), probe_threshold=np.float32(0.0))


def block_inputs(R: int, B: int, H: int, Dh: int, F: int, Lmax: int, ctx_len, seed: int, copies: int = 1):
    """A draft block (layer) at M = R * B: weights bf16 ~ N(0, 0.02^2) of
    qkv [3 H Dh, d], o [d, H Dh], gate_up [2F, d], down [d, F] (d = H Dh),
    norm gains ln1, ln2 ~ 1 + N(0, 0.1^2) in bf16; hidden states h [R * B, d]
    ~ N(0, 1); context keys and values bf16 [R, Lmax, d] ~ N(0, 1); the given
    context lengths. ``copies`` > 1 draws that many weight sets (layers)."""
    d = H * Dh
    layers = []
    for c in range(copies):
        base = S_LAYER + 16 * (20 + c)
        w = dict(qkv=normal_bf16(seed, base, (3 * d, d)), o=normal_bf16(seed, base + 1, (d, d)),
                 gate_up=normal_bf16(seed, base + 2, (2 * F, d)), down=normal_bf16(seed, base + 3, (d, F)))
        w["ln1"] = bf16_bits_rne(1.0 + normal_f32(seed, base + 4, (d,), 0.1))
        w["ln2"] = bf16_bits_rne(1.0 + normal_f32(seed, base + 5, (d,), 0.1))
        layers.append(w)
    h = normal_f32(seed, S_LAYER + 16 * 19, (R * B, d))
    k_ctx = normal_bf16(seed, S_LAYER + 16 * 19 + 1, (R, Lmax, d), 1.0)
    v_ctx = normal_bf16(seed, S_LAYER + 16 * 19 + 2, (R, Lmax, d), 1.0)
    return dict(h=h, layers=layers, k_ctx=k_ctx, v_ctx=v_ctx, ctx_len=np.asarray(ctx_len, np.int32),
                R=R, B=B, H=H, Dh=Dh, F=F, d=d, Lmax=Lmax, eps=np.float32(1e-6))


def draft_forward_inputs(R: int, B: int, H: int, Dh: int, F: int, Lmax: int, ctx_len, layers: int, n_fc: int,
                         seed: int) -> dict:
    """A drafter of ``layers`` blocks at M = R * B: the blocks of block_inputs
    (weights and a context cache per block), fc bf16 [d, n_fc d] ~ N(0, 0.02^2)
    and its input x_in [R * B, n_fc d] ~ N(0, 1), and a final norm gain
    norm [d] ~ 1 + N(0, 0.1^2) in bf16."""
    d = H * Dh
    blk = block_inputs(R, B, H, Dh, F, Lmax, ctx_len, seed, copies=layers)
    k_ctx = [blk["k_ctx"]] + [normal_bf16(seed, S_LAYER + 16 * (60 + c), (R, Lmax, d), 1.0) for c in range(1, layers)]
    v_ctx = [blk["v_ctx"]] + [normal_bf16(seed, S_LAYER + 16 * (60 + c) + 1, (R, Lmax, d), 1.0)
                              for c in range(1, layers)]
    fc = normal_bf16(seed, S_LAYER + 16 * 58, (d, n_fc * d))
    x_in = normal_f32(seed, S_LAYER + 16 * 58 + 1, (R * B, n_fc * d))
    norm = bf16_bits_rne(1.0 + normal_f32(seed, S_LAYER + 16 * 58 + 2, (d,), 0.1))
    return dict(blk, k_ctx=k_ctx, v_ctx=v_ctx, fc=fc, x_in=x_in, norm=norm, n_fc=n_fc)


def fused_layer(ws: dict) -> dict:
    """The same layer with the projections that share an input concatenated
    along N: qkv [3 * 4096, 4096] (rows q, then k, then v) and gate_up
    [2 * 12288, 4096]; o and down unchanged. Output columns follow the same
    order, so y_qkv[:, :4096] is q, and so on."""
    return dict(qkv=np.concatenate([ws["q"], ws["k"], ws["v"]]), o=ws["o"],
                gate_up=np.concatenate([ws["gate"], ws["up"]]), down=ws["down"])


FUSED_INPUT = dict(qkv="q", o="o", gate_up="gate", down="down")  # fused projection -> its input's name
