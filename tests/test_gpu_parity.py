"""Parity of every C-ABI entry point with the fp64 oracle on an MI355X.

Inputs come from the seeded generator; expected values only from the oracle.
Each case prints its name, seed and shape before touching the GPU.
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


def _bf(bits, dev):
    return _ops().bf16_from_bits(bits, dev)


# ---------------------------------------------------------------------------
# GEMV: projections and lm_head
# ---------------------------------------------------------------------------

GEMV_CASES = [
    # (M, N, K): tiles, ragged N tails, K tails (K % 64 != 0), every row packing
    (1, 1, 8), (4, 4096, 256), (7, 4096 + 8, 264), (7, 17, 4096), (8, 1000, 520),
    (9, 333, 264), (15, 4096, 5120), (16, 2049, 1032), (17, 515, 264), (33, 1024, 512),
    (72, 3203, 640), (130, 300, 136), (7, 4096, 7424), (3, 32000 + 3, 256),
    (5, 1000, 1032), (8, 777, 3000), (2, 4099, 2048), (7, 16, 1096),
]


@pytest.mark.parametrize("M,N,K", GEMV_CASES)
@pytest.mark.parametrize("entry", ["proj_smallm", "lm_head"])
def test_gemv_matches_oracle(dev, entry, M, N, K):
    seed = 7000 + M * 31 + N + K
    say(f"[gemv {entry}] M={M} N={N} K={K} seed={seed}")
    W, X = synth.gemv_inputs(M, N, K, seed)
    y = getattr(_ops(), entry)(_bf(W, dev), _up(X, dev))
    torch.cuda.synchronize()
    logits_close(y.cpu().numpy(), oracle.gemv(W, X), f"{entry} M={M} N={N} K={K}")


MWIDE_CASES = [
    # (M, N, K) with 16 < M <= 80, one launch: every count of A blocks (a hi
    # and a lo block per 16 rows, one shared block for an odd last group of
    # at most 8), ragged N (past a multiple of 128 and of 16), K tails
    # (K % 128 != 0, one k-group of 8), K of several pipeline rounds
    (17, 300, 136), (24, 1000 + 5, 776), (25, 129, 8), (32, 515, 1032), (40, 2000 + 3, 264),
    (41, 128, 5120), (48, 700, 520), (49, 1000, 1544), (56, 257, 776), (64, 1001, 264),
    (65, 3000, 1032), (72, 4000 + 3, 5120), (73, 515, 776), (80, 1027, 2056),
]


@pytest.mark.parametrize("M,N,K", MWIDE_CASES)
def test_gemv_medium_m_matches_oracle(dev, M, N, K):
    """The batched lm_head's small-GEMM path: every output within the
    tolerance of the oracle, reruns bit-identical, and a residual added to
    the outputs in place."""
    seed = 7300 + M * 31 + N + K
    say(f"[gemv medium M] M={M} N={N} K={K} seed={seed}")
    W, X = synth.gemv_inputs(M, N, K, seed)
    ops = _ops()
    Wd, Xd = _bf(W, dev), _up(X, dev)
    y = ops.lm_head(Wd, Xd)
    y2 = ops.lm_head(Wd, Xd)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "rerun differs"
    ref = oracle.gemv(W, X)
    logits_close(y.cpu().numpy(), ref, f"lm_head M={M} N={N} K={K}")
    r = torch.randn(M, N, device=dev, generator=torch.Generator(device=dev).manual_seed(seed))
    r0 = r.clone()
    ops.proj_smallm_add(Wd, Xd, r, out=r)
    torch.cuda.synchronize()
    assert torch.equal(r, r0 + y), "residual not added to the same outputs"


SPLIT_CASES = [
    # (M, N, K) with M > 16: every count of A blocks, ragged N (past a
    # multiple of 256, one row, fewer rows than a block), K of one 64-wide
    # chunk (the second half empty), an odd number of chunks, K tails
    # (K % 64 != 0), several launches of at most 80 rows
    (17, 300, 136), (24, 1000 + 5, 776), (25, 129, 8), (32, 515, 1032), (41, 257, 5120),
    (49, 1000, 1544), (56, 1, 64), (64, 1001, 264), (65, 3000, 1032), (72, 4000 + 3, 5120),
    (73, 515, 200), (80, 1027, 2056), (81, 700, 1000), (160, 513, 320),
    # the batched lane's d with 84 and 90 rows (two launch parts each)
    (84, 9003, 5120), (90, 2003, 4096),
]


@pytest.mark.parametrize("M,N,K", SPLIT_CASES)
def test_lm_head_split_matches_oracle(dev, M, N, K):
    """dspark_lm_head_split (K in two halves, the second finisher adds):
    every output within the tolerance of the oracle; reruns bit-identical;
    every ticket word 0 after each call; a workspace sized for a larger
    shape serves a smaller one; and the outputs equal dspark_lm_head's up to
    rounding."""
    seed = 7500 + M * 31 + N + K
    say(f"[lm_head split] M={M} N={N} K={K} seed={seed}")
    W, X = synth.gemv_inputs(M, N, K, seed)
    ops = _ops()
    Wd, Xd = _bf(W, dev), _up(X, dev)
    n = ops.lm_head_split_workspace_bytes(N, K, M)
    assert n > 0
    ws = torch.zeros(ops.lm_head_split_workspace_bytes(N + 1000, K, M) + 4096, dtype=torch.uint8, device=dev)
    y = ops.lm_head_split(Wd, Xd, ws)
    torch.cuda.synchronize()
    ticks = (((N + 255) // 256 + 7) // 8) * 8
    assert int(ws[: 4 * ticks].count_nonzero().item()) == 0, "a ticket word was left set"
    y2 = ops.lm_head_split(Wd, Xd, ws)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "rerun differs"
    ref = oracle.gemv(W, X)
    logits_close(y.cpu().numpy(), ref, f"lm_head_split M={M} N={N} K={K}")
    one = ops.lm_head(Wd, Xd)
    torch.cuda.synchronize()
    assert torch.allclose(y, one, rtol=1e-5, atol=1e-5)


def test_lm_head_split_full_size_and_graph(dev):
    """The batched lane's lm_head [72 x 5120] x [32000 x 5120] through the
    split, sampled rows against the oracle; the same call recorded in a HIP
    graph and replayed (eager work between replays) gives the same bits."""
    M, N, K, seed = 72, 32000, 5120, 7641
    say(f"[lm_head split full] M={M} N={N} K={K} seed={seed}")
    W, X = synth.gemv_inputs(M, N, K, seed)
    ops = _ops()
    Wd, Xd = _bf(W, dev), _up(X, dev)
    ws = ops.lm_head_split_workspace(N, K, M, dev)
    out = torch.empty(M, N, device=dev)
    ops.lm_head_split(Wd, Xd, ws, out=out)
    torch.cuda.synchronize()
    eager = out.clone()
    rows = np.random.default_rng(seed).choice(N, 512, replace=False)
    logits_close(eager.cpu().numpy()[:, rows], oracle.gemv(W[rows], X), "lm_head_split full sampled")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ops.lm_head_split(Wd, Xd, ws, out=out)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ops.lm_head_split(Wd, Xd, ws, out=out)
    for rep in range(3):
        out.fill_(7.0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs"
        _ = ops.lm_head(Wd, Xd[:20])  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["draft_layer"])
def test_draft_layer_projections(dev, name):
    inp = synth.layer_inputs()
    for proj, Wb in inp["layers"][0].items():
        X = inp["X"][proj]
        say(f"[proj {proj}] W {Wb.shape} X {X.shape} seed={inp['seed']}")
        y = _ops().proj_smallm(_bf(Wb, dev), _up(X, dev))
        torch.cuda.synchronize()
        logits_close(y.cpu().numpy(), oracle.gemv(Wb, X), f"proj {proj}")


def test_draft_layer_fused_projections(dev):
    """q/k/v as one GEMV over the concatenated weight (and gate/up likewise):
    each slice of the output matches the oracle of its own projection."""
    inp = synth.layer_inputs()
    ws = inp["layers"][0]
    fused = synth.fused_layer(ws)
    parts = dict(qkv=["q", "k", "v"], o=["o"], gate_up=["gate", "up"], down=["down"])
    for nm, Wb in fused.items():
        X = inp["X"][synth.FUSED_INPUT[nm]]
        say(f"[proj fused {nm}] W {Wb.shape} X {X.shape} seed={inp['seed']}")
        y = _ops().proj_smallm(_bf(Wb, dev), _up(X, dev))
        torch.cuda.synchronize()
        y = y.cpu().numpy()
        col = 0
        for part in parts[nm]:
            n = ws[part].shape[0]
            logits_close(y[:, col:col + n], oracle.gemv(ws[part], inp["X"][part]), f"proj {nm}/{part}")
            col += n
        assert col == y.shape[1]


SCHED_CASES = [
    # (rows, V, d): the scheduled kernel takes vocabularies of more than 16
    # tiles of 16 rows per CU (V > 65536 on 256 CUs): a ragged last unit of
    # 32 rows, two K phases (the second full, then partial), a single row
    # with one partial k-block; smaller vocabularies run dspark_lm_head's
    # kernels and leave the counter alone
    (5, 70001, 1024), (8, 66003, 4096), (3, 70000, 2056), (1, 65601, 8), (7, 33, 256), (7, 19200, 256),
    # 65 static units per workgroup: its LDS holds 64 units' outputs, so it
    # writes them out mid-way and goes on
    (2, 600001, 8),
]


@pytest.mark.parametrize("rows,V,d", SCHED_CASES)
def test_lm_head_sched_matches_oracle(dev, rows, V, d):
    """Rows handed out by a counter: every row computed once, the counter
    left at 0 by every call, reruns bit-identical."""
    seed = 7700 + rows + V + d
    say(f"[lm_head sched] rows={rows} V={V} d={d} seed={seed}")
    W, X = synth.gemv_inputs(rows, V, d, seed)
    ops = _ops()
    Wd, Xd = _bf(W, dev), _up(X, dev)
    cnt = ops.lm_head_counter(dev)
    y = ops.lm_head_sched(Wd, Xd, cnt)
    y2 = ops.lm_head_sched(Wd, Xd, cnt)
    torch.cuda.synchronize()
    assert int(cnt.item()) == 0, "the counter was not left at 0"
    assert torch.equal(y, y2), "rerun differs"
    logits_close(y.cpu().numpy(), oracle.gemv(W, X), f"lm_head sched rows={rows} V={V} d={d}")


def test_lm_head_sched_full_size(dev):
    """At the Qwen3-8B head's shape the scheduled lm_head gives the bits of
    dspark_lm_head (the same summation order for every logit), whichever
    workgroup computed a row; shapes it does not take (9 rows) run
    dspark_lm_head's kernels and leave the counter alone."""
    cfg = synth.CONFIGS["qwen3_8b_head"]
    V, d, rows = cfg["V"], cfg["d"], cfg["B"]
    seed = synth.config_seed("qwen3_8b_head")
    say(f"[lm_head sched full] V={V} d={d} rows={rows}")
    ops = _ops()
    W = _bf(synth.normal_bf16(seed, synth.S_W_LM, (V, d)), dev)
    H = _up(synth.normal_f32(seed, synth.S_H, (9, d)), dev)
    cnt = ops.lm_head_counter(dev)
    ref = ops.lm_head(W, H[:rows].contiguous())
    for rep in range(3):
        y = ops.lm_head_sched(W, H[:rows].contiguous(), cnt)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"call {rep} differs from dspark_lm_head"
        assert int(cnt.item()) == 0
    cnt.fill_(5)
    y9 = ops.lm_head_sched(W, H, cnt)
    torch.cuda.synchronize()
    assert int(cnt.item()) == 5, "a shape outside the scheduled kernel touched the counter"
    assert torch.equal(y9, ops.lm_head(W, H))


@pytest.mark.parametrize("nbytes,groups,threads", [(1 << 30, 256, 1024), (40 * 256 * 1024 + 4096, 8, 256), (0, 4, 512),
                                                    (3 * 256 * 1024, 16, 1024)])
def test_stream_read_sched_reads_every_byte_once(dev, nbytes, groups, threads):
    """The scheduled read (static runs, then units from the counter) folds
    to the same word as the plain read, so every 16-byte piece was read once
    by one workgroup; the counter is left at 0 (also with fewer units than
    workgroups, or none)."""
    say(f"[stream read sched] bytes={nbytes} groups={groups} threads={threads}")
    ops = _ops()
    g = torch.Generator(device="cpu").manual_seed(nbytes % 1000 + groups)
    buf = torch.randint(0, 2 ** 31 - 1, (max(nbytes // 4, 1),), dtype=torch.int32, generator=g).to(dev)
    cnt = ops.lm_head_counter(dev)
    a = ops.stream_read(buf, groups, threads, nbytes=nbytes)
    for _ in range(2):
        b = ops.stream_read_sched(buf, groups, threads, cnt, nbytes=nbytes)
        torch.cuda.synchronize()
        assert int(cnt.item()) == 0
        fa = int(np.bitwise_xor.reduce(a.cpu().numpy().astype(np.uint32)))
        fb = int(np.bitwise_xor.reduce(b.cpu().numpy().astype(np.uint32)))
        assert fa == fb, "the scheduled read did not read every piece once"


def test_lm_head_full_size_sampled(dev):
    """Qwen3-8B-shaped head at full size in the benchmark's launch
    configuration; oracle on sampled vocabulary rows incl. the ragged tail."""
    cfg = synth.CONFIGS["qwen3_8b_head"]
    V, d, rows = cfg["V"], cfg["d"], cfg["B"]
    seed = synth.config_seed("qwen3_8b_head")
    say(f"[lm_head full] V={V} d={d} rows={rows} seed={seed}")
    W = synth.normal_bf16(seed, synth.S_W_LM, (V, d))
    H = synth.normal_f32(seed, synth.S_H, (rows, d))
    y = _ops().lm_head(_bf(W, dev), _up(H, dev)).cpu().numpy()
    pick = np.unique(np.concatenate([np.arange(32), np.arange(V - 48, V),
                                     np.random.default_rng(1).choice(V, 4000, replace=False)]))
    logits_close(y[:, pick], oracle.gemv_rows(W, H, pick), "lm_head sampled")


# ---------------------------------------------------------------------------
# GEMV over Q8_0 weights
# ---------------------------------------------------------------------------

GEMV_Q8_CASES = [
    # (M, N, K): one block, K not a multiple of the 128-entry wave segment,
    # several phases with a partial last one, ragged N, both row packings,
    # more than 16 rows (several launches). Up to 16 tiles per workgroup
    # (N up to ~65k rows on 256 CUs) take the short kernel, one tile or
    # several; longer workgroups the streaming kernel, with one K phase or
    # several (last three cases).
    (1, 1, 32), (7, 4096, 4096), (7, 4099, 96), (15, 1000, 160), (16, 2049, 4128), (3, 300, 7424),
    (8, 33, 64), (9, 777, 2080), (20, 515, 256), (4, 65, 5120), (7, 16, 12288), (15, 4096, 4128),
    (7, 70001, 160), (15, 66003, 2080), (5, 90017, 4160),
]


@pytest.mark.parametrize("M,N,K", GEMV_Q8_CASES)
@pytest.mark.parametrize("entry", ["proj_smallm_q8", "lm_head_q8"])
def test_gemv_q8_matches_oracle(dev, entry, M, N, K):
    seed = 7100 + M * 31 + N + K
    say(f"[gemv {entry}] M={M} N={N} K={K} seed={seed}")
    Wq, Wd, X = synth.gemv_q8_inputs(M, N, K, seed)
    q, d = _ops().q8_from_numpy(Wq, Wd, dev)
    y = getattr(_ops(), entry)(q, d, _up(X, dev))
    torch.cuda.synchronize()
    logits_close(y.cpu().numpy(), oracle.gemv_q8(Wq, Wd, X), f"{entry} M={M} N={N} K={K}")


def test_gemv_q8_scale_edge_values(dev):
    """Scales of either sign, subnormal and the largest binary16, quants at
    -128 and 127: every block's scale lands on its own 32 entries."""
    M, N, K = 5, 70, 192
    g = np.random.default_rng(77)
    say(f"[gemv q8 edge scales] M={M} N={N} K={K}")
    Wq = g.integers(-128, 128, size=(N, K)).astype(np.int8)
    Wq[0, :] = -128
    Wq[1, :] = 127
    e = g.integers(1, 22, size=(N, K // 32))
    Wd = ((g.integers(0, 2, size=e.shape) << 15) | (e << 10) | g.integers(0, 1024, size=e.shape)).astype(np.uint16)
    Wd[2, :] = 0x0001  # least subnormal
    Wd[3, :] = 0x7BFF  # 65504
    Wd[4, :] = 0x8000  # -0
    X = (g.standard_normal((M, K)) * 0.01).astype(np.float32)
    q, d = _ops().q8_from_numpy(Wq, Wd, dev)
    y = _ops().proj_smallm_q8(q, d, _up(X, dev))
    torch.cuda.synchronize()
    logits_close(y.cpu().numpy(), oracle.gemv_q8(Wq, Wd, X), "q8 edge scales")


def test_lm_head_q8_full_size_sampled(dev):
    """Qwen3-8B-shaped head with Q8_0 weights at full size; oracle on sampled
    rows incl. the ragged tail; reruns bit-identical; a row's output does not
    depend on the other rows (M = 7 vs M = 1, same packing)."""
    cfg = synth.CONFIGS["qwen3_8b_head"]
    V, d, rows = cfg["V"], cfg["d"], cfg["B"]
    seed = synth.config_seed("qwen3_8b_head")
    say(f"[lm_head q8 full] V={V} d={d} rows={rows} seed={seed}")
    Wq, Wd, H = synth.gemv_q8_inputs(rows, V, d, seed)
    q, dd = _ops().q8_from_numpy(Wq, Wd, dev)
    Hd = _up(H, dev)
    y = _ops().lm_head_q8(q, dd, Hd)
    y2 = _ops().lm_head_q8(q, dd, Hd)
    y1 = _ops().lm_head_q8(q, dd, Hd[3:4].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "rerun differs"
    assert torch.equal(y[3:4], y1), "row 3 depends on the other rows"
    y = y.cpu().numpy()
    pick = np.unique(np.concatenate([np.arange(32), np.arange(V - 48, V),
                                     np.random.default_rng(1).choice(V, 3000, replace=False)]))
    logits_close(y[:, pick], oracle.gemv_q8_rows(Wq, Wd, H, pick), "lm_head q8 sampled")


@pytest.mark.parametrize("N,K", [(9000, 4096), (151936, 4096), (4096, 12288), (248320, 5120)])
def test_gemv_invariants(dev, N, K):
    """Deterministic reruns; a row's output does not depend on the other rows
    (bit-identical for every M within a row class: 1..8 and 9..16); equal
    weight rows give equal outputs wherever they sit."""
    say(f"[gemv invariants] N={N} K={K}")
    W, X = synth.gemv_inputs(16, N, K, 99)
    W[N // 2 + 5] = W[17]
    W[N - 1] = W[17]
    Wd, Xd = _bf(W, dev), _up(X, dev)
    ops = _ops()
    y8a, y8b = ops.lm_head(Wd, Xd[:8].contiguous()), ops.lm_head(Wd, Xd[:8].contiguous())
    y7 = ops.lm_head(Wd, Xd[:7].contiguous())
    y1 = ops.lm_head(Wd, Xd[3:4].contiguous())
    y16 = ops.lm_head(Wd, Xd)
    y9 = ops.lm_head(Wd, Xd[:9].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(y8a, y8b)
    assert torch.equal(y7, y8a[:7])
    assert torch.equal(y1[0], y8a[3])
    assert torch.equal(y9, y16[:9])
    for y in (y8a, y16):
        assert torch.equal(y[:, N // 2 + 5], y[:, 17]) and torch.equal(y[:, N - 1], y[:, 17])


# ---------------------------------------------------------------------------
# Markov loop
# ---------------------------------------------------------------------------

MARKOV_CASES = [
    # (R, B, k, V, r)
    (1, 4, 4, 4096, 32), (1, 7, 7, 1, 8), (1, 3, 2, 5, 8), (2, 5, 5, 17, 16), (1, 7, 7, 20011, 256),
    (3, 6, 4, 4099, 264), (8, 9, 9, 32000 + 7, 256), (16, 2, 2, 3001, 64), (5, 3, 3, 2000, 1024),
    (1, 15, 15, 9000, 128), (16, 3, 2, 300000, 32),
]


@pytest.mark.parametrize("R,B,k,V,r", MARKOV_CASES)
def test_markov_matches_oracle(dev, R, B, k, V, r):
    seed = 500 + R * 7 + V + r
    say(f"[markov] R={R} B={B} k={k} V={V} r={r} seed={seed}")
    base, w1, w2, prev0, _ = synth.markov_inputs(R, B, V, r, seed)
    ids = _ops().markov_sample(_up(base, dev), _bf(w1, dev), _bf(w2, dev), _up(prev0, dev), k)
    torch.cuda.synchronize()
    check_markov(ids.cpu().numpy(), base, w1, w2, prev0, k)


def test_markov_workspace_reused_across_shapes(dev):
    """One zero-filled workspace serves a sequence of calls whose step
    count, request count and grid size go up and down: the loop leaves its
    key slots clean for the next call without a clearing launch."""
    ws = _ops().markov_workspace(1, 1, 1, dev)
    seq = [(1, 7, 7, 20011, 256), (16, 2, 2, 3001, 64), (1, 15, 15, 9000, 128), (2, 5, 5, 17, 16),
           (8, 9, 9, 32007, 256), (1, 3, 2, 5, 8), (1, 15, 15, 9000, 128), (3, 6, 4, 4099, 264)]
    for n, (R, B, k, V, r) in enumerate(seq):
        seed = 4100 + n
        say(f"[markov reuse {n}] R={R} B={B} k={k} V={V} r={r} seed={seed}")
        base, w1, w2, prev0, _ = synth.markov_inputs(R, B, V, r, seed)
        ids = _ops().markov_sample(_up(base, dev), _bf(w1, dev), _bf(w2, dev), _up(prev0, dev), k, workspace=ws)
        torch.cuda.synchronize()
        check_markov(ids.cpu().numpy(), base, w1, w2, prev0, k)


def _markov_case(dev, R, B, k, V, r, seed):
    base, w1, w2, prev0, _ = synth.markov_inputs(R, B, V, r, seed)
    return (base, w1, w2, prev0), (_up(base, dev), _bf(w1, dev), _bf(w2, dev), _up(prev0, dev), k)


@pytest.mark.parametrize("mark", [1, 7])
def test_markov_marked_workspace_repairs_itself(dev, mark):
    """A workspace marked as a grid-wide wait that gave up leaves it (the
    state word set from the host: 1, or any value but 0 and 2) is repaired by
    the next call, whose ids are -2; the call after that samples normally,
    with no zero-fill by the caller."""
    R, B, k, V, r = 2, 5, 5, 3000, 64
    say(f"[markov repair] mark={mark} R={R} V={V} r={r}")
    host, args = _markov_case(dev, R, B, k, V, r, 91)
    ws = _ops().markov_workspace(R, k, V, dev)
    good = _ops().markov_sample(*args, workspace=ws).clone()
    ws[0] = mark  # low byte of the state word
    ids = _ops().markov_sample(*args, workspace=ws)
    torch.cuda.synchronize()
    assert torch.all(ids == -2)
    for _ in range(3):
        ids = _ops().markov_sample(*args, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(ids, good)
    assert int(ws[:4].view(torch.int32)[0]) == 0, "the state word is back to normal"
    check_markov(ids.cpu().numpy(), host[0], host[1], host[2], host[3], k)


def test_markov_repair_inside_a_replayed_graph(dev):
    """The repair under graph replay: the replay that finds the mark repairs
    (-2); the next replay of the same recorded launch recognises the repair
    as its own and only drops the record (-2); every later replay samples."""
    R, B, k, V, r = 1, 7, 7, 20011, 256
    say(f"[markov repair in graph] R={R} V={V} r={r}")
    _, args = _markov_case(dev, R, B, k, V, r, 92)
    ops = _ops()
    ws = ops.markov_workspace(R, k, V, dev)
    out = torch.empty(R, k, dtype=torch.int64, device=dev)
    good = ops.markov_sample(*args, workspace=ws).clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ops.markov_sample(*args, workspace=ws, out=out)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ops.markov_sample(*args, workspace=ws, out=out)
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, good)
    ws[0] = 1
    want = ["repair", "own record", "sample", "sample"]
    for rep, what in enumerate(want):
        out.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        if what == "sample":
            assert torch.equal(out, good), f"replay {rep}"
        else:
            assert torch.all(out == -2), f"replay {rep} ({what})"
        _ = ops.markov_sample(*args)  # eager work (own workspace) between replays
        torch.cuda.synchronize()


def test_markov_forced_give_up_then_recovers(dev):
    """A poll bound of one poll (set from the host) makes the grid-wide waits
    of an ordinary call give up: that call's ids are -2 and every kernel
    exits normally. With the default bound restored, the next call repairs
    the workspace (-2) and the one after it samples correctly."""
    R, B, k, V, r = 1, 7, 7, 151936, 256
    say(f"[markov forced give-up] R={R} V={V} r={r}")
    host, args = _markov_case(dev, R, B, k, V, r, 93)
    ops = _ops()
    ws = ops.markov_workspace(R, k, V, dev)
    good = ops.markov_sample(*args, workspace=ws).clone()
    gave_up = False
    for attempt in range(3):
        prev = ops.markov_set_spin_limit(1)
        try:
            ids = ops.markov_sample(*args, workspace=ws)
        finally:
            ops.markov_set_spin_limit(0)
        torch.cuda.synchronize()
        if torch.all(ids == -2):
            gave_up = True
            ids = ops.markov_sample(*args, workspace=ws)
            torch.cuda.synchronize()
            assert torch.all(ids == -2), "the call after a give-up repairs"
        else:
            assert torch.equal(ids, good), f"attempt {attempt}: neither -2 nor correct"
        ids = ops.markov_sample(*args, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(ids, good)
        if gave_up:
            break
    assert prev == 1 << 18
    assert gave_up, "a one-poll bound never gave up (the path was not exercised)"
    check_markov(ids.cpu().numpy(), host[0], host[1], host[2], host[3], k)


def test_markov_beside_a_long_gemv_on_another_stream(dev):
    """The loop launched while lm_head GEMVs queued on another stream of the
    same process hold compute units: its workgroups may start late, which
    the bounded waits absorb. The ids are correct, or (if a wait gave up)
    -2 followed by the documented repair."""
    R, B, k, V, r = 1, 7, 7, 151936, 256
    say(f"[markov beside gemv] R={R} V={V} r={r}")
    host, args = _markov_case(dev, R, B, k, V, r, 94)
    ops = _ops()
    ws = ops.markov_workspace(R, k, V, dev)
    good = ops.markov_sample(*args, workspace=ws).clone()
    W = (torch.randn(151936, 4096, device=dev) * 0.02).to(torch.bfloat16)
    H = torch.randn(7, 4096, device=dev)
    y = torch.empty(7, 151936, device=dev)
    torch.cuda.synchronize()
    s2 = torch.cuda.Stream()
    outcomes = []
    for trial in range(3):
        with torch.cuda.stream(s2):
            for _ in range(6):
                ops.lm_head(W, H, out=y)
        ids = ops.markov_sample(*args, workspace=ws)  # current stream, beside them
        torch.cuda.synchronize()
        if torch.all(ids == -2):
            outcomes.append("gave up")
            again = ops.markov_sample(*args, workspace=ws)
            torch.cuda.synchronize()
            assert torch.all(again == -2)
        else:
            outcomes.append("ok")
            assert torch.equal(ids, good), f"trial {trial}"
        ids = ops.markov_sample(*args, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(ids, good)
    say(f"[markov beside gemv] outcomes {outcomes}")
    check_markov(ids.cpu().numpy(), host[0], host[1], host[2], host[3], k)


def test_markov_d2t_and_sentinel(dev):
    R, B, k, V, r = 4, 5, 5, 3000, 64
    say(f"[markov d2t+sentinel] R={R} V={V} r={r}")
    base, w1, w2, prev0, _ = synth.markov_inputs(R, B, V, r, 77)
    prev0[1] = V        # out of range -> -1 row
    prev0[3] = -5
    d2t = synth.d2t_map(V, 77)
    ids = _ops().markov_sample(_up(base, dev), _bf(w1, dev), _bf(w2, dev), _up(prev0, dev), k, d2t=_up(d2t, dev))
    torch.cuda.synchronize()
    ids = ids.cpu().numpy()
    assert np.all(ids[1] == -1) and np.all(ids[3] == -1)
    check_markov(ids, base, w1, w2, prev0, k, d2t=d2t)


@pytest.mark.parametrize("exact", [True, False])
def test_markov_constructed_ties(dev, exact):
    """27B-lane shape with 5% of base rows given a duplicated top value at two
    indices; with exact=True markov_w2's rows are equal too, so the scores
    tie exactly and the lower index must win."""
    cfg = synth.CONFIGS["lane27b"]
    R, B, V, r = cfg["num_reqs"], cfg["B"], cfg["V"], cfg["r"]
    seed = synth.config_seed("lane27b")
    say(f"[markov ties exact={exact}] V={V} r={r} B={B} seed={seed}")
    base, w1, w2, prev0, ties = synth.markov_inputs(R, B, V, r, seed, tie_frac=0.05, tie_exact=exact)
    ids = _ops().markov_sample(_up(base, dev), _bf(w1, dev), _bf(w2, dev), _up(prev0, dev), B)
    torch.cuda.synchronize()
    ids = ids.cpu().numpy()
    if exact:
        for (q, i, a, b) in ties:
            assert ids[q, i] == a, f"tie row {i}: ids {ids[q, i]} expected lower index {a} of ({a}, {b})"
    check_markov(ids, base, w1, w2, prev0, B)


def test_markov_full_size_and_invariants(dev):
    """Qwen3-8B head shape at full size: exact ids, deterministic reruns,
    and batched requests equal to single-request runs."""
    cfg = synth.CONFIGS["qwen3_8b_head"]
    B, V, r = cfg["B"], cfg["V"], cfg["r"]
    say(f"[markov full] V={V} r={r} B={B}")
    base, w1, w2, prev0, _ = synth.markov_inputs(3, B, V, r, synth.config_seed("qwen3_8b_head"))
    bd, w1d, w2d, pd = _up(base, dev), _bf(w1, dev), _bf(w2, dev), _up(prev0, dev)
    a = _ops().markov_sample(bd, w1d, w2d, pd, B)
    b = _ops().markov_sample(bd, w1d, w2d, pd, B)
    singles = [_ops().markov_sample(bd[q:q + 1].contiguous(), w1d, w2d, pd[q:q + 1].contiguous(), B) for q in range(3)]
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    for q in range(3):
        assert torch.equal(a[q], singles[q][0])
    check_markov(a.cpu().numpy(), base, w1, w2, prev0, B)


@pytest.mark.parametrize("R,B", [(1, 15), (9, 6)])
def test_markov_lane27b_size(dev, R, B):
    """The 27B lane's vocabulary (248320 x 256): markov_w2 does not fit on
    chip with eight waves per workgroup, so the loop runs one wave per SIMD
    with tiles in AGPRs; R = 9 has waves poll several requests each. Exact
    ids (near-ties reported), 5% tie rows with exactly equal scores."""
    cfg = synth.CONFIGS["lane27b"]
    V, r = cfg["V"], cfg["r"]
    seed = synth.config_seed("lane27b") + R
    say(f"[markov lane27b] R={R} B={B} V={V} r={r} seed={seed}")
    base, w1, w2, prev0, ties = synth.markov_inputs(R, B, V, r, seed, tie_frac=cfg["tie_frac"])
    bd, w1d, w2d, pd = _up(base, dev), _bf(w1, dev), _bf(w2, dev), _up(prev0, dev)
    ids = _ops().markov_sample(bd, w1d, w2d, pd, B)
    again = _ops().markov_sample(bd, w1d, w2d, pd, B)
    torch.cuda.synchronize()
    assert torch.equal(ids, again)
    check_markov(ids.cpu().numpy(), base, w1, w2, prev0, B)


# ---------------------------------------------------------------------------
# Probe
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,D", [(1, 8), (4, 256), (7, 4096), (15, 5120), (72, 5120), (7, 7424), (3, 7432)])
def test_probe_matches_oracle(dev, M, D):
    seed = 900 + M + D
    say(f"[probe] M={M} D={D} seed={seed}")
    x, w = synth.probe_inputs(M, D, seed)
    logit, passed = _ops().conf_probe(_up(x, dev), _bf(w, dev), 0.25, 0.0)
    torch.cuda.synchronize()
    ref_l, ref_p = oracle.conf_probe(x, w, 0.25, 0.0)
    probe_close(logit.cpu().numpy(), passed.cpu().numpy(), ref_l, ref_p, 0.0)


def test_probe_threshold_boundary(dev):
    """Logit exactly equal to the threshold passes (integer-valued data)."""
    say("[probe boundary]")
    x = np.zeros((3, 16), np.float32)
    x[:, 0], x[:, 1] = 2.0, 2.0
    w = np.zeros(16, np.float32)
    w[0], w[1] = 1.0, -0.5
    wb = synth.bf16_bits_rne(w)
    logit, passed = _ops().conf_probe(_up(x, dev), _bf(wb, dev), 0.0, 1.0)
    torch.cuda.synchronize()
    assert np.all(logit.cpu().numpy() == 1.0) and np.all(passed.cpu().numpy() == 1)
    logit, passed = _ops().conf_probe(_up(x, dev), _bf(wb, dev), -0.5, 1.0)
    torch.cuda.synchronize()
    assert np.all(passed.cpu().numpy() == 0)


# ---------------------------------------------------------------------------
# A whole round, chained, and under graph capture
# ---------------------------------------------------------------------------

def _round_tensors(name, dev):
    inp = synth.round_inputs(name)
    t = dict(W=_bf(inp["W_lm"], dev), H=_up(inp["H"], dev), w1=_bf(inp["w1"], dev), w2=_bf(inp["w2"], dev),
             prev0=_up(inp["prev0"], dev), pw=_bf(inp["probe_w"], dev))
    return inp, t


def _run_round(inp, t, logits=None, ids=None, ws=None, lg=None, ps=None):
    """The round as separate calls, with the lm_head run like the round's
    own: scheduled (dspark_lm_head_sched) on a counter of its own, or, for
    more than 16 rows, split (dspark_lm_head_split) in a workspace of its
    own."""
    ops = _ops()
    R, B, V = inp["num_reqs"], inp["B"], inp["V"]
    if R * B > 16:
        split_ws = ops.lm_head_split_workspace(V, t["W"].shape[1], R * B, t["H"].device)
        logits = ops.lm_head_split(t["W"], t["H"], split_ws, out=logits)
    else:
        logits = ops.lm_head_sched(t["W"], t["H"], ops.lm_head_counter(t["H"].device), out=logits)
    ids = ops.markov_sample(logits.view(R, B, V), t["w1"], t["w2"], t["prev0"], inp["k"], out=ids, workspace=ws)
    lg, ps = ops.conf_probe(t["H"], t["pw"], float(inp["probe_bias"]), float(inp["probe_threshold"]),
                            logit_out=lg, pass_out=ps)
    return logits, ids, lg, ps


@pytest.mark.parametrize("name", ["tiny", "qwen3_8b_head", "reduced_vocab_batched", "lane27b"])
def test_round_chained(dev, name):
    inp, t = _round_tensors(name, dev)
    say(f"[round {name}] seed={inp['seed']}")
    logits, ids, lg, ps = _run_round(inp, t)
    torch.cuda.synchronize()
    ref = oracle.draft_round(inp["W_lm"], inp["H"], inp["w1"], inp["w2"], inp["prev0"], inp["num_reqs"],
                             inp["B"], inp["k"], inp["probe_w"], inp["probe_bias"], inp["probe_threshold"])
    logits_close(logits.cpu().numpy(), ref["base"], f"round {name} logits")
    # The GPU loop ran on the GPU's own fp32 logits; ids are compared against
    # the oracle loop on the oracle's fp32 logits, with the near-tie rule.
    check_markov(ids.cpu().numpy(), ref["base32"], inp["w1"], inp["w2"], inp["prev0"], inp["k"])
    probe_close(lg.cpu().numpy(), ps.cpu().numpy(), ref["logit"], ref["passed"], float(inp["probe_threshold"]))


@pytest.mark.parametrize("name", ["tiny", "qwen3_8b_head"])
def test_draft_round_dirty_lm_counter(dev, name):
    """A workspace whose lm_head counter word is not 0 (never zero-filled):
    that round's ids are all -2 and the word goes back to 0; the next round
    gives the ids of a clean workspace."""
    inp, t = _round_tensors(name, dev)
    say(f"[draft_round dirty counter {name}] seed={inp['seed']}")
    ops = _ops()
    R, B, k, V = inp["num_reqs"], inp["B"], inp["k"], inp["V"]
    clean = ops.draft_round(t["W"], t["H"], t["w1"], t["w2"], t["prev0"], B, k)["ids"].clone()
    ws = ops.markov_workspace(R, k, V, dev)
    word = ops.markov_lm_counter_offset() // 4
    ws.view(torch.int32)[word] = 12345
    out = ops.draft_round(t["W"], t["H"], t["w1"], t["w2"], t["prev0"], B, k, workspace=ws)
    torch.cuda.synchronize()
    assert (out["ids"] == -2).all(), "a round on a dirty lm_head counter was not reported"
    assert int(ws.view(torch.int32)[word].item()) == 0, "the counter word was not set back to 0"
    again = ops.draft_round(t["W"], t["H"], t["w1"], t["w2"], t["prev0"], B, k, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(again["ids"], clean)


def test_draft_round_dirty_split_tickets(dev):
    """The batched round's split lm_head on ticket words that are not 0 (a
    workspace never zero-filled): a word past 1 makes that round's ids -2;
    the loop leaves every ticket word 0, and the next round equals a round
    on a clean workspace, bit for bit."""
    inp, t = _round_tensors("reduced_vocab_batched", dev)
    ops = _ops()
    R, B, k, V = inp["num_reqs"], inp["B"], inp["k"], inp["V"]
    d = t["W"].shape[1]
    say(f"[draft_round dirty split tickets] seed={inp['seed']}")
    clean = ops.draft_round(t["W"], t["H"], t["w1"], t["w2"], t["prev0"], B, k)
    clean = {n: x.clone() for n, x in clean.items() if x is not None}
    ws = ops.draft_round_workspace(R, B, k, V, d, dev)
    at = (ops.markov_workspace_bytes(R, k, V) + 255) // 256 * 64  # int32 index of the first ticket word
    n = ((V + 255) // 256 + 7) // 8 * 8
    for val in (12345, 1):
        ws.view(torch.int32)[at: at + n] = val
        out = ops.draft_round(t["W"], t["H"], t["w1"], t["w2"], t["prev0"], B, k, workspace=ws)
        torch.cuda.synchronize()
        if val > 1:
            assert (out["ids"] == -2).all(), "a round on dirty ticket words was not reported"
        assert int(ws.view(torch.int32)[at: at + n].count_nonzero().item()) == 0, "ticket words left set"
        again = ops.draft_round(t["W"], t["H"], t["w1"], t["w2"], t["prev0"], B, k, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(again["ids"], clean["ids"]) and torch.equal(again["base"], clean["base"])


@pytest.mark.parametrize("name", ["tiny", "qwen3_8b_head", "reduced_vocab_batched", "lane27b"])
def test_draft_round_fused(dev, name):
    """dspark_draft_round (the probe inside the Markov launch) gives the same
    bits as the three separate calls, and matches the oracle."""
    inp, t = _round_tensors(name, dev)
    say(f"[draft_round {name}] seed={inp['seed']}")
    R, B, k = inp["num_reqs"], inp["B"], inp["k"]
    sep = [x.clone() for x in _run_round(inp, t)]
    out = _ops().draft_round(t["W"], t["H"], t["w1"], t["w2"], t["prev0"], B, k, probe_w=t["pw"],
                             probe_bias=float(inp["probe_bias"]), probe_threshold=float(inp["probe_threshold"]))
    torch.cuda.synchronize()
    assert torch.equal(out["base"].view(R * B, -1), sep[0])
    assert torch.equal(out["ids"], sep[1])
    assert torch.equal(out["logit"], sep[2])
    assert torch.equal(out["passed"], sep[3])
    if name in ("tiny", "reduced_vocab_batched"):
        ref = oracle.draft_round(inp["W_lm"], inp["H"], inp["w1"], inp["w2"], inp["prev0"], R, B, k,
                                 inp["probe_w"], inp["probe_bias"], inp["probe_threshold"])
        logits_close(out["base"].view(R * B, -1).cpu().numpy(), ref["base"], f"draft_round {name} logits")
        check_markov(out["ids"].cpu().numpy(), ref["base32"], inp["w1"], inp["w2"], inp["prev0"], k)
        probe_close(out["logit"].cpu().numpy(), out["passed"].cpu().numpy(), ref["logit"], ref["passed"],
                    float(inp["probe_threshold"]))


# (R, B, k, V, d, r): one workgroup (V <= 256: the probe runs after workgroup
# 0's last step), and more probe rows than the waves that compute them.
SMALL_ROUNDS = [(2, 3, 3, 200, 64, 16), (16, 2, 2, 600, 136, 64), (3, 5, 4, 1000, 8, 8),
                # 84 and 90 drafted rows: the split lm_head in two launch parts inside the round
                (12, 7, 7, 3000, 512, 64), (10, 9, 9, 2000, 256, 32)]


@pytest.mark.parametrize("R,B,k,V,d,r", SMALL_ROUNDS)
def test_draft_round_small_grids(dev, R, B, k, V, d, r):
    seed = 5100 + V + d
    say(f"[draft_round small] R={R} B={B} k={k} V={V} d={d} r={r} seed={seed}")
    W, H = synth.gemv_inputs(R * B, V, d, seed)
    _, w1, w2, prev0, _ = synth.markov_inputs(R, 1, V, r, seed)
    _, pw = synth.probe_inputs(1, d, seed)
    thr = 0.01
    out = _ops().draft_round(_bf(W, dev), _up(H, dev), _bf(w1, dev), _bf(w2, dev), _up(prev0, dev), B, k,
                             probe_w=_bf(pw, dev), probe_bias=-0.02, probe_threshold=thr)
    torch.cuda.synchronize()
    ref = oracle.draft_round(W, H, w1, w2, prev0, R, B, k, pw, -0.02, thr)
    logits_close(out["base"].view(R * B, -1).cpu().numpy(), ref["base"], "draft_round small logits")
    check_markov(out["ids"].cpu().numpy(), ref["base32"], w1, w2, prev0, k)
    probe_close(out["logit"].cpu().numpy(), out["passed"].cpu().numpy(), ref["logit"], ref["passed"], thr)
    lg, ps = _ops().conf_probe(_up(H, dev), _bf(pw, dev), -0.02, thr)
    torch.cuda.synchronize()
    assert torch.equal(out["logit"], lg) and torch.equal(out["passed"], ps)


@pytest.mark.parametrize("R,B,k,V,r,M,D", [(1, 7, 7, 151936, 256, 7, 7424), (8, 9, 9, 32000, 256, 3, 7432),
                                             (2, 3, 2, 200, 16, 40, 64)])
def test_markov_sample_probe(dev, R, B, k, V, r, M, D):
    """The loop and a probe of unrelated shape in one launch: the same bits as
    dspark_markov_sample and dspark_conf_probe called separately."""
    seed = 7300 + M
    say(f"[markov_sample_probe] R={R} B={B} k={k} V={V} r={r} probe M={M} D={D} seed={seed}")
    base, w1, w2, prev0, _ = synth.markov_inputs(R, B, V, r, seed)
    x, pw = synth.probe_inputs(M, D, seed)
    args = (_up(base, dev), _bf(w1, dev), _bf(w2, dev), _up(prev0, dev), k)
    probe = dict(x=_up(x, dev), w=_bf(pw, dev), bias=0.125, threshold=0.0)
    ids = _ops().markov_sample(*args, probe=probe)
    ids_sep = _ops().markov_sample(*args)
    lg, ps = _ops().conf_probe(probe["x"], probe["w"], 0.125, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids_sep)
    assert torch.equal(probe["logit_out"], lg) and torch.equal(probe["pass_out"], ps)
    ref_l, ref_p = oracle.conf_probe(x, pw, 0.125, 0.0)
    probe_close(lg.cpu().numpy(), ps.cpu().numpy(), ref_l, ref_p, 0.0)
    if V <= 32000:
        check_markov(ids.cpu().numpy(), base, w1, w2, prev0, k)


def test_draft_round_without_probe_and_repair(dev):
    """Without probe_w the round writes no probe output; on a workspace
    marked by a wait that gave up, the round's ids are -2 (it repairs the
    workspace), its probe is still computed, and the next round is normal."""
    inp, t = _round_tensors("tiny", dev)
    say("[draft_round no probe / repair] tiny")
    R, B, V, k = inp["num_reqs"], inp["B"], inp["V"], inp["k"]
    ws = _ops().markov_workspace(R, k, V, dev)
    lg = torch.full((R * B,), 7.0, device=dev)
    out = _ops().draft_round(t["W"], t["H"], t["w1"], t["w2"], t["prev0"], B, k, workspace=ws, logit_out=lg)
    torch.cuda.synchronize()
    assert out["logit"] is None and torch.all(lg == 7.0)
    good = out["ids"].clone()
    ws[0] = 1  # the state word, as a wait that gave up leaves it
    out = _ops().draft_round(t["W"], t["H"], t["w1"], t["w2"], t["prev0"], B, k, probe_w=t["pw"], workspace=ws)
    torch.cuda.synchronize()
    assert torch.all(out["ids"] == -2)
    ref_lg, ref_ps = _ops().conf_probe(t["H"], t["pw"])
    torch.cuda.synchronize()
    assert torch.equal(out["logit"], ref_lg) and torch.equal(out["passed"], ref_ps)
    out = _ops().draft_round(t["W"], t["H"], t["w1"], t["w2"], t["prev0"], B, k, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out["ids"], good)


@pytest.mark.parametrize("name", ["tiny", "qwen3_8b_head"])
def test_draft_round_pinned_host_outputs(dev, name):
    """ids, probe logits and gates stored by the kernels straight into pinned
    host memory (slices of one buffer) equal the device-memory results."""
    inp, t = _round_tensors(name, dev)
    say(f"[draft_round pinned outputs] {name}")
    R, B, k = inp["num_reqs"], inp["B"], inp["k"]
    rows = R * B
    host = torch.zeros(R * k * 8 + rows * 8, dtype=torch.uint8, pin_memory=True)
    ids = host[: R * k * 8].view(torch.int64).view(R, k)
    lg = host[R * k * 8: R * k * 8 + rows * 4].view(torch.float32)
    ps = host[R * k * 8 + rows * 4:].view(torch.int32)
    kw = dict(probe_w=t["pw"], probe_bias=float(inp["probe_bias"]), probe_threshold=float(inp["probe_threshold"]))
    ref = _ops().draft_round(t["W"], t["H"], t["w1"], t["w2"], t["prev0"], B, k, **kw)
    _ops().draft_round(t["W"], t["H"], t["w1"], t["w2"], t["prev0"], B, k, ids_out=ids, logit_out=lg, pass_out=ps,
                       **kw)
    torch.cuda.synchronize()
    assert torch.equal(ids, ref["ids"].cpu())
    assert torch.equal(lg, ref["logit"].cpu()) and torch.equal(ps, ref["passed"].cpu())
    lg2 = torch.zeros(rows, dtype=torch.float32, pin_memory=True)
    _ops().conf_probe(t["H"], t["pw"], float(inp["probe_bias"]), float(inp["probe_threshold"]), logit_out=lg2,
                      want_pass=False)
    torch.cuda.synchronize()
    assert torch.equal(lg2, ref["logit"].cpu())


def test_draft_round_graph_replay(dev):
    """dspark_draft_round recorded in a HIP graph and replayed with eager work
    between replays: every replay equals the eager result."""
    inp, t = _round_tensors("reduced_vocab_batched", dev)
    say("[draft_round graph replay] reduced_vocab_batched")
    R, B, V, k = inp["num_reqs"], inp["B"], inp["V"], inp["k"]
    ops = _ops()
    bufs = dict(base_out=torch.empty(R, B, V, device=dev), ids_out=torch.empty(R, k, dtype=torch.int64, device=dev),
                logit_out=torch.empty(R * B, device=dev), pass_out=torch.empty(R * B, dtype=torch.int32, device=dev),
                workspace=ops.draft_round_workspace(R, B, k, V, t["W"].shape[1], dev))

    def run():
        return ops.draft_round(t["W"], t["H"], t["w1"], t["w2"], t["prev0"], B, k, probe_w=t["pw"], **bufs)
    eager = {n: x.clone() for n, x in run().items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(4):
        for n in ("base_out", "ids_out", "logit_out"):
            bufs[n].fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        for n, b in zip(("base_out", "ids_out", "logit_out", "pass_out"), ("base", "ids", "logit", "passed")):
            assert torch.equal(bufs[n], eager[b]), f"replay {rep}: {n} differs"
        _ = ops.lm_head(t["W"], t["H"])  # eager work between replays
        torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# The Markov loop and the round over Q8_0 weights
# ---------------------------------------------------------------------------

def _q8(q, d, dev):
    return _ops().q8_from_numpy(q, d, dev)


MARKOV_Q8_CASES = [
    # (R, B, k, V, r): one block; one workgroup with 3 blocks of a 4-block
    # k-loop; 16 requests over 3 workgroups; the batched lane; the
    # Qwen3-8B head at full size
    (1, 4, 4, 4096, 32), (3, 5, 5, 3000, 64), (2, 3, 3, 200, 96), (16, 2, 2, 600, 128),
    (8, 9, 9, 32000, 256), (1, 7, 7, 151936, 256),
]


@pytest.mark.parametrize("R,B,k,V,r", MARKOV_Q8_CASES)
def test_markov_q8_matches_oracle(dev, R, B, k, V, r):
    seed = 8100 + R * 7 + V + r
    say(f"[markov q8] R={R} B={B} k={k} V={V} r={r} seed={seed}")
    base, w1q, w1d, w2q, w2d, prev0 = synth.markov_q8_inputs(R, B, V, r, seed)
    ids = _ops().markov_sample_q8(_up(base, dev), *_q8(w1q, w1d, dev), *_q8(w2q, w2d, dev), _up(prev0, dev), k)
    ids2 = _ops().markov_sample_q8(_up(base, dev), *_q8(w1q, w1d, dev), *_q8(w2q, w2d, dev), _up(prev0, dev), k)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2), "rerun differs"
    check_markov(ids.cpu().numpy(), base, oracle.q8_0_to_f64(w1q, w1d), oracle.q8_0_to_f64(w2q, w2d), prev0, k)


@pytest.mark.parametrize("R,B", [(1, 15), (9, 6)])
def test_markov_q8_lane27b_size(dev, R, B):
    """The 27B lane's draft vocabulary (248320 x 256): in Q8_0 every
    markov_w2 tile of a workgroup fits on chip."""
    V, r, k = 248320, 256, B
    seed = 8200 + R
    say(f"[markov q8 lane27b] R={R} B={B} V={V} seed={seed}")
    base, w1q, w1d, w2q, w2d, prev0 = synth.markov_q8_inputs(R, B, V, r, seed)
    ids = _ops().markov_sample_q8(_up(base, dev), *_q8(w1q, w1d, dev), *_q8(w2q, w2d, dev), _up(prev0, dev), k)
    torch.cuda.synchronize()
    check_markov(ids.cpu().numpy(), base, oracle.q8_0_to_f64(w1q, w1d), oracle.q8_0_to_f64(w2q, w2d), prev0, k)


def test_markov_q8_constructed_ties(dev):
    """Exact ties in Q8_0: tie rows' pair (a, b) share the top base value and
    markov_w2 row b is a copy of row a (quants and scales): index a wins."""
    R, B, V, r = 2, 6, 5000, 64
    say(f"[markov q8 ties] R={R} V={V} r={r}")
    base, w1q, w1d, w2q, w2d, prev0 = synth.markov_q8_inputs(R, B, V, r, 93)
    g = np.random.default_rng(5)
    ties = []
    for q in range(R):
        for i in range(B):
            a, b = sorted(int(x) for x in g.choice(V, 2, replace=False))
            base[q, i, a] = base[q, i, b] = synth.TIE_VALUE
            w2q[b], w2d[b] = w2q[a], w2d[a]
            ties.append((q, i, a))
    ids = _ops().markov_sample_q8(_up(base, dev), *_q8(w1q, w1d, dev), *_q8(w2q, w2d, dev), _up(prev0, dev), B)
    torch.cuda.synchronize()
    ids = ids.cpu().numpy()
    for q, i, a in ties:
        assert ids[q, i] == a, f"request {q} step {i}: {ids[q, i]} instead of {a}"


def test_markov_q8_and_bf16_share_a_workspace(dev):
    """bf16 and Q8_0 calls alternate on one workspace (the key slots and the
    call counter are shared): each equals its result on a fresh workspace."""
    R, B, k, V, r = 3, 5, 5, 3000, 64
    say("[markov q8/bf16 shared workspace]")
    base, w1q, w1d, w2q, w2d, prev0 = synth.markov_q8_inputs(R, B, V, r, 97)
    _, w1, w2, _, _ = synth.markov_inputs(R, B, V, r, 97)
    bq = (_up(base, dev), *_q8(w1q, w1d, dev), *_q8(w2q, w2d, dev), _up(prev0, dev), k)
    bb = (_up(base, dev), _bf(w1, dev), _bf(w2, dev), _up(prev0, dev), k)
    ref_q = _ops().markov_sample_q8(*bq).clone()
    ref_b = _ops().markov_sample(*bb).clone()
    ws = _ops().markov_workspace(R, k, V, dev)
    for _ in range(3):
        a = _ops().markov_sample_q8(*bq, workspace=ws)
        b = _ops().markov_sample(*bb, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(a, ref_q) and torch.equal(b, ref_b)


def test_markov_q8_fused_probe(dev):
    R, B, k, V, r = 1, 7, 7, 151936, 256
    say("[markov q8 + probe] qwen3_8b_head shape, probe 7 x 4096")
    base, w1q, w1d, w2q, w2d, prev0 = synth.markov_q8_inputs(R, B, V, r, 99)
    x, pw = synth.probe_inputs(7, 4096, 99)
    probe = dict(x=_up(x, dev), w=_bf(pw, dev), bias=0.25, threshold=0.0)
    args = (_up(base, dev), *_q8(w1q, w1d, dev), *_q8(w2q, w2d, dev), _up(prev0, dev), k)
    ids = _ops().markov_sample_q8(*args, probe=probe)
    ids2 = _ops().markov_sample_q8(*args)
    lg, ps = _ops().conf_probe(probe["x"], probe["w"], 0.25, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2)
    assert torch.equal(probe["logit_out"], lg) and torch.equal(probe["pass_out"], ps)


def _round_q8_tensors(inp, dev):
    return dict(Wq=_q8(inp["Wq_lm"], inp["Wd_lm"], dev), w1=_q8(inp["w1q"], inp["w1d"], dev),
                w2=_q8(inp["w2q"], inp["w2d"], dev), H=_up(inp["H"], dev), prev0=_up(inp["prev0"], dev),
                pw=_bf(inp["probe_w"], dev))


Q8_LDD_CASES = [
    # (M, N, K, ldd): the 27B-lane shape with three and two K phases, rows
    # padded to 128-byte lines and an odd stride (single-scale loads); a
    # dense-aligned K; an odd block count; the short kernel.
    (15, 70001, 5120, 192), (7, 66003, 5120, 161), (7, 9000, 4096, 192), (9, 5003, 160, 64), (3, 300, 7424, 256),
    # more than 16 rows: two launches over the same padded scales
    (20, 5003, 5120, 192),
]


@pytest.mark.parametrize("M,N,K,ldd", Q8_LDD_CASES)
def test_lm_head_q8_padded_scales_equal_dense(dev, M, N, K, ldd):
    """Scale rows ldd apart, the padding filled with NaN: the logits of the
    dense layout bit for bit (no padding is read as a scale)."""
    seed = 7150 + M + N + K + ldd
    say(f"[lm_head q8 ldd] M={M} N={N} K={K} ldd={ldd} seed={seed}")
    Wq, Wd, X = synth.gemv_q8_inputs(M, N, K, seed)
    q, d = _ops().q8_from_numpy(Wq, Wd, dev)
    dp = torch.full((N, ldd), float("nan"), dtype=torch.float16, device=dev)
    dp[:, :K // 32] = d
    Xd = _up(X, dev)
    y0 = _ops().lm_head_q8(q, d, Xd)
    y1 = _ops().lm_head_q8(q, dp, Xd)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1), "padded scale rows changed the logits"
    if K % 32 == 0 and (K // 32) % 64 != 0:
        y2 = _ops().lm_head_q8(q, _ops().q8_pad_scales(d), Xd)
        torch.cuda.synchronize()
        assert torch.equal(y0, y2)


def test_draft_round_q8_padded_scales_equal_dense(dev):
    """dspark_draft_round_q8_ld with the lm_head's scale rows padded to whole
    lines: base logits, ids and probe equal to the dense round's bit for bit,
    and the ids right against the oracle."""
    R, B, k, V, d, r = 2, 4, 3, 3000, 5120, 64
    seed = 8310
    say(f"[draft_round q8 ldd] R={R} B={B} k={k} V={V} d={d} r={r}")
    Wq, Wd, H = synth.gemv_q8_inputs(R * B, V, d, seed)
    _, w1q, w1d, w2q, w2d, prev0 = synth.markov_q8_inputs(R, 1, V, r, seed)
    _, pw = synth.probe_inputs(1, d, seed)
    inp = dict(Wq_lm=Wq, Wd_lm=Wd, H=H, w1q=w1q, w1d=w1d, w2q=w2q, w2d=w2d, prev0=prev0, probe_w=pw)
    t = _round_q8_tensors(inp, dev)
    q, dd = t["Wq"]
    dp = _ops().q8_pad_scales(dd)
    assert dp.shape[1] == 192
    a = _ops().draft_round_q8(q, dd, t["H"], *t["w1"], *t["w2"], t["prev0"], B, k, probe_w=t["pw"])
    b = _ops().draft_round_q8(q, dp, t["H"], *t["w1"], *t["w2"], t["prev0"], B, k, probe_w=t["pw"])
    torch.cuda.synchronize()
    for key in ("base", "ids", "logit", "passed"):
        assert torch.equal(a[key], b[key]), key
    ref = oracle.draft_round_q8(Wq, Wd, H, w1q, w1d, w2q, w2d, prev0, R, B, k, pw, 0.0, 0.0)
    logits_close(b["base"].view(R * B, V).cpu().numpy(), ref["base"], "draft_round_q8_ld logits")
    check_markov(b["ids"].cpu().numpy(), ref["base32"], oracle.q8_0_to_f64(w1q, w1d),
                 oracle.q8_0_to_f64(w2q, w2d), prev0, k)


def test_draft_round_q8_small(dev):
    """A small Q8_0 round against the oracle and against the separate calls."""
    R, B, k, V, d, r = 2, 4, 3, 3000, 256, 64
    seed = 8300
    say(f"[draft_round q8 small] R={R} B={B} k={k} V={V} d={d} r={r}")
    Wq, Wd, H = synth.gemv_q8_inputs(R * B, V, d, seed)
    _, w1q, w1d, w2q, w2d, prev0 = synth.markov_q8_inputs(R, 1, V, r, seed)
    _, pw = synth.probe_inputs(1, d, seed)
    inp = dict(Wq_lm=Wq, Wd_lm=Wd, H=H, w1q=w1q, w1d=w1d, w2q=w2q, w2d=w2d, prev0=prev0, probe_w=pw)
    t = _round_q8_tensors(inp, dev)
    out = _ops().draft_round_q8(*t["Wq"], t["H"], *t["w1"], *t["w2"], t["prev0"], B, k, probe_w=t["pw"],
                                probe_threshold=0.01)
    base = _ops().lm_head_q8(*t["Wq"], t["H"])
    ids = _ops().markov_sample_q8(base.view(R, B, V), *t["w1"], *t["w2"], t["prev0"], k)
    lg, ps = _ops().conf_probe(t["H"], t["pw"], 0.0, 0.01)
    torch.cuda.synchronize()
    assert torch.equal(out["base"].view(R * B, V), base) and torch.equal(out["ids"], ids)
    assert torch.equal(out["logit"], lg) and torch.equal(out["passed"], ps)
    ref = oracle.draft_round_q8(Wq, Wd, H, w1q, w1d, w2q, w2d, prev0, R, B, k, pw, 0.0, 0.01)
    logits_close(base.cpu().numpy(), ref["base"], "draft_round_q8 logits")
    check_markov(out["ids"].cpu().numpy(), ref["base32"], oracle.q8_0_to_f64(w1q, w1d),
                 oracle.q8_0_to_f64(w2q, w2d), prev0, k)
    probe_close(lg.cpu().numpy(), ps.cpu().numpy(), ref["logit"], ref["passed"], 0.01)


def test_draft_round_q8_full_size(dev):
    """The Qwen3-8B head in Q8_0 at full size: the fused round equals the
    separate calls bit for bit; the loop is checked against the oracle on the
    GPU's own base logits, the base logits on sampled rows."""
    inp = synth.round_inputs("qwen3_8b_head_q8")
    R, B, k, V = inp["num_reqs"], inp["B"], inp["k"], inp["V"]
    say(f"[draft_round q8 full] qwen3_8b_head_q8 seed={inp['seed']}")
    t = _round_q8_tensors(inp, dev)
    out = _ops().draft_round_q8(*t["Wq"], t["H"], *t["w1"], *t["w2"], t["prev0"], B, k, probe_w=t["pw"])
    base = _ops().lm_head_q8(*t["Wq"], t["H"])
    ids = _ops().markov_sample_q8(base.view(R, B, V), *t["w1"], *t["w2"], t["prev0"], k)
    torch.cuda.synchronize()
    assert torch.equal(out["base"].view(R * B, V), base) and torch.equal(out["ids"], ids)
    b = base.cpu().numpy()
    pick = np.unique(np.concatenate([np.arange(16), np.arange(V - 16, V),
                                     np.random.default_rng(2).choice(V, 1500, replace=False)]))
    logits_close(b[:, pick], oracle.gemv_q8_rows(inp["Wq_lm"], inp["Wd_lm"], inp["H"], pick), "q8 round logits")
    check_markov(out["ids"].cpu().numpy(), b.reshape(R, B, V), oracle.q8_0_to_f64(inp["w1q"], inp["w1d"]),
                 oracle.q8_0_to_f64(inp["w2q"], inp["w2d"]), inp["prev0"], k)
    ref_l, ref_p = oracle.conf_probe(inp["H"], inp["probe_w"], 0.0, 0.0)
    probe_close(out["logit"].cpu().numpy(), out["passed"].cpu().numpy(), ref_l, ref_p, 0.0)


# ---------------------------------------------------------------------------
# The rest of the draft block: RMSNorm, SiLU gate, residual GEMV, attention
# ---------------------------------------------------------------------------

def _close(a, b, what, rtol=1e-5, atol=1e-5):
    a = np.asarray(a, np.float64)
    err = np.abs(a - b)
    ok = err <= atol + rtol * np.abs(b)
    assert ok.all(), f"{what}: max err {err.max():.3e} at {np.unravel_index(np.argmax(err), err.shape)}"


@pytest.mark.parametrize("M,D", [(7, 4096), (3, 7424), (1, 5), (16, 4100), (72, 5120)])
def test_rmsnorm_matches_oracle(dev, M, D):
    say(f"[rmsnorm] M={M} D={D}")
    g = np.random.default_rng(M + D)
    x = (g.standard_normal((M, D)) * 2).astype(np.float32)
    gamma = synth.bf16_bits_rne((1 + 0.1 * g.standard_normal(D)).astype(np.float32))
    y = _ops().rmsnorm(_up(x, dev), _bf(gamma, dev), 1e-6)
    torch.cuda.synchronize()
    _close(y.cpu().numpy(), oracle.rmsnorm(x, gamma, 1e-6), f"rmsnorm M={M} D={D}")


@pytest.mark.parametrize("M,F", [(7, 12288), (1, 3), (9, 1000)])
def test_silu_gate_matches_oracle(dev, M, F):
    say(f"[silu gate] M={M} F={F}")
    g = np.random.default_rng(M * F)
    gu = (g.standard_normal((M, 2 * F)) * 4).astype(np.float32)
    a = _ops().silu_gate(_up(gu, dev))
    torch.cuda.synchronize()
    _close(a.cpu().numpy(), oracle.silu_gate(gu, F), f"silu gate M={M} F={F}", rtol=2e-6, atol=1e-6)


@pytest.mark.parametrize("M,N,K", [(7, 4096, 4096), (7, 4096, 12288), (3, 1000, 264), (20, 515, 256), (90, 600, 512)])
def test_proj_smallm_add(dev, M, N, K):
    """Y = residual + X W^T, also in place (residual = Y)."""
    seed = 7300 + M + N + K
    say(f"[proj add] M={M} N={N} K={K} seed={seed}")
    W, X = synth.gemv_inputs(M, N, K, seed)
    res = synth.normal_f32(seed, synth.S_BASE, (M, N))
    Wd, Xd = _bf(W, dev), _up(X, dev)
    y = _ops().proj_smallm_add(Wd, Xd, _up(res, dev))
    r2 = _up(res, dev)
    _ops().proj_smallm_add(Wd, Xd, r2, out=r2)
    plain = _ops().proj_smallm(Wd, Xd)
    torch.cuda.synchronize()
    assert torch.equal(y, r2), "in-place result differs"
    assert torch.equal(y, _up(res, dev) + plain), "residual epilogue is not y + residual in fp32"
    logits_close(y.cpu().numpy(), oracle.gemv(W, X) + res.astype(np.float64), f"proj add M={M} N={N} K={K}")


NORM_CASES = [
    # (M, N, K): packed rows with one tile per workgroup and several phases,
    # several tiles; hi/lo rows with a partial last phase, several tiles;
    # ragged N with one short phase; the smallest shape; 8 packed rows
    (7, 4096, 4096), (7, 12288, 4096), (15, 4096, 4128), (16, 24576, 4096), (3, 1000, 264), (1, 2, 8),
    (8, 777, 2080),
]


@pytest.mark.parametrize("M,N,K", NORM_CASES)
def test_proj_smallm_norm_matches_oracle(dev, M, N, K):
    """rmsnorm fused into the projection: Y = rmsnorm(X; gamma, eps) W^T
    against the oracle's rmsnorm followed by its gemv."""
    seed = 7350 + M + N + K
    say(f"[proj norm] M={M} N={N} K={K} seed={seed}")
    W, X = synth.gemv_inputs(M, N, K, seed)
    X = X * np.float32(3.0) + np.float32(0.5)  # rows with a mean: the norm must not centre them
    gamma = synth.bf16_bits_rne(1.0 + synth.normal_f32(seed, synth.S_BASE, (K,), 0.2))
    eps = 1e-6
    assert _ops().proj_smallm_norm_fits(N, K, M)
    y = _ops().proj_smallm_norm(_bf(W, dev), _up(X, dev), _bf(gamma, dev), eps)
    torch.cuda.synchronize()
    logits_close(y.cpu().numpy(), oracle.gemv(W, oracle.rmsnorm(X, gamma, eps)), f"proj norm M={M} N={N} K={K}")


def test_proj_smallm_norm_row_properties(dev):
    """A row's output depends on that row alone (same bits for M = 7 and for
    the row by itself), and at eps = 0 scaling X by 8 changes no bit (every
    step of the factor is exact under a power-of-two scale)."""
    M, N, K = 7, 12288, 4096
    say(f"[proj norm rows] M={M} N={N} K={K}")
    W, X = synth.gemv_inputs(M, N, K, 7399)
    gamma = _bf(synth.bf16_bits_rne(1.0 + synth.normal_f32(7399, synth.S_BASE, (K,), 0.2)), dev)
    Wd, Xd = _bf(W, dev), _up(X, dev)
    ops = _ops()
    y = ops.proj_smallm_norm(Wd, Xd, gamma, 0.0)
    y3 = ops.proj_smallm_norm(Wd, Xd[3:4].contiguous(), gamma, 0.0)
    y8 = ops.proj_smallm_norm(Wd, Xd * 8.0, gamma, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(y[3:4], y3), "row 3 depends on the other rows"
    assert torch.equal(y, y8), "scaling X by 8 changed the result"
    assert not ops.proj_smallm_norm_fits(N, K, 17)


ATTN_CASES = [
    # (R, B, H, Dh, Lmax, ctx_len, causal)
    (1, 7, 32, 128, 512, [512], False), (1, 7, 32, 128, 512, [300], True), (2, 3, 4, 64, 128, [0, 100], False),
    (2, 16, 2, 256, 100, [100, 37], True), (1, 1, 1, 8, 0, [0], False), (3, 5, 3, 32, 40, [40, 0, 17], True),
    # keys come in chunks of 64: Lk = 64 and 65 exactly, two full chunks, a long context, Dh = 24 (three 8-dim groups)
    (2, 7, 2, 128, 58, [57, 58], True), (1, 7, 3, 64, 121, [121], False), (2, 7, 4, 128, 4000, [4000, 1234], True),
    (2, 4, 3, 24, 70, [70, 1], True),
]


@pytest.mark.parametrize("R,B,H,Dh,Lmax,lens,causal", ATTN_CASES)
def test_attention_ragged_matches_oracle(dev, R, B, H, Dh, Lmax, lens, causal):
    seed = 7400 + R * B * H + Dh + Lmax
    say(f"[attention] R={R} B={B} H={H} Dh={Dh} Lmax={Lmax} lens={lens} causal={causal}")
    g = np.random.default_rng(seed)
    HD = H * Dh
    qkv = g.standard_normal((R * B, 3 * HD)).astype(np.float32)
    kc = synth.bf16_bits_rne(g.standard_normal((R, max(Lmax, 1), HD)).astype(np.float32))[:, :Lmax]
    vc = synth.bf16_bits_rne(g.standard_normal((R, max(Lmax, 1), HD)).astype(np.float32))[:, :Lmax]
    kcd = _bf(np.ascontiguousarray(kc), dev).view(R, Lmax, HD) if Lmax else torch.zeros((R, 0, HD), dtype=torch.bfloat16, device=dev)
    vcd = _bf(np.ascontiguousarray(vc), dev).view(R, Lmax, HD) if Lmax else torch.zeros((R, 0, HD), dtype=torch.bfloat16, device=dev)
    out = _ops().attention_ragged(_up(qkv, dev), R, B, H, Dh, kcd, vcd,
                                  torch.tensor(lens, dtype=torch.int32, device=dev), causal)
    out2 = _ops().attention_ragged(_up(qkv, dev), R, B, H, Dh, kcd, vcd,
                                   torch.tensor(lens, dtype=torch.int32, device=dev), causal)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "rerun differs"
    kc_ = kc if Lmax else np.zeros((R, 0, HD), np.uint16)
    vc_ = vc if Lmax else np.zeros((R, 0, HD), np.uint16)
    ref = oracle.attention_ragged(qkv[:, :HD], qkv[:, HD:2 * HD], qkv[:, 2 * HD:], R, B, H, Dh, kc_, vc_, lens, causal)
    _close(out.cpu().numpy(), ref, "attention", rtol=1e-4, atol=1e-5)


def test_attention_workspace_needs_no_clearing(dev):
    """Every partial result is written before it is read: a workspace full of
    NaN bit patterns, shared by a large and then a smaller call, gives the
    results of fresh workspaces bit for bit."""
    say("[attention] dirty shared workspace")
    ops = _ops()
    g = np.random.default_rng(7411)
    ws = torch.full((ops.attention_workspace_bytes(2, 7, 4, 128, 700),), 0xFF, dtype=torch.uint8, device=dev)
    for (R, B, H, Dh, Lmax, lens, causal) in [(2, 7, 4, 128, 700, [700, 3], True), (1, 5, 2, 64, 90, [80], False)]:
        HD = H * Dh
        qkv = _up(g.standard_normal((R * B, 3 * HD)).astype(np.float32), dev)
        kc = _bf(synth.bf16_bits_rne(g.standard_normal((R, Lmax, HD)).astype(np.float32)), dev).view(R, Lmax, HD)
        vc = _bf(synth.bf16_bits_rne(g.standard_normal((R, Lmax, HD)).astype(np.float32)), dev).view(R, Lmax, HD)
        ln = torch.tensor(lens, dtype=torch.int32, device=dev)
        a = ops.attention_ragged(qkv, R, B, H, Dh, kc, vc, ln, causal, workspace=ws)
        b = ops.attention_ragged(qkv, R, B, H, Dh, kc, vc, ln, causal)
        torch.cuda.synchronize()
        assert torch.isfinite(a).all() and torch.equal(a, b), f"shared workspace changed the result R={R} Lmax={Lmax}"


@pytest.mark.parametrize("R,B,H,Dh,F,Lmax,lens", [(1, 7, 2, 128, 512, 64, [64]), (1, 7, 32, 128, 12288, 512, [512]),
                                                  (2, 4, 4, 64, 1024, 96, [96, 20]),
                                                  # M = 21 and M = 84: the small-GEMM path and its split launches
                                                  (3, 7, 4, 64, 512, 80, [80, 33, 0]),
                                                  (12, 7, 2, 64, 256, 40, [40, 1, 7, 13, 0, 40, 39, 2, 25, 31, 8, 16])])
def test_draft_block_forward_matches_oracle(dev, R, B, H, Dh, F, Lmax, lens):
    """One whole draft block (rmsnorm, qkv, attention, o + residual, rmsnorm,
    gate/up, SiLU gate, down + residual) through the C ABI, against the fp64
    composition."""
    seed = 7500 + H * Dh + F
    say(f"[draft block] R={R} B={B} H={H} Dh={Dh} F={F} Lmax={Lmax} lens={lens} seed={seed}")
    inp = synth.block_inputs(R, B, H, Dh, F, Lmax, lens, seed)
    w = {k: _bf(v, dev) for k, v in inp["layers"][0].items()}
    kc = _bf(inp["k_ctx"], dev).view(R, Lmax, H * Dh)
    vc = _bf(inp["v_ctx"], dev).view(R, Lmax, H * Dh)
    y = _ops().draft_block_forward(_up(inp["h"], dev), w, R, B, H, Dh, kc, vc,
                                   torch.tensor(lens, dtype=torch.int32, device=dev), float(inp["eps"]))
    torch.cuda.synchronize()
    ref = oracle.draft_block_forward(inp["h"], inp["layers"][0], R, B, H, Dh, inp["k_ctx"], inp["v_ctx"],
                                     inp["ctx_len"], float(inp["eps"]))
    logits_close(y.cpu().numpy(), ref, f"draft block d={H * Dh}")


@pytest.mark.parametrize("R,B,H,Dh,F,Lmax,lens,causal", [(1, 7, 32, 128, 12288, 512, [512], False),
                                                         (2, 4, 4, 64, 1024, 96, [96, 20], True)])
def test_draft_block_single_call_equals_calls(dev, R, B, H, Dh, F, Lmax, lens, causal):
    """dspark_draft_block gives the bits of its eight entry points called one
    by one, also when h_out is h_in."""
    seed = 7600 + H * Dh + F
    say(f"[draft block one call] R={R} B={B} H={H} Dh={Dh} F={F} Lmax={Lmax} lens={lens} causal={causal} seed={seed}")
    ops = _ops()
    inp = synth.block_inputs(R, B, H, Dh, F, Lmax, lens, seed)
    w = {k: _bf(v, dev) for k, v in inp["layers"][0].items()}
    kc = _bf(inp["k_ctx"], dev).view(R, Lmax, H * Dh)
    vc = _bf(inp["v_ctx"], dev).view(R, Lmax, H * Dh)
    ln = torch.tensor(lens, dtype=torch.int32, device=dev)
    h = _up(inp["h"], dev)
    eps = float(inp["eps"])
    one = ops.draft_block_forward(h, w, R, B, H, Dh, kc, vc, ln, eps, causal)
    calls = ops.draft_block_forward_calls(h, w, R, B, H, Dh, kc, vc, ln, eps, causal)
    inplace = h.clone()
    ops.draft_block_forward(inplace, w, R, B, H, Dh, kc, vc, ln, eps, causal, out=inplace)
    torch.cuda.synchronize()
    assert torch.equal(one, calls)
    assert torch.equal(one, inplace)


@pytest.mark.parametrize("R,B,H,Dh,F,Lmax,lens,layers,n_fc,V,r", [(2, 3, 2, 64, 256, 40, [40, 9], 3, 2, 1000, 16),
                                                                 (1, 7, 32, 128, 12288, 512, [512], 2, 1, 4096, 256)])
def test_draft_forward_round_matches_oracle(dev, R, B, H, Dh, F, Lmax, lens, layers, n_fc, V, r):
    """A whole synthetic draft round: fc, the blocks (each with its own
    context cache), the final norm, then dspark_draft_round on the result;
    hidden states, logits, ids and probe against the fp64 oracle."""
    seed = 7700 + layers * 10 + n_fc
    d = H * Dh
    k = B
    say(f"[draft forward + round] R={R} B={B} d={d} F={F} layers={layers} n_fc={n_fc} V={V} r={r} seed={seed}")
    ops = _ops()
    inp = synth.draft_forward_inputs(R, B, H, Dh, F, Lmax, lens, layers, n_fc, seed)
    W_lm, _ = synth.gemv_inputs(1, V, d, seed)
    _, w1, w2, prev0, _ = synth.markov_inputs(R, 1, V, r, seed)
    _, pw = synth.probe_inputs(1, d, seed)
    eps = float(inp["eps"])
    hid = ops.draft_forward(_up(inp["x_in"], dev), _bf(inp["fc"], dev),
                            [{kk: _bf(v, dev) for kk, v in w.items()} for w in inp["layers"]],
                            [_bf(c, dev).view(R, Lmax, d) for c in inp["k_ctx"]],
                            [_bf(c, dev).view(R, Lmax, d) for c in inp["v_ctx"]], R, B, H, Dh,
                            torch.tensor(lens, dtype=torch.int32, device=dev), _bf(inp["norm"], dev), eps)
    out = ops.draft_round(_bf(W_lm, dev), hid, _bf(w1, dev), _bf(w2, dev), _up(prev0, dev), B, k,
                          probe_w=_bf(pw, dev), probe_bias=0.0, probe_threshold=0.0)
    torch.cuda.synchronize()
    ref_h = oracle.draft_forward(inp["x_in"], inp["fc"], inp["layers"], inp["k_ctx"], inp["v_ctx"], inp["ctx_len"],
                                 inp["norm"], eps, R, B, H, Dh)
    logits_close(hid.cpu().numpy(), ref_h, f"draft forward hidden ({layers} blocks)")
    ref = oracle.draft_round(W_lm, ref_h.astype(np.float32), w1, w2, prev0, R, B, k, pw, 0.0, 0.0)
    logits_close(out["base"].view(R * B, -1).cpu().numpy(), ref["base"], "draft forward round logits")
    check_markov(out["ids"].cpu().numpy(), ref["base32"], w1, w2, prev0, k)
    probe_close(out["logit"].cpu().numpy(), out["passed"].cpu().numpy(), ref["logit"], ref["passed"], 0.0)


def test_round_graph_replay(dev):
    """The whole round recorded once in a HIP graph and replayed, with eager
    work between replays: every replay equals the eager result."""
    inp, t = _round_tensors("tiny", dev)
    say("[round graph replay] tiny")
    R, B, V, k = inp["num_reqs"], inp["B"], inp["V"], inp["k"]
    ops = _ops()
    logits = torch.empty(R * B, V, device=dev)
    ids = torch.empty(R, k, dtype=torch.int64, device=dev)
    ws = ops.markov_workspace(R, k, V, dev)
    lg = torch.empty(R * B, device=dev)
    ps = torch.empty(R * B, dtype=torch.int32, device=dev)
    eager = [x.clone() for x in _run_round(inp, t, logits, ids, ws, lg, ps)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _run_round(inp, t, logits, ids, ws, lg, ps)  # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _run_round(inp, t, logits, ids, ws, lg, ps)
    for rep in range(4):
        logits.fill_(7.0)
        ids.fill_(-7)
        lg.fill_(7.0)
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((logits, ids, lg, ps), eager):
            assert torch.equal(a, b), f"replay {rep} differs"
        _ = ops.lm_head(t["W"], t["H"])  # eager work between replays
        torch.cuda.synchronize()


def test_draft_forward_graph_replay(dev):
    """fc, two blocks, the final norm and the round recorded once in a HIP
    graph and replayed, with eager work between replays: every replay equals
    the eager result (the attention and the block record no memset)."""
    R, B, H, Dh, F, Lmax, lens, V, r = 2, 3, 2, 64, 256, 40, [40, 9], 1000, 16
    seed = 7801
    say(f"[draft forward graph replay] R={R} B={B} d={H * Dh} seed={seed}")
    ops = _ops()
    inp = synth.draft_forward_inputs(R, B, H, Dh, F, Lmax, lens, 2, 1, seed)
    W_lm, _ = synth.gemv_inputs(1, V, H * Dh, seed)
    _, w1, w2, prev0, _ = synth.markov_inputs(R, 1, V, r, seed)
    _, pw = synth.probe_inputs(1, H * Dh, seed)
    x_in, fc, norm = _up(inp["x_in"], dev), _bf(inp["fc"], dev), _bf(inp["norm"], dev)
    layers = [{kk: _bf(v, dev) for kk, v in w.items()} for w in inp["layers"]]
    kcs = [_bf(c, dev).view(R, Lmax, H * Dh) for c in inp["k_ctx"]]
    vcs = [_bf(c, dev).view(R, Lmax, H * Dh) for c in inp["v_ctx"]]
    ln = torch.tensor(lens, dtype=torch.int32, device=dev)
    Wl, w1d, w2d, p0, pwd = _bf(W_lm, dev), _bf(w1, dev), _bf(w2, dev), _up(prev0, dev), _bf(pw, dev)
    scratch = {}
    hid = torch.empty(R * B, H * Dh, device=dev)
    base = torch.empty(R, B, V, device=dev)
    ids = torch.empty(R, B, dtype=torch.int64, device=dev)
    lg = torch.empty(R * B, device=dev)
    ps = torch.empty(R * B, dtype=torch.int32, device=dev)
    mws = ops.draft_round_workspace(R, B, B, V, H * Dh, dev)

    def run():
        ops.draft_forward(x_in, fc, layers, kcs, vcs, R, B, H, Dh, ln, norm, float(inp["eps"]), scratch=scratch,
                          out=hid)
        ops.draft_round(Wl, hid, w1d, w2d, p0, B, B, probe_w=pwd, base_out=base, ids_out=ids, logit_out=lg,
                        pass_out=ps, workspace=mws)
    run()
    torch.cuda.synchronize()
    eager = [x.clone() for x in (hid, base, ids, lg, ps)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()  # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(4):
        for x in (hid, base, lg):
            x.fill_(7.0)
        ids.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((hid, base, ids, lg, ps), eager):
            assert torch.equal(a, b), f"replay {rep} differs"
        _ = ops.proj_smallm(fc, x_in)  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("R,B,H,Dh,F,Lmax,lens,causal", [(1, 7, 2, 64, 256, 0, [0], False),
                                                         (2, 5, 2, 64, 256, 0, [0, 0], True),
                                                         (2, 7, 4, 64, 512, 70, [70, 3], True)])
def test_draft_block_edges_match_oracle(dev, R, B, H, Dh, F, Lmax, lens, causal):
    """Whole blocks with no context at all (the block attends to itself only)
    and with causal block attention, against the fp64 composition."""
    seed = 7900 + Lmax + 10 * R + (1 if causal else 0)
    say(f"[draft block edges] R={R} B={B} H={H} Dh={Dh} F={F} Lmax={Lmax} lens={lens} causal={causal} seed={seed}")
    inp = synth.block_inputs(R, B, H, Dh, F, Lmax, lens, seed)
    w = {k: _bf(v, dev) for k, v in inp["layers"][0].items()}
    d = H * Dh
    if Lmax:
        kc = _bf(inp["k_ctx"], dev).view(R, Lmax, d)
        vc = _bf(inp["v_ctx"], dev).view(R, Lmax, d)
    else:
        kc = torch.zeros((R, 0, d), dtype=torch.bfloat16, device=dev)
        vc = torch.zeros((R, 0, d), dtype=torch.bfloat16, device=dev)
    y = _ops().draft_block_forward(_up(inp["h"], dev), w, R, B, H, Dh, kc, vc,
                                   torch.tensor(lens, dtype=torch.int32, device=dev), float(inp["eps"]), causal)
    torch.cuda.synchronize()
    kc_ = inp["k_ctx"] if Lmax else np.zeros((R, 0, d), np.uint16)
    vc_ = inp["v_ctx"] if Lmax else np.zeros((R, 0, d), np.uint16)
    ref = oracle.draft_block_forward(inp["h"], inp["layers"][0], R, B, H, Dh, kc_, vc_, inp["ctx_len"],
                                     float(inp["eps"]), causal)
    logits_close(y.cpu().numpy(), ref, f"draft block edge Lmax={Lmax} causal={causal}")
