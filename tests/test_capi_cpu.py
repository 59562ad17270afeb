"""The C ABI without a GPU: the library loads, exports every symbol the
header declares, and rejects invalid arguments before any HIP call."""
import ctypes
import os
import re

import pytest

from gemv_markov_argmax_amd import build as B

HEADER = os.path.join(B.ROOT, "include", "dspark.h")
OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_WORKSPACE, ERR_HIP = range(6)


@pytest.fixture(scope="module")
def L():
    if B.needs_build():
        B.build()
    from gemv_markov_argmax_amd import ops
    return ops.lib()


def declared():
    code = open(HEADER).read()
    code = re.sub(r"/\*.*?\*/", "", code, flags=re.S)
    code = re.sub(r"//[^\n]*", "", code)
    return sorted(set(re.findall(r"\b(dspark_[a-z0-9_]+)\s*\(", code)))


def test_header_declares_the_entry_points():
    names = declared()
    for n in ["dspark_proj_smallm", "dspark_lm_head", "dspark_lm_head_sched", "dspark_lm_head_split",
              "dspark_lm_head_split_workspace_bytes", "dspark_draft_round_workspace_bytes",
              "dspark_markov_sample", "dspark_conf_probe",
              "dspark_markov_sample_probe", "dspark_draft_round", "dspark_proj_smallm_q8", "dspark_lm_head_q8",
              "dspark_markov_sample_q8", "dspark_draft_round_q8", "dspark_lm_head_q8_ld",
              "dspark_draft_round_q8_ld", "dspark_rmsnorm", "dspark_silu_gate",
              "dspark_proj_smallm_add", "dspark_proj_smallm_norm", "dspark_proj_smallm_norm_fits",
              "dspark_attention_ragged",
              "dspark_markov_workspace_bytes",
              "dspark_status_string"]:
        assert n in names


def test_library_exports_every_declared_symbol(L):
    missing = [n for n in declared() if not hasattr(L, n)]
    assert not missing, missing


def test_status_strings(L):
    from gemv_markov_argmax_amd import ops
    for code in range(6):
        assert ops.status_string(code).startswith("DSPARK_")
    assert "UNKNOWN" in ops.status_string(99)


A = 0x10000      # 16-byte-aligned fake device addresses: never dereferenced,
A2 = 0x20000     # every call below fails validation before any HIP call
MIS = 0x10002


def test_lm_head_sched_errors(L):
    f = L.dspark_lm_head_sched
    assert f(None, 16, 64, A, 7, A2, A, None) == ERR_NULL
    assert f(A, 16, 64, A, 7, A2, None, None) == ERR_NULL      # no counter
    assert f(A, 16, 12, A, 7, A2, A, None) == ERR_SHAPE        # d % 8 != 0
    assert f(A, 16, 64, A, 7, A2, A + 2, None) == ERR_ALIGN    # misaligned counter
    assert f(A, 16, 64, MIS, 7, A2, A, None) == ERR_ALIGN


def test_lm_head_split_workspace_bytes(L):
    f = L.dspark_lm_head_split_workspace_bytes
    assert f(0, 64, 72) == 0 and f(100, 0, 72) == 0 and f(100, 64, 0) == 0
    assert f(32000, 5120, 16) == 0                      # 16 rows or fewer: no split
    assert f(32000, (1 << 21) + 8, 72) == 0             # a 256-row K half past the 32-bit buffer range
    n = f(32000, 5120, 72)
    # ticket words for 128 blocks of 256 rows (125 padded to a multiple of 8),
    # then two partials of 80 rows x 256 columns per block
    assert n == 512 + 2 * 128 * 80 * 256 * 4
    assert f(32000, 5120, 17) == f(32000, 5120, 80) == f(32000, 5120, 500) == n  # parts of <= 80 rows reuse it
    assert f(1, 8, 17) == 256 + 2 * 8 * 80 * 256 * 4


def test_lm_head_split_errors(L):
    f = L.dspark_lm_head_split
    n = L.dspark_lm_head_split_workspace_bytes(3000, 64, 72)
    assert f(None, 3000, 64, A, 72, A2, A, n, None) == ERR_NULL
    assert f(A, 3000, 64, None, 72, A2, A, n, None) == ERR_NULL
    assert f(A, 3000, 12, A, 72, A2, A, n, None) == ERR_SHAPE      # d % 8 != 0
    assert f(A, 3000, 64, A, 0, A2, A, n, None) == ERR_SHAPE
    assert f(A, 3000, 64, MIS, 72, A2, A, n, None) == ERR_ALIGN
    assert f(A, 3000, 64, A, 72, A2, None, n, None) == ERR_WORKSPACE
    assert f(A, 3000, 64, A, 72, A2, A, n - 1, None) == ERR_WORKSPACE
    assert f(A, 3000, 64, A, 72, A2, A + 16, n, None) == ERR_ALIGN  # the workspace is 256-byte aligned


def test_draft_round_workspace_bytes(L):
    f = L.dspark_draft_round_workspace_bytes
    mk = L.dspark_markov_workspace_bytes(8, 9, 32000)
    assert f(1, 7, 7, 151936, 4096) == L.dspark_markov_workspace_bytes(1, 7, 151936)  # 7 rows: no split
    at = (mk + 255) // 256 * 256
    assert f(8, 9, 9, 32000, 5120) == at + L.dspark_lm_head_split_workspace_bytes(32000, 5120, 72)
    assert f(0, 9, 9, 32000, 5120) == 0 and f(8, 0, 9, 32000, 5120) == 0 and f(8, 9, 33, 32000, 5120) == 0
    assert f(8, 9, 9, 32000, 0) == 0


def test_gemv_errors(L):
    for fn in (L.dspark_proj_smallm, L.dspark_lm_head):
        assert fn(None, 16, 64, A, 7, A2, None) == ERR_NULL
        assert fn(A, 16, 64, None, 7, A2, None) == ERR_NULL
        assert fn(A, 16, 64, A, 7, None, None) == ERR_NULL
        assert fn(A, 0, 64, A, 7, A2, None) == ERR_SHAPE
        assert fn(A, 16, 0, A, 7, A2, None) == ERR_SHAPE
        assert fn(A, 16, 12, A, 7, A2, None) == ERR_SHAPE      # K % 8 != 0
        assert fn(A, 16, 64, A, 0, A2, None) == ERR_SHAPE
        assert fn(A, 16, (1 << 22) + 8, A, 7, A2, None) == ERR_SHAPE  # K past the 32-bit buffer ranges
        assert fn(MIS, 16, 64, A, 7, A2, None) == ERR_ALIGN
        assert fn(A, 16, 64, MIS, 7, A2, None) == ERR_ALIGN
        assert fn(A, 16, 64, A, 7, A2 + 1, None) == ERR_ALIGN


def test_gemv_q8_errors(L):
    for fn in (L.dspark_proj_smallm_q8, L.dspark_lm_head_q8):
        assert fn(None, A, 16, 64, A, 7, A2, None) == ERR_NULL
        assert fn(A, None, 16, 64, A, 7, A2, None) == ERR_NULL
        assert fn(A, A, 16, 64, None, 7, A2, None) == ERR_NULL
        assert fn(A, A, 16, 64, A, 7, None, None) == ERR_NULL
        assert fn(A, A, 0, 64, A, 7, A2, None) == ERR_SHAPE
        assert fn(A, A, 16, 16, A, 7, A2, None) == ERR_SHAPE      # K < 32
        assert fn(A, A, 16, 80, A, 7, A2, None) == ERR_SHAPE      # K % 32 != 0
        assert fn(A, A, 16, 64, A, 0, A2, None) == ERR_SHAPE
        assert fn(A, A, 16, (1 << 22) + 32, A, 7, A2, None) == ERR_SHAPE
        assert fn(A + 8, A, 16, 64, A, 7, A2, None) == ERR_ALIGN  # quants need 16 bytes
        assert fn(A, A + 1, 16, 64, A, 7, A2, None) == ERR_ALIGN  # scales need 2
        assert fn(A, A, 16, 64, MIS, 7, A2, None) == ERR_ALIGN


def test_lm_head_q8_ld_errors(L):
    f = L.dspark_lm_head_q8_ld
    assert f(None, A, 2, 16, 64, A, 7, A2, None) == ERR_NULL
    assert f(A, A, 2, 16, 80, A, 7, A2, None) == ERR_SHAPE       # K % 32 != 0
    assert f(A, A, 1, 16, 64, A, 7, A2, None) == ERR_SHAPE       # fewer scales per row than K / 32
    assert f(A, A, 67, 16, 64, A, 7, A2, None) == ERR_SHAPE      # more than one line of padding
    assert f(A, A + 1, 64, 16, 64, A, 7, A2, None) == ERR_ALIGN
    assert f(A, A, 64, 16, 64, MIS, 7, A2, None) == ERR_ALIGN


def test_markov_errors(L):
    f = L.dspark_markov_sample
    ws = L.dspark_markov_workspace_bytes(1, 7, 151936)
    assert ws > 0
    good = dict(base=A, R=1, B=7, V=151936, w1=A, w2=A2, r=256, d2t=None, prev0=A, k=7, ids=A2, ws=A, wsb=ws)

    def call(**kw):
        a = dict(good, **kw)
        return f(a["base"], a["R"], a["B"], a["V"], a["w1"], a["w2"], a["r"], a["d2t"], a["prev0"], a["k"],
                 a["ids"], a["ws"], a["wsb"], None)
    assert call(base=None) == ERR_NULL
    assert call(w1=None) == ERR_NULL
    assert call(prev0=None) == ERR_NULL
    assert call(ids=None) == ERR_NULL
    assert call(R=0) == ERR_SHAPE
    assert call(R=17) == ERR_SHAPE
    assert call(k=8) == ERR_SHAPE          # k > B
    assert call(k=0) == ERR_SHAPE
    assert call(B=40, k=33) == ERR_SHAPE   # k > 32
    assert call(r=12) == ERR_SHAPE         # r % 8 != 0
    assert call(r=2048) == ERR_SHAPE
    assert call(V=0) == ERR_SHAPE
    assert call(w1=MIS) == ERR_ALIGN
    assert call(base=A + 2) == ERR_ALIGN
    assert call(d2t=A + 4) == ERR_ALIGN
    assert call(ws=None) == ERR_WORKSPACE
    assert call(wsb=ws - 1) == ERR_WORKSPACE


def test_markov_spin_limit_setting(L):
    """The poll bound is host state only: setting it makes no HIP call."""
    f = L.dspark_markov_set_spin_limit
    first = f(5)
    assert first == 1 << 18          # the default
    assert f(0) == 5                 # 0 restores the default
    assert f(0) == 1 << 18


def test_markov_noalloc_errors(L):
    """The allocation-free loop rejects what dspark_markov_sample rejects,
    before its static workspace is set up or anything is launched."""
    f = L.dspark_markov_sample_noalloc
    good = dict(base=A, R=1, B=7, V=151936, w1=A, w2=A2, r=256, d2t=None, prev0=A, k=7, ids=A2)

    def call(**kw):
        a = dict(good, **kw)
        return f(a["base"], a["R"], a["B"], a["V"], a["w1"], a["w2"], a["r"], a["d2t"], a["prev0"], a["k"],
                 a["ids"], None)
    assert call(base=None) == ERR_NULL
    assert call(w2=None) == ERR_NULL
    assert call(ids=None) == ERR_NULL
    assert call(R=17) == ERR_SHAPE         # beyond the static workspace
    assert call(B=40, k=33) == ERR_SHAPE   # beyond the static workspace
    assert call(k=8) == ERR_SHAPE
    assert call(r=12) == ERR_SHAPE
    assert call(w1=MIS) == ERR_ALIGN
    assert call(ids=A2 + 4) == ERR_ALIGN


def test_stream_read_errors(L):
    f = L.dspark_stream_read
    assert f(None, 4096, 8, 256, A, None) == ERR_NULL
    assert f(A, 4096, 8, 256, None, None) == ERR_NULL
    assert f(A, 4096, 0, 256, A2, None) == ERR_SHAPE
    assert f(A, 4096, 65537, 256, A2, None) == ERR_SHAPE
    assert f(A, 4096, 8, 128, A2, None) == ERR_SHAPE
    assert f(A, 4100, 8, 256, A2, None) == ERR_SHAPE   # bytes % 16 != 0
    assert f(MIS, 4096, 8, 256, A2, None) == ERR_ALIGN
    assert f(A, 4096, 8, 256, A2 + 2, None) == ERR_ALIGN


def test_stream_read_sched_errors(L):
    f = L.dspark_stream_read_sched
    assert f(None, 4096, 8, 256, A, A2, None) == ERR_NULL
    assert f(A, 4096, 8, 256, None, A2, None) == ERR_NULL     # no counter
    assert f(A, 4096, 8, 256, A, None, None) == ERR_NULL
    assert f(A, 4096, 8, 128, A, A2, None) == ERR_SHAPE
    assert f(A, 4100, 8, 256, A, A2, None) == ERR_SHAPE
    assert f(A, 4096, 8, 256, A + 2, A2, None) == ERR_ALIGN


def test_markov_workspace_bytes(L):
    f = L.dspark_markov_workspace_bytes
    assert f(0, 7, 100) == 0 and f(17, 7, 100) == 0 and f(1, 0, 100) == 0 and f(1, 7, 0) == 0
    assert f(1, 33, 100) == 0
    # one layout for every valid shape, so a workspace can be reused across shapes
    assert f(8, 9, 32000) == f(1, 9, 32000) == f(16, 32, 300000) == f(1, 1, 1) > 0


def test_probe_errors(L):
    f = L.dspark_conf_probe
    assert f(None, 7, 64, A, 0.0, 0.0, A2, None, None) == ERR_NULL
    assert f(A, 7, 64, None, 0.0, 0.0, A2, None, None) == ERR_NULL
    assert f(A, 7, 64, A, 0.0, 0.0, None, None, None) == ERR_NULL
    assert f(A, 0, 64, A, 0.0, 0.0, A2, None, None) == ERR_SHAPE
    assert f(A, 7, 60, A, 0.0, 0.0, A2, None, None) == ERR_SHAPE
    assert f(MIS, 7, 64, A, 0.0, 0.0, A2, None, None) == ERR_ALIGN
    assert f(A, 7, 64, A, 0.0, 0.0, A2, A2 + 2, None) == ERR_ALIGN


def test_markov_sample_probe_errors(L):
    f = L.dspark_markov_sample_probe
    ws = L.dspark_markov_workspace_bytes(1, 7, 151936)
    good = dict(base=A, R=1, B=7, V=151936, w1=A, w2=A2, r=256, d2t=None, prev0=A, k=7, ids=A2, ws=A, wsb=ws,
                x=A2, M=7, D=4096, pw=A, logit=A2, ps=None)

    def call(**kw):
        a = dict(good, **kw)
        return f(a["base"], a["R"], a["B"], a["V"], a["w1"], a["w2"], a["r"], a["d2t"], a["prev0"], a["k"],
                 a["ids"], a["ws"], a["wsb"], a["x"], a["M"], a["D"], a["pw"], 0.0, 0.0, a["logit"], a["ps"], None)
    assert call(base=None) == ERR_NULL
    assert call(x=None) == ERR_NULL
    assert call(pw=None) == ERR_NULL
    assert call(logit=None) == ERR_NULL
    assert call(k=8) == ERR_SHAPE
    assert call(M=0) == ERR_SHAPE
    assert call(D=12) == ERR_SHAPE
    assert call(x=MIS) == ERR_ALIGN
    assert call(ps=A + 2) == ERR_ALIGN
    assert call(wsb=ws - 1) == ERR_WORKSPACE


def test_markov_q8_errors(L):
    f = L.dspark_markov_sample_q8
    ws = L.dspark_markov_workspace_bytes(1, 7, 151936)
    good = dict(base=A, R=1, B=7, V=151936, w1q=A, w1d=A2, w2q=A2, w2d=A, r=256, d2t=None, prev0=A, k=7, ids=A2,
                ws=A, wsb=ws, px=None, pm=0, pd=0, pw=None, lo=None, ps=None)

    def call(**kw):
        a = dict(good, **kw)
        return f(a["base"], a["R"], a["B"], a["V"], a["w1q"], a["w1d"], a["w2q"], a["w2d"], a["r"], a["d2t"],
                 a["prev0"], a["k"], a["ids"], a["ws"], a["wsb"], a["px"], a["pm"], a["pd"], a["pw"], 0.0, 0.0,
                 a["lo"], a["ps"], None)
    assert call(w1q=None) == ERR_NULL
    assert call(w2d=None) == ERR_NULL
    assert call(px=A, pm=7, pd=64, pw=None, lo=A2) == ERR_NULL   # a probe needs its weights
    assert call(r=48) == ERR_SHAPE                                # r % 32 != 0
    assert call(r=512) == ERR_SHAPE                               # r > 256
    assert call(r=16) == ERR_SHAPE
    assert call(k=8) == ERR_SHAPE
    assert call(R=17) == ERR_SHAPE
    assert call(px=A, pm=7, pd=60, pw=A, lo=A2) == ERR_SHAPE      # probe D % 8 != 0
    assert call(w1q=A + 8) == ERR_ALIGN
    assert call(w2d=A + 1) == ERR_ALIGN
    assert call(wsb=ws - 1) == ERR_WORKSPACE


def test_draft_round_q8_errors(L):
    f = L.dspark_draft_round_q8
    ws = L.dspark_markov_workspace_bytes(1, 7, 151936)
    good = dict(Wq=A, Wd=A2, V=151936, d=4096, H=A2, R=1, B=7, w1q=A, w1d=A2, w2q=A2, w2d=A, r=256, d2t=None,
                prev0=A, k=7, pw=A, base=A2, ids=A, lo=A2, ps=None, ws=A, wsb=ws)

    def call(**kw):
        a = dict(good, **kw)
        return f(a["Wq"], a["Wd"], a["V"], a["d"], a["H"], a["R"], a["B"], a["w1q"], a["w1d"], a["w2q"], a["w2d"],
                 a["r"], a["d2t"], a["prev0"], a["k"], a["pw"], 0.0, 0.0, a["base"], a["ids"], a["lo"], a["ps"],
                 a["ws"], a["wsb"], None)
    assert call(Wq=None) == ERR_NULL
    assert call(lo=None) == ERR_NULL
    assert call(d=4100) == ERR_SHAPE      # d % 32 != 0
    assert call(r=1024) == ERR_SHAPE
    assert call(R=0) == ERR_SHAPE
    assert call(Wd=A + 1) == ERR_ALIGN
    assert call(ws=None) == ERR_WORKSPACE


def test_draft_round_q8_ld_errors(L):
    f = L.dspark_draft_round_q8_ld
    ws = L.dspark_markov_workspace_bytes(1, 7, 151936)
    good = dict(Wq=A, Wd=A2, ldd=192, V=151936, d=5120, H=A2, R=1, B=7, w1q=A, w1d=A2, w2q=A2, w2d=A, r=256,
                d2t=None, prev0=A, k=7, pw=A, base=A2, ids=A, lo=A2, ps=None, ws=A, wsb=ws)

    def call(**kw):
        a = dict(good, **kw)
        return f(a["Wq"], a["Wd"], a["ldd"], a["V"], a["d"], a["H"], a["R"], a["B"], a["w1q"], a["w1d"], a["w2q"],
                 a["w2d"], a["r"], a["d2t"], a["prev0"], a["k"], a["pw"], 0.0, 0.0, a["base"], a["ids"], a["lo"],
                 a["ps"], a["ws"], a["wsb"], None)
    assert call(Wq=None) == ERR_NULL
    assert call(ldd=159) == ERR_SHAPE     # d / 32 = 160 scales per row at least
    assert call(ldd=225) == ERR_SHAPE     # at most 64 of padding
    assert call(d=4100) == ERR_SHAPE
    assert call(Wd=A + 1) == ERR_ALIGN
    assert call(ws=None) == ERR_WORKSPACE


def test_draft_round_errors(L):
    f = L.dspark_draft_round
    ws = L.dspark_markov_workspace_bytes(1, 7, 151936)
    good = dict(W=A, V=151936, d=4096, H=A2, R=1, B=7, w1=A, w2=A2, r=256, d2t=None, prev0=A, k=7, pw=A,
                base=A2, ids=A, logit=A2, ps=None, ws=A, wsb=ws)

    def call(**kw):
        a = dict(good, **kw)
        return f(a["W"], a["V"], a["d"], a["H"], a["R"], a["B"], a["w1"], a["w2"], a["r"], a["d2t"], a["prev0"],
                 a["k"], a["pw"], 0.0, 0.0, a["base"], a["ids"], a["logit"], a["ps"], a["ws"], a["wsb"], None)
    assert call(W=None) == ERR_NULL
    assert call(H=None) == ERR_NULL
    assert call(base=None) == ERR_NULL
    assert call(w2=None) == ERR_NULL
    assert call(ids=None) == ERR_NULL
    assert call(logit=None) == ERR_NULL                 # a probe needs its output
    assert call(R=0) == ERR_SHAPE
    assert call(R=17) == ERR_SHAPE
    assert call(B=0) == ERR_SHAPE
    assert call(d=4100) == ERR_SHAPE                    # d % 8 != 0
    assert call(k=8) == ERR_SHAPE                       # k > B
    assert call(r=2048) == ERR_SHAPE
    assert call(H=MIS) == ERR_ALIGN
    assert call(base=A + 2) == ERR_ALIGN
    assert call(pw=MIS) == ERR_ALIGN
    assert call(ps=A + 2) == ERR_ALIGN
    assert call(ws=None) == ERR_WORKSPACE
    assert call(wsb=ws - 1) == ERR_WORKSPACE
    # 8 requests x 9 rows: the round's lm_head splits K, so the workspace
    # holds the loop's and the split's
    big = L.dspark_draft_round_workspace_bytes(8, 9, 9, 32000, 5120)
    batched = dict(V=32000, d=5120, R=8, B=9, k=9, wsb=big)
    assert call(**dict(batched, wsb=L.dspark_markov_workspace_bytes(8, 9, 32000))) == ERR_WORKSPACE
    assert call(**dict(batched, wsb=big - 1)) == ERR_WORKSPACE
    assert call(**dict(batched, ws=A + 64)) == ERR_ALIGN


def test_block_errors(L):
    assert L.dspark_rmsnorm(None, 7, 64, A, 1e-6, A2, None) == ERR_NULL
    assert L.dspark_rmsnorm(A, 0, 64, A, 1e-6, A2, None) == ERR_SHAPE
    assert L.dspark_rmsnorm(A, 7, 64, A, -1.0, A2, None) == ERR_SHAPE
    assert L.dspark_rmsnorm(MIS, 7, 64, A, 1e-6, A2, None) == ERR_ALIGN
    assert L.dspark_silu_gate(None, 7, 64, A2, None) == ERR_NULL
    assert L.dspark_silu_gate(A, 7, 0, A2, None) == ERR_SHAPE
    assert L.dspark_proj_smallm_add(A, 16, 64, A, 7, None, A2, None) == ERR_NULL
    assert L.dspark_proj_smallm_add(A, 16, 12, A, 7, A, A2, None) == ERR_SHAPE
    assert L.dspark_proj_smallm_add(A, 16, 64, A, 7, A + 2, A2, None) == ERR_ALIGN
    # the fused norm: arguments checked like dspark_proj_smallm's, then gamma
    # and eps; without a device no shape qualifies for the fused kernel
    g = L.dspark_proj_smallm_norm
    assert L.dspark_proj_smallm_norm_fits(4096, 4096, 7) == 0
    assert L.dspark_proj_smallm_norm_fits(4096, 4096, 17) == 0
    assert g(None, 16, 64, A, 7, A2, 1e-6, A2, None) == ERR_NULL
    assert g(A, 16, 64, A, 7, None, 1e-6, A2, None) == ERR_NULL
    assert g(A, 16, 12, A, 7, A2, 1e-6, A2, None) == ERR_SHAPE       # K % 8 != 0
    assert g(A, 16, 64, A, 7, A2, -1.0, A2, None) == ERR_SHAPE
    assert g(A, 16, 64, A, 17, A2, 1e-6, A2, None) == ERR_SHAPE      # more than 16 rows
    assert g(A, 16, 64, MIS, 7, A2, 1e-6, A2, None) == ERR_ALIGN
    f = L.dspark_attention_ragged
    need = L.dspark_attention_workspace_bytes(1, 7, 32, 128, 512)
    assert need == 32 * 9 * 7 * 130 * 4                       # 9 chunks of 64 keys, m, l and o per chunk
    assert L.dspark_attention_workspace_bytes(1, 17, 32, 128, 512) == 0
    ok = dict(q=A, k=A2, v=A, ld=3 * 4096, R=1, B=7, H=32, Dh=128, kc=A, vc=A2, Lmax=512, lens=A, c=0, out=A2,
              ws=A, nws=need)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["k"], a["v"], a["ld"], a["R"], a["B"], a["H"], a["Dh"], a["kc"], a["vc"], a["Lmax"],
                 a["lens"], a["c"], a["out"], a["ws"], a["nws"], None)
    assert call(q=None) == ERR_NULL
    assert call(kc=None) == ERR_NULL
    assert call(B=17) == ERR_SHAPE
    assert call(Dh=100) == ERR_SHAPE                 # Dh % 8 != 0
    assert call(Dh=512) == ERR_SHAPE
    assert call(Lmax=-1) == ERR_SHAPE
    assert call(Lmax=4000) == ERR_WORKSPACE          # more chunks than the workspace holds
    assert call(ws=None) == ERR_WORKSPACE
    assert call(nws=need - 1) == ERR_WORKSPACE
    assert call(ws=A + 8) == ERR_ALIGN
    assert call(ld=4094) == ERR_SHAPE
    assert call(k=A2 + 4) == ERR_ALIGN


def test_binding_has_no_cpu_path(L):
    import torch
    from gemv_markov_argmax_amd import ops
    W = torch.zeros(16, 64, dtype=torch.bfloat16)
    X = torch.zeros(7, 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        ops.proj_smallm(W, X)
    with pytest.raises(ValueError, match="GPU tensor"):
        ops.conf_probe(X, torch.zeros(64, dtype=torch.bfloat16))


def test_draft_block_rejects_bad_arguments(L):
    need = L.dspark_draft_block_workspace_bytes(1, 7, 32, 128, 4096, 12288, 512)
    assert need > 0
    assert L.dspark_draft_block_workspace_bytes(1, 7, 32, 128, 4096, 12283, 512) == 0     # F % 8 != 0
    ok = dict(wqkv=A, wo=A2, wgu=A, wd=A2, ln1=A, ln2=A2, d=4096, F=12288, H=32, Dh=128, R=1, B=7, hin=A, hout=A2,
              kc=A, vc=A2, Lmax=512, lens=A, eps=1e-6, c=0, ws=A, nws=need)

    def call(**kw):
        a = dict(ok, **kw)
        return L.dspark_draft_block(a["wqkv"], a["wo"], a["wgu"], a["wd"], a["ln1"], a["ln2"], a["d"], a["F"], a["H"],
                                    a["Dh"], a["R"], a["B"], a["hin"], a["hout"], a["kc"], a["vc"], a["Lmax"],
                                    a["lens"], a["eps"], a["c"], a["ws"], a["nws"], None)
    assert call(wo=None) == ERR_NULL
    assert call(ln2=None) == ERR_NULL
    assert call(vc=None) == ERR_NULL
    assert call(d=4092) == ERR_SHAPE
    assert call(B=17) == ERR_SHAPE
    assert call(eps=-1.0) == ERR_SHAPE
    assert call(ws=None) == ERR_WORKSPACE
    assert call(nws=need - 1) == ERR_WORKSPACE
    assert call(ws=A + 16) == ERR_ALIGN                  # the workspace needs 256-byte alignment
    assert call(hin=A + 4) == ERR_ALIGN
    assert call(ln1=A + 1) == ERR_ALIGN
