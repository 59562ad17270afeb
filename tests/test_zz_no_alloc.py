"""The allocation-free Markov loop (dspark_markov_sample_noalloc), called
through the C ABI, against the workspace entry point dspark_markov_sample on
the same inputs: ids identical, two calls in a row, the second smaller, so
the second call runs on the static workspace the first one left."""
import ctypes

import numpy as np
import pytest

from gemv_markov_argmax_amd import synth
from parity import check_markov, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gemv_markov_argmax_amd import ops
    ops.lib()
    return torch.device("cuda:0")


def _call_both(dev, R, B, k, V, r, seed, d2t):
    from gemv_markov_argmax_amd import ops
    L = ops.lib()
    base, w1, w2, prev0, _ = synth.markov_inputs(R, B, V, r, seed)
    prev0 = prev0.copy()
    if R > 1:
        prev0[R - 1] = V + 5  # an invalid prev0: that request's ids are -1 on both paths
    bd = torch.from_numpy(base).to(dev)
    w1d, w2d = ops.bf16_from_bits(w1, dev), ops.bf16_from_bits(w2, dev)
    pd = torch.from_numpy(prev0).to(dev)
    dm = torch.from_numpy(d2t).to(dev) if d2t is not None else None
    dptr = dm.data_ptr() if dm is not None else None
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    got = torch.full((R, k), -9, dtype=torch.int64, device=dev)
    st = L.dspark_markov_sample_noalloc(bd.data_ptr(), R, B, V, w1d.data_ptr(), w2d.data_ptr(), r, dptr,
                                        pd.data_ptr(), k, got.data_ptr(), stream)
    assert st == 0, ops.status_string(st)
    ws = ops.markov_workspace(R, k, V, dev)
    want = torch.full((R, k), -9, dtype=torch.int64, device=dev)
    st = L.dspark_markov_sample(bd.data_ptr(), R, B, V, w1d.data_ptr(), w2d.data_ptr(), r, dptr, pd.data_ptr(), k,
                                want.data_ptr(), ws.data_ptr(), ws.numel(), stream)
    assert st == 0, ops.status_string(st)
    torch.cuda.synchronize()
    return got.cpu().numpy(), want.cpu().numpy(), (base, w1, w2, prev0)


def test_noalloc_matches_workspace_entry_point(dev):
    cases = [(4, 9, 9, 32000, 256, 7301, True), (1, 7, 3, 4099, 64, 7302, False)]  # second: smaller
    for n, (R, B, k, V, r, seed, with_d2t) in enumerate(cases):
        say(f"[noalloc call {n}] R={R} B={B} k={k} V={V} r={r} seed={seed} d2t={with_d2t}")
        d2t = synth.d2t_map(V, seed) if with_d2t else None
        got, want, (base, w1, w2, prev0) = _call_both(dev, R, B, k, V, r, seed, d2t)
        assert np.array_equal(got, want), f"call {n}: {got} vs {want}"
        if R > 1:
            assert np.all(got[R - 1] == -1)
        check_markov(got, base, w1, w2, prev0, k, d2t=d2t)  # and the oracle agrees
