"""Thin ctypes binding of libdspark.so (argument marshalling only).

Every computation runs in the library's HIP kernels on the tensors' device;
PyTorch only supplies device memory and the current stream. There is no CPU
fallback: CPU tensors, wrong dtypes and a missing library raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdspark.so")
_lib = None

_p = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t

SIGNATURES = {
    "dspark_status_string": (ctypes.c_char_p, [_i]),
    "dspark_proj_smallm": (_i, [_p, _i, _i, _p, _i, _p, _p]),
    "dspark_lm_head": (_i, [_p, _i, _i, _p, _i, _p, _p]),
    "dspark_lm_head_sched": (_i, [_p, _i, _i, _p, _i, _p, _p, _p]),
    "dspark_lm_head_split_workspace_bytes": (_sz, [_i, _i, _i]),
    "dspark_lm_head_split": (_i, [_p, _i, _i, _p, _i, _p, _p, _sz, _p]),
    "dspark_draft_round_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "dspark_proj_smallm_q8": (_i, [_p, _p, _i, _i, _p, _i, _p, _p]),
    "dspark_lm_head_q8": (_i, [_p, _p, _i, _i, _p, _i, _p, _p]),
    "dspark_lm_head_q8_ld": (_i, [_p, _p, _i, _i, _i, _p, _i, _p, _p]),
    "dspark_markov_sample_q8": (_i, [_p, _i, _i, _i, _p, _p, _p, _p, _i, _p, _p, _i, _p, _p, _sz,
                                     _p, _i, _i, _p, _f, _f, _p, _p, _p]),
    "dspark_draft_round_q8": (_i, [_p, _p, _i, _i, _p, _i, _i, _p, _p, _p, _p, _i, _p, _p, _i, _p, _f, _f,
                                   _p, _p, _p, _p, _p, _sz, _p]),
    "dspark_draft_round_q8_ld": (_i, [_p, _p, _i, _i, _i, _p, _i, _i, _p, _p, _p, _p, _i, _p, _p, _i, _p, _f, _f,
                                      _p, _p, _p, _p, _p, _sz, _p]),
    "dspark_rmsnorm": (_i, [_p, _i, _i, _p, _f, _p, _p]),
    "dspark_silu_gate": (_i, [_p, _i, _i, _p, _p]),
    "dspark_proj_smallm_add": (_i, [_p, _i, _i, _p, _i, _p, _p, _p]),
    "dspark_proj_smallm_norm_fits": (_i, [_i, _i, _i]),
    "dspark_proj_smallm_norm": (_i, [_p, _i, _i, _p, _i, _p, _f, _p, _p]),
    "dspark_attention_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "dspark_attention_ragged": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _i, _p, _i, _p, _p, _sz, _p]),
    "dspark_draft_block_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "dspark_draft_block": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _i, _p, _f, _i,
                                _p, _sz, _p]),
    "dspark_markov_workspace_bytes": (_sz, [_i, _i, _i]),
    "dspark_markov_set_spin_limit": (ctypes.c_uint32, [ctypes.c_uint32]),
    "dspark_stream_read": (_i, [_p, _sz, _i, _i, _p, _p]),
    "dspark_stream_read_sched": (_i, [_p, _sz, _i, _i, _p, _p, _p]),
    "dspark_markov_sample_noalloc": (_i, [_p, _i, _i, _i, _p, _p, _i, _p, _p, _i, _p, _p]),
    "dspark_markov_sample": (_i, [_p, _i, _i, _i, _p, _p, _i, _p, _p, _i, _p, _p, _sz, _p]),
    "dspark_conf_probe": (_i, [_p, _i, _i, _p, _f, _f, _p, _p, _p]),
    "dspark_markov_sample_probe": (_i, [_p, _i, _i, _i, _p, _p, _i, _p, _p, _i, _p, _p, _sz,
                                        _p, _i, _i, _p, _f, _f, _p, _p, _p]),
    "dspark_draft_round": (_i, [_p, _i, _i, _p, _i, _i, _p, _p, _i, _p, _p, _i, _p, _f, _f,
                                _p, _p, _p, _p, _p, _sz, _p]),
}


class DsparkError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libdspark.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m gemv_markov_argmax_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().dspark_status_string(status).decode()


def _check(status: int) -> None:
    if status != 0:
        raise DsparkError(status, status_string(status))


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str, ndim: int | None = None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    return t


_hip = None


def _host_device_ptr(t: torch.Tensor) -> int:
    """The device address of a pinned host tensor (hipHostGetDevicePointer of
    the HIP runtime this process already uses)."""
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
        _hip.hipHostGetDevicePointer.restype = ctypes.c_int
        _hip.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_uint]
    p = ctypes.c_void_p()
    err = _hip.hipHostGetDevicePointer(ctypes.byref(p), ctypes.c_void_p(t.data_ptr()), 0)
    if err != 0 or not p.value:
        raise RuntimeError(f"hipHostGetDevicePointer failed ({err}): the host tensor is not mapped for the device")
    return p.value


def _out_ptr(t: torch.Tensor, dtype: torch.dtype, name: str, ndim: int | None = None) -> int:
    """Address of a small result array: a GPU tensor, or a pinned host tensor
    (the kernel then stores the results straight into host memory)."""
    if isinstance(t, torch.Tensor) and not t.is_cuda and t.is_pinned():
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if not t.is_contiguous() or (ndim is not None and t.dim() != ndim):
            raise ValueError(f"{name} must be contiguous with {ndim} dims")
        return _host_device_ptr(t)
    return _dev(t, dtype, name, ndim).data_ptr()


def _gemv(entry, W, X, out):
    _dev(W, torch.bfloat16, "W", 2)
    _dev(X, torch.float32, "X", 2)
    N, K = W.shape
    M = X.shape[0]
    if X.shape[1] != K:
        raise ValueError(f"X has {X.shape[1]} columns, W has {K}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=W.device)
    _dev(out, torch.float32, "out", 2)
    if tuple(out.shape) != (M, N):
        raise ValueError("out must be [M, N]")
    _check(entry(W.data_ptr(), N, K, X.data_ptr(), M, out.data_ptr(), _stream(W)))
    return out


def lm_head_counter(device) -> torch.Tensor:
    """A zeroed counter for lm_head_sched (one 32-bit word of device memory)."""
    return torch.zeros(1, dtype=torch.int32, device=device)


def lm_head_sched(W_lm: torch.Tensor, H: torch.Tensor, counter: torch.Tensor, out: torch.Tensor | None = None,
                  counter_offset: int = 0) -> torch.Tensor:
    """Base logits with the weight rows handed out by a counter
    (dspark_lm_head_sched). ``counter``: device memory whose word at byte
    ``counter_offset`` reads 0 (lm_head_counter(), or a Markov workspace at
    offset markov_lm_counter_offset()); every call leaves it 0."""
    _dev(W_lm, torch.bfloat16, "W_lm", 2)
    _dev(H, torch.float32, "H", 2)
    if not counter.is_cuda:
        raise ValueError("counter must be a GPU tensor")
    if counter_offset < 0 or counter_offset + 4 > counter.numel() * counter.element_size():
        raise ValueError("counter word out of range")
    V, d = W_lm.shape
    rows = H.shape[0]
    if H.shape[1] != d:
        raise ValueError(f"H has {H.shape[1]} columns, W_lm has {d}")
    if out is None:
        out = torch.empty((rows, V), dtype=torch.float32, device=W_lm.device)
    _dev(out, torch.float32, "out", 2)
    if tuple(out.shape) != (rows, V):
        raise ValueError("out must be [rows, V]")
    _check(lib().dspark_lm_head_sched(W_lm.data_ptr(), V, d, H.data_ptr(), rows, out.data_ptr(),
                                      counter.data_ptr() + counter_offset, _stream(W_lm)))
    return out


def lm_head_split_workspace_bytes(V: int, d: int, rows: int) -> int:
    return int(lib().dspark_lm_head_split_workspace_bytes(V, d, rows))


def lm_head_split_workspace(V: int, d: int, rows: int, device) -> torch.Tensor | None:
    """A zero-filled workspace for dspark_lm_head_split (None where the split
    does not apply); reusable by calls of the same or smaller sizes."""
    n = lm_head_split_workspace_bytes(V, d, rows)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n > 0 else None


def lm_head_split(W_lm: torch.Tensor, H: torch.Tensor, workspace: torch.Tensor | None,
                  out: torch.Tensor | None = None) -> torch.Tensor:
    """Base logits [rows, V] = H @ W_lm^T with d split in two halves taken by
    different workgroups (dspark_lm_head_split). ``workspace``: uint8 device
    memory of lm_head_split_workspace_bytes(V, d, rows), zero-filled once
    (None where that is 0)."""
    _dev(W_lm, torch.bfloat16, "W_lm", 2)
    _dev(H, torch.float32, "H", 2)
    V, d = W_lm.shape
    rows = H.shape[0]
    if H.shape[1] != d:
        raise ValueError(f"H has {H.shape[1]} columns, W_lm has {d}")
    if out is None:
        out = torch.empty((rows, V), dtype=torch.float32, device=W_lm.device)
    _dev(out, torch.float32, "out", 2)
    if tuple(out.shape) != (rows, V):
        raise ValueError("out must be [rows, V]")
    wp, wn = None, 0
    if workspace is not None:
        _dev(workspace, torch.uint8, "workspace", 1)
        wp, wn = workspace.data_ptr(), workspace.numel()
    _check(lib().dspark_lm_head_split(W_lm.data_ptr(), V, d, H.data_ptr(), rows, out.data_ptr(), wp, wn,
                                      _stream(W_lm)))
    return out


def markov_lm_counter_offset() -> int:
    """Byte offset of the word of a Markov workspace that dspark_draft_round
    gives its lm_head as counter."""
    return 64


def proj_smallm(W: torch.Tensor, X: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Y = X @ W^T for bf16 W [N, K] and fp32 X [M, K] (dspark_proj_smallm)."""
    return _gemv(lib().dspark_proj_smallm, W, X, out)


def lm_head(W_lm: torch.Tensor, H: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Base logits [rows, V] = H @ W_lm^T (dspark_lm_head)."""
    return _gemv(lib().dspark_lm_head, W_lm, H, out)


def _gemv_q8(entry, Wq, Wd, X, out):
    _dev(Wq, torch.int8, "Wq", 2)
    _dev(Wd, torch.float16, "Wd", 2)
    _dev(X, torch.float32, "X", 2)
    N, K = Wq.shape
    M = X.shape[0]
    if X.shape[1] != K or K % 32 != 0 or tuple(Wd.shape) != (N, K // 32):
        raise ValueError("Wq [N, K] (K % 32 == 0), Wd [N, K / 32] and X [M, K] required")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=X.device)
    _dev(out, torch.float32, "out", 2)
    if tuple(out.shape) != (M, N):
        raise ValueError("out must be [M, N]")
    _check(entry(Wq.data_ptr(), Wd.data_ptr(), N, K, X.data_ptr(), M, out.data_ptr(), _stream(Wq)))
    return out


def proj_smallm_q8(Wq: torch.Tensor, Wd: torch.Tensor, X: torch.Tensor, out: torch.Tensor | None = None):
    """Y = X @ dequant(W).T for Q8_0 weights (dspark_proj_smallm_q8): Wq int8 [N, K],
    Wd float16 [N, K / 32] (the block scales), X fp32 [M, K]."""
    return _gemv_q8(lib().dspark_proj_smallm_q8, Wq, Wd, X, out)


def lm_head_q8(Wq: torch.Tensor, Wd: torch.Tensor, H: torch.Tensor, out: torch.Tensor | None = None):
    """Base logits from a Q8_0 lm_head (dspark_lm_head_q8). Wd may have
    padded rows, [V, ldd] with d / 32 <= ldd <= d / 32 + 64 (as q8_pad_scales
    makes them); the call is then dspark_lm_head_q8_ld."""
    V, d = Wq.shape
    if Wd.dim() != 2 or Wd.shape[0] != V or Wd.shape[1] == d // 32:
        return _gemv_q8(lib().dspark_lm_head_q8, Wq, Wd, H, out)
    ldd = Wd.shape[1]
    _dev(Wq, torch.int8, "Wq", 2)
    _dev(Wd, torch.float16, "Wd", 2)
    _dev(H, torch.float32, "H", 2)
    M = H.shape[0]
    if H.shape[1] != d or d % 32 != 0:
        raise ValueError("Wq [V, d] (d % 32 == 0) and H [rows, d] required")
    if out is None:
        out = torch.empty((M, V), dtype=torch.float32, device=H.device)
    _dev(out, torch.float32, "out", 2)
    if tuple(out.shape) != (M, V):
        raise ValueError("out must be [rows, V]")
    _check(lib().dspark_lm_head_q8_ld(Wq.data_ptr(), Wd.data_ptr(), ldd, V, d, H.data_ptr(), M, out.data_ptr(),
                                      _stream(Wq)))
    return out


def q8_pad_scales(Wd: torch.Tensor, line: int = 64) -> torch.Tensor:
    """Q8_0 scale rows padded with zeros to a multiple of ``line`` values (64
    binary16 values: whole 128-byte lines), for dspark_lm_head_q8_ld and
    dspark_draft_round_q8_ld. A layout made once when the weights are packed;
    the products are the same, bit for bit."""
    N, kb = Wd.shape
    ldd = (kb + line - 1) // line * line
    if ldd == kb:
        return Wd
    out = torch.zeros((N, ldd), dtype=Wd.dtype, device=Wd.device)
    out[:, :kb] = Wd
    return out


def proj_smallm_add(W: torch.Tensor, X: torch.Tensor, residual: torch.Tensor, out: torch.Tensor | None = None):
    """Y = residual + X @ W.T (dspark_proj_smallm_add); out may be residual itself."""
    _dev(W, torch.bfloat16, "W", 2)
    _dev(X, torch.float32, "X", 2)
    _dev(residual, torch.float32, "residual", 2)
    N, K = W.shape
    M = X.shape[0]
    if X.shape[1] != K or tuple(residual.shape) != (M, N):
        raise ValueError("W [N, K], X [M, K] and residual [M, N] required")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=X.device)
    _dev(out, torch.float32, "out", 2)
    _check(lib().dspark_proj_smallm_add(W.data_ptr(), N, K, X.data_ptr(), M, residual.data_ptr(), out.data_ptr(),
                                        _stream(W)))
    return out


def proj_smallm_norm_fits(N: int, K: int, M: int) -> bool:
    """Whether dspark_proj_smallm_norm takes this shape (dspark_proj_smallm_norm_fits)."""
    return bool(lib().dspark_proj_smallm_norm_fits(N, K, M))


def proj_smallm_norm(W: torch.Tensor, X: torch.Tensor, gamma: torch.Tensor, eps: float,
                     out: torch.Tensor | None = None):
    """Y = rmsnorm(X; gamma, eps) @ W.T with the norm fused into the projection
    (dspark_proj_smallm_norm); gamma bf16 [K]."""
    _dev(W, torch.bfloat16, "W", 2)
    _dev(X, torch.float32, "X", 2)
    _dev(gamma, torch.bfloat16, "gamma", 1)
    N, K = W.shape
    M = X.shape[0]
    if X.shape[1] != K or gamma.shape[0] != K:
        raise ValueError("W [N, K], X [M, K] and gamma [K] required")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=X.device)
    _dev(out, torch.float32, "out", 2)
    _check(lib().dspark_proj_smallm_norm(W.data_ptr(), N, K, X.data_ptr(), M, gamma.data_ptr(), float(eps),
                                         out.data_ptr(), _stream(W)))
    return out


def rmsnorm(x: torch.Tensor, gamma: torch.Tensor, eps: float, out: torch.Tensor | None = None):
    """x / sqrt(mean(x^2) + eps) * gamma per row (dspark_rmsnorm); gamma bf16 [D]."""
    _dev(x, torch.float32, "x", 2)
    _dev(gamma, torch.bfloat16, "gamma", 1)
    M, D = x.shape
    if gamma.shape[0] != D:
        raise ValueError("gamma must have D entries")
    if out is None:
        out = torch.empty_like(x)
    _dev(out, torch.float32, "out", 2)
    _check(lib().dspark_rmsnorm(x.data_ptr(), M, D, gamma.data_ptr(), float(eps), out.data_ptr(), _stream(x)))
    return out


def silu_gate(gu: torch.Tensor, out: torch.Tensor | None = None):
    """silu(gu[:, :F]) * gu[:, F:] (dspark_silu_gate)."""
    _dev(gu, torch.float32, "gu", 2)
    M, F2 = gu.shape
    if F2 % 2:
        raise ValueError("gu must have an even number of columns")
    if out is None:
        out = torch.empty((M, F2 // 2), dtype=torch.float32, device=gu.device)
    _dev(out, torch.float32, "out", 2)
    _check(lib().dspark_silu_gate(gu.data_ptr(), M, F2 // 2, out.data_ptr(), _stream(gu)))
    return out


def attention_workspace_bytes(R: int, B: int, H: int, Dh: int, Lmax: int) -> int:
    return int(lib().dspark_attention_workspace_bytes(R, B, H, Dh, Lmax))


def attention_ragged(qkv: torch.Tensor, R: int, B: int, H: int, Dh: int, k_ctx: torch.Tensor, v_ctx: torch.Tensor,
                     ctx_len: torch.Tensor, block_causal: bool = False, out: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None):
    """Attention of the draft positions (dspark_attention_ragged). qkv fp32
    [R * B, 3 H Dh] holds q, k and v as three column blocks (the fused qkv
    projection's output); k_ctx, v_ctx bf16 [R, Lmax, H Dh]; ctx_len int32 [R].
    ``workspace`` (uint8, at least attention_workspace_bytes) is allocated when
    not given."""
    _dev(qkv, torch.float32, "qkv", 2)
    _dev(k_ctx, torch.bfloat16, "k_ctx", 3)
    _dev(v_ctx, torch.bfloat16, "v_ctx", 3)
    _dev(ctx_len, torch.int32, "ctx_len", 1)
    HD = H * Dh
    if tuple(qkv.shape) != (R * B, 3 * HD) or k_ctx.shape[0] != R or k_ctx.shape[2] != HD or v_ctx.shape != k_ctx.shape:
        raise ValueError("qkv [R * B, 3 H Dh] and k_ctx, v_ctx [R, Lmax, H Dh] required")
    if out is None:
        out = torch.empty((R * B, HD), dtype=torch.float32, device=qkv.device)
    _dev(out, torch.float32, "out", 2)
    if workspace is None:
        workspace = torch.empty(max(attention_workspace_bytes(R, B, H, Dh, k_ctx.shape[1]), 16), dtype=torch.uint8,
                                device=qkv.device)
    _dev(workspace, torch.uint8, "workspace", 1)
    base = qkv.data_ptr()
    _check(lib().dspark_attention_ragged(base, base + HD * 4, base + 2 * HD * 4, 3 * HD, R, B, H, Dh,
                                         k_ctx.data_ptr(), v_ctx.data_ptr(), k_ctx.shape[1], ctx_len.data_ptr(),
                                         1 if block_causal else 0, out.data_ptr(), workspace.data_ptr(),
                                         workspace.numel(), _stream(qkv)))
    return out


def draft_block_workspace_bytes(R: int, B: int, H: int, Dh: int, d: int, F: int, Lmax: int) -> int:
    return int(lib().dspark_draft_block_workspace_bytes(R, B, H, Dh, d, F, Lmax))


def draft_block_forward(h: torch.Tensor, w: dict, R: int, B: int, H: int, Dh: int, k_ctx: torch.Tensor,
                        v_ctx: torch.Tensor, ctx_len: torch.Tensor, eps: float, block_causal: bool = False,
                        scratch: dict | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """One draft block (layer) in one C-ABI call (dspark_draft_block): the
    fused qkv projection with the rmsnorm in front of it, attention, o with
    the residual, the fused gate/up projection with its rmsnorm, the SiLU
    gate, and down with the residual. w
    holds bf16 tensors qkv [3 H Dh, d], o [d, H Dh], gate_up [2F, d],
    down [d, F], ln1, ln2 [d]. ``scratch`` (a dict) keeps the workspace
    between calls; ``out`` may be h itself."""
    M, d = h.shape
    F = w["down"].shape[1]
    _dev(h, torch.float32, "h", 2)
    for name in ("qkv", "o", "gate_up", "down", "ln1", "ln2"):
        _dev(w[name], torch.bfloat16, name, 2 if name not in ("ln1", "ln2") else 1)
    _dev(k_ctx, torch.bfloat16, "k_ctx", 3)
    _dev(v_ctx, torch.bfloat16, "v_ctx", 3)
    _dev(ctx_len, torch.int32, "ctx_len", 1)
    if M != R * B or k_ctx.shape[0] != R or v_ctx.shape != k_ctx.shape or k_ctx.shape[2] != H * Dh:
        raise ValueError("h [R * B, d] and k_ctx, v_ctx [R, Lmax, H Dh] required")
    Lmax = k_ctx.shape[1]
    n = draft_block_workspace_bytes(R, B, H, Dh, d, F, Lmax)
    sc = scratch if scratch is not None else {}
    if "ws" not in sc or sc["ws"].numel() < n + 256:
        sc["ws"] = torch.empty(max(n, 1) + 256, dtype=torch.uint8, device=h.device)
    ws = sc["ws"]
    off = (-ws.data_ptr()) % 256
    if out is None:
        out = torch.empty_like(h)
    _dev(out, torch.float32, "out", 2)
    _check(lib().dspark_draft_block(w["qkv"].data_ptr(), w["o"].data_ptr(), w["gate_up"].data_ptr(),
                                    w["down"].data_ptr(), w["ln1"].data_ptr(), w["ln2"].data_ptr(), d, F, H, Dh, R,
                                    B, h.data_ptr(), out.data_ptr(), k_ctx.data_ptr(), v_ctx.data_ptr(), Lmax,
                                    ctx_len.data_ptr(), float(eps), 1 if block_causal else 0, ws.data_ptr() + off,
                                    ws.numel() - off, _stream(h)))
    return out


def draft_forward(x_in: torch.Tensor, fc: torch.Tensor, layers: list, k_ctx: list, v_ctx: list, R: int, B: int,
                  H: int, Dh: int, ctx_len: torch.Tensor, norm: torch.Tensor, eps: float, block_causal: bool = False,
                  scratch: dict | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """The drafter's forward up to the lm_head's input: h = x_in fc^T
    (dspark_proj_smallm), each block in order (dspark_draft_block, with its
    own context cache), then the final norm (dspark_rmsnorm). Returns the
    normed hidden states [R * B, d]."""
    sc = scratch if scratch is not None else {}
    M, d = x_in.shape[0], fc.shape[0]
    if "h" not in sc or tuple(sc["h"].shape) != (M, d):
        sc["h"] = torch.empty((M, d), dtype=torch.float32, device=x_in.device)
    h = proj_smallm(fc, x_in, out=sc["h"])
    for w, kc, vc in zip(layers, k_ctx, v_ctx):
        draft_block_forward(h, w, R, B, H, Dh, kc, vc, ctx_len, eps, block_causal, scratch=sc, out=h)
    return rmsnorm(h, norm, eps, out=out)


def draft_block_forward_calls(h: torch.Tensor, w: dict, R: int, B: int, H: int, Dh: int, k_ctx: torch.Tensor,
                              v_ctx: torch.Tensor, ctx_len: torch.Tensor, eps: float, block_causal: bool = False,
                              out: torch.Tensor | None = None) -> torch.Tensor:
    """The same block as separate C-ABI calls: proj_smallm_norm (or rmsnorm
    then proj_smallm where its shape or the norm weights' alignment rule it
    out), attention_ragged, proj_smallm_add, proj_smallm_norm (or rmsnorm
    then proj_smallm), silu_gate, proj_smallm_add; dspark_draft_block must
    match it bit for bit."""
    M, d = h.shape
    F = w["down"].shape[1]

    def normed_proj(W, x, gamma):
        if proj_smallm_norm_fits(W.shape[0], W.shape[1], x.shape[0]) and gamma.data_ptr() % 16 == 0:
            return proj_smallm_norm(W, x, gamma, eps)
        return proj_smallm(W, rmsnorm(x, gamma, eps))

    qkv = normed_proj(w["qkv"], h, w["ln1"])
    attn = attention_ragged(qkv, R, B, H, Dh, k_ctx, v_ctx, ctx_len, block_causal)
    h2 = proj_smallm_add(w["o"], attn, h)
    gu = normed_proj(w["gate_up"], h2, w["ln2"])
    act = silu_gate(gu)
    return proj_smallm_add(w["down"], act, h2, out=out if out is not None else torch.empty_like(h))


def q8_from_numpy(q, d_bits, device):
    """Upload Q8_0 weights (int8 quants, uint16 binary16 scale bits) as torch tensors."""
    import numpy as np
    qt = torch.from_numpy(np.ascontiguousarray(q, dtype=np.int8)).to(device)
    dt = torch.from_numpy(np.ascontiguousarray(d_bits, dtype=np.uint16).view(np.float16)).to(device)
    return qt, dt


def markov_workspace_bytes(num_reqs: int, k: int, V: int) -> int:
    return int(lib().dspark_markov_workspace_bytes(num_reqs, k, V))


def markov_workspace(num_reqs: int, k: int, V: int, device) -> torch.Tensor:
    """A zero-filled workspace for dspark_markov_sample; reusable for calls of any shape."""
    n = markov_workspace_bytes(num_reqs, k, V)
    if n == 0:
        raise ValueError("sizes out of range for the Markov loop")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def draft_round_workspace_bytes(num_reqs: int, B: int, k: int, V: int, d: int) -> int:
    return int(lib().dspark_draft_round_workspace_bytes(num_reqs, B, k, V, d))


def draft_round_workspace(num_reqs: int, B: int, k: int, V: int, d: int, device) -> torch.Tensor:
    """A zero-filled workspace for dspark_draft_round: the Markov loop's, then
    (num_reqs * B > 16) the split lm_head's."""
    n = draft_round_workspace_bytes(num_reqs, B, k, V, d)
    if n == 0:
        raise ValueError("sizes out of range for the draft round")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def stream_read(buf: torch.Tensor, groups: int, threads: int, sink: torch.Tensor | None = None,
                nbytes: int | None = None) -> torch.Tensor:
    """Streaming read of a device tensor's bytes (dspark_stream_read, a
    measurement aid); returns the per-workgroup sink words."""
    if not buf.is_cuda:
        raise ValueError("buf must be a device tensor")
    n = buf.numel() * buf.element_size() if nbytes is None else int(nbytes)
    if sink is None:
        sink = torch.empty(groups, dtype=torch.int32, device=buf.device)
    _check(lib().dspark_stream_read(buf.data_ptr() if n else None, n, groups, threads, sink.data_ptr(),
                                    _stream(buf)))
    return sink


def stream_read_sched(buf: torch.Tensor, groups: int, threads: int, counter: torch.Tensor,
                      sink: torch.Tensor | None = None, nbytes: int | None = None) -> torch.Tensor:
    """The same read with the scheduled lm_head's schedule
    (dspark_stream_read_sched); ``counter`` as for lm_head_sched."""
    if not buf.is_cuda or not counter.is_cuda:
        raise ValueError("buf and counter must be device tensors")
    n = buf.numel() * buf.element_size() if nbytes is None else int(nbytes)
    if sink is None:
        sink = torch.empty(groups, dtype=torch.int32, device=buf.device)
    _check(lib().dspark_stream_read_sched(buf.data_ptr() if n else None, n, groups, threads, counter.data_ptr(),
                                          sink.data_ptr(), _stream(buf)))
    return sink


def markov_set_spin_limit(polls: int) -> int:
    """Bound of the Markov loop's grid-wide waits, in polls (0: the default);
    returns the previous setting (dspark_markov_set_spin_limit)."""
    return int(lib().dspark_markov_set_spin_limit(int(polls)))


def markov_sample_noalloc(base: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, prev0: torch.Tensor, k: int,
                          d2t: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """markov_sample with the library's static per-device workspace
    (dspark_markov_sample_noalloc). ``out`` int64 [R, k] must be given by a
    caller that may not allocate; it is allocated here otherwise."""
    _dev(base, torch.float32, "base", 3)
    _dev(w1, torch.bfloat16, "w1", 2)
    _dev(w2, torch.bfloat16, "w2", 2)
    _dev(prev0, torch.int64, "prev0", 1)
    R, B, V = base.shape
    r = w1.shape[1]
    if tuple(w1.shape) != (V, r) or tuple(w2.shape) != (V, r):
        raise ValueError("w1 and w2 must both be [V, r]")
    if prev0.shape[0] != R:
        raise ValueError("prev0 must have num_reqs entries")
    d2t_ptr = None
    if d2t is not None:
        _dev(d2t, torch.int64, "d2t", 1)
        if d2t.shape[0] != V:
            raise ValueError("d2t must have V entries")
        d2t_ptr = d2t.data_ptr()
    if out is None:
        out = torch.empty((R, k), dtype=torch.int64, device=base.device)
    if tuple(out.shape) != (R, k):
        raise ValueError("out must be [num_reqs, k]")
    out_ptr = _out_ptr(out, torch.int64, "out", 2)
    _check(lib().dspark_markov_sample_noalloc(base.data_ptr(), R, B, V, w1.data_ptr(), w2.data_ptr(), r, d2t_ptr,
                                              prev0.data_ptr(), k, out_ptr, _stream(base)))
    return out


def markov_sample(base: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, prev0: torch.Tensor, k: int,
                  d2t: torch.Tensor | None = None, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, probe: dict | None = None) -> torch.Tensor:
    """Drafted ids [R, k] int64 of the on-device Markov loop (dspark_markov_sample).

    base fp32 [R, B, V]; w1, w2 bf16 [V, r]; prev0 int64 [R]; d2t int64 [V] or None.
    ``probe``, when given, is a dict with the arguments of conf_probe (x, w,
    and optionally bias, threshold, logit_out, pass_out): the probe then runs
    in the same launch (dspark_markov_sample_probe) and its outputs are
    written to probe["logit_out"] and probe["pass_out"] (allocated here when
    absent).
    """
    _dev(base, torch.float32, "base", 3)
    _dev(w1, torch.bfloat16, "w1", 2)
    _dev(w2, torch.bfloat16, "w2", 2)
    _dev(prev0, torch.int64, "prev0", 1)
    R, B, V = base.shape
    r = w1.shape[1]
    if tuple(w1.shape) != (V, r) or tuple(w2.shape) != (V, r):
        raise ValueError("w1 and w2 must both be [V, r]")
    if prev0.shape[0] != R:
        raise ValueError("prev0 must have num_reqs entries")
    d2t_ptr = None
    if d2t is not None:
        _dev(d2t, torch.int64, "d2t", 1)
        if d2t.shape[0] != V:
            raise ValueError("d2t must have V entries")
        d2t_ptr = d2t.data_ptr()
    if out is None:
        out = torch.empty((R, k), dtype=torch.int64, device=base.device)
    if tuple(out.shape) != (R, k):
        raise ValueError("out must be [num_reqs, k]")
    out_ptr = _out_ptr(out, torch.int64, "out", 2)
    if workspace is None:
        workspace = markov_workspace(R, k, V, base.device)
    _dev(workspace, torch.uint8, "workspace", 1)
    if probe is None:
        _check(lib().dspark_markov_sample(base.data_ptr(), R, B, V, w1.data_ptr(), w2.data_ptr(), r, d2t_ptr,
                                          prev0.data_ptr(), k, out_ptr, workspace.data_ptr(),
                                          workspace.numel(), _stream(base)))
        return out
    x, pw = probe["x"], probe["w"]
    lo, pa, lo_ptr, pa_ptr = _probe_outputs(x, pw, probe.get("logit_out"), probe.get("pass_out"),
                                            probe.get("want_pass", True))
    probe["logit_out"], probe["pass_out"] = lo, pa
    _check(lib().dspark_markov_sample_probe(
        base.data_ptr(), R, B, V, w1.data_ptr(), w2.data_ptr(), r, d2t_ptr, prev0.data_ptr(), k, out_ptr,
        workspace.data_ptr(), workspace.numel(), x.data_ptr(), x.shape[0], x.shape[1], pw.data_ptr(),
        float(probe.get("bias", 0.0)), float(probe.get("threshold", 0.0)), lo_ptr, pa_ptr, _stream(base)))
    return out


def _probe_outputs(x, w, logit_out, pass_out, want_pass):
    _dev(x, torch.float32, "x", 2)
    _dev(w, torch.bfloat16, "w", 1)
    M, D = x.shape
    if w.shape[0] != D:
        raise ValueError("w must have D entries")
    if logit_out is None:
        logit_out = torch.empty(M, dtype=torch.float32, device=x.device)
    lo_ptr = _out_ptr(logit_out, torch.float32, "logit_out", 1)
    if pass_out is None and want_pass:
        pass_out = torch.empty(M, dtype=torch.int32, device=x.device)
    pa_ptr = None if pass_out is None else _out_ptr(pass_out, torch.int32, "pass_out", 1)
    if logit_out.shape[0] != M or (pass_out is not None and pass_out.shape[0] != M):
        raise ValueError("logit_out and pass_out must have M entries")
    return logit_out, pass_out, lo_ptr, pa_ptr


def conf_probe(x: torch.Tensor, w: torch.Tensor, bias: float = 0.0, threshold: float = 0.0,
               logit_out: torch.Tensor | None = None, pass_out: torch.Tensor | None = None,
               want_pass: bool = True):
    """(logit fp32 [M], pass int32 [M] or None) of the confidence probe (dspark_conf_probe)."""
    logit_out, pass_out, lo_ptr, pa_ptr = _probe_outputs(x, w, logit_out, pass_out, want_pass)
    M, D = x.shape
    _check(lib().dspark_conf_probe(x.data_ptr(), M, D, w.data_ptr(), float(bias), float(threshold),
                                   lo_ptr, pa_ptr, _stream(x)))
    return logit_out, pass_out


def draft_round(W_lm: torch.Tensor, H: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, prev0: torch.Tensor,
                B: int, k: int, probe_w: torch.Tensor | None = None, probe_bias: float = 0.0,
                probe_threshold: float = 0.0, d2t: torch.Tensor | None = None,
                base_out: torch.Tensor | None = None, ids_out: torch.Tensor | None = None,
                logit_out: torch.Tensor | None = None, pass_out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None, want_pass: bool = True) -> dict:
    """One draft round (dspark_draft_round): lm_head, Markov loop and, when
    probe_w is given, the probe on every row of H. Returns a dict with base
    fp32 [R, B, V], ids int64 [R, k], logit fp32 [R*B] and pass int32 [R*B]
    (the last two None without a probe).

    W_lm bf16 [V, d]; H fp32 [R*B, d]; w1, w2 bf16 [V, r]; prev0 int64 [R].
    """
    _dev(W_lm, torch.bfloat16, "W_lm", 2)
    _dev(H, torch.float32, "H", 2)
    _dev(w1, torch.bfloat16, "w1", 2)
    _dev(w2, torch.bfloat16, "w2", 2)
    _dev(prev0, torch.int64, "prev0", 1)
    V, d = W_lm.shape
    R = prev0.shape[0]
    r = w1.shape[1]
    if tuple(H.shape) != (R * B, d):
        raise ValueError("H must be [num_reqs * B, d]")
    if tuple(w1.shape) != (V, r) or tuple(w2.shape) != (V, r):
        raise ValueError("w1 and w2 must both be [V, r]")
    dev = H.device
    d2t_ptr = None
    if d2t is not None:
        _dev(d2t, torch.int64, "d2t", 1)
        if d2t.shape[0] != V:
            raise ValueError("d2t must have V entries")
        d2t_ptr = d2t.data_ptr()
    if base_out is None:
        base_out = torch.empty((R, B, V), dtype=torch.float32, device=dev)
    _dev(base_out, torch.float32, "base_out", 3)
    if tuple(base_out.shape) != (R, B, V):
        raise ValueError("base_out must be [num_reqs, B, V]")
    if ids_out is None:
        ids_out = torch.empty((R, k), dtype=torch.int64, device=dev)
    if tuple(ids_out.shape) != (R, k):
        raise ValueError("ids_out must be [num_reqs, k]")
    ids_ptr = _out_ptr(ids_out, torch.int64, "ids_out", 2)
    pw_ptr = lo_ptr = pa_ptr = None
    if probe_w is not None:
        if probe_w.shape[0] != d:
            raise ValueError("probe_w must have d entries")
        logit_out, pass_out, lo_ptr, pa_ptr = _probe_outputs(H, probe_w, logit_out, pass_out, want_pass)
        pw_ptr = probe_w.data_ptr()
    else:
        logit_out = pass_out = None
    if workspace is None:
        workspace = draft_round_workspace(R, B, k, V, d, dev)
    _dev(workspace, torch.uint8, "workspace", 1)
    _check(lib().dspark_draft_round(W_lm.data_ptr(), V, d, H.data_ptr(), R, B, w1.data_ptr(), w2.data_ptr(), r,
                                    d2t_ptr, prev0.data_ptr(), k, pw_ptr, float(probe_bias), float(probe_threshold),
                                    base_out.data_ptr(), ids_ptr, lo_ptr, pa_ptr, workspace.data_ptr(),
                                    workspace.numel(), _stream(H)))
    return dict(base=base_out, ids=ids_out, logit=logit_out, passed=pass_out)


def _q8_pair(q, d, V, r, name):
    _dev(q, torch.int8, name + "q", 2)
    _dev(d, torch.float16, name + "d", 2)
    if tuple(q.shape) != (V, r) or tuple(d.shape) != (V, r // 32):
        raise ValueError(f"{name}: quants [V, r] and scales [V, r / 32] required")


def markov_sample_q8(base: torch.Tensor, w1q: torch.Tensor, w1d: torch.Tensor, w2q: torch.Tensor,
                     w2d: torch.Tensor, prev0: torch.Tensor, k: int, d2t: torch.Tensor | None = None,
                     out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                     probe: dict | None = None) -> torch.Tensor:
    """Drafted ids [R, k] of the Markov loop over Q8_0 markov weights
    (dspark_markov_sample_q8): w1q, w2q int8 [V, r]; w1d, w2d float16
    [V, r / 32]. ``probe`` as in markov_sample (same launch)."""
    _dev(base, torch.float32, "base", 3)
    _dev(prev0, torch.int64, "prev0", 1)
    R, B, V = base.shape
    r = w1q.shape[1]
    _q8_pair(w1q, w1d, V, r, "w1")
    _q8_pair(w2q, w2d, V, r, "w2")
    if prev0.shape[0] != R:
        raise ValueError("prev0 must have num_reqs entries")
    d2t_ptr = None
    if d2t is not None:
        _dev(d2t, torch.int64, "d2t", 1)
        if d2t.shape[0] != V:
            raise ValueError("d2t must have V entries")
        d2t_ptr = d2t.data_ptr()
    if out is None:
        out = torch.empty((R, k), dtype=torch.int64, device=base.device)
    if tuple(out.shape) != (R, k):
        raise ValueError("out must be [num_reqs, k]")
    out_ptr = _out_ptr(out, torch.int64, "out", 2)
    if workspace is None:
        workspace = markov_workspace(R, k, V, base.device)
    _dev(workspace, torch.uint8, "workspace", 1)
    px = pw = lo_ptr = pa_ptr = None
    pm = pd = 0
    bias = thr = 0.0
    if probe is not None:
        x, w = probe["x"], probe["w"]
        lo, pa, lo_ptr, pa_ptr = _probe_outputs(x, w, probe.get("logit_out"), probe.get("pass_out"),
                                                probe.get("want_pass", True))
        probe["logit_out"], probe["pass_out"] = lo, pa
        px, pw, pm, pd = x.data_ptr(), w.data_ptr(), x.shape[0], x.shape[1]
        bias, thr = float(probe.get("bias", 0.0)), float(probe.get("threshold", 0.0))
    _check(lib().dspark_markov_sample_q8(base.data_ptr(), R, B, V, w1q.data_ptr(), w1d.data_ptr(), w2q.data_ptr(),
                                         w2d.data_ptr(), r, d2t_ptr, prev0.data_ptr(), k, out_ptr,
                                         workspace.data_ptr(), workspace.numel(), px, pm, pd, pw, bias, thr,
                                         lo_ptr, pa_ptr, _stream(base)))
    return out


def draft_round_q8(Wq: torch.Tensor, Wd: torch.Tensor, H: torch.Tensor, w1q: torch.Tensor, w1d: torch.Tensor,
                   w2q: torch.Tensor, w2d: torch.Tensor, prev0: torch.Tensor, B: int, k: int,
                   probe_w: torch.Tensor | None = None, probe_bias: float = 0.0, probe_threshold: float = 0.0,
                   d2t: torch.Tensor | None = None, base_out: torch.Tensor | None = None,
                   ids_out: torch.Tensor | None = None, logit_out: torch.Tensor | None = None,
                   pass_out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                   want_pass: bool = True) -> dict:
    """One draft round over Q8_0 weights (dspark_draft_round_q8); returns the
    dict of draft_round."""
    _dev(Wq, torch.int8, "Wq", 2)
    _dev(Wd, torch.float16, "Wd", 2)
    _dev(H, torch.float32, "H", 2)
    _dev(prev0, torch.int64, "prev0", 1)
    V, d = Wq.shape
    R = prev0.shape[0]
    r = w1q.shape[1]
    if Wd.shape[0] != V or not (d // 32 <= Wd.shape[1] <= d // 32 + 64) or tuple(H.shape) != (R * B, d):
        raise ValueError("Wq [V, d], Wd [V, ldd] (d / 32 <= ldd <= d / 32 + 64) and H [num_reqs * B, d] required")
    ldd = Wd.shape[1]
    _q8_pair(w1q, w1d, V, r, "w1")
    _q8_pair(w2q, w2d, V, r, "w2")
    dev = H.device
    d2t_ptr = None
    if d2t is not None:
        _dev(d2t, torch.int64, "d2t", 1)
        if d2t.shape[0] != V:
            raise ValueError("d2t must have V entries")
        d2t_ptr = d2t.data_ptr()
    if base_out is None:
        base_out = torch.empty((R, B, V), dtype=torch.float32, device=dev)
    _dev(base_out, torch.float32, "base_out", 3)
    if tuple(base_out.shape) != (R, B, V):
        raise ValueError("base_out must be [num_reqs, B, V]")
    if ids_out is None:
        ids_out = torch.empty((R, k), dtype=torch.int64, device=dev)
    if tuple(ids_out.shape) != (R, k):
        raise ValueError("ids_out must be [num_reqs, k]")
    ids_ptr = _out_ptr(ids_out, torch.int64, "ids_out", 2)
    pw_ptr = lo_ptr = pa_ptr = None
    if probe_w is not None:
        if probe_w.shape[0] != d:
            raise ValueError("probe_w must have d entries")
        logit_out, pass_out, lo_ptr, pa_ptr = _probe_outputs(H, probe_w, logit_out, pass_out, want_pass)
        pw_ptr = probe_w.data_ptr()
    else:
        logit_out = pass_out = None
    if workspace is None:
        workspace = markov_workspace(R, k, V, dev)
    _dev(workspace, torch.uint8, "workspace", 1)
    if ldd == d // 32:
        _check(lib().dspark_draft_round_q8(Wq.data_ptr(), Wd.data_ptr(), V, d, H.data_ptr(), R, B, w1q.data_ptr(),
                                           w1d.data_ptr(), w2q.data_ptr(), w2d.data_ptr(), r, d2t_ptr,
                                           prev0.data_ptr(), k, pw_ptr, float(probe_bias), float(probe_threshold),
                                           base_out.data_ptr(), ids_ptr, lo_ptr, pa_ptr, workspace.data_ptr(),
                                           workspace.numel(), _stream(H)))
    else:
        _check(lib().dspark_draft_round_q8_ld(Wq.data_ptr(), Wd.data_ptr(), ldd, V, d, H.data_ptr(), R, B,
                                              w1q.data_ptr(), w1d.data_ptr(), w2q.data_ptr(), w2d.data_ptr(), r,
                                              d2t_ptr, prev0.data_ptr(), k, pw_ptr, float(probe_bias),
                                              float(probe_threshold), base_out.data_ptr(), ids_ptr, lo_ptr, pa_ptr,
                                              workspace.data_ptr(), workspace.numel(), _stream(H)))
    return dict(base=base_out, ids=ids_out, logit=logit_out, passed=pass_out)


def bf16_from_bits(bits, device) -> torch.Tensor:
    """Upload numpy uint16 bf16 bit patterns as a torch.bfloat16 device tensor."""
    import numpy as np
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
