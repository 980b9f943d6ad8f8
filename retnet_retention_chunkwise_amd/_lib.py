"""ctypes binding of libretention (argument marshalling only).

Every computation runs in the HIP kernels of libretention.so; this module checks
torch tensors (device, dtype, shape, contiguity), passes their device pointers
and the current HIP stream through the C ABI, and turns a non-zero status into
an exception.  There is no CPU fallback: without the built library every call
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple, Union

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libretention.so")

RET_F32, RET_BF16 = 0, 1
RET_OK, RET_ERR_INVALID_ARG, RET_ERR_UNSUPPORTED, RET_ERR_HIP = 0, 1, 2, 3
MAX_DK, MAX_DV, MAX_CHUNK = 256, 512, 128

# (name, restype, argtypes) of every symbol include/libretention.h declares
_vp, _fp, _i, _sz = ctypes.c_void_p, ctypes.POINTER(ctypes.c_float), ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "retention_parallel_fwd": (_i, [_vp, _vp, _vp, _fp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]),
    "retention_chunkwise_fwd": (_i, [_vp, _vp, _vp, _fp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "retention_chunkwise_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "retention_chunkwise_fwd_group_norm": (_i, [_vp, _vp, _vp, _fp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _i, _i,
                                                _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "retention_chunkwise_fwd_group_norm_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "retention_testing_gn_wait": (_i, [_i, _i]),
    "retention_chunkwise_fwd_noalloc": (_i, [_vp, _vp, _vp, _fp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "retention_recurrent_step": (_i, [_vp, _vp, _vp, _fp, _vp, _vp, _i, _i, _i, _i, _i, _vp]),
    "retention_group_norm": (_i, [_vp, _vp, _vp, ctypes.c_float, _vp, _i, _i, _i, _i, _i, _vp]),
    "retention_chunkwise_bwd": (_i, [_vp, _vp, _vp, _fp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i,
                                     _i, _vp, _sz, _vp]),
    "retention_chunkwise_bwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "retention_last_error": (ctypes.c_char_p, []),
    "retention_version": (_i, []),
}


class RetentionError(RuntimeError):
    """A libretention call returned a non-zero status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"[status {status}] {message}")
        self.status = status


_lib = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libretention.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"libretention is not built ({p} missing); run `python -m retnet_retention_chunkwise_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def last_error() -> str:
    return load().retention_last_error().decode()


def version() -> int:
    return int(load().retention_version())


def _check(status: int):
    if status != RET_OK:
        raise RetentionError(status, last_error())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return RET_F32
    if t.dtype == torch.bfloat16:
        return RET_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (cuda/HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _gamma_array(gamma: Union[Sequence[float], torch.Tensor], H: int):
    if isinstance(gamma, torch.Tensor):
        vals = gamma.detach().to("cpu", torch.float32).reshape(-1).tolist()
    else:
        vals = [float(g) for g in gamma]
    if len(vals) != H:
        raise ValueError(f"gamma has {len(vals)} entries, expected H={H}")
    return (ctypes.c_float * H)(*vals)


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _out_check(t: torch.Tensor, shape, dtype, device, name):
    """A caller-supplied output: shape and dtype first (a kernel writes exactly
    that many elements of that size), then device and contiguity."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
    _dev(t, name)
    if t.device != device:
        raise ValueError(f"{name} must be on {device}")


def _state_check(s: Optional[torch.Tensor], shape, device, name):
    if s is None:
        return
    _dev(s, name)
    if s.dtype != torch.float32 or tuple(s.shape) != tuple(shape) or s.device != device:
        raise ValueError(f"{name} must be float32 {tuple(shape)} on {device}")


def _qkv_shapes(q, k, v):
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("expected q, k [B,H,T,dk] and v [B,H,T,dv]")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    B, H, T, dk = q.shape
    return B, H, T, dk, v.shape[-1], _dt(q)


def _qkv_devices(q, k, v):
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must share a device")


def _qkv(q, k, v):
    dims = _qkv_shapes(q, k, v)
    _qkv_devices(q, k, v)
    return dims


def chunkwise_workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, C: int, dtype: torch.dtype) -> int:
    dt = RET_BF16 if dtype == torch.bfloat16 else RET_F32
    n = int(load().retention_chunkwise_workspace_bytes(B, H, T, dk, dv, C, dt))
    if n == ctypes.c_size_t(-1).value:
        raise RetentionError(RET_ERR_INVALID_ARG, "arguments rejected by retention_chunkwise_workspace_bytes")
    return n


def chunkwise_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gamma, C: int,
                  state_in: Optional[torch.Tensor] = None, state_out: Union[torch.Tensor, bool, None] = True,
                  y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None
                  ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise retention forward on the GPU (retention_chunkwise_fwd).

    q, k [B,H,T,dk]; v [B,H,T,dv] (float32 or bfloat16, contiguous, on the GPU);
    gamma: H decays in [0, 1]; C: chunk length.  state_in: optional fp32
    [B,H,dk,dv].  state_out: a tensor to fill, True to allocate one, or
    False/None for none (may be the same tensor as state_in).
    Returns (y, state_out).
    """
    lib = load()
    B, H, T, dk, dv, dt = _qkv_shapes(q, k, v)
    if y is not None:
        _out_check(y, (B, H, T, dv), q.dtype, q.device, "y")
    _qkv_devices(q, k, v)
    sshape = (B, H, dk, dv)
    _state_check(state_in, sshape, q.device, "state_in")
    if state_out is True:
        state_out = torch.empty(sshape, dtype=torch.float32, device=q.device)
    elif state_out is False:
        state_out = None
    _state_check(state_out, sshape, q.device, "state_out")
    if y is None:
        y = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    need = int(lib.retention_chunkwise_workspace_bytes(B, H, T, dk, dv, int(C), dt))
    ws_bytes = 0
    if need and need != ctypes.c_size_t(-1).value:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_bytes = workspace.numel() * workspace.element_size()
    elif workspace is not None:
        ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.retention_chunkwise_fwd(_ptr(q), _ptr(k), _ptr(v), _gamma_array(gamma, H), _ptr(state_in),
                                     _ptr(state_out), _ptr(y), B, H, T, dk, dv, int(C), dt, _ptr(workspace),
                                     ws_bytes, _stream(q.device))
    _check(st)
    return y, state_out


def chunkwise_fwd_group_norm(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gamma, C: int,
                             weight: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
                             eps: float = 1e-5, state_in: Optional[torch.Tensor] = None,
                             state_out: Union[torch.Tensor, bool, None] = True, y: Optional[torch.Tensor] = None,
                             workspace: Optional[torch.Tensor] = None, check: bool = False
                             ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """The chunkwise forward with the per-head GroupNorm of its output fused in
    (retention_chunkwise_fwd_group_norm): y = group_norm(chunkwise_fwd(...)).
    weight, bias: optional fp32 [H,dv].  Returns (y, state_out).

    The fused kernel reports a wait that gave up (the column tiles of a head
    not all resident at once; y is then wrong) in the workspace's first 32-bit
    word: pass a workspace and read it with fused_group_norm_failed(), or pass
    check=True to wait for the call here and raise RuntimeError if it is set."""
    lib = load()
    B, H, T, dk, dv, dt = _qkv_shapes(q, k, v)
    if y is not None:
        _out_check(y, (B, H, T, dv), q.dtype, q.device, "y")
    _qkv_devices(q, k, v)
    sshape = (B, H, dk, dv)
    _state_check(state_in, sshape, q.device, "state_in")
    if state_out is True:
        state_out = torch.empty(sshape, dtype=torch.float32, device=q.device)
    elif state_out is False:
        state_out = None
    _state_check(state_out, sshape, q.device, "state_out")
    for t, n in ((weight, "weight"), (bias, "bias")):
        if t is not None:
            _dev(t, n)
            if t.dtype != torch.float32 or tuple(t.shape) != (H, dv) or t.device != q.device:
                raise ValueError(f"{n} must be float32 ({H}, {dv}) on {q.device}")
    if y is None:
        y = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    need = int(lib.retention_chunkwise_fwd_group_norm_workspace_bytes(B, H, T, dk, dv, int(C), dt))
    ws_bytes = 0
    if need and need != ctypes.c_size_t(-1).value:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_bytes = workspace.numel() * workspace.element_size()
    elif workspace is not None:
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.retention_chunkwise_fwd_group_norm(_ptr(q), _ptr(k), _ptr(v), _gamma_array(gamma, H), _ptr(state_in),
                                                  _ptr(state_out), _ptr(weight), _ptr(bias), float(eps), _ptr(y), B,
                                                  H, T, dk, dv, int(C), dt, _ptr(workspace), ws_bytes,
                                                  _stream(q.device)))
    if check and fused_group_norm_failed(workspace, B, H, T, dk, dv, C, q.dtype):
        raise RuntimeError("retention_chunkwise_fwd_group_norm: a workgroup gave up waiting for the statistics "
                           "of another column tile (the tiles of a head were not all resident); y is wrong")
    return y, state_out


def fused_group_norm_failed(workspace: Optional[torch.Tensor], B: int, H: int, T: int, dk: int, dv: int, C: int,
                            dtype: torch.dtype) -> bool:
    """Whether the last chunkwise_fwd_group_norm call with this workspace and
    shape ran the fused kernel and one of its waits gave up (error word 1).
    Waits for the current stream (it reads the word back)."""
    lib = load()
    dt = RET_BF16 if dtype == torch.bfloat16 else RET_F32
    need = int(lib.retention_chunkwise_fwd_group_norm_workspace_bytes(B, H, T, dk, dv, int(C), dt))
    plain = int(lib.retention_chunkwise_workspace_bytes(B, H, T, dk, dv, int(C), dt))
    if workspace is None or need == plain or need == ctypes.c_size_t(-1).value:
        return False  # the forward and the standalone GroupNorm: no error word
    return int(workspace[:4].view(torch.int32).item()) != 0


def testing_gn_wait(spin_limit: int = 1 << 16, silent_tile: int = -1) -> None:
    """retention_testing_gn_wait: failure-path testing of the fused GroupNorm
    (poll limit of its waits; a column tile that publishes no statistics).
    The defaults restore normal operation."""
    _check(load().retention_testing_gn_wait(int(spin_limit), int(silent_tile)))


def chunkwise_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gamma, C: int,
                          state_in: Optional[torch.Tensor] = None, state_out: Optional[torch.Tensor] = None,
                          y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """retention_chunkwise_fwd_noalloc: chunkwise_fwd with the workspace of
    segmented calls in the library's static device scratch, so that the call
    itself allocates nothing (pass y and, if wanted, state_out preallocated).
    Calls that overlap in time on one GPU race on that scratch.  Returns y."""
    lib = load()
    B, H, T, dk, dv, dt = _qkv_shapes(q, k, v)
    if y is not None:
        _out_check(y, (B, H, T, dv), q.dtype, q.device, "y")
    _qkv_devices(q, k, v)
    sshape = (B, H, dk, dv)
    _state_check(state_in, sshape, q.device, "state_in")
    _state_check(state_out, sshape, q.device, "state_out")
    if y is None:
        y = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    _check(lib.retention_chunkwise_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _gamma_array(gamma, H), _ptr(state_in),
                                               _ptr(state_out), _ptr(y), B, H, T, dk, dv, int(C), dt,
                                               _stream(q.device)))
    return y


def chunkwise_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gamma, C: int, grad_y: torch.Tensor,
                  state_in: Optional[torch.Tensor] = None, grad_state_out: Optional[torch.Tensor] = None,
                  grad_state_in: Union[torch.Tensor, bool, None] = True, workspace: Optional[torch.Tensor] = None
                  ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor, Optional[torch.Tensor]]:
    """Gradients of chunkwise_fwd on the GPU (retention_chunkwise_bwd).

    q, k, v, gamma, C, state_in: the forward call's arguments.  grad_y: [B,H,T,dv]
    in the input dtype; grad_state_out: optional fp32 [B,H,dk,dv].
    grad_state_in: a tensor to fill (may be grad_state_out), True to allocate
    one, or False/None for none.  workspace: device scratch (allocated here when
    the call needs one and none is given).  Returns (grad_q, grad_k, grad_v,
    grad_state_in).
    """
    lib = load()
    B, H, T, dk, dv, dt = _qkv(q, k, v)
    _dev(grad_y, "grad_y")
    if grad_y.shape != v.shape or grad_y.dtype != v.dtype or grad_y.device != v.device:
        raise ValueError("grad_y must match v in shape, dtype and device")
    sshape = (B, H, dk, dv)
    _state_check(state_in, sshape, q.device, "state_in")
    _state_check(grad_state_out, sshape, q.device, "grad_state_out")
    if grad_state_in is True:
        grad_state_in = torch.empty(sshape, dtype=torch.float32, device=q.device)
    elif grad_state_in is False:
        grad_state_in = None
    _state_check(grad_state_in, sshape, q.device, "grad_state_in")
    gq = torch.empty_like(q)
    gk = torch.empty_like(k)
    gv = torch.empty_like(v)
    need = int(lib.retention_chunkwise_bwd_workspace_bytes(B, H, T, dk, dv, int(C), dt))
    ws_bytes = 0
    if need and need != ctypes.c_size_t(-1).value:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_bytes = workspace.numel() * workspace.element_size()
    elif workspace is not None:
        ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.retention_chunkwise_bwd(_ptr(q), _ptr(k), _ptr(v), _gamma_array(gamma, H), _ptr(state_in),
                                     _ptr(grad_y), _ptr(grad_state_out), _ptr(gq), _ptr(gk), _ptr(gv),
                                     _ptr(grad_state_in), B, H, T, dk, dv, int(C), dt, _ptr(workspace), ws_bytes,
                                     _stream(q.device))
    _check(st)
    return gq, gk, gv, grad_state_in


def group_norm(y: torch.Tensor, weight: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
               eps: float = 1e-5, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-head GroupNorm of a [B,H,T,dv] retention output (retention_group_norm).

    weight, bias: optional fp32 [H,dv] device tensors.  out: a tensor to fill
    (may be y itself), or None to allocate one.
    """
    lib = load()
    _dev(y, "y")
    if y.dim() != 4:
        raise ValueError("expected y [B,H,T,dv]")
    B, H, T, dv = y.shape
    dt = _dt(y)
    for t, n in ((weight, "weight"), (bias, "bias")):
        if t is not None:
            _dev(t, n)
            if t.dtype != torch.float32 or tuple(t.shape) != (H, dv) or t.device != y.device:
                raise ValueError(f"{n} must be float32 ({H}, {dv}) on {y.device}")
    if out is None:
        out = torch.empty_like(y)
    else:
        _dev(out, "out")
        if out.shape != y.shape or out.dtype != y.dtype or out.device != y.device:
            raise ValueError("out must match y")
    _check(lib.retention_group_norm(_ptr(y), _ptr(weight), _ptr(bias), float(eps), _ptr(out), B, H, T, dv, dt,
                                    _stream(y.device)))
    return out


def parallel_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gamma,
                 state_in: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Parallel-form retention forward on the GPU (retention_parallel_fwd)."""
    lib = load()
    B, H, T, dk, dv, dt = _qkv_shapes(q, k, v)
    if y is not None:
        _out_check(y, (B, H, T, dv), q.dtype, q.device, "y")
    _qkv_devices(q, k, v)
    _state_check(state_in, (B, H, dk, dv), q.device, "state_in")
    if y is None:
        y = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    st = lib.retention_parallel_fwd(_ptr(q), _ptr(k), _ptr(v), _gamma_array(gamma, H), _ptr(state_in), _ptr(y),
                                    B, H, T, dk, dv, dt, _stream(q.device))
    _check(st)
    return y


def recurrent_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gamma, state: torch.Tensor,
                   y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode step on the GPU (retention_recurrent_step): state <- gamma*state + k^T v
    in place, returns y = q state.  q, k [B,H,dk]; v [B,H,dv]; state fp32 [B,H,dk,dv]."""
    lib = load()
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[:2] != q.shape[:2]:
        raise ValueError("expected q, k [B,H,dk] and v [B,H,dv]")
    B, H, dk = q.shape
    dv = v.shape[-1]
    dt = _dt(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    if y is not None:
        _out_check(y, (B, H, dv), q.dtype, q.device, "y")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must share a device")
    _state_check(state, (B, H, dk, dv), q.device, "state")
    if y is None:
        y = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
    st = lib.retention_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _gamma_array(gamma, H), _ptr(state), _ptr(y),
                                      B, H, dk, dv, dt, _stream(q.device))
    _check(st)
    return y
