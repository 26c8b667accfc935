"""MI355X (gfx950) In-Place Activated BatchNorm.

A thin ctypes binding of libiabn.so, whose C ABI is declared in include/iabn.h.
Every function here only marshals arguments -- torch tensors become device
pointers, the stream defaults to torch's current stream -- and calls the entry
point of the same name; all computation happens in the library's HIP kernels.
PyTorch provides device memory and streams only.

The library must be built (``__graft_entry__.build()`` or
``python place_batchnorm_activation_amd/build.py``); importing this package
without it raises ImportError.  There is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # loaded first: the library then binds to torch's HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libiabn.so")

NCHW, NHWC = 0, 1
F32, BF16, F16 = 0, 1, 2
ACT_IDENTITY, ACT_LEAKY_RELU, ACT_ELU = 0, 1, 2

LAYOUTS = {"NCHW": NCHW, "NHWC": NHWC}
ACTS = {"identity": ACT_IDENTITY, "leaky_relu": ACT_LEAKY_RELU, "elu": ACT_ELU}
STATUS = {0: "IABN_OK", 1: "IABN_ERR_INVALID_ARG", 2: "IABN_ERR_UNSUPPORTED",
          3: "IABN_ERR_WORKSPACE", 4: "IABN_ERR_MISALIGNED", 5: "IABN_ERR_HIP"}

if not os.path.exists(LIB_PATH):
    raise ImportError("libiabn.so is not built (expected at %s); run __graft_entry__.build()"
                      % LIB_PATH)

lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_F = ctypes.c_float
_INT = ctypes.c_int
_SZ = ctypes.c_size_t

lib.iabn_status_string.argtypes = [_INT]
lib.iabn_status_string.restype = ctypes.c_char_p
lib.iabn_version.argtypes = []
lib.iabn_version.restype = _INT
lib.iabn_workspace_size.argtypes = [_I64, _I64, _I64, _I64, _INT, _INT]
lib.iabn_workspace_size.restype = _SZ
_SHAPE = [_I64, _I64, _I64, _I64, _INT, _INT]
lib.iabn_forward_train.argtypes = [_P] + _SHAPE + [_P, _P, _P, _P, _P, _P, _INT, _F, _F, _F, _P,
                                                   _SZ, _P]
lib.iabn_forward_train_noalloc.argtypes = [_P] + _SHAPE + [_P, _P, _P, _P, _P, _P, _INT, _F, _F,
                                                           _F, _P]
lib.iabn_forward_stats.argtypes = [_P] + _SHAPE + [_P, _P, _P, _P, _P, _P, _F, _F, _P, _SZ, _P]
lib.iabn_forward_apply.argtypes = [_P] + _SHAPE + [_INT, _F, _P, _SZ, _P]
lib.iabn_forward_eval.argtypes = [_P] + _SHAPE + [_P, _P, _P, _P, _INT, _F, _F, _P]
lib.iabn_backward.argtypes = [_P, _P, _P] + _SHAPE + [_P, _P, _P, _P, _P, _INT, _F, _P, _SZ, _P]
lib.iabn_backward_reduce.argtypes = [_P, _P] + _SHAPE + [_P, _P, _P, _P, _P, _INT, _F, _P, _SZ,
                                                         _P]
lib.iabn_backward_apply.argtypes = [_P, _P, _P] + _SHAPE + [_INT, _F, _P, _SZ, _P]
lib.iabn_backward_eval.argtypes = [_P, _P, _P] + _SHAPE + [_P, _P, _P, _F, _P, _P, _INT, _F, _P,
                                                           _SZ, _P]
lib.iabn_set_grouped_kernels.argtypes = [_INT]
lib.iabn_set_grouped_kernels.restype = _INT
lib.iabn_workspace_status.argtypes = [_P, _SZ, _INT, ctypes.POINTER(_INT), _P]
lib.iabn_workspace_status.restype = _INT
lib.iabn_forward_train_ckpt.argtypes = [_P, _P] + _SHAPE + [_P, _P, _P, _P, _P, _P, _INT, _F, _F,
                                                            _F, _P, _SZ, _P]
lib.iabn_recompute_from_xhat.argtypes = [_P, _P] + _SHAPE + [_P, _P, _INT, _F, _P]
lib.iabn_backward_ckpt.argtypes = [_P, _P, _P] + _SHAPE + [_P, _P, _P, _P, _P, _INT, _F, _P, _SZ,
                                                           _P]
lib.iabn_describe_plan.argtypes = _SHAPE + [_INT, _INT, ctypes.c_char_p, _SZ]
lib.iabn_describe_plan.restype = _INT
for _fn in ("iabn_forward_train", "iabn_forward_train_noalloc", "iabn_forward_train_ckpt",
            "iabn_recompute_from_xhat", "iabn_backward_ckpt", "iabn_forward_stats",
            "iabn_forward_apply", "iabn_forward_eval", "iabn_backward", "iabn_backward_reduce",
            "iabn_backward_apply", "iabn_backward_eval"):
    getattr(lib, _fn).restype = _INT


class IABNError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s returned %s (%s)" % (fn, STATUS.get(status, status),
                                                  lib.iabn_status_string(status).decode()))


def _ptr(t) -> Optional[int]:
    """Tensor -> device address; None -> NULL; an int is taken as an address."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _vec(t) -> Optional[int]:
    """A per-channel vector (gamma, beta, statistics, gradients) -> device address:
    the library reads and writes them as float32, so any other dtype is refused
    (its bytes would be misread)."""
    if t is None or isinstance(t, int):
        return t
    if t.dtype != torch.float32:
        raise TypeError("per-channel vectors are float32, got %s" % t.dtype)
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


_TORCH_DTYPES = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}


def _dtype_code(t) -> int:
    code = _TORCH_DTYPES.get(t.dtype)
    if code is None:
        raise TypeError("storage dtype must be float32, bfloat16 or float16, got %s" % t.dtype)
    return code


def _dtype_arg(dtype) -> int:
    """A storage dtype given as a torch dtype or as the library's code."""
    if isinstance(dtype, torch.dtype):
        if dtype not in _TORCH_DTYPES:
            raise TypeError("storage dtype must be float32, bfloat16 or float16, got %s" % dtype)
        return _TORCH_DTYPES[dtype]
    return int(dtype)


def _code(v, table):
    return table[v] if isinstance(v, str) else int(v)


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise IABNError(fn, status)


def status_string(status: int) -> str:
    return lib.iabn_status_string(status).decode()


def iabn_version() -> int:
    return lib.iabn_version()


class ExchangeTimeout(RuntimeError):
    """A kernel whose workgroups exchange partial sums gave up waiting for a
    partner: the outputs of the calls since the workspace was last checked may
    hold NaN."""


def iabn_set_grouped_kernels(enabled: Optional[bool] = None) -> bool:
    """Allow (True) or forbid (False) the kernels whose workgroups wait on one
    another, process-wide; None only reads the setting.  Returns the previous
    setting."""
    return bool(lib.iabn_set_grouped_kernels(-1 if enabled is None else int(bool(enabled))))


def iabn_workspace_status(ws, clear: bool = True, stream=None) -> bool:
    """Whether a wait of an exchanging kernel ran out on this workspace since the
    word was last cleared (synchronises the stream)."""
    flag = _INT(0)
    _check("iabn_workspace_status",
           lib.iabn_workspace_status(_ptr(ws), ws.numel() * ws.element_size(), int(clear),
                                     ctypes.byref(flag), _stream(stream)))
    return bool(flag.value)


def check_workspace(ws, stream=None) -> None:
    """Raise ExchangeTimeout if an exchanging kernel timed out on this workspace
    (reads and clears the word; synchronises the stream)."""
    if iabn_workspace_status(ws, True, stream):
        raise ExchangeTimeout("a grouped kernel gave up waiting for a partner workgroup; "
                              "outputs since the last check may hold NaN "
                              "(iabn_set_grouped_kernels(False) avoids these kernels)")


def iabn_workspace_size(N, C, H, W, layout, dtype) -> int:
    """dtype: F32/BF16/F16 code or a torch dtype."""
    return lib.iabn_workspace_size(N, C, H, W, _code(layout, LAYOUTS), _dtype_arg(dtype))


def workspace(N, C, H, W, layout, dtype, device="cuda") -> torch.Tensor:
    """A workspace tensor of the size the library asks for (at least its 256-byte
    header)."""
    n = max(256, iabn_workspace_size(N, C, H, W, layout, dtype))
    return torch.empty(n, dtype=torch.uint8, device=device)


def _ws(ws):
    return (None, 0) if ws is None else (ws.data_ptr(), ws.numel() * ws.element_size())


def iabn_forward_train(x, N, C, H, W, layout, gamma, beta, running_mean, running_var, save_mean,
                       save_invstd, act, act_param, eps, momentum, workspace, stream=None):
    wp, wb = _ws(workspace)
    _check("iabn_forward_train", lib.iabn_forward_train(
        _ptr(x), N, C, H, W, _code(layout, LAYOUTS), _dtype_code(x), _vec(gamma), _vec(beta),
        _vec(running_mean), _vec(running_var), _vec(save_mean), _vec(save_invstd),
        _code(act, ACTS), act_param, eps, momentum, wp, wb, _stream(stream)))


def iabn_forward_train_noalloc(x, N, C, H, W, layout, gamma, beta, running_mean, running_var,
                               save_mean, save_invstd, act, act_param, eps, momentum, stream=None):
    """iabn_forward_train with the library's static per-device scratch as workspace
    (no allocation; shapes within IABN_NOALLOC_SCRATCH_BYTES of workspace)."""
    _check("iabn_forward_train_noalloc", lib.iabn_forward_train_noalloc(
        _ptr(x), N, C, H, W, _code(layout, LAYOUTS), _dtype_code(x), _vec(gamma), _vec(beta),
        _vec(running_mean), _vec(running_var), _vec(save_mean), _vec(save_invstd),
        _code(act, ACTS), act_param, eps, momentum, _stream(stream)))


NOALLOC_SCRATCH_BYTES = 8 << 20


def iabn_forward_stats(x, N, C, H, W, layout, gamma, beta, running_mean, running_var, save_mean,
                       save_invstd, eps, momentum, workspace, stream=None):
    wp, wb = _ws(workspace)
    _check("iabn_forward_stats", lib.iabn_forward_stats(
        _ptr(x), N, C, H, W, _code(layout, LAYOUTS), _dtype_code(x), _vec(gamma), _vec(beta),
        _vec(running_mean), _vec(running_var), _vec(save_mean), _vec(save_invstd), eps,
        momentum, wp, wb, _stream(stream)))


def iabn_forward_apply(x, N, C, H, W, layout, act, act_param, workspace, stream=None):
    wp, wb = _ws(workspace)
    _check("iabn_forward_apply", lib.iabn_forward_apply(
        _ptr(x), N, C, H, W, _code(layout, LAYOUTS), _dtype_code(x), _code(act, ACTS), act_param,
        wp, wb, _stream(stream)))


def iabn_forward_eval(x, N, C, H, W, layout, gamma, beta, running_mean, running_var, act,
                      act_param, eps, stream=None):
    _check("iabn_forward_eval", lib.iabn_forward_eval(
        _ptr(x), N, C, H, W, _code(layout, LAYOUTS), _dtype_code(x), _vec(gamma), _vec(beta),
        _vec(running_mean), _vec(running_var), _code(act, ACTS), act_param, eps,
        _stream(stream)))


def iabn_backward(y, dy, dx, N, C, H, W, layout, gamma, beta, save_invstd, dgamma, dbeta, act,
                  act_param, workspace, stream=None):
    wp, wb = _ws(workspace)
    _check("iabn_backward", lib.iabn_backward(
        _ptr(y), _ptr(dy), _ptr(dx), N, C, H, W, _code(layout, LAYOUTS), _dtype_code(y),
        _vec(gamma), _vec(beta), _vec(save_invstd), _vec(dgamma), _vec(dbeta), _code(act, ACTS),
        act_param, wp, wb, _stream(stream)))


def iabn_backward_reduce(y, dy, N, C, H, W, layout, gamma, beta, save_invstd, dgamma, dbeta, act,
                         act_param, workspace, stream=None):
    wp, wb = _ws(workspace)
    _check("iabn_backward_reduce", lib.iabn_backward_reduce(
        _ptr(y), _ptr(dy), N, C, H, W, _code(layout, LAYOUTS), _dtype_code(y), _vec(gamma),
        _vec(beta), _vec(save_invstd), _vec(dgamma), _vec(dbeta), _code(act, ACTS), act_param,
        wp, wb, _stream(stream)))


def iabn_backward_apply(y, dy, dx, N, C, H, W, layout, act, act_param, workspace, stream=None):
    wp, wb = _ws(workspace)
    _check("iabn_backward_apply", lib.iabn_backward_apply(
        _ptr(y), _ptr(dy), _ptr(dx), N, C, H, W, _code(layout, LAYOUTS), _dtype_code(y),
        _code(act, ACTS), act_param, wp, wb, _stream(stream)))


def iabn_backward_eval(y, dy, dx, N, C, H, W, layout, gamma, beta, running_var, eps, dgamma,
                       dbeta, act, act_param, workspace, stream=None):
    wp, wb = _ws(workspace)
    _check("iabn_backward_eval", lib.iabn_backward_eval(
        _ptr(y), _ptr(dy), _ptr(dx), N, C, H, W, _code(layout, LAYOUTS), _dtype_code(y),
        _vec(gamma), _vec(beta), _vec(running_var), eps, _vec(dgamma), _vec(dbeta),
        _code(act, ACTS), act_param, wp, wb, _stream(stream)))


def iabn_forward_train_ckpt(x, y, N, C, H, W, layout, gamma, beta, running_mean, running_var,
                            save_mean, save_invstd, act, act_param, eps, momentum, workspace,
                            stream=None):
    """Optimized checkpointing forward: xhat written over x, the layer output into y."""
    wp, wb = _ws(workspace)
    _check("iabn_forward_train_ckpt", lib.iabn_forward_train_ckpt(
        _ptr(x), _ptr(y), N, C, H, W, _code(layout, LAYOUTS), _dtype_code(x), _vec(gamma),
        _vec(beta), _vec(running_mean), _vec(running_var), _vec(save_mean), _vec(save_invstd),
        _code(act, ACTS), act_param, eps, momentum, wp, wb, _stream(stream)))


def iabn_recompute_from_xhat(xhat, y, N, C, H, W, layout, gamma, beta, act, act_param,
                             stream=None):
    _check("iabn_recompute_from_xhat", lib.iabn_recompute_from_xhat(
        _ptr(xhat), _ptr(y), N, C, H, W, _code(layout, LAYOUTS), _dtype_code(xhat), _vec(gamma),
        _vec(beta), _code(act, ACTS), act_param, _stream(stream)))


def iabn_backward_ckpt(xhat, dy, dx, N, C, H, W, layout, gamma, beta, save_invstd, dgamma, dbeta,
                       act, act_param, workspace, stream=None):
    wp, wb = _ws(workspace)
    _check("iabn_backward_ckpt", lib.iabn_backward_ckpt(
        _ptr(xhat), _ptr(dy), _ptr(dx), N, C, H, W, _code(layout, LAYOUTS), _dtype_code(xhat),
        _vec(gamma), _vec(beta), _vec(save_invstd), _vec(dgamma), _vec(dbeta), _code(act, ACTS),
        act_param, wp, wb, _stream(stream)))


def iabn_describe_plan(N, C, H, W, layout, dtype, act, aligned16=True) -> str:
    """Which kernels iabn_forward_train / iabn_backward launch for this problem."""
    buf = ctypes.create_string_buffer(256)
    n = lib.iabn_describe_plan(N, C, H, W, _code(layout, LAYOUTS), _dtype_arg(dtype),
                               _code(act, ACTS),
                               1 if aligned16 else 0, buf, 256)
    if n < 0:
        raise ValueError("invalid problem description")
    return buf.value.decode()


def shape_of(t: torch.Tensor, layout) -> tuple:
    """(N, C, H, W) of a contiguous 4-d storage tensor: [N,C,H,W] for NCHW,
    [N,H,W,C] for NHWC."""
    if _code(layout, LAYOUTS) == NCHW:
        N, C, H, W = t.shape
    else:
        N, H, W, C = t.shape
    return int(N), int(C), int(H), int(W)
