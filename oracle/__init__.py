"""fp64 CPU oracle for In-Place Activated BatchNorm -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU baseline may import this
package.  It wraps oracle/liboracle.so (plain C, built from iabn_oracle.c) with
ctypes.  Arrays are numpy float64 in logical NCHW order; per-channel vectors are
float64 of length C.  Nothing here shares code with the HIP library.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

from . import build as _build

ACT = {"identity": 0, "leaky_relu": 1, "elu": 2}
STORE = {"f64": 0, "f32": 1, "bf16": 2, "f16": 3}

_lib = None
_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.c_int64


_lib_path = None


def use_library(path: Optional[str]) -> None:
    """Point the wrapper at another build of iabn_oracle.c (None: the default).
    Used by the mutation test, which plants mistakes in copies of the source."""
    global _lib, _lib_path
    _lib, _lib_path = None, path


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = _lib_path or _build.LIB
    if _lib_path is None and not os.path.exists(path):
        _build.build()
    lib = ctypes.CDLL(path)
    lib.orc_forward_train.argtypes = [_I64, _I64, _I64, _D, _D, _D, ctypes.c_int, ctypes.c_double,
                                      ctypes.c_double, ctypes.c_double, _D, _D, _D, _D, _D, _D]
    lib.orc_forward_eval.argtypes = [_I64, _I64, _I64, _D, _D, _D, _D, _D, ctypes.c_int,
                                     ctypes.c_double, ctypes.c_double, _D]
    lib.orc_backward_from_y.argtypes = [_I64, _I64, _I64, _D, _D, _D, _D, _D, ctypes.c_int,
                                        ctypes.c_double, _D, _D, _D, _D]
    lib.orc_backward_eval.argtypes = [_I64, _I64, _I64, _D, _D, _D, _D, _D, ctypes.c_double,
                                      ctypes.c_int, ctypes.c_double, _D, _D, _D]
    lib.orc_backward_from_y_form2.argtypes = [_I64, _I64, _I64, _D, _D, _D, _D, _D, ctypes.c_int,
                                              ctypes.c_double, _D, _D, _D]
    lib.orc_backward_from_x.argtypes = [_I64, _I64, _I64, _D, _D, _D, _D, ctypes.c_int,
                                        ctypes.c_double, ctypes.c_double, _D, _D, _D]
    lib.orc_forward_train_ckpt.argtypes = [_I64, _I64, _I64, _D, _D, _D, ctypes.c_int,
                                           ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                           _D, _D, _D, _D, _D, _D, _D]
    lib.orc_recompute_from_xhat.argtypes = [_I64, _I64, _I64, _D, _D, _D, ctypes.c_int,
                                            ctypes.c_double, _D]
    lib.orc_backward_from_xhat.argtypes = [_I64, _I64, _I64, _D, _D, _D, _D, _D, ctypes.c_int,
                                           ctypes.c_double, _D, _D, _D]
    lib.orc_round_storage.argtypes = [_D, _I64, ctypes.c_int]
    lib.orc_num_threads.argtypes = []
    for f in (lib.orc_forward_train, lib.orc_forward_eval, lib.orc_backward_from_y,
              lib.orc_backward_eval, lib.orc_backward_from_y_form2, lib.orc_backward_from_x, lib.orc_round_storage,
              lib.orc_num_threads, lib.orc_forward_train_ckpt, lib.orc_recompute_from_xhat,
              lib.orc_backward_from_xhat):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(_D)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _shape(x: np.ndarray):
    N, C, H, W = x.shape
    return N, C, H * W


def num_threads() -> int:
    return int(_load().orc_num_threads())


def forward_train(x, gamma, beta, act="leaky_relu", act_param=0.01, eps=1e-5, momentum=0.1,
                  running_mean=None, running_var=None, storage="f64"):
    """Training forward.  x: [N,C,H,W].  Returns dict y (rounded to `storage`), mean, var,
    invstd and, when given, the updated running_mean / running_var (fp64 copies)."""
    x = _f64(x)
    N, C, HW = _shape(x)
    y = np.empty_like(x)
    mean, var, inv = np.empty(C), np.empty(C), np.empty(C)
    rm = None if running_mean is None else _f64(running_mean).copy()
    rv = None if running_var is None else _f64(running_var).copy()
    rc = _load().orc_forward_train(N, C, HW, _p(x), _p(_f64(gamma)), _p(_f64(beta)), ACT[act],
                                   float(act_param), float(eps), float(momentum), _p(y),
                                   _p(mean), _p(var), _p(inv), _p(rm), _p(rv))
    if rc != 0:
        raise ValueError("oracle forward_train rejected its arguments")
    round_storage(y, storage)
    return {"y": y, "mean": mean, "var": var, "invstd": inv, "running_mean": rm, "running_var": rv}


def forward_eval(x, gamma, beta, running_mean, running_var, act="leaky_relu", act_param=0.01,
                 eps=1e-5, storage="f64"):
    x = _f64(x)
    N, C, HW = _shape(x)
    y = np.empty_like(x)
    rc = _load().orc_forward_eval(N, C, HW, _p(x), _p(_f64(gamma)), _p(_f64(beta)),
                                  _p(_f64(running_mean)), _p(_f64(running_var)), ACT[act],
                                  float(act_param), float(eps), _p(y))
    if rc != 0:
        raise ValueError("oracle forward_eval rejected its arguments")
    round_storage(y, storage)
    return y


def backward_from_y(y, dy, gamma, beta, invstd, act="leaky_relu", act_param=0.01,
                    want_xhat=False):
    """Backward from the stored output y (form I).  Returns dict dx, dgamma, dbeta[, xhat]."""
    y, dy = _f64(y), _f64(dy)
    N, C, HW = _shape(y)
    dx = np.empty_like(y)
    dg, db = np.empty(C), np.empty(C)
    xh = np.empty_like(y) if want_xhat else None
    rc = _load().orc_backward_from_y(N, C, HW, _p(y), _p(dy), _p(_f64(gamma)), _p(_f64(beta)),
                                     _p(_f64(invstd)), ACT[act], float(act_param), _p(dx),
                                     _p(dg), _p(db), _p(xh))
    if rc != 0:
        raise ValueError("oracle backward_from_y rejected its arguments")
    out = {"dx": dx, "dgamma": dg, "dbeta": db}
    if want_xhat:
        out["xhat"] = xh
    return out


def backward_eval(y, dy, gamma, beta, running_var, act="leaky_relu", act_param=0.01, eps=1e-5):
    """Backward through the inference forward (frozen running statistics), from
    the stored y.  Returns dict dx, dgamma, dbeta."""
    y, dy = _f64(y), _f64(dy)
    N, C, HW = _shape(y)
    dx = np.empty_like(y)
    dg, db = np.empty(C), np.empty(C)
    rc = _load().orc_backward_eval(N, C, HW, _p(y), _p(dy), _p(_f64(gamma)), _p(_f64(beta)),
                                   _p(_f64(running_var)), float(eps), ACT[act], float(act_param),
                                   _p(dx), _p(dg), _p(db))
    if rc != 0:
        raise ValueError("oracle backward_eval rejected its arguments")
    return {"dx": dx, "dgamma": dg, "dbeta": db}


def backward_from_y_form2(y, dy, gamma, beta, invstd, act="leaky_relu", act_param=0.01):
    y, dy = _f64(y), _f64(dy)
    N, C, HW = _shape(y)
    dx = np.empty_like(y)
    dg, db = np.empty(C), np.empty(C)
    rc = _load().orc_backward_from_y_form2(N, C, HW, _p(y), _p(dy), _p(_f64(gamma)),
                                           _p(_f64(beta)), _p(_f64(invstd)), ACT[act],
                                           float(act_param), _p(dx), _p(dg), _p(db))
    if rc != 0:
        raise ValueError("oracle backward_from_y_form2 rejected its arguments")
    return {"dx": dx, "dgamma": dg, "dbeta": db}


def backward_from_x(x, dy, gamma, beta, act="leaky_relu", act_param=0.01, eps=1e-5):
    """Conventional backward of a block that stores x."""
    x, dy = _f64(x), _f64(dy)
    N, C, HW = _shape(x)
    dx = np.empty_like(x)
    dg, db = np.empty(C), np.empty(C)
    rc = _load().orc_backward_from_x(N, C, HW, _p(x), _p(dy), _p(_f64(gamma)), _p(_f64(beta)),
                                     ACT[act], float(act_param), float(eps), _p(dx), _p(dg),
                                     _p(db))
    if rc != 0:
        raise ValueError("oracle backward_from_x rejected its arguments")
    return {"dx": dx, "dgamma": dg, "dbeta": db}


def forward_train_ckpt(x, gamma, beta, act="leaky_relu", act_param=0.01, eps=1e-5, momentum=0.1,
                       running_mean=None, running_var=None, storage="f64"):
    """Training forward of optimized checkpointing: the block keeps xhat.  Returns
    dict xhat and y (both rounded to `storage`), mean, var, invstd and, when given,
    the updated running statistics."""
    x = _f64(x)
    N, C, HW = _shape(x)
    xh, y = np.empty_like(x), np.empty_like(x)
    mean, var, inv = np.empty(C), np.empty(C), np.empty(C)
    rm = None if running_mean is None else _f64(running_mean).copy()
    rv = None if running_var is None else _f64(running_var).copy()
    rc = _load().orc_forward_train_ckpt(N, C, HW, _p(x), _p(_f64(gamma)), _p(_f64(beta)),
                                        ACT[act], float(act_param), float(eps), float(momentum),
                                        _p(xh), _p(y), _p(mean), _p(var), _p(inv), _p(rm), _p(rv))
    if rc != 0:
        raise ValueError("oracle forward_train_ckpt rejected its arguments")
    round_storage(xh, storage)
    round_storage(y, storage)
    return {"xhat": xh, "y": y, "mean": mean, "var": var, "invstd": inv, "running_mean": rm,
            "running_var": rv}


def recompute_from_xhat(xhat, gamma, beta, act="leaky_relu", act_param=0.01, storage="f64"):
    """y = act(gamma xhat + beta), rounded to `storage`."""
    xhat = _f64(xhat)
    N, C, HW = _shape(xhat)
    y = np.empty_like(xhat)
    rc = _load().orc_recompute_from_xhat(N, C, HW, _p(xhat), _p(_f64(gamma)), _p(_f64(beta)),
                                         ACT[act], float(act_param), _p(y))
    if rc != 0:
        raise ValueError("oracle recompute_from_xhat rejected its arguments")
    round_storage(y, storage)
    return y


def backward_from_xhat(xhat, dy, gamma, beta, invstd, act="leaky_relu", act_param=0.01):
    """Backward from the checkpoint xhat.  Returns dict dx, dgamma, dbeta."""
    xhat, dy = _f64(xhat), _f64(dy)
    N, C, HW = _shape(xhat)
    dx = np.empty_like(xhat)
    dg, db = np.empty(C), np.empty(C)
    rc = _load().orc_backward_from_xhat(N, C, HW, _p(xhat), _p(dy), _p(_f64(gamma)),
                                        _p(_f64(beta)), _p(_f64(invstd)), ACT[act],
                                        float(act_param), _p(dx), _p(dg), _p(db))
    if rc != 0:
        raise ValueError("oracle backward_from_xhat rejected its arguments")
    return {"dx": dx, "dgamma": dg, "dbeta": db}


def round_storage(v: np.ndarray, storage: str) -> np.ndarray:
    """Round an fp64 array in place to the values representable in `storage`."""
    assert v.dtype == np.float64 and v.flags.c_contiguous
    rc = _load().orc_round_storage(_p(v), v.size, STORE[storage])
    if rc != 0:
        raise ValueError(storage)
    return v
