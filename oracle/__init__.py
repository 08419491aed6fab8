"""fp64 CPU oracle of the selective (S6) scan -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never loads it and
shares no code with it.  The arithmetic lives in ``scan_oracle.c`` (plain C,
double precision, one sequential loop per (batch, channel) row); this module
only compiles it with gcc and marshals numpy arrays into it.

Sources, cited by page title and section:
  [MFS] "从零理解 Mamba：选择性状态空间模型（Selective SSM）到 Mamba Block" (eutaboo.com)
  [MUN] "【临时文档---算法介绍】Mamba-UNet" (blog.csdn.net)
  [VIM] "Vision Mamba：从状态空间模型到视觉革命的跨越" (x-humanoid.csdn.net)
  [S4M] "从S4到Mamba：选择性状态空间模型的演进与革新" (jsqmd.com)

Every function here is pinned against something other than itself.
``tests/test_oracle_pins.py`` pins the scan, the step and the Conv1d against
closed forms, brute force and invariants the pages fix (LTI convolution [MFS
§2.3, eq (3a)(3b)], the A = 0 cumulative sum, associativity of the affine
scan [MFS §5], the first-order limit of the ZOH rule [MUN §4], flip
equivariance [VIM §2.2], the N = 1 gated-RNN case [MFS §6.2 Step 5, Theorem
1], the recurrent/step form [MFS §2.3], the Conv1d's impulse response and
numpy's convolution).  ``tests/test_oracle_bwd_pins.py`` pins the backward
pass against central finite differences of the forward oracle for every
gradient, and checks that it is linear in dout.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "scan_oracle.c")
_CONV_SRC = os.path.join(_HERE, "conv_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

DIR_FWD, DIR_BWD, DIR_BIDIR, DIR_CROSS2D = 0, 1, 2, 3
DTYPE_F32, DTYPE_BF16 = 0, 1


class _Dims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("dim", ctypes.c_int64), ("seqlen", ctypes.c_int64),
        ("dstate", ctypes.c_int64), ("height", ctypes.c_int64), ("width", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("dir_mode", ctypes.c_int32),
        ("delta_softplus", ctypes.c_int32), ("exact_zoh", ctypes.c_int32),
    ]


class _Inputs(ctypes.Structure):
    _fields_ = [
        ("u", ctypes.c_void_p), ("delta", ctypes.c_void_p), ("B", ctypes.c_void_p),
        ("C", ctypes.c_void_p), ("z", ctypes.c_void_p), ("A", ctypes.c_void_p),
        ("D", ctypes.c_void_p), ("delta_bias", ctypes.c_void_p),
        ("initial_state", ctypes.c_void_p),
    ]


def build(force: bool = False) -> str:
    """Compile scan_oracle.c and conv_oracle.c into liboracle.so with gcc (no GPU code involved)."""
    with _lock:
        stale = not os.path.exists(_LIB) or any(os.path.getmtime(_LIB) < os.path.getmtime(f) for f in (_SRC, _CONV_SRC))
        if force or stale:
            tmp = _LIB + ".tmp%d" % os.getpid()
            subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
                                   "-o", tmp, _SRC, _CONV_SRC, "-lm"])
            os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.oracle_scan_rows.restype = ctypes.c_int
        lib.oracle_scan_rows.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(_Inputs),
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_scan_bwd.restype = ctypes.c_int
        lib.oracle_scan_bwd.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(_Inputs), ctypes.c_void_p] + \
            [ctypes.c_void_p] * 9
        lib.oracle_conv1d.restype = ctypes.c_int
        lib.oracle_conv1d.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_scan_step.restype = ctypes.c_int
        lib.oracle_scan_step.argtypes = [ctypes.POINTER(_Dims)] + [ctypes.c_void_p] * 10
        lib.oracle_softplus.restype = ctypes.c_double
        lib.oracle_softplus.argtypes = [ctypes.c_double]
        lib.oracle_silu.restype = ctypes.c_double
        lib.oracle_silu.argtypes = [ctypes.c_double]
        lib.oracle_token.restype = ctypes.c_int64
        lib.oracle_token.argtypes = [ctypes.POINTER(_Dims), ctypes.c_int, ctypes.c_int64]
        lib.oracle_num_dirs.restype = ctypes.c_int
        lib.oracle_num_dirs.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def num_dirs(dir_mode: int) -> int:
    return {DIR_FWD: 1, DIR_BWD: 1, DIR_BIDIR: 2, DIR_CROSS2D: 4}[dir_mode]


def _dtype_code(arr: np.ndarray) -> int:
    if arr.dtype == np.float32:
        return DTYPE_F32
    if arr.dtype == np.uint16:
        return DTYPE_BF16
    raise TypeError("oracle inputs must be float32 or bfloat16 bit patterns (uint16), got %s" % arr.dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if dtype is not None and a.dtype != dtype:
        raise TypeError("expected %s, got %s" % (dtype, a.dtype))
    return a


def _dims(batch, dim, seqlen, dstate, dtype, dir_mode, delta_softplus, exact_zoh, height=0, width=0):
    return _Dims(batch, dim, seqlen, dstate, height, width, dtype, dir_mode,
                 1 if delta_softplus else 0, 1 if exact_zoh else 0)


def scan(u, delta, A, B, C, D=None, z=None, delta_bias=None, *, dir_mode=DIR_FWD,
         height=0, width=0, delta_softplus=True, exact_zoh=False, initial_state=None,
         rows=None, nthreads=None):
    """Run the oracle.

    Layouts (token-major, all C-contiguous; K = number of scan directions):
      u      [B][Ku][L][D]  (Ku = 1 for the cross scan, else K; the K axis is
                             omitted for K = 1, i.e. [B][L][D])
      delta  [B][K][L][D],  B, C [B][K][L][N],  z [B][L][D]
      A [K][D][N] float32, D and delta_bias [K][D] float32,
      initial_state [B][K][D][N] float32 or None.
    bf16 tensors are passed as uint16 bit patterns.

    rows: None for every (b, d) row, else an int array of shape [R, 2] with
      (b, d) pairs.
    Returns (out, last_state): for rows=None, out is [B][L][D] float64 and
      last_state [B][K][D][N]; otherwise out is [R][L] and last_state [R][K][N].
    """
    lib = _load()
    K = num_dirs(dir_mode)
    u = _c(u)
    dt = _dtype_code(u)
    delta, B, C, z = (_c(x) for x in (delta, B, C, z))
    for x in (delta, B, C) + ((z,) if z is not None else ()):
        if x.dtype != u.dtype:
            raise TypeError("u, delta, B, C, z must share one dtype")
    A = _c(A, np.float32)
    D = _c(D, np.float32)
    delta_bias = _c(delta_bias, np.float32)
    initial_state = _c(initial_state, np.float32)
    Bsz = u.shape[0]
    L = delta.shape[-2]
    Dm = delta.shape[-1]
    N = B.shape[-1]
    Ku = 1 if dir_mode == DIR_CROSS2D else K
    if u.size != Bsz * Ku * L * Dm or delta.size != Bsz * K * L * Dm:
        raise ValueError("u/delta shapes do not match the direction mode")
    if B.size != Bsz * K * L * N or C.size != Bsz * K * L * N or A.size != K * Dm * N:
        raise ValueError("B/C/A shapes do not match")
    if z is not None and z.size != Bsz * L * Dm:
        raise ValueError("z shape does not match")
    g = _dims(Bsz, Dm, L, N, dt, dir_mode, delta_softplus, exact_zoh, height, width)
    ins = _Inputs(_ptr(u), _ptr(delta), _ptr(B), _ptr(C), _ptr(z), _ptr(A), _ptr(D),
                  _ptr(delta_bias), _ptr(initial_state))
    full = rows is None
    if full:
        bb, dd = np.meshgrid(np.arange(Bsz, dtype=np.int64), np.arange(Dm, dtype=np.int64), indexing="ij")
        rb, rd = np.ascontiguousarray(bb.ravel()), np.ascontiguousarray(dd.ravel())
    else:
        rows = np.asarray(rows, dtype=np.int64).reshape(-1, 2)
        rb, rd = np.ascontiguousarray(rows[:, 0]), np.ascontiguousarray(rows[:, 1])
    R = rb.shape[0]
    out = np.empty((R, L), dtype=np.float64)
    st = np.empty((R, K, N), dtype=np.float64)
    if nthreads is None:
        nthreads = min(16, os.cpu_count() or 1)
    rc = lib.oracle_scan_rows(ctypes.byref(g), ctypes.byref(ins), rb.ctypes.data, rd.ctypes.data, R,
                              out.ctypes.data, st.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_scan_rows failed with %d" % rc)
    if full:
        out = np.ascontiguousarray(out.reshape(Bsz, Dm, L).transpose(0, 2, 1))
        st = np.ascontiguousarray(st.reshape(Bsz, Dm, K, N).transpose(0, 2, 1, 3))
    return out, st


def step(state, u_t, delta_t, A, B_t, C_t, D=None, z_t=None, delta_bias=None, *,
         delta_softplus=True, exact_zoh=False):
    """One recurrent step of a forward scan.  state [B][D][N] float64 is updated
    in place; returns out [B][D] float64."""
    lib = _load()
    u_t = _c(u_t)
    dt = _dtype_code(u_t)
    delta_t, B_t, C_t, z_t = (_c(x) for x in (delta_t, B_t, C_t, z_t))
    if state.dtype != np.float64 or not state.flags["C_CONTIGUOUS"]:
        raise TypeError("state must be a C-contiguous float64 array")
    A = _c(A, np.float32)
    D = _c(D, np.float32)
    delta_bias = _c(delta_bias, np.float32)
    Bsz, Dm = u_t.shape[0], u_t.shape[-1]
    N = B_t.shape[-1]
    if state.size != Bsz * Dm * N:
        raise ValueError("state shape does not match")
    g = _dims(Bsz, Dm, 1, N, dt, DIR_FWD, delta_softplus, exact_zoh)
    out = np.empty((Bsz, Dm), dtype=np.float64)
    rc = lib.oracle_scan_step(ctypes.byref(g), state.ctypes.data, _ptr(u_t), _ptr(delta_t), _ptr(A),
                              _ptr(B_t), _ptr(C_t), _ptr(D), _ptr(z_t), _ptr(delta_bias), out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_scan_step failed with %d" % rc)
    return out


def softplus(x: float) -> float:
    return _load().oracle_softplus(float(x))


def silu(x: float) -> float:
    return _load().oracle_silu(float(x))


def token(dir_mode: int, k: int, p: int, seqlen: int, height: int = 0, width: int = 0) -> int:
    g = _dims(1, 1, seqlen, 1, 0, dir_mode, True, False, height, width)
    return _load().oracle_token(ctypes.byref(g), k, p)


def conv1d(x, weight, bias=None, *, reverse=False, activation=True):
    """Causal depthwise Conv1d + SiLU (conv_oracle.c): x [B][L][D] (float32 or
    bfloat16 bits as uint16), weight [D][W] float32, bias [D] float32 or None.
    Returns float64 [B][L][D]."""
    lib = _load()
    x = np.ascontiguousarray(x)
    Bsz, L, Dm = x.shape
    w = _c(weight, np.float32)
    if w.shape[0] != Dm:
        raise ValueError("weight must be [D][W]")
    b = None if bias is None else _c(bias, np.float32)
    out = np.empty((Bsz, L, Dm), np.float64)
    rc = lib.oracle_conv1d(Bsz, Dm, L, _dtype_code(x), w.shape[1], 1 if reverse else 0, 1 if activation else 0,
                           _ptr(x), _ptr(w), _ptr(b), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_conv1d: invalid arguments")
    return out


def scan_bwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, dout=None, *, dir_mode=DIR_FWD, height=0,
             width=0, delta_softplus=True, exact_zoh=False, initial_state=None):
    """Gradients of L = sum(dout * out) with respect to every input of ``scan``
    (oracle_scan_bwd, float64).  Same layouts as ``scan``; dout is [B][L][D] in
    the input type.  Returns a dict of float64 arrays shaped like the inputs:
    du, ddelta, dA, dB, dC, dD, dz (None without z), ddelta_bias, dinit."""
    lib = _load()
    K = num_dirs(dir_mode)
    u = _c(u)
    dt = _dtype_code(u)
    delta, B, C, z, dout = (_c(x) for x in (delta, B, C, z, dout))
    for x in (delta, B, C, dout) + ((z,) if z is not None else ()):
        if x.dtype != u.dtype:
            raise TypeError("u, delta, B, C, z, dout must share one dtype")
    A = _c(A, np.float32)
    D = _c(D, np.float32)
    delta_bias = _c(delta_bias, np.float32)
    initial_state = _c(initial_state, np.float32)
    Bsz, L, Dm, N = u.shape[0], delta.shape[-2], delta.shape[-1], B.shape[-1]
    Ku = 1 if dir_mode == DIR_CROSS2D else K
    if dout.size != Bsz * L * Dm:
        raise ValueError("dout must be [B][L][D]")
    g = _dims(Bsz, Dm, L, N, dt, dir_mode, delta_softplus, exact_zoh, height, width)
    ins = _Inputs(_ptr(u), _ptr(delta), _ptr(B), _ptr(C), _ptr(z), _ptr(A), _ptr(D),
                  _ptr(delta_bias), _ptr(initial_state))
    kx = () if K == 1 else (K,)
    ux = () if Ku == 1 else (Ku,)
    out = dict(du=np.empty((Bsz,) + ux + (L, Dm)), ddelta=np.empty((Bsz,) + kx + (L, Dm)),
               dA=np.empty(kx + (Dm, N)), dB=np.empty((Bsz,) + kx + (L, N)), dC=np.empty((Bsz,) + kx + (L, N)),
               dD=np.empty(kx + (Dm,)), dz=None if z is None else np.empty((Bsz, L, Dm)),
               ddelta_bias=np.empty(kx + (Dm,)), dinit=np.empty((Bsz,) + kx + (Dm, N)))
    rc = lib.oracle_scan_bwd(ctypes.byref(g), ctypes.byref(ins), _ptr(dout), _ptr(out["du"]), _ptr(out["ddelta"]),
                             _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dz"]),
                             _ptr(out["ddelta_bias"]), _ptr(out["dinit"]))
    if rc != 0:
        raise ValueError("oracle_scan_bwd failed with %d" % rc)
    return out
