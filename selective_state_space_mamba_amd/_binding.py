"""ctypes binding of libmamba_scan.so (declared in include/mamba_scan.h).

Argument marshalling only: tensors become device pointers, shapes become a
``mamba_dims`` struct, torch's current stream becomes the ``hipStream_t``.
Every step of the scan runs in the library's HIP kernels; there is no
fallback, and loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmamba_scan.so")

MAMBA_OK, MAMBA_ERR_INVALID, MAMBA_ERR_UNSUPPORTED, MAMBA_ERR_WORKSPACE, MAMBA_ERR_HIP, MAMBA_ERR_SCRATCH = \
    0, -1, -2, -3, -4, -5
NOALLOC_SCRATCH_BYTES = 32 << 20
DIR_FWD, DIR_BWD, DIR_BIDIR, DIR_CROSS2D = 0, 1, 2, 3
DTYPE_F32, DTYPE_BF16 = 0, 1
EXPORTED = ("mamba_conv1d_silu", "mamba_scan_bwd", "mamba_scan_bwd_workspace_bytes", "mamba_scan_fwd_workspace_bytes",
            "mamba_scan_fwd", "mamba_scan_fwd_noalloc", "mamba_scan_fwd_save", "mamba_scan_saved_bytes",
            "mamba_scan_step",
            "mamba_status_string")


class MambaDims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("dim", ctypes.c_int64), ("seqlen", ctypes.c_int64),
        ("dstate", ctypes.c_int64), ("height", ctypes.c_int64), ("width", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("delta_softplus", ctypes.c_int32), ("exact_zoh", ctypes.c_int32),
        ("initial_state", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class MambaError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__("%s failed: %s (%d)" % (where, status_string(code), code))
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the built library (no build here; see selective_state_space_mamba_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libmamba_scan.so is not built (%s); run `python -m selective_state_space_mamba_amd.build` "
                           "or __graft_entry__.build()" % path)
    # torch's wheel bundles its own HIP runtime under the same soname
    # (libamdhip64.so.7) but asks for it as libamdhip64.so: loaded after torch,
    # the library binds to torch's runtime (one runtime, shared streams and
    # memory); loaded first, it would pull in the system runtime and torch a
    # second one.  So torch is imported first.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.mamba_scan_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.mamba_scan_fwd_workspace_bytes.argtypes = [ctypes.POINTER(MambaDims), i32]
    lib.mamba_scan_fwd.restype = i32
    lib.mamba_scan_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(MambaDims), i32, vp, vp, vp]
    lib.mamba_scan_fwd_noalloc.restype = i32
    lib.mamba_scan_fwd_noalloc.argtypes = lib.mamba_scan_fwd.argtypes
    lib.mamba_scan_step.restype = i32
    lib.mamba_scan_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(MambaDims), vp, vp]
    lib.mamba_scan_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.mamba_scan_bwd_workspace_bytes.argtypes = [ctypes.POINTER(MambaDims), i32]
    lib.mamba_scan_bwd.restype = i32
    lib.mamba_scan_bwd.argtypes = [vp] * 9 + [ctypes.POINTER(MambaDims), i32] + [vp] * 9 + [vp, ctypes.c_size_t, vp]
    lib.mamba_scan_saved_bytes.restype = ctypes.c_size_t
    lib.mamba_scan_saved_bytes.argtypes = [ctypes.POINTER(MambaDims), i32, i32]
    lib.mamba_scan_fwd_save.restype = i32
    lib.mamba_scan_fwd_save.argtypes = [vp] * 8 + [ctypes.POINTER(MambaDims), i32, vp, vp, vp, ctypes.c_size_t, vp]
    lib.mamba_conv1d_silu.restype = i32
    lib.mamba_conv1d_silu.argtypes = [vp, vp, vp, ctypes.POINTER(MambaDims), i32, i32, vp, vp]
    lib.mamba_status_string.restype = ctypes.c_char_p
    lib.mamba_status_string.argtypes = [i32]
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load_library().mamba_status_string(int(code)).decode()


def num_dirs(dir_mode: int) -> int:
    return {DIR_FWD: 1, DIR_BWD: 1, DIR_BIDIR: 2, DIR_CROSS2D: 4}[dir_mode]


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError("u/delta/B/C/z must be float32 or bfloat16, got %s" % t.dtype)


def _stream(stream) -> int | None:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _foreign_stream(stream):
    """The launch stream as a torch stream when it is not torch's current
    stream, else None.  A wrapper that will allocate (outputs, workspace,
    saved state) then calls itself again with that stream current, so that
    its tensors come from the caching allocator's pool of the stream the
    library launches on and a workspace dropped on return is not handed to
    another stream while the launch may still be using it.  A call given all
    its buffers skips the check (it costs a few microseconds of host time)."""
    import torch
    if stream is None:
        return None
    ts = torch.cuda.ExternalStream(stream) if isinstance(stream, int) else stream
    return None if ts.cuda_stream == torch.cuda.current_stream(ts.device).cuda_stream else ts


def make_dims(batch, dim, seqlen, dstate, dtype, *, height=0, width=0, delta_softplus=True, exact_zoh=False,
              initial_state=None, workspace=None, workspace_bytes=0) -> MambaDims:
    return MambaDims(int(batch), int(dim), int(seqlen), int(dstate), int(height), int(width), int(dtype),
                     1 if delta_softplus else 0, 1 if exact_zoh else 0, _ptr(initial_state), _ptr(workspace),
                     int(workspace_bytes))


def workspace_bytes(dims: MambaDims, dir_mode: int) -> int:
    n = load_library().mamba_scan_fwd_workspace_bytes(ctypes.byref(dims), int(dir_mode))
    if n == ctypes.c_size_t(-1).value:
        raise MambaError(MAMBA_ERR_INVALID, "mamba_scan_fwd_workspace_bytes")
    return n


def bwd_workspace_bytes(dims: MambaDims, dir_mode: int) -> int:
    n = load_library().mamba_scan_bwd_workspace_bytes(ctypes.byref(dims), int(dir_mode))
    if n == ctypes.c_size_t(-1).value:
        raise MambaError(MAMBA_ERR_UNSUPPORTED, "mamba_scan_bwd_workspace_bytes")
    return n


def saved_bytes(dims: MambaDims, dir_mode: int, gated: bool) -> int:
    n = load_library().mamba_scan_saved_bytes(ctypes.byref(dims), int(dir_mode), 1 if gated else 0)
    if n == ctypes.c_size_t(-1).value:
        raise MambaError(MAMBA_ERR_UNSUPPORTED, "mamba_scan_saved_bytes")
    return n


def _check(t, name, shape, dtype, device):
    if t is None:
        return
    if t.shape == shape and t.dtype == dtype and t.is_contiguous() and t.device == device:
        return  # (the common case, without building messages)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


def _check_buffer(t, name, device):
    """A caller's workspace or saved-state buffer: any dtype, passed on as its
    bytes, so it must be one contiguous block on the device of the inputs."""
    if t is None:
        return
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


def _torch_f32():
    import torch
    return torch.float32


def _check_fwd_shapes(u, delta, A, B, C, D, z, delta_bias, initial_state, dir_mode, K, Bsz, L, Dm, N, tdt, dev):
    f32 = _torch_f32()
    kx = () if K == 1 else (K,)
    ux = () if (K == 1 or dir_mode == DIR_CROSS2D) else (K,)
    _check(u, "u", (Bsz,) + ux + (L, Dm), tdt, dev)
    _check(delta, "delta", (Bsz,) + kx + (L, Dm), tdt, dev)
    _check(B, "B", (Bsz,) + kx + (L, N), tdt, dev)
    _check(C, "C", (Bsz,) + kx + (L, N), tdt, dev)
    _check(z, "z", (Bsz, L, Dm), tdt, dev)
    _check(A, "A", kx + (Dm, N), f32, dev)
    _check(D, "D", kx + (Dm,), f32, dev)
    _check(delta_bias, "delta_bias", kx + (Dm,), f32, dev)
    _check(initial_state, "initial_state", (Bsz,) + kx + (Dm, N), f32, dev)


def scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, *, dir_mode=DIR_FWD, height=0, width=0,
             delta_softplus=True, exact_zoh=False, initial_state=None, out=None, last_state=None,
             want_last_state=True, workspace=None, stream=None):
    """mamba_scan_fwd on torch tensors.

    Shapes (K directions; the K axis is absent when K = 1; u has no K axis for
    the cross scan): u [B][K][L][D], delta [B][K][L][D], A [K][D][N],
    B/C [B][K][L][N], D/delta_bias [K][D], z [B][L][D].
    Returns (out [B][L][D], last_state [B][K][D][N] or None)."""
    out, last_state, _ = _fwd(u, delta, A, B, C, D, z, delta_bias, dir_mode, height, width, delta_softplus,
                              exact_zoh, initial_state, out, last_state, want_last_state, workspace, stream,
                              False, None)
    return out, last_state


def scan_fwd_noalloc(u, delta, A, B, C, D=None, z=None, delta_bias=None, *, dir_mode=DIR_FWD, height=0,
                     width=0, delta_softplus=True, exact_zoh=False, initial_state=None, out, last_state=None,
                     stream=None):
    """mamba_scan_fwd_noalloc on torch tensors: the forward pass with its scratch
    taken from the library's static device array (no workspace argument).  The
    caller passes out [B][L][D] and, if wanted, last_state [B][K][D][N]; this
    wrapper allocates nothing.  Returns (out, last_state)."""
    lib = load_library()
    K = num_dirs(dir_mode)
    dev = u.device
    dt = _dtype_code(u)
    tdt = u.dtype
    Bsz, L, Dm = delta.shape[0], delta.shape[-2], delta.shape[-1]
    N = B.shape[-1]
    _check_fwd_shapes(u, delta, A, B, C, D, z, delta_bias, initial_state, dir_mode, K, Bsz, L, Dm, N, tdt, dev)
    _check(out, "out", (Bsz, L, Dm), tdt, dev)
    _check(last_state, "last_state", (Bsz,) + (() if K == 1 else (K,)) + (Dm, N), _torch_f32(), dev)
    dims = make_dims(Bsz, Dm, L, N, dt, height=height, width=width, delta_softplus=delta_softplus,
                     exact_zoh=exact_zoh, initial_state=initial_state)
    rc = lib.mamba_scan_fwd_noalloc(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                    _ptr(delta_bias), ctypes.byref(dims), int(dir_mode), _ptr(out),
                                    _ptr(last_state), _stream(stream))
    if rc != MAMBA_OK:
        raise MambaError(rc, "mamba_scan_fwd_noalloc")
    return out, last_state


def scan_fwd_save(u, delta, A, B, C, D=None, z=None, delta_bias=None, *, dir_mode=DIR_FWD, height=0, width=0,
                  delta_softplus=True, exact_zoh=False, initial_state=None, out=None, last_state=None,
                  want_last_state=True, workspace=None, saved=None, stream=None):
    """mamba_scan_fwd_save on torch tensors: scan_fwd that also fills the
    saved forward state for scan_bwd(..., saved=...).  saved: a uint8 device
    tensor of at least saved_bytes(dims, dir_mode, z is not None) bytes, or
    None to allocate one.  Returns (out, last_state, saved)."""
    return _fwd(u, delta, A, B, C, D, z, delta_bias, dir_mode, height, width, delta_softplus, exact_zoh,
                initial_state, out, last_state, want_last_state, workspace, stream, True, saved)


def _fwd(u, delta, A, B, C, D, z, delta_bias, dir_mode, height, width, delta_softplus, exact_zoh, initial_state,
         out, last_state, want_last_state, workspace, stream, save, saved):
    import torch
    allocates = (out is None or workspace is None or (last_state is None and want_last_state)
                 or (save and saved is None))
    ts = _foreign_stream(stream) if allocates else None
    if ts is not None:
        with torch.cuda.stream(ts):
            return _fwd(u, delta, A, B, C, D, z, delta_bias, dir_mode, height, width, delta_softplus, exact_zoh,
                        initial_state, out, last_state, want_last_state, workspace, ts, save, saved)
    lib = load_library()
    K = num_dirs(dir_mode)
    dev = u.device
    dt = _dtype_code(u)
    tdt = u.dtype
    Bsz, L, Dm = delta.shape[0], delta.shape[-2], delta.shape[-1]
    N = B.shape[-1]
    kx = () if K == 1 else (K,)
    _check_fwd_shapes(u, delta, A, B, C, D, z, delta_bias, initial_state, dir_mode, K, Bsz, L, Dm, N, tdt, dev)
    if out is None:
        out = torch.empty((Bsz, L, Dm), dtype=tdt, device=dev)
    _check(out, "out", (Bsz, L, Dm), tdt, dev)
    if last_state is None and want_last_state:
        last_state = torch.empty((Bsz,) + kx + (Dm, N), dtype=torch.float32, device=dev)
    _check(last_state, "last_state", (Bsz,) + kx + (Dm, N), torch.float32, dev)
    dims = make_dims(Bsz, Dm, L, N, dt, height=height, width=width, delta_softplus=delta_softplus,
                     exact_zoh=exact_zoh, initial_state=initial_state)
    _check_buffer(workspace, "workspace", dev)
    _check_buffer(saved, "saved", dev)
    need = workspace_bytes(dims, dir_mode)
    if need > 0:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        dims.workspace = workspace.data_ptr()
        dims.workspace_bytes = workspace.numel() * workspace.element_size()
    if not save:
        rc = lib.mamba_scan_fwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                _ptr(delta_bias), ctypes.byref(dims), int(dir_mode), _ptr(out), _ptr(last_state),
                                _stream(stream))
        if rc != MAMBA_OK:
            raise MambaError(rc, "mamba_scan_fwd")
        return out, last_state, None
    if saved is None:
        saved = torch.empty(saved_bytes(dims, dir_mode, z is not None), dtype=torch.uint8, device=dev)
    rc = lib.mamba_scan_fwd_save(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                 _ptr(delta_bias), ctypes.byref(dims), int(dir_mode), _ptr(out), _ptr(last_state),
                                 _ptr(saved), saved.numel() * saved.element_size(), _stream(stream))
    if rc != MAMBA_OK:
        raise MambaError(rc, "mamba_scan_fwd_save")
    return out, last_state, saved


def scan_bwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, *, dout, dir_mode=DIR_FWD, height=0, width=0,
             delta_softplus=True, exact_zoh=False, initial_state=None, want_dinit=True, workspace=None,
             saved=None, stream=None):
    """mamba_scan_bwd on torch tensors: gradients of sum(dout * out) for the
    scan_fwd call with the same arguments.  Returns a dict with du, ddelta,
    dA, dB, dC (shaped like their inputs), dD and ddelta_bias (None when D or
    delta_bias is None), dz (None without z) and dinit ([B][K][D][N] float32,
    None unless want_dinit).  saved: the buffer scan_fwd_save returned for
    the same arguments (the forward recompute is then skipped), or None."""
    import torch
    ts = _foreign_stream(stream)
    if ts is not None:
        with torch.cuda.stream(ts):
            return scan_bwd(u, delta, A, B, C, D, z, delta_bias, dout=dout, dir_mode=dir_mode, height=height,
                            width=width, delta_softplus=delta_softplus, exact_zoh=exact_zoh,
                            initial_state=initial_state, want_dinit=want_dinit, workspace=workspace, saved=saved,
                            stream=ts)
    lib = load_library()
    K = num_dirs(dir_mode)
    dev = u.device
    dt = _dtype_code(u)
    tdt = u.dtype
    Bsz, L, Dm = delta.shape[0], delta.shape[-2], delta.shape[-1]
    N = B.shape[-1]
    kx = () if K == 1 else (K,)
    ux = () if (K == 1 or dir_mode == DIR_CROSS2D) else (K,)
    _check(u, "u", (Bsz,) + ux + (L, Dm), tdt, dev)
    _check(delta, "delta", (Bsz,) + kx + (L, Dm), tdt, dev)
    _check(B, "B", (Bsz,) + kx + (L, N), tdt, dev)
    _check(C, "C", (Bsz,) + kx + (L, N), tdt, dev)
    _check(z, "z", (Bsz, L, Dm), tdt, dev)
    _check(dout, "dout", (Bsz, L, Dm), tdt, dev)
    _check(A, "A", kx + (Dm, N), torch.float32, dev)
    _check(D, "D", kx + (Dm,), torch.float32, dev)
    _check(delta_bias, "delta_bias", kx + (Dm,), torch.float32, dev)
    _check(initial_state, "initial_state", (Bsz,) + kx + (Dm, N), torch.float32, dev)
    g = dict(du=torch.empty_like(u), ddelta=torch.empty_like(delta), dA=torch.empty_like(A),
             dB=torch.empty_like(B), dC=torch.empty_like(C),
             dD=None if D is None else torch.empty_like(D), dz=None if z is None else torch.empty_like(z),
             ddelta_bias=None if delta_bias is None else torch.empty_like(delta_bias),
             dinit=torch.empty((Bsz,) + kx + (Dm, N), dtype=torch.float32, device=dev) if want_dinit else None)
    dims = make_dims(Bsz, Dm, L, N, dt, height=height, width=width, delta_softplus=delta_softplus,
                     exact_zoh=exact_zoh, initial_state=initial_state)
    _check_buffer(workspace, "workspace", dev)
    _check_buffer(saved, "saved", dev)
    need = bwd_workspace_bytes(dims, dir_mode)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    dims.workspace = workspace.data_ptr()
    dims.workspace_bytes = workspace.numel() * workspace.element_size()
    rc = lib.mamba_scan_bwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                            _ptr(dout), ctypes.byref(dims), int(dir_mode), _ptr(g["du"]), _ptr(g["ddelta"]),
                            _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]),
                            _ptr(g["ddelta_bias"]), _ptr(g["dinit"]), _ptr(saved),
                            0 if saved is None else saved.numel() * saved.element_size(), _stream(stream))
    if rc != MAMBA_OK:
        raise MambaError(rc, "mamba_scan_bwd")
    return g


def scan_step(state, u_t, delta_t, A, B_t, C_t, D=None, z_t=None, delta_bias=None, *, delta_softplus=True,
              exact_zoh=False, out=None, stream=None):
    """mamba_scan_step on torch tensors: state [B][D][N] float32 (updated in
    place), u_t/delta_t/z_t [B][D], B_t/C_t [B][N], A [D][N], D/delta_bias [D].
    Returns out [B][D]."""
    import torch
    ts = _foreign_stream(stream) if out is None else None
    if ts is not None:
        with torch.cuda.stream(ts):
            return scan_step(state, u_t, delta_t, A, B_t, C_t, D, z_t, delta_bias, delta_softplus=delta_softplus,
                             exact_zoh=exact_zoh, out=out, stream=ts)
    lib = load_library()
    dev = u_t.device
    dt = _dtype_code(u_t)
    tdt = u_t.dtype
    Bsz, Dm = u_t.shape
    N = B_t.shape[-1]
    _check(state, "state", (Bsz, Dm, N), torch.float32, dev)
    for name, t, shp in (("delta_t", delta_t, (Bsz, Dm)), ("B_t", B_t, (Bsz, N)), ("C_t", C_t, (Bsz, N)),
                         ("z_t", z_t, (Bsz, Dm))):
        _check(t, name, shp, tdt, dev)
    _check(A, "A", (Dm, N), torch.float32, dev)
    _check(D, "D", (Dm,), torch.float32, dev)
    _check(delta_bias, "delta_bias", (Dm,), torch.float32, dev)
    if out is None:
        out = torch.empty((Bsz, Dm), dtype=tdt, device=dev)
    _check(out, "out", (Bsz, Dm), tdt, dev)
    dims = make_dims(Bsz, Dm, 1, N, dt, delta_softplus=delta_softplus, exact_zoh=exact_zoh)
    rc = lib.mamba_scan_step(_ptr(state), _ptr(u_t), _ptr(delta_t), _ptr(A), _ptr(B_t), _ptr(C_t), _ptr(D),
                             _ptr(z_t), _ptr(delta_bias), ctypes.byref(dims), _ptr(out), _stream(stream))
    if rc != MAMBA_OK:
        raise MambaError(rc, "mamba_scan_step")
    return out


class ScanStepper:
    """Repeated mamba_scan_step calls of a decode loop [MFS §2.3]: the state,
    A, D and delta_bias, the options and the launch stream are checked and
    marshalled once here; each call then checks only its own [B][D] and
    [B][N] tensors (shape, dtype, contiguity, device) and makes one C call.
    state is updated in place on every call, as by scan_step.  stream: the
    launch stream (torch stream or raw handle), fixed at construction; None
    takes torch's current stream at construction time."""

    def __init__(self, state, A, D=None, delta_bias=None, *, dtype, delta_softplus=True, exact_zoh=False,
                 stream=None):
        import torch
        self._lib = load_library()
        dev = state.device
        if state.dim() != 3:
            raise ValueError("state must be [B][D][N], got %s" % (tuple(state.shape),))
        Bsz, Dm, N = state.shape
        dt = _dtype_code(torch.empty(0, dtype=dtype))
        _check(state, "state", (Bsz, Dm, N), torch.float32, dev)
        _check(A, "A", (Dm, N), torch.float32, dev)
        _check(D, "D", (Dm,), torch.float32, dev)
        _check(delta_bias, "delta_bias", (Dm,), torch.float32, dev)
        self._keep = (state, A, D, delta_bias)  # the pointers below stay valid while these live
        self._dims = make_dims(Bsz, Dm, 1, N, dt, delta_softplus=delta_softplus, exact_zoh=exact_zoh)
        self._dims_ref = ctypes.byref(self._dims)
        self._state, self._A, self._D, self._bias = _ptr(state), _ptr(A), _ptr(D), _ptr(delta_bias)
        self._stream = _stream(stream)
        self._bd = torch.Size((Bsz, Dm))
        self._bn = torch.Size((Bsz, N))
        self._dtype = dtype
        self._device = dev
        self._args = None

    def _ok(self, t, name, shape):
        if not (t.shape == shape and t.dtype == self._dtype and t.is_contiguous() and t.device == self._device):
            _check(t, name, shape, self._dtype, self._device)  # raises with the reason

    def bind(self, u_t, delta_t, B_t, C_t, z_t=None, *, out):
        """Checks and keeps one set of per-token buffers for step(): a decode
        loop that writes each token's u, delta, B, C (and z) into these same
        tensors then makes one C call per token, with no per-call checks."""
        bd, bn = self._bd, self._bn
        self._ok(u_t, "u_t", bd)
        self._ok(delta_t, "delta_t", bd)
        self._ok(B_t, "B_t", bn)
        self._ok(C_t, "C_t", bn)
        if z_t is not None:
            self._ok(z_t, "z_t", bd)
        self._ok(out, "out", bd)
        self._bound = (u_t, delta_t, B_t, C_t, z_t, out)  # kept alive with their pointers
        self._args = (self._state, u_t.data_ptr(), delta_t.data_ptr(), self._A, B_t.data_ptr(), C_t.data_ptr(),
                      self._D, None if z_t is None else z_t.data_ptr(), self._bias, self._dims_ref, out.data_ptr(),
                      self._stream)
        return self

    def step(self):
        """One step on the bound buffers (bind() first); returns the bound out."""
        if self._args is None:
            raise RuntimeError("ScanStepper.step() needs bind() first")
        rc = self._lib.mamba_scan_step(*self._args)
        if rc != MAMBA_OK:
            raise MambaError(rc, "mamba_scan_step")
        return self._bound[5]

    def __call__(self, u_t, delta_t, B_t, C_t, z_t=None, *, out):
        """One step: u_t, delta_t, z_t, out [B][D]; B_t, C_t [B][N]."""
        bd, bn = self._bd, self._bn
        self._ok(u_t, "u_t", bd)
        self._ok(delta_t, "delta_t", bd)
        self._ok(B_t, "B_t", bn)
        self._ok(C_t, "C_t", bn)
        if z_t is not None:
            self._ok(z_t, "z_t", bd)
        self._ok(out, "out", bd)
        rc = self._lib.mamba_scan_step(self._state, u_t.data_ptr(), delta_t.data_ptr(), self._A, B_t.data_ptr(),
                                       C_t.data_ptr(), self._D, None if z_t is None else z_t.data_ptr(),
                                       self._bias, self._dims_ref, out.data_ptr(), self._stream)
        if rc != MAMBA_OK:
            raise MambaError(rc, "mamba_scan_step")
        return out


def conv1d_silu(x, weight, bias=None, *, reverse=False, out=None, stream=None):
    """mamba_conv1d_silu on torch tensors: x [B][L][D] (bfloat16 or float32),
    weight [D][W] float32, bias [D] float32 or None.  Returns out [B][L][D]."""
    import torch
    ts = _foreign_stream(stream) if out is None else None
    if ts is not None:
        with torch.cuda.stream(ts):
            return conv1d_silu(x, weight, bias, reverse=reverse, out=out, stream=ts)
    lib = load_library()
    dev = x.device
    Bsz, L, Dm = x.shape
    if weight.dim() != 2 or weight.shape[0] != Dm:
        raise ValueError("weight must be [D][W], got %s" % (tuple(weight.shape),))
    W = weight.shape[1]
    _check(weight, "weight", (Dm, W), torch.float32, dev)
    _check(bias, "bias", (Dm,), torch.float32, dev)
    if out is None:
        out = torch.empty_like(x)
    _check(out, "out", (Bsz, L, Dm), x.dtype, dev)
    _check(x, "x", (Bsz, L, Dm), x.dtype, dev)
    dims = make_dims(Bsz, Dm, L, 1, _dtype_code(x))
    rc = lib.mamba_conv1d_silu(_ptr(x), _ptr(weight), _ptr(bias), ctypes.byref(dims), int(W), 1 if reverse else 0,
                               _ptr(out), _stream(stream))
    if rc != MAMBA_OK:
        raise MambaError(rc, "mamba_conv1d_silu")
    return out
