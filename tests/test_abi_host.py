"""Host-side checks of the C ABI (no GPU work): the library loads, exports every
function include/mamba_scan.h declares, sizes its workspace as a pure
function of the problem, and rejects invalid calls before touching the GPU."""
import ctypes
import os
import re

import pytest

import selective_state_space_mamba_amd as ms

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000  # 16-byte aligned stand-in pointer: every call below fails validation first


def header_functions():
    src = open(os.path.join(ROOT, "include", "mamba_scan.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mamba_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ms.LIB_PATH):
        from selective_state_space_mamba_amd import build
        build.build(force=False)
    return ms.load_library()


def test_exports_every_declared_function(lib):
    declared = header_functions()
    assert declared == sorted(ms.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_exports_nothing_else(lib):
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", ms.LIB_PATH], stdout=subprocess.PIPE, text=True,
                         check=True).stdout
    text_syms = sorted(line.split()[-1] for line in out.splitlines() if line.split()[1:2] == ["T"])
    assert text_syms == header_functions()


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, 7):
        assert len(ms.status_string(code)) > 0
    assert ms.status_string(0) == "ok"


def dims(**kw):
    base = dict(batch=2, dim=64, seqlen=100, dstate=16, dtype=ms.DTYPE_BF16)
    base.update(kw)
    return ms.make_dims(base.pop("batch"), base.pop("dim"), base.pop("seqlen"), base.pop("dstate"),
                        base.pop("dtype"), **base)


def test_workspace_bytes_pure_function(lib):
    assert ms.workspace_bytes(dims(), ms.DIR_FWD) == 0  # short sequence, enough rows: no split
    bi = ms.workspace_bytes(dims(), ms.DIR_BIDIR)
    assert bi >= 2 * 2 * 100 * 64 * 4  # per-direction fp32 rows
    assert ms.workspace_bytes(dims(), ms.DIR_BIDIR) == bi
    cross = ms.workspace_bytes(dims(seqlen=96, height=8, width=12), ms.DIR_CROSS2D)
    assert cross >= 4 * 2 * 96 * 64 * 4
    # a long sequence with few rows is split in time: aggregate state + ΣΔ per chunk
    long = ms.workspace_bytes(dims(batch=1, seqlen=1 << 16), ms.DIR_FWD)
    assert long > 0 and long % 256 == 0
    with pytest.raises(ms.MambaError):
        ms.workspace_bytes(dims(seqlen=0), ms.DIR_FWD)


def call_fwd(lib, d, mode=ms.DIR_FWD, **ptrs):
    p = dict(u=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, z=None, bias=None, out=FAKE, last=None)
    p.update(ptrs)
    return lib.mamba_scan_fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["bias"],
                              ctypes.byref(d), mode, p["out"], p["last"], None)


def test_fwd_validation(lib):
    assert call_fwd(lib, dims(), u=None) == ms._binding.MAMBA_ERR_INVALID
    assert call_fwd(lib, dims(), out=None) == ms._binding.MAMBA_ERR_INVALID
    assert call_fwd(lib, dims(batch=0)) == ms._binding.MAMBA_ERR_INVALID
    assert call_fwd(lib, dims(seqlen=-3)) == ms._binding.MAMBA_ERR_INVALID
    assert call_fwd(lib, dims(dtype=5)) == ms._binding.MAMBA_ERR_INVALID
    assert call_fwd(lib, dims(), mode=9) == ms._binding.MAMBA_ERR_INVALID
    assert call_fwd(lib, dims(seqlen=96, height=8, width=11), mode=ms.DIR_CROSS2D) == ms._binding.MAMBA_ERR_INVALID
    assert call_fwd(lib, dims(seqlen=96), mode=ms.DIR_CROSS2D) == ms._binding.MAMBA_ERR_INVALID
    # any state size 1..64 and (float32) any channel count that is a multiple of 4
    for n in (1, 3, 12, 24, 48, 63, 64):
        assert ms.workspace_bytes(dims(dstate=n), ms.DIR_FWD) >= 0
    assert ms.workspace_bytes(dims(dim=36, dtype=ms.DTYPE_F32), ms.DIR_FWD) >= 0
    assert call_fwd(lib, dims(dstate=65)) == ms._binding.MAMBA_ERR_UNSUPPORTED
    assert call_fwd(lib, dims(dim=34, dtype=ms.DTYPE_F32)) == ms._binding.MAMBA_ERR_UNSUPPORTED
    assert call_fwd(lib, dims(dim=36, dtype=ms.DTYPE_BF16)) == ms._binding.MAMBA_ERR_UNSUPPORTED
    # 32-bit slice offsets: (seqlen + 64) * dim * sizeof(dtype) must stay below 2^31 bytes
    dim = 1 << 16
    lmax = (2**31 - 1) // (dim * 2) - 64
    assert ms.workspace_bytes(dims(batch=1, dim=dim, seqlen=lmax), ms.DIR_FWD) >= 0
    assert call_fwd(lib, dims(batch=1, dim=dim, seqlen=lmax + 1)) == ms._binding.MAMBA_ERR_UNSUPPORTED
    # token indices and row strides are 24-bit multiply operands: seqlen and dim * 4 below 2^24
    assert ms.workspace_bytes(dims(batch=1, dim=8, seqlen=(1 << 24) - 1), ms.DIR_FWD) >= 0
    assert call_fwd(lib, dims(batch=1, dim=8, seqlen=1 << 24)) == ms._binding.MAMBA_ERR_UNSUPPORTED
    assert ms.workspace_bytes(dims(batch=1, dim=(1 << 22) - 8, seqlen=64), ms.DIR_FWD) >= 0
    assert call_fwd(lib, dims(batch=1, dim=1 << 22, seqlen=64)) == ms._binding.MAMBA_ERR_UNSUPPORTED
    assert call_fwd(lib, dims(dstate=128)) == ms._binding.MAMBA_ERR_UNSUPPORTED
    assert call_fwd(lib, dims(dim=60)) == ms._binding.MAMBA_ERR_UNSUPPORTED
    assert call_fwd(lib, dims(), u=FAKE + 4) == ms._binding.MAMBA_ERR_UNSUPPORTED
    assert call_fwd(lib, dims(), z=FAKE + 2) == ms._binding.MAMBA_ERR_UNSUPPORTED
    # multi-direction modes need the workspace
    assert call_fwd(lib, dims(), mode=ms.DIR_BIDIR) == ms._binding.MAMBA_ERR_WORKSPACE
    d = dims(workspace=FAKE, workspace_bytes=16)
    assert call_fwd(lib, d, mode=ms.DIR_BIDIR) == ms._binding.MAMBA_ERR_WORKSPACE


def test_step_validation(lib):
    def step(d, **ptrs):
        p = dict(state=FAKE, u=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, out=FAKE)
        p.update(ptrs)
        return lib.mamba_scan_step(p["state"], p["u"], p["delta"], p["A"], p["B"], p["C"], None, None, None,
                                   ctypes.byref(d), p["out"], None)
    assert step(dims(), state=None) == ms._binding.MAMBA_ERR_INVALID
    assert step(dims(dim=0)) == ms._binding.MAMBA_ERR_INVALID
    assert step(dims(dstate=65)) == ms._binding.MAMBA_ERR_UNSUPPORTED
    assert step(dims(dim=36)) == ms._binding.MAMBA_ERR_UNSUPPORTED  # bf16: a multiple of 8
    assert step(dims(), B=FAKE + 8) == ms._binding.MAMBA_ERR_UNSUPPORTED
    assert lib.mamba_scan_step(None, None, None, None, None, None, None, None, None, None, None, None) == \
        ms._binding.MAMBA_ERR_INVALID


def test_conv1d_validation(lib):
    d = dims(dim=64, seqlen=10)
    conv = lambda dd, width=4, x=FAKE, w=FAKE, b=None, out=FAKE: lib.mamba_conv1d_silu(
        x, w, b, ctypes.byref(dd), width, 0, out, None)
    assert conv(d, x=None) == ms._binding.MAMBA_ERR_INVALID
    assert conv(d, w=None) == ms._binding.MAMBA_ERR_INVALID
    assert conv(d, out=None) == ms._binding.MAMBA_ERR_INVALID
    assert conv(d, width=0) == ms._binding.MAMBA_ERR_INVALID
    assert conv(dims(dim=64, seqlen=0)) == ms._binding.MAMBA_ERR_INVALID
    assert conv(dims(dim=64, dtype=7)) == ms._binding.MAMBA_ERR_INVALID
    assert conv(d, width=5) == ms._binding.MAMBA_ERR_UNSUPPORTED
    assert conv(dims(dim=60)) == ms._binding.MAMBA_ERR_UNSUPPORTED
    assert conv(d, x=FAKE + 8) == ms._binding.MAMBA_ERR_UNSUPPORTED
    assert conv(d, w=FAKE + 2) == ms._binding.MAMBA_ERR_UNSUPPORTED


def test_bwd_workspace_and_validation(lib):
    d = dims()
    need = ms.bwd_workspace_bytes(d, ms.DIR_FWD)
    # at least: per-direction fp32 rows, 32-step checkpoints, dB/dC partials per 16-channel block
    L, Dm, N, Bz = 100, 64, 16, 2
    assert need >= 4 * (Bz * L * Dm + Bz * 4 * Dm * N + 2 * (Dm // 16) * Bz * L * N)
    assert need % 256 == 0 and ms.bwd_workspace_bytes(d, ms.DIR_FWD) == need
    cross = ms.bwd_workspace_bytes(dims(seqlen=96, height=8, width=12), ms.DIR_CROSS2D)
    assert cross >= 4 * 4 * Bz * 96 * Dm * 2  # per-direction rows and per-direction du
    assert ms.bwd_workspace_bytes(dims(dstate=32), ms.DIR_FWD) > need  # N = 32 is built
    assert ms.bwd_workspace_bytes(dims(dstate=12), ms.DIR_FWD) > 0  # any N up to 64
    # above 32 states: groups of 16 states, with fp32 parts of du and ddelta per group
    n64 = ms.bwd_workspace_bytes(dims(dstate=64), ms.DIR_FWD)
    assert n64 >= 4 * (2 * 4 * Bz * L * Dm + 2 * (Dm // 16) * Bz * L * 64)
    assert ms.bwd_workspace_bytes(dims(dstate=33), ms.DIR_FWD) > 0
    for bad in (dims(dstate=65), dims(seqlen=0), dims(dim=60), dims(dim=36, dtype=ms.DTYPE_F32)):
        with pytest.raises(ms.MambaError):
            ms.bwd_workspace_bytes(bad, ms.DIR_FWD)

    def bwd(dd, mode=ms.DIR_FWD, **ptrs):
        p = dict(u=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, z=None, bias=None, dout=FAKE, du=FAKE,
                 ddelta=FAKE, dA=FAKE, dB=FAKE, dC=FAKE, dD=None, dz=None, dbias=None, dinit=None, saved=None,
                 saved_bytes=0)
        p.update(ptrs)
        return lib.mamba_scan_bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["bias"], p["dout"],
                                  ctypes.byref(dd), mode, p["du"], p["ddelta"], p["dA"], p["dB"], p["dC"], p["dD"],
                                  p["dz"], p["dbias"], p["dinit"], p["saved"], p["saved_bytes"], None)
    E = ms._binding
    assert bwd(d, dout=None) == E.MAMBA_ERR_INVALID
    assert bwd(d, dB=None) == E.MAMBA_ERR_INVALID
    assert bwd(dims(batch=0)) == E.MAMBA_ERR_INVALID
    assert bwd(d, mode=7) == E.MAMBA_ERR_INVALID
    assert bwd(dims(dstate=65)) == E.MAMBA_ERR_UNSUPPORTED
    assert bwd(dims(dstate=40)) == E.MAMBA_ERR_WORKSPACE  # built (state groups); no workspace given
    assert bwd(dims(dim=36, dtype=ms.DTYPE_F32)) == E.MAMBA_ERR_UNSUPPORTED  # forward-only channel count
    assert bwd(d, dz=FAKE + 2) == E.MAMBA_ERR_UNSUPPORTED
    assert bwd(d) == E.MAMBA_ERR_WORKSPACE  # the backward pass always needs its workspace
    assert bwd(dims(workspace=FAKE, workspace_bytes=need - 256)) == E.MAMBA_ERR_WORKSPACE
    # a saved forward state too small for the call (with z and dz it must hold the rows), or misaligned
    ws = dict(workspace=FAKE, workspace_bytes=need)
    ck = ms.saved_bytes(d, ms.DIR_FWD, False)
    assert bwd(dims(**ws), saved=FAKE, saved_bytes=ck - 4) == E.MAMBA_ERR_WORKSPACE
    assert bwd(dims(**ws), saved=FAKE, saved_bytes=ck, z=FAKE, dz=FAKE) == E.MAMBA_ERR_WORKSPACE
    assert bwd(dims(**ws), saved=FAKE + 8, saved_bytes=10 * ck) == E.MAMBA_ERR_WORKSPACE


def test_saved_state_size_and_fwd_save_validation(lib):
    L, Dm, N, Bz = 100, 64, 16, 2
    d = dims()
    ck = ms.saved_bytes(d, ms.DIR_FWD, False)
    # the state before every 16th position (ceil(L/16) of them at N <= 16), 256-byte aligned, then the
    # fp32 output rows
    assert ck == (Bz * 7 * Dm * N * 4 + 255) // 256 * 256
    assert ms.saved_bytes(d, ms.DIR_FWD, True) == ck + Bz * L * Dm * 4
    cross = dims(seqlen=96, height=8, width=12)
    assert ms.saved_bytes(cross, ms.DIR_CROSS2D, True) == 4 * Bz * 6 * Dm * N * 4 + 4 * Bz * 96 * Dm * 4
    # 17..32 states, every 32nd position; above 32 (state groups of 16), every 16th again
    assert ms.saved_bytes(dims(dstate=32), ms.DIR_FWD, False) == (Bz * 4 * Dm * 32 * 4 + 255) // 256 * 256
    assert ms.saved_bytes(dims(dstate=48), ms.DIR_FWD, False) == (Bz * 7 * Dm * 48 * 4 + 255) // 256 * 256
    for bad in (dims(dstate=65), dims(seqlen=0), dims(dim=60)):
        with pytest.raises(ms.MambaError):
            ms.saved_bytes(bad, ms.DIR_FWD, False)

    def fwd_save(dd, mode=ms.DIR_FWD, **ptrs):
        p = dict(u=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, z=None, bias=None, out=FAKE, last=None,
                 saved=FAKE, saved_bytes=ck)
        p.update(ptrs)
        return lib.mamba_scan_fwd_save(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["bias"],
                                       ctypes.byref(dd), mode, p["out"], p["last"], p["saved"], p["saved_bytes"],
                                       None)
    E = ms._binding
    assert fwd_save(d, saved=None) == E.MAMBA_ERR_INVALID
    assert fwd_save(d, out=None) == E.MAMBA_ERR_INVALID
    assert fwd_save(dims(batch=0)) == E.MAMBA_ERR_INVALID
    assert fwd_save(dims(dstate=65)) == E.MAMBA_ERR_UNSUPPORTED  # what the backward pass cannot read
    assert fwd_save(dims(dstate=48)) == E.MAMBA_ERR_WORKSPACE  # built; ck is too small for 48 states
    assert fwd_save(d, saved=FAKE + 4) == E.MAMBA_ERR_UNSUPPORTED
    assert fwd_save(d, saved_bytes=ck - 1) == E.MAMBA_ERR_WORKSPACE
    assert fwd_save(d, z=FAKE) == E.MAMBA_ERR_WORKSPACE  # with a gate the rows are saved too
    assert fwd_save(d, mode=ms.DIR_BIDIR, saved_bytes=10 ** 9) == E.MAMBA_ERR_WORKSPACE  # the forward's own


def test_binding_rejects_scattered_buffers(lib):
    """The torch binding passes a caller's workspace and saved-state buffers on
    as plain byte ranges, so it refuses a non-contiguous view before any call
    into the library (CPU tensors: the check comes first)."""
    import torch
    Bz, L, Dm, N = 1, 64, 8, 4
    u = torch.zeros(Bz, L, Dm)
    A = -torch.ones(Dm, N)
    Bm = torch.zeros(Bz, L, N)
    scattered = torch.zeros(64, 8, dtype=torch.uint8).t()
    assert not scattered.is_contiguous()
    with pytest.raises(ValueError, match="workspace must be contiguous"):
        ms.scan_fwd(u, u, A, Bm, Bm, workspace=scattered)
    with pytest.raises(ValueError, match="saved must be contiguous"):
        ms.scan_fwd_save(u, u, A, Bm, Bm, saved=scattered)
    with pytest.raises(ValueError, match="workspace must be contiguous"):
        ms.scan_bwd(u, u, A, Bm, Bm, dout=u, workspace=scattered)


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU: --gpus above 1 (or a multi-rank launch) exits
    with a message before touching a GPU."""
    import subprocess
    import sys
    for args, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True, text=True,
                           env=dict(os.environ, **env), timeout=120)
        assert r.returncode == 2, (args, env, r.returncode)
        assert "measures one GPU" in r.stderr
        assert r.stdout == ""


def test_fwd_noalloc_validation(lib):
    """mamba_scan_fwd_noalloc validates like mamba_scan_fwd, ignores the dims'
    workspace, and refuses (before any GPU work) a problem whose scratch would
    not fit the library's static array."""
    E = ms._binding

    def call(d, mode=ms.DIR_FWD, **ptrs):
        p = dict(u=FAKE, delta=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, z=None, bias=None, out=FAKE, last=None)
        p.update(ptrs)
        return lib.mamba_scan_fwd_noalloc(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["bias"],
                                          ctypes.byref(d), mode, p["out"], p["last"], None)
    assert call(dims(), u=None) == E.MAMBA_ERR_INVALID
    assert call(dims(batch=0)) == E.MAMBA_ERR_INVALID
    assert call(dims(), mode=9) == E.MAMBA_ERR_INVALID
    assert call(dims(dim=60)) == E.MAMBA_ERR_UNSUPPORTED
    assert call(dims(), u=FAKE + 4) == E.MAMBA_ERR_UNSUPPORTED
    # the scratch limit: per-direction fp32 rows of a bidirectional scan, K*B*L*D*4 bytes
    cap = E.NOALLOC_SCRATCH_BYTES
    big = dims(batch=1, dim=1024, seqlen=cap // (2 * 1024 * 4) + 64)
    assert ms.workspace_bytes(big, ms.DIR_BIDIR) > cap
    assert call(big, mode=ms.DIR_BIDIR) == E.MAMBA_ERR_SCRATCH
    # the workspace fields are ignored: a workspace that mamba_scan_fwd would
    # accept does not lift the limit
    need = ms.workspace_bytes(big, ms.DIR_BIDIR)
    big.workspace, big.workspace_bytes = FAKE, need
    assert call(big, mode=ms.DIR_BIDIR) == E.MAMBA_ERR_SCRATCH
    assert "static scratch" in ms.status_string(E.MAMBA_ERR_SCRATCH)
