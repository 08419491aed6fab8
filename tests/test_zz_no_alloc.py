"""GPU check of mamba_scan_fwd_noalloc: the forward pass whose scratch comes
from the library's static device array.  Called through the C ABI, it must
give exactly what mamba_scan_fwd (same kernels, caller-owned workspace) gives,
on two calls in a row, the second with a smaller problem, each of which needs
scratch (per-direction rows and time-split carries)."""
import numpy as np
import pytest

import selective_state_space_mamba_amd as ms
from selective_state_space_mamba_amd import inputs as I

from scanutil import assert_close, dev_inputs, from_dev, oracle_fwd, torch

pytestmark = pytest.mark.gpu

CASES = [
    # bidirectional, long enough to be split in time: rows and carries in the scratch
    I.Workload("noalloc_split_bidir_f32", 1, 64, 8500, 16, I.DIR_BIDIR, "f32", True, 401),
    # then a smaller cross scan (rows only), on the same static array
    I.Workload("noalloc_cross2d_bf16", 2, 64, 240, 16, I.DIR_CROSS2D, "bf16", False, 402, 12, 20),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    ms.load_library()
    yield


def _run(w, x, noalloc, stream):
    t = torch()
    xd = dev_inputs(x)
    K = w.ndirs
    out = t.empty((w.batch, w.seqlen, w.dim), dtype=xd["u"].dtype, device="cuda:0")
    st = t.empty((w.batch,) + (() if K == 1 else (K,)) + (w.dim, w.dstate), dtype=t.float32, device="cuda:0")
    out.fill_(7.0)
    st.fill_(7.0)
    fn = ms.scan_fwd_noalloc if noalloc else ms.scan_fwd
    with t.cuda.stream(stream):
        fn(xd["u"], xd["delta"], xd["A"], xd["B"], xd["C"], xd.get("D"), xd.get("z"), xd.get("delta_bias"),
           dir_mode=w.dir_mode, height=w.height, width=w.width, out=out, last_state=st, stream=stream)
    t.cuda.synchronize()
    return out, st


def test_noalloc_matches_fwd_on_two_calls():
    t = torch()
    stream = t.cuda.Stream()
    for i, w in enumerate(CASES):
        print("[gpu case] noalloc call %d: %s" % (i + 1, w), flush=True)
        need = ms.workspace_bytes(ms.make_dims(w.batch, w.dim, w.seqlen, w.dstate,
                                               ms.DTYPE_BF16 if w.dtype == "bf16" else ms.DTYPE_F32,
                                               height=w.height, width=w.width), w.dir_mode)
        assert 0 < need <= ms._binding.NOALLOC_SCRATCH_BYTES
        if i > 0:
            assert need < prev_need  # the second call is the smaller one
        prev_need = need
        x = I.make_inputs(w)
        out_s, st_s = _run(w, x, True, stream)
        out_w, st_w = _run(w, x, False, stream)
        assert t.equal(out_s.view(t.int16) if out_s.dtype == t.bfloat16 else out_s,
                       out_w.view(t.int16) if out_w.dtype == t.bfloat16 else out_w), w.name
        assert t.equal(st_s, st_w), w.name
        # and both meet the oracle (the parity bar of every forward test)
        ref_out, ref_st = oracle_fwd(w, x)
        assert_close(w.name + " out", from_dev(out_s), ref_out, w.dtype)
        assert_close(w.name + " last_state", from_dev(st_s), ref_st.reshape(tuple(st_s.shape)), w.dtype)


def test_noalloc_rejects_oversized_problem():
    t = torch()
    w = I.Workload("noalloc_too_big", 1, 1024, 4200, 16, I.DIR_BIDIR, "bf16", True, 403)
    d = ms.make_dims(w.batch, w.dim, w.seqlen, w.dstate, ms.DTYPE_BF16)
    assert ms.workspace_bytes(d, w.dir_mode) > ms._binding.NOALLOC_SCRATCH_BYTES
    u = t.zeros((1, 2, w.seqlen, w.dim), dtype=t.bfloat16, device="cuda:0")
    A = -t.ones((2, w.dim, w.dstate), dtype=t.float32, device="cuda:0")
    Bm = t.zeros((1, 2, w.seqlen, w.dstate), dtype=t.bfloat16, device="cuda:0")
    out = t.empty((1, w.seqlen, w.dim), dtype=t.bfloat16, device="cuda:0")
    with pytest.raises(ms.MambaError) as ei:
        ms.scan_fwd_noalloc(u, u, A, Bm, Bm, dir_mode=w.dir_mode, out=out)
    assert ei.value.code == ms._binding.MAMBA_ERR_SCRATCH
