"""GPU parity of the causal depthwise Conv1d + SiLU prologue (through the C ABI)
against the fp64 CPU oracle on the same seeded inputs, and of the prologue
feeding the scan.

Sources, cited by page title and section:
  [MFS] "从零理解 Mamba：选择性状态空间模型（Selective SSM）到 Mamba Block" (eutaboo.com):
        §6.2 Step 2, §8 (d_conv = 4)
  [VIM] "Vision Mamba：从状态空间模型到视觉革命的跨越" (x-humanoid.csdn.net): §2.2
"""
import numpy as np
import pytest

import oracle
import selective_state_space_mamba_amd as ms
from selective_state_space_mamba_amd import inputs as I

from scanutil import assert_close, dev_inputs, from_dev, gpu_fwd, oracle_fwd, to_dev, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    ms.load_library()
    yield


def run_conv(Bsz, L, Dm, W, dtype, seed, reverse=False, with_bias=True):
    x = I.make_conv_inputs(Bsz, L, Dm, W, dtype, seed)
    bias = x["bias"] if with_bias else None
    print("[gpu case] conv B=%d L=%d D=%d W=%d %s reverse=%s bias=%s" % (Bsz, L, Dm, W, dtype, reverse, with_bias),
          flush=True)
    got = ms.conv1d_silu(to_dev(x["x"]), to_dev(x["weight"]), to_dev(bias), reverse=reverse)
    torch().cuda.synchronize()
    want = oracle.conv1d(x["x"], x["weight"], bias, reverse=reverse)
    assert_close("conv", from_dev(got), want, dtype)
    return x, got, want


@pytest.mark.parametrize("W", [1, 2, 3, 4])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("reverse", [False, True])
def test_conv_parity(W, dtype, reverse):
    run_conv(2, 77, 72, W, dtype, 200 + W, reverse=reverse)


def test_conv_no_bias_long_ragged():
    run_conv(3, 300, 136, 4, "bf16", 211, with_bias=False)
    run_conv(1, 33, 8, 4, "f32", 212)
    run_conv(1, 1, 16, 4, "f32", 213)


def test_conv_rejects_unsupported():
    x = to_dev(np.zeros((1, 8, 16), np.float32))
    w5 = to_dev(np.zeros((16, 5), np.float32))
    with pytest.raises(ms.MambaError):
        ms.conv1d_silu(x, w5)


def test_conv_full_size_mamba130m():
    w = I.WORKLOADS["mamba130m_layer"]
    run_conv(w.batch, w.seqlen, w.dim, 4, "bf16", 214)


def test_conv_feeds_the_scan():
    """u = silu(conv(x)) on the GPU, then the scan, against the oracle's conv
    (rounded to the input type as the GPU stores it) then the oracle's scan."""
    w = I.Workload("conv_scan", 2, 72, 150, 16, I.DIR_FWD, "bf16", True, 215)
    xin = I.make_inputs(w)
    cx = I.make_conv_inputs(w.batch, w.seqlen, w.dim, 4, w.dtype, 216)
    u_dev = ms.conv1d_silu(to_dev(cx["x"]), to_dev(cx["weight"]), to_dev(cx["bias"]))
    xd = dev_inputs(xin)
    xd["u"] = u_dev
    out, st = gpu_fwd(w, xd)
    u_ref = I.bf16_bits(oracle.conv1d(cx["x"], cx["weight"], cx["bias"]).astype(np.float32))
    ref = dict(xin)
    ref["u"] = u_ref
    ref_out, ref_st = oracle_fwd(w, ref)
    assert_close("conv+scan out", from_dev(out), ref_out, "bf16")
    assert_close("conv+scan state", from_dev(st), ref_st[:, 0], "bf16")
