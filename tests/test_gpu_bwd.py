"""GPU parity of the backward pass (mamba_scan_bwd, through the C ABI) against
the fp64 backward oracle on the same seeded inputs.

The training pass recomputes the states and runs the adjoint recurrence
[MFS §5; S4M §2.3].  Small cases span several 16-channel blocks and 32-step
segments with ragged tails, every direction mode, state sizes 1..64 (above 32 in
groups of 16 states, the last one partial at 33 and 40), both
input-term rules, softplus on and off, the optional gate, skip, bias and
initial state, and the time-split forward recompute.  The specified workloads
run at full size, checked on a channel subset over the whole batch (every
per-channel gradient, dA, dD, ddelta_bias included) and on whole batch items
(dB, dC, which sum over every channel).
Sources, cited by page title and section:
  [MFS] "从零理解 Mamba：选择性状态空间模型（Selective SSM）到 Mamba Block" (eutaboo.com)
  [S4M] "从S4到Mamba：选择性状态空间模型的演进与革新" (jsqmd.com)
"""
import numpy as np
import pytest

import oracle
import selective_state_space_mamba_amd as ms
from selective_state_space_mamba_amd import inputs as I

from scanutil import assert_close, dev_inputs, from_dev, saturate, to_dev, torch

pytestmark = pytest.mark.gpu

# gradients in the element type of their input, and the float32 ones
TYPED = ("du", "ddelta", "dB", "dC", "dz")
FP32 = ("dA", "dD", "ddelta_bias", "dinit")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    ms.load_library()  # fails loudly when the HIP library is missing
    yield


def announce(msg):
    print("[gpu case] " + msg, flush=True)


def init_state(w, seed):
    K = w.ndirs
    kx = () if K == 1 else (K,)
    r = np.random.Generator(np.random.PCG64([seed, 3]))
    return r.standard_normal((w.batch,) + kx + (w.dim, w.dstate)).astype(np.float32)


def gpu_bwd(w, x, dout, *, softplus=True, exact=False, init=None):
    xd = dev_inputs(x)
    g = ms.scan_bwd(xd["u"], xd["delta"], xd["A"], xd["B"], xd["C"], xd.get("D"), xd.get("z"), xd.get("delta_bias"),
                    dout=to_dev(dout), dir_mode=w.dir_mode, height=w.height, width=w.width,
                    delta_softplus=softplus, exact_zoh=exact, initial_state=to_dev(init))
    torch().cuda.synchronize()
    return {k: (None if v is None else from_dev(v)) for k, v in g.items()}


def oracle_bwd(w, x, dout, *, softplus=True, exact=False, init=None, height=None, width=None):
    return oracle.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x.get("D"), x.get("z"), x.get("delta_bias"),
                           dout=dout, dir_mode=w.dir_mode, height=w.height if height is None else height,
                           width=w.width if width is None else width, delta_softplus=softplus, exact_zoh=exact,
                           initial_state=init)


def compare(name, w, got, ref, keys=TYPED + FP32, index=None):
    for k in keys:
        if ref.get(k) is None or got.get(k) is None:
            assert got.get(k) is None or ref.get(k) is None
            continue
        gv = got[k] if index is None else index(k, got[k])
        rv = ref[k].reshape(gv.shape)
        assert_close("%s %s" % (name, k), gv, rv, w.dtype if k in TYPED else "f32")


W = I.Workload
SMALL = [
    # name, workload, softplus, exact, init, D/bias present
    ("fwd_bf16", W("fwd_bf16", 2, 40, 100, 16, I.DIR_FWD, "bf16", True, 31), True, False, False, True),
    ("fwd_f32_n4_exact_init", W("fwd_f32_n4", 1, 24, 77, 4, I.DIR_FWD, "f32", True, 32), True, True, True, True),
    ("bwd_bf16_n8", W("bwd_bf16_n8", 2, 32, 70, 8, I.DIR_BWD, "bf16", True, 33), True, False, True, True),
    ("bidir_f32_init", W("bidir_f32", 2, 16, 45, 16, I.DIR_BIDIR, "f32", True, 34), True, False, True, True),
    ("bidir_bf16_n2", W("bidir_bf16_n2", 1, 48, 64, 2, I.DIR_BIDIR, "bf16", False, 35), True, False, False, True),
    ("cross2d_bf16", W("cross2d_bf16", 2, 32, 45, 16, I.DIR_CROSS2D, "bf16", False, 36, 5, 9), True, False, False,
     True),
    ("cross2d_f32_n1_gated", W("cross2d_f32_n1", 1, 16, 66, 1, I.DIR_CROSS2D, "f32", True, 37, 11, 6), True, False,
     True, True),
    ("cross2d_f32_exact", W("cross2d_f32_ex", 1, 16, 36, 4, I.DIR_CROSS2D, "f32", True, 41, 6, 6), True, True, True,
     True),
    ("fwd_f32_nosoftplus_noskip", W("fwd_f32_nsp", 1, 16, 33, 16, I.DIR_FWD, "f32", False, 38), False, False, False,
     False),
    ("split_fwd_bf16", W("split_fwd_bf16", 1, 64, 4133, 16, I.DIR_FWD, "bf16", True, 39), True, False, True, True),
    ("split_bidir_f32", W("split_bidir_f32", 1, 16, 2500, 8, I.DIR_BIDIR, "f32", True, 42), True, True, False, True),
    # edge cases: one position, half a channel block, segment boundaries, a one-row grid
    ("L1_D8_bf16_n2", W("L1_D8", 1, 8, 1, 2, I.DIR_FWD, "bf16", True, 44), True, False, True, True),
    ("L31_bidir_f32", W("L31_bidir", 2, 24, 31, 16, I.DIR_BIDIR, "f32", True, 45), True, False, False, True),
    ("L33_bwd_bf16_n4", W("L33_bwd", 3, 40, 33, 4, I.DIR_BWD, "bf16", False, 46), True, False, True, True),
    ("L32_fwd_f32_n1", W("L32_fwd", 1, 16, 32, 1, I.DIR_FWD, "f32", True, 47), True, False, False, False),
    ("grid_1x37_f32", W("grid_1x37", 1, 16, 37, 8, I.DIR_CROSS2D, "f32", True, 48, 1, 37), True, False, True, True),
    ("exact_nosoftplus_init_bf16", W("ex_nsp", 2, 32, 65, 16, I.DIR_FWD, "bf16", True, 49), False, True, True, True),
    ("n32_fwd_bf16_init", W("n32_fwd", 2, 40, 90, 32, I.DIR_FWD, "bf16", True, 55), True, False, True, True),
    ("n32_bidir_f32_exact", W("n32_bidir", 1, 24, 70, 32, I.DIR_BIDIR, "f32", True, 56), True, True, False, True),
    ("n32_cross2d_bf16", W("n32_cross", 1, 16, 48, 32, I.DIR_CROSS2D, "bf16", True, 57, 6, 8), True, False, False,
     True),
    ("n32_split_fwd_f32", W("n32_split", 1, 16, 2300, 32, I.DIR_FWD, "f32", True, 58), True, False, True, True),
    ("n3_fwd_f32_init", W("n3_fwd", 2, 24, 70, 3, I.DIR_FWD, "f32", True, 59), True, False, True, True),
    ("n12_bidir_bf16", W("n12_bidir", 1, 40, 66, 12, I.DIR_BIDIR, "bf16", True, 60), True, False, False, True),
    ("n24_cross2d_f32_exact", W("n24_cross", 1, 16, 42, 24, I.DIR_CROSS2D, "f32", True, 62, 6, 7), True, True,
     False, True),
    ("n20_split_bwd_bf16", W("n20_split", 1, 16, 2200, 20, I.DIR_BWD, "bf16", True, 63), True, False, True, True),
    # above 32 states: groups of 16 states (the last group partial at 33 and 40)
    ("n64_fwd_bf16_init", W("n64_fwd", 2, 40, 90, 64, I.DIR_FWD, "bf16", True, 64), True, False, True, True),
    ("n48_bidir_f32_exact", W("n48_bidir", 1, 24, 70, 48, I.DIR_BIDIR, "f32", True, 65), True, True, False, True),
    ("n40_cross2d_bf16_init", W("n40_cross", 1, 16, 48, 40, I.DIR_CROSS2D, "bf16", True, 66, 6, 8), True, False,
     True, True),
    ("n33_fwd_f32_nosoftplus", W("n33_fwd", 2, 24, 41, 33, I.DIR_FWD, "f32", True, 67), False, False, False, True),
    ("n64_split_bwd_f32", W("n64_split", 1, 16, 2300, 64, I.DIR_BWD, "f32", True, 68), True, False, True, True),
    # the forward recompute in 64-position tiles (checkpoints inside the tile)
    ("t64_fwd_bf16_init", W("t64_fwd", 2, 40, 1100, 16, I.DIR_FWD, "bf16", True, 69), True, False, True, True),
    ("t64_cross2d_f32", W("t64_cross", 1, 16, 1024, 16, I.DIR_CROSS2D, "f32", True, 70, 32, 32), True, False, False,
     True),
]


def small_inputs(case):
    name, w, softplus, exact, with_init, skip = case
    x = I.make_inputs(w)
    if not skip:
        x["D"] = None
        x["delta_bias"] = None
    if not softplus:  # Δ = delta itself: keep it positive
        r = np.random.Generator(np.random.PCG64([w.seed, 4]))
        dl = r.uniform(0.01, 0.3, x["delta"].shape).astype(np.float32)
        x["delta"] = I.bf16_bits(dl) if w.dtype == "bf16" else dl
        if x["delta_bias"] is not None:  # the inverse-softplus bias would make Δ negative
            x["delta_bias"] = r.uniform(0.0, 0.05, x["delta_bias"].shape).astype(np.float32)
    dout = I.make_dout(w)
    init = init_state(w, w.seed) if with_init else None
    return x, dout, init


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_bwd_small(case):
    name, w, softplus, exact, with_init, skip = case
    announce("bwd %s %s softplus=%s exact=%s init=%s" % (name, w, softplus, exact, with_init))
    x, dout, init = small_inputs(case)
    got = gpu_bwd(w, x, dout, softplus=softplus, exact=exact, init=init)
    ref = oracle_bwd(w, x, dout, softplus=softplus, exact=exact, init=init)
    compare(name, w, got, ref)


def test_bwd_exact_mixed_A():
    """Exact rule with A = 0 and |ΔA| around the series switch."""
    w = W("exact_mixedA", 2, 32, 100, 16, I.DIR_FWD, "bf16", True, 40)
    announce("bwd %s" % (w,))
    x = I.make_inputs(w)
    A = x["A"].copy()
    A[:, 0::4] = 0.0
    A[:, 1::4] = -1e-3
    A[:, 2::4] = -3.0
    x["A"] = A
    dout = I.make_dout(w)
    got = gpu_bwd(w, x, dout, exact=True)
    ref = oracle_bwd(w, x, dout, exact=True)
    compare("exact_mixedA", w, got, ref)


@pytest.mark.parametrize("case", [SMALL[0], SMALL[3], SMALL[6]], ids=["fwd_bf16", "bidir_f32", "cross2d_f32_n1"])
def test_bwd_saturated_softplus_and_gate(case):
    """Every gradient with Δraw and z far outside their usual range (softplus
    underflowing and past its clamp, the gate's exponential overflowing)."""
    name, w, softplus, exact, with_init, skip = case
    announce("bwd saturated %s %s" % (name, w))
    x, dout, init = small_inputs(case)
    x = saturate(w, x, w.seed)
    got = gpu_bwd(w, x, dout, softplus=softplus, exact=exact, init=init)
    ref = oracle_bwd(w, x, dout, softplus=softplus, exact=exact, init=init)
    compare("saturated_" + name, w, got, ref)


def test_bwd_optional_outputs_absent():
    """Without dD, dz, ddelta_bias and dinit buffers the other gradients are unchanged."""
    w = W("opt_absent", 1, 32, 64, 16, I.DIR_BIDIR, "f32", True, 43)
    announce("bwd %s" % (w,))
    x = I.make_inputs(w)
    xd = dev_inputs(x)
    dout = to_dev(I.make_dout(w))
    full = ms.scan_bwd(xd["u"], xd["delta"], xd["A"], xd["B"], xd["C"], xd["D"], xd["z"], xd["delta_bias"], dout=dout,
                       dir_mode=w.dir_mode)
    lib = ms.load_library()
    dims = ms.make_dims(w.batch, w.dim, w.seqlen, w.dstate, ms.DTYPE_F32)
    t = torch()
    ws = t.empty(ms.bwd_workspace_bytes(dims, w.dir_mode), dtype=t.uint8, device="cuda:0")
    dims.workspace, dims.workspace_bytes = ws.data_ptr(), ws.numel()
    part = {k: t.empty_like(full[k]) for k in ("du", "ddelta", "dA", "dB", "dC")}
    p = lambda v: None if v is None else v.data_ptr()
    import ctypes
    rc = lib.mamba_scan_bwd(p(xd["u"]), p(xd["delta"]), p(xd["A"]), p(xd["B"]), p(xd["C"]), p(xd["D"]), p(xd["z"]),
                            p(xd["delta_bias"]), p(dout), ctypes.byref(dims), w.dir_mode, p(part["du"]),
                            p(part["ddelta"]), p(part["dA"]), p(part["dB"]), p(part["dC"]), None, None, None, None,
                            None, 0, t.cuda.current_stream().cuda_stream)
    assert rc == 0
    t.cuda.synchronize()
    for k in part:
        assert t.equal(part[k], full[k]), k


def saved_vs_recompute(name, w, xd, dout, init=None, softplus=True, exact=False):
    """mamba_scan_fwd_save returns mamba_scan_fwd's out and last_state, and the
    backward from its saved state equals the recomputing backward bit for bit
    (both take the same states from the same forward plan)."""
    t = torch()
    kw = dict(dir_mode=w.dir_mode, height=w.height, width=w.width, delta_softplus=softplus, exact_zoh=exact,
              initial_state=init)
    args = (xd["u"], xd["delta"], xd["A"], xd["B"], xd["C"], xd.get("D"), xd.get("z"), xd.get("delta_bias"))
    out0, st0 = ms.scan_fwd(*args, **kw)
    out1, st1, saved = ms.scan_fwd_save(*args, **kw)
    g0 = ms.scan_bwd(*args, dout=dout, **kw)
    g1 = ms.scan_bwd(*args, dout=dout, saved=saved, **kw)
    t.cuda.synchronize()
    assert t.equal(out0, out1), name + " out"
    assert t.equal(st0, st1), name + " last_state"
    for k in g0:
        assert (g0[k] is None) == (g1[k] is None), k
        if g0[k] is not None:
            assert t.equal(g0[k], g1[k]), "%s %s" % (name, k)


SAVED = [c for c in SMALL if c[0] in ("fwd_bf16", "fwd_f32_n4_exact_init", "bwd_bf16_n8", "bidir_f32_init",
                                      "cross2d_bf16", "cross2d_f32_n1_gated", "split_fwd_bf16", "split_bidir_f32",
                                      "L1_D8_bf16_n2", "exact_nosoftplus_init_bf16", "n32_fwd_bf16_init",
                                      "n3_fwd_f32_init", "n12_bidir_bf16", "n64_fwd_bf16_init",
                                      "n40_cross2d_bf16_init", "n64_split_bwd_f32", "t64_fwd_bf16_init",
                                      "t64_cross2d_f32")]


@pytest.mark.parametrize("case", SAVED, ids=[c[0] for c in SAVED])
def test_saved_state_small(case):
    name, w, softplus, exact, with_init, skip = case
    announce("saved %s %s" % (name, w))
    x, dout, init = small_inputs(case)
    saved_vs_recompute(name, w, dev_inputs(x), to_dev(dout), to_dev(init), softplus, exact)


@pytest.mark.parametrize("wname", ["mamba130m_layer", "vmamba_ss2d", "vim_bidir_224"])
def test_saved_state_full_size(wname):
    w = I.WORKLOADS[wname]
    announce("saved full %s" % (w,))
    saved_vs_recompute(wname, w, dev_inputs(I.make_inputs(w)), to_dev(I.make_dout(w)))


# (workload, check whole batch items): the 97k-token Vim image has one batch
# item, which the oracle would need over every channel (minutes); its dB and
# dC are covered by the split cases above at smaller sizes.
FULL = [("mamba130m_layer", True), ("vim_bidir_224", True), ("vmamba_ss2d", True), ("vim_bidir_1248", False)]


@pytest.mark.parametrize("wname,items", FULL, ids=[f[0] for f in FULL])
def test_bwd_full_size(wname, items):
    """The full workload on the GPU (the long one with a time-split adjoint);
    the oracle on 24 channels over the whole batch and, where affordable, on
    the first and last batch items over every channel."""
    w = I.WORKLOADS[wname]
    announce("bwd full %s" % (w,))
    x = I.make_inputs(w)
    dout = I.make_dout(w)
    got = gpu_bwd(w, x, dout)
    # channel subset: every gradient but dB, dC (sums over all channels)
    r = np.random.Generator(np.random.PCG64([w.seed, 5]))
    S = np.unique(np.concatenate([[0, w.dim - 1], r.choice(w.dim, 22, replace=False)]))
    xs = dict(x)
    for k in ("u", "delta", "z"):
        xs[k] = None if x[k] is None else np.ascontiguousarray(x[k][..., S])
    xs["A"] = np.ascontiguousarray(x["A"][..., S, :])
    xs["D"] = np.ascontiguousarray(x["D"][..., S])
    xs["delta_bias"] = np.ascontiguousarray(x["delta_bias"][..., S])
    ws = w.with_(dim=len(S))
    ref = oracle_bwd(ws, xs, np.ascontiguousarray(dout[..., S]))

    def chan(k, v):
        return v[..., S, :] if k in ("dA", "dinit") else v[..., S]
    compare(wname + " channels", ws, got, ref, keys=("du", "ddelta", "dz", "dA", "dD", "ddelta_bias", "dinit"),
            index=chan)
    # whole batch items: dB, dC
    for b in ((0, w.batch - 1) if items else ()):
        xb = dict(x)
        for k in ("u", "delta", "z", "B", "C"):
            xb[k] = None if x[k] is None else np.ascontiguousarray(x[k][b:b + 1])
        wb = w.with_(batch=1)
        refb = oracle_bwd(wb, xb, np.ascontiguousarray(dout[b:b + 1]))
        compare("%s batch %d" % (wname, b), wb, got, refb, keys=("dB", "dC", "du"),
                index=lambda k, v: v[b:b + 1])


def test_bwd_long_context_channels():
    """The long-context workload (one batch item, 262,144 tokens: fp32 output
    rows of exactly 2^31 bytes and an 8-chunk time-split adjoint), checked on
    24 channels; the gradients are sliced on the GPU before the copy back."""
    w = I.WORKLOADS["long_context"]
    announce("bwd full %s (channel subset)" % (w,))
    x = I.make_inputs(w)
    dout = I.make_dout(w)
    xd = dev_inputs(x)
    g = ms.scan_bwd(xd["u"], xd["delta"], xd["A"], xd["B"], xd["C"], xd["D"], xd["z"], xd["delta_bias"],
                    dout=to_dev(dout))
    r = np.random.Generator(np.random.PCG64([w.seed, 5]))
    S = np.unique(np.concatenate([[0, w.dim - 1], r.choice(w.dim, 22, replace=False)]))
    St = torch().from_numpy(S).to("cuda:0")
    got = {k: from_dev(v.index_select(-2 if k in ("dA", "dinit") else -1, St))
           for k, v in g.items() if k in ("du", "ddelta", "dz", "dA", "dD", "ddelta_bias", "dinit")}
    del g, xd
    xs = dict(x)
    for k in ("u", "delta", "z"):
        xs[k] = np.ascontiguousarray(x[k][..., S])
    xs["A"] = np.ascontiguousarray(x["A"][..., S, :])
    xs["D"] = np.ascontiguousarray(x["D"][..., S])
    xs["delta_bias"] = np.ascontiguousarray(x["delta_bias"][..., S])
    ws = w.with_(dim=len(S))
    ref = oracle_bwd(ws, xs, np.ascontiguousarray(dout[..., S]))
    compare("long_context channels", ws, got, ref, keys=tuple(got))
