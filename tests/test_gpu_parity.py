"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on the
same seeded inputs, plus properties that hold at any size.

Small cases span several 64-channel blocks and 32-step tiles with ragged
tails, every direction mode, every supported state size, the time-split path,
and the optional arguments.  The five specified workloads run at full size in
the launch configuration the benchmark times, checked on sampled (b, d) rows
that the oracle computes one by one.
"""
import os

import numpy as np
import pytest

import oracle
import selective_state_space_mamba_amd as ms
from selective_state_space_mamba_amd import inputs as I

from scanutil import (TOL, assert_close, dev_inputs, errors, from_dev, gpu_fwd, oracle_fwd, sample_rows, saturate,
                      to_dev, torch)

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    ms.load_library()  # fails loudly when the HIP library is missing
    yield


def announce(msg):
    print("[gpu case] " + msg, flush=True)


def run_and_check(w, x=None, name=None, **kw):
    x = x if x is not None else I.make_inputs(w)
    announce("%s %s" % (name or w.name, w))
    out, st = gpu_fwd(w, dev_inputs(x), **kw)
    ref_out, ref_st = oracle_fwd(w, x, **{k: v for k, v in kw.items() if k in ("delta_softplus", "exact_zoh")},
                                 initial_state=(None if kw.get("initial_state") is None
                                                else kw["initial_state"].cpu().numpy()))
    assert_close((name or w.name) + " out", from_dev(out), ref_out, w.dtype)
    if st is not None:
        assert_close((name or w.name) + " last_state", from_dev(st), ref_st.reshape(from_dev(st).shape),
                     "f32" if w.dtype == "f32" else "bf16")
    return out, st, ref_out, ref_st


# ---------------------------------------------------------------------------------------------
# the tiny float32 workload, also against the stored oracle fixture

def test_tiny_f32_workload():
    w = I.WORKLOADS["tiny_f32"]
    out, st, ref_out, ref_st = run_and_check(w)
    want = np.loadtxt(os.path.join(GOLDEN, "tiny_f32_oracle.txt"))
    got = np.concatenate([from_dev(out).ravel(), from_dev(st).ravel()])
    emax, _ = errors(got[:out.numel()], want[:out.numel()])
    assert emax <= TOL["f32"]["max"]


SMALL = {
    "fwd_bf16_ragged": I.Workload("fwd_bf16_ragged", 2, 136, 300, 16, I.DIR_FWD, "bf16", True, 11),
    "fwd_f32_ragged": I.Workload("fwd_f32_ragged", 2, 136, 300, 16, I.DIR_FWD, "f32", True, 12),
    "bwd_bf16": I.Workload("bwd_bf16", 2, 72, 133, 16, I.DIR_BWD, "bf16", True, 13),
    "bwd_f32": I.Workload("bwd_f32", 1, 64, 77, 16, I.DIR_BWD, "f32", False, 14),
    "bidir_bf16": I.Workload("bidir_bf16", 3, 72, 197, 16, I.DIR_BIDIR, "bf16", True, 15),
    "bidir_f32": I.Workload("bidir_f32", 2, 16, 45, 4, I.DIR_BIDIR, "f32", True, 16),
    "cross2d_bf16": I.Workload("cross2d_bf16", 2, 64, 240, 16, I.DIR_CROSS2D, "bf16", False, 17, 12, 20),
    "cross2d_f32_gated": I.Workload("cross2d_f32_gated", 1, 16, 35, 8, I.DIR_CROSS2D, "f32", True, 18, 5, 7),
    "cross2d_tall_f32": I.Workload("cross2d_tall_f32", 1, 24, 66, 4, I.DIR_CROSS2D, "f32", False, 19, 33, 2),
    "split_fwd_bf16": I.Workload("split_fwd_bf16", 1, 64, 4133, 16, I.DIR_FWD, "bf16", True, 20),
    "split_fwd_f32": I.Workload("split_fwd_f32", 1, 72, 5000, 16, I.DIR_FWD, "f32", True, 21),
    "split_bwd_bf16": I.Workload("split_bwd_bf16", 1, 64, 3001, 16, I.DIR_BWD, "bf16", True, 22),
    "split_bidir_bf16": I.Workload("split_bidir_bf16", 1, 64, 3000, 16, I.DIR_BIDIR, "bf16", True, 23),
    "split_cross2d_bf16": I.Workload("split_cross2d_bf16", 1, 32, 2304, 16, I.DIR_CROSS2D, "bf16", False, 24, 48, 48),
    # many rows, short sequences: one state per thread
    "rows768_bf16": I.Workload("rows768_bf16", 12, 1024, 70, 16, I.DIR_FWD, "bf16", True, 25),
    "rows768_cross2d_f32": I.Workload("rows768_cross2d_f32", 3, 1024, 36, 16, I.DIR_CROSS2D, "f32", False, 26, 6, 6),
    "wide4_bidir_bf16": I.Workload("wide4_bidir_bf16", 16, 1536, 20, 16, I.DIR_BIDIR, "bf16", True, 27),
    # rows for at least 16 waves per SIMD at N = 16: 2 states per thread (with a
    # ragged channel block and a ragged tile)
    "g2_fwd_bf16": I.Workload("g2_fwd_bf16", 64, 1032, 45, 16, I.DIR_FWD, "bf16", True, 32),
    "g2_bidir_f32": I.Workload("g2_bidir_f32", 32, 1032, 37, 16, I.DIR_BIDIR, "f32", True, 33),
    # few rows, long sequence: split in time (N = 16, 8 and 4)
    "split_long_fwd_bf16": I.Workload("split_long_fwd_bf16", 1, 64, 9000, 16, I.DIR_FWD, "bf16", True, 28),
    "split_long_bidir_f32": I.Workload("split_long_bidir_f32", 1, 64, 8500, 16, I.DIR_BIDIR, "f32", True, 29),
    "split_long_fwd_bf16_n8": I.Workload("split_long_fwd_bf16_n8", 1, 64, 9000, 8, I.DIR_FWD, "bf16", True, 30),
    "split_long_bidir_f32_n4": I.Workload("split_long_bidir_f32_n4", 1, 72, 5000, 4, I.DIR_BIDIR, "f32", True, 31),
    # one state per thread at N = 16 on 1024 positions or more: 64-position tiles
    # (ragged last tile, the bidirectional fold, the cross scan's column order)
    "t64_fwd_f32": I.Workload("t64_fwd_f32", 2, 48, 1100, 16, I.DIR_FWD, "f32", True, 34),
    "t64_bidir_bf16": I.Workload("t64_bidir_bf16", 2, 40, 1500, 16, I.DIR_BIDIR, "bf16", True, 35),
    "t64_cross2d_bf16": I.Workload("t64_cross2d_bf16", 1, 32, 1024, 16, I.DIR_CROSS2D, "bf16", False, 36, 32, 32),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_workloads(name):
    run_and_check(SMALL[name])


@pytest.mark.parametrize("N", [1, 2, 4, 8, 32, 64])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_state_sizes(N, dtype):
    w = I.Workload("N%d_%s" % (N, dtype), 2, 80, 70, N, I.DIR_FWD, dtype, True, 100 + N)
    run_and_check(w)


def test_state_size_64_bidir():
    run_and_check(I.Workload("N64_bidir", 1, 64, 50, 64, I.DIR_BIDIR, "f32", True, 131))


# state sizes that are not a power of two (run padded to the next one, the
# extra states held at zero) and float32 channel counts that are a multiple
# of 4 but not of 8
ODD = {
    "N3_fwd_f32": I.Workload("N3_fwd_f32", 2, 80, 70, 3, I.DIR_FWD, "f32", True, 141),
    "N3_fwd_bf16": I.Workload("N3_fwd_bf16", 2, 80, 71, 3, I.DIR_FWD, "bf16", True, 142),
    "N12_fwd_bf16": I.Workload("N12_fwd_bf16", 2, 136, 97, 12, I.DIR_FWD, "bf16", True, 143),
    "N12_bidir_f32": I.Workload("N12_bidir_f32", 2, 72, 65, 12, I.DIR_BIDIR, "f32", True, 144),
    "N24_cross2d_bf16": I.Workload("N24_cross2d_bf16", 1, 64, 63, 24, I.DIR_CROSS2D, "bf16", False, 145, 7, 9),
    "N48_fwd_f32": I.Workload("N48_fwd_f32", 1, 72, 90, 48, I.DIR_FWD, "f32", True, 146),
    "N48_bwd_bf16": I.Workload("N48_bwd_bf16", 2, 64, 50, 48, I.DIR_BWD, "bf16", True, 147),
    "N12_split_bf16": I.Workload("N12_split_bf16", 1, 64, 5000, 12, I.DIR_FWD, "bf16", True, 148),
    "D36_fwd_f32": I.Workload("D36_fwd_f32", 2, 36, 77, 16, I.DIR_FWD, "f32", True, 149),
    "D36_bidir_f32": I.Workload("D36_bidir_f32", 2, 36, 45, 16, I.DIR_BIDIR, "f32", True, 150),
    "D36_cross2d_f32_N5": I.Workload("D36_cross2d_f32_N5", 1, 36, 30, 5, I.DIR_CROSS2D, "f32", True, 151, 5, 6),
    "D100_split_f32_N24": I.Workload("D100_split_f32_N24", 1, 100, 4100, 24, I.DIR_FWD, "f32", True, 152),
}


@pytest.mark.parametrize("name", sorted(ODD))
def test_odd_state_sizes_and_channel_counts(name):
    run_and_check(ODD[name])


def test_options_softplus_off_no_skip_no_gate_no_bias():
    w = I.Workload("opts", 2, 64, 90, 16, I.DIR_FWD, "f32", False, 31)
    x = I.make_inputs(w)
    x["delta"] = np.abs(x["delta"]) * np.float32(0.1)  # softplus off: keep Δ positive and small
    x["D"] = None
    x["delta_bias"] = None
    run_and_check(w, x, name="softplus_off", delta_softplus=False)


def test_initial_state():
    for mode, K in ((I.DIR_FWD, 1), (I.DIR_BIDIR, 2)):
        w = I.Workload("init", 2, 72, 150, 16, mode, "bf16", True, 32)
        x = I.make_inputs(w)
        r = np.random.Generator(np.random.PCG64(5))
        shape = (2, 72, 16) if K == 1 else (2, K, 72, 16)
        init = r.standard_normal(shape).astype(np.float32)
        run_and_check(w, x, name="init_state_%d" % mode, initial_state=to_dev(init))
    # and through the time-split path
    w = I.Workload("init_split", 1, 64, 3000, 16, I.DIR_FWD, "bf16", True, 33)
    init = np.random.Generator(np.random.PCG64(6)).standard_normal((1, 64, 16)).astype(np.float32)
    run_and_check(w, I.make_inputs(w), name="init_state_split", initial_state=to_dev(init))


SATURATED = [
    (I.Workload("saturated_fwd", 2, 48, 150, 16, I.DIR_FWD, "bf16", True, 52), False),
    (I.Workload("saturated_bidir", 1, 32, 97, 16, I.DIR_BIDIR, "f32", True, 53), True),
    (I.Workload("saturated_cross", 1, 16, 48, 8, I.DIR_CROSS2D, "bf16", True, 54, 6, 8), False),
]


@pytest.mark.parametrize("w,exact", SATURATED, ids=[c[0].name for c in SATURATED])
def test_saturated_softplus_and_gate(w, exact):
    """Δraw and z far outside their usual range [MFS §4.1 (softplus), §6.2 Step 6
    (silu gate)]: finite results equal to the oracle's, also row by row
    ((b, d) over the sequence, each against its own largest value), so that
    the rows with large Δ do not hide the others."""
    x = saturate(w, I.make_inputs(w), w.seed)
    out, _, ref_out, _ = run_and_check(w, x, name=w.name + ("_exact" if exact else ""), exact_zoh=exact)
    got = from_dev(out)
    ref = ref_out.reshape(got.shape)
    scale = np.max(np.abs(ref), axis=1)
    err = np.max(np.abs(got - ref), axis=1) / np.where(scale > 0, scale, 1.0)
    print("%s: row-wise max err %.3e" % (w.name, err.max()), flush=True)
    assert err.max() <= TOL[w.dtype]["max"], err.max()


def test_no_last_state():
    w = I.Workload("nolast", 1, 64, 64, 16, I.DIR_FWD, "bf16", True, 34)
    x = I.make_inputs(w)
    out, st = ms.scan_fwd(*[to_dev(x[k]) for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")],
                          want_last_state=False)
    torch().cuda.synchronize()
    assert st is None
    ref, _ = oracle_fwd(w, x)
    assert_close("nolast", from_dev(out), ref, "bf16")


# ---------------------------------------------------------------------------------------------
# exact properties

def test_bf16_output_is_round_to_nearest_even():
    """C = 0, D = 1.5, no gate: out = bf16(1.5·u), where 1.5·u is exact in fp32 and
    often a tie at bf16 precision, so the rounding mode is visible bit for bit."""
    w = I.Workload("rne", 1, 64, 96, 4, I.DIR_FWD, "bf16", False, 41)
    x = I.make_inputs(w)
    x["C"] = np.zeros_like(x["C"])
    x["D"] = np.full_like(x["D"], 1.5)
    announce("rne")
    out, _ = gpu_fwd(w, dev_inputs(x))
    got = out.view(torch().int16).cpu().numpy().view(np.uint16)
    want = I.bf16_bits(I.bf16_to_f32(x["u"]) * np.float32(1.5))
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("mode,K", [(I.DIR_FWD, 1), (I.DIR_BWD, 1), (I.DIR_BIDIR, 2), (I.DIR_CROSS2D, 4)])
def test_one_hot_state_layout(mode, K):
    """A single u = 1 at the first scan position of one (b, k, d) row and B = e_n:
    last_state is nonzero exactly at [b, k, d, n]."""
    Bsz, H, W, Dm, N = 2, 6, 8, 72, 16
    L = H * W
    r = np.random.Generator(np.random.PCG64(42 + mode))
    Ku = 1 if mode == I.DIR_CROSS2D else K
    for trial in range(2):
        bs, ks, ds, ns = int(r.integers(Bsz)), int(r.integers(K)), int(r.integers(Dm)), int(r.integers(N))
        first = oracle.token(mode, ks, 0, L, H, W)
        u = np.zeros((Bsz, Ku, L, Dm), np.float32)
        u[bs, 0 if Ku == 1 else ks, first, ds] = 1.0
        delta = r.uniform(0.05, 0.3, (Bsz, K, L, Dm)).astype(np.float32)
        B = np.zeros((Bsz, K, L, N), np.float32)
        B[bs, ks, first, ns] = 1.0
        C = r.standard_normal((Bsz, K, L, N)).astype(np.float32)
        A = -r.uniform(0.5, 2, (K, Dm, N)).astype(np.float32)
        sq = lambda a: a.reshape(a.shape[:1] + a.shape[2:]) if a.shape[1] == 1 else a
        x = dict(u=sq(u), delta=sq(delta), B=sq(B), C=sq(C), A=A[0] if K == 1 else A)
        w = I.Workload("onehot", Bsz, Dm, L, N, mode, "f32", False, 0, H if mode == I.DIR_CROSS2D else 0,
                       W if mode == I.DIR_CROSS2D else 0)
        announce("one-hot mode %d trial %d" % (mode, trial))
        _, st = gpu_fwd(w, dev_inputs(x), delta_softplus=False)
        st = st.cpu().numpy().reshape(Bsz, K, Dm, N)
        nz = np.argwhere(st != 0)
        assert nz.tolist() == [[bs, ks, ds, ns]]
        _, ref = oracle_fwd(w, x, delta_softplus=False)
        assert abs(st[bs, ks, ds, ns] - ref[bs, ks, ds, ns]) <= 2e-6 * abs(ref[bs, ks, ds, ns])


def test_reversed_scan_is_flipped_forward_bitwise():
    w = I.Workload("flip", 2, 72, 150, 16, I.DIR_FWD, "bf16", True, 43)
    x = I.make_inputs(w)
    flip = lambda a: np.ascontiguousarray(a[:, ::-1])
    xf = dict(x, u=flip(x["u"]), delta=flip(x["delta"]), B=flip(x["B"]), C=flip(x["C"]), z=flip(x["z"]))
    announce("flip")
    fo, fs = gpu_fwd(w, dev_inputs(xf))
    bo, bs = gpu_fwd(w.with_(dir_mode=I.DIR_BWD), dev_inputs(x))
    np.testing.assert_array_equal(bo.flip(1).cpu().view(torch().int16).numpy(), fo.cpu().view(torch().int16).numpy())
    np.testing.assert_array_equal(bs.cpu().numpy(), fs.cpu().numpy())


def test_repeatable_overwrites_everything_and_stays_in_bounds():
    t = torch()
    for w in (SMALL["fwd_bf16_ragged"], SMALL["bidir_bf16"], SMALL["cross2d_bf16"], SMALL["split_fwd_bf16"]):
        x = I.make_inputs(w)
        xd = dev_inputs(x)
        announce("poison/guard %s" % w.name)
        Bsz, L, Dm, N, K = w.batch, w.seqlen, w.dim, w.dstate, w.ndirs
        guard = 4096
        ob = t.full((Bsz * L * Dm + guard,), float("nan"), dtype=t.bfloat16, device="cuda:0")
        sb = t.full((Bsz * K * Dm * N + guard,), float("nan"), dtype=t.float32, device="cuda:0")
        out = ob[:Bsz * L * Dm].view(Bsz, L, Dm)
        st = sb[:Bsz * K * Dm * N].view((Bsz, Dm, N) if K == 1 else (Bsz, K, Dm, N))
        ms.scan_fwd(xd["u"], xd["delta"], xd["A"], xd["B"], xd["C"], xd["D"], xd["z"], xd["delta_bias"],
                    dir_mode=w.dir_mode, height=w.height, width=w.width, out=out, last_state=st)
        t.cuda.synchronize()
        assert not t.isnan(out).any() and not t.isnan(st).any()
        assert t.isnan(ob[Bsz * L * Dm:]).all() and t.isnan(sb[Bsz * K * Dm * N:]).all()
        first = (out.clone(), st.clone())
        ms.scan_fwd(xd["u"], xd["delta"], xd["A"], xd["B"], xd["C"], xd["D"], xd["z"], xd["delta_bias"],
                    dir_mode=w.dir_mode, height=w.height, width=w.width, out=out, last_state=st)
        t.cuda.synchronize()
        assert t.equal(out.view(t.int16), first[0].view(t.int16)) and t.equal(st, first[1])


def test_cross_scan_transpose_symmetry():
    """H = W: transposing the grid swaps directions 0<->1 and 2<->3."""
    w = I.Workload("tr", 1, 64, 144, 16, I.DIR_CROSS2D, "f32", True, 44, 12, 12)
    x = I.make_inputs(w)
    H = 12
    T = lambda a: np.ascontiguousarray(a.reshape(a.shape[:-2] + (H, H, a.shape[-1])).swapaxes(-3, -2).reshape(a.shape))
    perm = [1, 0, 3, 2]
    xt = dict(u=T(x["u"]), delta=T(x["delta"][:, perm]), B=T(x["B"][:, perm]), C=T(x["C"][:, perm]),
              z=T(x["z"]), A=np.ascontiguousarray(x["A"][perm]), D=np.ascontiguousarray(x["D"][perm]),
              delta_bias=np.ascontiguousarray(x["delta_bias"][perm]))
    announce("transpose")
    o1, s1 = gpu_fwd(w, dev_inputs(x))
    o2, s2 = gpu_fwd(w, dev_inputs(xt))
    assert_close("transpose out", from_dev(o2), T(from_dev(o1)), "f32")
    assert_close("transpose state", from_dev(s2), from_dev(s1)[:, perm], "f32")


# ---------------------------------------------------------------------------------------------
# decode step

def run_decode(w, L0, steps, rows=None, exact_zoh=False, saturated=False):
    x = I.make_inputs(w, seqlen=L0 + steps)
    if saturated:
        x = saturate(w, x, w.seed)
    head = {k: (v[:, :L0] if k in ("u", "delta", "B", "C", "z") else v) for k, v in x.items()}
    xd = dev_inputs({k: (np.ascontiguousarray(v) if v is not None else None) for k, v in head.items()})
    announce("decode %s L0=%d steps=%d" % (w.name, L0, steps))
    _, st = gpu_fwd(w.with_(seqlen=L0), xd, exact_zoh=exact_zoh)
    state = st.contiguous()
    # step-major copies so that each step's [B][D] / [B][N] slice is contiguous
    tail = {k: to_dev(np.ascontiguousarray(x[k][:, L0:].swapaxes(0, 1))) for k in ("u", "delta", "B", "C", "z")}
    outs = []
    for s in range(steps):
        # (fresh allocations: a [B][N] slice of small N is not 16-byte aligned)
        t = {k: tail[k][s].clone() for k in tail}
        outs.append(ms.scan_step(state, t["u"], t["delta"], xd["A"], t["B"], t["C"], xd["D"], t["z"],
                                 xd["delta_bias"], exact_zoh=exact_zoh))
    torch().cuda.synchronize()
    got = np.stack([from_dev(o) for o in outs], axis=1)  # [B][steps][D]
    ref_out, ref_st = oracle_fwd(w.with_(seqlen=L0 + steps), x, rows=rows, exact_zoh=exact_zoh)
    return got, from_dev(state), ref_out, ref_st


def test_decode_continues_scan_small():
    w = I.Workload("dec", 2, 72, 0, 16, I.DIR_FWD, "bf16", True, 51)
    got, st, ref_out, ref_st = run_decode(w, 100, 40)
    assert_close("decode out", got, ref_out[:, 100:], "bf16")
    assert_close("decode state", st, ref_st[:, 0], "bf16")
    wf = I.Workload("decf", 1, 16, 0, 4, I.DIR_FWD, "f32", True, 52)
    got, st, ref_out, ref_st = run_decode(wf, 64, 16)
    assert_close("decode f32 out", got, ref_out[:, 64:], "f32")
    assert_close("decode f32 state", st, ref_st[:, 0], "f32")


def test_decode_saturated_softplus_and_gate():
    """Decode steps (and the scan before them) with Δraw and z far outside
    their usual range, as in the saturated forward cases."""
    for w, exact in ((I.Workload("dec_sat", 2, 72, 0, 16, I.DIR_FWD, "bf16", True, 55), False),
                     (I.Workload("dec_sat_f32", 1, 40, 0, 8, I.DIR_FWD, "f32", True, 56), True)):
        got, st, ref_out, ref_st = run_decode(w, 70, 24, exact_zoh=exact, saturated=True)
        assert_close(w.name + " out", got, ref_out[:, 70:], w.dtype)
        assert_close(w.name + " state", st, ref_st[:, 0], w.dtype)


@pytest.mark.parametrize("N", [1, 2, 8, 32, 64])
def test_decode_state_sizes(N):
    w = I.Workload("dec_N%d" % N, 2, 40, 0, N, I.DIR_FWD, "f32", True, 54 + N)
    got, st, ref_out, ref_st = run_decode(w, 50, 12)
    assert_close("decode N=%d out" % N, got, ref_out[:, 50:], "f32")
    assert_close("decode N=%d state" % N, st, ref_st[:, 0], "f32")


@pytest.mark.parametrize("N,dtype,dim", [(3, "f32", 40), (12, "bf16", 72), (24, "f32", 36), (48, "bf16", 64)])
def test_decode_odd_state_sizes(N, dtype, dim):
    w = I.Workload("dec_N%d" % N, 2, dim, 0, N, I.DIR_FWD, dtype, True, 60 + N)
    got, st, ref_out, ref_st = run_decode(w, 45, 10)
    assert_close("decode N=%d out" % N, got, ref_out[:, 45:], dtype)
    assert_close("decode N=%d state" % N, st, ref_st[:, 0], dtype)


def test_decode_exact_zoh():
    w = I.Workload("dec_exact", 2, 64, 0, 16, I.DIR_FWD, "f32", True, 53)
    got, st, ref_out, ref_st = run_decode(w, 80, 24, exact_zoh=True)
    assert_close("decode exact out", got, ref_out[:, 80:], "f32")
    assert_close("decode exact state", st, ref_st[:, 0], "f32")


@pytest.mark.parametrize("N,dtype", [(16, "bf16"), (12, "f32")])
def test_stepper_is_scan_step(N, dtype):
    """ScanStepper runs the same kernel as scan_step: equal outputs and state,
    bit for bit, over 24 steps from a scanned state; a mis-shaped tensor is
    refused before any launch."""
    t = torch()
    w = I.Workload("stepper", 3, 40, 0, N, I.DIR_FWD, dtype, True, 54)
    steps = 24
    x = I.make_inputs(w, seqlen=32 + steps)
    xd = dev_inputs({k: (np.ascontiguousarray(v[:, :32]) if k in ("u", "delta", "B", "C", "z") else v)
                     for k, v in x.items()})
    announce("stepper N=%d %s" % (N, dtype))
    _, st = gpu_fwd(w.with_(seqlen=32), xd)
    st_a = st.contiguous().clone()
    st_b = st.contiguous().clone()
    tail = {k: to_dev(np.ascontiguousarray(x[k][:, 32:].swapaxes(0, 1))) for k in ("u", "delta", "B", "C", "z")}
    stepper = ms.ScanStepper(st_b, xd["A"], xd["D"], xd["delta_bias"], dtype=tail["u"].dtype)
    for s in range(steps):
        a = {k: tail[k][s].clone() for k in tail}
        oa = ms.scan_step(st_a, a["u"], a["delta"], xd["A"], a["B"], a["C"], xd["D"], a["z"], xd["delta_bias"])
        ob = stepper(a["u"], a["delta"], a["B"], a["C"], a["z"], out=t.empty_like(oa))
        assert t.equal(oa, ob), s
    t.cuda.synchronize()
    assert t.equal(st_a, st_b)
    # bound buffers: each token copied into the same tensors, one call per step
    st_c = st.contiguous().clone()
    bound = {k: t.empty_like(tail[k][0]) for k in tail}
    ob = t.empty_like(tail["u"][0])
    stepper_c = ms.ScanStepper(st_c, xd["A"], xd["D"], xd["delta_bias"], dtype=tail["u"].dtype)
    stepper_c.bind(bound["u"], bound["delta"], bound["B"], bound["C"], bound["z"], out=ob)
    st_a = st.contiguous().clone()
    for s in range(steps):
        for k in tail:
            bound[k].copy_(tail[k][s])
        a = {k: tail[k][s].clone() for k in tail}  # (fresh allocations: 16-byte aligned)
        oa = ms.scan_step(st_a, a["u"], a["delta"], xd["A"], a["B"], a["C"], xd["D"], a["z"], xd["delta_bias"])
        assert t.equal(oa, stepper_c.step()), s
    t.cuda.synchronize()
    assert t.equal(st_a, st_c)
    bad = tail["B"][0][:, :N - 1].contiguous()
    with pytest.raises(ValueError):
        stepper(tail["u"][0], tail["delta"][0], bad, tail["C"][0], tail["z"][0], out=t.empty_like(tail["u"][0]))


# ---------------------------------------------------------------------------------------------
# exact zero-order hold of the input term

EXACT = {
    "exact_fwd_f32": I.Workload("exact_fwd_f32", 2, 136, 300, 16, I.DIR_FWD, "f32", True, 61),
    "exact_fwd_bf16": I.Workload("exact_fwd_bf16", 2, 72, 133, 16, I.DIR_FWD, "bf16", True, 62),
    "exact_bidir_bf16": I.Workload("exact_bidir_bf16", 2, 72, 197, 16, I.DIR_BIDIR, "bf16", True, 63),
    "exact_cross2d_f32": I.Workload("exact_cross2d_f32", 1, 16, 35, 8, I.DIR_CROSS2D, "f32", True, 64, 5, 7),
    "exact_split_f32": I.Workload("exact_split_f32", 1, 72, 5000, 16, I.DIR_FWD, "f32", True, 65),
    "exact_rows768_bf16": I.Workload("exact_rows768_bf16", 12, 1024, 70, 16, I.DIR_FWD, "bf16", True, 66),
    "exact_N4_f32": I.Workload("exact_N4_f32", 2, 80, 70, 4, I.DIR_FWD, "f32", True, 67),
    "exact_N64_f32": I.Workload("exact_N64_f32", 1, 64, 50, 64, I.DIR_FWD, "f32", True, 68),
}


@pytest.mark.parametrize("name", sorted(EXACT))
def test_exact_zoh(name):
    run_and_check(EXACT[name], exact_zoh=True)


def test_exact_zoh_small_and_zero_decay():
    """A spread over zero, tiny and large magnitudes, so that both the series
    and the direct branch of (e^{ΔA} - 1)/A and the A = 0 limit are taken."""
    w = I.Workload("exact_mixed_A", 2, 64, 120, 16, I.DIR_FWD, "f32", True, 69)
    x = I.make_inputs(w)
    r = np.random.Generator(np.random.PCG64(70))
    A = -np.exp(r.uniform(np.log(1e-4), np.log(30.0), size=x["A"].shape)).astype(np.float32)
    A[:, ::5] = 0.0  # every fifth state does not decay
    x["A"] = A
    run_and_check(w, x, name="exact_mixed_A", exact_zoh=True)
    run_and_check(w, x, name="simplified_mixed_A")


def test_exact_zoh_is_the_gated_rnn():
    """One state, A = -1, B = C = 1, no skip, no gate: with exact hold the scan is
    h_t = (1 - g_t) h_{t-1} + g_t u_t with g_t = sigmoid(delta_t + bias), computed
    here directly in float64 (independent of the oracle)."""
    w = I.Workload("gated_rnn", 2, 64, 257, 1, I.DIR_FWD, "f32", False, 71)
    x = I.make_inputs(w)
    x["A"] = np.full_like(x["A"], -1.0)
    x["B"] = np.ones_like(x["B"])
    x["C"] = np.ones_like(x["C"])
    x["D"] = None
    announce("gated rnn")
    out, _ = gpu_fwd(w, dev_inputs(x), exact_zoh=True)
    s = x["delta"].astype(np.float64) + x["delta_bias"].astype(np.float64)[None, None, :]
    g = 1.0 / (1.0 + np.exp(-s))
    u = x["u"].astype(np.float64)
    h = np.zeros((w.batch, w.dim))
    want = np.empty_like(u)
    for t in range(w.seqlen):
        h = (1.0 - g[:, t]) * h + g[:, t] * u[:, t]
        want[:, t] = h
    assert_close("gated rnn", from_dev(out), want, "f32")


# ---------------------------------------------------------------------------------------------
# the specified workloads at full size, sampled rows

def block_rows(rng, batch, dim, block=16):
    """For every batch and every block of `block` channels: both edge
    channels and one channel drawn inside the block."""
    rows = set()
    for b in range(batch):
        for d0 in range(0, dim, block):
            d1 = min(dim, d0 + block) - 1
            rows.update({(b, d0), (b, d1), (b, int(rng.integers(d0, d1 + 1)))})
    return np.array(sorted(rows), dtype=np.int64)


def full_size_check(w, rows="all", seed=7, exact_zoh=False):
    """The whole output and last state against the oracle (rows="all"), or the
    (b, d) rows of an int array [R, 2]."""
    x = I.make_inputs(w)
    announce("full-size %s exact_zoh=%s rows=%s" % (w.name, exact_zoh, "all" if isinstance(rows, str) else len(rows)))
    out, st = gpu_fwd(w, dev_inputs(x), exact_zoh=exact_zoh)
    o = from_dev(out)
    s = from_dev(st).reshape(w.batch, w.ndirs, w.dim, w.dstate)
    if isinstance(rows, str):
        ref_out, ref_st = oracle_fwd(w, x, exact_zoh=exact_zoh)
        assert_close(w.name + " out (every row)", o, ref_out, w.dtype)
        assert_close(w.name + " last_state (every row)", s, ref_st.reshape(s.shape), w.dtype)
        return
    ref_out, ref_st = oracle_fwd(w, x, rows=rows, exact_zoh=exact_zoh)
    got_o = np.stack([o[b, :, d] for b, d in rows])
    got_s = np.stack([s[b, :, d] for b, d in rows])
    assert_close(w.name + " out (%d rows)" % len(rows), got_o, ref_out, w.dtype)
    assert_close(w.name + " last_state (%d rows)" % len(rows), got_s, ref_st, w.dtype)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["mamba130m_layer", "vim_bidir_224", "vmamba_ss2d"])
def test_full_size_workloads_every_row(name):
    full_size_check(I.WORKLOADS[name])


@pytest.mark.slow
@pytest.mark.parametrize("name", ["long_context", "vim_bidir_1248"])
def test_full_size_long_workloads(name):
    """Few rows, long sequences: three channels of every 16-channel block (the
    two edges and one inside), every token of each."""
    w = I.WORKLOADS[name]
    full_size_check(w, rows=block_rows(np.random.Generator(np.random.PCG64(7)), w.batch, w.dim))


@pytest.mark.parametrize("name", ["mamba130m_layer", "vim_bidir_224"])
def test_full_size_exact_zoh(name):
    """The exact input-term rule in the launch configuration the benchmark
    times for it, sampled rows against the oracle."""
    w = I.WORKLOADS[name]
    full_size_check(w, rows=sample_rows(np.random.Generator(np.random.PCG64(7)), w.batch, w.dim, 48),
                    exact_zoh=True)


@pytest.mark.slow
def test_full_size_decode_512_steps():
    """512 decode steps continuing the full 2048-token scan, every row."""
    w = I.WORKLOADS["mamba130m_layer"]
    got, st, ref_out, ref_st = run_decode(w, w.seqlen, I.DECODE_STEPS)
    assert_close("decode512 out (every row)", got, ref_out[:, w.seqlen:], "bf16")
    assert_close("decode512 state (every row)", st, ref_st[:, 0], "bf16")
