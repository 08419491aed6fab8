"""Pins of the fp64 CPU oracle against what the pages and the mathematics fix.

Each test ties the oracle to something other than itself: a hand-worked
example, a closed form, brute force by a different formula, or an invariant.
They are chosen so that a plausible slip in the oracle (a wrong sign in the
exponent, B and C swapped, readout before the update, a wrong scan order or
state layout, a dropped skip term) fails at least one of them.

Sources, cited by page title and section:
  [MFS] "从零理解 Mamba：选择性状态空间模型（Selective SSM）到 Mamba Block" (eutaboo.com)
  [S4M] "从S4到Mamba：选择性状态空间模型的演进与革新" (jsqmd.com)
  [MUN] "【临时文档---算法介绍】Mamba-UNet" (blog.csdn.net)
  [VIM] "Vision Mamba：从状态空间模型到视觉革命的跨越" (x-humanoid.csdn.net)
"""
import math
import os

import numpy as np
import pytest

import oracle
from selective_state_space_mamba_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
F32 = np.float32


def rng(seed=0):
    return np.random.Generator(np.random.PCG64(seed))


def _rand_problem(r, Bsz=1, L=12, Dm=3, N=4, K=1, Ku=None, pos_delta=True):
    Ku = K if Ku is None else Ku
    sh = lambda *s: tuple(x for x in s)
    u = r.standard_normal(sh(Bsz, Ku, L, Dm)).astype(F32)
    if pos_delta:  # softplus off: delta is Δ itself, keep it positive and modest
        delta = r.uniform(0.01, 0.5, sh(Bsz, K, L, Dm)).astype(F32)
    else:
        delta = r.standard_normal(sh(Bsz, K, L, Dm)).astype(F32)
    B = r.standard_normal(sh(Bsz, K, L, N)).astype(F32)
    C = r.standard_normal(sh(Bsz, K, L, N)).astype(F32)
    A = -r.uniform(0.2, 3.0, (K, Dm, N)).astype(F32)
    D = r.standard_normal((K, Dm)).astype(F32)
    z = r.standard_normal((Bsz, L, Dm)).astype(F32)
    bias = np.zeros((K, Dm), F32)
    return dict(u=u, delta=delta, B=B, C=C, A=A, D=D, z=z, delta_bias=bias)


# --- hand example [MFS §2.2 eq (2a)(2b); MFS eq (4); MUN §4] ------------------------------

def test_hand_example_n1():
    rows = np.loadtxt(os.path.join(GOLDEN, "hand_example_n1.txt"))
    u = np.array([1.0, -2.0, 4.0], F32).reshape(1, 3, 1)
    delta = np.full((1, 3, 1), 0.5, F32)
    B = np.ones((1, 3, 1), F32)
    C = np.full((1, 3, 1), 2.0, F32)
    A = np.full((1, 1), -2.0, F32)
    D = np.full((1,), 0.25, F32)
    out, st = oracle.scan(u, delta, A, B, C, D, None, None, delta_softplus=False)
    np.testing.assert_allclose(out[0, :, 0], rows[:, 1], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(st[0, 0, 0, 0], rows[-1, 2], rtol=1e-14)


# --- P1: LTI case equals the convolution y = x * K, K_j = C Ā^j B̄ [MFS §2.3 eq (3a)(3b)] ---

@pytest.mark.parametrize("N", [1, 4])
def test_lti_convolution_bruteforce(N):
    r = rng(1)
    L, Dm = 24, 2
    dl = r.uniform(0.05, 0.4, Dm).astype(F32)       # Δ constant over time (LTI), per channel
    Bv = r.standard_normal(N).astype(F32)
    Cv = r.standard_normal(N).astype(F32)
    A = -r.uniform(0.3, 2.0, (Dm, N)).astype(F32)
    D = r.standard_normal(Dm).astype(F32)
    u = r.standard_normal((1, L, Dm)).astype(F32)
    delta = np.broadcast_to(dl, (1, L, Dm)).astype(F32).copy()
    B = np.broadcast_to(Bv, (1, L, N)).astype(F32).copy()
    C = np.broadcast_to(Cv, (1, L, N)).astype(F32).copy()
    out, _ = oracle.scan(u, delta, A, B, C, D, None, None, delta_softplus=False)
    for d in range(Dm):
        dd = float(dl[d])
        abar = np.exp(dd * A[d].astype(np.float64))
        Kj = np.array([np.sum(Cv * abar ** j * dd * Bv) for j in range(L)])  # kernel (CB̄, CĀB̄, ...)
        x = u[0, :, d].astype(np.float64)
        y = np.array([sum(Kj[j] * x[t - j] for j in range(t + 1)) for t in range(L)]) + D[d] * x
        np.testing.assert_allclose(out[0, :, d], y, rtol=1e-12, atol=1e-12)


# --- Unrolled time-varying recurrence (selection: Δ_t, B_t, C_t vary) [MFS §4.1 Algorithm 2] --

def test_time_varying_unrolled_bruteforce():
    r = rng(2)
    p = _rand_problem(r, Bsz=2, L=16, Dm=3, N=5)
    u, delta = p["u"][:, 0], p["delta"][:, 0]
    B, C, A, D = p["B"][:, 0], p["C"][:, 0], p["A"][0], p["D"][0]
    out, st = oracle.scan(u, delta, A, B, C, D, None, None, delta_softplus=False)
    Bsz, L, Dm = u.shape
    N = B.shape[-1]
    for b in range(Bsz):
        for d in range(Dm):
            dl = delta[b, :, d].astype(np.float64)
            cum = np.concatenate([[0.0], np.cumsum(dl)])  # cum[t+1] = Σ_{r<=t} Δ_r
            for t in range(L):
                y = 0.0
                for s in range(t + 1):
                    decay = np.exp(A[d].astype(np.float64) * (cum[t + 1] - cum[s + 1]))  # Π_{r=s+1..t} Ā_r
                    y += np.sum(C[b, t] * decay * dl[s] * B[b, s]) * u[b, s, d]
                y += float(D[d]) * float(u[b, t, d])
                assert abs(out[b, t, d] - y) <= 1e-11 * max(1.0, abs(y))
            hN = sum(np.exp(A[d].astype(np.float64) * (cum[L] - cum[s + 1])) * dl[s] * B[b, s] * u[b, s, d]
                     for s in range(L))
            np.testing.assert_allclose(st[b, 0, d], hN, rtol=1e-11, atol=1e-12)


# --- P2: A = 0 gives a cumulative sum of Δ·B·u (also under exact ZOH) ------------------------

@pytest.mark.parametrize("exact", [False, True])
def test_A_zero_cumsum(exact):
    r = rng(3)
    p = _rand_problem(r, Bsz=1, L=20, Dm=2, N=3)
    u, delta, B, C, D = p["u"][:, 0], p["delta"][:, 0], p["B"][:, 0], p["C"][:, 0], p["D"][0]
    A = np.zeros((2, 3), F32)
    out, st = oracle.scan(u, delta, A, B, C, D, None, None, delta_softplus=False, exact_zoh=exact)
    for d in range(2):
        inc = delta[0, :, d, None].astype(np.float64) * B[0].astype(np.float64) * u[0, :, d, None]
        h = np.cumsum(inc, axis=0)
        y = np.sum(C[0] * h, axis=1) + float(D[d]) * u[0, :, d].astype(np.float64)
        np.testing.assert_allclose(out[0, :, d], y, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(st[0, 0, d], h[-1], rtol=1e-12)


# --- P3: associativity of the affine pair and any chunking of the scan [MFS §5] ----------------

def test_affine_composition_associative():
    r = rng(4)
    comp = lambda p2, p1: (p2[0] * p1[0], p2[0] * p1[1] + p2[1])  # (a2,b2)∘(a1,b1)
    for _ in range(100):
        x, y, z = [tuple(r.uniform(-2, 2, 2)) for _ in range(3)]
        l, rr = comp(z, comp(y, x)), comp(comp(z, y), x)
        assert abs(l[0] - rr[0]) < 1e-12 and abs(l[1] - rr[1]) < 1e-12


@pytest.mark.parametrize("split", [1, 5, 11])
def test_chunked_scan_equals_sequential(split):
    """Two chunks combined through their affine aggregate equal one pass.

    Chunk 2 is scanned from zero; its state aggregate is P2·h1 + S2 with
    P2 = exp(A·ΣΔ over chunk 2), and its outputs gain Σ_n C_tn·Π_{r<=t}Ā_rn·h1."""
    r = rng(5)
    p = _rand_problem(r, Bsz=1, L=16, Dm=2, N=4)
    u, delta, B, C, A, D = (p[k][:, 0] if p[k].ndim == 4 else p[k][0] for k in ("u", "delta", "B", "C", "A", "D"))
    full_out, full_st = oracle.scan(u, delta, A, B, C, D, None, None, delta_softplus=False)
    o1, s1 = oracle.scan(u[:, :split], delta[:, :split], A, B[:, :split], C[:, :split], D, None, None,
                         delta_softplus=False)
    o2, s2 = oracle.scan(u[:, split:], delta[:, split:], A, B[:, split:], C[:, split:], D, None, None,
                         delta_softplus=False)
    h1 = s1[0, 0]                                            # [D][N]
    cum = np.cumsum(delta[0, split:].astype(np.float64), axis=0)  # [L2][D]
    P = np.exp(cum[:, :, None] * A[None].astype(np.float64))      # [L2][D][N]
    corr = np.einsum("tn,tdn,dn->td", C[0, split:].astype(np.float64), P, h1)
    np.testing.assert_allclose(o1[0], full_out[0, :split], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(o2[0] + corr, full_out[0, split:], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(P[-1] * h1 + s2[0, 0], full_st[0, 0], rtol=1e-11, atol=1e-12)


def test_initial_state_continuation():
    r = rng(6)
    p = _rand_problem(r, Bsz=2, L=14, Dm=3, N=4)
    u, delta, B, C, A, D, z = (p[k][:, 0] if p[k].ndim == 4 else (p[k][0] if k in ("A", "D") else p[k])
                               for k in ("u", "delta", "B", "C", "A", "D", "z"))
    full_out, full_st = oracle.scan(u, delta, A, B, C, D, z, None, delta_softplus=False)
    s = 6
    _, st1 = oracle.scan(u[:, :s], delta[:, :s], A, B[:, :s], C[:, :s], D, z[:, :s], None, delta_softplus=False)
    o2, st2 = oracle.scan(u[:, s:], delta[:, s:], A, B[:, s:], C[:, s:], D, z[:, s:], None,
                          delta_softplus=False, initial_state=st1.astype(F32))
    # the carried state is rounded to float32 when passed back in, so compare to fp32 rounding
    np.testing.assert_allclose(o2, full_out[:, s:], rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(st2, full_st, rtol=1e-5, atol=1e-6)


# --- P4: small-Δ limit Ā ≈ I + ΔA [MUN §4, first-order Taylor] --------------------------------

def test_first_order_limit():
    A = np.array([[-1.0, -4.0, -16.0, 2.0]], F32)
    dl = 1e-6
    out, st = oracle.scan(np.zeros((1, 1, 1), F32), np.full((1, 1, 1), dl, F32), A,
                          np.zeros((1, 1, 4), F32), np.zeros((1, 1, 4), F32), None, None, None,
                          delta_softplus=False, initial_state=np.ones((1, 1, 4), F32))
    dA = np.float64(np.float32(dl)) * A[0].astype(np.float64)
    err = np.abs(st[0, 0, 0] - (1.0 + dA))
    assert np.all(err <= dA ** 2), err
    assert np.all(np.abs(st[0, 0, 0] - (1.0 - dA)) > 1e-7)  # the wrong sign is far off


# --- P5: reversed scan is the forward scan of the flipped sequence; BIDIR sums both [VIM §2.2] --

def test_flip_equivariance_and_bidir_sum():
    r = rng(7)
    p = _rand_problem(r, Bsz=2, L=13, Dm=3, N=4, K=2, pos_delta=False)
    bias = r.uniform(-3, 0, (2, 3)).astype(F32)
    f = lambda k, x: x[:, k]
    fwd, sf = oracle.scan(f(0, p["u"]), f(0, p["delta"]), p["A"][0], f(0, p["B"]), f(0, p["C"]),
                          p["D"][0], None, bias[0], dir_mode=oracle.DIR_FWD)
    bwd, sb = oracle.scan(f(1, p["u"]), f(1, p["delta"]), p["A"][1], f(1, p["B"]), f(1, p["C"]),
                          p["D"][1], None, bias[1], dir_mode=oracle.DIR_BWD)
    flip = lambda x: np.ascontiguousarray(x[:, ::-1])
    bwd2, sb2 = oracle.scan(flip(f(1, p["u"])), flip(f(1, p["delta"])), p["A"][1], flip(f(1, p["B"])),
                            flip(f(1, p["C"])), p["D"][1], None, bias[1], dir_mode=oracle.DIR_FWD)
    np.testing.assert_array_equal(bwd, bwd2[:, ::-1])
    np.testing.assert_array_equal(sb, sb2)
    bi, sbi = oracle.scan(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], None, bias,
                          dir_mode=oracle.DIR_BIDIR)
    np.testing.assert_array_equal(bi, fwd + bwd)
    np.testing.assert_array_equal(sbi[:, 0], sf[:, 0])
    np.testing.assert_array_equal(sbi[:, 1], sb[:, 0])
    big, _ = oracle.scan(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], bias,
                         dir_mode=oracle.DIR_BIDIR)
    zz = p["z"].astype(np.float64)
    np.testing.assert_allclose(big, (fwd + bwd) * zz / (1 + np.exp(-zz)), rtol=1e-13, atol=1e-14)


# --- P6: Theorem 1: N = 1 reduces to a gated RNN [MFS §6.2 Step 5, eq (5)] -------------------

@pytest.mark.parametrize("exact", [True, False])
def test_theorem1_gated_rnn(exact):
    r = rng(8)
    L = 40
    s = r.standard_normal((1, L, 1)).astype(F32) * 2
    x = r.standard_normal((1, L, 1)).astype(F32)
    ones = np.ones((1, L, 1), F32)
    out, st = oracle.scan(x, s, np.full((1, 1), -1.0, F32), ones, ones, None, None, np.zeros(1, F32),
                          delta_softplus=True, exact_zoh=exact)
    g = 1.0 / (1.0 + np.exp(-s[0, :, 0].astype(np.float64)))  # g_t = σ(s_t)
    h, hs = 0.0, []
    for t in range(L):
        inp = g[t] if exact else -math.log1p(-g[t])         # exact B̄ = g; simplified B̄ = Δ = -log(1-g)
        h = (1.0 - g[t]) * h + inp * float(x[0, t, 0])
        hs.append(h)
    np.testing.assert_allclose(out[0, :, 0], hs, rtol=1e-12, atol=1e-13)


# --- P7: recurrent step continues a scan [MFS §2.3, recurrent form] --------------------------

def test_step_continues_scan():
    w = I.WORKLOADS["tiny_f32"].with_(batch=2, dim=8, dstate=4)
    x = I.make_inputs(w, seqlen=40)
    L0 = 32
    full, full_st = oracle.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"])
    _, st = oracle.scan(x["u"][:, :L0], x["delta"][:, :L0], x["A"], x["B"][:, :L0], x["C"][:, :L0],
                        x["D"], x["z"][:, :L0], x["delta_bias"])
    state = np.ascontiguousarray(st[:, 0])
    for t in range(L0, 40):
        o = oracle.step(state, x["u"][:, t], x["delta"][:, t], x["A"], x["B"][:, t], x["C"][:, t], x["D"],
                        x["z"][:, t], x["delta_bias"])
        np.testing.assert_allclose(o, full[:, t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(state, full_st[:, 0], rtol=1e-12, atol=1e-13)


# --- P8: one-hot input lands at exactly one state slot, with the closed-form value -------------

@pytest.mark.parametrize("mode,K", [(oracle.DIR_FWD, 1), (oracle.DIR_BWD, 1), (oracle.DIR_BIDIR, 2),
                                    (oracle.DIR_CROSS2D, 4)])
def test_one_hot_state_layout(mode, K):
    Bsz, H, W, Dm, N = 2, 3, 4, 5, 4
    L = H * W
    r = rng(9)
    Ku = 1 if mode == oracle.DIR_CROSS2D else K
    for trial in range(3):
        bs, ks, ds, ns = r.integers(Bsz), r.integers(K), r.integers(Dm), r.integers(N)
        first = oracle.token(mode, ks, 0, L, H, W)
        u = np.zeros((Bsz, Ku, L, Dm), F32)
        u[bs, 0 if Ku == 1 else ks, first, ds] = 1.0
        delta = r.uniform(0.05, 0.3, (Bsz, K, L, Dm)).astype(F32)
        B = np.zeros((Bsz, K, L, N), F32)
        B[bs, ks, first, ns] = 1.0
        C = r.standard_normal((Bsz, K, L, N)).astype(F32)
        A = -r.uniform(0.5, 2, (K, Dm, N)).astype(F32)
        _, st = oracle.scan(u, delta, A, B, C, None, None, None, dir_mode=mode, height=H, width=W,
                            delta_softplus=False)
        nz = np.argwhere(st != 0)
        assert nz.tolist() == [[bs, ks, ds, ns]]
        later = sum(float(delta[bs, ks, oracle.token(mode, ks, p, L, H, W), ds]) for p in range(1, L))
        want = float(delta[bs, ks, first, ds]) * math.exp(float(A[ks, ds, ns]) * later)
        assert abs(st[bs, ks, ds, ns] - want) <= 1e-13 * abs(want)


# --- P9: skip-only and zero gate; silu(z) - silu(-z) = z [MFS §6.2 Step 6] -----------------

def test_gate_and_skip():
    r = rng(10)
    p = _rand_problem(r, Bsz=1, L=10, Dm=3, N=4)
    u, delta, B, C, A, D, z = p["u"][:, 0], p["delta"][:, 0], p["B"][:, 0], p["C"][:, 0], p["A"][0], p["D"][0], p["z"]
    out0, _ = oracle.scan(u, delta, A, B, C, D, np.zeros_like(z), None, delta_softplus=False)
    assert np.all(out0 == 0)
    acc, _ = oracle.scan(u, delta, A, B, C, D, None, None, delta_softplus=False)
    op, _ = oracle.scan(u, delta, A, B, C, D, z, None, delta_softplus=False)
    om, _ = oracle.scan(u, delta, A, B, C, D, np.ascontiguousarray(-z), None, delta_softplus=False)
    np.testing.assert_allclose(op - om, acc * z, rtol=1e-12, atol=1e-13)
    skip, _ = oracle.scan(u, delta, A, B, np.zeros_like(C), D, None, None, delta_softplus=False)
    np.testing.assert_array_equal(skip, (D[None, None, :].astype(np.float64) * u))
    for zz in (-40.0, 0.0, 1.0, 40.0):
        assert abs(oracle.silu(zz) - oracle.silu(-zz) - zz) < 1e-14 * max(1, abs(zz))
    assert oracle.silu(-800.0) == 0.0 or abs(oracle.silu(-800.0)) < 1e-300


# --- P10: cross-scan orders: hand table, transpose symmetry, H = 1 [S4M §3] -------------------

def test_cross_scan_orders_hand_table():
    rows = np.loadtxt(os.path.join(GOLDEN, "ss2d_orders_2x3.txt"), dtype=np.int64)
    for row in rows:
        k, toks = int(row[0]), row[1:]
        got = [oracle.token(oracle.DIR_CROSS2D, k, p, 6, 2, 3) for p in range(6)]
        assert got == toks.tolist(), (k, got)
    assert [oracle.token(oracle.DIR_FWD, 0, p, 5) for p in range(5)] == [0, 1, 2, 3, 4]
    assert [oracle.token(oracle.DIR_BWD, 0, p, 5) for p in range(5)] == [4, 3, 2, 1, 0]
    for p in range(7):  # H = 1: the column-major order is the row-major order
        assert oracle.token(oracle.DIR_CROSS2D, 1, p, 7, 1, 7) == p
        assert oracle.token(oracle.DIR_CROSS2D, 3, p, 7, 1, 7) == 6 - p


def test_cross_scan_transpose_swaps_directions():
    r = rng(11)
    Bsz, H, Dm, N = 2, 4, 3, 4
    L = H * H
    p = _rand_problem(r, Bsz=Bsz, L=L, Dm=Dm, N=N, K=4, Ku=1, pos_delta=False)
    bias = r.uniform(-3, 0, (4, Dm)).astype(F32)
    T = lambda x: np.ascontiguousarray(x.reshape(x.shape[:-2] + (H, H, x.shape[-1])).swapaxes(-3, -2)
                                       .reshape(x.shape))
    perm = [1, 0, 3, 2]
    out, st = oracle.scan(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], bias,
                          dir_mode=oracle.DIR_CROSS2D, height=H, width=H)
    out2, st2 = oracle.scan(T(p["u"]), T(p["delta"][:, perm]), p["A"][perm], T(p["B"][:, perm]),
                            T(p["C"][:, perm]), p["D"][perm], T(p["z"]), bias[perm],
                            dir_mode=oracle.DIR_CROSS2D, height=H, width=H)
    np.testing.assert_allclose(out2, T(out), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st2, st[:, perm], rtol=1e-13, atol=1e-14)


# --- P11: softplus identities [MFS §4.1 τΔ; MUN §4 softplus] -----------------------------------

def test_softplus_identities():
    assert abs(oracle.softplus(0.0) - math.log(2.0)) < 1e-16
    for x in (-30.0, -5.0, -0.3, 0.7, 3.0, 25.0):
        assert abs(oracle.softplus(x) - oracle.softplus(-x) - x) < 1e-14 * max(1.0, abs(x))
    assert abs(oracle.softplus(-30.0) / math.exp(-30.0) - 1.0) < 1e-12
    assert oracle.softplus(60.0) == 60.0
    # softplus enters the scan as Δ: with N = 1, A = 0, B = C = 1, u = 1 the output is ΣΔ
    s = np.array([[[-2.0], [0.5], [3.0]]], F32)
    out, _ = oracle.scan(np.ones((1, 3, 1), F32), s, np.zeros((1, 1), F32), np.ones((1, 3, 1), F32),
                         np.ones((1, 3, 1), F32), None, None, np.full(1, 0.25, F32))
    want = np.cumsum([math.log1p(math.exp(float(v) + 0.25)) for v in s[0, :, 0]])
    np.testing.assert_allclose(out[0, :, 0], want, rtol=1e-14)


# --- determinism over thread count; bf16 inputs read from the same bits -------------------------

def test_thread_count_independent_and_bf16_decode():
    w = I.WORKLOADS["tiny_f32"].with_(dtype="bf16", batch=3, dim=24)
    x = I.make_inputs(w)
    a = oracle.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"], nthreads=1)
    b = oracle.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"], nthreads=7)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    f = {k: (I.bf16_to_f32(v) if v is not None and v.dtype == np.uint16 else v) for k, v in x.items()}
    c = oracle.scan(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"], f["delta_bias"])
    np.testing.assert_array_equal(a[0], c[0])
    rows = np.array([[2, 5], [0, 23]])
    r_out, r_st = oracle.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"], rows=rows)
    np.testing.assert_array_equal(r_out[0], a[0][2, :, 5])
    np.testing.assert_array_equal(r_st[1], a[1][0, :, 23])


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, np.inf, 0.0], F32)
    # 1+2^-8 is a tie between 1 and 1+2^-7: ties go to the even mantissa (1.0)
    got = I.bf16_to_f32(I.bf16_bits(x))
    np.testing.assert_array_equal(got, np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, np.inf, 0.0], F32))


def test_stored_tiny_oracle_output_unchanged():
    """Regression fixture written by tests/golden/make_golden.py (oracle only)."""
    path = os.path.join(GOLDEN, "tiny_f32_oracle.txt")
    want = np.loadtxt(path)
    x = I.make_inputs(I.WORKLOADS["tiny_f32"])
    out, st = oracle.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"])
    got = np.concatenate([out.reshape(-1), st.reshape(-1)])
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------------------------
# causal depthwise Conv1d + SiLU that produces u [MFS §6.2 Step 2; MFS §8 d_conv = 4;
# VIM §2.2 (each direction convolved); S4M §3 (depthwise convolution, then SiLU)]

def _conv_problem(r, Bsz=2, L=23, Dm=5, W=4):
    x = r.standard_normal((Bsz, L, Dm)).astype(F32)
    w = r.standard_normal((Dm, W)).astype(F32)
    b = r.standard_normal(Dm).astype(F32)
    return x, w, b


def test_conv_impulse_response_is_the_taps_in_causal_order():
    """A unit impulse at token t0 of one channel: the pre-activation output at
    t0 + k is tap W-1-k (the last tap weighs the current token), zero before t0
    (causal) and after t0 + W - 1."""
    r = rng(40)
    L, Dm, W, t0, d = 20, 3, 4, 7, 1
    x = np.zeros((1, L, Dm), F32)
    x[0, t0, d] = 1.0
    w = r.standard_normal((Dm, W)).astype(F32)
    pre = oracle.conv1d(x, w, None, activation=False)
    want = np.zeros(L)
    for k in range(W):
        want[t0 + k] = w[d, W - 1 - k]
    np.testing.assert_array_equal(pre[0, :, d], want)
    assert np.all(pre[0, :, [0, 2]] == 0.0)


def test_conv_matches_numpy_convolve_and_silu():
    """Pre-activation = bias + full linear convolution with the reversed taps,
    truncated to the first L outputs (numpy.convolve); output = z·sigmoid(z)."""
    r = rng(41)
    for W in (1, 2, 3, 4):
        x, w, b = _conv_problem(r, W=W)
        pre = oracle.conv1d(x, w, b, activation=False)
        out = oracle.conv1d(x, w, b)
        for bb in range(x.shape[0]):
            for d in range(x.shape[2]):
                ref = np.convolve(x[bb, :, d].astype(np.float64), w[d, ::-1].astype(np.float64))[: x.shape[1]]
                np.testing.assert_allclose(pre[bb, :, d], ref + float(b[d]), rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(out, pre / (1.0 + np.exp(-pre)), rtol=1e-14, atol=0)


def test_conv_identity_taps_and_linearity():
    r = rng(42)
    x, w, b = _conv_problem(r)
    ident = np.zeros_like(w)
    ident[:, -1] = 1.0
    np.testing.assert_array_equal(oracle.conv1d(x, ident, None, activation=False), x.astype(np.float64))
    x2 = r.standard_normal(x.shape).astype(F32)
    lhs = oracle.conv1d((x + x2).astype(F32), w, None, activation=False)
    rhs = oracle.conv1d(x, w, None, activation=False) + oracle.conv1d(x2, w, None, activation=False)
    # x + x2 is rounded to float32 before the convolution
    np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-5)


def test_conv_reverse_is_flipped_forward():
    r = rng(43)
    x, w, b = _conv_problem(r)
    fwd_of_flip = oracle.conv1d(np.ascontiguousarray(x[:, ::-1]), w, b)
    np.testing.assert_array_equal(oracle.conv1d(x, w, b, reverse=True), fwd_of_flip[:, ::-1])


def test_conv_bf16_inputs_widen_exactly():
    r = rng(44)
    x, w, b = _conv_problem(r)
    xb = I.bf16_bits(x)
    np.testing.assert_array_equal(oracle.conv1d(xb, w, b), oracle.conv1d(I.bf16_to_f32(xb), w, b))
