"""Pins of the fp64 backward oracle (oracle.scan_bwd) against central finite
differences of the forward oracle: every gradient entry of every input, for
every direction mode, both input-term rules, softplus on and off, with gate,
skip, bias and initial state.  Finite differences need no derivation, so a
slip anywhere in the adjoint recurrence or in a chain-rule factor fails here.

The training pass recomputes states and runs the adjoint recurrence [MFS §5;
S4M §2.3]; the forward it differentiates is the pinned forward oracle.
Sources, cited by page title and section:
  [MFS] "从零理解 Mamba：选择性状态空间模型（Selective SSM）到 Mamba Block" (eutaboo.com)
  [S4M] "从S4到Mamba：选择性状态空间模型的演进与革新" (jsqmd.com)
"""
import numpy as np
import pytest

import oracle

F32 = np.float32


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def problem(r, mode, softplus, gated, with_init, exact, Bsz=2, H=2, W=3, Dm=3, N=3):
    L = H * W
    K = oracle.num_dirs(mode)
    Ku = 1 if mode == oracle.DIR_CROSS2D else K
    kx = () if K == 1 else (K,)
    ux = () if Ku == 1 else (Ku,)
    x = {
        "u": r.standard_normal((Bsz,) + ux + (L, Dm)).astype(F32),
        "delta": (r.standard_normal((Bsz,) + kx + (L, Dm)) if softplus
                  else r.uniform(0.05, 0.6, (Bsz,) + kx + (L, Dm))).astype(F32),
        "B": r.standard_normal((Bsz,) + kx + (L, N)).astype(F32),
        "C": r.standard_normal((Bsz,) + kx + (L, N)).astype(F32),
        "A": (-r.uniform(0.2, 2.0, kx + (Dm, N))).astype(F32),
        "D": r.standard_normal(kx + (Dm,)).astype(F32),
        "delta_bias": (r.uniform(-1.0, 0.5, kx + (Dm,)) if softplus else r.uniform(0.0, 0.2, kx + (Dm,))).astype(F32),
        "z": r.standard_normal((Bsz, L, Dm)).astype(F32) if gated else None,
        "initial_state": r.standard_normal((Bsz,) + kx + (Dm, N)).astype(F32) if with_init else None,
    }
    if exact:
        x["A"].reshape(-1)[::4] = 0.0  # the A = 0 limit of the exact rule
    dout = r.standard_normal((Bsz, L, Dm)).astype(F32)
    kw = dict(dir_mode=mode, height=H if mode == oracle.DIR_CROSS2D else 0,
              width=W if mode == oracle.DIR_CROSS2D else 0, delta_softplus=softplus, exact_zoh=exact)
    return x, dout, kw


def loss(x, dout, kw):
    out, _ = oracle.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                         initial_state=x["initial_state"], nthreads=1, **kw)
    return float(np.sum(dout.astype(np.float64) * out))


def fd_grad(x, name, dout, kw):
    arr = x[name]
    g = np.empty(arr.shape)
    flat = arr.reshape(-1)
    for i in range(flat.size):
        v = flat[i]
        h = F32(1e-3 * max(1.0, abs(float(v))))
        vp, vm = F32(v + h), F32(v - h)
        flat[i] = vp
        lp = loss(x, dout, kw)
        flat[i] = vm
        lm = loss(x, dout, kw)
        flat[i] = v
        g.reshape(-1)[i] = (lp - lm) / (float(vp) - float(vm))
    return g


GRAD_OF = {"u": "du", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "z": "dz",
           "delta_bias": "ddelta_bias", "initial_state": "dinit"}

CASES = [
    ("fwd", oracle.DIR_FWD, True, True, True, False),
    ("fwd_exact", oracle.DIR_FWD, True, True, True, True),
    ("fwd_nosoftplus", oracle.DIR_FWD, False, False, False, False),
    ("bwd", oracle.DIR_BWD, True, True, False, False),
    ("bidir", oracle.DIR_BIDIR, True, True, True, False),
    ("bidir_exact_nosoftplus", oracle.DIR_BIDIR, False, True, False, True),
    ("cross2d", oracle.DIR_CROSS2D, True, False, True, False),
    ("cross2d_exact", oracle.DIR_CROSS2D, True, True, False, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_finite_differences(case):
    name, mode, softplus, gated, with_init, exact = case
    r = rng(300 + CASES.index(case))
    x, dout, kw = problem(r, mode, softplus, gated, with_init, exact)
    g = oracle.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"], dout,
                        initial_state=x["initial_state"], **kw)
    for inp, gname in GRAD_OF.items():
        if x[inp] is None:
            continue
        fd = fd_grad(x, inp, dout, kw)
        got = g[gname]
        assert got.shape == fd.shape, (inp, got.shape, fd.shape)
        scale = max(1.0, float(np.max(np.abs(fd))))
        err = float(np.max(np.abs(got - fd))) / scale
        assert err < 2e-5, (name, inp, err)


def test_backward_with_zero_dout_is_zero_and_linear_in_dout():
    r = rng(320)
    x, dout, kw = problem(r, oracle.DIR_BIDIR, True, True, True, False)
    args = (x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"])
    g0 = oracle.scan_bwd(*args, np.zeros_like(dout), initial_state=x["initial_state"], **kw)
    assert all(np.all(v == 0.0) for v in g0.values() if v is not None)
    g1 = oracle.scan_bwd(*args, dout, initial_state=x["initial_state"], **kw)
    g2 = oracle.scan_bwd(*args, (2 * dout).astype(F32), initial_state=x["initial_state"], **kw)
    for k in g1:
        if g1[k] is not None:
            np.testing.assert_allclose(g2[k], 2 * g1[k], rtol=1e-12, atol=1e-15)
