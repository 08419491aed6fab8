"""The scan entry points (forward, backward, decode step) inside captured HIP
graphs and on concurrent streams.

A launch-bound loop (the one-token decode step, or many short scans) can be
captured once as a HIP graph and replayed with no host work per call.  The
library allocates nothing, clears nothing with memset and keeps no state
between calls, so a captured sequence of its launches must reproduce the eager
results exactly.  Each graph here is replayed several times, with other eager
work and synchronisations between the replays, and every replay is compared
bit for bit with the eager result.  Independent calls on two streams at once
must also give the results of the same calls made one after the other.
"""
import numpy as np
import pytest

import selective_state_space_mamba_amd as ms
from selective_state_space_mamba_amd import inputs as I

from scanutil import dev_inputs, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    ms.load_library()
    yield


def announce(msg):
    print("[gpu case] " + msg, flush=True)


W = I.Workload
GRAPH_FWD = [
    # a long sequence with few rows: time split (aggregate pass, fold, workspace)
    W("graph_split", 1, 64, 4133, 16, I.DIR_FWD, "bf16", True, 61),
    W("graph_bidir", 2, 32, 300, 16, I.DIR_BIDIR, "bf16", True, 62),
    W("graph_cross", 1, 32, 96, 8, I.DIR_CROSS2D, "f32", False, 63, 8, 12),
]


def fwd_call(w, xd, out, st, ws, stream):
    ms.scan_fwd(xd["u"], xd["delta"], xd["A"], xd["B"], xd["C"], xd.get("D"), xd.get("z"), xd.get("delta_bias"),
                dir_mode=w.dir_mode, height=w.height, width=w.width, out=out, last_state=st, workspace=ws,
                stream=stream)


@pytest.mark.parametrize("w", GRAPH_FWD, ids=[w.name for w in GRAPH_FWD])
def test_fwd_graph_replays(w):
    t = torch()
    announce("graph fwd %s" % (w,))
    xd = dev_inputs(I.make_inputs(w))
    other = dev_inputs(I.make_inputs(w.with_(seed=w.seed + 100)))
    dims = ms.make_dims(w.batch, w.dim, w.seqlen, w.dstate, ms.DTYPE_BF16 if w.dtype == "bf16" else ms.DTYPE_F32,
                        height=w.height, width=w.width)
    ws = t.empty(max(ms.workspace_bytes(dims, w.dir_mode), 256), dtype=t.uint8, device="cuda:0")
    kx = () if w.ndirs == 1 else (w.ndirs,)
    tdt = xd["u"].dtype
    out_e = t.empty((w.batch, w.seqlen, w.dim), dtype=tdt, device="cuda:0")
    st_e = t.empty((w.batch,) + kx + (w.dim, w.dstate), dtype=t.float32, device="cuda:0")
    out_g, st_g = t.empty_like(out_e), t.empty_like(st_e)
    out_o, st_o = t.empty_like(out_e), t.empty_like(st_e)
    s = t.cuda.current_stream()
    fwd_call(w, xd, out_e, st_e, ws, s)
    t.cuda.synchronize()
    graph = t.cuda.CUDAGraph()
    cs = t.cuda.Stream()
    cs.wait_stream(s)
    with t.cuda.graph(graph, stream=cs):
        fwd_call(w, xd, out_g, st_g, ws, cs)
    t.cuda.synchronize()
    for rep in range(3):
        out_g.fill_(0)
        st_g.fill_(0)
        fwd_call(w, other, out_o, st_o, ws, s)  # eager work on the same workspace between replays
        t.cuda.synchronize()
        graph.replay()
        t.cuda.synchronize()
        assert t.equal(out_g, out_e), "%s replay %d out" % (w.name, rep)
        assert t.equal(st_g, st_e), "%s replay %d last_state" % (w.name, rep)


def test_step_graph_replays():
    """Eight decode steps captured once; each replay restarts from the same state."""
    t = torch()
    w = W("graph_step", 4, 64, 16, 16, I.DIR_FWD, "bf16", True, 64)
    announce("graph step %s" % (w,))
    x = I.make_inputs(w)
    xd = dev_inputs(x)
    st0 = t.from_numpy(np.random.Generator(np.random.PCG64([w.seed, 3])).standard_normal(
        (w.batch, w.dim, w.dstate)).astype(np.float32)).to("cuda:0")
    cols = {k: [xd[k][:, i].contiguous() for i in range(8)] for k in ("u", "delta", "B", "C", "z")}

    def steps(st, outs, stream):
        for i in range(8):
            ms.scan_step(st, cols["u"][i], cols["delta"][i], xd["A"], cols["B"][i], cols["C"][i], xd["D"],
                         cols["z"][i], xd["delta_bias"], out=outs[i], stream=stream)
    s = t.cuda.current_stream()
    st_e = st0.clone()
    outs_e = [t.empty_like(cols["u"][0]) for _ in range(8)]
    steps(st_e, outs_e, s)
    t.cuda.synchronize()
    st_g = st0.clone()
    outs_g = [t.empty_like(cols["u"][0]) for _ in range(8)]
    graph = t.cuda.CUDAGraph()
    cs = t.cuda.Stream()
    cs.wait_stream(s)
    t.cuda.synchronize()
    with t.cuda.graph(graph, stream=cs):
        steps(st_g, outs_g, cs)
    t.cuda.synchronize()
    for rep in range(3):
        st_g.copy_(st0)
        for o in outs_g:
            o.fill_(0)
        t.cuda.synchronize()
        graph.replay()
        t.cuda.synchronize()
        assert t.equal(st_g, st_e), "replay %d state" % rep
        for i in range(8):
            assert t.equal(outs_g[i], outs_e[i]), "replay %d step %d" % (rep, i)


def test_two_streams():
    """Two independent forward scans and a backward pass on two streams at once
    equal the same calls made one after the other."""
    t = torch()
    w1 = W("streams_a", 2, 64, 700, 16, I.DIR_FWD, "bf16", True, 65)
    w2 = W("streams_b", 2, 32, 300, 16, I.DIR_BIDIR, "bf16", True, 66)
    announce("two streams %s %s" % (w1, w2))
    x1, x2 = dev_inputs(I.make_inputs(w1)), dev_inputs(I.make_inputs(w2))
    dout1 = dev_inputs({"g": I.make_dout(w1)})["g"]

    def run(s1, s2):
        with t.cuda.stream(s1):
            o1, st1 = ms.scan_fwd(x1["u"], x1["delta"], x1["A"], x1["B"], x1["C"], x1["D"], x1["z"],
                                  x1["delta_bias"], stream=s1)
            g1 = ms.scan_bwd(x1["u"], x1["delta"], x1["A"], x1["B"], x1["C"], x1["D"], x1["z"], x1["delta_bias"],
                             dout=dout1, stream=s1)
        with t.cuda.stream(s2):
            o2, st2 = ms.scan_fwd(x2["u"], x2["delta"], x2["A"], x2["B"], x2["C"], x2["D"], x2["z"],
                                  x2["delta_bias"], dir_mode=w2.dir_mode, stream=s2)
        t.cuda.synchronize()
        return o1, st1, o2, st2, g1
    seq = run(t.cuda.current_stream(), t.cuda.current_stream())
    sa, sb = t.cuda.Stream(), t.cuda.Stream()
    par = run(sa, sb)
    for a, b in zip(seq[:4], par[:4]):
        assert t.equal(a, b)
    for k in seq[4]:
        if seq[4][k] is not None:
            assert t.equal(seq[4][k], par[4][k]), k


def test_side_stream_allocations_belong_to_the_launch_stream():
    """Calls on a stream other than torch's current one (a torch stream, then a
    raw handle), with no workspace given, allocate their workspace and outputs
    from the launch stream's pool.  Right after each call the current stream
    fills fresh allocations of the workspace's size; had the dropped workspace
    gone back to the current stream's pool, those fills could overwrite it
    while the scan still ran.  Every result equals the plain call's."""
    t = torch()
    w = W("side_split", 1, 64, 4133, 16, I.DIR_FWD, "bf16", True, 67)  # time split: needs a workspace
    announce("side stream %s" % (w,))
    xd = dev_inputs(I.make_inputs(w))
    dout = dev_inputs({"g": I.make_dout(w)})["g"]
    dims = ms.make_dims(w.batch, w.dim, w.seqlen, w.dstate, ms.DTYPE_BF16)
    ws_need = ms.workspace_bytes(dims, w.dir_mode)
    bws_need = ms.bwd_workspace_bytes(dims, w.dir_mode)
    assert ws_need > 0

    def fwd(stream=None):
        return ms.scan_fwd(xd["u"], xd["delta"], xd["A"], xd["B"], xd["C"], xd["D"], xd["z"], xd["delta_bias"],
                           stream=stream)

    def bwd(stream=None):
        return ms.scan_bwd(xd["u"], xd["delta"], xd["A"], xd["B"], xd["C"], xd["D"], xd["z"], xd["delta_bias"],
                           dout=dout, stream=stream)

    ref_out, ref_st = fwd()
    ref_g = bwd()
    t.cuda.synchronize()
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    got, junk = [], []
    for rep in range(4):
        handle = s if rep % 2 == 0 else s.cuda_stream
        got.append((fwd(handle), bwd(handle)))
        junk += [t.empty(n, dtype=t.uint8, device="cuda:0").fill_(255) for n in (ws_need, bws_need)]
    t.cuda.synchronize()
    for rep, ((o, st), g) in enumerate(got):
        assert t.equal(o, ref_out) and t.equal(st, ref_st), "call %d" % rep
        for k, v in ref_g.items():
            if v is not None:
                assert t.equal(g[k], v), "call %d %s" % (rep, k)


GRAPH_BWD = [
    W("graph_bwd_split", 1, 64, 4133, 16, I.DIR_FWD, "bf16", True, 68),  # time-split recompute and adjoint
    W("graph_bwd_bidir", 2, 32, 300, 16, I.DIR_BIDIR, "bf16", True, 69),
    W("graph_bwd_cross", 1, 32, 96, 8, I.DIR_CROSS2D, "f32", True, 70, 8, 12),
]


@pytest.mark.parametrize("w", GRAPH_BWD, ids=[w.name for w in GRAPH_BWD])
def test_bwd_graph_replays(w):
    """The backward pass (forward recompute, adjoint sweep, sums) captured once
    and replayed, with other eager backward calls between the replays."""
    t = torch()
    announce("graph bwd %s" % (w,))
    xd = dev_inputs(I.make_inputs(w))
    other = dev_inputs(I.make_inputs(w.with_(seed=w.seed + 100)))
    dout = dev_inputs({"g": I.make_dout(w)})["g"]

    def bwd(x, stream=None):
        return ms.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x.get("D"), x.get("z"), x.get("delta_bias"),
                           dout=dout, dir_mode=w.dir_mode, height=w.height, width=w.width, stream=stream)

    ref = bwd(xd)
    t.cuda.synchronize()
    graph = t.cuda.CUDAGraph()
    cs = t.cuda.Stream()
    cs.wait_stream(t.cuda.current_stream())
    with t.cuda.graph(graph, stream=cs):
        got = bwd(xd, cs)
    t.cuda.synchronize()
    for rep in range(3):
        for v in got.values():
            if v is not None:
                v.fill_(0)
        bwd(other)  # eager work between replays
        t.cuda.synchronize()
        graph.replay()
        t.cuda.synchronize()
        for k, v in ref.items():
            if v is not None:
                assert t.equal(got[k], v), "%s replay %d %s" % (w.name, rep, k)
