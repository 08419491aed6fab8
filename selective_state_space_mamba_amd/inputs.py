"""Seeded synthetic inputs for the selective scan.

This module only draws random numbers and rounds them to the storage dtype;
it holds none of the scan's arithmetic, so the HIP path and the CPU oracle can
both be fed from it without sharing any of the method.

Recipe (every workload):
  * generator ``numpy.random.Generator(PCG64(seed))``; draws in the order
    dt, u, delta, z, B, C, D (A is deterministic);
  * A[k, d, n] = -(n + 1) for every direction k and channel d (S4D-real);
  * dt[k, d] log-uniform in [1e-3, 1e-1] and delta_bias = log(expm1(dt)),
    the inverse of softplus, so that softplus(delta_bias) = dt;
  * u, delta, z, B, C, D standard normal float32; u, delta, z, B, C are then
    rounded to bfloat16 (round to nearest even) for the bf16 workloads and kept
    as uint16 bit patterns; A, D and delta_bias stay float32.

Layouts (token-major, C-contiguous; K scan directions):
  u [B][Ku][L][D] (Ku = 1 for the cross scan, otherwise K; the K axis is
  dropped when K = 1), delta [B][K][L][D], B and C [B][K][L][N], z [B][L][D],
  A [K][D][N], D and delta_bias [K][D].
"""
from __future__ import annotations

import dataclasses

import numpy as np

DIR_FWD, DIR_BWD, DIR_BIDIR, DIR_CROSS2D = 0, 1, 2, 3
_NDIRS = {DIR_FWD: 1, DIR_BWD: 1, DIR_BIDIR: 2, DIR_CROSS2D: 4}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    dim: int
    seqlen: int
    dstate: int
    dir_mode: int
    dtype: str  # "f32" or "bf16"
    gated: bool
    seed: int
    height: int = 0
    width: int = 0

    @property
    def ndirs(self) -> int:
        return _NDIRS[self.dir_mode]

    @property
    def elements(self) -> int:
        return self.ndirs * self.batch * self.dim * self.seqlen * self.dstate

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads the scan is specified on (the Vim one in two sizes).
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 16, 64, 4, DIR_FWD, "f32", True, 1001),
    "mamba130m_layer": Workload("mamba130m_layer", 8, 1536, 2048, 16, DIR_FWD, "bf16", True, 1002),
    "long_context": Workload("long_context", 1, 2048, 262144, 16, DIR_FWD, "bf16", True, 1003),
    "vim_bidir_224": Workload("vim_bidir_224", 128, 768, 197, 16, DIR_BIDIR, "bf16", True, 1041),
    "vim_bidir_1248": Workload("vim_bidir_1248", 1, 768, 97344, 16, DIR_BIDIR, "bf16", True, 1042),
    "vmamba_ss2d": Workload("vmamba_ss2d", 32, 192, 4096, 16, DIR_CROSS2D, "bf16", False, 1005,
                            height=64, width=64),
}
DECODE_STEPS = 512  # decode steps that continue the mamba130m_layer scan


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in, flat_out = x.reshape(-1), out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_in.size, step):
        v = flat_in[s:s + step].view(np.uint32)
        r = (v + (np.uint32(0x7FFF) + ((v >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
        r = r.astype(np.uint16)
        nan = np.isnan(flat_in[s:s + step])
        if nan.any():
            r[nan] = np.uint16(0x7FC0)
        flat_out[s:s + step] = r
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    return (np.ascontiguousarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng, shape, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return bf16_bits(x) if dtype == "bf16" else x


def make_inputs(w: Workload, seqlen: int | None = None) -> dict:
    """Draw one input set for workload ``w`` (optionally with another sequence length)."""
    L = w.seqlen if seqlen is None else seqlen
    K, Bsz, Dm, N = w.ndirs, w.batch, w.dim, w.dstate
    Ku = 1 if w.dir_mode == DIR_CROSS2D else K
    rng = np.random.Generator(np.random.PCG64(w.seed))
    A = np.ascontiguousarray(np.broadcast_to(-(np.arange(N, dtype=np.float32) + 1.0), (K, Dm, N)))
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=(K, Dm)))
    delta_bias = np.log(np.expm1(dt)).astype(np.float32)
    ushape = (Bsz, L, Dm) if Ku == 1 else (Bsz, Ku, L, Dm)
    dshape = (Bsz, L, Dm) if K == 1 else (Bsz, K, L, Dm)
    bshape = (Bsz, L, N) if K == 1 else (Bsz, K, L, N)
    u = _normal(rng, ushape, w.dtype)
    delta = _normal(rng, dshape, w.dtype)
    z = _normal(rng, (Bsz, L, Dm), w.dtype)
    B = _normal(rng, bshape, w.dtype)
    C = _normal(rng, bshape, w.dtype)
    D = rng.standard_normal(size=(K, Dm), dtype=np.float32)
    if K == 1:
        A, D, delta_bias = A.reshape(Dm, N), D.reshape(Dm), delta_bias.reshape(Dm)
    return dict(u=u, delta=delta, z=z if w.gated else None, B=B, C=C, A=A, D=D,
                delta_bias=delta_bias)


def make_conv_inputs(batch: int, seqlen: int, dim: int, width: int, dtype: str, seed: int) -> dict:
    """Inputs of the causal depthwise Conv1d + SiLU prologue: x [B][L][D] standard
    normal (rounded to bf16 for bf16), weight [D][W] and bias [D] uniform in
    ±1/sqrt(W) (the default initialisation of a depthwise Conv1d, fan-in W)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = _normal(rng, (batch, seqlen, dim), dtype)
    bound = 1.0 / np.sqrt(width)
    weight = rng.uniform(-bound, bound, size=(dim, width)).astype(np.float32)
    bias = rng.uniform(-bound, bound, size=dim).astype(np.float32)
    return dict(x=x, weight=weight, bias=bias)


def make_dout(w: Workload, seqlen: int | None = None) -> np.ndarray:
    """Upstream gradient dout [B][L][D] of the backward pass: standard normal,
    rounded to bf16 for bf16 workloads, from its own stream of the workload's seed."""
    L = w.seqlen if seqlen is None else seqlen
    rng = np.random.Generator(np.random.PCG64([w.seed, 2]))
    return _normal(rng, (w.batch, L, w.dim), w.dtype)


def make_inputs_device(w: Workload, device, seed: int | None = None) -> dict:
    """The make_inputs recipe drawn on a GPU with torch's generator, for the
    throughput measurement of workloads too large to draw quickly on the host:
    the same shapes and distributions (A = -(n + 1); dt log-uniform in
    [1e-3, 1e-1] and delta_bias = log(expm1(dt)); u, delta, z, B, C, D standard
    normal, rounded to bfloat16 to nearest even for the bf16 workloads), not the
    same values as make_inputs.  Returns torch tensors on `device`."""
    import torch
    K, Bsz, L, Dm, N = w.ndirs, w.batch, w.seqlen, w.dim, w.dstate
    Ku = 1 if w.dir_mode == DIR_CROSS2D else K
    g = torch.Generator(device=device)
    g.manual_seed(w.seed if seed is None else seed)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def normal(shape):
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(tdt)

    A = -(torch.arange(N, device=device, dtype=torch.float32) + 1.0).expand(K, Dm, N).contiguous()
    lo, hi = float(np.log(1e-3)), float(np.log(1e-1))
    dt = torch.exp(torch.rand((K, Dm), generator=g, device=device, dtype=torch.float64) * (hi - lo) + lo)
    delta_bias = torch.log(torch.expm1(dt)).to(torch.float32)
    ushape = (Bsz, L, Dm) if Ku == 1 else (Bsz, Ku, L, Dm)
    dshape = (Bsz, L, Dm) if K == 1 else (Bsz, K, L, Dm)
    bshape = (Bsz, L, N) if K == 1 else (Bsz, K, L, N)
    x = dict(u=normal(ushape), delta=normal(dshape), z=normal((Bsz, L, Dm)) if w.gated else None,
             B=normal(bshape), C=normal(bshape), A=A,
             D=torch.randn((K, Dm), generator=g, device=device, dtype=torch.float32), delta_bias=delta_bias)
    if K == 1:
        x["A"], x["D"], x["delta_bias"] = x["A"].reshape(Dm, N), x["D"].reshape(Dm), x["delta_bias"].reshape(Dm)
    return x


def host_channel_sample(w: Workload, xd: dict, channels) -> dict:
    """The inputs of a subset of channels (all batches, directions, tokens and
    states), copied from device tensors made by make_inputs_device to numpy
    arrays in the layout make_inputs returns (bf16 as uint16 bit patterns).
    Channels are independent rows of the scan, so the subset is a workload of
    its own with dim = len(channels)."""
    import torch
    idx = torch.as_tensor(np.asarray(channels, dtype=np.int64), device=xd["u"].device)

    def host(t, last_is_channel=True):
        if t is None:
            return None
        if last_is_channel:
            t = t.index_select(t.dim() - 1, idx)
        t = t.contiguous().cpu()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    out = {k: host(xd[k]) for k in ("u", "delta", "z", "D", "delta_bias")}
    out["A"] = host(xd["A"].index_select(xd["A"].dim() - 2, idx), last_is_channel=False)
    out["B"] = host(xd["B"], last_is_channel=False)
    out["C"] = host(xd["C"], last_is_channel=False)
    return out
