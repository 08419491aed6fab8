// scan_row.h -- the row-per-lane form of the selective-scan forward kernel.
//
// Sources, cited by page title and section:
//   [MFS] "从零理解 Mamba：选择性状态空间模型（Selective SSM）到 Mamba Block" (eutaboo.com)
//   [S4M] "从S4到Mamba：选择性状态空间模型的演进与革新" (jsqmd.com)
//   [MUN] "【临时文档---算法介绍】Mamba-UNet" (blog.csdn.net)
//   [VIM] "Vision Mamba：从状态空间模型到视觉革命的跨越" (x-humanoid.csdn.net)
//
// Work decomposition of scan_row_kernel: one wave (the whole workgroup) scans
// 64 consecutive channels of one (direction k, batch b) over one time chunk,
// and each lane owns one channel with all N of its states in registers.  The
// recurrence of a state never leaves its lane and the readout Σ_n C·h is an
// in-lane FMA chain [MFS §2.2 eq (2a)(2b)], so the kernel needs no LDS, no
// barrier and no cross-lane instruction:
//   * u, Δraw, z of the lane's channel are read per token with buffer loads
//     (the wave's 64 lanes read one contiguous row segment of the token-major
//     layout), issued PD tokens ahead of use;
//   * B_t and C_t are the same for every lane of the wave: they are read with
//     scalar loads into SGPRs, one (token, 8-state block) ahead, from fp32
//     copies padded to NP states that widen_bc_kernel writes first (so the
//     scalar unit, which the 64 waves of a CU share, only steps addresses);
//   * per token: Δ' = softplus(Δraw + bias)·log2 e once, then per state
//     Ā = 2^(Δ'·A) (one v_exp_f32), h = Ā·h + (Δ'·u·ln 2)·B and y += C·h
//     [MFS §6.2 Step 4 eq (4); MUN §4], then the D·u skip and the silu(z)
//     gate [MFS §6.2 Step 6];
//   * a sequence is split into chunks when its rows alone cannot fill the
//     GPU: an aggregate pass (AGG) scans every chunk but the last from a zero
//     state and stores its end state and ΣΔ'; the output pass starts chunk c
//     from the fold of the aggregates of chunks 0..c-1 [MFS §5; S4M §2.2].
// State sizes that are not a power of two run in the next power-of-two
// instantiation with the extra states held at A = 0, B = C = 0 (they stay 0
// and add nothing to the readout).
#pragma once

#include <type_traits>

#include "device_math.h"
#include "scan_kernels.h"

namespace mscan {

// Pointers into the constant address space: loads through them with a
// wave-uniform address become scalar (s_load) loads into SGPRs.
typedef const __attribute__((address_space(4))) uint32_t* cu32_ptr;

__device__ __forceinline__ cu32_ptr as_const_u32(const void* p) {
  return (cu32_ptr)(const __attribute__((address_space(4))) void*)(p);
}

// Scalar loads of NB consecutive fp32 values of a B or C row (from the padded
// fp32 copy), kept in SGPRs.
template <int NB>
struct RowBlock {
  uint32_t w[NB];
  __device__ __forceinline__ void load(const float* base, uint32_t e) {
    cu32_ptr q = as_const_u32(base);
#pragma unroll
    for (int j = 0; j < NB; ++j) w[j] = q[e + j];
  }
  __device__ __forceinline__ float get(int j) const { return __uint_as_float(w[j]); }
};

// B and C widened to fp32 rows of NP values, zero past the N values of each
// row: for each of B then C, a zero row, the [B][K][L][NP] rows, a zero row.
// One thread per output value.
template <typename TIn>
__global__ void __launch_bounds__(256) widen_bc_kernel(const TIn* __restrict__ B, const TIn* __restrict__ C,
                                                       float* __restrict__ out, int64_t rows, int N, int lognp) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per = (rows + 2) << lognp;
  if (i >= 2 * per) return;
  const bool isC = i >= per;
  const int64_t r = isC ? i - per : i;
  const int64_t row = (r >> lognp) - 1;  // -1 and rows: the padding
  const int n = (int)(r & ((1 << lognp) - 1));
  out[i] = (n < N && row >= 0 && row < rows) ? to_f32((isC ? C : B)[row * N + n]) : 0.f;
}

// Token order of one direction, walked one scan position at a time by the
// scalar unit without division or branches.  A row-major traversal is the
// column-major traversal of an L x 1 grid, so both are one walk over an
// Hs x Ws grid: scan position q visits token (q mod Hs)·Ws + q div Hs, and
// the next token is the current one plus Ws, or, where the row index wraps,
// plus 1 - (Hs - 1)·Ws (backwards: minus Ws, or (Hs - 1)·Ws - 1).  The step
// constants are shared by every walker of the direction.
struct WalkSteps {
  int dr, rwrap, rreset, dstep, dwrap, Hs, Ws;
  bool rev;
  __device__ __forceinline__ void init(int kind, int L, int H, int W) {
    const bool colwise = kind >= KIND_COL_FWD;
    rev = kind == KIND_ROW_REV || kind == KIND_COL_REV;
    Hs = colwise ? H : L;
    Ws = colwise ? W : 1;
    dr = rev ? -1 : 1;
    rwrap = rev ? -1 : Hs;
    rreset = rev ? Hs - 1 : 0;
    dstep = rev ? -Ws : Ws;
    dwrap = rev ? (Hs - 1) * Ws - 1 : 1 - (Hs - 1) * Ws;
  }
};
struct TokenWalk {
  int tok, r;
  __device__ __forceinline__ void init(const WalkSteps& w, int pbeg, int L) {
    const int q = w.rev ? L - 1 - pbeg : pbeg;
    r = q % w.Hs;
    tok = r * w.Ws + q / w.Hs;
  }
  __device__ __forceinline__ void next(const WalkSteps& w) {
    r += w.dr;
    const bool wrap = r == w.rwrap;
    r = wrap ? w.rreset : r;
    tok += wrap ? w.dwrap : w.dstep;
  }
};

// Makes the scalar registers of `v` count as read here, so that the wait for
// the scalar loads that fill them is placed here and not later.
template <int NW>
__device__ __forceinline__ void settle(const uint32_t (&v)[NW]) {
#pragma unroll
  for (int j = 0; j < NW; ++j) asm volatile("" ::"s"(v[j]));
}

// Scan positions ahead of use at which u, Δraw and z are loaded.
#ifndef MSCAN_ROW_PD
#define MSCAN_ROW_PD 8
#endif
constexpr int kRowPrefetch = MSCAN_ROW_PD;

// MODE: what the pass produces.
//   ROW_AGG      the aggregate pass: each chunk's end state from a zero state, and ΣΔ'
//   ROW_OUT      the output row of a one-direction scan, ungated, to out
//   ROW_OUT_GATE the same, gated by silu(z)
//   ROW_ROWS     the ungated fp32 row of each direction, to ws_y (several
//                directions; the merge kernel sums and gates them)
//   ROW_ANY      any output: the ungated fp32 rows (several directions, or kept
//                for the backward pass), out (gated when z is given), the
//                state checkpoints of the backward pass -- each when its
//                pointer is set
enum : int { ROW_AGG = 0, ROW_OUT = 1, ROW_OUT_GATE = 2, ROW_ROWS = 3, ROW_ANY = 4 };

// One wave = 64 channels of one (direction k, batch b) over one chunk of scan
// positions; lane = channel, all NP states of it in registers.  FULL: N == NP.
template <typename TIn, int NP, bool FULL, int MODE, bool EXACT>
__global__ void __launch_bounds__(64) scan_row_kernel(const ScanParams p) {
  constexpr bool AGG = MODE == ROW_AGG;
  constexpr bool ANY = MODE == ROW_ANY;
  const bool GATED = MODE == ROW_OUT_GATE || (ANY && p.z != nullptr && p.out != nullptr && p.K == 1);
  constexpr int NB = NP < 8 ? NP : 8;  // states per scalar-load block
  constexpr int NBLK = NP / NB;
  constexpr int PD = kRowPrefetch;
  const int lane = threadIdx.x;

  int bid = blockIdx.x;
  const int dblk = bid % p.nblk_d;
  bid /= p.nblk_d;
  const int c = bid % p.grid_chunks;
  bid /= p.grid_chunks;
  const int b = bid % p.Bsz;
  const int k = bid / p.Bsz;

  const int D = p.Dm, L = p.L, N = p.N;
  const int d = dblk * 64 + lane;
  const bool dvalid = d < D;
  const int dc = dvalid ? d : D - 1;  // loads of lanes past D read a valid channel
  const int kind = (p.kinds >> (2 * k)) & 3;
  const int ku = (p.Ku == 1) ? 0 : k;
  const int pbeg = c * p.chunk_len;
  const int pend = min(L, pbeg + p.chunk_len);
  const bool direct = MODE == ROW_OUT || MODE == ROW_OUT_GATE || (ANY && p.out != nullptr && p.K == 1);
  const bool rows_out = MODE == ROW_ROWS || (ANY && p.ws_y != nullptr);
  const bool ckpt = ANY && p.ckpt != nullptr;

  constexpr uint32_t ES = sizeof(TIn);
  const uint32_t slice = (uint32_t)((int64_t)L * D * ES);
  const auto rs_u = make_rsrc(static_cast<const TIn*>(p.u) + (int64_t)(b * p.Ku + ku) * L * D, slice);
  const auto rs_dl = make_rsrc(static_cast<const TIn*>(p.delta) + (int64_t)(b * p.K + k) * L * D, slice);
  const auto rs_z = make_rsrc(GATED ? static_cast<const TIn*>(p.z) + (int64_t)b * L * D : nullptr, GATED ? slice : 0u);
  const auto rs_out = make_rsrc(direct ? static_cast<TIn*>(p.out) + (int64_t)b * L * D : nullptr, direct ? slice : 0u);
  const auto rs_ws = make_rsrc(rows_out ? p.ws_y + ((int64_t)k * p.Bsz + b) * L * D : nullptr,
                               rows_out ? (uint32_t)((int64_t)L * D * 4) : 0u);
  // the (direction, batch) slice of the padded fp32 copies of B and C (each
  // copy is preceded and followed by one zero row)
  const int64_t bc_rows = (int64_t)p.Bsz * p.K * L;
  const float* Bw = p.bcw + ((int64_t)b * p.K + k) * L * NP;  // the row before the slice
  const float* Cw = Bw + (bc_rows + 2) * NP;

  // ---- per-lane constants and the starting state ----
  float Al2[NP], h[NP], invA[EXACT ? NP : 1];
#pragma unroll
  for (int n = 0; n < NP; ++n) {
    Al2[n] = (FULL || n < N) ? p.A[((int64_t)k * D + dc) * N + n] : 0.f;  // 2^(Δ'·A) = e^(Δ·A)
    if constexpr (EXACT) invA[n] = Al2[n] != 0.f ? 1.0f / Al2[n] : 0.f;
    h[n] = 0.f;
  }
  const int64_t agg_row = ((int64_t)k * p.Bsz + b) * (p.nchunks - 1);
  if (c == 0) {
    if (p.init_state) {
#pragma unroll
      for (int n = 0; n < NP; ++n)
        if (FULL || n < N) h[n] = p.init_state[(((int64_t)b * p.K + k) * D + dc) * N + n];
    }
  } else if (!AGG) {
    // fold the aggregates of chunks 0..c-1: h <- 2^(ΣΔ'_j·A)·h + S_j, the
    // aggregates of FB chunks loaded together before their updates (about
    // 64 registers of them), so chunk c waits for ceil(c / FB) memory round
    // trips instead of c
    constexpr int FB = NP >= 64 ? 1 : 64 / NP < kFoldBatch ? 64 / NP : kFoldBatch;
    for (int j0 = 0; j0 < c; j0 += FB) {
      float dsv[FB], Sv[FB][NP];
#pragma unroll
      for (int q = 0; q < FB; ++q) {
        const int jj = min(j0 + q, c - 1);  // (past c: the last aggregate again, unused)
        dsv[q] = p.agg_dsum[(agg_row + jj) * D + dc];
        const float* S = p.agg_state + ((agg_row + jj) * D + dc) * N;
#pragma unroll
        for (int n = 0; n < NP; ++n) Sv[q][n] = (FULL || n < N) ? S[n] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < FB; ++q) {
        if (j0 + q < c) {
#pragma unroll
          for (int n = 0; n < NP; ++n)
            if (FULL || n < N) h[n] = __builtin_fmaf(ex2(dsv[q] * Al2[n]), h[n], Sv[q][n]);
        }
      }
    }
  }
  const float bias = p.delta_bias ? p.delta_bias[k * D + dc] : 0.f;
  const float Dd = p.D ? p.D[k * D + dc] : 0.f;

  const uint32_t voff = (uint32_t)dc * ES;
  const uint32_t voff4 = (uint32_t)dc * 4u;
  const uint32_t rowb = (uint32_t)D * ES;
  const int nsteps = pend - pbeg;

  // ---- u, Δraw, z loaded PD positions ahead into a ring of register sets ----
  TIn rdl[PD], ru[PD], rz[PD];
  WalkSteps ws;
  ws.init(kind, L, p.H, p.W);
  TokenWalk lw;  // the next position to load
  lw.init(ws, pbeg, L);
  // (past the chunk end the walk goes on into positions that are never used;
  // their loads are clamped to a token of the slice)
  auto issue = [&](int slot) {
    const uint32_t soff = (uint32_t)min(max(lw.tok, 0), L - 1) * rowb;
    rdl[slot] = buf_load(rs_dl, voff, soff, (TIn*)nullptr);
    ru[slot] = buf_load(rs_u, voff, soff, (TIn*)nullptr);
    if (GATED) rz[slot] = buf_load(rs_z, voff, soff, (TIn*)nullptr);
    lw.next(ws);
  };
#pragma unroll
  for (int s = 0; s < PD; ++s) issue(s);

  // ---- B and C by scalar loads, one (position, 8-state block) ahead ----
  TokenWalk tw;  // the position being scanned
  tw.init(ws, pbeg, L);
  TokenWalk bw = tw;  // the position of the next B/C block to load
  // B and C blocks in two buffers used in turn: while block i is computed
  // from one buffer, block i + 1 loads into the other
  // (the prefetch of the block after the chunk's last one reads the next row
  // of the walk, token -1 or L at worst: the copies have a zero row of
  // padding before and after each of B and C, and addresses are taken from
  // the row before the slice so that they stay non-negative)
  int bblk = 0;
  RowBlock<NB> bufB[2], bufC[2];
  auto bc_addr = [&]() { return (uint32_t)(bw.tok + 1) * (uint32_t)NP + (uint32_t)(bblk * NB); };
  auto advance_bc = [&]() {
    if (++bblk == NBLK) {
      bblk = 0;
      bw.next(ws);
    }
  };
  bufB[0].load(Bw, bc_addr());
  if constexpr (!AGG) bufC[0].load(Cw, bc_addr());
  advance_bc();

  float dsum = 0.f;
  // The scan loop, instantiated with and without the softplus of Δ (a
  // uniform choice, kept out of the loop body).  Whole groups of PD positions
  // refill every slot of the load ring unconditionally (so each slot carries
  // one value around the loop and the waits stay PD positions behind the
  // loads); the last nsteps mod PD positions follow without refills.
  auto scan = [&](auto softplus_tag) {
    constexpr bool SP = decltype(softplus_tag)::value;
    auto do_step = [&](const int j, const int step, const bool refill) {
      const int pp = pbeg + step;
      if (ckpt && (pp & (p.ckpt_every - 1)) == 0 && dvalid) {
        // the state before this position, every ckpt_every (a power of two)
        // positions, for the backward pass
        float* S = p.ckpt + ((((int64_t)k * p.Bsz + b) * p.ckpt_tiles + pp / p.ckpt_every) * D + d) * N;
#pragma unroll
        for (int n = 0; n < NP; ++n)
          if (FULL || n < N) S[n] = h[n];
      }
      const float x = to_f32(rdl[j]) + bias;
      const float dl = SP ? softplus_log2(x) : x * kLog2e;  // Δ' = Δ·log2 e
      const float uu = to_f32(ru[j]);
      float zz = 0.f;
      if (GATED) zz = to_f32(rz[j]);
      if (refill) issue(j);  // refill this slot PD positions ahead
      const float du = EXACT ? uu : dl * (uu * kLn2);  // Δ·u (B unscaled)
      float y = 0.f;
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk) {
        // this block's values (loaded one block earlier) are waited for here,
        // then the next block's loads are issued: a scalar-load wait covers
        // every scalar load in flight, so the next loads must come after the
        // wait for these (NBLK * PD is even, so each block's buffer is fixed)
        const int cur = (j * NBLK + blk) & 1;
        const RowBlock<NB>& curB = bufB[cur];
        const RowBlock<NB>& curC = bufC[cur];
        settle(curB.w);
        if constexpr (!AGG) settle(curC.w);
        __builtin_amdgcn_sched_barrier(0);
        bufB[cur ^ 1].load(Bw, bc_addr());  // (the last position's row again at the end)
        if constexpr (!AGG) bufC[cur ^ 1].load(Cw, bc_addr());
        advance_bc();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int jn = 0; jn < NB; ++jn) {
          const int n = blk * NB + jn;
          const float t = dl * Al2[n];
          const float a = ex2(t);
          if constexpr (EXACT) {
            const float cf = zoh_coef_b2(a, t, dl, invA[n]);  // (e^{ΔA} - 1)/A
            h[n] = __builtin_fmaf(cf * du, curB.get(jn), a * h[n]);
          } else {
            h[n] = __builtin_fmaf(du, curB.get(jn), a * h[n]);
          }
          if constexpr (!AGG) y = __builtin_fmaf(curC.get(jn), h[n], y);
        }
      }
      if constexpr (AGG) {
        dsum += dl;
      } else {
        y = __builtin_fmaf(Dd, uu, y);
        if (dvalid) {
          if (rows_out) buf_store(y, rs_ws, voff4, (uint32_t)tw.tok * (uint32_t)D * 4u);  // ungated
          if (GATED) y *= silu_f(zz);
          if (direct) store_out(y, rs_out, voff, (uint32_t)tw.tok * rowb, (TIn*)nullptr);
        }
      }
      tw.next(ws);
    };
    int s0 = 0;
    for (; s0 + PD <= nsteps; s0 += PD) {
#pragma unroll
      for (int j = 0; j < PD; ++j) do_step(j, s0 + j, true);
    }
#pragma unroll
    for (int j = 0; j < PD - 1; ++j)
      if (s0 + j < nsteps) do_step(j, s0 + j, false);
  };
  if (p.softplus)
    scan(std::true_type{});
  else
    scan(std::false_type{});

  if (!dvalid) return;
  if constexpr (AGG) {
    float* S = p.agg_state + ((agg_row + c) * D + d) * N;
#pragma unroll
    for (int n = 0; n < NP; ++n)
      if (FULL || n < N) S[n] = h[n];
    p.agg_dsum[(agg_row + c) * D + d] = dsum;
  } else if (c == p.nchunks - 1 && p.last_state) {
    float* S = p.last_state + (((int64_t)b * p.K + k) * D + d) * N;
#pragma unroll
    for (int n = 0; n < NP; ++n)
      if (FULL || n < N) S[n] = h[n];
  }
}

}  // namespace mscan
