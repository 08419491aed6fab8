// scan_kernels.h -- gfx950 HIP kernels of the selective (S6) scan.
//
// Sources, cited by page title and section:
//   [MFS] "从零理解 Mamba：选择性状态空间模型（Selective SSM）到 Mamba Block" (eutaboo.com)
//   [S4M] "从S4到Mamba：选择性状态空间模型的演进与革新" (jsqmd.com)
//   [MUN] "【临时文档---算法介绍】Mamba-UNet" (blog.csdn.net)
//   [VIM] "Vision Mamba：从状态空间模型到视觉革命的跨越" (x-humanoid.csdn.net)
//
// Work decomposition of scan_chunk_kernel (one workgroup):
//   * CB consecutive channels d of one (direction k, batch b); thread i owns
//     channel i mod CB and G of the N states of that channel, held in
//     registers for the whole scan (NG = N/G threads share a channel);
//   * a contiguous range ("chunk") of scan positions; a sequence is split
//     into several chunks only when (k, b, channel-block) rows alone cannot
//     fill the GPU.  Chunks are joined by the associativity of the affine
//     step h -> a·h + b [MFS §5; S4M §2.2, chunked scan with aggregation]:
//     a first pass (AGG = true) scans each chunk from a zero state and
//     records its end state S_c and ΣΔ over the chunk (the chunk's decay is
//     exp(A·ΣΔ) since Ā_t = exp(Δ_t·A)); the output pass folds the aggregates
//     of the chunks before it into its starting state;
//   * the chunk is streamed in tiles of TT scan positions (32, or 64 for one
//     state per thread at N = 16 on long sequences): u, Δraw, z are read
//     through buffer descriptors, two adjacent channels per thread and load
//     with 16-channel blocks (each token's channel row is contiguous in the
//     token-major layout whatever the traversal order), two tiles ahead of
//     use, then staged in LDS as
//     (Δ', Δ'·u) pairs -- Δ' = Δ·log2 e, softplus and the product computed once
//     per (token, channel) -- next to B·ln 2 and C rows shared by the channels;
//   * per scan step and state: Ā = 2^(Δ'·A) = exp(Δ·A) (one v_exp_f32),
//     h = Ā·h + (Δ'u)·(B ln 2), and the partial readout Σ C·h over the
//     thread's G states [MFS §2.2 eq (2a)(2b); §6.2 Step 4 eq (4); MUN §4];
//   * the NG partial readouts meet in LDS (NG/4 with 16-channel blocks, whose
//     waves first sum their 4 state rows in registers); the epilogue adds them,
//     adds the D·u skip [MUN §4], applies the silu(z) gate [MFS §6.2 Step 6]
//     and stores the output row.  With several directions the ungated fp32
//     row goes to a workspace slice instead and merge_dirs_kernel sums the
//     directions in order and gates [VIM §2.2; S4M §3].
// No B·D·L·N intermediate is ever written to memory.
#pragma once

#include "device_math.h"

namespace mscan {

// Quads (4 scan steps) ahead at which the scan loop reads its LDS operands:
// 2 with one state per thread in 16-channel blocks (the 130M layer: 147.0 ->
// 143.6 µs on MI355X), 1 otherwise (2 states per thread have no registers to
// spare: Vim-224 234 -> 286 µs).
#ifndef MSCAN_LDS_PD
#define MSCAN_LDS_PD 0  // 0: the choice above; 1, 2, 3: that depth everywhere
#endif

// Chunk aggregates whose loads are issued together when a chunk of a time
// split folds the aggregates of the chunks before it.
#ifndef MSCAN_FOLD_BATCH
#define MSCAN_FOLD_BATCH 8
#endif
constexpr int kFoldBatch = MSCAN_FOLD_BATCH;

// Traversal kinds: token index of scan position p.
enum : int { KIND_ROW_FWD = 0, KIND_ROW_REV = 1, KIND_COL_FWD = 2, KIND_COL_REV = 3 };

__device__ __forceinline__ int token_of(int kind, int p, int L, int H, int W) {
  if (kind == KIND_ROW_FWD) return p;
  if (kind == KIND_ROW_REV) return L - 1 - p;
  const int q = (kind == KIND_COL_FWD) ? p : L - 1 - p;
  return (q % H) * W + q / H;
}

struct ScanParams {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;           // may be null
  const void* z;            // may be null
  const float* delta_bias;  // may be null
  const float* init_state;  // [Bsz][K][D][N] or null
  void* out;                // [Bsz][L][D]: written here with one direction (K = 1), else by the
                            // direction merge; null: no output row
  float* ws_y;              // [K][Bsz][L][D] ungated fp32 rows (several directions; with one
                            // direction, kept for the backward pass) or null
  float* last_state;        // [Bsz][K][D][N] or null
  float* agg_state;         // [K][Bsz][nchunks-1][D][N]
  float* agg_dsum;          // [K][Bsz][nchunks-1][D]
  float* ckpt;              // [K][Bsz][ckpt_tiles][D][N] state before every ckpt_every-th
                            // position (ckpt_every 16 or 32, a divisor of the tile), or null
  float* bcw;               // row kernel: B then C widened to fp32 rows of NP values, [Bsz][K][L][NP] each
  int Bsz, Dm, L, H, W;
  int N;                    // state size (the row kernel may run a larger power-of-two instantiation)
  int K, Ku;
  int kinds;                // 4 x 2-bit traversal kind, direction k at bits 2k..2k+1
  int nchunks;              // chunks per sequence (>= 1)
  int chunk_len;            // scan positions per chunk (multiple of the tile)
  int grid_chunks;          // chunks covered by this launch's grid
  int nblk_d;               // channel blocks of 64
  int softplus;
  int ckpt_tiles;           // checkpoint rows per sequence: ceil(L / ckpt_every)
  int ckpt_every;           // positions between checkpoints
  int prio;                 // 1: the scan loop runs at raised wave priority (16-channel blocks)
  int kbase;                // first direction of this launch's grid
  int fold;                 // 1 (two directions only): the launch's direction, k = 1, adds
                            // direction 0's row from ws_y to its own output and writes the
                            // gated result to out (no merge kernel, no row of its own)
};
// Template flag EXACT of the kernels below: exact zero-order-hold input term
// ((e^{ΔA} - 1)/A)·B·u instead of Δ·B·u [MFS §6.2 Step 4, eq (4)].

// Maps blockIdx.x to the logical workgroup index so that the 64/CB workgroups
// covering one 64-channel (128-byte bf16) row segment run on the same XCD:
// consecutive blockIdx values go round-robin to the 8 XCDs, each with its own L2.
__device__ __forceinline__ int logical_block(int bid, int nblocks, int S) {
  if (S == 1) return bid;
  const int span = 8 * S;
  const int full = nblocks / span * span;
  if (bid >= full) return bid;
  const int j = (bid / span) * 8 + (bid % 8);  // group of S logical blocks
  const int s = (bid / 8) % S;
  return j * S + s;
}

// One workgroup scans CB consecutive channels of one (direction k, batch b) over
// one chunk of scan positions.  Thread i owns channel c = i % CB and the state
// group ng = i / CB (states ng*G .. ng*G+G-1); NT = CB*N/G threads.  For the
// staging and the epilogue the same thread owns channel c and the TPT = TT/NG
// consecutive scan positions ng*TPT .. ng*TPT+TPT-1 of each tile.
template <typename TIn, int N, int G, int CB, int TT, bool AGG, bool EXACT>
// (64-position tiles: a 4-waves-per-SIMD register budget, 128 VGPRs; without
// it the in-tile checkpoints take the kernel to 132 and 3 waves)
__global__ void __launch_bounds__(CB * N / G, TT == 64 ? 4 : 1) scan_chunk_kernel(const ScanParams p) {
  constexpr int NG = N / G;    // state groups per channel
  constexpr int NT = CB * NG;  // threads per workgroup
  static_assert(NT % 64 == 0 && NT <= 1024, "whole waves");
  static_assert(TT % NG == 0, "tile splits evenly over state groups");
  constexpr int TPT = TT / NG;            // tile positions staged per thread
  constexpr int EQ = N < 4 ? N : 4;       // B/C elements per load unit
  constexpr int UPR = N / EQ;             // load units per token row
  constexpr int BCU = TT * UPR;           // load units per tile per tensor
  constexpr int BCI = (BCU + NT - 1) / NT;
  constexpr int YS = TT + 4;              // partial-readout row: stride 36 dwords, conflict-free b128
  constexpr int DS = 2 * TT + 4;          // (Δ', Δu) row of one channel: 68 dwords, conflict-free b128
  constexpr int BS = TT + 4;              // B or C row of one state: 36 dwords
  static_assert(TT % 4 == 0 && TPT % 2 == 0, "the scan loop runs 4 steps per iteration");
  static_assert(G <= 4, "at most 4 states per thread");

  // Every LDS row is time-contiguous, so one 16-byte read serves 2 steps of
  // (Δ', Δu) or 4 steps of B or C.
  __shared__ float s_dd[CB * DS];              // [c][2t] = Δ'_t, [c][2t+1] = Δ_t·u_t
  __shared__ float s_B[N * BS];                // [n][t] = B_t[n]·ln 2
  __shared__ float s_C[AGG ? 4 : N * BS];      // [n][t] = C_t[n]
  // Partial readouts, time-contiguous.  With 16-channel blocks a wave holds 4
  // state rows of the same 16 channels; they are summed in registers first
  // (two cross-lane swap stages), so each output has NG/4 partials.
  constexpr int NY = CB == 16 ? NG / 4 : NG;
  // Wave priorities (s_setprio) of a tile's phases.  The few waves per SIMD
  // are in different phases at any time; letting the arbiter prefer one phase
  // shortens the chain of tiles of every wave.  Measured on MI355X: with
  // 16-channel blocks and few waves per SIMD (p.prio, set by the plan),
  // preferring the scan loop (scan 1, epilogue and staging 0) took the 130M
  // layer from 151 to 139 µs (3 waves per SIMD) and the 130M-shaped layer at
  // N = 32 / 64 from 220 / 401 to 204 / 367 µs; with many waves no preference
  // is better (Vim-224 at 24 waves per SIMD 211 -> 206 µs, the 262k-token
  // context 4.22 -> 4.02 ms); with 64-channel blocks (now only N = 1 and 2),
  // preferring staging over the scan (staging 2, scan 1, epilogue 0) took
  // Vim-224 from 245 to 238 µs when it still ran on them.
  constexpr int P_EPI = 0;
  constexpr int P_STAGE = CB == 16 ? 0 : 2;
  // Staging and epilogue ownership.  With 16-channel blocks (PAIR) a thread
  // stages and stores two adjacent channels at PPT consecutive positions of a
  // tile: one 32-bit (bf16) or 64-bit (f32) load per tensor and position and
  // one store per position, half the memory instructions of one channel at
  // two positions.  With 64-channel blocks a thread keeps one channel at TPT
  // positions (the wave's row offsets are then scalars).
  constexpr bool PAIR = CB == 16;
  constexpr int NPR = CB / 2;                           // channel pairs per block
  constexpr int PPT = PAIR ? TT * NPR / NT : TPT;       // positions staged per thread
  constexpr int EPT = PAIR ? 2 * PPT : TPT;             // (position, channel) elements per thread
  static_assert(!PAIR || (TT * NPR) % NT == 0, "a tile's pairs split evenly over the threads");
  // partial readouts: [group][position][channel] with 16-channel blocks (two
  // adjacent channels of a position are one 8-byte read), [group][channel][position]
  // with 64 (each thread writes 4 steps of its channel at once)
  __shared__ float s_y[AGG ? 1 : NY][AGG ? 1 : (PAIR ? TT : CB)][AGG ? 4 : (PAIR ? CB : YS)];

  const int tid = threadIdx.x;
  const int cl = tid % CB;  // channel within the block
  // state group (scan) / position group (staging, epilogue); wave-uniform when
  // a wave spans the whole 64-channel block, and then kept in a scalar register
  const int ng = CB == 64 ? __builtin_amdgcn_readfirstlane(tid / CB) : tid / CB;

  const int nblocks = gridDim.x;
  int bid = logical_block(blockIdx.x, nblocks, 64 / CB < 1 ? 1 : 64 / CB);
  const int dblk = bid % p.nblk_d;
  bid /= p.nblk_d;
  const int c = bid % p.grid_chunks;
  bid /= p.grid_chunks;
  const int b = bid % p.Bsz;
  const int k = p.kbase + bid / p.Bsz;

  const int D = p.Dm, L = p.L;
  const int d0 = dblk * CB;
  const int d = d0 + cl;
  const bool dvalid = d < D;
  const int kind = (p.kinds >> (2 * k)) & 3;
  const int ku = (p.Ku == 1) ? 0 : k;
  const int pbeg = c * p.chunk_len;
  const int pend = min(L, pbeg + p.chunk_len);

  // u, Δraw, z, out and the per-direction fp32 rows are read and written through
  // buffer descriptors over this (k, b) slice: a scalar row offset plus the
  // lane's constant channel offset, no per-access vector address arithmetic.
  constexpr uint32_t ES = sizeof(TIn);
  const uint32_t slice = (uint32_t)((int64_t)L * D * ES);
  const TIn* u_slice = static_cast<const TIn*>(p.u) + (int64_t)(b * p.Ku + ku) * L * D;
  const TIn* dl_slice = static_cast<const TIn*>(p.delta) + (int64_t)(b * p.K + k) * L * D;
  const auto rs_u = make_rsrc(u_slice, slice);
  const auto rs_dl = make_rsrc(dl_slice, slice);
  const auto rs_z = make_rsrc(p.z ? static_cast<const TIn*>(p.z) + (int64_t)b * L * D : nullptr, p.z ? slice : 0u);
  // the gated output row is written here with one direction, or by the
  // folding last direction; the ungated fp32 rows whenever ws_y is given
  // (except by the folding direction, which reads them)
  const bool fold = !AGG && p.fold != 0;
  const bool direct = !AGG && p.out != nullptr && (p.K == 1 || fold);
  const auto rs_ws = make_rsrc(p.ws_y ? p.ws_y + ((int64_t)k * p.Bsz + b) * L * D : nullptr,
                               p.ws_y ? (uint32_t)((int64_t)L * D * 4) : 0u);
  const auto rs_out = make_rsrc(direct ? static_cast<TIn*>(p.out) + (int64_t)b * L * D : nullptr, direct ? slice : 0u);
  // direction 0's fp32 row, read by the folding direction
  const auto rs_fold = make_rsrc(fold ? p.ws_y + (int64_t)b * L * D : nullptr, fold ? (uint32_t)((int64_t)L * D * 4) : 0u);
  const TIn* __restrict__ B_base = static_cast<const TIn*>(p.B) + (int64_t)(b * p.K + k) * L * N;
  const TIn* __restrict__ C_base = static_cast<const TIn*>(p.C) + (int64_t)(b * p.K + k) * L * N;
  const bool gated = direct && p.z != nullptr;

  // ---- per-lane constants and the starting state ----
  float Al2[G], h[G], invA[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const int n = ng * G + j;
    Al2[j] = dvalid ? p.A[((int64_t)k * D + d) * N + n] : 0.f;  // 2^(Δ'·A) = e^(Δ·A)
    invA[j] = Al2[j] != 0.f ? 1.0f / Al2[j] : 0.f;
    h[j] = 0.f;
  }
  const int64_t agg_row = ((int64_t)k * p.Bsz + b) * (p.nchunks - 1);
  if (c == 0) {
    if (p.init_state && dvalid) {
#pragma unroll
      for (int j = 0; j < G; ++j) h[j] = p.init_state[(((int64_t)b * p.K + k) * D + d) * N + ng * G + j];
    }
  } else if (!AGG && dvalid) {
    // fold the aggregates of chunks 0..c-1: h <- exp(A·ΣΔ_j)·h + S_j, ΣΔ_j kept as ΣΔ'_j.
    // The aggregates of kFoldBatch chunks are loaded together before their
    // updates, so chunk c waits for ceil(c / kFoldBatch) memory round trips
    // instead of c (the loads do not depend on h; only the updates chain).
    for (int j0 = 0; j0 < c; j0 += kFoldBatch) {
      float dsv[kFoldBatch], Sv[kFoldBatch][G];
#pragma unroll
      for (int q = 0; q < kFoldBatch; ++q) {
        const int jj = min(j0 + q, c - 1);  // (past c: the last aggregate again, unused)
        dsv[q] = p.agg_dsum[(agg_row + jj) * D + d];
        const float* S = p.agg_state + ((agg_row + jj) * D + d) * N + ng * G;
#pragma unroll
        for (int j = 0; j < G; ++j) Sv[q][j] = S[j];
      }
#pragma unroll
      for (int q = 0; q < kFoldBatch; ++q) {
        if (j0 + q < c) {
#pragma unroll
          for (int j = 0; j < G; ++j) h[j] = __builtin_fmaf(ex2(dsv[q] * Al2[j]), h[j], Sv[q][j]);
        }
      }
    }
  }
  // the staging and epilogue elements of this thread: channels e0 (and e0 + 1
  // with PAIR) at positions ppos0 .. ppos0 + PPT - 1 of each tile; pairs are
  // aligned and D is a multiple of 8, so both channels of a pair exist or neither
  const int e0 = PAIR ? 2 * (tid % NPR) : cl;
  const int ppos0 = PAIR ? (tid / NPR) * PPT : ng * TPT;
  const bool evalid = d0 + e0 < D;
  float bias2[2], Dd2[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int de = d0 + e0 + (PAIR ? j : 0);
    bias2[j] = (evalid && p.delta_bias) ? p.delta_bias[k * D + de] : 0.f;
    Dd2[j] = (evalid && p.D) ? p.D[k * D + de] : 0.f;
  }
  // The state registers may still be waiting on the loads above; settle them
  // here so that no wait on global loads lands inside the scan loop, where it
  // would also wait for the next tile's prefetch.
  __builtin_amdgcn_s_waitcnt(0);

  // Row-major traversals (every direction except the cross scan's column-major
  // ones) visit a tile's tokens as one contiguous run: token row offsets are
  // then scalars and each access is a scalar base plus the lane's channel.
  const bool rowwise = kind < KIND_COL_FWD;
  const bool rev = kind == KIND_ROW_REV;
  auto token = [&](int pp) { return rowwise ? (rev ? L - 1 - pp : pp) : token_of(kind, pp, L, p.H, p.W); };

  // raw (undecoded) loads of one tile; two sets rotate so that a tile's loads
  // are issued two tiles before it is staged
  struct Raw {
    Pair<TIn> pdl[PAIR ? PPT : 1], pu[PAIR ? PPT : 1], pz[PAIR ? PPT : 1];
    TIn dl[PAIR ? 1 : TPT], u[PAIR ? 1 : TPT], z[PAIR ? 1 : TPT];
    Small<TIn, EQ> B[BCI], C[BCI];
  };
  Raw r0, r1;
  float Du[EPT], gate[EPT], folded[EPT];
  if constexpr (PAIR) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      r0.pdl[i].zero(); r0.pu[i].zero(); r0.pz[i].zero();
      r1.pdl[i].zero(); r1.pu[i].zero(); r1.pz[i].zero();
    }
  } else {
#pragma unroll
    for (int i = 0; i < TPT; ++i) r0.dl[i] = r0.u[i] = r0.z[i] = r1.dl[i] = r1.u[i] = r1.z[i] = TIn(0);
  }
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    Du[i] = 0.f;
    gate[i] = 1.f;
    folded[i] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < BCI; ++i) {
    r0.B[i].zero();
    r0.C[i].zero();
    r1.B[i].zero();
    r1.C[i].zero();
  }

  // Element offsets of this thread's channel; rows outside the chunk and
  // channels beyond D are clamped to valid addresses (their values are zeroed
  // at staging and never stored).
  // (a pair's first channel is clamped to D - 2: D is even)
  const int dlast = D - (PAIR ? 2 : 1) - d0;
  const uint32_t voff_in = (uint32_t)(d0 + min(e0, dlast)) * ES;
  const uint32_t voff_ws = (uint32_t)(d0 + min(e0, dlast)) * 4u;
  const uint32_t voff_out = (uint32_t)(d0 + min(e0, dlast)) * ES;
  const bool dfull = d0 + CB <= D;
  // Byte offset of the token row of scan position pp (clamped into the chunk)
  // for a row of D elements of es bytes.  Tokens and row strides are below
  // 2^24 (checked on the host), so the full-rate 24-bit multiply serves.
  auto row_off = [&](int pp, uint32_t es) { return __umul24((uint32_t)token(min(pp, pend - 1)), (uint32_t)D * es); };
  // Loads are issued unconditionally (rows clamped into the chunk), so the
  // wait before staging covers exactly the older of the two tiles in flight.
  auto load_tile = [&](int p0, Raw& r) {
    if constexpr (PAIR) {
#pragma unroll
      for (int i = 0; i < PPT; ++i) {
        const uint32_t voff = voff_in + row_off(p0 + ppos0 + i, ES);
        r.pdl[i].load(rs_dl, voff);
        r.pu[i].load(rs_u, voff);
        if (gated) r.pz[i].load(rs_z, voff);
      }
    } else {
#pragma unroll
      for (int i = 0; i < TPT; ++i) {
        // the row offset is a scalar only when the wave's rows are one row (CB = 64)
        const uint32_t roff = row_off(p0 + ng * TPT + i, ES);
        const uint32_t soff = CB == 64 ? roff : 0u;
        const uint32_t voff = CB == 64 ? voff_in : voff_in + roff;
        r.dl[i] = buf_load(rs_dl, voff, soff, (TIn*)nullptr);
        r.u[i] = buf_load(rs_u, voff, soff, (TIn*)nullptr);
        if (gated) r.z[i] = buf_load(rs_z, voff, soff, (TIn*)nullptr);
      }
    }
#pragma unroll
    for (int i = 0; i < BCI; ++i) {
      const int q = min(tid + i * NT, BCU - 1);
      const int tt = q / UPR, nq = q % UPR;
      const uint32_t off = __umul24((uint32_t)token(min(p0 + tt, pend - 1)), (uint32_t)N) + nq * EQ;
      r.B[i].load(B_base + off);
      if constexpr (!AGG) r.C[i].load(C_base + off);
    }
  };

  auto stage_tile = [&](int p0, const Raw& r) {
    __builtin_amdgcn_s_setprio(P_STAGE);
    if constexpr (PAIR) {
      // (Δ', Δu) of channels e0, e0 + 1 at positions ppos0 .. ppos0 + PPT - 1
      float dd[2][2 * PPT];
#pragma unroll
      for (int i = 0; i < PPT; ++i) {
        const int tt = ppos0 + i;
        const float okf = ((p0 + tt < pend) && evalid) ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float x = r.pdl[i].get(j) + bias2[j];
          const float dl = (p.softplus ? softplus_log2(x) : x * kLog2e) * okf;  // Δ' = Δ·log2 e
          const float uu = r.pu[i].get(j) * okf;
          dd[j][2 * i] = dl;
          dd[j][2 * i + 1] = EXACT ? uu : dl * uu;
          if constexpr (!AGG) {
            Du[2 * i + j] = Dd2[j] * uu;
            if (gated) gate[2 * i + j] = silu_f(r.pz[i].get(j));
          }
        }
      }
      if constexpr (!AGG) {
        if (fold) {
          // the folded row at this thread's epilogue elements, read a whole
          // tile before its use
#pragma unroll
          for (int i = 0; i < PPT; ++i) {
            Pair<float> f2;
            f2.load(rs_fold, voff_ws + row_off(p0 + ppos0 + i, 4u));
            folded[2 * i] = f2.get(0);
            folded[2 * i + 1] = f2.get(1);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float* row = &s_dd[(e0 + j) * DS + 2 * ppos0];
        if constexpr (PPT == 1) {
          *reinterpret_cast<float2*>(row) = make_float2(dd[j][0], dd[j][1]);
        } else {
#pragma unroll
          for (int m = 0; m < PPT / 2; ++m)
            *reinterpret_cast<float4*>(row + 4 * m) =
                make_float4(dd[j][4 * m], dd[j][4 * m + 1], dd[j][4 * m + 2], dd[j][4 * m + 3]);
        }
      }
    } else {
    float dd[2 * TPT];
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int tt = ng * TPT + i;
      // Branch-free: compute on whatever the registers hold (finite values of
      // clamped rows and channels), then zero rows past the chunk end and
      // channels past D by a 0/1 factor -- cheaper than a select per value.
      const float okf = ((p0 + tt < pend) && dvalid) ? 1.f : 0.f;
      const float x = to_f32(r.dl[i]) + bias2[0];
      const float dl = (p.softplus ? softplus_log2(x) : x * kLog2e) * okf;  // Δ' = Δ·log2 e
      const float uu = to_f32(r.u[i]) * okf;
      dd[2 * i] = dl;
      dd[2 * i + 1] = EXACT ? uu : dl * uu;
      if constexpr (!AGG) {
        Du[i] = Dd2[0] * uu;
        if (gated) gate[i] = silu_f(to_f32(r.z[i]));
      }
    }
    if constexpr (!AGG) {
      if (fold) {
        // direction 0's row at this thread's epilogue positions (a fold is
        // planned for two directions only), read here, a whole tile before
        // its use: one load per position and no wait for it until then
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
          const uint32_t roff = row_off(p0 + ng * TPT + i, 4u);
          folded[i] = buf_load(rs_fold, CB == 64 ? voff_ws : voff_ws + roff, CB == 64 ? roff : 0u, (float*)nullptr);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < TPT / 2; ++m)
      *reinterpret_cast<float4*>(&s_dd[cl * DS + 2 * ng * TPT + 4 * m]) =
          make_float4(dd[4 * m], dd[4 * m + 1], dd[4 * m + 2], dd[4 * m + 3]);
    }
#pragma unroll
    for (int i = 0; i < BCI; ++i) {
      const int q = tid + i * NT;
      if (q < BCU) {
        const int tt = q / UPR, nq = q % UPR;
        const float okq = p0 + tt < pend ? 1.f : 0.f;
        const float bscale = okq * (EXACT ? 1.f : kLn2);  // Δ·B = Δ'·(B·ln 2)
#pragma unroll
        for (int e = 0; e < EQ; ++e) {
          s_B[(nq * EQ + e) * BS + tt] = r.B[i].get(e) * bscale;
          if constexpr (!AGG) s_C[(nq * EQ + e) * BS + tt] = r.C[i].get(e) * okq;
        }
      }
    }
  };

  float dsum = 0.f;
  // one tile: barrier, scan, barrier, epilogue (the next tile is staged by the caller)
  auto process_tile = [&](int p0) {
    // the state before position pos, for the recomputation of the backward
    // pass (at the tile start, and inside the tile every ckpt_every positions)
    auto checkpoint = [&](int pos) {
      if (!AGG && p.ckpt && dvalid && pos < pend) {
        float* S = p.ckpt + ((((int64_t)k * p.Bsz + b) * p.ckpt_tiles + pos / p.ckpt_every) * D + d) * N + ng * G;
#pragma unroll
        for (int j = 0; j < G; ++j) S[j] = h[j];
      }
    };
    checkpoint(p0);
    __syncthreads();
    const int tlen = min(TT, pend - p0);
    // Rows of the tile past the chunk end were staged as Δ' = 0, Δu = 0, B = C = 0:
    // such a step leaves the state exactly unchanged (Ā = 2^0 = 1, input 0), so
    // the loop runs branch-free over whole groups of 4 steps.  Software-pipelined
    // over two register sets: the operands of the next two steps are read from
    // LDS while the current two compute.
    const int tend = (tlen + 3) & ~3;
    // Operands of 4 steps: two 16-byte reads of (Δ', Δu) and one of B and of C
    // per state.  Software-pipelined over two sets: the next 4 steps' operands
    // are read while the current 4 compute.
    struct Ops {
      float dl[4], du[4];
      float B[G][4], C[G][4];
    };
    auto read_ops = [&](Ops& o, int tt) {
      const float4 d01 = *reinterpret_cast<const float4*>(&s_dd[cl * DS + 2 * tt]);
      const float4 d23 = *reinterpret_cast<const float4*>(&s_dd[cl * DS + 2 * tt + 4]);
      o.dl[0] = d01.x; o.du[0] = d01.y; o.dl[1] = d01.z; o.du[1] = d01.w;
      o.dl[2] = d23.x; o.du[2] = d23.y; o.dl[3] = d23.z; o.du[3] = d23.w;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float4 bv = *reinterpret_cast<const float4*>(&s_B[(ng * G + j) * BS + tt]);
        o.B[j][0] = bv.x; o.B[j][1] = bv.y; o.B[j][2] = bv.z; o.B[j][3] = bv.w;
        if constexpr (!AGG) {
          const float4 cv = *reinterpret_cast<const float4*>(&s_C[(ng * G + j) * BS + tt]);
          o.C[j][0] = cv.x; o.C[j][1] = cv.y; o.C[j][2] = cv.z; o.C[j][3] = cv.w;
        }
      }
    };
    // Four steps: the exps and input products do not depend on the state; the
    // state updates and partial readouts follow in step order.
    auto quad = [&](const Ops& o, int tt) {
      float a[4][G], bu[4][G];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < G; ++j) {
          const float t = o.dl[r] * Al2[j];  // Δ'·A = ΔA / ln 2
          a[r][j] = ex2(t);
          if constexpr (EXACT) {
            // (e^{ΔA} - 1)/A · B·u
            bu[r][j] = zoh_coef_b2(a[r][j], t, o.dl[r], invA[j]) * (o.du[r] * o.B[j][r]);
          } else {
            bu[r][j] = o.du[r] * o.B[j][r];
          }
        }
      float y[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < G; ++j) {
          h[j] = __builtin_fmaf(a[r][j], h[j], bu[r][j]);
          if constexpr (!AGG) y[r] = __builtin_fmaf(o.C[j][r], h[j], y[r]);
        }
      if constexpr (AGG) dsum += (o.dl[0] + o.dl[1]) + (o.dl[2] + o.dl[3]);
      else if constexpr (CB == 16) {
        // Steps (0, 2) and (1, 3): swapping lanes 32-63 of one with lanes 0-31
        // of the other and adding sums the wave's two halves (rows 0+2, 1+3),
        // steps 0/1 landing in the low half and 2/3 in the high half; the
        // same with odd/even 16-lane rows then sums rows 0+1 (2+3), leaving
        // in row r the 4-row sum of step r.
        const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(y[0]), __float_as_uint(y[2]), false, false);
        const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(y[1]), __float_as_uint(y[3]), false, false);
        const float z02 = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);
        const float z13 = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);
        const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(z02), __float_as_uint(z13), false, false);
        s_y[ng >> 2][tt + (ng & 3)][cl] = __uint_as_float(q[0]) + __uint_as_float(q[1]);
      } else {
        *reinterpret_cast<float4*>(&s_y[ng][cl][tt]) = make_float4(y[0], y[1], y[2], y[3]);
      }
    };
    if (CB == 64 || p.prio) __builtin_amdgcn_s_setprio(1);
    constexpr int PDQ = MSCAN_LDS_PD ? MSCAN_LDS_PD : (G == 1 && CB == 16 ? 2 : 1);
    if constexpr (PDQ > 1) {
      // operands read PDQ quads ahead, in a ring of register sets
      constexpr int NQ = TT / 4;
      Ops ring[PDQ + 1];
#pragma unroll
      for (int q = 0; q < PDQ && q < NQ; ++q) read_ops(ring[q], 4 * q);
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        if (4 * q < tend) {
          if (q + PDQ < NQ) read_ops(ring[(q + PDQ) % (PDQ + 1)], 4 * (q + PDQ));
          quad(ring[q % (PDQ + 1)], 4 * q);
          // (inside the tile, the state before every ckpt_every-th position:
          // ckpt_every is 16 or 32)
          if constexpr (TT == 32) {
            if (4 * q + 4 == 16 && p.ckpt_every == 16) checkpoint(p0 + 16);
          } else if (4 * q + 4 < TT && (4 * q + 4) % 16 == 0 && ((4 * q + 4) % 32 == 0 || p.ckpt_every == 16)) {
            checkpoint(p0 + 4 * q + 4);
          }
        }
      }
    } else {
      Ops o0, o1;
      read_ops(o0, 0);
#pragma unroll
      for (int tt = 0; tt < TT; tt += 8) {
        if (tt < tend) {
          read_ops(o1, tt + 4);
          quad(o0, tt);
          if (tt + 4 < tend) {
            read_ops(o0, min(tt + 8, TT - 4));  // the last prefetch re-reads rows that go unused
            quad(o1, tt + 4);
            if constexpr (TT == 32) {
              if (tt + 8 == 16 && p.ckpt_every == 16) checkpoint(p0 + 16);
            } else if (tt + 8 < TT && (tt + 8) % 16 == 0 && ((tt + 8) % 32 == 0 || p.ckpt_every == 16)) {
              checkpoint(p0 + tt + 8);
            }
          }
        }
      }
    }
    __builtin_amdgcn_s_setprio(P_EPI);
    __syncthreads();
    if constexpr (!AGG && PAIR) {
      // epilogue: channels e0, e0 + 1 at positions ppos0 .. ppos0 + PPT - 1
      // (the partials added in group order, as below)
#pragma unroll
      for (int i = 0; i < PPT; ++i) {
        const int tt = ppos0 + i;
        float y0 = Du[2 * i], y1 = Du[2 * i + 1];
#pragma unroll
        for (int g = 0; g < NY; ++g) {
          const float2 v = *reinterpret_cast<const float2*>(&s_y[g][tt][e0]);
          y0 += v.x;
          y1 += v.y;
        }
        const int pp = p0 + tt;
        if (pp < pend && evalid) {
          if (p.ws_y && !fold) store_pair(y0, y1, rs_ws, voff_ws + row_off(pp, 4u), (float*)nullptr);
          if (direct) {
            float o0 = fold ? folded[2 * i] + y0 : y0;
            float o1 = fold ? folded[2 * i + 1] + y1 : y1;
            if (gated) {
              o0 *= gate[2 * i];
              o1 *= gate[2 * i + 1];
            }
            store_pair(o0, o1, rs_out, voff_out + row_off(pp, ES), (TIn*)nullptr);
          }
        }
      }
    } else if constexpr (!AGG) {
      // epilogue: this thread's channel at positions ng*TPT .. ng*TPT+TPT-1
      float yv[TPT];
#pragma unroll
      for (int i = 0; i < TPT; ++i) yv[i] = Du[i];
#pragma unroll
      for (int g = 0; g < NY; ++g) {
#pragma unroll
        for (int i = 0; i < TPT; ++i) yv[i] += s_y[g][cl][ng * TPT + i];
      }
      // (neither row: the recompute of a backward pass that needs only the
      // state checkpoints)
#pragma unroll
      for (int i = 0; i < TPT; ++i) {
        const int pp = p0 + ng * TPT + i;
        if (pp < pend && (dfull || dvalid)) {
          if (p.ws_y && !fold) {
            const uint32_t roff = row_off(pp, 4u);
            buf_store(yv[i], rs_ws, CB == 64 ? voff_ws : voff_ws + roff, CB == 64 ? roff : 0u);
          }
          if (direct) {
            const uint32_t roff = row_off(pp, ES);
            const float yo = fold ? folded[i] + yv[i] : yv[i];
            store_out(gated ? yo * gate[i] : yo, rs_out, CB == 64 ? voff_out : voff_out + roff,
                      CB == 64 ? roff : 0u, (TIn*)nullptr);
          }
        }
      }
    }
  };
  if (pbeg < pend) {
    load_tile(pbeg, r0);
    load_tile(pbeg + TT, r1);
    stage_tile(pbeg, r0);
  }
  for (int p0 = pbeg; p0 < pend; p0 += 2 * TT) {
    load_tile(p0 + 2 * TT, r0);  // two tiles ahead
    process_tile(p0);
    if (p0 + TT < pend) {
      stage_tile(p0 + TT, r1);
      load_tile(p0 + 3 * TT, r1);
      process_tile(p0 + TT);
      if (p0 + 2 * TT < pend) stage_tile(p0 + 2 * TT, r0);
    }
  }

  if (!dvalid) return;
  if constexpr (AGG) {
    float* S = p.agg_state + ((agg_row + c) * D + d) * N + ng * G;
#pragma unroll
    for (int j = 0; j < G; ++j) S[j] = h[j];
    if (ng == 0) p.agg_dsum[(agg_row + c) * D + d] = dsum;
  } else if (c == p.nchunks - 1 && p.last_state) {
    float* S = p.last_state + (((int64_t)b * p.K + k) * D + d) * N + ng * G;
#pragma unroll
    for (int j = 0; j < G; ++j) S[j] = h[j];
  }
}

// out[b][t][d] = (Σ_k ws_y[k][b][t][d]) · silu(z[b][t][d]), directions added in
// ascending k; one thread per V consecutive elements (V = 8 when the channel
// count is a multiple of 8, else 1).
template <typename TIn, int V>
__global__ void __launch_bounds__(256) merge_dirs_kernel(const float* __restrict__ ws_y, const TIn* __restrict__ z,
                                                         TIn* __restrict__ out, int K, int64_t nvec,
                                                         int64_t plane) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nvec) return;
  const int64_t off = i * V;
  float y8[V];
  if constexpr (V == 8) {
    const float4 a = reinterpret_cast<const float4*>(ws_y + off)[0];
    const float4 bq = reinterpret_cast<const float4*>(ws_y + off)[1];
    y8[0] = a.x; y8[1] = a.y; y8[2] = a.z; y8[3] = a.w;
    y8[4] = bq.x; y8[5] = bq.y; y8[6] = bq.z; y8[7] = bq.w;
    for (int k = 1; k < K; ++k) {
      const float4 a2 = reinterpret_cast<const float4*>(ws_y + k * plane + off)[0];
      const float4 b2 = reinterpret_cast<const float4*>(ws_y + k * plane + off)[1];
      y8[0] += a2.x; y8[1] += a2.y; y8[2] += a2.z; y8[3] += a2.w;
      y8[4] += b2.x; y8[5] += b2.y; y8[6] += b2.z; y8[7] += b2.w;
    }
    if (z) {
      Vec<TIn, 8> zz;
      zz.load(z + off);
#pragma unroll
      for (int j = 0; j < 8; ++j) y8[j] *= silu_f(zz.get(j));
    }
    storeV<8>(out + off, y8);
  } else {
    y8[0] = ws_y[off];
    for (int k = 1; k < K; ++k) y8[0] += ws_y[k * plane + off];
    if (z) y8[0] *= silu_f(load1(z + off));
    store1(out + off, y8[0]);
  }
}

// One recurrent step [MFS §2.3]: one thread per (b, d) holding all N states.
struct StepParams {
  float* state;
  const void* u_t;
  const void* delta_t;
  const float* A;
  const void* B_t;
  const void* C_t;
  const float* D;
  const void* z_t;
  const float* delta_bias;
  void* out;
  int Bsz, Dm, softplus;
};

// One token.  TPC = N/G threads per (batch, channel), each with G <= 4
// consecutive states (one 16-byte state load and store); the readout is summed
// over the channel's TPC lanes with xor shuffles and lane 0 of the group adds
// the skip, gates and stores.  Consecutive threads take consecutive state
// groups, so the state traffic is coalesced.
template <typename TIn, int N, bool EXACT>
__global__ void __launch_bounds__(256) scan_step_kernel(const StepParams p) {
  constexpr int G = N < 4 ? N : 4;  // states per thread
  constexpr int TPC = N / G;        // threads per channel (a power of two, at most 16)
  const int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t i = gi / TPC;  // (b, d)
  const int n0 = (int)(gi % TPC) * G;
  // (a channel's TPC lanes are all in range or all out: TPC divides the wave)
  if (i >= (int64_t)p.Bsz * p.Dm) return;
  const int b = (int)(i / p.Dm), d = (int)(i - (int64_t)b * p.Dm);
  const float x = load1(static_cast<const TIn*>(p.delta_t) + i) + (p.delta_bias ? p.delta_bias[d] : 0.f);
  const float dl = p.softplus ? softplus_log2(x) : x * kLog2e;  // Δ' = Δ·log2 e
  const float uu = load1(static_cast<const TIn*>(p.u_t) + i);
  const float du = dl * uu * kLn2;  // Δ·u
  float* st = p.state + i * N + n0;
  const float* Ad = p.A + (int64_t)d * N + n0;
  Small<float, G> hv, Av;
  Small<TIn, G> Bs, Cs;
  hv.load(st);
  Av.load(Ad);
  Bs.load(static_cast<const TIn*>(p.B_t) + (int64_t)b * N + n0);
  Cs.load(static_cast<const TIn*>(p.C_t) + (int64_t)b * N + n0);
  float hs[G];
  float y = 0.f;
#pragma unroll
  for (int e = 0; e < G; ++e) {
    const float An = Av.get(e);
    const float a = ex2(dl * An);  // e^(Δ·A) = 2^(Δ'·A)
    float bu = du * Bs.get(e);
    if constexpr (EXACT) bu = zoh_coef(a, dl * An * kLn2, dl * kLn2, An != 0.f ? 1.0f / An : 0.f) * (uu * Bs.get(e));
    hs[e] = __builtin_fmaf(a, hv.get(e), bu);
    y = __builtin_fmaf(Cs.get(e), hs[e], y);
  }
  if constexpr (G == 4) {
    *reinterpret_cast<float4*>(st) = make_float4(hs[0], hs[G > 1 ? 1 : 0], hs[G > 2 ? 2 : 0], hs[G > 3 ? 3 : 0]);
  } else {
#pragma unroll
    for (int e = 0; e < G; ++e) st[e] = hs[e];
  }
#pragma unroll
  for (int m = 1; m < TPC; m <<= 1) y += __shfl_xor(y, m, TPC);
  if (n0 != 0) return;
  y += (p.D ? p.D[d] : 0.f) * uu;
  if (p.z_t) y *= silu_f(load1(static_cast<const TIn*>(p.z_t) + i));
  store1(static_cast<TIn*>(p.out) + i, y);
}

// One token for any state size (those that are not a power of two): one
// thread per (batch, channel) walking its N states.
template <typename TIn, bool EXACT>
__global__ void __launch_bounds__(256) scan_step_any_kernel(const StepParams p, int N) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // (b, d)
  if (i >= (int64_t)p.Bsz * p.Dm) return;
  const int b = (int)(i / p.Dm), d = (int)(i - (int64_t)b * p.Dm);
  const float x = load1(static_cast<const TIn*>(p.delta_t) + i) + (p.delta_bias ? p.delta_bias[d] : 0.f);
  const float dl = p.softplus ? softplus_log2(x) : x * kLog2e;  // Δ' = Δ·log2 e
  const float uu = load1(static_cast<const TIn*>(p.u_t) + i);
  const float du = dl * uu * kLn2;  // Δ·u
  float* st = p.state + i * N;
  const float* Ad = p.A + (int64_t)d * N;
  const TIn* Bt = static_cast<const TIn*>(p.B_t) + (int64_t)b * N;
  const TIn* Ct = static_cast<const TIn*>(p.C_t) + (int64_t)b * N;
  float y = 0.f;
  for (int n = 0; n < N; ++n) {
    const float An = Ad[n];
    const float a = ex2(dl * An);  // e^(Δ·A) = 2^(Δ'·A)
    const float Bn = load1(Bt + n);
    float bu = du * Bn;
    if constexpr (EXACT) bu = zoh_coef(a, dl * An * kLn2, dl * kLn2, An != 0.f ? 1.0f / An : 0.f) * (uu * Bn);
    const float hn = __builtin_fmaf(a, st[n], bu);
    st[n] = hn;
    y = __builtin_fmaf(load1(Ct + n), hn, y);
  }
  y += (p.D ? p.D[d] : 0.f) * uu;
  if (p.z_t) y *= silu_f(load1(static_cast<const TIn*>(p.z_t) + i));
  store1(static_cast<TIn*>(p.out) + i, y);
}

}  // namespace mscan
