// scan_kernels.h -- gfx950 HIP kernels of the selective (S6) scan.
//
// Sources, cited by page title and section:
//   [MFS] "从零理解 Mamba：选择性状态空间模型（Selective SSM）到 Mamba Block" (eutaboo.com)
//   [S4M] "从S4到Mamba：选择性状态空间模型的演进与革新" (jsqmd.com)
//   [MUN] "【临时文档---算法介绍】Mamba-UNet" (blog.csdn.net)
//   [VIM] "Vision Mamba：从状态空间模型到视觉革命的跨越" (x-humanoid.csdn.net)
//
// Work decomposition of scan_chunk_kernel (one workgroup):
//   * 64 consecutive channels d of one (direction k, batch b), one lane per
//     channel; the N states of a channel are split over NW = N/G waves, each
//     lane holding G states h[n] in registers for the whole scan;
//   * a contiguous range ("chunk") of scan positions; a sequence is split
//     into several chunks only when (k, b, channel-block) rows alone cannot
//     fill the GPU.  Chunks are joined by the associativity of the affine
//     step h -> a·h + b [MFS §5; S4M §2.2, chunked scan with aggregation]:
//     a first pass (AGG = true) scans each chunk from a zero state and
//     records its end state S_c and ΣΔ over the chunk (the chunk's decay is
//     exp(A·ΣΔ) since Ā_t = exp(Δ_t·A)); the output pass folds the aggregates
//     of the chunks before it into its starting state;
//   * the chunk is streamed in tiles of TT scan positions: 128-bit coalesced
//     loads of u, Δraw, z rows (each token's 64-channel row is contiguous in
//     the token-major layout whatever the traversal order), prefetched one
//     tile ahead into registers, then staged in LDS as (Δ, Δ·u) pairs (softplus
//     and the Δ·u product computed once per (token, channel)) and fp32 B, C
//     rows shared by every channel;
//   * per scan step and state: Ā = 2^(Δ·A·log2 e) (one v_exp_f32),
//     h = Ā·h + (Δu)·B, and the partial readout Σ C·h over the lane's G
//     states [MFS §2.2 eq (2a)(2b); §6.2 Step 4 eq (4); MUN §4];
//   * the NW partial readouts meet in LDS; the epilogue adds them in wave
//     order, adds the D·u skip [MUN §4], applies the silu(z) gate [MFS §6.2
//     Step 6] and stores 16-byte rows of the output.  With several
//     directions the ungated fp32 row goes to a workspace slice instead and
//     merge_dirs_kernel sums the directions in order and gates
//     [VIM §2.2; S4M §3].
// No B·D·L·N intermediate is ever written to memory.
#pragma once

#include "device_math.h"

namespace mscan {

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
  void* out;                // [Bsz][L][D] (single direction)
  float* ws_y;              // [K][Bsz][L][D] ungated fp32 rows (several directions) or null
  float* last_state;        // [Bsz][K][D][N] or null
  float* agg_state;         // [K][Bsz][nchunks-1][D][N]
  float* agg_dsum;          // [K][Bsz][nchunks-1][D]
  int Bsz, Dm, L, H, W;
  int K, Ku;
  int kinds;                // 4 x 2-bit traversal kind, direction k at bits 2k..2k+1
  int nchunks;              // chunks per sequence (>= 1)
  int chunk_len;            // scan positions per chunk (multiple of the tile)
  int grid_chunks;          // chunks covered by this launch's grid
  int nblk_d;               // channel blocks of 64
  int softplus;
};

template <typename TIn, int N, int G, int TT, bool AGG>
__global__ void __launch_bounds__(64 * (N / G)) scan_chunk_kernel(const ScanParams p) {
  constexpr int NW = N / G;
  constexpr int NT = 64 * NW;
  constexpr int SPT = (TT * 8) / NT;  // (token, 8-channel group) slots per thread per tile
  static_assert(SPT * NT == TT * 8, "tile must split evenly into 8-channel slots");
  constexpr int EQ = N < 4 ? N : 4;   // B/C elements per load unit
  constexpr int UPR = N / EQ;         // load units per token row
  constexpr int BCU = TT * UPR;       // load units per tile per tensor
  constexpr int BCI = (BCU + NT - 1) / NT;

  __shared__ float2 s_dd[TT][64];  // (Δ, Δ·u) per scan step and channel
  __shared__ float s_B[TT][N];
  __shared__ float s_C[AGG ? 1 : TT][N];
  __shared__ float s_y[AGG ? 1 : NW][AGG ? 1 : TT][64];  // partial readouts per wave

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;

  int bid = blockIdx.x;
  const int dblk = bid % p.nblk_d;
  bid /= p.nblk_d;
  const int c = bid % p.grid_chunks;
  bid /= p.grid_chunks;
  const int b = bid % p.Bsz;
  const int k = bid / p.Bsz;

  const int D = p.Dm, L = p.L;
  const int d0 = dblk * 64;
  const int d = d0 + lane;
  const bool dvalid = d < D;
  const int kind = (p.kinds >> (2 * k)) & 3;
  const int ku = (p.Ku == 1) ? 0 : k;
  const int pbeg = c * p.chunk_len;
  const int pend = min(L, pbeg + p.chunk_len);

  const TIn* __restrict__ u_base = static_cast<const TIn*>(p.u) + (int64_t)(b * p.Ku + ku) * L * D;
  const TIn* __restrict__ dl_base = static_cast<const TIn*>(p.delta) + (int64_t)(b * p.K + k) * L * D;
  const TIn* __restrict__ z_base = p.z ? static_cast<const TIn*>(p.z) + (int64_t)b * L * D : nullptr;
  const TIn* __restrict__ B_base = static_cast<const TIn*>(p.B) + (int64_t)(b * p.K + k) * L * N;
  const TIn* __restrict__ C_base = static_cast<const TIn*>(p.C) + (int64_t)(b * p.K + k) * L * N;
  const bool gated = !AGG && (z_base != nullptr) && (p.ws_y == nullptr);

  // ---- per-lane constants and the starting state ----
  float Al2[G], h[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const int n = wave * G + j;
    Al2[j] = dvalid ? p.A[((int64_t)k * D + d) * N + n] * kLog2e : 0.f;
    h[j] = 0.f;
  }
  const int64_t agg_row = ((int64_t)k * p.Bsz + b) * (p.nchunks - 1);
  if (c == 0) {
    if (p.init_state && dvalid) {
#pragma unroll
      for (int j = 0; j < G; ++j) h[j] = p.init_state[(((int64_t)b * p.K + k) * D + d) * N + wave * G + j];
    }
  } else if (!AGG && dvalid) {
    // fold the aggregates of chunks 0..c-1: h <- exp(A·ΣΔ_j)·h + S_j
    for (int jj = 0; jj < c; ++jj) {
      const float ds = p.agg_dsum[(agg_row + jj) * D + d];
      const float* S = p.agg_state + ((agg_row + jj) * D + d) * N + wave * G;
#pragma unroll
      for (int j = 0; j < G; ++j) h[j] = __builtin_fmaf(ex2(ds * Al2[j]), h[j], S[j]);
    }
  }

  // The state registers may still be waiting on the loads above; settle them
  // here so that no wait on global loads lands inside the scan loop, where it
  // would also wait for the next tile's prefetch.
  __builtin_amdgcn_s_waitcnt(0);

  // ---- per-slot constants: channel group of this thread's slots is fixed ----
  const int c8 = tid & 7;
  const int dg = d0 + c8 * 8;
  const bool gvalid = dg < D;
  float bias8[8], D8[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    bias8[j] = (gvalid && p.delta_bias) ? p.delta_bias[k * D + dg + j] : 0.f;
    D8[j] = (gvalid && p.D) ? p.D[k * D + dg + j] : 0.f;
  }

  Vec8<TIn> rdl[SPT], ru[SPT], rz[SPT];
  Small<TIn, EQ> rB[BCI], rC[BCI];
  float Du[SPT][8], gate[SPT][8];
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    rdl[i].zero();
    ru[i].zero();
    rz[i].zero();
  }
#pragma unroll
  for (int i = 0; i < BCI; ++i) {
    rB[i].zero();
    rC[i].zero();
  }

  auto load_tile = [&](int p0) {
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int tt = (tid + i * NT) >> 3;
      const int pp = p0 + tt;
      if (pp < pend && gvalid) {
        const int64_t off = (int64_t)token_of(kind, pp, L, p.H, p.W) * D + dg;
        rdl[i].load(dl_base + off);
        ru[i].load(u_base + off);
        if (gated) rz[i].load(z_base + off);
      }
    }
#pragma unroll
    for (int i = 0; i < BCI; ++i) {
      const int q = tid + i * NT;
      if (q < BCU) {
        const int tt = q / UPR, nq = q % UPR;
        const int pp = p0 + tt;
        if (pp < pend) {
          const int64_t off = (int64_t)token_of(kind, pp, L, p.H, p.W) * N + nq * EQ;
          rB[i].load(B_base + off);
          if constexpr (!AGG) rC[i].load(C_base + off);
        }
      }
    }
  };

  auto stage_tile = [&](int p0) {
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int tt = (tid + i * NT) >> 3;
      const bool ok = (p0 + tt < pend) && gvalid;
      float2 dd[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // branch-free: compute on whatever the registers hold, then select
        const float x = rdl[i].get(j) + bias8[j];
        const float sp = softplus_f(x);
        const float dl = ok ? (p.softplus ? sp : x) : 0.f;
        const float uu = ok ? ru[i].get(j) : 0.f;
        dd[j] = make_float2(dl, dl * uu);
        if constexpr (!AGG) {
          Du[i][j] = D8[j] * uu;
          if (gated) gate[i][j] = silu_f(rz[i].get(j));
        }
      }
      float4* dst = reinterpret_cast<float4*>(&s_dd[tt][c8 * 8]);
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[j] = make_float4(dd[2 * j].x, dd[2 * j].y, dd[2 * j + 1].x, dd[2 * j + 1].y);
    }
#pragma unroll
    for (int i = 0; i < BCI; ++i) {
      const int q = tid + i * NT;
      if (q < BCU) {
        const int tt = q / UPR, nq = q % UPR;
        const bool ok = p0 + tt < pend;
#pragma unroll
        for (int e = 0; e < EQ; ++e) {
          s_B[tt][nq * EQ + e] = ok ? rB[i].get(e) : 0.f;
          if constexpr (!AGG) s_C[tt][nq * EQ + e] = ok ? rC[i].get(e) : 0.f;
        }
      }
    }
  };

  float dsum = 0.f;
  if (pbeg < pend) {
    load_tile(pbeg);
    stage_tile(pbeg);
  }
  for (int p0 = pbeg; p0 < pend; p0 += TT) {
    const bool has_next = p0 + TT < pend;
    if (has_next) load_tile(p0 + TT);  // in flight during this tile's scan
    __syncthreads();
    const int tlen = min(TT, pend - p0);
    for (int tt = 0; tt < tlen; ++tt) {
      const float2 dd = s_dd[tt][lane];
      float y = 0.f;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const int n = wave * G + j;
        const float a = ex2(dd.x * Al2[j]);
        h[j] = __builtin_fmaf(a, h[j], dd.y * s_B[tt][n]);
        if constexpr (!AGG) y = __builtin_fmaf(s_C[tt][n], h[j], y);
      }
      if constexpr (!AGG) s_y[wave][tt][lane] = y;
      if constexpr (AGG) dsum += dd.x;
    }
    __syncthreads();
    if constexpr (!AGG) {
#pragma unroll
      for (int i = 0; i < SPT; ++i) {
        const int tt = (tid + i * NT) >> 3;
        const int pp = p0 + tt;
        if (pp < pend && gvalid) {
          float y8[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) y8[j] = Du[i][j];
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            const float4 a = reinterpret_cast<const float4*>(&s_y[w][tt][c8 * 8])[0];
            const float4 bq = reinterpret_cast<const float4*>(&s_y[w][tt][c8 * 8])[1];
            y8[0] += a.x; y8[1] += a.y; y8[2] += a.z; y8[3] += a.w;
            y8[4] += bq.x; y8[5] += bq.y; y8[6] += bq.z; y8[7] += bq.w;
          }
          const int64_t off = (int64_t)token_of(kind, pp, L, p.H, p.W) * D + dg;
          if (p.ws_y) {
            store8(p.ws_y + ((int64_t)k * p.Bsz + b) * L * D + off, y8);
          } else {
            if (gated) {
#pragma unroll
              for (int j = 0; j < 8; ++j) y8[j] *= gate[i][j];
            }
            store8(static_cast<TIn*>(p.out) + (int64_t)b * L * D + off, y8);
          }
        }
      }
    }
    if (has_next) stage_tile(p0 + TT);
  }

  if (!dvalid) return;
  if constexpr (AGG) {
    float* S = p.agg_state + ((agg_row + c) * D + d) * N + wave * G;
#pragma unroll
    for (int j = 0; j < G; ++j) S[j] = h[j];
    if (wave == 0) p.agg_dsum[(agg_row + c) * D + d] = dsum;
  } else if (c == p.nchunks - 1 && p.last_state) {
    float* S = p.last_state + (((int64_t)b * p.K + k) * D + d) * N + wave * G;
#pragma unroll
    for (int j = 0; j < G; ++j) S[j] = h[j];
  }
}

// out[b][t][d] = (Σ_k ws_y[k][b][t][d]) · silu(z[b][t][d]), directions added in
// ascending k; one thread per 8 consecutive channels.
template <typename TIn>
__global__ void __launch_bounds__(256) merge_dirs_kernel(const float* __restrict__ ws_y, const TIn* __restrict__ z,
                                                         TIn* __restrict__ out, int K, int64_t nrows8,
                                                         int64_t plane) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nrows8) return;
  const int64_t off = i * 8;
  float y8[8];
  {
    const float4 a = reinterpret_cast<const float4*>(ws_y + off)[0];
    const float4 bq = reinterpret_cast<const float4*>(ws_y + off)[1];
    y8[0] = a.x; y8[1] = a.y; y8[2] = a.z; y8[3] = a.w;
    y8[4] = bq.x; y8[5] = bq.y; y8[6] = bq.z; y8[7] = bq.w;
  }
  for (int k = 1; k < K; ++k) {
    const float4 a = reinterpret_cast<const float4*>(ws_y + k * plane + off)[0];
    const float4 bq = reinterpret_cast<const float4*>(ws_y + k * plane + off)[1];
    y8[0] += a.x; y8[1] += a.y; y8[2] += a.z; y8[3] += a.w;
    y8[4] += bq.x; y8[5] += bq.y; y8[6] += bq.z; y8[7] += bq.w;
  }
  if (z) {
    Vec8<TIn> zz;
    zz.load(z + off);
#pragma unroll
    for (int j = 0; j < 8; ++j) y8[j] *= silu_f(zz.get(j));
  }
  store8(out + off, y8);
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

template <typename TIn, int N>
__global__ void __launch_bounds__(256) scan_step_kernel(const StepParams p) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= p.Bsz * p.Dm) return;
  const int b = i / p.Dm, d = i - b * p.Dm;
  const TIn* Bt = static_cast<const TIn*>(p.B_t) + (int64_t)b * N;
  const TIn* Ct = static_cast<const TIn*>(p.C_t) + (int64_t)b * N;
  const float x = load1(static_cast<const TIn*>(p.delta_t) + i) + (p.delta_bias ? p.delta_bias[d] : 0.f);
  const float dl = p.softplus ? softplus_f(x) : x;
  const float uu = load1(static_cast<const TIn*>(p.u_t) + i);
  const float du = dl * uu;
  float* st = p.state + (int64_t)i * N;
  const float* Ad = p.A + (int64_t)d * N;
  float y = 0.f;
#pragma unroll
  for (int n0 = 0; n0 < N; n0 += 4) {
    constexpr int E = N < 4 ? N : 4;
    float hs[E];
    Small<float, E> hv;
    Small<TIn, E> Bs, Cs;
    hv.load(st + n0);
    Bs.load(Bt + n0);
    Cs.load(Ct + n0);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float a = ex2(dl * (Ad[n0 + e] * kLog2e));
      hs[e] = __builtin_fmaf(a, hv.get(e), du * Bs.get(e));
      y = __builtin_fmaf(Cs.get(e), hs[e], y);
    }
    if (E == 4) {
      *reinterpret_cast<float4*>(st + n0) = make_float4(hs[0], hs[E > 1 ? 1 : 0], hs[E > 2 ? 2 : 0], hs[E > 3 ? 3 : 0]);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) st[n0 + e] = hs[e];
    }
  }
  y += (p.D ? p.D[d] : 0.f) * uu;
  if (p.z_t) y *= silu_f(load1(static_cast<const TIn*>(p.z_t) + i));
  store1(static_cast<TIn*>(p.out) + i, y);
}

}  // namespace mscan
