// scan_bwd.h -- gfx950 HIP kernels of the backward (gradient) pass of the
// selective scan.
//
// Sources, cited by page title and section:
//   [MFS] "从零理解 Mamba：选择性状态空间模型（Selective SSM）到 Mamba Block" (eutaboo.com)
//   [S4M] "从S4到Mamba：选择性状态空间模型的演进与革新" (jsqmd.com)
//
// The training pass recomputes the states instead of storing them [MFS §5;
// S4M §2.3].  For a loss with gradient dout on the output, per direction k,
// batch b, channel d and state n (scan position p visiting token t):
//   dy = dout·silu(z);  dz = dout·y_all·silu'(z)              (bwd_prep_kernel)
//   λ_p = C_t·dy_t + Ā_{p+1}·λ_{p+1}                           (adjoint of h_p)
//   dΔ_p = Σ_n [λ h_{p-1} A Ā + λ (∂B̄/∂Δ)·u],  du_t = Σ_n λ B̄_n + D·dy_t
//   dA += λ h_{p-1} Δ Ā (+ λ (∂c/∂A) B u for the exact rule)
//   dB_t = Σ_d λ·(Δ or c)·u,  dC_t = Σ_d dy_t·h_p,  dD = Σ dy·u
//   ddelta = dΔ·σ(x) (softplus) = dΔ·(1 - e^{-Δ}),  ddelta_bias = Σ ddelta
//   dinit = Ā_0·λ_0
// The forward pass with state checkpoints every 32 positions runs first
// (scan_chunk_kernel with ScanParams::ckpt); scan_bwd_kernel then walks each
// (direction, batch, 16-channel block) backwards one 32-position segment at a
// time: it recomputes the segment's states from its checkpoint into
// registers, then runs the adjoint recurrence over the two 16-position
// halves.  Sums over states go through LDS (like the forward readout); sums
// over the block's 16 channels (dB, dC) through a register butterfly across
// each 16-lane row; sums over blocks and batches in bwd_sum_kernel.
#pragma once

#include "scan_kernels.h"

namespace mscan {

// ---- row butterfly (16 lanes of a row hold the 16 channels of one state) ----
__device__ __forceinline__ float bwd_quad_perm_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4e, 0xf, 0xf, false));
}
__device__ __forceinline__ float bwd_quad_perm_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xb1, 0xf, 0xf, false));
}
// Lanes 0-7 of each row return x + x[j+8], lanes 8-15 return y + y[j-8]; the
// two adds write disjoint lane banks of one register.  The leading s_nop
// covers the wait states a DPP read needs after a vector write of its source.
__device__ __forceinline__ float bwd_bfly8(float x, float y) {
  float r;
  asm("s_nop 1\n\t"
      "v_add_f32_dpp %0, %1, %1 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %0, %2, %2 row_ror:8 row_mask:0xf bank_mask:0xc"
      : "=&v"(r)
      : "v"(x), "v"(y));
  return r;
}
// Lanes with bit 2 of j clear return x + x[j+4], the others y + y[j-4].
__device__ __forceinline__ float bwd_bfly4(float x, float y) {
  float r;
  asm("s_nop 1\n\t"
      "v_add_f32_dpp %0, %1, %1 row_ror:12 row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %0, %2, %2 row_ror:4 row_mask:0xf bank_mask:0xa"
      : "=&v"(r)
      : "v"(x), "v"(y));
  return r;
}
// v[s] (s = 0..15) per lane; returns, in lane j of each 16-lane row, the sum
// over the row's lanes of v[j].
__device__ __forceinline__ float row_sum_transpose16(const float (&v)[16], int j) {
  float r8[8], r4[4], r2[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) r8[i] = bwd_bfly8(v[i], v[i + 8]);    // step i + 8*bit3(j)
#pragma unroll
  for (int i = 0; i < 4; ++i) r4[i] = bwd_bfly4(r8[i], r8[i + 4]);  // + 4*bit2(j)
  const bool b1 = (j & 2) != 0, b0 = (j & 1) != 0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float send = b1 ? r4[i] : r4[i + 2];
    const float keep = b1 ? r4[i + 2] : r4[i];
    r2[i] = keep + bwd_quad_perm_xor2(send);
  }
  const float send = b0 ? r2[0] : r2[1];
  const float keep = b0 ? r2[1] : r2[0];
  return keep + bwd_quad_perm_xor1(send);  // step j
}

struct BwdParams {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;           // may be null
  const float* delta_bias;  // may be null
  const float* ckpt;        // [K][Bsz][ntiles][Dm][N] states at every 32-position tile start
  const float* dy;          // [Bsz][L][Dm] float32
  void* du;                 // [Bsz][Ku][L][Dm] (Ku = K), or null when du_part is used
  float* du_part;           // [K][Bsz][L][Dm] (the cross scan shares u), or null
  void* ddelta;             // [Bsz][K][L][Dm]
  float* dB_part;           // [nblk_d][Bsz][K][L][N]
  float* dC_part;           // [nblk_d][Bsz][K][L][N]
  float* dA_part;           // [Bsz][K][Dm][N]
  float* dD_part;           // [Bsz][K][Dm]
  float* dbias_part;        // [Bsz][K][Dm]
  float* dinit;             // [Bsz][K][Dm][N] or null
  int Bsz, Dm, L, H, W, K, Ku, kinds, nblk_d, ntiles, softplus;
};

// dy = dout·silu(z), dz = dout·y_all·silu'(z) with y_all = Σ_k y_k (ungated);
// without a gate dy = dout.  One thread per element.
template <typename TIn>
__global__ void __launch_bounds__(256) bwd_prep_kernel(const float* __restrict__ ws_y, const TIn* __restrict__ z,
                                                       const TIn* __restrict__ dout, float* __restrict__ dy,
                                                       TIn* __restrict__ dz, int K, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float go = to_f32(load1(dout + i));
  if (z == nullptr) {
    dy[i] = go;
    return;
  }
  float y = 0.f;
  if (dz)
    for (int k = 0; k < K; ++k) y += ws_y[k * n + i];
  const float zz = to_f32(load1(z + i));
  const float sg = rcp(1.0f + ex2(-zz * kLog2e));
  dy[i] = go * zz * sg;
  if (dz) store1(dz + i, go * y * sg * __builtin_fmaf(zz, 1.0f - sg, 1.0f));
}

// out[i] = Σ_s in[s·stride + i], s = 0 .. nslices-1 in order.
template <typename TOut>
__global__ void __launch_bounds__(256) bwd_sum_kernel(const float* __restrict__ in, int64_t nslices, int64_t stride,
                                                      int64_t n, TOut* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float acc = 0.f;
  for (int64_t s = 0; s < nslices; ++s) acc += in[s * stride + i];
  store1(out + i, acc);
}

// One workgroup: 16 channels of one (direction, batch) for the whole
// sequence, walked backwards.  Thread tid: channel cl = tid % 16, state
// n = tid / 16 (rows n >= N only pad small N to a whole wave).
template <typename TIn, int N, bool EXACT>
__global__ void __launch_bounds__(16 * (N < 4 ? 4 : N)) scan_bwd_kernel(const BwdParams p) {
  constexpr int CB = 16;
  constexpr int NGP = N < 4 ? 4 : N;  // thread rows
  constexpr int NT = CB * NGP;
  constexpr int TS = 32;              // segment (the forward checkpoint interval)
  constexpr int TH = 16;              // half segment (one butterfly)
  constexpr int TPS = TS / NGP;       // positions staged per thread per segment
  constexpr int TPH = TH / NGP > 0 ? TH / NGP : 1;  // positions summed per thread per half
  constexpr int PS = TS + 4;          // padded row of a per-channel or per-state array
  constexpr int YS = TH + 4;          // padded partial row
  static_assert(TS % NGP == 0 && TH % 4 == 0, "segment splits over the thread rows");
  static_assert(N <= 16, "one state per thread");

  __shared__ __attribute__((aligned(16))) float s_dl[CB * PS];   // Δ' = Δ·log2 e
  __shared__ __attribute__((aligned(16))) float s_u[CB * PS];    // u
  __shared__ __attribute__((aligned(16))) float s_dy[CB * PS];   // dy
  __shared__ __attribute__((aligned(16))) float s_B[N * PS];
  __shared__ __attribute__((aligned(16))) float s_C[N * PS];
  __shared__ __attribute__((aligned(16))) float s_pd[N][CB][YS];  // per-state parts of dΔ
  __shared__ __attribute__((aligned(16))) float s_pu[N][CB][YS];  // per-state parts of du
  __shared__ float s_red[2][NGP][CB];

  const int tid = threadIdx.x;
  const int cl = tid % CB;
  const int ng = tid / CB;
  const bool nvalid = ng < N;
  const int n = nvalid ? ng : 0;

  const int nblocks = gridDim.x;
  int bid = logical_block(blockIdx.x, nblocks, 4);
  const int dblk = bid % p.nblk_d;
  bid /= p.nblk_d;
  const int b = bid % p.Bsz;
  const int k = bid / p.Bsz;

  const int D = p.Dm, L = p.L;
  const int d0 = dblk * CB;
  const int d = d0 + cl;
  const bool dvalid = d < D;
  const int dc = dvalid ? d : D - 1;
  const int kind = (p.kinds >> (2 * k)) & 3;
  const int ku = (p.Ku == 1) ? 0 : k;
  const bool rowwise = kind < KIND_COL_FWD;
  const bool rev = kind == KIND_ROW_REV;
  auto token = [&](int pp) __attribute__((always_inline)) {
    return rowwise ? (rev ? L - 1 - pp : pp) : token_of(kind, pp, L, p.H, p.W);
  };

  const TIn* u_s = static_cast<const TIn*>(p.u) + (int64_t)(b * p.Ku + ku) * L * D;
  const TIn* dl_s = static_cast<const TIn*>(p.delta) + (int64_t)(b * p.K + k) * L * D;
  const TIn* B_s = static_cast<const TIn*>(p.B) + (int64_t)(b * p.K + k) * L * N;
  const TIn* C_s = static_cast<const TIn*>(p.C) + (int64_t)(b * p.K + k) * L * N;
  const float* dy_s = p.dy + (int64_t)b * L * D;

  const float Anat = (nvalid && dvalid) ? p.A[((int64_t)k * D + d) * N + n] : 0.f;
  const float invA = Anat != 0.f ? 1.0f / Anat : 0.f;
  const float bias = (dvalid && p.delta_bias) ? p.delta_bias[k * D + d] : 0.f;
  const float Dd = (dvalid && p.D) ? p.D[k * D + d] : 0.f;

  float carry = 0.f;  // Ā_{p+1}·λ_{p+1}
  float dA_acc = 0.f, dD_acc = 0.f, dbias_acc = 0.f;

  // (Every read of the staging arrays comes before the last barrier of the
  // previous segment, so staging needs no barrier of its own.)
  for (int seg = p.ntiles - 1; seg >= 0; --seg) {
    const int p0 = seg * TS;
    // ---- stage the segment: per (position, channel) and per (position, state) ----
#pragma unroll
    for (int i = 0; i < TPS; ++i) {
      const int tt = ng * TPS + i;
      const int pp = p0 + tt;
      const float okf = (pp < L && dvalid) ? 1.f : 0.f;
      const int64_t off = (int64_t)token(min(pp, L - 1)) * D + dc;
      const float x = to_f32(load1(dl_s + off)) + bias;
      s_dl[cl * PS + tt] = (p.softplus ? softplus_log2(x) : x * kLog2e) * okf;
      s_u[cl * PS + tt] = to_f32(load1(u_s + off)) * okf;
      s_dy[cl * PS + tt] = dy_s[off] * okf;
    }
    for (int q = tid; q < N * TS; q += NT) {
      const int nn = q % N, tt = q / N;
      const int pp = p0 + tt;
      const float okf = pp < L ? 1.f : 0.f;
      const int64_t off = (int64_t)token(min(pp, L - 1)) * N + nn;
      s_B[nn * PS + tt] = to_f32(load1(B_s + off)) * okf;
      s_C[nn * PS + tt] = to_f32(load1(C_s + off)) * okf;
    }
    __syncthreads();

    // ---- recompute the segment's states from its checkpoint ----
    const float h0 = (nvalid && dvalid) ? p.ckpt[((((int64_t)k * p.Bsz + b) * p.ntiles + seg) * D + d) * N + n] : 0.f;
    float hs[TS], as[TS];
    {
      float h = h0;
#pragma unroll
      for (int s = 0; s < TS; ++s) {
        const float dl = s_dl[cl * PS + s];
        const float uu = s_u[cl * PS + s];
        const float Bv = s_B[n * PS + s];
        const float a = ex2(dl * Anat);
        const float dt = dl * kLn2;
        const float c = EXACT ? zoh_coef(a, dt * Anat, dt, invA) : dt;
        h = __builtin_fmaf(a, h, c * Bv * uu);
        hs[s] = h;
        as[s] = a;
      }
    }

    // The adjoint reads the staged values again from LDS: kept live from the
    // recompute they would take five registers per position.
    asm volatile("" ::: "memory");

    // ---- the adjoint over the two halves, later half first ----
#pragma unroll
    for (int half = 1; half >= 0; --half) {
      float pB[TH], pC[TH];
#pragma unroll
      for (int s4 = TH - 4; s4 >= 0; s4 -= 4) {
        float pd4[4], pu4[4];
#pragma unroll
        for (int r = 3; r >= 0; --r) {
          const int s = half * TH + s4 + r;
          const float dl = s_dl[cl * PS + s];
          const float uu = s_u[cl * PS + s];
          const float dyv = s_dy[cl * PS + s];
          const float Bv = s_B[n * PS + s];
          const float Cv = s_C[n * PS + s];
          const float a = as[s];
          const float hp = s > 0 ? hs[s - 1] : h0;
          const float dt = dl * kLn2;
          const float l = __builtin_fmaf(Cv, dyv, carry);
          const float ga = l * hp;
          float c = dt, dcdt = 1.f;
          if constexpr (EXACT) {
            c = zoh_coef(a, dt * Anat, dt, invA);
            dcdt = a;  // dc/dΔ = e^{ΔA}
            dA_acc = __builtin_fmaf(l * zoh_coef_dA(a, dt * Anat, dt, c, invA), Bv * uu, dA_acc);
          }
          pd4[r] = __builtin_fmaf(ga * Anat, a, l * dcdt * Bv * uu);
          pu4[r] = l * c * Bv;
          dA_acc = __builtin_fmaf(ga * dt, a, dA_acc);
          pB[s4 + r] = l * c * uu;
          pC[s4 + r] = dyv * hs[s];
          carry = a * l;
        }
        if (nvalid) {
          *reinterpret_cast<float4*>(&s_pd[n][cl][s4]) = make_float4(pd4[0], pd4[1], pd4[2], pd4[3]);
          *reinterpret_cast<float4*>(&s_pu[n][cl][s4]) = make_float4(pu4[0], pu4[1], pu4[2], pu4[3]);
        }
      }
      // dB, dC: sums over the row's 16 channels; lane cl ends with step cl
      const float sB = row_sum_transpose16(pB, cl);
      const float sC = row_sum_transpose16(pC, cl);
      {
        const int pp = p0 + half * TH + cl;
        if (nvalid && pp < L) {
          const int64_t off = ((((int64_t)dblk * p.Bsz + b) * p.K + k) * L + token(pp)) * N + n;
          p.dB_part[off] = sB;
          p.dC_part[off] = sC;
        }
      }
      __syncthreads();
      // ---- sums over states, per (position, channel) ----
#pragma unroll
      for (int i = 0; i < TPH; ++i) {
        const int sh = ng * TPH + i;  // position within the half
        if (sh < TH) {
          const int s = half * TH + sh;
          const int pp = p0 + s;
          float dd = 0.f, duu = 0.f;
#pragma unroll
          for (int g = 0; g < N; ++g) {
            dd += s_pd[g][cl][sh];
            duu += s_pu[g][cl][sh];
          }
          const float dl = s_dl[cl * PS + s];
          const float uu = s_u[cl * PS + s];
          const float dyv = s_dy[cl * PS + s];
          // σ(x) = 1 - e^{-Δ} for Δ = softplus(x)
          const float dx = p.softplus ? dd * (1.0f - ex2(-dl)) : dd;
          duu = __builtin_fmaf(Dd, dyv, duu);
          dD_acc = __builtin_fmaf(dyv, uu, dD_acc);
          dbias_acc += dx;
          if (pp < L && dvalid) {
            const int t = token(pp);
            store1(static_cast<TIn*>(p.ddelta) + ((int64_t)(b * p.K + k) * L + t) * D + d, dx);
            if (p.du_part) p.du_part[(((int64_t)k * p.Bsz + b) * L + t) * D + d] = duu;
            else store1(static_cast<TIn*>(p.du) + ((int64_t)(b * p.Ku + ku) * L + t) * D + d, duu);
          }
        }
      }
      __syncthreads();  // the partial rows are rewritten by the next half
    }
  }

  // ---- per-(b, k, d) and per-(b, k, d, n) results ----
  s_red[0][ng][cl] = dD_acc;
  s_red[1][ng][cl] = dbias_acc;
  __syncthreads();
  if (dvalid) {
    if (nvalid) {
      const int64_t o = (((int64_t)b * p.K + k) * D + d) * N + n;
      p.dA_part[o] = dA_acc;
      if (p.dinit) p.dinit[o] = carry;
    }
    if (ng == 0) {
      float sD = 0.f, sb = 0.f;
#pragma unroll
      for (int g = 0; g < NGP; ++g) {
        sD += s_red[0][g][cl];
        sb += s_red[1][g][cl];
      }
      p.dD_part[((int64_t)b * p.K + k) * D + d] = sD;
      p.dbias_part[((int64_t)b * p.K + k) * D + d] = sb;
    }
  }
}

}  // namespace mscan
