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
//   dy = dout·silu(z);  dz = dout·y_all·silu'(z)     (staging; bwd_dz_kernel for K > 1)
//   λ_p = C_t·dy_t + Ā_{p+1}·λ_{p+1}                           (adjoint of h_p)
//   dΔ_p = Σ_n [λ h_{p-1} A Ā + λ (∂B̄/∂Δ)·u],  du_t = Σ_n λ B̄_n + D·dy_t
//   dA += λ h_{p-1} Δ Ā (+ λ (∂c/∂A) B u for the exact rule)
//   dB_t = Σ_d λ·(Δ or c)·u,  dC_t = Σ_d dy_t·h_p,  dD = Σ dy·u
//   ddelta = dΔ·σ(x) (softplus) = dΔ·(1 - e^{-Δ}),  ddelta_bias = Σ ddelta
//   dinit = Ā_0·λ_0
// With the simplified rule (B̄ = Δ·B) the channel's u and Δ factor out of the
// state sums: dΔ_p = Σ_n λ h_{p-1} A Ā + u·Σ_n λ B_n and du = Δ·Σ_n λ B_n + D·dy,
// so the per-state terms are λ h_{p-1} Ā A_n and λ B_n (and Δ·u is staged once).
// The forward pass with state checkpoints every 16 positions (32 at 17..32
// states) runs first
// (scan_chunk_kernel with ScanParams::ckpt); scan_bwd_kernel then walks each
// (direction, batch, 16-channel block) backwards one segment (16 positions,
// 32 for N = 17..32) at a time: it recomputes the segment's states from its
// checkpoint into registers, then runs the adjoint recurrence over its
// 16-position halves.  Sums over states go through LDS (like the forward readout); sums
// over the block's 16 channels (dB, dC) through a register butterfly across
// each 16-lane row; sums over blocks and batches in bwd_sum_kernel.  Above 32
// states the states are split into groups of 16, one workgroup each; their
// shares of the per-channel sums (du, ddelta, ddelta_bias) are added in
// bwd_sum_kernel.
#pragma once

#include "scan_kernels.h"

namespace mscan {

#ifndef MSCAN_BWD_WAVES
#define MSCAN_BWD_WAVES 2  // waves per SIMD the adjoint kernel's register budget is sized for (3 spills)
#endif
#ifndef MSCAN_BWD_WAVES16
// The same for 16 thread rows (N = 9..16 and the state groups above 32): 128
// VGPRs with 1 to 3 spilled, 4 waves per SIMD.  Measured on MI355X against the
// 2-wave budget (129 VGPRs, 3 waves), both builds in one process: Vim-224's
// backward 878 -> 818 us; the 130M layer, whose rows fill 3 waves per SIMD,
// and the cross scan unchanged (545 / 548, 2225 / 2226).
#define MSCAN_BWD_WAVES16 4
#endif
#ifndef MSCAN_BWD_WAVES_EXACT
#define MSCAN_BWD_WAVES_EXACT 1  // the same for the exact rule (with 16-position segments it fits 198 VGPRs anyway)
#endif
#ifndef MSCAN_BWD_SEG
#define MSCAN_BWD_SEG 16  // segment length (the forward's checkpoint interval) up to 16 states
#endif
#ifndef MSCAN_BWD_KEEP_ABAR
#define MSCAN_BWD_KEEP_ABAR 1  // 1: keep the segment's e^{ΔA} from the recompute (32 registers) instead of recomputing
#endif

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
struct BwdParams {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;           // may be null
  const float* delta_bias;  // may be null
  const float* ckpt;        // [K][Bsz][ntiles][Dm][N] states before every segment (TS positions)
  const void* dout;         // [Bsz][L][Dm]
  const void* z;            // [Bsz][L][Dm] or null (no gate)
  const float* ws_y;        // [K][Bsz][L][Dm] ungated output rows of the forward recompute, or null
                            // (no gate or no dz: not needed)
  void* dz;                 // [Bsz][L][Dm]: written while staging when dz_here
  int dz_here;              // one direction and a gate: dz from this direction's row
  void* du;                 // [Bsz][Ku][L][Dm] (Ku = K), or null when du_part is used
  float* du_part;           // [ngroups][K][Bsz][L][Dm] (the cross scan shares u) or
                            // [ngroups][Bsz][K][L][Dm] (groups, u per direction), or null
  void* ddelta;             // [Bsz][K][L][Dm]
  float* dB_part;           // [nblk_d][Bsz][K][L][N]
  float* dC_part;           // [nblk_d][Bsz][K][L][N]
  float* dA_part;           // [nchunks][Bsz][K][Dm][N]
  float* dD_part;           // [ngroups][nchunks][Bsz][K][Dm] (zero past group 0)
  float* dbias_part;        // [ngroups][nchunks][Bsz][K][Dm]
  float* dinit;             // [Bsz][K][Dm][N] or null
  // State groups (N above 32): the grid holds ngroups workgroups per (channel
  // block, chunk, batch, direction), group g taking states 16g .. 16g+15 (the
  // last may hold fewer); the sums over states of a channel's gradients are
  // then partial per group: ddelta and du go as fp32 parts to ddelta_part and
  // du_part, dbias as parts per group, and D·dy, dD and dz come from group 0.
  float* ddelta_part;       // [ngroups][Bsz][K][L][Dm] with ngroups > 1, else null
  // time split: the adjoint of chunk c starts from the carry of chunks c+1..
  float* agg_S;             // [K][Bsz][nchunks-1][Dm][N]: carry out of chunk j >= 1 from a zero carry in
  float* agg_dsum;          // [K][Bsz][nchunks-1][Dm]: ΣΔ over chunk j
  int nchunks, chunk_len;   // chunks per sequence (chunk_len a multiple of 32)
  int chunk0, grid_chunks;  // chunks chunk0 .. chunk0+grid_chunks-1 are this launch's
  int Bsz, Dm, L, H, W, K, Ku, kinds, nblk_d, ntiles, softplus;
  int N;                    // state size (the kernel may run a larger power-of-two instantiation,
                            // or groups of NP states)
  int ngroups;              // state groups (1: all N states in one workgroup)
};

// dz = dout·y_all·silu'(z), y_all = Σ_k y_k (ungated), silu'(z) = σ(z)·(1 + z·(1 - σ(z))),
// for several directions (with one, scan_bwd_kernel writes dz while staging).
// Eight consecutive elements per thread (n is a multiple of 8: the channel
// count is).
template <typename TIn>
__global__ void __launch_bounds__(256) bwd_dz_kernel(const float* __restrict__ ws_y, const TIn* __restrict__ z,
                                                     const TIn* __restrict__ dout, TIn* __restrict__ dz, int K,
                                                     int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i >= n) return;
  Vec<TIn, 8> go, zv;
  go.load(dout + i);
  zv.load(z + i);
  float y8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < K; ++k) {
    Vec<float, 8> yk;
    yk.load(ws_y + k * n + i);
#pragma unroll
    for (int c = 0; c < 8; ++c) y8[c] += yk.get(c);
  }
  float g8[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float zz = zv.get(c);
    const float sg = rcp(1.0f + ex2(-zz * kLog2e));
    g8[c] = go.get(c) * y8[c] * sg * __builtin_fmaf(zz, 1.0f - sg, 1.0f);
  }
  storeV<8>(dz + i, g8);
}

// out[i] = Σ_s in[s·stride + i], s = 0 .. nslices-1 in order; V consecutive
// elements per thread (V = 4 needs n and stride multiples of 4).  blockIdx.y
// selects one of two independent (in, out) pairs, so that two sums share a
// launch.
template <typename TOut, int V>
__global__ void __launch_bounds__(256) bwd_sum_kernel(const float* __restrict__ in0, TOut* __restrict__ out0,
                                                      const float* __restrict__ in1, TOut* __restrict__ out1,
                                                      int64_t nslices, int64_t stride, int64_t n) {
  const float* __restrict__ in = blockIdx.y == 0 ? in0 : in1;
  TOut* __restrict__ out = blockIdx.y == 0 ? out0 : out1;
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * V;
  if (i >= n) return;
  if constexpr (V == 4) {
    // 16 slices' loads in flight per thread (the sum stays in slice order)
    constexpr int U = 16;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    int64_t s = 0;
    for (; s + U <= nslices; s += U) {
      float4 v[U];
#pragma unroll
      for (int j = 0; j < U; ++j) v[j] = *reinterpret_cast<const float4*>(in + (s + j) * stride + i);
#pragma unroll
      for (int j = 0; j < U; ++j) {
        acc[0] += v[j].x;
        acc[1] += v[j].y;
        acc[2] += v[j].z;
        acc[3] += v[j].w;
      }
    }
    for (; s < nslices; ++s) {
      const float4 v = *reinterpret_cast<const float4*>(in + s * stride + i);
      acc[0] += v.x;
      acc[1] += v.y;
      acc[2] += v.z;
      acc[3] += v.w;
    }
    storeV<4>(out + i, acc);
  } else {
    float acc = 0.f;
    for (int64_t s = 0; s < nslices; ++s) acc += in[s * stride + i];
    store1(out + i, acc);
  }
}

// v[r] (r = 0..3) per lane, scaled by f; returns in row r of the wave (lanes
// 16r..16r+15) the sum over the wave's 4 rows of v[r] at the same column.
// Swapping lanes 32-63 of one register with lanes 0-31 of another and adding
// sums the two 32-lane halves (steps 0/1 land in the low half, 2/3 in the
// high half); the same with odd/even 16-lane rows sums the rows within a half.
__device__ __forceinline__ float sum_rows4(const float (&v)[4], float f) {
  const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0] * f), __float_as_uint(v[2] * f), false, false);
  const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[1] * f), __float_as_uint(v[3] * f), false, false);
  const float z02 = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);
  const float z13 = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(z02), __float_as_uint(z13), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Lane-mask select: m all ones gives x, all zeros gives y (one v_bfi_b32).
__device__ __forceinline__ float bsel(uint32_t m, float x, float y) {
  return __uint_as_float((__float_as_uint(x) & m) | (__float_as_uint(y) & ~m));
}

// v[s] (s = 0..15) per lane; returns, in lane j of each 16-lane row, the sum
// over the row's lanes of v[j].  m1, m0: all-ones masks of bit 1 and bit 0 of j.
__device__ __forceinline__ float row_sum_transpose16(const float (&v)[16], uint32_t m1, uint32_t m0) {
  float r8[8], r4[4], r2[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) r8[i] = bwd_bfly8(v[i], v[i + 8]);    // step i + 8*bit3(j)
#pragma unroll
  for (int i = 0; i < 4; ++i) r4[i] = bwd_bfly4(r8[i], r8[i + 4]);  // + 4*bit2(j)
#pragma unroll
  for (int i = 0; i < 2; ++i)  // + 2*bit1(j): keep that half, send the other to lane j^2
    r2[i] = bsel(m1, r4[i + 2], r4[i]) + bwd_quad_perm_xor2(bsel(m1, r4[i], r4[i + 2]));
  return bsel(m0, r2[1], r2[0]) + bwd_quad_perm_xor1(bsel(m0, r2[0], r2[1]));  // step j
}

// One workgroup: 16 channels of one (direction, batch) over one time chunk
// (the whole sequence unless it is split), walked backwards.  Thread tid: channel cl = tid % 16, state
// n = tid / 16 (rows n >= N only pad small N to a whole wave).  The global
// loads of the next (earlier) segment are issued before the current one is
// computed, and the staged rows hold Δ in natural units (the exp takes
// A·log2 e).
//
// AGG: the aggregate pass of a time split.  It runs only the adjoint carry
// (λ = C·dy + carry, carry = Ā·λ, which needs no states) from a zero carry at
// the chunk's end and stores the carry out of the chunk and its ΣΔ; the main
// pass then starts chunk c from the fold over the later chunks j,
// carry <- S_j + e^{A·ΣΔ_j}·carry (the carry's dependence on its start value
// is the product of the chunk's decays).
// (The exact rule's two coefficient series needed more registers than a
// 2-wave budget with 32-position segments; it keeps a 1-wave budget, within
// which the 16-position segment's kernel takes 198 VGPRs: 2 waves per SIMD.)
//
// NP: the instantiation's power-of-two state count; FULL: N == NP (N a
// compile-time constant), else N = p.N < NP and the thread rows n >= N hold
// no state (as the rows past N do for N < 4).
//
// GRP: a state group of a larger N (p.ngroups groups of NP states; the row
// stride of A, B, C, the checkpoints and the per-state gradients is p.N).
template <typename TIn, int NP, bool FULL, bool EXACT, bool AGG, bool GRP = false>
__global__ void __launch_bounds__(16 * (NP < 4 ? 4 : NP),
                                  EXACT ? MSCAN_BWD_WAVES_EXACT : (NP == 16 ? MSCAN_BWD_WAVES16 : MSCAN_BWD_WAVES))
    scan_bwd_kernel(const BwdParams p) {
  constexpr int CB = 16;
  constexpr int NGP = NP < 4 ? 4 : NP;  // thread rows
  constexpr int NT = CB * NGP;
  // segment = the forward's checkpoint interval: 16 positions (registers for
  // 16 recomputed states and decays per thread: 146 VGPRs at N = 16, 3 waves
  // per SIMD, against 206 and 2 waves with 32), 32 for 32 thread rows (each
  // row stages one position per segment)
  constexpr int TS = NGP > MSCAN_BWD_SEG ? NGP : MSCAN_BWD_SEG;
  constexpr int TH = 16;              // half segment (one butterfly)
  constexpr int TPS = TS / NGP;       // positions staged per thread per segment
  constexpr int TPH = TH / NGP > 0 ? TH / NGP : 1;  // positions summed per thread per half
  constexpr int PS = TS + 4;          // padded row of a per-channel or per-state array
  constexpr int YS = TH + 4;          // padded partial row
  constexpr int QI = (NP * TS + NT - 1) / NT;  // B (and C) elements staged per thread per segment (at most)
  static_assert(TS % NGP == 0 && TH % 4 == 0, "segment splits over the thread rows");
  static_assert(NP <= 32, "one state per thread, at most 512 threads");
  static_assert(!GRP || !FULL, "a group's state count is read at run time");
  // grid: (group,) channel block, chunk, batch, direction
  const int nblocks = gridDim.x;
  int bid = logical_block(blockIdx.x, nblocks, 4);
  const int gi = GRP ? bid % p.ngroups : 0;  // state group
  if (GRP) bid /= p.ngroups;
  const int n0 = GRP ? gi * NP : 0;           // its first state
  const int NS = GRP ? p.N : (FULL ? NP : p.N);  // states per row of A, B, C, checkpoints, per-state gradients
  const int N = GRP ? min(NP, p.N - n0) : NS;    // states of this workgroup
  constexpr bool KEEP_ABAR = MSCAN_BWD_KEEP_ABAR;

  __shared__ __attribute__((aligned(16))) float s_dt[CB * PS];   // Δ
  __shared__ __attribute__((aligned(16))) float s_u[CB * PS];    // u
  __shared__ __attribute__((aligned(16))) float s_dy[CB * PS];   // dy
  // Δ·u, shared by the channel's states (the simplified rule's input term)
  __shared__ __attribute__((aligned(16))) float s_du[EXACT ? 4 : CB * PS];
  __shared__ __attribute__((aligned(16))) float s_B[NP * PS];
  __shared__ __attribute__((aligned(16))) float s_C[NP * PS];
  // Parts of dΔ and du per wave: each wave first sums its 4 state rows in
  // registers, so a (position, channel) gathers NW = NGP/4 parts.
  constexpr int NW = NGP / 4;
  __shared__ __attribute__((aligned(16))) float s_pd[NW][CB][YS];
  __shared__ __attribute__((aligned(16))) float s_pu[NW][CB][YS];
  // (the final per-channel sums reuse s_pd: 2·NGP·CB floats, after the last barrier)
  static_assert(2 * NGP <= NW * YS, "room for the final sums");

  const int tid = threadIdx.x;
  const int cl = tid % CB;
  const int ng = tid / CB;
  const bool nvalid = ng < N;
  const int n = nvalid ? ng : 0;
  const uint32_t m1 = (cl & 2) ? ~0u : 0u, m0 = (cl & 1) ? ~0u : 0u;
  const float nvf = nvalid ? 1.f : 0.f;  // rows past N add nothing to the state sums

  const int dblk = bid % p.nblk_d;
  bid /= p.nblk_d;
  const int c = p.chunk0 + bid % p.grid_chunks;
  bid /= p.grid_chunks;
  const int b = bid % p.Bsz;
  const int k = bid / p.Bsz;

  const int D = p.Dm, L = p.L;
  const int seg_lo = c * p.chunk_len / TS;                            // the chunk's first segment
  const int seg_hi = (min(L, (c + 1) * p.chunk_len) + TS - 1) / TS - 1;  // and its last
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
  const TIn* B_s = static_cast<const TIn*>(p.B) + (int64_t)(b * p.K + k) * L * NS + n0;
  const TIn* C_s = static_cast<const TIn*>(p.C) + (int64_t)(b * p.K + k) * L * NS + n0;
  const TIn* go_s = static_cast<const TIn*>(p.dout) + (int64_t)b * L * D;
  const bool gated = p.z != nullptr;
  const TIn* z_s = gated ? static_cast<const TIn*>(p.z) + (int64_t)b * L * D : go_s;  // (no gate: unused loads)
  // the direction's fp32 output row for dz; without dz_here every lane loads
  // element 0 (one cache line, unused; of dout when there are no rows)
  const float* y_s = p.ws_y ? p.ws_y + ((int64_t)k * p.Bsz + b) * L * D : static_cast<const float*>(p.dout);
  const int64_t y_mask = p.dz_here ? ~(int64_t)0 : 0;
  const float* ck_s = p.ckpt + ((int64_t)k * p.Bsz + b) * p.ntiles * D * NS;
  const bool own = nvalid && dvalid;  // this thread's (channel, state) exists
  const int64_t ck_off = own ? (int64_t)d * NS + n0 + n : 0;

  // Stores inside the segment loop go through buffer descriptors over this
  // workgroup's slices (each at most 2^31 bytes: the plan's limits), every
  // one issued unconditionally: a lane with nothing to store takes the offset
  // kDrop, past its slice, and a descriptor of 0 bytes drops every lane (dz
  // without dz_here, the du layout not in use).  With no store under a branch
  // the compiler counts the memory operations issued after a prefetch
  // exactly, so staging waits for the prefetched rows only, not for the
  // stores issued since.
  constexpr uint32_t ES = sizeof(TIn);
  const uint32_t rowb = (uint32_t)D * ES;  // bytes per token row
  const uint32_t slice = (uint32_t)((int64_t)L * D * ES);
  const bool du32 = p.du_part != nullptr;
  const bool dz_here = p.dz_here && gi == 0;  // (dz: the same from every group)
  const auto rs_dz = make_rsrc(dz_here ? static_cast<TIn*>(p.dz) + (int64_t)b * L * D : nullptr,
                               dz_here ? slice : 0u);
  const auto rs_ddt = make_rsrc(GRP ? nullptr : static_cast<TIn*>(p.ddelta) + (int64_t)(b * p.K + k) * L * D,
                                GRP ? 0u : slice);
  // (groups: the fp32 parts of ddelta)
  const auto rs_ddt32 = make_rsrc(GRP ? p.ddelta_part + (((int64_t)gi * p.Bsz + b) * p.K + k) * L * D : nullptr,
                                  GRP ? (uint32_t)((int64_t)L * D * 4) : 0u);
  const auto rs_du = make_rsrc(du32 ? nullptr : static_cast<TIn*>(p.du) + (int64_t)(b * p.Ku + ku) * L * D,
                               du32 ? 0u : slice);
  const int64_t du_row = p.Ku != p.K ? ((int64_t)gi * p.K + k) * p.Bsz + b : ((int64_t)gi * p.Bsz + b) * p.K + k;
  const auto rs_du32 = make_rsrc(du32 ? p.du_part + du_row * L * D : nullptr,
                                 du32 ? (uint32_t)((int64_t)L * D * 4) : 0u);
  const int64_t bc_slice = (((int64_t)dblk * p.Bsz + b) * p.K + k) * L * NS;
  const auto rs_dB = make_rsrc(p.dB_part + bc_slice, (uint32_t)((int64_t)L * NS * 4));
  const auto rs_dC = make_rsrc(p.dC_part + bc_slice, (uint32_t)((int64_t)L * NS * 4));

  const float Anat = own ? p.A[((int64_t)k * D + d) * NS + n0 + n] : 0.f;
  const float Al2 = Anat * kLog2e;  // e^{ΔA} = 2^{Δ·A·log2 e}
  const float invA = Anat != 0.f ? 1.0f / Anat : 0.f;
  const float bias = (dvalid && p.delta_bias) ? p.delta_bias[k * D + d] : 0.f;
  const float Dd = (dvalid && p.D && gi == 0) ? p.D[k * D + d] : 0.f;  // (D·dy: group 0's du part)

  // raw global values of one segment (rows clamped into the sequence; padded
  // rows are zeroed at staging)
  struct Raw {
    TIn dl[TPS], u[TPS], go[TPS], zr[TPS], B[QI], C[QI];
    float y[TPS], h0;
  };
  auto load_seg = [&](int seg, Raw& r) __attribute__((always_inline)) {
    const int p0 = seg * TS;
#pragma unroll
    for (int i = 0; i < TPS; ++i) {
      const int64_t off = (int64_t)token(min(p0 + ng * TPS + i, L - 1)) * D + dc;
      r.dl[i] = dl_s[off];
      r.go[i] = go_s[off];
      r.zr[i] = z_s[off];
      if constexpr (!AGG) {
        r.u[i] = u_s[off];
        r.y[i] = y_s[off & y_mask];
      }
    }
#pragma unroll
    for (int i = 0; i < QI; ++i) {
      const int q = min(tid + i * NT, N * TS - 1);
      const int64_t off = (int64_t)token(min(p0 + q / N, L - 1)) * NS + q % N;
      if constexpr (!AGG) r.B[i] = B_s[off];
      r.C[i] = C_s[off];
    }
    if constexpr (!AGG) r.h0 = ck_s[(int64_t)seg * D * NS + ck_off];
  };
  auto stage_seg = [&](int seg, const Raw& r) __attribute__((always_inline)) {
    const int p0 = seg * TS;
#pragma unroll
    for (int i = 0; i < TPS; ++i) {
      const int tt = ng * TPS + i;
      const float okf = (p0 + tt < L && dvalid) ? 1.f : 0.f;
      const float x = to_f32(r.dl[i]) + bias;
      const float dtv = (p.softplus ? softplus_log2(x) * kLn2 : x) * okf;
      s_dt[cl * PS + tt] = dtv;
      if constexpr (!AGG) {
        const float uu = to_f32(r.u[i]) * okf;
        s_u[cl * PS + tt] = uu;
        if constexpr (!EXACT) s_du[cl * PS + tt] = dtv * uu;
      }
      // dy = dout·silu(z); with one direction also dz = dout·y·silu'(z)
      const float g = to_f32(r.go[i]);
      float dyv = g, dzv = 0.f;
      if (gated) {
        const float zz = to_f32(r.zr[i]);
        const float sg = rcp(1.0f + ex2(-zz * kLog2e));
        dyv = g * zz * sg;
        if constexpr (!AGG) dzv = g * r.y[i] * sg * __builtin_fmaf(zz, 1.0f - sg, 1.0f);
      }
      if constexpr (!AGG) {
        const int pp = min(p0 + tt, L - 1);
        const uint32_t off = __umul24((uint32_t)token(pp), rowb) + (uint32_t)dc * ES;
        store_out(dzv, rs_dz, (gated && p0 + tt < L && dvalid) ? off : kDrop, 0u, (TIn*)nullptr);
      }
      s_dy[cl * PS + tt] = dyv * okf;
    }
#pragma unroll
    for (int i = 0; i < QI; ++i) {
      const int q = tid + i * NT;
      if (QI * NT == N * TS || q < N * TS) {
        const float okf = p0 + q / N < L ? 1.f : 0.f;
        if constexpr (!AGG) s_B[(q % N) * PS + q / N] = to_f32(r.B[i]) * okf;
        s_C[(q % N) * PS + q / N] = to_f32(r.C[i]) * okf;
      }
    }
  };

  float carry = 0.f;  // Ā_{p+1}·λ_{p+1}
  if constexpr (!AGG) {
    // the carry into this chunk: fold the later chunks' aggregates
    // (the aggregates of kFoldBatch chunks loaded together before their updates)
    if (own) {
      const int64_t arow = ((int64_t)k * p.Bsz + b) * (p.nchunks - 1);
      for (int j0 = p.nchunks - 1; j0 > c; j0 -= kFoldBatch) {
        float dsv[kFoldBatch], Sv[kFoldBatch];
#pragma unroll
        for (int q = 0; q < kFoldBatch; ++q) {
          const int64_t r = arow + (max(j0 - q, c + 1) - 1);  // (past c + 1: chunk c + 1 again, unused)
          dsv[q] = p.agg_dsum[r * D + d];
          Sv[q] = p.agg_S[(r * D + d) * NS + n0 + n];
        }
#pragma unroll
        for (int q = 0; q < kFoldBatch; ++q)
          if (j0 - q > c) carry = __builtin_fmaf(ex2(dsv[q] * Al2), carry, Sv[q]);
      }
    }
  }
  float dA_acc = 0.f, dD_acc = 0.f, dbias_acc = 0.f, dsum = 0.f;

  // The loop is rotated: a segment's rows are loaded at the start of the
  // segment after it (in walk order) and staged at its end, so no load in
  // flight crosses the loop's back edge.  (Every read of the staging arrays
  // comes before the last barrier of a segment, so staging needs no barrier
  // of its own.)  Wave priorities: the recompute and the adjoint steps 1,
  // staging and the per-position sums 0 (the cross scan's backward: 2.72 ->
  // 2.65 ms).
  Raw raw;
  float h0n = 0.f;
  auto stage = [&](int seg) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(0);
    stage_seg(seg, raw);
    // the checkpoint is waited for here, with the staged rows
    h0n = (!AGG && own) ? raw.h0 : 0.f;
    asm volatile("" ::"v"(h0n));
  };
  load_seg(seg_hi, raw);
  stage(seg_hi);
  for (int seg = seg_hi; seg >= seg_lo; --seg) {
    const int p0 = seg * TS;
    const float h0 = h0n;
    __syncthreads();
    load_seg(seg > seg_lo ? seg - 1 : seg, raw);  // (the last segment reloads its own rows, unused)

    if constexpr (AGG) {
#pragma unroll 8
      for (int s = TS - 1; s >= 0; --s) {
        const float dt = s_dt[cl * PS + s];
        const float l = __builtin_fmaf(s_C[n * PS + s], s_dy[cl * PS + s], carry);
        carry = ex2(dt * Al2) * l;
        dsum += dt;
      }
      __syncthreads();  // the staging arrays are rewritten by the next segment
    } else {

    // ---- recompute the segment's states from its checkpoint ----
    __builtin_amdgcn_s_setprio(1);
    float hs[TS], as[KEEP_ABAR ? TS : 1];
    {
      float h = h0;
#pragma unroll
      for (int s = 0; s < TS; ++s) {
        const float dt = s_dt[cl * PS + s];
        const float Bv = s_B[n * PS + s];
        const float a = ex2(dt * Al2);
        if constexpr (EXACT) {
          const float c = zoh_coef(a, dt * Anat, dt, invA);
          h = __builtin_fmaf(a, h, c * s_u[cl * PS + s] * Bv);
        } else {
          h = __builtin_fmaf(a, h, s_du[cl * PS + s] * Bv);  // (Δ·u)·B
        }
        hs[s] = h;
        if constexpr (KEEP_ABAR) as[s] = a;
      }
    }
    // The adjoint reads the staged values again from LDS: kept live from the
    // recompute they would take five registers per position.
    asm volatile("" ::: "memory");

    // ---- the adjoint over the two halves, later half first ----
#pragma unroll
    for (int half = TS / TH - 1; half >= 0; --half) {
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int qt = 1; qt >= 0; --qt) {
        // dB and dC terms of the quarter's 8 steps: [r] dB of step r, [8 + r] dC
        float pBC[16];
#pragma unroll
        for (int s4 = 4; s4 >= 0; s4 -= 4) {
          float pd4[4], pu4[4];
#pragma unroll
          for (int r = 3; r >= 0; --r) {
            const int sq = s4 + r;                 // step within the quarter
            const int s = half * TH + qt * 8 + sq;  // step within the segment
            const float dt = s_dt[cl * PS + s];
            const float dyv = s_dy[cl * PS + s];
            const float Bv = s_B[n * PS + s];
            const float Cv = s_C[n * PS + s];
            const float a = KEEP_ABAR ? as[s] : ex2(dt * Al2);
            const float hp = s > 0 ? hs[s - 1] : h0;
            const float l = __builtin_fmaf(Cv, dyv, carry);  // λ
            const float ga = l * hp;
            const float lB = l * Bv;
            if constexpr (EXACT) {
              const float uu = s_u[cl * PS + s];
              const float x = dt * Anat;
              const float c = zoh_coef(a, x, dt, invA);
              // dc/dΔ = e^{ΔA}; dc/dA from zoh_coef_dA
              pd4[r] = __builtin_fmaf(ga * Anat, a, a * lB * uu);
              pu4[r] = lB * c;
              dA_acc = __builtin_fmaf(lB * zoh_coef_dA(a, x, dt, c, invA), uu, dA_acc);
              pBC[sq] = l * c * uu;
              dA_acc = __builtin_fmaf(ga * dt, a, dA_acc);
            } else {
              // dΔ = Σ_n λ h_{p-1} Ā A_n + u·Σ_n λ B_n and du = Δ·Σ_n λ B_n:
              // the per-state parts are λ h_{p-1} Ā A_n and λ B_n, the
              // channel's u and Δ enter once per position in the sums below
              const float gaa = ga * a;
              pd4[r] = gaa * Anat;
              pu4[r] = lB;
              dA_acc = __builtin_fmaf(gaa, dt, dA_acc);
              pBC[sq] = l * s_du[cl * PS + s];  // λ·(Δ·u)
            }
            pBC[8 + sq] = dyv * hs[s];
            carry = a * l;
          }
          // the 4 steps' parts summed over the wave's 4 state rows: row r of
          // the wave ends with step r
          const int sh = qt * 8 + s4 + (ng & 3);  // position within the half
          s_pd[ng >> 2][cl][sh] = sum_rows4(pd4, nvf);
          s_pu[ng >> 2][cl][sh] = sum_rows4(pu4, nvf);
        }
        // sums over the row's 16 channels: lane cl < 8 ends with dB of step
        // cl, lane cl >= 8 with dC of step cl - 8
        const float sBC = row_sum_transpose16(pBC, m1, m0);
        const int pp = p0 + half * TH + qt * 8 + (cl & 7);
        const uint32_t off = __umul24((uint32_t)token(min(pp, L - 1)), (uint32_t)NS * 4u) + (uint32_t)(n0 + n) * 4u;
        const bool ok = nvalid && pp < L;
        buf_store(sBC, rs_dB, (ok && cl < 8) ? off : kDrop, 0u);
        buf_store(sBC, rs_dC, (ok && cl >= 8) ? off : kDrop, 0u);
      }
      __syncthreads();
      // ---- sums over states, per (position, channel) ----
      __builtin_amdgcn_s_setprio(0);
      // (with 32 thread rows, rows 16..31 have no position of the half: they
      // repeat the last one, add nothing and store nothing)
      constexpr bool ALLROWS = TPH * NGP <= TH;
#pragma unroll
      for (int i = 0; i < TPH; ++i) {
        const int sh0 = ng * TPH + i;  // position within the half
        const bool hv = ALLROWS || sh0 < TH;
        const int sh = hv ? sh0 : TH - 1;
        const float hf = hv ? 1.f : 0.f;
        const int s = half * TH + sh;
        const int pp = p0 + s;
        float dd = 0.f, duu = 0.f;
#pragma unroll
        for (int g = 0; g < NW; ++g) {
          dd += s_pd[g][cl][sh];
          duu += s_pu[g][cl][sh];
        }
        const float dt = s_dt[cl * PS + s];
        const float uu = s_u[cl * PS + s];
        const float dyv = s_dy[cl * PS + s];
        if constexpr (!EXACT) {  // duu holds Σ_n λ B_n
          dd = __builtin_fmaf(uu, duu, dd);
          duu *= dt;
        }
        // softplus'(x) = sigmoid(x) = 1 - e^{-Δ}
        const float dx = p.softplus ? dd * (1.0f - ex2(-dt * kLog2e)) : dd;
        duu = __builtin_fmaf(Dd, dyv, duu);
        dD_acc = __builtin_fmaf(dyv * hf, uu, dD_acc);
        dbias_acc = __builtin_fmaf(dx, hf, dbias_acc);
        const uint32_t t = (uint32_t)token(min(pp, L - 1));
        const bool ok = hv && pp < L && dvalid;
        const uint32_t roff = __umul24(t, rowb) + (uint32_t)dc * ES;
        const uint32_t roff4 = __umul24(t, (uint32_t)D * 4u) + (uint32_t)dc * 4u;
        if constexpr (GRP)
          buf_store(dx, rs_ddt32, ok ? roff4 : kDrop, 0u);
        else
          store_out(dx, rs_ddt, ok ? roff : kDrop, 0u, (TIn*)nullptr);
        store_out(duu, rs_du, ok ? roff : kDrop, 0u, (TIn*)nullptr);
        buf_store(duu, rs_du32, ok ? roff4 : kDrop, 0u);
      }
      __syncthreads();  // the partial rows are rewritten by the next half
    }
    }  // !AGG
    if (seg > seg_lo) stage(seg - 1);
  }

  if constexpr (AGG) {
    if (dvalid) {
      const int64_t r = ((int64_t)k * p.Bsz + b) * (p.nchunks - 1) + (c - 1);
      if (nvalid) p.agg_S[(r * D + d) * NS + n0 + n] = carry;
      if (ng == 0 && gi == 0) p.agg_dsum[r * D + d] = dsum;
    }
    return;
  }

  // ---- per-(b, k, d) and per-(b, k, d, n) results ----
  float* s_red = &s_pd[0][0][0];  // [2][NGP][CB]
  s_red[ng * CB + cl] = dD_acc;
  s_red[(NGP + ng) * CB + cl] = dbias_acc;
  __syncthreads();
  if (dvalid) {
    if (nvalid) {
      const int64_t o = (((int64_t)b * p.K + k) * D + d) * NS + n0 + n;
      p.dA_part[(int64_t)c * p.Bsz * p.K * D * NS + o] = dA_acc;
      if (p.dinit && c == 0) p.dinit[o] = carry;
    }
    if (ng == 0) {
      float sD = 0.f, sb = 0.f;
#pragma unroll
      for (int g = 0; g < NGP; ++g) {
        sD += s_red[g * CB + cl];
        sb += s_red[(NGP + g) * CB + cl];
      }
      const int64_t o = ((((int64_t)gi * p.nchunks + c) * p.Bsz + b) * p.K + k) * D + d;
      p.dD_part[o] = gi == 0 ? sD : 0.f;  // (dD: the same sum in every group)
      p.dbias_part[o] = sb;
    }
  }
}

}  // namespace mscan
