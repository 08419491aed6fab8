// conv_kernels.h -- gfx950 HIP kernel of the causal depthwise Conv1d + SiLU
// that produces the scan input u.
//
// Sources, cited by page title and section:
//   [MFS] "从零理解 Mamba：选择性状态空间模型（Selective SSM）到 Mamba Block" (eutaboo.com):
//         §6.2 Step 2 (small depthwise causal 1-D convolution before the SSM),
//         §8 (d_conv = 4)
//   [VIM] "Vision Mamba：从状态空间模型到视觉革命的跨越" (x-humanoid.csdn.net): §2.2
//         (each scan direction convolved on its own)
//   [S4M] "从S4到Mamba：选择性状态空间模型的演进与革新" (jsqmd.com): §3 (depthwise
//         convolution, then SiLU)
//
// out(s) = silu(bias[d] + Σ_{j<W} w[d][j]·x(s - (W-1) + j)), x = 0 before the
// start, along the sequence or along the reversed sequence.
//
// The kernel is bound by HBM traffic: each thread owns 8 consecutive channels
// (one 16-byte bf16 vector) and a run of T positions, reads the T + W - 1 rows
// it needs once (a sliding window in registers) and writes T rows.  Threads
// with consecutive indices take consecutive channel vectors, so a wave reads
// and writes contiguous row segments.
#pragma once

#include "device_math.h"

namespace mscan {

struct ConvParams {
  const void* x;      // [Bsz][L][Dm]
  const float* w;     // [Dm][W]
  const float* bias;  // [Dm] or null
  void* out;          // [Bsz][L][Dm]
  int Bsz, L, Dm, reverse;
};

template <typename TIn, int W, int T>
__global__ void __launch_bounds__(256) conv1d_silu_kernel(const ConvParams p) {
  constexpr int V = 8;
  const int nvec = p.Dm / V;
  const int nrun = (p.L + T - 1) / T;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)p.Bsz * nrun * nvec) return;
  const int dv = (int)(i % nvec);
  const int64_t rest = i / nvec;
  const int run = (int)(rest % nrun);
  const int b = (int)(rest / nrun);
  const int d0 = dv * V;
  const int s0 = run * T;
  const int L = p.L;

  float w[W][V], bias[V];
#pragma unroll
  for (int c = 0; c < V; ++c) {
    bias[c] = p.bias ? p.bias[d0 + c] : 0.f;
#pragma unroll
    for (int j = 0; j < W; ++j) w[j][c] = p.w[(d0 + c) * W + j];
  }
  const TIn* xb = static_cast<const TIn*>(p.x) + (int64_t)b * L * p.Dm + d0;
  TIn* ob = static_cast<TIn*>(p.out) + (int64_t)b * L * p.Dm + d0;
  auto row = [&](int s) { return (int64_t)(p.reverse ? L - 1 - s : s) * p.Dm; };

  // Before output position s: win[j] holds position s - W + j for j >= 1; each
  // step shifts the window down one slot and takes position s into slot W-1,
  // so that win[j] holds position s - (W-1) + j while s is computed.
  float win[W][V];
#pragma unroll
  for (int j = 0; j < W; ++j) {
    const int s = s0 - W + j;
    if (j >= 1 && s >= 0) {
      Vec<TIn, V> v;
      v.load(xb + row(s));
#pragma unroll
      for (int c = 0; c < V; ++c) win[j][c] = v.get(c);
    } else {
#pragma unroll
      for (int c = 0; c < V; ++c) win[j][c] = 0.f;
    }
  }
  // Rows arrive in groups of RG, the next group's loads issued before the
  // current group is computed.  Rows past the end are clamped to the last row
  // (their outputs are not stored), so the loads carry no branch.
  constexpr int RG = T < 8 ? T : 8;
  static_assert(T % RG == 0, "whole row groups");
  Vec<TIn, V> rows[2][RG];
  auto load_group = [&](int g, Vec<TIn, V>(&dst)[RG]) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < RG; ++r) dst[r].load(xb + row(min(s0 + g * RG + r, L - 1)));
  };
  load_group(0, rows[0]);
#pragma unroll
  for (int g = 0; g < T / RG; ++g) {
    if (g + 1 < T / RG) load_group(g + 1, rows[(g + 1) & 1]);
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const int s = s0 + g * RG + r;
#pragma unroll
      for (int j = 0; j + 1 < W; ++j)
#pragma unroll
        for (int c = 0; c < V; ++c) win[j][c] = win[j + 1][c];
      float y[V];
#pragma unroll
      for (int c = 0; c < V; ++c) {
        win[W - 1][c] = rows[g & 1][r].get(c);
        float acc = bias[c];
#pragma unroll
        for (int j = 0; j < W; ++j) acc = __builtin_fmaf(w[j][c], win[j][c], acc);
        y[c] = silu_f(acc);
      }
      if (s < L) {
        if constexpr (sizeof(TIn) == 2) {
          // non-temporal 16-byte store: the output is not read again here,
          // and keeping it out of the caches measured 31 -> 25 us on an
          // [8][2048][1536] bf16 input (4.1 TB/s, 93 % of a plain copy)
          const u32x4 v = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                           pack_bf16x2(y[6], y[7])};
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(ob + row(s)));
        } else {
          typedef float f32x4 __attribute__((ext_vector_type(4)));
          const f32x4 v0 = {y[0], y[1], y[2], y[3]}, v1 = {y[4], y[5], y[6], y[7]};
          __builtin_nontemporal_store(v0, reinterpret_cast<f32x4*>(ob + row(s)));
          __builtin_nontemporal_store(v1, reinterpret_cast<f32x4*>(ob + row(s)) + 1);
        }
      }
    }
  }
}

}  // namespace mscan
