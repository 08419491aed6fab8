/*
 * conv_oracle.c -- plain fp64 CPU oracle of the causal depthwise Conv1d + SiLU
 * that produces the scan input u.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this code.  The product path
 * (the HIP library) shares no code, header, table or helper with it.
 *
 * Sources (web pages; cited by title and section):
 *   [MFS] "从零理解 Mamba：选择性状态空间模型（Selective SSM）到 Mamba Block
 *          （面向医学图像分割的基础铺垫）" (eutaboo.com): §6.2 Step 2 (a small
 *          depthwise causal 1-D convolution mixes neighbouring tokens before
 *          the selective SSM), §8 (the module is built with d_conv = 4)
 *   [VIM] "Vision Mamba：从状态空间模型到视觉革命的跨越" (x-humanoid.csdn.net):
 *          §2.2 VimBlock (each scan direction is convolved on its own)
 *   [S4M] "从S4到Mamba：选择性状态空间模型的演进与革新" (jsqmd.com): §3 (depthwise
 *          convolution, then SiLU, ahead of the scan)
 *
 * For batch b, channel d and sequence position s (s = t, or s = L-1-t along
 * the reversed sequence), with W taps w[d][0..W-1]:
 *   pre(s) = bias[d] + sum_{j=0}^{W-1} w[d][j] * x(s - (W-1) + j),  x(s) = 0 for s < 0
 *   out    = silu(pre) = pre / (1 + exp(-pre))   (or pre when activation is 0)
 * so tap W-1 weighs the current token and tap 0 the oldest one.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static double ldx(const void* p, int dtype, int64_t i) {
  if (dtype == 1) {
    uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
  }
  return (double)((const float*)p)[i];
}

/* x, out: [batch][seqlen][dim] (x float32 values or bfloat16 bit patterns;
 * out float64); w: [dim][width]; bias: [dim] or NULL.  Returns 0, or -1 on
 * invalid sizes. */
int oracle_conv1d(int64_t batch, int64_t dim, int64_t seqlen, int32_t dtype, int32_t width, int32_t reverse,
                  int32_t activation, const void* x, const float* w, const float* bias, double* out) {
  if (batch <= 0 || dim <= 0 || seqlen <= 0 || width <= 0 || !x || !w || !out) return -1;
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t d = 0; d < dim; ++d) {
      for (int64_t s = 0; s < seqlen; ++s) {
        double acc = bias ? (double)bias[d] : 0.0;
        for (int32_t j = 0; j < width; ++j) {
          const int64_t q = s - (width - 1) + j;
          if (q < 0) continue;
          const int64_t tq = reverse ? seqlen - 1 - q : q;
          acc += (double)w[d * width + j] * ldx(x, dtype, (b * seqlen + tq) * dim + d);
        }
        const int64_t t = reverse ? seqlen - 1 - s : s;
        out[(b * seqlen + t) * dim + d] = activation ? acc / (1.0 + exp(-acc)) : acc;
      }
    }
  }
  return 0;
}
