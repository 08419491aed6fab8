/*
 * mamba_scan.h -- C ABI of the MI355X (gfx950) selective-scan library
 * (libmamba_scan.so).
 *
 * The library computes the S6 selective scan of the Mamba layer and its
 * bidirectional (Vision Mamba) and four-way cross-scan (VMamba SS2D) forms,
 * plus a one-token recurrent step.  Sources, cited by page title and section:
 *   [MFS] "从零理解 Mamba：选择性状态空间模型（Selective SSM）到 Mamba Block
 *          （面向医学图像分割的基础铺垫）" (eutaboo.com)
 *   [S4M] "从S4到Mamba：选择性状态空间模型的演进与革新" (jsqmd.com)
 *   [MUN] "【临时文档---算法介绍】Mamba-UNet" (blog.csdn.net)
 *   [VIM] "Vision Mamba：从状态空间模型到视觉革命的跨越" (x-humanoid.csdn.net)
 *
 * What one scan direction k computes for batch b and channel d, visiting the
 * tokens t in that direction's order, with h[n] = 0 (or initial_state) before
 * the first token:
 *   Δ     = softplus(delta[t] + delta_bias[d])      [MFS §4.1 Algorithm 2; MUN §4]
 *   Ā_n   = exp(Δ·A[d][n])                          [MFS §6.2 Step 4, eq (4)]
 *   h[n]  = Ā_n·h[n] + Δ·B[t][n]·u[t]               [MFS §2.2 eq (2a); MUN §4: B̄ ≈ ΔB]
 *           (exact_zoh: ((Ā_n - 1)/A[d][n])·B[t][n]·u[t] [MFS §6.2 eq (4)])
 *   y_k   = Σ_n C[t][n]·h[n] + D[d]·u[t]            [MFS eq (2b); MUN §4: y = Ch + Dx]
 * and the output is out[t] = (Σ_k y_k[t])·silu(z[t]) [MFS §6.2 Step 6; VIM §2.2].
 *
 * Conventions common to every entry point
 *   - Every tensor is dense, row-major and C-contiguous, and indexed by token
 *     position in the original (grid) order, never by scan order.
 *   - All pointers are device pointers (HIP device memory) unless stated
 *     otherwise.  The caller owns every buffer.  The library allocates no
 *     memory and is safe to call from several host threads.  Calls on the
 *     same buffers must not overlap.  Its only state is the static device
 *     scratch of mamba_scan_fwd_noalloc (and that scratch's address on each
 *     device, looked up once).
 *   - Calls are asynchronous on `stream` (0 = the null stream).  The return
 *     value reports host-side validation and launch errors only; faults during
 *     execution surface at the next synchronisation of the stream.
 *   - Device pointers must be 16-byte aligned.
 */
#ifndef MAMBA_SCAN_H
#define MAMBA_SCAN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden visibility; these are its only exports. */
#define MAMBA_API __attribute__((visibility("default")))

/* Return codes. */
typedef enum {
  MAMBA_OK = 0,
  MAMBA_ERR_INVALID = -1,     /* NULL required pointer, size <= 0, L != H*W, unknown mode or dtype */
  MAMBA_ERR_UNSUPPORTED = -2, /* valid but not built: N above 64 (for the backward and
                                 mamba_scan_fwd_save also dim not a multiple of 8), dim
                                 not a multiple of 8 (bf16) or 4 (f32), a pointer
                                 not 16-byte aligned, or sizes beyond
                                 the 32-bit offsets used inside one (batch, direction) slice:
                                 (seqlen+64)*dim*sizeof(dtype) below 2^31 bytes, and for
                                 several directions (and for mamba_scan_bwd) seqlen*dim*4
                                 at most 2^31 bytes; seqlen and dim*4 below 2^24 */
  MAMBA_ERR_WORKSPACE = -3,   /* workspace NULL or smaller than mamba_scan_fwd_workspace_bytes() */
  MAMBA_ERR_HIP = -4,         /* the HIP runtime rejected a launch */
  MAMBA_ERR_SCRATCH = -5      /* mamba_scan_fwd_noalloc: the problem needs more scratch than the
                                 library's static array holds (MAMBA_NOALLOC_SCRATCH_BYTES) */
} mamba_status;

/* Size of the static device scratch that mamba_scan_fwd_noalloc uses. */
#define MAMBA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* Scan directions.  K is the number of directions each mode runs.
 *   MAMBA_DIR_FWD      K=1: tokens 0..L-1.
 *   MAMBA_DIR_BWD      K=1: tokens L-1..0.
 *   MAMBA_DIR_BIDIR    K=2: k=0 forward, k=1 reversed, summed [VIM §2.2, VimBlock].
 *   MAMBA_DIR_CROSS2D  K=4 over an H×W grid, token t = row*W + col [S4M §3, SS2D]:
 *                      k=0 row-major, k=1 column-major (t = (p mod H)*W + p div H at
 *                      scan position p), k=2 row-major reversed, k=3 column-major
 *                      reversed; the four outputs are summed at each grid position. */
typedef enum {
  MAMBA_DIR_FWD = 0,
  MAMBA_DIR_BWD = 1,
  MAMBA_DIR_BIDIR = 2,
  MAMBA_DIR_CROSS2D = 3
} mamba_dir_mode;

/* Element type of u, delta, z, B, C and out (A, D, delta_bias and states are
 * always float32).  bf16 outputs are rounded to nearest, ties to even, once,
 * after the direction sum and the gate. */
typedef enum { MAMBA_DTYPE_F32 = 0, MAMBA_DTYPE_BF16 = 1 } mamba_dtype;

/* Problem description shared by the entry points (host memory). */
typedef struct {
  int64_t batch;   /* B >= 1 */
  int64_t dim;     /* D >= 1, the channel count (d_inner); a multiple of 8 for bf16, of 4 for f32 */
  int64_t seqlen;  /* L >= 1 tokens (ignored by mamba_scan_step) */
  int64_t dstate;  /* N, state size per channel: 1..64 */
  int64_t height;  /* MAMBA_DIR_CROSS2D only: grid rows H, with H*W == L; else 0 */
  int64_t width;   /* MAMBA_DIR_CROSS2D only: grid columns W; else 0 */
  int32_t dtype;          /* mamba_dtype */
  int32_t delta_softplus; /* 1: Δ = softplus(delta + bias); 0: Δ = delta + bias */
  int32_t exact_zoh;      /* 0: input term Δ·B·u (the simplified rule [MUN §4]);
                             1: exact zero-order hold ((e^{ΔA} - 1)/A)·B·u, Δ·B·u where
                             A = 0 [MFS §6.2 Step 4, eq (4)] */
  const float* initial_state; /* optional device pointer, [B][K][D][N] float32: state before
                                 each direction's first token; NULL = zeros */
  void* workspace;            /* device scratch owned by the caller (may be NULL when
                                 mamba_scan_fwd_workspace_bytes() returns 0) */
  size_t workspace_bytes;     /* size of workspace */
} mamba_dims;

/*
 * Bytes of device workspace mamba_scan_fwd needs for these dims and mode
 * (time-split carries of long sequences, per-direction partial outputs of
 * the multi-direction modes, and for the one-channel-per-lane kernel that
 * serves long single-direction sequences and state sizes that are not a
 * power of two, float32 copies of B and C padded to a power-of-two N).  A pure function of its arguments: it makes no
 * HIP call.  Returns 0 when no workspace is needed, and (size_t)-1 when the
 * arguments are invalid.  The workspace contents need not be initialised.
 */
MAMBA_API size_t mamba_scan_fwd_workspace_bytes(const mamba_dims* dims, int dir_mode);

/*
 * Selective-scan forward pass [MFS §6.2 Step 4 and Step 6; VIM §2.2; S4M §3].
 *
 * Layouts (K from dir_mode; Ku = 1 for MAMBA_DIR_CROSS2D, whose four
 * directions share u, else Ku = K; an axis of size 1 may be read as absent):
 *   u           [B][Ku][L][D]  dtype
 *   delta       [B][K][L][D]   dtype   (Δ before bias and softplus)
 *   A           [K][D][N]      float32 (continuous-time diagonal A, normally < 0)
 *   B, C        [B][K][L][N]   dtype   (input-dependent B_t, C_t)
 *   D           [K][D]         float32 or NULL (no skip term)
 *   z           [B][L][D]      dtype or NULL (no gate)
 *   delta_bias  [K][D]         float32 or NULL (zero bias)
 *   out         [B][L][D]      dtype, written; must not alias any input
 *   last_state  [B][K][D][N]   float32 or NULL: the state after each
 *                              direction's final scan step (for a reversed
 *                              direction, after token 0)
 * Errors: MAMBA_ERR_INVALID / _UNSUPPORTED / _WORKSPACE before any GPU work;
 * MAMBA_ERR_HIP if a launch is rejected.
 */
MAMBA_API int mamba_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                   const float* D, const void* z, const float* delta_bias, const mamba_dims* dims,
                   int dir_mode, void* out, float* last_state, hipStream_t stream);

/*
 * mamba_scan_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, layouts, results and errors as mamba_scan_fwd, except that
 * dims->workspace and dims->workspace_bytes are ignored: the scratch the scan
 * needs (mamba_scan_fwd_workspace_bytes(dims, dir_mode) bytes) comes from a
 * static device array of MAMBA_NOALLOC_SCRATCH_BYTES (32 MiB) inside the
 * library, one per device, which each device holds until the process ends.
 * The call allocates and frees nothing.  A problem that needs more scratch
 * returns MAMBA_ERR_SCRATCH before any GPU work.  The scratch is looked up
 * (hipGetSymbolAddress) on the first call on each device, the device of
 * `stream` (the current device for the null stream); MAMBA_ERR_HIP if that
 * fails.  Nothing in the scratch has to start at zero: every call writes
 * what it reads.  Calls that overlap in time on one device (concurrent
 * streams, several host threads) share that device's array and race; the
 * caller serialises them.  The caller still passes every input and output.
 */
MAMBA_API int mamba_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B,
                                     const void* C, const float* D, const void* z, const float* delta_bias,
                                     const mamba_dims* dims, int dir_mode, void* out, float* last_state,
                                     hipStream_t stream);

/*
 * One recurrent step of a forward scan (decode) [MFS §2.3: the recurrent form
 * updates the state one token at a time].  For every batch b and channel d it
 * applies the forward-scan update to `state` for one token and writes that
 * token's gated output.
 *   state        [B][D][N]  float32, read and updated in place (same layout as
 *                           last_state of a MAMBA_DIR_FWD scan)
 *   u_t, delta_t [B][D]     dtype
 *   A            [D][N]     float32
 *   B_t, C_t     [B][N]     dtype
 *   D            [D]        float32 or NULL
 *   z_t          [B][D]     dtype or NULL
 *   delta_bias   [D]        float32 or NULL
 *   out          [B][D]     dtype, written; must not alias any input
 * dims->seqlen, height, width, initial_state and workspace are ignored.
 */
MAMBA_API int mamba_scan_step(float* state, const void* u_t, const void* delta_t, const float* A,
                    const void* B_t, const void* C_t, const float* D, const void* z_t,
                    const float* delta_bias, const mamba_dims* dims, void* out, hipStream_t stream);

/*
 * Causal depthwise Conv1d followed by SiLU, the step that produces the scan
 * input u from the expanded activations [MFS §6.2 Step 2 (a small depthwise
 * causal 1-D convolution before the SSM); MFS §8 (d_conv = 4); VIM §2.2 (each
 * direction convolved on its own); S4M §3 (depthwise convolution, then SiLU)].
 * For batch b, channel d and sequence position s, with W = width taps:
 *   out(s) = silu(bias[d] + Σ_{j=0}^{W-1} weight[d][j]·x(s - (W-1) + j)),
 *   x(s) = 0 for s < 0 (tap W-1 weighs the current token),
 * where s is the token index t, or L-1-t when reverse is nonzero (the
 * convolution runs along the reversed sequence, as for a backward scan).
 *   x       [B][L][D]  dtype
 *   weight  [D][W]     float32 (a depthwise Conv1d weight [D][1][W] without its middle axis)
 *   bias    [D]        float32 or NULL
 *   out     [B][L][D]  dtype, written; must not alias x
 * Uses dims->batch, dim, seqlen and dtype only.  Errors: MAMBA_ERR_INVALID
 * (NULL pointer, size <= 0, unknown dtype), MAMBA_ERR_UNSUPPORTED (width above
 * 4, dim not a multiple of 8, x or out not 16-byte aligned), MAMBA_ERR_HIP.
 */
MAMBA_API int mamba_conv1d_silu(const void* x, const float* weight, const float* bias, const mamba_dims* dims,
                                int width, int reverse, void* out, hipStream_t stream);

/*
 * Bytes of device workspace mamba_scan_bwd needs for these dims and mode.  A
 * pure function of its arguments; (size_t)-1 when the arguments are invalid
 * or the backward pass is not built for them.  The workspace is never 0.
 */
MAMBA_API size_t mamba_scan_bwd_workspace_bytes(const mamba_dims* dims, int dir_mode);

/*
 * Bytes of the saved forward state that mamba_scan_fwd_save writes and
 * mamba_scan_bwd can read in place of its forward recompute: the state before
 * every 16th position (every 32nd when N is 17..32), [K][B][ceil(L/16 or
 * 32)][D][N] float32, and, when gated is
 * nonzero (a scan with z whose dz will be asked for), after it (at a 256-byte
 * aligned offset) the ungated per-direction outputs [K][B][L][D] float32.
 * A pure function of its arguments; (size_t)-1 when the arguments are invalid
 * or the backward pass is not built for them (as mamba_scan_bwd_workspace_bytes).
 */
MAMBA_API size_t mamba_scan_saved_bytes(const mamba_dims* dims, int dir_mode, int gated);

/*
 * mamba_scan_fwd that also writes the saved forward state (layout above, with
 * the rows when z is not NULL) into saved, a device buffer of saved_bytes
 * owned by the caller, so that the training pass's backward need not recompute
 * the states [MFS §5 and S4M §2.3 recompute them instead; this trades that
 * recomputation for the buffer: 151 MB for a batch-8, 2048-token, 1536-channel
 * layer].  out and last_state are those of mamba_scan_fwd for the same
 * arguments.  Same errors as mamba_scan_fwd, plus MAMBA_ERR_INVALID for a
 * NULL saved and MAMBA_ERR_WORKSPACE when saved_bytes is below
 * mamba_scan_saved_bytes(dims, dir_mode, z != NULL); built for dstate N in
 * 1..64 and a channel count that is a multiple of 8, like the backward pass.
 */
MAMBA_API int mamba_scan_fwd_save(const void* u, const void* delta, const float* A, const void* B, const void* C,
                                  const float* D, const void* z, const float* delta_bias, const mamba_dims* dims,
                                  int dir_mode, void* out, float* last_state, void* saved, size_t saved_bytes,
                                  hipStream_t stream);

/*
 * Selective-scan backward pass: gradients of a loss with respect to every
 * input of mamba_scan_fwd, given dout = ∂loss/∂out [MFS §5 and S4M §2.3: the
 * training pass keeps only the inputs and recomputes the states].  Same
 * inputs, layouts, dims and dir_mode as mamba_scan_fwd (dims->initial_state,
 * if set, is the state the forward started from); the gradients have the
 * layout and element type of their input:
 *   dout         [B][L][D]    dtype (read)
 *   du           [B][Ku][L][D] dtype   (the cross scan sums its four directions)
 *   ddelta       [B][K][L][D]  dtype   (with respect to delta before bias and softplus)
 *   dA           [K][D][N]     float32
 *   dB, dC       [B][K][L][N]  dtype
 *   dD           [K][D]        float32, or NULL: not computed
 *   dz           [B][L][D]     dtype,   or NULL: not computed (ignored without z)
 *   ddelta_bias  [K][D]        float32, or NULL: not computed
 *   dinit        [B][K][D][N]  float32, or NULL: gradient of the initial state
 * Per direction, with λ the adjoint of the state (λ = C·dy + Ā_next·λ_next
 * backwards over the scan order) and dy = dout·silu(z):
 *   du = Σ_n λ·c·B + D·dy,  dΔ = Σ_n λ·(A·Ā·h_prev + (∂c/∂Δ)·B·u),
 *   dA = Σ λ·(Δ·Ā·h_prev + (∂c/∂A)·B·u),  dB = Σ_d λ·c·u,  dC = Σ_d dy·h,
 *   dD = Σ dy·u,  dz = dout·(Σ_k y_k)·silu'(z),  ddelta = dΔ·sigmoid(delta + bias)
 * (c = Δ, or (Ā - 1)/A with exact_zoh).  The gradient outputs must not alias
 * any input or each other.  Built for dstate N in 1..64 and a channel count
 * that is a multiple of 8; other N and channel counts give
 * MAMBA_ERR_UNSUPPORTED (above 32 states the states are taken in groups of
 * 16, each group's share of du and ddelta summed in float32 before the
 * conversion to dtype).  dims->workspace must hold
 * mamba_scan_bwd_workspace_bytes() bytes; its contents need not be
 * initialised.  saved: NULL to recompute the forward states, or the buffer
 * mamba_scan_fwd_save wrote for these same inputs, dims and dir_mode (read
 * only; with z and dz it must hold the rows); the gradients are then the
 * same, bit for bit, and the recompute is skipped.  MAMBA_ERR_WORKSPACE when
 * saved is given with saved_bytes below mamba_scan_saved_bytes(dims, dir_mode,
 * z && dz) or is not 16-byte aligned.  Other errors as for mamba_scan_fwd.
 */
MAMBA_API int mamba_scan_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                             const float* D, const void* z, const float* delta_bias, const void* dout,
                             const mamba_dims* dims, int dir_mode, void* du, void* ddelta, float* dA, void* dB,
                             void* dC, float* dD, void* dz, float* ddelta_bias, float* dinit, const void* saved,
                             size_t saved_bytes, hipStream_t stream);

/* Static, human-readable text for a status code (never NULL). */
MAMBA_API const char* mamba_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_SCAN_H */
