// mamba_scan.hip -- C ABI of the gfx950 selective-scan library: argument
// validation and the launch plan.  The kernels live in scan_kernels.h, their
// launch code in scan_launch.h (instantiated by scan_inst.hip); the interface
// is documented in include/mamba_scan.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mamba_scan.h"
#include "conv_kernels.h"
#include "scan_launch.h"

#include <mutex>

using namespace mscan;

// Scratch of mamba_scan_fwd_noalloc: the workspace it would otherwise take from
// the caller (per-direction rows, time-split carries), as one static device
// array.  Each device the library runs on holds its own copy until the process
// ends.  In host code `scratch` names a host-side stand-in, not the device
// array: host code only ever uses the address that hipGetSymbolAddress returns
// for the device (scratch_of_stream below).
constexpr size_t kScratchBytes = MAMBA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mutex;
char* g_scratch[kScratchDevices];  // device address of `scratch` per device, once looked up

int num_dirs(int mode) { return mode == MAMBA_DIR_BIDIR ? 2 : mode == MAMBA_DIR_CROSS2D ? 4 : 1; }

// 2-bit traversal kind of each direction.
int kinds_of(int mode) {
  switch (mode) {
    case MAMBA_DIR_FWD: return KIND_ROW_FWD;
    case MAMBA_DIR_BWD: return KIND_ROW_REV;
    case MAMBA_DIR_BIDIR: return KIND_ROW_FWD | (KIND_ROW_REV << 2);
    default: return KIND_ROW_FWD | (KIND_COL_FWD << 2) | (KIND_ROW_REV << 4) | (KIND_COL_REV << 6);
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#ifndef MSCAN_FORCE_KERNEL
#define MSCAN_FORCE_KERNEL 0  // 1: the channel-block kernel wherever it applies, 2: the row kernel everywhere
#endif
#ifndef MSCAN_ROW_TARGET_WAVES
#define MSCAN_ROW_TARGET_WAVES 8192  // waves wanted from the row kernel's split (up to 16 states)
#endif
#ifndef MSCAN_ROW_MIN_CHUNK
#define MSCAN_ROW_MIN_CHUNK 256  // shortest time chunk of the row kernel's split
#endif

// Which forward kernel: scan_row_kernel (one channel per lane, every state in
// its registers) or scan_chunk_kernel (channel blocks with the states spread
// over lanes).  Only the row kernel takes state sizes that are not a power of
// two and channel counts that are not a multiple of 8.
bool choose_rows(const mamba_dims* g, int K) {
  const int64_t N = g->dstate;
  if ((N & (N - 1)) != 0 || g->dim % 8 != 0) return true;
  if (MSCAN_FORCE_KERNEL == 1) return false;
  if (MSCAN_FORCE_KERNEL == 2) return true;
  // The row kernel (rows of 64 channels, one wave each) also serves a single
  // direction whose channel blocks are too few to fill the GPU, where both
  // kernels split the sequence in time.  Measured on MI355X (row vs channel
  // block, µs): the 262k-token context 3997 vs 4150; elsewhere it loses --
  // 130M layer 253 vs 142, Vim-224 217 vs 208, 97k-token Vim 1322 vs 1253,
  // SS2D 910 vs 634.
  const int64_t blk_waves = (int64_t)K * g->batch * ((g->dim + 15) / 16) * (N < 4 ? 1 : N) / 4;
  return K == 1 && blk_waves < MSCAN_TARGET_WAVES / 2 && g->seqlen >= 2 * MSCAN_MIN_CHUNK;
}

// Launch plan of the row kernel: 64 channels per wave, split in time into
// enough chunks for ~MSCAN_TARGET_WAVES waves when the rows are fewer.
int plan_rows(const mamba_dims* g, int K, Plan* pl) {
  const int64_t L = g->seqlen, N = g->dstate;
  pl->row = 1;
  pl->tile = kTile;  // (unused by the row kernel)
  pl->cb = 64;
  pl->g = (int)N;
  pl->prio = 0;
  pl->nblk_d = (int)((g->dim + 63) / 64);
  const int64_t rows = (int64_t)K * g->batch * pl->nblk_d;
  // Up to 16 states the kernel fits 4 waves per SIMD (at most 119 VGPRs), and
  // the split aims at two rounds of 4 per SIMD.  Measured on MI355X with the
  // builds loaded side by side in one process, the 262k-token context in 96
  // chunks (3 waves per SIMD) 3997 µs, 128 (one round of 4) 3687-3709, 256
  // (two rounds) 3277-3307, 512 3774.  Larger states keep 3 per SIMD.
  const int64_t target = pl->np <= 16 ? MSCAN_ROW_TARGET_WAVES : MSCAN_TARGET_WAVES;
  int64_t nch = 1;
  if (rows < target) {
    nch = (target + rows - 1) / rows;
    if (nch > L / MSCAN_ROW_MIN_CHUNK) nch = L / MSCAN_ROW_MIN_CHUNK;
    if (nch > MSCAN_MAX_CHUNKS) nch = MSCAN_MAX_CHUNKS;
    if (nch < 1) nch = 1;
  }
  if (MSCAN_FORCE_CHUNKS > 0) nch = MSCAN_FORCE_CHUNKS < L ? MSCAN_FORCE_CHUNKS : L;
  const int64_t clen = (L + nch - 1) / nch;
  nch = (L + clen - 1) / clen;
  if (pl->nblk_d * nch * g->batch * K > INT32_MAX) return MAMBA_ERR_UNSUPPORTED;
  pl->nchunks = (int)nch;
  pl->chunk_len = (int)clen;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  pl->ws_y_bytes = K > 1 ? up((size_t)K * g->batch * L * g->dim * sizeof(float)) : 0;
  pl->agg_state_bytes = nch > 1 ? up((size_t)K * g->batch * (nch - 1) * g->dim * N * sizeof(float)) : 0;
  pl->agg_dsum_bytes = nch > 1 ? up((size_t)K * g->batch * (nch - 1) * g->dim * sizeof(float)) : 0;
  pl->bc_bytes = up(2 * ((size_t)K * g->batch * L + 2) * pl->np * sizeof(float));  // B, C: rows + 2 padding rows each
  return MAMBA_OK;
}

// Validates the sizes (no pointers) and derives the launch plan.  A pure
// function of dims and mode.
int make_plan(const mamba_dims* g, int mode, Plan* pl) {
  if (!g) return MAMBA_ERR_INVALID;
  if (mode < MAMBA_DIR_FWD || mode > MAMBA_DIR_CROSS2D) return MAMBA_ERR_INVALID;
  if (g->dtype != MAMBA_DTYPE_F32 && g->dtype != MAMBA_DTYPE_BF16) return MAMBA_ERR_INVALID;
  if (g->batch <= 0 || g->dim <= 0 || g->seqlen <= 0 || g->dstate <= 0) return MAMBA_ERR_INVALID;
  if (mode == MAMBA_DIR_CROSS2D &&
      (g->height <= 0 || g->width <= 0 || g->height > INT32_MAX || g->width > INT32_MAX ||
       g->height * g->width != g->seqlen))
    return MAMBA_ERR_INVALID;
  const int64_t N = g->dstate;
  if (N > 64) return MAMBA_ERR_UNSUPPORTED;
  if (g->dim % (g->dtype == MAMBA_DTYPE_BF16 ? 8 : 4) != 0) return MAMBA_ERR_UNSUPPORTED;
  const int K = num_dirs(mode);
  // token and grid indices are 32-bit inside the kernels; element offsets are 64-bit
  if (g->seqlen > INT32_MAX / 2 || g->dim > INT32_MAX / 2 || g->batch > INT32_MAX / 8 ||
      g->batch * g->dim > INT32_MAX / 4)
    return MAMBA_ERR_UNSUPPORTED;
  // token indices and token-row strides in bytes (up to 4 bytes per element)
  // are multiplied as 24-bit operands
  if (g->seqlen >= ((int64_t)1 << 24) || g->dim * 4 >= ((int64_t)1 << 24)) return MAMBA_ERR_UNSUPPORTED;
  // each (batch, direction) slice of L x D elements is addressed through a
  // buffer descriptor with 32-bit offsets (fp32 rows for several directions)
  const int64_t es = g->dtype == MAMBA_DTYPE_BF16 ? 2 : 4;
  // (64 rows of margin: prefetches past either end of the sequence must still
  // map to offsets outside the slice without wrapping)
  // (fp32 rows: at most 2^31 bytes per slice, so every offset stays below 2^31)
  if ((g->seqlen + 64) * g->dim * es > INT32_MAX || (K > 1 && g->seqlen * g->dim * 4 > ((int64_t)1 << 31)))
    return MAMBA_ERR_UNSUPPORTED;
  pl->K = K;
  pl->Ku = (mode == MAMBA_DIR_CROSS2D) ? 1 : K;
  // Layout and time split.  Waves wanted: MSCAN_TARGET_WAVES (3 per SIMD),
  // since one wave alone issues vector instructions at about half the SIMD rate.
  // Measured on MI355X: the 16-channel blocks beat the 64-channel ones at
  // every size tried once the wave priorities were in (N = 16: Vim-224
  // 239 -> 219 µs, a batch-32 130M-shaped layer 646 -> 491 µs; that layer at
  // N = 8: 306 -> 140 µs, at N = 4: 440 -> 148 µs), so every N >= 4 uses
  // them; N = 1 and 2 have only the 64-channel layout.  Rows short of waves
  // (long sequences with few rows) are split in time, the 16-channel layout
  // into enough chunks for ~24 waves per SIMD (32 -> 48 or 64 chunks: -2 to
  // -3 % on the long workloads).
  const int64_t L = g->seqlen;
  pl->np = 1;
  while (pl->np < N) pl->np *= 2;
  if (choose_rows(g, K)) return plan_rows(g, K, pl);
  pl->row = 0;
  pl->bc_bytes = 0;
  const int cb = layout_of((int)N).cb;
  const int64_t rows = (int64_t)K * g->batch * ((g->dim + cb - 1) / cb);
  // 2 states per thread at N = 16 when there are waves to spare, or when the
  // rows are so few that a time split supplies the waves (97k-token Vim:
  // 1290 -> 1257 µs; the 262k-token context unchanged)
  const int64_t waves1 = rows * (threads_of(16, 1) / 64);
  const bool split_needed = waves1 < MSCAN_TARGET_WAVES / 2 && L >= 2 * MSCAN_MIN_CHUNK;
  const int g16 = (N == 16 && (waves1 >= kG2Waves || split_needed)) ? 2 : 1;
  const int64_t waves = rows * (threads_of((int)N, g16) / 64);
  int64_t nch = 1;
  // Smaller state sizes have fewer waves per row and split into shorter
  // chunks: N = 1, 2 (64-channel blocks, one thread per channel) down to 128
  // positions (the 130M-shaped layer at N = 1: 370 -> 173 µs in 16 chunks;
  // 64- or 32-position chunks for 2 or 4 times the waves: 206 and 278 µs),
  // N = 4, 8 down to 256 (N = 4: 149 -> 139 µs); N >= 16 keeps 1024 (shorter
  // chunks cost the 97k-token Vim image and the long context 1.5-2 %).
  const int64_t min_chunk = cb == 64 ? 128 : N < 16 ? 256 : MSCAN_MIN_CHUNK;
  auto split = [&](int64_t target) {
    int64_t c = (target + waves - 1) / waves;
    if (c > L / min_chunk) c = L / min_chunk;
    if (c > MSCAN_MAX_CHUNKS) c = MSCAN_MAX_CHUNKS;
    return c < 1 ? (int64_t)1 : c;
  };
  if (waves < MSCAN_TARGET_WAVES / 2 && L >= 2 * min_chunk)
    nch = split(cb == 16 ? 8 * MSCAN_TARGET_WAVES : MSCAN_TARGET_WAVES);
  if (MSCAN_FORCE_CHUNKS > 0) nch = MSCAN_FORCE_CHUNKS < L ? MSCAN_FORCE_CHUNKS : L;
  if (nch < 1) nch = 1;
  pl->cb = cb;
  pl->g = layout_of((int)N, g16).g;
  // the scan loop's raised wave priority pays with few waves per SIMD and
  // costs with many (the kernel's priority note): below 16 per SIMD (a
  // batch-32 130M-shaped layer at 12: 478 µs with it, 482 without)
  pl->prio = waves * nch < 16 * 1024 ? 1 : 0;
  pl->nblk_d = (int)((g->dim + cb - 1) / cb);
  // 64-position tiles for one state per thread at N = 16 on sequences of
  // 1024 positions or more: half the barriers and per-tile work per position.
  // Measured on MI355X with the builds side by side in one process (µs): the
  // cross scan 595.5 -> 564.8, the 130M layer 133.9 -> 132.0; two states per
  // thread lose with them (Vim-224 189 -> 263, the 97k-token Vim 1157 ->
  // 1289), and short sequences would pad a larger share of their last tile.
  pl->tile = (N == 16 && g16 == 1 && L >= 1024) ? 2 * kTile : kTile;
  int64_t clen = (L + nch - 1) / nch;
  clen = (clen + pl->tile - 1) / pl->tile * pl->tile;
  nch = (L + clen - 1) / clen;
  if (pl->nblk_d * nch * g->batch * K > INT32_MAX) return MAMBA_ERR_UNSUPPORTED;
  pl->nchunks = (int)nch;
  pl->chunk_len = (int)clen;
  const size_t al = 256;
  auto up = [&](size_t x) { return (x + al - 1) / al * al; };
  pl->ws_y_bytes = K > 1 ? up((size_t)K * g->batch * L * g->dim * sizeof(float)) : 0;
  pl->agg_state_bytes = nch > 1 ? up((size_t)K * g->batch * (nch - 1) * g->dim * N * sizeof(float)) : 0;
  pl->agg_dsum_bytes = nch > 1 ? up((size_t)K * g->batch * (nch - 1) * g->dim * sizeof(float)) : 0;
  return MAMBA_OK;
}


// Workspace of the backward pass, in this order (each region 256-byte aligned):
// the forward recompute's time-split carries, the per-direction fp32 output
// rows, state checkpoints every 16 (N above 16: 32) positions, the per-channel-block partial
// sums of dB and dC, the per-direction du of the cross scan, the per-chunk
// and per-batch partial sums of dA, dD and ddelta_bias, and the adjoint's
// time-split carries.
constexpr int kBwdBlock = 16;     // channels per workgroup of scan_bwd_kernel
constexpr int kBwdSlots = 512;    // adjoint workgroups resident at once (2 per CU; 1 at N = 32)
#ifndef MSCAN_BWD_SLOTS16
#define MSCAN_BWD_SLOTS16 1024  // the same with 16 thread rows (4 waves per SIMD: 4 per CU)
#endif
constexpr int kBwdMinChunk = 1024;  // shortest time chunk of a split adjoint
constexpr int kBwdGroup = 16;     // states per group above 32 states
struct BwdPlan {
  Plan fwd;
  int nblk, ntiles, every, nchunks, chunk_len, ngroups;
  size_t agg, ws_y, ckpt, dB, dC, du, ddelta, dA, dD, dbias, bagg_S, bagg_dsum, total;
};

int make_bwd_plan(const mamba_dims* g, int mode, BwdPlan* bp) {
  const int rc = make_plan(g, mode, &bp->fwd);
  if (rc != MAMBA_OK) return rc;
  // one state per thread (16 channels x N states per workgroup, N rounded up
  // to a power of two, at most 512 threads; above 32 states, groups of 16
  // states in workgroups of their own) and checkpoints at multiples of the
  // tile
  if (g->dstate > 64 || kTile != 32) return MAMBA_ERR_UNSUPPORTED;
  // the per-element kernels of the backward (dz of several directions, the
  // sums) take 8 consecutive channels per thread
  if (g->dim % 8 != 0) return MAMBA_ERR_UNSUPPORTED;
  // the recompute always keeps per-direction fp32 rows (32-bit slice offsets)
  if (g->seqlen * g->dim * 4 > ((int64_t)1 << 31)) return MAMBA_ERR_UNSUPPORTED;
  const Plan& pl = bp->fwd;
  const int64_t K = pl.K, Bz = g->batch, L = g->seqlen, Dm = g->dim, N = g->dstate;
  bp->nblk = (int)((Dm + kBwdBlock - 1) / kBwdBlock);
  // state groups: above 32 states, workgroups of 16 states each (the sums over
  // states of a channel's gradients are then summed over the groups)
  const int64_t G = N > 32 ? (N + kBwdGroup - 1) / kBwdGroup : 1;
  bp->ngroups = (int)G;
  // checkpoint interval = the adjoint's segment: 16 positions, 32 for 17..32
  // states (the adjoint kernel's segment for 32 thread rows)
  bp->every = (N > 16 && G == 1) ? 32 : 16;
  bp->ntiles = (int)((L + bp->every - 1) / bp->every);
  // Time split of the adjoint when its rows fill less than one round of
  // workgroups: up to two rounds, chunks of at least kBwdMinChunk positions.
  const int64_t rows = (int64_t)bp->nblk * Bz * K * G;
  // Split below half a round of 16-thread-row workgroups (4 per CU since the
  // adjoint's 4-wave budget), into chunks for two rounds.  Measured on MI355X
  // with the builds side by side in one process: two rounds of 1024 instead
  // of 512 slots, the 97k-token Vim's backward 5239 -> 4479 µs, the 262k-token
  // context's 17271 -> 16824; splitting the 130M layer's 768 rows (2 chunks)
  // 544 -> 623, so it stays unsplit.
  const int64_t slots = (N > 16 && G == 1) ? kBwdSlots / 2 : (N > 8 ? MSCAN_BWD_SLOTS16 : kBwdSlots);
  const int64_t split_below = (N > 16 && G == 1) ? kBwdSlots / 2 : kBwdSlots;
  int64_t nch = 1;
  if (rows < split_below) {
    nch = (2 * slots + rows - 1) / rows;
    if (nch > L / kBwdMinChunk) nch = L / kBwdMinChunk;
    if (nch > 256) nch = 256;
    if (nch < 1) nch = 1;
  }
  int64_t clen = (L + nch - 1) / nch;
  clen = (clen + kTile - 1) / kTile * kTile;
  nch = (L + clen - 1) / clen;
  bp->nchunks = (int)nch;
  bp->chunk_len = (int)clen;
  if (rows * nch > INT32_MAX) return MAMBA_ERR_UNSUPPORTED;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t f4 = sizeof(float);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += up(bytes);
    return at;
  };
  bp->agg = take(pl.agg_state_bytes + pl.agg_dsum_bytes + pl.bc_bytes);
  bp->ws_y = take((size_t)K * Bz * L * Dm * f4);
  bp->ckpt = take((size_t)K * Bz * bp->ntiles * Dm * N * f4);
  bp->dB = take((size_t)bp->nblk * Bz * K * L * N * f4);
  bp->dC = take((size_t)bp->nblk * Bz * K * L * N * f4);
  // du and ddelta in fp32 parts: du of the cross scan per direction (its u is
  // shared), both per state group with groups
  bp->du = (pl.Ku != K || G > 1) ? take((size_t)G * K * Bz * L * Dm * f4) : off;
  bp->ddelta = G > 1 ? take((size_t)G * K * Bz * L * Dm * f4) : off;
  bp->dA = take((size_t)nch * Bz * K * Dm * N * f4);
  bp->dD = take((size_t)G * nch * Bz * K * Dm * f4);
  bp->dbias = take((size_t)G * nch * Bz * K * Dm * f4);
  bp->bagg_S = take((size_t)K * Bz * (nch - 1) * Dm * N * f4);
  bp->bagg_dsum = take((size_t)K * Bz * (nch - 1) * Dm * f4);
  bp->total = off;
  return MAMBA_OK;
}

template <typename TIn>
int launch_bwd_dz(const float* ws_y, const void* z, const void* dout, void* dz, int K, int64_t n,
                  hipStream_t stream) {
  const unsigned blocks = (unsigned)((n / 8 + 255) / 256);
  hipLaunchKernelGGL((bwd_dz_kernel<TIn>), dim3(blocks), dim3(256), 0, stream, ws_y, static_cast<const TIn*>(z),
                     static_cast<const TIn*>(dout), static_cast<TIn*>(dz), K, n);
  return hipGetLastError() == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

// Sums over packed partial slices (stride == n at every call); a second
// (in1, out1) pair of the same shape, if given, shares the launch.
template <typename TOut>
int launch_bwd_sum(const float* in, int64_t nslices, int64_t stride, int64_t n, void* out, hipStream_t stream,
                   const float* in1 = nullptr, void* out1 = nullptr) {
  const unsigned pairs = in1 ? 2u : 1u;
  TOut* o0 = static_cast<TOut*>(out);
  TOut* o1 = static_cast<TOut*>(in1 ? out1 : out);
  if (n % 4 == 0 && stride % 4 == 0) {
    const unsigned blocks = (unsigned)((n / 4 + 255) / 256);
    hipLaunchKernelGGL((bwd_sum_kernel<TOut, 4>), dim3(blocks, pairs), dim3(256), 0, stream, in, o0,
                       in1 ? in1 : in, o1, nslices, stride, n);
  } else {
    const unsigned blocks = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL((bwd_sum_kernel<TOut, 1>), dim3(blocks, pairs), dim3(256), 0, stream, in, o0,
                       in1 ? in1 : in, o1, nslices, stride, n);
  }
  return hipGetLastError() == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}


#ifndef MSCAN_CONV_RUN
#define MSCAN_CONV_RUN 16
#endif
constexpr int kConvRun = MSCAN_CONV_RUN;  // positions per thread of the Conv1d kernel

template <typename TIn, int W>
int launch_conv(const ConvParams& p, hipStream_t stream) {
  const int64_t threads = (int64_t)p.Bsz * ((p.L + kConvRun - 1) / kConvRun) * (p.Dm / 8);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  hipLaunchKernelGGL((conv1d_silu_kernel<TIn, W, kConvRun>), dim3(blocks), dim3(256), 0, stream, p);
  return hipGetLastError() == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

template <typename TIn>
int dispatch_conv(int width, const ConvParams& p, hipStream_t stream) {
  switch (width) {
    case 1: return launch_conv<TIn, 1>(p, stream);
    case 2: return launch_conv<TIn, 2>(p, stream);
    case 3: return launch_conv<TIn, 3>(p, stream);
    case 4: return launch_conv<TIn, 4>(p, stream);
    default: return MAMBA_ERR_UNSUPPORTED;
  }
}

// ScanParams of a forward pass over these dims (the output, workspace and
// checkpoint pointers are set by the caller).
ScanParams scan_params(const void* u, const void* delta, const float* A, const void* B, const void* C,
                       const float* D, const void* z, const float* delta_bias, const mamba_dims* dims,
                       int dir_mode, const Plan& pl) {
  ScanParams p{};
  p.u = u;
  p.delta = delta;
  p.A = A;
  p.B = B;
  p.C = C;
  p.D = D;
  p.z = z;
  p.delta_bias = delta_bias;
  p.init_state = dims->initial_state;
  p.Bsz = (int)dims->batch;
  p.Dm = (int)dims->dim;
  p.L = (int)dims->seqlen;
  p.H = dir_mode == MAMBA_DIR_CROSS2D ? (int)dims->height : 1;
  p.W = dir_mode == MAMBA_DIR_CROSS2D ? (int)dims->width : (int)dims->seqlen;
  p.N = (int)dims->dstate;
  p.K = pl.K;
  p.Ku = pl.Ku;
  p.kinds = kinds_of(dir_mode);
  p.nchunks = pl.nchunks;
  p.chunk_len = pl.chunk_len;
  p.nblk_d = pl.nblk_d;
  p.softplus = dims->delta_softplus ? 1 : 0;
  return p;
}

int dispatch_fwd(const mamba_dims* dims, const ScanParams& p, const Plan& pl, hipStream_t stream) {
  const bool exact = dims->exact_zoh != 0;
  if (pl.row) {
    if (dims->dtype == MAMBA_DTYPE_BF16)
      return exact ? dispatch_rows_bf16_exact(p, pl, stream) : dispatch_rows_bf16_simple(p, pl, stream);
    return exact ? dispatch_rows_f32_exact(p, pl, stream) : dispatch_rows_f32_simple(p, pl, stream);
  }
  if (dims->dtype == MAMBA_DTYPE_BF16)
    return exact ? dispatch_scan_bf16_exact(dims->dstate, p, pl, stream)
                 : dispatch_scan_bf16_simple(dims->dstate, p, pl, stream);
  return exact ? dispatch_scan_f32_exact(dims->dstate, p, pl, stream)
               : dispatch_scan_f32_simple(dims->dstate, p, pl, stream);
}

// Saved forward state (mamba_scan_fwd_save -> mamba_scan_bwd): the state
// before every 16th position (32nd at 17..32 states), [K][B][ntiles][D][N] fp32, then, for a
// gated scan, the ungated per-direction rows [K][B][L][D] fp32 (dz needs them).
struct SavedLayout {
  BwdPlan bp;
  size_t rows, total;
};

int saved_layout(const mamba_dims* g, int mode, bool rows, SavedLayout* s) {
  const int rc = make_bwd_plan(g, mode, &s->bp);
  if (rc != MAMBA_OK) return rc;
  const size_t f4 = sizeof(float);
  const int64_t K = s->bp.fwd.K;
  const size_t ck = ((size_t)K * g->batch * s->bp.ntiles * g->dim * g->dstate * f4 + 255) / 256 * 256;
  s->rows = ck;
  s->total = ck + (rows ? (size_t)K * g->batch * g->seqlen * g->dim * f4 : 0);
  return MAMBA_OK;
}

// Points the forward pass's scratch regions into a workspace laid out as Plan
// describes: the per-direction rows at ws (when rows is true), the other
// regions from rest on (ws + pl.ws_y_bytes in a whole forward workspace).
void set_workspace(ScanParams* p, const Plan& pl, char* ws, bool rows, char* rest) {
  if (rows) p->ws_y = pl.ws_y_bytes ? reinterpret_cast<float*>(ws) : nullptr;
  char* w = rest;
  size_t off = 0;
  p->agg_state = pl.agg_state_bytes ? reinterpret_cast<float*>(w + off) : nullptr;
  off += pl.agg_state_bytes;
  p->agg_dsum = pl.agg_dsum_bytes ? reinterpret_cast<float*>(w + off) : nullptr;
  off += pl.agg_dsum_bytes;
  p->bcw = pl.bc_bytes ? reinterpret_cast<float*>(w + off) : nullptr;
}

// Validation shared by the forward entry points (pointers, alignment, plan).
int check_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C, const float* D,
              const void* z, const float* delta_bias, const mamba_dims* dims, int dir_mode, const void* out,
              const float* last_state, Plan* pl) {
  const int rc = make_plan(dims, dir_mode, pl);
  if (rc != MAMBA_OK) return rc;
  if (!u || !delta || !A || !B || !C || !out) return MAMBA_ERR_INVALID;
  const void* ptrs[] = {u, delta, A, B, C, D, z, delta_bias, out, last_state, dims->initial_state};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return MAMBA_ERR_UNSUPPORTED;
  return MAMBA_OK;
}

// The forward pass with its workspace at ws (pl.total() bytes, or none).
int run_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C, const float* D,
            const void* z, const float* delta_bias, const mamba_dims* dims, int dir_mode, void* out,
            float* last_state, const Plan& pl, char* ws, hipStream_t stream) {
  ScanParams p = scan_params(u, delta, A, B, C, D, z, delta_bias, dims, dir_mode, pl);
  p.out = out;
  set_workspace(&p, pl, ws, true, ws + pl.ws_y_bytes);
  p.last_state = last_state;
  p.fold = 1;  // the per-direction rows are not kept: the last direction may sum them
  return dispatch_fwd(dims, p, pl, stream);
}

// Device address of the static scratch on the device of `stream` (the
// current device for the null stream), looked up once per device with that
// device current and kept for the life of the process.
int scratch_of_stream(hipStream_t stream, char** out) {
  int dev = -1;
  if (stream != nullptr) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return MAMBA_ERR_HIP;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return MAMBA_ERR_HIP;
  }
  if (dev < 0 || dev >= kScratchDevices) return MAMBA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return MAMBA_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return MAMBA_ERR_HIP;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return MAMBA_ERR_HIP;
    if (e != hipSuccess || ptr == nullptr) return MAMBA_ERR_HIP;
    g_scratch[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch[dev];
  return MAMBA_OK;
}

}  // namespace

extern "C" {

size_t mamba_scan_fwd_workspace_bytes(const mamba_dims* dims, int dir_mode) {
  Plan pl;
  if (make_plan(dims, dir_mode, &pl) != MAMBA_OK) return (size_t)-1;
  return pl.total();
}

int mamba_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                   const float* D, const void* z, const float* delta_bias, const mamba_dims* dims,
                   int dir_mode, void* out, float* last_state, hipStream_t stream) {
  Plan pl;
  const int rc = check_fwd(u, delta, A, B, C, D, z, delta_bias, dims, dir_mode, out, last_state, &pl);
  if (rc != MAMBA_OK) return rc;
  const size_t need = pl.total();
  if (need > 0 && (!dims->workspace || dims->workspace_bytes < need || !aligned16(dims->workspace)))
    return MAMBA_ERR_WORKSPACE;
  return run_fwd(u, delta, A, B, C, D, z, delta_bias, dims, dir_mode, out, last_state, pl,
                 static_cast<char*>(dims->workspace), stream);
}

int mamba_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B, const void* C,
                           const float* D, const void* z, const float* delta_bias, const mamba_dims* dims,
                           int dir_mode, void* out, float* last_state, hipStream_t stream) {
  Plan pl;
  int rc = check_fwd(u, delta, A, B, C, D, z, delta_bias, dims, dir_mode, out, last_state, &pl);
  if (rc != MAMBA_OK) return rc;
  const size_t need = pl.total();
  if (need > kScratchBytes) return MAMBA_ERR_SCRATCH;
  char* ws = nullptr;
  if (need > 0) {
    rc = scratch_of_stream(stream, &ws);
    if (rc != MAMBA_OK) return rc;
  }
  return run_fwd(u, delta, A, B, C, D, z, delta_bias, dims, dir_mode, out, last_state, pl, ws, stream);
}

size_t mamba_scan_saved_bytes(const mamba_dims* dims, int dir_mode, int gated) {
  SavedLayout sl;
  if (saved_layout(dims, dir_mode, gated != 0, &sl) != MAMBA_OK) return (size_t)-1;
  return sl.total;
}

int mamba_scan_fwd_save(const void* u, const void* delta, const float* A, const void* B, const void* C,
                        const float* D, const void* z, const float* delta_bias, const mamba_dims* dims,
                        int dir_mode, void* out, float* last_state, void* saved, size_t saved_bytes,
                        hipStream_t stream) {
  SavedLayout sl;
  int rc = saved_layout(dims, dir_mode, z != nullptr, &sl);
  if (rc != MAMBA_OK) return rc;
  const Plan& pl = sl.bp.fwd;
  if (!u || !delta || !A || !B || !C || !out || !saved) return MAMBA_ERR_INVALID;
  const void* ptrs[] = {u, delta, A, B, C, D, z, delta_bias, out, last_state, dims->initial_state, saved};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return MAMBA_ERR_UNSUPPORTED;
  if (saved_bytes < sl.total) return MAMBA_ERR_WORKSPACE;
  const size_t need = pl.total();
  if (need > 0 && (!dims->workspace || dims->workspace_bytes < need || !aligned16(dims->workspace)))
    return MAMBA_ERR_WORKSPACE;

  ScanParams p = scan_params(u, delta, A, B, C, D, z, delta_bias, dims, dir_mode, pl);
  p.out = out;
  char* ws = static_cast<char*>(dims->workspace);
  char* sv = static_cast<char*>(saved);
  // gated: the per-direction rows go to the saved buffer (the merge reads
  // them there); ungated with several directions: to the workspace as usual
  set_workspace(&p, pl, ws, true, ws + pl.ws_y_bytes);
  if (z) p.ws_y = reinterpret_cast<float*>(sv + sl.rows);
  p.last_state = last_state;
  p.ckpt = reinterpret_cast<float*>(sv);
  p.ckpt_tiles = sl.bp.ntiles;
  p.ckpt_every = sl.bp.every;
  return dispatch_fwd(dims, p, pl, stream);
}

size_t mamba_scan_bwd_workspace_bytes(const mamba_dims* dims, int dir_mode) {
  BwdPlan bp;
  if (make_bwd_plan(dims, dir_mode, &bp) != MAMBA_OK) return (size_t)-1;
  return bp.total;
}

int mamba_scan_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                   const float* D, const void* z, const float* delta_bias, const void* dout,
                   const mamba_dims* dims, int dir_mode, void* du, void* ddelta, float* dA, void* dB, void* dC,
                   float* dD, void* dz, float* ddelta_bias, float* dinit, const void* saved,
                   size_t saved_bytes, hipStream_t stream) {
  SavedLayout sl;
  int rc = saved_layout(dims, dir_mode, z && dz, &sl);
  if (rc != MAMBA_OK) return rc;
  const BwdPlan& bp = sl.bp;
  if (saved && (saved_bytes < sl.total || !aligned16(saved))) return MAMBA_ERR_WORKSPACE;
  if (!u || !delta || !A || !B || !C || !dout || !du || !ddelta || !dA || !dB || !dC) return MAMBA_ERR_INVALID;
  const void* ptrs[] = {u, delta, A, B, C, D, z, delta_bias, dout, du, ddelta, dA, dB, dC, dD, dz,
                        ddelta_bias, dinit, dims->initial_state};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return MAMBA_ERR_UNSUPPORTED;
  if (!dims->workspace || dims->workspace_bytes < bp.total || !aligned16(dims->workspace))
    return MAMBA_ERR_WORKSPACE;
  const Plan& pl = bp.fwd;
  char* ws = static_cast<char*>(dims->workspace);
  auto wsf = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  const bool bf16 = dims->dtype == MAMBA_DTYPE_BF16;
  const bool exact = dims->exact_zoh != 0;
  const int64_t N = dims->dstate;

  // 1. state checkpoints (and, for dz, the per-direction fp32 output rows):
  // from the saved forward state, else by a forward recompute
  ScanParams p = scan_params(u, delta, A, B, C, D, z, delta_bias, dims, dir_mode, pl);
  if (saved) {
    p.ckpt = reinterpret_cast<float*>(const_cast<void*>(saved));
    p.ws_y = (z && dz) ? reinterpret_cast<float*>(static_cast<char*>(const_cast<void*>(saved)) + sl.rows) : nullptr;
  } else {
    p.out = nullptr;
    p.ws_y = (z && dz) ? wsf(bp.ws_y) : nullptr;  // the rows serve dz alone
    // the forward plan's split carries and B/C copies at bp.agg (its rows
    // region, unused here, is left out of the reservation)
    set_workspace(&p, pl, nullptr, false, ws + bp.agg);
    p.last_state = nullptr;
    p.ckpt = wsf(bp.ckpt);
    p.ckpt_tiles = bp.ntiles;
    p.ckpt_every = bp.every;
    rc = dispatch_fwd(dims, p, pl, stream);
    if (rc != MAMBA_OK) return rc;
  }

  // 2. dz of several directions (it needs their sum; with one direction the
  // reverse sweep writes dz while staging)
  const int64_t nrow = dims->batch * dims->seqlen * dims->dim;
  const bool dz_here = z && dz && pl.K == 1;
  if (z && dz && !dz_here) {
    rc = bf16 ? launch_bwd_dz<uint16_t>(p.ws_y, z, dout, dz, pl.K, nrow, stream)
              : launch_bwd_dz<float>(p.ws_y, z, dout, dz, pl.K, nrow, stream);
    if (rc != MAMBA_OK) return rc;
  }

  // 3. the reverse sweep (dy = dout·silu(z) computed while staging)
  BwdParams q{};
  q.u = u;
  q.delta = delta;
  q.A = A;
  q.B = B;
  q.C = C;
  q.D = D;
  q.delta_bias = delta_bias;
  q.ckpt = p.ckpt;
  q.dout = dout;
  q.z = z;
  q.ws_y = p.ws_y;
  q.dz = dz_here ? dz : nullptr;
  q.dz_here = dz_here ? 1 : 0;
  const bool shared_u = pl.Ku != pl.K;
  const bool groups = bp.ngroups > 1;
  q.du = (shared_u || groups) ? nullptr : du;
  q.du_part = (shared_u || groups) ? wsf(bp.du) : nullptr;
  q.ddelta = ddelta;
  q.ddelta_part = groups ? wsf(bp.ddelta) : nullptr;
  q.ngroups = bp.ngroups;
  q.dB_part = wsf(bp.dB);
  q.dC_part = wsf(bp.dC);
  q.dA_part = wsf(bp.dA);
  q.dD_part = wsf(bp.dD);
  q.dbias_part = wsf(bp.dbias);
  q.dinit = dinit;
  q.Bsz = p.Bsz;
  q.Dm = p.Dm;
  q.L = p.L;
  q.H = p.H;
  q.W = p.W;
  q.K = p.K;
  q.Ku = p.Ku;
  q.kinds = p.kinds;
  q.nblk_d = bp.nblk;
  q.ntiles = bp.ntiles;
  q.nchunks = bp.nchunks;
  q.chunk_len = bp.chunk_len;
  q.agg_S = wsf(bp.bagg_S);
  q.agg_dsum = wsf(bp.bagg_dsum);
  q.softplus = p.softplus;
  q.N = (int)dims->dstate;
  rc = bf16 ? (exact ? dispatch_bwd_bf16_exact(N, q, stream) : dispatch_bwd_bf16_simple(N, q, stream))
            : (exact ? dispatch_bwd_f32_exact(N, q, stream) : dispatch_bwd_f32_simple(N, q, stream));
  if (rc != MAMBA_OK) return rc;

  // 4. sums over channel blocks (dB, dC), directions (du of the cross scan),
  // state groups (du, ddelta) and batches (dA, dD, ddelta_bias)
  const int64_t K = pl.K, Bz = dims->batch, Dm = dims->dim, G = bp.ngroups;
  const int64_t nbc = Bz * K * dims->seqlen * N;
  // du parts: [G][K] slices of [B][L][D] (shared u) or [G] slices of [B][K][L][D]
  const int64_t du_sl = shared_u ? G * K : G, du_n = shared_u ? nrow : nrow * K;
  if (bf16) {
    rc = launch_bwd_sum<uint16_t>(q.dB_part, bp.nblk, nbc, nbc, dB, stream, q.dC_part, dC);
    if (rc == MAMBA_OK && (shared_u || groups)) rc = launch_bwd_sum<uint16_t>(q.du_part, du_sl, du_n, du_n, du, stream);
    if (rc == MAMBA_OK && groups) rc = launch_bwd_sum<uint16_t>(q.ddelta_part, G, nrow * K, nrow * K, ddelta, stream);
  } else {
    rc = launch_bwd_sum<float>(q.dB_part, bp.nblk, nbc, nbc, dB, stream, q.dC_part, dC);
    if (rc == MAMBA_OK && (shared_u || groups)) rc = launch_bwd_sum<float>(q.du_part, du_sl, du_n, du_n, du, stream);
    if (rc == MAMBA_OK && groups) rc = launch_bwd_sum<float>(q.ddelta_part, G, nrow * K, nrow * K, ddelta, stream);
  }
  // (the dA parts are [chunk][batch][K][...]: one slice per (chunk, batch); the
  // dD and ddelta_bias parts [group][chunk][batch][K][...])
  const int64_t nsl = (int64_t)bp.nchunks * Bz;
  const int64_t nsl_g = G * nsl;
  if (rc == MAMBA_OK) rc = launch_bwd_sum<float>(q.dA_part, nsl, K * Dm * N, K * Dm * N, dA, stream);
  if (rc == MAMBA_OK && dD && ddelta_bias)
    rc = launch_bwd_sum<float>(q.dD_part, nsl_g, K * Dm, K * Dm, dD, stream, q.dbias_part, ddelta_bias);
  else if (rc == MAMBA_OK && dD)
    rc = launch_bwd_sum<float>(q.dD_part, nsl_g, K * Dm, K * Dm, dD, stream);
  else if (rc == MAMBA_OK && ddelta_bias)
    rc = launch_bwd_sum<float>(q.dbias_part, nsl_g, K * Dm, K * Dm, ddelta_bias, stream);
  return rc;
}

int mamba_scan_step(float* state, const void* u_t, const void* delta_t, const float* A, const void* B_t,
                    const void* C_t, const float* D, const void* z_t, const float* delta_bias,
                    const mamba_dims* dims, void* out, hipStream_t stream) {
  if (!dims || !state || !u_t || !delta_t || !A || !B_t || !C_t || !out) return MAMBA_ERR_INVALID;
  if (dims->dtype != MAMBA_DTYPE_F32 && dims->dtype != MAMBA_DTYPE_BF16) return MAMBA_ERR_INVALID;
  if (dims->batch <= 0 || dims->dim <= 0 || dims->dstate <= 0) return MAMBA_ERR_INVALID;
  const int64_t N = dims->dstate;
  if (N > 64) return MAMBA_ERR_UNSUPPORTED;
  if (dims->dim % (dims->dtype == MAMBA_DTYPE_BF16 ? 8 : 4) != 0 || dims->batch * dims->dim > INT32_MAX / 64)
    return MAMBA_ERR_UNSUPPORTED;
  const void* ptrs[] = {state, u_t, delta_t, A, B_t, C_t, D, z_t, delta_bias, out};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return MAMBA_ERR_UNSUPPORTED;
  StepParams p{state, u_t, delta_t, A, B_t, C_t, D, z_t, delta_bias, out,
               (int)dims->batch, (int)dims->dim, dims->delta_softplus ? 1 : 0};
  const bool exact = dims->exact_zoh != 0;
  if (dims->dtype == MAMBA_DTYPE_BF16)
    return exact ? dispatch_step_bf16_exact(N, p, stream) : dispatch_step_bf16_simple(N, p, stream);
  return exact ? dispatch_step_f32_exact(N, p, stream) : dispatch_step_f32_simple(N, p, stream);
}

int mamba_conv1d_silu(const void* x, const float* weight, const float* bias, const mamba_dims* dims, int width,
                      int reverse, void* out, hipStream_t stream) {
  if (!dims || !x || !weight || !out) return MAMBA_ERR_INVALID;
  if (dims->dtype != MAMBA_DTYPE_F32 && dims->dtype != MAMBA_DTYPE_BF16) return MAMBA_ERR_INVALID;
  if (dims->batch <= 0 || dims->dim <= 0 || dims->seqlen <= 0 || width <= 0) return MAMBA_ERR_INVALID;
  if (width > 4 || dims->dim % 8 != 0) return MAMBA_ERR_UNSUPPORTED;
  if (dims->seqlen > INT32_MAX / 2 || dims->dim > INT32_MAX / 2 || dims->batch > INT32_MAX / 2 ||
      dims->batch * ((dims->seqlen + kConvRun - 1) / kConvRun) * (dims->dim / 8) > (int64_t)INT32_MAX * 64)
    return MAMBA_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(out) || ((uintptr_t)weight & 3u) || (bias && ((uintptr_t)bias & 3u)))
    return MAMBA_ERR_UNSUPPORTED;
  ConvParams p{x, weight, bias, out, (int)dims->batch, (int)dims->seqlen, (int)dims->dim, reverse ? 1 : 0};
  if (dims->dtype == MAMBA_DTYPE_BF16) return dispatch_conv<uint16_t>(width, p, stream);
  return dispatch_conv<float>(width, p, stream);
}

const char* mamba_status_string(int status) {
  switch (status) {
    case MAMBA_OK: return "ok";
    case MAMBA_ERR_INVALID: return "invalid argument (null pointer, non-positive size, L != H*W, or unknown mode/dtype)";
    case MAMBA_ERR_UNSUPPORTED: return "unsupported (state size, channel count, alignment or size limit)";
    case MAMBA_ERR_WORKSPACE: return "workspace missing or smaller than the *_workspace_bytes() figure";
    case MAMBA_ERR_HIP: return "HIP runtime rejected a kernel launch";
    case MAMBA_ERR_SCRATCH: return "mamba_scan_fwd_noalloc: the problem needs more than the library's 32 MiB static scratch";
    default: return "unknown status";
  }
}

}  // extern "C"
