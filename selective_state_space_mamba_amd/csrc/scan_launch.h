// scan_launch.h -- launch plan types and the templated launch code of the
// selective-scan kernels.  The kernel instantiations are spread over several
// translation units (scan_inst.hip, compiled once per element type and
// input-term rule) that export the dispatch functions declared at the end.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mamba_scan.h"
#include "scan_bwd.h"
#include "scan_kernels.h"

namespace mscan {


#ifndef MSCAN_TILE
#define MSCAN_TILE 32
#endif
inline constexpr int kTile = MSCAN_TILE;  // scan positions per LDS tile

#ifndef MSCAN_TARGET_WAVES
#define MSCAN_TARGET_WAVES 3072  // resident waves wanted: 3 per SIMD (one wave issues VALU at half rate)
#endif
#ifndef MSCAN_FORCE_CHUNKS
#define MSCAN_FORCE_CHUNKS 0
#endif
#ifndef MSCAN_MIN_CHUNK
#define MSCAN_MIN_CHUNK 1024     // shortest time chunk worth a separate aggregate pass
#endif
#ifndef MSCAN_MAX_CHUNKS
#define MSCAN_MAX_CHUNKS 256
#endif

// Workgroup layouts: CB channels per workgroup, G states per thread,
// CB*N/G threads.  State sizes from 4 up use 16-channel blocks with one state
// per thread (N/16 from N = 16 on, at most 4), whose waves hold 4 state rows
// of the same 16 channels; N = 1 and 2, which cannot fill a wave that way,
// use 64-channel blocks with all N states in each thread.  At N = 16 a
// problem with many rows takes 2 states per thread instead (kG2Waves).
struct Layout {
  int cb, g;
};
inline constexpr Layout layout_of(int N, int g16 = 1) {
  return N < 4 ? Layout{64, N} : N == 16 ? Layout{16, g16} : Layout{16, N < 16 ? 1 : N / 16};
}
inline constexpr int threads_of(int N, int g16 = 1) { return layout_of(N, g16).cb * N / layout_of(N, g16).g; }
// Measured on MI355X (130M-shaped layers, Vim-224): 2 states per thread at
// N = 16 win once 1 state per thread would give 24 or more waves per SIMD
// (batch 64: 942 -> 910 µs; Vim-224: 220 -> 210 µs) and lose below 12
// (batch 32: 482 -> 497; the 130M layer at 3 waves per SIMD: 140 -> 180).
inline constexpr int64_t kG2Waves = 16 * 1024;

struct Plan {
  int K, Ku, cb, g, nblk_d, nchunks, chunk_len, prio;
  size_t ws_y_bytes, agg_state_bytes, agg_dsum_bytes;
  size_t total() const { return ws_y_bytes + agg_state_bytes + agg_dsum_bytes; }
};


// Dispatchers exported by the instantiation units: N is the state size, the
// suffix the element type (bf16 / f32) and the input-term rule (exact
// zero-order hold or Δ·B·u).
#define MSCAN_DECLARE_DISPATCH(SUFFIX)                                                        \
  int dispatch_scan_##SUFFIX(int64_t N, const ScanParams& p, const Plan& pl, hipStream_t s); \
  int dispatch_step_##SUFFIX(int64_t N, const StepParams& p, hipStream_t s);              \
  int dispatch_bwd_##SUFFIX(int64_t N, const BwdParams& p, hipStream_t s);
MSCAN_DECLARE_DISPATCH(bf16_simple)
MSCAN_DECLARE_DISPATCH(bf16_exact)
MSCAN_DECLARE_DISPATCH(f32_simple)
MSCAN_DECLARE_DISPATCH(f32_exact)

#ifdef MSCAN_INSTANTIATE
template <typename TIn, int N, int G16, bool EXACT>
int launch_chunks(ScanParams p, const Plan& pl, hipStream_t stream) {
  constexpr Layout lay = layout_of(N, G16);
  constexpr int NT = threads_of(N, G16);
  if (pl.nchunks > 1) {
    p.grid_chunks = pl.nchunks - 1;
    p.prio = pl.prio;
    const unsigned blocks = (unsigned)(pl.nblk_d * p.grid_chunks * p.Bsz * p.K);
    hipLaunchKernelGGL((scan_chunk_kernel<TIn, N, lay.g, lay.cb, kTile, true, EXACT>), dim3(blocks), dim3(NT), 0, stream, p);
    if (hipGetLastError() != hipSuccess) return MAMBA_ERR_HIP;
  }
  p.grid_chunks = pl.nchunks;
  const unsigned blocks = (unsigned)(pl.nblk_d * p.grid_chunks * p.Bsz * p.K);
  p.prio = pl.prio;
  hipLaunchKernelGGL((scan_chunk_kernel<TIn, N, lay.g, lay.cb, kTile, false, EXACT>), dim3(blocks), dim3(NT), 0, stream, p);
  return hipGetLastError() == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

template <typename TIn, int N, bool EXACT>
int launch_scan(const ScanParams& p, const Plan& pl, hipStream_t stream) {
  int rc;
  if constexpr (N == 16) {
    rc = pl.g == 2 ? launch_chunks<TIn, N, 2, EXACT>(p, pl, stream) : launch_chunks<TIn, N, 1, EXACT>(p, pl, stream);
  } else {
    rc = launch_chunks<TIn, N, 1, EXACT>(p, pl, stream);
  }
  if (rc != MAMBA_OK) return rc;
  if (p.ws_y && p.out && p.K > 1) {  // (with one direction the scan wrote out itself)
    const int64_t rows8 = (int64_t)p.Bsz * p.L * p.Dm / 8;
    const unsigned mblocks = (unsigned)((rows8 + 255) / 256);
    hipLaunchKernelGGL((merge_dirs_kernel<TIn>), dim3(mblocks), dim3(256), 0, stream, p.ws_y,
                       static_cast<const TIn*>(p.z), static_cast<TIn*>(p.out), p.K, rows8,
                       (int64_t)p.Bsz * p.L * p.Dm);
    if (hipGetLastError() != hipSuccess) return MAMBA_ERR_HIP;
  }
  return MAMBA_OK;
}

template <typename TIn, bool EXACT>
int dispatch_scan(int64_t N, const ScanParams& p, const Plan& pl, hipStream_t s) {
  switch (N) {
    case 1: return launch_scan<TIn, 1, EXACT>(p, pl, s);
    case 2: return launch_scan<TIn, 2, EXACT>(p, pl, s);
    case 4: return launch_scan<TIn, 4, EXACT>(p, pl, s);
    case 8: return launch_scan<TIn, 8, EXACT>(p, pl, s);
    case 16: return launch_scan<TIn, 16, EXACT>(p, pl, s);
    case 32: return launch_scan<TIn, 32, EXACT>(p, pl, s);
    case 64: return launch_scan<TIn, 64, EXACT>(p, pl, s);
    default: return MAMBA_ERR_UNSUPPORTED;
  }
}

template <typename TIn, int N, bool EXACT>
int launch_step(const StepParams& p, hipStream_t stream) {
  constexpr int TPC = N < 4 ? 1 : N / 4;  // threads per (batch, channel)
  const unsigned blocks = (unsigned)(((int64_t)p.Bsz * p.Dm * TPC + 255) / 256);
  hipLaunchKernelGGL((scan_step_kernel<TIn, N, EXACT>), dim3(blocks), dim3(256), 0, stream, p);
  return hipGetLastError() == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

template <typename TIn, bool EXACT>
int dispatch_step(int64_t N, const StepParams& p, hipStream_t s) {
  switch (N) {
    case 1: return launch_step<TIn, 1, EXACT>(p, s);
    case 2: return launch_step<TIn, 2, EXACT>(p, s);
    case 4: return launch_step<TIn, 4, EXACT>(p, s);
    case 8: return launch_step<TIn, 8, EXACT>(p, s);
    case 16: return launch_step<TIn, 16, EXACT>(p, s);
    case 32: return launch_step<TIn, 32, EXACT>(p, s);
    case 64: return launch_step<TIn, 64, EXACT>(p, s);
    default: return MAMBA_ERR_UNSUPPORTED;
  }
}

template <typename TIn, int N, bool EXACT>
int launch_bwd(BwdParams p, hipStream_t stream) {
  constexpr int NT = 16 * (N < 4 ? 4 : N);
  if (p.nchunks > 1) {  // aggregate pass over chunks 1.. (the carry alone: no input-term rule)
    p.chunk0 = 1;
    p.grid_chunks = p.nchunks - 1;
    const unsigned blocks = (unsigned)(p.nblk_d * p.grid_chunks * p.Bsz * p.K);
    hipLaunchKernelGGL((scan_bwd_kernel<TIn, N, false, true>), dim3(blocks), dim3(NT), 0, stream, p);
    if (hipGetLastError() != hipSuccess) return MAMBA_ERR_HIP;
  }
  p.chunk0 = 0;
  p.grid_chunks = p.nchunks;
  const unsigned blocks = (unsigned)(p.nblk_d * p.grid_chunks * p.Bsz * p.K);
  hipLaunchKernelGGL((scan_bwd_kernel<TIn, N, EXACT, false>), dim3(blocks), dim3(NT), 0, stream, p);
  return hipGetLastError() == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

template <typename TIn, bool EXACT>
int dispatch_bwd(int64_t N, const BwdParams& p, hipStream_t s) {
  switch (N) {
    case 1: return launch_bwd<TIn, 1, EXACT>(p, s);
    case 2: return launch_bwd<TIn, 2, EXACT>(p, s);
    case 4: return launch_bwd<TIn, 4, EXACT>(p, s);
    case 8: return launch_bwd<TIn, 8, EXACT>(p, s);
    case 16: return launch_bwd<TIn, 16, EXACT>(p, s);
    default: return MAMBA_ERR_UNSUPPORTED;
  }
}

#endif  // MSCAN_INSTANTIATE

}  // namespace mscan
