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
#include "scan_row.h"

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
#ifndef MSCAN_FOLD
#define MSCAN_FOLD 1
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
#ifndef MSCAN_G2_WAVES
#define MSCAN_G2_WAVES (16 * 1024)
#endif
inline constexpr int64_t kG2Waves = MSCAN_G2_WAVES;

// Workspace of a forward pass, in this order (each region 256-byte aligned):
// the per-direction fp32 rows, the time-split aggregates (end states, ΣΔ'),
// and for the row kernel the fp32 copies of B and C.
struct Plan {
  int K, Ku, cb, g, nblk_d, nchunks, chunk_len, prio;
  int tile;  // scan positions per LDS tile of the channel-block kernel (kTile or 2 kTile)
  int row;  // 1: scan_row_kernel (one channel per lane, all states in registers); 0: scan_chunk_kernel
  int np;   // the row kernel's power-of-two state count (>= N)
  size_t ws_y_bytes, agg_state_bytes, agg_dsum_bytes, bc_bytes;
  size_t total() const { return ws_y_bytes + agg_state_bytes + agg_dsum_bytes + bc_bytes; }
};


// Dispatchers exported by the instantiation units: N is the state size, the
// suffix the element type (bf16 / f32) and the input-term rule (exact
// zero-order hold or Δ·B·u).
#define MSCAN_DECLARE_DISPATCH(SUFFIX)                                                        \
  int dispatch_scan_##SUFFIX(int64_t N, const ScanParams& p, const Plan& pl, hipStream_t s); \
  int dispatch_rows_##SUFFIX(const ScanParams& p, const Plan& pl, hipStream_t s);           \
  int dispatch_step_##SUFFIX(int64_t N, const StepParams& p, hipStream_t s);              \
  int dispatch_bwd_##SUFFIX(int64_t N, const BwdParams& p, hipStream_t s);
MSCAN_DECLARE_DISPATCH(bf16_simple)
MSCAN_DECLARE_DISPATCH(bf16_exact)
MSCAN_DECLARE_DISPATCH(f32_simple)
MSCAN_DECLARE_DISPATCH(f32_exact)

#if defined(MSCAN_INSTANTIATE) || defined(MSCAN_INSTANTIATE_ROWS)
template <typename TIn>
int launch_merge(const ScanParams& p, hipStream_t stream) {
  const int64_t n = (int64_t)p.Bsz * p.L * p.Dm;
  if (p.Dm % 8 == 0) {
    const int64_t rows8 = n / 8;
    const unsigned mblocks = (unsigned)((rows8 + 255) / 256);
    hipLaunchKernelGGL((merge_dirs_kernel<TIn, 8>), dim3(mblocks), dim3(256), 0, stream, p.ws_y,
                       static_cast<const TIn*>(p.z), static_cast<TIn*>(p.out), p.K, rows8, n);
  } else {
    const unsigned mblocks = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL((merge_dirs_kernel<TIn, 1>), dim3(mblocks), dim3(256), 0, stream, p.ws_y,
                       static_cast<const TIn*>(p.z), static_cast<TIn*>(p.out), p.K, n, n);
  }
  return hipGetLastError() == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

#endif

#ifdef MSCAN_INSTANTIATE
// Whether the channel-block kernel's last direction folds the other
// direction's row into the output (p.fold, set by the plain forward pass: the
// rows are not kept) instead of a merge kernel summing the rows afterwards.
// Two directions only -- measured on MI355X (fold vs merge, µs): 97k-token
// Vim 1270 vs 1315, Vim-224 234 vs 236; the cross scan's fourth direction
// alone fills a quarter of the GPU and loses: 999 vs 674.
inline bool folds(const ScanParams& p) { return MSCAN_FOLD && p.fold && p.K == 2 && p.out && p.ws_y; }

template <typename TIn, int N, int G16, bool EXACT, int TT>
int launch_chunks_tt(ScanParams p, const Plan& pl, hipStream_t stream) {
  constexpr Layout lay = layout_of(N, G16);
  constexpr int NT = threads_of(N, G16);
  if (pl.nchunks > 1) {
    p.grid_chunks = pl.nchunks - 1;
    p.prio = pl.prio;
    const unsigned blocks = (unsigned)(pl.nblk_d * p.grid_chunks * p.Bsz * p.K);
    hipLaunchKernelGGL((scan_chunk_kernel<TIn, N, lay.g, lay.cb, TT, true, EXACT>), dim3(blocks), dim3(NT), 0, stream, p);
    if (hipGetLastError() != hipSuccess) return MAMBA_ERR_HIP;
  }
  p.grid_chunks = pl.nchunks;
  p.prio = pl.prio;
  // directions kbase .. kbase+kcount-1 in one grid
  auto run = [&](int kbase, int kcount, int fold) {
    ScanParams q = p;
    q.kbase = kbase;
    q.fold = fold;
    const unsigned blocks = (unsigned)(pl.nblk_d * q.grid_chunks * q.Bsz * kcount);
    hipLaunchKernelGGL((scan_chunk_kernel<TIn, N, lay.g, lay.cb, TT, false, EXACT>), dim3(blocks), dim3(NT), 0,
                       stream, q);
    return hipGetLastError() == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
  };
  if (folds(p)) {
    // direction 0 writes its row, then direction 1 adds it to its own output
    // in its epilogue
    const int rc = run(0, p.K - 1, 0);
    return rc != MAMBA_OK ? rc : run(p.K - 1, 1, 1);
  }
  return run(0, p.K, 0);
}

// 64-position tiles for one state per thread at N = 16 on long sequences
// (Plan::tile, set by the plan), 32 elsewhere.
template <typename TIn, int N, int G16, bool EXACT>
int launch_chunks(const ScanParams& p, const Plan& pl, hipStream_t stream) {
  if constexpr (N == 16 && G16 == 1) {
    if (pl.tile == 2 * kTile) return launch_chunks_tt<TIn, N, G16, EXACT, 2 * kTile>(p, pl, stream);
  }
  return launch_chunks_tt<TIn, N, G16, EXACT, kTile>(p, pl, stream);
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
  // (K = 1 or folded: the scan wrote out)
  if (p.ws_y && p.out && p.K > 1 && !folds(p)) return launch_merge<TIn>(p, stream);
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
  if ((N & (N - 1)) != 0) {
    const unsigned blocks = (unsigned)(((int64_t)p.Bsz * p.Dm + 255) / 256);
    hipLaunchKernelGGL((scan_step_any_kernel<TIn, EXACT>), dim3(blocks), dim3(256), 0, s, p, (int)N);
    return hipGetLastError() == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
  }
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

template <typename TIn, int NP, bool FULL, bool EXACT>
int launch_bwd(BwdParams p, hipStream_t stream) {
  constexpr int NT = 16 * (NP < 4 ? 4 : NP);
  if (p.nchunks > 1) {  // aggregate pass over chunks 1.. (the carry alone: no input-term rule)
    p.chunk0 = 1;
    p.grid_chunks = p.nchunks - 1;
    const unsigned blocks = (unsigned)(p.nblk_d * p.grid_chunks * p.Bsz * p.K);
    hipLaunchKernelGGL((scan_bwd_kernel<TIn, NP, FULL, false, true>), dim3(blocks), dim3(NT), 0, stream, p);
    if (hipGetLastError() != hipSuccess) return MAMBA_ERR_HIP;
  }
  p.chunk0 = 0;
  p.grid_chunks = p.nchunks;
  const unsigned blocks = (unsigned)(p.nblk_d * p.grid_chunks * p.Bsz * p.K);
  hipLaunchKernelGGL((scan_bwd_kernel<TIn, NP, FULL, EXACT, false>), dim3(blocks), dim3(NT), 0, stream, p);
  return hipGetLastError() == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

// State sizes that are not a power of two run the next power-of-two
// instantiation with the state count read at run time.
template <typename TIn, int NP, bool EXACT>
int launch_bwd_np(const BwdParams& p, hipStream_t s) {
  if constexpr (NP <= 2) return launch_bwd<TIn, NP, true, EXACT>(p, s);
  else return p.N == NP ? launch_bwd<TIn, NP, true, EXACT>(p, s) : launch_bwd<TIn, NP, false, EXACT>(p, s);
}

// Above 32 states: p.ngroups workgroups of 16 states per (channel block,
// chunk, batch, direction), the group the fastest-varying grid index.
template <typename TIn, bool EXACT>
int launch_bwd_groups(BwdParams p, hipStream_t stream) {
  constexpr int NP = 16, NT = 16 * NP;
  if (p.nchunks > 1) {  // aggregate pass over chunks 1..
    p.chunk0 = 1;
    p.grid_chunks = p.nchunks - 1;
    const unsigned blocks = (unsigned)((int64_t)p.nblk_d * p.grid_chunks * p.Bsz * p.K * p.ngroups);
    hipLaunchKernelGGL((scan_bwd_kernel<TIn, NP, false, false, true, true>), dim3(blocks), dim3(NT), 0, stream, p);
    if (hipGetLastError() != hipSuccess) return MAMBA_ERR_HIP;
  }
  p.chunk0 = 0;
  p.grid_chunks = p.nchunks;
  const unsigned blocks = (unsigned)((int64_t)p.nblk_d * p.grid_chunks * p.Bsz * p.K * p.ngroups);
  hipLaunchKernelGGL((scan_bwd_kernel<TIn, NP, false, EXACT, false, true>), dim3(blocks), dim3(NT), 0, stream, p);
  return hipGetLastError() == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

template <typename TIn, bool EXACT>
int dispatch_bwd(int64_t N, const BwdParams& p, hipStream_t s) {
  if (N < 1 || N > 64) return MAMBA_ERR_UNSUPPORTED;
  if (N > 32) return p.ngroups == (N + 15) / 16 ? launch_bwd_groups<TIn, EXACT>(p, s) : MAMBA_ERR_UNSUPPORTED;
  if (N <= 1) return launch_bwd_np<TIn, 1, EXACT>(p, s);
  if (N <= 2) return launch_bwd_np<TIn, 2, EXACT>(p, s);
  if (N <= 4) return launch_bwd_np<TIn, 4, EXACT>(p, s);
  if (N <= 8) return launch_bwd_np<TIn, 8, EXACT>(p, s);
  if (N <= 16) return launch_bwd_np<TIn, 16, EXACT>(p, s);
  return launch_bwd_np<TIn, 32, EXACT>(p, s);
}

#endif  // MSCAN_INSTANTIATE


#ifdef MSCAN_INSTANTIATE_ROWS
template <typename TIn, int NP, bool FULL, bool EXACT>
int launch_rows(ScanParams p, const Plan& pl, hipStream_t stream) {
  {
    const int64_t rows = (int64_t)p.Bsz * p.K * p.L;
    const unsigned wblocks = (unsigned)((2 * (rows + 2) * NP + 255) / 256);
    int lognp = 0;
    while ((1 << lognp) < NP) ++lognp;
    hipLaunchKernelGGL((widen_bc_kernel<TIn>), dim3(wblocks), dim3(256), 0, stream, static_cast<const TIn*>(p.B),
                       static_cast<const TIn*>(p.C), p.bcw, rows, p.N, lognp);
    if (hipGetLastError() != hipSuccess) return MAMBA_ERR_HIP;
  }
  if (pl.nchunks > 1) {
    p.grid_chunks = pl.nchunks - 1;
    const unsigned blocks = (unsigned)(pl.nblk_d * p.grid_chunks * p.Bsz * p.K);
    hipLaunchKernelGGL((scan_row_kernel<TIn, NP, FULL, ROW_AGG, EXACT>), dim3(blocks), dim3(64), 0, stream, p);
    if (hipGetLastError() != hipSuccess) return MAMBA_ERR_HIP;
  }
  p.grid_chunks = pl.nchunks;
  const unsigned blocks = (unsigned)(pl.nblk_d * p.grid_chunks * p.Bsz * p.K);
  if (p.ckpt || (p.K == 1 && p.ws_y) || (p.K == 1 && !p.out) || (p.K != 1 && !p.ws_y))
    hipLaunchKernelGGL((scan_row_kernel<TIn, NP, FULL, ROW_ANY, EXACT>), dim3(blocks), dim3(64), 0, stream, p);
  else if (p.K != 1)
    hipLaunchKernelGGL((scan_row_kernel<TIn, NP, FULL, ROW_ROWS, EXACT>), dim3(blocks), dim3(64), 0, stream, p);
  else if (p.z)
    hipLaunchKernelGGL((scan_row_kernel<TIn, NP, FULL, ROW_OUT_GATE, EXACT>), dim3(blocks), dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL((scan_row_kernel<TIn, NP, FULL, ROW_OUT, EXACT>), dim3(blocks), dim3(64), 0, stream, p);
  return hipGetLastError() == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

template <typename TIn, int NP, bool EXACT>
int launch_scan_rows(const ScanParams& p, const Plan& pl, hipStream_t stream) {
  // (state sizes up to 2 are powers of two: no padded instantiation)
  int rc;
  if constexpr (NP <= 2) rc = launch_rows<TIn, NP, true, EXACT>(p, pl, stream);
  else rc = p.N == NP ? launch_rows<TIn, NP, true, EXACT>(p, pl, stream)
                      : launch_rows<TIn, NP, false, EXACT>(p, pl, stream);
  if (rc != MAMBA_OK) return rc;
  if (p.ws_y && p.out && p.K > 1) return launch_merge<TIn>(p, stream);
  return MAMBA_OK;
}

template <typename TIn, bool EXACT>
int dispatch_rows(const ScanParams& p, const Plan& pl, hipStream_t s) {
  switch (pl.np) {
    case 1: return launch_scan_rows<TIn, 1, EXACT>(p, pl, s);
    case 2: return launch_scan_rows<TIn, 2, EXACT>(p, pl, s);
    case 4: return launch_scan_rows<TIn, 4, EXACT>(p, pl, s);
    case 8: return launch_scan_rows<TIn, 8, EXACT>(p, pl, s);
    case 16: return launch_scan_rows<TIn, 16, EXACT>(p, pl, s);
    case 32: return launch_scan_rows<TIn, 32, EXACT>(p, pl, s);
    case 64: return launch_scan_rows<TIn, 64, EXACT>(p, pl, s);
    default: return MAMBA_ERR_UNSUPPORTED;
  }
}
#endif  // MSCAN_INSTANTIATE_ROWS

}  // namespace mscan
