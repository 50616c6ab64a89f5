// Per-family launch dispatch over the supported shapes and dtypes.  Each
// family's translation unit includes this file once with its own FAMILY.
#pragma once

#include "sk_read.hpp"
#include "sk_tile.hpp"

namespace sk {

// The flush over a device-side list of due sequences: the scan, then the
// loop over the listed tiles with a workgroup per tile of the first p.nseq
// list entries (about twice what a ragged phase brings due at a step).
template <void (*LOOP)(Params)>
static void launch_scanned_flush(int threads, size_t lds, const Params& p, hipStream_t st) {
  hipLaunchKernelGGL(due_scan_kernel<0>, dim3(1), dim3(DUE_SCAN_THREADS), 0, st, p);
  hipLaunchKernelGGL(LOOP, dim3(p.nseq * p.H), dim3(threads), lds, st, p);
}

template <int FAM, int DK, int DV, typename AT, typename UT, int WMAX>
static int launch_tile(int mode, int coef, const Params& p, hipStream_t st) {
  const dim3 grid((p.seq_list ? p.nseq : p.B) * p.H), block(TileShape<DK, DV>::THREADS);
  constexpr size_t lds_flush = TileLds<FAM, DK, DV, WMAX, MODE_FLUSH, 0>::BYTES;
  constexpr size_t lds_flush_map = TileLds<FAM, DK, DV, WMAX, MODE_FLUSH, 1>::BYTES;
  constexpr size_t lds_full = TileLds<FAM, DK, DV, WMAX, MODE_FULL, 0>::BYTES;
  constexpr size_t lds_replay = TileLds<FAM, DK, DV, WMAX, MODE_REPLAY, 0>::BYTES;
  // (the flush of a layer with dense-fallback heads is its own instantiation)
  const bool dense = p.ndense > 0;
  if (mode == MODE_FLUSH && p.seq_count) {
    constexpr int NT = TileShape<DK, DV>::THREADS;
    if (coef && dense)
      launch_scanned_flush<tile_kernel<FAM, DK, DV, AT, UT, MODE_FLUSH, WMAX, 1, true, true>>(NT, lds_flush_map, p, st);
    else if (coef)
      launch_scanned_flush<tile_kernel<FAM, DK, DV, AT, UT, MODE_FLUSH, WMAX, 1, false, true>>(NT, lds_flush_map, p, st);
    else if (dense)
      launch_scanned_flush<tile_kernel<FAM, DK, DV, AT, UT, MODE_FLUSH, WMAX, 0, true, true>>(NT, lds_flush, p, st);
    else
      launch_scanned_flush<tile_kernel<FAM, DK, DV, AT, UT, MODE_FLUSH, WMAX, 0, false, true>>(NT, lds_flush, p, st);
    return 0;
  }
  if (mode == MODE_FLUSH && coef && dense)
    hipLaunchKernelGGL((tile_kernel<FAM, DK, DV, AT, UT, MODE_FLUSH, WMAX, 1, true>), grid, block, lds_flush_map, st, p);
  else if (mode == MODE_FLUSH && coef)
    hipLaunchKernelGGL((tile_kernel<FAM, DK, DV, AT, UT, MODE_FLUSH, WMAX, 1, false>), grid, block, lds_flush_map, st, p);
  else if (mode == MODE_FLUSH && dense)
    hipLaunchKernelGGL((tile_kernel<FAM, DK, DV, AT, UT, MODE_FLUSH, WMAX, 0, true>), grid, block, lds_flush, st, p);
  else if (mode == MODE_FLUSH)
    hipLaunchKernelGGL((tile_kernel<FAM, DK, DV, AT, UT, MODE_FLUSH, WMAX, 0, false>), grid, block, lds_flush, st, p);
  else if (mode == MODE_FULL)
    hipLaunchKernelGGL((tile_kernel<FAM, DK, DV, AT, UT, MODE_FULL, WMAX, 0, false>), grid, block, lds_full, st, p);
  else if (mode == MODE_REPLAY)
    hipLaunchKernelGGL((tile_kernel<FAM, DK, DV, AT, UT, MODE_REPLAY, WMAX, 0, false>), grid, block, lds_replay, st, p);
  else
    return -4;
  return 0;
}

template <int FAM, int DK, int DV, typename AT, typename UT, int WMAX, int COEF>
static void launch_read(const Params& p, hipStream_t st) {
  if constexpr (FAM == FAM_M2) {
    const dim3 pgrid(PrepGrid<COEF, DK, UT, WMAX>::blocks(p.B), p.G);
    constexpr int CS = m2_read_split(DV, WMAX);
    const dim3 rgrid(m2_read_blocks(p.B, p.G, p.HPG, CS));
    hipLaunchKernelGGL((m2_prep_kernel<DK, AT, UT, WMAX, COEF>), pgrid, dim3(CQ_THREADS), 0, st, p);
    hipLaunchKernelGGL((m2_read_kernel<DK, DV, AT, UT, WMAX, CS>), rgrid, dim3(64 * M2R_WPB), 0, st, p);
    if (p.ndense > 0)
      hipLaunchKernelGGL((m2_dense_read_kernel<DK, DV, AT, UT, WMAX>), dim3(p.B * p.ndense), dim3(64), 0,
                         st, p);
  } else {
    if (p.pullback == 2)
      hipLaunchKernelGGL((dn_read_kernel<FAM, DK, DV, AT, UT, WMAX, COEF, 2>), dim3(dn_read_blocks(p.B, p.H)),
                         dim3(64 * DN_TPW), 0, st, p);
    else if (p.pullback == 1)
      hipLaunchKernelGGL((dn_read_kernel<FAM, DK, DV, AT, UT, WMAX, COEF, 1>), dim3(dn_read_blocks(p.B, p.H)),
                         dim3(64 * DN_TPW), 0, st, p);
    else
      hipLaunchKernelGGL((dn_read_kernel<FAM, DK, DV, AT, UT, WMAX, COEF, 0>), dim3(dn_read_blocks(p.B, p.H)),
                         dim3(64 * DN_TPW), 0, st, p);
    if (p.ndense > 0)
      hipLaunchKernelGGL((dn_dense_read_kernel<DK, DV, AT, UT>), dim3(p.B * p.ndense), dim3(DND_THREADS), 0,
                         st, p);
  }
}

template <int FAM, int DK, int DV, typename AT, typename UT>
static int launch_shape(int mode, int coef, const Params& p, hipStream_t st) {
  if (p.B <= 0 || p.H <= 0) return 0;
  if (mode == MODE_READ) {
    if (p.W <= 16) {
      if (coef) launch_read<FAM, DK, DV, AT, UT, 16, 1>(p, st);
      else launch_read<FAM, DK, DV, AT, UT, 16, 0>(p, st);
    } else {
      if (coef) launch_read<FAM, DK, DV, AT, UT, 32, 1>(p, st);
      else launch_read<FAM, DK, DV, AT, UT, 32, 0>(p, st);
    }
  } else if (p.W <= 16) {
    if (int rc = launch_tile<FAM, DK, DV, AT, UT, 16>(mode, coef, p, st)) return rc;
  } else {
    if (int rc = launch_tile<FAM, DK, DV, AT, UT, 32>(mode, coef, p, st)) return rc;
  }
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

template <int FAM, typename AT, typename UT>
static int launch_dtype(int mode, int coef, int dk, int dv, const Params& p, hipStream_t st) {
  if (dk == 16 && dv == 32) return launch_shape<FAM, 16, 32, AT, UT>(mode, coef, p, st);
  if (dk == 64 && dv == 64) return launch_shape<FAM, 64, 64, AT, UT>(mode, coef, p, st);
  if (dk == 128 && dv == 64) return launch_shape<FAM, 128, 64, AT, UT>(mode, coef, p, st);
  if (dk == 128 && dv == 128) return launch_shape<FAM, 128, 128, AT, UT>(mode, coef, p, st);
  return -2;
}


}  // namespace sk
