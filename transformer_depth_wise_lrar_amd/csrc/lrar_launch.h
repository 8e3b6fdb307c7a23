// Kernel parameter blocks and launchers of liblrattnres (internal; not installed).
// Every launcher assumes its arguments were validated by the entry points in lrar_api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "lrar_device.h"

namespace lrar {

// The read (lrar_forward) and the merge (lrar_merge, which adds a prior accumulator).
struct ReadParams {
  SrcList src;
  int n;
  int d, r;
  int64_t T;
  double eps;
  const float* q;
  void* out;
  int64_t out_ld;
  float* alpha;  // nullable
  int64_t alpha_ld;
  // nullable: per row the scores z_i (columns 0..n-1) and 1 / rho_i (columns n..2n-1)
  double* saved;
  int64_t saved_ld;
  // merge only
  const float* m_in;
  const float* l_in;
  const void* acc;
  int64_t acc_ld;
  float* m_out;  // nullable
  float* l_out;  // nullable
  // separate-key read only: the spread key piece chosen by tile_keys_piece
  int key_piece;
  // merge with the partial-sum update fused in: b_out = b_prev + src[0] (b_prev nullable)
  const void* b_prev;
  int64_t b_prev_ld;
  void* b_out;
  int64_t b_out_ld;
  // register-tile read only, set by its launcher: the row tiles [tile_begin, tile_end) of one
  // launch
  int64_t tile_begin, tile_end;
};

// A spread key piece of ks elements per lane, reduced row-locally (rowred) or over the lanes.
constexpr int key_piece_code(int ks, bool rowred) { return 2 * ks + (rowred ? 1 : 0); }

enum class ReadKind { kTwoPass, kOnline, kMerge, kMergeAccumulate };

// Phase-1 statistics (lrar_forward_stats).
struct StatsParams {
  SrcList src;
  int n;
  int d, r;
  int64_t T;
  double eps;
  int nq;
  const float* q;
  int64_t q_ld;
  float* m;
  float* l;
  int64_t ml_ld;
  void* acc;
  int64_t acc_ld;
  int64_t acc_qstride;
};

// Backward (lrar_backward).
struct BwdParams {
  SrcList src;
  DstList dsrc;
  int n;
  int d, r;
  int64_t T;
  double eps;
  const float* q;
  const void* dout;  // float32 or bf16, the gradient type
  int64_t dout_ld;
  int accumulate;
  // nullable: the forward's saved statistics (z_i, then 1 / rho_i, per row); when given, the
  // key pass does not score the keys again
  const double* saved;
  int64_t saved_ld;
  float* dq;
  void* workspace;  // [grid + reduce groups][r] float64 dq partials
  int key_stash;    // set by the row-tile launcher: pass B reads the key units from LDS
};

// Column-chunked two-pass read (any width; also the merge when a row does not fit a tile).
// key_mode is a RowKeyMode: the sliced key, the full-width-RMS control or separate key rows
// (keys, only for kKeySeparate); the merge (kind kMerge) takes the sliced key.
hipError_t launch_read(const ReadParams& p, ReadKind kind, int io_bf16, int vec, int acc_bf16,
                       hipStream_t s, int key_mode = kKeySlice, const SrcList* keys = nullptr);
// b_out = b + o on [T, d] rows of the element type (b may be null), for the fused Phase-2
// update of rows too wide for a tile.
hipError_t launch_add_rows(const void* b, int64_t b_ld, const void* o, int64_t o_ld, void* bout,
                           int64_t bout_ld, int64_t T, int d, int io_bf16, int vec,
                           hipStream_t s);
// Register-tile read (online, two-pass or merge) for rows of at most tile_max_chunks() chunks
// of 64 units.
hipError_t launch_tile(const ReadParams& p, ReadKind kind, int io_bf16, int vec, int acc_bf16,
                       hipStream_t s);
int tile_max_chunks();
// The full-width-RMS control read and the separate-key read on register tiles (one pass).
hipError_t launch_tile_fullrms(const ReadParams& p, int io_bf16, int vec, hipStream_t s);
hipError_t launch_tile_keys(const ReadParams& p, const SrcList& keys, int io_bf16, int vec,
                            hipStream_t s);
// Spread key piece for a separate key of r elements whose rows all start at multiples of
// align_bytes (a power of two), with esize-byte elements; 0 if none serves this key.
int tile_keys_piece(int r, int align_bytes, int esize, int vec);

hipError_t launch_stats(const StatsParams& p, int io_bf16, int vec, int acc_bf16, hipStream_t s);

// Phase 1 on whole workgroups (lrar_stats_tile.hip): vector path, at most kStatsMaxSrc sources,
// queries in groups of stats_tile_query_group() (0 if one query's LDS slice does not fit).
constexpr int kStatsMaxSrc = 8;
constexpr int kStatsMaxQ = 12;
constexpr int kStatsKeySlots = 2;  // key unit slots loaded together per source
int stats_tile_query_group(int d, int r, int vec);
hipError_t launch_stats_tile(const StatsParams& p, int io_bf16, int acc_bf16, int qg,
                             hipStream_t s);

// Backward: grid size (workgroups) used for T rows, and the launcher.
int backward_grid(int64_t T);
// Lanes' register window for dq partials must cover the key; false if this shape needs more.
bool backward_supported(int d, int r, int vec);
size_t backward_workspace(int64_t T, int r);
// Workspace bytes for `grid` workgroup rows of dq partials (backward_workspace uses
// backward_grid(T)).
size_t backward_workspace_rows(int grid, int r);
// ws_grid > 0: the workspace holds that many workgroup rows (at most backward_grid(T)) and the
// launch uses at most that many workgroups.
hipError_t launch_backward(const BwdParams& p, int io_bf16, int grad_bf16, int vec,
                           hipStream_t s, int ws_grid = 0);
// Row-tile backward for the vector path (lrar_backward_tile.hip): writes the dq partials of
// *grid <= max_blocks workgroups into block_dq.
int backward_tile_max_chunks();
hipError_t launch_backward_tile(const BwdParams& p, int io_bf16, int grad_bf16, double* block_dq,
                                int max_blocks, int* grid, hipStream_t s);

// The calibration streams (lrar_copy, lrar_read_stream): workgroups, and 16-byte loads in flight
// per lane.
constexpr int kCalibBlocks = 1024;
constexpr int kCopyUnroll = 2;
constexpr int kReadUnroll = 4;
hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t s);
hipError_t launch_read_stream(const void* src, size_t bytes, void* sink, hipStream_t s);
// A kernel's traffic as a plain stream (lrar_mix_stream), in the launch shape given.
hipError_t launch_mix_stream(const SrcList& src, int n, int64_t T, int d, const DstList& out,
                             int nout, bool f32_out, int waves_per_cu, int waves_per_row,
                             int depth, int slots, int rows_per_wave, int lockstep,
                             hipStream_t s);

}  // namespace lrar
