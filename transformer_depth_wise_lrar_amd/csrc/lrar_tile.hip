// Dispatch of the register-tile read (lrar_tile_impl.h) to its per-mode instantiations.

#include "lrar_launch.h"

namespace lrar {

hipError_t launch_tile_online(const ReadParams& p, int io_bf16, int vec, hipStream_t s);
hipError_t launch_tile_twopass(const ReadParams& p, int io_bf16, int vec, hipStream_t s);
hipError_t launch_tile_merge(const ReadParams& p, int io_bf16, int vec, int acc_bf16,
                             hipStream_t s);
hipError_t launch_tile_merge_acc(const ReadParams& p, int io_bf16, int vec, int acc_bf16,
                                 hipStream_t s);

int tile_max_chunks() { return 32; }

hipError_t launch_tile(const ReadParams& p, ReadKind kind, int io_bf16, int vec, int acc_bf16,
                       hipStream_t s) {
  if (kind == ReadKind::kMerge) return launch_tile_merge(p, io_bf16, vec, acc_bf16, s);
  if (kind == ReadKind::kMergeAccumulate)
    return launch_tile_merge_acc(p, io_bf16, vec, acc_bf16, s);
  if (kind == ReadKind::kOnline) return launch_tile_online(p, io_bf16, vec, s);
  return launch_tile_twopass(p, io_bf16, vec, s);
}

}  // namespace lrar
