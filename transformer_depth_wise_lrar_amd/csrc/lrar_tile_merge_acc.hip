// Instantiation of the register-tile read, merge mode with the partial-sum update fused in
// (Phase 2 of the two-phase schedule; see lrar_tile_impl.h).
#include "lrar_tile_impl.h"

namespace lrar {

hipError_t launch_tile_merge_acc(const ReadParams& p, int io_bf16, int vec, int acc_bf16,
                                 hipStream_t s) {
  if (io_bf16) {
    if (acc_bf16) return vec > 1 ? launch_tile_nu<bf16_bits, 8, kTileMergeAcc, bf16_bits>(p, s)
                                 : launch_tile_nu<bf16_bits, 1, kTileMergeAcc, bf16_bits>(p, s);
    return vec > 1 ? launch_tile_nu<bf16_bits, 8, kTileMergeAcc, float>(p, s)
                   : launch_tile_nu<bf16_bits, 1, kTileMergeAcc, float>(p, s);
  }
  if (acc_bf16) return vec > 1 ? launch_tile_nu<float, 4, kTileMergeAcc, bf16_bits>(p, s)
                               : launch_tile_nu<float, 1, kTileMergeAcc, bf16_bits>(p, s);
  return vec > 1 ? launch_tile_nu<float, 4, kTileMergeAcc, float>(p, s)
                 : launch_tile_nu<float, 1, kTileMergeAcc, float>(p, s);
}

}  // namespace lrar
