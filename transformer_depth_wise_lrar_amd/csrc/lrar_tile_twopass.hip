// Instantiation of the register-tile read, two-pass mode (see lrar_tile_impl.h).
#include "lrar_tile_impl.h"

namespace lrar {

hipError_t launch_tile_twopass(const ReadParams& p, int io_bf16, int vec, hipStream_t s) {
  if (io_bf16) return vec > 1 ? launch_tile_nu<bf16_bits, 8, kTileTwoPass, float>(p, s)
                              : launch_tile_nu<bf16_bits, 1, kTileTwoPass, float>(p, s);
  return vec > 1 ? launch_tile_nu<float, 4, kTileTwoPass, float>(p, s)
                 : launch_tile_nu<float, 1, kTileTwoPass, float>(p, s);
}

}  // namespace lrar
