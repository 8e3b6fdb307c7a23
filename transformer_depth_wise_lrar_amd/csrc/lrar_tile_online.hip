// Instantiation of the register-tile read, online mode (see lrar_tile_impl.h).
#include "lrar_tile_impl.h"

namespace lrar {

hipError_t launch_tile_online(const ReadParams& p, int io_bf16, int vec, hipStream_t s) {
  if (io_bf16) return vec > 1 ? launch_tile_nu<bf16_bits, 8, kTileOnline, float>(p, s)
                              : launch_tile_nu<bf16_bits, 1, kTileOnline, float>(p, s);
  return vec > 1 ? launch_tile_nu<float, 4, kTileOnline, float>(p, s)
                 : launch_tile_nu<float, 1, kTileOnline, float>(p, s);
}

}  // namespace lrar
