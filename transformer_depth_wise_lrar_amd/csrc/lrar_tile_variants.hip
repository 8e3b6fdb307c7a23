// Instantiation of the register-tile read for the full-width-RMS control read and the
// separate-key read (see lrar_tile_impl.h).
#include "lrar_tile_impl.h"

namespace lrar {

hipError_t launch_tile_fullrms(const ReadParams& p, int io_bf16, int vec, hipStream_t s) {
  if (io_bf16) return vec > 1 ? launch_tile_nu<bf16_bits, 8, kTileFullRms, float>(p, s)
                              : launch_tile_nu<bf16_bits, 1, kTileFullRms, float>(p, s);
  return vec > 1 ? launch_tile_nu<float, 4, kTileFullRms, float>(p, s)
                 : launch_tile_nu<float, 1, kTileFullRms, float>(p, s);
}

hipError_t launch_tile_keys(const ReadParams& p, const SrcList& keys, int io_bf16, int vec,
                            hipStream_t s) {
  if (io_bf16) return vec > 1 ? launch_tile_nu<bf16_bits, 8, kTileKeys, float>(p, keys, s)
                              : launch_tile_nu<bf16_bits, 1, kTileKeys, float>(p, keys, s);
  return vec > 1 ? launch_tile_nu<float, 4, kTileKeys, float>(p, keys, s)
                 : launch_tile_nu<float, 1, kTileKeys, float>(p, keys, s);
}

// The pieces in order of preference: row-local sums over lanes 0..31 with the smallest piece
// that fits there, then sums over all 64 lanes. A piece must divide r (so no lane reads past
// the key) and its loads must be aligned; the element path loads single elements only.
int tile_keys_piece(int r, int align_bytes, int esize, int vec) {
  const int lanes_local = kWave / 2;
  for (int pass = 0; pass < 2; ++pass) {
    const bool rowred = pass == 0;
    const int lanes = rowred ? lanes_local : kWave;
    for (int ks = 1; ks <= 8; ks *= 2) {
      if (vec == 1 && ks > 1) break;
      const int bytes = ks * esize < 16 ? ks * esize : 16;
      if (r % ks == 0 && r / ks <= lanes && align_bytes % bytes == 0)
        return key_piece_code(ks, rowred);
    }
  }
  return 0;
}

}  // namespace lrar
