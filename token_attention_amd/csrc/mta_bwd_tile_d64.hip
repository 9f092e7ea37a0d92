// Fused backward tile kernels for head size 64 (one translation unit per head size).
#include "mta_bwd_tile.h"

namespace mta {

hipError_t launch_bwd_tiles_d64(const bwt::BwArgs& a, int ch, int mode, int spec, size_t lds, unsigned grid,
                                 hipStream_t st) {
  return bwt::launch_tiles<64>(a, ch, mode, spec, lds, grid, st);
}

}  // namespace mta
