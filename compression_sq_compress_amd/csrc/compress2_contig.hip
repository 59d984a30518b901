// compress2 kernel instances writing records to contiguous slots.
#include "compress2_kernel.h"

namespace sq {
template void launch_compress2_pg<false>(int, bool, bool, int, dim3, size_t, hipStream_t,
                                              const Compress2Args &);
}  // namespace sq

namespace sq {
void launch_compress2_norm(int d, int rsc, dim3 grid, size_t lds, hipStream_t s, const Compress2Args &a) {
  switch (d) {
    case 32: launch_compress2_g<32, false, true, false, true>(rsc, grid, lds, s, a); break;
    case 64: launch_compress2_g<64, false, true, false, true>(rsc, grid, lds, s, a); break;
    default: launch_compress2_g<128, false, true, false, true>(rsc, grid, lds, s, a); break;
  }
}
}  // namespace sq
