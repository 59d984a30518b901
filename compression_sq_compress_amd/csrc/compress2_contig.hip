// compress2 kernel instances writing records to contiguous slots.
#include "compress2_kernel.h"

namespace sq {
template void launch_compress2_pg<false>(int, bool, bool, int, dim3, size_t, hipStream_t,
                                              const Compress2Args &);
}  // namespace sq
