// compress2 kernel instances writing records to a paged pool.
#include "compress2_kernel.h"

namespace sq {
template void launch_compress2_pg<true>(int, bool, bool, int, dim3, size_t, hipStream_t,
                                              const Compress2Args &);
}  // namespace sq
