// Fused decode kernel instances: 3 and 4 query heads per launch, contiguous key and value records.
#include "decode_dispatch.h"

namespace sq {
template bool dispatch_g<3, 1>(bool, int, int, int, dim3, size_t, hipStream_t, const AttendArgs &);
template bool dispatch_g<4, 1>(bool, int, int, int, dim3, size_t, hipStream_t, const AttendArgs &);
}  // namespace sq
