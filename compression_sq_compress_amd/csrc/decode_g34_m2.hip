// Fused decode kernel instances: 3 and 4 query heads per launch, paged key and value records.
#include "decode_dispatch.h"

namespace sq {
template bool dispatch_g<3, 2>(bool, int, int, int, dim3, size_t, hipStream_t, const AttendArgs &);
template bool dispatch_g<4, 2>(bool, int, int, int, dim3, size_t, hipStream_t, const AttendArgs &);
}  // namespace sq
