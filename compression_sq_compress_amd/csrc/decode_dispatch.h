// Instances of the fused decode kernel and their dispatch by table placement,
// pipeline depth and waves per workgroup (sq_decode, sq_decode_paged).  Each
// (query heads per launch, mode) is instantiated in a translation unit of its
// own (decode_g*.hip) so that the build compiles them in parallel.
#pragma once
#include "attend_kernel.h"

namespace sq {

// Waves per workgroup the fused kernel is built for, by table placement:
// column tables share LDS among 8, 12 or 16 single-buffered waves, packed and
// device-memory tables among 4 or 8.
template <int G, int LM, int NP, int WPB, int FM>
void launch_one(dim3 grid, size_t lds, hipStream_t s, const AttendArgs &a) {
  hipLaunchKernelGGL((attend_partial_kernel<G, LM, NP, WPB, 1, FM>), grid, dim3(64 * WPB), lds, s, a);
}

template <int G, int LM, int NP, int WPB, int FM>
bool fits() {  // no static LDS (tables at address 0) and no scratch
  static const bool ok = [] {
    hipFuncAttributes fa{};
    return hipFuncGetAttributes(&fa, reinterpret_cast<const void *>(&attend_partial_kernel<G, LM, NP, WPB, 1, FM>)) ==
               hipSuccess && fa.sharedSizeBytes == 0 && fa.localSizeBytes == 0;
  }();
  return ok;
}

template <int G, int LM, int NP, int FM>
bool dispatch_np(bool run, int wpb, dim3 grid, size_t lds, hipStream_t s, const AttendArgs &a) {
  if constexpr (LM == LM_COL) {
    switch (wpb) {
      case 16: if (run) launch_one<G, LM, NP, 16, FM>(grid, lds, s, a); return fits<G, LM, NP, 16, FM>();
      case 12: if (run) launch_one<G, LM, NP, 12, FM>(grid, lds, s, a); return fits<G, LM, NP, 12, FM>();
      case 8: if (run) launch_one<G, LM, NP, 8, FM>(grid, lds, s, a); return fits<G, LM, NP, 8, FM>();
      default: return false;
    }
  } else {
    switch (wpb) {
      case 8: if (run) launch_one<G, LM, NP, 8, FM>(grid, lds, s, a); return fits<G, LM, NP, 8, FM>();
      case 4: if (run) launch_one<G, LM, NP, 4, FM>(grid, lds, s, a); return fits<G, LM, NP, 4, FM>();
      default: return false;
    }
  }
}

template <int G, int FM>
bool dispatch_g(bool run, int lm, int np, int wpb, dim3 grid, size_t lds, hipStream_t s, const AttendArgs &a) {
  auto by_np = [&](auto lmc) {
    constexpr int LM = decltype(lmc)::value;
    if (np == 1) return dispatch_np<G, LM, 1, FM>(run, wpb, grid, lds, s, a);
    if (np == 2) return dispatch_np<G, LM, 2, FM>(run, wpb, grid, lds, s, a);
    return dispatch_np<G, LM, 4, FM>(run, wpb, grid, lds, s, a);
  };
  if (lm == LM_COL) return by_np(std::integral_constant<int, LM_COL>());
  if (lm == LM_PACK) return by_np(std::integral_constant<int, LM_PACK>());
  return by_np(std::integral_constant<int, LM_GLB>());
}

}  // namespace sq
