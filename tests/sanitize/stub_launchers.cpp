// Launchers for the host-only sanitizer build of the C-ABI layer: the fuzz
// never reaches a launch (every call it makes fails validation first), so
// each stub aborts if it is ever called.
#include <cstdlib>

#include "fsa_internal.h"

namespace fsa {
hipError_t launch_build_index(const Geometry&, const int32_t*, const int32_t*, const fsa_index&, void*, hipStream_t) {
  std::abort();
}
hipError_t launch_stats(const Geometry&, const int32_t*, const void*, const void*, const fsa_index&, float*, float*,
                        void*, hipStream_t) {
  std::abort();
}
hipError_t launch_main(const Geometry&, const int32_t*, const void*, const void*, const void*, const fsa_index&,
                       const float*, void*, void*, hipStream_t) {
  std::abort();
}
hipError_t launch_reduce(const Geometry&, const fsa_index&, const void*, void*, bool, const void*, float*, float*,
                         hipStream_t) {
  std::abort();
}
hipError_t launch_bwd(const Geometry&, const int32_t*, const void*, const void*, const void*, const void*, const void*,
                      const float*, const fsa_index&, void*, void*, void*, void*, hipStream_t) {
  std::abort();
}
hipError_t launch_select(const Geometry&, const int32_t*, const float*, int64_t, int, int, int32_t*, hipStream_t) {
  std::abort();
}
hipError_t launch_nsa(const Geometry&, const int32_t*, const void*, const void*, const void*, const int32_t*, void*,
                      float*, hipStream_t) {
  std::abort();
}
}  // namespace fsa
