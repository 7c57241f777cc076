// Measurement kernel: the MFMA throughput this GPU sustains, for reporting
// the main kernel against a measured (not only the nominal) matrix-core peak.
// Each wave keeps eight independent accumulators so that back-to-back
// v_mfma_f32_32x32x16 instructions never wait on each other.
#include "fsa_internal.h"

namespace fsa {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void k_mfma_loop(float* __restrict__ sink, int iters) {
  using V8 = typename Vec8<T>::type;
  V8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (T)(threadIdx.x * 1e-3f + e);
    b[e] = (T)(e * 1e-3f);
  }
  f32x16 c[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) c[k] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = mfma32(a, b, c[k]);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[k][r];
  // keeps the loop alive; the sum never equals this value for these inputs
  if (s == -1.0f) sink[threadIdx.x] = s;
}

}  // namespace
}  // namespace fsa

using namespace fsa;

extern "C" int32_t fsa_mfma_loop(int32_t dtype, int32_t workgroups, int32_t iters, float* sink, void* stream) {
  if (sink == nullptr) return FSA_ERR_NULL;
  if (workgroups < 1 || iters < 1) return FSA_ERR_SHAPE;
  if (dtype != FSA_DTYPE_BF16 && dtype != FSA_DTYPE_FP16) return FSA_ERR_DTYPE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == FSA_DTYPE_BF16)
    hipLaunchKernelGGL(k_mfma_loop<__bf16>, dim3(workgroups), dim3(256), 0, s, sink, iters);
  else
    hipLaunchKernelGGL(k_mfma_loop<_Float16>, dim3(workgroups), dim3(256), 0, s, sink, iters);
  return hipGetLastError() == hipSuccess ? FSA_OK : FSA_ERR_HIP;
}
