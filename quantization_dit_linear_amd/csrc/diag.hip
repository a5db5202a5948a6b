// diag.hip -- the matrix-core throughput probe of orbitquant_diag.h: every
// wave keeps 32 independent 16x16x32 fp16 MFMA accumulators in flight, so
// the matrix pipe never waits on a result; the loop holds nothing else.
#include <hip/hip_runtime.h>

#include "../../include/orbitquant.h"
#include "../../include/orbitquant_diag.h"

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(512) void mfma_probe_kernel(float *__restrict__ sink, int iters) {
  half8 a, b;
#pragma unroll
  for (int e = 0; e < 8; e++) {
    a[e] = (_Float16)(((int)threadIdx.x + e) & 7);
    b[e] = (_Float16)(e - 3);
  }
  floatx4 c[32];
#pragma unroll
  for (int i = 0; i < 32; i++) c[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int i = 0; i < 32; i++) c[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c[i], 0, 0, 0);
  }
  floatx4 s = c[0];
#pragma unroll
  for (int i = 1; i < 32; i++) s += c[i];
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
}

}  // namespace

extern "C" int oq_diag_mfma_f16(int blocks, int iters, float *sink, void *stream) {
  if (!sink || blocks < 1 || iters < 1) return OQ_EINVAL;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(512), 0, (hipStream_t)stream, sink,
                     iters);
  return hipGetLastError() == hipSuccess ? OQ_OK : OQ_EDEVICE;
}
