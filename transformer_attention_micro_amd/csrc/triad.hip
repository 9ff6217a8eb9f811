// HBM bandwidth calibration: the STREAM triad a[i] = b[i] + s * c[i]
// (page "TileOPs-Metax benchmarks/hardware", sections "HBM Bandwidth" and
// "Methodology": two reads and one write per element, 128-bit vector
// accesses, GPU-side event timing).  12 bytes move per fp32 element.
#include "kb_device.hpp"

namespace {

__global__ void triad_vec_kernel(float4 *__restrict__ a, const float4 *__restrict__ b,
                                 const float4 *__restrict__ c, float s, size_t n4) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const float4 x = b[i], y = c[i];
    a[i] = make_float4(fmaf(s, y.x, x.x), fmaf(s, y.y, x.y), fmaf(s, y.z, x.z), fmaf(s, y.w, x.w));
  }
}

__global__ void triad_scalar_kernel(float *__restrict__ a, const float *__restrict__ b,
                                    const float *__restrict__ c, float s, size_t lo, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = lo + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    a[i] = fmaf(s, c[i], b[i]);
}

}  // namespace

hipError_t kb_launch_triad(float *a, const float *b, const float *c, float s, size_t n, int block,
                           hipStream_t stream) {
  const bool aligned = ((uintptr_t)a | (uintptr_t)b | (uintptr_t)c) % 16 == 0;
  const size_t n4 = aligned ? n / 4 : 0;
  if (n4) {
    const size_t blocks = (n4 + block - 1) / block;
    const unsigned grid = (unsigned)(blocks < (1u << 20) ? blocks : (1u << 20));
    hipLaunchKernelGGL(triad_vec_kernel, dim3(grid), dim3(block), 0, stream, (float4 *)a,
                       (const float4 *)b, (const float4 *)c, s, n4);
  }
  if (4 * n4 < n) {
    const size_t rest = n - 4 * n4;
    const size_t blocks = (rest + block - 1) / block;
    const unsigned grid = (unsigned)(blocks < (1u << 20) ? blocks : (1u << 20));
    hipLaunchKernelGGL(triad_scalar_kernel, dim3(grid), dim3(block), 0, stream, a, b, c, s, 4 * n4, n);
  }
  return hipGetLastError();
}
