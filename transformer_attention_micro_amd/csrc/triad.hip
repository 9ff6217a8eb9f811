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

// Reference bandwidth kernels of the same page ("HBM Bandwidth": copy,
// read-only and write-only beside the triad), 128-bit accesses, grid-stride.
__global__ void copy_vec_kernel(float4 *__restrict__ a, const float4 *__restrict__ b, size_t n4) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) a[i] = b[i];
}

// Read-only: every element is read and summed; the sum is stored (into a,
// within its n elements) only in the case that it equals `s`, which callers
// make impossible (NaN), so no bytes are written.
__global__ void read_vec_kernel(float *__restrict__ a, const float4 *__restrict__ b, float s, size_t n4) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  float acc = 0.f;
  for (size_t i = t; i < n4; i += stride) {
    const float4 x = b[i];
    acc += (x.x + x.y) + (x.z + x.w);
  }
  if (acc == s && t < 4 * n4) a[t] = acc;
}

__global__ void write_vec_kernel(float4 *__restrict__ a, float s, size_t n4) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
    a[i] = make_float4(s, s, s, s);
}

}  // namespace

// kind 1 copy (a = b), 2 read (b), 3 write (a = s); n a multiple of 4 and
// 16-byte aligned operands (checked by the caller).
hipError_t kb_launch_stream(int kind, float *a, const float *b, float s, size_t n, int block,
                            hipStream_t stream) {
  const size_t n4 = n / 4;
  const size_t blocks = (n4 + block - 1) / block;
  const unsigned grid = (unsigned)(blocks < (1u << 20) ? blocks : (1u << 20));
  switch (kind) {
    case 1:
      hipLaunchKernelGGL(copy_vec_kernel, dim3(grid), dim3(block), 0, stream, (float4 *)a, (const float4 *)b, n4);
      break;
    case 2:
      hipLaunchKernelGGL(read_vec_kernel, dim3(grid), dim3(block), 0, stream, a, (const float4 *)b, s, n4);
      break;
    case 3:
      hipLaunchKernelGGL(write_vec_kernel, dim3(grid), dim3(block), 0, stream, (float4 *)a, s, n4);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

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
