// Per-tensor FP8 (e4m3) quantisation: the operand preparation for the FP8
// forward. The pages name an FP8 forward path (page "r/mlscaling", FA3
// bullet) without a recipe; the one here is per-tensor amax scaling:
//   amax = max |x|;  code = e4m3_rne(x * (448 / amax));  descale = amax / 448.
// Three kernels on one stream: zero the accumulator, reduce amax with an
// unsigned atomic max on the float bits (valid for non-negative floats),
// then encode; the last one also turns amax into the descale in place.
#include "common.hpp"
#include "launch.hpp"

namespace fa {

__global__ void quant_init_kernel(float* acc) { *acc = 0.f; }

__global__ void __launch_bounds__(256) quant_amax_kernel(const float* __restrict__ x, size_t n, float* acc) {
  __shared__ float red[4];
  float m = 0.f;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) m = fmaxf(m, fabsf(x[i]));
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    atomicMax(reinterpret_cast<unsigned int*>(acc), __float_as_uint(m));
  }
}

// Encodes 4 consecutive elements per thread; `acc` holds amax on entry and
// the descale on exit (written after every block has read amax: the encode
// grid reads it once, and only the finish kernel overwrites it).
__global__ void __launch_bounds__(256) quant_encode_kernel(const float* __restrict__ x, size_t n,
                                                           unsigned char* __restrict__ codes, const float* acc) {
  const float amax = *acc;
  const float s = amax > 0.f ? 448.f / amax : 1.f;
  const size_t stride = (size_t)gridDim.x * blockDim.x * 4;
  for (size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
    if (i + 4 <= n) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(x + i);
      int w = cvt_fp8x2<false>(v[0] * s, v[1] * s, 0);
      w = cvt_fp8x2<true>(v[2] * s, v[3] * s, w);
      *reinterpret_cast<int*>(codes + i) = w;
    } else {
      for (size_t j = i; j < n; ++j) codes[j] = (unsigned char)(cvt_fp8x2<false>(x[j] * s, 0.f, 0) & 0xff);
    }
  }
}

__global__ void quant_finish_kernel(float* acc) {
  const float amax = *acc;
  *acc = amax > 0.f ? amax / 448.f : 1.f;
}

hipError_t quantize_fp8_launch(const float* x, size_t n, void* codes, float* descale, hipStream_t st) {
  hipLaunchKernelGGL(quant_init_kernel, dim3(1), dim3(1), 0, st, descale);
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(quant_amax_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, n, descale);
  size_t eblocks = (n + 1023) / 1024;
  if (eblocks > 8192) eblocks = 8192;
  hipLaunchKernelGGL(quant_encode_kernel, dim3((unsigned)eblocks), dim3(256), 0, st, x, n,
                     reinterpret_cast<unsigned char*>(codes), descale);
  hipLaunchKernelGGL(quant_finish_kernel, dim3(1), dim3(1), 0, st, descale);
  return hipGetLastError();
}

}  // namespace fa
