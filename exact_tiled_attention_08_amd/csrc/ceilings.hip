// Measured ceilings for the roofline denominators: what this GPU actually
// sustains for the two resources the attention kernels are bound by.
//
//  * ceiling_mfma_kernel: nothing but v_mfma_f32_32x32x16_bf16 on register
//    operands, four independent accumulator chains per wave, two waves per
//    SIMD -- the matrix-core rate the prefill can at best approach.  The rate
//    depends on the data: on random operands the chip holds a lower clock
//    than on small constants (power), so both are measured.
//  * ceiling_read_kernel: a streaming read of a large buffer with 16-byte
//    nontemporal loads, each work-group on its own contiguous run with eight
//    loads in flight per lane -- the HBM rate the decode can at best approach.
//
// These are measurement aids; no attention entry point uses them.
#include "fa_ceilings.h"

#include <hip/hip_runtime.h>

#include "fa_device.hpp"

namespace fa {

// Each wave holds eight A and eight B fragments and cycles through them, so
// the operands change from product to product as they do in a real kernel.
// With `src` they are random bf16 values; without, small constants (few bits
// toggle, so the matrix cores draw far less power and the clock stays high).
template <bool DATA>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void ceiling_mfma_kernel(
    const bf16x8* __restrict__ src, float* out, int iters) {
  const int tid = threadIdx.x;
  bf16x8 a[8], b[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    if (DATA) {
      a[u] = src[((size_t)blockIdx.x * 16 + u) * 256 + tid];
      b[u] = src[((size_t)blockIdx.x * 16 + 8 + u) * 256 + tid];
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        a[u][t] = (__bf16)((float)((tid + t + u) & 7) * 0.0078125f);
        b[u][t] = (__bf16)((float)((tid * 3 + t + u) & 7) * 0.0078125f);
      }
    }
  }
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = mfma32x32x16(a[u], b[(u + c) & 7], acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[(size_t)blockIdx.x * 256 + tid] = s;
}

// Each work-group streams its own contiguous run of the buffer (a whole
// multiple of 256 x 8 16-byte units), eight nontemporal loads in flight per
// lane; the units past the last run are read grid-stride.
__global__ __launch_bounds__(256) void ceiling_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                           unsigned* out) {
  constexpr int U = 8;
  const size_t per = (n16 / gridDim.x) / (256 * U) * (256 * U);
  const u32x4* p = src + (size_t)blockIdx.x * per + threadIdx.x;
  unsigned acc = 0;
  for (size_t i = 0; i < per; i += 256 * U) {
    u32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = __builtin_nontemporal_load(p + i + u * 256);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= x[u][0] ^ x[u][1] ^ x[u][2] ^ x[u][3];
  }
  for (size_t i = (size_t)gridDim.x * per + (size_t)blockIdx.x * 256 + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * 256) {
    const u32x4 x = __builtin_nontemporal_load(src + i);
    acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace fa

extern "C" {

int fa_ceiling_mfma(const void* src, float* out, int blocks, int iters, void* stream) {
  if (out == nullptr || blocks < 1 || iters < 1 || ((uintptr_t)src % 16) != 0) return -1;
  if (src != nullptr)
    hipLaunchKernelGGL(fa::ceiling_mfma_kernel<true>, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       (const fa::bf16x8*)src, out, iters);
  else
    hipLaunchKernelGGL(fa::ceiling_mfma_kernel<false>, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       (const fa::bf16x8*)nullptr, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int fa_ceiling_read(const void* src, size_t bytes, unsigned* out, int blocks, void* stream) {
  if (src == nullptr || out == nullptr || blocks < 1 || bytes % 16 != 0 || ((uintptr_t)src % 16) != 0) return -1;
  hipLaunchKernelGGL(fa::ceiling_read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     (const fa::u32x4*)src, bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
