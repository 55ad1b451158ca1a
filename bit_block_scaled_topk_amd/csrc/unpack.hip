// unpack.hip -- exact NVFP4 -> bf16 unpack that drops the per-tensor global
// (gllm PR #91, "bf16 NVFP4 GEMM (CUDA)"): the e2m1 magnitudes carry 2
// significant bits and an e4m3 scale 4, so their product needs 6 and bf16's 8
// hold it without rounding.  One thread per 32-element
// group: a 16-byte code load, two scale bytes, 64 bytes of bf16 out.
#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace moe {

namespace {

__global__ void __launch_bounds__(256)
k_unpack_bf16(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales, long rows,
              int cols, uint16_t *__restrict__ out) {
  const int gpr = cols / 32;  // groups per row
  long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= rows * gpr) return;
  long r = gid / gpr;
  int g = (int)(gid - r * gpr);
  u32x4_t c = *(const u32x4_t *)(codes + (size_t)r * (cols / 2) + (size_t)g * 16);
  const uint8_t *sp = scales + (size_t)r * (cols / 16) + (size_t)g * 2;
  float s0, s1;
  e4m3x2_to_f32((uint32_t)sp[0] | ((uint32_t)sp[1] << 8), s0, s1);
  u32x4_t *o = (u32x4_t *)(out + (size_t)r * cols + (size_t)g * 32);
  o[0] = dq8_bf16(c[0], s0);
  o[1] = dq8_bf16(c[1], s0);
  o[2] = dq8_bf16(c[2], s1);
  o[3] = dq8_bf16(c[3], s1);
}

}  // namespace

hipError_t launch_unpack_bf16(const uint8_t *codes, const uint8_t *scales, long rows, int cols,
                              uint16_t *out, hipStream_t stream) {
  long groups = rows * (cols / 32);
  long blocks = (groups + 255) / 256;
  hipLaunchKernelGGL(k_unpack_bf16, dim3((unsigned)blocks), dim3(256), 0, stream, codes, scales, rows, cols,
                     out);
  return hipGetLastError();
}

}  // namespace moe
