// Attainable-peak probe for the roofline of the LM-head GEMM: the GEMM's
// matrix-core work with its memory traffic taken away.  Each workgroup has
// the GEMM's eight waves (two per SIMD); each wave keeps eight 32 x 32
// accumulators (the GEMM's 128 x 64 wave tile) and issues
// v_mfma_f32_32x32x16_bf16 on operands held in registers, loaded once from
// the caller's buffer (their bit patterns set the power the matrix cores
// draw, and with it the clock).  No LDS, no global traffic in the loop.
#include "common.hpp"

namespace dflash2 {
namespace {

__global__ __launch_bounds__(512) void probe_mfma_kernel(const uint16_t* __restrict__ operands,
                                                         int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // each lane's four A and two B fragments (16 bytes each), as in the GEMM
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(operands) +
                       ((size_t)(blockIdx.x * 8 + wave) * 64 + lane) * 6;
  bf16x8_t fa[4], fb[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) fa[i] = __builtin_bit_cast(bf16x8_t, src[i]);
#pragma unroll
  for (int j = 0; j < 2; ++j) fb[j] = __builtin_bit_cast(bf16x8_t, src[4 + j]);
  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc[i][j][r];
  out[(size_t)blockIdx.x * 512 + threadIdx.x] = s;
}

}  // namespace

size_t probe_mfma_operand_bytes(int nwg) { return (size_t)nwg * 8 * 64 * 6 * 16; }

hipError_t launch_probe_mfma(const void* operands, int nwg, int iters, float* out,
                             hipStream_t s) {
  hipLaunchKernelGGL(probe_mfma_kernel, dim3((unsigned)nwg), dim3(512), 0, s,
                     static_cast<const uint16_t*>(operands), iters, out);
  return hipGetLastError();
}

}  // namespace dflash2
