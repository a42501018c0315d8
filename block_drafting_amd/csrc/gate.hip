// Context gate of the gated pair score ("DFlash 2: Keep Drafting Parallel",
// section "A lightweight path selector", eq. S_t(a,b)): the match between the
// previous token's embedding A(a) and the candidate's B(b) is weighted
// channel by channel by H(h_t), a function of the drafter's hidden state at
// position t.  Here H is a sigmoid of a linear map of h_t:
//   gate[m, k] = sigmoid( sum_c h[m, c] * Wg[k, c] ),   Wg [r, H] (K-contiguous).
//
// bf16: a [M x H] x [H x r] product with r <= 256 is far too narrow for the
// LM-head tiling, so each workgroup owns one 32 x 32 output tile and splits
// the K range over its eight waves.  A wave multiplies straight from global
// memory (its operand fragment per k-step is one 16-byte run of a row, the
// whole tile's rows stay hot in L2 across the workgroups that share them),
// then the eight partial tiles are added in LDS in wave order, so the result
// does not depend on timing.
#include "common.hpp"

namespace dflash2 {
namespace {

__device__ __forceinline__ float sigmoid(float x) { return 1.0f / (1.0f + expf(-x)); }

constexpr int kGateWaves = 8;
constexpr int kGateBatch = 4;  // k-steps whose loads are issued together

__global__ __launch_bounds__(64 * kGateWaves) void gate_bf16_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ Wg, float* __restrict__ gate,
    int M, int H, int r) {
  __shared__ float part[kGateWaves][16][64];
  const int m0 = blockIdx.x * 32;
  const int n0 = blockIdx.y * 32;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // Lane l supplies row l % 32 of each 32-row operand and k values
  // 8 * (l / 32) .. +7 of each 16-wide k-step.  Rows past the edge repeat the
  // last row (their results are never stored).
  const int rowsA = min(32, M - m0);
  const int rowsB = min(32, r - n0);
  const int ra = min(lane & 31, rowsA - 1);
  const int rb = min(lane & 31, rowsB - 1);
  const int kof = (lane >> 5) * 8;
  const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(h + (size_t)m0 * H), (short)0, rowsA * H * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(Wg + (size_t)n0 * H), (short)0, rowsB * H * 2, 0x00020000);
  const int offA = (ra * H + kof) * 2;
  const int offB = (rb * H + kof) * 2;

  const int ksteps = (H + 15) / 16;
  const int per = (ksteps + kGateWaves - 1) / kGateWaves;
  const int ks0 = min(ksteps, wave * per);
  const int ks1 = min(ksteps, ks0 + per);
  f32x16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  for (int ks = ks0; ks < ks1; ks += kGateBatch) {
    u32x4_t a[kGateBatch], b[kGateBatch];
#pragma unroll
    for (int u = 0; u < kGateBatch; ++u) {
      // steps past ks1 re-read step ks (in range) and are discarded below
      const int kk = ks + u < ks1 ? ks + u : ks;
      a[u] = __builtin_amdgcn_raw_buffer_load_b128(rsA, offA + kk * 32, 0, 0);
      b[u] = __builtin_amdgcn_raw_buffer_load_b128(rsB, offB + kk * 32, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kGateBatch; ++u) {
      // H % 16 == 8 leaves the upper half of the last k-step past the row end
      const bool live = ks + u < ks1 && (ks + u) * 16 + kof < H;
      const u32x4_t z = {0, 0, 0, 0};
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8_t, live ? a[u] : z),
          __builtin_bit_cast(bf16x8_t, live ? b[u] : z), acc, 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) part[wave][i][lane] = acc[i];
  __syncthreads();
  for (int o = tid; o < 16 * 64; o += 64 * kGateWaves) {
    const int reg = o >> 6;
    const int ln = o & 63;
    float s = part[0][reg][ln];
#pragma unroll
    for (int w = 1; w < kGateWaves; ++w) s += part[w][reg][ln];
    // accumulator register reg of lane ln holds C[row][col]:
    const int row = 8 * (reg >> 2) + 4 * (ln >> 5) + (reg & 3);
    const int col = ln & 31;
    if (row < rowsA && col < rowsB) gate[(size_t)(m0 + row) * r + n0 + col] = sigmoid(s);
  }
}

// fp32 operands (small models): one thread per output, plain fp32 dot.
__global__ __launch_bounds__(256) void gate_f32_kernel(const float* __restrict__ h,
                                                       const float* __restrict__ Wg,
                                                       float* __restrict__ gate, int M, int H,
                                                       int r) {
  const long long o = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (o >= (long long)M * r) return;
  const int m = (int)(o / r);
  const int k = (int)(o - (long long)m * r);
  const f32x4_t* hr = reinterpret_cast<const f32x4_t*>(h + (size_t)m * H);
  const f32x4_t* wr = reinterpret_cast<const f32x4_t*>(Wg + (size_t)k * H);
  float s = 0.f;
  for (int c = 0; c < H / 4; ++c) {
    const f32x4_t x = hr[c];
    const f32x4_t w = wr[c];
    s = fmaf(x[0], w[0], s);
    s = fmaf(x[1], w[1], s);
    s = fmaf(x[2], w[2], s);
    s = fmaf(x[3], w[3], s);
  }
  gate[o] = sigmoid(s);
}

}  // namespace

hipError_t launch_context_gate(const void* h, const void* Wg, float* gate, int M, int H, int r,
                               int dtype, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (dtype == 1) {
    const dim3 grid((unsigned)((M + 31) / 32), (unsigned)((r + 31) / 32));
    hipLaunchKernelGGL(gate_bf16_kernel, grid, dim3(64 * kGateWaves), 0, s,
                       static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(Wg), gate, M,
                       H, r);
  } else {
    const long long n = (long long)M * r;
    hipLaunchKernelGGL(gate_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       static_cast<const float*>(h), static_cast<const float*>(Wg), gate, M, H,
                       r);
  }
  return hipGetLastError();
}

}  // namespace dflash2
