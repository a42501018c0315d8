// Context gate of the gated pair score ("DFlash 2: Keep Drafting Parallel",
// section "A lightweight path selector", eq. S_t(a,b)): the match between the
// previous token's embedding A(a) and the candidate's B(b) is weighted
// channel by channel by H(h_t), a function of the drafter's hidden state at
// position t.  Here H is a sigmoid of a linear map of h_t:
//   gate[m, k] = sigmoid( sum_c h[m, c] * Wg[k, c] ),   Wg [r, H] (K-contiguous).
//
// bf16: a [M x H] x [H x r] product with r <= 256 is far too narrow for the
// LM-head tiling, so each workgroup owns one 32 x 32 output tile and walks
// the whole K range.  The operand rows are staged through LDS in K slices:
// every 16-byte load of a slice belongs to a run of 16 threads reading 256
// contiguous bytes of one row, so each cache line is fetched whole (matrix
// fragments gathered straight from global memory touch 32 rows per
// instruction and run at a fraction of the L2 bandwidth).  The four waves
// take alternate k-steps of each slice; their partial tiles are added in LDS
// in wave order, so the result does not depend on timing.
#include "common.hpp"

namespace dflash2 {
namespace {

__device__ __forceinline__ float sigmoid(float x) { return 1.0f / (1.0f + expf(-x)); }

// W waves share each tile; W = 8 takes 256-wide K slices (twice the bytes
// in flight per tile, for launches of at most one tile per CU), W = 4
// 128-wide ones (two tiles per CU).  (Sixteen waves with 512-wide slices,
// half the serial chain of slices, ran no faster: a tile's operand stream is
// bound by its CU's L2 bandwidth, not by the chain.)
template <int W>
struct GateCfg {
  static constexpr int kWaves = W;
  static constexpr int kBK = 32 * W;                          // k per LDS slice
  static constexpr int kLd = kBK + 8;                         // padded LDS row (bf16)
  static constexpr int kCpr = kBK / 8;                        // 16-byte chunks per row slice
  static constexpr int kRowsPerPass = 64 * W / kCpr;          // 16
  static constexpr int kPasses = 32 / kRowsPerPass;           // 2 per operand
};

template <int W>
__global__ __launch_bounds__(64 * W) void gate_bf16_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ Wg, float* __restrict__ gate,
    int M, int H, int r) {
  using C = GateCfg<W>;
  constexpr int kGateWaves = C::kWaves;
  constexpr int kGateBK = C::kBK;
  constexpr int kGateLd = C::kLd;
  constexpr int kGateCpr = C::kCpr;
  constexpr int kGateRowsPerPass = C::kRowsPerPass;
  constexpr int kGatePasses = C::kPasses;
  // [buf][A/B] operand slices; after the K loop the same bytes hold the
  // waves' partial tiles
  constexpr int kStageBytes = 2 * 2 * 32 * kGateLd * 2;
  constexpr int kPartBytes = kGateWaves * 16 * 64 * 4;
  __shared__ __attribute__((aligned(16)))
  uint8_t smem[kStageBytes > kPartBytes ? kStageBytes : kPartBytes];
  auto stage = reinterpret_cast<uint16_t(*)[2][32 * kGateLd]>(smem);
  auto part = reinterpret_cast<float(*)[16][64]>(smem);
  const int m0 = blockIdx.x * 32;
  const int n0 = blockIdx.y * 32;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rowsA = min(32, M - m0);
  const int rowsB = min(32, r - n0);
  // Loader role: rows (tid / kGateCpr) + 16 p of each operand, chunk tid % kGateCpr.
  // Rows past the edge repeat the last row (their results are never stored).
  const int lrow = tid / kGateCpr;
  const int lk = (tid % kGateCpr) * 8;
  const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(h + (size_t)m0 * H), (short)0, rowsA * H * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(Wg + (size_t)n0 * H), (short)0, rowsB * H * 2, 0x00020000);
  int offA[kGatePasses], offB[kGatePasses];
#pragma unroll
  for (int p = 0; p < kGatePasses; ++p) {
    offA[p] = (min(lrow + p * kGateRowsPerPass, rowsA - 1) * H + lk) * 2;
    offB[p] = (min(lrow + p * kGateRowsPerPass, rowsB - 1) * H + lk) * 2;
  }
  const int nslices = (H + kGateBK - 1) / kGateBK;
  // Two register staging sets keep two slices of loads in flight while the
  // one before them is multiplied.  Slices past the end re-read the last
  // slice (in range, never used).
  u32x4_t R0[2 * kGatePasses], R1[2 * kGatePasses];
  auto gload = [&](u32x4_t(&R)[2 * kGatePasses], int sl) {
    const int k = min(sl, nslices - 1) * kGateBK;
    const bool in = k + lk < H;  // H % 8 == 0: a chunk is wholly inside or outside
    const u32x4_t z = {0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p < kGatePasses; ++p) {
      const u32x4_t va = __builtin_amdgcn_raw_buffer_load_b128(rsA, offA[p] + k * 2, 0, 0);
      const u32x4_t vb = __builtin_amdgcn_raw_buffer_load_b128(rsB, offB[p] + k * 2, 0, 0);
      R[p] = in ? va : z;
      R[kGatePasses + p] = in ? vb : z;
    }
  };
  auto sstore = [&](const u32x4_t(&R)[2 * kGatePasses], int buf) {
#pragma unroll
    for (int p = 0; p < kGatePasses; ++p) {
      const int at = (lrow + p * kGateRowsPerPass) * kGateLd + lk;
      *reinterpret_cast<u32x4_t*>(&stage[buf][0][at]) = R[p];
      *reinterpret_cast<u32x4_t*>(&stage[buf][1][at]) = R[kGatePasses + p];
    }
  };

  f32x16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  // MFMA fragment of lane l: row l % 32, k values 8 (l / 32) .. +7 of a k-step.
  const int frag = (lane & 31) * kGateLd + (lane >> 5) * 8;
  auto multiply = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kGateBK / 16 / kGateWaves; ++j) {
      const int ks = wave + j * kGateWaves;
      const bf16x8_t fa = *reinterpret_cast<const bf16x8_t*>(&stage[buf][0][frag + ks * 16]);
      const bf16x8_t fb = *reinterpret_cast<const bf16x8_t*>(&stage[buf][1][frag + ks * 16]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc, 0, 0, 0);
    }
  };
  gload(R0, 0);
  gload(R1, 1);
  sstore(R0, 0);
  __syncthreads();
  // Slice sl sits in LDS buffer sl & 1; the set that carried it reloads
  // slice sl + 2, the other set (slice sl + 1) is stored after the MFMAs.
  for (int sl = 0; sl < nslices; sl += 2) {
    gload(R0, sl + 2);
    multiply(0);
    sstore(R1, 1);
    __syncthreads();
    if (sl + 1 >= nslices) break;
    gload(R1, sl + 3);
    multiply(1);
    sstore(R0, 0);
    __syncthreads();
  }
  __syncthreads();  // every wave is done with the stages
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
    const uint16_t* hb = static_cast<const uint16_t*>(h);
    const uint16_t* wb = static_cast<const uint16_t*>(Wg);
    if ((long long)grid.x * grid.y <= 256)
      hipLaunchKernelGGL(gate_bf16_kernel<8>, grid, dim3(64 * 8), 0, s, hb, wb, gate, M, H, r);
    else
      hipLaunchKernelGGL(gate_bf16_kernel<4>, grid, dim3(64 * 4), 0, s, hb, wb, gate, M, H, r);
  } else {
    const long long n = (long long)M * r;
    hipLaunchKernelGGL(gate_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       static_cast<const float*>(h), static_cast<const float*>(Wg), gate, M, H,
                       r);
  }
  return hipGetLastError();
}

}  // namespace dflash2
