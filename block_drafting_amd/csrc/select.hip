// Max-plus path walk over precomputed pair scores ("DFlash 2: Keep Drafting
// Parallel", section "A lightweight path selector": the one serial step walks
// the scores from the last verified token).  This walk is the exact best
// path (Viterbi):
//   d_0 = S0,  d_t[j] = max_i fl32(d_{t-1}[i] + S[t-1,i,j]),  lowest i on ties,
//   final slot = lowest j attaining max d_{L-1}, then follow the back-pointers.
//
// One wavefront per block.  Lane (q, j) = (lane >> 4, lane & 15) scans the
// four predecessors i = 4q..4q+3 of candidate j; two cross-row exchanges
// (xor 16, xor 32) finish the max with the lowest-index tie rule.  Scores of
// step t+1 are prefetched while step t reduces.
#include "walk.hpp"

namespace dflash2 {
namespace {

__global__ __launch_bounds__(64) void path_select_kernel(const float* __restrict__ S0,
                                                         const float* __restrict__ S,
                                                         const int32_t* __restrict__ top_idx,
                                                         int L, int32_t* __restrict__ path_slot,
                                                         int32_t* __restrict__ path_tok,
                                                         float* __restrict__ path_score) {
  __shared__ float delta[kTopK];
  __shared__ uint8_t back[64][kTopK];
  __shared__ uint8_t sslot[kMaxWalk];
  const int b = blockIdx.x;
  viterbi_walk<true>(S0 + (size_t)b * kTopK, S + (size_t)b * (L - 1) * kTopK * kTopK, top_idx, b,
                     L, delta, &back[1][0], kTopK, path_slot, path_tok, path_score, sslot);
}

// The greedy walk's next row depends on the last argmax, so the wave first
// copies every row the walk might visit ((L-1) x 16 x 16 floats, all loads in
// flight at once) into LDS and then walks there: one memory latency per block
// instead of one per position.
__global__ __launch_bounds__(64) void path_greedy_kernel(const float* __restrict__ S0,
                                                         const float* __restrict__ S,
                                                         const int32_t* __restrict__ top_idx,
                                                         int L, int32_t* __restrict__ path_slot,
                                                         int32_t* __restrict__ path_tok,
                                                         float* __restrict__ path_score) {
  extern __shared__ f32x4_t stage[];  // (L-1) * 64 vectors of 4 scores
  constexpr int kUnroll = 8;
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int n4 = (L - 1) * kTopK * kTopK / 4;
  const f32x4_t* src = reinterpret_cast<const f32x4_t*>(S + (size_t)b * (L - 1) * kTopK * kTopK);
  for (int base = 0; base < n4; base += 64 * kUnroll) {
    f32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int e = base + u * 64 + lane;
      if (e < n4) v[u] = src[e];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int e = base + u * 64 + lane;
      if (e < n4) stage[e] = v[u];
    }
  }
  __syncthreads();
  greedy_walk(S0 + (size_t)b * kTopK, reinterpret_cast<const float*>(stage), top_idx, b, L,
              path_slot, path_tok, path_score, nullptr);
}

__global__ __launch_bounds__(256) void verify_greedy_kernel(const int32_t* __restrict__ path_tok,
                                                            const int32_t* __restrict__ target,
                                                            int B, int L,
                                                            int32_t* __restrict__ accept_len,
                                                            int32_t* __restrict__ next_tok) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int32_t* p = path_tok + (size_t)b * L;
  const int32_t* g = target + (size_t)b * (L + 1);
  int n = 0;
  while (n < L && p[n] == g[n]) ++n;
  accept_len[b] = n + 1;
  if (next_tok) next_tok[b] = g[n];
}

}  // namespace

hipError_t launch_path_select(const float* S0, const float* S, const int32_t* top_idx, int B,
                              int L, int greedy, int32_t* path_slot, int32_t* path_tok,
                              float* path_score, hipStream_t s) {
  if (B == 0) return hipSuccess;
  if (greedy) {
    const size_t lds = (size_t)(L - 1) * kTopK * kTopK * sizeof(float);
    hipLaunchKernelGGL(path_greedy_kernel, dim3((unsigned)B), dim3(64), lds, s, S0, S, top_idx, L,
                       path_slot, path_tok, path_score);
  } else {
    hipLaunchKernelGGL(path_select_kernel, dim3((unsigned)B), dim3(64), 0, s, S0, S, top_idx, L,
                       path_slot, path_tok, path_score);
  }
  return hipGetLastError();
}

hipError_t launch_verify_greedy(const int32_t* path_tok, const int32_t* target, int B, int L,
                                int32_t* accept_len, int32_t* next_tok, hipStream_t s) {
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(verify_greedy_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, s,
                     path_tok, target, B, L, accept_len, next_tok);
  return hipGetLastError();
}

}  // namespace dflash2
