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
#include "common.hpp"

namespace dflash2 {
namespace {

__device__ __forceinline__ void better(float& bv, int& bi, float ov, int oi) {
  if (ov > bv || (ov == bv && oi < bi)) {
    bv = ov;
    bi = oi;
  }
}

__global__ __launch_bounds__(64) void path_select_kernel(const float* __restrict__ S0,
                                                         const float* __restrict__ S,
                                                         const int32_t* __restrict__ top_idx,
                                                         int L, int32_t* __restrict__ path_slot,
                                                         int32_t* __restrict__ path_tok,
                                                         float* __restrict__ path_score) {
  __shared__ float delta[kTopK];
  __shared__ uint8_t back[64][kTopK];
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int j = lane & 15;
  const int q = lane >> 4;
  if (lane < kTopK) delta[lane] = S0[(size_t)b * kTopK + lane];
  const float* Sb = S + (size_t)b * (L - 1) * kTopK * kTopK;
  float s_next[4];
  if (L > 1) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) s_next[ii] = Sb[(q * 4 + ii) * kTopK + j];
  }
  __syncthreads();
  for (int t = 1; t < L; ++t) {
    float s_cur[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) s_cur[ii] = s_next[ii];
    if (t + 1 < L) {
      const float* St = Sb + (size_t)t * kTopK * kTopK;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) s_next[ii] = St[(q * 4 + ii) * kTopK + j];
    }
    float bv = delta[q * 4] + s_cur[0];
    int bi = q * 4;
#pragma unroll
    for (int ii = 1; ii < 4; ++ii) {
      const float v = delta[q * 4 + ii] + s_cur[ii];
      if (v > bv) {
        bv = v;
        bi = q * 4 + ii;
      }
    }
    better(bv, bi, __shfl_xor(bv, 16, 64), __shfl_xor(bi, 16, 64));
    better(bv, bi, __shfl_xor(bv, 32, 64), __shfl_xor(bi, 32, 64));
    __syncthreads();
    if (q == 0) {
      delta[j] = bv;
      back[t][j] = (uint8_t)bi;
    }
    __syncthreads();
  }
  if (lane == 0) {
    int js = 0;
    float best = delta[0];
    for (int jj = 1; jj < kTopK; ++jj) {
      if (delta[jj] > best) {
        best = delta[jj];
        js = jj;
      }
    }
    path_score[b] = best;
    int slot = js;
    for (int t = L - 1; t >= 0; --t) {
      path_slot[(size_t)b * L + t] = slot;
      if (path_tok) path_tok[(size_t)b * L + t] = top_idx[((size_t)b * L + t) * kTopK + slot];
      if (t > 0) slot = back[t][slot];
    }
  }
}

// Index-tracking max over one aligned group of 16 lanes (lowest slot on ties);
// every lane of the group ends with the winner.
__device__ __forceinline__ void argmax16(float& bv, int& bi) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) better(bv, bi, __shfl_xor(bv, m, 64), __shfl_xor(bi, m, 64));
}

// Best-successor walk, the post's own decoder: p_0 = argmax S0, then
// p_t = argmax_j S[t-1, p_{t-1}, j], lowest slot on ties; the score is the fp32
// running sum along the walk.  Each step depends on the previous argmax, so
// the wave first copies every row the walk might visit ((L-1) x 16 x 16
// floats, all loads in flight at once) into LDS and then walks there: one
// memory latency per block instead of one per position.  Lanes j = lane & 15
// hold candidate j; the four quarters of the wave walk the same block.
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
  const int j = lane & 15;
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
  float bv = S0[(size_t)b * kTopK + j];
  int p = j;
  argmax16(bv, p);
  float score = bv;
  const size_t row = (size_t)b * L;
  if (lane == 0) {
    path_slot[row] = p;
    if (path_tok) path_tok[row] = top_idx[row * kTopK + p];
  }
  __syncthreads();
  const float* sS = reinterpret_cast<const float*>(stage);
  for (int t = 1; t < L; ++t) {
    bv = sS[((t - 1) * kTopK + p) * kTopK + j];
    int bi = j;
    argmax16(bv, bi);
    score = score + bv;
    p = bi;
    if (lane == 0) {
      path_slot[row + t] = p;
      if (path_tok) path_tok[row + t] = top_idx[(row + t) * kTopK + p];
    }
  }
  if (lane == 0) path_score[b] = score;
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
