// Path walks over the pair scores of one block, by one wavefront ("DFlash 2:
// Keep Drafting Parallel", section "A lightweight path selector": the one
// serial step walks the scores from the last verified token; sampling draws
// from the same scores).  Shared by the walk kernels (scores staged from
// global memory) and the fused scores-and-walk kernels (scores computed into
// LDS), so both run the same arithmetic.
#pragma once
#include "common.hpp"

namespace dflash2 {

__device__ __forceinline__ void walk_better(float& bv, int& bi, float ov, int oi) {
  if (ov > bv || (ov == bv && oi < bi)) {
    bv = ov;
    bi = oi;
  }
}

// Index-tracking max over one aligned group of 16 lanes (lowest slot on ties);
// every lane of the group ends with the winner.
__device__ __forceinline__ void walk_argmax16(float& bv, int& bi) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) walk_better(bv, bi, __shfl_xor(bv, m, 64), __shfl_xor(bi, m, 64));
}

// Orders the wave's LDS accesses around a step.  WG_SYNC: the workgroup is
// this one wave (a workgroup barrier is free); otherwise other waves of the
// workgroup do not take part, and a wave's LDS operations already execute in
// program order, so only the compiler must not move them.
template <bool WG_SYNC>
__device__ __forceinline__ void walk_sync() {
  if (WG_SYNC)
    __syncthreads();
  else
    __builtin_amdgcn_wave_barrier();
}

// Max-plus (Viterbi) walk: d_0 = S0,  d_t[j] = max_i fl32(d_{t-1}[i] + S[t-1,i,j]),
// lowest i on ties, final slot = lowest j attaining max d_{L-1}, then follow
// the back-pointers.  Lane (q, j) = (lane >> 4, lane & 15) scans the four
// predecessors i = 4q..4q+3 of candidate j; two cross-row exchanges (xor 16,
// xor 32) finish the max with the lowest-index tie rule.  Scores of step t+1
// are prefetched while step t reduces.  S0b [16], Sb [(L-1) x 16 x 16] of this
// block; delta [16] (which may be S0b itself) and the back-pointer rows are
// this wave's LDS scratch: row t (t >= 1, 16 bytes) sits at back1 + (t-1) * bstride.
// Row t is written after every score of step t-1 has been read, so the rows
// may overwrite score blocks already walked (bstride = one block).  When
// sslot is given, lane 0 also leaves the walked slots there.
template <bool WG_SYNC>
__device__ void viterbi_walk(const float* S0b, const float* Sb, const int32_t* top_idx, int b,
                             int L, float* delta, uint8_t* back1, int bstride,
                             int32_t* path_slot, int32_t* path_tok, float* path_score,
                             uint8_t* sslot) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15;
  const int q = lane >> 4;
  if (lane < kTopK) delta[lane] = S0b[lane];
  float s_next[4];
  if (L > 1) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) s_next[ii] = Sb[(q * 4 + ii) * kTopK + j];
  }
  walk_sync<WG_SYNC>();
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
    walk_better(bv, bi, __shfl_xor(bv, 16, 64), __shfl_xor(bi, 16, 64));
    walk_better(bv, bi, __shfl_xor(bv, 32, 64), __shfl_xor(bi, 32, 64));
    walk_sync<WG_SYNC>();
    if (q == 0) {
      delta[j] = bv;
      back1[(t - 1) * bstride + j] = (uint8_t)bi;
    }
    walk_sync<WG_SYNC>();
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
      if (sslot) sslot[t] = (uint8_t)slot;
      if (path_tok) path_tok[(size_t)b * L + t] = top_idx[((size_t)b * L + t) * kTopK + slot];
      if (t > 0) slot = back1[(t - 1) * bstride + slot];
    }
  }
}

// Best-successor walk, the post's own decoder: p_0 = argmax S0, then
// p_t = argmax_j S[t-1, p_{t-1}, j], lowest slot on ties; the score is the fp32
// running sum along the walk.  sS: this block's scores in LDS.  Lanes
// j = lane & 15 hold candidate j; the four quarters of the wave walk the same
// block.  When sslot is given, lane 0 also leaves the walked slots there.
__device__ __forceinline__ void greedy_walk(const float* S0b, const float* sS,
                                            const int32_t* top_idx, int b, int L,
                                            int32_t* path_slot, int32_t* path_tok,
                                            float* path_score, uint8_t* sslot) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15;
  float bv = S0b[j];
  int p = j;
  walk_argmax16(bv, p);
  float score = bv;
  const size_t row = (size_t)b * L;
  if (lane == 0) {
    path_slot[row] = p;
    if (sslot) sslot[0] = (uint8_t)p;
    if (path_tok) path_tok[row] = top_idx[row * kTopK + p];
  }
  for (int t = 1; t < L; ++t) {
    bv = sS[((t - 1) * kTopK + p) * kTopK + j];
    int bi = j;
    walk_argmax16(bv, bi);
    score = score + bv;
    p = bi;
    if (lane == 0) {
      path_slot[row + t] = p;
      if (sslot) sslot[t] = (uint8_t)p;
      if (path_tok) path_tok[row + t] = top_idx[(row + t) * kTopK + p];
    }
  }
  if (lane == 0) path_score[b] = score;
}

// Sampling walk at temperature T = 1 / inv_t, the sampling twin of the greedy
// walk: position t's slot is drawn from softmax(row / T) of the successors of
// the slot drawn before, by inverse CDF in slot order with the uniform u[t].
// s: this lane's S0 value (candidate j = lane & 15); sS: this block's scores
// in LDS; u [L]: this block's uniforms; q receives every position's proposal.
__device__ __forceinline__ void sample_walk(float s, const float* sS, const int32_t* top_idx,
                                            const float* u, float inv_t, int b, int L,
                                            int32_t* path_slot, int32_t* path_tok, float* q) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15;
  const size_t row = (size_t)b * L;
  int p = 0;
  for (int t = 0; t < L; ++t) {
    if (t > 0) s = sS[((t - 1) * kTopK + p) * kTopK + j];
    // softmax over the 16 lanes of each quarter (all four quarters agree)
    float m = s;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const float e = expf((s - m) * inv_t);
    float z = e;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) z += __shfl_xor(z, o, 64);
    const float qj = e / z;
    // inclusive prefix sum in slot order
    float c = qj;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const float n = __shfl_up(c, o, 16);
      if (j >= o) c += n;
    }
    const float ut = u[t];
    // first slot with u < c_j = number of slots with c_j <= u; rounding can
    // leave u above every c_j: then the last slot with q > 0
    const uint64_t le = __ballot(c <= ut) & 0xffffull;
    const uint64_t pos = __ballot(qj > 0.f) & 0xffffull;
    const int first = __popcll(le);
    const int last = pos ? 63 - __clzll(pos) : 0;  // no finite score: slot 0 (q is NaN)
    p = min(first, last);
    if (lane < kTopK) q[(row + t) * kTopK + j] = qj;
    if (lane == 0) {
      path_slot[row + t] = p;
      if (path_tok) path_tok[row + t] = top_idx[(row + t) * kTopK + p];
    }
  }
}

}  // namespace dflash2
