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

template <int J>
__device__ __forceinline__ void walk_better_xor(float& bv, int& bi) {
  walk_better(bv, bi, __uint_as_float(xor_lane<J>(__float_as_uint(bv))),
              (int)xor_lane<J>((uint32_t)bi));
}

// Index-tracking max over one aligned group of 16 lanes (lowest slot on ties);
// every lane of the group ends with the winner.  DPP exchanges.
__device__ __forceinline__ void walk_argmax16(float& bv, int& bi) {
  walk_better_xor<1>(bv, bi);
  walk_better_xor<2>(bv, bi);
  walk_better_xor<4>(bv, bi);
  walk_better_xor<8>(bv, bi);
}

// Max / sum over one aligned group of 16 lanes, in the butterfly order
// 1, 2, 4, 8 (DPP exchanges).
__device__ __forceinline__ float group16_max(float v) {
  v = fmaxf(v, __uint_as_float(xor_lane<1>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(xor_lane<2>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(xor_lane<4>(__float_as_uint(v))));
  return fmaxf(v, __uint_as_float(xor_lane<8>(__float_as_uint(v))));
}
__device__ __forceinline__ float group16_sum(float v) {
  v += __uint_as_float(xor_lane<1>(__float_as_uint(v)));
  v += __uint_as_float(xor_lane<2>(__float_as_uint(v)));
  v += __uint_as_float(xor_lane<4>(__float_as_uint(v)));
  return v + __uint_as_float(xor_lane<8>(__float_as_uint(v)));
}

// Inclusive prefix sum within each group of 16 lanes (a DPP row): row_shr
// 1, 2, 4, 8, a lane with no source adding nothing.
__device__ __forceinline__ float group16_scan(float v) {
  const int j = threadIdx.x & 15;
  float n;
  n = __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x111, 0xf, 0xf, false));
  if (j >= 1) v += n;
  n = __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x112, 0xf, 0xf, false));
  if (j >= 2) v += n;
  n = __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x114, 0xf, 0xf, false));
  if (j >= 4) v += n;
  n = __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x118, 0xf, 0xf, false));
  if (j >= 8) v += n;
  return v;
}

// Every walk ends the same way: lane t (t < L) holds the slot walked at
// position t; it writes path_slot (and sslot when given) and looks up its
// token, all positions at once (one memory round trip per block instead of
// one per position).  Returns the token in lanes t < L, -1 elsewhere.
__device__ __forceinline__ int walk_finish(int my_slot, const int32_t* top_idx, int b, int L,
                                           int32_t* path_slot, int32_t* path_tok,
                                           uint8_t* sslot) {
  const int lane = threadIdx.x & 63;
  int tok = -1;
  if (lane < L) {
    const size_t rt = (size_t)b * L + lane;
    path_slot[rt] = my_slot;
    if (sslot) sslot[lane] = (uint8_t)my_slot;
    tok = top_idx[rt * kTopK + my_slot];
    if (path_tok) path_tok[rt] = tok;
  }
  return tok;
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
// may overwrite score blocks already walked (bstride = one block).  sslot
// (LDS, L bytes) receives the walked slots.  Returns lane t's token (t < L).
template <bool WG_SYNC>
__device__ int viterbi_walk(const float* S0b, const float* Sb, const int32_t* top_idx, int b,
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
    walk_better_xor<16>(bv, bi);
    walk_better_xor<32>(bv, bi);
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
      sslot[t] = (uint8_t)slot;
      if (t > 0) slot = back1[(t - 1) * bstride + slot];
    }
  }
  walk_sync<WG_SYNC>();
  const int my_slot = lane < L ? sslot[lane] : 0;
  return walk_finish(my_slot, top_idx, b, L, path_slot, path_tok, nullptr);
}

// Best-successor walk, the post's own decoder: p_0 = argmax S0, then
// p_t = argmax_j S[t-1, p_{t-1}, j], lowest slot on ties; the score is the fp32
// running sum along the walk.  sS: this block's scores in LDS.  Lanes
// j = lane & 15 hold candidate j; the four quarters of the wave walk the same
// block.  When sslot is given, the walked slots are left there.  Returns
// lane t's token (t < L).
__device__ __forceinline__ int greedy_walk(const float* S0b, const float* sS,
                                           const int32_t* top_idx, int b, int L,
                                           int32_t* path_slot, int32_t* path_tok,
                                           float* path_score, uint8_t* sslot) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15;
  float bv = S0b[j];
  int p = j;
  walk_argmax16(bv, p);
  float score = bv;
  int my_slot = p;  // lane t keeps the slot of position t
  for (int t = 1; t < L; ++t) {
    bv = sS[((t - 1) * kTopK + p) * kTopK + j];
    int bi = j;
    walk_argmax16(bv, bi);
    score = score + bv;
    p = bi;
    if (lane == t) my_slot = p;
  }
  if (lane == 0) path_score[b] = score;
  return walk_finish(my_slot, top_idx, b, L, path_slot, path_tok, sslot);
}

// Backward messages of the whole-path distribution P(path) proportional to
// exp(score / T), the sampling twin of the max-plus walk: beta[L-1][.] = 0,
//   beta[t][i] = log sum_j exp(S[t, i, j] / T + beta[t+1][j]),  t = L-2 .. 0,
// in fp32 with each row shifted by its maximum.  Lane (q, j) = (lane >> 4,
// lane & 15) holds S[t, 4q + ii, j] for ii < 4; each row's max and sum reduce
// over the 16 lanes of its quarter (DPP), and lane (q, ii) writes row 4q + ii.
// sS: this block's scores in LDS; beta: [L][16] in LDS.  One wave.
__device__ __forceinline__ void path_messages(const float* sS, float inv_t, int L, float* beta) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15;
  const int q = lane >> 4;
  if (lane < kTopK) beta[(L - 1) * kTopK + lane] = 0.f;
  __builtin_amdgcn_wave_barrier();
  for (int t = L - 2; t >= 0; --t) {
    const float bn = beta[(t + 1) * kTopK + j];
    float mine = 0.f;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const float a = sS[(t * kTopK + 4 * q + ii) * kTopK + j] * inv_t + bn;
      const float m = group16_max(a);
      const float z = group16_sum(expf(a - m));
      if (j == ii) mine = m + logf(z);
    }
    __builtin_amdgcn_wave_barrier();
    if (j < 4) beta[t * kTopK + 4 * q + j] = mine;
    __builtin_amdgcn_wave_barrier();
  }
}

// Sampling walk at temperature T = 1 / inv_t.  Without messages (beta
// NULL), the sampling twin of the greedy walk: position t's slot is drawn
// from softmax(row / T) of the successors of the slot drawn before.  With
// the backward messages of path_messages, a draw of the whole path from
// exp(score / T): position t's slot is drawn from softmax(row / T +
// beta[t]), the conditional of slot t given the slots before it.  Draws are
// by inverse CDF in slot order with the uniform u[t].  s: this lane's S0
// value (candidate j = lane & 15); sS: this block's scores in LDS; u [L]:
// this block's uniforms; q receives every position's proposal.
__device__ __forceinline__ int sample_walk(float s, const float* sS, const int32_t* top_idx,
                                           const float* u, float inv_t, int b, int L,
                                           int32_t* path_slot, int32_t* path_tok, float* q,
                                           const float* beta = nullptr) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15;
  const size_t row = (size_t)b * L;
  const float my_u = lane < L ? u[lane] : 0.f;  // the uniforms, one per lane, loaded up front
  int p = 0;
  int my_slot = 0;  // lane t keeps the slot of position t
  for (int t = 0; t < L; ++t) {
    if (t > 0) s = sS[((t - 1) * kTopK + p) * kTopK + j];
    // softmax over the 16 lanes of each quarter (all four quarters agree)
    float e;
    if (beta) {
      const float a = s * inv_t + beta[t * kTopK + j];
      e = expf(a - group16_max(a));
    } else {
      const float m = group16_max(s);
      e = expf((s - m) * inv_t);
    }
    const float z = group16_sum(e);
    const float qj = e / z;
    // inclusive prefix sum in slot order
    const float c = group16_scan(qj);
    const float ut = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(my_u), t));
    // first slot with u < c_j = number of slots with c_j <= u; rounding can
    // leave u above every c_j: then the last slot with q > 0
    const uint64_t le = __ballot(c <= ut) & 0xffffull;
    const uint64_t pos = __ballot(qj > 0.f) & 0xffffull;
    const int first = __popcll(le);
    const int last = pos ? 63 - __clzll(pos) : 0;  // no finite score: slot 0 (q is NaN)
    p = min(first, last);
    if (lane < kTopK) q[(row + t) * kTopK + j] = qj;
    if (lane == t) my_slot = p;
  }
  return walk_finish(my_slot, top_idx, b, L, path_slot, path_tok, nullptr);
}

}  // namespace dflash2
