// Sampling at T > 0 and lossless verification ("DFlash 2: Keep Drafting
// Parallel", section "A lightweight path selector": besides the greedy walk,
// sampling draws from the same precomputed scores, and rejection sampling
// restores the target's exact distribution).
//
// path_sample_kernel    the sampling twin of the greedy walk: position t's
//                       slot is drawn from softmax(row / T) of the successors
//                       of the slot drawn before, by inverse CDF with the
//                       caller's uniforms.  One wave per block, scores staged
//                       in LDS as in the greedy walk.
// target_lse_kernel     log sum_v exp(z[v] / T) of every target row: one
//                       streaming pass with a running max, rescaled once per
//                       batch of 16 values (HBM-bound).
// verify_rejection_kernel  the speculative-sampling rule: accept x_t when
//                       u * q_t(x_t) < p_t(x_t); at the first rejection (or
//                       after L acceptances) draw the verifier's token from
//                       max(0, p - q) (or p) by inverse CDF in token order.
//                       One workgroup per block; the draw sums p over
//                       256-token tiles wave by wave, moves the 16
//                       candidates' corrections into their tiles, scans the
//                       tile sums, then scans inside the chosen tile.
// verify_rejection_lazy_kernel  the same rule with each target row's
//                       log-sum-exp computed here, only for the rows the
//                       accept test reaches: one pass per row keeps every
//                       tile's (reference max, sum) in LDS, which also gives
//                       the draw's tile masses at the row where the test stops.
// stage_rows_kernel     the first rows of every block summed up front, all
//                       blocks at once, with the row pass's own batch code;
//                       the lazy kernel (STAGED) then starts from those sums.
//
// The sampling walk itself (sample_walk) lives in walk.hpp, shared with the
// fused scores-and-walk kernel.
#include <type_traits>

#include "walk.hpp"

namespace dflash2 {
namespace {

// ---------------------------------------------------------------- path sampling
__global__ __launch_bounds__(64) void path_sample_kernel(
    const float* __restrict__ S0, const float* __restrict__ S, const int32_t* __restrict__ top_idx,
    const float* __restrict__ u, float inv_t, int L, int joint, int32_t* __restrict__ path_slot,
    int32_t* __restrict__ path_tok, float* __restrict__ q) {
  extern __shared__ f32x4_t stage[];  // (L-1) * 64 vectors of 4 scores
  __shared__ float sbeta[kMaxWalk * kTopK];  // backward messages (whole-path draws)
  constexpr int kUnroll = 8;
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int j = lane & 15;
  const int n4 = (L - 1) * kTopK * kTopK / 4;
  const f32x4_t* src = reinterpret_cast<const f32x4_t*>(S + (size_t)b * (L - 1) * kTopK * kTopK);
  for (int base = 0; base < n4; base += 64 * kUnroll) {
    f32x4_t v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int e = base + k * 64 + lane;
      if (e < n4) v[k] = src[e];
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int e = base + k * 64 + lane;
      if (e < n4) stage[e] = v[k];
    }
  }
  float s = S0[(size_t)b * kTopK + j];
  const size_t row = (size_t)b * L;
  __syncthreads();
  const float* sS = reinterpret_cast<const float*>(stage);
  if (joint) path_messages(sS, inv_t, L, sbeta);
  sample_walk(s, sS, top_idx, u + row, inv_t, b, L, path_slot, path_tok, q,
              joint ? sbeta : nullptr);
}

// ---------------------------------------------------------------- target log-sum-exp
// Running (max, sum) pairs in base 2: a value a contributes 2^(a - m).
// Exponentials use the hardware exp2 (v_exp_f32, about 1 ulp).
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ void lse_merge(float& m, float& s, float om, float os) {
  const float nm = fmaxf(m, om);
  if (nm == -__builtin_inff()) return;  // both empty
  s = s * exp2f(m - nm) + os * exp2f(om - nm);
  m = nm;
}

// One batch of values (already scaled to base 2) into (m, s): one rescale
// per batch instead of a branch per value.  -inf values carry no mass.
template <int N>
__device__ __forceinline__ void lse_batch(float& m, float& s, const float (&a)[N]) {
  float bm = a[0];
#pragma unroll
  for (int i = 1; i < N; ++i) bm = fmaxf(bm, a[i]);
  const float nm = fmaxf(m, bm);
  if (nm == -__builtin_inff()) return;
  float acc = s * exp2f(m - nm);
#pragma unroll
  for (int i = 0; i < N; ++i) acc += exp2f(a[i] - nm);
  s = acc;
  m = nm;
}

__global__ __launch_bounds__(256) void target_lse_kernel(const float* __restrict__ z, int V,
                                                         float scale2, float* __restrict__ lse) {
  __shared__ float red_m[4], red_s[4];
  const size_t r = blockIdx.x;
  const float* row = z + r * V;
  const int tid = threadIdx.x;
  constexpr float kNeg = -__builtin_inff();
  float m = kNeg, s = 0.f;
  if ((V & 3) == 0) {  // 16-byte loads (rows stay 16-byte aligned)
    const f32x4_t* r4 = reinterpret_cast<const f32x4_t*>(row);
    const int n4 = V >> 2;
    constexpr int kU = 4;
    for (int base = tid; base < n4; base += 256 * kU) {
      f32x4_t v[kU];
#pragma unroll
      for (int k = 0; k < kU; ++k) {
        const int e = base + k * 256;
        v[k] = e < n4 ? r4[e] : f32x4_t{kNeg, kNeg, kNeg, kNeg};
      }
      float a[4 * kU];
#pragma unroll
      for (int k = 0; k < kU; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) a[4 * k + i] = v[k][i] * scale2;
      lse_batch(m, s, a);
    }
  } else {
    for (int e = tid; e < V; e += 256) {
      const float a[1] = {row[e] * scale2};
      lse_batch(m, s, a);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) lse_merge(m, s, __shfl_xor(m, o, 64), __shfl_xor(s, o, 64));
  if ((tid & 63) == 0) {
    red_m[tid >> 6] = m;
    red_s[tid >> 6] = s;
  }
  __syncthreads();
  if (tid == 0) {
    float mm = red_m[0], ss = red_s[0];
    for (int w = 1; w < 4; ++w) lse_merge(mm, ss, red_m[w], red_s[w]);
    lse[r] = (mm + log2f(ss)) * kLn2;  // back to natural log
  }
}

// ---------------------------------------------------------------- rejection verification
// Wave reductions through DPP / lane-swap exchanges (xor_lane), several
// times cheaper per step than a __shfl_xor (an LDS permute each).
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __uint_as_float(xor_lane<1>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(xor_lane<2>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(xor_lane<4>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(xor_lane<8>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(xor_lane<16>(__float_as_uint(v))));
  return fmaxf(v, __uint_as_float(xor_lane<32>(__float_as_uint(v))));
}

// N independent wave sums (every lane ends with the totals), the N chains
// interleaved.
template <int N>
__device__ __forceinline__ void wave_sum_n(float (&v)[N]) {
  auto step = [&](auto jtag) {
    constexpr int J = decltype(jtag)::value;
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] += __uint_as_float(xor_lane<J>(__float_as_uint(v[k])));
  };
  step(std::integral_constant<int, 1>{});
  step(std::integral_constant<int, 2>{});
  step(std::integral_constant<int, 4>{});
  step(std::integral_constant<int, 8>{});
  step(std::integral_constant<int, 16>{});
  step(std::integral_constant<int, 32>{});
}

// Inclusive prefix sum across the wave in six DPP steps: row_shr 1, 2, 4,
// 8 scan each 16-lane row (a lane with no source adds 0), then row_bcast 15
// adds row 0's total to row 1 and row 2's to row 3, and row_bcast 31 adds
// the total of rows 0-1 to rows 2 and 3.
__device__ __forceinline__ float wave_scan_incl(float v) {
  auto add = [&](auto ctag, auto mtag) {
    constexpr int C = decltype(ctag)::value;
    constexpr int R = decltype(mtag)::value;
    v += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), C, R, 0xf, false));
  };
  add(std::integral_constant<int, 0x111>{}, std::integral_constant<int, 0xf>{});  // row_shr:1
  add(std::integral_constant<int, 0x112>{}, std::integral_constant<int, 0xf>{});  // row_shr:2
  add(std::integral_constant<int, 0x114>{}, std::integral_constant<int, 0xf>{});  // row_shr:4
  add(std::integral_constant<int, 0x118>{}, std::integral_constant<int, 0xf>{});  // row_shr:8
  add(std::integral_constant<int, 0x142>{}, std::integral_constant<int, 0xa>{});  // row_bcast:15
  add(std::integral_constant<int, 0x143>{}, std::integral_constant<int, 0xc>{});  // row_bcast:31
  return v;
}

__device__ __forceinline__ int wave_min_int(int v) {
  v = min(v, (int)xor_lane<1>((uint32_t)v));
  v = min(v, (int)xor_lane<2>((uint32_t)v));
  v = min(v, (int)xor_lane<4>((uint32_t)v));
  v = min(v, (int)xor_lane<8>((uint32_t)v));
  v = min(v, (int)xor_lane<16>((uint32_t)v));
  return min(v, (int)xor_lane<32>((uint32_t)v));
}

constexpr int kTile = 256;      // tokens per tile: 64 lanes x 4
constexpr int kTileBatch = 8;   // tiles a wave has in flight
constexpr int kVerWaves = 16;   // 128 KB of the row in flight per workgroup

// Masses of the four tokens v0 .. v0+3 of the drawn row (0 past V):
// p(v) = 2^(zr[v] * s2 - l2), less the candidate's q at the rejected
// position (resid), clamped at 0.  praw gets p itself.
__device__ __forceinline__ void token_masses(const float* __restrict__ zr, int V, float s2,
                                             float l2, bool resid, const int32_t* cand_id,
                                             const float* cand_q, int v0, float (&r)[4],
                                             float (&praw)[4]) {
  float zv[4];
  if ((V & 3) == 0 && v0 + 4 <= V) {
    const f32x4_t x = *reinterpret_cast<const f32x4_t*>(zr + v0);
#pragma unroll
    for (int i = 0; i < 4; ++i) zv[i] = x[i];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) zv[i] = v0 + i < V ? zr[v0 + i] : -__builtin_inff();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float p = v0 + i < V ? exp2f(zv[i] * s2 - l2) : 0.f;
    float m = p;
    if (resid) {
#pragma unroll
      for (int c = 0; c < kTopK; ++c)
        if (cand_id[c] == v0 + i) m = fmaxf(m - cand_q[c], 0.f);
    }
    r[i] = m;
    praw[i] = p;
  }
}

// Fallback of the draw when the tile it chose holds no token with mass (the
// prefix overshot every tile, u within rounding of 1, or the chosen tile's
// sum was rounding residue): the last token with mass, searching the tiles
// below `k` from the top down, then the tiles above it; if no tile has one,
// the last token with p > 0 of the first tile that has any, starting with
// tile k's (lastp, -1 if none); if none, V - 1.  After an overshoot k is the
// last tile, so these are the last tokens of the row with residual mass and
// with p > 0.  At most ntiles - 1 tile passes; rare, so kept out of line.
__device__ __attribute__((noinline)) int draw_fallback(const float* __restrict__ zr, int V,
                                                       float s2, float l2, bool resid,
                                                       const int32_t* cand_id,
                                                       const float* cand_q, int k, int ntiles,
                                                       int lastp, int lane) {
  for (int step = 1; step < ntiles; ++step) {
    const int t = k - step >= 0 ? k - step : k - step + ntiles;  // k-1, ..., 0, ntiles-1, ..., k+1
    const int v0 = t * kTile + lane * 4;
    float r[4], pr[4];
    token_masses(zr, V, s2, l2, resid, cand_id, cand_q, v0, r, pr);
    int lr = -1, lp = -1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (r[i] > 0.f) lr = v0 + i;
      if (pr[i] > 0.f) lp = v0 + i;
    }
    lr = -wave_min_int(-lr);
    lp = -wave_min_int(-lp);
    if (lastp < 0) lastp = lp;
    if (lr >= 0) return lr;
  }
  return lastp >= 0 ? lastp : V - 1;
}

// Steps 3-4 of the draw, run by one wave: the candidates' residual
// corrections -min(p, q) into their tiles (in slot order), the inclusive
// prefix of the tile sums in token order, 64 at a time, the first tile whose
// prefix passes u * total, then the first token inside it whose running sum
// passes.  tsum [ntiles] holds each 256-token tile's mass of p; zr is the
// drawn row, p(v) = 2^(zr[v] * s2 - l2).  Writes accept_len = n + 1 and the
// token, always an id in [0, V).
__device__ __forceinline__ void draw_token(float* tsum, int ntiles, const float* __restrict__ zr, int V, float s2,
                           float l2, bool resid, const int32_t* cand_id, const float* cand_q,
                           float u, int lane, int32_t* accept_len, int32_t* next_tok, int n) {
  if (resid) {
    // lanes 0..15 load their candidate's logit together; lane 0 then
    // applies the corrections in slot order from registers (one memory
    // round trip instead of sixteen dependent ones)
    float corr = 0.f;
    int ct = -1;
    if (lane < kTopK) {
      const int v = cand_id[lane];
      if (v >= 0 && v < V) {
        const float p = exp2f(zr[v] * s2 - l2);
        corr = fminf(p, cand_q[lane]);
        ct = v / kTile;
      }
    }
#pragma unroll
    for (int c = 0; c < kTopK; ++c) {
      const int t = __builtin_amdgcn_readlane(ct, c);
      const float cv = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(corr), c));
      if (lane == 0 && t >= 0) tsum[t] -= cv;
    }
  }
  // Inclusive prefix of the tile masses (negative corrections clamped to
  // 0): lane l sums its own run of consecutive tiles, one wave scan adds the
  // runs before it, and the lane writes its run's prefixes.  The first tile
  // whose prefix passes u * total is the lowest one over all lanes.
  __builtin_amdgcn_wave_barrier();
  const int per = (ntiles + 63) / 64;
  const int lo = min(lane * per, ntiles), hi = min(lo + per, ntiles);
  float mine_t = 0.f;
  for (int i = lo; i < hi; ++i) mine_t += fmaxf(tsum[i], 0.f);
  const float incl_t = wave_scan_incl(mine_t);
  const float carry = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(incl_t), 63));
  const float target = u * carry;
  float run_t = incl_t - mine_t;
  int first = 0x7fffffff;
  for (int i = lo; i < hi; ++i) {
    run_t += fmaxf(tsum[i], 0.f);
    tsum[i] = run_t;
    if (first == 0x7fffffff && run_t > target) first = i;
  }
  __builtin_amdgcn_wave_barrier();
  int k = wave_min_int(first);
  const bool over = k == 0x7fffffff;  // rounding: u * total passed every prefix
  if (over) k = ntiles - 1;
  // 4. inside tile k: the first token whose running sum passes the target
  const float base = k > 0 ? tsum[k - 1] : 0.f;
  const int v0 = k * kTile + lane * 4;
  float r[4], pr[4];
  token_masses(zr, V, s2, l2, resid, cand_id, cand_q, v0, r, pr);
  const float mine = r[0] + r[1] + r[2] + r[3];
  const float c = wave_scan_incl(mine);
  float run = base + (c - mine);
  int hit = 0x7fffffff;
  int lastv = -1, lastp = -1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    run += r[i];
    if (hit == 0x7fffffff && r[i] > 0.f && run > target) hit = v0 + i;
    if (r[i] > 0.f) lastv = v0 + i;
    if (pr[i] > 0.f) lastp = v0 + i;
  }
  hit = over ? 0x7fffffff : wave_min_int(hit);  // an overshoot takes the last token with mass
  lastv = -wave_min_int(-lastv);
  if (hit == 0x7fffffff && lastv < 0)
    lastv = draw_fallback(zr, V, s2, l2, resid, cand_id, cand_q, k, ntiles,
                          -wave_min_int(-lastp), lane);
  if (lane == 0) {
    *accept_len = n + 1;
    *next_tok = hit != 0x7fffffff ? hit : lastv;
  }
}

template <bool VEC>
__global__ __launch_bounds__(64 * kVerWaves) void verify_rejection_kernel(
    const int32_t* __restrict__ path_slot, const int32_t* __restrict__ path_tok,
    const float* __restrict__ q, const int32_t* __restrict__ top_idx,
    const float* __restrict__ z, const float* __restrict__ lse, float inv_t,
    const float* __restrict__ u_acc, const float* __restrict__ u_res, int L, int V,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ next_tok) {
  extern __shared__ float tsum[];  // tile sums, then their inclusive prefix
  __shared__ int s_n;
  __shared__ int32_t cand_id[kTopK];
  __shared__ float cand_q[kTopK];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const size_t brow = (size_t)b * L;
  const size_t zrow = (size_t)b * (L + 1);
  // 1. every position's accept test at once (thread t, t < L; a token
  //    outside [0, V) or a slot outside [0, 16) fails), then n = the
  //    number of leading passes
  if (tid == 0) s_n = L;
  __syncthreads();
  if (tid < L) {
    const size_t bt = brow + tid;
    const int x = path_tok[bt];
    const int sl = path_slot[bt];
    bool pass = false;
    if (x >= 0 && x < V && sl >= 0 && sl < kTopK) {
      const float qx = q[bt * kTopK + sl];
      const float px = expf(z[(zrow + tid) * V + x] * inv_t - lse[zrow + tid]);
      pass = u_acc[bt] * qx < px;
    }
    if (!pass) atomicMin(&s_n, tid);
  }
  __syncthreads();
  const int n = s_n;
  const bool resid = n < L;  // draw from max(0, p - q) at the rejected position, else from p
  if (tid < kTopK) {
    cand_id[tid] = resid ? top_idx[(brow + n) * kTopK + tid] : -1;
    cand_q[tid] = resid ? q[(brow + n) * kTopK + tid] : 0.f;
  }
  const float* zr = z + (zrow + n) * V;
  // p(v) = 2^(z[v] * s2 - l2): base-2 form of exp(z / T - lse)
  const float s2 = inv_t * kLog2e;
  const float l2 = lse[zrow + n] * kLog2e;
  const int ntiles = (V + kTile - 1) / kTile;
  // 2. tile sums of p (candidates corrected below): wave w takes
  //    kTileBatch consecutive tiles at a time (8w .. 8w+7, then 128 further
  //    on), so each wave streams 8 KB runs of the row.  All the batch's
  //    loads go out before the first use (indices clamped into the row,
  //    tokens past V masked).
  for (int t0 = wave * kTileBatch; t0 < ntiles; t0 += kVerWaves * kTileBatch) {
    f32x4_t raw[kTileBatch];
#pragma unroll
    for (int k = 0; k < kTileBatch; ++k) {
      const int v0 = (t0 + k) * kTile + lane * 4;
      if constexpr (VEC) {
        raw[k] = *reinterpret_cast<const f32x4_t*>(zr + min(v0, V - 4));  // V % 4 == 0
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) raw[k][i] = zr[min(v0 + i, V - 1)];
      }
    }
    float acc[kTileBatch];
#pragma unroll
    for (int k = 0; k < kTileBatch; ++k) {
      acc[k] = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if ((t0 + k) * kTile + lane * 4 + i < V) acc[k] += exp2f(raw[k][i] * s2 - l2);
    }
    wave_sum_n<kTileBatch>(acc);
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < kTileBatch; ++k)
        if (t0 + k < ntiles) tsum[t0 + k] = acc[k];
    }
  }
  __syncthreads();
  // 3-4. wave 0 draws the verifier's token from the tile sums
  if (wave == 0)
    draw_token(tsum, ntiles, zr, V, s2, l2, resid, cand_id, cand_q, u_res[b], lane,
               accept_len + b, next_tok + b, n);
}

// The loads of one batch (tile_batch below): lane l takes 16 bytes of each
// of the kTileBatch tiles, index clamped into the row.
template <bool VEC>
__device__ __forceinline__ void tile_batch_load(const float* __restrict__ zr, int V, int t0,
                                                int lane, f32x4_t (&raw)[kTileBatch]) {
#pragma unroll
  for (int k = 0; k < kTileBatch; ++k) {
    const int v0 = (t0 + k) * kTile + lane * 4;
    if constexpr (VEC) {
      raw[k] = *reinterpret_cast<const f32x4_t*>(zr + min(v0, V - 4));  // V % 4 == 0
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) raw[k][i] = zr[min(v0 + i, V - 1)];
    }
  }
}

__device__ __forceinline__ void tile_batch_sum(const f32x4_t (&raw)[kTileBatch], int V, int t0,
                                               int lane, float s2, float& bm, float& tile,
                                               float& bs) {
  static_assert(kTileBatch == 8, "the reduce-scatter below is sized for 8 tiles");
  constexpr float kNeg = -__builtin_inff();
  float zv[kTileBatch][4];
  bm = kNeg;
  if ((t0 + kTileBatch) * kTile <= V) {  // the whole batch inside the row (uniform)
#pragma unroll
    for (int k = 0; k < kTileBatch; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        zv[k][i] = raw[k][i] * s2;
        bm = fmaxf(bm, zv[k][i]);
      }
  } else {
#pragma unroll
    for (int k = 0; k < kTileBatch; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        zv[k][i] = (t0 + k) * kTile + lane * 4 + i < V ? raw[k][i] * s2 : kNeg;
        bm = fmaxf(bm, zv[k][i]);
      }
  }
  bm = wave_max(bm);
  const float ref = bm == kNeg ? 0.f : bm;  // an empty batch sums exp2(-inf) = 0
  // The hardware exponential without exp2f's denormal-range fix-up: a term
  // below 2^-126 cannot change a sum that holds the batch maximum's 1.
  float v[kTileBatch];
#pragma unroll
  for (int k = 0; k < kTileBatch; ++k) {
    v[k] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[k] += __builtin_amdgcn_exp2f(zv[k][i] - ref);
  }
  // Reduce-scatter over lane bits 5, 4, 3: each step a lane keeps half of
  // its tiles (the upper half when the bit is set) and adds its partner's
  // sums of them, so after three steps lane l holds tile (l >> 3) & 7 of
  // the batch; a butterfly over bits 2..0 finishes that tile in its group
  // of 8 lanes, and one over bits 3..5 the batch total (13 exchanges in
  // place of 48).
  auto half = [&](auto dtag, int n) {
    constexpr int D = decltype(dtag)::value;
    const bool hi = (lane & D) != 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < n / 2) {
        const float send = hi ? v[j] : v[j + n / 2];
        const float keep = hi ? v[j + n / 2] : v[j];
        v[j] = keep + __uint_as_float(xor_lane<D>(__float_as_uint(send)));
      }
  };
  half(std::integral_constant<int, 32>{}, 8);
  half(std::integral_constant<int, 16>{}, 4);
  half(std::integral_constant<int, 8>{}, 2);
  tile = v[0];
  tile += __uint_as_float(xor_lane<4>(__float_as_uint(tile)));
  tile += __uint_as_float(xor_lane<2>(__float_as_uint(tile)));
  tile += __uint_as_float(xor_lane<1>(__float_as_uint(tile)));
  bs = tile;
  bs += __uint_as_float(xor_lane<8>(__float_as_uint(bs)));
  bs += __uint_as_float(xor_lane<16>(__float_as_uint(bs)));
  bs += __uint_as_float(xor_lane<32>(__float_as_uint(bs)));
}

// One batch of a target row: kTileBatch consecutive tiles from tile t0,
// values scaled by s2 (base 2), tokens past V as -inf.  Every lane ends with
// the batch maximum bm (the tiles' common reference, 0 in its place when
// the batch is empty) and the total bs of 2^(value - reference); lane l
// holds in `tile` the sum of tile t0 + ((l >> 3) & 7).  Every load is issued
// before the first use (index clamped into the row): a use or a per-lane
// branch between two loads makes each wait for the one before.  The lazy
// verification's row pass and the staged rows share this code, so their
// sums are the same bit for bit.
template <bool VEC>
__device__ __forceinline__ void tile_batch(const float* __restrict__ zr, int V, int t0, int lane,
                                           float s2, float& bm, float& tile, float& bs) {
  f32x4_t raw[kTileBatch];
  tile_batch_load<VEC>(zr, V, t0, lane, raw);
  tile_batch_sum(raw, V, t0, lane, s2, bm, tile, bs);
}

// Per (block, row) record of a staged row: the tiles' batch maxima [ntiles],
// the tiles' sums [ntiles], then the batches' maxima [nbatch] and totals
// [nbatch].
__host__ __device__ constexpr size_t staged_row_floats(int ntiles) {
  return 2 * (size_t)ntiles + 2 * (size_t)((ntiles + kTileBatch - 1) / kTileBatch);
}

// The first `rows` target rows of every block, all at once: one wave per
// kStageBatches consecutive batches of kTileBatch tiles, (block, row,
// batches) in that order, writing the batches' record entries.  A wave
// issues the loads of all its batches before summing the first.  No wave
// depends on another.  One batch per wave (8 KB of the row) is the fastest:
// with two or four, fewer waves are resident and each one's exponentials
// and reductions run longer after its loads land.
constexpr int kStageBatches = 1;

template <bool VEC>
__global__ __launch_bounds__(256) void stage_rows_kernel(const float* __restrict__ z, float s2,
                                                         int L, int V, int rows, int nwaves,
                                                         float* __restrict__ staged) {
  const int lane = threadIdx.x & 63;
  const int g = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (g >= nwaves) return;  // whole waves
  const int ntiles = (V + kTile - 1) / kTile;
  const int nbatch = (ntiles + kTileBatch - 1) / kTileBatch;
  const int per_row = (nbatch + kStageBatches - 1) / kStageBatches;  // waves per row
  const int j0 = (g % per_row) * kStageBatches;
  const int bt = g / per_row;
  const int t = bt % rows, b = bt / rows;
  const float* zr = z + ((size_t)b * (L + 1) + t) * V;
  f32x4_t raw[kStageBatches][kTileBatch];
#pragma unroll
  for (int i = 0; i < kStageBatches; ++i)  // a batch past the row reads (clamped) and is dropped
    tile_batch_load<VEC>(zr, V, min(j0 + i, nbatch - 1) * kTileBatch, lane, raw[i]);
  float* rec = staged + (size_t)bt * staged_row_floats(ntiles);
#pragma unroll
  for (int i = 0; i < kStageBatches; ++i) {
    const int j = j0 + i;
    if (j >= nbatch) break;  // uniform
    float bm, tile, bs;
    tile_batch_sum(raw[i], V, j * kTileBatch, lane, s2, bm, tile, bs);
    const int tk = j * kTileBatch + ((lane >> 3) & 7);  // the tile this lane's group holds
    if ((lane & 7) == 0 && tk < ntiles) {
      rec[tk] = bm;
      rec[ntiles + tk] = tile;
    }
    if (lane == 0) {
      rec[2 * ntiles + j] = bm;
      rec[2 * ntiles + nbatch + j] = bs;
    }
  }
}

// Rejection verification that computes the normaliser of a target row only
// when the accept test reaches it: row t is read once, as 256-token tiles
// whose (reference maximum, sum of 2^(z * s2 - reference)) stay in LDS; the
// tiles give the row's log-sum-exp for the test and, at the row where the
// walk stops, the tile masses of the draw, so the stopping row is not read
// again.  A block that stops at position n reads n + 1 rows instead of all
// L + 1.  The accept rule and the draw are those of verify_rejection_kernel.
// STAGED: rows below `rows` come from stage_rows_kernel's records instead,
// merged in the order the row pass would merge them.
template <bool VEC, bool STAGED>
__global__ __launch_bounds__(64 * kVerWaves) void verify_rejection_lazy_kernel(
    const int32_t* __restrict__ path_slot, const int32_t* __restrict__ path_tok,
    const float* __restrict__ q, const int32_t* __restrict__ top_idx,
    const float* __restrict__ z, float s2, const float* __restrict__ u_acc,
    const float* __restrict__ u_res, int L, int V, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ next_tok, const float* __restrict__ staged, int rows) {
  extern __shared__ float tiles[];  // [ntiles] reference maxima, then [ntiles] sums
  __shared__ int32_t s_x[kMaxWalk];
  __shared__ float s_thr[kMaxWalk];
  __shared__ float s_wm[kVerWaves], s_ws[kVerWaves];
  __shared__ float s_l2;
  __shared__ int s_stop;
  __shared__ int32_t cand_id[kTopK];
  __shared__ float cand_q[kTopK];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const size_t brow = (size_t)b * L;
  const size_t zrow = (size_t)b * (L + 1);
  const int ntiles = (V + kTile - 1) / kTile;
  float* tref = tiles;
  float* tsum = tiles + ntiles;
  constexpr float kNeg = -__builtin_inff();
  // the accept tests' inputs: token (-1: fails), threshold u * q(slot)
  if (tid < L) {
    const size_t bt = brow + tid;
    const int x = path_tok[bt];
    const int sl = path_slot[bt];
    const bool ok = x >= 0 && x < V && sl >= 0 && sl < kTopK;
    s_x[tid] = ok ? x : -1;
    s_thr[tid] = ok ? u_acc[bt] * q[bt * kTopK + sl] : 0.f;
  }
  __syncthreads();
  int n = L;
  for (int t = 0; t <= L; ++t) {
    const float* zr = z + (zrow + t) * V;
    const int x = t < L ? s_x[t] : -1;
    float zx = 0.f;
    if (tid == 0 && x >= 0) zx = zr[x];  // in flight during the pass
    // wave w takes kTileBatch consecutive tiles at a time (8 KB runs of the
    // row: 14% faster per row than tiles strided across the waves); each
    // batch shares one reference maximum.  A staged row's batches were summed
    // ahead (stage_rows_kernel, the same arithmetic); its waves merge their
    // batches' (maximum, total) in the same order.
    float Mw = kNeg, Sw = 0.f;
    if (STAGED && t < rows) {
      // lane i loads the record of batch wave + 16 i (every load in one
      // round trip; at most 64 batches per wave as V <= 2^21), then the
      // wave merges them in batch order
      const float* rec = staged + ((size_t)b * rows + t) * staged_row_floats(ntiles);
      const int nbatch = (ntiles + kTileBatch - 1) / kTileBatch;
      const int nbw = (nbatch - wave + kVerWaves - 1) / kVerWaves;  // this wave's batches
      float pm = kNeg, ps = 0.f;
      if (lane < nbw) {
        const int j = wave + kVerWaves * lane;
        pm = rec[2 * ntiles + j];
        ps = rec[2 * ntiles + nbatch + j];
      }
      for (int i = 0; i < nbw; ++i)
        lse_merge(Mw, Sw, __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                              __builtin_bit_cast(int, pm), i)),
                  __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                __builtin_bit_cast(int, ps), i)));
    } else {
      for (int t0 = wave * kTileBatch; t0 < ntiles; t0 += kVerWaves * kTileBatch) {
        float bm, tile, bs;
        tile_batch<VEC>(zr, V, t0, lane, s2, bm, tile, bs);
        const int tk = t0 + ((lane >> 3) & 7);  // the tile this lane's group holds
        if ((lane & 7) == 0 && tk < ntiles) {
          tref[tk] = bm;
          tsum[tk] = tile;
        }
        lse_merge(Mw, Sw, bm, bs);
      }
    }
    if (lane == 0) {
      s_wm[wave] = Mw;
      s_ws[wave] = Sw;
    }
    __syncthreads();
    if (tid == 0) {
      float mm = s_wm[0], ss = s_ws[0];
      for (int w = 1; w < kVerWaves; ++w) lse_merge(mm, ss, s_wm[w], s_ws[w]);
      const float l2 = mm + log2f(ss);
      s_l2 = l2;
      s_stop = t == L || !(x >= 0 && s_thr[t] < exp2f(zx * s2 - l2));
    }
    __syncthreads();
    if (s_stop) {
      n = t;
      break;
    }
  }
  const float l2 = s_l2;
  const bool resid = n < L;  // draw from max(0, p - q) at the rejected position, else from p
  if (tid < kTopK) {
    cand_id[tid] = resid ? top_idx[(brow + n) * kTopK + tid] : -1;
    cand_q[tid] = resid ? q[(brow + n) * kTopK + tid] : 0.f;
  }
  // tile masses of p: sum * 2^(reference - l2) (a staged row's tiles from
  // its record, read by the thread that uses them)
  const float* srec = STAGED && n < rows
                          ? staged + ((size_t)b * rows + n) * staged_row_floats(ntiles)
                          : nullptr;
  for (int i = tid; i < ntiles; i += 64 * kVerWaves) {
    const float r = srec ? srec[i] : tref[i];
    const float sm = srec ? srec[ntiles + i] : tsum[i];
    tsum[i] = r == kNeg ? 0.f : sm * exp2f(r - l2);
  }
  __syncthreads();
  if (wave == 0)
    draw_token(tsum, ntiles, z + (zrow + n) * V, V, s2, l2, resid, cand_id, cand_q, u_res[b],
               lane, accept_len + b, next_tok + b, n);
}

}  // namespace

hipError_t launch_path_sample(const float* S0, const float* S, const int32_t* top_idx,
                              const float* u, float temperature, int B, int L, int joint,
                              int32_t* path_slot, int32_t* path_tok, float* q, hipStream_t s) {
  if (B == 0) return hipSuccess;
  const size_t lds = (size_t)(L - 1) * kTopK * kTopK * sizeof(float);
  hipLaunchKernelGGL(path_sample_kernel, dim3((unsigned)B), dim3(64), lds, s, S0, S, top_idx, u,
                     1.0f / temperature, L, joint, path_slot, path_tok, q);
  return hipGetLastError();
}

hipError_t launch_target_lse(const float* z, int R, int V, float temperature, float* lse,
                             hipStream_t s) {
  if (R == 0) return hipSuccess;
  hipLaunchKernelGGL(target_lse_kernel, dim3((unsigned)R), dim3(256), 0, s, z, V,
                     kLog2e / temperature, lse);
  return hipGetLastError();
}

template <bool STAGED>
static void launch_lazy(const int32_t* path_slot, const int32_t* path_tok, const float* q,
                        const int32_t* top_idx, const float* z, float temperature,
                        const float* u_acc, const float* u_res, int B, int L, int V,
                        int32_t* accept_len, int32_t* next_tok, const float* staged, int rows,
                        hipStream_t s) {
  // 16-byte loads when the rows are 16-byte aligned (z is, and V % 4 == 0)
  if ((V & 3) == 0 && (reinterpret_cast<uintptr_t>(z) & 15) == 0)
    hipLaunchKernelGGL((verify_rejection_lazy_kernel<true, STAGED>), dim3((unsigned)B),
                       dim3(64 * kVerWaves), verify_rejection_lazy_lds(V), s, path_slot, path_tok,
                       q, top_idx, z, kLog2e / temperature, u_acc, u_res, L, V, accept_len,
                       next_tok, staged, rows);
  else
    hipLaunchKernelGGL((verify_rejection_lazy_kernel<false, STAGED>), dim3((unsigned)B),
                       dim3(64 * kVerWaves), verify_rejection_lazy_lds(V), s, path_slot, path_tok,
                       q, top_idx, z, kLog2e / temperature, u_acc, u_res, L, V, accept_len,
                       next_tok, staged, rows);
}

hipError_t launch_verify_rejection_lazy(const int32_t* path_slot, const int32_t* path_tok,
                                        const float* q, const int32_t* top_idx, const float* z,
                                        float temperature, const float* u_acc, const float* u_res,
                                        int B, int L, int V, int32_t* accept_len,
                                        int32_t* next_tok, hipStream_t s) {
  if (B == 0) return hipSuccess;
  launch_lazy<false>(path_slot, path_tok, q, top_idx, z, temperature, u_acc, u_res, B, L, V,
                     accept_len, next_tok, nullptr, 0, s);
  return hipGetLastError();
}

size_t verify_rejection_staged_bytes(int B, int V, int rows) {
  const int ntiles = (V + kTile - 1) / kTile;
  return (size_t)B * (size_t)rows * staged_row_floats(ntiles) * sizeof(float);
}

hipError_t launch_verify_rejection_staged(const int32_t* path_slot, const int32_t* path_tok,
                                          const float* q, const int32_t* top_idx, const float* z,
                                          float temperature, const float* u_acc,
                                          const float* u_res, int B, int L, int V, int rows,
                                          float* staged, int32_t* accept_len, int32_t* next_tok,
                                          hipStream_t s) {
  if (B == 0) return hipSuccess;
  const int ntiles = (V + kTile - 1) / kTile;
  const int nbatch = (ntiles + kTileBatch - 1) / kTileBatch;
  const int per_row = (nbatch + kStageBatches - 1) / kStageBatches;
  const long long nwaves = (long long)B * rows * per_row;  // < 2^31: checked by the caller
  const unsigned grid = (unsigned)((nwaves + 3) / 4);
  if ((V & 3) == 0 && (reinterpret_cast<uintptr_t>(z) & 15) == 0)
    hipLaunchKernelGGL(stage_rows_kernel<true>, dim3(grid), dim3(256), 0, s, z,
                       kLog2e / temperature, L, V, rows, (int)nwaves, staged);
  else
    hipLaunchKernelGGL(stage_rows_kernel<false>, dim3(grid), dim3(256), 0, s, z,
                       kLog2e / temperature, L, V, rows, (int)nwaves, staged);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_lazy<true>(path_slot, path_tok, q, top_idx, z, temperature, u_acc, u_res, B, L, V,
                    accept_len, next_tok, staged, rows, s);
  return hipGetLastError();
}

size_t verify_rejection_lds(int V) { return (size_t)((V + kTile - 1) / kTile) * sizeof(float); }

size_t verify_rejection_lazy_lds(int V) { return 2 * verify_rejection_lds(V); }

hipError_t launch_verify_rejection(const int32_t* path_slot, const int32_t* path_tok,
                                   const float* q, const int32_t* top_idx, const float* z,
                                   const float* lse, float temperature, const float* u_acc,
                                   const float* u_res, int B, int L, int V, int32_t* accept_len,
                                   int32_t* next_tok, hipStream_t s) {
  if (B == 0) return hipSuccess;
  if ((V & 3) == 0 && (reinterpret_cast<uintptr_t>(z) & 15) == 0)
    hipLaunchKernelGGL(verify_rejection_kernel<true>, dim3((unsigned)B), dim3(64 * kVerWaves),
                       verify_rejection_lds(V), s, path_slot, path_tok, q, top_idx, z, lse,
                       1.0f / temperature, u_acc, u_res, L, V, accept_len, next_tok);
  else
    hipLaunchKernelGGL(verify_rejection_kernel<false>, dim3((unsigned)B), dim3(64 * kVerWaves),
                       verify_rejection_lds(V), s, path_slot, path_tok, q, top_idx, z, lse,
                       1.0f / temperature, u_acc, u_res, L, V, accept_len, next_tok);
  return hipGetLastError();
}

}  // namespace dflash2
