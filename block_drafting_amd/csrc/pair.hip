// Adjacent-pair scores ("DFlash 2: Keep Drafting Parallel", section
// "A lightweight path selector", eq. S_t(a,b)) in low-rank form
//   S_t[i, j] = logit_t(c_{t,j}) + (U[c_{t-1,i}] * g_t) . V[c_{t,j}],
// with the last verified token as the previous token of position 0.  g_t is
// the context gate of position t (an r-vector); without one it is all ones.
//
// One wavefront per (block, position) computes the whole 16 x 16 match
// matrix as one fp32 matrix-core product, [16 x r] x [r x 16], with
// v_mfma_f32_16x16x4f32.  The four k-rows of each MFMA step are four
// contiguous quarters of the rank: lane l = 16 q + i feeds row i of the
// previous-token factors and column i of the candidate factors with the
// elements k = q * rc + s (rc = ceil(r / 4)) at step s, so every lane
// gathers one contiguous run of each factor row straight into registers
// (16-byte loads, all in flight at once) and no LDS is needed.  Products and
// sums are fp32, as in a plain fp32 dot.
#include "walk.hpp"

namespace dflash2 {
namespace {

// Raw storage of RC consecutive elements of one factor row.
template <typename T, int RC>
struct Chunk;
template <int RC>
struct Chunk<uint16_t, RC> {
  static constexpr int kRuns = RC / 8;  // 16-byte runs of 8 bf16
  u32x4_t w[kRuns];
  __device__ __forceinline__ float get(int k) const {
    const uint32_t v = w[k >> 3][(k >> 1) & 3];
    return (k & 1) ? bf16_hi(v) : bf16_lo(v);
  }
};
template <int RC>
struct Chunk<float, RC> {
  static constexpr int kRuns = RC / 4;  // 16-byte runs of 4 fp32
  u32x4_t w[kRuns];
  __device__ __forceinline__ float get(int k) const { return __uint_as_float(w[k >> 2][k & 3]); }
};

// Elements [k0, k0 + n) of row `id` of F [V, r] (n <= RC); elements past n
// read as 0.  An id outside [0, V) gives a NaN row; `zero` gives a zero row.
// VEC: the run start k0 and n are whole 16-byte runs and rows are 16-byte
// aligned, so each run is one vector load; else element by element.
template <typename T, int RC, bool VEC>
__device__ __forceinline__ void load_chunk(Chunk<T, RC>& c, const T* __restrict__ F, int id, int V,
                                           int r, int k0, int n, bool zero) {
  constexpr int kPer = 16 / sizeof(T);
  const bool bad = !zero && (id < 0 || id >= V);
  const bool live = !zero && !bad;
  const T* row = F + (size_t)(live ? id : 0) * r + k0;
  const uint32_t nan_bits = sizeof(T) == 2 ? 0x7fc0u : 0x7fc00000u;
#pragma unroll
  for (int q = 0; q < Chunk<T, RC>::kRuns; ++q) {
    const int k = q * kPer;
    if (VEC) {
      const uint32_t f = sizeof(T) == 2 ? (nan_bits | nan_bits << 16) : nan_bits;
      if (live && k < n)
        c.w[q] = *reinterpret_cast<const u32x4_t*>(row + k);
      else if (bad && k < n)
        c.w[q] = u32x4_t{f, f, f, f};
      else
        c.w[q] = u32x4_t{0u, 0u, 0u, 0u};
    } else {
      uint32_t v[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        uint32_t bits = 0u;
        if (k + e < n) {
          if (bad)
            bits = nan_bits;
          else if (live)
            bits = sizeof(T) == 2 ? (uint32_t)reinterpret_cast<const uint16_t*>(row)[k + e]
                                  : __float_as_uint(reinterpret_cast<const float*>(row)[k + e]);
        }
        if (sizeof(T) == 2)
          v[e >> 1] |= bits << (16 * (e & 1));
        else
          v[e] = bits;
      }
      c.w[q] = u32x4_t{v[0], v[1], v[2], v[3]};
    }
  }
}

// RC: the most elements one lane holds per factor row (>= ceil(r / 4)).
// The 16 x 16 block of position t of block b, computed by one wave: lane
// l = 16 q + i ends with tv = the logit of candidate i and, in res[e], the
// match of previous candidate 4 q + e with candidate i, so the score
// S_t[4 q + e][i] is tv + res[e] (for t = 0, row 0 holds the anchor's).
template <typename T, int RC, bool VEC>
__device__ __forceinline__ void pair_block(const float* __restrict__ top_val,
                                           const int32_t* __restrict__ top_idx,
                                           const int32_t* __restrict__ anchor_tok,
                                           const T* __restrict__ U, const T* __restrict__ Vf,
                                           const float* __restrict__ gate, int b, int t, int L,
                                           int V, int r, int lane, float& tv, f32x4_t& res) {
  const int i = lane & 15;  // row of the previous factors / column of the current ones
  const int q = lane >> 4;  // quarter of the rank this lane feeds
  const int rc = (r + 3) >> 2;
  const int k0 = q * rc;
  const int n = min(rc, r - k0);  // may be <= 0 for tiny r: then all padding
  const size_t bt = (size_t)b * L + t;
  const int32_t* cur = top_idx + bt * kTopK;

  int prev_id = 0;
  bool prev_zero = false;
  if (t == 0) {
    prev_zero = anchor_tok == nullptr;       // no match term at t = 0
    if (!prev_zero) prev_id = anchor_tok[b];  // the same row for all 16 i
  } else {
    prev_id = cur[i - kTopK];
  }
  Chunk<T, RC> cu, cv;
  load_chunk<T, RC, VEC>(cu, U, prev_id, V, r, k0, n, prev_zero);
  load_chunk<T, RC, VEC>(cv, Vf, cur[i], V, r, k0, n, false);
  float g[RC];
  if (gate) {
    const float* gr = gate + bt * r + k0;
#pragma unroll
    for (int s = 0; s < RC; s += 4) {
      if (VEC && s < n) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(gr + s);
        g[s] = v[0];
        g[s + 1] = v[1];
        g[s + 2] = v[2];
        g[s + 3] = v[3];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) g[s + e] = (!VEC && s + e < n) ? gr[s + e] : 1.0f;
      }
    }
  }
  tv = top_val[bt * kTopK + i];

  // C[i][j] = sum_k A[i][k] B[k][j]; two accumulators alternate so that
  // consecutive steps do not wait on each other.
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f};
  f32x4_t acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < RC; ++s) {
    float a = cu.get(s);
    if (gate) a *= g[s];
    const float bb = cv.get(s);
    if (s & 1)
      acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bb, acc1, 0, 0, 0);
    else
      acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bb, acc0, 0, 0, 0);
  }
  // Lane l holds C[4 (l / 16) + e][l % 16] in element e: column j = i, whose
  // own logit this lane already holds.
#pragma unroll
  for (int e = 0; e < 4; ++e) res[e] = acc0[e] + acc1[e];
}

template <typename T, int RC, bool VEC>
__global__ __launch_bounds__(64) void pair_score_kernel(const float* __restrict__ top_val,
                                                        const int32_t* __restrict__ top_idx,
                                                        const int32_t* __restrict__ anchor_tok,
                                                        const T* __restrict__ U,
                                                        const T* __restrict__ Vf,
                                                        const float* __restrict__ gate, int L,
                                                        int V, int r, float* __restrict__ S0,
                                                        float* __restrict__ S) {
  const int b = blockIdx.x / L;
  const int t = blockIdx.x - b * L;
  const int lane = threadIdx.x;
  const int i = lane & 15;
  const int q = lane >> 4;
  float tv;
  f32x4_t res;
  pair_block<T, RC, VEC>(top_val, top_idx, anchor_tok, U, Vf, gate, b, t, L, V, r, lane, tv, res);
  if (t == 0) {
    if (q == 0) S0[(size_t)b * kTopK + i] = tv + res[0];
    return;
  }
  float* dst = S + ((size_t)b * (L - 1) + (t - 1)) * kTopK * kTopK;
#pragma unroll
  for (int e = 0; e < 4; ++e) dst[(4 * q + e) * kTopK + i] = tv + res[e];
}

// The scores of block b, one wave per position (t = wave, wave + waves, ...):
// each 16 x 16 block to LDS (sS [(L-1) x 16 x 16], sS0 [16]) and, when
// S0out / Sout are given, to global memory too.
template <typename T, int RC, bool VEC>
__device__ __forceinline__ void pair_phase(const float* __restrict__ top_val,
                                           const int32_t* __restrict__ top_idx,
                                           const int32_t* __restrict__ anchor_tok,
                                           const T* __restrict__ U, const T* __restrict__ Vf,
                                           const float* __restrict__ gate, int b, int L, int V,
                                           int r, float* sS, float* sS0, float* __restrict__ S0out,
                                           float* __restrict__ Sout) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int nw = blockDim.x >> 6;
  const int i = lane & 15;
  const int q = lane >> 4;
  for (int t = wave; t < L; t += nw) {
    float tv;
    f32x4_t res;
    pair_block<T, RC, VEC>(top_val, top_idx, anchor_tok, U, Vf, gate, b, t, L, V, r, lane, tv,
                           res);
    if (t == 0) {
      if (q == 0) {
        const float v = tv + res[0];
        sS0[i] = v;
        if (S0out) S0out[(size_t)b * kTopK + i] = v;
      }
    } else {
      float* dl = sS + (size_t)(t - 1) * kTopK * kTopK;
      float* dg = Sout ? Sout + ((size_t)b * (L - 1) + (t - 1)) * kTopK * kTopK : nullptr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = tv + res[e];
        dl[(4 * q + e) * kTopK + i] = v;
        if (dg) dg[(4 * q + e) * kTopK + i] = v;
      }
    }
  }
}

// Pair scores, path walk and greedy verification of one block in one
// workgroup: the step's three latency-bound stages in one launch, with the
// scores kept in LDS between them.  Waves take the positions t = wave,
// wave + waves, ... and leave each 16 x 16 block in LDS (and, when S0out /
// Sout are given, in global memory too); wave 0 then walks the scores in LDS
// (the max-plus walk keeps its back-pointer rows in score blocks it has
// already walked) and compares the walked tokens with the targets.  Every
// part runs the separate kernels' arithmetic, so the results are the same
// bit for bit.  LDS: (L-1) x 1 KiB of scores plus 128 bytes.  Up to 16 waves
// per block; 8 where r > 128, whose score registers would not fit 16.
template <int RC>
constexpr int pwv_max_waves() { return RC >= 32 ? 8 : 16; }

template <typename T, int RC, bool VEC, bool GREEDY>
__global__ __launch_bounds__(64 * pwv_max_waves<RC>()) void pair_walk_verify_kernel(
    const float* __restrict__ top_val, const int32_t* __restrict__ top_idx,
    const int32_t* __restrict__ anchor_tok, const T* __restrict__ U, const T* __restrict__ Vf,
    const float* __restrict__ gate, const int32_t* __restrict__ target, int L, int V, int r,
    float* __restrict__ S0out, float* __restrict__ Sout, int32_t* __restrict__ path_slot,
    int32_t* __restrict__ path_tok, float* __restrict__ path_score,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ next_tok) {
  extern __shared__ float sS[];         // (L - 1) x 16 x 16 scores
  __shared__ float sS0[kTopK];          // S0, then the max-plus walk's running maxima
  __shared__ uint8_t sslot[kMaxWalk];   // walked slots
  const int b = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  // wave 0 loads the targets now (lane t: target t, t <= min(L, 63)); they
  // are in registers by the time the walk ends
  int gt = 0;
  if (wave == 0 && lane <= L) gt = target[(size_t)b * (L + 1) + lane];
  pair_phase<T, RC, VEC>(top_val, top_idx, anchor_tok, U, Vf, gate, b, L, V, r, sS, sS0, S0out,
                         Sout);
  __syncthreads();
  if (wave != 0) return;
  int tok;
  if (GREEDY)
    tok = greedy_walk(sS0, sS, top_idx, b, L, path_slot, path_tok, path_score, sslot);
  else
    tok = viterbi_walk<false>(sS0, sS, top_idx, b, L, sS0, reinterpret_cast<uint8_t*>(sS),
                              kTopK * kTopK * (int)sizeof(float), path_slot, path_tok,
                              path_score, sslot);
  // Greedy verification: accepted = the longest prefix of walked tokens equal
  // to the targets, plus the target after it.
  const uint64_t mm = __ballot(lane < L && tok != gt);
  const int n = mm ? (int)__builtin_ctzll(mm) : L;
  // the target after the accepted prefix; at n = 64 (L = 64, all accepted)
  // it has no lane and is read from memory
  const int gn = __builtin_amdgcn_readlane(gt, n & 63);
  if (lane == 0) {
    accept_len[b] = n + 1;
    if (next_tok) next_tok[b] = n < 64 ? gn : target[(size_t)b * (L + 1) + n];
  }
}

// Pair scores and the sampling walk of one block in one workgroup (the
// sampling twin of pair_walk_verify_kernel; the rejection verification needs
// the target logits and runs on its own).  Bit for bit the separate calls.
template <typename T, int RC, bool VEC>
__global__ __launch_bounds__(64 * pwv_max_waves<RC>()) void pair_sample_kernel(
    const float* __restrict__ top_val, const int32_t* __restrict__ top_idx,
    const int32_t* __restrict__ anchor_tok, const T* __restrict__ U, const T* __restrict__ Vf,
    const float* __restrict__ gate, const float* __restrict__ u, float inv_t, int L, int V, int r,
    int joint, float* __restrict__ S0out, float* __restrict__ Sout,
    int32_t* __restrict__ path_slot, int32_t* __restrict__ path_tok, float* __restrict__ qout) {
  extern __shared__ float sS[];  // (L - 1) x 16 x 16 scores
  __shared__ float sS0[kTopK];
  __shared__ float sbeta[kMaxWalk * kTopK];  // backward messages (whole-path draws)
  const int b = blockIdx.x;
  pair_phase<T, RC, VEC>(top_val, top_idx, anchor_tok, U, Vf, gate, b, L, V, r, sS, sS0, S0out,
                         Sout);
  __syncthreads();
  if ((threadIdx.x >> 6) != 0) return;
  if (joint) path_messages(sS, inv_t, L, sbeta);
  sample_walk(sS0[threadIdx.x & 15], sS, top_idx, u + (size_t)b * L, inv_t, b, L, path_slot,
              path_tok, qout, joint ? sbeta : nullptr);
}

template <typename T, int RC>
void launch_rc(bool vec, dim3 grid, hipStream_t s, const float* top_val, const int32_t* top_idx,
               const int32_t* anchor_tok, const void* U, const void* Vf, const float* gate, int L,
               int V, int r, float* S0, float* S) {
  const T* u = static_cast<const T*>(U);
  const T* v = static_cast<const T*>(Vf);
  if (vec)
    hipLaunchKernelGGL((pair_score_kernel<T, RC, true>), grid, dim3(64), 0, s, top_val, top_idx,
                       anchor_tok, u, v, gate, L, V, r, S0, S);
  else
    hipLaunchKernelGGL((pair_score_kernel<T, RC, false>), grid, dim3(64), 0, s, top_val, top_idx,
                       anchor_tok, u, v, gate, L, V, r, S0, S);
}

template <typename T>
void launch_t(bool vec, dim3 grid, hipStream_t s, const float* top_val, const int32_t* top_idx,
              const int32_t* anchor_tok, const void* U, const void* Vf, const float* gate, int L,
              int V, int r, float* S0, float* S) {
  const int rc = (r + 3) / 4;
  if (rc <= 8)
    launch_rc<T, 8>(vec, grid, s, top_val, top_idx, anchor_tok, U, Vf, gate, L, V, r, S0, S);
  else if (rc <= 16)
    launch_rc<T, 16>(vec, grid, s, top_val, top_idx, anchor_tok, U, Vf, gate, L, V, r, S0, S);
  else if (rc <= 32)
    launch_rc<T, 32>(vec, grid, s, top_val, top_idx, anchor_tok, U, Vf, gate, L, V, r, S0, S);
  else
    launch_rc<T, 64>(vec, grid, s, top_val, top_idx, anchor_tok, U, Vf, gate, L, V, r, S0, S);
}

}  // namespace

hipError_t launch_pair_score(const float* top_val, const int32_t* top_idx,
                             const int32_t* anchor_tok, const void* U, const void* Vf,
                             const float* gate, int B, int L, int V, int r, int dtype, float* S0,
                             float* S, hipStream_t s) {
  if (B == 0) return hipSuccess;
  const dim3 grid((unsigned)((long long)B * L));
  // 16-byte runs: every lane's quarter (r / 4 elements) must be whole runs
  // and every row, gate row and base 16-byte aligned.
  const uintptr_t bases = reinterpret_cast<uintptr_t>(U) | reinterpret_cast<uintptr_t>(Vf) |
                          reinterpret_cast<uintptr_t>(gate);
  if (dtype == 1) {
    const bool vec = r % 32 == 0 && (bases & 15) == 0;
    launch_t<uint16_t>(vec, grid, s, top_val, top_idx, anchor_tok, U, Vf, gate, L, V, r, S0, S);
  } else {
    const bool vec = r % 16 == 0 && (bases & 15) == 0;
    launch_t<float>(vec, grid, s, top_val, top_idx, anchor_tok, U, Vf, gate, L, V, r, S0, S);
  }
  return hipGetLastError();
}

namespace {
template <typename T, int RC, bool GREEDY>
void launch_pwv_rc(bool vec, dim3 grid, size_t lds, hipStream_t s,
                   const float* top_val, const int32_t* top_idx, const int32_t* anchor_tok,
                   const void* U, const void* Vf, const float* gate, const int32_t* target, int L,
                   int V, int r, float* S0, float* S, int32_t* path_slot, int32_t* path_tok,
                   float* path_score, int32_t* accept_len, int32_t* next_tok) {
  const T* u = static_cast<const T*>(U);
  const T* v = static_cast<const T*>(Vf);
  const dim3 block((unsigned)(64 * min(L, pwv_max_waves<RC>())));
  if (vec)
    hipLaunchKernelGGL((pair_walk_verify_kernel<T, RC, true, GREEDY>), grid, block, lds, s,
                       top_val, top_idx, anchor_tok, u, v, gate, target, L, V, r, S0, S,
                       path_slot, path_tok, path_score, accept_len, next_tok);
  else
    hipLaunchKernelGGL((pair_walk_verify_kernel<T, RC, false, GREEDY>), grid, block, lds, s,
                       top_val, top_idx, anchor_tok, u, v, gate, target, L, V, r, S0, S,
                       path_slot, path_tok, path_score, accept_len, next_tok);
}

template <typename T, bool GREEDY>
void launch_pwv_t(bool vec, dim3 grid, size_t lds, hipStream_t s,
                  const float* top_val, const int32_t* top_idx, const int32_t* anchor_tok,
                  const void* U, const void* Vf, const float* gate, const int32_t* target, int L,
                  int V, int r, float* S0, float* S, int32_t* path_slot, int32_t* path_tok,
                  float* path_score, int32_t* accept_len, int32_t* next_tok) {
  const int rc = (r + 3) / 4;
#define DFLASH2_PWV(RC)                                                                         \
  launch_pwv_rc<T, RC, GREEDY>(vec, grid, lds, s, top_val, top_idx, anchor_tok, U, Vf,   \
                               gate, target, L, V, r, S0, S, path_slot, path_tok, path_score,   \
                               accept_len, next_tok)
  if (rc <= 8)
    DFLASH2_PWV(8);
  else if (rc <= 16)
    DFLASH2_PWV(16);
  else if (rc <= 32)
    DFLASH2_PWV(32);
  else
    DFLASH2_PWV(64);
#undef DFLASH2_PWV
}
}  // namespace

hipError_t launch_pair_walk_verify(const float* top_val, const int32_t* top_idx,
                                   const int32_t* anchor_tok, const void* U, const void* Vf,
                                   const float* gate, const int32_t* target, int B, int L, int V,
                                   int r, int dtype, int greedy, float* S0, float* S,
                                   int32_t* path_slot, int32_t* path_tok, float* path_score,
                                   int32_t* accept_len, int32_t* next_tok, hipStream_t s) {
  if (B == 0) return hipSuccess;
  const dim3 grid((unsigned)B);
  const size_t lds = (size_t)(L - 1) * kTopK * kTopK * sizeof(float);
  const uintptr_t bases = reinterpret_cast<uintptr_t>(U) | reinterpret_cast<uintptr_t>(Vf) |
                          reinterpret_cast<uintptr_t>(gate);
  if (dtype == 1) {
    const bool vec = r % 32 == 0 && (bases & 15) == 0;
    if (greedy)
      launch_pwv_t<uint16_t, true>(vec, grid, lds, s, top_val, top_idx, anchor_tok, U, Vf,
                                   gate, target, L, V, r, S0, S, path_slot, path_tok, path_score,
                                   accept_len, next_tok);
    else
      launch_pwv_t<uint16_t, false>(vec, grid, lds, s, top_val, top_idx, anchor_tok, U, Vf,
                                    gate, target, L, V, r, S0, S, path_slot, path_tok, path_score,
                                    accept_len, next_tok);
  } else {
    const bool vec = r % 16 == 0 && (bases & 15) == 0;
    if (greedy)
      launch_pwv_t<float, true>(vec, grid, lds, s, top_val, top_idx, anchor_tok, U, Vf,
                                gate, target, L, V, r, S0, S, path_slot, path_tok, path_score,
                                accept_len, next_tok);
    else
      launch_pwv_t<float, false>(vec, grid, lds, s, top_val, top_idx, anchor_tok, U, Vf,
                                 gate, target, L, V, r, S0, S, path_slot, path_tok, path_score,
                                 accept_len, next_tok);
  }
  return hipGetLastError();
}

namespace {
template <typename T, int RC>
void launch_ps_rc(bool vec, dim3 grid, size_t lds, hipStream_t s, const float* top_val,
                  const int32_t* top_idx, const int32_t* anchor_tok, const void* U, const void* Vf,
                  const float* gate, const float* u, float inv_t, int L, int V, int r, int joint,
                  float* S0, float* S, int32_t* path_slot, int32_t* path_tok, float* q) {
  const T* uu = static_cast<const T*>(U);
  const T* vv = static_cast<const T*>(Vf);
  const dim3 block((unsigned)(64 * min(L, pwv_max_waves<RC>())));
  if (vec)
    hipLaunchKernelGGL((pair_sample_kernel<T, RC, true>), grid, block, lds, s, top_val, top_idx,
                       anchor_tok, uu, vv, gate, u, inv_t, L, V, r, joint, S0, S, path_slot,
                       path_tok, q);
  else
    hipLaunchKernelGGL((pair_sample_kernel<T, RC, false>), grid, block, lds, s, top_val, top_idx,
                       anchor_tok, uu, vv, gate, u, inv_t, L, V, r, joint, S0, S, path_slot,
                       path_tok, q);
}

template <typename T>
void launch_ps_t(bool vec, dim3 grid, size_t lds, hipStream_t s, const float* top_val,
                 const int32_t* top_idx, const int32_t* anchor_tok, const void* U, const void* Vf,
                 const float* gate, const float* u, float inv_t, int L, int V, int r, int joint,
                 float* S0, float* S, int32_t* path_slot, int32_t* path_tok, float* q) {
  const int rc = (r + 3) / 4;
#define DFLASH2_PS(RC)                                                                          \
  launch_ps_rc<T, RC>(vec, grid, lds, s, top_val, top_idx, anchor_tok, U, Vf, gate, u, inv_t, L, \
                      V, r, joint, S0, S, path_slot, path_tok, q)
  if (rc <= 8)
    DFLASH2_PS(8);
  else if (rc <= 16)
    DFLASH2_PS(16);
  else if (rc <= 32)
    DFLASH2_PS(32);
  else
    DFLASH2_PS(64);
#undef DFLASH2_PS
}
}  // namespace

hipError_t launch_pair_sample(const float* top_val, const int32_t* top_idx,
                              const int32_t* anchor_tok, const void* U, const void* Vf,
                              const float* gate, const float* u, float temperature, int B, int L,
                              int V, int r, int dtype, int joint, float* S0, float* S,
                              int32_t* path_slot, int32_t* path_tok, float* q, hipStream_t s) {
  if (B == 0) return hipSuccess;
  const dim3 grid((unsigned)B);
  const size_t lds = (size_t)(L - 1) * kTopK * kTopK * sizeof(float);
  const float inv_t = 1.0f / temperature;
  const uintptr_t bases = reinterpret_cast<uintptr_t>(U) | reinterpret_cast<uintptr_t>(Vf) |
                          reinterpret_cast<uintptr_t>(gate);
  if (dtype == 1)
    launch_ps_t<uint16_t>(r % 32 == 0 && (bases & 15) == 0, grid, lds, s, top_val, top_idx,
                          anchor_tok, U, Vf, gate, u, inv_t, L, V, r, joint, S0, S, path_slot,
                          path_tok, q);
  else
    launch_ps_t<float>(r % 16 == 0 && (bases & 15) == 0, grid, lds, s, top_val, top_idx,
                       anchor_tok, U, Vf, gate, u, inv_t, L, V, r, joint, S0, S, path_slot,
                       path_tok, q);
  return hipGetLastError();
}

}  // namespace dflash2
