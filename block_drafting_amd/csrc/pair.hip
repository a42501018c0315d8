// Adjacent-pair scores ("DFlash 2: Keep Drafting Parallel", section
// "A lightweight path selector", eq. S_t(a,b)) in low-rank form
//   S_t[i, j] = logit_t(c_{t,j}) + (U[c_{t-1,i}] * g_t) . V[c_{t,j}],
// with the last verified token as the previous token of position 0.  g_t is
// the context gate of position t (an r-vector); without one it is all ones.
//
// One wavefront per (block, position): it gathers the 16 (or 1) previous
// factor rows and the 16 current factor rows into LDS as fp32, then each lane
// produces four neighbouring outputs (one 16-byte store).  All pairs of all
// positions are independent, so the whole tensor is scored in one launch.
#include "common.hpp"

namespace dflash2 {
namespace {

template <typename T>
__device__ __forceinline__ float widen(T v);
template <>
__device__ __forceinline__ float widen<float>(float v) { return v; }
template <>
__device__ __forceinline__ float widen<uint16_t>(uint16_t v) {
  return __uint_as_float((uint32_t)v << 16);
}

// Gather `rows` factor rows (ids[0..rows)) of rank r into lds (stride r+1).
// Ids outside [0, V) fill their row with NaN.  When a row is a whole number
// of 16-byte runs (VEC), every lane issues all of its runs before using any,
// so the wave pays one memory latency for the random rows instead of one per
// element.
template <typename T, bool VEC>
__device__ void gather_rows(const T* __restrict__ F, const int32_t* ids, int rows, int r, int V,
                            float* lds) {
  const int lane = threadIdx.x;
  if (VEC) {
    constexpr int kPer = 16 / sizeof(T);        // elements per 16-byte run
    constexpr int kMaxRuns = 16 * 256 / kPer / 64;  // runs per lane at r = 256
    const int cpr = r / kPer;                    // runs per row
    const int total = rows * cpr;
    u32x4_t buf[kMaxRuns];
    int rowof[kMaxRuns];
#pragma unroll
    for (int q = 0; q < kMaxRuns; ++q) {
      const int e = lane + q * 64;
      rowof[q] = -1;
      if (e < total) {
        const int row = e / cpr;
        const int id = ids[row];
        if (id >= 0 && id < V) {
          buf[q] = *reinterpret_cast<const u32x4_t*>(F + (size_t)id * r + (e - row * cpr) * kPer);
          rowof[q] = row;
        } else {
          rowof[q] = -2 - row;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kMaxRuns; ++q) {
      const int e = lane + q * 64;
      if (e >= total) continue;
      const int row = rowof[q] >= 0 ? rowof[q] : -2 - rowof[q];
      float* dst = lds + row * (r + 1) + (e - row * cpr) * kPer;
      if (rowof[q] < 0) {
#pragma unroll
        for (int k = 0; k < kPer; ++k) dst[k] = __builtin_nanf("");
      } else if (sizeof(T) == 2) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          dst[2 * k] = bf16_lo(buf[q][k]);
          dst[2 * k + 1] = bf16_hi(buf[q][k]);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) dst[k] = __uint_as_float(buf[q][k]);
      }
    }
    return;
  }
  for (int e = lane; e < rows * r; e += 64) {
    const int row = e / r;
    const int k = e - row * r;
    const int id = ids[row];
    lds[row * (r + 1) + k] =
        (id >= 0 && id < V) ? widen<T>(F[(size_t)id * r + k]) : __builtin_nanf("");
  }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(64) void pair_score_kernel(const float* __restrict__ top_val,
                                                        const int32_t* __restrict__ top_idx,
                                                        const int32_t* __restrict__ anchor_tok,
                                                        const T* __restrict__ U,
                                                        const T* __restrict__ Vf,
                                                        const float* __restrict__ gate, int L,
                                                        int V, int r, float* __restrict__ S0,
                                                        float* __restrict__ S) {
  extern __shared__ float lds[];
  const int b = blockIdx.x / L;
  const int t = blockIdx.x - b * L;
  const int lane = threadIdx.x;
  const int stride = r + 1;
  float* su = lds;                 // previous-token factors, up to 16 rows
  float* sv = lds + 16 * stride;   // current-candidate factors, 16 rows
  const int32_t* cur = top_idx + ((size_t)b * L + t) * kTopK;
  const float* tv = top_val + ((size_t)b * L + t) * kTopK;

  float* sg = lds + 32 * stride;   // gate of this position
  if (gate) {
    const float* g = gate + ((size_t)b * L + t) * r;
    for (int k = lane; k < r; k += 64) sg[k] = g[k];
  }
  gather_rows<T, VEC>(Vf, cur, kTopK, r, V, sv);
  if (t == 0) {
    if (anchor_tok) gather_rows<T, VEC>(U, anchor_tok + b, 1, r, V, su);
    __syncthreads();
    if (gate && anchor_tok) {
      for (int k = lane; k < r; k += 64) su[k] *= sg[k];
      __syncthreads();
    }
    if (lane < kTopK) {
      float acc = 0.f;
      if (anchor_tok) {
        for (int k = 0; k < r; ++k) acc = fmaf(su[k], sv[lane * stride + k], acc);
      } else if (cur[lane] < 0 || cur[lane] >= V) {
        acc = __builtin_nanf("");
      }
      S0[(size_t)b * kTopK + lane] = tv[lane] + acc;
    }
    return;
  }
  gather_rows<T, VEC>(U, cur - kTopK, kTopK, r, V, su);
  __syncthreads();
  if (gate) {
    // A(a) (.) H(h_t): scale the previous-token rows once, before the dots
    for (int e = lane; e < kTopK * r; e += 64) {
      const int i = e / r;
      const int k = e - i * r;
      su[i * stride + k] *= sg[k];
    }
    __syncthreads();
  }
  const int i = lane >> 2;
  const int j0 = (lane & 3) * 4;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const float* ui = su + i * stride;
  for (int k = 0; k < r; ++k) {
    const float u = ui[k];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = fmaf(u, sv[(j0 + q) * stride + k], acc[q]);
  }
  f32x4_t out;
#pragma unroll
  for (int q = 0; q < 4; ++q) out[q] = tv[j0 + q] + acc[q];
  float* dst = S + (((size_t)b * (L - 1) + (t - 1)) * kTopK + i) * kTopK + j0;
  *reinterpret_cast<f32x4_t*>(dst) = out;
}

}  // namespace

hipError_t launch_pair_score(const float* top_val, const int32_t* top_idx,
                             const int32_t* anchor_tok, const void* U, const void* Vf,
                             const float* gate, int B, int L, int V, int r, int dtype, float* S0,
                             float* S, hipStream_t s) {
  if (B == 0) return hipSuccess;
  const size_t lds = ((size_t)2 * kTopK * (r + 1) + (gate ? r : 0)) * sizeof(float);
  const dim3 grid((unsigned)((long long)B * L));
  const bool vec_bf16 = r % 8 == 0 && ((reinterpret_cast<uintptr_t>(U) | reinterpret_cast<uintptr_t>(Vf)) & 15) == 0;
  const bool vec_f32 = r % 4 == 0 && ((reinterpret_cast<uintptr_t>(U) | reinterpret_cast<uintptr_t>(Vf)) & 15) == 0;
  const uint16_t* Ub = static_cast<const uint16_t*>(U);
  const uint16_t* Vb = static_cast<const uint16_t*>(Vf);
  const float* Uf = static_cast<const float*>(U);
  const float* Vff = static_cast<const float*>(Vf);
  if (dtype == 1 && vec_bf16)
    hipLaunchKernelGGL((pair_score_kernel<uint16_t, true>), grid, dim3(64), lds, s, top_val, top_idx,
                       anchor_tok, Ub, Vb, gate, L, V, r, S0, S);
  else if (dtype == 1)
    hipLaunchKernelGGL((pair_score_kernel<uint16_t, false>), grid, dim3(64), lds, s, top_val,
                       top_idx, anchor_tok, Ub, Vb, gate, L, V, r, S0, S);
  else if (vec_f32)
    hipLaunchKernelGGL((pair_score_kernel<float, true>), grid, dim3(64), lds, s, top_val, top_idx,
                       anchor_tok, Uf, Vff, gate, L, V, r, S0, S);
  else
    hipLaunchKernelGGL((pair_score_kernel<float, false>), grid, dim3(64), lds, s, top_val, top_idx,
                       anchor_tok, Uf, Vff, gate, L, V, r, S0, S);
  return hipGetLastError();
}

}  // namespace dflash2
