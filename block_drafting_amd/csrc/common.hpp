// Internal declarations shared by the HIP sources of libdflash2 (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dflash2 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTopK = 16;
constexpr int kWave = 64;
constexpr int kMaxWalk = 64;  // longest block a path walk takes (one slot per lane)

// bf16 storage <-> fp32 arithmetic.  A bf16 value is the upper half of an
// IEEE single, so widening is a shift; narrowing uses the gfx950 hardware
// convert (round to nearest even).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Value of lane (lane ^ J) for 32-bit data.  Partners within a 16-lane row
// use DPP (quad_perm; xor 4 = quad reverse after row_half_mirror; xor 8 =
// row_half_mirror after row_mirror); xor 16 and xor 32 use the gfx950 lane
// swaps (v_permlane16_swap: odd rows of the first operand trade places with
// even rows of the second; v_permlane32_swap: the upper half of the first
// with the lower half of the second; with both operands v, a lane finds its
// partner in the first result when it sits in the odd row / upper half,
// else in the second).  All are VALU operations, no LDS traffic.
template <int J>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  if constexpr (J == 1) {
    return __builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xf, 0xf, false);  // quad_perm [1,0,3,2]
  } else if constexpr (J == 2) {
    return __builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xf, 0xf, false);  // quad_perm [2,3,0,1]
  } else if constexpr (J == 4) {
    const uint32_t h = __builtin_amdgcn_update_dpp(0u, v, 0x141, 0xf, 0xf, false);
    return __builtin_amdgcn_update_dpp(0u, h, 0x1B, 0xf, 0xf, false);
  } else if constexpr (J == 8) {
    const uint32_t m = __builtin_amdgcn_update_dpp(0u, v, 0x140, 0xf, 0xf, false);
    return __builtin_amdgcn_update_dpp(0u, m, 0x141, 0xf, 0xf, false);
  } else if constexpr (J == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (threadIdx.x & 16) ? r[0] : r[1];
  } else {
    static_assert(J == 32, "xor partner 1, 2, 4, 8, 16 or 32");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (threadIdx.x & 32) ? r[0] : r[1];
  }
}

// Workgroup i of a launch runs on XCD i mod 8, and each XCD has its own L2.
// Bijection from dispatch order to tile order that gives XCD x a contiguous
// range of tiles, so tiles that share operand rows share an L2.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_tile(int pid, int ntiles) {
  const int xcd = pid % kXcds;
  const int local = pid / kXcds;
  const int q = ntiles / kXcds;
  const int rem = ntiles % kXcds;
  return xcd < rem ? xcd * (q + 1) + local : rem * (q + 1) + (xcd - rem) * q + local;
}

// ---------------------------------------------------------------- launches
// Each returns hipSuccess or the launch error; arguments are already valid.
hipError_t launch_twotap_conv(const void* x, const void* anchor_h, void* y, const float* k0,
                              const float* k1, const float* proj, int groups, int B, int L,
                              int H, int dtype, hipStream_t s);

hipError_t launch_twotap_conv_mm(const void* x, const void* anchor_h, void* y, const float* k0,
                                 const float* k1, const void* projT, int groups, int B, int L,
                                 int H, hipStream_t s);

// Columns per tile maximum (the bf16 GEMM's N tile).
constexpr int kTileMaxCols = 256;

// The LM-head weight in the GEMM's tiled layout (dtype code 2 of launch_lmhead).
size_t lmhead_pack_bytes(int V, int H);
hipError_t launch_lmhead_pack(const void* W, void* Wp, int V, int H, hipStream_t s);
hipError_t launch_lmhead(const void* h, const void* W, float* logits, float* tmax, int M, int H,
                         int V, int dtype, hipStream_t s);

// Candidate form of the bf16 GEMM + tile maxima (logits kept only where the
// top-16 may need them): per (row, N tile) a count cnt (kCandDense: the
// tile's logits were stored) and kCandSlots (value bits, column) slots; gmax
// [M, 16] is the GEMM's own scratch (reset by the launch).  dtype 1 or 2.
constexpr int kCandSlots = 4;
constexpr int kCandDense = -1;
hipError_t launch_lmhead_cand(const void* h, const void* W, float* logits, float* tmax,
                              uint32_t* gmax, int* cnt, void* slots, int M, int H, int V,
                              int dtype, hipStream_t s);
hipError_t launch_topk16_cand(const float* logits, const float* tmax, const int* cnt,
                              const void* slots, float* top_val, int32_t* top_idx, int M, int V,
                              hipStream_t s);

int topk16_splits(int M, int V);
size_t topk16_workspace_bytes(int M, int V);
hipError_t launch_topk16(const float* logits, float* top_val, int32_t* top_idx, int M, int V,
                         void* workspace, hipStream_t s);
hipError_t launch_topk16_tilemax(const float* logits, const float* tmax, float* top_val,
                                 int32_t* top_idx, int M, int V, hipStream_t s);

// Pair scores + walk (greedy != 0: best successor, else max-plus) + greedy
// verification of each block in one launch; S0 / S may be NULL.
hipError_t launch_pair_walk_verify(const float* top_val, const int32_t* top_idx,
                                   const int32_t* anchor_tok, const void* U, const void* Vf,
                                   const float* gate, const int32_t* target, int B, int L, int V,
                                   int r, int dtype, int greedy, float* S0, float* S,
                                   int32_t* path_slot, int32_t* path_tok, float* path_score,
                                   int32_t* accept_len, int32_t* next_tok, hipStream_t s);
// Pair scores + the sampling walk of each block in one launch; S0 / S may be NULL.
// joint != 0: the whole path drawn from exp(score / T) (backward messages),
// else the chain sampler.
hipError_t launch_pair_sample(const float* top_val, const int32_t* top_idx,
                              const int32_t* anchor_tok, const void* U, const void* Vf,
                              const float* gate, const float* u, float temperature, int B, int L,
                              int V, int r, int dtype, int joint, float* S0, float* S,
                              int32_t* path_slot, int32_t* path_tok, float* q, hipStream_t s);
hipError_t launch_pair_score(const float* top_val, const int32_t* top_idx,
                             const int32_t* anchor_tok, const void* U, const void* Vf,
                             const float* gate, int B, int L, int V, int r, int dtype, float* S0,
                             float* S, hipStream_t s);

hipError_t launch_context_gate(const void* h, const void* Wg, float* gate, int M, int H, int r,
                               int dtype, hipStream_t s);

hipError_t launch_path_select(const float* S0, const float* S, const int32_t* top_idx, int B,
                              int L, int greedy, int32_t* path_slot, int32_t* path_tok,
                              float* path_score, hipStream_t s);

hipError_t launch_path_sample(const float* S0, const float* S, const int32_t* top_idx,
                              const float* u, float temperature, int B, int L, int joint,
                              int32_t* path_slot, int32_t* path_tok, float* q, hipStream_t s);

hipError_t launch_target_lse(const float* z, int R, int V, float temperature, float* lse,
                             hipStream_t s);

size_t verify_rejection_lds(int V);
// The staged rows' records ([B, rows] of them) and the two-launch form of the
// lazy verification that fills them first.
size_t verify_rejection_staged_bytes(int B, int V, int rows);
hipError_t launch_verify_rejection_staged(const int32_t* path_slot, const int32_t* path_tok,
                                          const float* q, const int32_t* top_idx, const float* z,
                                          float temperature, const float* u_acc,
                                          const float* u_res, int B, int L, int V, int rows,
                                          float* staged, int32_t* accept_len, int32_t* next_tok,
                                          hipStream_t s);
size_t verify_rejection_lazy_lds(int V);
hipError_t launch_verify_rejection_lazy(const int32_t* path_slot, const int32_t* path_tok,
                                        const float* q, const int32_t* top_idx, const float* z,
                                        float temperature, const float* u_acc, const float* u_res,
                                        int B, int L, int V, int32_t* accept_len,
                                        int32_t* next_tok, hipStream_t s);
hipError_t launch_verify_rejection(const int32_t* path_slot, const int32_t* path_tok,
                                   const float* q, const int32_t* top_idx, const float* z,
                                   const float* lse, float temperature, const float* u_acc,
                                   const float* u_res, int B, int L, int V, int32_t* accept_len,
                                   int32_t* next_tok, hipStream_t s);

// Attainable-peak probe: the GEMM's matrix-core work without memory traffic.
size_t probe_mfma_operand_bytes(int nwg);
hipError_t launch_probe_mfma(const void* operands, int nwg, int iters, float* out, hipStream_t s);

hipError_t launch_verify_greedy(const int32_t* path_tok, const int32_t* target, int B, int L,
                                int32_t* accept_len, int32_t* next_tok, hipStream_t s);

}  // namespace dflash2
