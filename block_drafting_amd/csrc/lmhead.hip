// LM-head logits z = h . W^T ("DFlash 2: Keep Drafting Parallel", section
// "A lightweight path selector": the pair score's unary term is the drafter's
// own logit, computed once per position).  The only dense contraction of the
// step: M = blocks x positions rows, N = vocabulary, K = hidden.
//
// bf16 path: v_mfma_f32_32x32x16_bf16 tiles.  A workgroup of eight waves
// (two per SIMD, so one wave's MFMAs cover the other's memory waits) owns a
// 256 x 256 output tile; each wave accumulates a 128 x 64 sub-tile.  K is
// walked in 64-wide slices through two padded LDS stages; both operands are
// K-contiguous, so every thread moves 16-byte runs of 8 bf16 with buffer
// loads into one of two register staging sets (two slices ahead of use)
// and writes them to LDS between MFMAs.
// Tiles are numbered so that the M-tiles sharing one W slice run back to back
// on the same XCD (workgroup i is dispatched to XCD i mod 8), so W is pulled
// from HBM about once and re-read from that XCD's L2.
//
// fp32 path (fp32 workloads): a plain per-output fp32 dot product.
//
// Optionally the kernel also writes, for every row, the maximum over each
// 256-column N tile (tmax [M, ceil(N / 256)]).  The 16th largest of a row's
// tile maxima bounds its 16th largest logit from below, so the top-16 only
// has to read the tiles whose maximum reaches that bound (usually 16 of the
// 594 at V = 151936) instead of the whole row.
#include <type_traits>

#include "common.hpp"

namespace dflash2 {
namespace {

// ord(): canonical floats (-0 -> +0, NaN -> -inf) onto uint32 in the same order.
__device__ __forceinline__ uint32_t cand_ord(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) u = 0xff800000u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float cand_val(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
constexpr uint32_t kCandOrdNegInf = 0x007fffffu;  // cand_ord(-inf)

template <int BM, int BN, int BK, int WM, int WN>
struct GemmCfg {
  static constexpr int kThreads = WM * WN * 64;
  static constexpr int kLdk = BK + 8;            // padded LDS row pitch (elements)
  static constexpr int kTm = BM / WM / 32;       // 32x32 blocks per wave along M
  static constexpr int kTn = BN / WN / 32;       // ... along N
  static constexpr int kChunksPerRow = BK / 8;   // 16-byte runs per tile row
  static constexpr int kAPer = BM * kChunksPerRow / kThreads;
  static constexpr int kBPer = BN * kChunksPerRow / kThreads;
  static constexpr int kStage = (BM + BN) * kLdk;  // elements per LDS stage
  static_assert(BM % (WM * 32) == 0 && BN % (WN * 32) == 0, "wave tile");
  static_assert(BK % 16 == 0, "k step");
  static_assert((BM * kChunksPerRow) % kThreads == 0, "A load split");
  static_assert((BN * kChunksPerRow) % kThreads == 0, "B load split");
};

// PACKED: W comes in the tiled layout of lmhead_pack_kernel (each 256-row x
// 64-column block contiguous), so every slice of a W tile is one 32 KB run.
//
// CAND (logits not wanted, only the top-16): a row of a tile writes its
// logits only when it cannot prove they are not needed.  Each row keeps 16
// group maxima in memory (group = N tile mod 16): every finished tile raises
// its group's entry to its row maximum (an atomic max of the order-preserving
// uint32 of the value).  The 16 group maxima are 16 distinct elements of the
// row, so their minimum theta is at most the row's 16th largest logit, at
// any moment and whatever a reader sees of the other tiles' updates (entries
// only grow).  A tile row that finds all 16 groups filled stores only its
// values >= theta, as (value bits, column) pairs in kCandSlots slots, with
// their count; a row whose groups are not all filled yet (the first round
// of tiles) or that has more than kCandSlots such values stores its 256
// logits to C and count kCandDense.  Every top-16 element of the row is
// then either in a stored tile or in a slot.
struct CandOut {
  uint32_t* gmax;  // [M, 16] group maxima (orders), reset to cand_ord(-inf) before the launch
  int* cnt;        // [M, ntiles] slots used, or kCandDense
  uint2* slots;    // [M, ntiles, kCandSlots] (value bits, column)
};

template <int BM, int BN, int BK, int WM, int WN, bool KTAIL, bool PACKED, bool CAND>
__global__ __launch_bounds__(WM* WN * 64) void lmhead_bf16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bw, float* __restrict__ C,
    float* __restrict__ tmax, int M, int N, int K, int mtiles, int ntiles, int nt0,
    CandOut cand) {
  using Cfg = GemmCfg<BM, BN, BK, WM, WN>;
  constexpr int kT = Cfg::kThreads;
  constexpr int kLdk = Cfg::kLdk;
  constexpr int kCpr = Cfg::kChunksPerRow;
  constexpr int kTm = Cfg::kTm;
  constexpr int kTn = Cfg::kTn;
  constexpr int kSteps = BK / 16;
  constexpr int kLoads = Cfg::kAPer + Cfg::kBPer;
  static_assert(kSteps >= 3 && kSteps % 2 == 0, "pipeline needs an even step count >= 4");
  static_assert(!CAND || kT >= BM, "one thread per tile row in the candidate epilogue");
  static_assert((WN + 2) * BM * 4 + BM * kCandSlots * 8 + 8 <= 2 * Cfg::kStage * 2,
                "epilogue LDS fits in the stages");
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * Cfg::kStage];

  // this launch's tiles: N tiles nt0, nt0 + 1, ... of all ntiles, M fastest
  const int tile = xcd_tile(blockIdx.x, (int)gridDim.x);
  const int mt = tile % mtiles;
  const int nt = nt0 + tile / mtiles;
  const int m0 = mt * BM;
  const int n0 = nt * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % WM;
  const int wn = wave / WM;

  // Each thread moves kLoads 16-byte runs per K slice through buffer loads:
  // one descriptor per operand tile (base = first row of the tile, size = the
  // rows that exist) and a 32-bit byte offset per run.  Every access is range
  // checked by the hardware: rows past the matrix edge, and the prefetches
  // past the end of K that the last slices issue, read as zero or as rows of
  // this tile that are never used, so the loads need no branches.
  constexpr int kRowStep = kT / kCpr;  // tile rows covered by one pass of the block
  const int row0 = tid / kCpr;
  const int kof = (tid % kCpr) * 8;
  const int rowsA = min(BM, M - m0);
  const int rowsB = min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(A + (size_t)m0 * K), (short)0, rowsA * K * 2, 0x00020000);
  const int nk = (K + BK - 1) / BK;  // K slices (the packed layout's blocks per tile)
  const __amdgpu_buffer_rsrc_t rsB =
      PACKED ? __builtin_amdgcn_make_buffer_rsrc(
                   const_cast<uint16_t*>(Bw + (size_t)nt * nk * BN * BK), (short)0,
                   nk * BN * BK * 2, 0x00020000)
             : __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Bw + (size_t)n0 * K),
                                                 (short)0, rowsB * K * 2, 0x00020000);
  const int voff0 = (row0 * K + kof) * 2;
  const int vstep = kRowStep * K * 2;
  // packed W: row r, chunk kof of slice s at ((s * BN + r) * BK + kof) * 2 bytes
  const int voffB0 = PACKED ? (row0 * BK + kof) * 2 : voff0;
  const int vstepB = PACKED ? kRowStep * BK * 2 : vstep;
  // Two register staging sets: the loads of slice c are issued while slice
  // c-3 is multiplied and written to LDS while slice c-1 is, so HBM latency
  // (first touch of a W row) has about two slices of MFMA work to hide under.
  // Slices past the end of K re-read the last slice (an L2 hit, never used).
  const int klast = (nk - 1) * BK;
  u32x4_t R0[kLoads], R1[kLoads];
  auto gload = [&](u32x4_t(&R)[kLoads], int k0) {
    k0 = min(k0, klast);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const bool isA = i < Cfg::kAPer;
      const int ii = isA ? i : i - Cfg::kAPer;
      // the whole offset sits in the per-lane part so the range check covers it
      const int off = isA ? voff0 + ii * vstep + k0 * 2
                          : voffB0 + ii * vstepB + (PACKED ? (k0 / BK) * (BN * BK * 2) : k0 * 2);
      u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(isA ? rsA : rsB, off, 0, 0);
      if (KTAIL && k0 + kof >= K) v = u32x4_t{0, 0, 0, 0};
      R[i] = v;
    }
  };
  // LDS destination of run i: row (row0 + ii * kRowStep) of the A or B part.
  const int dst0 = row0 * kLdk + kof;
  auto sstore = [&](const u32x4_t(&R)[kLoads], uint16_t* stage) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const bool isA = i < Cfg::kAPer;
      const int ii = isA ? i : i - Cfg::kAPer;
      *reinterpret_cast<u32x4_t*>(stage + dst0 + ((isA ? 0 : BM) + ii * kRowStep) * kLdk) = R[i];
    }
  };

  f32x16_t acc[kTm][kTn];
#pragma unroll
  for (int i = 0; i < kTm; ++i)
#pragma unroll
    for (int j = 0; j < kTn; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Fragment offsets (elements) inside a stage: lane l supplies row l % 32 of
  // a 32-row block and the 8 k values starting at 8 * (l / 32).
  const int a_frag = (wm * (BM / WM) + (lane & 31)) * kLdk + (lane >> 5) * 8;
  const int b_frag = (BM + wn * (BN / WN) + (lane & 31)) * kLdk + (lane >> 5) * 8;
  bf16x8_t FA[2][kTm], FB[2][kTn];
  auto fread = [&](const uint16_t* st, int kk, int slot) {
#pragma unroll
    for (int i = 0; i < kTm; ++i)
      FA[slot][i] = __builtin_bit_cast(
          bf16x8_t, *reinterpret_cast<const u32x4_t*>(st + a_frag + i * 32 * kLdk + kk * 16));
#pragma unroll
    for (int j = 0; j < kTn; ++j)
      FB[slot][j] = __builtin_bit_cast(
          bf16x8_t, *reinterpret_cast<const u32x4_t*>(st + b_frag + j * 32 * kLdk + kk * 16));
  };
  auto mfma = [&](int slot) {
#pragma unroll
    for (int i = 0; i < kTm; ++i)
#pragma unroll
      for (int j = 0; j < kTn; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FA[slot][i], FB[slot][j], acc[i][j], 0,
                                                            0, 0);
  };

  // One K slice (kSteps k-steps of 16).  Rs holds slice kt+1 on entry; it is
  // written to the other LDS stage during step 1 and reloaded with slice
  // kt+3 right after (the earlier the loads go out, the more of their
  // latency the next two slices hide: ~2% faster than issuing them after
  // the barrier).
  //   step kk:   read fragments of step kk+1 | 16 MFMAs on step kk
  //   step 1:    + the stage writes, one per MFMA, then the global loads of slice kt+3
  //   step S-2:  + barrier
  //   step S-1:  the fragment reads come from the next stage (visible after the barrier)
  // The body has no branches: a conditional body makes the register
  // allocator spill the accumulators.
  auto slice = [&](int kt, u32x4_t(&Rs)[kLoads]) {
    const uint16_t* cur = lds + (kt & 1) * Cfg::kStage;
    uint16_t* nxt = lds + ((kt & 1) ^ 1) * Cfg::kStage;
#pragma unroll
    for (int kk = 0; kk < kSteps; ++kk) {
      if (kk + 1 < kSteps) {
        fread(cur, kk + 1, (kk + 1) & 1);
      } else {
        fread(nxt, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      mfma(kk & 1);
      if (kk == 1) {
        sstore(Rs, nxt);
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // one LDS write
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (kk == 1) {
        gload(Rs, (kt + 3) * BK);  // Rs is in LDS now: reload it at once
        __builtin_amdgcn_sched_barrier(0);
      }
      if (kk == kSteps - 2) {
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  gload(R0, 0);
  gload(R1, BK);
  sstore(R0, lds);
  __syncthreads();
  gload(R0, 2 * BK);
  fread(lds, 0, 0);
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    slice(kt, R1);
    slice(kt + 1, R0);
  }
  if (kt < nk) slice(kt, R1);

  // Accumulator layout of a 32x32 block: register r of lane l holds
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32.  Half-waves store 128-byte runs.
  // CAND: this row's group maxima, loaded during the last exchange steps
  // (earlier they would compete with the 64 values per lane for registers)
  u32x4_t gq[4];
  float* red = reinterpret_cast<float*>(lds);  // [WN][BM]; the stages are done
  float* cth = red + WN * BM;                  // CAND: per row, theta (-inf: dense)
  int* cpos = reinterpret_cast<int*>(cth + BM);  // CAND: per row, slots taken
  uint2* cslot = reinterpret_cast<uint2*>(cpos + BM);  // CAND: per row, kCandSlots slots
  int* cflag = reinterpret_cast<int*>(cslot + BM * kCandSlots);  // CAND: [0] some row dense,
                                                                 // [1] every row dense
  if (tmax) {
    // Maximum of every row over this tile's BN columns (columns past N
    // excluded, NaN ignored by fmaxf).  Each lane holds kTm * 16 rows of its
    // half-wave's 32 columns; a reduce-scatter across the 32 lanes (each
    // exchange step halves the values a lane keeps: 62 lane exchanges in
    // place of 64 full butterflies) leaves every lane two finished rows,
    // and the WN waves of a row band meet in LDS.
    static_assert(kTm * 16 == 64, "reduce-scatter sized for 64 rows per lane");
    float v[64];
#pragma unroll
    for (int i = 0; i < kTm; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = -INFINITY;
#pragma unroll
        for (int j = 0; j < kTn; ++j) {
          const int col = n0 + wn * (BN / WN) + j * 32 + (lane & 31);
          if (col < N) x = fmaxf(x, acc[i][j][r]);
        }
        v[i * 16 + r] = x;
      }
    // step with partner lane ^ D on N values: the lane with bit D set keeps
    // the upper half, the other the lower half, each taking the partner's max
    auto step = [&](auto dtag, int n) {
      constexpr int D = decltype(dtag)::value;
      const bool hi = (lane & D) != 0;
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        if (k < n / 2) {
          const float send = hi ? v[k] : v[k + n / 2];
          const float keep = hi ? v[k + n / 2] : v[k];
          const float recv = __uint_as_float(xor_lane<D>(__float_as_uint(send)));
          v[k] = fmaxf(keep, recv);
        }
      }
    };
    step(std::integral_constant<int, 1>{}, 64);
    step(std::integral_constant<int, 2>{}, 32);
    step(std::integral_constant<int, 4>{}, 16);
    if (CAND && tid < BM && m0 + tid < M) {
      // relaxed atomic loads: other workgroups raise these entries meanwhile,
      // and any value read is a valid (possibly older, so lower) group
      // maximum.  Workgroup scope reads this XCD's L2, which its own
      // workgroups' atomics keep up to date; an agent-scope load reads a
      // copy further out that lags it, which lowers the bound and makes
      // more tile rows overflow their slots.
      uint32_t* gm = cand.gmax + (size_t)(m0 + tid) * 16;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          gq[q][e] = __hip_atomic_load(gm + 4 * q + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    step(std::integral_constant<int, 8>{}, 8);
    step(std::integral_constant<int, 16>{}, 4);
    __syncthreads();  // every wave is done with the stages
    // v[j] now holds value index 32 b0 + 16 b1 + 8 b2 + 4 b3 + 2 b4 + j
    // (b_s = bit s of the lane within its half), index = i * 16 + r
    const int l5 = lane & 31;
    const int base = ((l5 & 1) << 5) | ((l5 & 2) << 3) | ((l5 & 4) << 1) | ((l5 & 8) >> 1) |
                     ((l5 & 16) >> 3);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int idx = base + j;
      const int i = idx >> 4;
      const int r = idx & 15;
      red[wn * BM + wm * (BM / WM) + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)] = v[j];
    }
    if (CAND && tid == 0) {
      cflag[0] = 0;
      cflag[1] = 1;
    }
    __syncthreads();
    for (int row = tid; row < BM; row += kT) {
      float v = red[row];
#pragma unroll
      for (int w = 1; w < WN; ++w) v = fmaxf(v, red[w * BM + row]);
      if (m0 + row < M) tmax[(size_t)(m0 + row) * ntiles + nt] = v;
      if constexpr (CAND) {
        float th = -INFINITY;
        if (m0 + row < M) {
          atomicMax(cand.gmax + (size_t)(m0 + row) * 16 + (nt & 15), cand_ord(v));
          uint32_t lo = gq[0][0];
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) lo = min(lo, gq[q][e]);
          if (lo > kCandOrdNegInf) th = cand_val(lo);  // all 16 groups filled
        }
        cth[row] = th;
        cpos[row] = 0;
        if (m0 + row < M) {
          if (th == -INFINITY) cflag[0] = 1;  // some row stores densely
          else cflag[1] = 0;                  // not every row does
        }
      }
    }
  }
  if constexpr (CAND) {
    // Tile rows with theta: their values >= theta into LDS slots (a ballot
    // per value; slot positions from an LDS counter per row), then one
    // thread per row writes the row's slots out.  Rows without theta (dense)
    // are skipped here and stored below.
    __syncthreads();
    const bool all_dense = cflag[1] != 0;
    if (!all_dense) {
#pragma unroll
      for (int i = 0; i < kTm; ++i) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int rl0 = wm * (BM / WM) + i * 32 + 8 * r4 + 4 * (lane >> 5);
          const f32x4_t t4 = *reinterpret_cast<const f32x4_t*>(cth + rl0);
#pragma unroll
          for (int j = 0; j < kTn; ++j) {
            const int col = n0 + wn * (BN / WN) + j * 32 + (lane & 31);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float x = acc[i][j][r4 * 4 + e];
              // bitwise operators: short-circuit forms compile to branches
              const bool pass = (x >= t4[e]) & (t4[e] != -INFINITY) & (col < N) &
                                (m0 + rl0 + e < M);
              if (__ballot(pass)) {
                if (pass) {
                  const int q = atomicAdd(cpos + rl0 + e, 1);
                  if (q < kCandSlots)
                    cslot[(rl0 + e) * kCandSlots + q] = uint2{__float_as_uint(x), (uint32_t)col};
                }
              }
            }
          }
        }
      }
      __syncthreads();
      // counts; a row with more values >= theta than slots stores densely
      for (int row = tid; row < BM; row += kT) {
        const int np = cpos[row];
        const bool dense = cth[row] == -INFINITY || np > kCandSlots;
        if (m0 + row < M) {
          const size_t rt = (size_t)(m0 + row) * ntiles + nt;
          cand.cnt[rt] = dense ? kCandDense : np;
          if (!dense)
            for (int q = 0; q < np; ++q) cand.slots[rt * kCandSlots + q] = cslot[row * kCandSlots + q];
        }
        if (dense) {
          cth[row] = -INFINITY;
          if (m0 + row < M) cflag[0] = 1;
        }
      }
      __syncthreads();
      if (!cflag[0]) return;  // no dense row in this tile (uniform)
    } else {
      for (int row = tid; row < BM; row += kT)
        if (m0 + row < M) cand.cnt[(size_t)(m0 + row) * ntiles + nt] = kCandDense;
    }
    // dense rows: every logit, as without CAND
#pragma unroll
    for (int i = 0; i < kTm; ++i) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int rl0 = wm * (BM / WM) + i * 32 + 8 * r4 + 4 * (lane >> 5);
        const f32x4_t t4 = *reinterpret_cast<const f32x4_t*>(cth + rl0);
#pragma unroll
        for (int j = 0; j < kTn; ++j) {
          const int col = n0 + wn * (BN / WN) + j * 32 + (lane & 31);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int row = m0 + rl0 + e;
            if (t4[e] == -INFINITY && col < N && row < M)
              __builtin_nontemporal_store(acc[i][j][r4 * 4 + e], C + (size_t)row * N + col);
          }
        }
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < kTm; ++i) {
#pragma unroll
    for (int j = 0; j < kTn; ++j) {
      const int col = n0 + wn * (BN / WN) + j * 32 + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * (BM / WM) + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < M) __builtin_nontemporal_store(acc[i][j][r], C + (size_t)row * N + col);
      }
    }
  }
}

// fp32 operands: a workgroup owns 64 vocabulary rows x 8 output rows.  The
// W rows are staged through LDS in 64-wide K chunks with coalesced 16-byte
// loads (a row per thread would read 64 rows per load instruction); thread
// (n, q) then accumulates outputs (2q, 2q + 1) of vocabulary row n, one
// fmaf per k in k order, so every output is the same sequential fp32 sum
// as a plain loop.
constexpr int kF32N = 64;   // vocabulary rows per workgroup
constexpr int kF32M = 8;    // output rows per workgroup
constexpr int kF32K = 64;   // K chunk
__global__ __launch_bounds__(256) void lmhead_f32_kernel(const float* __restrict__ A,
                                                         const float* __restrict__ W,
                                                         float* __restrict__ C, int M, int N,
                                                         int K) {
  __shared__ float ws[kF32N][kF32K + 1];  // padded: lanes of a wave read 64 rows, 64 banks
  __shared__ float as[kF32M][kF32K];
  const int n0 = blockIdx.x * kF32N;
  const int m0 = blockIdx.y * kF32M;
  const int tid = threadIdx.x;
  const int nl = tid & 63;   // vocabulary row of this thread
  const int q = tid >> 6;    // output rows 2q, 2q + 1
  const int rows = min(kF32N, N - n0);
  float acc0 = 0.f, acc1 = 0.f;
  for (int kc = 0; kc < K; kc += kF32K) {
    const int kn = min(kF32K, K - kc);  // a multiple of 4 (K % 8 == 0)
    // 64 rows x kn floats: 16 threads per row, 16 bytes each, four passes
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int r = (tid >> 4) + 16 * pass;
      const int c = (tid & 15) * 4;
      if (r < rows && c < kn) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(W + (size_t)(n0 + r) * K + kc + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) ws[r][c + i] = v[i];
      }
    }
    for (int e = tid; e < kF32M * kF32K; e += 256) {
      const int mm = e / kF32K, c = e - mm * kF32K;
      if (m0 + mm < M && c < kn) as[mm][c] = A[(size_t)(m0 + mm) * K + kc + c];
    }
    __syncthreads();
    for (int k = 0; k < kn; ++k) {
      const float w = ws[nl][k];
      acc0 = fmaf(as[2 * q][k], w, acc0);
      acc1 = fmaf(as[2 * q + 1][k], w, acc1);
    }
    __syncthreads();
  }
  if (nl < rows) {
    if (m0 + 2 * q < M) C[(size_t)(m0 + 2 * q) * N + n0 + nl] = acc0;
    if (m0 + 2 * q + 1 < M) C[(size_t)(m0 + 2 * q + 1) * N + n0 + nl] = acc1;
  }
}

// Row maxima of every kTileMaxCols-column tile of finished logits (the
// fp32 path, whose GEMM does not produce them): one wave per (row, tile).
__global__ __launch_bounds__(256) void tilemax_kernel(const float* __restrict__ z, int M, int V,
                                                      int nt, float* __restrict__ tmax) {
  const long long w = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (long long)M * nt) return;
  const int lane = threadIdx.x & 63;
  const int m = (int)(w / nt);
  const int t = (int)(w - (long long)m * nt);
  float v = -INFINITY;
  for (int c = t * kTileMaxCols + lane; c < min(V, (t + 1) * kTileMaxCols); c += 64)
    v = fmaxf(v, z[(size_t)m * V + c]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  if (lane == 0) tmax[w] = v;
}

template <int BM, int BN, int BK, int WM, int WN, bool PACKED, bool CAND>
hipError_t launch_bf16_part(const uint16_t* h, const uint16_t* W, float* z, float* tmax, int M,
                            int H, int V, int nt0, int ntl, CandOut cand, hipStream_t s) {
  static_assert(BN == kTileMaxCols, "tile maxima follow the N tiles");
  const int mt = (M + BM - 1) / BM;
  const int nt = (V + BN - 1) / BN;
  if (H % BK == 0)
    hipLaunchKernelGGL((lmhead_bf16_kernel<BM, BN, BK, WM, WN, false, PACKED, CAND>),
                       dim3((unsigned)(mt * ntl)), dim3(WM * WN * 64), 0, s, h, W, z, tmax, M, V,
                       H, mt, nt, nt0, cand);
  else
    hipLaunchKernelGGL((lmhead_bf16_kernel<BM, BN, BK, WM, WN, true, PACKED, CAND>),
                       dim3((unsigned)(mt * ntl)), dim3(WM * WN * 64), 0, s, h, W, z, tmax, M, V,
                       H, mt, nt, nt0, cand);
  return hipGetLastError();
}

// All N tiles of the product.  One M tile of 256 rows (129 <= M <= 256) whose
// last round of N tiles fills at most half the CUs runs that round as
// 128-row tiles in a second launch: the same columns on twice the
// workgroups, each reading half of h (M = 256, K = 2560, V = 151936: 594
// tiles, 82 in the third round).
template <bool PACKED, bool CAND>
hipError_t launch_bf16(const uint16_t* h, const uint16_t* W, float* z, float* tmax, int M, int H,
                       int V, CandOut cand, hipStream_t s) {
  constexpr int kCus = 256;
  const int nt = (V + 255) / 256;
  const int tail = nt % kCus;
  if (M > 128 && M <= 256 && nt > kCus && tail <= kCus / 2) {
    hipError_t e = launch_bf16_part<256, 256, 64, 2, 4, PACKED, CAND>(h, W, z, tmax, M, H, V, 0,
                                                                      nt - tail, cand, s);
    if (e != hipSuccess || tail == 0) return e;
    return launch_bf16_part<128, 256, 64, 1, 8, PACKED, CAND>(h, W, z, tmax, M, H, V, nt - tail,
                                                              tail, cand, s);
  }
  return launch_bf16_part<256, 256, 64, 2, 4, PACKED, CAND>(h, W, z, tmax, M, H, V, 0, nt, cand, s);
}

// Group maxima back to "unfilled" before a candidate launch.
__global__ __launch_bounds__(256) void cand_reset_kernel(uint32_t* __restrict__ gmax,
                                                         long long n) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) gmax[i] = kCandOrdNegInf;
}

// The packed W layout: [ceil(V / 256)][ceil(H / 64)][256][64] bf16, rows past
// V and columns past H zero.  One thread per 16-byte run of the output.
constexpr int kPackRows = 256;
constexpr int kPackCols = 64;
__global__ __launch_bounds__(256) void lmhead_pack_kernel(const uint16_t* __restrict__ W,
                                                          uint16_t* __restrict__ Wp, int V, int H,
                                                          long long runs) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= runs) return;
  const int nkt = (H + kPackCols - 1) / kPackCols;
  const int c8 = (int)(i % (kPackCols / 8));            // run within the 64 columns
  const long long rb = i / (kPackCols / 8);              // (tile, slice, row)
  const int r = (int)(rb % kPackRows);
  const long long ts = rb / kPackRows;
  const int slice = (int)(ts % nkt);
  const long long tile = ts / nkt;
  const long long n = tile * kPackRows + r;
  const int k = slice * kPackCols + c8 * 8;
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (n < V && k < H) v = *reinterpret_cast<const u32x4_t*>(W + n * H + k);  // H % 8 == 0
  *reinterpret_cast<u32x4_t*>(Wp + i * 8) = v;
}

}  // namespace

hipError_t launch_lmhead(const void* h, const void* W, float* logits, float* tmax, int M, int H,
                         int V, int dtype, hipStream_t s) {
  if (M == 0) return hipSuccess;
  static_assert(kPackRows == 256 && kPackCols == 64, "the packed layout follows the bf16 tiles");
  if (dtype == 1 || dtype == 2) {  // 2: W packed by launch_lmhead_pack
    const uint16_t* hb = static_cast<const uint16_t*>(h);
    const uint16_t* Wb = static_cast<const uint16_t*>(W);
    if (dtype == 2)
      return launch_bf16<true, false>(hb, Wb, logits, tmax, M, H, V, {}, s);
    return launch_bf16<false, false>(hb, Wb, logits, tmax, M, H, V, {}, s);
  }
  const dim3 grid((unsigned)((V + kF32N - 1) / kF32N), (unsigned)((M + kF32M - 1) / kF32M));
  hipLaunchKernelGGL(lmhead_f32_kernel, grid, dim3(256), 0, s, static_cast<const float*>(h),
                     static_cast<const float*>(W), logits, M, V, H);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !tmax) return e;
  const int nt = (V + kTileMaxCols - 1) / kTileMaxCols;
  const long long waves = (long long)M * nt;
  hipLaunchKernelGGL(tilemax_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, logits, M,
                     V, nt, tmax);
  return hipGetLastError();
}

hipError_t launch_lmhead_cand(const void* h, const void* W, float* logits, float* tmax,
                              uint32_t* gmax, int* cnt, void* slots, int M, int H, int V,
                              int dtype, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const long long n = (long long)M * kTopK;
  hipLaunchKernelGGL(cand_reset_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, gmax,
                     n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const CandOut cand{gmax, cnt, static_cast<uint2*>(slots)};
  const uint16_t* hb = static_cast<const uint16_t*>(h);
  const uint16_t* Wb = static_cast<const uint16_t*>(W);
  if (dtype == 2)
    return launch_bf16<true, true>(hb, Wb, logits, tmax, M, H, V, cand, s);
  return launch_bf16<false, true>(hb, Wb, logits, tmax, M, H, V, cand, s);
}

size_t lmhead_pack_bytes(int V, int H) {
  return (size_t)((V + kPackRows - 1) / kPackRows) * ((H + kPackCols - 1) / kPackCols) *
         kPackRows * kPackCols * 2;
}

hipError_t launch_lmhead_pack(const void* W, void* Wp, int V, int H, hipStream_t s) {
  const long long runs = (long long)(lmhead_pack_bytes(V, H) / 16);
  if (runs == 0) return hipSuccess;
  hipLaunchKernelGGL(lmhead_pack_kernel, dim3((unsigned)((runs + 255) / 256)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(W), static_cast<uint16_t*>(Wp), V, H, runs);
  return hipGetLastError();
}

}  // namespace dflash2
