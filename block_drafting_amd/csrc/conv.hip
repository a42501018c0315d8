// Two-tap dynamic depthwise conv ("DFlash 2: Keep Drafting Parallel",
// section "A lightweight local convolution", eq. Conv_k and Fig. 4):
//   y_t = (k0 + D_t[g,0]) * x_t + (k1 + D_t[g,1]) * x_{t-1},  x_{-1} = anchor,
//   D_t[g,j] = x_t . proj[:, 2g+j].
// HBM-bound elementwise work: every thread moves 16-byte vectors (8 bf16 or
// 4+4 fp32 channels); the correction needs a row reduction first, or, with
// one correction per 16 channels, a matrix product (conv_mm_kernel).
//
// Arithmetic is fp64 (taps, corrections, products and the sum), then one
// rounding to the storage type: fp64 -> fp32 by round-to-odd, then fp32 ->
// bf16 by the hardware round-to-nearest-even.  Round-to-odd at 24 bits
// followed by rounding to 8 bits equals a single correct rounding, so each
// output is the exactly rounded value of the formula (up to the 2^-53
// relative error of the fp64 evaluation).  Chained convs therefore do not
// drift apart from the definition through double rounding.  The kernel is
// HBM-bound, so the fp64 rate is not the limit.
#include "common.hpp"

namespace dflash2 {
namespace {

// Eight consecutive channels of one row, widened to fp32.
template <typename T>
struct Row8;

// fp64 -> fp32 rounding to odd: truncate toward zero and make the last bit 1
// when anything was cut off.
__device__ __forceinline__ float f64_to_f32_odd(double v) {
  float f = (float)v;
  uint32_t u = __float_as_uint(f);
  const double back = (double)f;
  if (back != v) {
    if (fabs(back) > fabs(v)) u -= 1;  // stepped past v: move one ulp toward zero
    u |= 1u;
  }
  return __uint_as_float(u);
}

template <>
struct Row8<uint16_t> {
  __device__ static void load(const uint16_t* p, double v[8]) {
    u32x4_t w = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = (double)bf16_lo(w[i]);
      v[2 * i + 1] = (double)bf16_hi(w[i]);
    }
  }
  __device__ static void store(uint16_t* p, const double v[8]) {
    u32x4_t w;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = pack_bf16x2(f64_to_f32_odd(v[2 * i]), f64_to_f32_odd(v[2 * i + 1]));
    *reinterpret_cast<u32x4_t*>(p) = w;
  }
};

template <>
struct Row8<float> {
  __device__ static void load(const float* p, double v[8]) {
    f32x4_t a = reinterpret_cast<const f32x4_t*>(p)[0];
    f32x4_t b = reinterpret_cast<const f32x4_t*>(p)[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = (double)a[i];
      v[4 + i] = (double)b[i];
    }
  }
  __device__ static void store(float* p, const double v[8]) {
    f32x4_t a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = (float)v[i];
      b[i] = (float)v[4 + i];
    }
    reinterpret_cast<f32x4_t*>(p)[0] = a;
    reinterpret_cast<f32x4_t*>(p)[1] = b;
  }
};

__device__ __forceinline__ void load_f32x8(const float* p, double v[8]) {
  f32x4_t a = reinterpret_cast<const f32x4_t*>(p)[0];
  f32x4_t b = reinterpret_cast<const f32x4_t*>(p)[1];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = (double)a[i];
    v[4 + i] = (double)b[i];
  }
}

// y for 8 channels from fp64 taps c0, c1.
template <typename T>
__device__ __forceinline__ void mix8(const T* xp, const T* pp, T* yp, const double c0[8],
                                     const double c1[8]) {
  double xv[8], pv[8], yv[8];
  Row8<T>::load(xp, xv);
  if (pp) {
    Row8<T>::load(pp, pv);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) pv[i] = 0.0;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) yv[i] = c0[i] * xv[i] + c1[i] * pv[i];
  Row8<T>::store(yp, yv);
}

// Static taps: one thread per 8 channels of one (block, position) row.
template <typename T>
__global__ __launch_bounds__(256) void conv_static_kernel(const T* __restrict__ x,
                                                          const T* __restrict__ anchor,
                                                          T* __restrict__ y,
                                                          const float* __restrict__ k0,
                                                          const float* __restrict__ k1,
                                                          int L, int H, long long total8) {
  const int H8 = H >> 3;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < total8;
       i += (long long)gridDim.x * blockDim.x) {
    const long long row = i / H8;
    const int c = (int)(i - row * H8) * 8;
    const int t = (int)(row % L);
    const long long b = row / L;
    const T* xp = x + row * H + c;
    const T* pp = t > 0 ? xp - H : (anchor ? anchor + b * H + c : nullptr);
    double c0[8], c1[8];
    load_f32x8(k0 + c, c0);
    load_f32x8(k1 + c, c1);
    mix8<T>(xp, pp, y + row * H + c, c0, c1);
  }
}

__device__ __forceinline__ double block_sum_256(double v, double* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  double s = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return s;
}

// One correction pair per row (groups == 1): a 256-thread block per row
// reduces x_t . proj[:,0] and x_t . proj[:,1], then mixes.
template <typename T>
__global__ __launch_bounds__(256) void conv_dyn1_kernel(const T* __restrict__ x,
                                                        const T* __restrict__ anchor,
                                                        T* __restrict__ y,
                                                        const float* __restrict__ k0,
                                                        const float* __restrict__ k1,
                                                        const float* __restrict__ proj, int L,
                                                        int H) {
  __shared__ double red[4];
  const long long row = blockIdx.x;
  const int t = (int)(row % L);
  const long long b = row / L;
  const T* xr = x + row * H;
  double d0 = 0.0, d1 = 0.0;
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
    double xv[8], p[16];
    Row8<T>::load(xr + c, xv);
    load_f32x8(proj + 2 * c, p);
    load_f32x8(proj + 2 * c + 8, p + 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      d0 += xv[i] * p[2 * i];
      d1 += xv[i] * p[2 * i + 1];
    }
  }
  d0 = block_sum_256(d0, red);
  d1 = block_sum_256(d1, red);
  const T* pr = t > 0 ? xr - H : (anchor ? anchor + b * H : nullptr);
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
    double c0[8], c1[8];
    load_f32x8(k0 + c, c0);
    load_f32x8(k1 + c, c1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      c0[i] += d0;
      c1[i] += d1;
    }
    mix8<T>(xr + c, pr ? pr + c : nullptr, y + row * H + c, c0, c1);
  }
}

// General group count: the row is staged in LDS as fp64, all 2*groups
// corrections are computed (threads over outputs, coalesced proj reads), then
// each channel mixes with its group's pair.  Dynamic LDS: (H + 2*groups) doubles.
template <typename T>
__global__ __launch_bounds__(256) void conv_dyng_kernel(const T* __restrict__ x,
                                                        const T* __restrict__ anchor,
                                                        T* __restrict__ y,
                                                        const float* __restrict__ k0,
                                                        const float* __restrict__ k1,
                                                        const float* __restrict__ proj,
                                                        int groups, int L, int H) {
  extern __shared__ double ldsd[];
  double* xs = ldsd;
  double* dl = ldsd + H;
  const long long row = blockIdx.x;
  const int t = (int)(row % L);
  const long long b = row / L;
  const T* xr = x + row * H;
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
    double xv[8];
    Row8<T>::load(xr + c, xv);
#pragma unroll
    for (int i = 0; i < 8; ++i) xs[c + i] = xv[i];
  }
  __syncthreads();
  const int q2 = 2 * groups;
  for (int q = threadIdx.x; q < q2; q += 256) {
    double acc = 0.0;
    for (int c = 0; c < H; ++c) acc += xs[c] * (double)proj[(long long)c * q2 + q];
    dl[q] = acc;
  }
  __syncthreads();
  const int per = H / groups;
  const T* pr = t > 0 ? xr - H : (anchor ? anchor + b * H : nullptr);
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
    double c0[8], c1[8];
    load_f32x8(k0 + c, c0);
    load_f32x8(k1 + c, c1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int g = (c + i) / per;
      c0[i] += dl[2 * g];
      c1[i] += dl[2 * g + 1];
    }
    mix8<T>(xr + c, pr ? pr + c : nullptr, y + row * H + c, c0, c1);
  }
}

// ---------------------------------------------------------------- corrections on the matrix cores
// The post's coefficients carry one correction pair per 16 channels, so the
// correction of a whole batch is a real product D = X . P^T, [M x H] by
// [H x 2G] (2G = H/8 at G = H/16, 13.4 GFLOP per application at 2048 rows of
// 5120).  One workgroup owns a 64-row x 64-column tile of D (32 groups) and
// then applies the conv to exactly the channels of those groups for its
// rows, so D never leaves the chip.
//
// Product: bf16 x and P^T (both K-contiguous), v_mfma_f32_32x32x16_bf16,
// fp32 accumulation.  Four waves own the four 32 x 32 quarters of the tile;
// with few tiles a second group of four takes the second half of every K
// slice (partial quarters added at the end).  K is staged through LDS in
// 128-wide slices per group, every 16-byte load part of a run of threads
// reading contiguous bytes of one row, with two register staging sets
// keeping two slices in flight.  Mix: fp64 from the
// fp32 corrections, rounded once as in the kernels above.
constexpr int kMmBM = 64;
constexpr int kMmBN = 64;
constexpr int kMmDLd = kMmBN + 1;  // fp32 D tile pitch

// KH wave groups of four (2 x 2 quarters of the tile) split each K slice.
template <int KH>
struct MmCfg {
  static constexpr int kThreads = 256 * KH;
  static constexpr int kBK = 128 * KH;                   // K per LDS slice: 128 per group
  static constexpr int kLd = kBK + 8;                    // padded LDS row (bf16)
  static constexpr int kCpr = kBK / 8;                   // 16-byte chunks per row slice
  static constexpr int kRowsPerPass = kThreads / kCpr;   // 16
  static constexpr int kPasses = kMmBM / kRowsPerPass;   // 4 per operand
  static constexpr int kLoads = 2 * kPasses;
  static_assert(16 * 64 * 4 * 4 + kMmBM * kMmDLd * 4 <= 2 * 2 * kMmBM * kLd * 2,
                "partial tiles and the D tile fit in the stages");
};
static_assert(kMmBM == kMmBN, "one loader layout serves both operands");

template <int KH>
__global__ __launch_bounds__(MmCfg<KH>::kThreads) void conv_mm_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ anchor,
    uint16_t* __restrict__ y, const float* __restrict__ k0, const float* __restrict__ k1,
    const uint16_t* __restrict__ pt, int M, int N, int H, int L, int gw, int mtiles,
    int ntiles) {
  using C = MmCfg<KH>;
  constexpr int kMmThreads = C::kThreads;
  constexpr int kMmKH = KH;
  constexpr int kMmBK = C::kBK;
  constexpr int kMmLd = C::kLd;
  constexpr int kMmCpr = C::kCpr;
  constexpr int kMmRowsPerPass = C::kRowsPerPass;
  constexpr int kMmPasses = C::kPasses;
  constexpr int kMmLoads = C::kLoads;
  __shared__ __attribute__((aligned(16))) uint16_t stage[2][2][kMmBM * kMmLd];  // [buf][x/P]
  // Tiles that share x rows run on one XCD: n fastest.
  const int tile = xcd_tile(blockIdx.x, mtiles * ntiles);
  const int mt = tile / ntiles;
  const int nt = tile - mt * ntiles;
  const int m0 = mt * kMmBM;
  const int n0 = nt * kMmBN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rowsA = min(kMmBM, M - m0);
  const int rowsB = min(kMmBN, N - n0);
  // Loader role: rows (tid / kMmCpr) + 16 p of each operand, chunk tid % kMmCpr.
  // Rows past the edge repeat the last row (their results are never used).
  const int lrow = tid / kMmCpr;
  const int lk = (tid % kMmCpr) * 8;
  const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x + (size_t)m0 * H), (short)0, rowsA * H * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(pt + (size_t)n0 * H), (short)0, rowsB * H * 2, 0x00020000);
  int offA[kMmPasses], offB[kMmPasses];
#pragma unroll
  for (int p = 0; p < kMmPasses; ++p) {
    offA[p] = (min(lrow + p * kMmRowsPerPass, rowsA - 1) * H + lk) * 2;
    offB[p] = (min(lrow + p * kMmRowsPerPass, rowsB - 1) * H + lk) * 2;
  }
  const int nslices = (H + kMmBK - 1) / kMmBK;
  // Slices past the end re-read the last slice (in range, never used).
  u32x4_t R0[kMmLoads], R1[kMmLoads];
  auto gload = [&](u32x4_t(&R)[kMmLoads], int sl) {
    const int k = min(sl, nslices - 1) * kMmBK;
    const bool in = k + lk < H;  // H % 8 == 0: a chunk is wholly inside or outside
    const u32x4_t z = {0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p < kMmPasses; ++p) {
      const u32x4_t va = __builtin_amdgcn_raw_buffer_load_b128(rsA, offA[p] + k * 2, 0, 0);
      const u32x4_t vb = __builtin_amdgcn_raw_buffer_load_b128(rsB, offB[p] + k * 2, 0, 0);
      R[p] = in ? va : z;
      R[kMmPasses + p] = in ? vb : z;
    }
  };
  auto sstore = [&](const u32x4_t(&R)[kMmLoads], int buf) {
#pragma unroll
    for (int p = 0; p < kMmPasses; ++p) {
      const int at = (lrow + p * kMmRowsPerPass) * kMmLd + lk;
      *reinterpret_cast<u32x4_t*>(&stage[buf][0][at]) = R[p];
      *reinterpret_cast<u32x4_t*>(&stage[buf][1][at]) = R[kMmPasses + p];
    }
  };
  f32x16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  // Wave (kh, wm, wn): K half kh of every slice, rows 32 wm.. and columns
  // 32 wn.. of the tile; lane l supplies fragment row l % 32 and k values
  // 8 (l / 32) .. +7 of a k-step.
  const int kh = KH > 1 ? wave >> 2 : 0;
  const int wm = wave & 1;
  const int wn = (wave >> 1) & 1;
  const int fa = (wm * 32 + (lane & 31)) * kMmLd + (lane >> 5) * 8 + kh * (kMmBK / kMmKH);
  const int fb = (wn * 32 + (lane & 31)) * kMmLd + (lane >> 5) * 8 + kh * (kMmBK / kMmKH);
  auto multiply = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < kMmBK / kMmKH / 16; ++ks) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&stage[buf][0][fa + ks * 16]);
      const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(&stage[buf][1][fb + ks * 16]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
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
  // The second K half's partial quarters meet the first's in LDS (over the
  // stages, which are free now), then the D tile goes to LDS: accumulator
  // register r of lane l holds C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
  float* part = reinterpret_cast<float*>(&stage[0][0][0]);  // [4 quarters][16][64]
  float* dt = part + 4 * 16 * 64;
  const int quarter = wave & 3;
  if (KH > 1) {
    if (kh == 1) {
#pragma unroll
      for (int r = 0; r < 16; ++r) part[(quarter * 16 + r) * 64 + lane] = acc[r];
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] += part[(quarter * 16 + r) * 64 + lane];
    }
  }
  if (kh == 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      dt[row * kMmDLd + wn * 32 + (lane & 31)] = acc[r];
    }
  }
  __syncthreads();
  // Mix the channels of this tile's groups for its rows.
  const int g0 = n0 >> 1;
  const int c0 = g0 * gw;
  const int c1 = min(N >> 1, g0 + kMmBN / 2) * gw;
  const int nvec = (c1 - c0) >> 3;
  // kMixU vectors of 8 channels per thread per round, all their loads in
  // flight before any arithmetic (a round trip per vector would dominate).
  const bool whole = (gw & 7) == 0;  // a vector never straddles two groups
  const int nv = rowsA * nvec;
  constexpr int kMixU = 4;
  for (int e0 = tid; e0 < nv; e0 += kMmThreads * kMixU) {
    u32x4_t xr[kMixU], pr[kMixU];
    f32x4_t ka[kMixU][2], kb[kMixU][2];
    int rw[kMixU], cc[kMixU];
#pragma unroll
    for (int u = 0; u < kMixU; ++u) {
      const int e = min(e0 + kMmThreads * u, nv - 1);  // tail rounds redo the last vector (not stored)
      const int row = e / nvec;
      const int c = c0 + (e - row * nvec) * 8;
      const int m = m0 + row;
      const int b = m / L;
      const int t = m - b * L;
      rw[u] = row;
      cc[u] = c;
      const uint16_t* xp = x + (size_t)m * H + c;
      xr[u] = *reinterpret_cast<const u32x4_t*>(xp);
      if (t > 0)
        pr[u] = *reinterpret_cast<const u32x4_t*>(xp - H);
      else if (anchor)
        pr[u] = *reinterpret_cast<const u32x4_t*>(anchor + (size_t)b * H + c);
      else
        pr[u] = u32x4_t{0u, 0u, 0u, 0u};
      ka[u][0] = *reinterpret_cast<const f32x4_t*>(k0 + c);
      ka[u][1] = *reinterpret_cast<const f32x4_t*>(k0 + c + 4);
      kb[u][0] = *reinterpret_cast<const f32x4_t*>(k1 + c);
      kb[u][1] = *reinterpret_cast<const f32x4_t*>(k1 + c + 4);
    }
#pragma unroll
    for (int u = 0; u < kMixU; ++u) {
      if (e0 + kMmThreads * u >= nv) break;
      const int c = cc[u];
      const float* drow = dt + rw[u] * kMmDLd;
      double d0[8], d1[8];
      if (whole) {
        const int col = 2 * (c / gw - g0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          d0[i] = (double)drow[col];
          d1[i] = (double)drow[col + 1];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int col = 2 * ((c + i) / gw - g0);
          d0[i] = (double)drow[col];
          d1[i] = (double)drow[col + 1];
        }
      }
      u32x4_t out;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        double yv[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int i = 2 * w + h;
          const double xv = (double)(h ? bf16_hi(xr[u][w]) : bf16_lo(xr[u][w]));
          const double pv = (double)(h ? bf16_hi(pr[u][w]) : bf16_lo(pr[u][w]));
          const double a0 = (double)ka[u][i >> 2][i & 3] + d0[i];
          const double a1 = (double)kb[u][i >> 2][i & 3] + d1[i];
          yv[h] = a0 * xv + a1 * pv;
        }
        out[w] = pack_bf16x2(f64_to_f32_odd(yv[0]), f64_to_f32_odd(yv[1]));
      }
      *reinterpret_cast<u32x4_t*>(y + (size_t)(m0 + rw[u]) * H + c) = out;
    }
  }
}

template <typename T>
hipError_t launch_typed(const void* x, const void* anchor_h, void* y, const float* k0,
                        const float* k1, const float* proj, int groups, int B, int L, int H,
                        hipStream_t s) {
  const T* xp = static_cast<const T*>(x);
  const T* ap = static_cast<const T*>(anchor_h);
  T* yp = static_cast<T*>(y);
  const long long rows = (long long)B * L;
  if (!proj) {
    const long long total8 = rows * (H / 8);
    long long blocks = (total8 + 255) / 256;
    if (blocks > (1 << 20)) blocks = 1 << 20;
    hipLaunchKernelGGL(conv_static_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, s, xp, ap,
                       yp, k0, k1, L, H, total8);
  } else if (groups == 1) {
    hipLaunchKernelGGL(conv_dyn1_kernel<T>, dim3((unsigned)rows), dim3(256), 0, s, xp, ap, yp,
                       k0, k1, proj, L, H);
  } else {
    const size_t lds = (size_t)(H + 2 * groups) * sizeof(double);
    hipLaunchKernelGGL(conv_dyng_kernel<T>, dim3((unsigned)rows), dim3(256), lds, s, xp, ap,
                       yp, k0, k1, proj, groups, L, H);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_twotap_conv_mm(const void* x, const void* anchor_h, void* y, const float* k0,
                                 const float* k1, const void* projT, int groups, int B, int L,
                                 int H, hipStream_t s) {
  const int M = B * L;
  const int N = 2 * groups;
  const int mtiles = (M + kMmBM - 1) / kMmBM;
  const int ntiles = (N + kMmBN - 1) / kMmBN;
  const unsigned tiles = (unsigned)(mtiles * ntiles);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* ab = static_cast<const uint16_t*>(anchor_h);
  uint16_t* yb = static_cast<uint16_t*>(y);
  const uint16_t* pb = static_cast<const uint16_t*>(projT);
  // One round of tiles over the CUs: two wave groups per tile (a tile's K
  // loop is latency-bound, the second group halves it; 135 KB of LDS, one
  // tile per CU).  More tiles than CUs: one group, two tiles per CU.
  if (tiles <= 256)
    hipLaunchKernelGGL(conv_mm_kernel<2>, dim3(tiles), dim3(MmCfg<2>::kThreads), 0, s, xb, ab, yb,
                       k0, k1, pb, M, N, H, L, H / groups, mtiles, ntiles);
  else
    hipLaunchKernelGGL(conv_mm_kernel<1>, dim3(tiles), dim3(MmCfg<1>::kThreads), 0, s, xb, ab, yb,
                       k0, k1, pb, M, N, H, L, H / groups, mtiles, ntiles);
  return hipGetLastError();
}

hipError_t launch_twotap_conv(const void* x, const void* anchor_h, void* y, const float* k0,
                              const float* k1, const float* proj, int groups, int B, int L,
                              int H, int dtype, hipStream_t s) {
  if (dtype == 1)
    return launch_typed<uint16_t>(x, anchor_h, y, k0, k1, proj, groups, B, L, H, s);
  return launch_typed<float>(x, anchor_h, y, k0, k1, proj, groups, B, L, H, s);
}

}  // namespace dflash2
