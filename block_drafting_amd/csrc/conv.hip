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
// drift apart from the definition through double rounding.  The
// ten-channel kernel takes the nearest fp32 value instead and falls back to
// round-to-odd only where that value is a bf16 midpoint (same result).
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

// ---------------------------------------------------------------- rows of a block per workgroup
// Raw storage of 8 consecutive channels (one 16-byte bf16 vector or two
// fp32 vectors), widened to fp64 on use.
template <typename T>
struct Raw8;
template <>
struct Raw8<uint16_t> {
  u32x4_t w;
  __device__ void load(const uint16_t* p) { w = *reinterpret_cast<const u32x4_t*>(p); }
  __device__ void zero() { w = u32x4_t{0u, 0u, 0u, 0u}; }
  __device__ void widen(double v[8]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = (double)bf16_lo(w[i]);
      v[2 * i + 1] = (double)bf16_hi(w[i]);
    }
  }
  // channel i (a compile-time index once unrolled)
  __device__ double at(int i) const {
    return (double)((i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]));
  }
};
template <>
struct Raw8<float> {
  f32x4_t a, b;
  __device__ void load(const float* p) {
    a = reinterpret_cast<const f32x4_t*>(p)[0];
    b = reinterpret_cast<const f32x4_t*>(p)[1];
  }
  __device__ void zero() {
    a = f32x4_t{0.f, 0.f, 0.f, 0.f};
    b = a;
  }
  __device__ void widen(double v[8]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = (double)a[i];
      v[4 + i] = (double)b[i];
    }
  }
  __device__ double at(int i) const { return (double)(i < 4 ? a[i] : b[i - 4]); }
};

// Eight output channels, each rounded once from fp64 as it is produced:
// bf16 by round-to-odd to fp32 then the hardware's nearest-even (one
// correct rounding), fp32 by nearest-even.
template <typename T>
struct Out8;
template <>
struct Out8<uint16_t> {
  float f[8];
  __device__ void set(int i, double v) { f[i] = f64_to_f32_odd(v); }
  __device__ void store(uint16_t* p) const {
    u32x4_t w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    *reinterpret_cast<u32x4_t*>(p) = w;
  }
};
template <>
struct Out8<float> {
  float f[8];
  __device__ void set(int i, double v) { f[i] = (float)v; }
  __device__ void store(float* p) const {
    reinterpret_cast<f32x4_t*>(p)[0] = f32x4_t{f[0], f[1], f[2], f[3]};
    reinterpret_cast<f32x4_t*>(p)[1] = f32x4_t{f[4], f[5], f[6], f[7]};
  }
};

// Value of lane (lane ^ D) for fp64 data (two 32-bit exchanges).
template <int D>
__device__ __forceinline__ double xor_f64(double v) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const uint32_t lo = xor_lane<D>((uint32_t)u);
  const uint32_t hi = xor_lane<D>((uint32_t)(u >> 32));
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// One reduce-scatter step over partner lane ^ D on the first N values: the
// lane with bit D set keeps the upper half, the other the lower half, each
// adding its partner's copy; the lane's value index advances accordingly.
template <int D, int N>
__device__ __forceinline__ void rs_step(double* v, int lane, int& idx) {
  const bool up = (lane & D) != 0;
#pragma unroll
  for (int k = 0; k < N / 2; ++k) {
    const double send = up ? v[k] : v[k + N / 2];
    const double keep = up ? v[k + N / 2] : v[k];
    v[k] = keep + xor_f64<D>(send);
  }
  if (up) idx += N / 2;
}

// Sums of N values (N a power of two, 2..32) over the 64 lanes of a wave:
// a reduce-scatter over partners 32, 16, ... (log2 N steps) leaves each lane
// one value, then full exchanges over the remaining partners finish it.
// Returns the total of value `idx`; the lanes whose low 6 - log2 N bits are
// zero hold each value once.
template <int N>
__device__ __forceinline__ double wave_reduce_scatter(double* v, int lane, int& idx) {
  static_assert(N >= 2 && N <= 32 && (N & (N - 1)) == 0, "2..32 values");
  idx = 0;
  rs_step<32, N>(v, lane, idx);
  if constexpr (N >= 4) rs_step<16, N / 2>(v, lane, idx); else v[0] += xor_f64<16>(v[0]);
  if constexpr (N >= 8) rs_step<8, N / 4>(v, lane, idx); else v[0] += xor_f64<8>(v[0]);
  if constexpr (N >= 16) rs_step<4, N / 8>(v, lane, idx); else v[0] += xor_f64<4>(v[0]);
  if constexpr (N >= 32) rs_step<2, N / 16>(v, lane, idx); else v[0] += xor_f64<2>(v[0]);
  v[0] += xor_f64<1>(v[0]);
  return v[0];
}

// NG groups of R consecutive positions of one block per workgroup (rows
// t0 .. t0 + NG*R - 1), every channel.  Thread i holds channel chunks i,
// i + blockDim, ... (CPT of them, 8 channels each) of a group's R rows in
// registers, so the taps (and the projection) are read once per workgroup,
// each row's predecessor is the previous row's registers (only t0's is
// read: x[b, t0 - 1], or the anchor at t0 = 0), and every load is issued
// before the first use.  The groups are software-pipelined: group g+1's
// rows are loading while group g reduces, mixes and stores.  DYN (one
// correction pair per row): each group's 2R dot products are summed in
// fp64, per wave by a reduce-scatter, then across the waves in LDS in wave
// order, so the result does not depend on timing.  The mix is the fp64
// formula with one rounding per output, as in the kernels above.
template <typename T, int R, int NG, int CPT, bool DYN>
__global__ __launch_bounds__(1024 / CPT) void conv_rows_kernel(const T* __restrict__ x,
                                                         const T* __restrict__ anchor,
                                                         T* __restrict__ y,
                                                         const float* __restrict__ k0,
                                                         const float* __restrict__ k1,
                                                         const float* __restrict__ proj, int L,
                                                         int H, int wgs_per_block) {
  constexpr int N = 2 * R;  // correction dot products of a group
  __shared__ double red[16 * N];
  __shared__ double tot[N];
  const int b = blockIdx.x / wgs_per_block;
  const int t0 = (blockIdx.x - b * wgs_per_block) * (R * NG);
  const int H8 = H >> 3;
  const int tid = threadIdx.x;
  const int nth = blockDim.x;
  Raw8<T> xr[2][CPT][R], pr[CPT];
  f32x4_t kv[CPT][4];       // k0 (2 vectors) then k1 (2 vectors) of the chunk
  f32x4_t pj[CPT][DYN ? 4 : 1];
  auto load_group = [&](Raw8<T>(&dst)[CPT][R], int g) {
    const int tg = t0 + g * R;
    const int nr = min(R, L - tg);
    const size_t base = ((size_t)b * L + tg) * H;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c8 = tid + j * nth;
      if (c8 < H8) {
#pragma unroll
        for (int r = 0; r < R; ++r)
          if (r < nr) dst[j][r].load(x + base + (size_t)r * H + c8 * 8);
      }
    }
  };
  load_group(xr[0], 0);
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int c8 = tid + j * nth;
    if (c8 < H8) {
      const int c = c8 * 8;
      if (t0 > 0)
        pr[j].load(x + ((size_t)b * L + t0 - 1) * H + c);
      else if (anchor)
        pr[j].load(anchor + (size_t)b * H + c);
      else
        pr[j].zero();
      if constexpr (DYN) {
#pragma unroll
        for (int q = 0; q < 4; ++q) pj[j][q] = reinterpret_cast<const f32x4_t*>(proj + 2 * c)[q];
      }
      kv[j][0] = reinterpret_cast<const f32x4_t*>(k0 + c)[0];
      kv[j][1] = reinterpret_cast<const f32x4_t*>(k0 + c)[1];
      kv[j][2] = reinterpret_cast<const f32x4_t*>(k1 + c)[0];
      kv[j][3] = reinterpret_cast<const f32x4_t*>(k1 + c)[1];
    }
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int tg = t0 + g * R;
    const int nr = min(R, L - tg);
    if (nr <= 0) break;  // uniform over the workgroup
    Raw8<T>(&cur)[CPT][R] = xr[g & 1];
    if (g > 0) {
      // the predecessor of this group's first row, before the next group's
      // loads reuse the buffer that holds it
#pragma unroll
      for (int j = 0; j < CPT; ++j) pr[j] = xr[(g - 1) & 1][j][R - 1];
    }
    if (g + 1 < NG && tg + R < L) load_group(xr[(g + 1) & 1], g + 1);
    double d[N];
#pragma unroll
    for (int i = 0; i < N; ++i) d[i] = 0.0;
    if constexpr (DYN) {
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        if (tid + j * nth < H8) {
          // channel by channel: the channel's two projection entries, then
          // its value in every row (few fp64 values live at once)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const double p0 = (double)pj[j][i / 2][2 * (i % 2)];
            const double p1 = (double)pj[j][i / 2][2 * (i % 2) + 1];
#pragma unroll
            for (int r = 0; r < R; ++r) {
              if (r < nr) {
                const double xv = cur[j][r].at(i);
                d[2 * r] += xv * p0;
                d[2 * r + 1] += xv * p1;
              }
            }
          }
        }
      }
      const int lane = tid & 63;
      const int wave = tid >> 6;
      int idx;
      const double part = wave_reduce_scatter<N>(d, lane, idx);
      if ((lane & (64 / N - 1)) == 0) red[wave * N + idx] = part;
      __syncthreads();
      if (tid < N) {
        double sacc = red[tid];
        for (int w = 1; w < (nth >> 6); ++w) sacc += red[w * N + tid];
        tot[tid] = sacc;
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < N; ++i) d[i] = tot[i];
    }
    const size_t base = ((size_t)b * L + tg) * H;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c8 = tid + j * nth;
      if (c8 < H8) {
        const int c = c8 * 8;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (r < nr) {
            const Raw8<T>& prev = r == 0 ? pr[j] : cur[j][r - 1];
            Out8<T> o;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const double c0 = (double)kv[j][i / 4][i % 4] + d[2 * r];
              const double c1 = (double)kv[j][2 + i / 4][i % 4] + d[2 * r + 1];
              o.set(i, c0 * cur[j][r].at(i) + c1 * prev.at(i));
            }
            o.store(y + base + (size_t)r * H + c);
          }
        }
      }
    }
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

// ---------------------------------------------------------------- bf16 rows, ten channels per thread
// The bf16 path for H a multiple of 640 up to 5120 (H = 5120: 512 threads,
// eight waves, two per SIMD).  Thread t owns channels [10t, 10t + 10) of
// every row of its workgroup: NG groups of R consecutive positions of one
// block.  Group g + PD's rows load while group g is mixed.
//
// Every access is a buffer access.  A group's descriptor ends at its last
// row inside the block, so rows past L read zeros and store nothing, and
// the loop body has no branches: the compiler then counts outstanding
// loads exactly and only waits for the group it is about to use.  With a
// projection the 2R partial dot products of a group are reduced over the
// wave (reduce-scatter), then over the waves in LDS in wave order (so the
// sum does not depend on timing) behind one barrier per group; the next
// group's loads stay in flight across it.
//
// Rounding (one correct rounding to bf16 of the fp64 value v): (float)v is
// the nearest fp32 value to v.  Every bf16 midpoint is an fp32 value, so
// v and (float)v lie on the same side of every midpoint unless (float)v
// is a midpoint itself (low 16 bits 0x8000); the nearest-even bf16 of
// (float)v is then v's.  When any lane of the wave meets a midpoint, the
// row takes the round-to-odd conversion above.
constexpr int kC10 = 10;         // channels per thread
constexpr int kC10Threads = 512;  // largest workgroup (H = 5120)
constexpr int kRsrcFlags = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           kRsrcFlags);
}

// Ten bf16 channels: a 16-byte and a 4-byte load (dword aligned).
struct Raw10 {
  uint32_t w[5];
  __device__ double at(int i) const {
    return (double)((i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]));
  }
  __device__ void load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = a[i];
    w[4] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 16, 0, 0);
  }
};

// NF fp32 values (NF = 4q or 4q + 2) from byte offset off.
template <int NF>
__device__ __forceinline__ void load_floats(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                            float (&f)[NF]) {
  typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int q = 0; q + 4 <= NF; q += 4) {
    const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(r, off + q * 4, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) f[q + i] = __uint_as_float(a[i]);
  }
  if constexpr (NF % 4 == 2) {
    const u32x2_t a = __builtin_bit_cast(
        u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off + (NF - 2) * 4, 0, 0));
    f[NF - 2] = __uint_as_float(a[0]);
    f[NF - 1] = __uint_as_float(a[1]);
  }
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// Two fp32 values to a bf16 pair, nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ bool on_bf16_midpoint(float f) {
  return (__float_as_uint(f) & 0xffffu) == 0x8000u;
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, l);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), l);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Corrections of conv_rows10_kernel: none (static taps), one pair per row
// from an [H, 2] projection, or one pair per group of gw >= 16 channels
// whose split-K partial sums conv_mm_partial_kernel left in the rows of y.
enum Conv10Mode { kStaticTaps = 0, kOnePair = 1, kSplitParts = 2 };
constexpr int kSplitK = 4;  // K splits of the per-group corrections

template <int R, int NG, int PD, int MODE>
__global__ __launch_bounds__(kC10Threads) void conv_rows10_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ anchor,
    uint16_t* __restrict__ y, const float* __restrict__ k0, const float* __restrict__ k1,
    const float* __restrict__ proj, int L, int H, int wgs_per_block, int ncols, int gw) {
  constexpr bool DYN = MODE == kOnePair;
  constexpr bool PARTS = MODE == kSplitParts;
  constexpr int C = kC10;
  constexpr int N = 2 * R;       // correction dot products of a group
  constexpr int NB = PD + 1;     // row buffers: the group in use and PD in flight
  constexpr int NWMAX = kC10Threads / 64;
  __shared__ double red[2][DYN ? NWMAX * N : 1];
  const int nw = (int)(blockDim.x >> 6);
  const int b = blockIdx.x / wgs_per_block;
  const int t0 = (blockIdx.x - b * wgs_per_block) * (R * NG);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const uint32_t row_bytes = (uint32_t)H * 2;
  const uint32_t cb = (uint32_t)tid * (2 * C);  // byte offset of the thread's channels in a row
  auto group_rsrc = [&](const uint16_t* base, int g) {
    const int tg = t0 + g * R;
    const int nr = max(0, min(R, L - tg));
    return byte_rsrc(base + ((size_t)b * L + tg) * H,
                     __builtin_amdgcn_readfirstlane((uint32_t)nr * row_bytes));
  };
  Raw10 xr[NB][R];
  // Split-K partials: row r of y holds float [kSplitK][ncols]; the thread's
  // channels belong to groups ga and ga + 1 at most (gw >= 16), whose four
  // columns 2 ga .. 2 ga + 3 one 16-byte load per split brings.  The last
  // group loads columns ncols - 4 .. ncols - 1 instead (psh = 2), so no load
  // runs past the row's partials; it has no second group.
  u32x4_t pa[PARTS ? NB : 1][PARTS ? R : 1][kSplitK];
  const int ga = PARTS ? (C * tid) / gw : 0;
  const int pbase = PARTS && ncols >= 4 ? min(2 * ga, ncols - 4) : 2 * ga;
  const bool psh = 2 * ga != pbase;
  auto load_group = [&](int g) {
    const __amdgpu_buffer_rsrc_t rx = group_rsrc(x, g);
#pragma unroll
    for (int r = 0; r < R; ++r) xr[g % NB][r].load(rx, cb + r * row_bytes);
    if constexpr (PARTS) {
      const __amdgpu_buffer_rsrc_t rp = group_rsrc(y, g);
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int k = 0; k < kSplitK; ++k)
          pa[g % NB][r][k] = __builtin_amdgcn_raw_buffer_load_b128(
              rp, r * row_bytes + (uint32_t)(k * ncols + pbase) * 4, 0, 0);
    }
  };
#pragma unroll
  for (int g = 0; g < PD && g < NG; ++g) load_group(g);
  float ka[C], kb[C], pj[DYN ? 2 * C : 2];
  double pv[C];  // the predecessor of the group's first row
  {
    const uint16_t* pp = t0 > 0 ? x + ((size_t)b * L + t0 - 1) * H
                                : (anchor ? anchor + (size_t)b * H : x);
    const uint32_t pbytes =
        __builtin_amdgcn_readfirstlane((t0 > 0 || anchor) ? row_bytes : 0u);  // 0: zeros
    Raw10 pr;
    pr.load(byte_rsrc(pp, pbytes), cb);
    if constexpr (DYN)
      load_floats<2 * C>(byte_rsrc(proj, (uint32_t)H * 8), (uint32_t)tid * (8 * C), pj);
    load_floats<C>(byte_rsrc(k0, (uint32_t)H * 4), (uint32_t)tid * (4 * C), ka);
    load_floats<C>(byte_rsrc(k1, (uint32_t)H * 4), (uint32_t)tid * (4 * C), kb);
#pragma unroll
    for (int i = 0; i < C; ++i) pv[i] = pr.at(i);
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if (t0 + g * R >= L) break;  // uniform over the workgroup
    if (g + PD < NG) load_group(g + PD);
    double xv[R][C];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < C; ++i) xv[r][i] = xr[g % NB][r].at(i);
    double d[N];
#pragma unroll
    for (int i = 0; i < N; ++i) d[i] = 0.0;
    if constexpr (DYN) {
      // channel by channel, every row of the group
#pragma unroll
      for (int i = 0; i < C; ++i) {
        const double p0 = (double)pj[2 * i];
        const double p1 = (double)pj[2 * i + 1];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          d[2 * r] += xv[r][i] * p0;
          d[2 * r + 1] += xv[r][i] * p1;
        }
      }
      int idx;
      const double part = wave_reduce_scatter<N>(d, lane, idx);
      if ((lane & (64 / N - 1)) == 0) red[g & 1][wave * N + idx] = part;
      // one barrier per group: red[g & 1] is next written two groups on,
      // after every wave has passed the barrier of the group in between
      __syncthreads();
      double tot = 0.0;
      if (lane < N) {
        tot = red[g & 1][lane];
        for (int w = 1; w < nw; ++w) tot += red[g & 1][w * N + lane];
      }
#pragma unroll
      for (int i = 0; i < N; ++i) d[i] = readlane_f64(tot, i);
    }
    // per-group corrections of the group's rows: the K splits in order
    double dp[PARTS ? R : 1][2][2];
    if constexpr (PARTS) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float sum[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sum[e] = __uint_as_float(pa[g % NB][r][0][e]);
#pragma unroll
          for (int k = 1; k < kSplitK; ++k) sum[e] += __uint_as_float(pa[g % NB][r][k][e]);
        }
        // The sums, and so the loads they read, must be done before the
        // barrier below: the barrier waits for LDS operations only, and left
        // to itself the compiler finishes some rows' sums after it, with
        // their loads still in flight when other waves store into these rows.
        asm volatile("" ::"v"(sum[0]), "v"(sum[1]), "v"(sum[2]), "v"(sum[3]));
        dp[r][0][0] = (double)(psh ? sum[2] : sum[0]);
        dp[r][0][1] = (double)(psh ? sum[3] : sum[1]);
        dp[r][1][0] = (double)sum[2];  // group ga + 1 (unused with psh)
        dp[r][1][1] = (double)sum[3];
      }
      // every thread has read these rows' partials before any writes them
      __syncthreads();
    }
    const int na = PARTS ? min(C, (ga + 1) * gw - C * tid) : C;  // channels in group ga
    const __amdgpu_buffer_rsrc_t ry = group_rsrc(y, g);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const double* prev = r == 0 ? pv : xv[r - 1];
      float f[C];
      uint64_t mid = 0;
      auto tap = [&](int i, double& c0, double& c1) {
        if constexpr (DYN) {
          c0 = (double)ka[i] + d[2 * r];
          c1 = (double)kb[i] + d[2 * r + 1];
        } else if constexpr (PARTS) {
          const int q = i < na ? 0 : 1;
          c0 = (double)ka[i] + dp[PARTS ? r : 0][q][0];
          c1 = (double)kb[i] + dp[PARTS ? r : 0][q][1];
        } else {
          c0 = (double)ka[i];
          c1 = (double)kb[i];
        }
      };
#pragma unroll
      for (int i = 0; i < C; ++i) {
        double c0, c1;
        tap(i, c0, c1);
        f[i] = (float)(c0 * xv[r][i] + c1 * prev[i]);
        mid |= __builtin_amdgcn_ballot_w64(on_bf16_midpoint(f[i]));
      }
      if (mid) {
#pragma unroll
        for (int i = 0; i < C; ++i) {
          double c0, c1;
          tap(i, c0, c1);
          f[i] = f64_to_f32_odd(c0 * xv[r][i] + c1 * prev[i]);
        }
      }
      const uint32_t off = cb + r * row_bytes;
      __builtin_amdgcn_raw_buffer_store_b128(
          u32x4_t{pk_bf16(f[0], f[1]), pk_bf16(f[2], f[3]), pk_bf16(f[4], f[5]),
                  pk_bf16(f[6], f[7])},
          ry, off, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(pk_bf16(f[8], f[9]), ry, off + 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C; ++i) pv[i] = xv[R - 1][i];
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

// ---------------------------------------------------------------- split-K per-group corrections
// For gw >= 16 channels per group the corrections of a batch can also be
// computed as kSplitK partial products over quarters of K, each workgroup a
// 128 x 160 tile of D over one quarter (0.72 MB of operands per workgroup
// against 1.28 MB for a whole-K 64 x 64 tile), and the fp32 partials parked
// in the rows of y: row m holds float [kSplitK][2G], which fits its 2H bytes
// exactly when G = H / 16.  conv_rows10_kernel<..., kSplitParts> then sums
// the quarters in order, mixes and overwrites each row.
//
// Eight waves: four bands of 32 rows x two halves of 80 columns, each a
// 2 x 5 grid of 16 x 16 blocks on v_mfma_f32_16x16x32_bf16 (lane l: row or
// column l % 16, k values 8 (l / 16) .. +7 of a 32-step; accumulator r:
// row 4 (l / 16) + r, column l % 16).  K is staged through LDS in 128-wide
// slices with two register staging sets, as in conv_mm_kernel.
constexpr int kSkBM = 128;
constexpr int kSkBN = 160;
constexpr int kSkBK = 128;
constexpr int kSkLd = kSkBK + 8;              // padded LDS row (bf16)
constexpr int kSkThreads = 512;
constexpr int kSkCpr = kSkBK / 8;             // 16-byte chunks per row slice
constexpr int kSkRows = kSkThreads / kSkCpr;  // rows per loader pass
constexpr int kSkPA = kSkBM / kSkRows;        // loads per thread: x
constexpr int kSkPB = kSkBN / kSkRows;        // ... P^T
constexpr int kSkLoads = kSkPA + kSkPB;
static_assert(kSkBM % kSkRows == 0 && kSkBN % kSkRows == 0, "whole loader passes");

__global__ __launch_bounds__(kSkThreads) void conv_mm_partial_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ pt, float* __restrict__ part,
    int M, int N, int H, int mtiles, int ntiles) {
  __shared__ __attribute__((aligned(16))) uint16_t stage[2][(kSkBM + kSkBN) * kSkLd];
  const int ntile = mtiles * ntiles;
  const int split = blockIdx.x / ntile;
  // tiles that share x rows run on one XCD: n fastest
  const int tile = xcd_tile(blockIdx.x - split * ntile, ntile);
  const int mt = tile / ntiles;
  const int nt = tile - mt * ntiles;
  const int m0 = mt * kSkBM;
  const int n0 = nt * kSkBN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rowsA = min(kSkBM, M - m0);
  const int rowsB = min(kSkBN, N - n0);
  const int kq = (H / 8 + kSplitK - 1) / kSplitK * 8;  // K per split (a multiple of 8)
  const int kbeg = split * kq;
  const int kend = min(H, kbeg + kq);
  const int lrow = tid / kSkCpr;
  const int lk = (tid % kSkCpr) * 8;
  // Rows past the edge repeat the last row (their results are not stored).
  const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x + (size_t)m0 * H), (short)0, rowsA * H * 2, kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(pt + (size_t)n0 * H), (short)0, rowsB * H * 2, kRsrcFlags);
  int off[kSkLoads];
#pragma unroll
  for (int p = 0; p < kSkPA; ++p) off[p] = (min(lrow + p * kSkRows, rowsA - 1) * H + lk) * 2;
#pragma unroll
  for (int p = 0; p < kSkPB; ++p)
    off[kSkPA + p] = (min(lrow + p * kSkRows, rowsB - 1) * H + lk) * 2;
  const int nsl = max(1, (kend - kbeg + kSkBK - 1) / kSkBK);
  // Slices past the end re-read the last slice (in range, never used);
  // chunks past the split's end read as zero.
  u32x4_t R0[kSkLoads], R1[kSkLoads];
  auto gload = [&](u32x4_t(&R)[kSkLoads], int sl) {
    const int k = kbeg + min(sl, nsl - 1) * kSkBK;
    const bool in = k + lk < kend;
    const u32x4_t z = {0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p < kSkLoads; ++p) {
      const u32x4_t v =
          __builtin_amdgcn_raw_buffer_load_b128(p < kSkPA ? rsA : rsB, off[p] + k * 2, 0, 0);
      R[p] = in ? v : z;
    }
  };
  auto sstore = [&](const u32x4_t(&R)[kSkLoads], int buf) {
#pragma unroll
    for (int p = 0; p < kSkLoads; ++p) {
      const int row = p < kSkPA ? lrow + p * kSkRows : kSkBM + lrow + (p - kSkPA) * kSkRows;
      *reinterpret_cast<u32x4_t*>(&stage[buf][row * kSkLd + lk]) = R[p];
    }
  };
  f32x4_t acc[2][5];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 5; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int wr = wave & 3;   // rows 32 wr ..
  const int wc = wave >> 2;  // columns 80 wc ..
  const int fa = (wr * 32 + (lane & 15)) * kSkLd + (lane >> 4) * 8;
  const int fb = (kSkBM + wc * 80 + (lane & 15)) * kSkLd + (lane >> 4) * 8;
  auto multiply = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < kSkBK / 32; ++ks) {
      bf16x8_t a[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(&stage[buf][fa + i * 16 * kSkLd + ks * 32]);
#pragma unroll
      for (int j = 0; j < 5; ++j) {
        const bf16x8_t bv =
            *reinterpret_cast<const bf16x8_t*>(&stage[buf][fb + j * 16 * kSkLd + ks * 32]);
#pragma unroll
        for (int i = 0; i < 2; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bv, acc[i][j], 0, 0, 0);
      }
    }
  };
  gload(R0, 0);
  gload(R1, 1);
  sstore(R0, 0);
  __syncthreads();
  // Slice sl sits in LDS buffer sl & 1; the set that carried it reloads
  // slice sl + 2, the other set (slice sl + 1) is stored after the MFMAs.
  for (int sl = 0; sl < nsl; sl += 2) {
    gload(R0, sl + 2);
    multiply(0);
    sstore(R1, 1);
    __syncthreads();
    if (sl + 1 >= nsl) break;
    gload(R1, sl + 3);
    multiply(1);
    sstore(R0, 0);
    __syncthreads();
  }
  const size_t pitch = (size_t)H / 2;  // floats per row of y
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 5; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wr * 32 + 16 * i + 4 * (lane >> 4) + r;
        const int col = wc * 80 + 16 * j + (lane & 15);
        if (row < rowsA && col < rowsB)
          part[(size_t)(m0 + row) * pitch + (size_t)split * N + n0 + col] = acc[i][j][r];
      }
}

// bf16 rows of H = 640 k <= 5120 channels: ten channels per thread.
bool conv10_fits(int H) { return H % 640 == 0 && H <= kC10 * kC10Threads; }

// Launches conv_rows10_kernel in the given mode; false (nothing launched)
// when the grid would not fit.  Positions per workgroup from a sweep at
// H = 5120 (kernel trace, us): 2048 rows with a projection, 2 x 4 rows (one
// ahead): 11.0 (8 rows of the eight-channel kernel below: 16.1; 2 x 4 rows
// with the next two ahead: 12.0; 4 x 2: 12.1); 4096 static rows, 8 single
// rows, two ahead: 14.1 (18.0); 512 static rows, 2 rows: 4.9 (5.3).  Fewer
// positions when that leaves under 256 workgroups.
bool launch_rows10(int mode, const uint16_t* xq, const uint16_t* aq, uint16_t* yq, const float* k0,
                   const float* k1, const float* proj, int ncols, int gw, int B, int L, int H,
                   hipStream_t s) {
  const long long rows = (long long)B * L;
  const long long units = rows / 256;
  int rn = 1;
  while (rn < 8 && rn * 2 <= L && rn * 2 <= units) rn *= 2;
  const int wpb = (L + rn - 1) / rn;
  const long long wgs = (long long)B * wpb;
  if (wgs > 0x7fffffffLL) return false;
  const dim3 grid((unsigned)wgs), blk((unsigned)(H / kC10));
#define DFLASH2_CONV10(RR, NN, PP, MM)                                                         \
  hipLaunchKernelGGL((conv_rows10_kernel<RR, NN, PP, MM>), grid, blk, 0, s, xq, aq, yq, k0, k1, \
                     proj, L, H, wpb, ncols, gw)
  if (mode == kOnePair) {
    if (rn == 8) DFLASH2_CONV10(2, 4, 1, kOnePair);
    else if (rn == 4) DFLASH2_CONV10(2, 2, 1, kOnePair);
    else if (rn == 2) DFLASH2_CONV10(2, 1, 1, kOnePair);
    else DFLASH2_CONV10(1, 1, 1, kOnePair);
  } else if (mode == kSplitParts) {
    if (rn == 8) DFLASH2_CONV10(2, 4, 1, kSplitParts);
    else if (rn == 4) DFLASH2_CONV10(2, 2, 1, kSplitParts);
    else if (rn == 2) DFLASH2_CONV10(2, 1, 1, kSplitParts);
    else DFLASH2_CONV10(1, 1, 1, kSplitParts);
  } else {
    if (rn == 8) DFLASH2_CONV10(1, 8, 2, kStaticTaps);
    else if (rn == 4) DFLASH2_CONV10(2, 2, 1, kStaticTaps);
    else if (rn == 2) DFLASH2_CONV10(2, 1, 1, kStaticTaps);
    else DFLASH2_CONV10(1, 1, 1, kStaticTaps);
  }
#undef DFLASH2_CONV10
  return true;
}

template <typename T>
hipError_t launch_typed(const void* x, const void* anchor_h, void* y, const float* k0,
                        const float* k1, const float* proj, int groups, int B, int L, int H,
                        hipStream_t s) {
  const T* xp = static_cast<const T*>(x);
  const T* ap = static_cast<const T*>(anchor_h);
  T* yp = static_cast<T*>(y);
  const long long rows = (long long)B * L;
  if constexpr (sizeof(T) == 2) {
    if ((!proj || groups == 1) && conv10_fits(H) &&
        launch_rows10(proj ? kOnePair : kStaticTaps, static_cast<const uint16_t*>(x),
                      static_cast<const uint16_t*>(anchor_h), static_cast<uint16_t*>(y), k0, k1,
                      proj, 0, 0, B, L, H, s))
      return hipGetLastError();
  }
  // Rows of a block per workgroup, measured at H = 5120 (20 launches back to
  // back): the corrections' workgroups take 8 rows (15.9 us per application
  // at 2048 rows against 18.3 for one row per workgroup, 16.0 with 4);
  // static taps take 2 rows up to 2047 rows (4.9 against 6.3 us at 512) and
  // 4 pipelined single rows from 2048 on (18.0 against 21.7 us at 4096).
  // One thread per 8-channel chunk, so H <= 8192 (1024 threads); wider
  // rows take the one-row kernels below.
  const int H8 = H / 8;
  if ((!proj || groups == 1) && H8 <= 1024) {
    int R = 1, NG = 1;
    if (proj) {
      const int rmax = sizeof(T) == 2 ? 8 : 2;  // fp32 rows take twice the registers
      while (R < rmax && R * 2 <= L && rows / (R * 2) >= 256) R *= 2;
    } else if (rows >= 2048 && L >= 4) {
      NG = 4;
    } else if (rows >= 512 && L >= 2) {
      R = 2;
    }
    const int nth = (H8 + 63) / 64 * 64;
    const int wpb = (L + R * NG - 1) / (R * NG);
    const long long wgs = (long long)B * wpb;
    if (wgs <= 0x7fffffffLL) {
      const dim3 grid((unsigned)wgs), blk((unsigned)nth);
#define DFLASH2_CONV_ROWS(RR, NN, CC, DD)                                                       \
  hipLaunchKernelGGL((conv_rows_kernel<T, RR, NN, CC, DD>), grid, blk, 0, s, xp, ap, yp, k0, k1, \
                     proj, L, H, wpb)
#define DFLASH2_CONV_ROWS_C(CC)                                  \
  do {                                                           \
    if (proj) {                                                  \
      if constexpr (sizeof(T) == 2) {                            \
        if (R == 8) DFLASH2_CONV_ROWS(8, 1, CC, true);           \
        else if (R == 4) DFLASH2_CONV_ROWS(4, 1, CC, true);      \
      }                                                          \
      if (R == 2) DFLASH2_CONV_ROWS(2, 1, CC, true);             \
      else if (R == 1) DFLASH2_CONV_ROWS(1, 1, CC, true);        \
    } else {                                                     \
      if (NG == 4) DFLASH2_CONV_ROWS(1, 4, CC, false);           \
      else if (R == 2) DFLASH2_CONV_ROWS(2, 1, CC, false);       \
      else DFLASH2_CONV_ROWS(1, 1, CC, false);                   \
    }                                                            \
  } while (0)
      DFLASH2_CONV_ROWS_C(1);
#undef DFLASH2_CONV_ROWS_C
#undef DFLASH2_CONV_ROWS
      return hipGetLastError();
    }
  }
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
  // Split-K (groups of gw >= 16 channels, whose partials fit in y's rows;
  // rows of H = 640 k <= 5120) when its partial tiles fill half the CUs.
  const int gw = H / groups;
  if (gw >= 16 && conv10_fits(H)) {
    const int smt = (M + kSkBM - 1) / kSkBM;
    const int snt = (N + kSkBN - 1) / kSkBN;
    const long long swgs = (long long)smt * snt * kSplitK;
    if (swgs >= 128 && swgs <= 0x7fffffffLL) {
      hipLaunchKernelGGL(conv_mm_partial_kernel, dim3((unsigned)swgs), dim3(kSkThreads), 0, s, xb,
                         pb, reinterpret_cast<float*>(yb), M, N, H, smt, snt);
      if (launch_rows10(kSplitParts, xb, ab, yb, k0, k1, nullptr, N, gw, B, L, H, s))
        return hipGetLastError();
    }
  }
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
