// Per-row top-16 of fp32 logits ("DFlash 2: Keep Drafting Parallel", section
// "A lightweight path selector": 16 candidates per position).
//
// Order: value descending, then token id ascending.  Each (value, id) pair is
// packed into one 64-bit key that is larger exactly when the pair ranks
// higher:  key = ord(value) << 32 | ~id,  ord() mapping canonical floats
// (-0 -> +0, NaN -> -inf) onto uint32 in the same order.  Every key of a
// real element is > 0, so 0 marks an empty list slot.
//
// A wavefront keeps its best 16 keys sorted in lanes 0..15 of each 16-lane
// row (the four rows hold the same list) and streams its share of the row
// with 16-byte loads.  An element is inspected only when its value is not
// below the current 16th value (one compare per element in the common case);
// survivors are compacted into a small LDS buffer and merged into the list
// by a 64-lane bitonic sort when the buffer fills.  A row may be split over
// several workgroups; their lists are merged by a one-wave-per-row kernel.
#include "common.hpp"

namespace dflash2 {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxSplits = 32;

__device__ __forceinline__ uint32_t ord_of(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) u = 0xff800000u;          // NaN ranks as -inf
  if (u == 0x80000000u) u = 0u;         // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float val_of(uint32_t o) {
  const uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t key_of(float f, uint32_t idx) {
  return ((uint64_t)ord_of(f) << 32) | (uint32_t)(~idx);
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}

// Sorted list of 16 keys per 16-lane row; slot = lane & 15.
struct WaveTop16 {
  uint64_t key;   // this lane's slot
  uint64_t thr;   // 16th key (wave-uniform)
  float thr_f;    // value of the 16th key; -inf while the list is not full

  __device__ void init() {
    key = 0;
    thr = 0;
    thr_f = -INFINITY;
  }
  __device__ void refresh() {
    thr = readlane64(key, 15);
    thr_f = thr ? val_of((uint32_t)(thr >> 32)) : -INFINITY;
  }
};

__device__ __forceinline__ uint64_t shfl64(uint64_t v, int src) {
  const uint32_t lo = __shfl((int)(uint32_t)v, src, 64);
  const uint32_t hi = __shfl((int)(uint32_t)(v >> 32), src, 64);
  return ((uint64_t)hi << 32) | lo;
}

template <int J>
__device__ __forceinline__ uint64_t xor_lane64(uint64_t v) {
  const uint32_t lo = xor_lane<J>((uint32_t)v);
  const uint32_t hi = xor_lane<J>((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

template <int K, int J>
__device__ __forceinline__ uint64_t bitonic_step(uint64_t v, int lane) {
  const uint64_t o = xor_lane64<J>(v);
  const bool keep_max = ((lane & J) == 0) == ((lane & K) == 0);
  return keep_max ? (v > o ? v : o) : (v < o ? v : o);
}

template <int K, int J>
__device__ __forceinline__ uint64_t bitonic_merge(uint64_t v, int lane) {
  v = bitonic_step<K, J>(v, lane);
  if constexpr (J > 1) v = bitonic_merge<K, J / 2>(v, lane);
  return v;
}

// Bitonic sort of one key per lane across the wavefront, descending (lane 0
// ends with the largest).
__device__ uint64_t wave_sort_desc(uint64_t v) {
  const int lane = threadIdx.x & 63;
  v = bitonic_merge<2, 1>(v, lane);
  v = bitonic_merge<4, 2>(v, lane);
  v = bitonic_merge<8, 4>(v, lane);
  v = bitonic_merge<16, 8>(v, lane);
  v = bitonic_merge<32, 16>(v, lane);
  v = bitonic_merge<64, 32>(v, lane);
  return v;
}

// A candidate may rank in the list unless it is strictly below the 16th value
// (NaN always passes here and is decided exactly by its key later).
__device__ __forceinline__ bool may_enter(float v, float thr_f) { return !(v < thr_f); }

// Per-wave candidate buffer in LDS (kBuf keys).  Survivors of the filter are
// appended with a ballot/mbcnt compaction; when the buffer would overflow, the
// list (16 keys) and the buffer (<= 48 keys) are merged by one 64-lane sort.
constexpr int kBuf = 48;

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

__device__ void flush(WaveTop16& top, const uint64_t* buf, int& count) {
  const int lane = threadIdx.x & 63;
  uint64_t v = lane < 16 ? top.key : (lane - 16 < count ? buf[lane - 16] : 0ull);
  v = wave_sort_desc(v);
  top.key = shfl64(v, lane & 15);
  top.refresh();
  count = 0;
}

// Append the keys of lanes with `pass` set (wave-uniform control flow).
__device__ void append(WaveTop16& top, uint64_t* buf, int& count, bool pass, uint64_t key) {
  const uint64_t m = __ballot(pass);
  if (!m) return;
  const int n = __popcll(m);
  if (count + n > kBuf && count) flush(top, buf, count);
  const int lane = threadIdx.x & 63;
  if (n > kBuf) {
    // more survivors than the buffer holds (adversarial order): keep the
    // batch's own best 16, which contain every survivor that can matter
    const uint64_t v = wave_sort_desc(pass ? key : 0ull);
    if (lane < 16) buf[lane] = v;
    count = 16;
    return;
  }
  if (pass) buf[count + lanes_below(m)] = key;
  count += n;
}

// Stream [c0, c1) of one row; VEC = 4 uses 16-byte loads (row and c0 16-byte
// aligned), VEC = 1 scalar loads.  The four waves of the block interleave in
// 64*VEC-element runs; each lane keeps kUnroll loads in flight.
//
// Warm start: on its first vector each lane finds its own largest key; the
// wave sorts those 64 keys and takes the top 16 as its initial list (they are
// real elements, so the list is exact); the other values of that vector go
// through the filter like every later one.
template <int VEC>
__device__ void scan_range(const float* __restrict__ row, int c0, int c1, WaveTop16& top,
                           uint64_t* buf) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  constexpr int kUnroll = 8;
  const int stride = kThreads * VEC;  // elements per block-wide step
  bool first = true;
  int count = 0;
  for (int base = c0 + wave * 64 * VEC; base < c1; base += stride * kUnroll) {
    float v[kUnroll][VEC];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int e = base + u * stride + lane * VEC;
      ok[u] = e < c1;
      if (VEC == 4) {
        f32x4_t q = ok[u] ? *reinterpret_cast<const f32x4_t*>(row + e) : f32x4_t{0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < VEC; ++k) v[u][k] = q[k];
      } else {
        v[u][0] = ok[u] ? row[e] : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int e0 = base + u * stride + lane * VEC;
      int skip = -1;  // the lane's own maximum, already in the list (warm start)
      if (first && u == 0) {
        first = false;
        uint64_t best = 0;
        if (ok[0]) {
#pragma unroll
          for (int k = 0; k < VEC; ++k) {
            const uint64_t c = key_of(v[0][k], (uint32_t)(e0 + k));
            if (c > best) {
              best = c;
              skip = k;
            }
          }
        }
        top.key = shfl64(wave_sort_desc(best), lane & 15);
        top.refresh();
      }
      bool any = false;
#pragma unroll
      for (int k = 0; k < VEC; ++k) any |= ok[u] && (k != skip) && may_enter(v[u][k], top.thr_f);
      if (!__ballot(any)) continue;
#pragma unroll
      for (int k = 0; k < VEC; ++k) {
        const bool p = ok[u] && (k != skip) && may_enter(v[u][k], top.thr_f);
        append(top, buf, count, p, key_of(v[u][k], (uint32_t)(e0 + k)));
      }
    }
  }
  if (count) flush(top, buf, count);
}

// Merge the four waves' lists of a block into wave 0 with one 64-lane sort.
__device__ void merge_block(WaveTop16& top, uint64_t* lds) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if (lane < 16) lds[wave * 16 + lane] = top.key;
  __syncthreads();
  if (wave == 0) {
    top.key = shfl64(wave_sort_desc(lds[lane]), lane & 15);
    top.refresh();
  }
}

__device__ __forceinline__ void write_final(const WaveTop16& top, float* val, int32_t* idx) {
  const int lane = threadIdx.x & 63;
  if (lane < 16) {
    val[lane] = val_of((uint32_t)(top.key >> 32));
    idx[lane] = (int32_t)(~(uint32_t)top.key);
  }
}

template <int VEC>
__global__ __launch_bounds__(kThreads) void topk16_scan_kernel(const float* __restrict__ logits,
                                                               int V, int splits, int chunk,
                                                               float* __restrict__ top_val,
                                                               int32_t* __restrict__ top_idx,
                                                               uint64_t* __restrict__ part) {
  __shared__ uint64_t lds[64];
  __shared__ uint64_t cand[kThreads / 64][kBuf];
  const int m = blockIdx.x / splits;
  const int sp = blockIdx.x - m * splits;
  const float* row = logits + (size_t)m * V;
  const int c0 = sp * chunk;
  const int c1 = min(V, c0 + chunk);
  WaveTop16 top;
  top.init();
  if (c0 < c1) scan_range<VEC>(row, c0, c1, top, cand[threadIdx.x >> 6]);
  merge_block(top, lds);
  if ((threadIdx.x >> 6) != 0) return;
  if (splits == 1) {
    write_final(top, top_val + (size_t)m * kTopK, top_idx + (size_t)m * kTopK);
  } else if ((threadIdx.x & 63) < 16) {
    part[((size_t)m * splits + sp) * kTopK + (threadIdx.x & 15)] = top.key;
  }
}

// One wave per row merges `splits` partial lists.
__global__ __launch_bounds__(64) void topk16_merge_kernel(const uint64_t* __restrict__ part,
                                                          int splits, float* __restrict__ top_val,
                                                          int32_t* __restrict__ top_idx) {
  const int m = blockIdx.x;
  const int lane = threadIdx.x;
  const uint64_t* p = part + (size_t)m * splits * kTopK;
  const int n = splits * kTopK;
  WaveTop16 top;
  top.init();
  // list (lanes 0..15) + the next 48 partial keys (lanes 16..63), one sort each
  for (int base = 0; base < n; base += 48) {
    const int e = base + lane - 16;
    const uint64_t c = lane < 16 ? top.key : (e < n ? p[e] : 0ull);
    top.key = shfl64(wave_sort_desc(c), lane & 15);
  }
  top.refresh();
  write_final(top, top_val + (size_t)m * kTopK, top_idx + (size_t)m * kTopK);
}

// Top-16 of a row that comes with its tile maxima tmax [nt] (tile t covers
// columns [256 t, 256 t + 256)).  Any 16 tile maxima are 16 distinct
// elements, so if tau is at most the 16th largest of some 16 of them, the
// row's 16th best value is >= tau and every top-16 element is >= tau and
// lies in a tile whose maximum is >= tau.  One wave per row, two sorts for
// the bound:
//  - each lane takes the maximum of its share of the tile maxima; the 16th
//    largest of those 64 lane maxima is a first bound, which ~35 tiles of a
//    151936-token row of Gaussian logits reach;
//  - when at most 64 tiles reach it, the 16th largest of their maxima is the
//    exact 16th largest tile maximum, which usually only 16 tiles reach.
// Only those tiles are read, kPruneBatch at a time in flight, and their
// elements >= tau are compacted into an LDS buffer with one ballot per 64
// elements.  The buffer is merged into the sorted list 48 keys per 64-lane
// sort.  Exact: the result is the full scan's, bit for bit.
constexpr int kPruneBatch = 16;
constexpr int kMaxChunk = 16;      // tile maxima per lane per pass (1024 tiles)
constexpr int kFewChunk = 10;      // rows of at most 640 tiles (V <= 163840) take 10
constexpr int kCandCap = 512;      // LDS candidate keys before a merge (a tile adds at most 256)

// Merge n keys of cand into the list (this lane's slot key), 48 per sort.
// Not inlined: the call sites sit inside unrolled loops and are rarely taken.
__device__ __attribute__((noinline)) uint64_t merge_keys(uint64_t key, const uint64_t* cand,
                                                          int n) {
  const int lane = threadIdx.x & 63;
  for (int b = 0; b < n; b += 48) {
    const int e = b + lane - 16;
    const uint64_t c = lane < 16 ? key : (e < n ? cand[e] : 0ull);
    key = shfl64(wave_sort_desc(c), lane & 15);
  }
  return key;
}

__device__ __forceinline__ void merge_cands(WaveTop16& top, const uint64_t* cand, int n) {
  top.key = merge_keys(top.key, cand, n);
  top.refresh();
}

// ord_of(-inf), the lowest order of any element (NaN ranks here too).
constexpr uint32_t kOrdNegInf = 0x007fffffu;

// The loops below are written without per-lane branches: every load is
// issued (indices clamped into the buffer, results masked), and a lane whose
// element is not kept writes to its own spare LDS slot instead of skipping
// the write.  Per-lane branches (one exec-mask branch per element) made the
// selection and compaction steps several times slower.
//
// CAND: the logits come from the GEMM's candidate form.  A tile whose count
// cnt[m, t] is kCandDense was stored whole; any other tile left only its
// values >= a lower bound of the row's 16th value (so every top-16 element
// of the tile) in kCandSlots (value bits, column) slots, the first cnt of
// them used.  Such a tile is read as those slots: lanes 0 and 1 load two
// slots each in place of the tile's 1 KB.
// CH: tile maxima per lane per pass; each wave's work is mostly instruction
// issue on a SIMD of its own, so rows of few tiles take a shorter unroll.
template <int VEC, bool CAND, int CH>
__global__ __launch_bounds__(64) void topk16_pruned_kernel(const float* __restrict__ logits,
                                                           const float* __restrict__ tmax, int V,
                                                           int nt, float* __restrict__ top_val,
                                                           int32_t* __restrict__ top_idx,
                                                           const int* __restrict__ cnt,
                                                           const uint2* __restrict__ slots) {
  static_assert(!CAND || kCandSlots == 4, "two slots per 16-byte load, lanes 0 and 1");
  constexpr int kList = 64 * CH;
  // LDS kept small (9.5 KB) so that many rows are in flight per CU.  A list
  // entry is tile * 8 + (count + 1), the count (CAND) of kCandDense = -1 ..
  // kCandSlots; the tile maxima's orders are only read for the first 64
  // entries (the tighter bound below), so later ones go to spare slots.
  static_assert(kCandDense == -1 && kCandSlots <= 6, "a count fits 3 bits");
  __shared__ uint64_t cand[kCandCap + 64];  // + one spare slot per lane
  __shared__ int list[kList + 64];
  __shared__ uint32_t lord[64 + 64];
  const int m = blockIdx.x;
  const int lane = threadIdx.x;
  const float* tm = tmax + (size_t)m * nt;
  const float* row = logits + (size_t)m * V;
  // 1. tau from the lane maxima.  o = order of a tile maximum, 0 for a tile
  // index past nt (every element's order is > 0).
  uint32_t lmax = 0;
  uint32_t o[CH];  // the last pass's orders (all of them when nt <= kList)
  int cn[CH];      // CAND: the same tiles' counts
  auto load_orders = [&](int c0) {
    float v[CH];
#pragma unroll
    for (int k = 0; k < CH; ++k) v[k] = tm[min(c0 + k * 64 + lane, nt - 1)];
    if constexpr (CAND) {
#pragma unroll
      for (int k = 0; k < CH; ++k)
        cn[k] = cnt[(size_t)m * nt + min(c0 + k * 64 + lane, nt - 1)];
    }
#pragma unroll
    for (int k = 0; k < CH; ++k)
      o[k] = ord_of(v[k]) & (0u - (uint32_t)(c0 + k * 64 + lane < nt));
  };
  for (int c0 = 0; c0 < nt; c0 += kList) {
    load_orders(c0);
#pragma unroll
    for (int k = 0; k < CH; ++k) lmax = max(lmax, o[k]);
  }
  const uint64_t srt = wave_sort_desc(((uint64_t)lmax << 32) | (uint32_t)(~lane));
  uint32_t tau = nt >= 16 ? (uint32_t)(readlane64(srt, 15) >> 32) : 0u;
  // 2. read the tiles that reach tau; keep their elements >= tau
  WaveTop16 top;
  top.init();
  int ncand = 0;
  for (int c0 = 0; c0 < nt; c0 += kList) {
    if (nt > kList) load_orders(c0);
    const uint32_t tmin = max(tau, 1u);
    int nsel = 0;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const bool s = o[k] >= tmin;
      const uint64_t sel = __ballot(s);
      const int below = lanes_below(sel);
      const int at = below + (s ? nsel : kList + lane - below);
      list[at] = (c0 + k * 64 + lane) * 8 + (CAND ? cn[k] + 1 : 0);
      lord[at < 64 ? at : 64 + lane] = o[k];
      nsel += __popcll(sel);
    }
    // Tighter bound: the 16th largest of the selected tiles' maxima (the 16
    // largest tile maxima are 16 distinct elements too).  Tiles below it are
    // dropped, usually leaving 16.
    if (nt >= 16 && nt <= kList && nsel > 16 && nsel <= 64) {
      const int t = lane < nsel ? list[lane] : 0;
      const uint32_t ot = lane < nsel ? lord[lane] : 0u;
      const uint64_t srt2 = wave_sort_desc(((uint64_t)ot << 32) | (uint32_t)(~lane));
      tau = (uint32_t)(readlane64(srt2, 15) >> 32);
      const bool s = lane < nsel && ot >= tau;
      const uint64_t sel = __ballot(s);
      __builtin_amdgcn_wave_barrier();
      list[s ? lanes_below(sel) : kList + lane] = t;
      __builtin_amdgcn_wave_barrier();
      nsel = __popcll(sel);
    }
    for (int b0 = 0; b0 < nsel; b0 += kPruneBatch) {
      const int ns = min(kPruneBatch, nsel - b0);
      f32x4_t q[kPruneBatch];
      int cbase[kPruneBatch];
      int ncn[kPruneBatch];  // CAND: slots used of a sparse tile, -1 for a stored tile
#pragma unroll
      for (int k = 0; k < kPruneBatch; ++k) {
        const int le = k < ns ? list[b0 + k] : 0;  // b0 + k < kList + 64
        const int tl = le >> 3;
        cbase[k] = tl * kTileMaxCols + lane * 4;
        const int c = cbase[k];
        ncn[k] = CAND ? __builtin_amdgcn_readfirstlane(k < ns ? (le & 7) - 1 : 0)
                      : kCandDense;
        if (CAND && ncn[k] != kCandDense) {
          // slots 2 lane, 2 lane + 1 as (v, col, v, col); lanes past 1 re-read
          const uint2* sp = slots + ((size_t)m * nt + tl) * kCandSlots + 2 * min(lane, 1);
          q[k] = *reinterpret_cast<const f32x4_t*>(sp);
        } else if (VEC == 4) {
          q[k] = *reinterpret_cast<const f32x4_t*>(row + min(c, V - 4));  // V % 4 == 0
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) q[k][i] = row[min(c + i, V - 1)];
        }
      }
      // Keep x when ord_of(x) >= floor.  For x not NaN that is x >= the
      // floor's value (ord_of maps -0 and +0 together, as IEEE compares
      // them); NaN ranks as -inf, kept only when the floor is at most -inf.
      const uint32_t floor_ord = top.thr ? max(tau, (uint32_t)(top.thr >> 32)) : tau;
      const bool nan_pass = floor_ord <= kOrdNegInf;
      const float floor_f = nan_pass ? -INFINITY : val_of(floor_ord);
#pragma unroll
      for (int k = 0; k < kPruneBatch; ++k) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int c = cbase[k] + i;
          float x = q[k][i];
          bool ok = c < V;
          if (CAND && ncn[k] != kCandDense) {  // wave-uniform
            if (i >= 2) continue;
            x = q[k][2 * i];
            c = (int)__float_as_uint(q[k][2 * i + 1]);
            ok = 2 * lane + i < ncn[k];
          }
          // bitwise operators: short-circuit forms compile to branches
          const bool p = (k < ns) & ok & ((x >= floor_f) | (nan_pass & (x != x)));
          const uint64_t pm = __ballot(p);
          if (pm) {
            const int below = lanes_below(pm);
            cand[below + (p ? ncand : kCandCap + lane - below)] = key_of(x, (uint32_t)c);
            ncand += __popcll(pm);
          }
        }
        if (ncand > kCandCap - 4 * 64) {  // keep the next tile's keys in range
          merge_cands(top, cand, ncand);
          ncand = 0;
        }
      }
    }
  }
  if (ncand) merge_cands(top, cand, ncand);
  write_final(top, top_val + (size_t)m * kTopK, top_idx + (size_t)m * kTopK);
}

template <bool CAND>
void launch_pruned(bool vec, bool few, const float* logits, const float* tmax, int V, int nt,
                   float* top_val, int32_t* top_idx, const int* cnt, const uint2* sl, int M,
                   hipStream_t s) {
  const dim3 g((unsigned)M), b(64);
  if (vec && few)
    hipLaunchKernelGGL((topk16_pruned_kernel<4, CAND, kFewChunk>), g, b, 0, s, logits, tmax, V,
                       nt, top_val, top_idx, cnt, sl);
  else if (vec)
    hipLaunchKernelGGL((topk16_pruned_kernel<4, CAND, kMaxChunk>), g, b, 0, s, logits, tmax, V,
                       nt, top_val, top_idx, cnt, sl);
  else if (few)
    hipLaunchKernelGGL((topk16_pruned_kernel<1, CAND, kFewChunk>), g, b, 0, s, logits, tmax, V,
                       nt, top_val, top_idx, cnt, sl);
  else
    hipLaunchKernelGGL((topk16_pruned_kernel<1, CAND, kMaxChunk>), g, b, 0, s, logits, tmax, V,
                       nt, top_val, top_idx, cnt, sl);
}

}  // namespace

hipError_t launch_topk16_tilemax(const float* logits, const float* tmax, float* top_val,
                                 int32_t* top_idx, int M, int V, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int nt = (V + kTileMaxCols - 1) / kTileMaxCols;
  const bool vec = (V % 4 == 0) && ((reinterpret_cast<uintptr_t>(logits) & 15) == 0);
  launch_pruned<false>(vec, nt <= 64 * kFewChunk, logits, tmax, V, nt, top_val, top_idx, nullptr,
                       nullptr, M, s);
  return hipGetLastError();
}

hipError_t launch_topk16_cand(const float* logits, const float* tmax, const int* cnt,
                              const void* slots, float* top_val, int32_t* top_idx, int M, int V,
                              hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int nt = (V + kTileMaxCols - 1) / kTileMaxCols;
  const uint2* sl = static_cast<const uint2*>(slots);  // 16-byte aligned
  const bool vec = (V % 4 == 0) && ((reinterpret_cast<uintptr_t>(logits) & 15) == 0);
  launch_pruned<true>(vec, nt <= 64 * kFewChunk, logits, tmax, V, nt, top_val, top_idx, cnt, sl,
                      M, s);
  return hipGetLastError();
}

int topk16_splits(int M, int V) {
  // About 512 blocks (2048 waves, each with 8 loads per lane in flight) and
  // chunks of at least 4096 values; fewer splits mean fewer lists to warm up.
  int s = M > 0 ? (512 + M - 1) / M : 1;
  const int by_len = V / 4096;
  if (s > by_len) s = by_len;
  if (s > kMaxSplits) s = kMaxSplits;
  return s < 1 ? 1 : s;
}

size_t topk16_workspace_bytes(int M, int V) {
  const int s = topk16_splits(M, V);
  return s > 1 ? (size_t)M * s * kTopK * sizeof(uint64_t) : 0;
}

hipError_t launch_topk16(const float* logits, float* top_val, int32_t* top_idx, int M, int V,
                         void* workspace, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int splits = topk16_splits(M, V);
  const bool vec = (V % 4 == 0) && ((reinterpret_cast<uintptr_t>(logits) & 15) == 0);
  int chunk = (V + splits - 1) / splits;
  chunk = (chunk + 3) & ~3;  // keep every chunk start 16-byte aligned
  uint64_t* part = static_cast<uint64_t*>(workspace);
  const dim3 grid((unsigned)((long long)M * splits));
  if (vec)
    hipLaunchKernelGGL(topk16_scan_kernel<4>, grid, dim3(kThreads), 0, s, logits, V, splits,
                       chunk, top_val, top_idx, part);
  else
    hipLaunchKernelGGL(topk16_scan_kernel<1>, grid, dim3(kThreads), 0, s, logits, V, splits,
                       chunk, top_val, top_idx, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  hipLaunchKernelGGL(topk16_merge_kernel, dim3((unsigned)M), dim3(64), 0, s, part, splits,
                     top_val, top_idx);
  return hipGetLastError();
}

}  // namespace dflash2
