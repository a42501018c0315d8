// extern "C" entry points of libdflash2: argument validation on the host,
// then kernel launches on the caller's stream.  Nothing is launched and no
// output is touched unless every check passes.
#include <mutex>

#include "dflash2.h"
#include "common.hpp"

#define DFLASH2_API extern "C" __attribute__((visibility("default")))

using namespace dflash2;

namespace {

constexpr int kVersion = 10000;  // 1.0.0

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }

size_t esize(int dtype) { return dtype == DFLASH2_F32 ? 4 : 2; }
bool valid_dtype(int dtype) { return dtype == DFLASH2_F32 || dtype == DFLASH2_BF16; }
// The LM-head calls also take bf16 h with W in the packed tile layout.
bool lmhead_dtype(int dtype) { return valid_dtype(dtype) || dtype == DFLASH2_BF16_PACKED; }
size_t w_bytes(int V, int H, int dtype) {
  return dtype == DFLASH2_BF16_PACKED ? lmhead_pack_bytes(V, H) : (size_t)V * H * esize(dtype);
}

// Byte ranges [a, a+na) and [b, b+nb) overlap.
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

int status_of(hipError_t e) { return e == hipSuccess ? DFLASH2_OK : DFLASH2_EHIP; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

const long long kInt32Max = 2147483647LL;

}  // namespace

DFLASH2_API int dflash2_version(void) { return kVersion; }

DFLASH2_API const char* dflash2_strerror(int status) {
  switch (status) {
    case DFLASH2_OK: return "ok";
    case DFLASH2_EINVAL: return "invalid argument (pointer, size, shape, alignment or aliasing)";
    case DFLASH2_EUNSUPPORTED: return "unsupported configuration";
    case DFLASH2_EHIP: return "HIP launch or runtime error";
    case DFLASH2_EWORKSPACE: return "workspace missing or too small";
    case DFLASH2_ESCRATCH:
      return "problem larger than the fixed scratch of the allocation-free call";
    default: return "unknown status";
  }
}

DFLASH2_API int dflash2_twotap_conv(const void* x, const void* anchor_h, void* y,
                                    const float* k0, const float* k1, const float* proj,
                                    int groups, int B, int L, int H, int dtype, void* stream) {
  if (!valid_dtype(dtype) || B < 0 || L < 1 || H < 8 || H % 8 != 0) return DFLASH2_EINVAL;
  if ((long long)B * L * H > (1LL << 40)) return DFLASH2_EINVAL;
  if (B == 0) return DFLASH2_OK;
  if (!x || !y || !k0 || !k1) return DFLASH2_EINVAL;
  if (!aligned16(x) || !aligned16(y) || !aligned16(k0) || !aligned16(k1)) return DFLASH2_EINVAL;
  if (anchor_h && !aligned16(anchor_h)) return DFLASH2_EINVAL;
  if (proj) {
    if (groups < 1 || H % groups != 0 || !aligned16(proj)) return DFLASH2_EINVAL;
    if (groups > 1 && (size_t)(H + 2 * groups) * sizeof(double) > 65536)
      return DFLASH2_EUNSUPPORTED;
    if ((long long)B * L > kInt32Max) return DFLASH2_EUNSUPPORTED;  // one workgroup per row
  }
  const size_t es = esize(dtype);
  const size_t xbytes = (size_t)B * L * H * es;
  // workgroups read the parameters while others already write y
  if (overlap(x, xbytes, y, xbytes) || overlap(k0, (size_t)H * 4, y, xbytes) ||
      overlap(k1, (size_t)H * 4, y, xbytes) ||
      (proj && overlap(proj, (size_t)H * 2 * groups * 4, y, xbytes)))
    return DFLASH2_EINVAL;
  if (anchor_h && overlap(anchor_h, (size_t)B * H * es, y, xbytes)) return DFLASH2_EINVAL;
  return status_of(launch_twotap_conv(x, anchor_h, y, k0, k1, proj, proj ? groups : 1, B, L, H,
                                      dtype, as_stream(stream)));
}

DFLASH2_API int dflash2_twotap_conv_mm(const void* x, const void* anchor_h, void* y,
                                       const float* k0, const float* k1, const void* projT,
                                       int groups, int B, int L, int H, int dtype, void* stream) {
  if (!valid_dtype(dtype) || B < 0 || L < 1 || H < 8 || H % 8 != 0) return DFLASH2_EINVAL;
  if (groups < 1 || H % groups != 0) return DFLASH2_EINVAL;
  if ((long long)B * L * H > (1LL << 40)) return DFLASH2_EINVAL;
  if (dtype != DFLASH2_BF16) return DFLASH2_EUNSUPPORTED;  // matrix cores take bf16 operands
  if (B == 0) return DFLASH2_OK;
  if (!x || !y || !k0 || !k1 || !projT) return DFLASH2_EINVAL;
  if (!aligned16(x) || !aligned16(y) || !aligned16(k0) || !aligned16(k1) || !aligned16(projT))
    return DFLASH2_EINVAL;
  if (anchor_h && !aligned16(anchor_h)) return DFLASH2_EINVAL;
  // 32-bit byte offsets inside a 64-row tile; tile and grid counts in int
  if (H > (1 << 21) || (long long)B * L > kInt32Max / 2) return DFLASH2_EUNSUPPORTED;
  const size_t xbytes = (size_t)B * L * H * 2;
  if (overlap(x, xbytes, y, xbytes) ||
      (anchor_h && overlap(anchor_h, (size_t)B * H * 2, y, xbytes)) ||
      overlap(projT, (size_t)2 * groups * H * 2, y, xbytes) ||
      overlap(k0, (size_t)H * 4, y, xbytes) || overlap(k1, (size_t)H * 4, y, xbytes))
    return DFLASH2_EINVAL;
  return status_of(launch_twotap_conv_mm(x, anchor_h, y, k0, k1, projT, groups, B, L, H,
                                         as_stream(stream)));
}

namespace {
int check_lmhead(const void* h, const void* W, int M, int H, int V, int dtype) {
  if (!lmhead_dtype(dtype) || M < 0 || H < 8 || H % 8 != 0 || V < kTopK) return DFLASH2_EINVAL;
  if ((long long)M * V > (1LL << 40) || (long long)V * H > (1LL << 40)) return DFLASH2_EINVAL;
  if (M > 0 && (!h || !W || !aligned16(h) || !aligned16(W))) return DFLASH2_EINVAL;
  if (H > (1 << 21)) return DFLASH2_EUNSUPPORTED;  // 32-bit tile offsets
  return DFLASH2_OK;
}
}  // namespace

DFLASH2_API int dflash2_lmhead_logits(const void* h, const void* W, float* logits, int M, int H,
                                      int V, int dtype, void* stream) {
  int st = check_lmhead(h, W, M, H, V, dtype);
  if (st != DFLASH2_OK) return st;
  if (M == 0) return DFLASH2_OK;
  if (!logits || !aligned16(logits)) return DFLASH2_EINVAL;
  const size_t zb = (size_t)M * V * sizeof(float);
  if (overlap(logits, zb, h, (size_t)M * H * esize(dtype)) ||
      overlap(logits, zb, W, w_bytes(V, H, dtype)))
    return DFLASH2_EINVAL;
  return status_of(launch_lmhead(h, W, logits, nullptr, M, H, V, dtype, as_stream(stream)));
}

static size_t tilemax_bytes(int M, int V) {
  return (size_t)M * ((V + kTileMaxCols - 1) / kTileMaxCols) * sizeof(float);
}

DFLASH2_API int dflash2_lmhead_logits_tilemax(const void* h, const void* W, float* logits,
                                              float* tilemax, int M, int H, int V, int dtype,
                                              void* stream) {
  int st = check_lmhead(h, W, M, H, V, dtype);
  if (st != DFLASH2_OK) return st;
  if (M == 0) return DFLASH2_OK;
  if (!logits || !aligned16(logits) || !tilemax || !aligned4(tilemax)) return DFLASH2_EINVAL;
  const size_t zb = (size_t)M * V * sizeof(float);
  const size_t tb = tilemax_bytes(M, V);
  const size_t es = esize(dtype);
  const size_t wb = w_bytes(V, H, dtype);
  if (overlap(logits, zb, h, (size_t)M * H * es) || overlap(logits, zb, W, wb) ||
      overlap(tilemax, tb, h, (size_t)M * H * es) || overlap(tilemax, tb, W, wb) ||
      overlap(tilemax, tb, logits, zb))
    return DFLASH2_EINVAL;
  return status_of(launch_lmhead(h, W, logits, tilemax, M, H, V, dtype, as_stream(stream)));
}

DFLASH2_API size_t dflash2_lmhead_pack_bytes(int V, int H) {
  if (V < 1 || H < 8 || H % 8 != 0 || (long long)V * H > (1LL << 40) || H > (1 << 21)) return 0;
  return lmhead_pack_bytes(V, H);
}

DFLASH2_API int dflash2_lmhead_pack(const void* W, void* Wp, int V, int H, void* stream) {
  if (V < 1 || H < 8 || H % 8 != 0 || (long long)V * H > (1LL << 40)) return DFLASH2_EINVAL;
  if (H > (1 << 21)) return DFLASH2_EUNSUPPORTED;
  if (!W || !Wp || !aligned16(W) || !aligned16(Wp)) return DFLASH2_EINVAL;
  if (overlap(W, (size_t)V * H * 2, Wp, lmhead_pack_bytes(V, H))) return DFLASH2_EINVAL;
  return status_of(launch_lmhead_pack(W, Wp, V, H, as_stream(stream)));
}

DFLASH2_API int dflash2_topk16_tilemax(const float* logits, const float* tilemax, float* top_val,
                                       int32_t* top_idx, int M, int V, int K, void* stream) {
  if (K != kTopK || M < 0 || V < kTopK || (long long)M * V > (1LL << 40)) return DFLASH2_EINVAL;
  if (M == 0) return DFLASH2_OK;
  if (!logits || !aligned4(logits) || !tilemax || !aligned4(tilemax)) return DFLASH2_EINVAL;
  if (!top_val || !top_idx || !aligned4(top_val) || !aligned4(top_idx)) return DFLASH2_EINVAL;
  const size_t zb = (size_t)M * V * sizeof(float);
  const size_t ob = (size_t)M * kTopK * 4;
  const size_t tb = tilemax_bytes(M, V);
  if (overlap(top_val, ob, logits, zb) || overlap(top_idx, ob, logits, zb) ||
      overlap(top_val, ob, tilemax, tb) || overlap(top_idx, ob, tilemax, tb) ||
      overlap(top_val, ob, top_idx, ob))
    return DFLASH2_EINVAL;
  return status_of(
      launch_topk16_tilemax(logits, tilemax, top_val, top_idx, M, V, as_stream(stream)));
}

DFLASH2_API size_t dflash2_topk16_workspace(int M, int V, int K) {
  if (M < 0 || V < kTopK || K != kTopK) return 0;
  return topk16_workspace_bytes(M, V);
}

namespace {
int check_topk_out(float* top_val, int32_t* top_idx, int M) {
  if (M > 0 && (!top_val || !top_idx || !aligned4(top_val) || !aligned4(top_idx)))
    return DFLASH2_EINVAL;
  return DFLASH2_OK;
}
}  // namespace

DFLASH2_API int dflash2_topk16(const float* logits, float* top_val, int32_t* top_idx, int M, int V,
                               int K, void* workspace, size_t workspace_bytes, void* stream) {
  if (K != kTopK || M < 0 || V < kTopK || (long long)M * V > (1LL << 40)) return DFLASH2_EINVAL;
  if (M == 0) return DFLASH2_OK;
  if (!logits || !aligned4(logits)) return DFLASH2_EINVAL;
  int st = check_topk_out(top_val, top_idx, M);
  if (st != DFLASH2_OK) return st;
  const size_t need = topk16_workspace_bytes(M, V);
  if (need > 0 && (!workspace || workspace_bytes < need ||
                   (reinterpret_cast<uintptr_t>(workspace) & 255) != 0))
    return DFLASH2_EWORKSPACE;
  const size_t zb = (size_t)M * V * sizeof(float);
  if (overlap(top_val, (size_t)M * kTopK * 4, logits, zb) ||
      overlap(top_idx, (size_t)M * kTopK * 4, logits, zb) ||
      overlap(top_val, (size_t)M * kTopK * 4, top_idx, (size_t)M * kTopK * 4) ||
      (need && overlap(workspace, need, logits, zb)))
    return DFLASH2_EINVAL;
  return status_of(launch_topk16(logits, top_val, top_idx, M, V, workspace, as_stream(stream)));
}

// Workspace of dflash2_logits_topk, each part 256-byte aligned: the tile
// maxima; when the caller gives no logits buffer, for bf16 the candidate
// form's group maxima [M, 16], counts [M, nt] and slots [M, nt, 4] (uint2),
// and then the logits [M, V] (only the tiles the GEMM stores are written).
namespace {
struct TopkWs {
  size_t gmax = 0, cnt = 0, slots = 0, z = 0, total = 0;
  bool cand = false;
};
size_t al256(size_t b) { return (b + 255) & ~(size_t)255; }
TopkWs topk_ws(int M, int V, int dtype, bool logits_given) {
  TopkWs w;
  const size_t nt = (size_t)((V + kTileMaxCols - 1) / kTileMaxCols);
  size_t at = al256(tilemax_bytes(M, V));
  w.cand = !logits_given && (dtype == DFLASH2_BF16 || dtype == DFLASH2_BF16_PACKED);
  if (w.cand) {
    w.gmax = at;
    at += al256((size_t)M * kTopK * 4);
    w.cnt = at;
    at += al256((size_t)M * nt * 4);
    w.slots = at;
    at += al256((size_t)M * nt * kCandSlots * 8);
  }
  w.z = at;
  if (!logits_given) at += (size_t)M * V * sizeof(float);
  w.total = at;
  return w;
}
}  // namespace

DFLASH2_API size_t dflash2_logits_topk_workspace(int M, int H, int V, int K, int dtype,
                                                 int logits_given) {
  if (K != kTopK || M < 0 || V < kTopK || H < 8 || !lmhead_dtype(dtype)) return 0;
  return topk_ws(M, V, dtype, logits_given != 0).total;
}

DFLASH2_API int dflash2_logits_topk(const void* h, const void* W, float* logits, float* top_val,
                                    int32_t* top_idx, int M, int H, int V, int K, int dtype,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  if (K != kTopK) return DFLASH2_EINVAL;
  int st = check_lmhead(h, W, M, H, V, dtype);
  if (st != DFLASH2_OK) return st;
  if (M == 0) return DFLASH2_OK;
  st = check_topk_out(top_val, top_idx, M);
  if (st != DFLASH2_OK) return st;
  if (logits && !aligned16(logits)) return DFLASH2_EINVAL;
  const size_t need = dflash2_logits_topk_workspace(M, H, V, K, dtype, logits != nullptr);
  if (need > 0 && (!workspace || workspace_bytes < need ||
                   (reinterpret_cast<uintptr_t>(workspace) & 255) != 0))
    return DFLASH2_EWORKSPACE;
  const TopkWs lay = topk_ws(M, V, dtype, logits != nullptr);
  char* wsb = static_cast<char*>(workspace);
  float* tmax = static_cast<float*>(workspace);
  float* z = logits ? logits : reinterpret_cast<float*>(wsb + lay.z);
  const size_t zb = (size_t)M * V * sizeof(float);
  const size_t es = esize(dtype);
  const size_t wb = w_bytes(V, H, dtype);
  if (overlap(z, zb, h, (size_t)M * H * es) || overlap(z, zb, W, wb) ||
      overlap(top_val, (size_t)M * kTopK * 4, z, zb) ||
      overlap(top_idx, (size_t)M * kTopK * 4, z, zb) ||
      (logits && need && overlap(workspace, need, logits, zb)))
    return DFLASH2_EINVAL;
  if (overlap(top_val, (size_t)M * kTopK * 4, workspace, need) ||
      overlap(top_idx, (size_t)M * kTopK * 4, workspace, need) ||
      overlap(workspace, need, h, (size_t)M * H * es) ||
      overlap(workspace, need, W, wb))
    return DFLASH2_EINVAL;
  hipStream_t s = as_stream(stream);
  if (lay.cand) {
    uint32_t* gmax = reinterpret_cast<uint32_t*>(wsb + lay.gmax);
    int* cnt = reinterpret_cast<int*>(wsb + lay.cnt);
    void* slots = wsb + lay.slots;
    hipError_t e = launch_lmhead_cand(h, W, z, tmax, gmax, cnt, slots, M, H, V, dtype, s);
    if (e != hipSuccess) return DFLASH2_EHIP;
    return status_of(launch_topk16_cand(z, tmax, cnt, slots, top_val, top_idx, M, V, s));
  }
  hipError_t e = launch_lmhead(h, W, z, tmax, M, H, V, dtype, s);
  if (e != hipSuccess) return DFLASH2_EHIP;
  return status_of(launch_topk16_tilemax(z, tmax, top_val, top_idx, M, V, s));
}

DFLASH2_API int dflash2_lmhead_candidates(const void* h, const void* W, int M, int H, int V,
                                          int dtype, void* workspace, size_t workspace_bytes,
                                          void* stream) {
  int st = check_lmhead(h, W, M, H, V, dtype);
  if (st != DFLASH2_OK) return st;
  if (dtype != DFLASH2_BF16 && dtype != DFLASH2_BF16_PACKED) return DFLASH2_EUNSUPPORTED;
  if (M == 0) return DFLASH2_OK;
  const TopkWs lay = topk_ws(M, V, dtype, false);
  if (!workspace || workspace_bytes < lay.total ||
      (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return DFLASH2_EWORKSPACE;
  if (overlap(workspace, lay.total, h, (size_t)M * H * 2) ||
      overlap(workspace, lay.total, W, w_bytes(V, H, dtype)))
    return DFLASH2_EINVAL;
  char* wsb = static_cast<char*>(workspace);
  return status_of(launch_lmhead_cand(
      h, W, reinterpret_cast<float*>(wsb + lay.z), reinterpret_cast<float*>(wsb),
      reinterpret_cast<uint32_t*>(wsb + lay.gmax), reinterpret_cast<int*>(wsb + lay.cnt),
      wsb + lay.slots, M, H, V, dtype, as_stream(stream)));
}

DFLASH2_API int dflash2_topk16_candidates(const void* workspace, size_t workspace_bytes,
                                          float* top_val, int32_t* top_idx, int M, int H, int V,
                                          int K, void* stream) {
  if (K != kTopK || M < 0 || V < kTopK || H < 8 || (long long)M * V > (1LL << 40))
    return DFLASH2_EINVAL;
  if (M == 0) return DFLASH2_OK;
  int st = check_topk_out(top_val, top_idx, M);
  if (st != DFLASH2_OK) return st;
  const TopkWs lay = topk_ws(M, V, DFLASH2_BF16, false);
  if (!workspace || workspace_bytes < lay.total ||
      (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return DFLASH2_EWORKSPACE;
  const size_t ob = (size_t)M * kTopK * 4;
  if (overlap(top_val, ob, workspace, lay.total) || overlap(top_idx, ob, workspace, lay.total) ||
      overlap(top_val, ob, top_idx, ob))
    return DFLASH2_EINVAL;
  const char* wsb = static_cast<const char*>(workspace);
  return status_of(launch_topk16_cand(
      reinterpret_cast<const float*>(wsb + lay.z), reinterpret_cast<const float*>(wsb),
      reinterpret_cast<const int*>(wsb + lay.cnt), wsb + lay.slots, top_val, top_idx, M, V,
      as_stream(stream)));
}

static int pair_score(const float* top_val, const int32_t* top_idx, const int32_t* anchor_tok,
                      const void* U, const void* Vf, const float* gate, int B, int L, int V, int r,
                      int dtype, float* S0, float* S, void* stream) {
  if (!valid_dtype(dtype) || B < 0 || L < 1 || L > DFLASH2_MAX_L || V < kTopK || r < 1 ||
      r > DFLASH2_MAX_RANK)
    return DFLASH2_EINVAL;
  if (B == 0) return DFLASH2_OK;
  if (!top_val || !top_idx || !U || !Vf || !S0 || (L > 1 && !S)) return DFLASH2_EINVAL;
  if ((long long)V * r > (1LL << 40) || (long long)B * L * kTopK > kInt32Max)
    return DFLASH2_EINVAL;
  if (!aligned4(top_val) || !aligned4(top_idx) || !aligned4(S0) || (S && !aligned16(S)) ||
      (anchor_tok && !aligned4(anchor_tok)) || (gate && !aligned4(gate)))
    return DFLASH2_EINVAL;
  const size_t es = esize(dtype);
  if (dtype == DFLASH2_BF16 ? ((reinterpret_cast<uintptr_t>(U) | reinterpret_cast<uintptr_t>(Vf)) & 1)
                            : (!aligned4(U) || !aligned4(Vf)))
    return DFLASH2_EINVAL;
  const size_t s0b = (size_t)B * kTopK * 4;
  const size_t sb = L > 1 ? (size_t)B * (L - 1) * kTopK * kTopK * 4 : 0;
  const size_t tb = (size_t)B * L * kTopK * 4;
  const void* ins[] = {top_val, top_idx, U, Vf, anchor_tok, gate};
  const size_t insz[] = {tb, tb, (size_t)V * r * es, (size_t)V * r * es, (size_t)B * 4,
                         (size_t)B * L * r * 4};
  for (int i = 0; i < 6; ++i) {
    if (overlap(S0, s0b, ins[i], insz[i]) || (sb && overlap(S, sb, ins[i], insz[i])))
      return DFLASH2_EINVAL;
  }
  if (sb && overlap(S0, s0b, S, sb)) return DFLASH2_EINVAL;
  return status_of(launch_pair_score(top_val, top_idx, anchor_tok, U, Vf, gate, B, L, V, r, dtype,
                                     S0, L > 1 ? S : nullptr, as_stream(stream)));
}

DFLASH2_API int dflash2_pair_score(const float* top_val, const int32_t* top_idx,
                                   const int32_t* anchor_tok, const void* U, const void* Vf,
                                   int B, int L, int V, int r, int dtype, float* S0, float* S,
                                   void* stream) {
  return pair_score(top_val, top_idx, anchor_tok, U, Vf, nullptr, B, L, V, r, dtype, S0, S,
                    stream);
}

DFLASH2_API int dflash2_pair_score_gated(const float* top_val, const int32_t* top_idx,
                                         const int32_t* anchor_tok, const void* U, const void* Vf,
                                         const float* gate, int B, int L, int V, int r, int dtype,
                                         float* S0, float* S, void* stream) {
  if (!gate && B > 0) return DFLASH2_EINVAL;
  return pair_score(top_val, top_idx, anchor_tok, U, Vf, gate, B, L, V, r, dtype, S0, S, stream);
}

DFLASH2_API int dflash2_context_gate(const void* h, const void* Wg, float* gate, int M, int H,
                                     int r, int dtype, void* stream) {
  if (!valid_dtype(dtype) || M < 0 || H < 8 || H % 8 != 0 || r < 1 || r > DFLASH2_MAX_RANK)
    return DFLASH2_EINVAL;
  if (M == 0) return DFLASH2_OK;
  if (!h || !Wg || !gate) return DFLASH2_EINVAL;
  if (!aligned16(h) || !aligned16(Wg) || !aligned4(gate)) return DFLASH2_EINVAL;
  if (H > (1 << 21) || (long long)M * r > kInt32Max) return DFLASH2_EUNSUPPORTED;
  const size_t es = esize(dtype);
  const size_t gb = (size_t)M * r * 4;
  if (overlap(gate, gb, h, (size_t)M * H * es) || overlap(gate, gb, Wg, (size_t)r * H * es))
    return DFLASH2_EINVAL;
  return status_of(launch_context_gate(h, Wg, gate, M, H, r, dtype, as_stream(stream)));
}

static int path_select(const float* S0, const float* S, const int32_t* top_idx, int B, int L,
                       int mode, int32_t* path_slot, int32_t* path_tok, float* path_score,
                       void* stream) {
  if (B < 0 || L < 1 || L > DFLASH2_MAX_L) return DFLASH2_EINVAL;
  if (mode != DFLASH2_PATH_VITERBI && mode != DFLASH2_PATH_GREEDY) return DFLASH2_EINVAL;
  if (B == 0) return DFLASH2_OK;
  if (!S0 || (L > 1 && !S) || !path_slot || !path_score) return DFLASH2_EINVAL;
  if (mode == DFLASH2_PATH_GREEDY && L > 1 && !aligned16(S)) return DFLASH2_EINVAL;
  if ((top_idx == nullptr) != (path_tok == nullptr)) return DFLASH2_EINVAL;
  if (!aligned4(S0) || (S && !aligned4(S)) || !aligned4(path_slot) || !aligned4(path_score) ||
      (top_idx && !aligned4(top_idx)) || (path_tok && !aligned4(path_tok)))
    return DFLASH2_EINVAL;
  const size_t s0b = (size_t)B * kTopK * 4;
  const size_t sb = L > 1 ? (size_t)B * (L - 1) * kTopK * kTopK * 4 : 0;
  const size_t tib = (size_t)B * L * kTopK * 4;
  const size_t pb = (size_t)B * L * 4;
  const void* outs[] = {path_slot, path_tok, path_score};
  const size_t outsz[] = {pb, pb, (size_t)B * 4};
  for (int i = 0; i < 3; ++i) {
    if (overlap(outs[i], outsz[i], S0, s0b) || (sb && overlap(outs[i], outsz[i], S, sb)) ||
        overlap(outs[i], outsz[i], top_idx, tib))
      return DFLASH2_EINVAL;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outsz[i], outs[j], outsz[j])) return DFLASH2_EINVAL;
  }
  return status_of(launch_path_select(S0, L > 1 ? S : nullptr, top_idx, B, L,
                                      mode == DFLASH2_PATH_GREEDY, path_slot, path_tok,
                                      path_score, as_stream(stream)));
}

DFLASH2_API int dflash2_path_select(const float* S0, const float* S, const int32_t* top_idx,
                                    int B, int L, int32_t* path_slot, int32_t* path_tok,
                                    float* path_score, void* stream) {
  return path_select(S0, S, top_idx, B, L, DFLASH2_PATH_VITERBI, path_slot, path_tok, path_score,
                     stream);
}

DFLASH2_API int dflash2_path_select_mode(const float* S0, const float* S, const int32_t* top_idx,
                                         int B, int L, int mode, int32_t* path_slot,
                                         int32_t* path_tok, float* path_score, void* stream) {
  return path_select(S0, S, top_idx, B, L, mode, path_slot, path_tok, path_score, stream);
}

static bool valid_temperature(float T) { return T > 0.f && T <= 1e30f && T == T; }

static bool valid_sample_mode(int mode) {
  return mode == DFLASH2_SAMPLE_CHAIN || mode == DFLASH2_SAMPLE_PATH;
}

static int path_sample(const float* S0, const float* S, const int32_t* top_idx, const float* u,
                       float temperature, int B, int L, int mode, int32_t* path_slot,
                       int32_t* path_tok, float* q, void* stream) {
  if (B < 0 || L < 1 || L > DFLASH2_MAX_L || !valid_temperature(temperature) ||
      !valid_sample_mode(mode))
    return DFLASH2_EINVAL;
  if (B == 0) return DFLASH2_OK;
  if (!S0 || (L > 1 && !S) || !u || !path_slot || !q) return DFLASH2_EINVAL;
  if ((top_idx == nullptr) != (path_tok == nullptr)) return DFLASH2_EINVAL;
  if (!aligned4(S0) || (L > 1 && !aligned16(S)) || !aligned4(u) || !aligned4(path_slot) ||
      !aligned4(q) || (top_idx && !aligned4(top_idx)) || (path_tok && !aligned4(path_tok)))
    return DFLASH2_EINVAL;
  const size_t s0b = (size_t)B * kTopK * 4;
  const size_t sb = L > 1 ? (size_t)B * (L - 1) * kTopK * kTopK * 4 : 0;
  const size_t tib = (size_t)B * L * kTopK * 4;
  const size_t pb = (size_t)B * L * 4;
  const void* ins[] = {S0, S, top_idx, u};
  const size_t insz[] = {s0b, sb, tib, pb};
  void* outs[] = {path_slot, path_tok, q};
  const size_t outsz[] = {pb, pb, tib};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 4; ++j)
      if (insz[j] && overlap(outs[i], outsz[i], ins[j], insz[j])) return DFLASH2_EINVAL;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outsz[i], outs[j], outsz[j])) return DFLASH2_EINVAL;
  }
  return status_of(launch_path_sample(S0, L > 1 ? S : nullptr, top_idx, u, temperature, B, L,
                                      mode == DFLASH2_SAMPLE_PATH, path_slot, path_tok, q,
                                      as_stream(stream)));
}

DFLASH2_API int dflash2_path_sample(const float* S0, const float* S, const int32_t* top_idx,
                                    const float* u, float temperature, int B, int L,
                                    int32_t* path_slot, int32_t* path_tok, float* q,
                                    void* stream) {
  return path_sample(S0, S, top_idx, u, temperature, B, L, DFLASH2_SAMPLE_CHAIN, path_slot,
                     path_tok, q, stream);
}

DFLASH2_API int dflash2_path_sample_mode(const float* S0, const float* S, const int32_t* top_idx,
                                         const float* u, float temperature, int B, int L,
                                         int mode, int32_t* path_slot, int32_t* path_tok,
                                         float* q, void* stream) {
  return path_sample(S0, S, top_idx, u, temperature, B, L, mode, path_slot, path_tok, q, stream);
}

DFLASH2_API int dflash2_target_lse(const float* z, int R, int V, float temperature, float* lse,
                                   void* stream) {
  if (R < 0 || V < 1 || !valid_temperature(temperature)) return DFLASH2_EINVAL;
  if ((long long)R * V > (1LL << 40)) return DFLASH2_EINVAL;
  if (R == 0) return DFLASH2_OK;
  if (!z || !lse || !aligned16(z) || !aligned4(lse)) return DFLASH2_EINVAL;
  if (overlap(lse, (size_t)R * 4, z, (size_t)R * V * 4)) return DFLASH2_EINVAL;
  return status_of(launch_target_lse(z, R, V, temperature, lse, as_stream(stream)));
}

DFLASH2_API int dflash2_verify_rejection(const int32_t* path_slot, const int32_t* path_tok,
                                         const float* q, const int32_t* top_idx, const float* z,
                                         const float* lse, float temperature, const float* u_acc,
                                         const float* u_res, int B, int L, int V,
                                         int32_t* accept_len, int32_t* next_tok, void* stream) {
  if (B < 0 || L < 1 || L > DFLASH2_MAX_L || V < kTopK || !valid_temperature(temperature))
    return DFLASH2_EINVAL;
  if ((long long)B * (L + 1) * V > (1LL << 40)) return DFLASH2_EINVAL;
  if (verify_rejection_lds(V) > 65536) return DFLASH2_EUNSUPPORTED;  // tile sums in LDS
  if (B == 0) return DFLASH2_OK;
  if (!path_slot || !path_tok || !q || !top_idx || !z || !lse || !u_acc || !u_res ||
      !accept_len || !next_tok)
    return DFLASH2_EINVAL;
  const void* all[] = {path_slot, path_tok, q, top_idx, z, lse, u_acc, u_res, accept_len,
                       next_tok};
  for (const void* p : all)
    if (!aligned4(p)) return DFLASH2_EINVAL;
  const size_t pb = (size_t)B * L * 4, tib = (size_t)B * L * kTopK * 4, ob = (size_t)B * 4;
  const void* ins[] = {path_slot, path_tok, q, top_idx, z, lse, u_acc, u_res};
  const size_t insz[] = {pb, pb, tib, tib, (size_t)B * (L + 1) * V * 4, (size_t)B * (L + 1) * 4,
                         pb, ob};
  for (int j = 0; j < 8; ++j)
    if (overlap(accept_len, ob, ins[j], insz[j]) || overlap(next_tok, ob, ins[j], insz[j]))
      return DFLASH2_EINVAL;
  if (overlap(accept_len, ob, next_tok, ob)) return DFLASH2_EINVAL;
  return status_of(launch_verify_rejection(path_slot, path_tok, q, top_idx, z, lse, temperature,
                                           u_acc, u_res, B, L, V, accept_len, next_tok,
                                           as_stream(stream)));
}

DFLASH2_API int dflash2_verify_rejection_lazy(const int32_t* path_slot, const int32_t* path_tok,
                                              const float* q, const int32_t* top_idx,
                                              const float* z, float temperature,
                                              const float* u_acc, const float* u_res, int B,
                                              int L, int V, int32_t* accept_len,
                                              int32_t* next_tok, void* stream) {
  if (B < 0 || L < 1 || L > DFLASH2_MAX_L || V < kTopK || !valid_temperature(temperature))
    return DFLASH2_EINVAL;
  if ((long long)B * (L + 1) * V > (1LL << 40)) return DFLASH2_EINVAL;
  if (verify_rejection_lazy_lds(V) > 65536) return DFLASH2_EUNSUPPORTED;  // tiles in LDS
  if (B == 0) return DFLASH2_OK;
  if (!path_slot || !path_tok || !q || !top_idx || !z || !u_acc || !u_res || !accept_len ||
      !next_tok)
    return DFLASH2_EINVAL;
  const void* all[] = {path_slot, path_tok, q, top_idx, z, u_acc, u_res, accept_len, next_tok};
  for (const void* p : all)
    if (!aligned4(p)) return DFLASH2_EINVAL;
  const size_t pb = (size_t)B * L * 4, tib = (size_t)B * L * kTopK * 4, ob = (size_t)B * 4;
  const void* ins[] = {path_slot, path_tok, q, top_idx, z, u_acc, u_res};
  const size_t insz[] = {pb, pb, tib, tib, (size_t)B * (L + 1) * V * 4, pb, ob};
  for (int j = 0; j < 7; ++j)
    if (overlap(accept_len, ob, ins[j], insz[j]) || overlap(next_tok, ob, ins[j], insz[j]))
      return DFLASH2_EINVAL;
  if (overlap(accept_len, ob, next_tok, ob)) return DFLASH2_EINVAL;
  return status_of(launch_verify_rejection_lazy(path_slot, path_tok, q, top_idx, z, temperature,
                                                u_acc, u_res, B, L, V, accept_len, next_tok,
                                                as_stream(stream)));
}

DFLASH2_API size_t dflash2_verify_rejection_staged_workspace(int B, int L, int V, int rows) {
  if (B < 0 || L < 1 || L > DFLASH2_MAX_L || V < kTopK || rows < 1 || rows > L + 1) return 0;
  return verify_rejection_staged_bytes(B, V, rows);
}

DFLASH2_API int dflash2_verify_rejection_staged(const int32_t* path_slot, const int32_t* path_tok,
                                                const float* q, const int32_t* top_idx,
                                                const float* z, float temperature,
                                                const float* u_acc, const float* u_res, int B,
                                                int L, int V, int rows, void* workspace,
                                                size_t workspace_bytes, int32_t* accept_len,
                                                int32_t* next_tok, void* stream) {
  if (B < 0 || L < 1 || L > DFLASH2_MAX_L || V < kTopK || !valid_temperature(temperature))
    return DFLASH2_EINVAL;
  if (rows < 1 || rows > L + 1) return DFLASH2_EINVAL;
  if ((long long)B * (L + 1) * V > (1LL << 40)) return DFLASH2_EINVAL;
  if (verify_rejection_lazy_lds(V) > 65536) return DFLASH2_EUNSUPPORTED;  // tiles in LDS
  if (B == 0) return DFLASH2_OK;
  if (!path_slot || !path_tok || !q || !top_idx || !z || !u_acc || !u_res || !accept_len ||
      !next_tok || !workspace)
    return DFLASH2_EINVAL;
  const size_t need = verify_rejection_staged_bytes(B, V, rows);
  if (workspace_bytes < need) return DFLASH2_EINVAL;
  const void* all[] = {path_slot, path_tok, q, top_idx, z, u_acc, u_res, accept_len, next_tok,
                       workspace};
  for (const void* p : all)
    if (!aligned4(p)) return DFLASH2_EINVAL;
  const size_t pb = (size_t)B * L * 4, tib = (size_t)B * L * kTopK * 4, ob = (size_t)B * 4;
  const void* ins[] = {path_slot, path_tok, q, top_idx, z, u_acc, u_res};
  const size_t insz[] = {pb, pb, tib, tib, (size_t)B * (L + 1) * V * 4, pb, ob};
  for (int j = 0; j < 7; ++j)
    if (overlap(accept_len, ob, ins[j], insz[j]) || overlap(next_tok, ob, ins[j], insz[j]) ||
        overlap(workspace, need, ins[j], insz[j]))
      return DFLASH2_EINVAL;
  if (overlap(accept_len, ob, next_tok, ob) || overlap(workspace, need, accept_len, ob) ||
      overlap(workspace, need, next_tok, ob))
    return DFLASH2_EINVAL;
  return status_of(launch_verify_rejection_staged(
      path_slot, path_tok, q, top_idx, z, temperature, u_acc, u_res, B, L, V, rows,
      static_cast<float*>(workspace), accept_len, next_tok, as_stream(stream)));
}

DFLASH2_API int dflash2_verify_greedy(const int32_t* path_tok, const int32_t* target, int B, int L,
                                      int32_t* accept_len, int32_t* next_tok, void* stream) {
  if (B < 0 || L < 1) return DFLASH2_EINVAL;
  if (B == 0) return DFLASH2_OK;
  if (!path_tok || !target || !accept_len) return DFLASH2_EINVAL;
  if (!aligned4(path_tok) || !aligned4(target) || !aligned4(accept_len) ||
      (next_tok && !aligned4(next_tok)))
    return DFLASH2_EINVAL;
  const size_t pb = (size_t)B * L * 4, tb = (size_t)B * (L + 1) * 4, ob = (size_t)B * 4;
  if (overlap(accept_len, ob, path_tok, pb) || overlap(accept_len, ob, target, tb) ||
      overlap(next_tok, ob, path_tok, pb) || overlap(next_tok, ob, target, tb) ||
      overlap(accept_len, ob, next_tok, ob))
    return DFLASH2_EINVAL;
  return status_of(
      launch_verify_greedy(path_tok, target, B, L, accept_len, next_tok, as_stream(stream)));
}

DFLASH2_API int dflash2_pair_select_verify(
    const float* top_val, const int32_t* top_idx, const int32_t* anchor_tok, const void* U,
    const void* Vf, const float* gate, const int32_t* target, int B, int L, int V, int r,
    int dtype, int mode, float* S0, float* S, int32_t* path_slot, int32_t* path_tok,
    float* path_score, int32_t* accept_len, int32_t* next_tok, void* stream) {
  if (!valid_dtype(dtype) || B < 0 || L < 1 || L > DFLASH2_MAX_L || V < kTopK || r < 1 ||
      r > DFLASH2_MAX_RANK)
    return DFLASH2_EINVAL;
  if (mode != DFLASH2_PATH_VITERBI && mode != DFLASH2_PATH_GREEDY) return DFLASH2_EINVAL;
  if (B == 0) return DFLASH2_OK;
  if (!top_val || !top_idx || !U || !Vf || !target || !path_slot || !path_score || !accept_len)
    return DFLASH2_EINVAL;
  if ((long long)V * r > (1LL << 40) || (long long)B * L * kTopK > kInt32Max)
    return DFLASH2_EINVAL;
  const void* a4[] = {top_val, top_idx, anchor_tok, gate,     target,     S0,
                      S,       path_slot, path_tok, path_score, accept_len, next_tok};
  for (const void* p : a4)
    if (p && !aligned4(p)) return DFLASH2_EINVAL;
  const size_t es = esize(dtype);
  if (dtype == DFLASH2_BF16 ? ((reinterpret_cast<uintptr_t>(U) | reinterpret_cast<uintptr_t>(Vf)) & 1)
                            : (!aligned4(U) || !aligned4(Vf)))
    return DFLASH2_EINVAL;
  const size_t tb = (size_t)B * L * kTopK * 4;
  const size_t pb = (size_t)B * L * 4;
  const size_t ob = (size_t)B * 4;
  const void* ins[] = {top_val, top_idx, U, Vf, anchor_tok, gate, target};
  const size_t insz[] = {tb, tb, (size_t)V * r * es, (size_t)V * r * es, ob,
                         (size_t)B * L * r * 4, (size_t)B * (L + 1) * 4};
  const void* outs[] = {S0, L > 1 ? S : nullptr, path_slot, path_tok, path_score, accept_len,
                        next_tok};
  const size_t outsz[] = {(size_t)B * kTopK * 4, (size_t)B * (L - 1) * kTopK * kTopK * 4, pb, pb,
                          ob, ob, ob};
  for (int o = 0; o < 7; ++o) {
    if (!outs[o]) continue;
    for (int k = 0; k < 7; ++k)
      if (overlap(outs[o], outsz[o], ins[k], insz[k])) return DFLASH2_EINVAL;
    for (int k = o + 1; k < 7; ++k)
      if (outs[k] && overlap(outs[o], outsz[o], outs[k], outsz[k])) return DFLASH2_EINVAL;
  }
  return status_of(launch_pair_walk_verify(
      top_val, top_idx, anchor_tok, U, Vf, gate, target, B, L, V, r, dtype,
      mode == DFLASH2_PATH_GREEDY, S0, L > 1 ? S : nullptr, path_slot, path_tok, path_score,
      accept_len, next_tok, as_stream(stream)));
}

static int pair_sample(const float* top_val, const int32_t* top_idx, const int32_t* anchor_tok,
                       const void* U, const void* Vf, const float* gate, const float* u,
                       float temperature, int B, int L, int V, int r, int dtype, int mode,
                       float* S0, float* S, int32_t* path_slot, int32_t* path_tok, float* q,
                       void* stream) {
  if (!valid_dtype(dtype) || B < 0 || L < 1 || L > DFLASH2_MAX_L || V < kTopK || r < 1 ||
      r > DFLASH2_MAX_RANK || !valid_temperature(temperature) || !valid_sample_mode(mode))
    return DFLASH2_EINVAL;
  if (B == 0) return DFLASH2_OK;
  if (!top_val || !top_idx || !U || !Vf || !u || !path_slot || !q) return DFLASH2_EINVAL;
  if ((long long)V * r > (1LL << 40) || (long long)B * L * kTopK > kInt32Max)
    return DFLASH2_EINVAL;
  const void* a4[] = {top_val, top_idx, anchor_tok, gate, u, S0, S, path_slot, path_tok, q};
  for (const void* p : a4)
    if (p && !aligned4(p)) return DFLASH2_EINVAL;
  const size_t es = esize(dtype);
  if (dtype == DFLASH2_BF16 ? ((reinterpret_cast<uintptr_t>(U) | reinterpret_cast<uintptr_t>(Vf)) & 1)
                            : (!aligned4(U) || !aligned4(Vf)))
    return DFLASH2_EINVAL;
  const size_t tb = (size_t)B * L * kTopK * 4;
  const size_t pb = (size_t)B * L * 4;
  const void* ins[] = {top_val, top_idx, U, Vf, anchor_tok, gate, u};
  const size_t insz[] = {tb, tb, (size_t)V * r * es, (size_t)V * r * es, (size_t)B * 4,
                         (size_t)B * L * r * 4, pb};
  const void* outs[] = {S0, L > 1 ? S : nullptr, path_slot, path_tok, q};
  const size_t outsz[] = {(size_t)B * kTopK * 4, (size_t)B * (L - 1) * kTopK * kTopK * 4, pb, pb,
                          tb};
  for (int o = 0; o < 5; ++o) {
    if (!outs[o]) continue;
    for (int k = 0; k < 7; ++k)
      if (overlap(outs[o], outsz[o], ins[k], insz[k])) return DFLASH2_EINVAL;
    for (int k = o + 1; k < 5; ++k)
      if (outs[k] && overlap(outs[o], outsz[o], outs[k], outsz[k])) return DFLASH2_EINVAL;
  }
  return status_of(launch_pair_sample(top_val, top_idx, anchor_tok, U, Vf, gate, u, temperature,
                                      B, L, V, r, dtype, mode == DFLASH2_SAMPLE_PATH, S0,
                                      L > 1 ? S : nullptr, path_slot, path_tok, q,
                                      as_stream(stream)));
}

DFLASH2_API int dflash2_pair_sample(const float* top_val, const int32_t* top_idx,
                                    const int32_t* anchor_tok, const void* U, const void* Vf,
                                    const float* gate, const float* u, float temperature, int B,
                                    int L, int V, int r, int dtype, float* S0, float* S,
                                    int32_t* path_slot, int32_t* path_tok, float* q,
                                    void* stream) {
  return pair_sample(top_val, top_idx, anchor_tok, U, Vf, gate, u, temperature, B, L, V, r, dtype,
                     DFLASH2_SAMPLE_CHAIN, S0, S, path_slot, path_tok, q, stream);
}

DFLASH2_API int dflash2_pair_sample_mode(const float* top_val, const int32_t* top_idx,
                                         const int32_t* anchor_tok, const void* U,
                                         const void* Vf, const float* gate, const float* u,
                                         float temperature, int B, int L, int V, int r,
                                         int dtype, int mode, float* S0, float* S,
                                         int32_t* path_slot, int32_t* path_tok, float* q,
                                         void* stream) {
  return pair_sample(top_val, top_idx, anchor_tok, U, Vf, gate, u, temperature, B, L, V, r, dtype,
                     mode, S0, S, path_slot, path_tok, q, stream);
}

// ---------------------------------------------------------------- attainable-peak probe
DFLASH2_API size_t dflash2_probe_mfma_operand_bytes(int workgroups) {
  if (workgroups < 1 || workgroups > (1 << 20)) return 0;
  return probe_mfma_operand_bytes(workgroups);
}

DFLASH2_API int dflash2_probe_mfma(const void* operands, int workgroups, int iters, float* out,
                                   void* stream) {
  if (workgroups < 1 || workgroups > (1 << 20) || iters < 1) return DFLASH2_EINVAL;
  if (!operands || !out || !aligned16(operands) || !aligned4(out)) return DFLASH2_EINVAL;
  if (overlap(out, (size_t)workgroups * 512 * 4, operands,
              probe_mfma_operand_bytes(workgroups)))
    return DFLASH2_EINVAL;
  return status_of(launch_probe_mfma(operands, workgroups, iters, out, as_stream(stream)));
}

// ---------------------------------------------------------------- allocation-free logits + top-16
// dflash2_logits_topk for callers that cannot allocate: the tile maxima
// between the GEMM and the top-16 live in this fixed device array (each GPU
// the library runs on holds its own copy until the process ends).  Host
// code never passes the array's name to a kernel: its device address on the
// current device is looked up once per device and kept.
static __device__ __align__(256) unsigned char scratch[DFLASH2_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call made with that device current).
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DFLASH2_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DFLASH2_EHIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return DFLASH2_OK;
}
}  // namespace

DFLASH2_API int dflash2_logits_topk_noalloc(const void* h, const void* W, float* logits,
                                            float* top_val, int32_t* top_idx, int M, int H,
                                            int V, int K, int dtype, void* stream) {
  if (K != kTopK) return DFLASH2_EINVAL;
  int st = check_lmhead(h, W, M, H, V, dtype);
  if (st != DFLASH2_OK) return st;
  if (M == 0) return DFLASH2_OK;
  st = check_topk_out(top_val, top_idx, M);
  if (st != DFLASH2_OK) return st;
  if (!logits || !aligned16(logits)) return DFLASH2_EINVAL;
  if (tilemax_bytes(M, V) > (size_t)DFLASH2_NOALLOC_SCRATCH_BYTES) return DFLASH2_ESCRATCH;
  const size_t zb = (size_t)M * V * sizeof(float);
  const size_t ob = (size_t)M * kTopK * 4;
  const size_t es = esize(dtype);
  const size_t wb = w_bytes(V, H, dtype);
  if (overlap(logits, zb, h, (size_t)M * H * es) || overlap(logits, zb, W, wb) ||
      overlap(top_val, ob, logits, zb) || overlap(top_idx, ob, logits, zb) ||
      overlap(top_val, ob, top_idx, ob))
    return DFLASH2_EINVAL;
  void* sp = nullptr;
  st = scratch_on_current_device(&sp);
  if (st != DFLASH2_OK) return st;
  float* tmax = static_cast<float*>(sp);
  hipStream_t s = as_stream(stream);
  hipError_t e = launch_lmhead(h, W, logits, tmax, M, H, V, dtype, s);
  if (e != hipSuccess) return DFLASH2_EHIP;
  return status_of(launch_topk16_tilemax(logits, tmax, top_val, top_idx, M, V, s));
}
