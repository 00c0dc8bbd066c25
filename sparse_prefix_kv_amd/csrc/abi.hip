// C ABI of libsprint.so (declared in include/sprint.h): host-side argument
// validation, workspace queries and dispatch to the kernel launchers.
// Every check runs before the first HIP call, so a rejected call touches no
// device state.
#include <math.h>
#include <stdint.h>

#include "../../include/sprint.h"
#include "sprint_internal.hpp"

using namespace sprint;

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool dev16(const void* p) { return p != nullptr && aligned(p, 16); }
bool dev4(const void* p) { return p != nullptr && aligned(p, 4); }
bool dtype_ok(int32_t dt) { return dt == SPRINT_F32 || dt == SPRINT_BF16; }
bool head_dim_ok(int32_t D) { return D == 64 || D == 128; }
// a * b * c < limit for a, b, c >= 0 and limit >= 1, without forming the
// product (which can overflow int64 for absurd sizes).
bool product_below(int64_t a, int64_t b, int64_t c, int64_t limit) {
  if (a == 0 || b == 0 || c == 0) return true;
  return a <= ((limit - 1) / c) / b;
}
// Arrays that kernels address through 32-bit buffer offsets stay below 2 GiB.
bool under_2gib(int64_t rows, int64_t row_bytes) {
  return product_below(rows, 1, row_bytes, static_cast<int64_t>(1) << 31);
}
// Arrays addressed through 64-bit offsets: a key row of at most 1 MiB (the
// kernels count a row's 16-byte vectors in 32 bits) and a whole stack under
// 2^48 bytes, the GPU's virtual address space, so no offset overflows.
constexpr int64_t kMaxRowBytes = int64_t(1) << 20;
constexpr int64_t kMaxArrayBytes = int64_t(1) << 48;
// Vocabulary and sequence-count limits that keep tile and grid counts in 32 bits.
constexpr int32_t kMaxVocab = (1 << 30) - 1;
constexpr int32_t kMaxSeqs = 1 << 24;
int64_t kv_row_bytes(int32_t Hkv, int32_t D, int32_t dtype) {
  return static_cast<int64_t>(Hkv) * D * (dtype == SPRINT_BF16 ? 2 : 4);
}
int status_of(hipError_t e) { return e == hipSuccess ? SPRINT_OK : SPRINT_EHIP; }
hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return SPRINT_OK;
  if (ws_bytes < need) return SPRINT_EWORKSPACE;
  if (!dev16(ws)) return SPRINT_EINVAL;
  return SPRINT_OK;
}

}  // namespace

extern "C" {

const char* sprint_strerror(int status) {
  switch (status) {
    case SPRINT_OK: return "ok";
    case SPRINT_EINVAL: return "invalid argument";
    case SPRINT_EUNSUPPORTED: return "unsupported shape or dtype";
    case SPRINT_EWORKSPACE: return "workspace too small";
    case SPRINT_EHIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int sprint_version(void) { return 100; }

int64_t sprint_keep_count(double r, int64_t n) {
  if (n <= 0 || !(r == r)) return 0;
  const double k = floor(r * static_cast<double>(n));
  if (k <= 0.0) return 0;
  if (k >= static_cast<double>(n)) return n;
  return static_cast<int64_t>(k);
}

int sprint_plan_keep(const int64_t* n_text, const int64_t* n_img, int32_t nseq, double r_text,
                     double r_img, int32_t* keep, int32_t* cu_kept, int64_t* total_kept) {
  if (!n_text || !n_img || !keep || !cu_kept || !total_kept || nseq < 1) return SPRINT_EINVAL;
  int64_t acc = 0;
  for (int32_t s = 0; s < nseq; ++s) {
    if (n_text[s] < 0 || n_img[s] < 0) return SPRINT_EINVAL;
    if (n_text[s] > INT32_MAX || n_img[s] > INT32_MAX - n_text[s]) return SPRINT_EINVAL;
  }
  cu_kept[0] = 0;
  for (int32_t s = 0; s < nseq; ++s) {
    const int64_t kt = sprint_keep_count(r_text, n_text[s]);
    const int64_t ki = sprint_keep_count(r_img, n_img[s]);
    keep[2 * s] = static_cast<int32_t>(kt);
    keep[2 * s + 1] = static_cast<int32_t>(ki);
    acc += kt + ki;
    if (acc > INT32_MAX) return SPRINT_EINVAL;
    cu_kept[s + 1] = static_cast<int32_t>(acc);
  }
  *total_kept = acc;
  return SPRINT_OK;
}

// ---------------------------------------------------------------- LM head
size_t lmhead_confidence_ws(int64_t M, int32_t H, int32_t V, int32_t dtype) {
  if (M < 1 || M > INT32_MAX || V < 1 || V > kMaxVocab || H < 1) return 0;
  return lmhead_ws_bytes(M, H, V, dtype);
}

int lmhead_confidence(const void* hidden, int64_t M, int32_t H, const void* W, int32_t V,
                      int32_t dtype, float* conf, int32_t* argmax, float* lse, void* ws,
                      size_t ws_bytes, void* stream) {
  if (!dtype_ok(dtype)) return SPRINT_EINVAL;
  if (M < 1 || V < 1 || H < 1 || M > INT32_MAX) return SPRINT_EINVAL;
  if (!dev16(hidden) || !dev16(W) || !dev4(conf) || !dev4(argmax)) return SPRINT_EINVAL;
  if (lse != nullptr && !aligned(lse, 4)) return SPRINT_EINVAL;
  if (H % 64 != 0 || H > 65536 || V > kMaxVocab) return SPRINT_EUNSUPPORTED;
  const int st = check_ws(ws, ws_bytes, lmhead_ws_bytes(M, H, V, dtype));
  if (st != SPRINT_OK) return st;
  return status_of(launch_lmhead(hidden, M, H, W, V, dtype, conf, argmax, lse, ws,
                                 as_stream(stream)));
}

size_t lmhead_confidence_unmask_ws(int32_t nseq, int32_t Lq, int32_t H, int32_t V,
                                   int32_t dtype) {
  if (nseq < 1 || nseq > kMaxSeqs || Lq < 1 || Lq > 64 || V < 1 || V > kMaxVocab || H < 1)
    return 0;
  return lmhead_unmask_ws_bytes(nseq, Lq, H, V, dtype);
}

int lmhead_confidence_unmask(const void* hidden, int32_t nseq, int32_t Lq, int32_t H,
                             const void* W, int32_t V, int32_t dtype, float* conf,
                             int32_t* argmax, float tau, int32_t steps_left, uint8_t* masked,
                             int32_t* tokens, int32_t* n_accepted, void* ws, size_t ws_bytes,
                             void* stream) {
  if (!dtype_ok(dtype)) return SPRINT_EINVAL;
  if (nseq < 1 || Lq < 1 || V < 1 || H < 1 || tau != tau) return SPRINT_EINVAL;
  if (Lq > 64 || nseq > kMaxSeqs) return SPRINT_EUNSUPPORTED;
  if (!dev16(hidden) || !dev16(W) || !dev4(conf) || !dev4(argmax) || masked == nullptr ||
      !dev4(tokens) || !dev4(n_accepted))
    return SPRINT_EINVAL;
  if (H % 64 != 0 || H > 65536 || V > kMaxVocab) return SPRINT_EUNSUPPORTED;
  const int st = check_ws(ws, ws_bytes, lmhead_unmask_ws_bytes(nseq, Lq, H, V, dtype));
  if (st != SPRINT_OK) return st;
  return status_of(launch_lmhead_unmask(hidden, nseq, Lq, H, W, V, dtype, conf, argmax, tau,
                                        steps_left, masked, tokens, n_accepted, ws,
                                        as_stream(stream)));
}

// ---------------------------------------------------------------- score
static int score_impl(const void* K, int32_t n_layers, int per_layer, const float* conf,
                      const int32_t* cu_len, int32_t nseq, int64_t total_L, int32_t Hkv,
                      int32_t D, int32_t dtype, float alpha, float* ibar, float* score, void* ws,
                      size_t ws_bytes, void* stream) {
  if (!dtype_ok(dtype) || nseq < 1 || total_L < 0 || total_L > INT32_MAX || Hkv < 1)
    return SPRINT_EINVAL;
  if (n_layers < 1 || n_layers > 65535) return SPRINT_EINVAL;
  if (!dev4(cu_len) || !isfinite(alpha)) return SPRINT_EINVAL;
  if (!head_dim_ok(D) || nseq > kMaxSeqs) return SPRINT_EUNSUPPORTED;
  const int64_t row = kv_row_bytes(Hkv, D, dtype);
  if (row > kMaxRowBytes || !product_below(n_layers, total_L, row, kMaxArrayBytes))
    return SPRINT_EUNSUPPORTED;
  if (total_L > 0 && (!dev16(K) || !dev4(conf) || !dev4(ibar) || !dev4(score)))
    return SPRINT_EINVAL;
  const int st = check_ws(ws, ws_bytes, score_ws_bytes(total_L, nseq, n_layers));
  if (st != SPRINT_OK) return st;
  return status_of(launch_score(K, n_layers, per_layer, conf, cu_len, nseq, total_L, Hkv, D,
                                dtype, alpha, ibar, score, ws, as_stream(stream)));
}

size_t sprint_score_ws(int64_t total_L, int32_t nseq) {
  if (total_L < 0 || total_L > INT32_MAX || nseq < 1 || nseq > kMaxSeqs) return 0;
  return score_ws_bytes(total_L, nseq, 1);
}

int sprint_score(const void* K, const float* conf, const int32_t* cu_len, int32_t nseq,
                 int64_t total_L, int32_t Hkv, int32_t D, int32_t dtype, float alpha, float* ibar,
                 float* score, void* ws, size_t ws_bytes, void* stream) {
  return score_impl(K, 1, 0, conf, cu_len, nseq, total_L, Hkv, D, dtype, alpha, ibar, score, ws,
                    ws_bytes, stream);
}

size_t sprint_score_layers_ws(int64_t total_L, int32_t nseq, int32_t n_layers) {
  if (total_L < 0 || total_L > INT32_MAX || nseq < 1 || nseq > kMaxSeqs || n_layers < 1 ||
      n_layers > 65535)
    return 0;
  return score_ws_bytes(total_L, nseq, n_layers);
}

int sprint_score_layers(const void* K, int32_t n_layers, const float* conf, const int32_t* cu_len,
                        int32_t nseq, int64_t total_L, int32_t Hkv, int32_t D, int32_t dtype,
                        float alpha, float* ibar, float* score, void* ws, size_t ws_bytes,
                        void* stream) {
  return score_impl(K, n_layers, 0, conf, cu_len, nseq, total_L, Hkv, D, dtype, alpha, ibar,
                    score, ws, ws_bytes, stream);
}

int sprint_score_per_layer(const void* K, int32_t n_layers, const float* conf,
                           const int32_t* cu_len, int32_t nseq, int64_t total_L, int32_t Hkv,
                           int32_t D, int32_t dtype, float alpha, float* ibar, float* score,
                           void* ws, size_t ws_bytes, void* stream) {
  return score_impl(K, n_layers, 1, conf, cu_len, nseq, total_L, Hkv, D, dtype, alpha, ibar,
                    score, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------- prune
static int prune_impl(const float* score, const uint8_t* modality, const int32_t* cu_len,
                      const int32_t* keep, const int32_t* cu_kept, int32_t nseq, int64_t total_L,
                      int64_t total_kept, const void* K, const void* V, int32_t n_layers,
                      int per_layer, int32_t Hkv, int32_t D, int32_t dtype, void* K_out,
                      void* V_out, int32_t* kept_idx, void* ws, size_t ws_bytes, void* stream) {
  if (!dtype_ok(dtype) || nseq < 1 || total_L < 0 || total_L > INT32_MAX || Hkv < 1)
    return SPRINT_EINVAL;
  if (n_layers < 1 || n_layers > 65535) return SPRINT_EINVAL;
  if (total_kept < 0 || total_kept > total_L) return SPRINT_EINVAL;
  if (!dev4(cu_len) || !dev4(keep) || !dev4(cu_kept)) return SPRINT_EINVAL;
  if (!head_dim_ok(D) || nseq > kMaxSeqs) return SPRINT_EUNSUPPORTED;
  const int64_t row = kv_row_bytes(Hkv, D, dtype);
  if (row > kMaxRowBytes || !product_below(n_layers, total_L, row, kMaxArrayBytes))
    return SPRINT_EUNSUPPORTED;
  // the pruned cache of a layer is written through 32-bit buffer offsets
  if (!under_2gib(total_kept, row)) return SPRINT_EUNSUPPORTED;
  if (total_L > 0 && (!dev4(score) || modality == nullptr || !dev16(K) || !dev16(V)))
    return SPRINT_EINVAL;
  if (total_kept > 0 && (!dev16(K_out) || !dev16(V_out) || !dev4(kept_idx))) return SPRINT_EINVAL;
  const int st = check_ws(ws, ws_bytes, prune_ws_bytes(total_L, nseq, per_layer ? n_layers : 1));
  if (st != SPRINT_OK) return st;
  return status_of(launch_prune(score, modality, cu_len, keep, cu_kept, nseq, total_L, total_kept,
                                K, V, n_layers, per_layer, Hkv, D, dtype, K_out, V_out, kept_idx,
                                ws, as_stream(stream)));
}

size_t sprint_prune_kv_ws(int64_t total_L, int32_t nseq) {
  if (total_L < 0 || total_L > INT32_MAX || nseq < 1 || nseq > kMaxSeqs) return 0;
  return prune_ws_bytes(total_L, nseq, 1);
}

int sprint_prune_kv(const float* score, const uint8_t* modality, const int32_t* cu_len,
                    const int32_t* keep, const int32_t* cu_kept, int32_t nseq, int64_t total_L,
                    int64_t total_kept, const void* K, const void* V, int32_t Hkv, int32_t D,
                    int32_t dtype, void* K_out, void* V_out, int32_t* kept_idx, void* ws,
                    size_t ws_bytes, void* stream) {
  return prune_impl(score, modality, cu_len, keep, cu_kept, nseq, total_L, total_kept, K, V, 1, 0,
                    Hkv, D, dtype, K_out, V_out, kept_idx, ws, ws_bytes, stream);
}

int sprint_prune_kv_layers(const float* score, const uint8_t* modality, const int32_t* cu_len,
                           const int32_t* keep, const int32_t* cu_kept, int32_t nseq,
                           int64_t total_L, int64_t total_kept, const void* K, const void* V,
                           int32_t n_layers, int32_t Hkv, int32_t D, int32_t dtype, void* K_out,
                           void* V_out, int32_t* kept_idx, void* ws, size_t ws_bytes,
                           void* stream) {
  return prune_impl(score, modality, cu_len, keep, cu_kept, nseq, total_L, total_kept, K, V,
                    n_layers, 0, Hkv, D, dtype, K_out, V_out, kept_idx, ws, ws_bytes, stream);
}

size_t sprint_prune_kv_per_layer_ws(int64_t total_L, int32_t nseq, int32_t n_layers) {
  if (total_L < 0 || total_L > INT32_MAX || nseq < 1 || nseq > kMaxSeqs || n_layers < 1 ||
      n_layers > 65535)
    return 0;
  return prune_ws_bytes(total_L, nseq, n_layers);
}

int sprint_prune_kv_per_layer(const float* score, const uint8_t* modality, const int32_t* cu_len,
                              const int32_t* keep, const int32_t* cu_kept, int32_t nseq,
                              int64_t total_L, int64_t total_kept, const void* K, const void* V,
                              int32_t n_layers, int32_t Hkv, int32_t D, int32_t dtype,
                              void* K_out, void* V_out, int32_t* kept_idx, void* ws,
                              size_t ws_bytes, void* stream) {
  return prune_impl(score, modality, cu_len, keep, cu_kept, nseq, total_L, total_kept, K, V,
                    n_layers, 1, Hkv, D, dtype, K_out, V_out, kept_idx, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------- attention
static int attend_shape_status(int32_t nseq, int32_t Lq, int32_t Hq, int32_t Hkv, int32_t D,
                               int32_t max_kv) {
  if (nseq < 1 || Lq < 1 || Hq < 1 || Hkv < 1 || max_kv < 0) return SPRINT_EINVAL;
  if (Hq % Hkv != 0) return SPRINT_EINVAL;
  if (!head_dim_ok(D) || Lq > 64 || static_cast<int64_t>(Hq / Hkv) * Lq > 256 || nseq > kMaxSeqs)
    return SPRINT_EUNSUPPORTED;
  // the block's rows stay under 2 GiB even in bf16 (checked per dtype later)
  if (!under_2gib(static_cast<int64_t>(nseq) * Lq, kv_row_bytes(Hkv, D, SPRINT_BF16)))
    return SPRINT_EUNSUPPORTED;
  return SPRINT_OK;
}

size_t block_attend_ws(int32_t nseq, int32_t Lq, int32_t Hq, int32_t Hkv, int32_t D,
                       int32_t max_kv, int32_t has_block) {
  if (attend_shape_status(nseq, Lq, Hq, Hkv, D, max_kv) != SPRINT_OK) return 0;
  // fp32 partials are the larger case; a bf16 call needs no more than this
  return attend_plan(nseq, Lq, Hq, Hkv, D, max_kv, has_block, SPRINT_F32).ws_bytes;
}

static int attend_check(const void* Q, int32_t nseq, int32_t Lq, int32_t Hq, const void* Kp,
                        const void* Vp, const int32_t* cu_kv, int64_t total_kv, int32_t max_kv,
                        const void* Kb, const void* Vb, int32_t Hkv, int32_t D, float scale,
                        int32_t dtype, void* O) {
  if (!dtype_ok(dtype)) return SPRINT_EINVAL;
  const int ss = attend_shape_status(nseq, Lq, Hq, Hkv, D, max_kv);
  if (ss != SPRINT_OK) return ss;
  if (total_kv < 0 || total_kv > INT32_MAX || !isfinite(scale) || !(scale > 0.f))
    return SPRINT_EINVAL;
  // K/V tiles are loaded through 32-bit buffer offsets
  const int64_t row = kv_row_bytes(Hkv, D, dtype);
  if (!under_2gib(total_kv, row) || !under_2gib(static_cast<int64_t>(nseq) * Lq, row))
    return SPRINT_EUNSUPPORTED;
  // one sequence's cache is all of [0, total_kv), which max_kv must cover
  if (nseq == 1 && total_kv > max_kv) return SPRINT_EINVAL;
  if (!dev16(Q) || !dev16(O) || !dev4(cu_kv)) return SPRINT_EINVAL;
  if ((Kb == nullptr) != (Vb == nullptr)) return SPRINT_EINVAL;
  if (Kb != nullptr && (!dev16(Kb) || !dev16(Vb))) return SPRINT_EINVAL;
  if (Kb == nullptr && max_kv < 1) return SPRINT_EINVAL;  // no keys at all
  if (total_kv > 0 && (!dev16(Kp) || !dev16(Vp))) return SPRINT_EINVAL;
  return SPRINT_OK;
}

int block_attend(const void* Q, int32_t nseq, int32_t Lq, int32_t Hq, const void* Kp,
                 const void* Vp, const int32_t* cu_kv, int64_t total_kv, int32_t max_kv,
                 const void* Kb, const void* Vb, int32_t Hkv, int32_t D, float scale,
                 int32_t dtype, void* O, void* ws, size_t ws_bytes, void* stream) {
  const int ck = attend_check(Q, nseq, Lq, Hq, Kp, Vp, cu_kv, total_kv, max_kv, Kb, Vb, Hkv, D,
                              scale, dtype, O);
  if (ck != SPRINT_OK) return ck;
  const AttnPlan plan = attend_plan(nseq, Lq, Hq, Hkv, D, max_kv, Kb != nullptr, dtype);
  const int st = check_ws(ws, ws_bytes, plan.ws_bytes);
  if (st != SPRINT_OK) return st;
  return status_of(launch_attend(Q, nseq, Lq, Hq, Kp, Vp, cu_kv, total_kv, Kb, Vb, Hkv, D, scale,
                                 dtype, O, plan, ws, as_stream(stream)));
}

int block_attend_noalloc(const void* Q, int32_t nseq, int32_t Lq, int32_t Hq, const void* Kp,
                         const void* Vp, const int32_t* cu_kv, int64_t total_kv, int32_t max_kv,
                         const void* Kb, const void* Vb, int32_t Hkv, int32_t D, float scale,
                         int32_t dtype, void* O, void* stream) {
  const int ck = attend_check(Q, nseq, Lq, Hq, Kp, Vp, cu_kv, total_kv, max_kv, Kb, Vb, Hkv, D,
                              scale, dtype, O);
  if (ck != SPRINT_OK) return ck;
  const AttnPlan plan = attend_plan(nseq, Lq, Hq, Hkv, D, max_kv, Kb != nullptr, dtype);
  if (plan.ws_bytes > kAttendScratchBytes) return SPRINT_EWORKSPACE;
  void* ws = nullptr;
  if (plan.ws_bytes > 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SPRINT_EHIP;
    ws = attend_scratch(dev);
    if (ws == nullptr) return SPRINT_EHIP;
  }
  return status_of(launch_attend(Q, nseq, Lq, Hq, Kp, Vp, cu_kv, total_kv, Kb, Vb, Hkv, D, scale,
                                 dtype, O, plan, ws, as_stream(stream)));
}

// ---------------------------------------------------------------- unmask
int unmask_select(const float* conf, const int32_t* argmax, int32_t nseq, int32_t Lq, float tau,
                  int32_t steps_left, uint8_t* masked, int32_t* tokens, int32_t* n_accepted,
                  void* stream) {
  if (nseq < 1 || Lq < 1 || tau != tau) return SPRINT_EINVAL;
  if (Lq > 64 || nseq > kMaxSeqs) return SPRINT_EUNSUPPORTED;
  if (!dev4(conf) || !dev4(argmax) || masked == nullptr || !dev4(tokens) || !dev4(n_accepted))
    return SPRINT_EINVAL;
  return status_of(launch_unmask(conf, argmax, nseq, Lq, tau, steps_left, masked, tokens,
                                 n_accepted, as_stream(stream)));
}

// ---------------------------------------------------------------- append
int sprint_append_rows(const void* old, const int32_t* cu_old, int32_t nseq, int64_t total_old,
                       const void* blk, int32_t n_blk, int64_t row_bytes, void* out,
                       int32_t* cu_out, void* stream) {
  if (nseq < 1 || n_blk < 0 || total_old < 0 || total_old > INT32_MAX || row_bytes < 1 ||
      row_bytes > (int64_t(1) << 31))
    return SPRINT_EINVAL;
  if (nseq > kMaxSeqs) return SPRINT_EUNSUPPORTED;
  if (!dev4(cu_old) || (cu_out != nullptr && (!aligned(cu_out, 4) || cu_out == cu_old)))
    return SPRINT_EINVAL;
  const int64_t total_rows = total_old + static_cast<int64_t>(nseq) * n_blk;
  if (total_rows > INT32_MAX) return SPRINT_EINVAL;
  if (total_old > 0 && old == nullptr) return SPRINT_EINVAL;
  if (n_blk > 0 && blk == nullptr) return SPRINT_EINVAL;
  if (total_rows > 0 && out == nullptr) return SPRINT_EINVAL;
  // out must not overlap either source
  const auto overlaps = [](const void* a, int64_t na, const void* b, int64_t nb) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return na > 0 && nb > 0 && pa < pb + static_cast<uintptr_t>(nb) &&
           pb < pa + static_cast<uintptr_t>(na);
  };
  const int64_t out_bytes = total_rows * row_bytes;
  if (overlaps(out, out_bytes, old, total_old * row_bytes) ||
      overlaps(out, out_bytes, blk, static_cast<int64_t>(nseq) * n_blk * row_bytes))
    return SPRINT_EINVAL;
  return status_of(launch_append_rows(old, cu_old, nseq, total_old, blk, n_blk, row_bytes, out,
                                      cu_out, as_stream(stream)));
}

// ---------------------------------------------------------------- MoE FFN
size_t moe_ffn_ws(int32_t M, int32_t H, int32_t n_experts, int32_t top_k, int32_t inter) {
  if (M < 1 || H < 1 || n_experts < 1 || top_k < 1 || inter < 1) return 0;
  if (!moe_shape_supported(H, inter, n_experts, top_k, M, SPRINT_BF16) &&
      !moe_shape_supported(H, inter, n_experts, top_k, M, SPRINT_F32))
    return 0;
  return moe_ws_bytes(M, H, n_experts, top_k, inter);
}

int moe_ffn(const void* x, int32_t M, int32_t H, const void* w_router, const float* bias,
            int32_t n_experts, int32_t top_k, float route_scale, const void* w_gate,
            const void* w_up, const void* w_down, int32_t inter, int32_t dtype,
            const void* residual, void* y, int32_t* expert_ids, float* gates, void* ws,
            size_t ws_bytes, void* stream) {
  if (!dtype_ok(dtype) || M < 1 || H < 1 || n_experts < 1 || top_k < 1 || inter < 1)
    return SPRINT_EINVAL;
  if (top_k > n_experts || !isfinite(route_scale)) return SPRINT_EINVAL;
  if (!dev16(x) || !dev16(w_router) || !dev4(bias) || !dev16(w_gate) || !dev16(w_up) ||
      !dev16(w_down) || !dev16(y) || !dev4(expert_ids) || !dev4(gates))
    return SPRINT_EINVAL;
  if (residual != nullptr && !dev16(residual)) return SPRINT_EINVAL;
  if (!moe_shape_supported(H, inter, n_experts, top_k, M, dtype)) return SPRINT_EUNSUPPORTED;
  const int st = check_ws(ws, ws_bytes, moe_ws_bytes(M, H, n_experts, top_k, inter));
  if (st != SPRINT_OK) return st;
  return status_of(launch_moe(x, M, H, w_router, bias, n_experts, top_k, route_scale, w_gate,
                              w_up, w_down, inter, dtype, residual, y, expert_ids, gates, ws,
                              as_stream(stream)));
}

}  // extern "C"
