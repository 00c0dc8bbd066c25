// Host-side launchers behind the C ABI.  Arguments reaching these functions
// have already been validated by abi.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sprint {

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---- key norm + composite score
// K is [n_layers, total_L, Hkv, D].  per_layer = 0: I is the mean over
// layers of each layer's mean-normalised key norm (ibar, score [total_L]);
// per_layer = 1: each layer's own I and s (ibar, score [n_layers, total_L]).
size_t score_ws_bytes(int64_t total_L, int nseq, int n_layers);
hipError_t launch_score(const void* K, int n_layers, int per_layer, const float* conf,
                        const int32_t* cu_len, int nseq, int64_t total_L, int Hkv, int D,
                        int dtype, float alpha, float* ibar, float* score, void* ws,
                        hipStream_t st);

// ---- per-modality top-k + compaction
// per_layer = 0: one kept set (from score [total_L]) compacts every layer's
// cache; per_layer = 1: layer l selects from score[l] and writes kept_idx[l]
// (n_sets = n_layers thresholds and chunk counts in the workspace).
size_t prune_ws_bytes(int64_t total_L, int nseq, int n_sets);
hipError_t launch_prune(const float* score, const uint8_t* modality, const int32_t* cu_len,
                        const int32_t* keep, const int32_t* cu_kept, int nseq, int64_t total_L,
                        int64_t total_kept, const void* K, const void* V, int n_layers,
                        int per_layer, int Hkv, int D, int dtype, void* K_out, void* V_out,
                        int32_t* kept_idx, void* ws, hipStream_t st);

// ---- block attention (split-KV + combine)
struct AttnPlan {
  int kps;         // keys per split (the last split of a sequence runs to its end)
  int n_splits;    // splits per (sequence, KV head)
  int rows;        // query rows per KV head = (Hq/Hkv) * Lq
  size_t ws_bytes;
};
AttnPlan attend_plan(int nseq, int Lq, int Hq, int Hkv, int D, int max_kv, int has_block,
                     int dtype);
// block_attend_noalloc: its partials live in a fixed device array of this
// many bytes; attend_scratch(device) is that array's address on the current
// device (device must be current), or null when it cannot be found.
constexpr size_t kAttendScratchBytes = size_t(16) << 20;
void* attend_scratch(int device);
hipError_t launch_attend(const void* Q, int nseq, int Lq, int Hq, const void* Kp, const void* Vp,
                         const int32_t* cu_kv, int64_t total_kv, const void* Kb, const void* Vb,
                         int Hkv, int D, float scale, int dtype, void* O, const AttnPlan& plan,
                         void* ws, hipStream_t st);

// ---- LM-head confidence (fused GEMM + streaming max / log-sum-exp, then merge)
size_t lmhead_ws_bytes(int64_t M, int H, int V, int dtype);
// The LM head of a denoising step fused with its unmasking step (M = nseq*Lq
// <= 64 on the register-ring path; other shapes run the two launches in
// turn).  Workspace: lmhead_ws_bytes(M, ...) then nseq arrival counters.
size_t lmhead_unmask_ws_bytes(int nseq, int Lq, int H, int V, int dtype);
hipError_t launch_lmhead_unmask(const void* X, int nseq, int Lq, int H, const void* W, int V,
                                int dtype, float* conf, int32_t* argmax, float tau,
                                int steps_left, uint8_t* masked, int32_t* tokens,
                                int32_t* n_accepted, void* ws, hipStream_t st);
hipError_t launch_lmhead(const void* X, int64_t M, int H, const void* W, int V, int dtype,
                         float* conf, int32_t* argmax, float* lse, void* ws, hipStream_t st);

// ---- unmask selection
hipError_t launch_unmask(const float* conf, const int32_t* argmax, int nseq, int Lq, float tau,
                         int steps_left, uint8_t* masked, int32_t* tokens, int32_t* n_accepted,
                         hipStream_t st);

// ---- prefix growth between blocks
hipError_t launch_append_rows(const void* old, const int32_t* cu_old, int nseq, int64_t total_old,
                              const void* blk, int n_blk, int64_t row_bytes, void* out,
                              int32_t* cu_out, hipStream_t st);

// ---- MoE FFN on synthetic weights
size_t moe_ws_bytes(int M, int H, int E, int top_k, int I);
bool moe_shape_supported(int H, int I, int E, int top_k, int M, int dtype);
hipError_t launch_moe(const void* x, int M, int H, const void* wr, const float* bias, int E,
                      int top_k, float scale, const void* wg, const void* wu, const void* wd,
                      int I, int dtype, const void* residual, void* y, int32_t* ids,
                      float* gates, void* ws, hipStream_t st);

}  // namespace sprint
