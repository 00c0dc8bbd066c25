// Modality-aware prefix pruning and KV compaction (LLaDA2.0-Uni, SPRINT
// "Sparse Prefix Retention": keep the top-floor(r*n) positions by score within
// each modality, then build a contiguous pruned cache once per block).
//
// Ranking key of position p: (score desc, position asc).  The score is mapped
// to an order-preserving uint32, so "the k-th largest" is found exactly by an
// MSB-first radix select (4 passes of 8 bits) per (sequence, modality)
// segment.  The result is a threshold key T and a tie cut: a position is
// kept iff key > T, or key == T and p <= tie_cut (the first ties by position).
//
// Launches:
//   1. topk_threshold_kernel  one 1024-thread block per segment (the keys of
//                             a sequence of up to 32768 positions read from
//                             HBM once, into LDS);
//   2. chunk_count_kernel     kept count of every 64-position chunk;
//   3. compact_kernel         per chunk: prefix of earlier chunk counts in the
//                             sequence -> output slots; writes kept_idx and
//                             copies the K and V rows (16-byte vectors), of
//                             every layer (grid y) when one kept set serves
//                             several layers' caches.
// With a kept set per layer, all three run once per layer (grid y), each
// layer on its own scores, thresholds, counts and kept_idx row.
// The copy dominates: 2 x kept x row bytes read and written, HBM-bound.
#include <limits.h>

#include "sprint_device.hpp"
#include "sprint_internal.hpp"

namespace sprint {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kLdsKeys = 32768;    // a sequence's keys kept in LDS (128 KB)
constexpr int kChunk = 64;
constexpr int kCopyThreads = 256;

struct SegThresh {
  uint32_t key;
  int32_t tie_cut;
};

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 ranks equal to +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ bool is_kept(uint32_t key, int64_t p, const SegThresh& t) {
  return key > t.key || (key == t.key && p <= static_cast<int64_t>(t.tie_cut));
}

__device__ __forceinline__ void clamp_seq(const int32_t* cu, int s, int64_t total, int64_t& a,
                                          int64_t& e) {
  a = cu[s];
  e = cu[s + 1];
  a = a < 0 ? 0 : (a > total ? total : a);
  e = e < a ? a : (e > total ? total : e);
}

// Block-wide inclusive scan of one int per thread (1024 threads).
__device__ __forceinline__ int block_incl_scan(int v, int* s_wave, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kWaves = kSelThreads / 64;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  if (lane == 63) s_wave[wave] = v;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int x = s_wave[w];
    if (w < wave) base += x;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return v + base;
}

__global__ __launch_bounds__(kSelThreads) void topk_threshold_kernel(
    const float* __restrict__ score, const uint8_t* __restrict__ modality,
    const int32_t* __restrict__ cu_len, const int32_t* __restrict__ keep, int nseq,
    int64_t total_L, SegThresh* __restrict__ thr) {
  // grid y: the layer whose scores select its own set (one layer otherwise)
  score += static_cast<int64_t>(blockIdx.y) * total_L;
  thr += static_cast<int64_t>(blockIdx.y) * nseq * 2;
  const int seg = blockIdx.x;
  const int s = seg >> 1;
  const uint8_t mod = static_cast<uint8_t>(seg & 1);
  int64_t a, e;
  clamp_seq(cu_len, s, total_L, a, e);
  const int k = keep[seg];
  __shared__ int hist[256];
  __shared__ int s_wave[kSelThreads / 64];
  __shared__ int s_bucket, s_above, s_total, s_found, s_nkeys;
  __shared__ uint32_t s_keys[kLdsKeys];
  if (k <= 0) {
    if (threadIdx.x == 0) thr[seg] = SegThresh{0xFFFFFFFFu, -1};
    return;
  }
  uint32_t prefix = 0, pmask = 0;
  int krem = k;
  int ties = 0;
  // A sequence of up to kLdsKeys positions has its modality's keys read from
  // HBM once, during the first pass, into LDS (in any order: the histograms
  // only count); the later passes read them there.  Longer sequences read
  // the scores again in every pass.
  const bool in_lds = e - a <= kLdsKeys;
  if (threadIdx.x == 0) s_nkeys = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (threadIdx.x < 256) hist[threadIdx.x] = 0;
    __syncthreads();
    if (in_lds && pass > 0) {
      const int nk = s_nkeys;
      for (int i = threadIdx.x; i < nk; i += kSelThreads) {
        const uint32_t key = s_keys[i];
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
      }
    } else {
      // eight chunks of the sequence per round, all their loads in flight
      // before any is used
      const int lane = threadIdx.x & 63;
      constexpr int kU = 8;
      for (int64_t p0 = a; p0 < e; p0 += kU * kSelThreads) {
        uint8_t md[kU];
        float sc[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int64_t p = p0 + u * kSelThreads + threadIdx.x;
          md[u] = p < e ? modality[p] : static_cast<uint8_t>(mod ^ 1);
          sc[u] = p < e ? score[p] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const bool mine = md[u] == mod;
          const uint32_t key = mine ? order_key(sc[u]) : 0u;
          if (mine && (key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
          if (in_lds) {
            // one LDS slot reservation per wave
            const uint64_t bal = __ballot(mine);
            int slot0 = 0;
            if (lane == 0 && bal) slot0 = atomicAdd(&s_nkeys, __popcll(bal));
            slot0 = __shfl(slot0, 0, 64);
            if (mine) s_keys[slot0 + __popcll(bal & ((1ull << lane) - 1ull))] = key;
          }
        }
      }
    }
    __syncthreads();
    // Suffix sums over the 256 digits (threads 0..255 = waves 0..3).  Every
    // wave of the block reaches both barriers below.
    int v = 0, h = 0;
    if (threadIdx.x < 256) {
      const int lane = threadIdx.x & 63;
      h = hist[threadIdx.x];
      v = h;  // inclusive suffix within the wave (higher digits = higher lanes)
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_down(v, off, 64);
        if (lane + off < 64) v += o;
      }
      if (lane == 0) s_wave[threadIdx.x >> 6] = v;  // wave total
    }
    __syncthreads();
    if (threadIdx.x < 256) {
      const int t = threadIdx.x, wave = t >> 6;
      int higher = 0;
      for (int w = wave + 1; w < 4; ++w) higher += s_wave[w];
      const int incl = v + higher;        // elements with digit >= t
      const int excl = incl - h;          // elements with digit >  t
      if (pass == 0 && t == 0) s_total = incl;
      if (excl < krem && krem <= incl) {
        s_bucket = t;
        s_above = excl;
      }
    }
    __syncthreads();
    if (pass == 0 && k >= s_total) {
      if (threadIdx.x == 0) thr[seg] = SegThresh{0u, INT_MAX};
      return;
    }
    const int b = s_bucket;
    krem -= s_above;
    prefix |= static_cast<uint32_t>(b) << shift;
    pmask |= 255u << shift;
    ties = hist[b];
    __syncthreads();
  }
  // prefix is now the exact key of the k-th largest; keep the first `krem`
  // of the `ties` positions that carry it.
  if (krem >= ties) {
    if (threadIdx.x == 0) thr[seg] = SegThresh{prefix, INT_MAX};
    return;
  }
  if (threadIdx.x == 0) s_found = 0;
  __syncthreads();
  int base = 0;
  for (int64_t p0 = a; p0 < e; p0 += kSelThreads) {
    const int64_t p = p0 + threadIdx.x;
    const int f = (p < e && modality[p] == mod && order_key(score[p]) == prefix) ? 1 : 0;
    int tot;
    const int incl = block_incl_scan(f, s_wave, tot);
    if (f && base + incl == krem) {
      thr[seg] = SegThresh{prefix, static_cast<int32_t>(p)};
      s_found = 1;
    }
    base += tot;
    __syncthreads();
    if (s_found) break;
  }
}

__device__ __forceinline__ bool kept_at(const float* __restrict__ score,
                                        const uint8_t* __restrict__ modality,
                                        const SegThresh* __restrict__ thr, int s, int64_t p) {
  const uint8_t m = modality[p];
  const SegThresh t = thr[2 * s + (m ? 1 : 0)];
  return is_kept(order_key(score[p]), p, t);
}

// One wave per 64-position chunk.
__global__ __launch_bounds__(64) void chunk_count_kernel(const float* __restrict__ score,
                                                         const uint8_t* __restrict__ modality,
                                                         const int32_t* __restrict__ cu_len,
                                                         int nseq, int64_t total_L,
                                                         const SegThresh* __restrict__ thr,
                                                         int32_t* __restrict__ counts) {
  SeqChunk sc;
  if (!find_seq_chunk(cu_len, nseq, kChunk, total_L, blockIdx.x, sc)) return;
  // grid y: the layer (its scores, thresholds and counts; one layer otherwise)
  score += static_cast<int64_t>(blockIdx.y) * total_L;
  thr += static_cast<int64_t>(blockIdx.y) * nseq * 2;
  counts += static_cast<int64_t>(blockIdx.y) * gridDim.x;
  const int64_t p = sc.begin + static_cast<int64_t>(sc.c) * kChunk + threadIdx.x;
  const bool f = p < sc.begin + sc.len && kept_at(score, modality, thr, sc.seq, p);
  const uint64_t bal = __ballot(f);
  if (threadIdx.x == 0) counts[blockIdx.x] = static_cast<int32_t>(__popcll(bal));
}

__global__ __launch_bounds__(kCopyThreads) void compact_kernel(
    const float* __restrict__ score, const uint8_t* __restrict__ modality,
    const int32_t* __restrict__ cu_len, const int32_t* __restrict__ cu_kept, int nseq,
    int64_t total_L, int64_t total_kept, const SegThresh* __restrict__ thr,
    const int32_t* __restrict__ counts, const char* __restrict__ K, const char* __restrict__ V,
    int row_vecs, char* __restrict__ K_out, char* __restrict__ V_out,
    int32_t* __restrict__ kept_idx, int per_layer) {
  SeqChunk sc;
  if (!find_seq_chunk(cu_len, nseq, kChunk, total_L, blockIdx.x, sc)) return;
  // layer blockIdx.y: its caches.  One shared set: layer 0 writes kept_idx.
  // A set per layer: the layer's own scores, thresholds, counts and kept_idx.
  const int64_t layer = blockIdx.y;
  K += layer * total_L * row_vecs * 16;
  V += layer * total_L * row_vecs * 16;
  K_out += layer * total_kept * row_vecs * 16;
  V_out += layer * total_kept * row_vecs * 16;
  const bool writes_idx = per_layer || layer == 0;
  if (per_layer) {
    score += layer * total_L;
    thr += layer * nseq * 2;
    counts += layer * gridDim.x;
    kept_idx += layer * total_kept;
  }
  __shared__ int64_t s_pos[kChunk];
  __shared__ int64_t s_slot0, s_limit;
  __shared__ int s_nk;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int pre = 0;
    for (int i = lane; i < sc.c; i += 64) pre += counts[sc.first + i];
    pre = wave_sum_i(pre);
    const int64_t p = sc.begin + static_cast<int64_t>(sc.c) * kChunk + lane;
    const bool f = p < sc.begin + sc.len && kept_at(score, modality, thr, sc.seq, p);
    const uint64_t bal = __ballot(f);
    const int rank = __popcll(bal & ((1ull << lane) - 1ull));
    int64_t limit = cu_kept[sc.seq + 1];
    if (limit > total_kept) limit = total_kept;
    const int64_t slot0 = static_cast<int64_t>(cu_kept[sc.seq]) + pre;
    if (f) {
      s_pos[rank] = p;
      const int64_t slot = slot0 + rank;
      if (writes_idx && slot >= 0 && slot < limit) kept_idx[slot] = static_cast<int32_t>(p);
    }
    if (lane == 0) {
      s_nk = __popcll(bal);
      s_slot0 = slot0;
      s_limit = limit;
    }
  }
  __syncthreads();
  const int nk = s_nk;
  const int64_t slot0 = s_slot0, limit = s_limit;
  const int64_t row_bytes = static_cast<int64_t>(row_vecs) * 16;
  const int units = nk * row_vecs;
  // four 16-byte vectors of K and of V per thread in flight per round; the
  // source rows are read once (non-temporal), the pruned cache is written
  // with ordinary stores since the denoising steps read it next
  constexpr int kU = 4;
  for (int u0 = threadIdx.x; u0 < units; u0 += kU * kCopyThreads) {
    u32x4 kv[kU], vv[kU];
    int64_t dst[kU];
    bool ok[kU];
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      const int u = u0 + i * kCopyThreads;
      const int r = u / row_vecs, v = u - r * row_vecs;
      const int64_t slot = slot0 + r;
      ok[i] = u < units && slot >= 0 && slot < limit;
      const int64_t src = ok[i] ? s_pos[r] * row_bytes + v * 16 : 0;
      dst[i] = slot * row_bytes + v * 16;
      kv[i] = ok[i] ? ld16_nt(K + src) : u32x4{0u, 0u, 0u, 0u};
      vv[i] = ok[i] ? ld16_nt(V + src) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < kU; ++i)
      if (ok[i]) {
        st16(K_out + dst[i], kv[i]);
        st16(V_out + dst[i], vv[i]);
      }
  }
}

}  // namespace

size_t prune_ws_bytes(int64_t total_L, int nseq, int n_sets) {
  const size_t thr =
      align_up(static_cast<size_t>(nseq) * 2 * n_sets * sizeof(SegThresh), 256);
  const size_t cnt =
      align_up(static_cast<size_t>(chunk_bound(total_L, nseq, kChunk)) * n_sets * 4, 256);
  return thr + cnt;
}

hipError_t launch_prune(const float* score, const uint8_t* modality, const int32_t* cu_len,
                        const int32_t* keep, const int32_t* cu_kept, int nseq, int64_t total_L,
                        int64_t total_kept, const void* K, const void* V, int n_layers,
                        int per_layer, int Hkv, int D, int dtype, void* K_out, void* V_out,
                        int32_t* kept_idx, void* ws, hipStream_t st) {
  if (total_L == 0) return hipSuccess;
  const int n_sets = per_layer ? n_layers : 1;
  SegThresh* thr = static_cast<SegThresh*>(ws);
  int32_t* counts = reinterpret_cast<int32_t*>(
      static_cast<char*>(ws) +
      align_up(static_cast<size_t>(nseq) * 2 * n_sets * sizeof(SegThresh), 256));
  const int es = dtype == 1 ? 2 : 4;
  const int row_vecs = Hkv * D * es / 16;
  const int64_t nchunk = chunk_bound(total_L, nseq, kChunk);
  topk_threshold_kernel<<<dim3(nseq * 2, n_sets), dim3(kSelThreads), 0, st>>>(
      score, modality, cu_len, keep, nseq, total_L, thr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  chunk_count_kernel<<<dim3(static_cast<unsigned>(nchunk), n_sets), dim3(64), 0, st>>>(
      score, modality, cu_len, nseq, total_L, thr, counts);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (total_kept == 0) return hipSuccess;
  compact_kernel<<<dim3(static_cast<unsigned>(nchunk), static_cast<unsigned>(n_layers)),
                   dim3(kCopyThreads), 0, st>>>(
      score, modality, cu_len, cu_kept, nseq, total_L, total_kept, thr, counts,
      static_cast<const char*>(K), static_cast<const char*>(V), row_vecs,
      static_cast<char*>(K_out), static_cast<char*>(V_out), kept_idx, per_layer);
  return hipGetLastError();
}

}  // namespace sprint
