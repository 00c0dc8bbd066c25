// Modality-aware prefix pruning and KV compaction (LLaDA2.0-Uni, SPRINT
// "Sparse Prefix Retention": keep the top-floor(r*n) positions by score within
// each modality, then build a contiguous pruned cache once per block).
//
// Ranking key of position p: (score desc, position asc).  The score is mapped
// to an order-preserving uint32, so "the k-th largest" is found exactly by an
// MSB-first radix select (windows of up to 8 bits) per (sequence, modality)
// segment.  The result is a threshold key T and a tie cut: a position is
// kept iff key > T, or key == T and p <= tie_cut (the first ties by position).
//
// Launches:
//   1. topk_threshold_kernel  one 1024-thread block per segment; the keys of
//                             a sequence of up to 32768 positions are read
//                             from HBM once and stay in registers (32 per
//                             thread) for every radix window; the histogram
//                             has a copy per lane so that keys crowding into
//                             few digits do not serialize the LDS atomics;
//                             once at most 64 keys share the prefix, one
//                             wave ranks them directly instead of further
//                             windows; each block also writes its
//                             modality's kept count of every 64-position
//                             chunk;
//   2. compact_kernel         per chunk: prefix of earlier chunk counts in the
//                             sequence -> output slots; writes kept_idx and
//                             copies the K and V rows (16-byte vectors), of
//                             every layer (grid y) when one kept set serves
//                             several layers' caches.
// With a kept set per layer, both run once per layer (grid y), each
// layer on its own scores, thresholds, counts and kept_idx row.
// The copy dominates: 2 x kept x row bytes read and written, HBM-bound.
#include <limits.h>

#include "sprint_device.hpp"
#include "sprint_internal.hpp"

namespace sprint {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kRegChunks = 2;      // 16-position chunks of keys held per thread
constexpr int kFewKeys = 64;       // keys under the prefix one wave ranks directly
constexpr int kChunk = 64;
constexpr int kCopyThreads = 256;

struct SegThresh {
  uint32_t key;
  int32_t tie_cut;
};

__device__ __forceinline__ uint32_t order_key(float f) {
  // non-negative: the sign bit set; negative: the two's complement, which
  // reverses their order and puts -0 on the key of +0.  No score has key 0.
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? 0u - u : u | 0x80000000u;
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

// Per-lane copies of the 256-digit histogram: digit d, copy c at
// d * kHistCopies + c, lane l counting into copy l % kHistCopies.  Two lanes
// of a wave share an address only when they are 32 apart and count the same
// digit, however the keys crowd into few digits (scores share their top
// exponent bits, so the first windows are far from uniform).
constexpr int kHistCopies = 32;

__device__ __forceinline__ void hist_count(int* hist, uint32_t digit) {
  atomicAdd(&hist[digit * kHistCopies + (threadIdx.x & (kHistCopies - 1))], 1);
}

// Radix-window selection step shared by both paths.  On entry every thread
// has counted its keys into hist.  Sums the copies of each digit into s_cnt
// (and clears them for the next window), taking `absent0` off digit 0 (slots
// counted there that hold no key).  Then every wave scans the 256 counts on
// its own and returns, in every thread, the digit that holds the krem-th
// largest key, the number of keys in higher digits, the number in it and the
// number counted.  Every thread of the block calls it.
struct WindowPick {
  int digit, above, count, total;
};

__device__ __forceinline__ int dpp_row_shr(int v, int ctrl_shift) {
  // lane i of a row of 16 reads lane i - n of that row, 0 below it
  switch (ctrl_shift) {
    case 1: return __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);
    case 2: return __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);
    case 4: return __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);
    default: return __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);
  }
}

__device__ __forceinline__ WindowPick pick_digit(int* hist, int* s_cnt, int krem, int absent0) {
  const int lane = threadIdx.x & 63;
  __syncthreads();  // every count is in
  {
    // digit d = threadIdx.x / 4: four threads sum 8 copies each
    const int d = threadIdx.x >> 2, part = threadIdx.x & 3;
    int4* hp = reinterpret_cast<int4*>(hist + d * kHistCopies + part * 8);
    const int4 x = hp[0], y = hp[1];
    hp[0] = make_int4(0, 0, 0, 0);
    hp[1] = make_int4(0, 0, 0, 0);
    int h = x.x + x.y + x.z + x.w + y.x + y.y + y.z + y.w;
    h += __builtin_amdgcn_mov_dpp(h, 0xB1, 0xF, 0xF, true);  // quad lanes 1,0,3,2
    h += __builtin_amdgcn_mov_dpp(h, 0x4E, 0xF, 0xF, true);  // quad lanes 2,3,0,1
    if (part == 0) s_cnt[d] = d == 0 ? h - absent0 : h;
  }
  __syncthreads();
  // lane l holds digits 252-4l .. 255-4l (the highest digits in lane 0); an
  // inclusive scan over the lanes counts the keys at or above each lane's
  // lowest digit
  const int4 c = *reinterpret_cast<const int4*>(s_cnt + 252 - 4 * lane);
  const int csum = c.x + c.y + c.z + c.w;
  int v = csum;
  v += dpp_row_shr(v, 1);
  v += dpp_row_shr(v, 2);
  v += dpp_row_shr(v, 4);
  v += dpp_row_shr(v, 8);
  const int r15 = __builtin_amdgcn_readlane(v, 15);
  const int r31 = __builtin_amdgcn_readlane(v, 31);
  const int r47 = __builtin_amdgcn_readlane(v, 47);
  const int row = lane >> 4;
  v += (row >= 1 ? r15 : 0) + (row >= 2 ? r31 : 0) + (row >= 3 ? r47 : 0);
  // the lane's digits from the highest down
  int acc = v - csum;  // keys above the lane's digits
  int found = -1, f_above = 0, f_cnt = 0;
  const int cnt[4] = {c.w, c.z, c.y, c.x};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (found < 0 && acc < krem && krem <= acc + cnt[q]) {
      found = 255 - 4 * lane - q;
      f_above = acc;
      f_cnt = cnt[q];
    }
    acc += cnt[q];
  }
  const uint64_t m = __ballot(found >= 0);
  WindowPick r{0, 0, 0, __builtin_amdgcn_readlane(v, 63)};
  if (m != 0ull) {
    const int src = __builtin_ctzll(m);
    r.digit = __builtin_amdgcn_readlane(found, src);
    r.above = __builtin_amdgcn_readlane(f_above, src);
    r.count = __builtin_amdgcn_readlane(f_cnt, src);
  }
  return r;
}

__global__ __launch_bounds__(kSelThreads) void topk_threshold_kernel(
    const float* __restrict__ score, const uint8_t* __restrict__ modality,
    const int32_t* __restrict__ cu_len, const int32_t* __restrict__ keep, int nseq,
    int64_t total_L, SegThresh* __restrict__ thr, int32_t* __restrict__ counts, int64_t nchunk) {
  // grid y: the layer whose scores select its own set (one layer otherwise)
  score += static_cast<int64_t>(blockIdx.y) * total_L;
  thr += static_cast<int64_t>(blockIdx.y) * nseq * 2;
  const int seg = blockIdx.x;
  const int s = seg >> 1;
  const uint8_t mod = static_cast<uint8_t>(seg & 1);
  // this segment's column of kept counts per 64-position chunk (chunk ids
  // run sequence by sequence, as the compaction numbers them)
  counts += (static_cast<int64_t>(blockIdx.y) * 2 + mod) * nchunk;
  int64_t a, e;
  clamp_seq(cu_len, s, total_L, a, e);
  const int nc = static_cast<int>((e - a + kChunk - 1) / kChunk);
  const int k = keep[seg];
  __shared__ __align__(16) int hist[256 * kHistCopies];
  __shared__ __align__(16) int s_cnt[256];
  __shared__ int s_cc[kSelThreads];
  __shared__ int s_wave[kSelThreads / 64];
  __shared__ int s_first[kSelThreads / 64];
  __shared__ int s_found;
  __shared__ int64_t s_cut;
  __shared__ uint32_t s_min[kSelThreads / 64], s_max[kSelThreads / 64];
  __shared__ uint32_t s_cand[kFewKeys];
  __shared__ int s_ncand;
  __shared__ uint32_t s_sel[3];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 256 * kHistCopies; i += kSelThreads) hist[i] = 0;
  s_cc[threadIdx.x] = 0;
  if (threadIdx.x == 0) s_ncand = 0;
  {
    // chunk id of the sequence's first chunk: chunks of the earlier ones
    int acc = 0;
    for (int s2 = threadIdx.x; s2 < s; s2 += kSelThreads) {
      int64_t a2, e2;
      clamp_seq(cu_len, s2, total_L, a2, e2);
      acc += static_cast<int>((e2 - a2 + kChunk - 1) / kChunk);
    }
    acc = wave_sum_i(acc);
    if (lane == 0) s_first[wave] = acc;
  }
  __syncthreads();
  int first_chunk = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) first_chunk += s_first[w];
  counts += first_chunk;
  if (k <= 0) {  // nothing kept
    if (threadIdx.x == 0) thr[seg] = SegThresh{0xFFFFFFFFu, -1};
    for (int c = threadIdx.x; c < nc; c += kSelThreads) counts[c] = 0;
    return;
  }
  if (e <= a) {  // empty sequence: nothing to read
    if (threadIdx.x == 0) thr[seg] = SegThresh{0u, INT_MAX};
    return;
  }
  uint32_t prefix = 0, pmask = 0;
  int krem = k;
  int ties = 0;

  // The positions from a rounded down to a multiple of 16 are cut into
  // chunks of 16; thread t holds chunks t and t + 1024.  When those cover the
  // sequence, every key is read from HBM once, into registers, and every
  // radix window counts from there.
  const int64_t a16 = a & ~static_cast<int64_t>(15);
  if (e - a16 <= kRegChunks * kSelThreads * 16) {
    // key 0 marks a slot outside the sequence or of the other modality.
    // Chunk j of a wave is active when it starts inside the sequence; the
    // slots of inactive chunks are never counted (shorter sequences skip
    // most of the work).
    uint32_t key[kRegChunks * 16];
    bool act[kRegChunks];
    int n_slots = 0;  // slots of the active chunks of the block
#pragma unroll
    for (int j = 0; j < kRegChunks; ++j) {
      act[j] = a16 + static_cast<int64_t>(j * kSelThreads + wave * 64) * 16 < e;
      const int64_t left = e - a16 - static_cast<int64_t>(j) * kSelThreads * 16;
      const int64_t waves = left <= 0 ? 0 : (left + 1023) / 1024;
      n_slots += static_cast<int>(waves < kSelThreads / 64 ? waves : kSelThreads / 64) * 1024;
    }
    int n_mine = 0;
    {
      u32x4 sv[kRegChunks][4], mv[kRegChunks];
      const bool vec = (reinterpret_cast<uintptr_t>(score) & 15) == 0 &&
                       (reinterpret_cast<uintptr_t>(modality) & 15) == 0;
      if (vec) {
        // 16-byte buffer loads; past the resource's end they read zeros
        int64_t span = total_L - a16;  // integer arithmetic: the resource stays scalar
        if (span > kRegChunks * kSelThreads * 16) span = kRegChunks * kSelThreads * 16;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(score + a16), 0, static_cast<int>(span * 4), 0x00020000);
        const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(modality + a16), 0, static_cast<int>(span), 0x00020000);
#pragma unroll
        for (int j = 0; j < kRegChunks; ++j) {
          const int q = j * kSelThreads + threadIdx.x;
#pragma unroll
          for (int c = 0; c < 4; ++c)
            sv[j][c] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, q * 64 + c * 16, 0, 0));
          mv[j] = __builtin_bit_cast(u32x4,
                                     __builtin_amdgcn_raw_buffer_load_b128(rm, q * 16, 0, 0));
        }
      }
      const uint32_t rep = mod ? 0x01010101u : 0u;
#pragma unroll
      for (int j = 0; j < kRegChunks; ++j) {
        if (!act[j]) {
#pragma unroll
          for (int i = 0; i < 16; ++i) key[j * 16 + i] = 0u;
          continue;
        }
        const int64_t c0 = a16 + static_cast<int64_t>(j * kSelThreads + threadIdx.x) * 16;
        // unaligned arrays, or the chunk that runs past the end of the
        // arrays: one position at a time (clamped into the sequence)
        if (!vec || (c0 < e && c0 + 16 > total_L)) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int64_t p = c0 + i;
            const int64_t pc = p < a ? a : (p >= e ? e - 1 : p);
            sv[j][i >> 2][i & 3] = __float_as_uint(score[pc]);
            const uint32_t sh = 8u * (i & 3);
            mv[j][i >> 2] = (mv[j][i >> 2] & ~(0xFFu << sh)) | (uint32_t{modality[pc]} << sh);
          }
        }
        // positions outside the sequence take modality byte 0xFF (neither)
        if (c0 < a || c0 + 16 > e) {
          const int lo = static_cast<int>(c0 < a ? a - c0 : 0);
          const int hi = static_cast<int>(c0 >= e ? 0 : (c0 + 16 > e ? e - c0 : 16));
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (i < lo || i >= hi) mv[j][i >> 2] |= 0xFFu << (8 * (i & 3));
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // bit 7 of each byte of z: that position is of this modality
          const uint32_t x = mv[j][w] ^ rep;
          const uint32_t z = ~(((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x) & 0x80808080u;
          n_mine += __popc(z);
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const uint32_t sel = static_cast<uint32_t>(static_cast<int>(z << (24 - 8 * b)) >> 31);
            key[j * 16 + w * 4 + b] = order_key(__uint_as_float(sv[j][w][b])) & sel;
          }
        }
      }
    }
    // the modality's key count and its smallest and largest key
    uint32_t kmin1 = 0xFFFFFFFFu, kmax = 0u;  // kmin1: smallest key - 1 (key 0 wraps)
#pragma unroll
    for (int r = 0; r < kRegChunks * 16; ++r) {
      kmin1 = min(kmin1, key[r] - 1u);
      kmax = max(kmax, key[r]);
    }
    int n_m = n_mine;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      kmin1 = min(kmin1, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmin1), o, 64)));
      kmax = max(kmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmax), o, 64)));
      n_m += __shfl_xor(n_m, o, 64);
    }
    if (lane == 0) {
      s_min[wave] = kmin1;
      s_max[wave] = kmax;
      s_wave[wave] = n_m;
    }
    __syncthreads();
    n_m = 0;
#pragma unroll
    for (int w = 0; w < kSelThreads / 64; ++w) {
      kmin1 = min(kmin1, s_min[w]);
      kmax = max(kmax, s_max[w]);
      n_m += s_wave[w];
    }
    // every position of the modality is kept when k >= n_m
    const bool all = k >= n_m;
    int64_t cut = INT_MAX;
    if (!all) {
      const uint32_t kmin = kmin1 + 1u;
      const int n_absent = n_slots - n_m;
      ties = n_m;
      // Windows of up to 8 bits from the highest bit where the smallest and
      // largest key differ (the bits above it are common to every key).  The
      // first window counts every slot: the key-0 slots all fall on digit 0
      // and are taken off there; later windows count the keys under the
      // prefix, which key 0 matches only while the prefix is 0.
      int hi = -1;
      if (kmin == kmax) {
        prefix = kmin;
        pmask = 0xFFFFFFFFu;
      } else {
        hi = 31 - __clz(static_cast<int>(kmin ^ kmax));
        pmask = hi == 31 ? 0u : ~((2u << hi) - 1u);
        prefix = kmin & pmask;
      }
      bool first = true;
      while (hi >= 0) {
        const int wbits = hi + 1 < 8 ? hi + 1 : 8;
        const int shift = hi + 1 - wbits;
        const uint32_t dmask = (1u << wbits) - 1u;
#pragma unroll
        for (int j = 0; j < kRegChunks; ++j) {
          if (!act[j]) continue;
          if (first) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
            hist_count(hist, __builtin_amdgcn_ubfe(key[j * 16 + i], shift, wbits));
          } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const bool in = (key[j * 16 + i] & pmask) == prefix;
              if (in) hist_count(hist, __builtin_amdgcn_ubfe(key[j * 16 + i], shift, wbits));
            }
          }
        }
        const WindowPick w =
            pick_digit(hist, s_cnt, krem, first || prefix == 0u ? n_absent : 0);
        first = false;
        krem -= w.above;
        ties = w.count;
        prefix |= static_cast<uint32_t>(w.digit) << shift;
        pmask |= dmask << shift;
        hi = shift - 1;
        if (hi >= 0 && ties <= kFewKeys) {
          // At most 64 keys left under the prefix: one wave ranks them
          // directly instead of further radix windows.  The key holding
          // rank krem among them (gt keys above it, eq equal to it, with
          // gt < krem <= gt + eq) is the threshold.
#pragma unroll
          for (int j = 0; j < kRegChunks; ++j) {
            if (!act[j]) continue;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const uint32_t kk = key[j * 16 + i];
              if (kk != 0u && (kk & pmask) == prefix) {
                const int slot = atomicAdd(&s_ncand, 1);
                if (slot < kFewKeys) s_cand[slot] = kk;
              }
            }
          }
          __syncthreads();
          if (wave == 0) {
            const int nk = min(__builtin_amdgcn_readfirstlane(s_ncand), kFewKeys);
            const uint32_t v = lane < nk ? s_cand[lane] : 0u;
            int gt = 0, eq = 0;
            for (int i = 0; i < nk; ++i) {
              const uint32_t u = __builtin_amdgcn_readlane(v, i);
              gt += u > v ? 1 : 0;
              eq += u == v ? 1 : 0;
            }
            const uint64_t hit = __ballot(lane < nk && gt < krem && krem <= gt + eq);
            const int src = hit ? __builtin_ctzll(hit) : 0;
            const uint32_t t = __builtin_amdgcn_readlane(v, src);
            const int tg = __builtin_amdgcn_readlane(gt, src);
            const int te = __builtin_amdgcn_readlane(eq, src);
            if (lane == 0) {
              s_sel[0] = t;
              s_sel[1] = static_cast<uint32_t>(tg);
              s_sel[2] = static_cast<uint32_t>(te);
            }
          }
          __syncthreads();
          prefix = s_sel[0];
          pmask = 0xFFFFFFFFu;
          krem -= static_cast<int>(s_sel[1]);
          ties = static_cast<int>(s_sel[2]);
          break;
        }
      }
      if (krem < ties) {
        // Tie cut: the krem-th position, in position order, whose key is the
        // threshold (never 0).  Position order is chunk 0 of threads 0..1023,
        // then chunk 1.
        int before = 0;
#pragma unroll
        for (int j = 0; j < kRegChunks; ++j) {
          uint32_t tie = 0;
#pragma unroll
          for (int i = 0; i < 16; ++i) tie |= (key[j * 16 + i] == prefix ? 1u : 0u) << i;
          const int c = __popc(tie);
          int tot;
          const int incl = block_incl_scan(c, s_wave, tot) + before;
          const int want = krem - (incl - c);  // 1-based rank of the cut in this chunk
          if (want >= 1 && want <= c) {
            int seen = 0, slot = 0;
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if ((tie >> i) & 1u) {
                ++seen;
                if (seen == want) slot = i;
              }
            s_cut = a16 + static_cast<int64_t>(j * kSelThreads + threadIdx.x) * 16 + slot;
          }
          before += tot;
        }
        __syncthreads();
        cut = s_cut;
      }
    }
    const uint32_t T = all ? 0u : prefix;
    if (threadIdx.x == 0) thr[seg] = SegThresh{T, static_cast<int32_t>(cut)};
    // Kept counts of the chunks.  Kept: key >= Tm when there is no tie cut
    // (Tm = 1 keeps every key of the modality), else key > T or key == T at
    // a position <= cut.
    const bool tie_cut = cut != INT_MAX;
    const uint32_t Tm = all ? 1u : T;
    int kc[kRegChunks];          // kept slots of chunk j
    uint32_t kmask[kRegChunks];  // the same as a bit mask (tie cut or unaligned start)
    const bool aligned = (a & 15) == 0;
#pragma unroll
    for (int j = 0; j < kRegChunks; ++j) {
      kc[j] = 0;
      kmask[j] = 0;
      if (!act[j]) continue;
      const int64_t c0 = a16 + static_cast<int64_t>(j * kSelThreads + threadIdx.x) * 16;
      if (!tie_cut && aligned) {
#pragma unroll
        for (int i = 0; i < 16; ++i) kc[j] += key[j * 16 + i] >= Tm ? 1 : 0;
      } else {
        const int64_t rel = cut - c0;  // slots 0..lim may tie
        const int lim = static_cast<int>(rel < -1 ? -1 : (rel > 15 ? 15 : rel));
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t kk = key[j * 16 + i];
          const bool kept = tie_cut ? (kk > T || (kk == T && i <= lim)) : kk >= Tm;
          kmask[j] |= (kept ? 1u : 0u) << i;
        }
        kc[j] = __popc(kmask[j]);
      }
    }
    if (aligned) {
      // 16-position chunk q of the sequence is quarter q % 4 of 64-position
      // chunk q / 4, and the four quarters sit in lanes 4c .. 4c+3
#pragma unroll
      for (int j = 0; j < kRegChunks; ++j) {
        if (!act[j]) continue;
        int v = kc[j];
        v += __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);  // quad lanes 1,0,3,2
        v += __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);  // quad lanes 2,3,0,1
        const int c = (j * kSelThreads + static_cast<int>(threadIdx.x)) >> 2;
        if ((threadIdx.x & 3) == 0 && c < nc) counts[c] = v;
      }
      return;
    }
    // unaligned start: a thread's 16 slots fall in at most two chunks
#pragma unroll
    for (int j = 0; j < kRegChunks; ++j) {
      const uint32_t km = kmask[j];
      if (km == 0u) continue;
      const int64_t c0 = a16 + static_cast<int64_t>(j * kSelThreads + threadIdx.x) * 16;
      const int r0 = static_cast<int>(c0 - a);  // -15 .. 32767
      const int C0 = r0 >> 6, C1 = (r0 + 15) >> 6;
      if (C0 == C1) {
        atomicAdd(&s_cc[C0], __popc(km));
      } else {
        // slots before a hold key 0, so `lo` is empty when C0 is -1
        const int ib = C1 * 64 - r0;
        const uint32_t lo = km & ((1u << ib) - 1u), up = km >> ib;
        if (lo != 0u) atomicAdd(&s_cc[C0], __popc(lo));
        if (up != 0u) atomicAdd(&s_cc[C1], __popc(up));
      }
    }
    __syncthreads();
    if (static_cast<int>(threadIdx.x) < nc) counts[threadIdx.x] = s_cc[threadIdx.x];  // nc <= 513
    return;
  }

  // Longer sequences: every window reads the scores from HBM again, in four
  // windows of 8 bits from the top.
  bool first = true, all = false;
  for (int hi = 31; hi >= 0; hi -= 8) {
    const int shift = hi - 7;
    constexpr int kU = 8;
    for (int64_t p0 = a; p0 < e; p0 += kU * kSelThreads) {
      uint32_t md[kU];
      float sc[kU];
      // every load of the round issued before any is used: positions past
      // the sequence read its last position and count as the other modality
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t p = p0 + u * kSelThreads + threadIdx.x;
        const bool in = p < e;
        const int64_t pc = in ? p : e - 1;
        const uint32_t m = modality[pc];
        md[u] = in ? m : static_cast<uint32_t>(mod ^ 1);
        sc[u] = score[pc];
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const uint32_t key = order_key(sc[u]);
        if (md[u] == mod && (key & pmask) == prefix) hist_count(hist, (key >> shift) & 0xFFu);
      }
    }
    const WindowPick w = pick_digit(hist, s_cnt, krem, 0);
    if (first) {
      if (k >= w.total) {  // every position of the modality is kept
        all = true;
        break;
      }
      first = false;
    }
    krem -= w.above;
    ties = w.count;
    prefix |= static_cast<uint32_t>(w.digit) << shift;
    pmask |= 0xFFu << shift;
  }
  // prefix is now the exact key of the k-th largest; keep the first `krem`
  // of the `ties` positions that carry it.
  int64_t cut = INT_MAX;
  if (!all && krem < ties) {
    if (threadIdx.x == 0) s_found = 0;
    __syncthreads();
    int base = 0;
    for (int64_t p0 = a; p0 < e; p0 += kSelThreads) {
      const int64_t p = p0 + threadIdx.x;
      const int f = (p < e && modality[p] == mod && order_key(score[p]) == prefix) ? 1 : 0;
      int tot;
      const int incl = block_incl_scan(f, s_wave, tot);
      if (f && base + incl == krem) {
        s_cut = p;
        s_found = 1;
      }
      base += tot;
      __syncthreads();
      if (s_found) break;
    }
    cut = s_cut;
  }
  const uint32_t T = all ? 0u : prefix;
  if (threadIdx.x == 0) thr[seg] = SegThresh{T, static_cast<int32_t>(cut)};
  // kept counts of the chunks, a wave per chunk
  for (int c = wave; c < nc; c += kSelThreads / 64) {
    const int64_t p = a + static_cast<int64_t>(c) * kChunk + lane;
    bool kept = false;
    if (p < e && modality[p] == mod) {
      const uint32_t kk = order_key(score[p]);
      kept = all || kk > T || (kk == T && p <= cut);
    }
    const uint64_t b = __ballot(kept);
    if (lane == 0) counts[c] = static_cast<int32_t>(__popcll(b));
  }
}


__device__ __forceinline__ bool kept_at(const float* __restrict__ score,
                                        const uint8_t* __restrict__ modality,
                                        const SegThresh* __restrict__ thr, int s, int64_t p) {
  const uint8_t m = modality[p];
  const SegThresh t = thr[2 * s + (m ? 1 : 0)];
  return is_kept(order_key(score[p]), p, t);
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
    counts += layer * 2 * gridDim.x;
    kept_idx += layer * total_kept;
  }
  __shared__ int64_t s_pos[kChunk];
  __shared__ int64_t s_slot0, s_limit;
  __shared__ int s_nk;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int pre = 0;
    // both modality columns of the earlier chunks of the sequence
    for (int i = lane; i < sc.c; i += 64)
      pre += counts[sc.first + i] + counts[gridDim.x + sc.first + i];
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
  // Four 16-byte vectors of K and of V per thread in flight per round.  The
  // source rows are read once (non-temporal); the pruned cache is written
  // with ordinary-policy buffer stores, since the denoising steps read it
  // next.  Nothing is branched: a unit past the chunk's last reads that last
  // unit, and a store that must not happen goes to an offset past the end of
  // the output resource, which the hardware drops.  (Loads or stores under a
  // per-lane condition compile to branches that wait for each load in turn.)
  const uint32_t out_bytes = static_cast<uint32_t>(total_kept * row_bytes);  // < 2^31 (host)
  const __amdgpu_buffer_rsrc_t rKo =
      __builtin_amdgcn_make_buffer_rsrc(K_out, 0, static_cast<int>(out_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t rVo =
      __builtin_amdgcn_make_buffer_rsrc(V_out, 0, static_cast<int>(out_bytes), 0x00020000);
  constexpr uint32_t kDrop = 0x80000000u;  // past every output resource
  constexpr int kU = 4;
  for (int u0 = threadIdx.x; u0 < units; u0 += kU * kCopyThreads) {
    u32x4 kv[kU], vv[kU];
    uint32_t dst[kU];
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      const int u = u0 + i * kCopyThreads;
      const int uc = u < units ? u : units - 1;
      const int r = uc / row_vecs, v = uc - r * row_vecs;
      const int64_t slot = slot0 + r;
      const bool ok = u < units && slot >= 0 && slot < limit;
      const int64_t src = s_pos[r] * row_bytes + v * 16;
      dst[i] = ok ? static_cast<uint32_t>(slot * row_bytes + v * 16) : kDrop;
      kv[i] = ld16_nt(K + src);
      vv[i] = ld16_nt(V + src);
    }
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      __builtin_amdgcn_raw_buffer_store_b128(kv[i], rKo, static_cast<int>(dst[i]), 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(vv[i], rVo, static_cast<int>(dst[i]), 0, 0);
    }
  }
}

}  // namespace

size_t prune_ws_bytes(int64_t total_L, int nseq, int n_sets) {
  const size_t thr =
      align_up(static_cast<size_t>(nseq) * 2 * n_sets * sizeof(SegThresh), 256);
  const size_t cnt =
      align_up(static_cast<size_t>(chunk_bound(total_L, nseq, kChunk)) * n_sets * 2 * 4, 256);
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
      score, modality, cu_len, keep, nseq, total_L, thr, counts, nchunk);
  hipError_t e = hipGetLastError();
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
