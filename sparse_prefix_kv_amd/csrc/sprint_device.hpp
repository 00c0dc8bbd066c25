// Device helpers for the SPRINT kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace sprint {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- bf16 <-> f32
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// Round to nearest even (finite inputs): gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Element traits: bf16 is stored as uint16 bit patterns.
struct BF16 {
  using storage = uint16_t;
  static constexpr int bytes = 2;
  __device__ static float to_f32(storage x) { return bf16_to_f32(x); }
  __device__ static storage from_f32(float f) { return f32_to_bf16(f); }
};
struct F32 {
  using storage = float;
  static constexpr int bytes = 4;
  __device__ static float to_f32(storage x) { return x; }
  __device__ static storage from_f32(float f) { return f; }
};

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ int shfl_xor_i(int v, int m) { return __shfl_xor(v, m, 64); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_f(v, m);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor_f(v, m));
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_i(v, m);
  return v;
}

// ---------------------------------------------------------------- MFMA
// 32x32 output tile, 16 reduction elements per call.  Lane l supplies, for
// A, row (l % 32) and for B, column (l % 32); both supply the 8 reduction
// elements of half (l / 32).  Any assignment of reduction indices to the
// (half, element) slots works as long as A and B use the same one.
// The accumulator holds C[row][col] with col = l % 32 and
// row = 8*(r/4) + 4*(l/32) + (r%4) for register r in 0..15.
__device__ __forceinline__ f32x16 mma32_k16(const bf16x8& a, const bf16x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// fp32 operands: the same slot layout, issued as 8 rank-2 fp32 MFMAs
// (element j of lane l pairs with element j of the B lane of the same half).
__device__ __forceinline__ f32x16 mma32_k16(const float (&a)[8], const float (&b)[8], f32x16 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], c, 0, 0, 0);
  return c;
}

// 16-byte vector load/store helpers.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// Non-temporal load for data streamed once (global_load ... nt): the caches
// do not keep the line, which on MI355X raises the rate of cold HBM streams.
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
// Cache-policy operand of buffer loads: non-temporal.
constexpr int kCpolNT = 2;
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// ---------------------------------------------------------------- unmask rule
// One unmasking step for one sequence, on one wave (lane i = block position,
// Lq <= 64), from each lane's loaded confidence, mask byte and argmax (lanes
// past Lq pass any value): accept every masked position whose confidence
// exceeds tau, and at least q = min(m, ceil(m / steps_left)) of the m masked
// ones (all of them when steps_left <= 0), ranked by (confidence descending,
// position ascending).  Writes the accepted tokens and mask bytes and, from
// lane 0, the number accepted.
__device__ __forceinline__ void unmask_rule(float c_ld, uint8_t m_ld, int32_t a_ld, int i, int Lq,
                                            float tau, int steps_left, int64_t base,
                                            uint8_t* masked, int32_t* tokens,
                                            int32_t* n_accepted_s) {
  const bool valid = i < Lq;
  const float c = valid ? c_ld : 0.f;
  const bool msk = valid && m_ld != 0;
  const uint64_t bal_m = __ballot(msk);
  const uint64_t bal_hi = __ballot(msk && c > tau);
  const int m = __popcll(bal_m);
  const int n_hi = __popcll(bal_hi);
  int q = m;
  if (steps_left > 0) {
    const int64_t ceil_q = (static_cast<int64_t>(m) + steps_left - 1) / steps_left;
    q = ceil_q < m ? static_cast<int>(ceil_q) : m;
  }
  const int count = n_hi > q ? n_hi : q;
  // rank = masked positions ahead in (confidence desc, position asc).  An
  // unmasked lane (lanes past Lq included) broadcasts -inf, which is neither
  // above nor equal to any finite confidence, so all 64 lanes are visited
  // without a branch.
  const float ck = msk ? c : -INFINITY;
  int rank = 0;
#pragma unroll
  for (int j = 0; j < 64; ++j) {
    const float cj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ck), j));
    rank += (cj > c || (cj == c && j < i)) ? 1 : 0;
  }
  if (msk && rank < count) {
    tokens[base + i] = a_ld;
    masked[base + i] = 0;
  }
  if (i == 0) *n_accepted_s = count;
}

// ---------------------------------------------------------------- sequence chunks
// Work is split into chunks of `chunk` positions that never cross a sequence
// boundary.  Chunk ids are numbered sequence by sequence; the grid holds an
// upper bound (total_L / chunk + nseq) and surplus blocks exit.
struct SeqChunk {
  int seq;        // sequence index
  int c;          // chunk index within the sequence
  int first;      // chunk id of the sequence's first chunk
  int nchunks;    // chunks in this sequence
  int64_t begin;  // first global row of the sequence
  int64_t len;    // sequence length
};

__device__ __forceinline__ bool find_seq_chunk(const int32_t* __restrict__ cu, int nseq, int chunk,
                                               int64_t total, int b, SeqChunk& out) {
  int acc = 0;
  for (int s = 0; s < nseq; ++s) {
    int64_t a = cu[s], e = cu[s + 1];
    a = a < 0 ? 0 : (a > total ? total : a);
    e = e < a ? a : (e > total ? total : e);
    const int64_t L = e - a;
    const int nc = static_cast<int>((L + chunk - 1) / chunk);
    if (b < acc + nc) {
      out.seq = s;
      out.c = b - acc;
      out.first = acc;
      out.nchunks = nc;
      out.begin = a;
      out.len = L;
      return true;
    }
    acc += nc;
  }
  return false;
}

__host__ __device__ inline int64_t chunk_bound(int64_t total, int nseq, int chunk) {
  return total / chunk + nseq;
}

}  // namespace sprint
