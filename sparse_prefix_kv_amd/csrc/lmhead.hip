// LM-head confidence with the softmax statistics fused into the GEMM
// (LLaDA2.0-Uni, SPRINT: c_i = max_v p(v|x_t) in "Sparse Prefix Retention",
// c_n = p(x0_hat|x_t) in "Non-uniform Token Unmasking").
//
// Z^T = W X^T is computed tile by tile on MFMA (A = vocabulary rows of W,
// B = token rows of X, both staged through LDS).  With that orientation the
// accumulator gives each lane one token column and 16 vocabulary rows, so the
// per-token (max, sum exp, argmax) of a tile is a lane-local loop plus one
// cross-half and one cross-wave merge.  Only 16 bytes per (token, vocabulary
// tile) leave the kernel; a merge kernel folds the tiles in vocabulary order.
// Ties keep the lowest vocabulary index.  Sums use exp2 with log2(e) scaling.
#include <limits.h>
#include <math.h>

#include "sprint_device.hpp"
#include "sprint_internal.hpp"

namespace sprint {
namespace {

constexpr int kKC = 64;  // reduction depth per LDS stage

struct Stat {
  float m;  // max logit
  float s;  // sum exp(z - m)
  int a;    // argmax (lowest index on ties)
};

__device__ __forceinline__ void merge(Stat& x, const Stat& y) {
  if (y.m == -INFINITY) return;
  if (x.m == -INFINITY) {
    x = y;
    return;
  }
  const float mn = fmaxf(x.m, y.m);
  x.s = x.s * exp2f((x.m - mn) * kLog2e) + y.s * exp2f((y.m - mn) * kLog2e);
  if (y.m > x.m || (y.m == x.m && y.a < x.a)) x.a = y.a;
  x.m = mn;
}

template <typename T>
struct LFrag;
template <>
struct LFrag<BF16> {
  using type = bf16x8;
  __device__ static type load(const uint16_t* p) { return as_bf16x8(ld16(p)); }
  __device__ static f32x16 mma(const type& a, const type& b, f32x16 c) { return mma32_k16(a, b, c); }
};
struct LF8 {
  float v[8];
};
template <>
struct LFrag<F32> {
  using type = LF8;
  __device__ static type load(const float* p) {
    type r;
    const u32x4 a = ld16(p), b = ld16(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r.v[i] = __uint_as_float(a[i]);
      r.v[4 + i] = __uint_as_float(b[i]);
    }
    return r;
  }
  __device__ static f32x16 mma(const type& a, const type& b, f32x16 c) {
    return mma32_k16(a.v, b.v, c);
  }
};

// Block = 4 waves laid out NWV (vocab) x NWT (tokens); each wave computes
// WV x WT tiles of 32x32.  Block tile = BV vocab rows x BT token rows.
template <typename T, int NWV, int NWT, int WV, int WT>
__global__ __launch_bounds__(256) void lmhead_tile_kernel(const char* __restrict__ X, int64_t M,
                                                          int H, const char* __restrict__ W,
                                                          int V, float4* __restrict__ part,
                                                          int n_vt) {
  using S = typename T::storage;
  using FR = LFrag<T>;
  static_assert(NWV * NWT == 4, "four waves");
  constexpr int BV = NWV * WV * 32, BT = NWT * WT * 32;
  constexpr int kEpv = 16 / sizeof(S);
  constexpr int kRow = kKC + kEpv;                 // padded LDS pitch (elements)
  constexpr int kVpr = kKC / kEpv;                 // 16-byte vectors per staged row
  __shared__ __align__(16) S sA[BV * kRow];
  __shared__ __align__(16) S sB[BT * kRow];
  __shared__ Stat red[NWT * WT * 32][NWV];

  const int vt = blockIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * BT;
  const int v0 = vt * BV;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wv = wave % NWV, wt = wave / NWV;
  const int q = lane & 31, hh = lane >> 5;
  const int64_t row_bytes = static_cast<int64_t>(H) * sizeof(S);

  f32x16 acc[WV][WT];
#pragma unroll
  for (int i = 0; i < WV; ++i)
#pragma unroll
    for (int j = 0; j < WT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  for (int k0 = 0; k0 < H; k0 += kKC) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < BV * kVpr; idx += 256) {
      const int r = idx / kVpr, v = idx - r * kVpr;
      const int vr = v0 + r;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (vr < V) x = ld16(W + vr * row_bytes + (static_cast<int64_t>(k0) + v * kEpv) * sizeof(S));
      st16(&sA[r * kRow + v * kEpv], x);
    }
    for (int idx = threadIdx.x; idx < BT * kVpr; idx += 256) {
      const int r = idx / kVpr, v = idx - r * kVpr;
      const int64_t tr = t0 + r;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (tr < M) x = ld16(X + tr * row_bytes + (static_cast<int64_t>(k0) + v * kEpv) * sizeof(S));
      st16(&sB[r * kRow + v * kEpv], x);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kKC / 16; ++ks) {
      typename FR::type a[WV], b[WT];
#pragma unroll
      for (int i = 0; i < WV; ++i)
        a[i] = FR::load(&sA[((wv * WV + i) * 32 + q) * kRow + 16 * ks + 8 * hh]);
#pragma unroll
      for (int j = 0; j < WT; ++j)
        b[j] = FR::load(&sB[((wt * WT + j) * 32 + q) * kRow + 16 * ks + 8 * hh]);
#pragma unroll
      for (int i = 0; i < WV; ++i)
#pragma unroll
        for (int j = 0; j < WT; ++j) acc[i][j] = FR::mma(a[i], b[j], acc[i][j]);
    }
  }

  // Epilogue: per token column, fold this wave's vocabulary rows.
#pragma unroll
  for (int j = 0; j < WT; ++j) {
    Stat st{-INFINITY, 0.f, INT_MAX};
#pragma unroll
    for (int i = 0; i < WV; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int v = v0 + (wv * WV + i) * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
        const float z = acc[i][j][r];
        if (v < V && z > st.m) {
          st.m = z;
          st.a = v;
        }
      }
    if (st.m != -INFINITY) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < WV; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int v = v0 + (wv * WV + i) * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (v < V) s += exp2f((acc[i][j][r] - st.m) * kLog2e);
        }
      st.s = s;
    }
    Stat other;
    other.m = shfl_xor_f(st.m, 32);
    other.s = shfl_xor_f(st.s, 32);
    other.a = shfl_xor_i(st.a, 32);
    if (hh == 0) {
      merge(st, other);
      red[(wt * WT + j) * 32 + q][wv] = st;
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < BT; c += 256) {
    const int64_t tok = t0 + c;
    if (tok >= M) continue;
    Stat st = red[c][0];
#pragma unroll
    for (int w = 1; w < NWV; ++w) merge(st, red[c][w]);
    part[tok * n_vt + vt] = make_float4(st.m, st.s, __int_as_float(st.a), 0.f);
  }
}

// One wave per row: each lane folds a strided subset of tiles in order, then
// a fixed butterfly merges the lanes.
__global__ __launch_bounds__(256) void lmhead_merge_kernel(const float4* __restrict__ part,
                                                           int64_t M, int n_vt,
                                                           float* __restrict__ conf,
                                                           int32_t* __restrict__ argmax,
                                                           float* __restrict__ lse) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (row >= M) return;
  Stat st{-INFINITY, 0.f, INT_MAX};
  for (int t = lane; t < n_vt; t += 64) {
    const float4 p = part[row * n_vt + t];
    merge(st, Stat{p.x, p.y, __float_as_int(p.z)});
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    Stat o;
    o.m = shfl_xor_f(st.m, m);
    o.s = shfl_xor_f(st.s, m);
    o.a = shfl_xor_i(st.a, m);
    // merge in a lane-symmetric way so every lane ends with the same value
    Stat lo = (lane & m) ? o : st;
    const Stat hi = (lane & m) ? st : o;
    merge(lo, hi);
    st = lo;
  }
  if (lane == 0) {
    conf[row] = 1.f / st.s;
    argmax[row] = st.a;
    if (lse) lse[row] = st.m + logf(st.s);
  }
}

struct TileShape {
  int BV, BT;
};

template <typename T, int NWV, int NWT, int WV, int WT>
hipError_t run_tiles(const void* X, int64_t M, int H, const void* W, int V, float4* part,
                     int n_vt, hipStream_t st) {
  constexpr int BT = NWT * WT * 32;
  const int64_t n_tt = (M + BT - 1) / BT;
  lmhead_tile_kernel<T, NWV, NWT, WV, WT><<<dim3(n_vt, static_cast<unsigned>(n_tt)), dim3(256), 0,
                                             st>>>(static_cast<const char*>(X), M, H,
                                                   static_cast<const char*>(W), V, part, n_vt);
  return hipGetLastError();
}

// Small M (a denoising step's block): 32 tokens x 128 vocabulary rows per
// block, so the grid spreads W over every CU.  Large M (the prefix pass):
// 128 x 128 tiles.
inline bool small_m(int64_t M) { return M <= 32; }
inline int tile_bv(int64_t M) { return small_m(M) ? 128 : 128; }

}  // namespace

size_t lmhead_ws_bytes(int64_t M, int H, int V, int dtype) {
  (void)H;
  (void)dtype;
  const int n_vt = (V + tile_bv(M) - 1) / tile_bv(M);
  return align_up(static_cast<size_t>(M) * n_vt * sizeof(float4), 256);
}

hipError_t launch_lmhead(const void* X, int64_t M, int H, const void* W, int V, int dtype,
                         float* conf, int32_t* argmax, float* lse, void* ws, hipStream_t st) {
  const int n_vt = (V + tile_bv(M) - 1) / tile_bv(M);
  float4* part = static_cast<float4*>(ws);
  hipError_t e;
  if (dtype == 1)
    e = small_m(M) ? run_tiles<BF16, 4, 1, 1, 1>(X, M, H, W, V, part, n_vt, st)
                   : run_tiles<BF16, 2, 2, 2, 2>(X, M, H, W, V, part, n_vt, st);
  else
    e = small_m(M) ? run_tiles<F32, 4, 1, 1, 1>(X, M, H, W, V, part, n_vt, st)
                   : run_tiles<F32, 2, 2, 2, 2>(X, M, H, W, V, part, n_vt, st);
  if (e != hipSuccess) return e;
  lmhead_merge_kernel<<<dim3(static_cast<unsigned>((M + 3) / 4)), dim3(256), 0, st>>>(
      part, M, n_vt, conf, argmax, lse);
  return hipGetLastError();
}

}  // namespace sprint
