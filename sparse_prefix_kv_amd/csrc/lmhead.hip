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

#include <algorithm>
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

// ---------------------------------------------------------------------------
// Large-M path (the prefix pass, M = L rows): 256 x 256 block tile, eight
// waves laid out 2 (vocab) x 4 (tokens), each owning 128 x 64 = 4 x 2 MFMA
// tiles (128 fp32 accumulators), so two waves share each SIMD and one wave's
// MFMAs cover the other's barrier and LDS latency.
//
// Global -> LDS: buffer loads straight into LDS (buffer_load_dwordx4 ... lds,
// 1 KB of contiguous LDS per wave instruction) into two stages of 64-deep K
// chunks (64 KB each: 256 W rows then 256 X rows of 128 bytes).  Every row
// access is one whole 128-byte line, which keeps the L2 request count (the
// L1's in-flight request capacity is the feed limit) at its minimum.  The two
// stages are distinct LDS arrays so the compiler can see that reads of one
// stage do not alias loads into the other; the loop is unrolled by two.
//
// Per chunk: four 16-deep k-slices of 8 MFMAs, the next slice's fragments
// read under the current slice's MFMAs.  Before the last slice's MFMAs each
// wave waits for its own loads of the next chunk and for its fragment reads,
// then a plain s_barrier (no fence: a fence would drain every outstanding
// load) hands the finished stage back; the chunk after next is then loaded
// into it while the last slice's MFMAs run.
//
// LDS layout: the 16-byte slot of k-chunk c in row R is c ^ ((R >> 1) & 7),
// so each 16-lane group of a ds_read_b128 fragment read covers all 64 banks.
//
// Blocks are mapped XCD-aware: block b runs on XCD b % 8, so each XCD gets a
// contiguous range of tile ids, ordered in groups of 8 token tiles so the
// ~32 blocks resident on one XCD share 4 W tiles and 8 X tiles in its L2.
// The grid is one block per CU; a block walks its XCD's range at a stride
// of the blocks per XCD and loads the next tile's first two chunks under the
// current tile's last two chunks.
constexpr int kGB = 256;                     // tile edge (vocab and tokens)
constexpr int kGKC = 64;                     // reduction depth per stage
constexpr int kGStageElems = 2 * kGB * kGKC; // A rows then B rows
constexpr int kGThreads = 512;
constexpr int kXcds = 8;
constexpr int kGroupM = 8;

#define SPRINT_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt immediate: at most n vector-memory ops pending, lgkm unrestricted
constexpr int vm_wait_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
// s_waitcnt immediate: vmcnt(0) and lgkmcnt(0)
constexpr int vm_lgkm_zero_imm() { return (7 << 4); }

// One 64-deep chunk of this wave's rows through buffer loads: instruction j
// fills rows 32*wave + 8*j + lane/8 of the A (W) and B (X) halves of the
// stage.  The swizzled k-chunk a lane fetches only depends on the parity of
// j, so the per-lane part of every address is one of two 32-bit offsets and
// the rest is a wave-uniform scalar offset.  The buffer descriptors span
// exactly W and X, so rows past V or M read as zeros.
__device__ __forceinline__ void gemm_dma(__amdgpu_buffer_rsrc_t rW, __amdgpu_buffer_rsrc_t rX,
                                         uint32_t soA, uint32_t soB, uint32_t rs_bytes,
                                         uint32_t offE, uint32_t offO, uint16_t* stA,
                                         uint16_t* stB) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rW, SPRINT_LDS(stA + j * 512), 16,
                                             (j & 1) ? offO : offE, soA + j * rs_bytes, 0, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rX, SPRINT_LDS(stB + j * 512), 16,
                                             (j & 1) ? offO : offE, soB + j * rs_bytes, 0, 0);
}

// Fragments of one 16-deep k-slice: 4 vocabulary tiles and 2 token tiles.
__device__ __forceinline__ void gemm_frags(const uint16_t* sA, const uint16_t* sB, int so,
                                           bf16x8 (&fa)[4], bf16x8 (&fb)[2]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) fa[i] = as_bf16x8(ld16(sA + i * 32 * kGKC + so));
#pragma unroll
  for (int j = 0; j < 2; ++j) fb[j] = as_bf16x8(ld16(sB + j * 32 * kGKC + so));
}

__device__ __forceinline__ void gemm_mma8(const bf16x8 (&fa)[4], const bf16x8 (&fb)[2],
                                          f32x16 (&acc)[4][2]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = mma32_k16(fa[i], fb[j], acc[i][j]);
}

// Issue order for one slice: MFMAs and fragment reads alternated; the full
// sched_barrier keeps later slices' reads from being hoisted.
__device__ __forceinline__ void gemm_interleave() {
#pragma unroll
  for (int g = 0; g < 6; ++g) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  __builtin_amdgcn_sched_barrier(0);
}

// Tile t of the vocabulary x token grid, in groups of kGroupM token tiles
// per vocabulary tile.
struct GemmTile {
  int vt, v0;
  int64_t t0;
};

__device__ __forceinline__ GemmTile gemm_tile(int t, int n_vt, int n_mt) {
  const int group = kGroupM * n_vt;
  const int first_m = (t / group) * kGroupM;
  const int gm = min(n_mt - first_m, kGroupM);
  const int r_in = t % group;
  const int mt = first_m + r_in % gm;
  const int vt = r_in / gm;
  return GemmTile{vt, vt * kGB, static_cast<int64_t>(mt) * kGB};
}

// Persistent: block b works on XCD b % 8 through the tiles of that XCD's
// range at stride (blocks per XCD), so the blocks resident on one XCD still
// hold consecutive tiles.  The first two K chunks of a block's next tile are
// loaded while the last two chunks of the current one are computed; the
// epilogue starts once they have landed.
__global__ __launch_bounds__(kGThreads) void lmhead_gemm_kernel(
    const uint16_t* __restrict__ X, int64_t M, int H, const uint16_t* __restrict__ W, int V,
    float4* __restrict__ part, int n_vt, int n_mt, int per_xcd) {
  __shared__ __align__(16) uint16_t st0[kGStageElems];
  __shared__ __align__(16) uint16_t st1[kGStageElems];
  __shared__ Stat red[kGB * 2];  // [256 tokens][2 vocab waves]
  __shared__ float4 res[kGB];    // a tile's result per token column
  const int n_tiles = n_vt * n_mt;
  const int xcd = blockIdx.x % kXcds, slots = gridDim.x / kXcds;
  const int tbase = xcd * per_xcd;
  int it = blockIdx.x / kXcds;  // position in the XCD's range
  if (it >= per_xcd || tbase + it >= n_tiles) return;
  GemmTile tile = gemm_tile(tbase + it, n_vt, n_mt);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wv = wave & 1, wt = wave >> 1;
  const int q = lane & 31, hh = lane >> 5;

  // Load plan: instruction j of this wave fills rows r = 32*wave + 8*j + lane/8,
  // slot lane%8, which holds k-chunk (lane%8) ^ ((r>>1)&7); that is
  // (lane&7) ^ ((lane>>4)&7) for even j and the same ^ 4 for odd j.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int c_even = (lane & 7) ^ ((lane >> 4) & 7);
  const uint32_t lrow_bytes = static_cast<uint32_t>(lane >> 3) * H * 2;
  const uint32_t offE = lrow_bytes + c_even * 16;
  const uint32_t offO = lrow_bytes + (c_even ^ 4) * 16;
  const uint32_t rs_bytes = static_cast<uint32_t>(16) * H;    // 8 rows of bf16
  const __amdgpu_buffer_rsrc_t rW = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(W), 0, static_cast<int>(static_cast<int64_t>(V) * H * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rX = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(X), 0, static_cast<int>(M * H * 2), 0x00020000);
  uint32_t soA = static_cast<uint32_t>(tile.v0 + 32 * wave_u) * H * 2;
  uint32_t soB = static_cast<uint32_t>(tile.t0 + 32 * wave_u) * H * 2;
  uint16_t* const dA0 = st0 + wave_u * 4 * 512;
  uint16_t* const dB0 = st0 + kGB * kGKC + wave_u * 4 * 512;
  uint16_t* const dA1 = st1 + wave_u * 4 * 512;
  uint16_t* const dB1 = st1 + kGB * kGKC + wave_u * 4 * 512;

  // Fragment reads: row R = wv*128 + i*32 + q (A) or wt*64 + j*32 + q (B),
  // k-chunk 2*ks + hh at slot (2*ks + hh) ^ ((q >> 1) & 7).
  const int sw = (q >> 1) & 7;
  int so[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) so[ks] = ((2 * ks + hh) ^ sw) * 8;
  const int aoff = (wv * 128 + q) * kGKC;
  const int boff = kGB * kGKC + (wt * 64 + q) * kGKC;

  // H is a multiple of 2 * kGKC, so a tile has an even number of chunks and
  // its chunk 0 always sits in st0
  const int nk = H / kGKC;
  gemm_dma(rW, rX, soA, soB, rs_bytes, offE, offO, dA0, dB0);
  gemm_dma(rW, rX, soA + 2 * kGKC, soB + 2 * kGKC, rs_bytes, offE, offO, dA1, dB1);
  // both chunks: with chunk 1 still pending on entry to the K loop, the
  // compiler can no longer tell the two stages' DMA apart and would wait
  // for every load at the loop head
  __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
  __builtin_amdgcn_s_barrier();

  // the previous tile's result waits in res until the next tile is under way
  bool pend = false;
  GemmTile prev = tile;

  while (true) {
    const int in = it + slots;
    const bool has_next = in < per_xcd && tbase + in < n_tiles;
    GemmTile nt = tile;
    uint32_t nsoA = 0, nsoB = 0;
    if (has_next) {
      nt = gemm_tile(tbase + in, n_vt, n_mt);
      nsoA = static_cast<uint32_t>(nt.v0 + 32 * wave_u) * H * 2;
      nsoB = static_cast<uint32_t>(nt.t0 + 32 * wave_u) * H * 2;
    }
    if (pend && tid < kGB && prev.t0 + tid < M) part[(prev.t0 + tid) * n_vt + prev.vt] = res[tid];
    pend = false;

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    bf16x8 fa0[4], fb0[2], fa1[4], fb1[2];
    gemm_frags(st0 + aoff, st0 + boff, so[0], fa0, fb0);

#define SPRINT_GEMM_STEP(CUR, NXT, DA, DB, U)                                                \
  {                                                                                          \
    const int kc = kb + (U);                                                                 \
    if (kc < nk) {                                                                           \
      gemm_frags(CUR + aoff, CUR + boff, so[1], fa1, fb1);                                   \
      gemm_mma8(fa0, fb0, acc);                                                              \
      gemm_interleave();                                                                     \
      gemm_frags(CUR + aoff, CUR + boff, so[2], fa0, fb0);                                   \
      gemm_mma8(fa1, fb1, acc);                                                              \
      gemm_interleave();                                                                     \
      gemm_frags(CUR + aoff, CUR + boff, so[3], fa1, fb1);                                   \
      gemm_mma8(fa0, fb0, acc);                                                              \
      gemm_interleave();                                                                     \
      __builtin_amdgcn_s_waitcnt(vm_lgkm_zero_imm());                                        \
      __builtin_amdgcn_s_barrier();                                                          \
      if (kc + 2 < nk) {                                                                     \
        const uint32_t k2 = 2u * (kc + 2) * kGKC;                                            \
        gemm_dma(rW, rX, soA + k2, soB + k2, rs_bytes, offE, offO, DA, DB);                  \
      } else if (has_next) {                                                                 \
        const uint32_t k2 = 2u * (kc + 2 - nk) * kGKC;                                       \
        gemm_dma(rW, rX, nsoA + k2, nsoB + k2, rs_bytes, offE, offO, DA, DB);                \
      }                                                                                      \
      if (kc + 1 < nk) gemm_frags(NXT + aoff, NXT + boff, so[0], fa0, fb0);                  \
      gemm_mma8(fa1, fb1, acc);                                                              \
    }                                                                                        \
  }
    for (int kb = 0; kb < nk; kb += 2) {
      SPRINT_GEMM_STEP(st0, st1, dA0, dB0, 0)
      SPRINT_GEMM_STEP(st1, st0, dA1, dB1, 1)
    }
#undef SPRINT_GEMM_STEP

    // the next tile's first two chunks land before the epilogue starts
    // (measured faster than running the epilogue under them)
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
    // Epilogue: per token column fold this wave's 128 vocabulary rows, then
    // the partner half-wave, then the other vocabulary wave through LDS.
    // Per column a lane holds 64 logits (4 tiles x 16); rows ascend with
    // (i, r).  One max, the lowest row holding it (scanning down, so the last
    // match written is the lowest row), then one pass of raw exp2 (arguments
    // <= 0) for the sum.  Rows past V exist only in the last vocabulary tile
    // and are masked to -inf there.
    const int vbase = tile.v0 + wv * 128 + 4 * hh;
    if (tile.v0 + kGB > V) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (vbase + i * 32 + 8 * (r >> 2) + (r & 3) >= V) acc[i][j][r] = -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[i][j][r]);
      // the position (i, r) of the lowest row holding the max as a 6-bit
      // code, an inline constant, so that no row index is held in a
      // register (64 row indices beside the accumulators made the compiler
      // spill); 64 = none (every logit NaN)
      int code = 64;
#pragma unroll
      for (int i = 3; i >= 0; --i)
#pragma unroll
        for (int r = 15; r >= 0; --r) code = acc[i][j][r] == mx ? i * 16 + r : code;
      int am = code == 64 ? INT_MAX
                          : vbase + (code >> 4) * 32 + 8 * ((code >> 2) & 3) + (code & 3);
      float sum = 0.f;
      if (mx != -INFINITY) {
        const float ml = mx * kLog2e;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sum += __builtin_amdgcn_exp2f(fmaf(acc[i][j][r], kLog2e, -ml));
      } else {
        am = INT_MAX;
      }
      Stat st{mx, sum, am};
      Stat other;
      other.m = shfl_xor_f(st.m, 32);
      other.s = shfl_xor_f(st.s, 32);
      other.a = shfl_xor_i(st.a, 32);
      if (hh == 0) {
        merge(st, other);
        red[(wt * 64 + j * 32 + q) * 2 + wv] = st;
      }
    }
    __syncthreads();
    if (tid < kGB) {
      const int c = tid;  // 256 token columns
      Stat st = red[c * 2 + 0];
      merge(st, red[c * 2 + 1]);
      res[c] = make_float4(st.m, st.s, __int_as_float(st.a), 0.f);
    }
    pend = true;
    prev = tile;
    if (!has_next) break;
    // the next tile's chunks 0 and 1 were loaded into st0 and st1 during the
    // last two chunks; red and res are next written after this tile's
    // barriers, res read by the same threads that wrote it
    __builtin_amdgcn_s_waitcnt(vm_lgkm_zero_imm());
    __builtin_amdgcn_s_barrier();
    it = in;
    tile = nt;
    soA = nsoA;
    soB = nsoB;
  }
  if (tid < kGB && prev.t0 + tid < M) part[(prev.t0 + tid) * n_vt + prev.vt] = res[tid];
}

// ---------------------------------------------------------------------------
// Small-M path (a denoising step: M = 32 or 64 block tokens).  The work is
// streaming W once from HBM (V*H*2 bytes against 2*M*V*H flops), so the
// kernel is built around bytes in flight: a block owns 128 vocabulary rows
// and the whole reduction, and streams 64-deep K chunks of those rows (16 KB)
// plus the matching X chunk (4 KB per 32 tokens, an L2 hit) through a ring
// of six LDS stages with buffer loads straight into LDS, five chunks ahead.
// Each wave turns a chunk into 4*NT MFMAs (32 vocabulary rows x 32*NT
// tokens), far below the time the chunk takes to arrive.  Same swizzle and
// epilogue fold as the large-M kernel.
constexpr int kSBV = 128;     // vocabulary rows per block
constexpr int kSStages = 6;

template <int NT>
__global__ __launch_bounds__(256) void lmhead_stream_kernel(const uint16_t* __restrict__ X,
                                                            int64_t M, int H,
                                                            const uint16_t* __restrict__ W, int V,
                                                            float4* __restrict__ part, int n_vt) {
  constexpr int kBT = 32 * NT;
  constexpr int kStElems = (kSBV + kBT) * kGKC;
  __shared__ __align__(16) uint16_t s0[kStElems];
  __shared__ __align__(16) uint16_t s1[kStElems];
  __shared__ __align__(16) uint16_t s2[kStElems];
  __shared__ __align__(16) uint16_t s3[kStElems];
  __shared__ __align__(16) uint16_t s4[kStElems];
  __shared__ __align__(16) uint16_t s5[kStElems];
  __shared__ Stat red[kBT][4];

  const int vt = blockIdx.x;
  const int v0 = vt * kSBV;
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * kBT;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int q = lane & 31, hh = lane >> 5;

  // DMA plan: instruction i of a stage half fills rows 8i + lane/8, slot
  // lane%8 = k-chunk (lane%8) ^ ((row >> 1) & 7), which depends only on the
  // parity of i.  W instructions 4*wave + j, X instructions wave + 4*p.
  const int c_even = (lane & 7) ^ ((lane >> 4) & 7);
  const uint32_t lrow_bytes = static_cast<uint32_t>(lane >> 3) * H * 2;
  const uint32_t offE = lrow_bytes + c_even * 16;
  const uint32_t offO = lrow_bytes + (c_even ^ 4) * 16;
  const uint32_t rs8 = static_cast<uint32_t>(16) * H;        // 8 rows of bf16
  const __amdgpu_buffer_rsrc_t rW = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(W), 0, static_cast<int>(static_cast<int64_t>(V) * H * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rX = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(X), 0, static_cast<int>(M * H * 2), 0x00020000);
  const uint32_t soA = static_cast<uint32_t>(v0 + 32 * wave) * H * 2;
  const uint32_t soB = static_cast<uint32_t>(t0 + 8 * wave) * H * 2;
  const uint32_t offX = (wave & 1) ? offO : offE;
  auto issue = [&](int kc, uint16_t* stage) {
    const uint32_t kb = static_cast<uint32_t>(kc) * (2 * kGKC);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rW, SPRINT_LDS(stage + (4 * wave + j) * 512), 16,
                                               (j & 1) ? offO : offE, soA + j * rs8 + kb, 0,
                                               kCpolNT);
#pragma unroll
    for (int p = 0; p < NT; ++p)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rX, SPRINT_LDS(stage + kSBV * kGKC + (wave + 4 * p) * 512), 16, offX,
          soB + p * 4 * rs8 + kb, 0, 0);
  };

  const int sw = (q >> 1) & 7;
  const int aoff = (32 * wave + q) * kGKC;
  const int boff = kSBV * kGKC + q * kGKC;
  f32x16 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[n][r] = 0.f;
  auto compute = [&](const uint16_t* stage) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int so = ((2 * ks + hh) ^ sw) * 8;
      const bf16x8 a = as_bf16x8(ld16(stage + aoff + so));
#pragma unroll
      for (int n = 0; n < NT; ++n)
        acc[n] = mma32_k16(a, as_bf16x8(ld16(stage + boff + n * 32 * kGKC + so)), acc[n]);
    }
  };

  const int nk = H / kGKC;
  constexpr int kPer = 4 + NT;     // vector-memory instructions per wave per chunk
  if (0 < nk) issue(0, s0);
  if (1 < nk) issue(1, s1);
  if (2 < nk) issue(2, s2);
  if (3 < nk) issue(3, s3);
  if (4 < nk) issue(4, s4);
#define SPRINT_STREAM_STEP(CUR, NXT, U)                                                   \
  {                                                                                       \
    const int kc = kb + (U);                                                              \
    if (kc < nk) {                                                                        \
      const int pend = min(kSStages - 2, nk - 1 - kc);                                    \
      if (pend >= 4)                                                                      \
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(4 * kPer));                                \
      else if (pend == 3)                                                                 \
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(3 * kPer));                                \
      else if (pend == 2)                                                                 \
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(2 * kPer));                                \
      else if (pend == 1)                                                                 \
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(kPer));                                    \
      else                                                                                \
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));                                       \
      __builtin_amdgcn_s_barrier();                                                       \
      if (kc + kSStages - 1 < nk) issue(kc + kSStages - 1, NXT);                          \
      compute(CUR);                                                                       \
    }                                                                                     \
  }
  for (int kb = 0; kb < nk; kb += kSStages) {
    SPRINT_STREAM_STEP(s0, s5, 0)
    SPRINT_STREAM_STEP(s1, s0, 1)
    SPRINT_STREAM_STEP(s2, s1, 2)
    SPRINT_STREAM_STEP(s3, s2, 3)
    SPRINT_STREAM_STEP(s4, s3, 4)
    SPRINT_STREAM_STEP(s5, s4, 5)
  }
#undef SPRINT_STREAM_STEP

  // Epilogue: per token column fold this wave's 32 vocabulary rows, the
  // partner half-wave, then the four waves (vocabulary order) through LDS.
  const int vbase = v0 + 32 * wave + 4 * hh;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    Stat st{-INFINITY, 0.f, INT_MAX};
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int v = vbase + 8 * (r >> 2) + (r & 3);
      if (v < V && acc[n][r] > st.m) {
        st.m = acc[n][r];
        st.a = v;
      }
    }
    if (st.m != -INFINITY) {
      const float ml = st.m * kLog2e;
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (vbase + 8 * (r >> 2) + (r & 3) < V) sum += exp2f(fmaf(acc[n][r], kLog2e, -ml));
      st.s = sum;
    }
    Stat other;
    other.m = shfl_xor_f(st.m, 32);
    other.s = shfl_xor_f(st.s, 32);
    other.a = shfl_xor_i(st.a, 32);
    if (hh == 0) {
      merge(st, other);
      red[n * 32 + q][wave] = st;
    }
  }
  __syncthreads();
  if (threadIdx.x < kBT) {
    const int c = threadIdx.x;
    const int64_t tok = t0 + c;
    if (tok < M) {
      Stat st = red[c][0];
#pragma unroll
      for (int w = 1; w < 4; ++w) merge(st, red[c][w]);
      part[tok * n_vt + vt] = make_float4(st.m, st.s, __int_as_float(st.a), 0.f);
    }
  }
}

// ---------------------------------------------------------------------------
// Small-M path through registers (M <= 64, H a multiple of 256): W is read
// with coalesced non-temporal loads (each wave instruction covers eight whole
// 128-byte row segments, the pattern that streams HBM fastest on MI355X)
// into a ring of four 64-deep chunks per wave, then written to a
// double-buffered LDS stage in the swizzled layout the MFMA fragment reads
// use.  One barrier per chunk: a stage is rewritten two chunks later, after
// every wave has passed the barrier that follows its last read.  The barrier
// is a bare s_barrier after an LDS-only wait, so the global loads in flight
// are never drained.  Same block shape and epilogue as the DMA kernel.
constexpr int kRRing = 4;      // 64-deep chunks in flight per wave

// s_waitcnt immediate: lgkmcnt(0), vmcnt and expcnt unrestricted
constexpr int lgkm_zero_imm() { return 15 | (7 << 4) | (3 << 14); }

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(lgkm_zero_imm());
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int NT, int NW>
__global__ __launch_bounds__(64 * NW) void lmhead_ring_kernel(const uint16_t* __restrict__ X,
                                                              int64_t M, int H,
                                                              const uint16_t* __restrict__ W,
                                                              int V, float4* __restrict__ part,
                                                              int n_vt,
                                                              int32_t* __restrict__ arrive,
                                                              int n_arrive) {
  constexpr int kBV = 32 * NW;               // vocabulary rows per block
  constexpr int kBT = 32 * NT;
  constexpr int kXP = 4 * NT / NW;           // X load instructions per wave per chunk
  static_assert(kXP * NW == 4 * NT, "X rows split evenly over the waves");
  constexpr int kStElems = (kBV + kBT) * kGKC;
  __shared__ __align__(16) uint16_t s0[kStElems];
  __shared__ __align__(16) uint16_t s1[kStElems];
  __shared__ Stat red[kBT][NW];

  const int vt = blockIdx.x;
  const int v0 = vt * kBV;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int q = lane & 31, hh = lane >> 5;
  const int lr = lane >> 3, lc = lane & 7;
  // the fused merge-and-unmask launch that follows counts its finished rows
  // per sequence in `arrive`; this launch starts every count at zero
  if (arrive != nullptr && vt == 0 && static_cast<int>(threadIdx.x) < n_arrive)
    arrive[threadIdx.x] = 0;

  // load plan: W rows 32*wave + 8*j + lr, X rows 8*(wave + NW*p) + lr, chunk
  // lc of each 64-deep slice; LDS slot lc ^ ((row >> 1) & 7).  Rows past V
  // or M are clamped (their results are discarded in the epilogue).
  const uint16_t* wsrc[4];
  int wdst[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int R = 32 * wave + 8 * j + lr;
    wsrc[j] = W + static_cast<int64_t>(min(v0 + R, V - 1)) * H + 8 * lc;
    wdst[j] = R * kGKC + ((lc ^ ((R >> 1) & 7)) << 3);
  }
  const uint16_t* xsrc[kXP];
  int xdst[kXP];
#pragma unroll
  for (int p = 0; p < kXP; ++p) {
    const int R = 8 * (wave + NW * p) + lr;
    xsrc[p] = X + min(static_cast<int64_t>(R), M - 1) * H + 8 * lc;
    xdst[p] = kBV * kGKC + R * kGKC + ((lc ^ ((R >> 1) & 7)) << 3);
  }
  // Each block walks the 64-deep chunks from its own starting chunk and
  // wraps around.  If every block read the same chunk column of its rows at
  // once, the concurrent 128-byte reads would all sit 4 KB apart across W;
  // spreading the blocks over the columns (start = Knuth's multiplicative
  // hash of the block index) streams HBM 10-18% faster, measured at V =
  // 32768 to 163840.  The k order is fixed per block, so results stay
  // reproducible.
  const int nk = H / kGKC;                 // a multiple of kRRing
  const int rot = static_cast<int>((static_cast<uint32_t>(vt) * 2654435761u) >> 16) % nk;
  u32x4 rw[kRRing][4], rx[kRRing][kXP];
  auto load = [&](int slot, int kc0) {
    const int kc = kc0 + rot < nk ? kc0 + rot : kc0 + rot - nk;
#pragma unroll
    for (int j = 0; j < 4; ++j) rw[slot][j] = ld16_nt(wsrc[j] + kc * kGKC);
#pragma unroll
    for (int p = 0; p < kXP; ++p) rx[slot][p] = ld16(xsrc[p] + kc * kGKC);
  };
  auto put = [&](int slot, uint16_t* stage) {
#pragma unroll
    for (int j = 0; j < 4; ++j) st16(stage + wdst[j], rw[slot][j]);
#pragma unroll
    for (int p = 0; p < kXP; ++p) st16(stage + xdst[p], rx[slot][p]);
  };

  const int sw = (q >> 1) & 7;
  const int aoff = (32 * wave + q) * kGKC;
  const int boff = kBV * kGKC + q * kGKC;
  f32x16 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[n][r] = 0.f;
  auto compute = [&](const uint16_t* stage) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int so = ((2 * ks + hh) ^ sw) * 8;
      const bf16x8 a = as_bf16x8(ld16(stage + aoff + so));
#pragma unroll
      for (int n = 0; n < NT; ++n)
        acc[n] = mma32_k16(a, as_bf16x8(ld16(stage + boff + n * 32 * kGKC + so)), acc[n]);
    }
  };

#pragma unroll
  for (int p = 0; p < kRRing; ++p) load(p, p);
  for (int c0 = 0; c0 < nk - kRRing; c0 += kRRing) {
#pragma unroll
    for (int p = 0; p < kRRing; ++p) {
      uint16_t* stage = (p & 1) ? s1 : s0;
      put(p, stage);
      load(p, c0 + kRRing + p);
      lds_barrier();
      compute(stage);
    }
  }
#pragma unroll
  for (int p = 0; p < kRRing; ++p) {
    uint16_t* stage = (p & 1) ? s1 : s0;
    put(p, stage);
    lds_barrier();
    compute(stage);
  }

  const int vbase = v0 + 32 * wave + 4 * hh;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    Stat st{-INFINITY, 0.f, INT_MAX};
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int v = vbase + 8 * (r >> 2) + (r & 3);
      if (v < V && acc[n][r] > st.m) {
        st.m = acc[n][r];
        st.a = v;
      }
    }
    if (st.m != -INFINITY) {
      const float ml = st.m * kLog2e;
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (vbase + 8 * (r >> 2) + (r & 3) < V) sum += exp2f(fmaf(acc[n][r], kLog2e, -ml));
      st.s = sum;
    }
    Stat other;
    other.m = shfl_xor_f(st.m, 32);
    other.s = shfl_xor_f(st.s, 32);
    other.a = shfl_xor_i(st.a, 32);
    if (hh == 0) {
      merge(st, other);
      red[n * 32 + q][wave] = st;
    }
  }
  __syncthreads();
  if (threadIdx.x < kBT) {
    const int c = threadIdx.x;
    if (c < M) {
      Stat st = red[c][0];
#pragma unroll
      for (int w = 1; w < NW; ++w) merge(st, red[c][w]);
      part[static_cast<int64_t>(c) * n_vt + vt] = make_float4(st.m, st.s, __int_as_float(st.a), 0.f);
    }
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

// Small M: one 256-thread block per row, so a row's tiles are read by 256
// threads at once (each folds tiles t = tid, tid + 256, ... in order, four
// loads in flight), then a fixed butterfly in each wave and the four waves in
// order.  The fold order depends only on n_vt: results are reproducible.
__global__ __launch_bounds__(256) void lmhead_merge_row_kernel(const float4* __restrict__ part,
                                                               int n_vt,
                                                               float* __restrict__ conf,
                                                               int32_t* __restrict__ argmax,
                                                               float* __restrict__ lse) {
  __shared__ Stat wst[4];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const float4* pr = part + row * n_vt;
  Stat st{-INFINITY, 0.f, INT_MAX};
  for (int t0 = tid; t0 < n_vt; t0 += 4 * 256) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = t0 + 256 * u;
      v[u] = t < n_vt ? pr[t] : make_float4(-INFINITY, 0.f, __int_as_float(INT_MAX), 0.f);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) merge(st, Stat{v[u].x, v[u].y, __float_as_int(v[u].z)});
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    Stat o;
    o.m = shfl_xor_f(st.m, m);
    o.s = shfl_xor_f(st.s, m);
    o.a = shfl_xor_i(st.a, m);
    Stat lo = (lane & m) ? o : st;
    const Stat hi = (lane & m) ? st : o;
    merge(lo, hi);
    st = lo;
  }
  if (lane == 0) wst[wave] = st;
  __syncthreads();
  if (tid == 0) {
    Stat r = wst[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) merge(r, wst[w]);
    conf[row] = 1.f / r.s;
    argmax[row] = r.a;
    if (lse) lse[row] = r.m + logf(r.s);
  }
}

// The last two launches of a denoising step in one (for the register-ring
// path, M = nseq * Lq <= 64): the merge of lmhead_merge_row_kernel for row
// blockIdx.x, then, in the block that finishes a sequence's last row, the
// unmasking step of that sequence (unmask_rule, as unmask_select applies
// it).  Each block stores its row's confidence and argmax with agent-scope
// atomic stores, which are coherent across the XCDs' L2 caches, waits for
// them to complete, and only then counts the row in arrive[sequence]; the
// block that sees the count reach Lq reads the sequence's rows back with
// agent-scope atomic loads.  No fence is needed (an agent-scope release or
// acquire writes back or invalidates a whole L2), and no block waits for
// another.  Results are bitwise those of the two separate launches.
__global__ __launch_bounds__(256) void lmhead_merge_unmask_kernel(
    const float4* __restrict__ part, int n_vt, float* conf, int32_t* argmax, int Lq, float tau,
    int steps_left, uint8_t* __restrict__ masked, int32_t* __restrict__ tokens,
    int32_t* __restrict__ n_accepted, int32_t* __restrict__ arrive) {
  __shared__ Stat wst[4];
  __shared__ int s_last;
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const float4* pr = part + row * n_vt;
  Stat st{-INFINITY, 0.f, INT_MAX};
  for (int t0 = tid; t0 < n_vt; t0 += 4 * 256) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = t0 + 256 * u;
      v[u] = t < n_vt ? pr[t] : make_float4(-INFINITY, 0.f, __int_as_float(INT_MAX), 0.f);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) merge(st, Stat{v[u].x, v[u].y, __float_as_int(v[u].z)});
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    Stat o;
    o.m = shfl_xor_f(st.m, m);
    o.s = shfl_xor_f(st.s, m);
    o.a = shfl_xor_i(st.a, m);
    Stat lo = (lane & m) ? o : st;
    const Stat hi = (lane & m) ? st : o;
    merge(lo, hi);
    st = lo;
  }
  if (lane == 0) wst[wave] = st;
  __syncthreads();
  const int seq = static_cast<int>(row / Lq);
  if (tid == 0) {
    Stat r = wst[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) merge(r, wst[w]);
    __hip_atomic_store(conf + row, 1.f / r.s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(argmax + row, r.a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // both stores are complete before the row is counted
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const int before = __hip_atomic_fetch_add(arrive + seq, 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    s_last = before == Lq - 1 ? 1 : 0;
  }
  __syncthreads();
  if (s_last == 0 || wave != 0) return;
  // every row of the sequence was stored before it was counted
  const int64_t base = static_cast<int64_t>(seq) * Lq;
  const int i = lane;
  const int64_t at = base + (i < Lq ? i : Lq - 1);
  const float c_ld = __hip_atomic_load(conf + at, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int32_t a_ld = __hip_atomic_load(argmax + at, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint8_t m_ld = masked[at];
  unmask_rule(c_ld, m_ld, a_ld, i, Lq, tau, steps_left, base, masked, tokens, n_accepted + seq);
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

// Kernel choice.  bf16, M <= 64 streams W once: through the register ring
// (H a multiple of 256), else through buffer-to-LDS loads (W and X each
// addressable by a 32-bit buffer descriptor).  Larger M runs the 256 x 256
// tile GEMM (H in whole 128-deep pairs of chunks).  Anything else (fp32,
// odd shapes) takes the generic tile kernel: 32 tokens x 128 vocabulary rows
// per block for M <= 32, 128 x 128 tiles otherwise.
inline bool small_m(int64_t M) { return M <= 32; }
inline bool bf16_buffers(int64_t M, int H, int V, int dtype) {
  return dtype == 1 && static_cast<int64_t>(V) * H * 2 < (int64_t(1) << 31) &&
         M * H * 2 < (int64_t(1) << 31);
}
inline bool ring_path(int64_t M, int H, int V, int dtype) {
  return dtype == 1 && M <= 64 && H % (kGKC * kRRing) == 0;
}
// Waves (32 vocabulary rows each) per ring block.  With the staggered chunk
// order, four-wave blocks stream faster than two-wave ones at every
// vocabulary size measured (V = 32768 to 163840, M = 32 and 64).
constexpr int kRingWaves = 4;
inline bool stream_path(int64_t M, int H, int V, int dtype) {
  return bf16_buffers(M, H, V, dtype) && M <= 64 && H % kGKC == 0;
}
inline bool gemm_path(int64_t M, int H, int V, int dtype) {
  return bf16_buffers(M, H, V, dtype) && M > 64 && H % (2 * kGKC) == 0;
}
inline int tile_bv(int64_t M, int H, int V, int dtype) {
  if (ring_path(M, H, V, dtype)) return 32 * kRingWaves;
  return gemm_path(M, H, V, dtype) ? kGB : 128;
}
}  // namespace

size_t lmhead_ws_bytes(int64_t M, int H, int V, int dtype) {
  const int n_vt = (V + tile_bv(M, H, V, dtype) - 1) / tile_bv(M, H, V, dtype);
  return align_up(static_cast<size_t>(M) * n_vt * sizeof(float4), 256);
}

hipError_t launch_lmhead(const void* X, int64_t M, int H, const void* W, int V, int dtype,
                         float* conf, int32_t* argmax, float* lse, void* ws, hipStream_t st) {
  const int n_vt = (V + tile_bv(M, H, V, dtype) - 1) / tile_bv(M, H, V, dtype);
  float4* part = static_cast<float4*>(ws);
  hipError_t e;
  if (ring_path(M, H, V, dtype)) {
    const uint16_t* x16 = static_cast<const uint16_t*>(X);
    const uint16_t* w16 = static_cast<const uint16_t*>(W);
    if (M <= 32)
      lmhead_ring_kernel<1, kRingWaves>
          <<<dim3(n_vt), dim3(64 * kRingWaves), 0, st>>>(x16, M, H, w16, V, part, n_vt,
                                                          nullptr, 0);
    else
      lmhead_ring_kernel<2, kRingWaves>
          <<<dim3(n_vt), dim3(64 * kRingWaves), 0, st>>>(x16, M, H, w16, V, part, n_vt,
                                                          nullptr, 0);
    e = hipGetLastError();
  } else if (stream_path(M, H, V, dtype)) {
    const dim3 grid(n_vt);
    if (M <= 32)
      lmhead_stream_kernel<1><<<grid, dim3(256), 0, st>>>(static_cast<const uint16_t*>(X), M, H,
                                                         static_cast<const uint16_t*>(W), V, part,
                                                         n_vt);
    else
      lmhead_stream_kernel<2><<<grid, dim3(256), 0, st>>>(static_cast<const uint16_t*>(X), M, H,
                                                         static_cast<const uint16_t*>(W), V, part,
                                                         n_vt);
    e = hipGetLastError();
  } else if (gemm_path(M, H, V, dtype)) {
    const int n_mt = static_cast<int>((M + kGB - 1) / kGB);
    const int per_xcd = (n_vt * n_mt + kXcds - 1) / kXcds;
    // one block per CU (the stages take most of the LDS), at most one per tile
    int dev = 0, cus = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int slots = std::max(1, std::min(cus / kXcds, per_xcd));
    lmhead_gemm_kernel<<<dim3(slots * kXcds), dim3(kGThreads), 0, st>>>(
        static_cast<const uint16_t*>(X), M, H, static_cast<const uint16_t*>(W), V, part, n_vt,
        n_mt, per_xcd);
    e = hipGetLastError();
  } else if (dtype == 1)
    e = small_m(M) ? run_tiles<BF16, 4, 1, 1, 1>(X, M, H, W, V, part, n_vt, st)
                   : run_tiles<BF16, 2, 2, 2, 2>(X, M, H, W, V, part, n_vt, st);
  else
    e = small_m(M) ? run_tiles<F32, 4, 1, 1, 1>(X, M, H, W, V, part, n_vt, st)
                   : run_tiles<F32, 2, 2, 2, 2>(X, M, H, W, V, part, n_vt, st);
  if (e != hipSuccess) return e;
  if (M <= 256)
    lmhead_merge_row_kernel<<<dim3(static_cast<unsigned>(M)), dim3(256), 0, st>>>(
        part, n_vt, conf, argmax, lse);
  else
    lmhead_merge_kernel<<<dim3(static_cast<unsigned>((M + 3) / 4)), dim3(256), 0, st>>>(
        part, M, n_vt, conf, argmax, lse);
  return hipGetLastError();
}

size_t lmhead_unmask_ws_bytes(int nseq, int Lq, int H, int V, int dtype) {
  const int64_t M = static_cast<int64_t>(nseq) * Lq;
  return lmhead_ws_bytes(M, H, V, dtype) + align_up(static_cast<size_t>(nseq) * 4, 256);
}

hipError_t launch_lmhead_unmask(const void* X, int nseq, int Lq, int H, const void* W, int V,
                                int dtype, float* conf, int32_t* argmax, float tau,
                                int steps_left, uint8_t* masked, int32_t* tokens,
                                int32_t* n_accepted, void* ws, hipStream_t st) {
  const int64_t M = static_cast<int64_t>(nseq) * Lq;
  if (!ring_path(M, H, V, dtype)) {
    // no fused form for this shape: the two calls, in order
    const hipError_t e =
        launch_lmhead(X, M, H, W, V, dtype, conf, argmax, nullptr, ws, st);
    if (e != hipSuccess) return e;
    return launch_unmask(conf, argmax, nseq, Lq, tau, steps_left, masked, tokens, n_accepted, st);
  }
  const int n_vt = (V + tile_bv(M, H, V, dtype) - 1) / tile_bv(M, H, V, dtype);
  float4* part = static_cast<float4*>(ws);
  int32_t* arrive =
      reinterpret_cast<int32_t*>(static_cast<char*>(ws) + lmhead_ws_bytes(M, H, V, dtype));
  const uint16_t* x16 = static_cast<const uint16_t*>(X);
  const uint16_t* w16 = static_cast<const uint16_t*>(W);
  if (M <= 32)
    lmhead_ring_kernel<1, kRingWaves>
        <<<dim3(n_vt), dim3(64 * kRingWaves), 0, st>>>(x16, M, H, w16, V, part, n_vt, arrive,
                                                        nseq);
  else
    lmhead_ring_kernel<2, kRingWaves>
        <<<dim3(n_vt), dim3(64 * kRingWaves), 0, st>>>(x16, M, H, w16, V, part, n_vt, arrive,
                                                        nseq);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  lmhead_merge_unmask_kernel<<<dim3(static_cast<unsigned>(M)), dim3(256), 0, st>>>(
      part, n_vt, conf, argmax, Lq, tau, steps_left, masked, tokens, n_accepted, arrive);
  return hipGetLastError();
}

}  // namespace sprint
