// Block attention of one denoising step: the block's queries attend without
// a mask to [prefix KV cache ; the block's own K/V] (LLaDA2.0-Uni: SPRINT
// "Sparse Prefix Retention" -- each step attends to the (pruned) prefix --
// and the block notation of "BDLM Loss").  GQA: query head h reads KV head
// floor(h*Hkv/Hq).
//
// Work decomposition (split-KV, flash-decoding style):
//   a block owns one KV head of one sequence and one contiguous key range,
//   and ALL R = (Hq/Hkv)*Lq query rows that read that head, as R/32 waves of
//   32 rows.  Every K/V byte is fetched once per step and shared through LDS.
//   The block's own K/V (the block keys) are the last tiles of the last range.
// K/V stages of 64 keys (two 32-key tiles) arrive by buffer loads straight
//   into LDS (buffer_load_dwordx4 ... lds, non-temporal).  bf16 blocks of up
//   to four waves run two blocks per CU, each with a ring of two stages (one
//   in flight) and at most 256 registers per lane, so every SIMD interleaves
//   two waves; other shapes use one block per CU with a ring of four stages
//   (three in flight).  The stages are distinct LDS arrays and the loop is
//   unrolled over them, so the compiler can see that reads of one stage do
//   not alias loads into another; each wave waits (vmcnt) for its own loads
//   of a stage, then a plain s_barrier (no fence, which would drain every
//   outstanding load) publishes it.
// Per tile and wave:
//   S^T = K Q^T on MFMA 32x32x16 (A = key rows from LDS, B = the wave's
//   queries held in registers).  The accumulator gives each lane one query
//   column and 16 keys, so the online-softmax max needs one cross-half swap
//   and the row sum stays lane-local.
//   O^T += V^T P^T with the probabilities taken straight from the S^T
//   accumulator as the B operand.  For bf16 the V^T operand comes from the
//   natural [key][d] layout through transposing LDS reads (ds_read_b64_tr_b16).
// LDS layouts are XOR-swizzled per 16-byte chunk (DMA writes are contiguous,
//   so no padding): K chunk c of row r sits in slot c ^ f(r) so the sixteen
//   rows of a ds_read_b128 pass cover all banks; bf16 V chunk c sits in slot
//   c ^ 4*(r & 3) (c ^ 4*((r >> 1) & 1) for 128-byte rows) so the four rows of
//   a transposing-read pass land on disjoint banks.
// A single key range writes O directly; otherwise each wave writes its rows'
//   partial (o / l in fp32 for fp32 inputs; for bf16 inputs in fp16 times a
//   power-of-two row scale that keeps every row in fp16's range, plus m in
//   log2 units, l and the scale) and a combine kernel merges the ranges.  The
//   last range of a sequence runs to its end, so a sequence longer than the
//   planned cache length is still attended in full.
#include <math.h>

#include <mutex>
#include <type_traits>

#include "sprint_device.hpp"
#include "sprint_internal.hpp"

namespace sprint {

// Key-range partials of block_attend_noalloc: a fixed device array (each GPU
// the library runs on holds its own copy until the process ends).  Host code
// never uses the array's name as an address: its device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) char scratch[kAttendScratchBytes];

namespace {

constexpr int kKT = 32;       // keys per MFMA tile (one S^T accumulator)
constexpr int kStages = 4;    // LDS ring depth

typedef _Float16 half_t;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

struct AttnArgs {
  const char* Q;
  const char* Kp;
  const char* Vp;
  const int32_t* cu_kv;
  const char* Kb;
  const char* Vb;
  char* O;
  void* part_o;    // [nseq*Hkv*n_splits*R, D] fp16 (bf16 inputs) or fp32: o / l, times 2^-e
  float* part_ml;  // [nseq*Hkv*n_splits*R, 4]  (m in log2 units, l, 2^e, unused)
  int nseq, Lq, Hq, Hkv, G, R, n_splits, kps, has_block, n_rg;
  int64_t total_kv;
  float scale_log2;
};

__device__ __forceinline__ f32x16 mma(const bf16x8& a, const bf16x8& b, f32x16 c) {
  return mma32_k16(a, b, c);
}
struct F8 {
  float v[8];
};
__device__ __forceinline__ f32x16 mma(const F8& a, const F8& b, f32x16 c) {
  return mma32_k16(a.v, b.v, c);
}

#define SPRINT_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt immediate: at most n vector-memory ops pending (clamped to the
// 6-bit field: waiting for fewer is always safe), lgkm unrestricted
constexpr int vm_wait_imm(int n) {
  return n > 63 ? vm_wait_imm(63) : (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14);
}

// Geometry of one pipeline stage (KS keys) for element type T and head dim D.
template <typename T, int D, int KS>
struct TileGeo {
  using S = typename T::storage;
  static constexpr bool kBf16 = sizeof(S) == 2;
  static constexpr int kRowBytes = D * static_cast<int>(sizeof(S));
  static constexpr int kChunks = kRowBytes / 16;              // 16-byte chunks per row
  static constexpr int kTileBytes = KS * kRowBytes;           // K (or V) rows of a stage
  static constexpr int kInstr = kTileBytes / 1024;            // 1 KB DMA instructions per tile
  static constexpr int kRowsPerInstr = 1024 / kRowBytes;
  // K: a ds_read_b128 pass reads 16 consecutive rows at one chunk; rows of
  // 256+ bytes start on bank 0, 128-byte rows alternate halves
  __host__ __device__ static constexpr int k_swz(int r) {
    return kChunks >= 16 ? (r & 15) : ((r >> 1) & (kChunks - 1));
  }
  // V (bf16 only): a transposing b64 pass reads 4 consecutive rows at 4 chunks
  __host__ __device__ static constexpr int v_swz(int r) {
    return kChunks >= 16 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
  }
};

// Max / sum of lanes q and q + 32 (gfx950 v_permlane32_swap: one VALU op
// instead of an LDS permute).  Both lanes of a pair get the same value.
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <typename T>
struct Frag;
template <>
struct Frag<BF16> {
  using type = bf16x8;
  // 8 consecutive elements starting at element e (multiple of 8) of a row
  // whose chunks are swizzled by `sw`
  __device__ static type load_row(const uint16_t* row, int e, int sw) {
    return as_bf16x8(ld16(row + (((e >> 3) ^ sw) << 3)));
  }
  __device__ static type zero() { return as_bf16x8(u32x4{0u, 0u, 0u, 0u}); }
  __device__ static type from8(const float (&x)[8]) {
    u32x4 u;
    u[0] = pack_bf16x2(x[0], x[1]);
    u[1] = pack_bf16x2(x[2], x[3]);
    u[2] = pack_bf16x2(x[4], x[5]);
    u[3] = pack_bf16x2(x[6], x[7]);
    return as_bf16x8(u);
  }
  __device__ static type qload(const uint16_t* p) { return as_bf16x8(ld16(p)); }
};
template <>
struct Frag<F32> {
  using type = F8;
  __device__ static type load_row(const float* row, int e, int sw) {
    type r;
    const u32x4 a = ld16(row + (((e >> 2) ^ sw) << 2));
    const u32x4 b = ld16(row + ((((e >> 2) + 1) ^ sw) << 2));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r.v[i] = __uint_as_float(a[i]);
      r.v[4 + i] = __uint_as_float(b[i]);
    }
    return r;
  }
  __device__ static type zero() {
    type r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r.v[i] = 0.f;
    return r;
  }
  __device__ static type from8(const float (&x)[8]) {
    type r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r.v[i] = x[i];
    return r;
  }
  __device__ static type qload(const float* p) {
    type r;
    const u32x4 a = ld16(p), b = ld16(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r.v[i] = __uint_as_float(a[i]);
      r.v[4 + i] = __uint_as_float(b[i]);
    }
    return r;
  }
};

// DMA of one tile (K or V rows) into a stage: this wave's instructions
// j = wave, wave + NW, ... (clamped to the last one: a repeat rewrites the
// same bytes).  Lane L of instruction j fills LDS bytes 1024*j + 16*L.
// `voff[p]` is that lane's byte offset within the tile (loop invariant),
// `soff` the tile's uniform offset.
__device__ __forceinline__ void tile_dma(__amdgpu_buffer_rsrc_t rs, uint32_t soff,
                                         const uint32_t* voff, char* stage, int wave, int nw,
                                         int np, int ni) {
#pragma unroll
  for (int p = 0; p < np; ++p) {
    const int j = wave + nw * p < ni ? wave + nw * p : ni - 1;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, SPRINT_LDS(stage + j * 1024), 16, voff[p], soff,
                                             0, kCpolNT);
  }
}

// ---------------------------------------------------------------- output rows
// A wave's 32 output rows leave through LDS: each lane stores its 4-column
// groups of row q (XOR-swizzled 16-byte chunks), then every lane copies one
// 16-byte chunk of a whole row, so global stores are full contiguous rows
// instead of 8-byte pieces scattered over 32 rows.
template <typename E>
__device__ __forceinline__ E out_cvt(float x);
template <>
__device__ __forceinline__ uint16_t out_cvt<uint16_t>(float x) {   // bf16 bits
  return f32_to_bf16(x);
}
template <>
__device__ __forceinline__ half_t out_cvt<half_t>(float x) {
  return static_cast<half_t>(x);
}

template <typename E, int D>
struct RowGeo {
  static constexpr int kCE = 16 / static_cast<int>(sizeof(E));   // elements per chunk
  static constexpr int kNC = D / kCE;                             // chunks per row
  static constexpr int kSw = kNC >= 16 ? 15 : kNC - 1;
  static constexpr int kRowBytes = D * static_cast<int>(sizeof(E));
  static constexpr int kWaveBytes = 32 * kRowBytes;
};

template <typename E, int D>
__device__ __forceinline__ void stage_rows(char* reg, const f32x16 (&acc)[D / 32], float inv,
                                           int q, int hh) {
  using G = RowGeo<E, D>;
  char* row = reg + q * G::kRowBytes;
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = 32 * mt + 8 * r4 + 4 * hh;     // first of 4 consecutive columns
      const int c = d / G::kCE, e = d % G::kCE;
      char* dst = row + ((c ^ (q & G::kSw)) * 16) + e * static_cast<int>(sizeof(E));
      if constexpr (sizeof(E) == 2) {
        E v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = out_cvt<E>(acc[mt][4 * r4 + i] * inv);
        *reinterpret_cast<uint2*>(dst) = __builtin_bit_cast(uint2, v);
      } else {
        *reinterpret_cast<f32x4*>(dst) =
            f32x4{acc[mt][4 * r4] * inv, acc[mt][4 * r4 + 1] * inv, acc[mt][4 * r4 + 2] * inv,
                  acc[mt][4 * r4 + 3] * inv};
      }
    }
}

// Copy the first `nrows` staged rows to global memory; row_ptr(r) gives the
// destination of row r.
template <typename E, int D, typename F>
__device__ __forceinline__ void flush_rows(const char* reg, int lane, int nrows, F row_ptr) {
  using G = RowGeo<E, D>;
  constexpr int kRowsPer = 64 / G::kNC;
  const int cc = lane % G::kNC, r0 = lane / G::kNC;
#pragma unroll
  for (int it = 0; it < 32 / kRowsPer; ++it) {
    const int rr = it * kRowsPer + r0;
    if (rr < nrows)
      st16(row_ptr(rr) + cc * 16, ld16(reg + rr * G::kRowBytes + ((cc ^ (rr & G::kSw)) * 16)));
  }
}

// STG = 4: one block per CU, a four-stage ring (three stages in flight).
// STG = 2: two blocks per CU, each with a two-stage ring (one stage in
//   flight) and at most 256 registers per lane.
template <typename T, int D, int NW, int NSUB, int STG>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(STG == 2 ? 2 : 1)))
void attend_split_kernel(AttnArgs args) {
  using S = typename T::storage;
  using FR = Frag<T>;
  constexpr int KS = kKT * NSUB;                          // keys per pipeline stage
  using GEO = TileGeo<T, D, KS>;
  constexpr bool kBf16 = GEO::kBf16;
  constexpr int kNI = GEO::kInstr;
  constexpr int kNWT = NW;                               // waves in the block
  constexpr int kP = (kNI + kNWT - 1) / kNWT;            // DMA instructions per wave per tensor
  constexpr int kStageBytes = 2 * GEO::kTileBytes;       // K tile then V tile
  __shared__ __align__(16) char st0[kStageBytes];
  __shared__ __align__(16) char st1[kStageBytes];
  constexpr int kRing = STG;
  __shared__ __align__(16) char st2[kRing == 4 ? kStageBytes : 16];
  __shared__ __align__(16) char st3[kRing == 4 ? kStageBytes : 16];

  const int split = blockIdx.x % args.n_splits;
  const int g = (blockIdx.x / args.n_splits) % args.Hkv;
  const int seq = blockIdx.x / (args.n_splits * args.Hkv);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rw = wave;                                 // row wave
  const int lane = threadIdx.x & 63;
  const int q = lane & 31, hh = lane >> 5;

  const int64_t kv_begin = args.cu_kv[seq];
  const int kv_len = args.cu_kv[seq + 1] - args.cu_kv[seq];
  const int n_keys = kv_len + (args.has_block ? args.Lq : 0);
  const int k0 = min(n_keys, split * args.kps);
  // the last range runs to the sequence's end, whatever the planned length,
  // so a sequence longer than the plan assumed is covered (only slower)
  const int k1 = split == args.n_splits - 1 ? n_keys : min(n_keys, k0 + args.kps);
  // tiles: the range's prefix keys [pk0, pk1), then its block keys [bk0, bk1)
  const int pk0 = min(k0, kv_len), pk1 = min(k1, kv_len);
  const int bk0 = max(k0, kv_len) - kv_len, bk1 = max(k1, kv_len) - kv_len;
  const int n_ptiles = (pk1 - pk0 + KS - 1) / KS;
  const int n_btiles = (bk1 - bk0 + KS - 1) / KS;
  const int nt = n_ptiles + n_btiles;

  const int rho = rw * 32 + q;
  const bool row_ok = rho < args.R;
  const int gi = row_ok ? rho / args.Lq : 0, qi = row_ok ? rho % args.Lq : 0;
  const int head = g * args.G + gi;

  // Query fragments: lane (q, half) holds row rho, dims [16*ds + 8*half, +8).
  typename FR::type qf[D / 16];
  {
    const S* qrow = reinterpret_cast<const S*>(args.Q) +
                    ((static_cast<int64_t>(seq) * args.Lq + qi) * args.Hq + head) * D;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds)
      qf[ds] = row_ok ? FR::qload(qrow + 16 * ds + 8 * hh) : FR::zero();
  }

  // Buffer descriptors over the prefix cache or the block's own K/V (reads
  // past either return zeros).  The descriptor of a tile is built from the
  // selected base pointer and size, both wave-uniform scalars: selecting
  // between two finished descriptors instead makes the compiler keep them in
  // scratch memory and drain every outstanding load before each tile.
  const int64_t row_stride = static_cast<int64_t>(args.Hkv) * GEO::kRowBytes;
  const int pbytes = static_cast<int>(args.total_kv * row_stride);
  const int bbytes = args.has_block
                         ? static_cast<int>(static_cast<int64_t>(args.nseq) * args.Lq * row_stride)
                         : 0;
  // per-lane byte offsets inside a tile: row * stride + swizzled chunk
  uint32_t vK[kP], vV[kP];
#pragma unroll
  for (int p = 0; p < kP; ++p) {
    const int j = wave + kNWT * p < kNI ? wave + kNWT * p : kNI - 1;
    const int row = j * GEO::kRowsPerInstr + lane / GEO::kChunks;
    const int slot = lane % GEO::kChunks;
    const int ck = slot ^ GEO::k_swz(row);
    const int cv = kBf16 ? (slot ^ GEO::v_swz(row)) : ck;
    vK[p] = static_cast<uint32_t>(row * row_stride + ck * 16);
    vV[p] = static_cast<uint32_t>(row * row_stride + cv * 16);
  }
  const uint32_t head_off = static_cast<uint32_t>(g * GEO::kRowBytes);
  const uint32_t pre_base = static_cast<uint32_t>((kv_begin + pk0) * row_stride) + head_off;
  const uint32_t blk_base =
      static_cast<uint32_t>((static_cast<int64_t>(seq) * args.Lq + bk0) * row_stride) + head_off;
  auto issue = [&](int t, char* stage) {
    const bool pre = t < n_ptiles;
    const char* kb = pre ? args.Kp : args.Kb;
    const char* vb = pre ? args.Vp : args.Vb;
    const int nb = pre ? pbytes : bbytes;
    const uint32_t so = (pre ? pre_base : blk_base) +
                        static_cast<uint32_t>((pre ? t : t - n_ptiles) * KS * row_stride);
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kb), 0, nb, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vb), 0, nb, 0x00020000);
    tile_dma(rk, so, vK, stage, wave, kNWT, kP, kNI);
    tile_dma(rv, so, vV, stage + GEO::kTileBytes, wave, kNWT, kP, kNI);
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc_o[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[mt][r] = 0.f;

  // K fragment reads: row q, chunk (16*ds + 8*hh) / chunk-elements
  const int ksw = GEO::k_swz(q);
  // bf16 V transposed reads: source lane i = lane & 15 of group G = lane >> 4
  // points at key 4*hh + (i >> 2), column 16*(G & 1) + 4*(i & 3) of a 32-column
  // slab; lane j of the group then receives column j of those four keys.
  const int vrow = 4 * hh + ((lane & 15) >> 2);
  const int vcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // One stage: NSUB independent 32-key S^T accumulators (their MFMA chains
  // interleave), one softmax update over all NSUB*32 keys, then P V.
  auto compute = [&](const char* stage, int t) {
    const S* sK = reinterpret_cast<const S*>(stage);
    const S* sV = reinterpret_cast<const S*>(stage + GEO::kTileBytes);
    const int valid = t < n_ptiles ? min(KS, pk1 - pk0 - t * KS)
                                   : min(KS, bk1 - bk0 - (t - n_ptiles) * KS);
    // S^T[key][query]; the K swizzle of row 32u + q equals that of row q
    f32x16 s[NSUB];
#pragma unroll
    for (int u = 0; u < NSUB; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[u][r] = 0.f;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds)
#pragma unroll
      for (int u = 0; u < NSUB; ++u)
        s[u] = mma(FR::load_row(sK + (32 * u + q) * D, 16 * ds + 8 * hh, ksw), qf[ds], s[u]);
    // online softmax in log2 units: m is kept scaled by scale*log2(e) (> 0)
    const float c = args.scale_log2;
    if (valid < KS) {
#pragma unroll
      for (int u = 0; u < NSUB; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * u + 8 * (r >> 2) + 4 * hh + (r & 3) >= valid) s[u][r] = -INFINITY;
    }
    float tmax = s[0][0];
#pragma unroll
    for (int u = 0; u < NSUB; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[u][r]);
    tmax = pair_max(tmax) * c;
    // Lazy rescaling: the reference maximum m_run moves only when a key
    // exceeds it by more than 2^8, so probabilities stay <= 256 (exact in
    // fp32 sums, and bf16 keeps its relative precision at any magnitude) and
    // the O rescale, which some lane of 32 queries would otherwise trigger on
    // almost every stage, becomes rare.  o = acc / l is independent of the
    // reference; the partials carry it as their m.
    const bool grow = tmax > m_run + 8.f;
    if (__ballot(grow)) {
      const float m_up = grow ? tmax : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_up);
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[mt][r] *= alpha;
      m_run = m_up;
    }
    const float m_new = m_run;
    float p[NSUB][16];
#pragma unroll
    for (int u = 0; u < NSUB; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[u][r] = __builtin_amdgcn_exp2f(fmaf(s[u][r], c, -m_new));
        l_run += p[u][r];
      }
    // O^T[d][query] += sum_key V[key][d] P[query][key]
#pragma unroll
    for (int u = 0; u < NSUB; ++u)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        float pk8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pk8[e] = p[u][8 * ks + e];
        const typename FR::type bq = FR::from8(pk8);
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) {
          typename FR::type a;
          if constexpr (kBf16) {
            typedef __attribute__((address_space(3))) s16x4* lds_s16x4;
            const int r0 = 32 * u + 16 * ks + vrow, r1 = r0 + 8;
            const int col = 32 * mt + vcol;
            const uint16_t* p0 =
                sV + r0 * D + ((((col >> 3) ^ GEO::v_swz(r0)) << 3) | (col & 7));
            const uint16_t* p1 =
                sV + r1 * D + ((((col >> 3) ^ GEO::v_swz(r1)) << 3) | (col & 7));
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(p0));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(p1));
            a = __builtin_bit_cast(bf16x8,
                                   __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int key = 32 * u + 16 * ks + 8 * (e >> 2) + 4 * hh + (e & 3);
              const int d = 32 * mt + q;
              a.v[e] = sV[key * D + ((((d >> 2) ^ GEO::k_swz(key)) << 2) | (d & 3))];
            }
          }
          acc_o[mt] = mma(a, bq, acc_o[mt]);
        }
      }
  };

  constexpr int kPer = 2 * kP;   // vector-memory instructions per wave per tile
  if constexpr (STG == 2) {
    // one stage in flight: at step t only tile t is outstanding
    if (0 < nt) issue(0, st0);
#define SPRINT_ATT_STEP2(CUR, NXT, U)                                                     \
  {                                                                                       \
    const int t = tb + (U);                                                               \
    if (t < nt) {                                                                         \
      __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));                                         \
      __builtin_amdgcn_s_barrier();                                                       \
      if (t + 1 < nt) issue(t + 1, NXT);                                                  \
      compute(CUR, t);                                                                    \
    }                                                                                     \
  }
    for (int tb = 0; tb < nt; tb += 2) {
      SPRINT_ATT_STEP2(st0, st1, 0)
      SPRINT_ATT_STEP2(st1, st0, 1)
    }
#undef SPRINT_ATT_STEP2
  } else {
  // prologue: three stages in flight
  if (0 < nt) issue(0, st0);
  if (1 < nt) issue(1, st1);
  if (2 < nt) issue(2, st2);
#define SPRINT_ATT_STEP(CUR, NXT3, U)                                                     \
  {                                                                                       \
    const int t = tb + (U);                                                               \
    if (t < nt) {                                                                         \
      if (t + 2 < nt)                                                                     \
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(2 * kPer));                                \
      else if (t + 1 < nt)                                                                \
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(kPer));                                    \
      else                                                                                \
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));                                       \
      __builtin_amdgcn_s_barrier();                                                       \
      if (t + 3 < nt) issue(t + 3, NXT3);                                                 \
      compute(CUR, t);                                                                    \
    }                                                                                     \
  }
  for (int tb = 0; tb < nt; tb += kStages) {
    SPRINT_ATT_STEP(st0, st3, 0)
    SPRINT_ATT_STEP(st1, st0, 1)
    SPRINT_ATT_STEP(st2, st1, 2)
    SPRINT_ATT_STEP(st3, st2, 3)
  }
#undef SPRINT_ATT_STEP
  }

  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int nrows = max(0, min(32, args.R - rw * 32));
  // this wave's staging region: after the barrier the stages are free
  __syncthreads();
  using PE = typename std::conditional<kBf16, half_t, float>::type;   // partial element
  constexpr int kOutWave = RowGeo<S, D>::kWaveBytes;
  constexpr int kPartWave = RowGeo<PE, D>::kWaveBytes;
  constexpr int kWaveBytes = kOutWave > kPartWave ? kOutWave : kPartWave;
  constexpr int kWps = kStageBytes / kWaveBytes;                      // wave regions per stage
  static_assert(kWps * kRing >= NW, "staging regions");
  const int sidx = rw / kWps;
  char* reg = (sidx == 0 ? st0 : sidx == 1 ? st1 : sidx == 2 ? st2 : st3) +
              (rw % kWps) * kWaveBytes;
  if (args.n_splits == 1) {
    // the block saw every key: write O directly
    stage_rows<S, D>(reg, acc_o, inv, q, hh);
    __syncthreads();
    flush_rows<S, D>(reg, lane, nrows, [&](int rr) {
        const int rh = rw * 32 + rr;
        const int hd = g * args.G + rh / args.Lq;
        return args.O + ((static_cast<int64_t>(seq) * args.Lq + rh % args.Lq) * args.Hq + hd) *
                            static_cast<int64_t>(D * sizeof(S));
      });
    return;
  }
  // Partial rows.  fp16 partials (bf16 inputs) carry a power-of-two row scale
  // 2^e chosen so the row's largest |o| lands in [2^14, 2^15): fp16's full
  // precision at any magnitude bf16 values can take, and no overflow.
  float pscale = 1.f, pmul = 1.f;
  if constexpr (kBf16) {
    float mx = 0.f;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fabsf(acc_o[mt][r]));
    mx = pair_max(mx * inv);
    int e = 0;
    if (mx > 0.f) {
      e = static_cast<int>((__float_as_uint(mx) >> 23) & 255u) - 127 - 14;
      e = e < -100 ? -100 : (e > 100 ? 100 : e);
    }
    pscale = __uint_as_float(static_cast<uint32_t>(127 - e) << 23);   // 2^-e
    pmul = __uint_as_float(static_cast<uint32_t>(127 + e) << 23);     // 2^e
  }
  const int64_t pbase =
      ((static_cast<int64_t>(seq) * args.Hkv + g) * args.n_splits + split) * args.R + rw * 32;
  stage_rows<PE, D>(reg, acc_o, inv * pscale, q, hh);
  __syncthreads();
  flush_rows<PE, D>(reg, lane, nrows, [&](int rr) {
    return static_cast<char*>(args.part_o) + (pbase + rr) * static_cast<int64_t>(D * sizeof(PE));
  });
  if (hh == 0 && row_ok)
    *reinterpret_cast<f32x4*>(args.part_ml + (pbase + q) * 4) = f32x4{m_run, l_tot, pmul, 0.f};
}

// Output rows (waves) per combine block: two, so that the 512 rows of a
// single sequence with 4 KV heads and 128 query rows each cover all 256
// CUs (four per block left half of them idle and measured 2-4% slower).
constexpr int kCombineWaves = 2;

// Combine the key ranges: one wave per output row (of one sequence and KV
// head).  A lane owns 8 columns and every (64/(D/8))-th range, so all of its
// loads for a batch of NB ranges are in flight together; it folds them
// with the running (m, l) in log2 units, then a butterfly over the lanes
// that share its columns merges the range groups.  The fold order is fixed,
// so the result is bitwise reproducible.  NB = 16 when one batch of 8 would
// not cover every range, so that up to 64 (D = 128) or 128 (D = 64) ranges
// take one memory round trip instead of two.
template <typename T, int D, int NB>
__global__ __launch_bounds__(64 * kCombineWaves) void attend_combine_kernel(AttnArgs args) {
  using S = typename T::storage;
  constexpr bool kBf16 = sizeof(S) == 2;
  constexpr int kCL = D / 8;        // lanes across the columns
  constexpr int kSG = 64 / kCL;     // lanes across the ranges
  constexpr int kNB = NB;           // ranges per lane per batch
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n_rb = (args.R + kCombineWaves - 1) / kCombineWaves;
  const int rb = blockIdx.x % n_rb;
  const int unit = blockIdx.x / n_rb;           // seq * Hkv + g
  const int rr = rb * kCombineWaves + wave;
  if (rr >= args.R) return;
  const int g = unit % args.Hkv, seq = unit / args.Hkv;
  const int cl = lane % kCL, sg = lane / kCL;
  const int d = cl * 8;
  const int64_t rstride = static_cast<int64_t>(args.R);
  const int64_t row0 = static_cast<int64_t>(unit) * args.n_splits * rstride + rr;
  float m = -INFINITY, l = 0.f;
  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.f;
  for (int base = sg; base < args.n_splits; base += kSG * kNB) {
    float ms[kNB], ls[kNB], mul[kNB], v[kNB][8];
    // Every load of the batch is issued unconditionally (a range past the
    // last reads range 0's row, which exists) and the values are selected
    // afterwards: loads under a per-lane condition compile to branches that
    // wait for each load before issuing the next.
    // (m, l) and 2^e are loaded apart: a 16-byte load whose last word is
    // never read lets that register be reused at once, which waits for the
    // load.
    bool okv[kNB];
    float2 mlv[kNB];
    float mulv[kNB];
    u32x4 hv0[kNB], hv1[kNB];
#pragma unroll
    for (int u = 0; u < kNB; ++u) {
      const int sp = base + kSG * u;
      okv[u] = sp < args.n_splits;
      const int64_t prow = row0 + static_cast<int64_t>(okv[u] ? sp : 0) * rstride;
      mlv[u] = *reinterpret_cast<const float2*>(args.part_ml + prow * 4);
      mulv[u] = args.part_ml[prow * 4 + 2];
      if constexpr (kBf16) {
        hv0[u] = ld16(static_cast<const half_t*>(args.part_o) + prow * D + d);
      } else {
        const float* src = static_cast<const float*>(args.part_o) + prow * D + d;
        hv0[u] = ld16(src);
        hv1[u] = ld16(src + 4);
      }
    }
#pragma unroll
    for (int u = 0; u < kNB; ++u) {
      ms[u] = okv[u] ? mlv[u].x : -INFINITY;
      ls[u] = okv[u] ? mlv[u].y : 0.f;
      mul[u] = mulv[u];
      if constexpr (kBf16) {
        const f16x8 hv = __builtin_bit_cast(f16x8, hv0[u]);
#pragma unroll
        for (int c = 0; c < 8; ++c) v[u][c] = okv[u] ? static_cast<float>(hv[c]) : 0.f;
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          v[u][c] = okv[u] ? __uint_as_float(hv0[u][c]) : 0.f;
          v[u][4 + c] = okv[u] ? __uint_as_float(hv1[u][c]) : 0.f;
        }
      }
    }
    // no early exit when every range so far is empty (mb = -inf): it would
    // make the partials' loads wait for the (m, l) loads; empty ranges
    // already get weight 0 and leave m at -inf
    float mb = m;
#pragma unroll
    for (int u = 0; u < kNB; ++u) mb = fmaxf(mb, ms[u]);
    const float a = m == -INFINITY ? 0.f : exp2f(m - mb);
    l *= a;
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] *= a;
#pragma unroll
    for (int u = 0; u < kNB; ++u) {
      const float w = ms[u] == -INFINITY ? 0.f : ls[u] * exp2f(ms[u] - mb);
      l += w;
      const float wv = w * mul[u];               // undo the partial's row scale
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = fmaf(wv, v[u][c], acc[c]);
    }
    m = mb;
  }
  // merge the range groups (the same arithmetic on both lanes of a pair)
#pragma unroll
  for (int o = kCL; o < 64; o <<= 1) {
    const float m2 = shfl_xor_f(m, o), l2 = shfl_xor_f(l, o);
    const float mn = fmaxf(m, m2);
    const float a = m == -INFINITY ? 0.f : exp2f(m - mn);
    const float b = m2 == -INFINITY ? 0.f : exp2f(m2 - mn);
    l = l * a + l2 * b;
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = acc[c] * a + shfl_xor_f(acc[c], o) * b;
    m = mn;
  }
  if (sg != 0) return;
  const float inv = 1.f / l;
  const int gi = rr / args.Lq, qi = rr % args.Lq;
  const int head = g * args.G + gi;
  S* out = reinterpret_cast<S*>(args.O) +
           ((static_cast<int64_t>(seq) * args.Lq + qi) * args.Hq + head) * D + d;
  if constexpr (kBf16) {
    u32x4 o;
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = pack_bf16x2(acc[2 * c] * inv, acc[2 * c + 1] * inv);
    st16(out, o);
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c) out[c] = acc[c] * inv;
  }
}

// bf16 stages hold 64 keys (two S^T tiles); fp32 stages 32 keys (LDS size).
template <typename T>
constexpr int nsub() {
  return sizeof(typename T::storage) == 2 ? 2 : 1;
}

// bf16 with up to four waves per block uses the two-stage, two-blocks-per-CU
// form (about 15% faster than the four-stage ring at every cache size measured,
// 3.5k to 28k keys); fp32 and eight-wave blocks keep the four-stage ring.
constexpr int kSplitStages = 2;

template <typename T, int D, int NW>
hipError_t launch_split(const AttnArgs& a, hipStream_t st) {
  const int blocks = a.nseq * a.Hkv * a.n_splits;
  constexpr int stg = (sizeof(typename T::storage) == 2 && NW <= 4) ? kSplitStages : 4;
  attend_split_kernel<T, D, NW, nsub<T>(), stg><<<dim3(blocks), dim3(64 * NW), 0, st>>>(a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_typed(const AttnArgs& a, hipStream_t st) {
  hipError_t e;
  if (a.n_rg <= 1)
    e = launch_split<T, D, 1>(a, st);
  else if (a.n_rg <= 2)
    e = launch_split<T, D, 2>(a, st);
  else if (a.n_rg <= 4)
    e = launch_split<T, D, 4>(a, st);
  else
    e = launch_split<T, D, 8>(a, st);
  if (e != hipSuccess || a.n_splits == 1) return e;
  const int blocks = a.nseq * a.Hkv * ((a.R + kCombineWaves - 1) / kCombineWaves);
  constexpr int kSG = 64 / (D / 8);  // lanes across the ranges
  if (a.n_splits > kSG * 8)
    attend_combine_kernel<T, D, 16><<<dim3(blocks), dim3(64 * kCombineWaves), 0, st>>>(a);
  else
    attend_combine_kernel<T, D, 8><<<dim3(blocks), dim3(64 * kCombineWaves), 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

AttnPlan attend_plan(int nseq, int Lq, int Hq, int Hkv, int D, int max_kv, int has_block,
                     int dtype) {
  AttnPlan p;
  p.rows = (Hq / Hkv) * Lq;
  const int64_t n_keys = static_cast<int64_t>(max_kv) + (has_block ? Lq : 0);
  const int64_t units = static_cast<int64_t>(nseq) * Hkv;
  // Keys per range: the largest power of two that still gives >= 192 blocks,
  // so most CUs stream a range, but at least two 64-key stages: below that a
  // block is all fixed latency, and more ranges only add partials to write
  // and combine (and past 256 blocks a second partial wave).
  int kps = 1 << 20;
  while (kps > 4 * kKT && units * ((n_keys + kps - 1) / kps) < 192) kps >>= 1;
  p.kps = kps;
  p.n_splits = static_cast<int>(n_keys > 0 ? (n_keys + kps - 1) / kps : 1);
  const size_t es = dtype == 1 ? 2 : 4;
  const size_t parts = static_cast<size_t>(units) * p.n_splits * p.rows;
  p.ws_bytes = p.n_splits == 1 ? 0
                               : align_up(parts * D * es, 256) +
                                     align_up(parts * 4 * sizeof(float), 256);
  return p;
}

hipError_t launch_attend(const void* Q, int nseq, int Lq, int Hq, const void* Kp, const void* Vp,
                         const int32_t* cu_kv, int64_t total_kv, const void* Kb, const void* Vb,
                         int Hkv, int D, float scale, int dtype, void* O, const AttnPlan& plan,
                         void* ws, hipStream_t st) {
  AttnArgs a;
  a.Q = static_cast<const char*>(Q);
  a.Kp = static_cast<const char*>(Kp);
  a.Vp = static_cast<const char*>(Vp);
  a.cu_kv = cu_kv;
  a.Kb = static_cast<const char*>(Kb);
  a.Vb = static_cast<const char*>(Vb);
  a.O = static_cast<char*>(O);
  const size_t es = dtype == 1 ? 2 : 4;
  const size_t parts = static_cast<size_t>(nseq) * Hkv * plan.n_splits * plan.rows;
  a.part_o = ws;
  a.part_ml = plan.n_splits == 1 ? nullptr
                                 : reinterpret_cast<float*>(static_cast<char*>(ws) +
                                                            align_up(parts * D * es, 256));
  a.nseq = nseq;
  a.Lq = Lq;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.R = plan.rows;
  a.n_splits = plan.n_splits;
  a.kps = plan.kps;
  a.has_block = (Kb != nullptr) ? 1 : 0;
  a.n_rg = (plan.rows + 31) / 32;
  a.total_kv = total_kv;
  a.scale_log2 = scale * kLog2e;
  if (dtype == 1) return D == 128 ? launch_typed<BF16, 128>(a, st) : launch_typed<BF16, 64>(a, st);
  return D == 128 ? launch_typed<F32, 128>(a, st) : launch_typed<F32, 64>(a, st);
}

void* attend_scratch(int device) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[device] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptr[device] = p;
  }
  return ptr[device];
}

}  // namespace sprint
