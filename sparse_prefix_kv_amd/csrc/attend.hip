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
// K/V tiles of 32 keys arrive by buffer loads straight into LDS
//   (buffer_load_dwordx4 ... lds) into a ring of four stages, three tiles
//   ahead of the one being used.  The stages are distinct LDS arrays and the
//   loop is unrolled by four, so the compiler can see that reads of one stage
//   do not alias loads into another; each wave waits (vmcnt) for its own
//   loads of a stage, then a plain s_barrier (no fence, which would drain
//   every outstanding load) publishes it.
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
//   partial (o / l in fp16 for bf16 inputs, fp32 otherwise, plus m and l in
//   log2 units) and a combine kernel merges the ranges.
#include <math.h>

#include "sprint_device.hpp"
#include "sprint_internal.hpp"

namespace sprint {
namespace {

constexpr int kKT = 32;       // keys per tile
constexpr int kStages = 4;    // LDS ring depth

typedef _Float16 half_t;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

struct AttnArgs {
  const char* Q;
  const char* Kp;
  const char* Vp;
  const int32_t* cu_kv;
  const char* Kb;
  const char* Vb;
  char* O;
  void* part_o;    // [nseq*Hkv*n_splits*R, D] fp16 (bf16 inputs) or fp32, normalized by l
  float* part_ml;  // [nseq*Hkv*n_splits*R, 2]  (m in log2 units, l)
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

// s_waitcnt immediate: at most n vector-memory ops pending, lgkm unrestricted
constexpr int vm_wait_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// Geometry of one tile for element type T and head dim D.
template <typename T, int D>
struct TileGeo {
  using S = typename T::storage;
  static constexpr bool kBf16 = sizeof(S) == 2;
  static constexpr int kRowBytes = D * static_cast<int>(sizeof(S));
  static constexpr int kChunks = kRowBytes / 16;              // 16-byte chunks per row
  static constexpr int kTileBytes = kKT * kRowBytes;
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
                                             0, 0);
  }
}

template <typename T, int D, int NW>
__global__ __launch_bounds__(64 * NW) void attend_split_kernel(AttnArgs args) {
  using S = typename T::storage;
  using FR = Frag<T>;
  using GEO = TileGeo<T, D>;
  constexpr bool kBf16 = GEO::kBf16;
  constexpr int kNI = GEO::kInstr;
  constexpr int kP = (kNI + NW - 1) / NW;                // DMA instructions per wave per tensor
  constexpr int kStageBytes = 2 * GEO::kTileBytes;       // K tile then V tile
  __shared__ __align__(16) char st0[kStageBytes];
  __shared__ __align__(16) char st1[kStageBytes];
  __shared__ __align__(16) char st2[kStageBytes];
  __shared__ __align__(16) char st3[kStageBytes];

  const int split = blockIdx.x % args.n_splits;
  const int g = (blockIdx.x / args.n_splits) % args.Hkv;
  const int seq = blockIdx.x / (args.n_splits * args.Hkv);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int q = lane & 31, hh = lane >> 5;

  const int64_t kv_begin = args.cu_kv[seq];
  const int kv_len = args.cu_kv[seq + 1] - args.cu_kv[seq];
  const int n_keys = kv_len + (args.has_block ? args.Lq : 0);
  const int k0 = min(n_keys, split * args.kps);
  const int k1 = min(n_keys, k0 + args.kps);
  // tiles: the range's prefix keys [pk0, pk1), then its block keys [bk0, bk1)
  const int pk0 = min(k0, kv_len), pk1 = min(k1, kv_len);
  const int bk0 = max(k0, kv_len) - kv_len, bk1 = max(k1, kv_len) - kv_len;
  const int n_ptiles = (pk1 - pk0 + kKT - 1) / kKT;
  const int n_btiles = (bk1 - bk0 + kKT - 1) / kKT;
  const int nt = n_ptiles + n_btiles;

  const int rho = wave * 32 + q;
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

  // Buffer descriptors over the prefix cache and the block's own K/V; reads
  // past either return zeros.
  const int64_t row_stride = static_cast<int64_t>(args.Hkv) * GEO::kRowBytes;
  const int pbytes = static_cast<int>(args.total_kv * row_stride);
  const int bbytes = args.has_block
                         ? static_cast<int>(static_cast<int64_t>(args.nseq) * args.Lq * row_stride)
                         : 0;
  const __amdgpu_buffer_rsrc_t rKp =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(args.Kp), 0, pbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rVp =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(args.Vp), 0, pbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rKb =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(args.Kb), 0, bbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rVb =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(args.Vb), 0, bbytes, 0x00020000);
  // per-lane byte offsets inside a tile: row * stride + swizzled chunk
  uint32_t vK[kP], vV[kP];
#pragma unroll
  for (int p = 0; p < kP; ++p) {
    const int j = wave + NW * p < kNI ? wave + NW * p : kNI - 1;
    const int row = j * GEO::kRowsPerInstr + lane / GEO::kChunks;
    const int slot = lane % GEO::kChunks;
    const int ck = slot ^ GEO::k_swz(row);
    const int cv = kBf16 ? (slot ^ GEO::v_swz(row)) : ck;
    vK[p] = static_cast<uint32_t>(row * row_stride + ck * 16);
    vV[p] = static_cast<uint32_t>(row * row_stride + cv * 16);
  }
  const uint32_t head_off = static_cast<uint32_t>(g * GEO::kRowBytes);
  auto issue = [&](int t, char* stage) {
    if (t < n_ptiles) {
      const uint32_t so =
          static_cast<uint32_t>((kv_begin + pk0 + t * kKT) * row_stride) + head_off;
      tile_dma(rKp, so, vK, stage, wave, NW, kP, kNI);
      tile_dma(rVp, so, vV, stage + GEO::kTileBytes, wave, NW, kP, kNI);
    } else {
      const uint32_t so = static_cast<uint32_t>(
                              (static_cast<int64_t>(seq) * args.Lq + bk0 + (t - n_ptiles) * kKT) *
                              row_stride) + head_off;
      tile_dma(rKb, so, vK, stage, wave, NW, kP, kNI);
      tile_dma(rVb, so, vV, stage + GEO::kTileBytes, wave, NW, kP, kNI);
    }
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

  auto compute = [&](const char* stage, int t) {
    const S* sK = reinterpret_cast<const S*>(stage);
    const S* sV = reinterpret_cast<const S*>(stage + GEO::kTileBytes);
    const int valid = t < n_ptiles ? min(kKT, pk1 - pk0 - t * kKT)
                                   : min(kKT, bk1 - bk0 - (t - n_ptiles) * kKT);
    // S^T[key][query]
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
    const S* krow = sK + q * D;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds)
      s = mma(FR::load_row(krow, 16 * ds + 8 * hh, ksw), qf[ds], s);
    // online softmax in log2 units: m is kept scaled by scale*log2(e) (> 0)
    const float c = args.scale_log2;
    if (valid < kKT) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + 4 * hh + (r & 3) >= valid) s[r] = -INFINITY;
    }
    float tmax = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, s[r]);
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 32)) * c;
    const float m_new = fmaxf(m_run, tmax);
    if (__ballot(m_new > m_run)) {       // rescale only when some lane's maximum moved
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[mt][r] *= alpha;
    }
    m_run = m_new;
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c, -m_new));
      l_run += p[r];
    }
    // O^T[d][query] += sum_key V[key][d] P[query][key]
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float pk8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pk8[e] = p[8 * ks + e];
      const typename FR::type bq = FR::from8(pk8);
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) {
        typename FR::type a;
        if constexpr (kBf16) {
          typedef __attribute__((address_space(3))) s16x4* lds_s16x4;
          const int r0 = 16 * ks + vrow, r1 = r0 + 8;
          const int col = 32 * mt + vcol;
          const uint16_t* p0 = sV + r0 * D + ((((col >> 3) ^ GEO::v_swz(r0)) << 3) | (col & 7));
          const uint16_t* p1 = sV + r1 * D + ((((col >> 3) ^ GEO::v_swz(r1)) << 3) | (col & 7));
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(p0));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(p1));
          a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int key = 16 * ks + 8 * (e >> 2) + 4 * hh + (e & 3);
            const int d = 32 * mt + q;
            a.v[e] = sV[key * D + ((((d >> 2) ^ GEO::k_swz(key)) << 2) | (d & 3))];
          }
        }
        acc_o[mt] = mma(a, bq, acc_o[mt]);
      }
    }
  };

  // prologue: three tiles in flight
  if (0 < nt) issue(0, st0);
  if (1 < nt) issue(1, st1);
  if (2 < nt) issue(2, st2);
  constexpr int kPer = 2 * kP;   // vector-memory instructions per wave per tile
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

  const float l_tot = l_run + shfl_xor_f(l_run, 32);
  if (!row_ok) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (args.n_splits == 1) {
    // the block saw every key: write O directly
    S* out = reinterpret_cast<S*>(args.O) +
             ((static_cast<int64_t>(seq) * args.Lq + qi) * args.Hq + head) * D;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        out[32 * mt + 8 * (r >> 2) + 4 * hh + (r & 3)] = T::from_f32(acc_o[mt][r] * inv);
    return;
  }
  const int64_t prow =
      ((static_cast<int64_t>(seq) * args.Hkv + g) * args.n_splits + split) * args.R + rho;
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = 32 * mt + 8 * r4 + 4 * hh;
      if constexpr (kBf16) {
        f16x4 v = {static_cast<half_t>(acc_o[mt][4 * r4 + 0] * inv),
                   static_cast<half_t>(acc_o[mt][4 * r4 + 1] * inv),
                   static_cast<half_t>(acc_o[mt][4 * r4 + 2] * inv),
                   static_cast<half_t>(acc_o[mt][4 * r4 + 3] * inv)};
        *reinterpret_cast<f16x4*>(static_cast<half_t*>(args.part_o) + prow * D + d) = v;
      } else {
        f32x4 v = {acc_o[mt][4 * r4 + 0] * inv, acc_o[mt][4 * r4 + 1] * inv,
                   acc_o[mt][4 * r4 + 2] * inv, acc_o[mt][4 * r4 + 3] * inv};
        *reinterpret_cast<f32x4*>(static_cast<float*>(args.part_o) + prow * D + d) = v;
      }
    }
  if (hh == 0) {
    args.part_ml[prow * 2 + 0] = m_run;
    args.part_ml[prow * 2 + 1] = l_tot;
  }
}

// Combine the key ranges: a block per (sequence, KV head, row group, 32-column
// slab).  Eight lanes per row fold (m, l) over the ranges in parallel; then
// every thread accumulates four columns of its row across the ranges with the
// weights l_s 2^(m_s - m), four ranges per batch of loads.
template <typename T, int D>
__global__ __launch_bounds__(256) void attend_combine_kernel(AttnArgs args) {
  using S = typename T::storage;
  constexpr bool kBf16 = sizeof(S) == 2;
  constexpr int kSlabs = D / 32;
  const int slab = blockIdx.x % kSlabs;
  const int rest = blockIdx.x / kSlabs;
  const int rg = rest % args.n_rg;
  const int g = (rest / args.n_rg) % args.Hkv;
  const int seq = rest / (args.n_rg * args.Hkv);
  const int row = threadIdx.x >> 3, sub = threadIdx.x & 7;
  const int rr = rg * 32 + row;
  const bool ok = rr < args.R;
  const int64_t ubase = (static_cast<int64_t>(seq) * args.Hkv + g) * args.n_splits;
  const int64_t rstride = static_cast<int64_t>(args.R);
  const float* pml = args.part_ml + (ubase * rstride + (ok ? rr : 0)) * 2;
  float m = -INFINITY;
  for (int sp = sub; sp < args.n_splits; sp += 8) m = fmaxf(m, pml[sp * rstride * 2]);
#pragma unroll
  for (int o = 4; o >= 1; o >>= 1) m = fmaxf(m, shfl_xor_f(m, o));
  float l = 0.f;
  for (int sp = sub; sp < args.n_splits; sp += 8) {
    const float ms = pml[sp * rstride * 2];
    l += ms == -INFINITY ? 0.f : pml[sp * rstride * 2 + 1] * exp2f(ms - m);
  }
#pragma unroll
  for (int o = 4; o >= 1; o >>= 1) l += shfl_xor_f(l, o);
  if (!ok) return;
  const int d = slab * 32 + sub * 4;
  const int64_t pofs = (ubase * rstride + rr) * D + d;
  auto load4 = [&](int sp) -> f32x4 {
    if constexpr (kBf16) {
      const f16x4 h = *reinterpret_cast<const f16x4*>(static_cast<const half_t*>(args.part_o) +
                                                      pofs + sp * rstride * D);
      return f32x4{static_cast<float>(h[0]), static_cast<float>(h[1]), static_cast<float>(h[2]),
                   static_cast<float>(h[3])};
    } else {
      return *reinterpret_cast<const f32x4*>(static_cast<const float*>(args.part_o) + pofs +
                                             sp * rstride * D);
    }
  };
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int sp = 0;
  for (; sp + 4 <= args.n_splits; sp += 4) {
    float ms[4], ls[4];
    f32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ms[u] = pml[(sp + u) * rstride * 2];
      ls[u] = pml[(sp + u) * rstride * 2 + 1];
      v[u] = load4(sp + u);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      acc += (ms[u] == -INFINITY ? 0.f : ls[u] * exp2f(ms[u] - m)) * v[u];
  }
  for (; sp < args.n_splits; ++sp) {
    const float ms = pml[sp * rstride * 2];
    const f32x4 v = load4(sp);
    acc += (ms == -INFINITY ? 0.f : pml[sp * rstride * 2 + 1] * exp2f(ms - m)) * v;
  }
  const float inv = 1.f / l;
  const int gi = rr / args.Lq, qi = rr % args.Lq;
  const int head = g * args.G + gi;
  S* out = reinterpret_cast<S*>(args.O) +
           ((static_cast<int64_t>(seq) * args.Lq + qi) * args.Hq + head) * D + d;
#pragma unroll
  for (int c = 0; c < 4; ++c) out[c] = T::from_f32(acc[c] * inv);
}

template <typename T, int D, int NW>
hipError_t launch_split(const AttnArgs& a, hipStream_t st) {
  const int blocks = a.nseq * a.Hkv * a.n_splits;
  attend_split_kernel<T, D, NW><<<dim3(blocks), dim3(64 * NW), 0, st>>>(a);
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
  const int blocks = a.nseq * a.Hkv * a.n_rg * (D / 32);
  attend_combine_kernel<T, D><<<dim3(blocks), dim3(256), 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

AttnPlan attend_plan(int nseq, int Lq, int Hq, int Hkv, int D, int max_kv, int has_block,
                     int dtype) {
  AttnPlan p;
  p.rows = (Hq / Hkv) * Lq;
  const int64_t n_keys = static_cast<int64_t>(max_kv) + (has_block ? Lq : 0);
  const int64_t units = static_cast<int64_t>(nseq) * Hkv;
  // Keys per range: the largest power of two (at least one tile) that still
  // gives >= 192 blocks, so most CUs stream a range.
  int kps = 1 << 20;
  while (kps > kKT && units * ((n_keys + kps - 1) / kps) < 192) kps >>= 1;
  p.kps = kps;
  p.n_splits = static_cast<int>(n_keys > 0 ? (n_keys + kps - 1) / kps : 1);
  const size_t es = dtype == 1 ? 2 : 4;
  const size_t parts = static_cast<size_t>(units) * p.n_splits * p.rows;
  p.ws_bytes = p.n_splits == 1 ? 0
                               : align_up(parts * D * es, 256) +
                                     align_up(parts * 2 * sizeof(float), 256);
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

}  // namespace sprint
