// Block attention of one denoising step: the block's queries attend without
// a mask to [prefix KV cache ; the block's own K/V] (LLaDA2.0-Uni: SPRINT
// "Sparse Prefix Retention" -- each step attends to the (pruned) prefix --
// and the block notation of "BDLM Loss").  GQA: query head h reads KV head
// floor(h*Hkv/Hq).
//
// Work decomposition (split-KV, flash-decoding style):
//   grid = (splits, Hkv, nseq); a block owns one KV head of one sequence and
//   one contiguous key range, and ALL (Hq/Hkv)*Lq query rows that read that
//   head, so every K/V byte is fetched from HBM once per step.  Each wave
//   owns 32 query rows.
// Per 32-key tile, staged through LDS:
//   S^T = K Q^T on bf16 MFMA 32x32x16 (A = key rows from LDS, B = the wave's
//   queries held in registers).  The accumulator gives each lane one query
//   column and 16 keys, so the online-softmax max needs one cross-half swap
//   and the row sum stays lane-local.
//   O^T += V^T P^T with the probabilities taken straight from the S^T
//   accumulator as the B operand (same lane/key slots, no shuffle); the
//   per-query rescale is lane-local too.
// Each split writes (o, m, l) partials in fp32 (m in log2 units); the combine
// kernel merges them and rounds O to the output dtype.
#include <math.h>

#include "sprint_device.hpp"
#include "sprint_internal.hpp"

namespace sprint {
namespace {

constexpr int kKT = 32;  // keys per LDS tile

struct AttnArgs {
  const char* Q;
  const char* Kp;
  const char* Vp;
  const int32_t* cu_kv;
  const char* Kb;
  const char* Vb;
  char* O;
  float* part_o;   // [nseq*Hkv*n_splits*R, D]
  float* part_ml;  // [nseq*Hkv*n_splits*R, 2]
  int nseq, Lq, Hq, Hkv, G, R, n_splits, kps, has_block;
  float scale_log2;
};

template <typename T>
struct Frag;
template <>
struct Frag<BF16> {
  using type = bf16x8;
  __device__ static type load(const uint16_t* p) { return as_bf16x8(ld16(p)); }
  __device__ static type zero() { return as_bf16x8(u32x4{0u, 0u, 0u, 0u}); }
  __device__ static type from8(const float (&x)[8]) {
    u32x4 u;
    u[0] = pack_bf16x2(x[0], x[1]);
    u[1] = pack_bf16x2(x[2], x[3]);
    u[2] = pack_bf16x2(x[4], x[5]);
    u[3] = pack_bf16x2(x[6], x[7]);
    return as_bf16x8(u);
  }
  __device__ static type gather8(const uint16_t* base, const int (&off)[8]) {
    u32x4 u;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      u[i] = static_cast<uint32_t>(base[off[2 * i]]) |
             (static_cast<uint32_t>(base[off[2 * i + 1]]) << 16);
    return as_bf16x8(u);
  }
};
struct F8 {
  float v[8];
};
template <>
struct Frag<F32> {
  using type = F8;
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
  __device__ static type gather8(const float* base, const int (&off)[8]) {
    type r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r.v[i] = base[off[i]];
    return r;
  }
};

__device__ __forceinline__ f32x16 mma(const bf16x8& a, const bf16x8& b, f32x16 c) {
  return mma32_k16(a, b, c);
}
__device__ __forceinline__ f32x16 mma(const F8& a, const F8& b, f32x16 c) {
  return mma32_k16(a.v, b.v, c);
}

template <typename T, int D>
__global__ __launch_bounds__(512) void attend_split_kernel(AttnArgs args) {
  using S = typename T::storage;
  using FR = Frag<T>;
  constexpr int kPad = 16 / sizeof(S);
  constexpr int kRow = D + kPad;                     // LDS row pitch (elements)
  constexpr int kVpr = D * static_cast<int>(sizeof(S)) / 16;  // 16-byte vectors per row
  constexpr int kEpv = 16 / sizeof(S);               // elements per vector
  __shared__ __align__(16) S sK[kKT * kRow];
  __shared__ __align__(16) S sV[kKT * kRow];

  const int split = blockIdx.x, g = blockIdx.y, seq = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q = lane & 31, hh = lane >> 5;
  const int64_t kv_begin = args.cu_kv[seq];
  const int kv_len = args.cu_kv[seq + 1] - args.cu_kv[seq];
  const int n_keys = kv_len + (args.has_block ? args.Lq : 0);
  const int k0 = split * args.kps;
  const int k1 = min(n_keys, k0 + args.kps);
  const int64_t pbase =
      ((static_cast<int64_t>(seq) * args.Hkv + g) * args.n_splits + split) * args.R;
  const int rho = wave * 32 + q;
  const bool row_ok = rho < args.R;

  if (k0 >= k1) {  // empty split: the combine skips it
    if (row_ok && hh == 0) {
      args.part_ml[(pbase + rho) * 2 + 0] = -INFINITY;
      args.part_ml[(pbase + rho) * 2 + 1] = 0.f;
    }
    return;
  }

  // Query fragments: lane (q, half) holds row rho, dims [16*ds + 8*half, +8).
  typename FR::type qf[D / 16];
  {
    const int gi = row_ok ? rho / args.Lq : 0, qi = row_ok ? rho % args.Lq : 0;
    const int head = g * args.G + gi;
    const S* qrow = reinterpret_cast<const S*>(args.Q) +
                    ((static_cast<int64_t>(seq) * args.Lq + qi) * args.Hq + head) * D;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds)
      qf[ds] = row_ok ? FR::load(qrow + 16 * ds + 8 * hh) : FR::zero();
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc_o[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[mt][r] = 0.f;

  const int64_t kv_stride = static_cast<int64_t>(args.Hkv) * D;  // elements per cache row
  for (int t0 = k0; t0 < k1; t0 += kKT) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < kKT * kVpr; idx += blockDim.x) {
      const int r = idx / kVpr, v = idx - r * kVpr;
      const int key = t0 + r;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (key < k1) {
        int64_t off;
        const char *kb, *vb;
        if (key < kv_len) {
          off = ((kv_begin + key) * kv_stride + static_cast<int64_t>(g) * D) * sizeof(S);
          kb = args.Kp;
          vb = args.Vp;
        } else {
          off = (((static_cast<int64_t>(seq) * args.Lq + (key - kv_len)) * args.Hkv + g) * D) *
                sizeof(S);
          kb = args.Kb;
          vb = args.Vb;
        }
        kv = ld16(kb + off + v * 16);
        vv = ld16(vb + off + v * 16);
      }
      st16(&sK[r * kRow + v * kEpv], kv);
      st16(&sV[r * kRow + v * kEpv], vv);
    }
    __syncthreads();

    // S^T[key][query] for the 32 keys of the tile.
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      const typename FR::type a = FR::load(&sK[q * kRow + 16 * ds + 8 * hh]);
      s = mma(a, qf[ds], s);
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = t0 + 8 * (r >> 2) + 4 * hh + (r & 3);
      const float x = key < k1 ? s[r] * args.scale_log2 : -INFINITY;
      s[r] = x;
      tmax = fmaxf(tmax, x);
    }
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = exp2f(m_run - m_new);
    float p[16];
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = exp2f(s[r] - m_new);
      psum += p[r];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[mt][r] *= alpha;

    // O^T[d][query] += sum_key V[key][d] P[query][key]
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float pk[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pk[e] = p[8 * ks + e];
      const typename FR::type b = FR::from8(pk);
      int off[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) off[e] = (16 * ks + 8 * (e >> 2) + 4 * hh + (e & 3)) * kRow + q;
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) {
        const typename FR::type a = FR::gather8(&sV[32 * mt], off);
        acc_o[mt] = mma(a, b, acc_o[mt]);
      }
    }
  }

  const float l_tot = l_run + shfl_xor_f(l_run, 32);
  if (row_ok) {
    float* po = args.part_o + (pbase + rho) * D;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * mt + 8 * r4 + 4 * hh;
        f32x4 v = {acc_o[mt][4 * r4 + 0], acc_o[mt][4 * r4 + 1], acc_o[mt][4 * r4 + 2],
                   acc_o[mt][4 * r4 + 3]};
        *reinterpret_cast<f32x4*>(po + d) = v;
      }
    if (hh == 0) {
      args.part_ml[(pbase + rho) * 2 + 0] = m_run;
      args.part_ml[(pbase + rho) * 2 + 1] = l_tot;
    }
  }
}

// One wave per output row (sequence, query, head).
template <typename T, int D>
__global__ __launch_bounds__(256) void attend_combine_kernel(AttnArgs args) {
  using S = typename T::storage;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  const int64_t total_rows = static_cast<int64_t>(args.nseq) * args.Lq * args.Hq;
  if (row >= total_rows) return;
  const int head = static_cast<int>(row % args.Hq);
  const int qi = static_cast<int>((row / args.Hq) % args.Lq);
  const int seq = static_cast<int>(row / (static_cast<int64_t>(args.Hq) * args.Lq));
  const int g = head / args.G, gi = head % args.G;
  const int rho = gi * args.Lq + qi;
  const int64_t base = (static_cast<int64_t>(seq) * args.Hkv + g) * args.n_splits;
  float m = -INFINITY;
  for (int sp = 0; sp < args.n_splits; ++sp)
    m = fmaxf(m, args.part_ml[((base + sp) * args.R + rho) * 2]);
  constexpr int kPer = D / 64;
  float o[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) o[j] = 0.f;
  float l = 0.f;
  for (int sp = 0; sp < args.n_splits; ++sp) {
    const int64_t pr = (base + sp) * args.R + rho;
    const float ms = args.part_ml[pr * 2];
    if (ms == -INFINITY) continue;
    const float w = exp2f(ms - m);
    l += args.part_ml[pr * 2 + 1] * w;
#pragma unroll
    for (int j = 0; j < kPer; ++j) o[j] += w * args.part_o[pr * D + lane + 64 * j];
  }
  const float inv = 1.f / l;
  S* out = reinterpret_cast<S*>(args.O) + row * D;
#pragma unroll
  for (int j = 0; j < kPer; ++j) out[lane + 64 * j] = T::from_f32(o[j] * inv);
}

template <typename T, int D>
hipError_t launch_typed(const AttnArgs& a, hipStream_t st) {
  const int waves = (a.R + 31) / 32;
  attend_split_kernel<T, D>
      <<<dim3(a.n_splits, a.Hkv, a.nseq), dim3(64 * waves), 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = static_cast<int64_t>(a.nseq) * a.Lq * a.Hq;
  attend_combine_kernel<T, D><<<dim3((rows + 3) / 4), dim3(256), 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

AttnPlan attend_plan(int nseq, int Lq, int Hq, int Hkv, int D, int max_kv, int has_block,
                     int dtype) {
  (void)dtype;
  AttnPlan p;
  p.rows = (Hq / Hkv) * Lq;
  const int64_t n_keys = static_cast<int64_t>(max_kv) + (has_block ? Lq : 0);
  const int64_t units = static_cast<int64_t>(nseq) * Hkv;
  // Largest key range per split that still gives >= 256 blocks; at least one tile.
  int kps = 2048;
  while (kps > kKT && units * ((n_keys + kps - 1) / kps) < 256) kps >>= 1;
  p.kps = kps;
  p.n_splits = static_cast<int>(n_keys > 0 ? (n_keys + kps - 1) / kps : 1);
  const size_t parts = static_cast<size_t>(units) * p.n_splits * p.rows;
  p.ws_bytes = align_up(parts * D * sizeof(float), 256) + align_up(parts * 2 * sizeof(float), 256);
  return p;
}

hipError_t launch_attend(const void* Q, int nseq, int Lq, int Hq, const void* Kp, const void* Vp,
                         const int32_t* cu_kv, const void* Kb, const void* Vb, int Hkv, int D,
                         float scale, int dtype, void* O, const AttnPlan& plan, void* ws,
                         hipStream_t st) {
  AttnArgs a;
  a.Q = static_cast<const char*>(Q);
  a.Kp = static_cast<const char*>(Kp);
  a.Vp = static_cast<const char*>(Vp);
  a.cu_kv = cu_kv;
  a.Kb = static_cast<const char*>(Kb);
  a.Vb = static_cast<const char*>(Vb);
  a.O = static_cast<char*>(O);
  const size_t parts = static_cast<size_t>(nseq) * Hkv * plan.n_splits * plan.rows;
  a.part_o = static_cast<float*>(ws);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                       align_up(parts * D * sizeof(float), 256));
  a.nseq = nseq;
  a.Lq = Lq;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.R = plan.rows;
  a.n_splits = plan.n_splits;
  a.kps = plan.kps;
  a.has_block = (Kb != nullptr) ? 1 : 0;
  a.scale_log2 = scale * kLog2e;
  if (dtype == 1) return D == 128 ? launch_typed<BF16, 128>(a, st) : launch_typed<BF16, 64>(a, st);
  return D == 128 ? launch_typed<F32, 128>(a, st) : launch_typed<F32, 64>(a, st);
}

}  // namespace sprint
