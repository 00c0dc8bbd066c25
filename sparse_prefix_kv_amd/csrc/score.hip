// Composite prefix score: mean-normalised key norm blended with the prefix
// confidence (LLaDA2.0-Uni, SPRINT "Sparse Prefix Retention").
//
// Two launches over chunks of 64 positions (a chunk never spans sequences):
//   1. keynorm_kernel: n_i = ||K[i]|| (fp32 accumulation) into `ibar`, plus
//      the chunk's sum of norms into the workspace;
//   2. score_kernel: every chunk re-derives its sequence's mean from the
//      chunk sums in one fixed order (so all chunks agree bitwise), then
//      writes I_i = n_i / mean and s_i = alpha*I_i + (1-alpha)*c_i in place.
// With several layers, launch 1 runs once per layer (grid y) into per-layer
// norms and chunk sums.  For one kept set shared by every layer's cache, I_i
// is the mean over layers of each layer's I_i, summed in layer order; for a
// set per layer, launch 2 also runs per layer and writes each layer's own
// I and s.  One layer gives exactly the single-layer arithmetic either way.
// HBM-bound: it reads each key row once (Hkv*D elements) and 12 bytes of
// per-position floats.  Eight lanes share a row: one wave instruction reads
// 128 contiguous bytes of eight rows (whole cache lines), and every lane has
// all of its loads for two rows in flight before it reduces.  Summation
// order is fixed (lane-strided vectors, then a butterfly), so results are
// bitwise reproducible.
#include "sprint_device.hpp"
#include "sprint_internal.hpp"

namespace sprint {
namespace {

constexpr int kChunk = 64;     // positions per block
constexpr int kThreads = 256;  // 4 waves x 2 passes x 8 rows = 64 rows
constexpr int kLanesPerRow = 8;

template <typename T>
__device__ __forceinline__ float sumsq16(u32x4 x);
template <>
__device__ __forceinline__ float sumsq16<BF16>(u32x4 x) {
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(x[i] << 16);
    const float hi = __uint_as_float(x[i] & 0xFFFF0000u);
    acc = fmaf(lo, lo, acc);
    acc = fmaf(hi, hi, acc);
  }
  return acc;
}
template <>
__device__ __forceinline__ float sumsq16<F32>(u32x4 x) {
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float f = __uint_as_float(x[i]);
    acc = fmaf(f, f, acc);
  }
  return acc;
}

// row_vecs = 16-byte vectors per key row (a multiple of 8 for D in {64, 128}).
template <typename T>
__global__ __launch_bounds__(kThreads) void keynorm_kernel(const char* __restrict__ K,
                                                           const int32_t* __restrict__ cu_len,
                                                           int nseq, int64_t total_L,
                                                           int row_vecs,
                                                           float* __restrict__ norms,
                                                           float* __restrict__ partial) {
  SeqChunk sc;
  if (!find_seq_chunk(cu_len, nseq, kChunk, total_L, blockIdx.x, sc)) return;
  // layer blockIdx.y: its cache, norms and chunk sums
  K += static_cast<int64_t>(blockIdx.y) * total_L * row_vecs * 16;
  norms += static_cast<int64_t>(blockIdx.y) * total_L;
  partial += static_cast<int64_t>(blockIdx.y) * gridDim.x;
  __shared__ float s_norm[kChunk];
  const int64_t p0 = sc.begin + static_cast<int64_t>(sc.c) * kChunk;
  const int64_t rem = sc.begin + sc.len - p0;
  const int n = rem < kChunk ? static_cast<int>(rem) : kChunk;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int gl = lane & (kLanesPerRow - 1), grp = lane / kLanesPerRow;
  const int64_t row_bytes = static_cast<int64_t>(row_vecs) * 16;
  // this lane's two rows: r_p = 16*wave + 8*p + grp
  const int r0 = 16 * wave + grp, r1 = r0 + 8;
  const bool ok0 = r0 < n, ok1 = r1 < n;
  const char* row0 = K + (p0 + (ok0 ? r0 : 0)) * row_bytes;
  const char* row1 = K + (p0 + (ok1 ? r1 : 0)) * row_bytes;
  float ss0 = 0.f, ss1 = 0.f;
#pragma unroll 4
  for (int v = gl; v < row_vecs; v += kLanesPerRow) {
    const u32x4 a = ok0 ? ld16_nt(row0 + v * 16) : u32x4{0u, 0u, 0u, 0u};
    const u32x4 b = ok1 ? ld16_nt(row1 + v * 16) : u32x4{0u, 0u, 0u, 0u};
    ss0 += sumsq16<T>(a);
    ss1 += sumsq16<T>(b);
  }
#pragma unroll
  for (int m = kLanesPerRow >> 1; m >= 1; m >>= 1) {
    ss0 += shfl_xor_f(ss0, m);
    ss1 += shfl_xor_f(ss1, m);
  }
  if (gl == 0) {
    if (ok0) {
      const float nv = sqrtf(ss0);
      s_norm[r0] = nv;
      norms[p0 + r0] = nv;
    }
    if (ok1) {
      const float nv = sqrtf(ss1);
      s_norm[r1] = nv;
      norms[p0 + r1] = nv;
    }
  }
  __syncthreads();
  if (wave == 0) {
    float acc = lane < n ? s_norm[lane] : 0.f;
    acc = wave_sum(acc);
    if (lane == 0) partial[blockIdx.x] = acc;
  }
}

// One wave per 64-position chunk.  norms: [n_layers, total_L] (may be ibar
// itself for one layer); partial: [n_layers, n_chunks].  per_layer: grid y
// is the layer, and each layer's own I and s go to ibar/score [n_layers,
// total_L] (one kept set per layer); otherwise I is the layer mean.
__global__ __launch_bounds__(64) void score_kernel(const float* __restrict__ conf,
                                                   const int32_t* __restrict__ cu_len, int nseq,
                                                   int64_t total_L, int n_layers, int per_layer,
                                                   const float* norms,
                                                   const float* __restrict__ partial, float alpha,
                                                   float* ibar, float* __restrict__ score) {
  SeqChunk sc;
  if (!find_seq_chunk(cu_len, nseq, kChunk, total_L, blockIdx.x, sc)) return;
  const int lane = threadIdx.x;
  const int64_t p = sc.begin + static_cast<int64_t>(sc.c) * kChunk + lane;
  const bool ok = p < sc.begin + sc.len;
  const int l0 = per_layer ? static_cast<int>(blockIdx.y) : 0;
  const int l1 = per_layer ? l0 + 1 : n_layers;
  // The position's confidence and norms do not depend on the chunk sums:
  // they are loaded first, so that their latency overlaps the sums'.
  const int64_t pc = ok ? p : sc.begin;
  const float cf = conf[pc];
  float ib = 0.f;
  for (int l = l0; l < l1; ++l) {
    const float nv = norms[static_cast<int64_t>(l) * total_L + pc];
    const float* part = partial + static_cast<int64_t>(l) * gridDim.x + sc.first;
    // lane-strided sum of the chunk sums, eight loads in flight per round,
    // added in index order (the same order, so the same bits, in every chunk)
    float acc = 0.f;
    int i = lane;
    for (; i + 7 * 64 < sc.nchunks; i += 8 * 64) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[i + 64 * u];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += v[u];
    }
    for (; i < sc.nchunks; i += 64) acc += part[i];
    acc = wave_sum(acc);
    const float mean = acc / static_cast<float>(sc.len);
    ib += mean > 0.f ? nv / mean : 1.f;
  }
  if (ok) {
    ib /= static_cast<float>(l1 - l0);
    const int64_t o = static_cast<int64_t>(l0) * total_L + p;
    ibar[o] = ib;
    score[o] = alpha * ib + (1.f - alpha) * cf;
  }
}

}  // namespace

size_t score_ws_bytes(int64_t total_L, int nseq, int n_layers) {
  const size_t part = align_up(static_cast<size_t>(chunk_bound(total_L, nseq, kChunk)) *
                                   n_layers * sizeof(float), 256);
  const size_t norms =
      n_layers > 1 ? align_up(static_cast<size_t>(total_L) * n_layers * sizeof(float), 256) : 0;
  return part + norms;
}

hipError_t launch_score(const void* K, int n_layers, int per_layer, const float* conf,
                        const int32_t* cu_len, int nseq, int64_t total_L, int Hkv, int D,
                        int dtype, float alpha, float* ibar, float* score, void* ws,
                        hipStream_t st) {
  if (total_L == 0) return hipSuccess;
  const int es = dtype == 1 ? 2 : 4;
  const int row_vecs = Hkv * D * es / 16;
  const int64_t nblk = chunk_bound(total_L, nseq, kChunk);
  float* partial = static_cast<float*>(ws);
  // one layer keeps its norms in ibar; several need their own array
  float* norms = n_layers > 1
                     ? reinterpret_cast<float*>(static_cast<char*>(ws) +
                                                align_up(static_cast<size_t>(nblk) * n_layers *
                                                             sizeof(float), 256))
                     : ibar;
  const dim3 grid(static_cast<unsigned>(nblk), static_cast<unsigned>(n_layers));
  if (dtype == 1)
    keynorm_kernel<BF16><<<grid, dim3(kThreads), 0, st>>>(
        static_cast<const char*>(K), cu_len, nseq, total_L, row_vecs, norms, partial);
  else
    keynorm_kernel<F32><<<grid, dim3(kThreads), 0, st>>>(
        static_cast<const char*>(K), cu_len, nseq, total_L, row_vecs, norms, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 sgrid(static_cast<unsigned>(nblk), per_layer ? static_cast<unsigned>(n_layers) : 1u);
  score_kernel<<<sgrid, dim3(64), 0, st>>>(conf, cu_len, nseq, total_L, n_layers, per_layer, norms,
                                           partial, alpha, ibar, score);
  return hipGetLastError();
}

}  // namespace sprint
