// Composite prefix score: mean-normalised key norm blended with the prefix
// confidence (LLaDA2.0-Uni, SPRINT "Sparse Prefix Retention").
//
// Two launches over chunks of 256 positions (a chunk never spans sequences):
//   1. keynorm_kernel: n_i = ||K[i]|| (fp32 accumulation) into `ibar`, plus
//      the chunk's sum of norms into the workspace;
//   2. score_kernel: every chunk re-derives its sequence's mean from the
//      chunk sums in one fixed order (so all chunks agree bitwise), then
//      writes I_i = n_i / mean and s_i = alpha*I_i + (1-alpha)*c_i in place.
// HBM-bound: it reads each key row once (Hkv*D elements) and 12 bytes of
// per-position floats.
#include "sprint_device.hpp"
#include "sprint_internal.hpp"

namespace sprint {
namespace {

constexpr int kChunk = 256;
constexpr int kThreads = 256;

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

// G lanes cooperate on one key row of `row_vecs` 16-byte vectors; G is the
// largest power of two <= min(64, row_vecs).
template <typename T>
__global__ __launch_bounds__(kThreads) void keynorm_kernel(const char* __restrict__ K,
                                                           const int32_t* __restrict__ cu_len,
                                                           int nseq, int64_t total_L,
                                                           int row_vecs, int G,
                                                           float* __restrict__ norms,
                                                           float* __restrict__ partial) {
  SeqChunk sc;
  if (!find_seq_chunk(cu_len, nseq, kChunk, total_L, blockIdx.x, sc)) return;
  __shared__ float s_norm[kChunk];
  const int64_t p0 = sc.begin + static_cast<int64_t>(sc.c) * kChunk;
  const int64_t rem = sc.begin + sc.len - p0;
  const int n = rem < kChunk ? static_cast<int>(rem) : kChunk;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int gl = lane & (G - 1), grp = lane / G, groups = 64 / G;
  const int rows_per_iter = (kThreads / 64) * groups;
  const int64_t row_bytes = static_cast<int64_t>(row_vecs) * 16;
  for (int r0 = 0; r0 < n; r0 += rows_per_iter) {
    const int r = r0 + wave * groups + grp;
    float ss = 0.f;
    if (r < n) {
      const char* row = K + (p0 + r) * row_bytes;
      for (int v = gl; v < row_vecs; v += G) ss += sumsq16<T>(ld16(row + v * 16));
    }
    for (int m = G >> 1; m >= 1; m >>= 1) ss += shfl_xor_f(ss, m);
    if (r < n && gl == 0) {
      const float nv = sqrtf(ss);
      s_norm[r] = nv;
      norms[p0 + r] = nv;
    }
  }
  __syncthreads();
  if (wave == 0) {
    float acc = 0.f;
    for (int i = lane; i < n; i += 64) acc += s_norm[i];
    acc = wave_sum(acc);
    if (lane == 0) partial[blockIdx.x] = acc;
  }
}

__global__ __launch_bounds__(kThreads) void score_kernel(const float* __restrict__ conf,
                                                         const int32_t* __restrict__ cu_len,
                                                         int nseq, int64_t total_L,
                                                         const float* __restrict__ partial,
                                                         float alpha, float* __restrict__ ibar,
                                                         float* __restrict__ score) {
  SeqChunk sc;
  if (!find_seq_chunk(cu_len, nseq, kChunk, total_L, blockIdx.x, sc)) return;
  __shared__ float s_mean;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    float acc = 0.f;
    for (int i = lane; i < sc.nchunks; i += 64) acc += partial[sc.first + i];
    acc = wave_sum(acc);
    if (lane == 0) s_mean = acc / static_cast<float>(sc.len);
  }
  __syncthreads();
  const float mean = s_mean;
  const int64_t p = sc.begin + static_cast<int64_t>(sc.c) * kChunk + threadIdx.x;
  if (p < sc.begin + sc.len) {
    const float ib = mean > 0.f ? ibar[p] / mean : 1.f;
    ibar[p] = ib;
    score[p] = alpha * ib + (1.f - alpha) * conf[p];
  }
}

}  // namespace

size_t score_ws_bytes(int64_t total_L, int nseq) {
  return align_up(static_cast<size_t>(chunk_bound(total_L, nseq, kChunk)) * sizeof(float), 256);
}

hipError_t launch_score(const void* K, const float* conf, const int32_t* cu_len, int nseq,
                        int64_t total_L, int Hkv, int D, int dtype, float alpha, float* ibar,
                        float* score, void* ws, hipStream_t st) {
  if (total_L == 0) return hipSuccess;
  const int es = dtype == 1 ? 2 : 4;
  const int row_vecs = Hkv * D * es / 16;
  int G = 1;
  while (G * 2 <= row_vecs && G * 2 <= 64) G *= 2;
  const int64_t nblk = chunk_bound(total_L, nseq, kChunk);
  float* partial = static_cast<float*>(ws);
  if (dtype == 1)
    keynorm_kernel<BF16><<<dim3(nblk), dim3(kThreads), 0, st>>>(
        static_cast<const char*>(K), cu_len, nseq, total_L, row_vecs, G, ibar, partial);
  else
    keynorm_kernel<F32><<<dim3(nblk), dim3(kThreads), 0, st>>>(
        static_cast<const char*>(K), cu_len, nseq, total_L, row_vecs, G, ibar, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  score_kernel<<<dim3(nblk), dim3(kThreads), 0, st>>>(conf, cu_len, nseq, total_L, partial,
                                                       alpha, ibar, score);
  return hipGetLastError();
}

}  // namespace sprint
