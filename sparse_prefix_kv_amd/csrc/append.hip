// Growth of the prefix between blocks (LLaDA2.0-Uni: block-wise generation in
// the SPRINT introduction -- B blocks generated one after another -- and
// "Sparse Prefix Retention": the first step of every block sees the complete
// cache, so a finished block's rows join the prefix before the next block's
// pass scores and prunes it again).
//
// Packed arrays (K, V, hidden states, modality) hold each sequence's rows
// back to back; appending n_blk rows to every sequence therefore moves every
// later sequence, and the op writes a new packed array:
//   out rows [a_s + s*n_blk, a_{s+1} + s*n_blk) = old rows [a_s, a_{s+1}),
//   then the n_blk rows of block s,
// with a_s = cu_old[s].  Rows are opaque bytes (bit copies).  One thread per
// 16-byte vector of the output when rows are whole vectors, per byte
// otherwise; the sequence of an output row comes from a binary search over
// the new row starts.  HBM-bound: (old + block) bytes read, as many written.
#include "sprint_device.hpp"
#include "sprint_internal.hpp"

namespace sprint {
namespace {

constexpr int kAppendThreads = 256;

__device__ __forceinline__ int64_t clamp64(int64_t v, int64_t lo, int64_t hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

// W = 16: vectors of 16 bytes (row_bytes a multiple of 16); W = 1: bytes.
template <int W>
__global__ __launch_bounds__(kAppendThreads) void append_rows_kernel(
    const char* __restrict__ old, const int32_t* __restrict__ cu_old, int nseq, int64_t total_old,
    const char* __restrict__ blk, int n_blk, int64_t row_bytes, int64_t total_units,
    char* __restrict__ out, int32_t* __restrict__ cu_out) {
  const int64_t u = static_cast<int64_t>(blockIdx.x) * kAppendThreads + threadIdx.x;
  if (cu_out != nullptr && blockIdx.x == 0) {
    for (int s = threadIdx.x; s <= nseq; s += kAppendThreads)
      cu_out[s] = static_cast<int32_t>(clamp64(cu_old[s], 0, total_old) +
                                       static_cast<int64_t>(s) * n_blk);
  }
  if (u >= total_units) return;
  const int64_t units_per_row = row_bytes / W;
  const int64_t r = u / units_per_row;
  const int64_t c = (u - r * units_per_row) * W;
  // sequence of output row r: the last s whose new start is <= r
  int lo = 0, hi = nseq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (clamp64(cu_old[mid], 0, total_old) + static_cast<int64_t>(mid) * n_blk <= r)
      lo = mid;
    else
      hi = mid - 1;
  }
  const int s = lo;
  const int64_t a = clamp64(cu_old[s], 0, total_old);
  const int64_t e = clamp64(cu_old[s + 1], a, total_old);
  const int64_t j = r - (a + static_cast<int64_t>(s) * n_blk);   // row within the new run
  const char* src = nullptr;
  if (j >= 0 && j < e - a)
    src = old + (a + j) * row_bytes;
  else if (j >= e - a && j < e - a + n_blk)
    src = blk + (static_cast<int64_t>(s) * n_blk + (j - (e - a))) * row_bytes;
  if (src == nullptr) return;   // inconsistent cu_old: leave the row alone
  if constexpr (W == 16)
    st16(out + r * row_bytes + c, ld16_nt(src + c));
  else
    out[r * row_bytes + c] = src[c];
}

}  // namespace

hipError_t launch_append_rows(const void* old, const int32_t* cu_old, int nseq, int64_t total_old,
                              const void* blk, int n_blk, int64_t row_bytes, void* out,
                              int32_t* cu_out, hipStream_t st) {
  const int64_t total_rows = total_old + static_cast<int64_t>(nseq) * n_blk;
  const bool vec = row_bytes % 16 == 0 && (reinterpret_cast<uintptr_t>(old) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(blk) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(out) & 15) == 0;
  const int64_t units = total_rows * (vec ? row_bytes / 16 : row_bytes);
  // at least one block so that cu_out is written
  const int64_t blocks = units > 0 ? (units + kAppendThreads - 1) / kAppendThreads : 1;
  const auto* o = static_cast<const char*>(old);
  const auto* b = static_cast<const char*>(blk);
  auto* d = static_cast<char*>(out);
  if (vec)
    append_rows_kernel<16><<<dim3(static_cast<unsigned>(blocks)), dim3(kAppendThreads), 0, st>>>(
        o, cu_old, nseq, total_old, b, n_blk, row_bytes, units, d, cu_out);
  else
    append_rows_kernel<1><<<dim3(static_cast<unsigned>(blocks)), dim3(kAppendThreads), 0, st>>>(
        o, cu_old, nseq, total_old, b, n_blk, row_bytes, units, d, cu_out);
  return hipGetLastError();
}

}  // namespace sprint
