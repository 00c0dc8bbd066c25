// Confidence-adaptive unmasking, one step (LLaDA2.0-Uni, SPRINT "Non-uniform
// Token Unmasking"): accept every masked position whose confidence exceeds
// tau, and at least ceil(m / (T - t)) of them, ranked by (confidence
// descending, position ascending).
//
// One wave per sequence, one lane per block position (Lq <= 64).  The rank of
// a masked position is the number of masked positions ahead of it in that
// order, computed by broadcasting every lane's confidence in turn (readlane:
// a scalar broadcast, no LDS round trip); unmask_rule holds the rule, which
// the LM head's fused merge-and-unmask kernel applies too.
#include "sprint_device.hpp"
#include "sprint_internal.hpp"

namespace sprint {
namespace {

__global__ __launch_bounds__(64) void unmask_kernel(const float* __restrict__ conf,
                                                    const int32_t* __restrict__ argmax, int Lq,
                                                    float tau, int steps_left,
                                                    uint8_t* __restrict__ masked,
                                                    int32_t* __restrict__ tokens,
                                                    int32_t* __restrict__ n_accepted) {
  const int s = blockIdx.x;
  const int i = threadIdx.x;
  const int64_t base = static_cast<int64_t>(s) * Lq;
  const bool valid = i < Lq;
  // Every lane loads (a lane past Lq reads position Lq - 1 and ignores it),
  // so the three loads are in flight together.
  const int64_t at = base + (valid ? i : Lq - 1);
  const float c_ld = conf[at];
  const uint8_t m_ld = masked[at];
  const int32_t a_ld = argmax[at];
  unmask_rule(c_ld, m_ld, a_ld, i, Lq, tau, steps_left, base, masked, tokens, n_accepted + s);
}

}  // namespace

hipError_t launch_unmask(const float* conf, const int32_t* argmax, int nseq, int Lq, float tau,
                         int steps_left, uint8_t* masked, int32_t* tokens, int32_t* n_accepted,
                         hipStream_t st) {
  unmask_kernel<<<dim3(nseq), dim3(64), 0, st>>>(conf, argmax, Lq, tau, steps_left, masked, tokens,
                                                 n_accepted);
  return hipGetLastError();
}

}  // namespace sprint
