// Backward instantiations (head dims 64 and 128).
#include "backward.hpp"
#include "kernels.hpp"

namespace attn {

hipError_t backward(int d, const BwdParams &p, bool causal, hipStream_t s) {
  if (d == 64) return causal ? launch_backward<64, 64, true>(p, s) : launch_backward<64, 64, false>(p, s);
  return causal ? launch_backward<128, 64, true>(p, s) : launch_backward<128, 64, false>(p, s);
}

}  // namespace attn
