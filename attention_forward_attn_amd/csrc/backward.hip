// Backward instantiations (head dim 128).
#include "backward.hpp"
#include "kernels.hpp"

namespace attn {

hipError_t backward_d128(const BwdParams &p, bool causal, hipStream_t s) {
  return causal ? launch_backward<128, 64, true>(p, s) : launch_backward<128, 64, false>(p, s);
}

}  // namespace attn
