// Prefill instantiations for head dim 256.
#include "kernels.hpp"
#include "prefill.hpp"

namespace attn {

hipError_t prefill_d256(const PrefillParams &p, int mask, int n_units, hipStream_t s) {
  switch (mask) {
    case kMaskNone: return launch_prefill<256, 4, 32, false, false, 1>(p, n_units, s);
    case kMaskCausal: return launch_prefill<256, 4, 32, true, false, 1>(p, n_units, s);
    default: return launch_prefill<256, 4, 32, true, true, 1>(p, n_units, s);
  }
}

}  // namespace attn
