// Prefill instantiations for head dim 256.
#include "kernels.hpp"
#include "prefill.hpp"

namespace attn {

hipError_t prefill_d256(const PrefillParams &p, int mask, int n_units, hipStream_t s) {
  switch (mask) {
    case kMaskNone: return launch_prefill<256, 4, 32, false, false>(p, n_units, s);
    case kMaskCausal: return launch_prefill<256, 4, 32, true, false>(p, n_units, s);
    default: return launch_prefill<256, 4, 32, true, true>(p, n_units, s);
  }
}

}  // namespace attn
