// Prefill instantiations for head dim 512 (two 256-wide halves per pair of waves).
#include "kernels.hpp"
#include "prefill.hpp"

namespace attn {

hipError_t prefill_d512(const PrefillParams &p, int mask, int n_units, hipStream_t s) {
  switch (mask) {
    case kMaskNone: return launch_prefill<512, 8, 32, false, false, 2, 256>(p, n_units, s);
    case kMaskCausal: return launch_prefill<512, 8, 32, true, false, 2, 256>(p, n_units, s);
    default: return launch_prefill<512, 8, 32, true, true, 2, 256>(p, n_units, s);
  }
}

hipError_t prefill_d512_chunked(const PrefillParams &p, const PrefillChunks &ck, hipStream_t s) {
  return launch_prefill_chunked<512, 8, 32, 2, 256>(p, ck, s);
}

}  // namespace attn
