// Prefill instantiations for head dim 256.
#include "kernels.hpp"
#include "prefill.hpp"

namespace attn {

hipError_t prefill_d256(const PrefillParams &p, int mask, int n_units, hipStream_t s) {
  switch (mask) {
    case kMaskNone: return launch_prefill_pp<256, 32, false, false, 4>(p, n_units, s);
    case kMaskCausal: return launch_prefill_pp<256, 32, true, false, 4>(p, n_units, s);
    default: return launch_prefill_pp<256, 32, true, true, 4>(p, n_units, s);
  }
}

hipError_t prefill_d256_queue(const PrefillParams &p, int mask, int n_units, int n_wg, uint32_t *queue,
                              hipStream_t s) {
  switch (mask) {
    case kMaskNone: return launch_prefill_pp_queue<256, 32, false, false, 4>(p, n_units, n_wg, queue, s);
    case kMaskCausal: return launch_prefill_pp_queue<256, 32, true, false, 4>(p, n_units, n_wg, queue, s);
    default: return launch_prefill_pp_queue<256, 32, true, true, 4>(p, n_units, n_wg, queue, s);
  }
}

}  // namespace attn
