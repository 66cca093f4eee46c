// Prefill instantiations for head dim 64: 8-wave workgroups of 256 rows (two per CU
// at 4 waves per SIMD); a sliding window keeps 4 waves on 128 rows.
#include "kernels.hpp"
#include "prefill.hpp"

namespace attn {

hipError_t prefill_d64(const PrefillParams &p, int mask, int n_units, hipStream_t s) {
  switch (mask) {
    case kMaskNone: return launch_prefill<64, 8, 64, false, false, 4>(p, n_units, s);
    case kMaskCausal: return launch_prefill<64, 8, 64, true, false, 4>(p, n_units, s);
    default: return launch_prefill<64, 4, 64, true, true, 4>(p, n_units, s);
  }
}

}  // namespace attn
