// Backward instantiations (head dims 64 and 128).
#include "backward.hpp"
#include "kernels.hpp"

namespace attn {

// Waves per workgroup: the staged tiles allow one workgroup per compute unit,
// so dQ runs 8 waves (two per SIMD); dK/dV keeps 4 (at 8 it spills).
constexpr int BWD_NWQ = 8;
constexpr int BWD_NWK = 4;
int backward_block_rows() { return 32 * BWD_NWQ; }
hipError_t backward(int d, const BwdParams &p, bool causal, hipStream_t s) {
  const bool window = p.window > 0;
  if (d == 64)
    return window   ? launch_backward<64, 64, true, true, BWD_NWQ, BWD_NWK>(p, s)
           : causal ? launch_backward<64, 64, true, false, BWD_NWQ, BWD_NWK>(p, s)
                    : launch_backward<64, 64, false, false, BWD_NWQ, BWD_NWK>(p, s);
  return window   ? launch_backward<128, 64, true, true, BWD_NWQ, BWD_NWK>(p, s)
         : causal ? launch_backward<128, 64, true, false, BWD_NWQ, BWD_NWK>(p, s)
                  : launch_backward<128, 64, false, false, BWD_NWQ, BWD_NWK>(p, s);
}

}  // namespace attn
