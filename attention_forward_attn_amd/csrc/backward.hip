// Backward instantiations (head dims 64, 128 and 256).
#include "backward.hpp"
#include "kernels.hpp"

namespace attn {

// Waves per workgroup: the staged tiles allow one workgroup per compute unit,
// so at d <= 128 dQ runs 8 waves (two per SIMD); dK/dV keeps 4 (at 8 it
// spills).  At d = 256 both run 4 waves over 32-row tiles: a wave holds its
// rows' Q and dO (or K and V) as MMA operands, 128 registers, beside a
// 32 x 256 fp32 accumulator per gradient, and two stages of 64-row tiles
// would not fit in LDS.
constexpr int BWD_NWQ = 8;
constexpr int BWD_NWK = 4;
constexpr int BWD_NW256 = 4;
// Ring stages (dQ, dK/dV): each tile is staged once (the tile engine's shared
// swizzle), so a stage is 32 KiB of K and V (dQ) or Q and dO plus the rows'
// LSE and D (dK/dV) at every head dim but 64 (16 KiB).
constexpr int BWD_NSQ = 2;
constexpr int BWD_NSK = 2;
constexpr int BWD_NSQ256 = 2;
constexpr int BWD_NSK256 = 2;
constexpr int BWD_BNQ256 = 64;  // keys per dQ tile at d = 256 (two stages of K and V: 128 KiB)
// Rows per dQ workgroup, at its smallest over the head dims (sizes the
// sink-gradient partials of the workspace, one per query tile).
int backward_block_rows() { return 32 * BWD_NW256; }
hipError_t backward(int d, const BwdParams &p, bool causal, hipStream_t s) {
  const bool window = p.window > 0;
  if (d == 64)
    return window   ? launch_backward<64, 64, true, true, BWD_NWQ, BWD_NWK, BWD_NSQ, BWD_NSK>(p, s)
           : causal ? launch_backward<64, 64, true, false, BWD_NWQ, BWD_NWK, BWD_NSQ, BWD_NSK>(p, s)
                    : launch_backward<64, 64, false, false, BWD_NWQ, BWD_NWK, BWD_NSQ, BWD_NSK>(p, s);
  if (d == 256)
    return window   ? launch_backward<256, 32, true, true, BWD_NW256, BWD_NW256, BWD_NSQ256, BWD_NSK256, BWD_BNQ256>(p, s)
           : causal ? launch_backward<256, 32, true, false, BWD_NW256, BWD_NW256, BWD_NSQ256, BWD_NSK256, BWD_BNQ256>(p, s)
                    : launch_backward<256, 32, false, false, BWD_NW256, BWD_NW256, BWD_NSQ256, BWD_NSK256, BWD_BNQ256>(p, s);
  return window   ? launch_backward<128, 64, true, true, BWD_NWQ, BWD_NWK, BWD_NSQ, BWD_NSK>(p, s)
         : causal ? launch_backward<128, 64, true, false, BWD_NWQ, BWD_NWK, BWD_NSQ, BWD_NSK>(p, s)
                  : launch_backward<128, 64, false, false, BWD_NWQ, BWD_NWK, BWD_NSQ, BWD_NSK>(p, s);
}

}  // namespace attn
