// Split-KV decode (with its in-launch merge) and LSE-merge instantiations.
#include "combine.hpp"
#include "decode.hpp"
#include "kernels.hpp"

namespace attn {

int decode_block_rows(int d) { return (d == 64 || d == 128 || d == 256) ? 128 : 0; }

hipError_t decode_split(int d, const DecodeParams &p, hipStream_t s) {
  switch (d) {
    case 64: return launch_decode_split<64, 4, 64, 2, 4>(p, s);
    case 128: return launch_decode_split<128, 4, 32, 2, 3>(p, s);
    default: return launch_decode_split<256, 4, 32, 2, 2>(p, s);
  }
}

hipError_t decode_split_paged(int d, const DecodeParams &p, hipStream_t s) {
  switch (d) {
    case 64: return launch_decode_split<64, 4, 64, 2, 4, true>(p, s);
    case 128: return launch_decode_split<128, 4, 32, 2, 3, true>(p, s);
    default: return launch_decode_split<256, 4, 32, 2, 2, true>(p, s);
  }
}

hipError_t decode_split_fp8(int d, const DecodeParams &p, hipStream_t s) {
  switch (d) {
    case 128: return launch_decode_split<128, 4, 32, 2, 3, false, true>(p, s);
    case 256: return launch_decode_split<256, 4, 32, 2, 2, false, true>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t decode_split_paged_fp8(int d, const DecodeParams &p, hipStream_t s) {
  switch (d) {
    case 128: return launch_decode_split<128, 4, 32, 2, 3, true, true>(p, s);
    case 256: return launch_decode_split<256, 4, 32, 2, 2, true, true>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t combine(const CombineParams &p, hipStream_t s) { return launch_combine<float>(p, s); }
hipError_t combine_bf16(const CombineParams &p, hipStream_t s) { return launch_combine<uint16_t>(p, s); }

}  // namespace attn
