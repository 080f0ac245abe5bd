// Bit-plane W_b A8 kernels for b = 1..4 (the policy is in bitplane.h).
#include "bitplane.h"

namespace qg {

size_t lds_bytes_bitplane(const Plan& pl, int G) { return skinny_lds_bytes<fmt::PolicyBP<1>>(pl, G); }

hipError_t launch_bitplane_lo(const Plan& pl, const GemmArgs& a, int bits, hipStream_t s) {
  switch (bits) {
    case 1: return dispatch_skinny<fmt::PolicyBP<1>>(pl, a, s);
    case 2: return dispatch_skinny<fmt::PolicyBP<2>>(pl, a, s);
    case 3: return dispatch_skinny<fmt::PolicyBP<3>>(pl, a, s);
    case 4: return dispatch_skinny<fmt::PolicyBP<4>>(pl, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qg
