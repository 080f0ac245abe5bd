// Bit-plane W_b A8 kernels for b = 5..8 (the policy is in bitplane.h).
#include "bitplane.h"

namespace qg {

hipError_t launch_bitplane_hi(const Plan& pl, const GemmArgs& a, int bits, hipStream_t s) {
  switch (bits) {
    case 5: return dispatch_skinny<fmt::PolicyBP<5>>(pl, a, s);
    case 6: return dispatch_skinny<fmt::PolicyBP<6>>(pl, a, s);
    case 7: return dispatch_skinny<fmt::PolicyBP<7>>(pl, a, s);
    case 8: return dispatch_skinny<fmt::PolicyBP<8>>(pl, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qg
