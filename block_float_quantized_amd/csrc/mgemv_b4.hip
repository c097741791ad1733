// Instantiates the matrix-core skinny matmul for BFP4 weights.
#include "mfma_gemv.hpp"

namespace bfp {

hipError_t mfma_gemv_launch_b4(const mg::MgArgs& a, bool x_bf16, hipStream_t s) {
  return x_bf16 ? mg::launch<4, 1>(a, s) : mg::launch<4, 2>(a, s);
}

}  // namespace bfp
