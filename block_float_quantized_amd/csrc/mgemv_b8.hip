// Instantiates the matrix-core skinny matmul for BFP8 weights.
#include "mfma_gemv.hpp"

namespace bfp {

hipError_t mfma_gemv_launch_b8(const mg::MgArgs& a, bool x_bf16, hipStream_t s) {
  return x_bf16 ? mg::launch<8, 1>(a, s) : mg::launch<8, 2>(a, s);
}

}  // namespace bfp
