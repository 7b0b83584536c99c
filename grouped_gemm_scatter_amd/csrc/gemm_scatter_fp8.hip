// Blockwise-scaled fp8 grouped GEMM with the receive-buffer sink epilogue.
#include "ep_kernels.h"

namespace ep {

hipError_t launch_gemm_fp8(const GemmArgs& a, int tile, int grid, hipStream_t st) {
  (void)a; (void)tile; (void)grid; (void)st;
  return hipErrorNotSupported;
}

}  // namespace ep
