// Instantiation of the GEMM mainloop for one operand mode: NVFP4 weight GEMM with NVFP4 activations.
#include "gemm_kernel.h"

namespace bi {

hipError_t launch_gemm_nvfp4a(const GemmRecipe &r, const GemmArgs &a, int grid, hipStream_t s) {
    return gemm_detail::launch_modes<OPND_NVFP4_ROWS, OPND_NVFP4_ROWS>(r, a, grid, s);
}

}  // namespace bi
