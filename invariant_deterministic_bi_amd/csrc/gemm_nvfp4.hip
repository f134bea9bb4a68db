// Instantiation of the GEMM mainloop for one operand mode: NVFP4 weight GEMM with bf16 activations.
#include "gemm_kernel.h"

namespace bi {

hipError_t launch_gemm_nvfp4(const GemmRecipe &r, const GemmArgs &a, int grid, hipStream_t s) {
    return gemm_detail::launch_modes<OPND_BF16_ROWS, OPND_NVFP4_ROWS>(r, a, grid, s);
}

}  // namespace bi
