// Instantiation of the GEMM mainloop for one operand mode: NVFP4 weight GEMM
// with bf16 activations, weight bytes streamed into a raw LDS ring (K % 64 == 0).
#include "gemm_kernel.h"

namespace bi {

hipError_t launch_gemm_nvfp4raw(const GemmRecipe &r, const GemmArgs &a, int grid, hipStream_t s) {
    return gemm_detail::launch_modes<OPND_BF16_ROWS, OPND_NVFP4_RAW>(r, a, grid, s);
}

}  // namespace bi
