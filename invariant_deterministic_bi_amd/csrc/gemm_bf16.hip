// Instantiation of the GEMM mainloop for one operand mode: dense bf16 GEMM: A and B both bf16 [rows, K].
#include "gemm_kernel.h"

namespace bi {

hipError_t launch_gemm_bf16(const GemmRecipe &r, const GemmArgs &a, int grid, hipStream_t s) {
    return gemm_detail::launch_modes<OPND_BF16_ROWS, OPND_BF16_ROWS>(r, a, grid, s);
}

}  // namespace bi
