// Instantiation of the GEMM mainloop for one operand mode: BMM: A bf16 [M, K], B bf16 [K, N].
#include "gemm_kernel.h"

namespace bi {

hipError_t launch_gemm_kn(const GemmRecipe &r, const GemmArgs &a, int grid, hipStream_t s) {
    return gemm_detail::launch_modes<OPND_BF16_ROWS, OPND_BF16_KN>(r, a, grid, s);
}

}  // namespace bi
