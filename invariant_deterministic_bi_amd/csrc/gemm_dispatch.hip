// Dispatch of a GEMM-family launch to the instantiation for its operand modes.
#include "bi_internal.h"

namespace bi {

hipError_t launch_gemm_bf16(const GemmRecipe &r, const GemmArgs &a, int grid, hipStream_t s);
hipError_t launch_gemm_kn(const GemmRecipe &r, const GemmArgs &a, int grid, hipStream_t s);
hipError_t launch_gemm_nvfp4(const GemmRecipe &r, const GemmArgs &a, int grid, hipStream_t s);
hipError_t launch_gemm_nvfp4raw(const GemmRecipe &r, const GemmArgs &a, int grid, hipStream_t s);
hipError_t launch_gemm_nvfp4a(const GemmRecipe &r, const GemmArgs &a, int grid, hipStream_t s);

hipError_t launch_gemm(int a_mode, int b_mode, const GemmRecipe &r, const GemmArgs &args,
                       int grid, hipStream_t stream) {
    if (a_mode == OPND_BF16_ROWS && b_mode == OPND_BF16_ROWS)
        return launch_gemm_bf16(r, args, grid, stream);
    if (a_mode == OPND_BF16_ROWS && b_mode == OPND_BF16_KN)
        return launch_gemm_kn(r, args, grid, stream);
    if (a_mode == OPND_BF16_ROWS && b_mode == OPND_NVFP4_ROWS)
        return launch_gemm_nvfp4(r, args, grid, stream);
    if (a_mode == OPND_BF16_ROWS && b_mode == OPND_NVFP4_RAW)
        return launch_gemm_nvfp4raw(r, args, grid, stream);
    if (a_mode == OPND_NVFP4_ROWS && b_mode == OPND_NVFP4_ROWS)
        return launch_gemm_nvfp4a(r, args, grid, stream);
    return hipErrorInvalidValue;
}

}  // namespace bi
