// The projection GEMM kernels and their launchers (see gemm_launch.hpp).
#include "gemm_launch.hpp"

namespace gqe {

void launch_proj_gemm_bf16(const ProjArgs& a, unsigned grid, hipStream_t st) {
    hipLaunchKernelGGL((proj_gemm_kernel<bf16, ProjBf16>), dim3(grid), dim3(ProjBf16::NTH), 0, st, a);
}
void launch_proj_gemm_f32(const ProjArgs& a, unsigned grid, hipStream_t st) {
    hipLaunchKernelGGL((proj_gemm_kernel<float, ProjF32>), dim3(grid), dim3(ProjF32::NTH), 0, st, a);
}
void launch_grouped_q_bf16(const GroupArgs& g, unsigned grid, hipStream_t st) {
    hipLaunchKernelGGL((grouped_q_kernel<bf16, GrpBf16>), dim3(grid), dim3(GrpBf16::NTH), 0, st, g);
}
void launch_grouped_q_f32(const GroupArgs& g, unsigned grid, hipStream_t st) {
    hipLaunchKernelGGL((grouped_q_kernel<float, GrpF32>), dim3(grid), dim3(GrpF32::NTH), 0, st, g);
}
void launch_skinny_proj(const ProjArgs& a, unsigned grid, hipStream_t st) {
    hipLaunchKernelGGL(skinny_proj_kernel<bf16>, dim3(grid), dim3(256), 0, st, a);
}

}  // namespace gqe
