// Tile configurations of the projection GEMMs and the host-side launchers of
// their kernels. The kernels are instantiated in gemm_launch.hip, a unit of
// their own: its compilation schedules for instruction-level parallelism
// (the K loop then keeps the next step's LDS fragment reads in flight behind
// the current step's MFMAs), which the attention kernels, compiled with the
// occupancy-first default, do not want.
#pragma once

#include "gemm.hpp"

namespace gqe {

// Projection GEMM: 128 x 128 tiles of eight waves (32 x 64 each), two
// workgroups per CU, four waves per SIMD.
#ifndef GQE_PROJ_CFG
#define GQE_PROJ_CFG 128, 128, 4, 2, 4
#endif
using ProjBf16 = TileCfg<bf16, GQE_PROJ_CFG>;
using ProjF32 = TileCfg<float, 128, 128, 2, 2>;
// The grouped routed-Q GEMM: 256 x 64 tiles (256 rows of one expert's
// segment, its 64 query columns), eight waves of 32 x 64, two workgroups per
// CU (80 KB of LDS each, 86 VGPRs), so four waves per SIMD. A wave's K step
// is short (8 MFMAs per 32-wide step), so the tile loads need many waves to
// hide behind: against 128 x 64 tiles at two per CU, 72 -> 58 us at T = 32K
// and 367 -> 288 us on the k = 2, D = 2048 workload.
#ifndef GQE_GRP_CFG
#define GQE_GRP_CFG 256, 64, 8, 1, 4
#endif
using GrpBf16 = TileCfg<bf16, GQE_GRP_CFG>;
using GrpF32 = TileCfg<float, 128, 64, 4, 1>;

// Enqueue the kernels on `st` with `grid` workgroups (block size from the
// configuration); errors surface through hipGetLastError.
void launch_proj_gemm_bf16(const ProjArgs& a, unsigned grid, hipStream_t st);
void launch_proj_gemm_f32(const ProjArgs& a, unsigned grid, hipStream_t st);
void launch_grouped_q_bf16(const GroupArgs& g, unsigned grid, hipStream_t st);
void launch_grouped_q_f32(const GroupArgs& g, unsigned grid, hipStream_t st);
void launch_skinny_proj(const ProjArgs& a, unsigned grid, hipStream_t st);

}  // namespace gqe
