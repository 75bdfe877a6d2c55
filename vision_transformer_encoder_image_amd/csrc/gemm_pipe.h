// Tile configurations of the multi-stage bf16 GEMM (gemm_pipe.hip).  Every
// configuration keeps at least 3 LDS stages (the stage being multiplied, the
// next one being read into fragments, and one or more copies in flight).
#pragma once

#include "common.h"

enum GemmPipeCfg {
  GEMM_PIPE_128x128_S4 = 0,     // 4 waves of 64x64, 4 LDS stages (128 KB)
  GEMM_PIPE_128x128_S3 = 1,     // 4 waves of 64x64, 3 stages (96 KB)
  GEMM_PIPE_256x128_S3 = 2,     // 4 waves of 128x64, 3 stages (144 KB)
  GEMM_PIPE_128x256_S3 = 3,     // 4 waves of 64x128, 3 stages (144 KB)
  GEMM_PIPE_256x128_W8_S3 = 4,  // 8 waves of 64x64, 3 stages (144 KB)
  GEMM_PIPE_256x256_K32_S4 = 5,     // 4 waves of 128x128, BK 32, 4 stages (128 KB)
  GEMM_PIPE_256x256_W8_K32_S4 = 6,  // 8 waves of 128x64, BK 32, 4 stages (128 KB)
  GEMM_PIPE_128x128_W2_K32_S4 = 7,  // 2 waves of 128x64, BK 32, 4 stages (64 KB), 2 per CU
  GEMM_PIPE_NCFG = 8,
};

hipError_t launch_gemm_pipe(int cfg, int epi, const GemmArgs& g, hipStream_t s);
// one tile per workgroup, 128x128 (gemm_tile.hip)
hipError_t launch_gemm_tile128(int epi, const GemmArgs& g, hipStream_t s);
