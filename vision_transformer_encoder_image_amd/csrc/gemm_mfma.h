// Tile configurations of the bf16 MFMA GEMM (gemm_mfma.hip).
#pragma once

#include "common.h"

enum GemmMfmaCfg {
  GEMM_MFMA_128x128 = 0,     // 8 waves of 32x64, 4 LDS stages of BK 64 (128 KB)
  GEMM_MFMA_256x128_W8 = 1,  // 8 waves of 64x64, 3 stages of BK 64 (144 KB)
  GEMM_MFMA_256x256_W8 = 2,  // 8 waves of 128x64, 4 stages of BK 32 (128 KB)
  GEMM_MFMA_192x256 = 3,     // 4 waves of 96x128 (accumulators in AGPRs), 4 stages of BK 32 (112 KB)
  GEMM_MFMA_64x64_W2 = 4,    // 2 waves of 32x64, 4 stages of BK 64 (64 KB: two workgroups per CU)
  GEMM_MFMA_NCFG = 5,
};

// g1 (optional): a second GEMM of the same configuration and epilogue in the
// same launch (its workgroups follow g's)
hipError_t launch_gemm_mfma(int cfg, int epi, const GemmArgs& g, hipStream_t s,
                            const GemmArgs* g1 = nullptr);

// Two GEMMs with different tile configurations (of one workgroup size) in one
// launch: g0's tiles (cfg0) take the lower workgroup ids.  hipErrorNotSupported
// when that pair of configurations is not built.
hipError_t launch_gemm_mfma_pair(int cfg0, int cfg1, int epi, const GemmArgs& g0,
                                 const GemmArgs& g1, hipStream_t s);

// Launch plan of one GEMM: cfg_main over columns [0, n_main), and when
// n_main < N a second launch of cfg_tail over [n_main, N).
struct GemmSplit {
  int cfg_main;
  int64_t n_main;
  int cfg_tail;
};
