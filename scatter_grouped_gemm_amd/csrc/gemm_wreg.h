// Internal interface of the register-streamed grouped GEMM (gemm_wreg.hip),
// used by the C entry points in gemm.hip for the compact layout.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct WregArgs {
  const uint8_t* A;        // activations [M][K] (bf16 or e4m3)
  const uint8_t* A_scale;  // FP8: [K/128][M] UE8M0 bytes
  const uint8_t* B;        // weights [G][N][K] (bf16 or e4m3)
  const uint8_t* B_scale;  // FP8: [G][N/128][K/128]
  void* C;                 // plain: bf16 [M][N]; SiLU: the activation [M][N/2]
  uint8_t* C_scale;        // SiLU with e4m3 output: [N/256][M]
  const int32_t* m_indices;
  int64_t M;
  int N, K, G;
};

// Epilogues of the register-streamed kernel (same meaning as the LDS-staged
// kernel's): plain bf16 product, SiLU-and-mul to bf16, SiLU-and-mul to e4m3.
constexpr int kWrEpiPlain = 0, kWrEpiSiluBf16 = 1, kWrEpiSiluFp8 = 2;

// True when the register-streamed kernel covers this compact GEMM (N a
// multiple of 256, one expert's weights under 2 GiB, at most 8160 row blocks).
bool wreg_supported(int64_t M, int N, int K, int G, bool fp8);

// Enqueue the compact grouped GEMM (fp8: e4m3 operands with 128x128 weight
// blocks and 128-channel activation scales; else bf16).
int32_t launch_wreg(const WregArgs& a, bool fp8, int epi, hipStream_t s);

}  // namespace moe
