// Launchers of the bf16 projection kernels (v41_gemm.hip); arguments are
// validated by the C ABI layer before a launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace v41 {

struct LinearArgs {
  const uint16_t* a;
  int64_t lda, a_gs;
  const uint16_t* w;
  int64_t ldw, w_gs;
  uint16_t* y;
  int64_t ldy, y_gs;
  int32_t M, N, K, groups;
  void* workspace;
  int64_t workspace_bytes;
};

int gemm_splits(int32_t M, int32_t N, int32_t K, int32_t groups);
int64_t gemm_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t groups);
hipError_t launch_linear_bf16(const LinearArgs& a, hipStream_t s);

}  // namespace v41
