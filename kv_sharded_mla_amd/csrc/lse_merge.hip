// Exact log-sum-exp merge of c rank partials (SGLang "Decode Context
// Parallelism", section "MLA decode dataflow"): lse = logsumexp_r lse_r,
// o = sum_r exp(lse_r - lse) * o_r, in the base of the partials.  On one GPU
// this kernel stands in for the group's packed all-to-all plus the merge.
// Memory-bound: reads c*(512+1)*4 bytes and writes 512*2 + 4 bytes per row.
#include "dcp_common.hpp"
#include "dcp_internal.hpp"

namespace dcp {

namespace {

// Two rows per 256-thread block; thread t of a row owns columns 4t..4t+3.
__global__ void __launch_bounds__(256)
lse_merge_kernel(int32_t c, int64_t rows, const float* __restrict__ o_part, const float* __restrict__ lse_part,
                 int32_t base2, uint16_t* __restrict__ o_out, float* __restrict__ lse_out) {
  const int64_t row = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 7);
  const int col4 = threadIdx.x & 127;
  if (row >= rows) return;
  f32x4 acc;
  float lse;
  merge_row4(o_part + row * kDv, rows * kDv, lse_part + row, rows, c, base2 != 0, col4, acc, lse);
  uint32_t lo = (uint32_t)f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
  uint32_t hi = (uint32_t)f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
  *reinterpret_cast<uint2*>(o_out + row * kDv + 4 * col4) = make_uint2(lo, hi);
  if (col4 == 0) lse_out[row] = lse;
}

}  // namespace

hipError_t launch_lse_merge(int32_t c, int64_t rows, const float* o_part, const float* lse_part, bool base2,
                            void* o_out, float* lse_out, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)((rows + 1) / 2)), dim3(256), 0, stream, c, rows, o_part,
                     lse_part, base2 ? 1 : 0, (uint16_t*)o_out, lse_out);
  return hipGetLastError();
}

}  // namespace dcp
