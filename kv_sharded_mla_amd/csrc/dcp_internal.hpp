// Host-side launchers behind the C ABI (argument checking happens in abi.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dcp {

hipError_t launch_alloc_virtual(int32_t c, int32_t page, const int32_t* free_stack, int32_t* free_top,
                                const int32_t* old_len, const int32_t* new_len, int32_t batch,
                                int32_t* block_table, int32_t bt_stride, int32_t* dev_status,
                                hipStream_t stream);

hipError_t launch_kv_write(int32_t c, int32_t interleave, int32_t page, int32_t num_pages, bool fp8, void* pools,
                           float* pool_scales, const int32_t* block_table, int32_t bt_stride,
                           const int32_t* seq_len, const int32_t* cu_new, int32_t batch,
                           int64_t n_rows, const void* rows, const float* row_scales,
                           int64_t* slot_out, int32_t* dev_status, hipStream_t stream);

hipError_t launch_kv_read(int32_t c, int32_t interleave, int32_t page, int32_t num_pages, bool fp8, const void* pools,
                          const float* pool_scales, const int32_t* block_table, int32_t bt_stride,
                          const int32_t* seq_len, const int32_t* cu_out, int32_t batch, int64_t n_rows,
                          void* rows_out, float* scales_out, int32_t* dev_status, hipStream_t stream);

hipError_t launch_kv_relayout(int32_t c, int32_t interleave, int32_t page, int32_t num_pages, bool fp8,
                              const void* src_pool, const float* src_scales, int32_t src_num_pages,
                              const int32_t* src_table, int32_t src_stride, const int32_t* seq_len, int32_t batch,
                              int32_t rank_begin, int32_t rank_count, void* pools, float* pool_scales,
                              const int32_t* block_table, int32_t bt_stride, int32_t* dev_status,
                              hipStream_t stream);

hipError_t launch_lse_merge(int32_t c, int64_t rows, const float* o_part, const float* lse_part,
                            bool base2, void* o_out, float* lse_out, hipStream_t stream);

// Work decomposition of one mla_decode_partial call.  The split of each
// (rank, request) into work items is planned on the device at every call;
// the host fixes the row blocking and bounds the number of items.
struct DecodePlan {
  int32_t rows;            // q_len * heads
  int32_t row_block;       // query rows per workgroup (16, 32 or 64)
  int32_t n_row_blocks;    // rows / row_block
  int32_t stage_tokens;    // tokens per LDS stage
  int64_t units;           // rank_count * batch
  int32_t items_target;    // work items per row block the device plan aims for
  int32_t t_min, t_max;    // item length bounds in stages
  int64_t max_items;       // bound on the items the device plan makes
  bool direct;             // no unit longer than t_min stages: one item per unit, no plan
  size_t off_ws_lse;       // workspace: partial o, then partial lse, then the plan
  size_t off_ints;
  size_t workspace_bytes;
};

DecodePlan plan_decode(int32_t c, int32_t interleave, int32_t page, bool fp8, int32_t rank_count, int32_t batch,
                       int32_t q_len, int32_t heads, int64_t max_seq_len);

struct DecodeArgs {
  int32_t c, interleave, page, num_pages;
  bool fp8;
  const void* pools;
  const float* pool_scales;
  int32_t rank_begin, rank_count;
  const void* q;
  int32_t batch, q_len, heads;
  const int32_t* block_table;
  int32_t bt_stride;
  const int32_t* seq_len;
  int64_t max_seq_len;
  float sm_scale;
  bool base2;
  bool causal;
  float* o_part;
  float* lse_part;
  void* workspace;
  int32_t* dev_status;
};

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream);

// Bytes of the file-scope scratch array the allocation-free decode entry
// point uses instead of a caller's workspace.
constexpr size_t kScratchBytes = (size_t)256 << 20;

// Device address of that array on the current device (looked up once per
// device; no allocation).
hipError_t decode_scratch(void** ptr);

int device_cu_count();

}  // namespace dcp
