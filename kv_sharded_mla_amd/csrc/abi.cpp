// C ABI entry points: host-side argument checks, then the kernel launchers.
// Every declaration and its contract is in include/dcp_mla.h.
#include <math.h>

#include "../../include/dcp_mla.h"
#include "dcp_internal.hpp"

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// interleave 0 means one token, as 1 does
int32_t interleave_of(const dcp_layout* l) { return l->interleave < 1 ? 1 : l->interleave; }

int check_layout(const dcp_layout* l) {
  if (!l) return DCP_ERR_INVALID_ARG;
  if (l->c < 1 || l->page < 1 || l->num_pages < 0) return DCP_ERR_INVALID_ARG;
  // every virtual page must give each rank exactly P positions
  if (l->interleave < 0 || l->page % interleave_of(l) != 0) return DCP_ERR_INVALID_ARG;
  if (l->kv_dtype != DCP_KV_BF16 && l->kv_dtype != DCP_KV_FP8_E4M3) return DCP_ERR_INVALID_ARG;
  // every slot index of the group must fit in int64 with room to spare
  if ((int64_t)l->num_pages * l->page > ((int64_t)1 << 40)) return DCP_ERR_UNSUPPORTED;
  return DCP_OK;
}

int row_bytes(const dcp_layout* l) { return l->kv_dtype == DCP_KV_BF16 ? 2 * DCP_D_QK : DCP_D_QK; }

int hip_status(hipError_t e) { return e == hipSuccess ? DCP_OK : DCP_ERR_HIP; }

// Argument checks shared by both decode entry points; on success fills the plan.
int check_decode(const dcp_layout* layout, const void* pools, const float* pool_scales, int32_t rank_begin,
                 int32_t rank_count, const void* q, int32_t batch, int32_t q_len, int32_t heads,
                 const int32_t* block_table, int32_t bt_stride, const int32_t* seq_len, int64_t max_seq_len,
                 float sm_scale, int32_t lse_base, const float* o_part, const float* lse_part, dcp::DecodePlan* pl) {
  if (int s = check_layout(layout)) return s;
  const bool fp8 = layout->kv_dtype == DCP_KV_FP8_E4M3;
  if (rank_begin < 0 || rank_count < 1 || (int64_t)rank_begin + rank_count > layout->c) return DCP_ERR_INVALID_ARG;
  if (batch < 0 || bt_stride < 1 || max_seq_len < 0) return DCP_ERR_INVALID_ARG;
  if (lse_base != DCP_LSE_BASE_E && lse_base != DCP_LSE_BASE_2) return DCP_ERR_INVALID_ARG;
  if (!isfinite(sm_scale)) return DCP_ERR_INVALID_ARG;
  if (q_len < 1 || q_len > DCP_MAX_Q_LEN || heads < 16 || heads % 16 != 0 || heads > 4096)
    return DCP_ERR_UNSUPPORTED;
  if (max_seq_len > INT32_MAX) return DCP_ERR_UNSUPPORTED;
  if (batch == 0) return DCP_OK;
  if (!pools || !q || !block_table || !seq_len || !o_part || !lse_part) return DCP_ERR_INVALID_ARG;
  if (fp8 && !pool_scales) return DCP_ERR_INVALID_ARG;
  if (!aligned(pools, 16) || !aligned(q, 16) || !aligned(o_part, 16) || !aligned(lse_part, 4))
    return DCP_ERR_ALIGNMENT;
  if (fp8 && !aligned(pool_scales, 4)) return DCP_ERR_ALIGNMENT;
  *pl = dcp::plan_decode(layout->c, interleave_of(layout), layout->page, fp8, rank_count, batch, q_len, heads,
                         max_seq_len);
  return DCP_OK;
}

int launch_decode_call(const dcp_layout* layout, const void* pools, const float* pool_scales, int32_t rank_begin,
                       int32_t rank_count, const void* q, int32_t batch, int32_t q_len, int32_t heads,
                       const int32_t* block_table, int32_t bt_stride, const int32_t* seq_len, int64_t max_seq_len,
                       float sm_scale, int32_t lse_base, int32_t causal, float* o_part, float* lse_part,
                       void* workspace, const dcp::DecodePlan& pl, int32_t* dev_status, hipStream_t stream) {
  const bool fp8 = layout->kv_dtype == DCP_KV_FP8_E4M3;
  dcp::DecodeArgs a{};
  a.c = layout->c;
  a.interleave = interleave_of(layout);
  a.page = layout->page;
  a.num_pages = layout->num_pages;
  a.fp8 = fp8;
  a.pools = pools;
  a.pool_scales = pool_scales;
  a.rank_begin = rank_begin;
  a.rank_count = rank_count;
  a.q = q;
  a.batch = batch;
  a.q_len = q_len;
  a.heads = heads;
  a.block_table = block_table;
  a.bt_stride = bt_stride;
  a.seq_len = seq_len;
  a.max_seq_len = max_seq_len;
  a.sm_scale = sm_scale;
  a.base2 = lse_base == DCP_LSE_BASE_2;
  a.causal = causal != 0;
  a.o_part = o_part;
  a.lse_part = lse_part;
  a.workspace = workspace;
  a.dev_status = dev_status;
  return hip_status(dcp::launch_decode(a, pl, stream));
}


}  // namespace

extern "C" {

int64_t dcp_pool_bytes(const dcp_layout* layout) {
  if (check_layout(layout) != DCP_OK) return -1;
  return (int64_t)layout->num_pages * layout->page * row_bytes(layout);
}

int dcp_alloc_virtual(const dcp_layout* layout, const int32_t* free_stack, int32_t* free_top,
                      const int32_t* old_len, const int32_t* new_len, int32_t batch, int32_t* block_table,
                      int32_t bt_stride, int32_t* dev_status, hipStream_t stream) {
  if (int s = check_layout(layout)) return s;
  if (batch < 0 || batch > 65536 || bt_stride < 1) return DCP_ERR_INVALID_ARG;
  if (!free_top) return DCP_ERR_INVALID_ARG;
  if (batch > 0 && (!old_len || !new_len || !block_table)) return DCP_ERR_INVALID_ARG;
  if (!free_stack && layout->num_pages > 0) return DCP_ERR_INVALID_ARG;
  if ((int64_t)layout->page * layout->c > INT32_MAX) return DCP_ERR_UNSUPPORTED;
  return hip_status(dcp::launch_alloc_virtual(layout->c, layout->page, free_stack, free_top, old_len, new_len,
                                              batch, block_table, bt_stride, dev_status, stream));
}

int dcp_kv_write(const dcp_layout* layout, void* pools, float* pool_scales, const int32_t* block_table,
                 int32_t bt_stride, const int32_t* seq_len, const int32_t* cu_new, int32_t batch, int64_t n_rows,
                 const void* rows, const float* row_scales, int64_t* slot_out, int32_t* dev_status,
                 hipStream_t stream) {
  if (int s = check_layout(layout)) return s;
  const bool fp8 = layout->kv_dtype == DCP_KV_FP8_E4M3;
  if (batch < 0 || n_rows < 0 || bt_stride < 1) return DCP_ERR_INVALID_ARG;
  if (n_rows > 0 && batch == 0) return DCP_ERR_INVALID_ARG;
  if (n_rows == 0) return DCP_OK;
  if (!pools || !block_table || !seq_len || !cu_new || !rows) return DCP_ERR_INVALID_ARG;
  if (fp8 && (!pool_scales || !row_scales)) return DCP_ERR_INVALID_ARG;
  if (!aligned(pools, 16) || !aligned(rows, 16)) return DCP_ERR_ALIGNMENT;
  if (fp8 && (!aligned(pool_scales, 4) || !aligned(row_scales, 4))) return DCP_ERR_ALIGNMENT;
  if (slot_out && !aligned(slot_out, 8)) return DCP_ERR_ALIGNMENT;
  return hip_status(dcp::launch_kv_write(layout->c, interleave_of(layout), layout->page, layout->num_pages, fp8, pools, pool_scales,
                                         block_table, bt_stride, seq_len, cu_new, batch, n_rows, rows, row_scales,
                                         slot_out, dev_status, stream));
}

int dcp_kv_read(const dcp_layout* layout, const void* pools, const float* pool_scales, const int32_t* block_table,
                int32_t bt_stride, const int32_t* seq_len, const int32_t* cu_out, int32_t batch, int64_t n_rows,
                void* rows_out, float* scales_out, int32_t* dev_status, hipStream_t stream) {
  if (int s = check_layout(layout)) return s;
  const bool fp8 = layout->kv_dtype == DCP_KV_FP8_E4M3;
  if (batch < 0 || batch > 65536 || n_rows < 0 || bt_stride < 1) return DCP_ERR_INVALID_ARG;
  if ((int64_t)layout->page * layout->c > (1 << 30)) return DCP_ERR_UNSUPPORTED;
  if (batch == 0) return DCP_OK;
  if (!pools || !block_table || !seq_len || !cu_out || (n_rows > 0 && !rows_out)) return DCP_ERR_INVALID_ARG;
  if (fp8 && (!pool_scales || (n_rows > 0 && !scales_out))) return DCP_ERR_INVALID_ARG;
  if (!aligned(pools, 16) || !aligned(rows_out, 16)) return DCP_ERR_ALIGNMENT;
  if (fp8 && (!aligned(pool_scales, 4) || !aligned(scales_out, 4))) return DCP_ERR_ALIGNMENT;
  return hip_status(dcp::launch_kv_read(layout->c, interleave_of(layout), layout->page, layout->num_pages, fp8, pools,
                                        pool_scales, block_table, bt_stride, seq_len, cu_out, batch, n_rows, rows_out,
                                        scales_out, dev_status, stream));
}

int dcp_kv_relayout(const dcp_layout* layout, const void* src_pool, const float* src_scales, int32_t src_num_pages,
                    const int32_t* src_block_table, int32_t src_bt_stride, const int32_t* seq_len, int32_t batch,
                    int32_t rank_begin, int32_t rank_count, void* pools, float* pool_scales,
                    const int32_t* block_table, int32_t bt_stride, int32_t* dev_status, hipStream_t stream) {
  if (int s = check_layout(layout)) return s;
  const bool fp8 = layout->kv_dtype == DCP_KV_FP8_E4M3;
  if (batch < 0 || batch > 65536 || bt_stride < 1 || src_bt_stride < 1 || src_num_pages < 0) return DCP_ERR_INVALID_ARG;
  if (rank_begin < 0 || rank_count < 1 || (int64_t)rank_begin + rank_count > layout->c) return DCP_ERR_INVALID_ARG;
  if ((int64_t)layout->page * layout->c > (1 << 30)) return DCP_ERR_UNSUPPORTED;
  if ((int64_t)src_num_pages * layout->page > ((int64_t)1 << 40)) return DCP_ERR_UNSUPPORTED;
  if (batch == 0) return DCP_OK;
  if (!src_pool || !src_block_table || !seq_len || !pools || !block_table) return DCP_ERR_INVALID_ARG;
  if (fp8 && (!src_scales || !pool_scales)) return DCP_ERR_INVALID_ARG;
  if (!aligned(src_pool, 16) || !aligned(pools, 16)) return DCP_ERR_ALIGNMENT;
  if (fp8 && (!aligned(src_scales, 4) || !aligned(pool_scales, 4))) return DCP_ERR_ALIGNMENT;
  return hip_status(dcp::launch_kv_relayout(layout->c, interleave_of(layout), layout->page, layout->num_pages, fp8,
                                            src_pool, src_scales, src_num_pages, src_block_table, src_bt_stride,
                                            seq_len, batch, rank_begin, rank_count, pools, pool_scales, block_table,
                                            bt_stride, dev_status, stream));
}

size_t mla_decode_workspace_size(const dcp_layout* layout, int32_t rank_count, int32_t batch, int32_t q_len,
                                 int32_t heads, int64_t max_seq_len) {
  if (check_layout(layout) != DCP_OK || rank_count < 1 || batch < 0 || q_len < 1 || q_len > DCP_MAX_Q_LEN ||
      heads < 16 || heads % 16 != 0 || max_seq_len < 0)
    return 0;
  dcp::DecodePlan pl = dcp::plan_decode(layout->c, interleave_of(layout), layout->page,
                                        layout->kv_dtype == DCP_KV_FP8_E4M3, rank_count, batch, q_len, heads,
                                        max_seq_len);
  return pl.workspace_bytes;
}

int mla_decode_partial(const dcp_layout* layout, const void* pools, const float* pool_scales, int32_t rank_begin,
                       int32_t rank_count, const void* q, int32_t batch, int32_t q_len, int32_t heads,
                       const int32_t* block_table, int32_t bt_stride, const int32_t* seq_len, int64_t max_seq_len,
                       float sm_scale, int32_t lse_base, int32_t causal, float* o_part, float* lse_part,
                       void* workspace, size_t workspace_bytes, int32_t* dev_status, hipStream_t stream) {
  dcp::DecodePlan pl{};
  const int s = check_decode(layout, pools, pool_scales, rank_begin, rank_count, q, batch, q_len, heads, block_table,
                             bt_stride, seq_len, max_seq_len, sm_scale, lse_base, o_part, lse_part, &pl);
  if (s != DCP_OK || batch == 0) return s;
  if (!workspace || workspace_bytes < pl.workspace_bytes) return DCP_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return DCP_ERR_ALIGNMENT;
  return launch_decode_call(layout, pools, pool_scales, rank_begin, rank_count, q, batch, q_len, heads, block_table,
                            bt_stride, seq_len, max_seq_len, sm_scale, lse_base, causal, o_part, lse_part, workspace,
                            pl, dev_status, stream);
}

int mla_decode_partial_noalloc(const dcp_layout* layout, const void* pools, const float* pool_scales,
                               int32_t rank_begin, int32_t rank_count, const void* q, int32_t batch, int32_t q_len,
                               int32_t heads, const int32_t* block_table, int32_t bt_stride, const int32_t* seq_len,
                               int64_t max_seq_len, float sm_scale, int32_t lse_base, int32_t causal, float* o_part,
                               float* lse_part, int32_t* dev_status, hipStream_t stream) {
  dcp::DecodePlan pl{};
  const int s = check_decode(layout, pools, pool_scales, rank_begin, rank_count, q, batch, q_len, heads, block_table,
                             bt_stride, seq_len, max_seq_len, sm_scale, lse_base, o_part, lse_part, &pl);
  if (s != DCP_OK || batch == 0) return s;
  if (pl.workspace_bytes > dcp::kScratchBytes) return DCP_ERR_WORKSPACE;
  void* ws = nullptr;
  if (dcp::decode_scratch(&ws) != hipSuccess) return DCP_ERR_HIP;
  return launch_decode_call(layout, pools, pool_scales, rank_begin, rank_count, q, batch, q_len, heads, block_table,
                            bt_stride, seq_len, max_seq_len, sm_scale, lse_base, causal, o_part, lse_part, ws, pl,
                            dev_status, stream);
}

size_t mla_decode_noalloc_scratch_bytes(void) { return dcp::kScratchBytes; }

int dcp_lse_merge(int32_t c, int64_t rows, const float* o_part, const float* lse_part, int32_t lse_base,
                  void* o_out, float* lse_out, hipStream_t stream) {
  if (c < 1 || rows < 0) return DCP_ERR_INVALID_ARG;
  if (lse_base != DCP_LSE_BASE_E && lse_base != DCP_LSE_BASE_2) return DCP_ERR_INVALID_ARG;
  if (rows == 0) return DCP_OK;
  if (!o_part || !lse_part || !o_out || !lse_out) return DCP_ERR_INVALID_ARG;
  if (!aligned(o_part, 16) || !aligned(o_out, 8) || !aligned(lse_part, 4) || !aligned(lse_out, 4))
    return DCP_ERR_ALIGNMENT;
  return hip_status(dcp::launch_lse_merge(c, rows, o_part, lse_part, lse_base == DCP_LSE_BASE_2, o_out, lse_out,
                                          stream));
}

const char* dcp_status_string(int status) {
  switch (status) {
    case DCP_OK: return "ok";
    case DCP_ERR_INVALID_ARG: return "invalid argument";
    case DCP_ERR_UNSUPPORTED: return "unsupported shape";
    case DCP_ERR_ALIGNMENT: return "pointer not aligned";
    case DCP_ERR_WORKSPACE: return "workspace too small";
    case DCP_ERR_HIP: return "HIP launch failed";
    case DCP_DEV_OUT_OF_PAGES: return "device: out of pages";
    case DCP_DEV_BAD_LENGTH: return "device: bad length";
    case DCP_DEV_TABLE_OVERFLOW: return "device: block table overflow";
    case DCP_DEV_BAD_PAGE: return "device: page id out of range";
    case DCP_DEV_DECODE_STALLED: return "device: decode wave stopped waiting for its partner";
    default: return "unknown status";
  }
}

}  // extern "C"
