/*
 * dcp_mla.h - C ABI of the MI355X (gfx950) decode-context-parallel MLA hot path.
 *
 * Decode context parallelism (DCP) stripes one request's latent KV cache over a
 * group of c ranks by token position: rank r owns the positions p with
 * p mod c = r (SGLang documentation page "Decode Context Parallelism",
 * introduction).  Each rank attends its own shard and returns a locally
 * normalised output o_r with its log-sum-exp lse_r; the group merges the
 * partials exactly (same page, section "MLA decode dataflow").
 *
 * One library instance serves either a real rank (rank_count = 1) or, on one
 * GPU, an emulated group of c owner pools laid out back to back in HBM
 * (rank_begin = 0, rank_count = c), with dcp_lse_merge standing in for the
 * group's all-to-all.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers named in the argument lists are DEVICE pointers unless marked
 *   "host".  The caller owns every buffer; the library allocates and frees
 *   nothing and keeps no state between calls (several streams may use it at
 *   once on disjoint buffers).
 * - Every call only enqueues work on `stream` (0 = the null stream) and never
 *   synchronises.
 * - A negative return value is a host-detected argument error: nothing was
 *   enqueued and no buffer changed.  DCP_ERR_HIP reports a failed launch.
 * - Errors that depend on device-resident values (lengths, page ids) are
 *   reported by raising *dev_status (int32, device) to the largest
 *   DCP_DEV_* code met; the caller clears it to 0 beforehand and reads it
 *   when convenient.  dev_status may be NULL to skip the report.
 * - bf16 values are raw 16-bit bfloat16 payloads.  The e4m3 KV format is OCP
 *   FP8 E4M3FN codes with one float32 scale per token row
 *   (value = decode(code) * scale).
 * - Latent rows are DCP_D_QK = 576 wide: 512 latent columns then 64 rope
 *   columns.  V is the first DCP_D_V = 512 columns of the same row (vLLM
 *   GLM-5.3 blog post, section "Why the numbers add up": QK over 576
 *   dimensions, PV over 512).
 * - Pool layout: rank r's pool is [num_pages][page][row] with
 *   row = 1152 bytes (bf16) or 576 bytes (e4m3); a pool's physical slot s is
 *   row s.  The c pools sit back to back (pool r at pools + r*pool_bytes).
 *   e4m3 scales live apart in float32 [c][num_pages*page].
 * - Block table: int32 [batch][bt_stride]; entry g of request b is the page
 *   id of its g-th virtual page.  The same table serves every rank (a
 *   virtual page id indexes one physical page in every owner pool).
 */
#ifndef DCP_MLA_H
#define DCP_MLA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DCP_D_QK 576
#define DCP_D_V 512
#define DCP_MAX_Q_LEN 8

/* Host-detected status (return values). */
typedef enum dcp_status {
  DCP_OK = 0,
  DCP_ERR_INVALID_ARG = -1, /* null pointer, negative size, bad enum value   */
  DCP_ERR_UNSUPPORTED = -2, /* shape outside what the kernels implement      */
  DCP_ERR_ALIGNMENT = -3,   /* a pointer is not 16-byte aligned              */
  DCP_ERR_WORKSPACE = -4,   /* workspace smaller than the size query returned */
  DCP_ERR_HIP = -5          /* kernel launch failed                          */
} dcp_status;

/* Device-detected status, written to *dev_status (largest code wins). */
enum {
  DCP_DEV_OK = 0,
  DCP_DEV_OUT_OF_PAGES = 1,   /* allocator: free stack too short            */
  DCP_DEV_BAD_LENGTH = 2,     /* a length is negative, shrinks, or exceeds max_seq_len */
  DCP_DEV_TABLE_OVERFLOW = 3, /* a position needs a block-table column >= bt_stride */
  DCP_DEV_BAD_PAGE = 4,       /* a block-table entry is outside [0, num_pages) */
  DCP_DEV_DECODE_STALLED = 5  /* decode: a wave stopped waiting for its partner
                                 wave (never expected; the outputs are invalid) */
};

enum { DCP_KV_BF16 = 0, DCP_KV_FP8_E4M3 = 1 };
enum { DCP_LSE_BASE_E = 0, DCP_LSE_BASE_2 = 1 };

/* Geometry of one DCP group's paged latent cache (host struct). */
typedef struct dcp_layout {
  int32_t c;          /* DCP group size, >= 1                                  */
  int32_t page;       /* physical page size P in tokens, >= 1                  */
  int32_t num_pages;  /* physical pages per owner pool; capacity C = num_pages*page */
  int32_t kv_dtype;   /* DCP_KV_BF16 or DCP_KV_FP8_E4M3                        */
  int32_t interleave; /* KV interleave size I in tokens (0 or 1: one token);
                         I must divide page.  vLLM study page "vLLM Decode
                         Context Parallelism", operation guide, configuration
                         example: consecutive chunks of I positions go to the
                         ranks in turn, owner(p) = floor(p / I) mod c.  Every
                         virtual page of P*c positions still gives each rank P
                         of them, so the block table stays the rank-local page
                         table.  A negative I, or one that does not divide
                         page: DCP_ERR_INVALID_ARG                            */
} dcp_layout;

/* Bytes of one rank's pool (num_pages * page * row bytes). */
int64_t dcp_pool_bytes(const dcp_layout* layout);

/*
 * dcp_alloc_virtual - grow requests in the shared virtual allocator.
 *
 * SGLang "Decode Context Parallelism", section "Virtual KV layout": the group
 * exposes one virtual allocator of capacity C*c with virtual pages of P*c
 * tokens; one virtual page maps to one physical page on every rank, so the
 * ranks stay balanced to within one token.
 *
 * Request b grows from old_len[b] to new_len[b] tokens and needs
 * ceil(new/(P*c)) - ceil(old/(P*c)) new virtual pages.  Pages are popped from
 * the top of free_stack (the k-th page taken overall is
 * free_stack[*free_top - 1 - k]) in (request, logical page) order and written
 * to block_table[b][ceil(old/(P*c)) + i].  *free_top is decreased by the
 * number taken.  All or nothing: on DCP_DEV_BAD_LENGTH (negative or shrinking
 * length), DCP_DEV_TABLE_OVERFLOW (a request needs more than bt_stride
 * pages) or DCP_DEV_OUT_OF_PAGES no entry and no *free_top changes.
 *
 *   free_stack   int32 [*free_top] page ids (read only)
 *   free_top     int32 [1], read and updated
 *   old_len, new_len  int32 [batch]
 *   block_table  int32 [batch][bt_stride]; columns below ceil(old/(P*c)) untouched
 * Runs one workgroup; batch <= 65536.
 */
int dcp_alloc_virtual(const dcp_layout* layout, const int32_t* free_stack, int32_t* free_top,
                      const int32_t* old_len, const int32_t* new_len, int32_t batch,
                      int32_t* block_table, int32_t bt_stride, int32_t* dev_status,
                      hipStream_t stream);

/*
 * dcp_kv_write - scatter new latent rows into their owner pools.
 *
 * SGLang "Decode Context Parallelism", section "Virtual KV layout": every
 * rank sees the same request-to-token map, keeps the positions it owns and
 * compacts them into its physical pool.  Position p of request b has virtual
 * slot v = block_table[b][p / (P*c)] * P*c + p mod (P*c); its owner is
 * v mod c and its physical slot there is v / c (interleave I: owner
 * floor(v / I) mod c, physical slot floor(v / (I*c)) * I + v mod I).
 *
 * Request b appends rows cu_new[b] .. cu_new[b+1]-1 (n_b rows) at positions
 * seq_len[b]-n_b .. seq_len[b]-1 (seq_len is the length after the append).
 * Row bytes are copied unchanged (plus the e4m3 scale).  A row that belongs
 * to no request (n < cu_new[0] or n >= cu_new[batch]) or whose position is
 * negative (DCP_DEV_BAD_LENGTH), whose table column is >= bt_stride
 * (DCP_DEV_TABLE_OVERFLOW) or whose page id is outside [0, num_pages)
 * (DCP_DEV_BAD_PAGE) is skipped and its slot_out is -1; other rows are
 * written.  Slots not addressed keep their bytes.
 *
 *   pools        c pools (see layout above), written
 *   pool_scales  float32 [c][num_pages*page] for e4m3, else NULL
 *   seq_len      int32 [batch]; cu_new int32 [batch+1], non-decreasing, normally
 *                with cu_new[0] = 0 and cu_new[batch] = n_rows
 *   rows         [n_rows][576] bf16 payloads, or [n_rows][576] e4m3 codes
 *   row_scales   float32 [n_rows] for e4m3, else NULL
 *   slot_out     optional int64 [n_rows]: owner * (num_pages*page) + physical slot
 */
int dcp_kv_write(const dcp_layout* layout, void* pools, float* pool_scales,
                 const int32_t* block_table, int32_t bt_stride, const int32_t* seq_len,
                 const int32_t* cu_new, int32_t batch, int64_t n_rows, const void* rows,
                 const float* row_scales, int64_t* slot_out, int32_t* dev_status,
                 hipStream_t stream);

/*
 * mla_decode_workspace_size - bytes of workspace mla_decode_partial needs for
 * these sizes (0 only for invalid arguments).  max_seq_len bounds every
 * seq_len[b].  The workspace holds the call's work plan (how each (rank,
 * request) is cut into KV splits, decided on the device from seq_len) and
 * the partial outputs of requests that are split.  When max_seq_len is short
 * enough that no (rank, request) can be split (at most 256 tokens per rank),
 * mla_decode_partial is one kernel launch and leaves the workspace untouched:
 * the size is then 256 bytes whatever the batch, and the buffer must still be
 * passed.
 */
size_t mla_decode_workspace_size(const dcp_layout* layout, int32_t rank_count, int32_t batch,
                                 int32_t q_len, int32_t heads, int64_t max_seq_len);

/*
 * mla_decode_partial - absorbed-MLA decode attention of each rank over its own
 * striped shard, returning the rank-local (o_r, lse_r).
 *
 * SGLang "Decode Context Parallelism", sections "MLA decode dataflow" and
 * "DCP x speculative decoding": each rank attends only its owned positions
 * through a rank-local page table built from owner(p) = p mod c and returns
 * a locally normalised output with its LSE; for target verification the
 * kernel is given the group size, the rank and the global KV length so that
 * causality is judged on global positions.
 *
 * Rank r's j-th owned token is global position p = j*c + r (interleave I:
 * p = floor(j / I)*I*c + r*I + j mod I) and sits at physical slot
 * block_table[b][j / P] * P + j mod P of pool r (the shared block table is
 * the rank-local page table).  For query row (b, i, h), with
 * i < q_len and global length L = seq_len[b], the visible positions are
 * p <= L - q_len + i when causal, all p < L otherwise.  Scores are
 * sm_scale * <q, K_p> over the 576 columns, (times the row's scale for e4m3);
 * o_r = softmax-weighted sum of K_p[0:512]; lse_r = log of the sum of
 * exp(scores) in the requested base.  A rank with no visible token returns
 * o_r = 0 and lse_r = -inf.
 *
 *   pools, pool_scales  pool of rank rank_begin followed by the next
 *                       rank_count-1 pools (a real rank passes its own pool
 *                       with rank_count = 1)
 *   q            bf16 [batch][q_len][heads][576]; heads % 16 == 0, q_len <= 8
 *   seq_len      int32 [batch], 0 <= seq_len[b] <= max_seq_len (host value)
 *   o_part       float32 [rank_count][batch][q_len][heads][512]
 *   lse_part     float32 [rank_count][batch][q_len][heads]
 *   workspace    device scratch of at least mla_decode_workspace_size(...)
 *                bytes, 16-byte aligned; contents are scratch, and calls that
 *                share one workspace must not overlap in time
 *
 * The call enqueues kernels only (no allocation, copy or memset), and the
 * split of the work is decided on the device from seq_len at every call: a
 * call captured in a HIP graph stays right when seq_len changes between
 * replays, as long as every length stays within the captured max_seq_len.
 *
 * Device status: DCP_DEV_BAD_LENGTH, DCP_DEV_TABLE_OVERFLOW and
 * DCP_DEV_BAD_PAGE as above; DCP_DEV_DECODE_STALLED if a wave of the e4m3
 * decode gave up its bounded wait for the wave it exchanges row maxima with.
 */
int mla_decode_partial(const dcp_layout* layout, const void* pools, const float* pool_scales,
                       int32_t rank_begin, int32_t rank_count, const void* q, int32_t batch,
                       int32_t q_len, int32_t heads, const int32_t* block_table,
                       int32_t bt_stride, const int32_t* seq_len, int64_t max_seq_len,
                       float sm_scale, int32_t lse_base, int32_t causal, float* o_part,
                       float* lse_part, void* workspace, size_t workspace_bytes,
                       int32_t* dev_status, hipStream_t stream);

/*
 * mla_decode_partial_noalloc - mla_decode_partial without a caller workspace.
 *
 * For callers that cannot allocate device memory at the call (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * work plan and the split partials go to a scratch array that the library
 * holds in device memory (one copy per GPU, kept until the process ends, of
 * mla_decode_noalloc_scratch_bytes() = 256 MiB); the call allocates and frees
 * nothing.  Arguments, outputs and errors are those of mla_decode_partial,
 * and the outputs are the same bit for bit; a call whose workspace size
 * (mla_decode_workspace_size) exceeds the scratch returns DCP_ERR_WORKSPACE
 * and enqueues nothing.  The scratch needs no clearing between calls (every
 * call writes what it reads), but every call on one GPU shares it: calls that
 * overlap in time on one GPU (several streams, or host threads) race and must
 * be serialised by the caller.  DCP_ERR_HIP if the scratch address cannot be
 * looked up on the current device.
 */
int mla_decode_partial_noalloc(const dcp_layout* layout, const void* pools, const float* pool_scales,
                               int32_t rank_begin, int32_t rank_count, const void* q, int32_t batch,
                               int32_t q_len, int32_t heads, const int32_t* block_table,
                               int32_t bt_stride, const int32_t* seq_len, int64_t max_seq_len,
                               float sm_scale, int32_t lse_base, int32_t causal, float* o_part,
                               float* lse_part, int32_t* dev_status, hipStream_t stream);

/* Bytes of the scratch array mla_decode_partial_noalloc uses (host call). */
size_t mla_decode_noalloc_scratch_bytes(void);

/*
 * dcp_lse_merge - exact merge of c partials (SGLang "Decode Context
 * Parallelism", section "MLA decode dataflow"): lse = logsumexp_r lse_r and
 * o = sum_r exp(lse_r - lse) * o_r, in base e or base 2 (the base of the
 * partials).  Partials with lse_r = -inf get weight 0; if every partial of a
 * row is -inf the row gets o = 0 and lse = -inf.
 *
 *   o_part   float32 [c][rows][512];  lse_part float32 [c][rows]
 *   o_out    bf16 [rows][512], rounded to nearest even
 *   lse_out  float32 [rows]
 */
int dcp_lse_merge(int32_t c, int64_t rows, const float* o_part, const float* lse_part,
                  int32_t lse_base, void* o_out, float* lse_out, hipStream_t stream);

/*
 * dcp_kv_read - gather every request's cached rows back into token order.
 *
 * SGLang "Decode Context Parallelism", decode cost model: an extend step,
 * which lies outside that model, may gather the cached prefix shards,
 * restore token order and then append the new tokens (dcp_kv_write).
 *
 * Position p (0 <= p < seq_len[b]) of request b is read from its owner pool
 * (slot as in dcp_kv_write, interleave included) and written to row
 * cu_out[b] + p of rows_out; bytes are copied unchanged (plus the e4m3
 * scale to scales_out).  A request with seq_len[b] < 0, with cu_out[b+1] -
 * cu_out[b] != seq_len[b] or with a span outside [0, n_rows) is skipped
 * (DCP_DEV_BAD_LENGTH), one that needs more than bt_stride virtual pages
 * too (DCP_DEV_TABLE_OVERFLOW), and so are the positions of a virtual page
 * whose id is outside [0, num_pages) (DCP_DEV_BAD_PAGE).  Rows not written
 * keep their bytes.
 *
 *   pools        c pools (see layout above), read only
 *   pool_scales  float32 [c][num_pages*page] for e4m3, else NULL
 *   seq_len      int32 [batch]; cu_out int32 [batch+1]
 *   rows_out     [n_rows][576] bf16 or e4m3 (16-byte aligned)
 *   scales_out   float32 [n_rows] for e4m3, else NULL
 * batch <= 65536; page * c <= 2^30 (else DCP_ERR_UNSUPPORTED).
 */
int dcp_kv_read(const dcp_layout* layout, const void* pools, const float* pool_scales,
                const int32_t* block_table, int32_t bt_stride, const int32_t* seq_len,
                const int32_t* cu_out, int32_t batch, int64_t n_rows, void* rows_out,
                float* scales_out, int32_t* dev_status, hipStream_t stream);

/*
 * dcp_kv_relayout - copy dense (DCP size 1) paged KV into striped owner pools.
 *
 * SGLang "Decode Context Parallelism", section "DCP x PD disaggregation":
 * dense prefill pages cannot be copied into striped decode storage as they
 * are; going from a DCP1 prefill to a DCP decode relays the tokens out,
 * selecting for each decode rank the rows it owns, and the exact token count
 * keeps stale rows of a partly filled last page out.
 *
 * The source is one pool of src_num_pages pages of `page` tokens in the
 * layout's KV dtype; position p of request b sits at slot
 * src_block_table[b][p / page] * page + p mod page.  For every p <
 * seq_len[b] whose owner (as in dcp_kv_write) is in [rank_begin, rank_begin
 * + rank_count), the row (and e4m3 scale) is copied to its slot in that
 * owner's pool through the shared virtual table block_table, which must
 * already hold the request's virtual pages (dcp_alloc_virtual).  Nothing
 * else is written: not the other ranks' rows, not the slots of a last page
 * past the request's length.  A request with seq_len[b] < 0 is skipped
 * (DCP_DEV_BAD_LENGTH), one whose pages do not fit either table too
 * (DCP_DEV_TABLE_OVERFLOW); a position whose page id in either table is
 * outside its pool is skipped (DCP_DEV_BAD_PAGE).  pools (and pool_scales)
 * hold the pools of ranks rank_begin .. rank_begin + rank_count - 1 back to
 * back, as in mla_decode_partial: a real decode rank r passes rank_begin = r,
 * rank_count = 1 and its own pool; the emulated group on one GPU passes 0,
 * c and all c pools.
 *
 *   src_pool       [src_num_pages*page][576] bf16 or e4m3, read only
 *   src_scales     float32 [src_num_pages*page] for e4m3, else NULL
 *   src_block_table int32 [batch][src_bt_stride]
 *   pools, pool_scales, block_table, bt_stride: as in dcp_kv_write
 * batch <= 65536; page * c <= 2^30 (else DCP_ERR_UNSUPPORTED).
 */
int dcp_kv_relayout(const dcp_layout* layout, const void* src_pool, const float* src_scales,
                    int32_t src_num_pages, const int32_t* src_block_table, int32_t src_bt_stride,
                    const int32_t* seq_len, int32_t batch, int32_t rank_begin, int32_t rank_count,
                    void* pools, float* pool_scales, const int32_t* block_table, int32_t bt_stride,
                    int32_t* dev_status, hipStream_t stream);

/* Static description of a status value (host or device code). */
const char* dcp_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DCP_MLA_H */
