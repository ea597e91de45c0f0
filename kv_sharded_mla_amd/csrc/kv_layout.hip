// Shared virtual allocator and owner-pool scatter for the DCP latent cache.
//
// Layout (SGLang "Decode Context Parallelism", section "Virtual KV layout"):
// virtual capacity C*c, virtual page P*c, owner(v) = v mod c,
// physical(v) = floor(v / c).  A virtual page id is a page index valid in every
// owner pool, so virtual page g covers physical slots [g*P, (g+1)*P) on each
// rank.  With a KV interleave size I (vLLM study page "vLLM Decode Context
// Parallelism", operation guide) runs of I slots go to the owners in turn:
// owner(v) = floor(v / I) mod c, physical(v) = floor(v / (I c)) I + v mod I,
// and since I divides P the page mapping above is unchanged.  Both kernels are
// integer/byte work and bit-exact by construction.
#include "dcp_common.hpp"
#include "dcp_internal.hpp"

#include "../../include/dcp_mla.h"

namespace dcp {

namespace {

constexpr int kAllocThreads = 1024;

__device__ __forceinline__ int64_t pages_for(int64_t len, int64_t vpage) { return (len + vpage - 1) / vpage; }

// One workgroup.  Thread t owns a contiguous run of requests; a block scan of
// the per-thread page needs gives each request its offset into the pop order.
__global__ void __launch_bounds__(kAllocThreads)
alloc_virtual_kernel(int32_t c, int32_t page, const int32_t* __restrict__ free_stack,
                     int32_t* __restrict__ free_top, const int32_t* __restrict__ old_len,
                     const int32_t* __restrict__ new_len, int32_t batch,
                     int32_t* __restrict__ block_table, int32_t bt_stride,
                     int32_t* __restrict__ dev_status) {
  __shared__ int64_t scan[kAllocThreads];
  __shared__ int flags[2];
  const int t = threadIdx.x;
  const int64_t vpage = (int64_t)page * c;
  const int per = (batch + kAllocThreads - 1) / kAllocThreads;
  const int b0 = t * per;
  const int b1 = min(batch, b0 + per);
  if (t < 2) flags[t] = 0;
  __syncthreads();
  int64_t need = 0;
  bool bad_len = false, overflow = false;
  for (int b = b0; b < b1; ++b) {
    int32_t o = old_len[b], n = new_len[b];
    if (o < 0 || n < o) {
      bad_len = true;
      continue;
    }
    int64_t pn = pages_for(n, vpage);
    if (pn > bt_stride) overflow = true;
    need += pn - pages_for(o, vpage);
  }
  if (bad_len) atomicOr(&flags[0], 1);
  if (overflow) atomicOr(&flags[1], 1);
  scan[t] = need;
  __syncthreads();
  // Hillis-Steele inclusive scan over 1024 entries.
  for (int off = 1; off < kAllocThreads; off <<= 1) {
    int64_t v = (t >= off) ? scan[t - off] : 0;
    __syncthreads();
    scan[t] += v;
    __syncthreads();
  }
  const int64_t total = scan[kAllocThreads - 1];
  const int64_t top = *free_top;
  int code = DCP_DEV_OK;
  if (flags[0]) code = DCP_DEV_BAD_LENGTH;
  else if (flags[1]) code = DCP_DEV_TABLE_OVERFLOW;
  else if (total > top) code = DCP_DEV_OUT_OF_PAGES;
  if (code != DCP_DEV_OK) {
    if (t == 0 && dev_status) atomicMax(dev_status, code);
    return;
  }
  int64_t k = scan[t] - need;  // pops taken before this thread's first request
  for (int b = b0; b < b1; ++b) {
    int64_t first = pages_for(old_len[b], vpage);
    int64_t nb = pages_for(new_len[b], vpage) - first;
    int32_t* row = block_table + (int64_t)b * bt_stride;
    for (int64_t i = 0; i < nb; ++i, ++k) row[first + i] = free_stack[top - 1 - k];
  }
  __syncthreads();
  if (t == 0) *free_top = (int32_t)(top - total);
}

// One wave per row: the row's request comes from a binary search of cu_new,
// its position from seq_len, its slot from the shared block table.
template <bool FP8>
__global__ void __launch_bounds__(256)
kv_write_kernel(int32_t c, int32_t il, int32_t page, int32_t num_pages, uint8_t* __restrict__ pools,
                float* __restrict__ pool_scales, const int32_t* __restrict__ block_table,
                int32_t bt_stride, const int32_t* __restrict__ seq_len,
                const int32_t* __restrict__ cu_new, int32_t batch, int64_t n_rows,
                const uint8_t* __restrict__ rows, const float* __restrict__ row_scales,
                int64_t* __restrict__ slot_out, int32_t* __restrict__ dev_status) {
  constexpr int kRowBytes = FP8 ? kDqk : 2 * kDqk;
  constexpr int kChunks = kRowBytes / 16;
  const int lane = threadIdx.x & 63;
  const int64_t vpage = (int64_t)page * c;
  const int64_t cap = (int64_t)num_pages * page;
  const int64_t pool_bytes = cap * kRowBytes;
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x / 64);
  for (int64_t n = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6); n < n_rows; n += nwaves) {
    // request b with cu_new[b] <= n < cu_new[b+1]
    int lo = 0, hi = batch;  // invariant: cu_new[lo] <= n, answer in [lo, hi)
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if ((int64_t)cu_new[mid] <= n) lo = mid; else hi = mid;
    }
    const int b = lo;
    const int64_t nb = (int64_t)cu_new[b + 1] - cu_new[b];
    const int64_t p = (int64_t)seq_len[b] - nb + (n - cu_new[b]);
    int code = DCP_DEV_OK;
    int64_t owner = 0, phys = 0;
    if (p < 0 || nb < 0 || n >= (int64_t)cu_new[batch]) {
      code = DCP_DEV_BAD_LENGTH;
    } else if (p / vpage >= bt_stride) {
      code = DCP_DEV_TABLE_OVERFLOW;
    } else {
      int32_t pg = block_table[(int64_t)b * bt_stride + p / vpage];
      if (pg < 0 || pg >= num_pages) {
        code = DCP_DEV_BAD_PAGE;
      } else {
        // chunks of il positions go to the ranks in turn (il divides the page)
        int64_t v = (int64_t)pg * vpage + p % vpage;
        owner = (v / il) % c;
        phys = (v / ((int64_t)il * c)) * il + v % il;
      }
    }
    if (code != DCP_DEV_OK) {
      if (lane == 0) {
        if (dev_status) atomicMax(dev_status, code);
        if (slot_out) slot_out[n] = -1;
      }
      continue;
    }
    const int4* src = reinterpret_cast<const int4*>(rows + n * kRowBytes);
    int4* dst = reinterpret_cast<int4*>(pools + owner * pool_bytes + phys * kRowBytes);
    for (int ch = lane; ch < kChunks; ch += 64) dst[ch] = src[ch];
    if (lane == 0) {
      if (FP8) pool_scales[owner * cap + phys] = row_scales[n];
      if (slot_out) slot_out[n] = owner * cap + phys;
    }
  }
}

}  // namespace

hipError_t launch_alloc_virtual(int32_t c, int32_t page, const int32_t* free_stack, int32_t* free_top,
                                const int32_t* old_len, const int32_t* new_len, int32_t batch,
                                int32_t* block_table, int32_t bt_stride, int32_t* dev_status,
                                hipStream_t stream) {
  hipLaunchKernelGGL(alloc_virtual_kernel, dim3(1), dim3(kAllocThreads), 0, stream, c, page, free_stack,
                     free_top, old_len, new_len, batch, block_table, bt_stride, dev_status);
  return hipGetLastError();
}

hipError_t launch_kv_write(int32_t c, int32_t interleave, int32_t page, int32_t num_pages, bool fp8, void* pools,
                           float* pool_scales, const int32_t* block_table, int32_t bt_stride,
                           const int32_t* seq_len, const int32_t* cu_new, int32_t batch,
                           int64_t n_rows, const void* rows, const float* row_scales,
                           int64_t* slot_out, int32_t* dev_status, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  int64_t blocks = (n_rows + 3) / 4;
  if (blocks > 16384) blocks = 16384;
  if (fp8)
    hipLaunchKernelGGL(kv_write_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, c, interleave, page, num_pages,
                       (uint8_t*)pools, pool_scales, block_table, bt_stride, seq_len, cu_new, batch, n_rows,
                       (const uint8_t*)rows, row_scales, slot_out, dev_status);
  else
    hipLaunchKernelGGL(kv_write_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, c, interleave, page, num_pages,
                       (uint8_t*)pools, pool_scales, block_table, bt_stride, seq_len, cu_new, batch, n_rows,
                       (const uint8_t*)rows, row_scales, slot_out, dev_status);
  return hipGetLastError();
}

}  // namespace dcp
