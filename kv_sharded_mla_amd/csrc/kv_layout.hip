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
  __shared__ int64_t wsum[kAllocThreads / 64];
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
  // inclusive scan of the page needs: within each wave by shuffles, then
  // over the 16 wave totals
  const int lane = t & 63, wv = t >> 6;
  int64_t incl = need;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int64_t total = 0;
#pragma unroll
  for (int i = 0; i < kAllocThreads / 64; ++i) {
    const int64_t x = wsum[i];
    if (i < wv) incl += x;
    total += x;
  }
  const int64_t top = *free_top;
  int code = DCP_DEV_OK;
  if (flags[0]) code = DCP_DEV_BAD_LENGTH;
  else if (flags[1]) code = DCP_DEV_TABLE_OVERFLOW;
  else if (total > top) code = DCP_DEV_OUT_OF_PAGES;
  if (code != DCP_DEV_OK) {
    if (t == 0 && dev_status) atomicMax(dev_status, code);
    return;
  }
  int64_t k = incl - need;  // pops taken before this thread's first request
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
    // rows outside [cu_new[0], cu_new[batch]) belong to no request
    if (p < 0 || nb < 0 || n >= (int64_t)cu_new[batch] || n < (int64_t)cu_new[0]) {
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

// ---- extend gather and DCP1 -> DCP c relayout -------------------------------
// Both walk one virtual page of one request per step: rank r's P slots of
// virtual page g (page id pg) sit contiguously in pool r at [pg*P, pg*P + P),
// and local slot s there holds position g*P*c + (s / I)*I*c + r*I + s mod I
// (the gather walks the page in token order, the relayout rank by rank: the
// stores of either are then contiguous, which measured faster than contiguous
// loads).
// Each wave copies whole rows (rows are wave-uniform, so the index arithmetic
// is scalar), a round of four copy units at a time with all loads issued
// before the stores.
// Workgroup (b, k) of a batch x G grid takes virtual pages k, k + G, ... of
// request b.

constexpr int kCopyThreads = 256;
constexpr int kRowsPerWave = 4;

// position of local slot s of rank r in virtual page g
__device__ __forceinline__ int64_t slot_position(int64_t g, int32_t s, int32_t r, int32_t c, int32_t il, int32_t page) {
  return g * page * c + (int64_t)(s / il) * il * c + (int64_t)r * il + s % il;
}

// A copy unit is 1152 bytes: one bf16 row, or two e4m3 rows (the second
// starting at chunk 36).  Lane l moves chunk l of each unit and lanes 0..7
// also chunk 64 + l, so a unit takes two vector loads and two stores.
template <bool FP8>
struct CopyUnits {
  static constexpr int kRows = FP8 ? 2 * kRowsPerWave : kRowsPerWave;   // rows per wave round
};

// Stores carry the non-temporal hint (the copied rows are not read back by
// this kernel): 1-2% faster on every measured workload than plain stores;
// the same hint on the loads gained nothing.
typedef int v4i __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void stv(int4* p, int4 v) {
  __builtin_nontemporal_store(v4i{v.x, v.y, v.z, v.w}, reinterpret_cast<v4i*>(p));
}

template <bool FP8>
__device__ __forceinline__ void copy_rows(const uint8_t* (&src)[CopyUnits<FP8>::kRows],
                                          uint8_t* (&dst)[CopyUnits<FP8>::kRows],
                                          const bool (&live)[CopyUnits<FP8>::kRows], int lane) {
  static_assert(kRowsPerWave == 4, "four named units below");
  // chunk k of unit i: row (FP8 && k >= 36 ? 2i + 1 : i * (FP8 ? 2 : 1)), chunk k mod 36 (e4m3) or k
  auto pick = [&](int i, int k, int& row, int& ch) {
    if (FP8) {
      row = 2 * i + (k >= 36 ? 1 : 0);
      ch = k >= 36 ? k - 36 : k;
    } else {
      row = i;
      ch = k;
    }
  };
  const int k1 = 64 + (lane < 8 ? lane : 0);
  auto ld = [&](int i, int4& x, int4& y) {
    int row, ch;
    pick(i, lane, row, ch);
    if (live[row]) x = reinterpret_cast<const int4*>(src[row])[ch];
    pick(i, k1, row, ch);
    if (lane < 8 && live[row]) y = reinterpret_cast<const int4*>(src[row])[ch];
  };
  auto st = [&](int i, const int4& x, const int4& y) {
    int row, ch;
    pick(i, lane, row, ch);
    if (live[row]) stv(reinterpret_cast<int4*>(dst[row]) + ch, x);
    pick(i, k1, row, ch);
    if (lane < 8 && live[row]) stv(reinterpret_cast<int4*>(dst[row]) + ch, y);
  };
  int4 a0 = {}, a1 = {}, a2 = {}, a3 = {}, t0 = {}, t1 = {}, t2 = {}, t3 = {};
  ld(0, a0, t0);
  ld(1, a1, t1);
  ld(2, a2, t2);
  ld(3, a3, t3);
  st(0, a0, t0);
  st(1, a1, t1);
  st(2, a2, t2);
  st(3, a3, t3);
}

// e4m3 scales of a round's rows: lane i moves row i's scale, one load and one
// store for the whole round
template <int NR>
__device__ __forceinline__ void copy_scales(const float* __restrict__ from, float* __restrict__ to,
                                            const int64_t (&sf)[NR], const int64_t (&stt)[NR], const bool (&live)[NR],
                                            int lane) {
  int64_t f = 0, t = 0;
  bool lv = false;
#pragma unroll
  for (int i = 0; i < NR; ++i)
    if (lane == i) {
      f = sf[i];
      t = stt[i];
      lv = live[i];
    }
  if (lv) to[t] = from[f];
}

template <bool FP8>
__global__ void __launch_bounds__(kCopyThreads)
kv_read_kernel(int32_t c, int32_t il, int32_t page, int32_t num_pages, int32_t G, const uint8_t* __restrict__ pools,
               const float* __restrict__ pool_scales, const int32_t* __restrict__ block_table, int32_t bt_stride,
               const int32_t* __restrict__ seq_len, const int32_t* __restrict__ cu_out, int64_t n_rows,
               uint8_t* __restrict__ rows_out, float* __restrict__ scales_out, int32_t* __restrict__ dev_status) {
  constexpr int64_t kRowBytes = FP8 ? kDqk : 2 * kDqk;
  constexpr int NR = CopyUnits<FP8>::kRows;
  const int b = blockIdx.x / G, k = blockIdx.x % G;
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t vpage = (int64_t)page * c;
  const int64_t cap = (int64_t)num_pages * page;
  const int32_t L = seq_len[b];
  if (L < 0 || cu_out[b] < 0 || cu_out[b + 1] > n_rows || (int64_t)cu_out[b + 1] - cu_out[b] != L) {
    if (k == 0 && threadIdx.x == 0 && dev_status) atomicMax(dev_status, DCP_DEV_BAD_LENGTH);
    return;
  }
  const int64_t n_vp = (L + vpage - 1) / vpage;
  if (n_vp > bt_stride) {
    if (k == 0 && threadIdx.x == 0 && dev_status) atomicMax(dev_status, DCP_DEV_TABLE_OVERFLOW);
    return;
  }
  uint8_t* out_b = rows_out + (int64_t)cu_out[b] * kRowBytes;
  const int32_t per_vp = page * c;   // rows of one virtual page, taken rank by rank
  for (int64_t g = k; g < n_vp; g += G) {
    const int32_t pg = block_table[(int64_t)b * bt_stride + g];
    if (pg < 0 || pg >= num_pages) {
      if (threadIdx.x == 0 && dev_status) atomicMax(dev_status, DCP_DEV_BAD_PAGE);
      continue;
    }
    for (int32_t i0 = wv * NR; i0 < per_vp; i0 += (kCopyThreads / 64) * NR) {
      const uint8_t* src[NR];
      uint8_t* dst[NR];
      bool live[NR];
      int64_t sc_from[NR], sc_to[NR];
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        // rows in token order, so that a round's stores are contiguous
        const int32_t o = i0 + i;
        const int64_t pos = g * per_vp + o;
        const int32_t r = (o / il) % c, s = (o / (il * c)) * il + o % il;
        live[i] = o < per_vp && pos < L;
        const int64_t slot = (int64_t)pg * page + s;
        src[i] = pools + ((int64_t)r * cap + slot) * kRowBytes;
        dst[i] = out_b + pos * kRowBytes;
        sc_from[i] = (int64_t)r * cap + slot;
        sc_to[i] = cu_out[b] + pos;
      }
      if (FP8) copy_scales<NR>(pool_scales, scales_out, sc_from, sc_to, live, lane);
      copy_rows<FP8>(src, dst, live, lane);
    }
  }
}

template <bool FP8>
__global__ void __launch_bounds__(kCopyThreads)
kv_relayout_kernel(int32_t c, int32_t il, int32_t page, int32_t num_pages, int32_t G, int32_t rank_begin,
                   int32_t rank_count, const uint8_t* __restrict__ src_pool, const float* __restrict__ src_scales,
                   int32_t src_num_pages, const int32_t* __restrict__ src_table, int32_t src_stride,
                   const int32_t* __restrict__ seq_len, uint8_t* __restrict__ pools, float* __restrict__ pool_scales,
                   const int32_t* __restrict__ block_table, int32_t bt_stride, int32_t* __restrict__ dev_status) {
  constexpr int64_t kRowBytes = FP8 ? kDqk : 2 * kDqk;
  constexpr int NR = CopyUnits<FP8>::kRows;
  const int b = blockIdx.x / G, k = blockIdx.x % G;
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t vpage = (int64_t)page * c;
  const int64_t cap = (int64_t)num_pages * page;
  const int32_t L = seq_len[b];
  if (L < 0) {
    if (k == 0 && threadIdx.x == 0 && dev_status) atomicMax(dev_status, DCP_DEV_BAD_LENGTH);
    return;
  }
  const int64_t n_vp = (L + vpage - 1) / vpage;
  if (n_vp > bt_stride || ((int64_t)L + page - 1) / page > src_stride) {
    if (k == 0 && threadIdx.x == 0 && dev_status) atomicMax(dev_status, DCP_DEV_TABLE_OVERFLOW);
    return;
  }
  const int32_t* st = src_table + (int64_t)b * src_stride;
  const int32_t per_vp = page * rank_count;   // rows of the covered ranks in one virtual page
  for (int64_t g = k; g < n_vp; g += G) {
    const int32_t pg = block_table[(int64_t)b * bt_stride + g];
    for (int32_t i0 = wv * NR; i0 < per_vp; i0 += (kCopyThreads / 64) * NR) {
      const uint8_t* src[NR];
      uint8_t* dst[NR];
      bool live[NR];
      int64_t sc_from[NR], sc_to[NR];
      int code = DCP_DEV_OK;
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const int32_t rl = i0 + i;
        const int32_t rr = rl / page, s = rl - rr * page;
        const int32_t r = rank_begin + rr;
        const int64_t pos = slot_position(g, s, r, c, il, page);
        live[i] = rl < per_vp && pos < L;
        const int32_t sp = live[i] ? st[pos / page] : 0;
        if (live[i] && (sp < 0 || sp >= src_num_pages || pg < 0 || pg >= num_pages)) {
          code = DCP_DEV_BAD_PAGE;
          live[i] = false;
        }
        const int64_t slot = (int64_t)pg * page + s;
        const int64_t sslot = (int64_t)sp * page + pos % page;
        src[i] = src_pool + sslot * kRowBytes;
        dst[i] = pools + ((int64_t)rr * cap + slot) * kRowBytes;
        sc_from[i] = sslot;
        sc_to[i] = (int64_t)rr * cap + slot;
      }
      if (code != DCP_DEV_OK && lane == 0 && dev_status) atomicMax(dev_status, code);
      if (FP8) copy_scales<NR>(src_scales, pool_scales, sc_from, sc_to, live, lane);
      copy_rows<FP8>(src, dst, live, lane);
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

namespace dcp {

namespace {
// workgroups per request: enough in all for a few per CU, at most one per virtual page
int32_t copy_split(int32_t batch, int32_t bt_stride) {
  const int32_t want = (4096 + batch - 1) / batch;
  return want < 1 ? 1 : (want > bt_stride ? bt_stride : want);
}
}  // namespace

hipError_t launch_kv_read(int32_t c, int32_t interleave, int32_t page, int32_t num_pages, bool fp8, const void* pools,
                          const float* pool_scales, const int32_t* block_table, int32_t bt_stride,
                          const int32_t* seq_len, const int32_t* cu_out, int32_t batch, int64_t n_rows,
                          void* rows_out, float* scales_out, int32_t* dev_status, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  const int32_t G = copy_split(batch, bt_stride);
  const dim3 grid((unsigned)((int64_t)batch * G)), block(kCopyThreads);
  if (fp8)
    hipLaunchKernelGGL(kv_read_kernel<true>, grid, block, 0, stream, c, interleave, page, num_pages, G,
                       (const uint8_t*)pools, pool_scales, block_table, bt_stride, seq_len, cu_out, n_rows,
                       (uint8_t*)rows_out, scales_out, dev_status);
  else
    hipLaunchKernelGGL(kv_read_kernel<false>, grid, block, 0, stream, c, interleave, page, num_pages, G,
                       (const uint8_t*)pools, pool_scales, block_table, bt_stride, seq_len, cu_out, n_rows,
                       (uint8_t*)rows_out, scales_out, dev_status);
  return hipGetLastError();
}

hipError_t launch_kv_relayout(int32_t c, int32_t interleave, int32_t page, int32_t num_pages, bool fp8,
                              const void* src_pool, const float* src_scales, int32_t src_num_pages,
                              const int32_t* src_table, int32_t src_stride, const int32_t* seq_len, int32_t batch,
                              int32_t rank_begin, int32_t rank_count, void* pools, float* pool_scales,
                              const int32_t* block_table, int32_t bt_stride, int32_t* dev_status,
                              hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  const int32_t G = copy_split(batch, bt_stride);
  const dim3 grid((unsigned)((int64_t)batch * G)), block(kCopyThreads);
  if (fp8)
    hipLaunchKernelGGL(kv_relayout_kernel<true>, grid, block, 0, stream, c, interleave, page, num_pages, G,
                       rank_begin, rank_count, (const uint8_t*)src_pool, src_scales, src_num_pages, src_table,
                       src_stride, seq_len, (uint8_t*)pools, pool_scales, block_table, bt_stride, dev_status);
  else
    hipLaunchKernelGGL(kv_relayout_kernel<false>, grid, block, 0, stream, c, interleave, page, num_pages, G,
                       rank_begin, rank_count, (const uint8_t*)src_pool, src_scales, src_num_pages, src_table,
                       src_stride, seq_len, (uint8_t*)pools, pool_scales, block_table, bt_stride, dev_status);
  return hipGetLastError();
}

}  // namespace dcp
