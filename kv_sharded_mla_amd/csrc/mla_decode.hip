// Paged split-KV absorbed-MLA decode over a DCP rank's striped shard (gfx950).
//
// Method (SGLang "Decode Context Parallelism", sections "MLA decode dataflow"
// and "DCP x speculative decoding"): rank r attends only the positions it
// owns, p = j*c + r, through a rank-local page table built from the cyclic
// owner map, judges causality on global positions, and returns a locally
// normalised output with its log-sum-exp.  Rank r's j-th token sits at slot
// block_table[b][j / P] * P + j mod P of its pool, because floor((jc+r)/(Pc))
// = floor(j/P) and floor(((jc+r) mod Pc)/c) = j mod P for r < c: the shared
// block table is the rank-local page table.
//
// Kernel shape.  A workgroup of 8 waves (16 for 64-row bf16 blocks) owns one
// (rank, request, KV split, block of 16*RGN query rows).  KV is streamed
// through an LDS ring of 36 KB stages (32 bf16 or 64 e4m3 tokens) filled by
// direct-to-LDS 16-byte loads (global_load_lds_dwordx4); every latent row is
// read from HBM once per workgroup and serves all of its query rows.  Per 32
// tokens:
//   S^T[32 tok x 16 rows] = K[32 x 576] . Q^T           (mfma 16x16x32 bf16, K from LDS,
//                                                       Q^T held in registers)
//   O^T[512 x 16 rows]   += V^T[512 x 32] . P^T         (V^T read from the same LDS rows
//                                                       with ds_read_b64_tr_b16 / tr_b8)
// The MFMA output layout of S^T (lane = 16g + j holds tokens 4g+i of row j)
// is used directly as the P^T operand of the PV product by pairing k-slot
// 8g+i with token 4g+i and k-slot 8g+4+i with token 16+4g+i; the transposed V
// reads supply the same token order.  Every value a lane accumulates belongs
// to its row j, so the softmax rescale is a per-lane scalar.
// Online softmax runs in fp32 in base 2 (scores pre-multiplied by
// sm_scale*log2 e); the running maximum is only raised when a tile exceeds it
// by more than kTau, so O is rescaled rarely (any common reference value gives
// the same result; probabilities stay below 2^kTau).
// e4m3 KV: codes are converted exactly to bf16 for the MFMA, the per-token
// scale multiplies the score and the probability that weights V.
#include <mutex>

#include "dcp_common.hpp"
#include "dcp_internal.hpp"

#include "../../include/dcp_mla.h"

namespace dcp {

namespace {

constexpr float kTau = 8.0f;
constexpr int kMaxTab = 512;  // page ids staged per workgroup
constexpr int kStageTok = 32; // tokens per LDS stage, bf16 KV (e4m3 KV: 64, the same bytes)
constexpr int kCombineBlocksPerCu = 8;  // split-combine workgroups per CU (grid-stride beyond)
constexpr int kItemMinStages = 8;       // shortest work item (each pays a q load and a partial write)
constexpr int kItemsPerCu = 2;          // work items the plan aims for per CU and row block

struct DecodeParams {
  const uint8_t* pools;
  const float* pool_scales;
  int64_t pool_bytes;
  int64_t cap;  // tokens per pool
  int32_t c, interleave, page, num_pages, rank_begin;
  const uint16_t* q;
  int32_t batch, q_len, heads, rows;
  const int32_t* block_table;
  int32_t bt_stride;
  const int32_t* seq_len;
  int64_t max_seq_len;
  float scale_log2;  // sm_scale * log2(e)
  int32_t out_base2;  // lse_part in base 2 (else base e)
  int32_t causal;
  float* o_part;    // [units][rows][512], unit = rank * batch + request
  float* lse_part;  // [units][rows]
  int32_t n_row_blocks;
  int32_t stage_tok;  // tokens per LDS stage (and the plan's unit of work)
  int32_t units;    // rank_count * batch
  int32_t direct;   // every unit is one item: no work plan, item i = unit i
  // work plan (written each call by decode_plan_kernel, in the workspace)
  int32_t max_items;
  int32_t items_target;  // work items per row block the plan aims for
  int32_t t_min, t_max;  // bounds of an item's length in stages
  // [ceil8(max_items)][8] one record per dispatch position: item (its
  // partial slot; -1 past the last item), unit, first and end rank-local
  // token, the request's KV length, 1 when the unit is a single item, 0, 0
  int32_t* drec;
  int32_t* n_items;      // [3]: work items, split units, most items of one unit
  int32_t* unit_first;   // [units] first item of the unit
  int32_t* unit_count;   // [units] items of the unit
  int32_t* split_units;  // [units] the units with several items
  float* ws_o;           // [max_items][rows][512] partials of units with several items
  float* ws_lse;         // [max_items][rows] (base 2)
  int32_t* dev_status;
};

// LDS layout of a stage: row r (token) of ROWB bytes holds its 16-byte chunk c
// at position c ^ swz(r).  The XOR stays inside aligned groups of 8 (bf16,
// 72 chunks per row) or 4 (e4m3, 36 chunks) so it permutes each row.  Without
// it the 1152- and 576-byte row strides put the 16 rows that one LDS read
// instruction touches on the same banks.
template <bool FP8>
__device__ __forceinline__ int swz(int r) {
  // e4m3 rows (576 B): chunk position bit 1 from row bit 2, bit 0 from row
  // bit 4.  Measured with the bank-conflict counter over every 2-bit linear
  // row swizzle: this one (one of 128 that measure zero) leaves both the
  // 16-byte K reads (rows 16t..16t+15, chunk 4u+g) and the 8-byte transposed V
  // reads (rows 4G+s and 16+4G+s) conflict-free; the row bits 2 and 3^4 used
  // before cost 4 conflict cycles per K read.
  if (FP8) return ((r >> 4) & 1) | (((r >> 2) & 1) << 1);
  return ((r >> 1) ^ r) & 7;  // no conflicts with 64 banks of 4 bytes
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// Direct-to-LDS loads: every active lane k of the wave copies 16 (or 4) bytes
// from its global address to LDS byte lds + 16k (or 4k); lds must be
// wave-uniform.  Written as inline asm so that the compiler's wait-count
// insertion does not treat the ring's later LDS reads as aliasing these
// writes.  m0 carries the LDS address; nothing else in these kernels uses m0
// (a host-side build check verifies this in the generated code).
// Cache policy of the direct-to-LDS loads (NT): the non-temporal hint lifts
// KV streaming from HBM from 6.14 to 7.26 TB/s, and is used when a work item
// has one row block.  Items with several row blocks re-read their KV from L2
// (one read per row block), which the hint defeats (15% slower).
template <bool NT>
__device__ __forceinline__ void dma16(const uint8_t* gbase, uint32_t voff, const void* lds) {
  // gbase is wave-uniform; readfirstlane pins it (and the LDS address) to SGPRs
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  // (readfirstlane returns a signed int: widen through uint32_t, never sign-extend)
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)gbase);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uintptr_t)gbase >> 32));
  const uint64_t gb = lo | (hi << 32);
  if (NT)
    __asm__ volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(m0), "v"(voff), "s"(gb) : "memory");
  else
    __asm__ volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0), "v"(voff), "s"(gb) : "memory");
}
template <bool NT>
__device__ __forceinline__ void dma16_abs(const uint8_t* gaddr, const void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  if (NT)
    __asm__ volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(m0), "v"(gaddr) : "memory");
  else
    __asm__ volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(gaddr) : "memory");
}
template <bool NT>
__device__ __forceinline__ void dma4_abs(const float* gaddr, const void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  if (NT)
    __asm__ volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off nt" ::"s"(m0), "v"(gaddr) : "memory");
  else
    __asm__ volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(m0), "v"(gaddr) : "memory");
}

// Workgroup barrier without the release fence of __syncthreads (which would
// wait for every direct-to-LDS load in flight).  The empty asm statements keep
// the compiler from moving memory accesses across it; LDS writes that other
// waves read after it are completed first with an explicit lgkmcnt(0).
__device__ __forceinline__ void wg_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Wait until at most `ahead` (<= A) stages of this wave's loads, NV each, are
// outstanding.
template <int NV, int A>
__device__ __forceinline__ void wait_stages(int ahead) {
  if constexpr (A == 0) {
    wait_vmcnt<0>();
  } else {
    if (ahead >= A) {
      wait_vmcnt<A * NV>();
      return;
    }
    wait_stages<NV, A - 1>(ahead);
  }
}
// Waves below NBIG issue NI loads per stage, the others NI-1; e4m3 adds one
// scale load per wave.
template <int NI, int NBIG, bool FP8, int MAXA>
__device__ __forceinline__ void wait_vmcnt_ahead(int w, int ahead) {
  if (w < NBIG) wait_stages<NI + (FP8 ? 1 : 0), MAXA>(ahead);
  else wait_stages<NI - 1 + (FP8 ? 1 : 0), MAXA>(ahead);
}

__device__ __forceinline__ bf16x8 cvt_fp8x8(i32x2 v) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)v[0], 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)v[0], 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)v[1], 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)v[1], 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Maximum of three floats in one instruction.  The scores it is used on are
// never NaN; written as asm because fmaxf would first quiet each operand.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  __asm__("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ float wave_max_g(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

__device__ __forceinline__ float wave_sum_g(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// Workgroup -> (row block, work unit).  Workgroup ids congruent mod 8 run on
// the same XCD; the row blocks of one unit get ids congruent mod 8 so their KV
// reads share that XCD's L2.  Each block of 8 consecutive work items is
// rotated across the XCDs by a mix of the block index, so that the splits
// and ranks of one request spread over all XCDs even when a ragged batch
// concentrates the work in a few units.
struct WgUnit {
  int rb;
  int64_t unit;
};
__device__ __forceinline__ WgUnit wg_unit(int64_t id, int n_row_blocks) {
  const int xcd = (int)(id & 7);
  const int64_t qq = id >> 3;
  const int64_t blk = qq / n_row_blocks;
  const int rot = (int)((blk + (blk >> 3) + (blk >> 6)) & 7);
  return WgUnit{(int)(qq % n_row_blocks), blk * 8 + ((xcd + rot) & 7)};
}

// Global KV length of request b, or 0 when it is negative, above max_seq_len
// or needs more pages than a block-table row holds (reported when `report`).
__device__ __forceinline__ int32_t request_len(const DecodeParams& p, int b, bool report) {
  const int32_t L = p.seq_len[b];
  const int64_t vp = (int64_t)p.page * p.c;
  if (L < 0 || (int64_t)L > p.max_seq_len) {
    if (report && p.dev_status) atomicMax(p.dev_status, DCP_DEV_BAD_LENGTH);
    return 0;
  }
  if ((int64_t)L > (int64_t)p.bt_stride * vp) {  // ceil(L / vp) > bt_stride
    if (report && p.dev_status) atomicMax(p.dev_status, DCP_DEV_TABLE_OVERFLOW);
    return 0;
  }
  return L;
}

// Positions below x that rank r owns when runs of il consecutive positions go
// to the ranks in turn: il per full cycle of il*c positions, plus the part of
// r's run in the last, partial cycle.
__device__ __forceinline__ int32_t owned_below(int32_t x, int32_t r, int32_t c, int32_t il) {
  if (x <= 0) return 0;
  const int64_t cyc = (int64_t)il * c;
  const int64_t full = x / cyc;
  const int64_t rest = x - full * cyc - (int64_t)r * il;
  return (int32_t)(full * il + (rest < 0 ? 0 : (rest > il ? il : rest)));
}

// Rank-local tokens of rank r that query row qi sees: every owned position
// below L, or (causal) at most L - q_len + qi, where a verification step's
// query qi sits.  Rank r's positions rise with its local index, so the
// visible ones are a prefix of its shard.
__device__ __forceinline__ int32_t visible_tokens(int32_t L, int32_t r, int32_t c, int32_t il, int32_t q_len,
                                                  int32_t qi, int32_t causal) {
  const int32_t lim = causal ? L - q_len + qi : L - 1;
  return owned_below((lim + 1 < L ? lim + 1 : L), r, c, il);
}

// Decode kernel: a workgroup owns RGN row blocks of 16 query rows (RGN = 4,
// 2 or 1).  Waves 0..RGN-1 produce: wave q owns row block q, computes its
// full S^T (every 16-token block of the tile, all 576 columns), the online
// softmax and P^T, and publishes P^T (with the rescale factors when the
// running maximum moved) in a double-buffered LDS area.  The consumers
// multiply V^T by the P^T of the previous tile for a slice of the 512 output
// columns of every row block, so each transposed V fragment feeds RGN MFMAs.
// One workgroup barrier per tile hands P^T over and recycles the stage the
// consumers finished; producer and consumers of a SIMD run different phases
// and overlap (all waves at the same priority: a raised producer priority
// measured 3-4% slower).  Two shapes:
// * 8 waves (two per SIMD, up to 256 registers each): waves 4-7 consume,
//   wave 4+c owning columns [128c, 128c+128), and also issue every
//   direct-to-LDS load, which keeps the producers' path from one barrier to
//   the next free of load issue and waits; waves RGN..3 (RGN < 4) only take
//   part in the barriers;
// * 16 waves for bf16 blocks of 64 rows (four per SIMD, at most 128
//   registers each): waves 4-11 consume, wave 4+c owning columns
//   [64c, 64c+64), and waves 12-15 only issue the loads.  Issuing a stage's
//   loads holds the issuing wave for most of a tile; here no wave that
//   computes is held (128-head workloads 5-7% faster than with 8 waves).
//   Loading waves for e4m3 measured no faster: with 64-token tiles (the token
//   scales read where used to fit 128 registers) or with 32-token tiles.
// In the 8-wave e4m3 kernel for blocks of 64 rows the producers split each
// 64-token tile instead: producer w scores 32 rows (two row blocks) over one
// half of the tokens, so each K fragment it reads and converts feeds two
// MFMAs (half the K reads and conversions of four 16-row producers; long
// e4m3 workload 742/748 -> 706/701 us); the two producers of the same rows
// exchange their tile's row maxima through LDS before the exponentials.
template <int RGN, bool FP8>
constexpr bool kLoaderWaves = RGN == 4 && !FP8;
template <int RGN, bool FP8>
constexpr int kPcThreads = kLoaderWaves<RGN, FP8> ? 1024 : 512;

template <int RGN, bool FP8, bool ALIGNED, bool NT>
__global__ void __launch_bounds__((kPcThreads<RGN, FP8>), 1) mla_decode_pc_kernel(DecodeParams p) {
  constexpr bool LDW = kLoaderWaves<RGN, FP8>;
  constexpr int NTHR = kPcThreads<RGN, FP8>;
  static_assert(RGN == 1 || RGN == 2 || RGN == 4, "row blocks per workgroup");
  constexpr int MB = 16 * RGN;            // query rows per workgroup
  constexpr int ROWB = FP8 ? kDqk : 2 * kDqk;
  constexpr int CH = ROWB / 16;
  // tokens per stage (one tile): a 36 KB stage either way, 32 bf16 or 64
  // e4m3 rows, so an e4m3 tile carries the bytes of a bf16 one for the same
  // per-tile costs (barrier, softmax reductions, flags)
  constexpr int STOK = FP8 ? 64 : 32;
  constexpr int NTB = STOK / 16;          // 16-token blocks of a tile (score MFMA rows)
  constexpr int NH = STOK / 32;           // 32-token halves of a tile (PV MFMA k-steps)
  constexpr int SBYTES = STOK * ROWB;     // 36864
  constexpr int NSTG = FP8 ? 3 : 4;       // ring stages
  constexpr int NI_ALL = SBYTES / 1024;   // 1 KB direct-to-LDS loads per stage
  constexpr int NLW = 4;                  // waves that issue the direct-to-LDS loads
  constexpr int NI_MAX = (NI_ALL + NLW - 1) / NLW;            // loads of the busiest loading wave
  constexpr int NBIG = NI_ALL % NLW == 0 ? NLW : NI_ALL % NLW;  // loading waves that issue NI_MAX
  constexpr int NDBC = LDW ? 4 : 8;       // output blocks per consumer wave
  constexpr int SCW = STOK / NLW;         // e4m3 token scales loaded per loading wave
  constexpr int KU = FP8 ? 9 : 18;        // k units (k-steps, or e4m3 k-step pairs)
  // e4m3 blocks of 64 rows: each producer scores 32 rows (two row blocks) over
  // one 32-token half of every 64-token tile, so each K fragment it reads and
  // converts feeds two MFMAs; the two producers of the same rows (waves w and
  // w ^ 2) agree on the running maximum through LDS once per tile
  constexpr bool TS = FP8 && RGN == 4 && !LDW;

  __shared__ __attribute__((aligned(1024))) uint8_t lds_kv[NSTG * SBYTES];
  __shared__ __attribute__((aligned(16))) float lds_sc[FP8 ? NSTG * STOK : 4];
  __shared__ int32_t lds_pt[kMaxTab];
  __shared__ __attribute__((aligned(16))) bf16x8 lds_p[2][RGN * NH * 64];
  __shared__ float lds_alpha[2][RGN * 16];
  __shared__ __attribute__((aligned(16))) int lds_resc[2][4];  // read as one 16-byte vector
  __shared__ float lds_l[RGN * 16];
  __shared__ float lds_lh[TS ? 2 : 1][TS ? RGN * 16 : 1];     // per-half row sums
  __shared__ float lds_xmax[TS ? 2 : 1][TS ? 4 * 32 : 1];     // row maxima per producer
  __shared__ int lds_xflag[4];                                  // tile a producer's maxima are for

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, j = lane & 15;
  const bool producer = w < RGN;
  const bool consumer = LDW ? (w >= 4 && w < 12) : w >= 4;
  const bool loader = LDW ? w >= 12 : w >= 4;  // with 8 waves the consumers load
  const int rbq = w & 3;                  // producer: its row block
  const int pair = w & 1, half = w >> 1;  // token-split producer: rows 32*pair.., tokens 32*half..
  const int cq = LDW ? w - 4 : (w & 3);   // consumer: its column group

  const WgUnit wu = wg_unit(blockIdx.x, p.n_row_blocks);
  const int rb = wu.rb;
  // Without a plan (every unit is one item) item i is unit i, whole.  With
  // one, the workgroups of dispatch position i read the plan's record i: a
  // single load gives the item, its unit and token range, the request's
  // length and whether the unit is split (each further dependent load would
  // add a memory round trip before the first tile).  The plan writes every
  // position the grid covers; a record outside its bounds (a workspace this
  // call's plan did not write) ends the workgroup before it indexes anything.
  // Item bounds and tile count are uniform: scalar registers.
  int64_t item;
  int32_t unit, L, j_begin, j_stop;
  bool single;
  if (p.direct) {
    if (wu.unit >= p.units) return;
    item = wu.unit;
    unit = (int32_t)wu.unit;
    L = request_len(p, unit % p.batch, tid == 0);
    j_begin = 0;
    j_stop = INT32_MAX;
    single = true;
  } else {
    const int4* rec = reinterpret_cast<const int4*>(p.drec) + 2 * wu.unit;
    const int4 r0 = rec[0], r1 = rec[1];
    const int32_t it = __builtin_amdgcn_readfirstlane(r0.x);
    unit = __builtin_amdgcn_readfirstlane(r0.y);
    j_begin = __builtin_amdgcn_readfirstlane(r0.z);
    j_stop = __builtin_amdgcn_readfirstlane(r0.w);
    L = __builtin_amdgcn_readfirstlane(r1.x);
    single = __builtin_amdgcn_readfirstlane(r1.y) != 0;
    // (ceil(L / vp) > bt_stride, without a 64-bit division)
    const int64_t vp = (int64_t)p.page * p.c;
    if ((uint32_t)it >= (uint32_t)p.max_items || (uint32_t)unit >= (uint32_t)p.units || j_begin < 0 || L < 0 ||
        (int64_t)L > p.max_seq_len || (int64_t)L > (int64_t)p.bt_stride * vp)
      return;
    item = it;
  }
  const int b = unit % p.batch;
  const int rl = unit / p.batch;
  const int32_t ri = p.rank_begin + rl, Pi = p.page;
  const int row0 = rb * MB + rbq * 16;    // producer's first row

  // all rank-local token indices fit in int32 (seq_len is int32)
  auto visible = [&](int qi) -> int32_t { return visible_tokens(L, ri, p.c, p.interleave, p.q_len, qi, p.causal); };
  const int32_t n_wg = visible((rb * MB + MB - 1) / p.heads);
  const int32_t j_end = __builtin_amdgcn_readfirstlane(min(n_wg, j_stop));
  const int32_t jlim = min(visible(row0 / p.heads), j_stop);
  // wave-uniform: every row of a 16-row block belongs to the same query index
  const int32_t jlim_s = __builtin_amdgcn_readfirstlane(jlim);
  int32_t jlim_ts[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    jlim_ts[i] = __builtin_amdgcn_readfirstlane(min(visible((rb * MB + (2 * pair + i) * 16) / p.heads), j_stop));
  const int n_st = j_end > j_begin ? (j_end - j_begin + STOK - 1) / STOK : 0;
  // The row blocks of one item walk its tiles from different starting points
  // (block rb starts rb tiles ahead, wrapping around): the block
  // that reaches a tile first takes the miss and the others find the rows in
  // L2, instead of every block waiting on the same misses.  The order of the
  // tiles does not change the result beyond rounding.
  const int rot = n_st > 0 ? rb % n_st : 0;
  auto tile_of = [&](int s) { const int x = s + rot; return x < n_st ? x : x - n_st; };
  // a unit with one item writes o_part / lse_part directly (single); the
  // items of a split unit write partials (lse in base 2) for the combine,
  // also when this row block sees none of the item's tokens (lse = -inf, o = 0)

  const uint8_t* pool = p.pools + (int64_t)rl * p.pool_bytes;
  const float* spool = FP8 ? p.pool_scales + (int64_t)rl * p.cap : nullptr;
  const int32_t* bt = p.block_table + (int64_t)b * p.bt_stride;
  const int32_t vp_first = j_begin / Pi;
  const int32_t n_tab = n_st > 0 ? (j_end - 1) / Pi - vp_first + 1 : 0;
  if (n_tab > kMaxTab) return;  // the plan's item length keeps it within the table
  {
    bool bad_page = false;
    for (int t = tid; t < n_tab; t += NTHR) {
      int32_t pg = bt[vp_first + t];
      if ((unsigned)pg >= (unsigned)p.num_pages) {
        bad_page = true;
        pg = 0;
      }
      lds_pt[t] = pg;
    }
    if (bad_page && p.dev_status) atomicMax(p.dev_status, DCP_DEV_BAD_PAGE);
  }
  if (tid < 8) lds_resc[tid >> 2][tid & 3] = -1;
  if (tid < 4) lds_xflag[tid] = -1;

  // One register array serves both roles, which are fixed per wave: a
  // producer keeps its Q^T fragments (18 x 16 bytes) in R[0..17], a consumer
  // its O^T accumulators (NDBC column blocks x RGN row blocks).
  constexpr int NQ = TS ? 36 : 18;
  constexpr int NR = NDBC * RGN > NQ ? NDBC * RGN : NQ;
  f32x4 R[NR];
  if (producer) {
#pragma unroll
    for (int i = 0; i < NQ / 18; ++i) {
      const int qr = TS ? rb * MB + (2 * pair + i) * 16 : row0;
      const uint16_t* qrow = p.q + ((int64_t)b * p.rows + qr + j) * kDqk;
#pragma unroll
      for (int kk = 0; kk < 18; ++kk) {
        const int col = FP8 ? 64 * (kk >> 1) + 16 * g + 8 * (kk & 1) : 32 * kk + 8 * g;
        R[18 * i + kk] = __builtin_bit_cast(f32x4, *reinterpret_cast<const bf16x8*>(qrow + col));
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < NR; ++i) R[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  auto qf = [&](int kk) { return __builtin_bit_cast(bf16x8, R[kk]); };
  // Q and the page table must have landed before the loop: the compiler does
  // not count the asm loads below, so a wait for Q placed inside the loop
  // would also drain every load in flight
  wait_vmcnt<0>();
  __syncthreads();

  // direct-to-LDS loads, issued by the loading waves: loading wave lw issues
  // loads lw, lw + 4, ... of a stage; load i fills LDS bytes [1024 i, 1024 i +
  // 1024), lane k the 16 bytes at 1024 i + 16 k, which hold chunk
  // (pos ^ swz(row)) of stage row `row` (pos = position inside the row)
  const int lw = w & 3;
  const int ni = loader ? (lw < NBIG ? NI_MAX : NI_MAX - 1) : 0;
  int dma_row[NI_MAX];
  uint32_t dma_off[NI_MAX];
  auto init_dma = [&]() {
#pragma unroll
    for (int t = 0; t < NI_MAX; ++t) {
      const int ci = (lw + NLW * t) * 64 + lane;
      const int row = min(ci / CH, STOK - 1);
      dma_row[t] = row;
      dma_off[t] = (uint32_t)(row * ROWB + ((ci % CH) ^ swz<FP8>(row)) * 16);
    }
  };
  auto slot_of = [&](int32_t jj) -> int64_t {
    const int32_t pidx = jj / Pi;
    return (int64_t)lds_pt[pidx - vp_first] * Pi + (jj - pidx * Pi);
  };
  // page-table entry of the page that holds stage s (whole-stage fast path:
  // a stage never straddles pages)
  auto stage_pidx = [&](int s) { return (j_begin + tile_of(s) * STOK) / Pi - vp_first; };
  // issue stage s; pg is the page id of the stage (whole-stage fast path)
  auto issue = [&](int s, int32_t pg) {
    uint8_t* dst = lds_kv + (s % NSTG) * SBYTES;
    float* dst_sc = lds_sc + (FP8 ? (s % NSTG) * STOK : 0);
    const int32_t j0 = j_begin + tile_of(s) * STOK;
    if (ALIGNED && j0 + STOK <= j_end) {
      const int64_t slot0 = (int64_t)pg * Pi + (j0 - (j0 / Pi) * Pi);
      const uint8_t* base = pool + slot0 * ROWB;
#pragma unroll
      for (int t = 0; t < NI_MAX; ++t)
        if (t < ni) dma16<NT>(base, dma_off[t], dst + (lw + NLW * t) * 1024);
      if (FP8 && lane < SCW) dma4_abs<NT>(spool + slot0 + SCW * lw + lane, dst_sc + SCW * lw);
    } else {
      // last stage of a split (rows past j_end repeat the last valid row) or
      // pages that a stage can straddle
#pragma unroll
      for (int t = 0; t < NI_MAX; ++t)
        if (t < ni) {
          const int32_t jj = min(j0 + dma_row[t], j_end - 1);
          dma16_abs<NT>(pool + slot_of(jj) * ROWB + (dma_off[t] - dma_row[t] * ROWB), dst + (lw + NLW * t) * 1024);
        }
      if (FP8) {
        const int32_t jj = min(j0 + SCW * lw + (lane & (SCW - 1)), j_end - 1);
        const float* src = spool + slot_of(jj);
        if (lane < SCW) dma4_abs<NT>(src, dst_sc + SCW * lw);
      }
    }
  };

  // producer K offsets (token blocks 0 and 1) and consumer V^T offsets (the
  // first 32 tokens); the swizzles leave row bit 5 alone, so token block
  // tb + 2 and the second half of a 64-token tile sit 32 rows further
  int koff[2][2], voff[2][4];
  auto init_koff = [&]() {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int row = 16 * tb + j;
      if (FP8) {
        koff[tb][0] = row * ROWB + 16 * (g ^ swz<true>(row));
        koff[tb][1] = koff[tb][0];
      } else {
#pragma unroll
        for (int par = 0; par < 2; ++par) koff[tb][par] = row * ROWB + 16 * ((4 * par + g) ^ swz<false>(row));
      }
    }
  };
  auto init_voff = [&]() {
    if (FP8) {
      const int s8 = (lane & 15) >> 1;
      const int vrow = s8 < 4 ? 4 * (lane >> 4) + s8 : 16 + 4 * (lane >> 4) + (s8 - 4);
#pragma unroll
      for (int m = 0; m < 4; ++m) voff[0][m] = vrow * ROWB + 16 * (m ^ swz<true>(vrow)) + 8 * (lane & 1);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int vrow = 16 * h + 4 * (lane >> 4) + ((lane >> 2) & 3);
        const int y = ((lane & 3) >> 1) ^ swz<false>(vrow);
#pragma unroll
        for (int m = 0; m < 4; ++m) voff[h][m] = vrow * ROWB + 16 * ((2 * m) ^ y) + 8 * (lane & 1);
      }
    }
  };

  float m_run = -INFINITY, l_run = 0.f;   // producer softmax state of row row0 + j

  auto produce = [&](int t) {
    const uint8_t* kv = lds_kv + (t % NSTG) * SBYTES;
    const float* sc = lds_sc + (FP8 ? (t % NSTG) * STOK : 0);
    const int32_t jt = j_begin + tile_of(t) * STOK;
    f32x4 sacc[NTB];
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) sacc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // e4m3 token scales of this lane's tokens, read before the score MFMAs
    // so that their LDS latency is hidden
    float tsc[4 * NTB];
    if (FP8) {
#pragma unroll
      for (int h = 0; h < NTB; ++h) {
        // token 16h + 4g + i of the stage: one 16-byte read per block (the 16
        // lanes of a row group read the same four scales)
        const f32x4 v = *reinterpret_cast<const f32x4*>(sc + 16 * h + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) tsc[4 * h + i] = v[i];
      }
    }
    // K fragments f = 2u + tb (k unit u, token block tb), kept PD loads ahead
    // of the MFMA that uses them; the schedule below pins that interleave.
    if (FP8) {
      constexpr int NF = NTB * KU, PD = 6;
      i32x4 kf[NF];
      // fragment f: k unit u of token block tb, token-block major (each
      // accumulator takes its MFMAs back to back)
      auto ftb = [](int f) { return f / KU; };
      auto fu = [](int f) { return f % KU; };
      auto kload = [&](int f) {
        return *reinterpret_cast<const i32x4*>(kv + koff[ftb(f) & 1][0] + (ftb(f) >> 1) * 32 * ROWB + 64 * fu(f));
      };
#pragma unroll
      for (int f = 0; f < PD; ++f) kf[f] = kload(f);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        if (f + PD < NF) kf[f + PD] = kload(f + PD);
        const int u = fu(f), tb = ftb(f);
        sacc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cvt_fp8x8(i32x2{kf[f][0], kf[f][1]}), qf(2 * u), sacc[tb], 0, 0, 0);
        sacc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cvt_fp8x8(i32x2{kf[f][2], kf[f][3]}), qf(2 * u + 1), sacc[tb], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, PD, 0);
#pragma unroll
      for (int f = 0; f < NF - PD; ++f) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * PD, 0);
    } else {
      // fragment f = KU*tb + u: each accumulator takes its 18 MFMAs back to back
      // (5 fragments ahead in 128 registers: 4 measured 1% slower, 6 spill)
      constexpr int NF = 2 * KU, PD = LDW ? 5 : 8;
      bf16x8 kf[NF];
      auto ftb = [](int f) { return f / KU; };
      auto fu = [](int f) { return f % KU; };
      auto kload = [&](int f) {
        const int tb = ftb(f), u = fu(f);
        return *reinterpret_cast<const bf16x8*>(kv + koff[tb][u & 1] + 128 * (u >> 1));
      };
#pragma unroll
      for (int f = 0; f < PD; ++f) kf[f] = kload(f);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        if (f + PD < NF) kf[f + PD] = kload(f + PD);
        sacc[ftb(f)] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[f], qf(fu(f)), sacc[ftb(f)], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, PD, 0);
#pragma unroll
      for (int f = 0; f < NF - PD; ++f) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, PD, 0);
    }
    // ---- online softmax (base 2); lane holds tokens t2*16 + 4g + i of row j.
    // The running maximum only moves when some score exceeds it by kTau; that
    // is detected with a ballot and only then is the row maximum formed
    // across the lanes of the row.  exp2 is the hardware instruction: a
    // probability below 2^-126 flushes to zero, far below what bf16 P keeps.
    constexpr int NY = 4 * NTB;
    float y[NY];
#pragma unroll
    for (int e = 0; e < NY; ++e) {
      y[e] = sacc[e >> 2][e & 3];
      if (FP8) y[e] *= tsc[e];
      y[e] *= p.scale_log2;
    }
    if (jt + STOK > jlim_s) {  // the tile reaches past this row block's last visible token
      // masked by adding -inf, so every y stays an arithmetic result (the max
      // below then needs no NaN canonicalisation)
#pragma unroll
      for (int e = 0; e < NY; ++e)
        y[e] += (jt + (e >> 2) * 16 + 4 * g + (e & 3) >= jlim_s) ? -INFINITY : 0.f;
    }
    float mloc = max3f(max3f(y[0], y[1], y[2]), max3f(y[3], y[4], y[5]), fmaxf(y[6], y[7]));
#pragma unroll
    for (int e = 8; e < NY; e += 8)
      mloc = max3f(mloc, max3f(y[e], y[e + 1], y[e + 2]), max3f(max3f(y[e + 3], y[e + 4], y[e + 5]), y[e + 6], y[e + 7]));
    float alpha = 1.f;
    const bool resc = __any(mloc > m_run + kTau);
    if (resc) {
      const float mt = wave_max_g(mloc);
      if (mt > m_run + kTau) {
        alpha = __builtin_amdgcn_exp2f(m_run - mt);
        m_run = mt;
      }
    }
    const float mref = m_run == -INFINITY ? 0.f : m_run;
    float psum = 0.f;
    // P^T of 32-token half h: token blocks 2h and 2h + 1 (the PV operand order)
    bf16x8 pf[NH];
#pragma unroll
    for (int e = 0; e < NY; ++e) {
      float pe = __builtin_amdgcn_exp2f(y[e] - mref);
      psum += pe;
      if (FP8) pe *= tsc[e];
      pf[e >> 3][e & 7] = (__bf16)pe;
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int h = 0; h < NH; ++h) lds_p[t & 1][(rbq * NH + h) * 64 + lane] = pf[h];
    if (resc) {
      if (g == 0) lds_alpha[t & 1][rbq * 16 + j] = alpha;
      if (lane == 0) lds_resc[t & 1][rbq] = t;
    }
  };

  // Token-split producer (e4m3 blocks of 64 rows): rows 32*pair..32*pair+31
  // (row blocks 2*pair and 2*pair+1), tokens 32*half..32*half+31 of each
  // 64-token tile.  Both producers of the same rows keep the same running
  // maximum m2 (each sees the other's tile maximum before its exponentials)
  // and their own partial sums l2 of their half, added up at the end.
  float m2[2] = {-INFINITY, -INFINITY}, l2[2] = {0.f, 0.f};
  auto produce_ts = [&](int t) {
    const uint8_t* kv = lds_kv + (t % NSTG) * SBYTES;
    const float* sc = lds_sc + (t % NSTG) * STOK + 32 * half;
    const int32_t jt = j_begin + tile_of(t) * STOK + 32 * half;  // first token of this half
    f32x4 sacc[2][2];  // [row block][16-token block of the half]
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int tl = 0; tl < 2; ++tl) sacc[i][tl] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int NF = 2 * KU, PD = 4;  // fragment f: token block f / KU, k unit f % KU
    i32x4 kf[NF];
    auto kload = [&](int f) {
      return *reinterpret_cast<const i32x4*>(kv + koff[f / KU][0] + half * 32 * ROWB + 64 * (f % KU));
    };
#pragma unroll
    for (int f = 0; f < PD; ++f) kf[f] = kload(f);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if (f + PD < NF) kf[f + PD] = kload(f + PD);
      const int tl = f / KU, u = f % KU;
      const bf16x8 a0 = cvt_fp8x8(i32x2{kf[f][0], kf[f][1]});
      const bf16x8 a1 = cvt_fp8x8(i32x2{kf[f][2], kf[f][3]});
#pragma unroll
      for (int i = 0; i < 2; ++i) sacc[i][tl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf(18 * i + 2 * u), sacc[i][tl], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 2; ++i) sacc[i][tl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf(18 * i + 2 * u + 1), sacc[i][tl], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, PD, 0);
#pragma unroll
    for (int f = 0; f < NF - PD; ++f) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * PD, 0);
    // scores in base 2 with the token scales, masked past the visible limit
    float y[2][8], rmax[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int e = 0; e < 8; ++e) y[i][e] = sacc[i][e >> 2][e & 3] * sc[16 * (e >> 2) + 4 * g + (e & 3)] * p.scale_log2;
      if (jt + 32 > jlim_ts[i]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) y[i][e] += (jt + 16 * (e >> 2) + 4 * g + (e & 3) >= jlim_ts[i]) ? -INFINITY : 0.f;
      }
      rmax[i] = wave_max_g(max3f(max3f(y[i][0], y[i][1], y[i][2]), max3f(y[i][3], y[i][4], y[i][5]), fmaxf(y[i][6], y[i][7])));
    }
    // exchange the row maxima of this half with the partner (same rows, the
    // other half); the partner runs the same tiles, so the wait ends; it is
    // bounded anyway, and a wave that gives up reports it
    // volatile LDS pointers (with the LDS address space, so that these stay
    // ds_read / ds_write and are not turned into flat accesses)
    volatile __attribute__((address_space(3))) float* xm = DCP_LDS(float, lds_xmax[t & 1]);
    volatile __attribute__((address_space(3))) int* xf = DCP_LDS(int, lds_xflag);
    if (g == 0) {
      xm[w * 32 + j] = rmax[0];
      xm[w * 32 + 16 + j] = rmax[1];
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the maxima are in LDS before the flag
    if (lane == 0) xf[w] = t;
    const int partner = w ^ 2;
    int spin = 0;
    while (__builtin_amdgcn_readfirstlane(xf[partner]) != t && spin < (1 << 20)) {
      __builtin_amdgcn_s_sleep(1);
      ++spin;
    }
    if (spin >= (1 << 20) && lane == 0 && p.dev_status) atomicMax(p.dev_status, DCP_DEV_DECODE_STALLED);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    bf16x8 pf[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float mt = fmaxf(rmax[i], xm[partner * 32 + 16 * i + j]);
      float alpha = 1.f;
      const bool resc = __any(mt > m2[i] + kTau);
      if (mt > m2[i] + kTau) {
        alpha = __builtin_amdgcn_exp2f(m2[i] - mt);
        m2[i] = mt;
      }
      const float mref = m2[i] == -INFINITY ? 0.f : m2[i];
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float pe = __builtin_amdgcn_exp2f(y[i][e] - mref);
        psum += pe;
        pe *= sc[16 * (e >> 2) + 4 * g + (e & 3)];
        pf[i][e] = (__bf16)pe;
      }
      l2[i] = l2[i] * alpha + psum;
      lds_p[t & 1][((2 * pair + i) * NH + half) * 64 + lane] = pf[i];
      if (resc && half == 0) {
        if (g == 0) lds_alpha[t & 1][(2 * pair + i) * 16 + j] = alpha;
        if (lane == 0) lds_resc[t & 1][2 * pair + i] = t;
      }
    }
  };

  auto consume = [&](int t) {
    const uint8_t* kv = lds_kv + (t % NSTG) * SBYTES;
    // P^T of the row blocks and the eight V^T fragments of 32-token half h
    bf16x8 pg[RGN], vf[NDBC];
    auto operands = [&](int h) {
#pragma unroll
      for (int q = 0; q < RGN; ++q) pg[q] = lds_p[t & 1][(q * NH + h) * 64 + lane];
#pragma unroll
      for (int d = 0; d < NDBC; ++d) {
        const int db = cq * NDBC + d;
        if (FP8) {
          i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              DCP_LDS(i32x2, kv + voff[0][db & 3] + 64 * (db >> 2) + h * 32 * ROWB));
          vf[d] = cvt_fp8x8(raw);
        } else {
          i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(DCP_LDS(i16x4, kv + voff[0][db & 3] + 128 * (db >> 2)));
          i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(DCP_LDS(i16x4, kv + voff[1][db & 3] + 128 * (db >> 2)));
          typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;
          i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          vf[d] = __builtin_bit_cast(bf16x8, v);
        }
      }
    };
    auto mfmas = [&]() {
#pragma unroll
      for (int d = 0; d < NDBC; ++d)
#pragma unroll
        for (int q = 0; q < RGN; ++q)
          R[d * RGN + q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[d], pg[q], R[d * RGN + q], 0, 0, 0);
    };
    // every LDS read of the first half is issued first (the rescale flags,
    // P^T and V^T); the rescale and the MFMAs then wait for them in issue
    // order
    const i32x4 resc = *reinterpret_cast<const i32x4*>(&lds_resc[t & 1][0]);
    operands(0);
    bool any_resc = false;
#pragma unroll
    for (int q = 0; q < RGN; ++q) any_resc |= resc[q] == t;
    if (any_resc) {
#pragma unroll
      for (int q = 0; q < RGN; ++q)
        if (resc[q] == t) {
          const float a = lds_alpha[t & 1][q * 16 + j];
#pragma unroll
          for (int d = 0; d < NDBC; ++d) R[d * RGN + q] *= a;
        }
    }
    mfmas();
#pragma unroll
    for (int h = 1; h < NH; ++h) {
      operands(h);
      mfmas();
    }
  };

  // one loop per role, so that each role's registers are live only in its own
  // loop; every loop passes the workgroup barrier once before the first tile
  // and once per tile (n_st times)
  if (producer) {
    init_koff();
    wg_barrier();
    for (int i = 0; i < n_st; ++i) {
      if constexpr (TS) produce_ts(i);
      else produce(i);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): P^T and the rescale factors are in LDS
      wg_barrier();
    }
  } else if (LDW && consumer) {
    init_voff();
    wg_barrier();
    for (int i = 0; i < n_st; ++i) {
      if (i >= 1) consume(i - 1);
      __builtin_amdgcn_s_waitcnt(0xC07F);
      wg_barrier();
    }
    if (n_st > 0) consume(n_st - 1);
  } else {
    if (consumer) init_voff();
    if (loader) {
      init_dma();
      // stages 0 .. NSTG-2 in flight; stage 0 resident before the first tile
      for (int s = 0; s < NSTG - 1 && s < n_st; ++s) issue(s, ALIGNED ? __builtin_amdgcn_readfirstlane(lds_pt[stage_pidx(s)]) : 0);
      if (n_st > 0) wait_vmcnt_ahead<NI_MAX, NBIG, FP8, NSTG - 2>(lw, min(NSTG - 2, n_st - 1));
    }
    wg_barrier();
    for (int i = 0; i <= n_st; ++i) {
      const bool refill = i + NSTG - 1 < n_st;
      int32_t pg_next = 0;
      // page id of the stage issued after this tile's barrier, read early
      if (loader && ALIGNED && refill) pg_next = lds_pt[stage_pidx(i + NSTG - 1)];
      if (consumer && i >= 1) consume(i - 1);
      if (i == n_st) break;
      // stage i+1 must be resident for the next producer tile
      if (loader && i + 1 < n_st) wait_vmcnt_ahead<NI_MAX, NBIG, FP8, NSTG - 2>(lw, min(NSTG - 3, n_st - 2 - i));
      __builtin_amdgcn_s_waitcnt(0xC07F);
      wg_barrier();
      // the consumers are done with stage i-1: refill its slot
      if (loader && refill) issue(i + NSTG - 1, __builtin_amdgcn_readfirstlane(pg_next));
    }
  }

  // ---- finalise
  float* o_out = single ? p.o_part + (int64_t)unit * p.rows * kDv : p.ws_o + item * p.rows * kDv;
  if (producer && TS) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float lh = wave_sum_g(l2[i]);
      if (g == 0) lds_lh[half][(2 * pair + i) * 16 + j] = lh;
    }
  } else if (producer) {
    const float l_tot = wave_sum_g(l_run);
    if (g == 0) {
      lds_l[rbq * 16 + j] = l_tot;
      const float lse2 = l_tot > 0.f ? m_run + log2f(l_tot) : -INFINITY;
      if (single)
        p.lse_part[(int64_t)unit * p.rows + row0 + j] = p.out_base2 ? lse2 : lse2 * kLn2;
      else
        p.ws_lse[item * p.rows + row0 + j] = lse2;
    }
  }
  __syncthreads();
  if (TS && producer && half == 0 && g == 0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = (2 * pair + i) * 16 + j;
      const float l_tot = lds_lh[0][r] + lds_lh[1][r];
      const float lse2 = l_tot > 0.f ? m2[i] + log2f(l_tot) : -INFINITY;
      if (single)
        p.lse_part[(int64_t)unit * p.rows + rb * MB + r] = p.out_base2 ? lse2 : lse2 * kLn2;
      else
        p.ws_lse[item * p.rows + rb * MB + r] = lse2;
    }
  }
  if (consumer) {
    const int64_t orow0 = rb * MB + j;
#pragma unroll
    for (int q = 0; q < RGN; ++q) {
      const float lq = TS ? lds_lh[0][q * 16 + j] + lds_lh[1][q * 16 + j] : lds_l[q * 16 + j];
      const float inv = lq > 0.f ? 1.0f / lq : 0.f;
      float* optr = o_out + (orow0 + q * 16) * kDv;
#pragma unroll
      for (int d = 0; d < NDBC; ++d) {
        const int col = (cq * NDBC + d) * 16 + 4 * g;
        *reinterpret_cast<f32x4*>(optr + col) = R[d * RGN + q] * inv;
      }
    }
  }
}

// ---- work plan --------------------------------------------------------------
// One workgroup cuts every unit (rank, request) into work items of whole
// 32-token stages.  The item length T (in stages) spreads the call's total
// work W over about items_target items per row block, which gives every CU
// a few items and keeps the largest at about half of a CU's share; T is
// clamped to [t_min, t_max] (t_max: an item's page ids fit the workgroup's
// LDS table).  A unit of s stages gets ceil(s / T) items: of equal length
// when the units are about equally long, else of T stages and a shorter
// last one.  The items' slots (where their partials go) list the units with
// several items first; the decode workgroups take the items in a dispatch
// order, longest first when the lengths are ragged, each position with a
// record of everything the workgroup needs before its first load.  Every
// unit gets at least one item (an empty one for a rank that sees no token),
// so its outputs are always written.
// Exclusive prefix sum over the NW waves of a workgroup (64-bit values):
// wave scans with shuffles, then the wave totals.  Returns the prefix and
// sets total.
template <int NW>
__device__ __forceinline__ int64_t block_excl_scan(int64_t v, int64_t* wtot, int64_t& total) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int64_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wtot[wv] = x;
  __syncthreads();
  int64_t before = 0;
  total = 0;
  for (int i = 0; i < NW; ++i) {
    const int64_t t = wtot[i];
    if (i < wv) before += t;
    total += t;
  }
  __syncthreads();
  return before + x - v;
}

// Two exclusive prefix sums over the NW waves at once (one pair of barriers
// for both).
template <int NW>
__device__ __forceinline__ void block_excl_scan2(int64_t va, int64_t vb, int64_t* wtot, int64_t& pa, int64_t& pb,
                                                 int64_t& ta, int64_t& tb) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int64_t a = va, b = vb;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t ya = __shfl_up(a, o), yb = __shfl_up(b, o);
    if (lane >= o) {
      a += ya;
      b += yb;
    }
  }
  if (lane == 63) {
    wtot[wv] = a;
    wtot[16 + wv] = b;
  }
  __syncthreads();
  int64_t ba = 0, bb = 0;
  ta = 0;
  tb = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int64_t x = wtot[i], y = wtot[16 + i];
    if (i < wv) {
      ba += x;
      bb += y;
    }
    ta += x;
    tb += y;
  }
  __syncthreads();
  pa = ba + a - va;
  pb = bb + b - vb;
}

// Sum and maximum over the NW waves of a workgroup (every thread gets both).
template <int NW>
__device__ __forceinline__ void block_sum_max(int64_t v, int32_t m, int64_t* wtot, int64_t& sum, int32_t& mx) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    v += __shfl_xor(v, o);
    const int32_t y = __shfl_xor(m, o);
    m = y > m ? y : m;
  }
  if (lane == 0) {
    wtot[wv] = v;
    wtot[16 + wv] = m;
  }
  __syncthreads();
  sum = 0;
  mx = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    sum += wtot[i];
    const int32_t y = (int32_t)wtot[16 + i];
    mx = y > mx ? y : mx;
  }
  __syncthreads();
}

// NTHR threads (64, 256 or 1024): at least one per unit up to 1024 units, so
// small batches plan in one or four waves instead of sixteen (the plan is a
// chain of short dependent steps, and sixteen waves on four SIMDs take turns
// at every one of them); the result does not depend on NTHR.
template <int NTHR>
__global__ void __launch_bounds__(NTHR) decode_plan_kernel(DecodeParams p) {
  constexpr int NW = NTHR / 64;
  __shared__ int64_t wtot[32];
  const int tid = threadIdx.x;
  // stages of unit u and its request's KV length (a length the decode cannot
  // take is reported here and counts as 0; the decode reads it from the
  // dispatch records)
  auto unit_stages = [&](int32_t u, int32_t& L) -> int32_t {
    const int b = u % p.batch, rl = u / p.batch;
    L = request_len(p, b, true);
    const int32_t n = visible_tokens(L, p.rank_begin + rl, p.c, p.interleave, p.q_len, p.q_len - 1, p.causal);
    return (n + p.stage_tok - 1) / p.stage_tok;
  };
  // the first chunk's stage counts and lengths stay in registers (one read
  // of seq_len)
  int32_t L0 = 0;
  const int32_t st0 = tid < p.units ? unit_stages(tid, L0) : 0;
  int64_t w = st0;
  int32_t mx = st0;
  for (int32_t u = tid + NTHR; u < p.units; u += NTHR) {
    int32_t Lu;
    const int32_t st = unit_stages(u, Lu);
    w += st;
    mx = st > mx ? st : mx;
  }
  int64_t W;
  int32_t st_max;
  block_sum_max<NW>(w, mx, wtot, W, st_max);
  // When the units are about equally long (the longest at most 1.25 x the
  // mean) there is no ragged tail to spread, and one item per CU and row
  // block beats two: each item pays a q load, a pipeline fill and, when its
  // unit is split, a partial write and its share of the combine.
  int64_t target = p.items_target;
  const bool uniform = (int64_t)st_max * p.units * 4 <= W * 5;
  if (uniform) target = target > 1 ? target / 2 : 1;
  int64_t T64 = (W + target - 1) / target;
  // within [t_min, t_max]: 32-bit from here on (item arithmetic stays in int32)
  const int32_t T = (int32_t)(T64 < p.t_min ? p.t_min : (T64 > p.t_max ? p.t_max : T64));
  // A unit of st stages gets ceil(st / T) items: equal ones when the units
  // are about equally long; with ragged lengths items of T stages and a
  // shorter last one (the last items then come in many lengths, and the
  // longest-first dispatch below places them to fill the tail).  Item k
  // covers stages [k len, min((k + 1) len, st)).
  auto plan_of = [&](int32_t st, int32_t& items, int32_t& len) {
    if (st == 0) {
      items = 1;
      len = 0;
      return;
    }
    items = (st + T - 1) / T;  // st < 2^26 stages, T <= t_max: no overflow
    if (!uniform) {
      len = T;
      return;
    }
    len = (st + items - 1) / items;
    items = (st + len - 1) / len;
  };
  // Slots: the items of units with several items first, then the
  // single-item units (a separate counting pass unless every unit fits one
  // chunk of NTHR).
  int64_t multi_total = 0;
  if (p.units > NTHR) {
    for (int32_t base = 0; base < p.units; base += NTHR) {
      const int32_t u = base + tid;
      int32_t items = 0, len = 0;
      int32_t Lu;
      if (u < p.units) plan_of(base == 0 ? st0 : unit_stages(u, Lu), items, len);
      int64_t tot;
      block_excl_scan<NW>(items > 1 ? items : 0, wtot, tot);
      multi_total += tot;
    }
  }
  // Dispatch order.  With ragged lengths (and at most 1024 units) the items
  // are dispatched longest first, ties by unit and then by position in the
  // unit, so the longest work starts first and the short items fill the
  // tail; otherwise in the order of their slots (split units first).  No
  // item is longer than T: the items of exactly T stages come first, in
  // unit order (an exclusive scan of their counts), then each unit's shorter
  // item (at most one per unit) at the count of the shorter items that are
  // longer, or as long in an earlier unit.  The slots (partials of split
  // units) stay contiguous per unit for the combine.
  __shared__ __attribute__((aligned(16))) int32_t s_key[NTHR];
  __shared__ int32_t s_pos[2][NTHR];  // first position of the T-stage items, of the shorter one
  const bool lpt = !uniform && p.units <= NTHR;  // NTHR >= units whenever units <= 1024
  if (lpt) {
    int32_t items = 0, len = 0, n_t = 0;
    if (tid < p.units) {
      plan_of(st0, items, len);
      n_t = st0 > 0 ? st0 / len : 0;  // items of exactly T = len stages
    }
    const int32_t rest = st0 - n_t * len;  // the shorter item's stages (0: empty unit)
    const bool has_rest = tid < p.units && n_t < items;
    // key: the item's length (clamped, it only orders the dispatch), then
    // the unit index reversed, so a larger key comes first; -1: no such item
    s_key[tid] = has_rest ? (min(rest, (1 << 20) - 1) << 10 | (1023 - tid)) : -1;
    int64_t n_t_total;
    const int64_t t_before = block_excl_scan<NW>(n_t, wtot, n_t_total);
    // tpu consecutive threads (a power of two, within one wave) count for one
    // unit, each over a slice of whole groups of four units
    int tpu = 1;
    while (tpu < 64 && tpu * 2 * p.units <= NTHR) tpu *= 2;
    const int u = tid / tpu, part = tid % tpu;
    int32_t before = 0;
    if (u < p.units) {
      const int32_t key = s_key[u];
      const int32_t per = ((p.units + tpu - 1) / tpu + 3) & ~3;
      const int32_t v0 = part * per, ve = min((p.units + 3) & ~3, v0 + per);
      auto count4 = [&](int32_t v) {
        const int4 k4 = *reinterpret_cast<const int4*>(&s_key[v]);
        return (k4.x > key) + (k4.y > key) + (k4.z > key) + (k4.w > key);
      };
      // four LDS reads in flight per step: the loop is latency-bound
      int32_t v = v0;
      for (; v + 16 <= ve; v += 16) before += count4(v) + count4(v + 4) + count4(v + 8) + count4(v + 12);
      for (; v < ve; v += 4) before += count4(v);
    }
    for (int o = 1; o < tpu; o <<= 1) before += __shfl_xor(before, o);
    if (tid < p.units) s_pos[0][tid] = (int32_t)t_before;
    if (u < p.units && part == 0) s_pos[1][u] = (int32_t)n_t_total + before;
    __syncthreads();
  }
  // item offsets: items of split units in the high 32 bits, single-item
  // units in the low 32 bits; a second scan numbers the split units
  int64_t carry = 0, carry_split = 0;
  for (int32_t base = 0; base < p.units; base += NTHR) {
    const int32_t u = base + tid;
    int32_t st = 0, items = 0, len = 0, L = L0;
    if (u < p.units) {
      st = base == 0 ? st0 : unit_stages(u, L);
      plan_of(st, items, len);
    }
    int64_t tot, tot_split, off, nsplit;
    block_excl_scan2<NW>(items > 1 ? ((int64_t)items << 32) : (int64_t)items, items > 1 ? 1 : 0, wtot, off, nsplit,
                         tot, tot_split);
    off += carry;
    nsplit += carry_split;
    if (p.units <= NTHR) multi_total = tot >> 32;
    if (u < p.units) {
      const int32_t first = items > 1 ? (int32_t)(off >> 32) : (int32_t)(multi_total + (off & 0xffffffffLL));
      p.unit_first[u] = first;
      p.unit_count[u] = items;
      const int32_t n_t = lpt && st > 0 ? st / len : 0;
      const int32_t pos_t = lpt ? s_pos[0][u] : first, pos_r = lpt ? s_pos[1][u] : first + n_t;
      for (int32_t k = 0; k < items; ++k) {
        const int32_t pos = k < n_t || !lpt ? pos_t + k : pos_r;
        int4* rec = reinterpret_cast<int4*>(p.drec) + 2 * (int64_t)pos;
        rec[0] = int4{first + k, u, k * len * p.stage_tok, min((k + 1) * len, st) * p.stage_tok};
        rec[1] = int4{L, items == 1 ? 1 : 0, 0, 0};
      }
      if (items > 1) p.split_units[nsplit] = u;
    }
    carry += tot;
    carry_split += tot_split;
  }
  // the positions past the last item that the decode grid covers
  const int64_t n_total = multi_total + (carry & 0xffffffffLL);
  for (int64_t pos = n_total + tid; pos < ((int64_t)p.max_items + 7) / 8 * 8; pos += NTHR)
    reinterpret_cast<int4*>(p.drec)[2 * pos] = int4{-1, 0, 0, 0};
  if (tid == 0) {
    p.n_items[0] = (int32_t)n_total;
    p.n_items[1] = (int32_t)carry_split;
    int32_t items_max = 0, len = 0;
    plan_of(st_max, items_max, len);
    p.n_items[2] = items_max;
  }
}

// Merge of the base-2 partials [0, n) of one row over columns 8t..8t+7:
// acc = sum_r 2^(l_r - m) o_r / tot and lse = m + log2 tot with m the largest
// l_r; no partial (or only empty ones): lse = -inf, acc = 0.  One pass over the
// partials, 8 at a time (their lse and columns loaded together, then the
// running maximum and sums rescaled as in the online softmax), so a pair
// costs one round of load latency per 8 partials.
__device__ __forceinline__ void merge_cols8(const float* __restrict__ o, int64_t o_stride,
                                            const float* __restrict__ lse, int64_t lse_stride, int n, int t,
                                            f32x4& a0, f32x4& a1, float& lse_out) {
  float m = -INFINITY, tot = 0.f;
  a0 = f32x4{0.f, 0.f, 0.f, 0.f};
  a1 = a0;
  for (int r0 = 0; r0 < n; r0 += 8) {
    float l[8];
    f32x4 v0[8], v1[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      l[k] = -INFINITY;
      if (r0 + k < n) {
        l[k] = lse[(r0 + k) * lse_stride];
        v0[k] = *reinterpret_cast<const f32x4*>(o + (r0 + k) * o_stride + 8 * t);
        v1[k] = *reinterpret_cast<const f32x4*>(o + (r0 + k) * o_stride + 8 * t + 4);
      }
    }
    float mb = m;
#pragma unroll
    for (int k = 0; k < 8; ++k) mb = fmaxf(mb, l[k]);
    if (mb == -INFINITY) continue;
    const float sc = exp2f(m - mb);  // 0 while nothing was summed (m = -inf)
    tot *= sc;
    a0 *= sc;
    a1 *= sc;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (l[k] != -INFINITY) {
        const float w = exp2f(l[k] - mb);
        tot += w;
        a0 += w * v0[k];
        a1 += w * v1[k];
      }
    m = mb;
  }
  if (m == -INFINITY) {
    lse_out = -INFINITY;
    return;
  }
  const float inv = 1.0f / tot;
  a0 *= inv;
  a1 *= inv;
  lse_out = m + log2f(tot);
}

__global__ void __launch_bounds__(256) split_combine_kernel(DecodeParams p) {
  __shared__ float s_lse[4];
  __shared__ f32x4 s_acc[4][64][2];
  const int grp = threadIdx.x >> 6, t = threadIdx.x & 63;
  const int64_t n_pairs = (int64_t)p.n_items[1] * p.rows;
  if (p.n_items[2] < 8) {
    // few items per unit: each 64-thread group merges a pair of its own
    for (int64_t pr = (int64_t)blockIdx.x * 4 + grp; pr < n_pairs; pr += (int64_t)gridDim.x * 4) {
      const int32_t unit = p.split_units[pr / p.rows];
      const int rr = (int)(pr % p.rows);
      const int64_t first = p.unit_first[unit];
      f32x4 o0, o1;
      float l2;
      merge_cols8(p.ws_o + (first * p.rows + rr) * kDv, (int64_t)p.rows * kDv, p.ws_lse + first * p.rows + rr,
                  p.rows, p.unit_count[unit], t, o0, o1, l2);
      const int64_t row = (int64_t)unit * p.rows + rr;
      *reinterpret_cast<f32x4*>(p.o_part + row * kDv + 8 * t) = o0;
      *reinterpret_cast<f32x4*>(p.o_part + row * kDv + 8 * t + 4) = o1;
      if (t == 0) p.lse_part[row] = p.out_base2 ? l2 : l2 * kLn2;
    }
    return;
  }
  for (int64_t pr = blockIdx.x; pr < n_pairs; pr += gridDim.x) {
    const int32_t unit = p.split_units[pr / p.rows];
    const int rr = (int)(pr % p.rows);
    const int64_t first = p.unit_first[unit];
    const int32_t cnt = p.unit_count[unit];
    const int32_t a = (int32_t)((int64_t)cnt * grp / 4), b = (int32_t)((int64_t)cnt * (grp + 1) / 4);
    f32x4 a0, a1;
    float l2;
    merge_cols8(p.ws_o + ((first + a) * p.rows + rr) * kDv, (int64_t)p.rows * kDv, p.ws_lse + (first + a) * p.rows + rr,
                p.rows, b - a, t, a0, a1, l2);
    s_acc[grp][t][0] = a0;
    s_acc[grp][t][1] = a1;
    if (t == 0) s_lse[grp] = l2;
    __syncthreads();
    if (grp == 0) {
      float m = -INFINITY;
#pragma unroll
      for (int k = 0; k < 4; ++k) m = fmaxf(m, s_lse[k]);
      f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = o0;
      float lse2 = -INFINITY;
      if (m != -INFINITY) {
        float tot = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (s_lse[k] != -INFINITY) {
            const float w = exp2f(s_lse[k] - m);
            tot += w;
            o0 += w * s_acc[k][t][0];
            o1 += w * s_acc[k][t][1];
          }
        const float inv = 1.0f / tot;
        o0 *= inv;
        o1 *= inv;
        lse2 = m + log2f(tot);
      }
      const int64_t row = (int64_t)unit * p.rows + rr;
      *reinterpret_cast<f32x4*>(p.o_part + row * kDv + 8 * t) = o0;
      *reinterpret_cast<f32x4*>(p.o_part + row * kDv + 8 * t + 4) = o1;
      if (t == 0) p.lse_part[row] = p.out_base2 ? lse2 : lse2 * kLn2;
    }
    __syncthreads();
  }
}

template <int RGN, bool FP8>
hipError_t launch_pc(const DecodeParams& prm, bool aligned, int64_t grid, hipStream_t stream) {
  const dim3 g((unsigned)grid), b(kPcThreads<RGN, FP8>);
  const bool nt = prm.n_row_blocks == 1;
  if (aligned && nt) hipLaunchKernelGGL((mla_decode_pc_kernel<RGN, FP8, true, true>), g, b, 0, stream, prm);
  else if (aligned) hipLaunchKernelGGL((mla_decode_pc_kernel<RGN, FP8, true, false>), g, b, 0, stream, prm);
  else if (nt) hipLaunchKernelGGL((mla_decode_pc_kernel<RGN, FP8, false, true>), g, b, 0, stream, prm);
  else hipLaunchKernelGGL((mla_decode_pc_kernel<RGN, FP8, false, false>), g, b, 0, stream, prm);
  return hipGetLastError();
}

// Scratch of the allocation-free entry point: the work plan and the split
// partials of one call, in a file-scope device array (one copy per GPU, held
// until the process ends).  Host code never passes `scratch` itself to a
// kernel (on the host it names a stand-in, not a device address): the device
// address is looked up once per device with hipGetSymbolAddress.
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

DecodePlan plan_decode(int32_t c, int32_t interleave, int32_t page, bool fp8, int32_t rank_count, int32_t batch,
                       int32_t q_len, int32_t heads, int64_t max_seq_len) {

  DecodePlan pl{};
  pl.rows = q_len * heads;
  const int rg = pl.rows % 64 == 0 ? 4 : (pl.rows % 32 == 0 ? 2 : 1);
  pl.row_block = 16 * rg;
  pl.n_row_blocks = pl.rows / pl.row_block;
  pl.stage_tokens = fp8 ? 2 * kStageTok : kStageTok;
  const int32_t stok = pl.stage_tokens;
  pl.units = (int64_t)rank_count * batch;
  // a rank owns at most ceil(L / (I c)) chunks of I positions of a request of L
  const int64_t cyc = (int64_t)interleave * c;
  const int64_t n_r_max = (max_seq_len + cyc - 1) / cyc * interleave;
  const int64_t stages_max = (n_r_max + stok - 1) / stok;
  // (capped at 2^27 stages, more than any unit holds: seq_len is int32)
  pl.t_max = (int32_t)std::min<int64_t>(int64_t(1) << 27, std::max<int64_t>(1, (int64_t)(kMaxTab - 1) * page / stok));
  // the shortest item: kItemMinStages 32-token stages' worth of tokens
  pl.t_min = std::min<int32_t>(std::max<int32_t>(1, kItemMinStages * kStageTok / stok), pl.t_max);
  pl.items_target = std::max<int32_t>(1, kItemsPerCu * device_cu_count() / pl.n_row_blocks);
  // the device plan makes at most units + max(items_target, units * ceil(stages_max / t_max)) items;
  // the item length T is at least t_min stages, so a unit of at most t_min
  // stages is one item: with no unit longer than that the call needs no
  // split combine
  pl.direct = stages_max <= pl.t_min;
  pl.max_items = pl.direct
                     ? pl.units
                     : pl.units + std::max<int64_t>(pl.items_target,
                                                    pl.units * ((stages_max + pl.t_max - 1) / pl.t_max));
  if (pl.direct) {
    // one launch that never touches the workspace: a token size that does not
    // grow with the batch
    pl.off_ws_lse = pl.off_ints = 0;
    pl.workspace_bytes = 256;
    return pl;
  }
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  pl.off_ws_lse = al((size_t)pl.max_items * pl.rows * kDv * sizeof(float));
  pl.off_ints = pl.off_ws_lse + al((size_t)pl.max_items * pl.rows * sizeof(float));
  // dispatch records (8 ints for each position the decode grid covers), the
  // item counts, then the per-unit lists
  pl.workspace_bytes =
      pl.off_ints + al((size_t)(8 * ((pl.max_items + 7) / 8 * 8) + 3 + 3 * pl.units) * sizeof(int32_t));
  return pl;
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& pl, hipStream_t stream) {
  if (a.batch == 0 || a.rank_count == 0) return hipSuccess;
  if (pl.max_items > INT32_MAX / 2 || pl.units > INT32_MAX / 2) return hipErrorInvalidValue;
  DecodeParams prm{};
  const int row_bytes = a.fp8 ? kDqk : 2 * kDqk;
  prm.pools = (const uint8_t*)a.pools;
  prm.pool_scales = a.pool_scales;
  prm.cap = (int64_t)a.num_pages * a.page;
  prm.pool_bytes = prm.cap * row_bytes;
  prm.c = a.c;
  prm.interleave = a.interleave;
  prm.page = a.page;
  prm.num_pages = a.num_pages;
  prm.rank_begin = a.rank_begin;
  prm.q = (const uint16_t*)a.q;
  prm.batch = a.batch;
  prm.q_len = a.q_len;
  prm.heads = a.heads;
  prm.rows = pl.rows;
  prm.block_table = a.block_table;
  prm.bt_stride = a.bt_stride;
  prm.seq_len = a.seq_len;
  prm.max_seq_len = a.max_seq_len;
  prm.scale_log2 = a.sm_scale * kLog2e;
  prm.out_base2 = a.base2 ? 1 : 0;
  prm.causal = a.causal ? 1 : 0;
  prm.o_part = a.o_part;
  prm.lse_part = a.lse_part;
  prm.n_row_blocks = pl.n_row_blocks;
  prm.stage_tok = pl.stage_tokens;
  prm.units = (int32_t)pl.units;
  prm.max_items = (int32_t)pl.max_items;
  prm.items_target = pl.items_target;
  prm.t_min = pl.t_min;
  prm.t_max = pl.t_max;
  uint8_t* ws = (uint8_t*)a.workspace;
  prm.ws_o = (float*)ws;
  prm.ws_lse = (float*)(ws + pl.off_ws_lse);
  int32_t* ints = (int32_t*)(ws + pl.off_ints);
  prm.drec = ints;  // 256-byte aligned: records load as two 16-byte words
  prm.n_items = ints + 8 * ((pl.max_items + 7) / 8 * 8);
  prm.unit_first = prm.n_items + 3;
  prm.unit_count = prm.unit_first + pl.units;
  prm.split_units = prm.unit_count + pl.units;
  prm.dev_status = a.dev_status;
  // a call whose units are all single items needs neither the plan nor the
  // split combine: one kernel launch
  prm.direct = pl.direct ? 1 : 0;
  hipError_t e = hipSuccess;
  if (!pl.direct) {
    if (pl.units <= 64)
      hipLaunchKernelGGL(decode_plan_kernel<64>, dim3(1), dim3(64), 0, stream, prm);
    else if (pl.units <= 256)
      hipLaunchKernelGGL(decode_plan_kernel<256>, dim3(1), dim3(256), 0, stream, prm);
    else
      hipLaunchKernelGGL(decode_plan_kernel<1024>, dim3(1), dim3(1024), 0, stream, prm);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const bool aligned = a.page % pl.stage_tokens == 0;
  const int64_t grid = (pl.max_items + 7) / 8 * 8 * pl.n_row_blocks;
  const int rg = pl.row_block / 16;
  if (a.fp8)
    e = rg == 4 ? launch_pc<4, true>(prm, aligned, grid, stream)
                : (rg == 2 ? launch_pc<2, true>(prm, aligned, grid, stream) : launch_pc<1, true>(prm, aligned, grid, stream));
  else
    e = rg == 4 ? launch_pc<4, false>(prm, aligned, grid, stream)
                : (rg == 2 ? launch_pc<2, false>(prm, aligned, grid, stream) : launch_pc<1, false>(prm, aligned, grid, stream));
  if (e != hipSuccess || pl.direct) return e;
  // at most (max_items - units) units are split; a grid-stride loop covers them
  const int64_t pairs_max = std::min<int64_t>(pl.max_items - pl.units, pl.units) * pl.rows;
  const int64_t cgrid =
      std::max<int64_t>(1, std::min<int64_t>(pairs_max, kCombineBlocksPerCu * device_cu_count()));
  hipLaunchKernelGGL(split_combine_kernel, dim3((unsigned)cgrid), dim3(256), 0, stream, prm);
  return hipGetLastError();
}

}  // namespace dcp
