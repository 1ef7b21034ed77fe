// Expert align: a stable counting sort of the (token, slot) assignments by
// expert, each expert segment padded to the GEMM block M.
//
// Block granularity per expert follows the combine bookkeeping of "[SGLang]
// Single Batch Overlap for MoE models" (combine signal section: one signal per
// expert and 64-token block); padding rows of the gathered batch ("DP
// Attention and TBO for DeepSeek-V4 on MI355X", PrefillDelayer section) carry
// no assignment and are skipped.
//
// Small batches: one 1024-thread workgroup, LDS histogram -> wave scan of the
// padded counts -> stable scatter in 1024-assignment chunks.  Large batches
// split the same steps over spans of 4096 assignments (three launches).  Inside a chunk, a lane's rank
// among the lanes of its wave with the same expert comes from nine ballots
// over the bits of the expert id; ranks across the chunk's 16 waves come from
// per-wave counts in LDS.  The result is unique and deterministic.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {
namespace {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / kWave;
constexpr int kMaxSeg = 257;  // 256 routed experts + 1 shared
constexpr int kBigTile = 128; // row tile of the GEMM kernels

// Expert of assignment a in the virtual [T, k + n_shared] slot grid, or -1.
// Slot k (when n_shared) is the shared expert E of every valid row (a row is
// valid iff its first routed id is valid).
__device__ __forceinline__ int seg_of(const int32_t* ids, int a, int k, int kk,
                                      int E) {
  const int t = a / kk, j = a - t * kk;
  if (j < k) {
    const int e = ids[(size_t)t * k + j];
    return (e >= 0 && e < E) ? e : -1;
  }
  const int e0 = ids[(size_t)t * k];
  return (e0 >= 0 && e0 < E) ? E : -1;
}

// Exclusive scan of the padded segment counts (cnt in LDS) by wave 0 into
// base (LDS) and offsets / n_post; wave 1 lists the 128-row tiles of the
// segments above big_thr rows; wave 2 lists the streaming kernels' work
// items (the rows of every other non-empty segment, kStreamItemRows at a
// time).  Ends with a barrier.
__device__ void scan_segments(const int* cnt, int* base, int nseg, int bm, int32_t* offsets,
                              int32_t* n_post, int big_thr, int min_tiles, int32_t* tile_seg,
                              int32_t* tile_row0, int32_t* n_tiles, int32_t* item_seg,
                              int32_t* item_row0, int32_t* n_items) {
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  if (wave == 0) {
    int local[5];
    int sum = 0;
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      const int seg = lane * 5 + q;
      const int c = seg < nseg ? cnt[seg] : 0;
      local[q] = (c + bm - 1) / bm * bm;
      sum += local[q];
    }
    int inc = sum;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(inc, off);
      if (lane >= off) inc += o;
    }
    int run = inc - sum;
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      const int seg = lane * 5 + q;
      if (seg < nseg) {
        base[seg] = run;
        offsets[seg] = run;
      }
      run += local[q];
    }
    if (lane == kWave - 1) {
      offsets[nseg] = inc;
      *n_post = inc;
    }
  } else if (wave == 1 && tile_seg != nullptr) {
    // 128-row tiles of the segments with more than big_thr rows (handled by
    // the tiled GEMM kernels), in segment order
    int local[5];
    int sum = 0;
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      const int seg = lane * 5 + q;
      const int c = seg < nseg ? cnt[seg] : 0;
      local[q] = c > big_thr ? (c + kBigTile - 1) / kBigTile : 0;
      sum += local[q];
    }
    int inc = sum;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(inc, off);
      if (lane >= off) inc += o;
    }
    int run = inc - sum;
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      for (int i = 0; i < local[q]; ++i) {
        tile_seg[run + i] = lane * 5 + q;
        tile_row0[run + i] = i * kBigTile;
      }
      run += local[q];
    }
    if (lane == kWave - 1) *n_tiles = inc >= min_tiles ? inc : 0;
  } else if (wave == 2 && item_seg != nullptr) {
    // the GEMM decision of wave 1 (its tile total against min_tiles), then
    // the items of the segments it leaves to the streaming kernels
    int c[5];
    int tiles = 0;
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      const int seg = lane * 5 + q;
      c[q] = seg < nseg ? cnt[seg] : 0;
      tiles += c[q] > big_thr ? (c[q] + kBigTile - 1) / kBigTile : 0;
    }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) tiles += __shfl_xor(tiles, off);
    const bool gemm = tile_seg != nullptr && tiles > 0 && tiles >= min_tiles;
    int local[5];
    int sum = 0;
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      local[q] = (gemm && c[q] > big_thr) ? 0 : (c[q] + kStreamItemRows - 1) / kStreamItemRows;
      sum += local[q];
    }
    int inc = sum;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(inc, off);
      if (lane >= off) inc += o;
    }
    int run = inc - sum;
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      for (int i = 0; i < local[q]; ++i) {
        item_seg[run + i] = lane * 5 + q;
        item_row0[run + i] = i * kStreamItemRows;
      }
      run += local[q];
    }
    if (lane == kWave - 1) *n_items = inc;
  }
  __syncthreads();
}

// Sentinels at the tail of each segment, and the expert of each block.
__device__ void pad_segments(const int* cnt, const int* base, int nseg, int bm,
                             int32_t* sorted_ids, int32_t* block_expert, int32_t* seg_count) {
  for (int seg = threadIdx.x; seg < nseg; seg += blockDim.x) {
    const int c = cnt[seg];
    if (seg_count) seg_count[seg] = c;
    const int p = (c + bm - 1) / bm * bm;
    const int o = base[seg];
    for (int i = c; i < p; ++i) sorted_ids[o + i] = -1;
    for (int b = 0; b < p / bm; ++b) block_expert[o / bm + b] = seg;
  }
}

// Stable scatter of the assignments [a0, a1), chunk by chunk in flat order;
// base[seg] (LDS) is the next free position of each segment and advances.
// on_pos(a, pos, entry) receives each valid assignment's position in the
// sorted list and its entry (t * k + j; t * k for the shared slot).  A chunk
// of padding rows only is skipped.  wcnt must be zero on entry and is zero
// on exit.
template <typename OnPos>
__device__ void scatter_range(const int32_t* ids, int a0, int a1, int k, int kk, int E,
                              int nseg, int* base, int (*wcnt)[kMaxSeg], OnPos on_pos) {
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int chunk = a0; chunk < a1; chunk += kAlignThreads) {
    const int a = chunk + tid;
    const int e = a < a1 ? seg_of(ids, a, k, kk, E) : -1;
    const unsigned key = static_cast<unsigned>(e + 1);  // 0..257: 9 bits
    uint64_t same = ~0ull;
#pragma unroll
    for (int b = 0; b < 9; ++b) {
      const bool bit = (key >> b) & 1u;
      const uint64_t bal = __ballot(bit);
      same &= bit ? bal : ~bal;
    }
    const int rank = __popcll(same & lt_mask);
    if (e >= 0 && rank == 0) wcnt[wave][e] = __popcll(same);
    if (!__syncthreads_or(e >= 0)) continue;
    if (e >= 0) {
      int pre = 0;
      for (int w = 0; w < wave; ++w) pre += wcnt[w][e];
      const int t = a / kk, j = a - t * kk;
      on_pos(a, base[e] + pre + rank, t * k + (j < k ? j : 0));
    }
    __syncthreads();
    for (int seg = tid; seg < nseg; seg += kAlignThreads) {
      int s = 0;
      for (int w = 0; w < kAlignWaves; ++w) {
        s += wcnt[w][seg];
        wcnt[w][seg] = 0;
      }
      base[seg] += s;
    }
    __syncthreads();
  }
}

// on_pos of the align: the sorted list and each assignment's position in it
struct StoreSorted {
  int32_t* sorted_ids;
  int32_t* slot_pos;
  __device__ void operator()(int a, int pos, int entry) const {
    sorted_ids[pos] = entry;
    if (slot_pos) slot_pos[a] = pos;
  }
};

// One 1024-thread block for the whole list (small batches).
__global__ __launch_bounds__(kAlignThreads) void align_kernel(
    const int32_t* __restrict__ ids, int T, int k, int E, int ns, int bm,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ offsets, int32_t* __restrict__ n_post,
    int32_t* __restrict__ slot_pos, int32_t* __restrict__ seg_count, int big_thr, int min_tiles,
    int32_t* __restrict__ tile_seg, int32_t* __restrict__ tile_row0,
    int32_t* __restrict__ n_tiles, int32_t* __restrict__ item_seg,
    int32_t* __restrict__ item_row0, int32_t* __restrict__ n_items) {
  __shared__ int cnt[kMaxSeg];
  __shared__ int base[kMaxSeg];
  __shared__ int wcnt[kAlignWaves][kMaxSeg];
  const int tid = threadIdx.x;
  const int nseg = E + ns;
  const int kk = k + ns;
  const int n_assign = T * kk;

  for (int i = tid; i < kMaxSeg; i += kAlignThreads) cnt[i] = 0;
  for (int i = tid; i < kAlignWaves * kMaxSeg; i += kAlignThreads)
    (&wcnt[0][0])[i] = 0;
  __syncthreads();

  for (int a = tid; a < n_assign; a += kAlignThreads) {
    const int e = seg_of(ids, a, k, kk, E);
    if (e >= 0) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  scan_segments(cnt, base, nseg, bm, offsets, n_post, big_thr, min_tiles, tile_seg, tile_row0,
                n_tiles, item_seg, item_row0, n_items);
  pad_segments(cnt, base, nseg, bm, sorted_ids, block_expert, seg_count);
  scatter_range(ids, 0, n_assign, k, kk, E, nseg, base, wcnt, StoreSorted{sorted_ids, slot_pos});
}

// Large batches, three launches over kAlignSpan-assignment spans:
// 1. per-span segment counts -> span_cnt[span][seg];
// 2. one block: totals, the scan, tiles, sentinels, and each span's start
//    inside each segment -> span_cnt[span][seg] (overwritten);
// 3. per span: the stable scatter from those starts.
// Spans are in flat assignment order, so the result equals the one-block
// kernel's.
constexpr int kAlignSpan = 4 * kAlignThreads;

__global__ __launch_bounds__(kAlignThreads) void align_count_kernel(
    const int32_t* __restrict__ ids, int T, int k, int E, int ns,
    int32_t* __restrict__ span_cnt) {
  __shared__ int cnt[kMaxSeg];
  const int tid = threadIdx.x;
  const int nseg = E + ns, kk = k + ns, n_assign = T * kk;
  for (int i = tid; i < kMaxSeg; i += kAlignThreads) cnt[i] = 0;
  __syncthreads();
  const int a0 = blockIdx.x * kAlignSpan, a1 = min(n_assign, a0 + kAlignSpan);
  for (int a = a0 + tid; a < a1; a += kAlignThreads) {
    const int e = seg_of(ids, a, k, kk, E);
    if (e >= 0) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int seg = tid; seg < nseg; seg += kAlignThreads)
    span_cnt[(size_t)blockIdx.x * nseg + seg] = cnt[seg];
}

__global__ __launch_bounds__(kAlignThreads) void align_scan_kernel(
    int n_span, int E, int ns, int bm, int32_t* __restrict__ span_cnt,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ offsets, int32_t* __restrict__ n_post,
    int32_t* __restrict__ seg_count, int big_thr, int min_tiles,
    int32_t* __restrict__ tile_seg, int32_t* __restrict__ tile_row0,
    int32_t* __restrict__ n_tiles, int32_t* __restrict__ item_seg,
    int32_t* __restrict__ item_row0, int32_t* __restrict__ n_items) {
  __shared__ int cnt[kMaxSeg];
  __shared__ int base[kMaxSeg];
  const int tid = threadIdx.x;
  const int nseg = E + ns;
  // the spans' counts of a segment, loaded 8 at a time rather than one per
  // loop trip (the align of an 8192-row top-8 batch: 28.5 -> 24.3 us)
  constexpr int kSpanBatch = 8;
  for (int seg = tid; seg < nseg; seg += kAlignThreads) {
    int c = 0;
    for (int sp0 = 0; sp0 < n_span; sp0 += kSpanBatch) {
      int v[kSpanBatch];
#pragma unroll
      for (int q = 0; q < kSpanBatch; ++q)
        v[q] = sp0 + q < n_span ? span_cnt[(size_t)(sp0 + q) * nseg + seg] : 0;
#pragma unroll
      for (int q = 0; q < kSpanBatch; ++q) c += v[q];
    }
    cnt[seg] = c;
  }
  __syncthreads();
  scan_segments(cnt, base, nseg, bm, offsets, n_post, big_thr, min_tiles, tile_seg, tile_row0,
                n_tiles, item_seg, item_row0, n_items);
  pad_segments(cnt, base, nseg, bm, sorted_ids, block_expert, seg_count);
  // each span's first position in the segment, replacing its count
  for (int seg = tid; seg < nseg; seg += kAlignThreads) {
    int run = base[seg];
    for (int sp0 = 0; sp0 < n_span; sp0 += kSpanBatch) {
      int v[kSpanBatch];
#pragma unroll
      for (int q = 0; q < kSpanBatch; ++q)
        v[q] = sp0 + q < n_span ? span_cnt[(size_t)(sp0 + q) * nseg + seg] : 0;
#pragma unroll
      for (int q = 0; q < kSpanBatch; ++q) {
        if (sp0 + q < n_span) span_cnt[(size_t)(sp0 + q) * nseg + seg] = run;
        run += v[q];
      }
    }
  }
}

__global__ __launch_bounds__(kAlignThreads) void align_scatter_kernel(
    const int32_t* __restrict__ ids, int T, int k, int E, int ns,
    const int32_t* __restrict__ span_start, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ slot_pos) {
  __shared__ int base[kMaxSeg];
  __shared__ int wcnt[kAlignWaves][kMaxSeg];
  const int tid = threadIdx.x;
  const int nseg = E + ns, kk = k + ns, n_assign = T * kk;
  for (int seg = tid; seg < nseg; seg += kAlignThreads)
    base[seg] = span_start[(size_t)blockIdx.x * nseg + seg];
  for (int i = tid; i < kAlignWaves * kMaxSeg; i += kAlignThreads)
    (&wcnt[0][0])[i] = 0;
  __syncthreads();
  const int a0 = blockIdx.x * kAlignSpan, a1 = min(n_assign, a0 + kAlignSpan);
  scatter_range(ids, a0, a1, k, kk, E, nseg, base, wcnt, StoreSorted{sorted_ids, slot_pos});
}

}  // namespace

int align_spans(int T, int k, int n_shared) {
  const long long n = (long long)T * (k + n_shared);
  return n > 2 * kAlignSpan ? (int)((n + kAlignSpan - 1) / kAlignSpan) : 0;
}

hipError_t launch_align(const int32_t* ids, int T, int k, int E, int n_shared,
                        int bm, int32_t* sorted_ids, int32_t* block_expert,
                        int32_t* offsets, int32_t* n_post, int32_t* slot_pos,
                        int32_t* seg_count, int big_thr, int min_tiles, int32_t* tile_seg,
                        int32_t* tile_row0, int32_t* n_tiles, int32_t* span_buf,
                        int32_t* item_seg, int32_t* item_row0, int32_t* n_items,
                        hipStream_t s) {
  const int n_span = align_spans(T, k, n_shared);
  if (n_span == 0 || span_buf == nullptr) {
    hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kAlignThreads), 0, s, ids, T, k,
                       E, n_shared, bm, sorted_ids, block_expert, offsets, n_post,
                       slot_pos, seg_count, big_thr, min_tiles, tile_seg, tile_row0, n_tiles,
                       item_seg, item_row0, n_items);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(align_count_kernel, dim3(n_span), dim3(kAlignThreads), 0, s, ids, T, k, E,
                     n_shared, span_buf);
  hipLaunchKernelGGL(align_scan_kernel, dim3(1), dim3(kAlignThreads), 0, s, n_span, E, n_shared,
                     bm, span_buf, sorted_ids, block_expert, offsets, n_post, seg_count,
                     big_thr, min_tiles, tile_seg, tile_row0, n_tiles, item_seg, item_row0,
                     n_items);
  hipLaunchKernelGGL(align_scatter_kernel, dim3(n_span), dim3(kAlignThreads), 0, s, ids, T, k,
                     E, n_shared, span_buf, sorted_ids, slot_pos);
  return hipGetLastError();
}

}  // namespace moe
