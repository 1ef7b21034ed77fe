// Data movement around the expert kernels: token rows into MFMA fragment
// order, the one-time fragment packing of the expert weights, and the
// top-k-weighted combine of the per-assignment expert outputs.
//
// Combine: out[t] = sum_j w[t,j] y(t,j) plus the always-on shared expert
// ("Step3 Inference Optimization on AMD Instinct MI308X", optimisation list:
// shared-expert MLP fused in the layer; "[SGLang] Single Batch Overlap for MoE
// models": combine after the down-projection GEMM).
#include "moe_common.h"
#include "moe_kernels.h"

#include <algorithm>
#include <climits>

namespace moe {
namespace {

// Token rows of the streaming kernels in MFMA A-fragment order (frag_index):
// a wave then fetches a whole fragment as 1 KB contiguous, which leaves more
// of the memory system to the weight stream.  The down projection's input h
// is written in the same order by the gate/up kernel.
//
// xp tile t = x rows of the sorted rows 16 t .. 16 t + 15.  Padding rows are
// not written: an MFMA keeps the rows of its token operand apart, so whatever
// they hold only reaches output rows that are never stored.
// Serves calls where the tiled GEMM may take the large segments (calls where
// every segment streams read x directly): the work is the items of the
// streaming segments, driven by the streaming kernels' item table.  Units
// (item, 16-row tile of the item, chunk of kpc K steps), looped over by a
// capped grid.
__global__ __launch_bounds__(256) void pack_x_items_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ seg_off, const int32_t* __restrict__ seg_cnt,
    const int32_t* __restrict__ item_seg, const int32_t* __restrict__ item_row0,
    const int32_t* __restrict__ n_items, int max_items, uint16_t* __restrict__ xp, int H,
    int k, int kpc, int n_kc) {
  constexpr int kTiles = kStreamItemRows / 16;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int m = lane % 16, g = lane / 16;
  const int n_units = min(*n_items, max_items) * kTiles * n_kc;
  for (int u = blockIdx.x; u < n_units; u += gridDim.x) {
    const int item = u / (kTiles * n_kc), rest = u - item * (kTiles * n_kc);
    const int tt = rest / n_kc, kc = rest - tt * n_kc;
    const int e = item_seg[item];
    const int r0 = item_row0[item] + 16 * tt;   // first row of the tile in its segment
    if (r0 >= seg_cnt[e]) continue;
    const int tile = (seg_off[e] + r0) / 16;    // segments start on 16-row boundaries
    const int sid = sorted_ids[tile * 16 + m];
    if (sid < 0) continue;                      // a padding row of the segment
    const uint16_t* src = x + (size_t)(sid / k) * H + 8 * g;
    uint16_t* dst = xp + (size_t)tile * 16 * H + 8 * lane;
    const int s0 = kc * kpc, s1 = min(H / 32, s0 + kpc);
#pragma unroll 8
    for (int s = s0 + wave; s < s1; s += 4)
      *reinterpret_cast<u32x4*>(dst + (size_t)s * 512) = ld16(src + 32 * s);
  }
}

// Token rows as two e4m3 terms for the fp8-MFMA gate/up GEMM: with one
// power-of-two scale per row, s = 2^(e - 8) where max_h |x[t,h]| = m 2^e
// (m in [0.5, 1); s = 1 for a zero row), every |x / s| is below 256;
// hi = e4m3(x / s) and lo = e4m3(x / s - hi), both rounded to nearest even,
// so x = s (hi + lo) up to the part of x / s - hi below e4m3's resolution
// (a bf16 value carries 8 significant bits, hi and lo 4 each).  Planes
// xq[0..T*H) (hi) and xq[T*H..2*T*H) (lo), row-major; sx[t] = s.  Padding
// rows are neither read nor written.  One wave per row, two passes over it
// (the second from cache).
__global__ __launch_bounds__(256) void xq_split_kernel(const uint16_t* __restrict__ x,
                                                       const uint8_t* __restrict__ valid,
                                                       uint8_t* __restrict__ xq,
                                                       float* __restrict__ sx, int T, int H) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T || (valid != nullptr && valid[t] == 0)) return;
  const uint16_t* row = x + (size_t)t * H;
  float amax = 0.f;
  for (int p = lane; p < H / 8; p += kWave) {
    const u32x4 v = ld16(row + 8 * p);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      amax = fmaxf(amax, fabsf(__uint_as_float(v[q] << 16)));
      amax = fmaxf(amax, fabsf(__uint_as_float(v[q] & 0xffff0000u)));
    }
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  int e = 0;
  (void)frexpf(amax, &e);
  const bool zero = !(amax > 0.f);
  const float inv = zero ? 1.f : ldexpf(1.f, 8 - e);   // 1 / s, exact
  if (lane == 0) sx[t] = zero ? 1.f : ldexpf(1.f, e - 8);
  uint8_t* hi = xq + (size_t)t * H;
  uint8_t* lo = hi + (size_t)T * H;
  for (int p = lane; p < H / 8; p += kWave) {
    const u32x4 v = ld16(row + 8 * p);
    float f[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f[2 * q] = __uint_as_float(v[q] << 16) * inv;
      f[2 * q + 1] = __uint_as_float(v[q] & 0xffff0000u) * inv;
    }
    int ch[2], cl[2];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      int c = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * w], f[4 * w + 1], 0, false);
      ch[w] = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * w + 2], f[4 * w + 3], c, true);
      const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(ch[w], false);
      const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8(ch[w], true);
      c = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * w] - h01[0], f[4 * w + 1] - h01[1], 0, false);
      cl[w] = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * w + 2] - h23[0], f[4 * w + 3] - h23[1], c, true);
    }
    *reinterpret_cast<u32x2*>(hi + 8 * p) = u32x2{(uint32_t)ch[0], (uint32_t)ch[1]};
    *reinterpret_cast<u32x2*>(lo + 8 * p) = u32x2{(uint32_t)cl[0], (uint32_t)cl[1]};
  }
}

// Weights in MFMA B-fragment order (the same tile / step / lane order as
// frag_index, over a [rows, K] matrix): block (16-row tile t, K step s) of
// 512 elements at (t * K/32 + s) * 512, lane 16 g + m holding row 16 t + m,
// columns 32 s + 8 g .. + 7.  One thread moves one lane's 8 elements
// (ESZ bytes each).
template <int ESZ>
__global__ __launch_bounds__(256) void pack_frag_kernel(const uint8_t* __restrict__ src,
                                                        uint8_t* __restrict__ dst,
                                                        size_t n_lanes, int K) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_lanes) return;
  const int lane = (int)(i & 63);
  const size_t blk = i >> 6;
  const size_t steps = (size_t)K / 32;
  const size_t t = blk / steps, st = blk - t * steps;
  const size_t row = t * 16 + (lane & 15);
  const size_t col = st * 32 + 8 * (lane >> 4);
  const uint8_t* p = src + (row * K + col) * ESZ;
  if constexpr (ESZ == 2)
    *reinterpret_cast<u32x4*>(dst + i * 16) = *reinterpret_cast<const u32x4*>(p);
  else
    *reinterpret_cast<u32x2*>(dst + i * 8) = *reinterpret_cast<const u32x2*>(p);
}

// Combine: one block per token row; fp32 sum over the k routed slots in slot
// order, then the shared expert, rounded once.  Padding rows -> 0.  y rows
// are fp32, or bf16 (YB) in fp8-weight layers.
constexpr int kMaxSlots = 17;

// Slot positions and weights of row t (shared slot: weight 1), loaded
// together with its id (a padding row's positions are stale and never used);
// false for a padding row.
__device__ __forceinline__ bool combine_slots(const int32_t* ids, const float* w,
                                              const int32_t* slot_pos, int t, int k, int kk,
                                              int (&pos)[kMaxSlots], float (&wt)[kMaxSlots]) {
  const bool valid = ids[(size_t)t * k] >= 0;
#pragma unroll
  for (int j = 0; j < kMaxSlots; ++j) {
    pos[j] = j < kk ? slot_pos[(size_t)t * kk + j] : 0;
    wt[j] = j < k ? w[(size_t)t * k + j] : 1.f;
  }
  return valid;
}

// Wave 0 of a waiting combine block: wait until the completion counters of
// the blocks that hold the assignments of rows [t0, t1) (padding rows have
// none) reach cw.target, then acquire at agent scope, so that the y rows the
// producers stored before their release are the ones read.  Lane l polls
// pairs (row, slot) l, l + 64, ...; the shared slot's block is in segment E.
// False when the wait ran out of time or an earlier one did.
__device__ bool wait_rows(const CombineWait& cw, const int32_t* ids, const int32_t* slot_pos,
                          int t0, int t1, int k, int kk) {
  const int lane = threadIdx.x;
  const int n_pairs = (t1 - t0) * kk;
  const uint64_t start = __builtin_amdgcn_s_memrealtime();
  for (int q0 = 0; q0 < n_pairs; q0 += kWave) {
    const int q = q0 + lane;
    const int32_t* c = nullptr;
    if (q < n_pairs) {
      const int t = t0 + q / kk, j = q % kk;
      if (ids[(size_t)t * k] >= 0) {
        const int e = j < k ? ids[(size_t)t * k + j] : cw.E;
        const int p = slot_pos[(size_t)t * kk + j];
        c = cw.sig + (size_t)e * cw.nb64 + ((p - cw.seg_off[e]) >> 6);
      }
    }
    for (;;) {
      const bool ready =
          c == nullptr ||
          __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= cw.target;
      if (__all(ready)) break;
      if (__any(__hip_atomic_load(cw.giveup, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0))
        return false;
      if (__builtin_amdgcn_s_memrealtime() - start > (uint64_t)cw.ticks) {
        if (lane == 0)
          __hip_atomic_store(cw.giveup, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return false;
      }
      __builtin_amdgcn_s_sleep(8);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return true;
}

// The waiting combine runs as a persistent grid of at most kWaitGrid blocks
// (one per CU), each taking groups of rows in row order, T / kWaitGrid rows
// per group but at least one and at most kWaitRows: one wait and one acquire
// per group.  A block per (row, column chunk), as the other
// modes launch, filled every CU slot with waiting blocks and starved the
// down kernels they wait for (prefill micro-batch: down GEMM 375 us -> 10 ms,
// until the waits ran out); an acquire per row invalidated the L2 so often
// that the down GEMM, whose tiles share W2 through it, ran at half speed.
constexpr int kWaitGrid = 256;
constexpr int kWaitRows = 32;
__host__ __device__ inline int wait_group_rows(int T) {
  return T / kWaitGrid < 1 ? 1 : (T / kWaitGrid > kWaitRows ? kWaitRows : T / kWaitGrid);
}

// Called by every thread of a COMBINE_WAIT block: true when the block may
// combine rows [t0, t1).  The caller passes a barrier before the next call.
__device__ bool wait_group(const CombineWait& cw, const int32_t* ids, const int32_t* slot_pos,
                           int t0, int t1, int k, int kk) {
  __shared__ int s_ok;
  if (threadIdx.x < kWave) {
    const bool ok = wait_rows(cw, ids, slot_pos, t0, t1, k, kk);
    if (threadIdx.x == 0) s_ok = ok ? 1 : 0;
  }
  __syncthreads();
  return s_ok != 0;
}

// The persistent loop of the waiting combine: part(t, by) combines column
// chunk by of row t; done flags are set for the rows combined.
template <typename Part>
__device__ __forceinline__ void wait_and_combine(const CombineWait& cw, const int32_t* ids,
                                                 const int32_t* slot_pos, int T, int k, int kk,
                                                 int gy, Part part) {
  const int rows = wait_group_rows(T);
  for (int t0 = blockIdx.x * rows; t0 < T; t0 += gridDim.x * rows) {
    const int t1 = min(T, t0 + rows);
    if (wait_group(cw, ids, slot_pos, t0, t1, k, kk)) {
      for (int t = t0; t < t1; ++t)
        for (int by = 0; by < gy; ++by) part(t, by);
      for (int i = threadIdx.x; i < (t1 - t0) * gy; i += blockDim.x)
        cw.done[(size_t)t0 * gy + i] = 1;
    }
    __syncthreads();
  }
}

// fp32 y rows, or 24-bit ones (Y24); y is read once: non-temporal loads.
// Part `by` of the gy column chunks of row t; MODE: COMBINE_ALL, or
// COMBINE_REST (skip a part whose done flag is set).
template <int NV, bool Y24, int MODE>
__device__ __forceinline__ void combine_part(
    const void* __restrict__ y, const int32_t* __restrict__ ids,
    const float* __restrict__ w, const int32_t* __restrict__ slot_pos,
    int H, int k, int ns, void* __restrict__ out, int out_bf16, const CombineWait& cw, int t,
    int by, int gy) {
  const int kk = k + ns;
  if constexpr (MODE == COMBINE_REST) {
    if (cw.done[(size_t)t * gy + by] != 0) return;
  }
  int pos[kMaxSlots];
  float wt[kMaxSlots];
  const bool valid = combine_slots(ids, w, slot_pos, t, k, kk, pos, wt);
  // NV groups of 4 columns per thread, each group coalesced across the block;
  // all loads of a thread are issued before the sums
  int n[NV];
  floatx4 acc[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    n[v] = ((by * NV + v) * 256 + threadIdx.x) * 4;
    acc[v] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  if (valid) {
#pragma unroll
    for (int j = 0; j < kMaxSlots; ++j) {
      if (j < kk) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          if (n[v] < H) {
            const size_t yi = (size_t)pos[j] * H + n[v];
            floatx4 val;
            if constexpr (Y24)
              val = unpack_y24(__builtin_nontemporal_load(
                  reinterpret_cast<const u32x3*>(static_cast<const uint8_t*>(y) + yi * 3)));
            else
              val = __builtin_nontemporal_load(
                  reinterpret_cast<const floatx4*>(static_cast<const float*>(y) + yi));
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[v][i] = fmaf(wt[j], val[i], acc[v][i]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    if (n[v] >= H) continue;
    if (out_bf16) {
      uint16_t* o = static_cast<uint16_t*>(out) + (size_t)t * H + n[v];
      u32x2 pk;
      pk[0] = (uint32_t)f32_to_bf16_bits(acc[v][0]) | ((uint32_t)f32_to_bf16_bits(acc[v][1]) << 16);
      pk[1] = (uint32_t)f32_to_bf16_bits(acc[v][2]) | ((uint32_t)f32_to_bf16_bits(acc[v][3]) << 16);
      *reinterpret_cast<u32x2*>(o) = pk;
    } else {
      *reinterpret_cast<floatx4*>(static_cast<float*>(out) + (size_t)t * H + n[v]) = acc[v];
    }
  }
}

template <int NV, bool Y24, int MODE>
__global__ __launch_bounds__(256) void combine_kernel(
    const void* __restrict__ y, const int32_t* __restrict__ ids,
    const float* __restrict__ w, const int32_t* __restrict__ slot_pos, int T,
    int H, int k, int ns, void* __restrict__ out, int out_bf16, CombineWait cw, int gy) {
  if constexpr (MODE == COMBINE_WAIT) {
    wait_and_combine(cw, ids, slot_pos, T, k, k + ns, gy, [&](int t, int by) {
      combine_part<NV, Y24, COMBINE_ALL>(y, ids, w, slot_pos, H, k, ns, out, out_bf16, cw, t,
                                         by, gy);
    });
  } else {
    combine_part<NV, Y24, MODE>(y, ids, w, slot_pos, H, k, ns, out, out_bf16, cw, blockIdx.x,
                                blockIdx.y, gridDim.y);
  }
}

// bf16 y rows (fp8-weight layers), bf16 out: 8 columns per thread, 16-byte
// non-temporal y loads, all issued before the sums.  Part `by` of the gy
// column chunks of row t; MODE: COMBINE_ALL or COMBINE_REST.
template <int MODE>
__device__ __forceinline__ void combine_ybf_part(
    const uint16_t* __restrict__ y, const int32_t* __restrict__ ids,
    const float* __restrict__ w, const int32_t* __restrict__ slot_pos, int H, int k, int ns,
    uint16_t* __restrict__ out, const CombineWait& cw, int t, int by, int gy) {
  const int kk = k + ns;
  const int n = (by * 256 + threadIdx.x) * 8;
  if constexpr (MODE == COMBINE_REST) {
    if (cw.done[(size_t)t * gy + by] != 0) return;
  }

  if (n >= H) return;   // H % 8 == 0: a thread's 8 columns are all in range
  int pos[kMaxSlots];
  float wt[kMaxSlots];
  const bool valid = combine_slots(ids, w, slot_pos, t, k, kk, pos, wt);
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  if (valid) {
    u32x4 val[kMaxSlots];
#pragma unroll
    for (int j = 0; j < kMaxSlots; ++j)
      if (j < kk)
        val[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(y + (size_t)pos[j] * H + n));
#pragma unroll
    for (int j = 0; j < kMaxSlots; ++j) {
      if (j < kk) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = fmaf(wt[j], __uint_as_float(val[j][q] << 16), acc[2 * q]);
          acc[2 * q + 1] = fmaf(wt[j], __uint_as_float(val[j][q] & 0xffff0000u), acc[2 * q + 1]);
        }
      }
    }
  }
  u32x4 pk;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    pk[q] = (uint32_t)f32_to_bf16_bits(acc[2 * q]) | ((uint32_t)f32_to_bf16_bits(acc[2 * q + 1]) << 16);
  *reinterpret_cast<u32x4*>(out + (size_t)t * H + n) = pk;
}

template <int MODE>
__global__ __launch_bounds__(256) void combine_ybf_kernel(
    const uint16_t* __restrict__ y, const int32_t* __restrict__ ids,
    const float* __restrict__ w, const int32_t* __restrict__ slot_pos, int T, int H, int k,
    int ns, uint16_t* __restrict__ out, CombineWait cw, int gy) {
  if constexpr (MODE == COMBINE_WAIT) {
    wait_and_combine(cw, ids, slot_pos, T, k, k + ns, gy, [&](int t, int by) {
      combine_ybf_part<COMBINE_ALL>(y, ids, w, slot_pos, H, k, ns, out, cw, t, by, gy);
    });
  } else {
    combine_ybf_part<MODE>(y, ids, w, slot_pos, H, k, ns, out, cw, blockIdx.x, blockIdx.y,
                           gridDim.y);
  }
}

}  // namespace

hipError_t launch_pack_x_items(const void* x, const int32_t* sorted_ids, const int32_t* seg_off,
                               const int32_t* seg_cnt, const int32_t* item_seg,
                               const int32_t* item_row0, const int32_t* n_items, int max_items,
                               void* xp, int H, int k, hipStream_t s) {
  if (H % 32 != 0 || max_items < 0) return hipErrorInvalidValue;
  const int kpc = 32;   // MFMA steps per unit
  const int n_kc = (H / 32 + kpc - 1) / kpc;
  // the largest grid the chip holds at once, or less when fewer units can exist
  constexpr int kPackItemsGrid = 2048;
  const long long bound = (long long)max_items * (kStreamItemRows / 16) * n_kc;
  const int grid = (int)std::max(1LL, std::min<long long>(bound, kPackItemsGrid));
  hipLaunchKernelGGL(pack_x_items_kernel, dim3(grid), dim3(256), 0, s,
                     static_cast<const uint16_t*>(x), sorted_ids, seg_off, seg_cnt, item_seg,
                     item_row0, n_items, max_items, static_cast<uint16_t*>(xp), H, k, kpc, n_kc);
  return hipGetLastError();
}

hipError_t launch_xq_split(const void* x, const uint8_t* valid, uint8_t* xq, float* sx, int T,
                           int H, hipStream_t s) {
  if (H % 8 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(xq_split_kernel, dim3((T + 3) / 4), dim3(256), 0, s,
                     static_cast<const uint16_t*>(x), valid, xq, sx, T, H);
  return hipGetLastError();
}

hipError_t launch_pack_weights(int wkind, const void* src, void* dst, size_t rows, int K,
                               hipStream_t s) {
  if (wkind == W_F32 || rows % 16 != 0 || K % 32 != 0) return hipErrorInvalidValue;
  const size_t n_lanes = rows * (size_t)K / 8;
  const size_t blocks = (n_lanes + 255) / 256;
  if (blocks > 0x7fffffffu) return hipErrorInvalidValue;
  if (wkind == W_BF16)
    hipLaunchKernelGGL(pack_frag_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), n_lanes, K);
  else
    hipLaunchKernelGGL(pack_frag_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), n_lanes, K);
  return hipGetLastError();
}

int combine_grid_y(int T, int H, int yfmt) {
  if (yfmt == Y_BF16) return (H + 2047) / 2048;
  const int nv = T >= 2048 ? 8 : (T >= 256 ? 2 : 1);
  return (H + 1024 * nv - 1) / (1024 * nv);
}

hipError_t launch_combine(const void* y, int yfmt, const int32_t* ids, const float* w,
                          const int32_t* slot_pos, int T, int H, int k,
                          int n_shared, void* out, bool out_bf16,
                          hipStream_t s, int mode, const CombineWait* cw) {
  if (mode != COMBINE_ALL && cw == nullptr) return hipErrorInvalidValue;
  const CombineWait cwv = cw != nullptr ? *cw : CombineWait{};
  const int gy = combine_grid_y(T, H, yfmt);
  if ((long long)T * gy > INT_MAX) return hipErrorInvalidValue;
  // the waiting combine: a persistent grid over groups of rows
  const int groups = (T + wait_group_rows(T) - 1) / wait_group_rows(T);
  const dim3 grid = mode == COMBINE_WAIT ? dim3(std::min(groups, kWaitGrid)) : dim3(T, gy);
  if (yfmt == Y_BF16) {
    if (!out_bf16 || H % 8 != 0) return hipErrorInvalidValue;
#define MOE_COMBINE_BF(MODE)                                                                  \
  hipLaunchKernelGGL(combine_ybf_kernel<MODE>, grid, dim3(256), 0, s,                          \
                     static_cast<const uint16_t*>(y), ids, w, slot_pos, T, H, k, n_shared,      \
                     static_cast<uint16_t*>(out), cwv, gy)
    if (mode == COMBINE_WAIT) MOE_COMBINE_BF(COMBINE_WAIT);
    else if (mode == COMBINE_REST) MOE_COMBINE_BF(COMBINE_REST);
    else MOE_COMBINE_BF(COMBINE_ALL);
#undef MOE_COMBINE_BF
    return hipGetLastError();
  }
  if (yfmt != Y_F32 && yfmt != Y_F24) return hipErrorInvalidValue;
  // two 4-column groups per thread once there are rows enough to fill the
  // chip; on large batches one block per row (up to 8192 columns): a quarter
  // of the blocks, each with 4x the loads in flight (gather_padded_e48, 86%
  // padding rows that only take zeros: 57.8 -> 50.5 us)
  const int ob = out_bf16 ? 1 : 0;
#define MOE_COMBINE(NV, Y24, MODE)                                                            \
  hipLaunchKernelGGL((combine_kernel<NV, Y24, MODE>), grid, dim3(256), 0, s, y, ids, w,         \
                     slot_pos, T, H, k, n_shared, out, ob, cwv, gy)
#define MOE_COMBINE_M(NV, Y24)                                                               \
  if (mode == COMBINE_WAIT) MOE_COMBINE(NV, Y24, COMBINE_WAIT);                               \
  else if (mode == COMBINE_REST) MOE_COMBINE(NV, Y24, COMBINE_REST);                          \
  else MOE_COMBINE(NV, Y24, COMBINE_ALL)
  const bool y24 = yfmt == Y_F24;
  if (T >= 2048) {
    if (y24) { MOE_COMBINE_M(8, true); } else { MOE_COMBINE_M(8, false); }
  } else if (T >= 256) {
    if (y24) { MOE_COMBINE_M(2, true); } else { MOE_COMBINE_M(2, false); }
  } else {
    if (y24) { MOE_COMBINE_M(1, true); } else { MOE_COMBINE_M(1, false); }
  }
#undef MOE_COMBINE_M
#undef MOE_COMBINE
  return hipGetLastError();
}

namespace {
// Zero two int32 ranges.
__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t* __restrict__ a, size_t na,
                                                       int32_t* __restrict__ b, size_t nb) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < na + nb; i += stride) {
    if (i < na) a[i] = 0;
    else b[i - na] = 0;
  }
}
}  // namespace

hipError_t launch_zero_i32(int32_t* a, size_t na, int32_t* b, size_t nb, hipStream_t s) {
  const size_t n = na + nb;
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<size_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(zero_i32_kernel, dim3(grid), dim3(256), 0, s, a, na, b, nb);
  return hipGetLastError();
}

}  // namespace moe
