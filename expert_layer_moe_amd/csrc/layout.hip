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

namespace moe {
namespace {

// Token rows of the streaming kernels in MFMA A-fragment order (frag_index):
// a wave then fetches a whole fragment as 1 KB contiguous, which leaves more
// of the memory system to the weight stream.  The down projection's input h
// is written in the same order by the gate/up kernel.
//
// xp tile t = x rows of the sorted rows 16 t .. 16 t + 15, for the tiles of
// segments left to the streaming kernels.  Padding rows are not written: an
// MFMA keeps the rows of its token operand apart, so whatever they hold only
// reaches output rows that are never stored.
// grid = (cap / 16, chunks of kpc steps).
__global__ __launch_bounds__(256) void pack_x_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ n_post,
    const int32_t* __restrict__ seg_cnt, int big_thr, const int32_t* __restrict__ gemm_tiles,
    uint16_t* __restrict__ xp, int H, int k, int kpc) {
  const int tile = blockIdx.x;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int m = lane % 16, g = lane / 16;
  // issued together (the slot is inside the list's capacity; past n_post it
  // holds a stale value that is never used): a short chain of dependent
  // loads matters in a kernel this small
  const int sid = sorted_ids[tile * 16 + m];
  if (tile * 16 >= *n_post) return;
  if (gemm_tiles != nullptr && seg_cnt[block_expert[tile]] > big_thr && *gemm_tiles > 0) return;
  const uint16_t* src = x + (size_t)(sid >= 0 ? sid / k : 0) * H + 8 * g;
  uint16_t* dst = xp + (size_t)tile * 16 * H + 8 * lane;
  const int s0 = blockIdx.y * kpc, s1 = min(H / 32, s0 + kpc);
  if (sid < 0) return;
#pragma unroll 8
  for (int s = s0 + wave; s < s1; s += 4)
    *reinterpret_cast<u32x4*>(dst + (size_t)s * 512) = ld16(src + 32 * s);
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

// fp32 y rows (y is read once: non-temporal loads)
template <int NV>
__global__ __launch_bounds__(256) void combine_kernel(
    const float* __restrict__ y, const int32_t* __restrict__ ids,
    const float* __restrict__ w, const int32_t* __restrict__ slot_pos, int T,
    int H, int k, int ns, void* __restrict__ out, int out_bf16) {
  const int t = blockIdx.x;
  const int kk = k + ns;
  int pos[kMaxSlots];
  float wt[kMaxSlots];
  const bool valid = combine_slots(ids, w, slot_pos, t, k, kk, pos, wt);
  // NV groups of 4 columns per thread, each group coalesced across the block;
  // all loads of a thread are issued before the sums
  int n[NV];
  floatx4 acc[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    n[v] = ((blockIdx.y * NV + v) * 256 + threadIdx.x) * 4;
    acc[v] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  if (valid) {
#pragma unroll
    for (int j = 0; j < kMaxSlots; ++j) {
      if (j < kk) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          if (n[v] < H) {
            const floatx4 val = __builtin_nontemporal_load(
                reinterpret_cast<const floatx4*>(y + (size_t)pos[j] * H + n[v]));
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

// bf16 y rows (fp8-weight layers), bf16 out: 8 columns per thread, 16-byte
// non-temporal y loads, all issued before the sums.
__global__ __launch_bounds__(256) void combine_ybf_kernel(
    const uint16_t* __restrict__ y, const int32_t* __restrict__ ids,
    const float* __restrict__ w, const int32_t* __restrict__ slot_pos, int H, int k, int ns,
    uint16_t* __restrict__ out) {
  const int t = blockIdx.x, kk = k + ns;
  const int n = (blockIdx.y * 256 + threadIdx.x) * 8;
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

}  // namespace

hipError_t launch_pack_x(const void* x, const int32_t* sorted_ids, const int32_t* block_expert,
                         const int32_t* n_post, const int32_t* seg_cnt, int big_thr,
                         const int32_t* gemm_tiles, void* xp, int H, int k, int bm,
                         int max_rows, hipStream_t s) {
  if (bm != 16 || H % 32 != 0) return hipErrorInvalidValue;
  const int kpc = 32;   // MFMA steps per block
  hipLaunchKernelGGL(pack_x_kernel, dim3(max_rows / 16, (H / 32 + kpc - 1) / kpc), dim3(256), 0,
                     s, static_cast<const uint16_t*>(x), sorted_ids, block_expert, n_post,
                     seg_cnt, big_thr, gemm_tiles, static_cast<uint16_t*>(xp), H, k, kpc);
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

hipError_t launch_combine(const void* y, bool y_bf16, const int32_t* ids, const float* w,
                          const int32_t* slot_pos, int T, int H, int k,
                          int n_shared, void* out, bool out_bf16,
                          hipStream_t s) {
  if (y_bf16) {
    if (!out_bf16 || H % 8 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(combine_ybf_kernel, dim3(T, (H + 2047) / 2048), dim3(256), 0, s,
                       static_cast<const uint16_t*>(y), ids, w, slot_pos, H, k, n_shared,
                       static_cast<uint16_t*>(out));
    return hipGetLastError();
  }
  const float* yf = static_cast<const float*>(y);
  // two 4-column groups per thread once there are rows enough to fill the chip
  if (T >= 256)
    hipLaunchKernelGGL(combine_kernel<2>, dim3(T, (H + 2047) / 2048), dim3(256), 0, s, yf, ids,
                       w, slot_pos, T, H, k, n_shared, out, out_bf16 ? 1 : 0);
  else
    hipLaunchKernelGGL(combine_kernel<1>, dim3(T, (H + 1023) / 1024), dim3(256), 0, s, yf, ids,
                       w, slot_pos, T, H, k, n_shared, out, out_bf16 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace moe
