// Expert grouped GEMMs and the weighted combine.
//
// gate/up: h = SiLU(W_gate x) * (W_up x) per sorted row (the expert MLP of a
// sparse MoE layer, "AMD Instinct MI355X: ATOM ...": sparse MoE experts,
// block-scale GEMMs); down: y = W2 h ("[SGLang] Single Batch Overlap for MoE
// models": the down-projection GEMM); combine: out[t] = sum_j w[t,j] y(t,j)
// plus the always-on shared expert ("Step3 Inference Optimization on AMD
// Instinct MI308X", optimisation list: shared-expert MLP fused in the layer).
//
// fp8 weights (same list: FP8 blockscale) are OCP e4m3fn codes with one fp32
// scale per 128x128 block; codes become bf16 exactly, MFMA accumulates each
// 128-wide K block separately, and the block's scale multiplies that partial
// sum in fp32 before it joins the accumulator.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {
namespace {

constexpr int kBM = 32;  // rows per block in the MFMA kernels

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x2 ld8(const void* p) {
  return *reinterpret_cast<const u32x2*>(p);
}

template <bool FP8>
__device__ __forceinline__ bf16x8 load_w8(const void* base, size_t elem_off) {
  if constexpr (FP8) {
    const u32x2 v = ld8(static_cast<const uint8_t*>(base) + elem_off);
    return fp8x8_to_bf16x8(v[0], v[1]);
  } else {
    return as_bf16x8(ld16(static_cast<const uint16_t*>(base) + elem_off));
  }
}

// Gate/up: block = kBM sorted rows of one expert x 32 intermediate columns
// (32 gate + the matching 32 up rows of W13).  4 waves in a 2x2 grid, each a
// 16-row x 16-column tile of both gate and up.  grid = (max_blocks, I/32).
template <bool FP8>
__global__ __launch_bounds__(256) void gate_up_mfma_kernel(
    const uint16_t* __restrict__ x, const void* __restrict__ w13,
    const float* __restrict__ s13, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ n_post,
    uint16_t* __restrict__ h, int H, int I, int k) {
  const int b = blockIdx.x;
  if (b * kBM >= *n_post) return;
  const int e = block_expert[b];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int wr = wave >> 1, wc = wave & 1;
  const int m = lane % 16, g = lane / 16;
  const int r = b * kBM + wr * 16 + m;
  const int sid = sorted_ids[r];
  const int tok = sid >= 0 ? sid / k : -1;
  const int c0 = blockIdx.y * 32 + wc * 16;  // first gate column of this wave
  const uint16_t* xa = x + (size_t)(tok >= 0 ? tok : 0) * H + 8 * g;
  const size_t wg_off = ((size_t)e * 2 * I + c0 + m) * H + 8 * g;
  const size_t wu_off = wg_off + (size_t)I * H;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  floatx4 accg = {0.f, 0.f, 0.f, 0.f}, accu = accg;
  if constexpr (!FP8) {
#pragma unroll 4
    for (int kk = 0; kk < H; kk += 32) {
      const bf16x8 a = as_bf16x8(tok >= 0 ? ld16(xa + kk) : zero);
      accg = mfma16x16x32(a, load_w8<false>(w13, wg_off + kk), accg);
      accu = mfma16x16x32(a, load_w8<false>(w13, wu_off + kk), accu);
    }
  } else {
    const int nkb = H / 128;
    const float* sg = s13 + ((size_t)e * (2 * I / 128) + c0 / 128) * nkb;
    const float* su = s13 + ((size_t)e * (2 * I / 128) + (I + c0) / 128) * nkb;
    for (int kb = 0; kb < nkb; ++kb) {
      floatx4 pg = {0.f, 0.f, 0.f, 0.f}, pu = pg;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int kk = kb * 128 + q * 32;
        const bf16x8 a = as_bf16x8(tok >= 0 ? ld16(xa + kk) : zero);
        pg = mfma16x16x32(a, load_w8<true>(w13, wg_off + kk), pg);
        pu = mfma16x16x32(a, load_w8<true>(w13, wu_off + kk), pu);
      }
      const float scg = sg[kb], scu = su[kb];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        accg[i] = fmaf(scg, pg[i], accg[i]);
        accu[i] = fmaf(scu, pu[i], accu[i]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = b * kBM + wr * 16 + 4 * g + i;
    h[(size_t)row * I + c0 + m] = f32_to_bf16_bits(silu_mul(accg[i], accu[i]));
  }
}

// Down: block = kBM sorted rows x 64 output columns; 4 waves in a 2x2 grid,
// each 16 rows x 32 columns (two MFMA tiles).  grid = (max_blocks, H/64).
template <bool FP8>
__global__ __launch_bounds__(256) void down_mfma_kernel(
    const uint16_t* __restrict__ h, const void* __restrict__ w2,
    const float* __restrict__ s2, const int32_t* __restrict__ block_expert,
    const int32_t* __restrict__ n_post, float* __restrict__ y, int H, int I) {
  const int b = blockIdx.x;
  if (b * kBM >= *n_post) return;
  const int e = block_expert[b];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int wr = wave >> 1, wc = wave & 1;
  const int m = lane % 16, g = lane / 16;
  const int r = b * kBM + wr * 16 + m;
  const uint16_t* ha = h + (size_t)r * I + 8 * g;
  const int n0 = blockIdx.y * 64 + wc * 32;
  const size_t w0 = ((size_t)e * H + n0 + m) * I + 8 * g;
  const size_t w1 = w0 + (size_t)16 * I;
  floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  if constexpr (!FP8) {
#pragma unroll 4
    for (int kk = 0; kk < I; kk += 32) {
      const bf16x8 a = as_bf16x8(ld16(ha + kk));
      acc0 = mfma16x16x32(a, load_w8<false>(w2, w0 + kk), acc0);
      acc1 = mfma16x16x32(a, load_w8<false>(w2, w1 + kk), acc1);
    }
  } else {
    const int nkb = I / 128;
    const float* sc = s2 + ((size_t)e * (H / 128) + n0 / 128) * nkb;
    for (int kb = 0; kb < nkb; ++kb) {
      floatx4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = p0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int kk = kb * 128 + q * 32;
        const bf16x8 a = as_bf16x8(ld16(ha + kk));
        p0 = mfma16x16x32(a, load_w8<true>(w2, w0 + kk), p0);
        p1 = mfma16x16x32(a, load_w8<true>(w2, w1 + kk), p1);
      }
      const float s = sc[kb];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc0[i] = fmaf(s, p0[i], acc0[i]);
        acc1[i] = fmaf(s, p1[i], acc1[i]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const size_t row = (size_t)(b * kBM + wr * 16 + 4 * g + i);
    y[row * H + n0 + m] = acc0[i];
    y[row * H + n0 + 16 + m] = acc1[i];
  }
}

// fp32 layers (small): one block per sorted row, plain FMA loops.
__global__ __launch_bounds__(256) void gate_up_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ w13,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ block_expert,
    const int32_t* __restrict__ n_post, float* __restrict__ h, int H, int I,
    int k, int bm) {
  const int r = blockIdx.x;
  if (r >= *n_post) return;
  const int sid = sorted_ids[r];
  const int e = block_expert[r / bm];
  for (int c = threadIdx.x; c < I; c += blockDim.x) {
    float gs = 0.f, us = 0.f;
    if (sid >= 0) {
      const float* xp = x + (size_t)(sid / k) * H;
      const float* wg = w13 + ((size_t)e * 2 * I + c) * H;
      const float* wu = wg + (size_t)I * H;
      for (int i = 0; i < H; ++i) {
        gs = fmaf(xp[i], wg[i], gs);
        us = fmaf(xp[i], wu[i], us);
      }
    }
    h[(size_t)r * I + c] = silu_mul(gs, us);
  }
}

__global__ __launch_bounds__(256) void down_f32_kernel(
    const float* __restrict__ h, const float* __restrict__ w2,
    const int32_t* __restrict__ block_expert, const int32_t* __restrict__ n_post,
    float* __restrict__ y, int H, int I, int bm) {
  const int r = blockIdx.x;
  if (r >= *n_post) return;
  const int e = block_expert[r / bm];
  const float* hp = h + (size_t)r * I;
  for (int n = threadIdx.x; n < H; n += blockDim.x) {
    const float* wp = w2 + ((size_t)e * H + n) * I;
    float s = 0.f;
    for (int i = 0; i < I; ++i) s = fmaf(hp[i], wp[i], s);
    y[(size_t)r * H + n] = s;
  }
}

// Combine: one block per token row; fp32 sum over the k routed slots in slot
// order, then the shared expert, rounded once.  Padding rows -> 0.
constexpr int kMaxSlots = 17;

__global__ __launch_bounds__(256) void combine_kernel(
    const float* __restrict__ y, const int32_t* __restrict__ ids,
    const float* __restrict__ w, const int32_t* __restrict__ slot_pos, int T,
    int H, int k, int ns, void* __restrict__ out, int out_bf16) {
  const int t = blockIdx.x;
  const bool valid = ids[(size_t)t * k] >= 0;
  const int kk = k + ns;
  int pos[kMaxSlots];
  float wt[kMaxSlots];
#pragma unroll
  for (int j = 0; j < kMaxSlots; ++j) {
    pos[j] = (valid && j < kk) ? slot_pos[(size_t)t * kk + j] : 0;
    wt[j] = (valid && j < k) ? w[(size_t)t * k + j] : 1.f;
  }
  for (int n = threadIdx.x * 4; n < H; n += blockDim.x * 4) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    if (valid) {
#pragma unroll
      for (int j = 0; j < kMaxSlots; ++j) {
        if (j < kk) {
          const floatx4 v = *reinterpret_cast<const floatx4*>(y + (size_t)pos[j] * H + n);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] = fmaf(wt[j], v[i], acc[i]);
        }
      }
    }
    if (out_bf16) {
      uint16_t* o = static_cast<uint16_t*>(out) + (size_t)t * H + n;
      u32x2 pk;
      pk[0] = (uint32_t)f32_to_bf16_bits(acc[0]) | ((uint32_t)f32_to_bf16_bits(acc[1]) << 16);
      pk[1] = (uint32_t)f32_to_bf16_bits(acc[2]) | ((uint32_t)f32_to_bf16_bits(acc[3]) << 16);
      *reinterpret_cast<u32x2*>(o) = pk;
    } else {
      *reinterpret_cast<floatx4*>(static_cast<float*>(out) + (size_t)t * H + n) = acc;
    }
  }
}

}  // namespace

hipError_t launch_gate_up(int wkind, const void* x, const void* w13,
                          const float* s13, const int32_t* sorted_ids,
                          const int32_t* block_expert, const int32_t* n_post,
                          void* h, int H, int I, int k, int bm, int max_rows,
                          hipStream_t s) {
  if (wkind == W_F32) {
    hipLaunchKernelGGL(gate_up_f32_kernel, dim3(max_rows), dim3(256), 0, s,
                       static_cast<const float*>(x), static_cast<const float*>(w13),
                       sorted_ids, block_expert, n_post, static_cast<float*>(h), H, I,
                       k, bm);
    return hipGetLastError();
  }
  if (bm != kBM) return hipErrorInvalidValue;
  dim3 grid(max_rows / kBM, I / 32);
  if (wkind == W_FP8)
    hipLaunchKernelGGL(gate_up_mfma_kernel<true>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(x), w13, s13, sorted_ids,
                       block_expert, n_post, static_cast<uint16_t*>(h), H, I, k);
  else
    hipLaunchKernelGGL(gate_up_mfma_kernel<false>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(x), w13, s13, sorted_ids,
                       block_expert, n_post, static_cast<uint16_t*>(h), H, I, k);
  return hipGetLastError();
}

hipError_t launch_down(int wkind, const void* h, const void* w2, const float* s2,
                       const int32_t* block_expert, const int32_t* n_post,
                       float* y, int H, int I, int bm, int max_rows,
                       hipStream_t s) {
  if (wkind == W_F32) {
    hipLaunchKernelGGL(down_f32_kernel, dim3(max_rows), dim3(256), 0, s,
                       static_cast<const float*>(h), static_cast<const float*>(w2),
                       block_expert, n_post, y, H, I, bm);
    return hipGetLastError();
  }
  if (bm != kBM) return hipErrorInvalidValue;
  dim3 grid(max_rows / kBM, H / 64);
  if (wkind == W_FP8)
    hipLaunchKernelGGL(down_mfma_kernel<true>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(h), w2, s2, block_expert, n_post,
                       y, H, I);
  else
    hipLaunchKernelGGL(down_mfma_kernel<false>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(h), w2, s2, block_expert, n_post,
                       y, H, I);
  return hipGetLastError();
}

hipError_t launch_combine(const float* y, const int32_t* ids, const float* w,
                          const int32_t* slot_pos, int T, int H, int k,
                          int n_shared, void* out, bool out_bf16,
                          hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel, dim3(T), dim3(256), 0, s, y, ids, w, slot_pos,
                     T, H, k, n_shared, out, out_bf16 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace moe
