// Router: logits, then top-k with softmax over the selected logits.
//
// Routing reading: top-k of the router logits per token ("Step3 Inference
// Optimization on AMD Instinct MI308X", Background: 3 of 48 experts), ties to
// the lower expert id, weights = softmax of the selected logits (the same as
// softmax over all experts, keep k, renormalise).
#include <float.h>
#include <math.h>

#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {
namespace {

// One wave computes a 16-row x 16-expert logits tile over one K chunk with
// bf16 MFMA; a 256-thread block holds 4 waves on 4 adjacent expert tiles that
// share the same 16 rows (the x fragment is then an L1 hit for 3 of them).
// grid = (ceil(T/16), ceil(E/64), ks).
__global__ __launch_bounds__(256) void route_logits_bf16_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ valid,
    const uint16_t* __restrict__ R, float* __restrict__ part, int T, int H,
    int E, int kchunk) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int row0 = blockIdx.x * 16;
  const int e0 = blockIdx.y * 64 + wave * 16;
  if (e0 >= E) return;
  const int m = lane % 16, g = lane / 16;
  const int row = row0 + m;
  const bool rv = row < T && (valid == nullptr || valid[row] != 0);
  if (__ballot(rv) == 0) return;   // no valid row: partials never read
  const int e = e0 + m;
  const bool ev = e < E;
  const int kb = blockIdx.z * kchunk;
  const int ke = min(H, kb + kchunk);
  const uint16_t* xp = x + (size_t)(rv ? row : 0) * H + 8 * g;
  const uint16_t* rp = R + (size_t)(ev ? e : 0) * H + 8 * g;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int k = kb; k < ke; k += 32) {
    u32x4 a = rv ? *reinterpret_cast<const u32x4*>(xp + k) : zero;
    u32x4 b = ev ? *reinterpret_cast<const u32x4*>(rp + k) : zero;
    acc = mfma16x16x32(as_bf16x8(a), as_bf16x8(b), acc);
  }
  if (!ev) return;
  float* dst = part + ((size_t)blockIdx.z * T) * E + e;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = row0 + 4 * g + i;
    if (r < T) dst[(size_t)r * E] = acc[i];
  }
}

// fp32 router (small layers): one thread per (row, expert), sequential FMA.
__global__ __launch_bounds__(256) void route_logits_f32_kernel(
    const float* __restrict__ x, const uint8_t* __restrict__ valid,
    const float* __restrict__ R, float* __restrict__ part, int T, int H, int E) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)T * E) return;
  const int t = (int)(idx / E), e = (int)(idx % E);
  float acc = 0.f;
  if (valid == nullptr || valid[t] != 0) {
    const float* xp = x + (size_t)t * H;
    const float* rp = R + (size_t)e * H;
    for (int h = 0; h < H; ++h) acc = fmaf(xp[h], rp[h], acc);
  }
  part[idx] = acc;
}

__device__ __forceinline__ bool beats(float av, int ae, float bv, int be) {
  return av > bv || (av == bv && ae < be);
}

// One step of a wave arg-max under (logit desc, id asc): take the pair held
// by the lane that the DPP pattern CTRL names, if it beats this lane's.
template <int CTRL>
__device__ __forceinline__ void argmax_dpp(float& bv, int& be) {
  const float ov =
      __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(bv), CTRL, 0xf, 0xf, false));
  const int oe = __builtin_amdgcn_update_dpp(0, be, CTRL, 0xf, 0xf, false);
  if (beats(ov, oe, bv, be)) {
    bv = ov;
    be = oe;
  }
}

// Wave-wide arg-max: within each 16-lane row by DPP (swap neighbours, swap
// pairs, rotate by 4, rotate by 8 — every lane then holds its row's best),
// then the four rows' bests read into scalars.  The order is total, so the
// result does not depend on the reduction's shape.
__device__ __forceinline__ void wave_argmax(float& bv, int& be) {
  argmax_dpp<0xb1>(bv, be);    // quad_perm [1, 0, 3, 2]
  argmax_dpp<0x4e>(bv, be);    // quad_perm [2, 3, 0, 1]
  argmax_dpp<0x124>(bv, be);   // row_ror 4
  argmax_dpp<0x128>(bv, be);   // row_ror 8
  float rv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 0));
  int re = __builtin_amdgcn_readlane(be, 0);
#pragma unroll
  for (int r = 16; r < kWave; r += 16) {
    const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), r));
    const int id = __builtin_amdgcn_readlane(be, r);
    if (beats(v, id, rv, re)) {
      rv = v;
      re = id;
    }
  }
  bv = rv;
  be = re;
}

// One wave per row: expert e lives in lane e % 64, register e / 64.
// k rounds of a wave-wide arg-max under (logit desc, id asc).
constexpr int kMaxTopk = 16;

__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ part, int ks, const uint8_t* __restrict__ valid,
    int T, int E, int k, int32_t* __restrict__ ids, float* __restrict__ w,
    float* __restrict__ logits_out) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const bool rv = valid == nullptr || valid[t] != 0;
  if (!rv) {
    if (lane < k) {
      ids[(size_t)t * k + lane] = -1;
      w[(size_t)t * k + lane] = 0.f;
    }
    if (logits_out)
      for (int e = lane; e < E; e += kWave) logits_out[(size_t)t * E + e] = 0.f;
    return;
  }
  float v[4];
  bool taken[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + kWave * i;
    taken[i] = e >= E;
    float s = 0.f;
    if (e < E) {
      // fixed summation order z = 0, 1, ...; loads issued 8 at a time
      const float* pp = part + (size_t)t * E + e;
      const size_t zs = (size_t)T * E;
      int z = 0;
      for (; z + 8 <= ks; z += 8) {
        float v8[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v8[q] = pp[(z + q) * zs];
#pragma unroll
        for (int q = 0; q < 8; ++q) s += v8[q];
      }
      for (; z < ks; ++z) s += pp[z * zs];
      if (logits_out) logits_out[(size_t)t * E + e] = s;
    }
    v[i] = s;
  }
  float top = 0.f, denom = 0.f, my_v = 0.f;
  int my_e = -1;
#pragma unroll
  for (int j = 0; j < kMaxTopk; ++j) {
    if (j < k) {
      float bv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!taken[i] && beats(v[i], lane + kWave * i, bv, be)) {
          bv = v[i];
          be = lane + kWave * i;
        }
      wave_argmax(bv, be);
      if (j == 0) top = bv;
      denom += expf(bv - top);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (be == lane + kWave * i) taken[i] = true;
      if (lane == j) {
        my_v = bv;
        my_e = be;
      }
    }
  }
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_e;
    w[(size_t)t * k + lane] = expf(my_v - top) / denom;
  }
}

}  // namespace

hipError_t launch_route_logits(bool bf16, const void* x, const uint8_t* valid,
                               const void* R, float* part, int T, int H, int E,
                               int ks, hipStream_t s) {
  if (bf16) {
    const int ksteps = H / 32;
    const int kchunk = 32 * (ksteps / ks);
    dim3 grid((T + 15) / 16, (E + 63) / 64, ks);
    hipLaunchKernelGGL(route_logits_bf16_kernel, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(x), valid,
                       static_cast<const uint16_t*>(R), part, T, H, E, kchunk);
  } else {
    const size_t n = (size_t)T * E;
    if ((n + 255) / 256 > 0x7fffffffu) return hipErrorInvalidValue;
    hipLaunchKernelGGL(route_logits_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       static_cast<const float*>(x), valid,
                       static_cast<const float*>(R), part, T, H, E);
  }
  return hipGetLastError();
}

hipError_t launch_route_topk(const float* part, int ks, const uint8_t* valid,
                             int T, int E, int k, int32_t* ids, float* w,
                             float* logits_out, hipStream_t s) {
  hipLaunchKernelGGL(route_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, part,
                     ks, valid, T, E, k, ids, w, logits_out);
  return hipGetLastError();
}

}  // namespace moe
