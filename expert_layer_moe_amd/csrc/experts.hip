// Weight-streaming expert grouped GEMMs (the decode regime, bound by HBM).
//
// gate/up: h = SiLU(W_gate x) * (W_up x) per sorted row (the expert MLP of a
// sparse MoE layer, "AMD Instinct MI355X: ATOM ...": sparse MoE experts,
// block-scale GEMMs); down: y = W2 h ("[SGLang] Single Batch Overlap for MoE
// models": the down-projection GEMM).  The shared expert of "Step3 Inference
// Optimization on AMD Instinct MI308X" (optimisation list) is one more
// segment.
//
// fp8 weights (same list: FP8 blockscale) are OCP e4m3fn codes with one fp32
// scale per 128x128 block; codes become bf16 exactly, MFMA accumulates each
// 128-wide K block separately, and the block's scale multiplies that partial
// sum in fp32 before it joins the accumulator.
#include "moe_common.h"
#include "moe_kernels.h"

#include <climits>
#include <type_traits>

namespace moe {
namespace {

// One lane's 8 weights of a fragment; NT: a non-temporal load (for weights
// that no other block of the launch reads).
template <bool FP8, bool NT = false>
__device__ __forceinline__ bf16x8 load_w8(const void* base, size_t elem_off) {
  if constexpr (FP8) {
    const u32x2* p = reinterpret_cast<const u32x2*>(static_cast<const uint8_t*>(base) + elem_off);
    const u32x2 v = NT ? __builtin_nontemporal_load(p) : *p;
    return fp8x8_to_bf16x8(v[0], v[1]);
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + elem_off);
    return as_bf16x8(NT ? __builtin_nontemporal_load(p) : *p);
  }
}

// The hardware hands block b to XCD b % 8.  Give each XCD a contiguous range
// of logical block ids, so that the blocks of one expert (which read the same
// token rows) share that XCD's L2.  nb must be a multiple of 8.
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  return (b & 7) * (nb >> 3) + (b >> 3);
}

// Unit u of the streaming kernels -> its segment (returned), column group
// cg and item it within the segment (rows 64 it ..).  The item table lists
// a segment's items together, so the segment's units form one range of
// n_items(seg) x n_cols units, ordered column-group major: the items of a
// segment that read the same weight columns are neighbours in dispatch
// order (same XCD, at the same time), which lets them share those weights
// through L2.
__device__ __forceinline__ int unit_of_segment(int u, int n_cols, const int32_t* item_seg,
                                               const int32_t* item_row0, const int32_t* seg_cnt,
                                               int& cg, int& it) {
  const int ig = u / n_cols;   // an item of the unit's segment
  const int e = item_seg[ig];
  const int ni = (seg_cnt[e] + kStreamItemRows - 1) / kStreamItemRows;
  const int i0 = ig - item_row0[ig] / kStreamItemRows;   // the segment's first item
  const int local = u - i0 * n_cols;
  cg = local / ni;
  it = local - cg * ni;
  return e;
}

// The streaming kernels loop over n_live work units (known only on the
// device) in rounds of gridDim.x (a multiple of 8): this block's unit of the
// round that starts at u0, or -1.  A partial round is remapped over its
// first round_up(live, 8) blocks, which spread over all XCDs.  Capping the
// grid, instead of sizing it for the worst case, keeps surplus blocks from
// holding the CUs' slots while they find they have nothing to do.
__device__ __forceinline__ int round_unit(int u0, int n_live) {
  const int rem = min((int)gridDim.x, n_live - u0);
  const int nb = (rem + 7) & ~7;
  if ((int)blockIdx.x >= nb) return -1;
  const int l = xcd_remap(blockIdx.x, nb);
  return l < rem ? u0 + l : -1;
}

// ---------------------------------------------------------------------------
// Weight-streaming gate/up for expert segments of a few tiles of rows (the
// decode regime, bound by HBM): one block per (work item, 4/KS groups of 16
// intermediate columns), a work item being a segment and up to MT = 4 of its
// 16-row tiles (the align's stream item table; a segment's items run side by
// side, so its weights come from HBM once and are shared through L2).  The
// block's waves split K = H into KS contiguous parts; a wave streams its part
// of 16 gate rows and the 16 matching up rows of W13 once for the item's
// tiles, issuing KU MFMA K-steps of loads ahead of their MFMAs.  Partial sums
// of the KS waves meet in LDS (fixed order), then h = SiLU(g) * u in bf16.
// Units: (item, column group), n_cg = ceil(I / (16 * 4 / KS)) per item.
// bf16: three waves per SIMD (164 VGPRs, no spills) keep more weight loads in
// flight; the fp8 variant keeps two (it would spill).
template <int KS, int MT, int KU, bool FP8, bool PW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(FP8 ? 2 : 3)))
void gate_up_stream_kernel(
    const uint16_t* __restrict__ xp, const void* __restrict__ w13,
    const float* __restrict__ s13, const int32_t* __restrict__ seg_off,
    const int32_t* __restrict__ seg_cnt, const int32_t* __restrict__ item_seg,
    const int32_t* __restrict__ item_row0, const int32_t* __restrict__ n_items,
    uint16_t* __restrict__ h, int H, int I, int max_items, int n_cg) {
  static_assert(MT * 16 == kStreamItemRows, "one work item per pass");
  constexpr int CGW = 4 / KS;
  __shared__ floatx4 red[KS > 1 ? 4 : 1][2][MT][kWave];
  const int n_live = min(*n_items, max_items) * n_cg;
  for (int u0 = 0; u0 < n_live; u0 += gridDim.x) {
    const int lid = round_unit(u0, n_live);
    if (lid < 0) continue;
    int cgb, it;
    const int e = unit_of_segment(lid, n_cg, item_seg, item_row0, seg_cnt, cgb, it);
    const int cnt = seg_cnt[e];
    const int row0 = seg_off[e];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int ks = wave % KS, cw = wave / KS;
    const int cg = cgb * CGW + cw;
    const bool col_ok = cg * 16 < I;
    const int m = lane % 16, g = lane / 16;
    const int klen = H / KS, kbeg = ks * klen;
    const int c0 = col_ok ? cg * 16 : 0;
    // this lane's element offset in the gate / up rows at step 0 of its K
    // part, and the distance of one MFMA K step (row-major: 32 elements along
    // the row; fragment-packed: the next 512-element block of the same tile)
    constexpr size_t wstep = PW ? 512 : 32;
    size_t wg_off, wu_off;
    if constexpr (PW) {
      const size_t tg = ((size_t)e * 2 * I + c0) / 16, tu = tg + I / 16;
      wg_off = (tg * (H / 32) + kbeg / 32) * 512 + 8 * lane;
      wu_off = (tu * (H / 32) + kbeg / 32) * 512 + 8 * lane;
    } else {
      wg_off = ((size_t)e * 2 * I + c0 + m) * H + kbeg + 8 * g;
      wu_off = wg_off + (size_t)I * H;
    }
    const float* sg = nullptr;
    const float* su = nullptr;
    if constexpr (FP8) {
      const int nkb = H / 128;
      sg = s13 + ((size_t)e * (2 * I / 128) + c0 / 128) * nkb;
      su = s13 + ((size_t)e * (2 * I / 128) + (I + c0) / 128) * nkb;
    }
    const u32x4 zero = {0u, 0u, 0u, 0u};
    // the item's 16-row tiles [tb, te) of the segment
    const int tb = it * MT, te = min((cnt + 15) >> 4, tb + MT);
    for (int t0 = tb; t0 < te; t0 += MT) {
      // fragment-ordered token tiles (row0 is a multiple of 16); step s of
      // tile t at xa + 512 s
      const uint16_t* xa[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        xa[mt] = xp + ((size_t)(row0 >> 4) + t0 + mt) * 16 * H + (size_t)(kbeg / 32) * 512 + 8 * lane;
      floatx4 ag[MT], au[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        ag[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
        au[mt] = ag[mt];
      }
      if (col_ok) {
        for (int kk = 0; kk < klen; kk += 32 * KU) {
          bf16x8 bg[KU], bu[KU], a[KU][MT];
#pragma unroll
          for (int u = 0; u < KU; ++u) {
            bg[u] = load_w8<FP8>(w13, wg_off + (size_t)(kk / 32 + u) * wstep);
            bu[u] = load_w8<FP8>(w13, wu_off + (size_t)(kk / 32 + u) * wstep);
          }
#pragma unroll
          for (int u = 0; u < KU; ++u)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              a[u][mt] = as_bf16x8(t0 + mt < te ? ld16(xa[mt] + (size_t)(kk / 32 + u) * 512) : zero);
          if constexpr (FP8) {
            floatx4 pg[MT], pu[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              pg[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
              pu[mt] = pg[mt];
            }
#pragma unroll
            for (int u = 0; u < KU; ++u)
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
                if (t0 + mt < te) {
                  pg[mt] = mfma16x16x32(a[u][mt], bg[u], pg[mt]);
                  pu[mt] = mfma16x16x32(a[u][mt], bu[u], pu[mt]);
                }
            const int kb = (kbeg + kk) >> 7;
            const float scg = sg[kb], scu = su[kb];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                ag[mt][i] = fmaf(scg, pg[mt][i], ag[mt][i]);
                au[mt][i] = fmaf(scu, pu[mt][i], au[mt][i]);
              }
          } else {
#pragma unroll
            for (int u = 0; u < KU; ++u)
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
                if (t0 + mt < te) {
                  ag[mt] = mfma16x16x32(a[u][mt], bg[u], ag[mt]);
                  au[mt] = mfma16x16x32(a[u][mt], bu[u], au[mt]);
                }
          }
        }
      }
      if constexpr (KS == 1) {
        if (col_ok) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = (t0 + mt) * 16 + 4 * g + i;
              if (r < cnt)
                h[frag_index(row0 + r, c0 + m, I)] = f32_to_bf16_bits(silu_mul(ag[mt][i], au[mt][i]));
            }
        }
      } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          red[wave][0][mt][lane] = ag[mt];
          red[wave][1][mt][lane] = au[mt];
        }
        __syncthreads();
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if ((mt % KS) == ks && t0 + mt < te && col_ok) {
            floatx4 G = red[cw * KS][0][mt][lane], U = red[cw * KS][1][mt][lane];
#pragma unroll
            for (int q = 1; q < KS; ++q) {
              const floatx4 g2 = red[cw * KS + q][0][mt][lane];
              const floatx4 u2 = red[cw * KS + q][1][mt][lane];
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                G[i] += g2[i];
                U[i] += u2[i];
              }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = (t0 + mt) * 16 + 4 * g + i;
              if (r < cnt) h[frag_index(row0 + r, c0 + m, I)] = f32_to_bf16_bits(silu_mul(G[i], U[i]));
            }
          }
        }
        __syncthreads();
      }
    }
  }
}

// Weight-streaming down projection: one block per (work item, 64*NT output
// columns); each wave streams NT 16-row tiles of W2 (full K = I) once for
// the item's (up to MT) 16-row tiles of h.  W2 is the MFMA's A operand, so
// a lane ends with 4 consecutive output columns of one row, stored as one
// piece of the row's y (16 bytes of fp32, or 8 of bf16 with fp8 weights).
// Units: (item, column group), n_ng = ceil(H / (64 * NT)) per item (NT = 4).
template <int MT, int NT, int KU, bool FP8, bool PW>
__global__ __launch_bounds__(256) void down_stream_kernel(
    const uint16_t* __restrict__ h, const void* __restrict__ w2,
    const float* __restrict__ s2, const int32_t* __restrict__ seg_off,
    const int32_t* __restrict__ seg_cnt, const int32_t* __restrict__ item_seg,
    const int32_t* __restrict__ item_row0, const int32_t* __restrict__ n_items,
    void* __restrict__ y, int H, int I, int max_items, int n_ng) {
  static_assert(MT * 16 == kStreamItemRows, "one work item per pass");
  const int n_live = min(*n_items, max_items) * n_ng;
  for (int u0 = 0; u0 < n_live; u0 += gridDim.x) {
    const int lid = round_unit(u0, n_live);
    if (lid < 0) continue;
    int ngb, it;
    const int e = unit_of_segment(lid, n_ng, item_seg, item_row0, seg_cnt, ngb, it);
    const int cnt = seg_cnt[e];
    const int row0 = seg_off[e];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int n0 = (ngb * 4 + wave) * NT * 16;
    if (n0 >= H) continue;   // no barriers here: waves go their own way
    const int m = lane % 16, g = lane / 16;
    constexpr size_t wstep = PW ? 512 : 32;   // elements per MFMA K step
    size_t wo[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = min(n0 + nt * 16, H - 16);
      if constexpr (PW) wo[nt] = (((size_t)e * H + n) / 16 * (I / 32)) * 512 + 8 * lane;
      else wo[nt] = ((size_t)e * H + n + m) * I + 8 * g;
    }
    const float* sc = nullptr;
    if constexpr (FP8) sc = s2 + (size_t)e * (H / 128) * (I / 128);
    const u32x4 zero = {0u, 0u, 0u, 0u};
    // the item's 16-row tiles [tb, te) of the segment
    const int tb = it * MT, te = min((cnt + 15) >> 4, tb + MT);
    for (int t0 = tb; t0 < te; t0 += MT) {
      // fragment-ordered h tiles (rows past cnt may hold anything: each token
      // row feeds only its own output column of the MFMA, never stored)
      const uint16_t* ha[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        ha[mt] = h + ((size_t)(row0 >> 4) + t0 + mt) * 16 * I + 8 * lane;
      floatx4 acc[MT][NT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
      // W2 of a segment with one item is read by this block alone: non-temporal
      // loads (measured faster); the items of a larger segment share it
      // through L2 (normal loads measured faster)
      auto k_loop = [&](auto nt_tag) {
        constexpr bool kNT = decltype(nt_tag)::value;
        for (int kk = 0; kk < I; kk += 32 * KU) {
          bf16x8 b[KU][NT], a[KU][MT];
#pragma unroll
          for (int u = 0; u < KU; ++u)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              b[u][nt] = load_w8<FP8, kNT>(w2, wo[nt] + (size_t)(kk / 32 + u) * wstep);
#pragma unroll
          for (int u = 0; u < KU; ++u)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              a[u][mt] = as_bf16x8(t0 + mt < te ? ld16(ha[mt] + (size_t)(kk / 32 + u) * 512) : zero);
          if constexpr (FP8) {
            floatx4 p[MT][NT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
              for (int nt = 0; nt < NT; ++nt) p[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < KU; ++u)
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
                if (t0 + mt < te)
#pragma unroll
                  for (int nt = 0; nt < NT; ++nt) p[mt][nt] = mfma16x16x32(b[u][nt], a[u][mt], p[mt][nt]);
            const int kb = kk >> 7;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              const float s = sc[((n0 + nt * 16) / 128) * (I / 128) + kb];
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[mt][nt][i] = fmaf(s, p[mt][nt][i], acc[mt][nt][i]);
            }
          } else {
#pragma unroll
            for (int u = 0; u < KU; ++u)
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
                if (t0 + mt < te)
#pragma unroll
                  for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma16x16x32(b[u][nt], a[u][mt], acc[mt][nt]);
          }
        }
      };
      // (fragment-packed weights only: a row-major K step reads half of each
      // 128-byte line, and the next step needs the line again)
      if (PW && cnt <= kStreamItemRows) k_loop(std::true_type{});
      else k_loop(std::false_type{});
      // acc[mt][nt] lane (m, g): row (t0 + mt) 16 + m, columns n0 + 16 nt + 4 g .. + 3
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = (t0 + mt) * 16 + m;
        if (r >= cnt) continue;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if (n0 + nt * 16 >= H) continue;
          store_y4<FP8>(y, (size_t)(row0 + r) * H + n0 + nt * 16 + 4 * g, acc[mt][nt]);
        }
      }
    }
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

}  // namespace

namespace {

int pick_ku(int len) {
  // largest K-steps-per-batch in {4, 2, 1} that tiles len (a batch of
  // 32 * {1,2,4} never straddles a 128-wide fp8 scale block)
  for (int ku = 4; ku > 1; ku >>= 1)
    if (len % (32 * ku) == 0) return ku;
  return 1;
}

struct GuArgs {
  dim3 grid;
  hipStream_t s;
  const uint16_t* xp;
  const void* w13;
  const float* s13;
  const int32_t* seg_off;
  const int32_t* seg_cnt;
  const int32_t* item_seg;
  const int32_t* item_row0;
  const int32_t* n_items;
  uint16_t* h;
  int H, I, max_items, n_cg;
};

template <int KS, int KU, bool FP8, bool PW>
void launch_gu(const GuArgs& a) {
  hipLaunchKernelGGL((gate_up_stream_kernel<KS, 4, KU, FP8, PW>), a.grid, dim3(256), 0, a.s,
                     a.xp, a.w13, a.s13, a.seg_off, a.seg_cnt, a.item_seg, a.item_row0,
                     a.n_items, a.h, a.H, a.I, a.max_items, a.n_cg);
}

// up to 4 K steps per batch, 2 with fp8 weights or without a K split (the
// limits keep every variant free of register spills)
template <int KS, bool FP8, bool PW>
void launch_gu_ku(int ku, const GuArgs& a) {
  if constexpr (!FP8 && KS > 1) {
    if (ku == 4) {
      launch_gu<KS, 4, FP8, PW>(a);
      return;
    }
  }
  if (ku >= 2) launch_gu<KS, 2, FP8, PW>(a);
  else launch_gu<KS, 1, FP8, PW>(a);
}

template <bool FP8, bool PW>
void launch_gu_ks(int ks, int ku, const GuArgs& a) {
  if (ks == 4) launch_gu_ku<4, FP8, PW>(ku, a);
  else if (ks == 2) launch_gu_ku<2, FP8, PW>(ku, a);
  else launch_gu_ku<1, FP8, PW>(ku, a);
}

struct DnArgs {
  dim3 grid;
  hipStream_t s;
  const uint16_t* h;
  const void* w2;
  const float* s2;
  const int32_t* seg_off;
  const int32_t* seg_cnt;
  const int32_t* item_seg;
  const int32_t* item_row0;
  const int32_t* n_items;
  void* y;
  int H, I, max_items, n_ng;
};

template <int KU, bool FP8, bool PW>
void launch_dn(const DnArgs& a) {
  hipLaunchKernelGGL((down_stream_kernel<4, 4, KU, FP8, PW>), a.grid, dim3(256), 0, a.s, a.h, a.w2,
                     a.s2, a.seg_off, a.seg_cnt, a.item_seg, a.item_row0, a.n_items, a.y, a.H,
                     a.I, a.max_items, a.n_ng);
}

template <bool FP8, bool PW>
void launch_dn_ku(int ku, const DnArgs& a) {
  if (ku == 4) launch_dn<4, FP8, PW>(a);
  else if (ku == 2) launch_dn<2, FP8, PW>(a);
  else launch_dn<1, FP8, PW>(a);
}

int round8(int v) { return (v + 7) / 8 * 8; }

// Grid of the streaming kernels: one block per unit up to this many, then
// blocks loop over units.
constexpr int kStreamGridCap = 4096;
int stream_grid(int bound) { return min(round8(bound), kStreamGridCap); }

}  // namespace

hipError_t launch_gate_up(int wkind, bool packed, const void* x, const void* w13,
                          const float* s13, const int32_t* sorted_ids,
                          const int32_t* block_expert, const int32_t* n_post,
                          const int32_t* seg_off, const int32_t* seg_cnt,
                          const int32_t* item_seg, const int32_t* item_row0,
                          const int32_t* n_items, int max_items, const void* xp, void* h,
                          int H, int I, int k, int bm, int max_rows, hipStream_t s) {
  if (wkind == W_F32) {
    hipLaunchKernelGGL(gate_up_f32_kernel, dim3(max_rows), dim3(256), 0, s,
                       static_cast<const float*>(x), static_cast<const float*>(w13),
                       sorted_ids, block_expert, n_post, static_cast<float*>(h), H, I,
                       k, bm);
    return hipGetLastError();
  }
  const bool fp8 = wkind == W_FP8;
  // K split across the block's waves: 4 parts when each part still holds
  // whole 32-wide MFMA steps (and, for fp8, whole 128-wide scale blocks).
  int ks = 4;
  while (ks > 1 && (H % ks != 0 || (H / ks) % (fp8 ? 128 : 32) != 0)) ks >>= 1;
  const int ku = pick_ku(H / ks);
  const int cgw = 4 / ks;
  const int n_cg = (I / 16 + cgw - 1) / cgw;
  if (bm != 16 || (long long)max_items * n_cg > INT_MAX - 8) return hipErrorInvalidValue;
  GuArgs a{dim3(stream_grid(max_items * n_cg)), s, static_cast<const uint16_t*>(xp), w13, s13,
           seg_off, seg_cnt, item_seg, item_row0, n_items, static_cast<uint16_t*>(h), H, I,
           max_items, n_cg};
  if (fp8) {
    if (packed) launch_gu_ks<true, true>(ks, ku, a);
    else launch_gu_ks<true, false>(ks, ku, a);
  } else {
    if (packed) launch_gu_ks<false, true>(ks, ku, a);
    else launch_gu_ks<false, false>(ks, ku, a);
  }
  return hipGetLastError();
}

hipError_t launch_down(int wkind, bool packed, const void* h, const void* w2, const float* s2,
                       const int32_t* block_expert, const int32_t* n_post,
                       const int32_t* seg_off, const int32_t* seg_cnt,
                       const int32_t* item_seg, const int32_t* item_row0,
                       const int32_t* n_items, int max_items, void* y, int H, int I,
                       int bm, int max_rows, hipStream_t s) {
  if (wkind == W_F32) {
    hipLaunchKernelGGL(down_f32_kernel, dim3(max_rows), dim3(256), 0, s,
                       static_cast<const float*>(h), static_cast<const float*>(w2),
                       block_expert, n_post, static_cast<float*>(y), H, I, bm);
    return hipGetLastError();
  }
  const bool fp8 = wkind == W_FP8;
  const int ku = pick_ku(I);
  const int n_ng = (H + 255) / 256;
  if ((long long)max_items * n_ng > INT_MAX - 8) return hipErrorInvalidValue;
  DnArgs a{dim3(stream_grid(max_items * n_ng)), s, static_cast<const uint16_t*>(h), w2, s2,
           seg_off, seg_cnt, item_seg, item_row0, n_items, y, H, I, max_items, n_ng};
  if (fp8) {
    if (packed) launch_dn_ku<true, true>(ku, a);
    else launch_dn_ku<true, false>(ku, a);
  } else {
    if (packed) launch_dn_ku<false, true>(ku, a);
    else launch_dn_ku<false, false>(ku, a);
  }
  return hipGetLastError();
}

}  // namespace moe
