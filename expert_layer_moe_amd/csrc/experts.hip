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

#include <algorithm>
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
// through L2.  With item non-null, *item = the unit's item in the table.
__device__ __forceinline__ int unit_of_segment(int u, int n_cols, const int32_t* item_seg,
                                               const int32_t* item_row0, const int32_t* seg_cnt,
                                               int& cg, int& it, int* item = nullptr) {
  const int ig = u / n_cols;   // an item of the unit's segment
  const int e = item_seg[ig];
  const int ni = (seg_cnt[e] + kStreamItemRows - 1) / kStreamItemRows;
  const int i0 = ig - item_row0[ig] / kStreamItemRows;   // the segment's first item
  const int local = u - i0 * n_cols;
  cg = local / ni;
  it = local - cg * ni;
  if (item != nullptr) *item = i0 + it;
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
// decode regime, bound by HBM): one block per (work item, column group), a
// work item being a segment and up to MT = 4 of its 16-row tiles (the align's
// stream item table; a segment's items run side by side, so its weights come
// from HBM once and are shared through L2).  The block's waves split K = H
// into KS contiguous parts; a wave streams its part of CGN 16-row tiles of
// gate rows and the matching up rows of W13 once for the item's tiles,
// issuing KU MFMA K-steps of loads ahead of their MFMAs.  Each token
// fragment a wave loads feeds the MFMAs of its CGN column tiles.  The token
// rows come from L2 once per column group; with one 16-column tile per wave
// those L2 reads cost decode_e48 about a fifth of the kernel (167 us, 134
// with them taken out in a timing copy), and two tiles per wave (CGN = 2,
// two waves per SIMD, no spills) halve them: 157 us, gather_padded_e48 258
// -> 240 us.  (Three or four tiles per wave: 179 / 153 us on decode_e48 but
// 233 / 254 on gather_padded_e48.)  Partial sums of the KS waves meet in LDS
// (fixed order, one column tile at a time), then h = SiLU(g) * u in bf16.
// Units: (item, column group), n_cg = ceil(I / (16 CGN 4 / KS)) per item.
// XD: the token rows come straight from x (token sorted_ids[r] / topk of
// sorted row r, row-major, 16 rows x 64 bytes per wave load) instead of the
// fragment-ordered copy xp: for calls where every segment streams (decode)
// x holds each token once where the copy holds it k times, and reading it
// measured faster than packing it (decode_e48 step 0.265 -> 0.255 ms,
// decode_e256_shared 0.500 -> 0.475 ms); with many rows per segment
// (gather_padded_e48) the copy is faster (gate/up 241 against 288 us).
// One unit (work item lid of the item table, column group) of the streaming
// gate/up; returns the index of the unit's item in the item table.  Called
// by every thread of a 256-thread block (the K-part sums meet in red).
template <int KS, int MT, int KU, int CGN, bool FP8, bool PW, bool XD>
__device__ __forceinline__ int gate_up_unit(
    int lid, const uint16_t* __restrict__ xp, const void* __restrict__ w13,
    const float* __restrict__ s13, const int32_t* __restrict__ seg_off,
    const int32_t* __restrict__ seg_cnt, const int32_t* __restrict__ item_seg,
    const int32_t* __restrict__ item_row0, uint16_t* __restrict__ h, int H, int I, int n_cg,
    const int32_t* __restrict__ sorted_ids, int topk,
    floatx4 (&red)[KS > 1 ? 4 : 1][2][MT][kWave]) {
  static_assert(MT * 16 == kStreamItemRows, "one work item per pass");
  constexpr int CGW = 4 / KS;   // waves side by side along the columns
  int cgb, it, item;
  const int e = unit_of_segment(lid, n_cg, item_seg, item_row0, seg_cnt, cgb, it, &item);
  const int cnt = seg_cnt[e];
  const int row0 = seg_off[e];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int ks = wave % KS, cw = wave / KS;
  const int m = lane % 16, g = lane / 16;
  const int klen = H / KS, kbeg = ks * klen;
  // the wave's column tiles j: columns c0[j] .. + 15 (a tile past I is
  // neither loaded nor stored)
  bool col_ok[CGN];
  int c0[CGN];
  // this lane's element offsets in the gate / up rows at step 0 of its K
  // part, and the distance of one MFMA K step (row-major: 32 elements along
  // the row; fragment-packed: the next 512-element block of the same tile)
  constexpr size_t wstep = PW ? 512 : 32;
  size_t wg_off[CGN], wu_off[CGN];
  const float* sg[CGN];
  const float* su[CGN];
#pragma unroll
  for (int j = 0; j < CGN; ++j) {
    const int c = ((cgb * CGW + cw) * CGN + j) * 16;
    col_ok[j] = c < I;
    c0[j] = col_ok[j] ? c : 0;
    if constexpr (PW) {
      const size_t tg = ((size_t)e * 2 * I + c0[j]) / 16, tu = tg + I / 16;
      wg_off[j] = (tg * (H / 32) + kbeg / 32) * 512 + 8 * lane;
      wu_off[j] = (tu * (H / 32) + kbeg / 32) * 512 + 8 * lane;
    } else {
      wg_off[j] = ((size_t)e * 2 * I + c0[j] + m) * H + kbeg + 8 * g;
      wu_off[j] = wg_off[j] + (size_t)I * H;
    }
    sg[j] = su[j] = nullptr;
    if constexpr (FP8) {
      const int nkb = H / 128;
      sg[j] = s13 + ((size_t)e * (2 * I / 128) + c0[j] / 128) * nkb;
      su[j] = s13 + ((size_t)e * (2 * I / 128) + (I + c0[j]) / 128) * nkb;
    }
  }
  const u32x4 zero = {0u, 0u, 0u, 0u};
  // the item's 16-row tiles [tb, te) of the segment
  const int tb = it * MT, te = min((cnt + 15) >> 4, tb + MT);
  for (int t0 = tb; t0 < te; t0 += MT) {
    // this lane's token row of each tile at the start of its K part:
    // fragment-ordered tiles of xp (row0 is a multiple of 16; step s of
    // tile t at xa + 512 s), or row m of the tile straight from x (XD;
    // step s at xa + 32 s; a padding row reads any row: the MFMA keeps rows
    // apart and its results are never stored)
    const uint16_t* xa[MT];
    constexpr size_t xstep = XD ? 32 : 512;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if constexpr (XD) {
        const int sid = t0 + mt < te ? sorted_ids[row0 + (t0 + mt) * 16 + m] : -1;
        xa[mt] = xp + (size_t)(sid >= 0 ? sid / topk : 0) * H + kbeg + 8 * g;
      } else {
        xa[mt] = xp + ((size_t)(row0 >> 4) + t0 + mt) * 16 * H + (size_t)(kbeg / 32) * 512 + 8 * lane;
      }
    }
    floatx4 ag[CGN][MT], au[CGN][MT];
#pragma unroll
    for (int j = 0; j < CGN; ++j)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        ag[j][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
        au[j][mt] = ag[j][mt];
      }
    // W13 of a segment with one item is read by this block alone:
    // non-temporal loads (measured faster on the decode batches); the items
    // of a larger segment share it through L2 (normal loads measured faster)
    auto k_loop = [&](auto nt_tag) {
      constexpr bool kNT = decltype(nt_tag)::value;
      // The blocks of one item read the same token rows; started at the
      // same K they would all ask the same L2 lines at once.  Where those
      // rows come straight from x (XD), each group of 32 columns starts
      // its K loop at its own batch (a fixed order per column, so the sums
      // do not depend on the block shape): decode_e48 gate/up 157 -> 149
      // us.  From the packed copy, asking at once is what lets the L2
      // serve them once: without the rotation gather_padded_e48's gate/up
      // fetches 1036 instead of 1263 MB, in the same time.
      const int nbat = klen / (32 * KU);
      const int rot = XD ? (c0[0] / 32) % nbat * (32 * KU) : 0;
      for (int kk0 = 0; kk0 < klen; kk0 += 32 * KU) {
        const int kk = kk0 + rot < klen ? kk0 + rot : kk0 + rot - klen;
        bf16x8 bg[KU][CGN], bu[KU][CGN], a[KU][MT];
#pragma unroll
        for (int u = 0; u < KU; ++u)
#pragma unroll
          for (int j = 0; j < CGN; ++j) {
            if (j == 0 || col_ok[j]) {
              bg[u][j] = load_w8<FP8, kNT>(w13, wg_off[j] + (size_t)(kk / 32 + u) * wstep);
              bu[u][j] = load_w8<FP8, kNT>(w13, wu_off[j] + (size_t)(kk / 32 + u) * wstep);
            } else {
              bg[u][j] = bu[u][j] = as_bf16x8(zero);
            }
          }
#pragma unroll
        for (int u = 0; u < KU; ++u)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            a[u][mt] = as_bf16x8(t0 + mt < te ? ld16(xa[mt] + (size_t)(kk / 32 + u) * xstep) : zero);
        if constexpr (FP8) {
#pragma unroll
          for (int j = 0; j < CGN; ++j) {
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
                  pg[mt] = mfma16x16x32(a[u][mt], bg[u][j], pg[mt]);
                  pu[mt] = mfma16x16x32(a[u][mt], bu[u][j], pu[mt]);
                }
            const int kb = (kbeg + kk) >> 7;
            const float scg = sg[j][kb], scu = su[j][kb];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                ag[j][mt][i] = fmaf(scg, pg[mt][i], ag[j][mt][i]);
                au[j][mt][i] = fmaf(scu, pu[mt][i], au[j][mt][i]);
              }
          }
        } else {
#pragma unroll
          for (int u = 0; u < KU; ++u)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              if (t0 + mt < te)
#pragma unroll
                for (int j = 0; j < CGN; ++j) {
                  ag[j][mt] = mfma16x16x32(a[u][mt], bg[u][j], ag[j][mt]);
                  au[j][mt] = mfma16x16x32(a[u][mt], bu[u][j], au[j][mt]);
                }
        }
      }
    };
    // (fragment-packed weights only, as for W2 in the down kernel)
    if (col_ok[0]) {
      if (PW && cnt <= kStreamItemRows) k_loop(std::true_type{});
      else k_loop(std::false_type{});
    }
#pragma unroll
    for (int j = 0; j < CGN; ++j) {
      if constexpr (KS == 1) {
        if (col_ok[j]) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = (t0 + mt) * 16 + 4 * g + i;
              if (r < cnt)
                h[frag_index(row0 + r, c0[j] + m, I)] =
                    f32_to_bf16_bits(silu_mul(ag[j][mt][i], au[j][mt][i]));
            }
        }
      } else {
        // column tile j of every wave through the one LDS buffer
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          red[wave][0][mt][lane] = ag[j][mt];
          red[wave][1][mt][lane] = au[j][mt];
        }
        __syncthreads();
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if ((mt % KS) == ks && t0 + mt < te && col_ok[j]) {
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
              if (r < cnt) h[frag_index(row0 + r, c0[j] + m, I)] = f32_to_bf16_bits(silu_mul(G[i], U[i]));
            }
          }
        }
        __syncthreads();
      }
    }
  }
  return item;
}

// The streaming gate/up launch: a capped grid looping over the units.
template <int KS, int MT, int KU, int CGN, bool FP8, bool PW, bool XD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(FP8 || CGN > 1 ? 2 : 3)))
void gate_up_stream_kernel(
    const uint16_t* __restrict__ xp, const void* __restrict__ w13,
    const float* __restrict__ s13, const int32_t* __restrict__ seg_off,
    const int32_t* __restrict__ seg_cnt, const int32_t* __restrict__ item_seg,
    const int32_t* __restrict__ item_row0, const int32_t* __restrict__ n_items,
    uint16_t* __restrict__ h, int H, int I, int max_items, int n_cg,
    const int32_t* __restrict__ sorted_ids, int topk) {
  static_assert(MT * 16 == kStreamItemRows, "one work item per pass");
  __shared__ floatx4 red[KS > 1 ? 4 : 1][2][MT][kWave];
  const int n_live = min(*n_items, max_items) * n_cg;
  for (int u0 = 0; u0 < n_live; u0 += gridDim.x) {
    const int lid = round_unit(u0, n_live);
    if (lid < 0) continue;
    gate_up_unit<KS, MT, KU, CGN, FP8, PW, XD>(lid, xp, w13, s13, seg_off, seg_cnt, item_seg,
                                             item_row0, h, H, I, n_cg, sorted_ids, topk, red);
  }
}

// Weight-streaming down projection: one block per (work item, 64*NT output
// columns); each wave streams NT 16-row tiles of W2 (full K = I) once for
// the item's (up to MT) 16-row tiles of h.  W2 is the MFMA's A operand, so
// a lane ends with 4 consecutive output columns of one row.  Written as they
// are, a store instruction would cover 16 rows x 64 bytes: every 128-byte
// line of y in two halves from different instructions, which cost decode_e48
// 16 us of its 91 (90.6 -> 74.2 us with the stores taken out in a timing
// copy).  So each wave passes its 16 x 64 tile through its own LDS rows
// first, and a store instruction writes 4 whole rows of the tile (4 x 256
// bytes of fp32, or 4 x 128 of bf16 with fp8 weights).
// Units: (item, column group), n_ng = ceil(H / (64 * NT)) per item (NT = 4).
// Y24: y rows as 24-bit floats (bf16-weight calls where every segment
// streams; the writes of y are what the kernel pays most for besides W2).
// One unit (work item lid of the item table, 256 output columns) of the
// streaming down projection, signals included; returns the unit's item.
template <int MT, int NT, int KU, bool FP8, bool PW, bool Y24>
__device__ __forceinline__ int down_unit(
    int lid, const uint16_t* __restrict__ h, const void* __restrict__ w2,
    const float* __restrict__ s2, const int32_t* __restrict__ seg_off,
    const int32_t* __restrict__ seg_cnt, const int32_t* __restrict__ item_seg,
    const int32_t* __restrict__ item_row0, void* __restrict__ y, int H, int I, int n_ng,
    BlockSignals bs, floatx4 (&ytile)[4][16][17]) {
  static_assert(MT * 16 == kStreamItemRows, "one work item per pass");
  static_assert(NT == 4, "the store pass moves 64-column tiles");
  int ngb, it, item;
  const int e = unit_of_segment(lid, n_ng, item_seg, item_row0, seg_cnt, ngb, it, &item);
  const int cnt = seg_cnt[e];
  const int row0 = seg_off[e];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int n0 = (ngb * 4 + wave) * NT * 16;
  // no barriers in a unit (waves go their own way) unless it raises a
  // completion signal at its end
  if (n0 < H) {
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
      // acc[mt][nt] lane (m, g): row (t0 + mt) 16 + m, columns n0 + 16 nt +
      // 4 g .. + 3.  Through LDS: lane l then holds row 4 q + l / 16 of the
      // tile, columns n0 + 4 (l % 16) .. + 3, for q = 0 .. 3.
      const int lr = lane / 16, lc = lane % 16;
      const bool col_in = n0 + 4 * lc < H;   // H is a multiple of 16
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (t0 + mt >= te) continue;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) ytile[wave][m][4 * nt + g] = acc[mt][nt];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int tr = 4 * q + lr;
          const int r = (t0 + mt) * 16 + tr;
          const floatx4 v = ytile[wave][tr][lc];
          if (r < cnt && col_in) {
            const size_t yi = (size_t)(row0 + r) * H + n0 + 4 * lc;
            if constexpr (Y24) store_y24(y, yi, v);
            else store_y4<FP8>(y, yi, v);
          }
        }
      }
    }
  }
  // the unit's rows (one 64-row block of the segment) x its 256 columns
  if (bs.sig != nullptr)
    signal_rows_done(bs, e, it * kStreamItemRows, min(kStreamItemRows, cnt - it * kStreamItemRows),
                     min(256, H - ngb * 256));
  return item;
}

// The streaming down launch: a capped grid looping over the units (with
// only non-null, just the units whose flag is set).
template <int MT, int NT, int KU, bool FP8, bool PW, bool Y24>
__global__ __launch_bounds__(256) void down_stream_kernel(
    const uint16_t* __restrict__ h, const void* __restrict__ w2,
    const float* __restrict__ s2, const int32_t* __restrict__ seg_off,
    const int32_t* __restrict__ seg_cnt, const int32_t* __restrict__ item_seg,
    const int32_t* __restrict__ item_row0, const int32_t* __restrict__ n_items,
    void* __restrict__ y, int H, int I, int max_items, int n_ng, BlockSignals bs,
    const int32_t* __restrict__ only) {
  static_assert(MT * 16 == kStreamItemRows, "one work item per pass");
  // per wave: one 16-row x 64-column tile of y on its way out (rows padded
  // to 68 floats against bank conflicts); only its own wave touches it
  __shared__ floatx4 ytile[4][16][17];
  const int n_live = min(*n_items, max_items) * n_ng;
  for (int u0 = 0; u0 < n_live; u0 += gridDim.x) {
    const int lid = round_unit(u0, n_live);
    if (lid < 0) continue;
    if (only != nullptr && only[lid] == 0) continue;
    down_unit<MT, NT, KU, FP8, PW, Y24>(lid, h, w2, s2, seg_off, seg_cnt, item_seg, item_row0, y,
                                        H, I, n_ng, bs, ytile);
  }
}

// Gate/up, SiLU*mul and down in one launch ("Step3 Inference Optimization on
// AMD Instinct MI308X", optimisation list: the MoE one-stage kernel), for
// calls where every segment streams, bf16 weights.  A block takes tickets
// from one counter until they run out: the first n_items * n_cg tickets are
// gate/up units, the next n_items * n_ng down units (the units of the two
// streaming kernels, run by the same code).  A gate/up unit stores its h
// columns, releases them at agent scope and counts itself in its item's
// counter; a down unit waits until its item's counter reaches n_cg,
// acquires, and runs.  Tickets are
// handed out in order to blocks that are running, so every gate/up unit a
// down unit waits for is held by a running block that waits for nothing: the
// waits end.  They are also bounded in time (the real-time counter); a wait
// that runs out sets the give-up flag (later waits then skip) and marks its
// unit, which the streaming down kernel's rest pass then runs.  h stays in
// the L2s and memory between the halves, as between the two launches.
template <int MT, int KUG, int KUD, int CGN, bool PW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void expert_mlp_kernel(
    const uint16_t* __restrict__ x, const void* __restrict__ w13, const void* __restrict__ w2,
    const int32_t* __restrict__ seg_off, const int32_t* __restrict__ seg_cnt,
    const int32_t* __restrict__ item_seg, const int32_t* __restrict__ item_row0,
    const int32_t* __restrict__ n_items, uint16_t* __restrict__ h, void* __restrict__ y, int H,
    int I, int max_items, int n_cg, int n_ng, const int32_t* __restrict__ sorted_ids, int topk,
    OneLaunch ol) {
  constexpr int KS = 4;   // bf16 weights; every segment streams: 24-bit y rows
  __shared__ floatx4 red[4][2][MT][kWave];
  __shared__ floatx4 ytile[4][16][17];
  __shared__ int s_tk, s_ok;
  const int n_it = min(*n_items, max_items);
  const int n_gu = n_it * n_cg, n_all = n_gu + n_it * n_ng;
  // The block's next ticket, the same in every thread.  Thread 0's work of
  // an iteration stays between two barriers: with the count-in of a gate/up
  // unit and the next ticket's atomic as one thread-0 stretch across the
  // loop's back edge, the compiler let lane 0 alone leave an inner loop to
  // take the ticket while the block's other lanes went back to the ticket
  // barrier, read the old ticket and ran the same unit again without end.
  auto next_ticket = [&]() -> int {
    if (threadIdx.x == 0) s_tk = atomicAdd(ol.ticket, 1);
    __syncthreads();
    const int t = __builtin_amdgcn_readfirstlane(s_tk);
    __syncthreads();
    return t;
  };
  for (int tk = next_ticket(); tk < n_all; tk = next_ticket()) {
    if (tk < n_gu) {
      const int item = gate_up_unit<KS, MT, KUG, CGN, false, PW, true>(
          tk, x, w13, nullptr, seg_off, seg_cnt, item_seg, item_row0, h, H, I, n_cg, sorted_ids,
          topk, red);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __hip_atomic_fetch_add(ol.item_done + item, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      const int lid = tk - n_gu;
      if (threadIdx.x < kWave) {
        int ngb, it, item;
        (void)unit_of_segment(lid, n_ng, item_seg, item_row0, seg_cnt, ngb, it, &item);
        const uint64_t start = __builtin_amdgcn_s_memrealtime();
        bool ok = true;
        while (__hip_atomic_load(ol.item_done + item, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
               n_cg) {
          if (__hip_atomic_load(ol.giveup, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0 ||
              __builtin_amdgcn_s_memrealtime() - start > (uint64_t)ol.ticks) {
            ok = false;
            break;
          }
          __builtin_amdgcn_s_sleep(8);
        }
        ok = __all(ok);
        if (ok) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        if (threadIdx.x == 0) {
          s_ok = ok ? 1 : 0;
          if (!ok) {
            ol.undone[lid] = 1;
            __hip_atomic_store(ol.giveup, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
      __syncthreads();
      if (s_ok)
        down_unit<MT, 4, KUD, false, PW, true>(lid, h, w2, nullptr, seg_off, seg_cnt, item_seg,
                                               item_row0, y, H, I, n_ng, BlockSignals{nullptr, 0},
                                               ytile);
    }
    __syncthreads();   // the iteration ends here for every thread
  }
}

// Down projection and combine in one launch, for calls where every segment
// streams and the batch holds at most kColsRows assignments (decode): one
// block per 32 output columns runs every segment's rows against its W2
// columns, keeps each assignment's output row (those 32 columns, fp32) in
// LDS, then forms out[t] = sum_j w[t,j] y(t,j) for those columns itself.
// No y rows go to memory and back, and no combine launch follows.  The
// block's 16 waves take the segments in turn; a wave streams its segment's
// two 16-column W2 tiles over K = I (the MFMA A operand) for up to MT = 2
// of the segment's 16-row h tiles at a time.  The sums run over K in the
// order of the streaming down kernel, and the combine in the order of the
// combine kernels (slot j = 0, 1, ...; the shared slot with weight 1).
constexpr int kColsRows = 1216;   // LDS rows: assignments (T (k + n_shared)); 152 KB
constexpr int kMaxSegments = 257;  // 256 routed experts + 1 shared

template <int KU, bool FP8, bool PW>
__global__ __launch_bounds__(1024) void down_cols_kernel(
    const uint16_t* __restrict__ h, const void* __restrict__ w2, const float* __restrict__ s2,
    const int32_t* __restrict__ seg_off, const int32_t* __restrict__ seg_cnt,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ ids,
    const float* __restrict__ wts, int T, int H, int I, int E, int ns, int k,
    uint16_t* __restrict__ out) {
  constexpr int NT = 2, MT = 2, NW = 16;
  // y(a)[32 columns] of assignment a = t (k + ns) + j, as 8 groups of 4
  __shared__ floatx4 ylds[kColsRows][NT * 4];
  // every segment's offset and row count, read once per block (the waves
  // would otherwise wait for them at each segment they start)
  __shared__ int s_off[kMaxSegments], s_cnt[kMaxSegments];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int m = lane % 16, g = lane / 16;
  const int c0 = blockIdx.x * NT * 16;
  const int nseg = E + ns, kk = k + ns;
  constexpr size_t wstep = PW ? 512 : 32;   // elements per MFMA K step
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int i = threadIdx.x; i < nseg; i += blockDim.x) {
    s_off[i] = seg_off[i];
    s_cnt[i] = seg_cnt[i];
  }
  __syncthreads();
  for (int seg = wave; seg < nseg; seg += NW) {
    const int cnt = s_cnt[seg];
    if (cnt == 0) continue;
    const int row0 = s_off[seg];
    size_t wo[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      // a tile past H (H % 32 == 16) re-reads the last one; never combined
      const int n = min(c0 + nt * 16, H - 16);
      if constexpr (PW) wo[nt] = (((size_t)seg * H + n) / 16 * (I / 32)) * 512 + 8 * lane;
      else wo[nt] = ((size_t)seg * H + n + m) * I + 8 * g;
    }
    const float* sc = nullptr;
    if constexpr (FP8) sc = s2 + (size_t)seg * (H / 128) * (I / 128);
    const int ntl = (cnt + 15) >> 4;
    for (int t0 = 0; t0 < ntl; t0 += MT) {
      const uint16_t* ha[MT];
      // list entries of this pass's rows, loaded ahead of the K loop
      int entry[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        ha[mt] = h + ((size_t)(row0 >> 4) + t0 + mt) * 16 * I + 8 * lane;
        const int r = (t0 + mt) * 16 + m;
        entry[mt] = r < cnt ? sorted_ids[row0 + r] : 0;
      }
      floatx4 acc[MT][NT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
      // W2 columns read once by this block (a segment in one pass):
      // non-temporal loads
      auto k_loop = [&](auto nt_tag) {
        constexpr bool kNT = decltype(nt_tag)::value;
        for (int k0 = 0; k0 < I; k0 += 32 * KU) {
          bf16x8 b[KU][NT], a[KU][MT];
#pragma unroll
          for (int u = 0; u < KU; ++u)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              b[u][nt] = load_w8<FP8, kNT>(w2, wo[nt] + (size_t)(k0 / 32 + u) * wstep);
#pragma unroll
          for (int u = 0; u < KU; ++u)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              a[u][mt] = as_bf16x8(t0 + mt < ntl ? ld16(ha[mt] + (size_t)(k0 / 32 + u) * 512) : zero);
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
                if (t0 + mt < ntl)
#pragma unroll
                  for (int nt = 0; nt < NT; ++nt) p[mt][nt] = mfma16x16x32(b[u][nt], a[u][mt], p[mt][nt]);
            const int kb = k0 >> 7;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              const float sv = sc[((size_t)min(c0 + nt * 16, H - 16) / 128) * (I / 128) + kb];
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[mt][nt][i] = fmaf(sv, p[mt][nt][i], acc[mt][nt][i]);
            }
          } else {
#pragma unroll
            for (int u = 0; u < KU; ++u)
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
                if (t0 + mt < ntl)
#pragma unroll
                  for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma16x16x32(b[u][nt], a[u][mt], acc[mt][nt]);
          }
        }
      };
      if (PW && ntl <= MT) k_loop(std::true_type{});
      else k_loop(std::false_type{});
      // acc[mt][nt] lane (m, g): columns c0 + 16 nt + 4 g .. + 3 of the
      // segment's row (t0 + mt) 16 + m, whose list entry is t k + j (t k for
      // the shared segment E)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = (t0 + mt) * 16 + m;
        if (t0 + mt >= ntl || r >= cnt) continue;
        const int tt = entry[mt] / k;
        const int a = seg < E ? entry[mt] + tt * ns : tt * kk + k;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) ylds[a][4 * nt + g] = acc[mt][nt];
      }
    }
  }
  __syncthreads();
  // out[t] for this block's columns: thread -> (token, group of 4 columns)
  for (int i = threadIdx.x; i < T * NT * 4; i += blockDim.x) {
    const int t = i / (NT * 4), q = i - t * (NT * 4);
    const int col = c0 + 4 * q;
    if (col >= H) continue;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    if (ids[(size_t)t * k] >= 0) {
      for (int j = 0; j < kk; ++j) {
        const float wt = j < k ? wts[(size_t)t * k + j] : 1.f;
        const floatx4 v = ylds[t * kk + j][q];
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = fmaf(wt, v[c], acc[c]);
      }
    }
    u32x2 pk;
    pk[0] = pack_bf16x2(acc[0], acc[1]);
    pk[1] = pack_bf16x2(acc[2], acc[3]);
    *reinterpret_cast<u32x2*>(out + (size_t)t * H + col) = pk;
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

// 16-column tiles per wave of the streaming gate/up (the kernel's CGN) with
// fragment-packed weights; row-major weights keep one (their 16-row x 64-byte
// loads: decode_e48 gate/up 198 us with one, 204 with two)
constexpr int kGuCgn = 2;

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
  const int32_t* sorted;   // with x_direct: the sorted row list, and
  int topk;                // its entries per token row
  bool x_direct;
};

template <int KS, int KU, bool FP8, bool PW>
void launch_gu(const GuArgs& a) {
#define MOE_GU(XD)                                                                              \
  hipLaunchKernelGGL((gate_up_stream_kernel<KS, 4, KU, PW ? kGuCgn : 1, FP8, PW, XD>), a.grid,   \
                     dim3(256), 0, a.s, a.xp, a.w13, a.s13, a.seg_off, a.seg_cnt, a.item_seg,    \
                     a.item_row0, a.n_items, a.h, a.H, a.I, a.max_items, a.n_cg, a.sorted, a.topk)
  if (a.x_direct) MOE_GU(true);
  else MOE_GU(false);
#undef MOE_GU
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
  BlockSignals bs;
  const int32_t* only;   // rest pass: just these units
};

template <int KU, bool FP8, bool PW, bool Y24>
void launch_dn(const DnArgs& a) {
  hipLaunchKernelGGL((down_stream_kernel<4, 4, KU, FP8, PW, Y24>), a.grid, dim3(256), 0, a.s, a.h, a.w2,
                     a.s2, a.seg_off, a.seg_cnt, a.item_seg, a.item_row0, a.n_items, a.y, a.H,
                     a.I, a.max_items, a.n_ng, a.bs, a.only);
}

template <bool FP8, bool PW, bool Y24 = false>
void launch_dn_ku(int ku, const DnArgs& a) {
  if (ku == 4) launch_dn<4, FP8, PW, Y24>(a);
  else if (ku == 2) launch_dn<2, FP8, PW, Y24>(a);
  else launch_dn<1, FP8, PW, Y24>(a);
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
                          int H, int I, int k, int bm, int max_rows, bool x_direct, hipStream_t s) {
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
  const int cgw = 4 / ks * (packed ? kGuCgn : 1);   // 16-column tiles per block
  const int n_cg = (I / 16 + cgw - 1) / cgw;
  if (bm % 16 != 0 || (long long)max_items * n_cg > INT_MAX - 8) return hipErrorInvalidValue;
  GuArgs a{dim3(stream_grid(max_items * n_cg)), s,
           static_cast<const uint16_t*>(x_direct ? x : xp), w13, s13, seg_off, seg_cnt, item_seg,
           item_row0, n_items, static_cast<uint16_t*>(h), H, I, max_items, n_cg, sorted_ids, k,
           x_direct};
  if (fp8) {
    if (packed) launch_gu_ks<true, true>(ks, ku, a);
    else launch_gu_ks<true, false>(ks, ku, a);
  } else {
    if (packed) launch_gu_ks<false, true>(ks, ku, a);
    else launch_gu_ks<false, false>(ks, ku, a);
  }
  return hipGetLastError();
}

bool down_cols_fits(int T, int k, int n_shared, int H, int I) {
  return (long long)T * (k + n_shared) <= kColsRows && H % 16 == 0 && I % 32 == 0;
}

hipError_t launch_down_cols(int wkind, bool packed, const void* h, const void* w2,
                            const float* s2, const int32_t* seg_off, const int32_t* seg_cnt,
                            const int32_t* sorted_ids, const int32_t* ids, const float* w,
                            int T, int H, int I, int E, int n_shared, int k, void* out,
                            hipStream_t s) {
  if (wkind == W_F32 || !down_cols_fits(T, k, n_shared, H, I)) return hipErrorInvalidValue;
  const bool fp8 = wkind == W_FP8;
  const int ku = pick_ku(I);
  const dim3 grid((H + 31) / 32);
#define MOE_DC(KU, F, P)                                                                       \
  hipLaunchKernelGGL((down_cols_kernel<KU, F, P>), grid, dim3(1024), 0, s,                      \
                     static_cast<const uint16_t*>(h), w2, s2, seg_off, seg_cnt, sorted_ids, ids, \
                     w, T, H, I, E, n_shared, k, static_cast<uint16_t*>(out))
#define MOE_DC_KU(F, P)            \
  if (ku == 4) MOE_DC(4, F, P);    \
  else if (ku == 2) MOE_DC(2, F, P); \
  else MOE_DC(1, F, P)
  if (fp8) {
    if (packed) { MOE_DC_KU(true, true); } else { MOE_DC_KU(true, false); }
  } else {
    if (packed) { MOE_DC_KU(false, true); } else { MOE_DC_KU(false, false); }
  }
#undef MOE_DC_KU
#undef MOE_DC
  return hipGetLastError();
}

bool expert_mlp_fits(int wkind, int H, int I) {
  return wkind == W_BF16 && H % 512 == 0 && I % 128 == 0;
}

hipError_t launch_expert_mlp(int wkind, bool packed, const void* x, const void* w13,
                             const void* w2, const int32_t* seg_off, const int32_t* seg_cnt,
                             const int32_t* sorted_ids, const int32_t* item_seg,
                             const int32_t* item_row0, const int32_t* n_items, int max_items,
                             void* h, void* y, int H, int I, int k, OneLaunch ol,
                             hipStream_t s) {
  if (!expert_mlp_fits(wkind, H, I)) return hipErrorInvalidValue;
  // the streaming gate/up's shape (a K split in 4, batches of 4 K steps:
  // the same K order, so the same sums); the down's batches of 2 K steps
  // instead of 4 (the same order of its K steps, so the same sums) keep the
  // merged kernel free of register spills
  const int cgn = packed ? kGuCgn : 1;
  const int n_cg = (I / 16 + cgn - 1) / cgn;
  const int n_ng = stream_down_groups(H);
  const long long units = (long long)max_items * (n_cg + n_ng);
  if (units > INT_MAX - 8) return hipErrorInvalidValue;
  // enough blocks for every slot of the chip (two per CU); they loop over
  // the tickets
  const dim3 grid((unsigned)std::min<long long>(round8((int)std::min<long long>(units, 1 << 20)),
                                                512));
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  uint16_t* hb = static_cast<uint16_t*>(h);
#define MOE_MLP(CG, P)                                                                          \
  hipLaunchKernelGGL((expert_mlp_kernel<4, 4, 2, CG, P>), grid, dim3(256), 0, s, xb, w13, w2,     \
                     seg_off, seg_cnt, item_seg, item_row0, n_items, hb, y, H, I, max_items, n_cg, \
                     n_ng, sorted_ids, k, ol)
  if (packed) MOE_MLP(kGuCgn, true);
  else MOE_MLP(1, false);
#undef MOE_MLP
  return hipGetLastError();
}

hipError_t launch_down(int wkind, bool packed, const void* h, const void* w2, const float* s2,
                       const int32_t* block_expert, const int32_t* n_post,
                       const int32_t* seg_off, const int32_t* seg_cnt,
                       const int32_t* item_seg, const int32_t* item_row0,
                       const int32_t* n_items, int max_items, void* y, int H, int I,
                       int bm, int max_rows, bool y24, hipStream_t s, BlockSignals bs,
                       const int32_t* only) {
  if (wkind == W_F32) {
    if (bs.sig != nullptr || only != nullptr) return hipErrorInvalidValue;
    hipLaunchKernelGGL(down_f32_kernel, dim3(max_rows), dim3(256), 0, s,
                       static_cast<const float*>(h), static_cast<const float*>(w2),
                       block_expert, n_post, static_cast<float*>(y), H, I, bm);
    return hipGetLastError();
  }
  const bool fp8 = wkind == W_FP8;
  const int ku = pick_ku(I);
  const int n_ng = stream_down_groups(H);
  if ((long long)max_items * n_ng > INT_MAX - 8) return hipErrorInvalidValue;
  DnArgs a{dim3(stream_grid(max_items * n_ng)), s, static_cast<const uint16_t*>(h), w2, s2,
           seg_off, seg_cnt, item_seg, item_row0, n_items, y, H, I, max_items, n_ng, bs, only};
  if (fp8) {
    if (packed) launch_dn_ku<true, true>(ku, a);
    else launch_dn_ku<true, false>(ku, a);
  } else {
    if (y24) {
      if (packed) launch_dn_ku<false, true, true>(ku, a);
      else launch_dn_ku<false, false, true>(ku, a);
    } else {
      if (packed) launch_dn_ku<false, true>(ku, a);
      else launch_dn_ku<false, false>(ku, a);
    }
  }
  return hipGetLastError();
}

}  // namespace moe
