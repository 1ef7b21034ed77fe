// LDS-tiled MFMA GEMMs for expert segments of many rows (the prefill regime,
// bound by MFMA issue rather than by HBM), and for the router of large
// batches.  Prefill is compute-bound ("Step3 Inference Optimization on AMD
// Instinct MI308X", results: prefill favours the part with more compute), so
// a block works on a 128-row tile of one expert's sorted rows; fp8 weights
// ("AMD Instinct MI355X: ATOM ...": block-scale GEMM; Step3 page: FP8
// blockscale) are dequantised as value(q) * s in fp32 rounded to bf16, except
// in the fp8 down projection, which scales fp32 partial sums.
//
//   gate_up_tall_kernel: 128 rows x (128 gate + 128 up columns), 32x32x16
//     MFMA; weights as the A operand straight from memory, x rows through
//     LDS, epilogue h = SiLU(g) * u.
//   down_tall_kernel / down_tall_f8s_kernel (K = I <= 256, bf16 / fp8 W2): the
//     128 h rows resident in LDS, a sweep over output columns, weights as the
//     A operand; y rows fp32 (bf16 with fp8 weights).
//   gemm_kernel (down for larger I, and the router of more than 128
//     experts): 128 rows x 256 weight rows, both operands staged through LDS
//     per 64-wide K window.
//   router_tall_kernel (router of up to 128 experts): gate_up_tall_kernel's
//     structure, R rows as the A operands.
//
// Fragment order everywhere: an LDS slot (16-row tile, step j) is 64 lanes x
// 16 B, lane g*16 + r holding row r, K = 32 j + 8 g + (0..7) of the window.
// Weights come row-major or already in that order (fragment-packed, one
// contiguous 1 KB / 512 B block per tile and step).
#include <type_traits>

#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {
namespace {

constexpr int kBM = 128;   // rows per block tile
constexpr int kBN = 256;   // weight rows per block tile
constexpr int kKW = 64;    // K window
constexpr int kASlots = kBM / 16 * 2;
constexpr int kBSlots = kBN / 16 * 2;
constexpr int kMaxScaleCols = kMaxGemmK / 128;   // fp8 scale blocks along K

__device__ __forceinline__ int xcd_remap_g(int b, int nb) {
  return (b & 7) * (nb >> 3) + (b >> 3);
}

// Logical id among n_live live blocks of a grid sized for the tile table's
// bound, or -1 for a surplus block: the live ids are remapped over the first
// round_up(n_live, 8) blocks, which spread over all XCDs (remapping over the
// whole grid would leave the XCDs of its surplus tail idle).
__device__ __forceinline__ int live_block_g(int n_live) {
  const int nb = (n_live + 7) & ~7;
  if ((int)blockIdx.x >= nb) return -1;
  const int lid = xcd_remap_g(blockIdx.x, nb);
  return lid < n_live ? lid : -1;
}

enum GemmOp { OP_DOWN = 1, OP_ROUTER = 2 };


// 16 fp8 codes -> 16 bf16 (value * s, rounded), as two 16-byte halves
__device__ __forceinline__ void fp8x16_scaled(u32x4 v, float s, u32x4& lo, u32x4& hi) {
  uint32_t out[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8(v[w], false);
    const auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8(v[w], true);
    out[2 * w] = pack_bf16x2(f01[0] * s, f01[1] * s);
    out[2 * w + 1] = pack_bf16x2(f23[0] * s, f23[1] * s);
  }
  lo = u32x4{out[0], out[1], out[2], out[3]};
  hi = u32x4{out[4], out[5], out[6], out[7]};
}

// Position of lane l's 16 bytes inside an LDS fragment slot of step j.  The
// XOR keeps both the MFMA reads (8 consecutive lanes, fixed l/16) and the
// staging writes (fixed row, 8 (l/16, j) pairs) on 8 distinct 16-byte bank
// groups, so neither side conflicts.
__device__ __forceinline__ int swz(int l, int j) { return l ^ (((l >> 4) << 1) | j); }

// Both operands through LDS; a wave of the 2 x 2 grid owns 64 rows x 8
// weight tiles of 16 rows (32 MFMA 16x16x32 tiles).  Register stages run two
// windows ahead (window w+2 in flight while w is multiplied and w+1 is
// written to LDS), and two LDS buffers alternate.
// OP_DOWN: A = h rows (K = I); weight rows nt*256 + wr of W2.
// OP_ROUTER: A = x rows (padding rows enter as zeros, never used); weight
//   rows nt*256 + wr of R.
// Weight rows past the end are clamped to the last row: they feed only
// output columns that are never stored.  grid.x = round_up(max_tiles * n_nt, 8).
template <int OP, bool FP8, bool PW>
__global__ __launch_bounds__(256) void gemm_kernel(
    const uint16_t* __restrict__ a_src, const void* __restrict__ w,
    const float* __restrict__ wscale, const int32_t* __restrict__ tile_seg,
    const int32_t* __restrict__ tile_row0, const int32_t* __restrict__ n_tiles_ptr,
    const int32_t* __restrict__ seg_off, const int32_t* __restrict__ seg_cnt,
    const uint8_t* __restrict__ valid, void* __restrict__ dst, int H, int I, int n_nt,
    int max_tiles, int T, int E, int ksplit, BlockSignals bs) {
  __shared__ u32x4 abuf[2][kASlots][kWave];   // 2 x 16 KB
  __shared__ u32x4 bbuf[2][kBSlots][kWave];   // 2 x 32 KB
  __shared__ float sscale[2][kMaxScaleCols];  // fp8: the two 128-row scale rows
  const int per_z = max_tiles * n_nt;
  // expert ops: ksplit 1, live blocks from the tile table
  const int lid0 = OP == OP_ROUTER ? xcd_remap_g(blockIdx.x, gridDim.x)
                                   : live_block_g(min(*n_tiles_ptr, max_tiles) * n_nt);
  if (lid0 < 0 || lid0 >= per_z * ksplit) return;
  const int z = lid0 / per_z, lid = lid0 - z * per_z;   // router: K chunk z
  const int mt_id = lid / n_nt, nt = lid - mt_id * n_nt;
  int e = 0, row_base, rows_here;
  if constexpr (OP == OP_ROUTER) {
    row_base = mt_id * kBM;
    rows_here = min(kBM, T - row_base);
  } else {
    if (mt_id >= *n_tiles_ptr) return;
    e = tile_seg[mt_id];
    const int r0 = tile_row0[mt_id];
    row_base = seg_off[e] + r0;        // first sorted row of the tile
    rows_here = min(kBM, seg_cnt[e] - r0);
  }
  const int K = OP == OP_DOWN ? I : H;     // row stride of both operands
  const int Kc = K / ksplit, kofs = z * Kc;  // this block's K range
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int wm = wave >> 1, wn = wave & 1;
  const int m = lane % 16, g = lane / 16;

  // ---- A staging: 4 x 16 B per thread per window (row tid/8 + 32 s,
  // 8-element piece tid%8 at K 8 piece = 32 j + 8 g of the window: lane group
  // g of step j); a wave instruction reads 8 rows x 128 B.
  const int asq = tid & 7;
  uint32_t aoff[4];
  int aslot[4];
  bool aon[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int row = (tid >> 3) + 32 * s;
    const int rr = min(row, rows_here - 1);
    size_t src_row;
    src_row = (size_t)(row_base + rr);
    aon[s] = true;
    if constexpr (OP == OP_ROUTER) aon[s] = valid == nullptr || valid[src_row] != 0;
    aoff[s] = (uint32_t)(src_row * K) + kofs + 8 * asq;
    const int j = asq >> 2, l = (asq & 3) * 16 + (row & 15);
    aslot[s] = ((row >> 4) * 2 + j) * kWave + swz(l, j);
  }

  if constexpr (OP == OP_ROUTER) {
    if (!__syncthreads_or(aon[0] || aon[1] || aon[2] || aon[3])) return;
  }

  // ---- B staging: 16-byte pieces per thread per window, written to LDS
  // slot (tile lt, step j) at the position of their lane.
  //  row-major bf16: 8 pieces (row tid/8 + 32 s, 8 elements at K 8 (tid%8),
  //    as for A);
  //  row-major fp8: 4 pieces (row tid/4 + 64 s, 16 codes at K 16 p, p = tid%4:
  //    lane groups 2 (p%2) and 2 (p%2) + 1 of step p/2);
  //  fragment-packed (PW): piece P = 256 s + tid runs over the window's 32
  //    fragment blocks (lt, j), 1 KB each in bf16 (one lane per piece) or
  //    512 B in fp8 (two lanes per piece).
  constexpr int BP = FP8 ? 4 : 8;
  constexpr uint32_t kWinStride = PW ? 1024 : kKW;   // elements per window
  const void* wexp;
  uint32_t boff[BP];
  int bslot[BP], bslot2[BP], bsr[BP];
  {
    size_t base = 0;
    if constexpr (OP == OP_DOWN) base = (size_t)e * H * I;
    wexp = FP8 ? static_cast<const void*>(static_cast<const uint8_t*>(w) + base)
               : static_cast<const void*>(static_cast<const uint16_t*>(w) + base);
#pragma unroll
    for (int s = 0; s < BP; ++s) {
      if constexpr (PW) {
        const int P = 256 * s + tid;
        const int blk = FP8 ? (P >> 5) : (P >> 6);
        const int l0 = FP8 ? 2 * (P & 31) : (P & 63);
        const int lt = blk >> 1, j = blk & 1;
        int gt;   // 16-row tile of the expert's matrix
        gt = min(nt * 16 + lt, H / 16 - 1);
        boff[s] = ((uint32_t)gt * (K / 32) + kofs / 32 + j) * 512 + 8 * l0;
        bslot[s] = (lt * 2 + j) * kWave + swz(l0, j);
        bslot2[s] = (lt * 2 + j) * kWave + swz(l0 + 1, j);
        bsr[s] = lt >> 3;
      } else {
        const int wr = FP8 ? (tid >> 2) + 64 * s : (tid >> 3) + 32 * s;
        const int piece = FP8 ? (tid & 3) : (tid & 7);
        int grow = nt * kBN + wr;
        const int nrows = OP == OP_DOWN ? H : E;
        grow = min(grow, nrows - 1);
        boff[s] = (uint32_t)grow * K + kofs + (FP8 ? 16 : 8) * piece;
        const int j = FP8 ? (piece >> 1) : (piece >> 2);
        const int g0 = FP8 ? 2 * (piece & 1) : (piece & 3);
        bslot[s] = ((wr >> 4) * 2 + j) * kWave + swz(g0 * 16 + (wr & 15), j);
        bslot2[s] = ((wr >> 4) * 2 + j) * kWave + swz((g0 + 1) * 16 + (wr & 15), j);
        bsr[s] = wr >> 7;
      }
    }
  }
  // fp8: weight rows wr < 128 of the tile use scale row 0, the others row 1
  // (rows nt*256 + 0..255 of W2)
  if constexpr (FP8) {
    const int nkb = K / 128;
    const float* sb = wscale + (size_t)e * (H / 128) * nkb;
    const int sr0 = min(2 * nt, H / 128 - 1);
    const int sr1 = min(2 * nt + 1, H / 128 - 1);
    for (int i = tid; i < 2 * nkb; i += 256)
      sscale[i / nkb][i % nkb] = sb[(size_t)(i < nkb ? sr0 : sr1) * nkb + i % nkb];
  }

  struct Stage {
    u32x4 a[4];
    u32x4 b[BP];
  };
  auto g_load = [&](Stage& S, int win) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      S.a[s] = *reinterpret_cast<const u32x4*>(a_src + aoff[s] + (uint32_t)win * kKW);
#pragma unroll
    for (int s = 0; s < BP; ++s) {
      if constexpr (FP8)
        S.b[s] = *reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(wexp) + boff[s] +
                                                 (uint32_t)win * kWinStride);
      else
        S.b[s] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(wexp) + boff[s] +
                                                 (uint32_t)win * kWinStride);
    }
  };
  auto l_store = [&](const Stage& S, int buf, int win) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int s = 0; s < 4; ++s) (&abuf[buf][0][0])[aslot[s]] = aon[s] ? S.a[s] : zero;
#pragma unroll
    for (int s = 0; s < BP; ++s) {
      if constexpr (FP8) {
        const float sc = sscale[bsr[s]][win >> 1];
        u32x4 lo, hi;
        fp8x16_scaled(S.b[s], sc, lo, hi);
        (&bbuf[buf][0][0])[bslot[s]] = lo;
        (&bbuf[buf][0][0])[bslot2[s]] = hi;
      } else {
        (&bbuf[buf][0][0])[bslot[s]] = S.b[s];
      }
    }
  };

  floatx4 acc[4][8];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[mt][q] = floatx4{0.f, 0.f, 0.f, 0.f};
  // LDS weight tile of wave column wn, tile q
  auto btile = [&](int q) -> int { return wn * 8 + q; };
  auto compute = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int p = swz(lane, j);
      bf16x8 a[4], b[8];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        a[mt] = __builtin_bit_cast(bf16x8, abuf[buf][(wm * 4 + mt) * 2 + j][p]);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        b[q] = __builtin_bit_cast(bf16x8, bbuf[buf][btile(q) * 2 + j][p]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[mt][q] = mfma16x16x32(a[mt], b[q], acc[mt][q]);
    }
  };

  // Two register stages (s0: even windows, s1: odd) and two LDS buffers;
  // the window count is even (the launchers check K % 128 == 0).
  // While window w is multiplied out of LDS, window w+1 waits in registers
  // and window w+2 is in flight; loads past the last window re-read it (in
  // bounds, never stored).  Fixed stage names keep the loop free of register
  // copies, so the compiler waits only on the stage it stores.
  const int nwin = Kc / kKW, last = nwin - 1;
  Stage s0, s1;
  g_load(s0, 0);
  g_load(s1, min(1, last));
  __syncthreads();   // scale rows
  l_store(s0, 0, 0);
  __syncthreads();
  g_load(s0, min(2, last));
  // sched_barrier(0) pins each stage's loads right after the barrier that
  // frees its registers, a full window ahead of their LDS store.
  for (int win = 0; win < nwin; win += 2) {
    compute(0);
    l_store(s1, 1, win + 1);
    __syncthreads();
    g_load(s1, min(win + 3, last));
    __builtin_amdgcn_sched_barrier(0);
    compute(1);
    l_store(s0, 0, win + 2);
    __syncthreads();
    g_load(s0, min(win + 4, last));
    __builtin_amdgcn_sched_barrier(0);
  }

  // epilogue: acc[mt][q] lane (m, g) element i = row wm*64 + mt*16 + 4g + i,
  // column m of LDS weight tile btile(q)
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 64 + mt * 16 + 4 * g + i;
      if (row >= rows_here) continue;
      const int ncols = OP == OP_DOWN ? H : E;
      // router: fp32 partial logits of K chunk z; down: y rows (bf16 with fp8
      // weights)
      const size_t ro = (size_t)(row_base + row) * ncols;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int n = nt * kBN + (wn * 8 + q) * 16 + m;
        if (n >= ncols) continue;
        if constexpr (OP == OP_DOWN && FP8)
          static_cast<uint16_t*>(dst)[ro + n] = f32_to_bf16_bits(acc[mt][q][i]);
        else
          static_cast<float*>(dst)[(size_t)z * T * E + ro + n] = acc[mt][q][i];
      }
    }
  if constexpr (OP == OP_DOWN) {
    // the tile's rows x its kBN columns
    if (bs.sig != nullptr)
      signal_rows_done(bs, e, tile_row0[mt_id], rows_here, min(kBN, H - nt * kBN));
  }
}

// 8 fp8 codes (two dwords) -> 8 bf16 of value(q) * s, rounded to nearest even
__device__ __forceinline__ bf16x8 fp8x8_scaled(u32x2 v, float s) {
  uint32_t out[4];
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8(v[w], false);
    const auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8(v[w], true);
    out[2 * w] = pack_bf16x2(f01[0] * s, f01[1] * s);
    out[2 * w + 1] = pack_bf16x2(f23[0] * s, f23[1] * s);
  }
  return __builtin_bit_cast(bf16x8, u32x4{out[0], out[1], out[2], out[3]});
}

// Down projection of the large segments for K = I = 32 KSTEPS (128 or 256),
// bf16 W2: a block keeps the h rows of one 128-row tile in LDS (MFMA fragment
// order, loaded once) and sweeps a chunk of output columns.  Each wave takes
// 64 output columns at a time: their W2 fragments (the MFMA A operand,
// straight from global memory) against the resident h fragments (the B
// operand), so a lane ends with 8 consecutive output columns of one row.
// grid.x = round_up(max_tiles * n_chunks, 8); chunk = 256 * CPW columns.
constexpr int kTallCPW = 4;   // 64-column tiles per wave per chunk

template <int KSTEPS, bool PW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void down_tall_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ w2,
    const int32_t* __restrict__ tile_seg, const int32_t* __restrict__ tile_row0,
    const int32_t* __restrict__ n_tiles_ptr, const int32_t* __restrict__ seg_off,
    const int32_t* __restrict__ seg_cnt, float* __restrict__ y, int H, int n_chunks,
    int max_tiles, BlockSignals bs) {
  constexpr int I = 32 * KSTEPS;
  __shared__ u32x4 hbuf[8 * KSTEPS][kWave];   // (row tile, step) slots, 1 KB each
  const int lid = live_block_g(min(*n_tiles_ptr, max_tiles) * n_chunks);
  if (lid < 0) return;
  const int mt_id = lid / n_chunks, ch = lid - mt_id * n_chunks;
  const int e = tile_seg[mt_id];
  const int r0 = tile_row0[mt_id];
  const int row_base = seg_off[e] + r0;
  const int rows_here = min(kBM, seg_cnt[e] - r0);
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int m = lane % 16, g = lane / 16;

  // h tile -> LDS: piece P = (row, 8-element piece kp); K = 8 kp = 32 s + 8 gg
#pragma unroll
  for (int i = 0; i < 128 * I / 8 / 256; ++i) {
    const int P = i * 256 + tid;
    const int row = P / (I / 8), kp = P - row * (I / 8);
    const int rr = min(row, rows_here - 1);
    const u32x4 v = ld16(h + (size_t)(row_base + rr) * I + 8 * kp);
    const int st = kp >> 2, gg = kp & 3;
    hbuf[(row >> 4) * KSTEPS + st][swz(gg * 16 + (row & 15), st & 1)] = v;
  }
  const size_t wexp = (size_t)e * H * I;   // first element of expert e's W2
  __syncthreads();

  const int c_beg = ch * 256 * kTallCPW;
  // W2 element offset of this lane's fragment of 16-column group n at step st
  // Tile q of the half at nh: its A row j is output column
  // nh + 8 (j / 4) + 4 q + j % 4, so that a lane's results of the two tiles
  // are 8 consecutive columns of one row (one 16- or 32-byte y store).  Lane
  // (g, m) loads row j = m: W2 row nh + dn, in 16-row block (nh + dn) / 16.
  auto woff = [&](int nh, int q, int st) -> size_t {
    const int dn = 8 * (m >> 2) + 4 * q + (m & 3);
    if constexpr (PW)
      return wexp + ((size_t)((nh + dn) / 16) * KSTEPS + st) * 512 + 8 * (16 * g + (dn & 15));
    else return wexp + (size_t)(nh + dn) * I + 32 * st + 8 * g;
  };
  auto tile_n0 = [&](int t) { return c_beg + (t * 4 + wave) * 64; };
  // A half tile (32 output columns) at a time.  A half's W2 codes are all
  // loaded before the previous half's y stores: the memory counter retires
  // in order, so the MFMAs of a half never wait for those stores (loading
  // only the first half of the K steps early, or a quarter, was slower).
  u32x4 wpre[KSTEPS][2];
  // normal (cached) loads: the tiles of one expert read the same W2 and
  // share it through L2 (non-temporal loads measured 510 against 420 us on
  // prefill_ub_fp8, fetching W2 from HBM once per tile)
  auto w_code = [&](int nh, int st, int q) -> u32x4 { return ld16(w2 + woff(nh, q, st)); };
  auto preload = [&](int nh) {
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st)
#pragma unroll
      for (int q = 0; q < 2; ++q) wpre[st][q] = w_code(nh, st, q);
  };
  floatx4 acc[2][8];
  auto half = [&]() {
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) acc[q][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st) {
      bf16x8 wa[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) wa[q] = as_bf16x8(wpre[st][q]);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const bf16x8 hb = __builtin_bit_cast(bf16x8, hbuf[mt * KSTEPS + st][swz(lane, st & 1)]);
#pragma unroll
        for (int q = 0; q < 2; ++q) acc[q][mt] = mfma16x16x32(wa[q], hb, acc[q][mt]);
      }
    }
  };
  auto store = [&](int nh) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const int row = mt * 16 + m;
      if (row >= rows_here) continue;
      // columns nh + 8 g .. + 7: tile 0's four, then tile 1's
      store_y8<false>(y, (size_t)(row_base + row) * H + nh + 8 * g, acc[0][mt], acc[1][mt]);
    }
  };
  if (tile_n0(0) < H) {
    preload(tile_n0(0));
    // scheduling barriers keep each half's loads, MFMAs and stores in their
    // phase (hoisting the later loads spills registers)
    for (int t = 0; t < kTallCPW; ++t) {
      const int n0 = tile_n0(t);
      half();
      __builtin_amdgcn_sched_barrier(0);
      preload(n0 + 32);
      store(n0);
      __builtin_amdgcn_sched_barrier(0);
      half();
      __builtin_amdgcn_sched_barrier(0);
      const bool more = t + 1 < kTallCPW && tile_n0(t + 1) < H;
      if (more) preload(tile_n0(t + 1));
      store(n0 + 32);
      __builtin_amdgcn_sched_barrier(0);
      if (!more) break;
    }
  }
  if (bs.sig != nullptr)
    signal_rows_done(bs, e, r0, rows_here, min(256 * kTallCPW, H - c_beg));
}

// The same down projection for fp8 W2.  A wave takes a 64-column tile in two
// halves of 64 rows (four 16-column A operands x four 16-row h operands per
// 32-wide K step) that share the tile's W2 codes, so each h fragment read
// from LDS feeds four MFMAs and each y row leaves as one 128-byte line (a
// line stored as two 64-byte halves some time apart reached HBM as two
// writes about a third of the time, measured).  The second half loads the
// next tile's codes of each K step once it has converted its own.  Codes
// become bf16 exactly; the 128x128 block scales multiply the fp32
// accumulators instead (the first K block's partial by s0 / s1 when the
// second begins, the sum by s1 at the end).
// Tile q's A row j is output column 32 (q / 2) + 8 (j / 4) + 4 (q % 2) + j % 4,
// so lane (g, m) ends with columns 8 g .. 8 g + 7 and 32 + 8 g .. 32 + 8 g + 7
// of its row.
// One block's tile in NH 64-row halves: 2, or 1 for a tile of at most 64
// rows (typically an expert's last), which then issues half the MFMAs.
template <int KSTEPS, bool PW, int NH>
__device__ __forceinline__ void down_f8s_tile(
    const uint16_t* __restrict__ h, const uint8_t* __restrict__ w2, const float* __restrict__ s2,
    uint16_t* __restrict__ y, int H, int e, int ch, int row_base, int rows_here,
    u32x4 (*hbuf)[kWave]) {
  constexpr int I = 32 * KSTEPS;
  constexpr int KB = I / 128;      // scale blocks along K
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int m = lane % 16, g = lane / 16;

  const int c_beg = ch * 256 * kTallCPW;
  auto tile_n0 = [&](int t) { return c_beg + (t * 4 + wave) * 64; };
  // wave-uniform bases and 32-bit lane offsets (no 64-bit address per lane)
  const uint8_t* wexp = w2 + (size_t)e * H * I;
  const float* sc = s2 + (size_t)e * (H / 128) * KB;
  auto w_code = [&](int n0, int st, int q) -> u32x2 {
    const uint32_t row = n0 + 32 * (q >> 1) + 8 * (m >> 2) + 4 * (q & 1) + (m & 3);
    uint32_t o;
    if constexpr (PW) o = ((row >> 4) * KSTEPS + st) * 512 + 8 * (16 * g + (row & 15));
    else o = row * I + 32 * st + 8 * g;
    return ld8(wexp + o);
  };
  u32x2 wq[KSTEPS][4];
  float sk[KB];
  auto load_scales = [&](int n0) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sk[kb] = sc[(n0 / 128) * KB + kb];
  };
  const int nt_w = min(kTallCPW, max(0, (H - tile_n0(0) + 255) / 256));
  if (nt_w > 0) {
    load_scales(tile_n0(0));
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st)
#pragma unroll
      for (int q = 0; q < 4; ++q) wq[st][q] = w_code(tile_n0(0), st, q);
  }
#pragma unroll
  for (int i = 0; i < 64 * NH * I / 8 / 256; ++i) {
    const int P = i * 256 + tid;
    const int row = P / (I / 8), kp = P - row * (I / 8);
    const int rr = min(row, rows_here - 1);
    const u32x4 v = ld16(h + (size_t)(row_base + rr) * I + 8 * kp);
    const int st = kp >> 2, gg = kp & 3;
    hbuf[(row >> 4) * KSTEPS + st][swz(gg * 16 + (row & 15), st & 1)] = v;
  }
  __syncthreads();

  uint16_t* ytile = y + (size_t)row_base * H;
  floatx4 acc[4][4];
  for (int t = 0; t < nt_w; ++t) {
    // the next tile's codes are loaded unconditionally (the last tile
    // reloads its own from L2): conditional loads leave register copies at
    // the loop's back edge that wait for every outstanding load and store
    const int n0 = tile_n0(t), n1 = tile_n0(min(t + 1, nt_w - 1));
    // acc = (A0 ratio + A1) fin = s0 A0 + s1 A1 for the two K blocks' partial
    // sums A0, A1.  A zero s1, or one below 2^-64 |s0| (whose ratio could
    // overflow), is replaced by s0 2^-64: an absolute change of at most
    // 2^-63 |s0 A1|.
    float ratio = 1.f, fin = sk[KB - 1];
    if constexpr (KB == 2) {
      const bool tiny = !(fabsf(sk[1]) >= fabsf(sk[0]) * 0x1p-64f) || sk[1] == 0.f;
      ratio = tiny ? 0x1p64f : sk[0] / sk[1];
      fin = tiny ? sk[0] * 0x1p-64f : sk[1];
    }
    load_scales(n1);
#pragma unroll
    for (int half = 0; half < NH; ++half) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[q][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < KSTEPS; ++st) {
        bf16x8 wa[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) wa[q] = fp8x8_to_bf16x8(wq[st][q][0], wq[st][q][1]);
        if (half == NH - 1) {
#pragma unroll
          for (int q = 0; q < 4; ++q) wq[st][q] = w_code(n1, st, q);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const bf16x8 hb =
              __builtin_bit_cast(bf16x8, hbuf[(4 * half + mt) * KSTEPS + st][swz(lane, st & 1)]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (KB == 2 && st == KSTEPS / 2) acc[q][mt] *= ratio;
            acc[q][mt] = mfma16x16x32(wa[q], hb, acc[q][mt]);
          }
        }
        // one K step at a time (hoisting later steps' loads spills registers)
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int row = (4 * half + mt) * 16 + m;
        if (row >= rows_here) continue;
        const uint32_t o = (uint32_t)row * H + n0 + 8 * g;
        store_y8<true>(ytile, o, acc[0][mt] * fin, acc[1][mt] * fin);
        store_y8<true>(ytile, o + 32, acc[2][mt] * fin, acc[3][mt] * fin);
      }
    }
  }
}

template <int KSTEPS, bool PW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void down_tall_f8s_kernel(
    const uint16_t* __restrict__ h, const uint8_t* __restrict__ w2, const float* __restrict__ s2,
    const int32_t* __restrict__ tile_seg, const int32_t* __restrict__ tile_row0,
    const int32_t* __restrict__ n_tiles_ptr, const int32_t* __restrict__ seg_off,
    const int32_t* __restrict__ seg_cnt, uint16_t* __restrict__ y, int H, int n_chunks,
    int max_tiles, BlockSignals bs) {
  __shared__ u32x4 hbuf[8 * KSTEPS][kWave];
  const int lid = live_block_g(min(*n_tiles_ptr, max_tiles) * n_chunks);
  if (lid < 0) return;
  const int mt_id = lid / n_chunks, ch = lid - mt_id * n_chunks;
  const int e = tile_seg[mt_id];
  const int r0 = tile_row0[mt_id];
  const int row_base = seg_off[e] + r0;
  const int rows_here = min(kBM, seg_cnt[e] - r0);
  if (rows_here <= kBM / 2)
    down_f8s_tile<KSTEPS, PW, 1>(h, w2, s2, y, H, e, ch, row_base, rows_here, hbuf);
  else
    down_f8s_tile<KSTEPS, PW, 2>(h, w2, s2, y, H, e, ch, row_base, rows_here, hbuf);
  if (bs.sig != nullptr)
    signal_rows_done(bs, e, r0, rows_here, min(256 * kTallCPW, H - ch * 256 * kTallCPW));
}

// Gate/up of the large segments: 128 sorted rows x (128 gate + the matching
// 128 up columns) per block.  Each wave owns 32 gate and the matching 32 up
// columns, whose W13 fragments it loads straight from memory (the MFMA A
// operands, fp8 dequantised in registers, two 64-wide K windows ahead), while
// the x rows of the window come through LDS (shared by the four waves, two
// buffers, one barrier per window) as four 32-row B operands of the 32x32x16
// MFMA.  The weights keep the 16-row fragment order (a lane reads 16 bytes of
// one of the two 16-row tiles of its 32 rows) and the x window the LDS layout
// of the 16x16x32 kernels: logical K 8 h + i (h = lane / 32) of MFMA step
// (j, sub) is the physical K 32 j + 8 (2 sub + h) + i of the window for both
// operands.  A lane ends with four runs of 4 consecutive gate columns and the
// same up columns of one row, so SiLU(g) * u is formed in registers and
// stored as 8 bytes.
template <bool FP8, bool PW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void gate_up_tall_kernel(
    const uint16_t* __restrict__ x, const void* __restrict__ w13, const float* __restrict__ s13,
    const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ tile_seg,
    const int32_t* __restrict__ tile_row0, const int32_t* __restrict__ n_tiles_ptr,
    const int32_t* __restrict__ seg_off, const int32_t* __restrict__ seg_cnt,
    uint16_t* __restrict__ h, int H, int I, int k, int n_nt, int max_tiles) {
  __shared__ u32x4 xbuf[2][kASlots][kWave];   // 2 x 16 KB
  __shared__ float sscale[2][kMaxScaleCols];  // fp8: gate / up scale rows
  const int lid = live_block_g(min(*n_tiles_ptr, max_tiles) * n_nt);
  if (lid < 0) return;
  const int mt_id = lid / n_nt, nt = lid - mt_id * n_nt;
  const int e = tile_seg[mt_id];
  const int r0 = tile_row0[mt_id];
  const int row_base = seg_off[e] + r0;
  const int rows_here = min(kBM, seg_cnt[e] - r0);
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int l32 = lane % 32, hh = lane / 32, m = lane % 16;

  // x staging: 4 x 16 B per thread per window, as gemm_kernel's A operand
  const int asq = tid & 7;
  uint32_t aoff[4];
  int aslot[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int row = (tid >> 3) + 32 * s;
    const int rr = min(row, rows_here - 1);
    aoff[s] = (uint32_t)((size_t)(sorted_ids[row_base + rr] / k) * H) + 8 * asq;
    const int j = asq >> 2, l = (asq & 3) * 16 + (row & 15);
    aslot[s] = ((row >> 4) * 2 + j) * kWave + swz(l, j);
  }
  // W13 of this wave: q = 0 its 32 gate rows, q = 1 the matching up rows; this
  // lane's row l32, K half hh.  Offsets of MFMA step (j, sub) of window win:
  // woff[q] + (2 win + j) wstep + sub wsub.
  const size_t wexp = (size_t)e * 2 * I * H;
  size_t woff[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = q * I + nt * 128 + wave * 32 + l32;
    if constexpr (PW) woff[q] = wexp + ((size_t)(row / 16) * (H / 32)) * 512 + 8 * (16 * hh + m);
    else woff[q] = wexp + (size_t)row * H + 8 * hh;
  }
  constexpr size_t wstep = PW ? 512 : 32;
  constexpr size_t wsub = PW ? 256 : 16;
  if constexpr (FP8) {
    const int nkb = H / 128;
    const float* sb = s13 + (size_t)e * (2 * I / 128) * nkb;
    for (int i = tid; i < 2 * nkb; i += 256)
      sscale[i / nkb][i % nkb] = sb[(size_t)(i < nkb ? nt : I / 128 + nt) * nkb + i % nkb];
  }

  struct XStage { u32x4 a[4]; };
  struct WStage { typename std::conditional<FP8, u32x2, u32x4>::type c[2][2][2]; };  // [j][sub][q]
  auto x_load = [&](XStage& S, int win) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      S.a[s] = *reinterpret_cast<const u32x4*>(x + aoff[s] + (uint32_t)win * kKW);
  };
  auto x_store = [&](const XStage& S, int buf) {
#pragma unroll
    for (int s = 0; s < 4; ++s) (&xbuf[buf][0][0])[aslot[s]] = S.a[s];
  };
  auto w_load = [&](WStage& W, int win) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const size_t o = woff[q] + (size_t)(2 * win + j) * wstep + sub * wsub;
          if constexpr (FP8) W.c[j][sub][q] = ld8(static_cast<const uint8_t*>(w13) + o);
          else W.c[j][sub][q] = ld16(static_cast<const uint16_t*>(w13) + o);
        }
  };
  floatx16 acc[2][4];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[q][n][r] = 0.f;
  auto compute = [&](const WStage& W, int buf, int win) {
    float sg = 1.f, su = 1.f;
    if constexpr (FP8) {
      sg = sscale[0][win >> 1];
      su = sscale[1][win >> 1];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        bf16x8 wa[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          if constexpr (FP8) wa[q] = fp8x8_scaled(W.c[j][sub][q], q == 0 ? sg : su);
          else wa[q] = as_bf16x8(W.c[j][sub][q]);
        }
        // token row 32 n + l32 (16-row tile 2 n + l32 / 16), K group 2 sub + hh
        const int xl = swz(16 * (2 * sub + hh) + m, j);
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const bf16x8 xb =
              __builtin_bit_cast(bf16x8, xbuf[buf][(2 * n + l32 / 16) * 2 + j][xl]);
#pragma unroll
          for (int q = 0; q < 2; ++q) acc[q][n] = mfma32x32x16(wa[q], xb, acc[q][n]);
        }
      }
  };

  // windows in pairs (the count H / 64 is even): stage names fixed, loads two
  // windows ahead (past the end they re-read the last window, unused)
  const int nwin = H / kKW, last = nwin - 1;
  XStage xs0, xs1;
  WStage ws0, ws1;
  x_load(xs0, 0);
  w_load(ws0, 0);
  x_load(xs1, min(1, last));
  w_load(ws1, min(1, last));
  __syncthreads();   // scale rows
  x_store(xs0, 0);
  __syncthreads();
  x_load(xs0, min(2, last));
  for (int win = 0; win < nwin; win += 2) {
    compute(ws0, 0, win);
    w_load(ws0, min(win + 2, last));
    x_store(xs1, 1);
    __syncthreads();
    x_load(xs1, min(win + 3, last));
    __builtin_amdgcn_sched_barrier(0);
    compute(ws1, 1, win + 1);
    w_load(ws1, min(win + 3, last));
    x_store(xs0, 0);
    __syncthreads();
    x_load(xs0, min(win + 4, last));
    __builtin_amdgcn_sched_barrier(0);
  }

  // acc[q][n] lane (l32, hh) register r: column 32 wave + 8 (r / 4) + 4 hh +
  // r % 4 of the block's 128 (gate q = 0, up q = 1), sorted row 32 n + l32
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int row = 32 * n + l32;
    if (row >= rows_here) continue;
    uint16_t* hr = h + (size_t)(row_base + row) * I + nt * 128 + wave * 32 + 4 * hh;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x2 pk;
      pk[0] = pack_bf16x2(silu_mul(acc[0][n][4 * c], acc[1][n][4 * c]),
                          silu_mul(acc[0][n][4 * c + 1], acc[1][n][4 * c + 1]));
      pk[1] = pack_bf16x2(silu_mul(acc[0][n][4 * c + 2], acc[1][n][4 * c + 2]),
                          silu_mul(acc[0][n][4 * c + 3], acc[1][n][4 * c + 3]));
      *reinterpret_cast<u32x2*>(hr + 8 * c) = pk;
    }
  }
}

// Gate/up of the large segments with fp8 weights on the fp8 MFMA (32x32x64,
// e4m3 x e4m3, fp32 accumulation).  The token rows come as two e4m3 terms
// that share one power-of-two row scale, x = s_t (hi + lo) (xq_split_kernel),
// so each 64-wide K step of W13 codes meets both terms and both MFMAs
// accumulate into one sum: the same MFMA cycles as the bf16 instruction on
// dequantised weights, with the weights' codes used as they are.  Block,
// wave and epilogue layout as gate_up_tall_kernel: 128 sorted rows x (128
// gate + the matching 128 up columns); each wave's 32 + 32 weight rows are
// the A operands straight from memory (a lane holds 32 codes of one row:
// K 32 hh .. 32 hh + 31 of the step, hh = lane / 32), the x codes of each
// 64-wide K window come through two LDS buffers (rows 80 bytes apart: the
// 16-byte operand reads of 8 consecutive lanes hit distinct banks) as the B
// operands (token 32 n + lane % 32, the same K bytes).
// Block scales of the weights (one per 128 rows x 128 K): the accumulator
// holds the sum in units of a current scale c, multiplied by c_old / c_new
// when a 128-wide K block begins; a scale smaller in magnitude than 2^-64 of
// the row block's largest (zero included) is raised to that bound, which
// keeps every ratio below 2^64 and the accumulator finite.  At the end the
// sum is multiplied by c and by the row scale s_t.
constexpr int kF8KW = 64;            // K window: one fp8 MFMA K step
constexpr int kF8RS = kF8KW + 16;    // LDS row stride of the x codes, bytes

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;

template <bool PW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void gate_up_f8x_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ sx, const uint8_t* __restrict__ w13,
    const float* __restrict__ s13, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ tile_seg, const int32_t* __restrict__ tile_row0,
    const int32_t* __restrict__ n_tiles_ptr, const int32_t* __restrict__ seg_off,
    const int32_t* __restrict__ seg_cnt, uint16_t* __restrict__ h, int T, int H, int I, int k,
    int n_nt, int max_tiles) {
  __shared__ __attribute__((aligned(16))) uint8_t xbuf[2][2][kBM][kF8RS];  // [buf][term][row][K]
  __shared__ float wsc[2][kMaxScaleCols];   // gate / up scale rows of weight row block nt
  __shared__ float wfloor[2];
  __shared__ float tsc[kBM];                // row scales of the tile's tokens
  const int lid = live_block_g(min(*n_tiles_ptr, max_tiles) * n_nt);
  if (lid < 0) return;
  const int mt_id = lid / n_nt, nt = lid - mt_id * n_nt;
  const int e = tile_seg[mt_id];
  const int r0 = tile_row0[mt_id];
  const int row_base = seg_off[e] + r0;
  const int rows_here = min(kBM, seg_cnt[e] - r0);
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int l32 = lane % 32, hh = lane / 32;

  // x staging: per window 2 terms x 128 rows x 64 B = 16 KB; a thread moves
  // 16-byte piece tid % 4 of rows tid / 4 and tid / 4 + 64, both terms
  const int xp = tid & 3;
  uint32_t xoff[2];
  int xrow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    xrow[i] = (tid >> 2) + 64 * i;
    const int rr = min(xrow[i], rows_here - 1);
    xoff[i] = (uint32_t)((size_t)(sorted_ids[row_base + rr] / k) * H) + 16 * xp;
  }
  const uint8_t* xlo = xq + (size_t)T * H;
  if (tid < kBM) tsc[tid] = sx[sorted_ids[row_base + min(tid, rows_here - 1)] / k];
  const int nkb = H / 128;
  {
    const float* sb = s13 + (size_t)e * (2 * I / 128) * nkb;
    for (int i = tid; i < 2 * nkb; i += 256)
      wsc[i / nkb][i % nkb] = sb[(size_t)(i < nkb ? nt : I / 128 + nt) * nkb + i % nkb];
  }

  // A operands: gate (q = 0) / up (q = 1) row of this lane, 32 codes at
  // K 64 w + 32 hh of window w
  const size_t wexp = (size_t)e * 2 * I * H;
  size_t woff[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = q * I + nt * 128 + wave * 32 + l32;
    if constexpr (PW) woff[q] = wexp + ((size_t)(row / 16) * (H / 32) + hh) * 512 + 8 * (row % 16);
    else woff[q] = wexp + (size_t)row * H + 32 * hh;
  }
  struct WStage { u32x4 c[2][2]; };   // [q][16-byte half]
  struct XStage { u32x4 a[2][2]; };   // [row i][term]
  auto w_load = [&](WStage& W, int win) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if constexpr (PW) {
        // fragment order: the 32 codes are four 8-byte pieces, 128 bytes apart
        const uint8_t* p = w13 + woff[q] + (size_t)win * 1024;
        const u32x2 a = ld8(p), b = ld8(p + 128), c = ld8(p + 256), d = ld8(p + 384);
        W.c[q][0] = u32x4{a[0], a[1], b[0], b[1]};
        W.c[q][1] = u32x4{c[0], c[1], d[0], d[1]};
      } else {
        const uint8_t* p = w13 + woff[q] + (size_t)win * kF8KW;
        W.c[q][0] = ld16(p);
        W.c[q][1] = ld16(p + 16);
      }
    }
  };
  auto x_load = [&](XStage& S, int win) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      S.a[i][0] = ld16(xq + xoff[i] + (uint32_t)win * kF8KW);
      S.a[i][1] = ld16(xlo + xoff[i] + (uint32_t)win * kF8KW);
    }
  };
  auto x_store = [&](const XStage& S, int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        *reinterpret_cast<u32x4*>(&xbuf[buf][t][xrow[i]][16 * xp]) = S.a[i][t];
  };

  floatx16 acc[2][4];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[q][n][r] = 0.f;
  float cur[2] = {1.f, 1.f};   // the accumulators' current scale unit
  auto compute = [&](const WStage& W, int buf, int win) {
    if ((win & 1) == 0) {
      // a 128-wide K block begins: move the sums to its scale
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float sc = wsc[q][win >> 1];
        const float se = fabsf(sc) < wfloor[q] ? (sc < 0.f ? -wfloor[q] : wfloor[q]) : sc;
        const float ratio = cur[q] / se;
        cur[q] = se;
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[q][n][r] *= ratio;
      }
    }
    i32x8 a[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      a[q] = i32x8{(int)W.c[q][0][0], (int)W.c[q][0][1], (int)W.c[q][0][2], (int)W.c[q][0][3],
                   (int)W.c[q][1][0], (int)W.c[q][1][1], (int)W.c[q][1][2], (int)W.c[q][1][3]};
    }
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint8_t* xr = &xbuf[buf][t][32 * n + l32][32 * hh];
        const u32x4 b0 = *reinterpret_cast<const u32x4*>(xr);
        const u32x4 b1 = *reinterpret_cast<const u32x4*>(xr + 16);
        const i32x8 b = i32x8{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                              (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
#pragma unroll
        for (int q = 0; q < 2; ++q)
          acc[q][n] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[q], b, acc[q][n], 0, 0, 0,
                                                                     0, 0, 0);
      }
  };

  // windows in pairs (H / 64 is even): stage names fixed, loads two windows
  // ahead (past the end they re-read the last window, unused)
  const int nwin = H / kF8KW, last = nwin - 1;
  XStage xs0, xs1;
  WStage ws0, ws1;
  x_load(xs0, 0);
  w_load(ws0, 0);
  x_load(xs1, min(1, last));
  w_load(ws1, min(1, last));
  __syncthreads();   // scale rows and token scales in LDS
  if (wave < 2) {
    // bound below which a block scale is raised: 2^-64 of the row block's
    // largest magnitude (the smallest normal float if all are zero)
    float m = 0.f;
    for (int i = lane; i < nkb; i += kWave) m = fmaxf(m, fabsf(wsc[wave][i]));
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (lane == 0) wfloor[wave] = fmaxf(m * 0x1p-64f, 0x1p-126f);
  }
  x_store(xs0, 0);
  __syncthreads();
  x_load(xs0, min(2, last));
  for (int win = 0; win < nwin; win += 2) {
    compute(ws0, 0, win);
    w_load(ws0, min(win + 2, last));
    x_store(xs1, 1);
    __syncthreads();
    x_load(xs1, min(win + 3, last));
    __builtin_amdgcn_sched_barrier(0);
    compute(ws1, 1, win + 1);
    w_load(ws1, min(win + 3, last));
    x_store(xs0, 0);
    __syncthreads();
    x_load(xs0, min(win + 4, last));
    __builtin_amdgcn_sched_barrier(0);
  }

  // acc[q][n] lane (l32, hh) register r: column 32 wave + 8 (r / 4) + 4 hh +
  // r % 4 of the block's 128 (gate q = 0, up q = 1), sorted row 32 n + l32
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int row = 32 * n + l32;
    if (row >= rows_here) continue;
    const float fg = cur[0] * tsc[row], fu = cur[1] * tsc[row];
    uint16_t* hr = h + (size_t)(row_base + row) * I + nt * 128 + wave * 32 + 4 * hh;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x2 pk;
      pk[0] = pack_bf16x2(silu_mul(acc[0][n][4 * c] * fg, acc[1][n][4 * c] * fu),
                          silu_mul(acc[0][n][4 * c + 1] * fg, acc[1][n][4 * c + 1] * fu));
      pk[1] = pack_bf16x2(silu_mul(acc[0][n][4 * c + 2] * fg, acc[1][n][4 * c + 2] * fu),
                          silu_mul(acc[0][n][4 * c + 3] * fg, acc[1][n][4 * c + 3] * fu));
      *reinterpret_cast<u32x2*>(hr + 8 * c) = pk;
    }
  }
}

// Router logits of large batches with gate_up_tall_kernel's structure:
// 128 consecutive token rows x 256 experts per block over one K chunk z of
// ks.  Each wave owns 64 experts: two 32-row A operands of R (row-major,
// straight from memory), while the x rows of each 64-wide K window come
// through LDS as four 32-row B operands of the 32x32x16 MFMA.  Padding rows
// are never read (zeros in LDS) and their partials are not written; a tile
// with no valid row exits.  part[z][t][e] fp32.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void router_tall_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ valid,
    const uint16_t* __restrict__ R, float* __restrict__ part, int T, int H, int E, int n_nt,
    int n_tiles, int ks) {
  __shared__ u32x4 xbuf[2][kASlots][kWave];   // 2 x 16 KB
  const int lid = xcd_remap_g(blockIdx.x, gridDim.x);
  if (lid >= n_tiles * n_nt * ks) return;
  // tile-major: the K chunks and expert groups of one row tile are neighbours
  const int tile = lid / (n_nt * ks), rest = lid - tile * (n_nt * ks);
  const int nt = rest / ks, z = rest - nt * ks;
  const int row_base = tile * kBM;
  const int rows_here = min(kBM, T - row_base);
  const int Kc = H / ks, kofs = z * Kc;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int l32 = lane % 32, hh = lane / 32, m = lane % 16;

  // x staging: 4 x 16 B per thread per window (rows tid / 8 + 32 s)
  const int asq = tid & 7;
  uint32_t aoff[4];
  int aslot[4];
  bool aon[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int row = (tid >> 3) + 32 * s;
    const int rr = min(row, rows_here - 1);
    aon[s] = row < rows_here && (valid == nullptr || valid[row_base + rr] != 0);
    aoff[s] = (uint32_t)((size_t)(row_base + rr) * H) + kofs + 8 * asq;
    const int j = asq >> 2, l = (asq & 3) * 16 + (row & 15);
    aslot[s] = ((row >> 4) * 2 + j) * kWave + swz(l, j);
  }
  if (!__syncthreads_or(aon[0] || aon[1] || aon[2] || aon[3])) return;
  // R rows of this wave: experts e0 + 32 q + l32, K half hh of each step
  const int e0 = nt * 256 + wave * 64;
  bool ron[2];
  size_t roff[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = e0 + 32 * q + l32;
    ron[q] = e < E;
    roff[q] = (size_t)(ron[q] ? e : 0) * H + kofs + 8 * hh;
  }
  const bool wave_on = e0 < E;
  const u32x4 zero = {0u, 0u, 0u, 0u};

  struct XStage { u32x4 a[4]; };
  struct WStage { u32x4 c[2][2][2]; };   // [j][sub][q]
  auto x_load = [&](XStage& S, int win) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      S.a[s] = aon[s] ? *reinterpret_cast<const u32x4*>(x + aoff[s] + (uint32_t)win * kKW) : zero;
  };
  auto x_store = [&](const XStage& S, int buf) {
#pragma unroll
    for (int s = 0; s < 4; ++s) (&xbuf[buf][0][0])[aslot[s]] = S.a[s];
  };
  auto w_load = [&](WStage& W, int win) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int q = 0; q < 2; ++q)
          W.c[j][sub][q] = ron[q] ? ld16(R + roff[q] + (size_t)win * kKW + 32 * j + 16 * sub) : zero;
  };
  floatx16 acc[2][4];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[q][n][r] = 0.f;
  auto compute = [&](const WStage& W, int buf) {
    if (!wave_on) return;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int xl = swz(16 * (2 * sub + hh) + m, j);
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const bf16x8 xb =
              __builtin_bit_cast(bf16x8, xbuf[buf][(2 * n + l32 / 16) * 2 + j][xl]);
#pragma unroll
          for (int q = 0; q < 2; ++q) acc[q][n] = mfma32x32x16(as_bf16x8(W.c[j][sub][q]), xb, acc[q][n]);
        }
      }
  };

  // windows in pairs (Kc / 64 is even: H % (128 ks) == 0)
  const int nwin = Kc / kKW, last = nwin - 1;
  XStage xs0, xs1;
  WStage ws0, ws1;
  x_load(xs0, 0);
  w_load(ws0, 0);
  x_load(xs1, min(1, last));
  w_load(ws1, min(1, last));
  x_store(xs0, 0);
  __syncthreads();
  x_load(xs0, min(2, last));
  for (int win = 0; win < nwin; win += 2) {
    compute(ws0, 0);
    w_load(ws0, min(win + 2, last));
    x_store(xs1, 1);
    __syncthreads();
    x_load(xs1, min(win + 3, last));
    __builtin_amdgcn_sched_barrier(0);
    compute(ws1, 1);
    w_load(ws1, min(win + 3, last));
    x_store(xs0, 0);
    __syncthreads();
    x_load(xs0, min(win + 4, last));
    __builtin_amdgcn_sched_barrier(0);
  }
  if (!wave_on) return;

  // acc[q][n] lane (l32, hh) register r: expert e0 + 32 q + 8 (r / 4) + 4 hh +
  // r % 4, token row 32 n + l32
  float* dst = part + (size_t)z * T * E;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int row = 32 * n + l32;
    if (row >= rows_here) continue;
    if (valid != nullptr && valid[row_base + row] == 0) continue;
    float* pr = dst + (size_t)(row_base + row) * E;
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int e = e0 + 32 * q + 8 * c + 4 * hh;
        if ((E & 3) == 0 && e + 3 < E) {
          *reinterpret_cast<floatx4*>(pr + e) =
              floatx4{acc[q][n][4 * c], acc[q][n][4 * c + 1], acc[q][n][4 * c + 2], acc[q][n][4 * c + 3]};
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (e + i < E) pr[e + i] = acc[q][n][4 * c + i];
        }
      }
  }
}

int round8g(int v) { return (v + 7) / 8 * 8; }

template <int OP, bool FP8, bool PW>
void launch_gemm(dim3 grid, hipStream_t s, const uint16_t* a, const void* w, const float* ws,
                 const int32_t* tseg, const int32_t* trow, const int32_t* ntiles,
                 const int32_t* seg_off, const int32_t* seg_cnt, void* dst, int H, int I,
                 int n_nt, int max_tiles, BlockSignals bs) {
  hipLaunchKernelGGL((gemm_kernel<OP, FP8, PW>), grid, dim3(256), 0, s, a, w, ws, tseg, trow,
                     ntiles, seg_off, seg_cnt, nullptr, dst, H, I, n_nt, max_tiles, 0, 0, 1, bs);
}

template <int OP>
void launch_gemm_w(bool fp8, bool packed, dim3 grid, hipStream_t s, const uint16_t* a,
                   const void* w, const float* ws, const int32_t* tseg, const int32_t* trow,
                   const int32_t* ntiles, const int32_t* seg_off, const int32_t* seg_cnt,
                   void* dst, int H, int I, int n_nt, int max_tiles, BlockSignals bs) {
#define MOE_GEMM_ARGS grid, s, a, w, ws, tseg, trow, ntiles, seg_off, seg_cnt, dst, H, I, n_nt, \
                      max_tiles, bs
  if (fp8) {
    if (packed) launch_gemm<OP, true, true>(MOE_GEMM_ARGS);
    else launch_gemm<OP, true, false>(MOE_GEMM_ARGS);
  } else {
    if (packed) launch_gemm<OP, false, true>(MOE_GEMM_ARGS);
    else launch_gemm<OP, false, false>(MOE_GEMM_ARGS);
  }
#undef MOE_GEMM_ARGS
}

}  // namespace

hipError_t launch_gate_up_gemm(bool fp8, bool packed, const void* x, const void* w13,
                               const float* s13, const int32_t* sorted_ids,
                               const int32_t* tile_seg, const int32_t* tile_row0,
                               const int32_t* n_tiles, const int32_t* seg_off,
                               const int32_t* seg_cnt, void* h, int H, int I, int k,
                               int max_tiles, const uint8_t* xq, const float* sx, int T,
                               hipStream_t s) {
  if (H % 128 != 0 || I % 128 != 0 || H > kMaxGemmK) return hipErrorInvalidValue;
  const int n_nt = I / 128;
  const dim3 grid(round8g(max_tiles * n_nt));
  if (fp8 && xq != nullptr) {
    // fp8 MFMA on the two-term token codes
    const uint8_t* wq = static_cast<const uint8_t*>(w13);
    uint16_t* hb = static_cast<uint16_t*>(h);
    if (packed)
      hipLaunchKernelGGL((gate_up_f8x_kernel<true>), grid, dim3(256), 0, s, xq, sx, wq, s13,
                         sorted_ids, tile_seg, tile_row0, n_tiles, seg_off, seg_cnt, hb, T, H, I,
                         k, n_nt, max_tiles);
    else
      hipLaunchKernelGGL((gate_up_f8x_kernel<false>), grid, dim3(256), 0, s, xq, sx, wq, s13,
                         sorted_ids, tile_seg, tile_row0, n_tiles, seg_off, seg_cnt, hb, T, H, I,
                         k, n_nt, max_tiles);
    return hipGetLastError();
  }
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  uint16_t* hb = static_cast<uint16_t*>(h);
#define MOE_GUT(F8, P)                                                                      \
  hipLaunchKernelGGL((gate_up_tall_kernel<F8, P>), grid, dim3(256), 0, s, xb, w13, s13,     \
                     sorted_ids, tile_seg, tile_row0, n_tiles, seg_off, seg_cnt, hb, H, I, k, \
                     n_nt, max_tiles)
  if (fp8) { if (packed) MOE_GUT(true, true); else MOE_GUT(true, false); }
  else { if (packed) MOE_GUT(false, true); else MOE_GUT(false, false); }
#undef MOE_GUT
  return hipGetLastError();
}

hipError_t launch_down_gemm(bool fp8, bool packed, const void* h, const void* w2,
                            const float* s2, const int32_t* tile_seg, const int32_t* tile_row0,
                            const int32_t* n_tiles, const int32_t* seg_off,
                            const int32_t* seg_cnt, void* y, int H, int I, int max_tiles,
                            hipStream_t s, BlockSignals bs) {
  if (I % 128 != 0 || I > kMaxGemmK) return hipErrorInvalidValue;
  if (I == 128 || I == 256) {
    const int n_chunks = (H + 256 * kTallCPW - 1) / (256 * kTallCPW);
    const dim3 grid(round8g(max_tiles * n_chunks));
    const uint16_t* hb = static_cast<const uint16_t*>(h);
#define MOE_TALL(KS, P)                                                                     \
  hipLaunchKernelGGL((down_tall_kernel<KS, P>), grid, dim3(256), 0, s, hb,                    \
                     static_cast<const uint16_t*>(w2), tile_seg, tile_row0, n_tiles, seg_off,  \
                     seg_cnt, static_cast<float*>(y), H, n_chunks, max_tiles, bs)
#define MOE_TALL8(KS, P)                                                                    \
  hipLaunchKernelGGL((down_tall_f8s_kernel<KS, P>), grid, dim3(256), 0, s, hb,                \
                     static_cast<const uint8_t*>(w2), s2, tile_seg, tile_row0, n_tiles, seg_off, \
                     seg_cnt, static_cast<uint16_t*>(y), H, n_chunks, max_tiles, bs)
    if (I == 128) {
      if (fp8) { if (packed) MOE_TALL8(4, true); else MOE_TALL8(4, false); }
      else { if (packed) MOE_TALL(4, true); else MOE_TALL(4, false); }
    } else {
      if (fp8) { if (packed) MOE_TALL8(8, true); else MOE_TALL8(8, false); }
      else { if (packed) MOE_TALL(8, true); else MOE_TALL(8, false); }
    }
#undef MOE_TALL
#undef MOE_TALL8
    return hipGetLastError();
  }
  const int n_nt = (H + kBN - 1) / kBN;
  launch_gemm_w<OP_DOWN>(fp8, packed, dim3(round8g(max_tiles * n_nt)), s,
                         static_cast<const uint16_t*>(h), w2, s2, tile_seg, tile_row0, n_tiles,
                         seg_off, seg_cnt, y, H, I, n_nt, max_tiles, bs);
  return hipGetLastError();
}

hipError_t launch_router_gemm(const void* x, const uint8_t* valid, const void* R,
                              float* part, int T, int H, int E, int ks, hipStream_t s) {
  if (ks < 1 || H % (128 * ks) != 0) return hipErrorInvalidValue;
  const int tiles = (T + kBM - 1) / kBM;
  if (E <= 128) {
    // gemm_kernel's 256-expert tiles would spend most of their MFMA work on
    // absent experts; router_tall_kernel's waves own 64 experts each and the
    // waves without any skip their MFMAs (gather_padded_e48, E = 48: 52 ->
    // 34 us; with E = 256 it measured 71 us against gemm_kernel's 63 us)
    dim3 grid(round8g(tiles * ks));
    hipLaunchKernelGGL(router_tall_kernel, grid, dim3(256), 0, s, static_cast<const uint16_t*>(x),
                       valid, static_cast<const uint16_t*>(R), part, T, H, E, 1, tiles, ks);
    return hipGetLastError();
  }
  const int n_nt = (E + kBN - 1) / kBN;
  dim3 grid(round8g(tiles * n_nt * ks));
  hipLaunchKernelGGL((gemm_kernel<OP_ROUTER, false, false>), grid, dim3(256), 0, s,
                     static_cast<const uint16_t*>(x), R, nullptr, nullptr, nullptr, nullptr,
                     nullptr, nullptr, valid, part, H, 0, n_nt, tiles, T, E, ks,
                     BlockSignals{nullptr, 0});
  return hipGetLastError();
}

}  // namespace moe
