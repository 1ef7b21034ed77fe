// Host-side launchers of the gfx950 kernels (internal to libmoe_amd).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---- route -----------------------------------------------------------------
// Partial router logits: part[z][t][e] = sum over the z-th K chunk of
// x[t,:] * R[e,:].  bf16 inputs use MFMA; fp32 inputs use a plain FMA loop
// (ks must be 1 then).  Rows with valid == 0 are not read; their partials
// may be left unwritten (the top-k kernel never reads them).
hipError_t launch_route_logits(bool bf16, const void* x, const uint8_t* valid,
                               const void* R, float* part, int T, int H, int E,
                               int ks, hipStream_t s);
// Sum the ks partials (fixed order), pick top-k, softmax over the picks.
hipError_t launch_route_topk(const float* part, int ks, const uint8_t* valid,
                             int T, int E, int k, int32_t* ids, float* w,
                             float* logits_out, hipStream_t s);

// ---- align -----------------------------------------------------------------
// Stable counting sort of assignments by expert (n_shared extra always-on
// segments of every valid row when n_shared > 0).  slot_pos (position of each
// assignment in the sorted list) and seg_count (unpadded rows per segment)
// may be null.
// With tile_seg non-null, also lists the 128-row tiles (segment, first row)
// of every segment with more than big_thr rows, and their number; fewer
// than min_tiles tiles (too few blocks to fill the chip) are dropped and
// n_tiles is 0, leaving every segment to the streaming kernels.  With
// item_seg non-null, lists the streaming kernels' work items: for every
// non-empty segment they take, its rows in groups of 64 (segment, first row),
// and their number.
// Batches of more than 8192 assignments use align_spans(T, k, n_shared) spans
// and need span_buf (that many x (E + n_shared) int32); with span_buf null
// one block does the whole list.
int align_spans(int T, int k, int n_shared);
hipError_t launch_align(const int32_t* ids, int T, int k, int E, int n_shared,
                        int bm, int32_t* sorted_ids, int32_t* block_expert,
                        int32_t* offsets, int32_t* n_post, int32_t* slot_pos,
                        int32_t* seg_count, int big_thr, int min_tiles, int32_t* tile_seg,
                        int32_t* tile_row0, int32_t* n_tiles, int32_t* span_buf,
                        int32_t* item_seg, int32_t* item_row0, int32_t* n_items,
                        hipStream_t s);

// ---- expert GEMMs ------------------------------------------------------------
enum WKind { W_F32 = 0, W_BF16 = 1, W_FP8 = 2 };

// Rows of one work item of the streaming kernels (four 16-row MFMA tiles).
constexpr int kStreamItemRows = 64;
// Bound on the work items of a batch of n_rows sorted assignments over nseg
// segments.
inline int max_stream_items(long long n_rows, int nseg) {
  return (int)(n_rows / kStreamItemRows + (n_rows < nseg ? n_rows : nseg));
}

// Largest K (H for gate/up, I for down) the tiled GEMM kernels take (fp8:
// their per-block table of 128-wide scale blocks).
constexpr int kMaxGemmK = 16384;

// bf16 streaming path: x rows of the sorted rows of the streaming kernels'
// segments, packed in MFMA fragment order into xp (max_rows x H bf16, 16-row
// tiles; padding rows 0).  bm must be 16.
hipError_t launch_pack_x(const void* x, const int32_t* sorted_ids, const int32_t* block_expert,
                         const int32_t* n_post, const int32_t* seg_cnt, int big_thr,
                         const int32_t* gemm_tiles, void* xp, int H, int k, int bm,
                         int max_rows, hipStream_t s);
// h[r, :] = SiLU(W_gate x_tok(r)) * (W_up x_tok(r)) for the sorted rows of
// the stream item table (item_seg, item_row0: a segment and the first of up
// to 64 of its rows; *n_items of them, at most max_items; segments at
// seg_off[e] .. + seg_cnt[e] of the sorted list).
// bf16: the token rows come from xp (launch_pack_x), and h rows of the
// streaming kernels' segments are written in fragment order too (16-row
// tiles; the GEMM kernels' rows stay row-major).  fp32 reads x directly.
hipError_t launch_gate_up(int wkind, bool packed, const void* x, const void* w13,
                          const float* s13, const int32_t* sorted_ids,
                          const int32_t* block_expert, const int32_t* n_post,
                          const int32_t* seg_off, const int32_t* seg_cnt,
                          const int32_t* item_seg, const int32_t* item_row0,
                          const int32_t* n_items, int max_items, const void* xp, void* h,
                          int H, int I, int k, int bm, int max_rows, hipStream_t s);
// Tiled GEMMs for segments with more than big_thr rows (the align's tile
// table), and the router GEMM for large batches.  K (H, I) % 128 == 0.
hipError_t launch_gate_up_gemm(bool fp8, bool packed, const void* x, const void* w13,
                               const float* s13, const int32_t* sorted_ids,
                               const int32_t* tile_seg, const int32_t* tile_row0,
                               const int32_t* n_tiles, const int32_t* seg_off,
                               const int32_t* seg_cnt, void* h, int H, int I, int k,
                               int max_tiles, hipStream_t s);
hipError_t launch_down_gemm(bool fp8, bool packed, const void* h, const void* w2, const float* s2,
                            const int32_t* tile_seg, const int32_t* tile_row0,
                            const int32_t* n_tiles, const int32_t* seg_off,
                            const int32_t* seg_cnt, void* y, int H, int I, int max_tiles,
                            hipStream_t s);
// Router GEMM: part[z][t][e] for K chunk z of ks (H % (128 ks) == 0); tiles
// with no valid row are skipped (their partials are never read).
hipError_t launch_router_gemm(const void* x, const uint8_t* valid, const void* R,
                              float* part, int T, int H, int E, int ks, hipStream_t s);
// y[r, :] = W2_e h[r, :] for every sorted row r (bf16 h in the layout
// launch_gate_up writes; y rows fp32, bf16 with fp8 weights).  packed:
// weights from launch_pack_weights.
hipError_t launch_down(int wkind, bool packed, const void* h, const void* w2, const float* s2,
                       const int32_t* block_expert, const int32_t* n_post,
                       const int32_t* seg_off, const int32_t* seg_cnt,
                       const int32_t* item_seg, const int32_t* item_row0,
                       const int32_t* n_items, int max_items, void* y, int H, int I,
                       int bm, int max_rows, hipStream_t s);
// Expert weights (bf16 / fp8, a [rows, K] row-major matrix, rows % 16 == 0,
// K % 32 == 0) -> MFMA fragment order: block (16-row tile t, 32-wide K step
// s) of 512 elements at (t K/32 + s) 512, lane 16 g + m holding row 16 t + m,
// columns 32 s + 8 g .. + 7.  `packed` kernels read this layout.
hipError_t launch_pack_weights(int wkind, const void* src, void* dst, size_t rows, int K,
                               hipStream_t s);
// out[t] = sum_j w[t,j] y[pos(t,j)] (+ shared rows), summed in fp32 and
// rounded once; y rows fp32, or bf16 when y_bf16.
hipError_t launch_combine(const void* y, bool y_bf16, const int32_t* ids, const float* w,
                          const int32_t* slot_pos, int T, int H, int k,
                          int n_shared, void* out, bool out_bf16,
                          hipStream_t s);

}  // namespace moe
