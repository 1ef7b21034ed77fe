// Host-side launchers of the gfx950 kernels (internal to libmoe_amd).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Completion signals of the expert output rows y, one counter per (segment,
// 64-row block of the segment) ("[SGLang] Single Batch Overlap for MoE
// models", combine-signal section: the down-projection GEMM reports each
// finished block so that its consumer can start on it).  sig[seg * nb64 + b]
// counts the columns of y stored for rows 64 b .. 64 b + 63 of segment seg;
// the block is complete when the count reaches H.  The down launchers raise
// them when sig is non-null (the counters must start at zero).
struct BlockSignals {
  int32_t* sig;   // null: the launch raises no signals
  int nb64;       // counters per segment: ceil(T / 64)
};

// The combine as the signals' consumer.  COMBINE_WAIT: each block waits
// (wave 0, bounded in time) until the counters of its row's assignments
// reach target, then combines that part of the row and sets its done flag;
// a wait that runs out of time sets *giveup, after which no block waits and
// rows are left undone.  COMBINE_REST: combine only the parts whose done
// flag is 0 (launched once the producer and the waiting combine have ended).
enum CombineMode { COMBINE_ALL = 0, COMBINE_WAIT = 1, COMBINE_REST = 2 };
struct CombineWait {
  const int32_t* sig;       // BlockSignals counters
  const int32_t* seg_off;   // segment starts in the sorted row list
  int nb64, target, E;      // target: H; E: the shared segment's index
  int32_t* done;            // [T][combine_grid_y]: zeroed before the producer runs
  int32_t* giveup;          // zeroed likewise
  long long ticks;          // time bound of one wait, in 100 MHz real-time ticks
};

// Gate/up and down of the streaming kernels in one launch (calls where every
// segment streams; see launch_expert_mlp).  All counters and flags must be
// zero at the launch.
struct OneLaunch {
  int32_t* ticket;      // next unit to take
  int32_t* item_done;   // [max_items]: gate/up units of each item finished
  int32_t* undone;      // [max_items * n_ng]: down units left to the rest pass
  int32_t* giveup;      // set once a wait runs out of time; later waits skip
  long long ticks;      // time bound of one wait, in 100 MHz real-time ticks
};

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

// bf16 streaming path, calls where the tiled GEMM may run: x rows of the
// sorted rows of the stream item table's items (the streaming segments),
// packed in MFMA fragment order into xp (sorted-list rows x H bf16, 16-row
// tiles; padding rows and rows of other segments left as they are).
hipError_t launch_pack_x_items(const void* x, const int32_t* sorted_ids, const int32_t* seg_off,
                               const int32_t* seg_cnt, const int32_t* item_seg,
                               const int32_t* item_row0, const int32_t* n_items, int max_items,
                               void* xp, int H, int k, hipStream_t s);
// h[r, :] = SiLU(W_gate x_tok(r)) * (W_up x_tok(r)) for the sorted rows of
// the stream item table (item_seg, item_row0: a segment and the first of up
// to 64 of its rows; *n_items of them, at most max_items; segments at
// seg_off[e] .. + seg_cnt[e] of the sorted list).
// bf16 / fp8 weights: the token rows come from xp (launch_pack_x_items), or
// straight from x (bf16 [T, H]) through sorted_ids when x_direct (calls where
// every segment streams); h rows of the streaming kernels' segments are
// written in fragment order (16-row tiles; the GEMM kernels' rows stay
// row-major).  fp32 reads x directly.
hipError_t launch_gate_up(int wkind, bool packed, const void* x, const void* w13,
                          const float* s13, const int32_t* sorted_ids,
                          const int32_t* block_expert, const int32_t* n_post,
                          const int32_t* seg_off, const int32_t* seg_cnt,
                          const int32_t* item_seg, const int32_t* item_row0,
                          const int32_t* n_items, int max_items, const void* xp, void* h,
                          int H, int I, int k, int bm, int max_rows, bool x_direct,
                          hipStream_t s);
// Tiled GEMMs for segments with more than big_thr rows (the align's tile
// table), and the router GEMM for large batches.  K (H, I) % 128 == 0.
// fp8 weights with xq non-null: the fp8-MFMA kernel on the two-term token
// codes (launch_xq_split); otherwise bf16 MFMA on dequantised weights.
hipError_t launch_gate_up_gemm(bool fp8, bool packed, const void* x, const void* w13,
                               const float* s13, const int32_t* sorted_ids,
                               const int32_t* tile_seg, const int32_t* tile_row0,
                               const int32_t* n_tiles, const int32_t* seg_off,
                               const int32_t* seg_cnt, void* h, int H, int I, int k,
                               int max_tiles, const uint8_t* xq, const float* sx, int T,
                               hipStream_t s);
// Valid token rows (bf16 [T, H]) as two e4m3 terms with one power-of-two
// scale per row: xq [2][T][H] (hi plane, lo plane), sx [T].
hipError_t launch_xq_split(const void* x, const uint8_t* valid, uint8_t* xq, float* sx, int T,
                           int H, hipStream_t s);
hipError_t launch_down_gemm(bool fp8, bool packed, const void* h, const void* w2, const float* s2,
                            const int32_t* tile_seg, const int32_t* tile_row0,
                            const int32_t* n_tiles, const int32_t* seg_off,
                            const int32_t* seg_cnt, void* y, int H, int I, int max_tiles,
                            hipStream_t s, BlockSignals bs = BlockSignals{nullptr, 0});
// Router GEMM: part[z][t][e] for K chunk z of ks (H % (128 ks) == 0); tiles
// with no valid row are skipped (their partials are never read).
hipError_t launch_router_gemm(const void* x, const uint8_t* valid, const void* R,
                              float* part, int T, int H, int E, int ks, hipStream_t s);
// Calls where every segment streams, bf16 / fp8 weights, at most 1216
// assignments (T (k + n_shared)): the down projection and the combine in one
// launch, out [T, H] bf16 written directly (padding rows zero).
bool down_cols_fits(int T, int k, int n_shared, int H, int I);
hipError_t launch_down_cols(int wkind, bool packed, const void* h, const void* w2,
                            const float* s2, const int32_t* seg_off, const int32_t* seg_cnt,
                            const int32_t* sorted_ids, const int32_t* ids, const float* w,
                            int T, int H, int I, int E, int n_shared, int k, void* out,
                            hipStream_t s);
// y[r, :] = W2_e h[r, :] for every sorted row r (bf16 h in the layout
// launch_gate_up writes; y rows fp32, bf16 with fp8 weights, 24-bit floats
// with bf16 weights when y24).  packed: weights from launch_pack_weights.
hipError_t launch_down(int wkind, bool packed, const void* h, const void* w2, const float* s2,
                       const int32_t* block_expert, const int32_t* n_post,
                       const int32_t* seg_off, const int32_t* seg_cnt,
                       const int32_t* item_seg, const int32_t* item_row0,
                       const int32_t* n_items, int max_items, void* y, int H, int I,
                       int bm, int max_rows, bool y24, hipStream_t s,
                       BlockSignals bs = BlockSignals{nullptr, 0},
                       const int32_t* only = nullptr);
// Output column groups per item of the streaming down kernel (its units per
// item).
inline int stream_down_groups(int H) { return (H + 255) / 256; }
// Calls where every segment streams: gate/up (token rows straight from x)
// and down in one launch, y rows as launch_down writes them (24-bit); down
// units whose wait ran out are flagged in
// ol.undone for launch_down(..., only = ol.undone).  Shapes: bf16 weights,
// H % 512 == 0, I % 128 == 0 (expert_mlp_fits).
bool expert_mlp_fits(int wkind, int H, int I);
hipError_t launch_expert_mlp(int wkind, bool packed, const void* x, const void* w13,
                             const void* w2, const int32_t* seg_off, const int32_t* seg_cnt,
                             const int32_t* sorted_ids, const int32_t* item_seg,
                             const int32_t* item_row0, const int32_t* n_items, int max_items,
                             void* h, void* y, int H, int I, int k, OneLaunch ol,
                             hipStream_t s);
// Expert weights (bf16 / fp8, a [rows, K] row-major matrix, rows % 16 == 0,
// K % 32 == 0) -> MFMA fragment order: block (16-row tile t, 32-wide K step
// s) of 512 elements at (t K/32 + s) 512, lane 16 g + m holding row 16 t + m,
// columns 32 s + 8 g .. + 7.  `packed` kernels read this layout.
hipError_t launch_pack_weights(int wkind, const void* src, void* dst, size_t rows, int K,
                               hipStream_t s);
// Formats of the expert output rows y.
enum YFmt { Y_F32 = 0, Y_BF16 = 1, Y_F24 = 2 };
// out[t] = sum_j w[t,j] y[pos(t,j)] (+ shared rows), summed in fp32 and
// rounded once; y rows in format yfmt.
hipError_t launch_combine(const void* y, int yfmt, const int32_t* ids, const float* w,
                          const int32_t* slot_pos, int T, int H, int k,
                          int n_shared, void* out, bool out_bf16,
                          hipStream_t s, int mode = COMBINE_ALL,
                          const CombineWait* cw = nullptr);
// Column chunks per row of the combine grid (at most (H + 1023) / 1024).
int combine_grid_y(int T, int H, int yfmt);
// a[0 .. na) = 0 and b[0 .. nb) = 0 (a fill kernel: safe under graph capture)
hipError_t launch_zero_i32(int32_t* a, size_t na, int32_t* b, size_t nb, hipStream_t s);

}  // namespace moe
