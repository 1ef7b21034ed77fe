/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE expert-layer forward library.
 *
 * One MoE expert layer, forward only, on one GPU's share of a DP-attention +
 * TP-MoE deployment ("DP Attention and TBO for DeepSeek-V4 on MI355X",
 * summary page, opening section: DP attention with TP MoE joined by
 * all_gather / reduce_scatter).  The input is the all-gathered token batch,
 * padded to the largest DP rank (same page, PrefillDelayer section), and the
 * experts are held with their intermediate dimension sliced as TP slices it,
 * so `out` is this GPU's partial sum, ready for a reduce_scatter.
 *
 * Steps: router logits -> top-k + softmax over the selected logits (ties to
 * the lower expert id) -> expert align (stable counting sort of the token /
 * expert assignments, each expert padded to the GEMM block M) -> gate/up
 * grouped GEMM with SiLU(gate)*up -> down grouped GEMM -> top-k-weighted
 * combine ("[SGLang] Single Batch Overlap for MoE models": down-projection
 * GEMM, then combine).  Optional always-on shared experts ("Step3 Inference
 * Optimization on AMD Instinct MI308X", optimisation list: shared-expert MLP
 * fused into the MoE layer) and fp8 e4m3 weights with 128x128 fp32 block
 * scales (same list: FP8 blockscale; "AMD Instinct MI355X: ATOM ...":
 * block-scale GEMM).
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless marked (host).  The caller owns every
 *    buffer; the library allocates no device memory and keeps no per-call
 *    state, so calls on different streams with distinct workspaces may run
 *    concurrently.
 *  - Calls only enqueue work on `stream` (a hipStream_t; NULL = the null
 *    stream).  They never synchronise, so they may be captured in a graph.
 *  - All arguments are validated before anything is launched; a non-zero
 *    return means nothing was enqueued (except MOE_ERR_HIP, returned when a
 *    launch itself fails).  Device faults surface at the caller's next
 *    synchronisation.  Nothing is printed and no exception crosses the ABI.
 *  - Layouts are dense row-major with the reduction (K) dimension contiguous;
 *    every pointer must be 16-byte aligned.
 *  - Rows with valid_rows[t] == 0 are never read (they may hold NaN).  Valid
 *    rows must be finite.
 */
#ifndef MOE_AMD_H
#define MOE_AMD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* moe_stream_t; /* a hipStream_t */

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, size out of range, bad topk/block_m */
  MOE_ERR_UNSUPPORTED = -2, /* dtype combination or shape the kernels do not cover */
  MOE_ERR_WORKSPACE = -3,   /* workspace_bytes below moe_workspace_size() */
  MOE_ERR_HIP = -4          /* a HIP launch / runtime call failed */
};

enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 };

/* Layout of w13 / w2 (see moe_pack_weights). */
enum moe_weight_layout { MOE_LAYOUT_ROW_MAJOR = 0, MOE_LAYOUT_FRAG16 = 1 };

/* Layer descriptor (host struct).
 *   T         gathered rows, padding rows included (>= 1)
 *   H         hidden size (multiple of 64; of 128 with bf16 activations)
 *   E         routed experts (1..256)
 *   n_shared  always-on shared experts, 0 or 1; stored after the routed
 *             experts at index E of w13 / w2; not covered by router_w
 *   I         per-GPU expert intermediate size (multiple of 32; of 128 with
 *             fp8 weights)
 *   act_dtype dtype of x, router_w and out: MOE_F32 or MOE_BF16
 *   w_dtype   dtype of w13 / w2: MOE_F32 (with F32 activations), MOE_BF16 or
 *             MOE_FP8_E4M3 (both with BF16 activations)
 *   w13_scale fp8 only: fp32 [E+n_shared, 2I/128, H/128] block scales
 *   w2_scale  fp8 only: fp32 [E+n_shared, H/128, I/128] block scales
 *   block_m   padding granularity of the expert segments in moe_forward's
 *             sorted row list: 0 (library default, 16), 16, 32, 64, 128 or
 *             256 (else MOE_ERR_INVALID_ARG).  The kernels work on 16-row MFMA
 *             tiles of a segment and the tiled GEMMs on 128-row tiles inside
 *             it, so every accepted value gives the same output bits; larger
 *             values only cost workspace
 *   w_layout  MOE_LAYOUT_ROW_MAJOR: w13 / w2 as documented at moe_forward;
 *             MOE_LAYOUT_FRAG16: the same weights re-laid out by
 *             moe_pack_weights (BF16 activations only)
 */
typedef struct moe_desc {
  int32_t T, H, E, n_shared, I;
  int32_t act_dtype, w_dtype;
  const float* w13_scale;
  const float* w2_scale;
  int32_t block_m;
  int32_t w_layout;
} moe_desc;

/* Bytes of workspace moe_forward / moe_route need for this layer and topk
 * (host, pure).  Returns 0 if the descriptor is invalid. */
size_t moe_workspace_size(const moe_desc* desc, int32_t topk);

/* Router: logits l[t,e] = sum_h x[t,h] * router_w[e,h] (fp32 accumulation),
 * then per valid row the topk experts of largest logit (ties to the lower
 * expert id), in slots of descending logit, with weights = softmax over the
 * selected logits (they sum to 1).  Padding rows get ids -1 and weights 0.
 *   x            [T, H] act_dtype
 *   valid_rows   [T] uint8 (0 = padding row) or NULL = all rows valid
 *   router_w     [E, H] act_dtype
 *   topk_ids     out [T, topk] int32
 *   topk_w       out [T, topk] fp32
 *   logits       out [T, E] fp32 or NULL (debug; padding rows get 0)
 *   workspace    >= moe_workspace_size(desc, topk) bytes
 * (Routing: "Step3 Inference Optimization on AMD Instinct MI308X",
 * Background: top-3 of 48 experts.) */
int moe_route(const moe_desc* desc, const void* x, const uint8_t* valid_rows,
              const void* router_w, int32_t topk, int32_t* topk_ids,
              float* topk_w, float* logits, void* workspace,
              size_t workspace_bytes, moe_stream_t stream);

/* Align: stable counting sort of the flat assignments a = t*topk + j by
 * expert id.  Expert segments in ascending expert order, ascending a inside a
 * segment; each segment padded with -1 to a multiple of block_m; experts with
 * no assignment get no block; ids of -1 are skipped.  With desc->n_shared = 1
 * the shared expert is one more segment (expert E, after the routed ones)
 * holding every row t with topk_ids[t][0] >= 0, entered as t*topk; so in
 * every segment, entry / topk is the token row.  Only desc->T, E and
 * n_shared are read.
 *   topk_ids        [T, topk] int32 (values in [0, E) or -1)
 *   block_m         1..256
 *   sorted_ids      out, capacity >= T*(topk+n_shared) + (E+n_shared)*(block_m-1)
 *   block_expert    out, capacity >= that / block_m: segment of each block
 *   expert_offsets  out [E+n_shared+1] int32: padded segment starts, last = total
 *   n_post_padded   out [1] int32: total padded length
 *   workspace       NULL, or >= 4*ceil(T*(topk+n_shared)/4096)*(E+n_shared)
 *                   bytes (moe_workspace_size(desc, topk) always suffices):
 *                   batches of more than 8192 assignments then run the count /
 *                   scan / scatter over 4096-assignment spans in parallel;
 *                   with NULL one workgroup sorts the whole list.  Both give
 *                   the same bits.  MOE_ERR_WORKSPACE if workspace_bytes is
 *                   too small.
 * Only the first n_post_padded / n_post_padded/block_m entries are written.
 * (Per-expert block granularity: "[SGLang] Single Batch Overlap for MoE
 * models", combine signal section, one signal per 64-token block; padding
 * rows of the gathered batch carry no assignment: "DP Attention and TBO for
 * DeepSeek-V4 on MI355X", PrefillDelayer section.) */
int moe_align(const moe_desc* desc, const int32_t* topk_ids, int32_t topk,
              int32_t block_m, int32_t* sorted_ids, int32_t* block_expert,
              int32_t* expert_offsets, int32_t* n_post_padded, void* workspace,
              size_t workspace_bytes, moe_stream_t stream);

/* The whole layer: route -> align -> gate/up GEMM with SiLU(g)*u -> down GEMM
 * -> combine out[t] = sum_j w[t,j] * y_{ids[t,j]}(x_t) (+ shared experts with
 * weight 1), accumulated in fp32 and rounded once to act_dtype.  Each expert's
 * output row y is kept in fp32; in bf16 when w_dtype is MOE_FP8_E4M3 (its
 * rounding, at most 2^-9 relative, sits well inside that path's error
 * budget); with bf16 weights, in 24-bit floats (at most 2^-16 relative) when
 * every expert segment of the call streams its weights.  Calls where every
 * segment streams and T*(topk+n_shared) <= 1216 keep the y rows in fp32 on
 * chip and combine them in the same launch, whatever w_dtype.  `out` is
 * fully overwritten; padding rows are set to 0.
 *   w13  [E+n_shared, 2I, H]: gate rows 0..I-1, then up rows I..2I-1
 *   w2   [E+n_shared, H, I]
 *   (fp8: uint8 e4m3fn codes; W = code value * block scale)
 *   out  [T, H] act_dtype (must not alias any input) */
int moe_forward(const moe_desc* desc, const void* x, const uint8_t* valid_rows,
                const void* router_w, const void* w13, const void* w2,
                int32_t topk, void* out, void* workspace,
                size_t workspace_bytes, moe_stream_t stream);

/* Number of int32 completion counters moe_forward_signaled takes:
 * (E + n_shared) * ceil(T / 64).  Host, pure; 0 for a NULL or malformed desc. */
size_t moe_block_signal_count(const moe_desc* desc);

/* moe_forward with per-(expert, 64-row block) completion signals and the
 * combine as their consumer on a second stream ("[SGLang] Single Batch
 * Overlap for MoE models", combine-signal section: the down-projection GEMM
 * marks each finished block so that the combine can start on it instead of
 * waiting for the whole GEMM).
 *   block_signal    [E + n_shared][ceil(T / 64)] int32, device, caller-owned,
 *                   moe_block_signal_count(desc) entries.  The call zeroes it
 *                   on `stream`; each down-projection block then adds, after
 *                   a release at agent scope, the number of output columns it
 *                   stored for the 64-row blocks of the expert's segment of
 *                   the sorted row list (rows 64 b .. 64 b + 63 of expert e:
 *                   entry [e][b]) that its rows cover.  A block is complete
 *                   when its entry reaches H; entries of blocks past an
 *                   expert's rows stay 0.  Once the call has completed every
 *                   block that holds rows reads exactly H.
 *   consumer_stream the stream the waiting combine runs on (may equal
 *                   `stream`).  It waits (an event) for the gate/up GEMM,
 *                   then combines each token row as soon as the blocks that
 *                   hold its expert rows are complete; `stream` then waits
 *                   for it (an event) and combines the rows, if any, that it
 *                   left because a wait ran past its time bound
 *                   (moe_set_signal_wait_us; 10 ms by default).  The call
 *                   returns with all work enqueued; `out` is complete when
 *                   `stream` reaches that point, and the bits equal
 *                   moe_forward's (same kernels, same summation order),
 *                   except that decode-sized calls do not take moe_forward's
 *                   one-launch down + combine (their y rows go through
 *                   memory as in larger calls).
 * Errors as moe_forward, plus MOE_ERR_INVALID_ARG for a NULL block_signal and
 * MOE_ERR_UNSUPPORTED for fp32 layers.  Two events are created and released
 * per call; nothing is allocated in device memory.  Calls must not share a
 * block_signal array or a workspace while either runs. */
int moe_forward_signaled(const moe_desc* desc, const void* x, const uint8_t* valid_rows,
                         const void* router_w, const void* w13, const void* w2,
                         int32_t topk, void* out, void* workspace,
                         size_t workspace_bytes, int32_t* block_signal,
                         moe_stream_t stream, moe_stream_t consumer_stream);

/* Time bound of each wait of moe_forward_signaled's waiting combine, in
 * microseconds (0 .. 1000000; default 10000).  Host, process-wide, read when
 * a call is enqueued.  With 0 a wait gives up at once unless its blocks are
 * already complete, which sends the rows to the rest pass on `stream` (tests
 * use it to exercise that pass; the output bits do not change).
 * MOE_ERR_INVALID_ARG outside the range. */
int moe_set_signal_wait_us(int32_t us);

/* Calls of moe_forward / moe_forward_noalloc where every expert segment
 * streams its weights (decode-sized batches): run the gate/up GEMM with
 * SiLU*mul and the down GEMM in one launch (1) or in two (0, the default)
 * ("Step3 Inference Optimization on AMD Instinct MI308X", optimisation list:
 * the MoE one-stage kernel).  In the one launch, blocks take the gate/up
 * units first and the down units after them from one counter; each gate/up
 * unit releases its h columns at agent scope and counts itself in its work
 * item, and each down unit waits for its item's count (bounded in time by
 * moe_set_signal_wait_us; a unit whose wait runs out is run by a rest pass
 * after the launch), so the output bits equal the two-launch path's with the
 * y rows in memory, i.e. except for calls of at most 1216 assignments, which
 * the default path combines on chip.  Applies to bf16 activations and
 * weights, H a multiple of 512 and I of 128; other calls, and
 * moe_forward_signaled, keep two launches.  Host, process-wide, read when a
 * call is planned (size workspaces after choosing).  MOE_ERR_INVALID_ARG
 * unless 0 or 1. */
int moe_set_one_launch(int32_t enable);

/* Bytes of the fixed device scratch that moe_forward_noalloc works in. */
#define MOE_SCRATCH_BYTES (64u << 20)

/* moe_forward for callers that cannot allocate device memory or pass a
 * workspace: code under HIP-graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, kernels and output bits as
 * moe_forward, minus the workspace: the layer runs in a static device array
 * of MOE_SCRATCH_BYTES (64 MiB) that each GPU holds from the library's load
 * until the process ends (enough for decode-sized batches: the 48-expert
 * top-3 layer of hidden 7168 and inter 640 takes 44 MiB at 256 rows).
 * Returns MOE_ERR_WORKSPACE, before any launch, when
 * moe_workspace_size(desc, topk) exceeds it.  Nothing is allocated and no
 * library routine that allocates is called; the first call on a GPU looks up
 * that GPU's copy of the array.  Every call on one GPU shares that GPU's
 * array, so calls that overlap in time on one GPU (two streams, two threads)
 * race and give undefined results: serialise them.  Nothing in the array
 * needs to start at zero (each call writes what it reads). */
int moe_forward_noalloc(const moe_desc* desc, const void* x, const uint8_t* valid_rows,
                        const void* router_w, const void* w13, const void* w2,
                        int32_t topk, void* out, moe_stream_t stream);

/* One-time re-layout of the expert weights (at load time) into the order in
 * which the layer's MFMA kernels fetch them, so that each wave-wide weight
 * load is one contiguous 1 KB (bf16) / 512 B (fp8) block instead of 16 rows x
 * 64 B; moe_forward then takes desc->w_layout = MOE_LAYOUT_FRAG16.  Every
 * 16-row x 32-column piece of a [rows, K] weight matrix (w13: rows = (E +
 * n_shared) 2I, K = H; w2: rows = (E + n_shared) H, K = I) becomes a block of
 * 512 elements at (t K/32 + s) 512 (t = row / 16, s = column / 32), whose
 * element 8 (16 g + m) + i is W[16 t + m][32 s + 8 g + i].  The packed arrays
 * have the sizes and dtypes of w13 / w2; block scales are unchanged.
 *   desc        as for moe_forward (T, w_layout and the scale pointers are
 *               not used); w_dtype BF16 or FP8_E4M3 with BF16 activations
 *   w13, w2     row-major weights (read)
 *   w13_packed, w2_packed  out, same sizes; must not alias the inputs
 * Enqueued on `stream`; the caller keeps the packed arrays for the layer's
 * lifetime.  Returns MOE_ERR_UNSUPPORTED for fp32 weights. */
int moe_pack_weights(const moe_desc* desc, const void* w13, const void* w2,
                     void* w13_packed, void* w2_packed, moe_stream_t stream);

/* Path choice inside moe_forward (host; process-wide, read when a call
 * starts).  Expert segments with more than gemm_min_rows rows go to the
 * LDS-tiled GEMM kernels when their 128-row tiles number at least
 * gemm_min_tiles (-1 = enough to fill the chip); all other segments stream
 * the expert weights.  Defaults: 128, -1.  gemm_min_rows = INT32_MAX keeps
 * every segment on the streaming kernels.  Both paths compute the same
 * layer; this only moves work between kernels (tuning, and tests that cover
 * both paths at small sizes).  Returns MOE_ERR_INVALID_ARG for
 * gemm_min_rows < 0 or gemm_min_tiles < -1. */
int moe_set_path_thresholds(int32_t gemm_min_rows, int32_t gemm_min_tiles);

/* Arithmetic of the tiled gate/up GEMM for fp8 weights (host; process-wide,
 * read when a call starts).  0 (default): bf16 MFMA on weights dequantised
 * to bf16 (q * s rounded); 1: the fp8 MFMA on the weights' codes as they
 * are, with each token row split into two e4m3 terms that share a
 * power-of-two row scale (x = s (hi + lo), exact for all but the smallest
 * elements of a row), two fp8 MFMAs where 0 issues four bf16 ones of the
 * same total cycles.  Both meet the fp8-weight error bound; 1 needs 2 T H +
 * 4 T bytes more workspace (moe_workspace_size follows the setting, so size
 * workspaces after choosing) and a pass that splits the token rows
 * ("Step3 Inference Optimization on AMD Instinct MI308X", optimisation list:
 * mixed BF16 / FP8-blockscale arithmetic).  Returns MOE_ERR_INVALID_ARG for
 * other values. */
int moe_set_fp8_mfma(int32_t enable);

/* Message for a status code (host; static string). */
const char* moe_status_str(int status);

/* ---- measurement hooks (host; not for the serving path) ------------------
 * moe_profile_enable(mask): for every stage s with bit s of mask set,
 * moe_forward records a hipEvent pair around that stage's kernel launch on
 * the call's stream (mask 0 = off, -1 = every stage).  moe_profile_read waits
 * for the recorded events, writes the summed milliseconds and launch counts
 * of each stage (index < moe_num_stages()) and clears the record.  Event
 * records perturb the timeline slightly; enable only the stages you time.
 * Recording creates events: benchmarks only. */
int moe_num_stages(void);
const char* moe_stage_name(int stage);
int moe_profile_enable(int stage_mask);
int moe_profile_read(double* stage_ms, int32_t* stage_launches, int32_t n);

#ifdef __cplusplus
}
#endif
#endif /* MOE_AMD_H */
