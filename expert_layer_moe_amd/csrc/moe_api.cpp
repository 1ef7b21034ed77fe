// C ABI of the MoE layer: validation, workspace layout, launch sequence.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <mutex>
#include <vector>

#include "../../include/moe.h"
#include "moe_kernels.h"

namespace {

constexpr int kMaxE = 256;
constexpr int kMaxTopk = 16;
constexpr int kDefaultBM = 16;
constexpr size_t kAlign = 256;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace layout of one moe_forward call.
struct Plan {
  int T, H, E, ns, I, k;
  int act, w;
  int bm, ks;
  int cap;        // capacity of the sorted row list (multiple of bm)
  bool router_gemm;  // tiled router GEMM (large batches) instead of the K split
  int big_thr;    // segments with more rows go to the tiled GEMM kernels
  int max_tiles;  // bound on their 128-row tiles
  int min_tiles;  // fewer tiles than this stay on the streaming kernels
  int max_items;  // bound on the streaming kernels' work items
  size_t off_part, off_ids, off_w, off_sorted, off_bexp, off_offs, off_npost,
      off_slot, off_cnt, off_tseg, off_trow, off_ntiles, off_iseg, off_irow, off_nitems,
      off_span, off_h, off_y, off_xq, off_sx, off_done, off_one, total;
  bool xsplit;    // fp8 weights on the GEMM path: token rows as two e4m3 terms
  int yfmt;       // format of the expert output rows y (moe::YFmt)
  bool down_cols; // down projection and combine in one launch (small batches)
  bool one_launch; // gate/up and down in one launch (moe_set_one_launch)
};

// Rows per segment above which the tiled GEMM kernels (128-row tiles, weight
// fragments reused across the tile) beat streaming the weights once per
// 64-row pass.
constexpr int kBigSegRows = 128;

// Path thresholds (moe_set_path_thresholds); read when a call is planned.
std::atomic<int> g_gemm_min_rows{kBigSegRows};
std::atomic<int> g_gemm_min_tiles{-1};   // -1: enough tiles to fill the chip
// fp8 weights on the tiled gate/up GEMM: fp8 MFMA on two-term token codes (1)
// or bf16 MFMA on dequantised weights (0, the default: the same MFMA cycles,
// measured no faster, and no split pass); moe_set_fp8_mfma
std::atomic<int> g_fp8_mfma{0};
// Calls where every segment streams: gate/up and down in one launch (1) or
// two (0, the default: measured faster); moe_set_one_launch
std::atomic<int> g_one_launch{0};

// Padding granularity of the expert segments in the sorted row list: every
// kernel works on 16-row MFMA tiles of a segment (the tiled GEMMs on 128-row
// tiles inside it), so any multiple of 16 up to 256 gives the same result.
bool valid_block_m(int bm) {
  return bm == 0 || bm == 16 || bm == 32 || bm == 64 || bm == 128 || bm == 256;
}
int block_m_of(const moe_desc* d) { return d->block_m ? d->block_m : kDefaultBM; }

int check_desc(const moe_desc* d, int32_t topk, bool need_scales = true) {
  if (d == nullptr) return MOE_ERR_INVALID_ARG;
  if (d->T < 1 || d->H < 1 || d->I < 1 || d->E < 1 || d->E > kMaxE)
    return MOE_ERR_INVALID_ARG;
  if (d->n_shared < 0 || d->n_shared > 1) return MOE_ERR_INVALID_ARG;
  if (topk < 1 || topk > d->E || topk > kMaxTopk) return MOE_ERR_INVALID_ARG;
  if (!valid_block_m(d->block_m)) return MOE_ERR_INVALID_ARG;
  if (d->w_layout != MOE_LAYOUT_ROW_MAJOR && d->w_layout != MOE_LAYOUT_FRAG16)
    return MOE_ERR_INVALID_ARG;
  if (d->w_layout == MOE_LAYOUT_FRAG16 && d->act_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (d->act_dtype == MOE_BF16 && d->H % 128 != 0) return MOE_ERR_UNSUPPORTED;
  const bool f32 = d->act_dtype == MOE_F32 && d->w_dtype == MOE_F32;
  const bool bf16 = d->act_dtype == MOE_BF16 && d->w_dtype == MOE_BF16;
  const bool fp8 = d->act_dtype == MOE_BF16 && d->w_dtype == MOE_FP8_E4M3;
  if (!f32 && !bf16 && !fp8) return MOE_ERR_UNSUPPORTED;
  if (d->H % 64 != 0 || d->I % 32 != 0) return MOE_ERR_UNSUPPORTED;
  if (fp8) {
    if (d->H % 128 != 0 || d->I % 128 != 0) return MOE_ERR_UNSUPPORTED;
    if (need_scales && (d->w13_scale == nullptr || d->w2_scale == nullptr))
      return MOE_ERR_INVALID_ARG;
  }
  // sizes must fit the kernels' 32-bit row indexing of the sorted row list,
  // and the 32-bit element offsets of h rows (sorted rows x I) in the tiled
  // down GEMM
  const long long rows = (long long)d->T * (topk + d->n_shared) +
                         (long long)(d->E + d->n_shared) * block_m_of(d);
  if (rows > (1LL << 30) || (long long)d->T * d->H > (1LL << 40))
    return MOE_ERR_UNSUPPORTED;
  if ((unsigned long long)rows * (unsigned long long)d->I >= (1ULL << 32))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Column chunks per row that the combine grid can have (the done flags of
// the waiting combine).
int done_chunks(int H) { return (H + 1023) / 1024; }

// Completion counters of moe_forward_signaled: (E + n_shared) segments x
// ceil(T / 64) blocks.
size_t signal_count(const moe_desc* d) {
  return (size_t)(d->E + d->n_shared) * (size_t)((d->T + 63) / 64);
}

// Words of the one-launch gate/up + down's counters and flags: ticket, give-up
// flag, one spare, then max_items item counts and max_items * n_ng flags.
size_t one_launch_words(int max_items, int H) {
  return 3 + (size_t)max_items * (1 + moe::stream_down_groups(H));
}

// The tiled kernels index x with 32-bit element offsets.
bool fits_tiled(const moe_desc* d) { return (long long)d->T * d->H < (1LL << 31); }

bool use_router_gemm(const moe_desc* d) {
  return d->act_dtype == MOE_BF16 && d->T >= 1024 && d->H % 128 == 0 && fits_tiled(d);
}

// K split of the router logits (the top-k kernel sums the ks partials in a
// fixed order).  The router GEMM's split depends on H and E only, so a
// row's logits do not depend on the batch it comes in (a split batch
// reproduces the unsplit one bit for bit).
int choose_ks(const moe_desc* d) {
  if (d->act_dtype != MOE_BF16) return 1;
  if (use_router_gemm(d)) {
    // more than 128 experts (the 256-expert GEMM, one block per CU): 4 K
    // chunks measured faster than 8 (fewer partials for the top-k to sum)
    const int max_ks = d->E > 128 ? 4 : 8;
    int ks = 1;
    while (ks < max_ks && d->H % (128 * ks * 2) == 0) ks *= 2;
    return ks;
  }
  const int ksteps = d->H / 32;
  const long long base = (long long)((d->T + 15) / 16) * ((d->E + 63) / 64);
  int ks = 1;
  while (base * ks < 512 && ksteps % (ks * 2) == 0) ks *= 2;
  return ks;
}

int make_plan(const moe_desc* d, int32_t topk, Plan* p) {
  const int st = check_desc(d, topk);
  if (st != MOE_OK) return st;
  p->T = d->T; p->H = d->H; p->E = d->E; p->ns = d->n_shared; p->I = d->I;
  p->k = topk; p->act = d->act_dtype; p->w = d->w_dtype;
  p->bm = block_m_of(d);
  p->ks = choose_ks(d);
  p->router_gemm = use_router_gemm(d);
  const int min_rows = g_gemm_min_rows.load();
  const bool gemm_shape = d->act_dtype == MOE_BF16 && d->I % 128 == 0 &&
                          d->H <= moe::kMaxGemmK && d->I <= moe::kMaxGemmK && fits_tiled(d);
  p->big_thr = gemm_shape ? min_rows : INT_MAX;
  const size_t kk = (size_t)topk + p->ns;
  // the GEMM path only pays once its gate/up launch fills the chip
  // (256 blocks of I/128 columns each)
  const int tiles_set = g_gemm_min_tiles.load();
  p->min_tiles = tiles_set >= 0
                     ? tiles_set
                     : (256 + p->I / 128 - 1) / (p->I / 128 > 0 ? p->I / 128 : 1);
  p->max_tiles = (int)(((size_t)p->T * kk + 127) / 128 + p->E + p->ns);
  // A segment holds at most T rows, and the 128-row tiles of the segments
  // above big_thr rows number at most T kk / 128 + T kk / (big_thr + 1) + 1:
  // when that cannot reach min_tiles the GEMM kernels would never run, so
  // they are not launched.
  if (p->big_thr != INT_MAX) {
    const size_t bound = (size_t)p->T * kk / 128 + (size_t)p->T * kk / ((size_t)p->big_thr + 1) + 1;
    if (p->T <= p->big_thr || bound < (size_t)p->min_tiles) p->big_thr = INT_MAX;
  }
  p->max_items = moe::max_stream_items((long long)p->T * kk, p->E + p->ns);
  p->cap = (int)round_up((size_t)p->T * kk + (size_t)(p->E + p->ns) * (p->bm - 1), p->bm);
  const size_t act_h = (p->act == MOE_F32) ? 4 : 2;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = round_up(o + bytes, kAlign); return r; };
  p->off_part = take((size_t)p->ks * p->T * p->E * 4);
  p->off_ids = take((size_t)p->T * topk * 4);
  p->off_w = take((size_t)p->T * topk * 4);
  p->off_sorted = take((size_t)p->cap * 4);
  p->off_bexp = take((size_t)(p->cap / p->bm) * 4);
  p->off_offs = take((size_t)(p->E + p->ns + 1) * 4);
  p->off_npost = take(4);
  p->off_slot = take((size_t)p->T * kk * 4);
  p->off_cnt = take((size_t)(p->E + p->ns) * 4);
  p->off_tseg = take((size_t)p->max_tiles * 4);
  p->off_trow = take((size_t)p->max_tiles * 4);
  p->off_ntiles = take(4);
  p->off_iseg = take((size_t)p->max_items * 4);
  p->off_irow = take((size_t)p->max_items * 4);
  p->off_nitems = take(4);
  p->off_span = take((size_t)moe::align_spans(p->T, p->k, p->ns) * (p->E + p->ns) * 4);
  p->off_h = take((size_t)p->cap * p->I * act_h);
  // y rows: bf16 with fp8 weights; with bf16 weights 24-bit floats when
  // every segment streams (only the streaming down kernel writes them), fp32
  // otherwise.  The room is that of fp32 rows with bf16 weights whatever the
  // format, so that the workspace size does not depend on the path
  // thresholds.  In calls where the tiled GEMM may run it also holds the
  // packed token rows of the streaming gate/up (cap x H bf16) until the down
  // kernels overwrite them.
  p->yfmt = p->w == MOE_FP8_E4M3 ? moe::Y_BF16
            : (p->w == MOE_BF16 && p->big_thr == INT_MAX) ? moe::Y_F24 : moe::Y_F32;
  p->off_y = take((size_t)p->cap * p->H * (p->w == MOE_FP8_E4M3 ? 2 : 4));
  // every segment streams and the batch's assignments fit the combined
  // down kernel's LDS rows: no y rows, no combine launch
  p->down_cols = p->big_thr == INT_MAX && p->w != MOE_F32 && p->act == MOE_BF16 &&
                 moe::down_cols_fits(p->T, p->k, p->ns, p->H, p->I);
  // two e4m3 code planes of the token rows and their scales (fp8 MFMA path):
  // room whenever the shape can take the tiled GEMM (so the workspace size
  // does not depend on the path thresholds); filled when it can run
  const bool xq_room = p->w == MOE_FP8_E4M3 && gemm_shape && g_fp8_mfma.load() != 0;
  p->xsplit = xq_room && p->big_thr != INT_MAX;
  p->off_xq = take(xq_room ? (size_t)2 * p->T * p->H : 0);
  p->off_sx = take(xq_room ? (size_t)p->T * 4 : 0);
  // done flags of the waiting combine (moe_forward_signaled): one per (row,
  // column chunk of the combine grid), then the give-up flag
  p->off_done = take(((size_t)p->T * done_chunks(p->H) + 1) * 4);
  // the one-launch gate/up + down: ticket, give-up flag, per-item counts,
  // per-down-unit rest flags
  p->off_one = take(one_launch_words(p->max_items, p->H) * 4);
  const int wk = p->w == MOE_FP8_E4M3 ? moe::W_FP8 : (p->w == MOE_BF16 ? moe::W_BF16 : moe::W_F32);
  p->one_launch = g_one_launch.load() != 0 && p->big_thr == INT_MAX && p->act == MOE_BF16 &&
                  moe::expert_mlp_fits(wk, p->H, p->I);
  if (p->one_launch) p->down_cols = false;
  p->total = o;
  return MOE_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// ---- measurement hooks -------------------------------------------------------
enum Stage {
  S_LOGITS = 0, S_TOPK, S_ALIGN, S_PACK_X, S_GATE_UP, S_GATE_UP_GEMM, S_DOWN, S_DOWN_GEMM,
  S_COMBINE, S_X_SPLIT, S_COMBINE_WAIT, S_EXPERT_MLP, S_COUNT
};
const char* kStageNames[S_COUNT] = {"route_logits", "route_topk", "align", "pack_x", "gate_up",
                                    "gate_up_gemm", "down", "down_gemm", "combine", "x_split",
                                    "combine_wait", "expert_mlp"};

struct ProfRecord {
  int stage;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
unsigned g_prof_mask = 0;  // bit s set: time stage s
std::vector<ProfRecord> g_prof;

struct StageTimer {
  int stage;
  hipStream_t s;
  hipEvent_t a = nullptr, b = nullptr;
  StageTimer(int st, hipStream_t str) : stage(st), s(str) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!(g_prof_mask >> st & 1u)) return;
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) {
      a = b = nullptr;
      return;
    }
    (void)hipEventRecord(a, s);
  }
  ~StageTimer() {
    if (a == nullptr) return;
    (void)hipEventRecord(b, s);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof.push_back({stage, a, b});
  }
};

hipError_t launch_logits(const Plan& p, const void* x, const uint8_t* valid,
                         const void* router_w, float* part, hipStream_t s) {
  if (p.router_gemm)
    return moe::launch_router_gemm(x, valid, router_w, part, p.T, p.H, p.E, p.ks, s);
  return moe::launch_route_logits(p.act == MOE_BF16, x, valid, router_w, part, p.T, p.H, p.E,
                                  p.ks, s);
}

// moe_forward_signaled: the caller's completion counters and the stream of
// the waiting combine.
struct SignalCtx {
  int32_t* sig;
  hipStream_t consumer;
};

// Events of one signaled call, created with it and released once its waits
// are enqueued (HIP frees an event whose record is pending when that
// completes).
struct CallEvents {
  hipEvent_t ev[2] = {nullptr, nullptr};
  ~CallEvents() {
    for (hipEvent_t e : ev)
      if (e != nullptr) (void)hipEventDestroy(e);
  }
  bool make() {
    for (hipEvent_t& e : ev)
      if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return false;
    return true;
  }
};

// Time bound of one wait of the waiting combine, in microseconds
// (moe_set_signal_wait_us; the kernels count 100 MHz real-time ticks): 10 ms
// by default, far above any down projection it waits for.  A wait that runs
// out hands its rows to the rest pass.
std::atomic<int> g_wait_us{10000};

// The launch sequence of one layer forward into a workspace of p.total bytes
// (arguments already validated).  With sc, the down kernels raise the
// per-(segment, 64-row block) completion counters sc->sig and the combine
// runs on sc->consumer as their consumer (COMBINE_WAIT), followed on s by
// the rest pass for whatever it left.
int forward_impl(const Plan& p, const moe_desc* desc, const void* x, const uint8_t* valid_rows,
                 const void* router_w, const void* w13, const void* w2, void* out,
                 void* workspace, hipStream_t s, const SignalCtx* sc = nullptr) {
  void* ws = workspace;
  float* part = at<float>(ws, p.off_part);
  int32_t* ids = at<int32_t>(ws, p.off_ids);
  float* wts = at<float>(ws, p.off_w);
  int32_t* sorted = at<int32_t>(ws, p.off_sorted);
  int32_t* bexp = at<int32_t>(ws, p.off_bexp);
  int32_t* offs = at<int32_t>(ws, p.off_offs);
  int32_t* npost = at<int32_t>(ws, p.off_npost);
  int32_t* slot = at<int32_t>(ws, p.off_slot);
  int32_t* cnt = at<int32_t>(ws, p.off_cnt);
  int32_t* tseg = at<int32_t>(ws, p.off_tseg);
  int32_t* trow = at<int32_t>(ws, p.off_trow);
  int32_t* ntiles = at<int32_t>(ws, p.off_ntiles);
  int32_t* iseg = at<int32_t>(ws, p.off_iseg);
  int32_t* irow = at<int32_t>(ws, p.off_irow);
  int32_t* nitems = at<int32_t>(ws, p.off_nitems);
  const bool gemm = p.big_thr != INT_MAX;
  void* h = at<void>(ws, p.off_h);
  void* y = at<void>(ws, p.off_y);
  const int wkind = p.w == MOE_F32 ? moe::W_F32 : (p.w == MOE_BF16 ? moe::W_BF16 : moe::W_FP8);
  const bool packed = desc->w_layout == MOE_LAYOUT_FRAG16;

  {
    StageTimer tm(S_LOGITS, s);
    if (launch_logits(p, x, valid_rows, router_w, part, s) != hipSuccess) return MOE_ERR_HIP;
  }
  {
    StageTimer tm(S_TOPK, s);
    if (moe::launch_route_topk(part, p.ks, valid_rows, p.T, p.E, p.k, ids, wts,
                               nullptr, s) != hipSuccess)
      return MOE_ERR_HIP;
  }
  {
    StageTimer tm(S_ALIGN, s);
    if (moe::launch_align(ids, p.T, p.k, p.E, p.ns, p.bm, sorted, bexp, offs, npost,
                          slot, cnt, p.big_thr, p.min_tiles, gemm ? tseg : nullptr, trow,
                          ntiles, at<int32_t>(ws, p.off_span), iseg, irow, nitems,
                          s) != hipSuccess)
      return MOE_ERR_HIP;
  }
  if (p.one_launch) {
    // gate/up and down in one launch, the down units a wait left in the
    // streaming down kernel's rest pass, then the combine
    int32_t* one = at<int32_t>(ws, p.off_one);
    const moe::OneLaunch ol{one, one + 3, one + 3 + p.max_items, one + 1,
                            100LL * g_wait_us.load()};
    if (moe::launch_zero_i32(one, one_launch_words(p.max_items, p.H), nullptr, 0, s) !=
        hipSuccess)
      return MOE_ERR_HIP;
    {
      StageTimer tm(S_EXPERT_MLP, s);
      if (moe::launch_expert_mlp(wkind, packed, x, w13, w2, offs, cnt, sorted, iseg, irow,
                                 nitems, p.max_items, h, y, p.H, p.I, p.k, ol, s) != hipSuccess)
        return MOE_ERR_HIP;
    }
    {
      StageTimer tm(S_DOWN, s);
      if (moe::launch_down(wkind, packed, h, w2, desc->w2_scale, bexp, npost, offs, cnt, iseg,
                           irow, nitems, p.max_items, y, p.H, p.I, p.bm, p.cap,
                           p.yfmt == moe::Y_F24, s, moe::BlockSignals{nullptr, 0},
                           ol.undone) != hipSuccess)
        return MOE_ERR_HIP;
    }
    StageTimer tm(S_COMBINE, s);
    if (moe::launch_combine(y, p.yfmt, ids, wts, slot, p.T, p.H, p.k, p.ns, out,
                            p.act == MOE_BF16, s) != hipSuccess)
      return MOE_ERR_HIP;
    return MOE_OK;
  }
  // the streaming gate/up reads the token rows straight from x when every
  // segment streams, else from a fragment-ordered copy of the streaming
  // segments' rows
  if (wkind != moe::W_F32 && gemm) {
    StageTimer tm(S_PACK_X, s);
    if (moe::launch_pack_x_items(x, sorted, offs, cnt, iseg, irow, nitems, p.max_items, y, p.H,
                                 p.k, s) != hipSuccess)
      return MOE_ERR_HIP;
  }
  {
    StageTimer tm(S_GATE_UP, s);
    if (moe::launch_gate_up(wkind, packed, x, w13, desc->w13_scale, sorted, bexp, npost, offs,
                            cnt, iseg, irow, nitems, p.max_items, y, h, p.H, p.I, p.k, p.bm,
                            p.cap, !gemm, s) != hipSuccess)
      return MOE_ERR_HIP;
  }
  // the counters and the done flags start at zero in every signaled call
  const int nb64 = (p.T + 63) / 64;
  int32_t* done = at<int32_t>(ws, p.off_done);
  const size_t n_done = (size_t)p.T * done_chunks(p.H);
  if (sc != nullptr &&
      moe::launch_zero_i32(sc->sig, (size_t)(p.E + p.ns) * nb64, done, n_done + 1, s) != hipSuccess)
    return MOE_ERR_HIP;
  uint8_t* xq = p.xsplit ? at<uint8_t>(ws, p.off_xq) : nullptr;
  float* sx = p.xsplit ? at<float>(ws, p.off_sx) : nullptr;
  if (p.xsplit) {
    StageTimer tm(S_X_SPLIT, s);
    if (moe::launch_xq_split(x, valid_rows, xq, sx, p.T, p.H, s) != hipSuccess) return MOE_ERR_HIP;
  }
  if (gemm) {
    StageTimer tm(S_GATE_UP_GEMM, s);
    if (moe::launch_gate_up_gemm(wkind == moe::W_FP8, packed, x, w13, desc->w13_scale, sorted, tseg,
                                 trow, ntiles, offs, cnt, h, p.H, p.I, p.k, p.max_tiles, xq, sx,
                                 p.T, s) != hipSuccess)
      return MOE_ERR_HIP;
  }
  // signaled calls: the waiting combine may start once h is complete
  CallEvents evs;
  if (sc != nullptr && (!evs.make() || hipEventRecord(evs.ev[0], s) != hipSuccess))
    return MOE_ERR_HIP;
  const moe::BlockSignals bs{sc != nullptr ? sc->sig : nullptr, nb64};
  if (p.down_cols) {
    // the down projection and the combine in one launch
    StageTimer tm(S_DOWN, s);
    if (moe::launch_down_cols(wkind, packed, h, w2, desc->w2_scale, offs, cnt, sorted, ids, wts,
                              p.T, p.H, p.I, p.E, p.ns, p.k, out, s) != hipSuccess)
      return MOE_ERR_HIP;
    return MOE_OK;
  }
  {
    StageTimer tm(S_DOWN, s);
    if (moe::launch_down(wkind, packed, h, w2, desc->w2_scale, bexp, npost, offs, cnt, iseg,
                         irow, nitems, p.max_items, y, p.H, p.I, p.bm, p.cap, p.yfmt == moe::Y_F24,
                         s, bs) != hipSuccess)
      return MOE_ERR_HIP;
  }
  if (gemm) {
    StageTimer tm(S_DOWN_GEMM, s);
    if (moe::launch_down_gemm(wkind == moe::W_FP8, packed, h, w2, desc->w2_scale, tseg, trow, ntiles,
                              offs, cnt, y, p.H, p.I, p.max_tiles, s, bs) != hipSuccess)
      return MOE_ERR_HIP;
  }
  if (sc != nullptr) {
    const moe::CombineWait cw{sc->sig, offs, nb64, p.H, p.E, done, done + n_done,
                              100LL * g_wait_us.load()};
    if (hipStreamWaitEvent(sc->consumer, evs.ev[0], 0) != hipSuccess) return MOE_ERR_HIP;
    {
      StageTimer tm(S_COMBINE_WAIT, sc->consumer);
      if (moe::launch_combine(y, p.yfmt, ids, wts, slot, p.T, p.H, p.k, p.ns, out,
                              p.act == MOE_BF16, sc->consumer, moe::COMBINE_WAIT, &cw) != hipSuccess)
        return MOE_ERR_HIP;
    }
    if (hipEventRecord(evs.ev[1], sc->consumer) != hipSuccess ||
        hipStreamWaitEvent(s, evs.ev[1], 0) != hipSuccess)
      return MOE_ERR_HIP;
    StageTimer tm(S_COMBINE, s);
    if (moe::launch_combine(y, p.yfmt, ids, wts, slot, p.T, p.H, p.k, p.ns, out,
                            p.act == MOE_BF16, s, moe::COMBINE_REST, &cw) != hipSuccess)
      return MOE_ERR_HIP;
    return MOE_OK;
  }
  {
    StageTimer tm(S_COMBINE, s);
    if (moe::launch_combine(y, p.yfmt, ids, wts, slot, p.T, p.H, p.k, p.ns, out,
                            p.act == MOE_BF16, s) != hipSuccess)
      return MOE_ERR_HIP;
  }
  return MOE_OK;
}


// ---- fixed device scratch of moe_forward_noalloc ------------------------------
// One array per GPU, held from the library's load until the process ends.
// Host code never uses its name as an address: the device address of each
// GPU's copy comes from hipGetSymbolAddress, resolved once per device.
constexpr size_t kScratchBytes = size_t(MOE_SCRATCH_BYTES);
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This GPU's scratch (the current device), or nullptr on a HIP error.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

size_t moe_workspace_size(const moe_desc* desc, int32_t topk) {
  Plan p;
  if (make_plan(desc, topk, &p) != MOE_OK) return 0;
  return p.total;
}

int moe_pack_weights(const moe_desc* desc, const void* w13, const void* w2, void* w13_packed,
                     void* w2_packed, moe_stream_t stream) {
  if (desc == nullptr) return MOE_ERR_INVALID_ARG;
  moe_desc d = *desc;
  d.w_layout = MOE_LAYOUT_FRAG16;
  const int st = check_desc(&d, 1, /*need_scales=*/false);
  if (st != MOE_OK) return st;
  if (!w13 || !w2 || !w13_packed || !w2_packed) return MOE_ERR_INVALID_ARG;
  const int wkind = d.w_dtype == MOE_BF16 ? moe::W_BF16 : moe::W_FP8;
  const size_t ne = (size_t)d.E + d.n_shared;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (moe::launch_pack_weights(wkind, w13, w13_packed, ne * 2 * d.I, d.H, s) != hipSuccess ||
      moe::launch_pack_weights(wkind, w2, w2_packed, ne * d.H, d.I, s) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

int moe_set_path_thresholds(int32_t gemm_min_rows, int32_t gemm_min_tiles) {
  if (gemm_min_rows < 0 || gemm_min_tiles < -1) return MOE_ERR_INVALID_ARG;
  g_gemm_min_rows.store(gemm_min_rows);
  g_gemm_min_tiles.store(gemm_min_tiles);
  return MOE_OK;
}

int moe_set_signal_wait_us(int32_t us) {
  if (us < 0 || us > 1000000) return MOE_ERR_INVALID_ARG;
  g_wait_us.store(us);
  return MOE_OK;
}

int moe_set_one_launch(int32_t enable) {
  if (enable != 0 && enable != 1) return MOE_ERR_INVALID_ARG;
  g_one_launch.store(enable);
  return MOE_OK;
}

int moe_set_fp8_mfma(int32_t enable) {
  if (enable != 0 && enable != 1) return MOE_ERR_INVALID_ARG;
  g_fp8_mfma.store(enable);
  return MOE_OK;
}

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported dtype combination or shape";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

int moe_route(const moe_desc* desc, const void* x, const uint8_t* valid_rows,
              const void* router_w, int32_t topk, int32_t* topk_ids,
              float* topk_w, float* logits, void* workspace,
              size_t workspace_bytes, moe_stream_t stream) {
  Plan p;
  const int st = make_plan(desc, topk, &p);
  if (st != MOE_OK) return st;
  if (!x || !router_w || !topk_ids || !topk_w || !workspace) return MOE_ERR_INVALID_ARG;
  if (workspace_bytes < p.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* part = at<float>(workspace, p.off_part);
  if (launch_logits(p, x, valid_rows, router_w, part, s) != hipSuccess) return MOE_ERR_HIP;
  if (moe::launch_route_topk(part, p.ks, valid_rows, p.T, p.E, p.k, topk_ids,
                             topk_w, logits, s) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

int moe_align(const moe_desc* desc, const int32_t* topk_ids, int32_t topk,
              int32_t block_m, int32_t* sorted_ids, int32_t* block_expert,
              int32_t* expert_offsets, int32_t* n_post_padded, void* workspace,
              size_t workspace_bytes, moe_stream_t stream) {
  if (desc == nullptr) return MOE_ERR_INVALID_ARG;
  if (desc->T < 1 || desc->E < 1 || desc->E > kMaxE) return MOE_ERR_INVALID_ARG;
  if (desc->n_shared < 0 || desc->n_shared > 1) return MOE_ERR_INVALID_ARG;
  if (topk < 1 || topk > desc->E || topk > kMaxTopk) return MOE_ERR_INVALID_ARG;
  if (block_m < 1 || block_m > 256) return MOE_ERR_INVALID_ARG;
  if (!topk_ids || !sorted_ids || !block_expert || !expert_offsets || !n_post_padded)
    return MOE_ERR_INVALID_ARG;
  const int ns = desc->n_shared;
  if ((long long)desc->T * (topk + ns) + (long long)(desc->E + ns) * block_m > (1LL << 30))
    return MOE_ERR_UNSUPPORTED;
  // batches of more than 8192 assignments: the span-parallel kernels when a
  // workspace is given, else one block does the whole list (same result)
  int32_t* span = nullptr;
  const int n_span = moe::align_spans(desc->T, topk, ns);
  if (n_span > 0 && workspace != nullptr) {
    if (workspace_bytes < (size_t)n_span * (desc->E + ns) * sizeof(int32_t))
      return MOE_ERR_WORKSPACE;
    span = static_cast<int32_t*>(workspace);
  }
  if (moe::launch_align(topk_ids, desc->T, topk, desc->E, ns, block_m, sorted_ids,
                        block_expert, expert_offsets, n_post_padded, nullptr, nullptr,
                        INT_MAX, 0, nullptr, nullptr, nullptr, span, nullptr, nullptr,
                        nullptr, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

int moe_forward(const moe_desc* desc, const void* x, const uint8_t* valid_rows,
                const void* router_w, const void* w13, const void* w2,
                int32_t topk, void* out, void* workspace,
                size_t workspace_bytes, moe_stream_t stream) {
  Plan p;
  const int st = make_plan(desc, topk, &p);
  if (st != MOE_OK) return st;
  if (!x || !router_w || !w13 || !w2 || !out || !workspace) return MOE_ERR_INVALID_ARG;
  if (workspace_bytes < p.total) return MOE_ERR_WORKSPACE;
  return forward_impl(p, desc, x, valid_rows, router_w, w13, w2, out, workspace,
                      static_cast<hipStream_t>(stream));
}

size_t moe_block_signal_count(const moe_desc* desc) {
  if (desc == nullptr || desc->T < 1 || desc->E < 1 || desc->n_shared < 0) return 0;
  return signal_count(desc);
}

int moe_forward_signaled(const moe_desc* desc, const void* x, const uint8_t* valid_rows,
                         const void* router_w, const void* w13, const void* w2, int32_t topk,
                         void* out, void* workspace, size_t workspace_bytes,
                         int32_t* block_signal, moe_stream_t stream,
                         moe_stream_t consumer_stream) {
  Plan p;
  const int st = make_plan(desc, topk, &p);
  if (st != MOE_OK) return st;
  if (!x || !router_w || !w13 || !w2 || !out || !workspace || !block_signal)
    return MOE_ERR_INVALID_ARG;
  // the fp32 kernels raise no signals
  if (p.w == MOE_F32 || p.act != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (workspace_bytes < p.total) return MOE_ERR_WORKSPACE;
  // the per-assignment y rows are the signals' subject: no one-launch down +
  // combine, and the down units are those of the streaming down kernel
  p.down_cols = false;
  p.one_launch = false;
  const SignalCtx sc{block_signal, static_cast<hipStream_t>(consumer_stream)};
  return forward_impl(p, desc, x, valid_rows, router_w, w13, w2, out, workspace,
                      static_cast<hipStream_t>(stream), &sc);
}

int moe_forward_noalloc(const moe_desc* desc, const void* x, const uint8_t* valid_rows,
                        const void* router_w, const void* w13, const void* w2,
                        int32_t topk, void* out, moe_stream_t stream) {
  Plan p;
  const int st = make_plan(desc, topk, &p);
  if (st != MOE_OK) return st;
  if (!x || !router_w || !w13 || !w2 || !out) return MOE_ERR_INVALID_ARG;
  if (p.total > kScratchBytes) return MOE_ERR_WORKSPACE;
  void* ws = device_scratch();
  if (ws == nullptr) return MOE_ERR_HIP;
  return forward_impl(p, desc, x, valid_rows, router_w, w13, w2, out, ws,
                      static_cast<hipStream_t>(stream));
}

int moe_num_stages(void) { return S_COUNT; }

const char* moe_stage_name(int stage) {
  return (stage >= 0 && stage < S_COUNT) ? kStageNames[stage] : "";
}

int moe_profile_enable(int stage_mask) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_mask = static_cast<unsigned>(stage_mask) & ((1u << S_COUNT) - 1u);
  return MOE_OK;
}

int moe_profile_read(double* stage_ms, int32_t* stage_launches, int32_t n) {
  if (stage_ms == nullptr || stage_launches == nullptr || n < 0) return MOE_ERR_INVALID_ARG;
  std::vector<ProfRecord> recs;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    recs.swap(g_prof);
  }
  for (int i = 0; i < n; ++i) {
    stage_ms[i] = 0.0;
    stage_launches[i] = 0;
  }
  int status = MOE_OK;
  for (const ProfRecord& r : recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      status = MOE_ERR_HIP;
    else if (r.stage < n) {
      stage_ms[r.stage] += ms;
      stage_launches[r.stage] += 1;
    }
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  return status;
}

}  // extern "C"
