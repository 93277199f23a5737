// Host side of the C ABI declared in include/hs2.h: argument validation, the
// workspace plan, and the launch sequence of each entry point.  Nothing here
// allocates, frees or synchronises, except the measurement entry point
// hs2_cross_decoder_step_timed, which synchronises its stream at the end.
// hs2_cross_decoder_step_static runs on a device buffer the library holds
// (a file-scope device array, below), not on a caller's workspace.

#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "hs2_internal.h"

namespace hs2 {
namespace {

static_assert(sizeof(hs2_shape) == 64, "hs2_shape layout is part of the ABI");
static_assert(sizeof(hs2_bridge_shape) == 40, "hs2_bridge_shape layout is part of the ABI");

thread_local int g_last_hip_error = 0;

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Compute units of the current device, read once per device (the decode full
// layer is planned as one work-group per compute unit).  Without a device to
// ask (a host-only process sizing a workspace) the MI355X's 256 are assumed.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return kDefaultCUs;
  }
  const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
  if (cached > 0) return cached;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    n = kDefaultCUs;
  }
  g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Validate a shape and lay out the workspace.  Returns HS2_OK or an error code.
int make_plan(const hs2_shape* sh, int n_layers, Plan* p) {
  if (!sh || !p) return HS2_ERR_INVALID_ARG;
  if (sh->ctx_len < 1 || sh->batch < 1 || sh->n_q_tokens < 1 || sh->n_q_heads < 1 ||
      sh->n_kv_heads < 1 || sh->head_dim < 1 || sh->top_k < 0 || sh->window < 0 ||
      n_layers < 0 || sh->decode_splits < 0 || sh->decode_select < 0 || sh->decode_select > 2)
    return HS2_ERR_INVALID_ARG;
  const int32_t bs = sh->select_block;
  if (bs != 0) {
    if (bs < 16 || bs > 256 || (bs & (bs - 1)) != 0 || sh->top_k % bs != 0)
      return HS2_ERR_INVALID_ARG;
    if ((sh->ctx_len + bs - 1) / bs > 16384) return HS2_ERR_UNSUPPORTED;
  }
  if (!(sh->scale > 0.0) || !isfinite(sh->scale)) return HS2_ERR_INVALID_ARG;
  if (sh->n_q_tokens > sh->ctx_len) return HS2_ERR_INVALID_ARG;
  if (sh->kv_capacity != 0 && sh->kv_capacity < sh->ctx_len) return HS2_ERR_INVALID_ARG;
  if (sh->n_q_heads % sh->n_kv_heads != 0) return HS2_ERR_INVALID_ARG;
  if (static_cast<int64_t>(sh->top_k) + sh->window < 1) return HS2_ERR_INVALID_ARG;
  if (sh->head_dim != kD || sh->n_q_heads != kG * sh->n_kv_heads) return HS2_ERR_UNSUPPORTED;
  if (sh->ctx_len >= (int64_t{1} << 31)) return HS2_ERR_UNSUPPORTED;
  if (sh->kv_capacity >= (int64_t{1} << 40)) return HS2_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(sh->top_k) + sh->window > kMaxSel) return HS2_ERR_UNSUPPORTED;
  const int64_t R = static_cast<int64_t>(sh->batch) * sh->n_q_tokens * sh->n_kv_heads;
  if (R > 65535) return HS2_ERR_UNSUPPORTED;

  Plan q{};
  q.S = sh->ctx_len;
  q.Spad = static_cast<int64_t>(align_up(static_cast<size_t>(q.S), 64));
  q.kvp = sh->kv_capacity != 0 ? sh->kv_capacity : q.S;
  q.bs = sh->select_block;
  q.B = sh->batch;
  q.T = sh->n_q_tokens;
  q.Hq = sh->n_q_heads;
  q.Hkv = sh->n_kv_heads;
  q.R = static_cast<int>(R);
  q.k = sh->top_k;
  q.w = sh->window;
  q.cap = sh->top_k + sh->window;
  q.n_layers = n_layers;
  q.n_cu = device_cu_count();
  q.scale = sh->scale;

  // full attention, decode: about one work-group per compute unit, so that
  // the stream runs in one round with no tail (a count that leaves some CUs a
  // second work-group streams much slower)
  {
    const int64_t target = q.n_cu;
    int64_t ns = ceil_div(target, R);
    ns = std::max<int64_t>(1, std::min<int64_t>(ns, ceil_div(q.S, 256)));
    if (sh->decode_splits > 0)   // the caller's split count
      ns = std::max<int64_t>(1, std::min<int64_t>(sh->decode_splits, ceil_div(q.S, 128)));
    ns = std::min<int64_t>(ns, int64_t{kMaxSplits});
    int64_t kps = align_up(static_cast<size_t>(ceil_div(q.S, ns)), 128);
    q.kps = static_cast<int>(kps);
    q.n_split = static_cast<int>(ceil_div(q.S, kps));
  }
  // selection from given scores: ~256 work-groups over the rows, at most 16384
  // keys per work-group (the compaction keeps 64 keys per thread in bit masks)
  {
    int64_t chunk = align_up(static_cast<size_t>(ceil_div(q.S * R, 256)), 2048);
    chunk = std::max<int64_t>(chunk, 4096);
    chunk = std::min<int64_t>(chunk, 16384);
    q.sel_chunk = static_cast<int>(chunk);
    q.sel_nchunk = static_cast<int>(ceil_div(q.S, chunk));
  }
  // fused selection: subtiles of 16 keys, ~256 work-groups, <= 8192 per group
  const int64_t nst = q.Spad / 16;
  {
    // bound histogram: about 256 work-groups
    int64_t hc = align_up(static_cast<size_t>(ceil_div(nst * R, 256)), 256);
    hc = std::min<int64_t>(std::max<int64_t>(hc, 256), 8192);
    q.hs_chunk = static_cast<int>(hc);
    q.hs_nchunk = static_cast<int>(ceil_div(nst, hc));
    // candidate-subtile lists: about 1024 work-groups, whole rounds of
    // kScoreRound subtiles, at most kMaxChunks per row
    int64_t cc = align_up(static_cast<size_t>(ceil_div(nst * R, 1024)), kScoreRound);
    cc = std::max<int64_t>(cc, kScoreRound);
    cc = std::max<int64_t>(cc, static_cast<int64_t>(align_up(static_cast<size_t>(ceil_div(nst, kMaxChunks)), kScoreRound)));
    q.cc_chunk = static_cast<int>(cc);
    q.cc_nchunk = static_cast<int>(ceil_div(nst, cc));
    // scoring: three work-groups per compute unit (all resident at once), each
    // taking an equal share of its row's candidate list, so that clustered
    // candidates do not queue on a few work-groups
    int64_t ns = std::min<int64_t>(ceil_div(3 * q.n_cu, R), std::min<int64_t>(kMaxChunks, nst));
    ns = std::max<int64_t>(ns, 1);
    q.sc_nchunk = static_cast<int>(ns);
    q.sc_chunk = static_cast<int>(ceil_div(nst, ns));   // list entries a region holds
  }
  // refinement of lse2 (decode): about two work-groups per compute unit over
  // all rows (all resident at once), each taking an equal share of its row's
  // dominant subtiles
  q.ref_nwg = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(ceil_div(2 * q.n_cu, R), 1024)));
  // sparse: slices of 128 keys over work-groups when rows are few
  q.sp_nch = (R >= 256) ? 1 : static_cast<int>(ceil_div(q.cap, kSparseChunk));

  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, kAlign);
    return o;
  };
  const size_t Rz = static_cast<size_t>(R);
  const size_t nsplit_rows = Rz * q.n_split;
  const bool decode = q.T == 1;
  q.off_part_m = take(decode ? nsplit_rows * kG * sizeof(float) : 0);
  q.off_part_l = take(decode ? nsplit_rows * kG * sizeof(double) : 0);
  q.off_part_o = take(decode ? nsplit_rows * kG * kD * sizeof(float) : 0);
  q.off_stmax = take(decode ? Rz * nst * kG * sizeof(float) : 0);
  // the quads' distances pay where the selection re-reads many subtiles: when
  // top_k is at least 1/64 of the context (a subtile then holds a selected
  // key with probability about 1/4 or more)
  q.quads = decode && q.k > 0 && q.S <= int64_t{64} * q.k;
  q.off_qdiff = take(q.quads ? Rz * nst * 4 * kG : 0);
  // the dense decode selection (short contexts): every key's importance, then
  // the prefill chunk's per-row selection; the caller may choose either way
  q.dense_dec = decode && (sh->decode_select == 2 ||
                           (sh->decode_select == 0 &&
                            Rz * static_cast<size_t>(q.S) * kD * 2 <= static_cast<size_t>(kDenseDecodeBytes)));
  q.n_ib = static_cast<int>(decode ? ceil_div(q.S, kDecImpKeys) : ceil_div(q.T, kImportanceTok));
  const bool row_select = !decode || q.dense_dec;   // the per-row selection kernel runs
  q.off_lse2 = take(Rz * kG * sizeof(double));
  q.off_ytop = take(Rz * kG * sizeof(float));
  q.off_hist = take(Rz * kNB * sizeof(uint32_t));
  q.off_info = take(Rz * sizeof(RowInfo));
  q.off_ukey = take(Rz * q.Spad * sizeof(uint32_t));
  q.off_cert = take(Rz * align_up(static_cast<size_t>(q.k), 64) * sizeof(int32_t));
  q.off_unc = take(Rz * kUncCap * sizeof(int32_t));
  q.off_unck = take(Rz * kUncCap * sizeof(uint64_t));
  q.off_hist_c = take(decode ? Rz * kNB * sizeof(uint32_t) : 0);
  q.off_clist = take(decode ? Rz * q.cc_nchunk * static_cast<size_t>(q.cc_chunk) * sizeof(int32_t) : 0);
  q.off_ccnt = take(decode ? Rz * q.cc_nchunk * sizeof(uint32_t) : 0);
  q.off_lo = take(decode ? Rz * sizeof(int32_t) : 0);
  const size_t cz = decode ? Rz * static_cast<size_t>(q.sc_nchunk) * q.sc_chunk * 16 : 0;
  q.off_cand_y = take(cz * sizeof(double));
  q.off_cand_idx = take(cz * sizeof(int32_t));
  q.off_cand_cnt = take(decode ? Rz * q.sc_nchunk * sizeof(uint32_t) : 0);
  // band lists: a whole row's worth in decode; in a prefill chunk (many rows)
  // a bounded list per row, but one entry per block for block selection, so
  // that any band of blocks is ranked exactly
  q.band_cap = row_select ? std::min<int64_t>(q.Spad, kPrefillBandCap) : 0;
  if (row_select && q.bs > 0) q.band_cap = std::max<int64_t>(q.band_cap, ceil_div(q.S, q.bs));
  q.off_band_idx = take(Rz * q.band_cap * sizeof(int32_t));
  q.off_band_key = take(Rz * q.band_cap * sizeof(uint64_t));
  // the fixed-point importance of a prefill chunk shares the key buffer of the
  // selection from given scores: no call uses both
  q.off_ybuf = q.off_ukey;
  // per (batch, KV head, importance work-group): that work-group's share of max |k|
  q.off_kmax = take(row_select ? static_cast<size_t>(q.B) * q.Hkv * q.n_ib * sizeof(uint32_t) : 0);
  q.off_ref_part = take(decode ? Rz * q.ref_nwg * sizeof(RefinePart) : 0);
  q.off_dsub = take(decode ? Rz * q.cc_nchunk * static_cast<size_t>(q.cc_chunk) * sizeof(int32_t) : 0);
  q.off_dsub_cnt = take(decode ? Rz * q.cc_nchunk * sizeof(uint32_t) : 0);
  q.off_cut = take(decode ? Rz * sizeof(float) : 0);
  q.off_lse2r = take(Rz * kG * sizeof(double));
  q.off_ref_stat = take(Rz * sizeof(RefineStat));
  q.off_dom_list = take(row_select ? Rz * kDomCap * sizeof(int32_t) : 0);
  const size_t sp_parts = q.sp_nch > 1 ? Rz * q.sp_nch * n_layers * kG : 0;
  q.off_sp_m = take(sp_parts * sizeof(float));
  q.off_sp_l = take(sp_parts * sizeof(float));
  q.off_sp_o = take(sp_parts * kD * sizeof(float));
  q.off_idx_bad = take(Rz * q.sp_nch * sizeof(uint32_t));
  q.off_swa = take(Rz * static_cast<size_t>(n_layers) * kG * kD * sizeof(float));
  q.total = off;
  *p = q;
  return HS2_OK;
}

int check_ws(const Plan& p, void* ws, size_t ws_bytes) {
  if (!ws) return HS2_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return HS2_ERR_INVALID_ARG;
  if (ws_bytes < p.total) return HS2_ERR_WORKSPACE;
  return HS2_OK;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return HS2_OK;
  g_last_hip_error = static_cast<int>(e);
  return HS2_ERR_HIP;
}

}  // namespace

int record_hip_error(hipError_t e) { return hip_status(e); }

namespace {

#define HS2_TRY(expr)                        \
  do {                                       \
    const int st_ = hip_status((expr));      \
    if (st_ != HS2_OK) return st_;           \
  } while (0)

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int run_full(const Plan& p, const u16* q, const u16* k, const u16* v, u16* out, float* lse,
             void* ws, hipStream_t st) {
  HS2_TRY(launch_full_decode_split(p, q, k, v, ws, st));
  HS2_TRY(launch_full_combine(p, out, lse, ws, st));
  return HS2_OK;
}

}  // namespace
}  // namespace hs2

using namespace hs2;

extern "C" {

size_t hs2_workspace_bytes(const hs2_shape* shape, int32_t n_sparse_layers) {
  Plan p;
  if (make_plan(shape, n_sparse_layers, &p) != HS2_OK) return 0;
  return p.total;
}

int hs2_full_attn_scores(const hs2_shape* shape, const hs2_bf16* q, const hs2_bf16* k,
                         const hs2_bf16* v, hs2_bf16* out, float* lse, float* scores, void* ws,
                         size_t ws_bytes, void* stream) {
  Plan p;
  int st = make_plan(shape, 0, &p);
  if (st != HS2_OK) return st;
  if (!q || !k || !v || !out) return HS2_ERR_INVALID_ARG;
  if ((st = check_ws(p, ws, ws_bytes)) != HS2_OK) return st;
  (void)hipGetLastError();
  const hipStream_t s = as_stream(stream);
  if (p.T != 1) {
    HS2_TRY(launch_full_prefill(p, q, k, v, out, lse, ws, s));
    if (scores) HS2_TRY(launch_prefill_scores(p, q, k, scores, s));
    return HS2_OK;
  }
  if ((st = run_full(p, q, k, v, out, lse, ws, s)) != HS2_OK) return st;
  // the refined normaliser (lse and the scores): the selection's subtile-bound
  // histogram places the refinement's cut and its candidate kernel lists the
  // dominant subtiles
  HS2_TRY(launch_subtile_hist(p, ws, s));
  HS2_TRY(launch_subtile_cand(p, ws, s));
  HS2_TRY(launch_lse_refine(p, q, k, ws, s));
  HS2_TRY(launch_lse_finalize(p, lse, ws, s));
  if (scores) HS2_TRY(launch_full_scores(p, q, k, scores, ws, s));
  return HS2_OK;
}

int hs2_topk_select(const hs2_shape* shape, const float* scores, int32_t* idx, int32_t* n_sel,
                    void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  int st = make_plan(shape, 0, &p);
  if (st != HS2_OK) return st;
  if (!scores || !idx || !n_sel) return HS2_ERR_INVALID_ARG;
  if ((st = check_ws(p, ws, ws_bytes)) != HS2_OK) return st;
  (void)hipGetLastError();
  const hipStream_t s = as_stream(stream);
  HS2_TRY(launch_scores_select(p, scores, idx, n_sel, ws, s));
  return HS2_OK;
}

int hs2_sparse_attn(const hs2_shape* shape, int32_t n_layers, const hs2_bf16* q,
                    const hs2_bf16* k, const hs2_bf16* v, const int32_t* idx,
                    const int32_t* n_sel, hs2_bf16* out, void* ws, size_t ws_bytes,
                    void* stream) {
  Plan p;
  int st = make_plan(shape, n_layers, &p);
  if (st != HS2_OK) return st;
  if (n_layers < 1 || !q || !k || !v || !idx || !n_sel || !out) return HS2_ERR_INVALID_ARG;
  if ((st = check_ws(p, ws, ws_bytes)) != HS2_OK) return st;
  (void)hipGetLastError();
  HS2_TRY(launch_sparse(p, q, k, v, idx, n_sel, out, ws, as_stream(stream)));
  return HS2_OK;
}

}  // extern "C"

namespace hs2 {
namespace {

// the argument checks of a step, before any workspace is looked at
int check_step_args(const Plan& p, int32_t n_sparse_layers, const hs2_bf16* q_full,
                    const hs2_bf16* q_sparse, const hs2_bf16* k, const hs2_bf16* v,
                    const hs2_bf16* out_full, const hs2_bf16* out_sparse, const int32_t* idx,
                    const int32_t* n_sel) {
  if (!q_full || !k || !v || !out_full || !idx || !n_sel) return HS2_ERR_INVALID_ARG;
  if (n_sparse_layers > 0 && (!q_sparse || !out_sparse)) return HS2_ERR_INVALID_ARG;
  return HS2_OK;
}

// one step's launches on a checked plan and workspace
int run_step(const Plan& p, int32_t n_sparse_layers, const hs2_bf16* q_full,
             const hs2_bf16* q_sparse, const hs2_bf16* k, const hs2_bf16* v, hs2_bf16* out_full,
             hs2_bf16* out_sparse, int32_t* idx, int32_t* n_sel, float* lse, float* scores,
             void* ws, hipStream_t s) {
  int st;
  if (p.T != 1) {
    HS2_TRY(launch_full_prefill(p, q_full, k, v, out_full, lse, ws, s));
    HS2_TRY(launch_prefill_importance(p, q_full, k, ws, s));
    HS2_TRY(launch_prefill_select(p, q_full, k, idx, n_sel, lse, ws, s));
    if (scores) HS2_TRY(launch_prefill_scores(p, q_full, k, scores, s));
    if (n_sparse_layers > 0)
      HS2_TRY(launch_sparse(p, q_sparse, k, v, idx, n_sel, out_sparse, ws, s));
    return HS2_OK;
  }
  if ((st = run_full(p, q_full, k, v, out_full, lse, ws, s)) != HS2_OK) return st;
  if (p.dense_dec) {
    HS2_TRY(launch_decode_importance(p, q_full, k, ws, s));
    HS2_TRY(launch_prefill_select(p, q_full, k, idx, n_sel, lse, ws, s));
  } else {
    HS2_TRY(launch_fused_select(p, q_full, k, idx, n_sel, lse, ws, s));
  }
  if (scores) HS2_TRY(launch_full_scores(p, q_full, k, scores, ws, s));
  if (n_sparse_layers > 0)
    HS2_TRY(launch_sparse(p, q_sparse, k, v, idx, n_sel, out_sparse, ws, s));
  return HS2_OK;
}

// ---- the library-held workspace of hs2_cross_decoder_step_static
//
// One buffer per GPU: a file-scope device array, so that it exists on every
// device the library's code object is loaded on.  Host code never passes the
// array's name to a kernel (on the host it names a stand-in, not device
// memory): each device's address is looked up once, with that device current,
// and kept in g_scratch_dev[device].
static __device__ __align__(256) unsigned char scratch[HS2_STATIC_SCRATCH_BYTES];

std::atomic<void*> g_scratch_dev[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's scratch address, looked up on its first use; nullptr
// with *err set when the lookup fails.
void* scratch_of_current_device(int* err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *err = hip_status(e);
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *err = HS2_ERR_UNSUPPORTED;
    return nullptr;
  }
  void* ptr = g_scratch_dev[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ptr = g_scratch_dev[dev].load(std::memory_order_relaxed);
  if (ptr) return ptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr) {
    *err = hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol);
    return nullptr;
  }
  g_scratch_dev[dev].store(ptr, std::memory_order_release);
  return ptr;
}

}  // namespace
}  // namespace hs2

extern "C" {

int hs2_cross_decoder_step(const hs2_shape* shape, int32_t n_sparse_layers,
                           const hs2_bf16* q_full, const hs2_bf16* q_sparse, const hs2_bf16* k,
                           const hs2_bf16* v, hs2_bf16* out_full, hs2_bf16* out_sparse,
                           int32_t* idx, int32_t* n_sel, float* lse, float* scores, void* ws,
                           size_t ws_bytes, void* stream) {
  Plan p;
  int st = make_plan(shape, n_sparse_layers, &p);
  if (st != HS2_OK) return st;
  if ((st = check_step_args(p, n_sparse_layers, q_full, q_sparse, k, v, out_full, out_sparse,
                            idx, n_sel)) != HS2_OK)
    return st;
  if ((st = check_ws(p, ws, ws_bytes)) != HS2_OK) return st;
  (void)hipGetLastError();
  return run_step(p, n_sparse_layers, q_full, q_sparse, k, v, out_full, out_sparse, idx, n_sel,
                  lse, scores, ws, as_stream(stream));
}

int hs2_cross_decoder_step_static(const hs2_shape* shape, int32_t n_sparse_layers,
                                  const hs2_bf16* q_full, const hs2_bf16* q_sparse,
                                  const hs2_bf16* k, const hs2_bf16* v, hs2_bf16* out_full,
                                  hs2_bf16* out_sparse, int32_t* idx, int32_t* n_sel,
                                  float* lse, float* scores, void* stream) {
  Plan p;
  int st = make_plan(shape, n_sparse_layers, &p);
  if (st != HS2_OK) return st;
  if ((st = check_step_args(p, n_sparse_layers, q_full, q_sparse, k, v, out_full, out_sparse,
                            idx, n_sel)) != HS2_OK)
    return st;
  if (p.total > HS2_STATIC_SCRATCH_BYTES) return HS2_ERR_SCRATCH;
  (void)hipGetLastError();
  void* ws = scratch_of_current_device(&st);
  if (!ws) return st;
  // the step's kernels clear every counter and histogram they accumulate into,
  // so the previous call's contents need no clearing here
  return run_step(p, n_sparse_layers, q_full, q_sparse, k, v, out_full, out_sparse, idx, n_sel,
                  lse, scores, ws, as_stream(stream));
}

int hs2_cross_decoder_step_timed(const hs2_shape* shape, int32_t n_sparse_layers,
                                 const hs2_bf16* q_full, const hs2_bf16* q_sparse,
                                 const hs2_bf16* k, const hs2_bf16* v, hs2_bf16* out_full,
                                 hs2_bf16* out_sparse, int32_t* idx, int32_t* n_sel, void* ws,
                                 size_t ws_bytes, void* stream, int32_t iters, float* phase_ms) {
  Plan p;
  int st = make_plan(shape, n_sparse_layers, &p);
  if (st != HS2_OK) return st;
  if (!q_full || !k || !v || !out_full || !idx || !n_sel || !phase_ms || iters < 1)
    return HS2_ERR_INVALID_ARG;
  if (n_sparse_layers > 0 && (!q_sparse || !out_sparse)) return HS2_ERR_INVALID_ARG;
  if ((st = check_ws(p, ws, ws_bytes)) != HS2_OK) return st;
  (void)hipGetLastError();
  const hipStream_t s = as_stream(stream);
  hipEvent_t ev[5];
  for (int i = 0; i < 5; ++i) {
    const hipError_t e = hipEventCreate(&ev[i]);
    if (e != hipSuccess) {
      for (int j = 0; j < i; ++j) (void)hipEventDestroy(ev[j]);
      return hip_status(e);
    }
  }
  double acc[4] = {0, 0, 0, 0};
  int rc = HS2_OK;
  for (int it = 0; it < iters && rc == HS2_OK; ++it) {
    float ms[4] = {0, 0, 0, 0};
    const bool decode = p.T == 1;
    rc = hip_status(hipEventRecord(ev[0], s));
    if (rc == HS2_OK)
      rc = hip_status(decode ? launch_full_decode_split(p, q_full, k, v, ws, s)
                             : launch_full_prefill(p, q_full, k, v, out_full, nullptr, ws, s));
    if (rc == HS2_OK) rc = hip_status(hipEventRecord(ev[1], s));
    if (rc == HS2_OK && decode) rc = hip_status(launch_full_combine(p, out_full, nullptr, ws, s));
    if (rc == HS2_OK) rc = hip_status(hipEventRecord(ev[2], s));
    const bool by_rows = !decode || p.dense_dec;   // importance pass, then the per-row selection
    if (rc == HS2_OK)
      rc = hip_status(!by_rows ? launch_fused_select(p, q_full, k, idx, n_sel, nullptr, ws, s)
                      : decode ? launch_decode_importance(p, q_full, k, ws, s)
                               : launch_prefill_importance(p, q_full, k, ws, s));
    if (rc == HS2_OK && by_rows)
      rc = hip_status(launch_prefill_select(p, q_full, k, idx, n_sel, nullptr, ws, s));
    if (rc == HS2_OK) rc = hip_status(hipEventRecord(ev[3], s));
    if (rc == HS2_OK && n_sparse_layers > 0)
      rc = hip_status(launch_sparse(p, q_sparse, k, v, idx, n_sel, out_sparse, ws, s));
    if (rc == HS2_OK) rc = hip_status(hipEventRecord(ev[4], s));
    if (rc == HS2_OK) rc = hip_status(hipEventSynchronize(ev[4]));
    for (int i = 0; i < 4 && rc == HS2_OK; ++i) {
      rc = hip_status(hipEventElapsedTime(&ms[i], ev[i], ev[i + 1]));
      acc[i] += ms[i];
    }
  }
  for (int i = 0; i < 5; ++i) (void)hipEventDestroy(ev[i]);
  if (rc != HS2_OK) return rc;
  for (int i = 0; i < 4; ++i) phase_ms[i] = static_cast<float>(acc[i] / iters);
  return HS2_OK;
}

int hs2_kv_bridge(const hs2_bridge_shape* shape, const hs2_bf16* hidden, const hs2_bf16* w_kv,
                  hs2_bf16* k, hs2_bf16* v, void* stream) {
  if (!shape || !hidden || !w_kv || !k || !v) return HS2_ERR_INVALID_ARG;
  const hs2_bridge_shape& s = *shape;
  if (s.batch < 1 || s.n_tokens < 1 || s.d_model < 1 || s.n_kv_heads < 1 || s.head_dim < 1 ||
      s.kv_capacity < 1 || s.pos0 < 0 || s.reserved != 0)
    return HS2_ERR_INVALID_ARG;
  if (s.pos0 > s.kv_capacity - s.n_tokens) return HS2_ERR_INVALID_ARG;
  if (s.head_dim != kD || s.d_model % 64 != 0) return HS2_ERR_UNSUPPORTED;
  // the many-token kernel addresses 256 rows of a tile with 32-bit byte offsets
  if (static_cast<int64_t>(s.batch) * s.n_tokens >= (int64_t{1} << 31) ||
      s.kv_capacity >= (int64_t{1} << 40) || s.n_kv_heads > 4096 || s.d_model > (1 << 20))
    return HS2_ERR_UNSUPPORTED;
  BridgeArgs a{};
  a.hidden = hidden;
  a.w = w_kv;
  a.k = k;
  a.v = v;
  a.kvp = s.kv_capacity;
  a.pos0 = s.pos0;
  a.M = s.batch * s.n_tokens;
  a.n_tok = s.n_tokens;
  a.dm = s.d_model;
  a.Hkv = s.n_kv_heads;
  (void)hipGetLastError();
  HS2_TRY(launch_kv_bridge(a, as_stream(stream)));
  return HS2_OK;
}

int hs2_sparse_attn_swa(const hs2_shape* shape, int32_t n_layers, const hs2_bf16* q,
                        const hs2_bf16* k, const hs2_bf16* v, const int32_t* idx,
                        const int32_t* n_sel, const hs2_bf16* k_loc, const hs2_bf16* v_loc,
                        hs2_bf16* out, void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  int st = make_plan(shape, n_layers, &p);
  if (st != HS2_OK) return st;
  if (n_layers < 1 || !q || !k || !v || !idx || !n_sel || !out) return HS2_ERR_INVALID_ARG;
  // the local caches have min(S, T + w - 1) rows: none (and may be NULL) when w = 0, T = 1
  const bool has_local = std::min<int64_t>(p.S, static_cast<int64_t>(p.T) + p.w - 1) > 0;
  if (has_local && (!k_loc || !v_loc)) return HS2_ERR_INVALID_ARG;
  if ((st = check_ws(p, ws, ws_bytes)) != HS2_OK) return st;
  (void)hipGetLastError();
  // (with no local rows the caches may be NULL: the window branch then reads nothing)
  HS2_TRY(launch_sparse(p, q, k, v, idx, n_sel, out, ws, as_stream(stream), true, k_loc, v_loc));
  return HS2_OK;
}

int hs2_workspace_region(const hs2_shape* shape, int32_t n_sparse_layers, int32_t region,
                         size_t* offset, size_t* bytes) {
  Plan p;
  const int st = make_plan(shape, n_sparse_layers, &p);
  if (st != HS2_OK) return st;
  if (!offset || !bytes) return HS2_ERR_INVALID_ARG;
  switch (region) {
    case HS2_WS_LSE2:
      *offset = p.off_lse2r;
      *bytes = static_cast<size_t>(p.R) * kG * sizeof(double);
      return HS2_OK;
    case HS2_WS_REFINE:
      *offset = p.off_ref_stat;
      *bytes = static_cast<size_t>(p.R) * sizeof(RefineStat);
      return HS2_OK;
    case HS2_WS_INDEX_CHECK:
      *offset = p.off_idx_bad;
      *bytes = static_cast<size_t>(p.R) * p.sp_nch * sizeof(uint32_t);
      return HS2_OK;
    default:
      return HS2_ERR_INVALID_ARG;
  }
}

const char* hs2_status_string(int status) {
  switch (status) {
    case HS2_OK: return "ok";
    case HS2_ERR_INVALID_ARG: return "invalid argument";
    case HS2_ERR_UNSUPPORTED: return "unsupported shape";
    case HS2_ERR_WORKSPACE: return "workspace too small";
    case HS2_ERR_HIP: return "HIP runtime error";
    case HS2_ERR_SCRATCH: return "shape needs more than the static scratch buffer";
    default: return "unknown status";
  }
}

int hs2_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
