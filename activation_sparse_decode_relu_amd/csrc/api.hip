// C ABI of the activation-sparse ReLU FFN decode library: argument checks,
// workspace layout and the kernel sequence of each call.
//
// Sequences (PowerInfer paper explainer, section "GPU-CPUハイブリッドアーキテクチャ",
// inference flow: predict, then compute only the predicted neurons).  One token with fp16
// activations and predictor and fp16 or int4 rows (the split path):
//   predict            pred_hidden -> act(mask only) -> down(index list only)
//   forward PREDICTED  pred_hidden -> act(predictor mask) -> down
//   forward EXACT      act(dense pre-activation mask) -> down
//   forward DENSE      act(every neuron) -> down
//   forward_masked     act(caller's list) -> down
// Batches of 2..16 on the matrix-core path (group -> down -> finish) and every other case on
// the vector path (group -> finish) follow the same pattern, with the mask source first.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <new>
#include <string>

#include "kernels.h"
#include "pi_ffn.h"

#include <mutex>

// The workspace of pi_ffn_forward_static (see static_scratch below).
static __device__ __align__(256) char scratch[PI_FFN_STATIC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

pi_status fail(pi_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pi_status ok() {
  g_last_error.clear();
  return PI_OK;
}

constexpr size_t kAlign = 256;
constexpr int kMaxBatch = pik::kMaxBatchTokens;
constexpr int kMaxD = 1 << 20;
constexpr int kMaxN = 1 << 24;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Layout {
  size_t h, mask, idx, count, abuf, partial, tickets, total;
  int group, waves, n_groups, n_words, max_partials, slices;
};

// Neurons per group workgroup and waves per workgroup for a layer.  Small
// layers use 32-neuron groups of 4 waves so that every compute unit gets work;
// large layers use 128-neuron groups of 8 waves, which keeps the group
// partials (groups x d floats) small.
void group_shape(int n, int* group, int* waves) {
  const int g32 = (n + 31) / 32;
  if (g32 <= 512) {
    *group = 32;
    *waves = 4;
  } else {
    *group = 128;
    *waves = 8;
  }
}

Layout layout_for(const pi_ffn_desc& d) {
  Layout L{};
  const size_t B = (size_t)d.max_batch, n = (size_t)d.d_ffn, dm = (size_t)d.d_model;
  group_shape(d.d_ffn, &L.group, &L.waves);
  L.n_groups = (d.d_ffn + L.group - 1) / L.group;
  L.n_words = (d.d_ffn + 31) / 32;
  size_t off = 0;
  // The split path's ticket counters come first, at the same offset and size for every
  // descriptor: handles of different shapes that share a workspace then share the tickets too,
  // which every call leaves at zero, and no other region of another layout overlaps them.
  L.slices = pik::split_slices(d.w_dtype, d.d_model);
  L.tickets = off; off = align_up(off + sizeof(unsigned) * (size_t)pik::kMaxDnSlices * pik::kTicketStride);
  L.h = off;       off = align_up(off + sizeof(float) * B * (size_t)(d.rank > 0 ? d.rank : 1));
  L.mask = off;    off = align_up(off + sizeof(unsigned) * (size_t)L.n_words);
  L.idx = off;     off = align_up(off + sizeof(int) * n);
  L.count = off;   off = align_up(off + sizeof(int));
  // activations handed from the group (or act) kernel to the down kernel: a[neuron][16] fp32 on
  // the batched matrix-core path, a[neuron] on the one-token split path
  const size_t a_stride = d.max_batch > pik::kMaxTokens ? pik::kMaxBatchTokens : (d.max_batch > 1 ? pik::kMaxTokens : 1);
  L.abuf = off;    off = align_up(off + sizeof(float) * n * a_stride);
  // partials: one [B][d] block per group workgroup (vector path, at most 16 tokens), or per down
  // chunk on the batched path; [chunks][d] on the split path
  L.max_partials = L.n_groups;
  if (d.max_batch > 1) L.max_partials = std::max(L.max_partials, pik::batch_down_chunks(d.d_model));
  const size_t split_part = (size_t)pik::split_chunks(d.w_dtype, d.d_model) * dm;
  const size_t vec_part = (size_t)L.n_groups * std::min(B, (size_t)pik::kMaxTokens) * dm;
  const size_t batch_part = d.max_batch > 1 ? (size_t)pik::batch_down_chunks(d.d_model) * B * dm : 0;
  L.partial = off; off = align_up(off + sizeof(float) * std::max(std::max(vec_part, batch_part), split_part));
  L.total = off;
  return L;
}

pi_status check_desc(const pi_ffn_desc* d) {
  if (d == nullptr) return fail(PI_ERR_INVALID, "desc is NULL");
  if (d->d_model <= 0 || d->d_model % 64 != 0 || d->d_model > kMaxD)
    return fail(PI_ERR_INVALID, "d_model=%d must be a positive multiple of 64 up to %d", d->d_model, kMaxD);
  if (d->d_ffn <= 0 || d->d_ffn > kMaxN)
    return fail(PI_ERR_INVALID, "d_ffn=%d must lie in [1, %d]", d->d_ffn, kMaxN);
  if (d->rank < 0 || d->rank % 64 != 0 || d->rank > kMaxD)
    return fail(PI_ERR_INVALID, "rank=%d must be 0 or a positive multiple of 64", d->rank);
  if (d->gated != 0 && d->gated != 1) return fail(PI_ERR_INVALID, "gated=%d must be 0 or 1", d->gated);
  if (d->max_batch < 1 || d->max_batch > kMaxBatch)
    return fail(PI_ERR_INVALID, "max_batch=%d must lie in [1, %d]", d->max_batch, kMaxBatch);
  if (d->w_dtype != PI_F32 && d->w_dtype != PI_F16 && d->w_dtype != PI_Q4G32)
    return fail(PI_ERR_INVALID, "w_dtype=%d is not a pi_dtype", d->w_dtype);
  if (d->p_dtype != PI_F32 && d->p_dtype != PI_F16)
    return fail(PI_ERR_INVALID, "p_dtype=%d must be PI_F32 or PI_F16", d->p_dtype);
  if (d->act_dtype != PI_F32 && d->act_dtype != PI_F16)
    return fail(PI_ERR_INVALID, "act_dtype=%d must be PI_F32 or PI_F16", d->act_dtype);
  if (d->rank > 0 && !(d->tau > 0.0f && d->tau < 1.0f))
    return fail(PI_ERR_INVALID, "tau=%g must lie in (0, 1)", (double)d->tau);
  if (d->max_batch > pik::kMaxTokens &&
      !pik::batch_large_supported(d->w_dtype, d->act_dtype, d->max_batch, d->d_model))
    return fail(PI_ERR_UNSUPPORTED,
                "max_batch=%d: more than %d tokens run on the matrix cores only (fp16 weights and activations, "
                "d_model a multiple of 128)", d->max_batch, pik::kMaxTokens);
  int group, waves;
  group_shape(d->d_ffn, &group, &waves);
  if (pik::group_cpl(d->w_dtype, d->d_model, waves) == 0)
    return fail(PI_ERR_UNSUPPORTED, "d_model=%d is larger than the library's per-wave slice allows", d->d_model);
  return PI_OK;
}

pi_status check_weights(const pi_ffn_desc* d, const pi_ffn_weights* w) {
  if (w == nullptr) return fail(PI_ERR_INVALID, "weights is NULL");
  const bool q4 = d->w_dtype == PI_Q4G32;
  struct Req { const void* p; bool need; const char* name; };
  const Req reqs[] = {
      {w->w_gate, d->gated == 1, "w_gate"}, {w->w_up, true, "w_up"},       {w->w_down_t, true, "w_down_t"},
      {w->s_gate, q4 && d->gated == 1, "s_gate"}, {w->s_up, q4, "s_up"},    {w->s_down, q4, "s_down"},
      {w->b, true, "b"},                      {w->p1, d->rank > 0, "p1"},   {w->p2, d->rank > 0, "p2"},
      {w->b_p, d->rank > 0, "b_p"},
  };
  for (const Req& r : reqs) {
    if (r.need && r.p == nullptr) return fail(PI_ERR_INVALID, "%s is NULL but required by the descriptor", r.name);
    if (!r.need && r.p != nullptr) return fail(PI_ERR_INVALID, "%s must be NULL for this descriptor", r.name);
    if (r.p != nullptr && !aligned16(r.p)) return fail(PI_ERR_INVALID, "%s is not 16-byte aligned", r.name);
  }
  return PI_OK;
}

}  // namespace

struct pi_ffn {
  pi_ffn_desc desc;
  pi_ffn_weights w;
  char* ws;
  size_t ws_bytes;
  Layout L;
  float thr;
  const unsigned* hot_words;   // predicted mode: the always-computed neurons (pi_ffn_set_hot), or NULL
  void* prof_start[PI_PHASE_COUNT];
  void* prof_stop[PI_PHASE_COUNT];

  float* h() const { return reinterpret_cast<float*>(ws + L.h); }
  unsigned* mask() const { return reinterpret_cast<unsigned*>(ws + L.mask); }
  int* idx() const { return reinterpret_cast<int*>(ws + L.idx); }
  int* count() const { return reinterpret_cast<int*>(ws + L.count); }
  float* partial() const { return reinterpret_cast<float*>(ws + L.partial); }
  float* abuf() const { return reinterpret_cast<float*>(ws + L.abuf); }
  unsigned* tickets() const { return reinterpret_cast<unsigned*>(ws + L.tickets); }
};

namespace {

hipError_t record_event(void* ev, hipStream_t s) { return hipEventRecord(static_cast<hipEvent_t>(ev), s); }

// Launch one phase, bracketed by the armed profiling events if any.
template <typename F>
pi_status run_phase(pi_ffn* h, int phase, hipStream_t s, const char* what, F&& launch) {
  void* ev0 = h->prof_start[phase];
  void* ev1 = h->prof_stop[phase];
  if (ev0 != nullptr) {
    h->prof_start[phase] = h->prof_stop[phase] = nullptr;
    const hipError_t er = record_event(ev0, s);
    if (er != hipSuccess) return fail(PI_ERR_HIP, "event record before %s failed: %s", what, hipGetErrorString(er));
  }
  const hipError_t e = launch();
  if (e != hipSuccess) return fail(PI_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  if (ev1 != nullptr) {
    const hipError_t er = record_event(ev1, s);
    if (er != hipSuccess) return fail(PI_ERR_HIP, "event record after %s failed: %s", what, hipGetErrorString(er));
  }
  return PI_OK;
}

pi_status check_call(pi_ffn* h, const void* x, int32_t batch, const void* y, bool need_y) {
  if (h == nullptr) return fail(PI_ERR_INVALID, "handle is NULL");
  if (batch < 1 || batch > h->desc.max_batch)
    return fail(PI_ERR_INVALID, "batch=%d must lie in [1, max_batch=%d]", batch, h->desc.max_batch);
  if (x == nullptr || !aligned16(x)) return fail(PI_ERR_INVALID, "x is NULL or not 16-byte aligned");
  if (need_y && (y == nullptr || !aligned16(y))) return fail(PI_ERR_INVALID, "y is NULL or not 16-byte aligned");
  return PI_OK;
}

pi_status check_opt_ptr(const void* p, const char* name) {
  if (p != nullptr && !aligned16(p)) return fail(PI_ERR_INVALID, "%s is not 16-byte aligned", name);
  return PI_OK;
}

// Index lists and counts are read and written as single int32 values.
pi_status check_int_ptr(const void* p, const char* name) {
  if (p != nullptr && (reinterpret_cast<uintptr_t>(p) & 3u) != 0)
    return fail(PI_ERR_INVALID, "%s is not 4-byte aligned", name);
  return PI_OK;
}

pik::GroupArgs group_args(const pi_ffn* h, const void* x, int B) {
  const pi_ffn_desc& d = h->desc;
  pik::GroupArgs a{};
  a.w_gate = h->w.w_gate;
  a.w_up = h->w.w_up;
  a.w_down_t = h->w.w_down_t;
  a.s_gate = static_cast<const _Float16*>(h->w.s_gate);
  a.s_up = static_cast<const _Float16*>(h->w.s_up);
  a.s_down = static_cast<const _Float16*>(h->w.s_down);
  a.b = h->w.b;
  a.p2 = h->w.p2;
  a.b_p = h->w.b_p;
  a.h = h->h();
  a.x = x;
  a.mask_words = h->mask();
  a.partial = h->partial();
  a.thr = h->thr;
  a.p_dtype = d.p_dtype;
  a.d = d.d_model;
  a.n = d.d_ffn;
  a.r = d.rank;
  a.B = B;
  a.G = h->L.group;
  a.nw = h->L.waves;
  a.gated = d.gated;
  a.hot_words = h->hot_words;
  return a;
}

// Which kernels a call runs.
struct Plan {
  bool batched;   // matrix-core batch path: group + down + finish kernels
  bool split;     // one-token split path: act + down kernels, no finish
};

Plan plan_for(const pi_ffn* h, int mode, int B) {
  (void)mode;
  const pi_ffn_desc& d = h->desc;
  Plan p{};
  p.batched = pik::batch_supported(d.w_dtype, d.act_dtype, d.p_dtype, B, d.d_model, d.rank) ||
              pik::batch_large_supported(d.w_dtype, d.act_dtype, B, d.d_model);
  p.split = !p.batched && pik::split_supported(d.w_dtype, d.act_dtype, d.p_dtype, B, d.d_model, d.rank, d.d_ffn);
  return p;
}

pi_status hidden_phase(pi_ffn* h, const void* x, int B, hipStream_t s) {
  const pi_ffn_desc& d = h->desc;
  return run_phase(h, PI_PHASE_PRED_HIDDEN, s, "pred_hidden", [&] {
    return pik::launch_pred_hidden(d.p_dtype, d.act_dtype, h->w.p1, x, d.d_model, d.rank, B, h->h(), s);
  });
}

// Runs the group kernel (and, on the batched matrix-core path, the down kernel) for this
// call; *partials receives the number of partials of y written.
pi_status group_phase(pi_ffn* h, int mode, const Plan& plan, const pik::GroupArgs& a, hipStream_t s, int* partials) {
  const pi_ffn_desc& d = h->desc;
  if (plan.batched) {
    pi_status st = run_phase(h, PI_PHASE_GROUP, s, "ffn_bgroup",
                             [&] { return pik::launch_ffn_bgroup(mode, a, h->abuf(), s); });
    if (st != PI_OK || a.mask_only) return st;
    const int chunks = pik::batch_down_chunks(d.d_model);
    *partials = chunks;
    return run_phase(h, PI_PHASE_DOWN, s, "ffn_bdown",
                     [&] { return pik::launch_ffn_bdown(mode, a, h->abuf(), chunks, s); });
  }
  *partials = h->L.n_groups;
  return run_phase(h, PI_PHASE_GROUP, s, "ffn_group",
                   [&] { return pik::launch_ffn_group(d.w_dtype, d.act_dtype, mode, a, s); });
}

pi_status forward_impl(pi_ffn* h, const void* x, int32_t batch, int32_t mask_mode, void* y, int32_t* idx_out,
                       int32_t* count_out, void* stream);

// The one-token split path: act, then down (y, and the index list when idx / count are given).
pi_status split_phases(pi_ffn* h, int mode, const pik::GroupArgs& a, void* y, int* idx, int* count, hipStream_t s) {
  const pi_ffn_desc& d = h->desc;
  pi_status st = run_phase(h, PI_PHASE_GROUP, s, "act", [&] { return pik::launch_act(d.w_dtype, mode, a, h->abuf(), s); });
  if (st != PI_OK) return st;
  pik::DownArgs D{};
  D.abuf = h->abuf();
  D.w_down_t = h->w.w_down_t;
  D.s_down = static_cast<const _Float16*>(h->w.s_down);
  D.mask = h->mask();
  D.list = a.list;
  D.list_count = a.list_count;
  D.partial = h->partial();
  D.tickets = h->tickets();
  D.y = y;
  D.idx_out = idx;
  D.count_out = count;
  D.n = d.d_ffn;
  D.d = d.d_model;
  D.chunks = pik::split_chunks(d.w_dtype, d.d_model);
  D.do_down = a.mask_only ? 0 : 1;
  return run_phase(h, PI_PHASE_DOWN, s, "down", [&] { return pik::launch_down(d.w_dtype, mode, D, s); });
}

// reduce: sum the partials into y; list: 0 = none, 1 = compact the mask words, 2 = 0..n-1
pi_status finish_phase(pi_ffn* h, int B, int partials, void* y, bool reduce, int list, int* idx, int* count,
                       hipStream_t s) {
  const pi_ffn_desc& d = h->desc;
  return run_phase(h, PI_PHASE_FINISH, s, "finish", [&] {
    return pik::launch_finish(d.act_dtype, h->partial(), partials, B, d.d_model, y, list == 1 ? h->mask() : nullptr,
                              d.d_ffn, list == 2 ? d.d_ffn : 0, idx, count, reduce, list != 0, s);
  });
}

// The whole step of pi_ffn_forward, on a handle (a caller's, or the static scratch's).
pi_status forward_impl(pi_ffn* h, const void* x, int32_t batch, int32_t mask_mode, void* y, int32_t* idx_out,
                       int32_t* count_out, void* stream) {
  pi_status st = check_call(h, x, batch, y, true);
  if (st != PI_OK) return st;
  if ((st = check_int_ptr(idx_out, "idx_out")) != PI_OK || (st = check_int_ptr(count_out, "count_out")) != PI_OK)
    return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const pi_ffn_desc& d = h->desc;
  const bool want_list = idx_out != nullptr || count_out != nullptr;
  int* idx = idx_out != nullptr ? idx_out : h->idx();
  int* count = count_out != nullptr ? count_out : h->count();
  pik::GroupArgs a = group_args(h, x, batch);
  int mode, list;
  switch (mask_mode) {
    case PI_MASK_PREDICTED:
      if (d.rank == 0) return fail(PI_ERR_INVALID, "PREDICTED mode needs a predictor (rank > 0)");
      mode = pik::MODE_PRED;
      list = 1;
      break;
    case PI_MASK_EXACT_RELU:
      mode = pik::MODE_EXACT;
      a.thr = 0.0f;   // the ReLU support: g > 0, whatever the predictor's tau
      list = 1;
      break;
    case PI_MASK_DENSE:
      mode = pik::MODE_DENSE;
      list = 2;
      break;
    default:
      return fail(PI_ERR_INVALID, "mask_mode=%d is not a pi_mask_mode", mask_mode);
  }
  if (batch > pik::kMaxTokens && mode == pik::MODE_PRED) {
    // Past 16 tokens the union of the per-token masks covers most of the layer (about 53 % at
    // 16 tokens under a 10 % firing rate, 88 % at 64), so every gate row is read anyway: the
    // predictor is not run, and the exact ReLU support is computed from the dense pre-activations.
    mode = pik::MODE_EXACT;
    a.thr = 0.0f;
  }
  int partials = 0;
  const Plan plan = plan_for(h, mode, batch);
  if (mode == pik::MODE_PRED && (st = hidden_phase(h, x, batch, s)) != PI_OK) return st;
  if (plan.split) {
    if ((st = split_phases(h, mode, a, y, want_list ? idx : nullptr, want_list ? count : nullptr, s)) != PI_OK)
      return st;
    return ok();
  }
  if ((st = group_phase(h, mode, plan, a, s, &partials)) != PI_OK) return st;
  if ((st = finish_phase(h, batch, partials, y, true, want_list ? list : 0, idx, count, s)) != PI_OK) return st;
  return ok();
}

// ---- the static scratch of pi_ffn_forward_static ----------------------------------------------------
// One array per GPU, held until the process ends.  In host code `scratch` is only a host-side
// stand-in for the symbol: its device address on the current GPU comes from hipGetSymbolAddress,
// taken once per device and kept, and only that address is ever handed to a kernel.
constexpr size_t kStaticScratchBytes = PI_FFN_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices];

pi_status static_scratch(char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PI_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(PI_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(PI_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return PI_OK;
}

}  // namespace

extern "C" {

int32_t pi_ffn_abi_version(void) { return PI_FFN_ABI_VERSION; }

const char* pi_last_error(void) { return g_last_error.c_str(); }

pi_status pi_ffn_workspace_bytes(const pi_ffn_desc* desc, size_t* bytes) {
  pi_status st = check_desc(desc);
  if (st != PI_OK) return st;
  if (bytes == nullptr) return fail(PI_ERR_INVALID, "bytes is NULL");
  *bytes = layout_for(*desc).total;
  return ok();
}

pi_status pi_ffn_create(const pi_ffn_desc* desc, const pi_ffn_weights* weights, void* workspace,
                        size_t workspace_bytes, void* stream, pi_ffn** out) {
  if (out == nullptr) return fail(PI_ERR_INVALID, "out is NULL");
  *out = nullptr;
  pi_status st = check_desc(desc);
  if (st != PI_OK) return st;
  if ((st = check_weights(desc, weights)) != PI_OK) return st;
  const Layout L = layout_for(*desc);
  if (workspace == nullptr) return fail(PI_ERR_WORKSPACE, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0)
    return fail(PI_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(PI_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);

  pi_ffn* h = new (std::nothrow) pi_ffn{};
  if (h == nullptr) return fail(PI_ERR_INVALID, "out of host memory");
  h->desc = *desc;
  h->w = *weights;
  h->ws = static_cast<char*>(workspace);
  h->ws_bytes = workspace_bytes;
  h->L = L;
  h->thr = desc->rank > 0 ? (float)std::log((double)desc->tau / (1.0 - (double)desc->tau)) : 0.0f;
  // Clear the mask words once so a predict() before any forward() never reads garbage.
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = pik::launch_fill_u32(h->mask(), L.n_words, 0u, s);
  if (e == hipSuccess) e = pik::launch_fill_u32(h->tickets(), pik::kMaxDnSlices * pik::kTicketStride, 0u, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    delete h;
    return fail(PI_ERR_HIP, "workspace initialisation failed: %s", hipGetErrorString(e));
  }
  *out = h;
  return ok();
}

pi_status pi_ffn_destroy(pi_ffn* h) {
  if (h == nullptr) return fail(PI_ERR_INVALID, "handle is NULL");
  delete h;
  return ok();
}

pi_status pi_ffn_predict(pi_ffn* h, const void* x, int32_t batch, int32_t* idx, int32_t* count, float* logits_dbg,
                         void* stream) {
  pi_status st = check_call(h, x, batch, nullptr, false);
  if (st != PI_OK) return st;
  if (batch > pik::kMaxTokens)
    return fail(PI_ERR_UNSUPPORTED, "batch=%d: the predictor runs on at most %d tokens", batch, pik::kMaxTokens);
  if (h->desc.rank == 0) return fail(PI_ERR_INVALID, "predict needs a predictor (rank > 0)");
  if (idx == nullptr || count == nullptr) return fail(PI_ERR_INVALID, "idx and count are required");
  if ((st = check_int_ptr(idx, "idx")) != PI_OK || (st = check_int_ptr(count, "count")) != PI_OK ||
      (st = check_opt_ptr(logits_dbg, "logits_dbg")) != PI_OK)
    return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  pik::GroupArgs a = group_args(h, x, batch);
  a.logits = logits_dbg;
  a.mask_only = 1;
  int partials = 0;
  const Plan plan = plan_for(h, pik::MODE_PRED, batch);
  if ((st = hidden_phase(h, x, batch, s)) != PI_OK) return st;
  if (plan.split) {
    if ((st = split_phases(h, pik::MODE_PRED, a, nullptr, idx, count, s)) != PI_OK) return st;
    return ok();
  }
  if ((st = group_phase(h, pik::MODE_PRED, plan, a, s, &partials)) != PI_OK) return st;
  if ((st = finish_phase(h, batch, partials, nullptr, false, 1, idx, count, s)) != PI_OK) return st;
  return ok();
}

pi_status pi_ffn_forward(pi_ffn* h, const void* x, int32_t batch, int32_t mask_mode, void* y, int32_t* idx_out,
                         int32_t* count_out, void* stream) {
  return forward_impl(h, x, batch, mask_mode, y, idx_out, count_out, stream);
}

pi_status pi_ffn_forward_static(const pi_ffn_desc* desc, const pi_ffn_weights* weights, const void* x, int32_t batch,
                                int32_t mask_mode, void* y, int32_t* idx_out, int32_t* count_out, void* stream) {
  pi_status st = check_desc(desc);
  if (st != PI_OK) return st;
  if ((st = check_weights(desc, weights)) != PI_OK) return st;
  const Layout L = layout_for(*desc);
  if (L.total > kStaticScratchBytes)
    return fail(PI_ERR_WORKSPACE, "this descriptor needs %zu bytes of workspace; the static scratch holds %zu",
                L.total, kStaticScratchBytes);
  char* ws = nullptr;
  if ((st = static_scratch(&ws)) != PI_OK) return st;
  pi_ffn h{};   // on the stack: this call allocates nothing
  h.desc = *desc;
  h.w = *weights;
  h.ws = ws;
  h.ws_bytes = kStaticScratchBytes;
  h.L = L;
  h.thr = desc->rank > 0 ? (float)std::log((double)desc->tau / (1.0 - (double)desc->tau)) : 0.0f;
  if ((st = check_call(&h, x, batch, y, true)) != PI_OK) return st;
  // the split path's tickets must be zero; the scratch's last user may have laid it out differently
  const hipError_t e =
      pik::launch_fill_u32(h.tickets(), pik::kMaxDnSlices * pik::kTicketStride, 0u, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PI_ERR_HIP, "clearing the static scratch's tickets failed: %s", hipGetErrorString(e));
  return forward_impl(&h, x, batch, mask_mode, y, idx_out, count_out, stream);
}

pi_status pi_ffn_forward_masked(pi_ffn* h, const void* x, int32_t batch, const int32_t* idx, const int32_t* count,
                                void* y, void* stream) {
  pi_status st = check_call(h, x, batch, y, true);
  if (st != PI_OK) return st;
  if (batch > pik::kMaxTokens)
    return fail(PI_ERR_UNSUPPORTED, "batch=%d: a given list runs on at most %d tokens", batch, pik::kMaxTokens);
  if (idx == nullptr || count == nullptr) return fail(PI_ERR_INVALID, "idx and count are required");
  if ((st = check_int_ptr(idx, "idx")) != PI_OK || (st = check_int_ptr(count, "count")) != PI_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  pik::GroupArgs a = group_args(h, x, batch);
  a.list = idx;
  a.list_count = count;
  int partials = 0;
  const Plan plan = plan_for(h, pik::MODE_LIST, batch);
  if (plan.split) {
    if ((st = split_phases(h, pik::MODE_LIST, a, y, nullptr, nullptr, s)) != PI_OK) return st;
    return ok();
  }
  if ((st = group_phase(h, pik::MODE_LIST, plan, a, s, &partials)) != PI_OK) return st;
  if ((st = finish_phase(h, batch, partials, y, true, 0, nullptr, nullptr, s)) != PI_OK) return st;
  return ok();
}

pi_status pi_ffn_set_hot(pi_ffn* h, const uint32_t* hot_words) {
  if (h == nullptr) return fail(PI_ERR_INVALID, "handle is NULL");
  const pi_ffn_desc& d = h->desc;
  if (hot_words != nullptr) {
    if ((reinterpret_cast<uintptr_t>(hot_words) & 3u) != 0) return fail(PI_ERR_INVALID, "hot_words is not 4-byte aligned");
    if (d.rank == 0) return fail(PI_ERR_INVALID, "a hot set needs a predictor (rank > 0) for the other neurons");
    if (d.max_batch != 1 || !pik::split_supported(d.w_dtype, d.act_dtype, d.p_dtype, 1, d.d_model, d.rank, d.d_ffn))
      return fail(PI_ERR_UNSUPPORTED,
                  "a hot set runs on the one-token path only: max_batch 1, fp16 activations and predictor, "
                  "fp16 rows with d a multiple of 512 up to 8192 or int4 rows with d a multiple of 2048 up to 8192");
  }
  h->hot_words = hot_words;
  return ok();
}

pi_status pi_ffn_launch_plan(const pi_ffn* h, int32_t batch, int32_t mask_mode, uint32_t* plan) {
  if (h == nullptr || plan == nullptr) return fail(PI_ERR_INVALID, "handle or plan is NULL");
  if (batch < 1 || batch > h->desc.max_batch)
    return fail(PI_ERR_INVALID, "batch=%d must lie in [1, max_batch=%d]", batch, h->desc.max_batch);
  int mode;
  switch (mask_mode) {
    case PI_MASK_PREDICTED:
      if (h->desc.rank == 0) return fail(PI_ERR_INVALID, "PREDICTED mode needs a predictor (rank > 0)");
      mode = pik::MODE_PRED;
      break;
    case PI_MASK_EXACT_RELU: mode = pik::MODE_EXACT; break;
    case PI_MASK_DENSE: mode = pik::MODE_DENSE; break;
    default: return fail(PI_ERR_INVALID, "mask_mode=%d is not a pi_mask_mode", mask_mode);
  }
  if (batch > pik::kMaxTokens && mode == pik::MODE_PRED) mode = pik::MODE_EXACT;   // as pi_ffn_forward
  const Plan p = plan_for(h, mode, batch);
  uint32_t bits = 1u << PI_PHASE_GROUP;
  if (!p.split) bits |= 1u << PI_PHASE_FINISH;
  if (mode == pik::MODE_PRED) bits |= 1u << PI_PHASE_PRED_HIDDEN;
  if (p.batched || p.split) bits |= 1u << PI_PHASE_DOWN;
  *plan = bits;
  return ok();
}

pi_status pi_probe_read(const void* buf, size_t bytes, uint32_t* sums, int32_t n_sums, void* stream) {
  if (buf == nullptr || sums == nullptr) return fail(PI_ERR_INVALID, "buf and sums are required");
  if (!aligned16(buf) || bytes % 16 != 0) return fail(PI_ERR_INVALID, "buf must be 16-byte aligned and bytes a multiple of 16");
  if (n_sums < 1 || n_sums > 65536) return fail(PI_ERR_INVALID, "n_sums=%d must lie in [1, 65536]", n_sums);
  const hipError_t e = pik::launch_read_probe(buf, bytes / 16, sums, n_sums, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PI_ERR_HIP, "read probe launch failed: %s", hipGetErrorString(e));
  return ok();
}

pi_status pi_ffn_profile_next(pi_ffn* h, int32_t phase, void* start_event, void* stop_event) {
  if (h == nullptr) return fail(PI_ERR_INVALID, "handle is NULL");
  if (phase < 0 || phase >= PI_PHASE_COUNT) return fail(PI_ERR_INVALID, "phase=%d is not a pi_phase", phase);
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(PI_ERR_INVALID, "start_event and stop_event must both be set or both be NULL");
  h->prof_start[phase] = start_event;
  h->prof_stop[phase] = stop_event;
  return ok();
}

}  // extern "C"
