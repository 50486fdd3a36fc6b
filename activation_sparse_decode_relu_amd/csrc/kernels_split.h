// The one-token step as two balanced kernels (fp16 activations; fp16 or int4 group-32 weights;
// fp16 predictor), after k_pred_hidden in predicted mode:
//
//   k_act   every wave: NPW consecutive neurons (or NPW consecutive entries of a caller's
//           list).  Mask source -> decisions -> mask bits (the profile's hot neurons, if given,
//           are selected without reading their predictor rows); then, for each selected neuron
//           in order, its gate and up rows (full rows, 16-byte loads per lane), two wave sums,
//           and a = ReLU(g) * u written to a[neuron] in fp32.  Gated layers: each wave gathers
//           its own selected neurons, with no barrier, so the waves of a compute unit drift
//           apart and predictor rows and gathered rows stream together.  Non-gated layers (one
//           row per neuron): after one barrier the workgroup's selected neurons are dealt
//           round-robin to its waves, so no wave gathers several while the others idle.
//   k_down  y over (column slice s, chunk c) tiles.  With a mask, chunk c is the selected
//           neurons of mask words [c * W / C, (c + 1) * W / C), which the tile scans itself;
//           with a list (or dense), list positions [c * count / C, (c + 1) * count / C).  For
//           each neuron in ascending order, its contiguous piece of its W_down^T row (one
//           16-byte load per lane, int4 8 bytes) times a[neuron]; the tile's eight waves are
//           summed in wave order into its partial.  The last tile of a slice to finish (a
//           ticket counter per slice) sums the C partials in chunk order, rounds y once to the
//           act dtype and resets the ticket.  Tile (0, 0) also scans the whole mask and writes
//           the index list and count.
//
// Every floating-point sum has one fixed order (a neuron's dot products, the chunk's neurons in
// list order, the waves, the chunks), so results are the same on every run whichever tile
// arrives last.  The step is the FFN equation of the PowerInfer paper explainer (section
// "ニューロン活性化のべき乗則分布") over the neurons the predictor (section "活性化予測器")
// selects, computed only for those neurons (section "GPU-CPUハイブリッドアーキテクチャ", inference
// flow); down rows are stored transposed so each selected neuron's down weights are contiguous.
#pragma once

#include "kernels_impl.h"

namespace pik {

constexpr int kDnSeg = 1024;          // list entries of a chunk staged in LDS at a time
constexpr int kCoherent = 16;         // buffer cache policy sc1: coherent across compute units
constexpr int kStreaming = 2;         // buffer cache policy nt: streamed past the caches
constexpr int kOutOfRange = (int)0x80000000u;  // offset past any record (rows < 2^31 bytes): reads zero
constexpr int kRsrcFlags = 0x00020000;   // buffer resource word 3: raw 32-bit data, no swizzle

// ---------------------------------------------------------------------------------------------
// The gate and up sums of one neuron over the full row, by one wave: every 16-byte piece of both
// rows (and, int4, their group scales) is requested before any is used.  x comes from the
// wave's registers (xq) or, XLDS, from the workgroup's LDS copy.
// ---------------------------------------------------------------------------------------------
template <int WT, int CPL, bool XLDS>
__device__ __forceinline__ void gate_up_sums(const GroupArgs& A, int id, bool need_gate, bool need_up,
                                             const XChunk<WT, DT_F16> (&xq)[XLDS ? 1 : CPL],
                                             const u32x4* s_x, float& gs, float& us) {
  constexpr int EPC = WFmt<WT>::EPC;
  const int lane = threadIdx.x & (WAVE - 1);
  const size_t rbytes = row_bytes(WT, A.d);
  const int spr = A.d / 32;
  const char* wgb = static_cast<const char*>(A.w_gate);
  const char* wub = static_cast<const char*>(A.w_up);
  u32x4 wg[CPL], wu[CPL];
  f16 rsg[CPL], rsu[CPL];
#pragma unroll
  for (int q = 0; q < CPL; ++q) {
    const int c = lane + q * WAVE;
    wg[q] = need_gate ? ld_stream(reinterpret_cast<const u32x4*>(wgb + rbytes * id) + c) : u32x4{0, 0, 0, 0};
    wu[q] = need_up ? ld_stream(reinterpret_cast<const u32x4*>(wub + rbytes * id) + c) : u32x4{0, 0, 0, 0};
    if constexpr (WT == DT_Q4) {
      const size_t so = (size_t)id * spr + c;
      rsg[q] = need_gate ? A.s_gate[so] : (f16)0.f;
      rsu[q] = need_up ? A.s_up[so] : (f16)0.f;
    }
  }
  // fp16 rows wider than 4096: keep every load above ahead of every use below.  The scheduler
  // otherwise interleaves them, leaving about a third of the rows in flight per wave (Llama2-70B
  // shape: 31.7 us for the kernel interleaved, 28.3 us with all loads ahead); for shorter rows
  // (LLaMA-7B, int4 Falcon-40B) its interleaving is 2-3 % faster.
  if constexpr (WT == DT_F16 && CPL > 8) __builtin_amdgcn_sched_barrier(0);
  float pg = 0.f, pu = 0.f;
#pragma unroll
  for (int q = 0; q < CPL; ++q) {
    XChunk<WT, DT_F16> xl;
    if constexpr (XLDS) xl.load(reinterpret_cast<const f16*>(s_x) + (size_t)(lane + q * WAVE) * EPC);
    const XChunk<WT, DT_F16>& xc = XLDS ? xl : xq[XLDS ? 0 : q];
    if (need_gate) dot_chunk<WT, DT_F16>(pg, wg[q], xc, WT == DT_Q4 ? (float)rsg[q] : 1.f);
    if (need_up) dot_chunk<WT, DT_F16>(pu, wu[q], xc, WT == DT_Q4 ? (float)rsu[q] : 1.f);
  }
  gs = need_gate ? wave_sum(pg) : 0.f;
  us = need_up ? wave_sum(pu) : 0.f;
}

// ---------------------------------------------------------------------------------------------
// k_act
// ---------------------------------------------------------------------------------------------
// XLDS: the workgroup stages x in LDS once and the waves read their chunks from there at each
// selected neuron, instead of each wave holding x in registers (64 VGPRs at d = 8192).
// W: waves per workgroup.  GT: 1 gated, 0 non-gated, -1 read from A.gated.  DEAL: the
// workgroup's selected neurons are dealt to its waves after a barrier, instead of each wave
// gathering its own.
template <int WT, int CPL, int MODE, int NPW, bool XLDS, int W, int GT = -1, bool DEAL = false>
__global__ __launch_bounds__(W * WAVE) void k_act(const GroupArgs A, float* __restrict__ abuf) {
  constexpr int EPC = WFmt<WT>::EPC;
  static_assert(NPW == 8 || NPW == 16 || NPW == 32, "mask bits are written as whole bytes");
  static_assert(!DEAL || XLDS, "dealt gathers read x from the workgroup's LDS copy");
  const int lane = threadIdx.x & (WAVE - 1);
  const int wid = blockIdx.x * W + (int)(threadIdx.x / WAVE);
  const int n = A.n, d = A.d;
  const int base = wid * NPW;
  const f16* xb = static_cast<const f16*>(A.x);
  constexpr int kXU = XLDS ? CPL * WAVE * EPC / 8 : 1;   // x as 16-byte units
  __shared__ u32x4 s_x[kXU];
  if constexpr (XLDS) {
    for (int k = threadIdx.x; k < kXU; k += W * WAVE) s_x[k] = reinterpret_cast<const u32x4*>(xb)[k];
    __syncthreads();
  }
  int limit = n;   // neurons (or list entries) that exist
  if (MODE == MODE_LIST) limit = min(max(*A.list_count, 0), n);
  const bool live = base < limit;   // dealt: a wave past the end still meets the barrier below
  if (!DEAL && !live) return;
  const int m = live ? min(NPW, limit - base) : 0;

  // lane j < m holds entry j's neuron id, its FFN bias b and (predicted mode) its predictor bias b_p
  int my_id = -1;
  if (lane < m) {
    my_id = (MODE == MODE_LIST) ? A.list[base + lane] : base + lane;
    if ((unsigned)my_id >= (unsigned)n) my_id = -1;   // a list entry out of range does nothing
  }
  float my_b = 0.f, my_bp = 0.f;
  if (my_id >= 0) {
    my_b = A.b[my_id];
    if (MODE == MODE_PRED) my_bp = A.b_p[my_id];
  }
  auto id_of = [&](int j) { return __builtin_amdgcn_readlane(my_id, j); };
  auto lane_f = [&](float v, int j) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), j));
  };

  const size_t rbytes = row_bytes(WT, d);
  const bool gated = GT >= 0 ? GT == 1 : A.gated != 0;

  // ---- decisions ------------------------------------------------------------------------------
  unsigned sel = 0u;        // bit j: entry j is computed (wave-uniform)
  float gval[NPW];          // exact mode: entry j's pre-activation, including b
  if (MODE == MODE_PRED) {
    // the profile's hot neurons (if any) are selected whatever the predictor would say, and their
    // P2 rows are never read
    unsigned hot = 0u;
    if (A.hot_words != nullptr && live) {
      static_assert(NPW <= 32 && 32 % NPW == 0, "a wave's hot bits lie in one word");
      hot = (A.hot_words[base / 32] >> (base % 32)) & (m >= 32 ? 0xFFFFFFFFu : ((1u << m) - 1u));
    }
    int rows[NPW];
#pragma unroll
    for (int j = 0; j < NPW; ++j) rows[j] = (j < m && !((hot >> j) & 1u)) ? base + j : -1;
    float zacc[NPW][1];
    rows_dot<DT_F16, DT_F32, 1, NPW, 2>(zacc, static_cast<const char*>(A.p2), row_bytes(DT_F16, A.r), nullptr, A.r,
                                         rows, A.h, 0, 1);
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
      const float z = wave_sum(zacc[j][0]) + lane_f(my_bp, j);
      if (j < m) {
        const bool is_hot = (hot >> j) & 1u;
        if (A.logits != nullptr && lane == 0) A.logits[base + j] = is_hot ? __builtin_inff() : z;
        if (is_hot || z > A.thr) sel |= 1u << j;
      }
    }
  } else if (MODE == MODE_EXACT) {
    // the dense pre-activation of every neuron of the wave, two rows at a time
    const void* wpre = gated ? A.w_gate : A.w_up;
    const f16* spre = gated ? A.s_gate : A.s_up;
#pragma unroll
    for (int j0 = 0; j0 < NPW; j0 += 2) {
      int rows[2] = {(j0 < m) ? base + j0 : -1, (j0 + 1 < m) ? base + j0 + 1 : -1};
      float gacc[2][1];
      rows_dot<WT, DT_F16, 1, 2, (WT == DT_Q4 ? 2 : 4)>(gacc, static_cast<const char*>(wpre), rbytes, spre, d, rows,
                                                          xb, 0, 1);
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = j0 + jj;
        gval[j] = wave_sum(gacc[jj][0]) + lane_f(my_b, j);
        if (j < m && gval[j] > A.thr) sel |= 1u << j;
      }
    }
  } else {   // dense, list: every entry that names a neuron
    const unsigned long long ok = __ballot(my_id >= 0);
    sel = (unsigned)ok & (m == 32 ? 0xFFFFFFFFu : ((1u << m) - 1u));
  }

  if (MODE == MODE_PRED || MODE == MODE_EXACT) {
    // this wave's NPW mask bits: whole bytes at neuron base (bits of neurons >= n are 0)
    if (lane == 0 && live) {
      unsigned char* mb = reinterpret_cast<unsigned char*>(A.mask_words) + base / 8;
      if (NPW == 8) *mb = (unsigned char)sel;
      else if (NPW == 16) *reinterpret_cast<unsigned short*>(mb) = (unsigned short)sel;
      else *reinterpret_cast<unsigned*>(mb) = sel;
    }
  }
  const bool need_gate = gated && MODE != MODE_EXACT;
  const bool need_up = gated || MODE != MODE_EXACT;   // exact, non-gated: a = ReLU(g) from the mask pass
  XChunk<WT, DT_F16> xq[XLDS ? 1 : CPL];
  if constexpr (DEAL) {
    // the workgroup's selected entries, dealt round-robin to its waves in entry order
    static_assert(NPW * W <= 32, "one selection word per workgroup");
    __shared__ unsigned s_sel[W];
    __shared__ int s_id[W * NPW];
    __shared__ float s_v[W * NPW];   // bias b, or (exact) the pre-activation
    const int w = threadIdx.x / WAVE;
    if (lane == 0) s_sel[w] = A.mask_only ? 0u : sel;
    if (lane < NPW) {
      s_id[w * NPW + lane] = my_id;
      s_v[w * NPW + lane] = my_b;
    }
    if (MODE == MODE_EXACT && lane == 0) {
#pragma unroll
      for (int j = 0; j < NPW; ++j) s_v[w * NPW + j] = gval[j];
    }
    __syncthreads();
    unsigned all = 0u;
#pragma unroll
    for (int v = 0; v < W; ++v) all |= s_sel[v] << (NPW * v);
    const int total = __popc(all);
    for (int k = w; k < total; k += W) {
      unsigned rest = all;
      for (int q = 0; q < k; ++q) rest &= rest - 1u;   // drop the k lowest set entries
      const int e = __ffs((int)rest) - 1;
      const int id = s_id[e];
      float gs, us;
      gate_up_sums<WT, CPL, XLDS>(A, id, need_gate, need_up, xq, s_x, gs, us);
      float a;
      if (MODE == MODE_EXACT) {
        const float g = s_v[e];
        a = gated ? fmaxf(g, 0.f) * us : fmaxf(g, 0.f);
      } else {
        const float bj = s_v[e];
        a = gated ? fmaxf(gs + bj, 0.f) * us : fmaxf(us + bj, 0.f);
      }
      if (lane == 0) abuf[id] = a;
    }
    return;
  }
  if (A.mask_only || sel == 0u) return;

  // ---- activations of the selected neurons ------------------------------------------------------
  if (!XLDS && (need_gate || need_up)) {
#pragma unroll
    for (int q = 0; q < (XLDS ? 1 : CPL); ++q) xq[q].load(xb + (size_t)(lane + q * WAVE) * EPC);
  }
  unsigned todo = sel;
  while (todo != 0u) {
    const int j = __ffs((int)todo) - 1;
    todo &= todo - 1u;
    const int id = id_of(j);
    float gs, us;
    gate_up_sums<WT, CPL, XLDS>(A, id, need_gate, need_up, xq, s_x, gs, us);
    float a;
    if (MODE == MODE_EXACT) {
      float g = 0.f;
#pragma unroll
      for (int jj = 0; jj < NPW; ++jj)
        if (jj == j) g = gval[jj];
      a = gated ? fmaxf(g, 0.f) * us : fmaxf(g, 0.f);
    } else {
      const float bj = lane_f(my_b, j);
      a = gated ? fmaxf(gs + bj, 0.f) * us : fmaxf(us + bj, 0.f);
    }
    if (lane == 0) abuf[id] = a;
  }
}

// ---------------------------------------------------------------------------------------------
// k_down
// ---------------------------------------------------------------------------------------------
// What one lane loads of a row piece: fp16 16 bytes (8 columns), int4 8 bytes (16 columns, half a
// scale group), so a slice is 512 (fp16) or 1024 (int4) columns and a wave's load of one row
// piece is 1 KB or 512 B of contiguous row.
template <int WT> struct DnLane;
template <> struct DnLane<DT_F16> {
  static constexpr int EL = 8;
  typedef u32x4 V;
  __device__ static V load(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kStreaming));
  }
  __device__ static void unpack(V w, float (&o)[8]) { Unpack<DT_F16>::run(w, o); }
};
template <> struct DnLane<DT_Q4> {
  static constexpr int EL = 16;
  typedef u32x2 V;
  __device__ static V load(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kStreaming));
  }
  __device__ static void unpack(V w, float (&o)[16]) {
    const unsigned ws[2] = {w.x ^ 0x88888888u, w.y ^ 0x88888888u};
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const f16x2 qq = q4pair(ws[k] >> (8 * p));
        o[8 * k + 2 * p] = (float)qq.x;
        o[8 * k + 2 * p + 1] = (float)qq.y;
      }
  }
};

template <int WT> constexpr int dn_slice_cols() { return WAVE * DnLane<WT>::EL; }

// Device-coherent 16-byte store and load of fp32 partials (cache policy sc1): visible to every
// compute unit once the store completes, without the whole-L2 writeback and invalidate an
// agent-scope fence performs.
__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t r, int byte_off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, byte_off, 0, kCoherent);
}
__device__ __forceinline__ f32x4 load_coherent(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kCoherent));
}

// NT: threads per tile.  LOCAL (mask modes): chunk c is the neurons of mask words
// [c * words / C, (c + 1) * words / C) instead of positions [c * count / C, (c + 1) * count / C) of
// the global list, so a tile reads and scans only its own words.
template <int WT, int MODE, int U, int NT, bool LOCAL>
__global__ __launch_bounds__(NT) void k_down(const DownArgs D) {
  using LD = DnLane<WT>;
  using V = typename LD::V;
  constexpr int EL = LD::EL;                    // columns per lane
  constexpr int SW = dn_slice_cols<WT>();       // columns per slice
  constexpr int NWV = NT / WAVE;                // waves per tile
  constexpr bool kMask = MODE == MODE_PRED || MODE == MODE_EXACT;
  // the wave index through readfirstlane: known wave-uniform, so a wave's share of the list and
  // its batch loop live in scalar registers (divided from threadIdx, the loop ran under exec masks)
  const int lane = threadIdx.x & (WAVE - 1), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  const int n = D.n, d = D.d, C = D.chunks;
  const int slice = blockIdx.x, chunk = blockIdx.y;
  const int col = slice * SW + lane * EL;       // this lane's first column
  const bool col_ok = col < d;

  __shared__ int s_ids[kDnSeg];
  __shared__ float s_red[NWV][SW];
  __shared__ f32x4 s_half[SW / 4];
  __shared__ unsigned s_last;

  // ---- tile (0, 0): the whole index list and count ------------------------------------------------
  const int n_words = (n + 31) / 32;
  const bool lister = slice == 0 && chunk == 0 && (D.idx_out != nullptr || D.count_out != nullptr);
  int g_w0 = 0, g_w1 = 0, g_total = 0, g_pos = 0;   // the global scan: this thread's words and place
  if (kMask && (lister || !LOCAL)) {
    const int wpt = (n_words + NT - 1) / NT;
    g_w0 = min((int)threadIdx.x * wpt, n_words);
    g_w1 = min(g_w0 + wpt, n_words);
    int c = 0;
    for (int w = g_w0; w < g_w1; ++w) c += __popc(mask_word(D.mask, w, n));
    g_pos = block_exclusive_scan<NT>(c, &g_total);
  } else if (MODE == MODE_DENSE) {
    g_total = n;
  } else if (MODE == MODE_LIST) {
    g_total = min(max(*D.list_count, 0), n);
  }
  if (lister) {
    if (D.idx_out != nullptr && kMask) {
      int p = g_pos;
      for (int w = g_w0; w < g_w1; ++w) {
        unsigned mw = mask_word(D.mask, w, n);
        while (mw) {
          const int b = __ffs((int)mw) - 1;
          D.idx_out[p++] = 32 * w + b;
          mw &= mw - 1u;
        }
      }
    } else if (D.idx_out != nullptr && MODE == MODE_DENSE) {
      for (int i = threadIdx.x; i < n; i += NT) D.idx_out[i] = i;
    }
    if (D.count_out != nullptr && threadIdx.x == 0) *D.count_out = g_total;
  }
  if (!D.do_down) return;

  // ---- this tile's chunk: [lo, hi) of the list, each thread's words and place in it ----------------
  int w0 = g_w0, w1 = g_w1, my_pos = g_pos, lo, hi;
  if (kMask && LOCAL) {
    const int cw0 = (int)((long long)chunk * n_words / C), cw1 = (int)((long long)(chunk + 1) * n_words / C);
    const int wpt = (cw1 - cw0 + NT - 1) / NT;
    w0 = min(cw0 + (int)threadIdx.x * wpt, cw1);
    w1 = min(w0 + wpt, cw1);
    int c = 0;
    for (int w = w0; w < w1; ++w) c += __popc(mask_word(D.mask, w, n));
    int local;
    my_pos = block_exclusive_scan<NT>(c, &local);
    lo = 0;
    hi = local;
  } else {
    lo = (int)((long long)chunk * g_total / C);
    hi = (int)((long long)(chunk + 1) * g_total / C);
  }
  const int rbytes = (int)row_bytes(WT, d);
  const int cbytes = (int)row_bytes(WT, (size_t)(col_ok ? col : 0));
  const int col_oob = col_ok ? 0 : kOutOfRange;
  const int spr = d / 32;
  // every load of a batch goes through a buffer resource, the row's offset in a scalar register
  // (an entry is the same for the whole wave) and the lane's column offset in a vector one.  An
  // entry past the list (or a column past d) gets an out-of-range column offset and reads zero,
  // so a batch is straight-line code and the compiler can wait for one batch while the next is in
  // flight (split_supported keeps n rows under 2^31 bytes).
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(D.w_down_t), 0,
                                                                        n * rbytes, kRsrcFlags);
  const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(D.abuf), 0, n * 4,
                                                                        kRsrcFlags);
  const __amdgpu_buffer_rsrc_t srs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<f16*>(D.s_down), 0, WT == DT_Q4 ? n * spr * 2 : 0, kRsrcFlags);
  float acc[EL];
#pragma unroll
  for (int e = 0; e < EL; ++e) acc[e] = 0.f;

  for (int s0 = lo; s0 < hi; s0 += kDnSeg) {
    const int s1 = min(hi, s0 + kDnSeg);
    __syncthreads();   // the previous segment is no longer read
    if (MODE == MODE_PRED || MODE == MODE_EXACT) {
      int p = my_pos;
      for (int w = w0; w < w1 && p < s1; ++w) {
        unsigned mw = mask_word(D.mask, w, n);
        const int pc = __popc(mw);
        if (p + pc <= s0) {   // every bit of this word lies before the segment
          p += pc;
          continue;
        }
        while (mw && p < s1) {
          const int b = __ffs((int)mw) - 1;
          if (p >= s0) s_ids[p - s0] = 32 * w + b;
          ++p;
          mw &= mw - 1u;
        }
      }
    } else if (MODE == MODE_DENSE) {
      for (int k = threadIdx.x; k < s1 - s0; k += NT) s_ids[k] = s0 + k;
    } else {
      for (int k = threadIdx.x; k < s1 - s0; k += NT) {
        const int id = D.list[s0 + k];
        s_ids[k] = ((unsigned)id < (unsigned)n) ? id : -1;
      }
    }
    __syncthreads();
    // wave v takes entries v, v + NWV, v + 2 NWV, ... of the segment, U at a time, two batches in
    // flight: the next batch's row pieces are requested before the current batch is multiplied
    const int cnt = s1 - s0;
    const int mine = cnt > wave ? (cnt - wave + NWV - 1) / NWV : 0;   // this wave's entries
    // a batch: U row pieces with their activations (one address for the whole wave) and int4 scales
    struct Batch {
      V w[U];
      float a[U];
      f16 sc[U];
    };
    auto load = [&](int i0, Batch& bt) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u;
        const int id = __builtin_amdgcn_readfirstlane(s_ids[wave + NWV * min(i, mine - 1)]);
        // the top bit, set when the entry lies past this wave's share or names no neuron, is
        // or-ed into the column offsets (bit arithmetic, not a select: a select on this
        // wave-uniform condition becomes a branch around each load)
        const int oob = ((mine - 1 - i) | id) & kOutOfRange;
        const int sid = max(id, 0);
        bt.w[u] = LD::load(wrs, cbytes | oob | col_oob, sid * rbytes);
        bt.a[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ars, oob, sid * 4, 0));
        if constexpr (WT == DT_Q4)
          bt.sc[u] = __builtin_bit_cast(f16, __builtin_amdgcn_raw_buffer_load_b16(
                                                  srs, ((col_ok ? col : 0) / 32) * 2 | oob | col_oob, sid * spr * 2, 0));
      }
    };
    auto apply = [&](int i0, const Batch& bt) {
      // entries past the list read zero weights and activations: acc + 0 * 0 leaves acc as it is
      // (acc starts at +0 and a sum that is exactly zero rounds to +0, so acc is never -0)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float wf[EL];
        LD::unpack(bt.w[u], wf);
        const float as = WT == DT_Q4 ? bt.a[u] * (float)bt.sc[u] : bt.a[u];
#pragma unroll
        for (int e = 0; e < EL; ++e) acc[e] = fmaf(as, wf[e], acc[e]);
      }
    };
    if (mine > 0) {
      // the scheduling barriers keep each batch's loads where they are written: issued before
      // the other batch is applied, so the wait before an apply leaves the next batch in flight
      Batch ba, bb;
      load(0, ba);
      for (int i0 = 0; i0 < mine; i0 += 2 * U) {
        load(i0 + U, bb);
        __builtin_amdgcn_sched_barrier(0);
        apply(i0, ba);
        __builtin_amdgcn_sched_barrier(0);
        if (i0 + U >= mine) break;
        load(i0 + 2 * U, ba);
        __builtin_amdgcn_sched_barrier(0);
        apply(i0 + U, bb);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ---- the tile's partial: its waves summed in order ------------------------------------------------
#pragma unroll
  for (int e = 0; e < EL; e += 4)
    *reinterpret_cast<f32x4*>(&s_red[wave][lane * EL + e]) = f32x4{acc[e], acc[e + 1], acc[e + 2], acc[e + 3]};
  __syncthreads();
  const int ncol = min(SW, d - slice * SW);
  const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(D.partial, 0, 0x7fffffff, kRsrcFlags);
  for (int q = threadIdx.x; q < ncol / 4; q += NT) {
    f32x4 v = *reinterpret_cast<const f32x4*>(&s_red[0][4 * q]);
#pragma unroll
    for (int w = 1; w < NWV; ++w) v += *reinterpret_cast<const f32x4*>(&s_red[w][4 * q]);
    store_coherent(prs, 4 * (chunk * d + slice * SW + 4 * q), v);
  }

  // ---- the last tile of the slice sums the chunks' partials in a fixed order -------------------------
  // Every wave waits for its partial stores to complete before the barrier; only then does the tile
  // take its ticket, so the tile that draws the last ticket finds every partial in place.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  unsigned* ticket = D.tickets + (size_t)slice * kTicketStride;
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(C - 1)
                 ? 1u : 0u;
  __syncthreads();
  if (s_last == 0u) return;
  // thread t: column quad t % Q of the slice, chunk group t / Q (chunks [g * per, (g + 1) * per));
  // every load of a group is issued before any is added; groups are then added in group order
  constexpr int Q = SW / 4, H = NT / Q, kPer = (kMaxDnChunks + H - 1) / H;
  static_assert(H >= 1 && NT % Q == 0, "a slice's quads must divide the workgroup");
  const int quad = threadIdx.x % Q, grp = threadIdx.x / Q;
  const int per = (C + H - 1) / H, c0 = grp * per;
  const bool qok = 4 * quad < ncol;
  f32x4 t[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u)
    t[u] = (qok && u < per && c0 + u < C) ? load_coherent(prs, 4 * ((c0 + u) * d + slice * SW + 4 * quad))
                                          : f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 v = t[0];
#pragma unroll
  for (int u = 1; u < kPer; ++u)
    if (u < per && c0 + u < C) v += t[u];
  // groups 1 .. H-1 hand their sums to group 0, which adds them in group order
  for (int g = 1; g < H; ++g) {
    if (grp == g) s_half[quad] = v;
    __syncthreads();
    if (grp == 0 && g * per < C) v += s_half[quad];
    __syncthreads();
  }
  if (grp == 0 && qok) {
    f16* yo = static_cast<f16*>(D.y) + (size_t)slice * SW + 4 * quad;
#pragma unroll
    for (int e = 0; e < 4; ++e) yo[e] = (f16)v[e];
  }
  if (threadIdx.x == 0) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // next call
}

}  // namespace pik
