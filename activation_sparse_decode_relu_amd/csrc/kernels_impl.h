// gfx950 kernels of the activation-sparse ReLU FFN decode step: the predictor's hidden layer
// (every route), the vector route and the kernels it shares.  The one-token route's k_act and
// k_down are in kernels_split.h, the matrix-core batches in kernels_batch.h.
//
// The step (PowerInfer paper explainer, section "活性化予測器" for the
// predictor, section "ニューロン活性化のべき乗則分布" for the FFN equation,
// section "GPU-CPUハイブリッドアーキテクチャ" for "compute only the predicted
// neurons"), on the vector route three kernels per call:
//
//   k_pred_hidden  h = ReLU(x P1^T)                                   HBM-bound GEMV
//   k_ffn_group    one workgroup per group of G neurons:
//                    mask   predictor logits z = h P2^T + b_p (or the dense
//                           pre-activation in exact mode), threshold, wave
//                           ballot -> the group's 64-bit mask words;
//                    gather the selected neurons' gate/up/down rows: each of
//                           the 8 waves owns one d-slice, so every row is read
//                           by 8 waves in 1 KiB pieces and the down rows are
//                           prefetched with the gate/up rows;
//                    act    a = ReLU(g) (.) u from a fixed-order sum of the
//                           waves' partial dot products;
//                    down   the group's partial y over its own neurons, each
//                           wave writing only its d-slice (no cross-wave sum).
//   k_finish       y = sum of the group partials in a fixed order (no atomics),
//                  plus one extra workgroup that compacts the mask words into
//                  the ascending index list.
//
// No kernel communicates between workgroups inside a launch; every hand-off
// goes through a kernel boundary.  Reductions use one fixed order, so results
// are bit-reproducible run to run.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace pik {

// Exclusive prefix sum over a workgroup of NT threads; *total gets the sum of all values.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* total) {
  __shared__ int s_wave[NT / WAVE];
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int nwaves = NT / WAVE;
  int incl = v;
#pragma unroll
  for (int off = 1; off < WAVE; off <<= 1) {
    const int y = __shfl_up(incl, off, WAVE);
    if (lane >= off) incl += y;
  }
  if (lane == WAVE - 1) s_wave[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < nwaves; ++w) {
    const int s = s_wave[w];
    if (w < wave) before += s;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// Mask word w of a layer with n neurons, with the bits of neurons >= n cleared.  Kernels that
// write the mask a byte at a time leave the unused tail bytes of the last word untouched, and a
// workspace shared between layers may hold another layer's bits there.
__device__ __forceinline__ unsigned mask_word(const unsigned* words, int w, int n) {
  const unsigned v = words[w];
  const int rem = n - 32 * w;
  return rem >= 32 ? v : (v & ((1u << rem) - 1u));
}

// Mask words (bit b of word w = neuron 32w + b) of n neurons -> ascending int32 indices +
// count, by one workgroup.  Each thread owns a contiguous run of words; a scan
// of the per-thread popcounts gives every thread its output offset, so the
// list comes out in order.
template <int NT>
__device__ inline void block_compact(const unsigned* words, int n, int* idx, int* count) {
  const int T = NT, tid = threadIdx.x;
  const int n_words = (n + 31) / 32;
  const int wpt = (n_words + T - 1) / T;
  const int w0 = min(tid * wpt, n_words), w1 = min(w0 + wpt, n_words);
  int c = 0;
  for (int w = w0; w < w1; ++w) c += __popc(mask_word(words, w, n));
  int total;
  int pos = block_exclusive_scan<NT>(c, &total);
  for (int w = w0; w < w1; ++w) {
    unsigned m = mask_word(words, w, n);
    while (m) {
      const int b = __ffs((int)m) - 1;
      idx[pos++] = w * 32 + b;
      m &= m - 1u;
    }
  }
  if (tid == 0) *count = total;
}

__global__ inline void k_fill_u32(unsigned* p, int n, unsigned v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// ---------------------------------------------------------------------------
// a1: h[t][j] = max(sum_k x[t][k] P1[j][k], 0).  One wave per row of P1; each
// chunk of the row is loaded once and applied to every token of the batch
// (tokens in blocks of 4, NB = the most tokens).
// ---------------------------------------------------------------------------
// One wave computes row `row` of h (every token of the batch).
template <int PT, int AT, int NB, int U>
__device__ __forceinline__ void hidden_row(const void* __restrict__ p1, const void* __restrict__ x, int d, int r,
                                           int B, float* __restrict__ h, int row) {
  using XT = typename VecT<AT>::T;
  constexpr int EPC = WFmt<PT>::EPC;
  constexpr int TB = NB < 4 ? NB : 4;             // tokens per block
  const int lane = threadIdx.x & (WAVE - 1);
  if (row < r) {
    const int nch = d / EPC;
    const u32x4* wrow = reinterpret_cast<const u32x4*>(static_cast<const char*>(p1) + row_bytes(PT, (size_t)row * d));
    const XT* xb = static_cast<const XT*>(x);
    float acc[NB];
#pragma unroll
    for (int t = 0; t < NB; ++t) acc[t] = 0.f;
    for (int c0 = 0; c0 < nch; c0 += WAVE * U) {
      u32x4 w[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * WAVE + lane;
        w[u] = c < nch ? ld_stream(wrow + c) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int t0 = 0; t0 < NB; t0 += TB) {
        if (t0 >= B) break;
        XChunk<PT, AT> xv[U][TB];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + u * WAVE + lane;
#pragma unroll
          for (int t = 0; t < TB; ++t) {
            if (c < nch && t0 + t < B) xv[u][t].load(xb + (size_t)(t0 + t) * d + (size_t)c * EPC);
            else xv[u][t].zero();
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int t = 0; t < TB; ++t) dot_chunk<PT, AT>(acc[t0 + t], w[u], xv[u][t], 1.f);
      }
    }
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const float s = wave_sum(acc[t]);
      if (lane == 0 && t < B) h[(size_t)t * r + row] = fmaxf(s, 0.f);
    }
  }
}

template <int PT, int AT, int NB, int U>
__global__ __launch_bounds__(256) void k_pred_hidden(const void* __restrict__ p1, const void* __restrict__ x,
                                                     int d, int r, int B, float* __restrict__ h) {
  hidden_row<PT, AT, NB, U>(p1, x, d, r, B, h, blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE);
}

// ---------------------------------------------------------------------------
// Partial dot products of RB rows against NB token vectors, per lane
// (chunks c = lane, lane+64, ... of each row).  Rows with id < 0 are skipped.
// ---------------------------------------------------------------------------
template <int RT, int VT, int NB, int RB, int U>
__device__ __forceinline__ void rows_dot(float (&acc)[RB][NB], const char* __restrict__ rbase, size_t rbytes,
                                         const f16* __restrict__ scales, int K, const int (&rows)[RB],
                                         const typename VecT<VT>::T* __restrict__ vec, int t0, int B) {
  constexpr int EPC = WFmt<RT>::EPC;
  const int lane = threadIdx.x & (WAVE - 1);
  const int nch = K / EPC;
#pragma unroll
  for (int j = 0; j < RB; ++j)
#pragma unroll
    for (int t = 0; t < NB; ++t) acc[j][t] = 0.f;
  for (int c0 = 0; c0 < nch; c0 += WAVE * U) {
    u32x4 w[RB][U];
    float sc[RB][U];
    XChunk<RT, VT> xv[U][NB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * WAVE + lane;
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        const bool ok = c < nch && rows[j] >= 0;
        w[j][u] = ok ? ld_stream(reinterpret_cast<const u32x4*>(rbase + rbytes * rows[j]) + c) : u32x4{0, 0, 0, 0};
        sc[j][u] = (RT == DT_Q4 && ok) ? (float)scales[(size_t)rows[j] * (K / 32) + c] : 1.f;
      }
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        if (c < nch && t0 + t < B) xv[u][t].load(vec + (size_t)(t0 + t) * K + (size_t)c * EPC);
        else xv[u][t].zero();
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < NB; ++t)
#pragma unroll
        for (int j = 0; j < RB; ++j) dot_chunk<RT, VT>(acc[j][t], w[j][u], xv[u][t], sc[j][u]);
  }
}

// Elements of one 16-byte weight chunk, as floats (q4: the group scale applied by the caller).
template <int WT> struct Unpack;
template <> struct Unpack<DT_F16> {
  static constexpr int N = 8;
  __device__ static void run(u32x4 w, float (&o)[8]) {
    const unsigned ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const f16x2 hh = as_h2(ws[p]);
      o[2 * p] = (float)hh.x;
      o[2 * p + 1] = (float)hh.y;
    }
  }
};
template <> struct Unpack<DT_F32> {
  static constexpr int N = 4;
  __device__ static void run(u32x4 w, float (&o)[4]) {
    const f32x4 v = __builtin_bit_cast(f32x4, w);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  }
};
template <> struct Unpack<DT_Q4> {
  static constexpr int N = 32;
  __device__ static void run(u32x4 w, float (&o)[32]) {
    const unsigned ws[4] = {w.x ^ 0x88888888u, w.y ^ 0x88888888u, w.z ^ 0x88888888u, w.w ^ 0x88888888u};
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const f16x2 qq = q4pair(ws[k] >> (8 * p));
        o[8 * k + 2 * p] = (float)qq.x;
        o[8 * k + 2 * p + 1] = (float)qq.y;
      }
  }
};

// ---------------------------------------------------------------------------
// k_ffn_group: mask, gather, activation and the partial down projection of
// one group of neurons (see the file header).
// ---------------------------------------------------------------------------
constexpr int kNWMax = 8;      // waves per group workgroup (4 or 8)
constexpr int kGMax = 128;     // largest group

// Selected neurons per gather batch: the batch's gate/up/down pieces are all in flight at once.
template <int WT, int CPL, int NB = 1> struct Batch {
  static constexpr int kBase = ((WT == DT_Q4) ? 4 : 8) / CPL / (NB > 1 ? 2 : 1);
  static constexpr int JB = kBase > 0 ? kBase : 1;
};
constexpr int kJBMax = 8;

template <int WT, int AT, int NB, int MODE, int CPL, int NW>
__global__ __launch_bounds__(NW * WAVE) void k_ffn_group(const GroupArgs A) {
  using XT = typename VecT<AT>::T;
  constexpr int EPC = WFmt<WT>::EPC;
  constexpr int NE = Unpack<WT>::N;
  constexpr int kJB = Batch<WT, CPL>::JB;
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int G = A.G, B = A.B, d = A.d, n = A.n;
  const int grp = blockIdx.x;
  const int g0 = grp * G;
  const XT* xb = static_cast<const XT*>(A.x);

  __shared__ unsigned s_wb[kNWMax];  // each wave's decision bits
  __shared__ int s_list[kGMax];
  __shared__ int s_m;
  __shared__ float s_g[(MODE == MODE_EXACT) ? kGMax * kMaxTokens : 1];
  __shared__ float s_part[kJBMax][2][NB][NW];
  __shared__ float s_a[kJBMax][NB];

  // ---- which neurons of the group are computed ------------------------------------------------
  if (MODE == MODE_PRED || MODE == MODE_EXACT) {
    const int rpw = G / NW;   // rows per wave: 4, 8, 16 or 32, so no wave's rows straddle a mask word
    // Lane l holds the bias of the wave's row l (b_p, or b in exact mode); it is fetched ahead of
    // the row loads and read back with readlane, so no global round trip precedes the row stream.
    float row_bias = 0.f;
    {
      const int row = g0 + wave * rpw + lane;
      if (lane < rpw && row < n) row_bias = (MODE == MODE_PRED) ? A.b_p[row] : A.b[row];
    }
    constexpr int RB = (MODE == MODE_PRED) ? 8 : 4;
    bool dec = false;
#pragma unroll 1
    for (int rb = 0; rb < rpw; rb += RB) {
      int rows[RB];
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        const int row = g0 + wave * rpw + rb + j;
        rows[j] = (rb + j < rpw && row < n) ? row : -1;
      }
      bool any[RB];
#pragma unroll
      for (int j = 0; j < RB; ++j) any[j] = false;
      for (int t0 = 0; t0 < B; t0 += NB) {
        float acc[RB][NB];
        if (MODE == MODE_PRED) {
          if (A.p_dtype == DT_F16)
            rows_dot<DT_F16, DT_F32, NB, RB, 2>(acc, static_cast<const char*>(A.p2), row_bytes(DT_F16, A.r), nullptr,
                                                 A.r, rows, A.h, t0, B);
          else
            rows_dot<DT_F32, DT_F32, NB, RB, 2>(acc, static_cast<const char*>(A.p2), row_bytes(DT_F32, A.r), nullptr,
                                                 A.r, rows, A.h, t0, B);
        } else {
          const void* wpre = A.gated ? A.w_gate : A.w_up;
          const f16* spre = A.gated ? A.s_gate : A.s_up;
          rows_dot<WT, AT, NB, RB, 4>(acc, static_cast<const char*>(wpre), row_bytes(WT, d), spre, d, rows, xb, t0, B);
        }
#pragma unroll
        for (int j = 0; j < RB; ++j) {
          // rb + j < rpw + RB <= 40: a valid lane even for the padding rows, whose value is unused
          const float bias = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, row_bias), rb + j));
#pragma unroll
          for (int t = 0; t < NB; ++t) {
            const float v = wave_sum(acc[j][t]) + bias;
            if (rows[j] >= 0 && t0 + t < B) {
              if (MODE == MODE_PRED && A.logits != nullptr && lane == 0) A.logits[(size_t)(t0 + t) * n + rows[j]] = v;
              if (MODE == MODE_EXACT && lane == 0) s_g[(wave * rpw + rb + j) * kMaxTokens + t0 + t] = v;
              any[j] = any[j] || (v > A.thr);
            }
          }
        }
      }
#pragma unroll
      for (int j = 0; j < RB; ++j)
        if (lane == rb + j) dec = any[j];
    }
    // lane j of the wave holds row (wave * rpw + j)
    const unsigned long long bits = __ballot(dec) & ((1ull << rpw) - 1ull);
    if (lane == 0) s_wb[wave] = (unsigned)bits;
    __syncthreads();
    // word q of the group = the bits of waves q * (32 / rpw) ... (q + 1) * (32 / rpw) - 1
    const int wpw = 32 / rpw;
    auto group_word = [&](int q) {
      unsigned w = 0u;
      for (int k = 0; k < wpw; ++k) w |= s_wb[q * wpw + k] << (k * rpw);
      return w;
    };
    const int n_gw = G / 32;
    if ((int)threadIdx.x < n_gw && g0 / 32 + (int)threadIdx.x < (n + 31) / 32)
      A.mask_words[g0 / 32 + threadIdx.x] = group_word(threadIdx.x);
    if ((int)threadIdx.x < G) {
      const int q = threadIdx.x / 32, bit = threadIdx.x % 32;
      const unsigned word = group_word(q);
      int pos = __popc(word & ((1u << bit) - 1u));
      for (int qq = 0; qq < q; ++qq) pos += __popc(group_word(qq));
      if ((word >> bit) & 1u) s_list[pos] = threadIdx.x;
    }
    if (threadIdx.x == 0) {
      int m = 0;
      for (int q = 0; q < n_gw; ++q) m += __popc(group_word(q));
      s_m = m;
    }
  } else if (MODE == MODE_DENSE) {
    const int m = max(0, min(G, n - g0));
    if ((int)threadIdx.x < G) s_list[threadIdx.x] = threadIdx.x;
    if (threadIdx.x == 0) s_m = m;
  } else {  // MODE_LIST: an even slice of the caller's list per workgroup
    const int cnt = min(max(*A.list_count, 0), n);
    const int per = (cnt + (int)gridDim.x - 1) / (int)gridDim.x;   // <= G since gridDim.x = ceil(n / G)
    const int e0 = grp * per;
    const int m = max(0, min(per, cnt - e0));
    if ((int)threadIdx.x < m) {
      const int id = A.list[e0 + threadIdx.x];
      s_list[threadIdx.x] = ((unsigned)id < (unsigned)n) ? id : -1;
    }
    if (threadIdx.x == 0) s_m = m;
  }
  __syncthreads();
  if (A.mask_only) return;
  const int m = s_m;

  // ---- this wave's d-slice -------------------------------------------------------------------
  const int nch = d / EPC;
  const int cpw = (nch + NW - 1) / NW;
  const int c_begin = wave * cpw, c_end = min(nch, c_begin + cpw);
  const size_t rbytes = row_bytes(WT, d);
  const char* wgb = static_cast<const char*>(A.w_gate);
  const char* wub = static_cast<const char*>(A.w_up);
  const char* wdb = static_cast<const char*>(A.w_down_t);
  const bool need_gate = A.gated && MODE != MODE_EXACT;
  const bool need_up = !(MODE == MODE_EXACT && !A.gated);

  for (int t0 = 0; t0 < B; t0 += NB) {
    float acc[CPL][NB][NE];
#pragma unroll
    for (int q = 0; q < CPL; ++q)
#pragma unroll
      for (int t = 0; t < NB; ++t)
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[q][t][e] = 0.f;

    XChunk<WT, AT> xq[CPL][NB];
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      const int c = c_begin + lane + q * WAVE;
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        if (c < c_end && t0 + t < B) xq[q][t].load(xb + (size_t)(t0 + t) * d + (size_t)c * EPC);
        else xq[q][t].zero();
      }
    }

    for (int j0 = 0; j0 < m; j0 += kJB) {
      int nid[kJB];
#pragma unroll
      for (int jj = 0; jj < kJB; ++jj) {
        const int j = j0 + jj;
        int id = -1;
        if (j < m) id = (MODE == MODE_LIST) ? s_list[j] : g0 + s_list[j];
        nid[jj] = id;
      }
      // the activation threads fetch their neuron's bias along with the batch's rows
      float bj = 0.f;
      bool act_ok = false;
      if ((int)threadIdx.x < kJB * NB) {
        const int j = j0 + (int)threadIdx.x / NB;
        if (j < m) {
          const int id = (MODE == MODE_LIST) ? s_list[j] : g0 + s_list[j];
          act_ok = id >= 0;
          if (MODE != MODE_EXACT && act_ok) bj = A.b[id];
        }
      }
      // issue every load of the batch: gate, up and down pieces of this wave's slice
      u32x4 wg[kJB][CPL], wu[kJB][CPL], wd[kJB][CPL];
      float sg[kJB][CPL], su[kJB][CPL], sd[kJB][CPL];
#pragma unroll
      for (int jj = 0; jj < kJB; ++jj)
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
          const int c = c_begin + lane + q * WAVE;
          const bool ok = nid[jj] >= 0 && c < c_end;
          const size_t off = rbytes * (size_t)(ok ? nid[jj] : 0);
          const size_t soff = (size_t)(ok ? nid[jj] : 0) * (d / 32) + c;
          wg[jj][q] = (ok && need_gate) ? ld_stream(reinterpret_cast<const u32x4*>(wgb + off) + c) : u32x4{0, 0, 0, 0};
          wu[jj][q] = (ok && need_up) ? ld_stream(reinterpret_cast<const u32x4*>(wub + off) + c) : u32x4{0, 0, 0, 0};
          wd[jj][q] = ok ? ld_stream(reinterpret_cast<const u32x4*>(wdb + off) + c) : u32x4{0, 0, 0, 0};
          sg[jj][q] = (WT == DT_Q4 && ok && need_gate) ? (float)A.s_gate[soff] : 1.f;
          su[jj][q] = (WT == DT_Q4 && ok && need_up) ? (float)A.s_up[soff] : 1.f;
          sd[jj][q] = (WT == DT_Q4 && ok) ? (float)A.s_down[soff] : 1.f;
        }
      // partial dot products over the slice, folded across the wave
      if (need_gate || need_up) {
#pragma unroll
        for (int jj = 0; jj < kJB; ++jj) {
          float pg[NB], pu[NB];
#pragma unroll
          for (int t = 0; t < NB; ++t) pg[t] = pu[t] = 0.f;
#pragma unroll
          for (int q = 0; q < CPL; ++q) {
            const int c = c_begin + lane + q * WAVE;
            if (nid[jj] >= 0 && c < c_end) {
#pragma unroll
              for (int t = 0; t < NB; ++t) {
                if (need_gate) dot_chunk<WT, AT>(pg[t], wg[jj][q], xq[q][t], sg[jj][q]);
                if (need_up) dot_chunk<WT, AT>(pu[t], wu[jj][q], xq[q][t], su[jj][q]);
              }
            }
          }
          if (j0 + jj < m) {
#pragma unroll
            for (int t = 0; t < NB; ++t) {
              const float vg = need_gate ? wave_sum(pg[t]) : 0.f;
              const float vu = wave_sum(pu[t]);
              if (lane == 0) {
                s_part[jj][0][t][wave] = vg;
                s_part[jj][1][t][wave] = vu;
              }
            }
          }
        }
      }
      __syncthreads();
      if ((int)threadIdx.x < kJB * NB) {
        const int jj = threadIdx.x / NB, t = threadIdx.x % NB;
        float a = 0.f;
        if (act_ok && t0 + t < B) {
          float sg_ = 0.f, su_ = 0.f;
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            sg_ += s_part[jj][0][t][w];
            su_ += s_part[jj][1][t][w];
          }
          if (MODE == MODE_EXACT) {
            const float g = s_g[s_list[j0 + jj] * kMaxTokens + t0 + t];
            a = A.gated ? fmaxf(g, 0.f) * su_ : fmaxf(g, 0.f);
          } else {
            a = A.gated ? fmaxf(sg_ + bj, 0.f) * su_ : fmaxf(su_ + bj, 0.f);
          }
        }
        s_a[jj][t] = a;
      }
      __syncthreads();
      // down: acc[slice] += a_j * W_downT[j][slice]
#pragma unroll
      for (int jj = 0; jj < kJB; ++jj) {
        if (j0 + jj < m) {
#pragma unroll
          for (int q = 0; q < CPL; ++q) {
            float wf[NE];
            Unpack<WT>::run(wd[jj][q], wf);
#pragma unroll
            for (int t = 0; t < NB; ++t) {
              const float as = s_a[jj][t] * sd[jj][q];
#pragma unroll
              for (int e = 0; e < NE; ++e) acc[q][t][e] = fmaf(as, wf[e], acc[q][t][e]);
            }
          }
        }
      }
    }
    // the group's partial of y for this wave's slice (zeros if nothing was selected)
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      const int c = c_begin + lane + q * WAVE;
      if (c < c_end) {
#pragma unroll
        for (int t = 0; t < NB; ++t) {
          if (t0 + t < B) {
            float* dst = A.partial + ((size_t)grp * B + t0 + t) * d + (size_t)c * EPC;
#pragma unroll
            for (int e = 0; e < NE; e += 4)
              *reinterpret_cast<f32x4*>(dst + e) = f32x4{acc[q][t][e], acc[q][t][e + 1], acc[q][t][e + 2], acc[q][t][e + 3]};
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// k_finish: y[t][c] = sum over groups g (in order) of partial[g][t][c], one grid row per
// token; the extra last workgroup of row 0 writes the index list (compacted mask words, or
// 0..n-1).
// ---------------------------------------------------------------------------
template <int OT>
__global__ __launch_bounds__(256) void k_finish(const float* __restrict__ partial, int NG, int B, int d,
                                                void* __restrict__ y, const unsigned* __restrict__ mask_words,
                                                int mask_n, int iota_n, int* __restrict__ idx_out,
                                                int* __restrict__ count_out, int n_col_blocks) {
  using YT = typename VecT<OT>::T;
  if ((int)blockIdx.x == n_col_blocks) {
    if (blockIdx.y != 0) return;
    if (mask_words != nullptr) {
      block_compact<256>(mask_words, mask_n, idx_out, count_out);
    } else if (iota_n > 0) {
      for (int i = threadIdx.x; i < iota_n; i += blockDim.x) idx_out[i] = i;
      if (threadIdx.x == 0) *count_out = iota_n;
    }
    return;
  }
  // 256 threads = 8 column quads (32 columns: one 128-byte line of each partial row) x 32 slices
  // of the groups.  Slice k sums groups k, k + 32, k + 64, ... in that order; the 32 slice sums
  // are then added pairwise in a fixed tree, so the result is the same on every run.
  constexpr int kQ = 8, kS = 32, kU = 12;
  __shared__ f32x4 s_red[kS][kQ];
  const int cq = threadIdx.x % kQ, sl = threadIdx.x / kQ;
  const int col = blockIdx.x * (4 * kQ) + cq * 4;
  const int t = blockIdx.y;
  f32x4 sum = {0.f, 0.f, 0.f, 0.f};
  if (col < d) {
    for (int g0 = sl; g0 < NG; g0 += kS * kU) {
      f32x4 v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int g = g0 + kS * u;
        v[u] = g < NG ? *reinterpret_cast<const f32x4*>(partial + ((size_t)g * B + t) * d + col)
                      : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) sum += v[u];
    }
  }
  s_red[sl][cq] = sum;
  __syncthreads();
#pragma unroll
  for (int stride = kS / 2; stride > 0; stride /= 2) {
    if (sl < stride) s_red[sl][cq] += s_red[sl + stride][cq];
    __syncthreads();
  }
  if (sl == 0 && col < d) {
    const f32x4 tot = s_red[0][cq];
    YT* yo = static_cast<YT*>(y) + (size_t)t * d + col;
#pragma unroll
    for (int e = 0; e < 4; ++e) yo[e] = from_f32<YT>(tot[e]);
  }
}

// Batch size B -> token block NB (1, or 4 with a loop over token blocks).
template <typename F>
inline hipError_t with_nb(int B, F&& f) {
  if (B == 1) return f(std::integral_constant<int, 1>{});
  return f(std::integral_constant<int, 4>{});
}

// Per-weight-format launchers, each compiled in its own translation unit.
hipError_t launch_ffn_group_f16(int at, int mode, const GroupArgs& a, int cpl, hipStream_t s);
hipError_t launch_ffn_group_f32(int at, int mode, const GroupArgs& a, int cpl, hipStream_t s);
hipError_t launch_ffn_group_q4(int at, int mode, const GroupArgs& a, int cpl, hipStream_t s);

}  // namespace pik
