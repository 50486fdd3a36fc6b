// gfx950 kernels of the activation-sparse ReLU FFN decode step.
//
// The step (PowerInfer paper explainer, section "活性化予測器" for the
// predictor, section "ニューロン活性化のべき乗則分布" for the FFN equation,
// section "GPU-CPUハイブリッドアーキテクチャ" for "compute only the predicted
// neurons"):
//
//   k_pred_hidden   h = ReLU(x P1^T)                               HBM-bound GEMV
//   k_rows_mask     v = rows . vec + bias; selected = OR_t v > thr;
//                   wave ballot -> 64-bit mask words; the last workgroup
//                   compacts the words into the ascending index list  HBM-bound GEMV
//   k_gather        for each selected neuron: a = ReLU(g) (.) u        row-gather GEMV
//   k_down          y = sum over selected i of a_i W_downT[i]: split over
//                   (column tile, neuron slice); fixed-order sum of the
//                   slices by the last workgroup of each tile; no atomics
//                   on values
//
// Every loop that reads weights issues 16-byte loads from 64 consecutive
// chunks of a row (1 KiB per wave instruction), several rows and chunks in
// flight per lane.  Reductions use one fixed order, so results are
// bit-reproducible run to run for a given launch shape.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace pik {

// ---------------------------------------------------------------------------
// Cross-workgroup hand-off: the last workgroup to arrive at a ticket sees
// every other workgroup's stores (release fence before the ticket, acquire
// fence after it).
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool arrive_last(unsigned* ticket, unsigned expected) {
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = atomicAdd(ticket, 1u);
    s_last = (prev == expected - 1u) ? 1 : 0;
  }
  __syncthreads();
  const bool last = s_last != 0;
  if (last) __threadfence();
  return last;
}

// Exclusive prefix sum over the workgroup; *total gets the sum of all values.
__device__ __forceinline__ int block_exclusive_scan(int v, int* total) {
  __shared__ int s_wave[16];
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int nwaves = blockDim.x / WAVE;
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

// Mask words -> ascending int32 indices + count, by one workgroup.  Each
// thread owns a contiguous run of words; a scan of the per-thread popcounts
// gives every thread its output offset, so the list comes out in order.
__device__ void block_compact(const unsigned long long* words, int n_words, int* idx, int* count) {
  const int T = blockDim.x, tid = threadIdx.x;
  const int wpt = (n_words + T - 1) / T;
  const int w0 = min(tid * wpt, n_words), w1 = min(w0 + wpt, n_words);
  int c = 0;
  for (int w = w0; w < w1; ++w) c += __popcll(__hip_atomic_load(words + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  int total;
  int pos = block_exclusive_scan(c, &total);
  for (int w = w0; w < w1; ++w) {
    unsigned long long m = __hip_atomic_load(words + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    while (m) {
      const int b = __ffsll((long long)m) - 1;
      idx[pos++] = w * 64 + b;
      m &= m - 1ull;
    }
  }
  if (tid == 0) *count = total;
}

__global__ void k_fill_u32(unsigned* p, int n, unsigned v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// ---------------------------------------------------------------------------
// a1: h[t][j] = max(sum_k x[t][k] P1[j][k], 0).  One wave per row of P1.
// ---------------------------------------------------------------------------
template <int PT, int AT, int NB, int U>
__global__ __launch_bounds__(256) void k_pred_hidden(const void* __restrict__ p1, const void* __restrict__ x,
                                                     int d, int r, int B, float* __restrict__ h) {
  using XT = typename VecT<AT>::T;
  constexpr int EPC = WFmt<PT>::EPC;
  const int lane = threadIdx.x & (WAVE - 1);
  const int row = blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE;
  if (row >= r) return;
  const int nch = d / EPC;
  const u32x4* wrow = reinterpret_cast<const u32x4*>(static_cast<const char*>(p1) + row_bytes(PT, (size_t)row * d));
  const XT* xb = static_cast<const XT*>(x);
  for (int t0 = 0; t0 < B; t0 += NB) {
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
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * WAVE + lane;
        if (c < nch) {
#pragma unroll
          for (int t = 0; t < NB; ++t)
            if (t0 + t < B) dot_chunk<PT, AT>(acc[t], w[u], xb + (size_t)(t0 + t) * d + (size_t)c * EPC, 1.f);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const float s = wave_sum(acc[t]);
      if (lane == 0 && t0 + t < B) h[(size_t)(t0 + t) * r + row] = fmaxf(s, 0.f);
    }
  }
}

// ---------------------------------------------------------------------------
// a2/a4 + a3: v[t][i] = rows[i] . vec[t] + bias[i]; selected_i = OR_t v[t][i] > thr.
// One workgroup (4 waves x 16 rows) per 64-row mask word; lane j of a wave
// holds the decision for its row j and a ballot packs them.  The last
// workgroup compacts all words into idx/count.
// ---------------------------------------------------------------------------
template <int WT, int VT, int NB, int RG, int U>
__global__ __launch_bounds__(256) void k_rows_mask(const void* __restrict__ rows, const f16* __restrict__ scales,
                                                   const void* __restrict__ vec, int K, int n,
                                                   const float* __restrict__ bias, float thr, int B,
                                                   float* __restrict__ vals_out,
                                                   unsigned long long* __restrict__ mask_words,
                                                   unsigned* __restrict__ ticket, int* __restrict__ idx_out,
                                                   int* __restrict__ count_out) {
  using V = typename VecT<VT>::T;
  constexpr int EPC = WFmt<WT>::EPC;
  constexpr int RPW = 16;  // rows per wave
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int row_base = blockIdx.x * 64 + wave * RPW;
  const int nch = K / EPC;
  const V* vb = static_cast<const V*>(vec);
  const char* rbase = static_cast<const char*>(rows);
  const size_t rbytes = row_bytes(WT, (size_t)K);
  bool dec = false;

#pragma unroll 1
  for (int rg = 0; rg < RPW; rg += RG) {
    const u32x4* wr[RG];
    const f16* sr[RG];
#pragma unroll
    for (int j = 0; j < RG; ++j) {
      const int row = min(row_base + rg + j, n - 1);
      wr[j] = reinterpret_cast<const u32x4*>(rbase + rbytes * row);
      sr[j] = (WT == DT_Q4) ? scales + (size_t)row * (K / 32) : nullptr;
    }
    bool any[RG];
#pragma unroll
    for (int j = 0; j < RG; ++j) any[j] = false;
    for (int t0 = 0; t0 < B; t0 += NB) {
      float acc[RG][NB];
#pragma unroll
      for (int j = 0; j < RG; ++j)
#pragma unroll
        for (int t = 0; t < NB; ++t) acc[j][t] = 0.f;
      for (int c0 = 0; c0 < nch; c0 += WAVE * U) {
        u32x4 w[RG][U];
        float sc[RG][U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + u * WAVE + lane;
#pragma unroll
          for (int j = 0; j < RG; ++j) {
            w[j][u] = c < nch ? ld_stream(wr[j] + c) : u32x4{0, 0, 0, 0};
            sc[j][u] = (WT == DT_Q4 && c < nch) ? (float)sr[j][c] : 1.f;
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + u * WAVE + lane;
          if (c < nch) {
#pragma unroll
            for (int t = 0; t < NB; ++t) {
              if (t0 + t < B) {
                const V* vp = vb + (size_t)(t0 + t) * K + (size_t)c * EPC;
#pragma unroll
                for (int j = 0; j < RG; ++j) dot_chunk<WT, VT>(acc[j][t], w[j][u], vp, sc[j][u]);
              }
            }
          }
        }
      }
#pragma unroll
      for (int j = 0; j < RG; ++j) {
        const int row = row_base + rg + j;
#pragma unroll
        for (int t = 0; t < NB; ++t) {
          const float s = wave_sum(acc[j][t]);
          if (row < n && t0 + t < B) {
            const float v = s + bias[row];
            if (vals_out != nullptr && lane == 0) vals_out[(size_t)(t0 + t) * n + row] = v;
            any[j] = any[j] || (v > thr);
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < RG; ++j)
      if (lane == rg + j) dec = any[j];
  }

  __shared__ unsigned long long s_sub[4];
  const unsigned long long bits = __ballot(dec) & 0xFFFFull;
  if (lane == 0) s_sub[wave] = bits;
  __syncthreads();
  if (threadIdx.x == 0)
    mask_words[blockIdx.x] = s_sub[0] | (s_sub[1] << 16) | (s_sub[2] << 32) | (s_sub[3] << 48);
  if (arrive_last(ticket, gridDim.x)) {
    block_compact(mask_words, gridDim.x, idx_out, count_out);
    if (threadIdx.x == 0) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------------------
// a5: row-gather GEMV over the selected neurons.  One wave per neuron,
// persistent grid-stride over ranks k < count (count read on the device).
//   GM_GATED        a = ReLU(W_gate[i].x + b_i) * (W_up[i].x)
//   GM_NONGATED     a = ReLU(W_up[i].x + b_i)
//   GM_EXACT_GATED  a = ReLU(g[i]) * (W_up[i].x)     (g from the dense pass)
// a is stored by rank: a[t][k].
// ---------------------------------------------------------------------------
template <int WT, int AT, int NB, int GM, int U>
__global__ __launch_bounds__(256) void k_gather(const void* __restrict__ w_gate, const void* __restrict__ w_up,
                                                const f16* __restrict__ s_gate, const f16* __restrict__ s_up,
                                                const float* __restrict__ bias, const float* __restrict__ g_ws,
                                                const void* __restrict__ x, int d, int n, int B,
                                                const int* __restrict__ idx, const int* __restrict__ count,
                                                int dense, float* __restrict__ a_ws, int* __restrict__ iota_out,
                                                int* __restrict__ count_out) {
  using XT = typename VecT<AT>::T;
  constexpr int EPC = WFmt<WT>::EPC;
  constexpr bool TWO = (GM == GM_GATED);
  const int lane = threadIdx.x & (WAVE - 1);
  const int gw = blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE;
  const int nw = gridDim.x * (blockDim.x / WAVE);
  // A caller-given list is bounded here: count is clamped to [0, n] and
  // entries outside [0, n) contribute nothing.
  const int cnt = dense ? n : min(max(*count, 0), n);
  const int nch = d / EPC;
  const size_t rbytes = row_bytes(WT, (size_t)d);
  const XT* xb = static_cast<const XT*>(x);
  if (dense && count_out != nullptr && gw == 0 && lane == 0) *count_out = n;

  for (int k = gw; k < cnt; k += nw) {
    const int i = dense ? k : idx[k];
    if (dense && iota_out != nullptr && lane == 0) iota_out[k] = k;
    if ((unsigned)i >= (unsigned)n) {
      if (lane == 0)
        for (int t = 0; t < B; ++t) a_ws[(size_t)t * n + k] = 0.f;
      continue;
    }
    const u32x4* ru = reinterpret_cast<const u32x4*>(static_cast<const char*>(w_up) + rbytes * i);
    const u32x4* rg = TWO ? reinterpret_cast<const u32x4*>(static_cast<const char*>(w_gate) + rbytes * i) : nullptr;
    const f16* su = (WT == DT_Q4) ? s_up + (size_t)i * (d / 32) : nullptr;
    const f16* sg = (WT == DT_Q4 && TWO) ? s_gate + (size_t)i * (d / 32) : nullptr;
    for (int t0 = 0; t0 < B; t0 += NB) {
      float au[NB], ag[NB];
#pragma unroll
      for (int t = 0; t < NB; ++t) au[t] = ag[t] = 0.f;
      for (int c0 = 0; c0 < nch; c0 += WAVE * U) {
        u32x4 wu[U], wg[U];
        float scu[U], scg[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + u * WAVE + lane;
          const bool ok = c < nch;
          wu[u] = ok ? ld_stream(ru + c) : u32x4{0, 0, 0, 0};
          scu[u] = (WT == DT_Q4 && ok) ? (float)su[c] : 1.f;
          if (TWO) {
            wg[u] = ok ? ld_stream(rg + c) : u32x4{0, 0, 0, 0};
            scg[u] = (WT == DT_Q4 && ok) ? (float)sg[c] : 1.f;
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + u * WAVE + lane;
          if (c < nch) {
#pragma unroll
            for (int t = 0; t < NB; ++t) {
              if (t0 + t < B) {
                const XT* xp = xb + (size_t)(t0 + t) * d + (size_t)c * EPC;
                dot_chunk<WT, AT>(au[t], wu[u], xp, scu[u]);
                if (TWO) dot_chunk<WT, AT>(ag[t], wg[u], xp, scg[u]);
              }
            }
          }
        }
      }
#pragma unroll
      for (int t = 0; t < NB; ++t) {
        const float su_ = wave_sum(au[t]);
        float a;
        if (GM == GM_GATED) {
          const float sg_ = wave_sum(ag[t]);
          a = fmaxf(sg_ + bias[i], 0.f) * su_;
        } else if (GM == GM_NONGATED) {
          a = fmaxf(su_ + bias[i], 0.f);
        } else {
          a = fmaxf(g_ws[(size_t)(t0 + t) * n + i], 0.f) * su_;
        }
        if (lane == 0 && t0 + t < B) a_ws[(size_t)(t0 + t) * n + k] = a;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// a6 + a7: y[t] = sum over ranks k < count of a[t][k] * W_downT[idx[k]].
// Workgroup (tile, s) owns output columns [tile*TW, (tile+1)*TW) and the ranks
// k = s*4 + wave (mod 4*S).  Waves fold into the workgroup's partial through
// LDS; the last of the S workgroups of a tile sums the S partials in order
// s = 0..S-1 and writes y.
//   ASRC_A      a[t][k] from the gather pass
//   ASRC_GRELU  a[t][k] = ReLU(g[t][idx[k]])      (non-gated exact mode: u = 1)
// ---------------------------------------------------------------------------
template <int WT> struct DownFmt;
template <> struct DownFmt<DT_F32> { static constexpr int EPL = 4; };
template <> struct DownFmt<DT_F16> { static constexpr int EPL = 8; };
template <> struct DownFmt<DT_Q4> { static constexpr int EPL = 16; };

template <int WT, int OT, int NB, int ASRC, int U>
__global__ __launch_bounds__(256) void k_down(const void* __restrict__ w_down_t, const f16* __restrict__ s_down,
                                              const float* __restrict__ a_ws, const float* __restrict__ g_ws,
                                              int d, int n, int B, const int* __restrict__ idx,
                                              const int* __restrict__ count, int dense, int S,
                                              float* __restrict__ partial, unsigned* __restrict__ tickets,
                                              void* __restrict__ y) {
  using YT = typename VecT<OT>::T;
  constexpr int EPL = DownFmt<WT>::EPL;
  constexpr int TW = WAVE * EPL;
  extern __shared__ float s_red[];  // [4][NB][TW]
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int tile = blockIdx.x, s = blockIdx.y;
  const int col0 = tile * TW + lane * EPL;
  const bool col_ok = col0 < d;
  const int cnt = dense ? n : min(max(*count, 0), n);
  const int stride = S * 4;
  const size_t rbytes = row_bytes(WT, (size_t)d);
  const char* wb = static_cast<const char*>(w_down_t);

  for (int t0 = 0; t0 < B; t0 += NB) {
    float acc[NB][EPL];
#pragma unroll
    for (int t = 0; t < NB; ++t)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[t][e] = 0.f;

    for (int k0 = s * 4 + wave; k0 < cnt; k0 += stride * U) {
      int ii[U];
      float av[U][NB];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = k0 + u * stride;
        int i = k < cnt ? (dense ? k : idx[k]) : -1;
        if ((unsigned)i >= (unsigned)n) i = -1;
        const bool ok = i >= 0;
        ii[u] = i;
#pragma unroll
        for (int t = 0; t < NB; ++t) {
          float a = 0.f;
          if (ok && t0 + t < B) {
            if (ASRC == ASRC_A) a = a_ws[(size_t)(t0 + t) * n + k];
            else a = fmaxf(g_ws[(size_t)(t0 + t) * n + ii[u]], 0.f);
          }
          av[u][t] = a;
        }
      }
      if (WT == DT_Q4) {
        u32x2 q[U];
        float sc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const bool ok = ii[u] >= 0 && col_ok;
          const char* rp = wb + rbytes * (ok ? ii[u] : 0);
          q[u] = ok ? ld_stream(reinterpret_cast<const u32x2*>(rp + col0 / 2)) : u32x2{0u, 0u};
          sc[u] = ok ? (float)s_down[(size_t)ii[u] * (d / 32) + col0 / 32] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float qf[16];
          const unsigned wds[2] = {q[u].x ^ 0x88888888u, q[u].y ^ 0x88888888u};
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const f16x2 qq = q4pair(wds[kk] >> (8 * p));
              qf[kk * 8 + 2 * p] = (float)qq.x;
              qf[kk * 8 + 2 * p + 1] = (float)qq.y;
            }
#pragma unroll
          for (int t = 0; t < NB; ++t) {
            const float as = av[u][t] * sc[u];
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[t][e] = fmaf(as, qf[e], acc[t][e]);
          }
        }
      } else {
        u32x4 w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const bool ok = ii[u] >= 0 && col_ok;
          const char* rp = wb + rbytes * (ok ? ii[u] : 0);
          w[u] = ok ? ld_stream(reinterpret_cast<const u32x4*>(rp + row_bytes(WT, (size_t)col0)))
                    : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float wf[EPL];
          if (WT == DT_F16) {
            const unsigned ws[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const f16x2 hh = as_h2(ws[p]);
              wf[2 * p] = (float)hh.x;
              wf[2 * p + 1] = (float)hh.y;
            }
          } else {
            const f32x4 v = __builtin_bit_cast(f32x4, w[u]);
            wf[0] = v.x; wf[1] = v.y; wf[2] = v.z; wf[3] = v.w;
          }
#pragma unroll
          for (int t = 0; t < NB; ++t)
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[t][e] = fmaf(av[u][t], wf[e], acc[t][e]);
        }
      }
    }

    // fold the 4 waves: wave w writes its columns, then each thread sums 4 values in order
#pragma unroll
    for (int t = 0; t < NB; ++t)
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_red[(wave * NB + t) * TW + lane * EPL + e] = acc[t][e];
    __syncthreads();
    for (int e = threadIdx.x; e < NB * TW; e += blockDim.x) {
      const int t = e / TW, j = e % TW;
      const int col = tile * TW + j;
      if (t0 + t < B && col < d) {
        const float v = ((s_red[(0 * NB + t) * TW + j] + s_red[(1 * NB + t) * TW + j]) +
                         s_red[(2 * NB + t) * TW + j]) + s_red[(3 * NB + t) * TW + j];
        partial[((size_t)s * B + t0 + t) * d + col] = v;
      }
    }
    __syncthreads();
  }

  if (arrive_last(tickets + tile, (unsigned)S)) {
    YT* yo = static_cast<YT*>(y);
    for (int e = threadIdx.x; e < B * TW; e += blockDim.x) {
      const int t = e / TW, j = e % TW;
      const int col = tile * TW + j;
      if (col >= d) continue;
      float sum = 0.f;
      for (int s2 = 0; s2 < S; ++s2)
        sum += __hip_atomic_load(partial + ((size_t)s2 * B + t) * d + col, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      yo[(size_t)t * d + col] = from_f32<YT>(sum);
    }
    if (threadIdx.x == 0) __hip_atomic_store(tickets + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers: runtime dtypes -> template instances.
// ---------------------------------------------------------------------------
namespace {
constexpr int kBlock = 256;

template <typename F>
hipError_t with_nb(int B, F&& f) {
  if (B == 1) return f(std::integral_constant<int, 1>{});
  return f(std::integral_constant<int, 4>{});
}
}  // namespace

int down_tile_width(int wt) {
  return WAVE * (wt == DT_F32 ? DownFmt<DT_F32>::EPL : (wt == DT_F16 ? DownFmt<DT_F16>::EPL : DownFmt<DT_Q4>::EPL));
}

hipError_t launch_fill_u32(unsigned* p, int n, unsigned v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_u32, dim3((n + kBlock - 1) / kBlock), dim3(kBlock), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_pred_hidden(int pt, int at, const void* p1, const void* x, int d, int r, int B, float* h,
                              hipStream_t s) {
  const dim3 grid((r + 3) / 4), block(kBlock);
  return with_nb(B, [&](auto nbc) -> hipError_t {
    constexpr int NB = decltype(nbc)::value;
    constexpr int U = 8;
    if (pt == DT_F16 && at == DT_F16)
      hipLaunchKernelGGL((k_pred_hidden<DT_F16, DT_F16, NB, U>), grid, block, 0, s, p1, x, d, r, B, h);
    else if (pt == DT_F16 && at == DT_F32)
      hipLaunchKernelGGL((k_pred_hidden<DT_F16, DT_F32, NB, U>), grid, block, 0, s, p1, x, d, r, B, h);
    else if (pt == DT_F32 && at == DT_F16)
      hipLaunchKernelGGL((k_pred_hidden<DT_F32, DT_F16, NB, U>), grid, block, 0, s, p1, x, d, r, B, h);
    else if (pt == DT_F32 && at == DT_F32)
      hipLaunchKernelGGL((k_pred_hidden<DT_F32, DT_F32, NB, U>), grid, block, 0, s, p1, x, d, r, B, h);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  });
}

hipError_t launch_rows_mask(int wt, int vt, const void* rows, const void* scales, const void* vec, int K, int n,
                            const float* bias, float thr, int B, float* vals_out,
                            unsigned long long* mask_words, unsigned* ticket, int* idx_out, int* count_out,
                            hipStream_t s) {
  const int n_words = (n + 63) / 64;
  const dim3 grid(n_words), block(kBlock);
  const f16* sc = static_cast<const f16*>(scales);
  return with_nb(B, [&](auto nbc) -> hipError_t {
    constexpr int NB = decltype(nbc)::value;
    constexpr int RG = 4, U = 4;
#define PIK_ROWS_MASK(W, V)                                                                                  \
  hipLaunchKernelGGL((k_rows_mask<W, V, NB, RG, U>), grid, block, 0, s, rows, sc, vec, K, n, bias, thr, B, \
                     vals_out, mask_words, ticket, idx_out, count_out)
    if (wt == DT_F16 && vt == DT_F16) PIK_ROWS_MASK(DT_F16, DT_F16);
    else if (wt == DT_F16 && vt == DT_F32) PIK_ROWS_MASK(DT_F16, DT_F32);
    else if (wt == DT_F32 && vt == DT_F32) PIK_ROWS_MASK(DT_F32, DT_F32);
    else if (wt == DT_F32 && vt == DT_F16) PIK_ROWS_MASK(DT_F32, DT_F16);
    else if (wt == DT_Q4 && vt == DT_F16) PIK_ROWS_MASK(DT_Q4, DT_F16);
    else if (wt == DT_Q4 && vt == DT_F32) PIK_ROWS_MASK(DT_Q4, DT_F32);
    else return hipErrorInvalidValue;
#undef PIK_ROWS_MASK
    return hipGetLastError();
  });
}

hipError_t launch_gather(int wt, int at, int gm, const void* w_gate, const void* w_up, const void* s_gate,
                         const void* s_up, const float* bias, const float* g_ws, const void* x, int d, int n,
                         int B, const int* idx, const int* count, int dense, float* a_ws, int* iota_out,
                         int* count_out, int grid_blocks, hipStream_t s) {
  const dim3 grid(grid_blocks), block(kBlock);
  const f16* sg = static_cast<const f16*>(s_gate);
  const f16* su = static_cast<const f16*>(s_up);
  return with_nb(B, [&](auto nbc) -> hipError_t {
    constexpr int NB = decltype(nbc)::value;
#define PIK_GATHER_GM(W, A, G, U)                                                                                \
  hipLaunchKernelGGL((k_gather<W, A, NB, G, U>), grid, block, 0, s, w_gate, w_up, sg, su, bias, g_ws, x, d, n, B, \
                     idx, count, dense, a_ws, iota_out, count_out)
#define PIK_GATHER(W, A, U)                                              \
  do {                                                                   \
    if (gm == GM_GATED) PIK_GATHER_GM(W, A, GM_GATED, U);                \
    else if (gm == GM_NONGATED) PIK_GATHER_GM(W, A, GM_NONGATED, U);     \
    else PIK_GATHER_GM(W, A, GM_EXACT_GATED, U);                         \
  } while (0)
    if (wt == DT_F16 && at == DT_F16) PIK_GATHER(DT_F16, DT_F16, 8);
    else if (wt == DT_F16 && at == DT_F32) PIK_GATHER(DT_F16, DT_F32, 8);
    else if (wt == DT_F32 && at == DT_F32) PIK_GATHER(DT_F32, DT_F32, 8);
    else if (wt == DT_F32 && at == DT_F16) PIK_GATHER(DT_F32, DT_F16, 8);
    else if (wt == DT_Q4 && at == DT_F16) PIK_GATHER(DT_Q4, DT_F16, 4);
    else if (wt == DT_Q4 && at == DT_F32) PIK_GATHER(DT_Q4, DT_F32, 4);
    else return hipErrorInvalidValue;
#undef PIK_GATHER
#undef PIK_GATHER_GM
    return hipGetLastError();
  });
}

hipError_t launch_down(int wt, int ot, int asrc, const void* w_down_t, const void* s_down, const float* a_ws,
                       const float* g_ws, int d, int n, int B, const int* idx, const int* count, int dense, int S,
                       float* partial, unsigned* tickets, void* y, hipStream_t s) {
  const int tw = down_tile_width(wt);
  const dim3 grid((d + tw - 1) / tw, S), block(kBlock);
  const f16* sd = static_cast<const f16*>(s_down);
  return with_nb(B, [&](auto nbc) -> hipError_t {
    constexpr int NB = decltype(nbc)::value;
    const size_t lds = sizeof(float) * 4 * NB * tw;
#define PIK_DOWN_A(W, O, A)                                                                                    \
  hipLaunchKernelGGL((k_down<W, O, NB, A, 4>), grid, block, lds, s, w_down_t, sd, a_ws, g_ws, d, n, B, idx, count, \
                     dense, S, partial, tickets, y)
#define PIK_DOWN(W, O)                                   \
  do {                                                   \
    if (asrc == ASRC_A) PIK_DOWN_A(W, O, ASRC_A);        \
    else PIK_DOWN_A(W, O, ASRC_GRELU);                   \
  } while (0)
    if (wt == DT_F16 && ot == DT_F16) PIK_DOWN(DT_F16, DT_F16);
    else if (wt == DT_F16 && ot == DT_F32) PIK_DOWN(DT_F16, DT_F32);
    else if (wt == DT_F32 && ot == DT_F32) PIK_DOWN(DT_F32, DT_F32);
    else if (wt == DT_F32 && ot == DT_F16) PIK_DOWN(DT_F32, DT_F16);
    else if (wt == DT_Q4 && ot == DT_F16) PIK_DOWN(DT_Q4, DT_F16);
    else if (wt == DT_Q4 && ot == DT_F32) PIK_DOWN(DT_Q4, DT_F32);
    else return hipErrorInvalidValue;
#undef PIK_DOWN
#undef PIK_DOWN_A
    return hipGetLastError();
  });
}

}  // namespace pik
