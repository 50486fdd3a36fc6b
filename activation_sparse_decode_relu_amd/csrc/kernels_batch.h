// Batched decode steps (2 to 64 tokens; fp16 weights, activations and predictor) on the
// CDNA4 matrix cores.
//
// With a batch, every gathered row serves B tokens, so the row-gather products become
// skinny GEMMs.  Tokens are padded to TT tiles of 16, the M dimension of the 16x16 MFMA
// tiles: TT = 1 up to 16 tokens (every mode), TT = 2 or 4 up to 32 or 64 tokens (the exact
// and dense modes: past 16 tokens the union of the per-token masks covers most of the layer,
// so every row is read and the predictor is not run).  A weight fragment, once loaded, is
// applied to every token tile.  Each of these products must, by construction, contract over
// the dimension that is contiguous in memory:
//
//   k_ffn_bgroup  one workgroup per group of 64 neurons, 4 waves, each wave taking a
//                 quarter of the contraction:
//                   mask  predicted: Z = H P2^T (fp32 MFMA: h stays fp32, the fp16
//                         predictor rows are widened exactly); exact: the dense
//                         pre-activation X W^T (fp16 MFMA, fp32 accumulation).  The union
//                         over the batch's tokens gives the group's mask words.
//                   act   gate and up products of the active neurons (fp16 MFMA, exact
//                         fp16 products, fp32 accumulation), a fixed-order sum of the four
//                         waves' partial tiles, a = ReLU(g + b) * u (or ReLU(u + b)),
//                         written to a[neuron][16 TT] in fp32.
//   k_ffn_bdown   y partials over (neuron chunk, 512-column slice): the contraction runs
//                 over neurons, which are strided in W_down^T, so it uses the fp32 MFMA
//                 whose lanes each supply a single element: lane l takes neuron (l / 16) of
//                 a 4-neuron step and 8 consecutive columns of that neuron's row, one
//                 column per output tile.  a stays fp32; the fp16 weights widen exactly.
//                 Past 16 tokens that fp32 MFMA would bound the kernel (2 B n d flops), so
//                 there each 32-neuron step runs on the fp16 MFMA instead: every a is split
//                 into two fp16 parts, hi = fp16(a) and lo = fp16(a - hi), whose exact
//                 products with the fp16 weights carry about 22 of a's 24 bits.  A step
//                 holding an |a| of 2^15 or more (which fp16 cannot split) keeps the fp32
//                 MFMA, so nothing overflows.
//
// The pages describe the single-token step (PowerInfer paper explainer, section
// "ニューロン活性化のべき乗則分布" for the FFN and "活性化予測器" for the predictor); the
// batch union is the reading that a row loaded once serves every token that fires it.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace pik {

typedef f16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kBG = 64;         // neurons per batched group workgroup
constexpr int kBNW = 4;         // waves per batched group workgroup
constexpr int kBT = kBG / 16;   // 16-neuron tiles per group
constexpr int kDW = 4;          // waves per down workgroup
constexpr int kDCols = 128;     // output columns per down wave: 8 MFMA tiles of 16
constexpr int kDSeg = 2048;     // neurons a down workgroup compacts into LDS at a time

// D[16][16] += A[16][4] B[4][16] (fp32): lane l gives A[l%16][l/16] and B[l/16][l%16] and
// holds D[4(l/16)+v][l%16] in element v.
__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// D[16][16] += A[16][32] B[32][16] (fp16 in, fp32 accumulate): lane l gives A[l%16][8(l/16)+e]
// and B[8(l/16)+e][l%16] for e = 0..7; D as above.
__device__ __forceinline__ f32x4 mma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                0);
}
__device__ __forceinline__ float half_at(u32x4 w, int e) { return (float)__builtin_bit_cast(f16x8, w)[e]; }
// a step's activations from this magnitude on stay on the fp32 MFMA (fp16 tops out at 65504)
constexpr float kSplitLimit = 32768.f;

// Partial tiles over this wave's share [k_begin, k_end) of a contraction of length K:
// acc[m][t] += X[tok][k] * W_m[row[t]][k] for the nt tiles in use; rows < 0, tokens >= B and
// k >= k_end contribute zeros.  Each batch of loads covers BS consecutive MFMA k-steps of every
// row in use, so a row is requested 64 * BS contiguous bytes at a time rather than 64: operand
// tiles read in longer row runs stream markedly faster.
constexpr int kBS = 4;   // MFMA k-steps (of 32) per load batch
// k-steps per load batch with TT token tiles: fewer with four tiles, whose accumulators take
// 128 registers
constexpr int bs_for(int TT) { return TT >= 4 ? 2 : kBS; }

template <int NM, int BS, int TT>
__device__ __forceinline__ void tiles_mma_f16(f32x4 (&acc)[NM][kBT][TT], const f16* const (&w)[NM],
                                              const int (&row)[kBT], int nt, const f16* __restrict__ x, int B, int K,
                                              int k_begin, int k_end) {
  const int lane = threadIdx.x & (WAVE - 1), li = lane & 15, lk = lane >> 4;
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int t = 0; t < kBT; ++t)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) acc[m][t][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = k_begin; k0 < k_end; k0 += 32 * BS) {
    // step st: lane (li, lk) reads 16 bytes of row li at element k0 + 32 * st + 8 * lk, so the
    // batch covers 64 * BS contiguous bytes of each row; X (token 16 tt + li) in the same order
    u32x4 xa[BS][TT], wv[BS][NM][kBT];
#pragma unroll
    for (int st = 0; st < BS; ++st) {
      const int kk = k0 + 32 * st + 8 * lk;
      const bool ok = k0 + 32 * st < k_end;
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const int tok = 16 * tt + li;
        xa[st][tt] = (tok < B && ok) ? *reinterpret_cast<const u32x4*>(x + (size_t)tok * K + kk) : u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int t = 0; t < kBT; ++t)
#pragma unroll
        for (int st = 0; st < BS; ++st) {
          const int kk = k0 + 32 * st + 8 * lk;
          const bool ok = k0 + 32 * st < k_end;
          wv[st][m][t] = (ok && t < nt && row[t] >= 0)
                             ? ld_cached(reinterpret_cast<const u32x4*>(w[m] + (size_t)row[t] * K + kk))
                             : u32x4{0, 0, 0, 0};
        }
#pragma unroll
    for (int st = 0; st < BS; ++st)
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int t = 0; t < kBT; ++t)
          if (t < nt)
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) acc[m][t][tt] = mma_f16(xa[st][tt], wv[st][m][t], acc[m][t][tt]);
  }
}

// Fixed-order sum over the waves of tile t's lane l partials, after each wave stored its own.
__device__ __forceinline__ f32x4 wave_tiles_sum(const f32x4 (*red)[2][kBT][WAVE], int m, int t, int l) {
  f32x4 s = red[0][m][t][l];
#pragma unroll
  for (int w = 1; w < kBNW; ++w) s += red[w][m][t][l];
  return s;
}

// The fixed-order sum over the waves of slot m of every token tile's accumulators: tile tt of
// this thread's 16-neuron tile (its wave) lands in out[tt].  acc holds this wave's partials of
// the kBT neuron tiles.
template <int TT>
__device__ __forceinline__ void waves_sum_tiles(f32x4 (*red)[2][kBT][WAVE], const f32x4 (&acc)[kBT][TT], int m,
                                                f32x4 (&out)[TT]) {
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
    for (int q = 0; q < kBT; ++q) red[wave][m][q][lane] = acc[q][tt];
    __syncthreads();
    out[tt] = wave_tiles_sum(red, m, wave, lane);
    __syncthreads();   // the slots are rewritten for the next token tile
  }
}

// TT: token tiles of 16 (B <= 16 TT); above one tile, only the exact and dense modes.
template <int MODE, int TT>
__global__ __launch_bounds__(kBNW * WAVE) void k_ffn_bgroup(const GroupArgs A, float* __restrict__ abuf) {
  static_assert(TT == 1 || MODE == MODE_EXACT || MODE == MODE_DENSE, "more than 16 tokens: exact or dense only");
  constexpr int TS = 16 * TT;          // a[neuron][TS]: the activation stride
  constexpr int BS = bs_for(TT);
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE, li = lane & 15, lk = lane >> 4;
  const int B = A.B, d = A.d, n = A.n;
  const int g0 = blockIdx.x * kBG;
  const f16* xb = static_cast<const f16*>(A.x);

  __shared__ f32x4 s_red[kBNW][2][kBT][WAVE];   // each wave's partial tiles
  __shared__ float s_pre[(MODE == MODE_EXACT) ? kBG * TS : 1];
  __shared__ unsigned s_tbits[kBT];
  __shared__ int s_list[kBG];
  __shared__ int s_m;

  // ---- which neurons of the group are computed ------------------------------------------------
  if (MODE == MODE_PRED || MODE == MODE_EXACT) {
    // this thread's tile (= its wave) and neuron, after the cross-wave sum
    const int t = wave, nrn = g0 + 16 * t + li;
    f32x4 z[TT];
    float bias = 0.f;
    if (MODE == MODE_PRED) {
      if (nrn < n) bias = A.b_p[nrn];
      const int r = A.r, kw = r / kBNW, kb = wave * kw;
      const f16* p2 = static_cast<const f16*>(A.p2);
      const float* hr = A.h + (size_t)li * r;
      f32x4 acc[kBT];
#pragma unroll
      for (int q = 0; q < kBT; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int k0 = kb; k0 < kb + kw; k0 += 32 * kBS) {
        u32x4 pw[kBS][kBT];
        f32x4 hv[kBS][2];
#pragma unroll
        for (int st = 0; st < kBS; ++st) {
          const int kk = k0 + 32 * st + 8 * lk;
          const bool ok = k0 + 32 * st < kb + kw;
#pragma unroll
          for (int q = 0; q < 2; ++q)
            hv[st][q] = (ok && li < B) ? *reinterpret_cast<const f32x4*>(hr + kk + 4 * q) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int q = 0; q < kBT; ++q) {
          const int row = g0 + 16 * q + li;
#pragma unroll
          for (int st = 0; st < kBS; ++st) {
            const int kk = k0 + 32 * st + 8 * lk;
            const bool ok = k0 + 32 * st < kb + kw;
            pw[st][q] = (ok && row < n) ? ld_cached(reinterpret_cast<const u32x4*>(p2 + (size_t)row * r + kk))
                                        : u32x4{0, 0, 0, 0};
          }
        }
#pragma unroll
        for (int st = 0; st < kBS; ++st)
#pragma unroll
          for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int q = 0; q < kBT; ++q) acc[q] = mma_f32(hv[st][e / 4][e % 4], half_at(pw[st][q], e), acc[q]);
      }
#pragma unroll
      for (int q = 0; q < kBT; ++q) s_red[wave][0][q][lane] = acc[q];
      __syncthreads();
      z[0] = wave_tiles_sum(s_red, 0, t, lane);
    } else {
      if (nrn < n) bias = A.b[nrn];
      int row[kBT];
#pragma unroll
      for (int q = 0; q < kBT; ++q) row[q] = (g0 + 16 * q + li < n) ? g0 + 16 * q + li : -1;
      const f16* const w[1] = {static_cast<const f16*>(A.gated ? A.w_gate : A.w_up)};
      f32x4 acc[1][kBT][TT];
      const int kw = d / kBNW;
      tiles_mma_f16<1, BS, TT>(acc, w, row, kBT, xb, B, d, wave * kw, (wave + 1) * kw);
      waves_sum_tiles<TT>(s_red, acc[0], 0, z);
    }
    bool dec = false;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tok = 16 * tt + 4 * lk + v;
        const float val = z[tt][v] + bias;
        if (MODE == MODE_EXACT) s_pre[(16 * t + li) * TS + tok] = val;
        if (nrn < n && tok < B) {
          if (MODE == MODE_PRED && A.logits != nullptr) A.logits[(size_t)tok * n + nrn] = val;
          dec = dec || (val > A.thr);
        }
      }
    // neuron li of tile t fires if any of its four lanes (token quarters) saw it fire
    const unsigned long long b = __ballot(dec);
    if (lane == 0) s_tbits[t] = (unsigned)((b | (b >> 16) | (b >> 32) | (b >> 48)) & 0xFFFFull);
    __syncthreads();
    const unsigned long long gmask = (unsigned long long)s_tbits[0] | ((unsigned long long)s_tbits[1] << 16) |
                                     ((unsigned long long)s_tbits[2] << 32) | ((unsigned long long)s_tbits[3] << 48);
    const int n_words = (n + 31) / 32;
    if ((int)threadIdx.x < kBG / 32 && g0 / 32 + (int)threadIdx.x < n_words)
      A.mask_words[g0 / 32 + threadIdx.x] = (unsigned)(gmask >> (32 * threadIdx.x));
    if ((int)threadIdx.x < kBG && ((gmask >> threadIdx.x) & 1ull))
      s_list[__popcll(gmask & ((1ull << threadIdx.x) - 1ull))] = threadIdx.x;
    if (threadIdx.x == 0) s_m = __popcll(gmask);
  } else if (MODE == MODE_DENSE) {
    if ((int)threadIdx.x < kBG) s_list[threadIdx.x] = threadIdx.x;
    if (threadIdx.x == 0) s_m = max(0, min(kBG, n - g0));
  } else {  // MODE_LIST: an even slice of the caller's list per workgroup
    const int cnt = min(max(*A.list_count, 0), n);
    const int per = (cnt + (int)gridDim.x - 1) / (int)gridDim.x;   // <= kBG since gridDim.x = ceil(n / kBG)
    const int e0 = blockIdx.x * per;
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
  if (m == 0) return;
  const int nt = (m + 15) / 16;

  // ---- gate / up products of the active neurons, the activation, a[neuron][token] -------------
  int row[kBT];
#pragma unroll
  for (int q = 0; q < kBT; ++q) {
    const int j = 16 * q + li;
    int id = -1;
    if (j < m) id = (MODE == MODE_LIST) ? s_list[j] : g0 + s_list[j];
    row[q] = id;
  }
  const int kw = d / kBNW, kb = wave * kw;
  const int t = wave;   // after the sum, thread (t, lane) finishes tile t
  const int slot = 16 * t + li;
  const int id = slot < m ? ((MODE == MODE_LIST) ? s_list[slot] : g0 + s_list[slot]) : -1;
  float bj = 0.f;
  if (MODE != MODE_EXACT && id >= 0) bj = A.b[id];
  f32x4 g[TT], u[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) g[tt] = u[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // tiles past nt hold zeros: their sums are computed and not used
  if (MODE == MODE_EXACT) {
    if (A.gated) {
      const f16* const w[1] = {static_cast<const f16*>(A.w_up)};
      f32x4 acc[1][kBT][TT];
      tiles_mma_f16<1, BS, TT>(acc, w, row, nt, xb, B, d, kb, kb + kw);
      waves_sum_tiles<TT>(s_red, acc[0], 1, u);
    }
  } else if (A.gated) {
    const f16* const w[2] = {static_cast<const f16*>(A.w_gate), static_cast<const f16*>(A.w_up)};
    f32x4 acc[2][kBT][TT];
    tiles_mma_f16<2, BS, TT>(acc, w, row, nt, xb, B, d, kb, kb + kw);
    waves_sum_tiles<TT>(s_red, acc[0], 0, g);
    waves_sum_tiles<TT>(s_red, acc[1], 1, u);
  } else {
    const f16* const w[1] = {static_cast<const f16*>(A.w_up)};
    f32x4 acc[1][kBT][TT];
    tiles_mma_f16<1, BS, TT>(acc, w, row, nt, xb, B, d, kb, kb + kw);
    waves_sum_tiles<TT>(s_red, acc[0], 1, u);
  }
  if (id >= 0 && slot < m && t < nt) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      f32x4 a;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tok = 16 * tt + 4 * lk + v;
        float av;
        if (MODE == MODE_EXACT) {
          const float pre = s_pre[s_list[slot] * TS + tok];
          av = A.gated ? fmaxf(pre, 0.f) * u[tt][v] : fmaxf(pre, 0.f);
        } else {
          av = A.gated ? fmaxf(g[tt][v] + bj, 0.f) * u[tt][v] : fmaxf(u[tt][v] + bj, 0.f);
        }
        a[v] = tok < B ? av : 0.f;
      }
      *reinterpret_cast<f32x4*>(abuf + (size_t)id * TS + 16 * tt + 4 * lk) = a;
    }
  }
}

// y partial of neuron chunk blockIdx.y over columns [blockIdx.x * 512, +512): the chunk is a
// range of mask words (predicted, exact), of neurons (dense) or of list entries (list).
// Steps of kDStep neurons: the workgroup reads each neuron's 1 KB row segment with one
// row-contiguous load (the pattern HBM streams best), stages the step in LDS, and each wave
// then reads its 128 columns back in the MFMA layout.  Two LDS buffers: the next step's rows
// are in flight while the current step is multiplied.
constexpr int kDStep = 32;                 // neurons per down step (two workgroups fit a CU's LDS)
constexpr int kDRow = kDW * kDCols;        // 512 columns: a 1 KB fp16 row segment
constexpr int kDPitch = kDRow + 8;         // LDS row pitch in halves (rows start 16 bytes apart in bank order)
constexpr int kDRowsPerWave = kDStep / kDW;

// TT: token tiles of 16, as in k_ffn_bgroup (a[neuron][16 TT]).
template <int MODE, int TT>
__global__ __launch_bounds__(kDW * WAVE) void k_ffn_bdown(const float* __restrict__ abuf, const f16* __restrict__ wd,
                                                          const unsigned* __restrict__ mask_words,
                                                          const int* __restrict__ list, const int* __restrict__ list_count,
                                                          int n, int d, int B, float* __restrict__ partial) {
  constexpr int TS = 16 * TT;
  // a of the step in LDS: [neuron][TS] for one token tile; past it [token][kAP] (neurons
  // contiguous, the row padded by 4 so the lanes' 16-byte reads spread over the banks), the
  // layout the fp16 MFMA's A operand reads
  constexpr int kAP = kDStep + 4;
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE, li = lane & 15, lk = lane >> 4;
  const int C = gridDim.y, c = blockIdx.y;
  const int cw = blockIdx.x * kDRow;               // first column of the workgroup's slice
  const int ncols = min(kDRow, d - cw);            // a multiple of 128
  const bool cols = wave * kDCols < ncols;         // this wave's 128 columns exist
  __shared__ int s_list[kDSeg];
  __shared__ int s_cnt;
  __shared__ f16 s_w[2][kDStep][kDPitch];
  __shared__ __attribute__((aligned(16))) float s_a[2][TT > 1 ? TS * kAP : kDStep * TS];
  auto a_at = [&](int buf, int nrn, int tok) -> float& {
    return TT > 1 ? s_a[buf][tok * kAP + nrn] : s_a[buf][nrn * TS + tok];
  };

  f32x4 acc[8][TT];
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[e][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

  int lo, hi;   // the chunk, in words (mask modes, dense) or list entries (list)
  if (MODE == MODE_LIST) {
    const int cnt = min(max(*list_count, 0), n);
    lo = (int)((long long)c * cnt / C);
    hi = (int)((long long)(c + 1) * cnt / C);
  } else {
    const int nw = (n + 31) / 32;
    lo = (int)((long long)c * nw / C);
    hi = (int)((long long)(c + 1) * nw / C);
  }
  // one step in registers: this wave's kDRowsPerWave rows (16 bytes per lane) and, for the first
  // 128 threads, 4 tokens' activations of one neuron in each token tile
  struct DRegs {
    u32x4 w[kDRowsPerWave];
    f32x4 a[TT];
  };
  constexpr int kSegUnits = (MODE == MODE_LIST) ? kDSeg : kDSeg / 32;
  for (int s0 = lo; s0 < hi; s0 += kSegUnits) {
    const int s1 = min(hi, s0 + kSegUnits);
    __syncthreads();   // the previous segment's list and buffers are no longer read
    if (MODE == MODE_PRED || MODE == MODE_EXACT) {
      if (wave == 0) {   // 64 lanes, one mask word each: in-wave scan of the popcounts
        const unsigned word = (s0 + lane < s1) ? mask_words[s0 + lane] : 0u;
        const int pc = __popc(word);
        int incl = pc;
#pragma unroll
        for (int off = 1; off < WAVE; off <<= 1) {
          const int y = __shfl_up(incl, off, WAVE);
          if (lane >= off) incl += y;
        }
        int pos = incl - pc;
        unsigned mw = word;
        while (mw) {
          const int bit = __ffs((int)mw) - 1;
          s_list[pos++] = 32 * (s0 + lane) + bit;
          mw &= mw - 1u;
        }
        if (lane == WAVE - 1) s_cnt = incl;
      }
    } else if (MODE == MODE_DENSE) {
      const int first = 32 * s0, last = min(n, 32 * s1);
      for (int j = threadIdx.x; j < last - first; j += blockDim.x) s_list[j] = first + j;
      if (threadIdx.x == 0) s_cnt = max(0, last - first);
    } else {
      for (int j = threadIdx.x; j < s1 - s0; j += blockDim.x) {
        const int id = list[s0 + j];
        s_list[j] = ((unsigned)id < (unsigned)n) ? id : -1;
      }
      if (threadIdx.x == 0) s_cnt = s1 - s0;
    }
    __syncthreads();
    const int cnt = s_cnt;
    auto load = [&](DRegs& r, int j0) {
#pragma unroll
      for (int i = 0; i < kDRowsPerWave; ++i) {
        const int j = j0 + wave * kDRowsPerWave + i;
        const int id = j < cnt ? s_list[j] : -1;
        r.w[i] = (id >= 0 && 8 * lane < ncols)
                     ? ld_stream(reinterpret_cast<const u32x4*>(wd + (size_t)id * d + cw) + lane)
                     : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) r.a[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (threadIdx.x < kDStep * 4) {
        const int j = j0 + (int)threadIdx.x / 4;
        const int id = j < cnt ? s_list[j] : -1;
        if (id >= 0) {
#pragma unroll
          for (int tt = 0; tt < TT; ++tt)
            r.a[tt] = *reinterpret_cast<const f32x4*>(abuf + (size_t)id * TS + 16 * tt + 4 * (threadIdx.x % 4));
        }
      }
    };
    // stages one step; returns whether an activation it staged is too large to split (TT > 1)
    auto stage = [&](const DRegs& r, int buf) -> int {
#pragma unroll
      for (int i = 0; i < kDRowsPerWave; ++i)
        *reinterpret_cast<u32x4*>(&s_w[buf][wave * kDRowsPerWave + i][8 * lane]) = r.w[i];
      int big = 0;
      if (threadIdx.x < kDStep * 4) {
        const int nrn = threadIdx.x / 4, t4 = 4 * (threadIdx.x % 4);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          if constexpr (TT > 1) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              a_at(buf, nrn, 16 * tt + t4 + v) = r.a[tt][v];
              big |= fabsf(r.a[tt][v]) >= kSplitLimit ? 1 : 0;
            }
          } else {
            *reinterpret_cast<f32x4*>(&s_a[buf][nrn * TS + t4]) = r.a[tt];
          }
        }
      }
      return big;
    };
    auto mma = [&](int buf) {
      if (!cols) return;
#pragma unroll
      for (int q = 0; q < kDStep / 4; ++q) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(&s_w[buf][4 * q + lk][wave * kDCols + 8 * li]);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          const float a = a_at(buf, 4 * q + lk, 16 * tt + li);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e][tt] = mma_f32(a, half_at(w, e), acc[e][tt]);
        }
      }
    };
    // The whole 32-neuron step on the fp16 MFMA (D[16][16] += A[16][32] B[32][16]): tile e of
    // token tile tt takes A = a[token 16 tt + li][neuron 8 lk + k] and B = W[neuron 8 lk + k]
    // [column 8 li + e], so its outputs land where the fp32 form puts them.
    auto mma_split = [&](int buf) {
      if (!cols) return;
      // this lane's 8 x 8 block of W: neurons 8 lk .. 8 lk + 7, columns 8 li .. 8 li + 7
      f16x8 wr[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        wr[k] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(&s_w[buf][8 * lk + k][wave * kDCols + 8 * li]));
      u32x4 ahi[TT], alo[TT];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const float* ar = &a_at(buf, 8 * lk, 16 * tt + li);
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(ar), a1 = *reinterpret_cast<const f32x4*>(ar + 4);
        const float av[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        f16x8 h, l;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          h[k] = (f16)av[k];
          l[k] = (f16)(av[k] - (float)h[k]);   // a - fp16(a) is exact in fp32
        }
        ahi[tt] = __builtin_bit_cast(u32x4, h);
        alo[tt] = __builtin_bit_cast(u32x4, l);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        f16x8 b;
#pragma unroll
        for (int k = 0; k < 8; ++k) b[k] = wr[k][e];
        const u32x4 bw = __builtin_bit_cast(u32x4, b);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          acc[e][tt] = mma_f16(ahi[tt], bw, acc[e][tt]);
          acc[e][tt] = mma_f16(alo[tt], bw, acc[e][tt]);
        }
      }
    };
    if (cnt == 0) continue;
    DRegs r;
    load(r, 0);
    int big = stage(r, 0);
    if constexpr (TT > 1) big = __syncthreads_or(big);
    else __syncthreads();
    int buf = 0;
    for (int j0 = 0; j0 < cnt; j0 += kDStep) {
      const bool more = j0 + kDStep < cnt;   // uniform
      if (more) load(r, j0 + kDStep);
      if (TT > 1 && !big) mma_split(buf);
      else mma(buf);
      const int nbig = more ? stage(r, buf ^ 1) : 0;
      if constexpr (TT > 1) big = __syncthreads_or(nbig);
      else __syncthreads();
      buf ^= 1;
    }
  }
  if (!cols) return;
  // tile (e, tt) holds columns cw + 128 * wave + 8 * (lane % 16) + e for tokens
  // 16 tt + 4 * (lane / 16) + v
  const int c0 = cw + wave * kDCols;
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int tok = 16 * tt + 4 * lk + v;
      if (tok < B) {
        float* dst = partial + ((size_t)c * B + tok) * d + c0 + 8 * li;
        *reinterpret_cast<f32x4*>(dst) = f32x4{acc[0][tt][v], acc[1][tt][v], acc[2][tt][v], acc[3][tt][v]};
        *reinterpret_cast<f32x4*>(dst + 4) = f32x4{acc[4][tt][v], acc[5][tt][v], acc[6][tt][v], acc[7][tt][v]};
      }
    }
}

}  // namespace pik
