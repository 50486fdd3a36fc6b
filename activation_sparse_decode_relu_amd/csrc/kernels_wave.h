// The one-token predicted step with wave-independent neuron ownership (fp16 weights,
// activations and predictor): k_ffn_wave for fp16 rows with d = 512 * CPLF up to 4096,
// k_ffn_wave2 (wave pairs, half a row each) for fp16 with d from 5120 to 8192 and int4.
//
// A workgroup owns a byte-aligned range of about n / (#CUs) neurons, one workgroup per CU, and
// splits it into 8 waves of at most kWRows consecutive neurons.  Each wave, on its own:
//   mask    its rows' predictor logits z = h P2^T + b_p (1 KB row-contiguous loads), the
//           threshold, and a ballot of its decisions;
//   gather  for each of its selected neurons in order, the full gate / up / down rows, the
//           activation a = ReLU(x W_gate + b) * (x W_up) from two wave sums, and
//           y += a * W_down^T row over the full d, in registers.
// There is no barrier between a wave's mask and gather phases, so the waves of a CU drift
// apart and the CU streams predictor rows and gathered rows at the same time instead of in
// two workgroup-wide phases.  At the end, each wave that selected something stores its y in
// its own LDS slot (a wave that selected nothing holds an exact +0 vector and stores nothing);
// after one barrier every thread adds the occupied slots in wave order into the workgroup's
// partial, so the result is the same on every run.
// The step is the PowerInfer paper explainer's FFN equation (section
// "ニューロン活性化のべき乗則分布") over the neurons its predictor (section "活性化予測器")
// selects (section "GPU-CPUハイブリッドアーキテクチャ", inference flow).
#pragma once

#include "kernels_impl.h"

namespace pik {

constexpr int kWWaves = 8;   // waves per workgroup
constexpr int kWRows = 8;    // most neurons one wave owns (a workgroup owns at most 64)

template <int CPLF>
__global__ __launch_bounds__(kWWaves * WAVE) void k_ffn_wave(const GroupArgs A, int n_units) {
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int n = A.n, d = A.d, r = A.r;
  // this workgroup's neurons: 8-neuron units [u0, u1), so its mask bits are whole bytes
  const int u0 = (int)((long long)blockIdx.x * n_units / gridDim.x);
  const int u1 = (int)((long long)(blockIdx.x + 1) * n_units / gridDim.x);
  const int r0 = 8 * u0, r1 = min(n, 8 * u1);
  const int rpw = (r1 - r0 + kWWaves - 1) / kWWaves;   // <= kWRows
  const int w0 = r0 + wave * rpw, w1 = min(r1, w0 + rpw);

  __shared__ unsigned s_bits[2];                    // the workgroup's decisions (at most 64 neurons)
  __shared__ unsigned s_busy;                       // bit w: wave w selected a neuron and stored its y
  constexpr int kCF = CPLF * WAVE;                  // 16-byte chunks in a row
  __shared__ f32x4 s_y[kWWaves][2 * (kCF + 1)];     // each wave's y: quad k of chunk c at k * (kCF + 1) + c

  if (threadIdx.x < 2) s_bits[threadIdx.x] = 0u;
  if (threadIdx.x == 0) s_busy = 0u;
  __syncthreads();

  // ---- mask: this wave's rows ------------------------------------------------------------------
  float row_bias = 0.f;
  if (lane < w1 - w0) row_bias = A.b_p[w0 + lane];
  int rows[kWRows];
#pragma unroll
  for (int j = 0; j < kWRows; ++j) rows[j] = (w0 + j < w1) ? w0 + j : -1;
  float zacc[kWRows][1];
  rows_dot<DT_F16, DT_F32, 1, kWRows, 2>(zacc, static_cast<const char*>(A.p2), row_bytes(DT_F16, r), nullptr, r, rows,
                                          A.h, 0, 1);
  unsigned mine = 0u;   // bit j: row w0 + j selected (wave-uniform)
#pragma unroll
  for (int j = 0; j < kWRows; ++j) {
    const float v = wave_sum(zacc[j][0]) +
                    __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, row_bias), j));
    if (rows[j] >= 0) {
      if (A.logits != nullptr && lane == 0) A.logits[rows[j]] = v;
      if (v > A.thr) mine |= 1u << j;
    }
  }

  // ---- gather: this wave's selected neurons, full rows, y over the full d ----------------------
  constexpr int NE = 8;
  float acc[CPLF][NE];
#pragma unroll
  for (int q = 0; q < CPLF; ++q)
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[q][e] = 0.f;
  if (!A.mask_only && mine != 0u) {
    const f16* xb = static_cast<const f16*>(A.x);
    XChunk<DT_F16, DT_F16> xq[CPLF];
#pragma unroll
    for (int q = 0; q < CPLF; ++q) xq[q].load(xb + (size_t)(lane + q * WAVE) * 8);
    const size_t rbytes = row_bytes(DT_F16, d);
    const char* wgb = static_cast<const char*>(A.w_gate);
    const char* wub = static_cast<const char*>(A.w_up);
    const char* wdb = static_cast<const char*>(A.w_down_t);
    unsigned todo = mine;
    while (todo != 0u) {
      const int j = __ffs((int)todo) - 1;
      todo &= todo - 1u;
      const int id = w0 + j;
      const float bj = A.b[id];
      u32x4 wg[CPLF], wu[CPLF], wd[CPLF];
#pragma unroll
      for (int q = 0; q < CPLF; ++q) {
        const int c = lane + q * WAVE;
        wg[q] = A.gated ? ld_stream(reinterpret_cast<const u32x4*>(wgb + rbytes * id) + c) : u32x4{0, 0, 0, 0};
        wu[q] = ld_stream(reinterpret_cast<const u32x4*>(wub + rbytes * id) + c);
        wd[q] = ld_stream(reinterpret_cast<const u32x4*>(wdb + rbytes * id) + c);
      }
      float pg = 0.f, pu = 0.f;
#pragma unroll
      for (int q = 0; q < CPLF; ++q) {
        if (A.gated) dot_chunk<DT_F16, DT_F16>(pg, wg[q], xq[q], 1.f);
        dot_chunk<DT_F16, DT_F16>(pu, wu[q], xq[q], 1.f);
      }
      const float g = A.gated ? wave_sum(pg) : 0.f;
      const float u = wave_sum(pu);
      const float a = A.gated ? fmaxf(g + bj, 0.f) * u : fmaxf(u + bj, 0.f);
#pragma unroll
      for (int q = 0; q < CPLF; ++q) {
        float wf[NE];
        Unpack<DT_F16>::run(wd[q], wf);
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[q][e] = fmaf(a, wf[e], acc[q][e]);
      }
    }
  }

  // ---- the workgroup's mask bytes and partial of y ---------------------------------------------
  if (lane == 0 && mine != 0u) {
    const int off = w0 - r0;   // < 64
    atomicOr(&s_bits[off / 32], mine << (off % 32));
    if (off % 32 + rpw > 32) atomicOr(&s_bits[off / 32 + 1], mine >> (32 - off % 32));
  }
  if (!A.mask_only && mine != 0u) {
#pragma unroll
    for (int q = 0; q < CPLF; ++q) {
      const int c = lane + q * WAVE;
      s_y[wave][c] = f32x4{acc[q][0], acc[q][1], acc[q][2], acc[q][3]};
      s_y[wave][kCF + 1 + c] = f32x4{acc[q][4], acc[q][5], acc[q][6], acc[q][7]};
    }
    if (lane == 0) atomicOr(&s_busy, 1u << wave);
  }
  __syncthreads();
  if ((int)threadIdx.x < u1 - u0) {
    const int bo = 8 * (int)threadIdx.x;
    reinterpret_cast<unsigned char*>(A.mask_words)[u0 + threadIdx.x] =
        (unsigned char)(s_bits[bo / 32] >> (bo % 32));
  }
  if (A.mask_only) return;
  const unsigned busy = s_busy;
  float* dst = A.partial + (size_t)blockIdx.x * d;
  for (int k = threadIdx.x; k < 2 * kCF; k += blockDim.x) {   // quad k of the row
    const int slot = (k & 1) * (kCF + 1) + (k >> 1);
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    bool first = true;
#pragma unroll
    for (int w = 0; w < kWWaves; ++w) {
      if ((busy >> w) & 1u) {
        v = first ? s_y[w][slot] : v + s_y[w][slot];
        first = false;
      }
    }
    *reinterpret_cast<f32x4*>(dst + 4 * k) = v;
  }
}


// ---------------------------------------------------------------------------------------------
// k_ffn_wave2: the same step on wave pairs, for layers whose rows do not fit one wave's
// registers: fp16 with d = 1024 * CPLH (5120 .. 8192), and int4 group-32 with d = 4096 * CPLH.
// The 8 waves form 4 pairs; the two waves of a pair take the two halves of d (and of r for the
// predictor).
//   mask    each pair computes the half-r partial logits of a quarter of the workgroup's
//           neurons; after a barrier one thread per neuron adds the halves (first + second)
//           and the bias, and the decisions become a ballot bit set and then the workgroup's
//           ascending list of selected neurons;
//   gather  the list is dealt round-robin to the pairs (pair p takes entries p, p + 4, ...), so
//           each pair handles at most ceil(selected / 4), NJ neurons per step.  For each step
//           both waves of the pair load their halves of the NJ neurons' rows, exchange their
//           partial gate and up sums through LDS (each wave raises its own LDS step counter and
//           waits for its partner's: both walk the same entries, so they take the same steps,
//           and the partner is a wave of the same workgroup that waits on nothing else), form
//           the activations identically, and add a * W_down^T over their half of d.
// At the end each pair's y halves are added in pair order through LDS, so the result is the
// same on every run.  int4 rows are one group of 32 per 16-byte chunk: a chunk's scale
// multiplies its partial gate / up sum, and multiplies a for its slice of the down row.
// ---------------------------------------------------------------------------------------------
constexpr int kW2Pairs = 4;                          // wave pairs per workgroup (8 waves)
constexpr int kW2Rows = 32;                          // predictor rows per pair
constexpr int kW2Max = kW2Pairs * kW2Rows;           // most neurons one workgroup owns (128)
constexpr int kW2Units = kW2Max / 8;

template <int WT, int CPLH, int NJ>   // chunks per lane of a half row; neurons per exchange step
__global__ __launch_bounds__(2 * kW2Pairs * WAVE) void k_ffn_wave2(const GroupArgs A, int n_units) {
  constexpr int EPC = WFmt<WT>::EPC;                 // elements per 16-byte chunk
  constexpr int kQH = CPLH * WAVE * EPC / 4;         // float4 quads in half a row
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int pair = wave >> 1, half = wave & 1;
  const int n = A.n, d = A.d, r = A.r;
  const int u0 = (int)((long long)blockIdx.x * n_units / gridDim.x);
  const int u1 = (int)((long long)(blockIdx.x + 1) * n_units / gridDim.x);
  const int r0 = 8 * u0, r1 = min(n, 8 * u1);        // r1 - r0 <= kW2Max
  const int dh = d / 2, rh = r / 2;                  // this wave's halves of d and r

  __shared__ unsigned s_bits[kW2Max / 32];
  __shared__ int s_list[kW2Max];                     // the selected neurons, ascending
  __shared__ unsigned s_busy;                        // bit p: pair p handled a neuron
  __shared__ int s_step[2 * kW2Pairs];               // steps each wave has published
  __shared__ float s_z[2][kW2Max];                   // partial logits by half of r
  __shared__ float s_gu[kW2Pairs][2][2][NJ][2];      // [pair][step parity][half][neuron][g, u]
  constexpr int kCH = CPLH * WAVE;                  // chunks in half a row
  __shared__ f32x4 s_y[2 * kW2Pairs][(EPC / 4) * (kCH + 1)];

  if (threadIdx.x == 0) s_busy = 0u;
  if ((int)threadIdx.x < 2 * kW2Pairs) s_step[threadIdx.x] = 0;

  // ---- mask: a quarter of the workgroup's rows per pair, this wave's half of r -----------------
  {
    const f16* p2 = static_cast<const f16*>(A.p2);
    const int rpp = (r1 - r0 + kW2Pairs - 1) / kW2Pairs;   // <= kW2Rows
    const int q0 = r0 + pair * rpp, q1 = min(r1, q0 + rpp);
    const bool cok = 8 * lane < rh;
    u32x4 pw[kW2Rows];
#pragma unroll
    for (int j = 0; j < kW2Rows; ++j)
      pw[j] = (q0 + j < q1 && cok)
                  ? ld_stream(reinterpret_cast<const u32x4*>(p2 + (size_t)(q0 + j) * r + half * rh) + lane)
                  : u32x4{0, 0, 0, 0};
    XChunk<DT_F16, DT_F32> hx;
    if (cok) hx.load(A.h + half * rh + 8 * lane);
    else hx.zero();
#pragma unroll
    for (int j = 0; j < kW2Rows; ++j) {
      float a = 0.f;
      dot_chunk<DT_F16, DT_F32>(a, pw[j], hx, 1.f);
      const float zp = wave_sum(a);
      if (lane == 0 && q0 + j < q1) s_z[half][q0 - r0 + j] = zp;
    }
  }
  __syncthreads();
  if (threadIdx.x < kW2Max) {   // waves 0 and 1: one neuron per thread
    const int t = threadIdx.x;
    bool sel = false;
    if (r0 + t < r1) {
      const float v = (s_z[0][t] + s_z[1][t]) + A.b_p[r0 + t];
      if (A.logits != nullptr) A.logits[r0 + t] = v;
      sel = v > A.thr;
    }
    const unsigned long long bal = __ballot(sel);
    if (lane == 0) {
      s_bits[2 * wave] = (unsigned)bal;
      s_bits[2 * wave + 1] = (unsigned)(bal >> 32);
    }
  }
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int w = 0; w < kW2Max / 32; ++w) total += __popc(s_bits[w]);
  if (threadIdx.x < kW2Max) {
    const int t = threadIdx.x, w = t / 32, b = t % 32;
    if ((s_bits[w] >> b) & 1u) {
      int pos = __popc(s_bits[w] & ((1u << b) - 1u));
      for (int k = 0; k < w; ++k) pos += __popc(s_bits[k]);
      s_list[pos] = r0 + t;
    }
  }
  __syncthreads();

  // ---- gather: list entries pair, pair + 4, ...; this wave's half of every row ----------------
  float acc[CPLH][EPC];
#pragma unroll
  for (int q = 0; q < CPLH; ++q)
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[q][e] = 0.f;
  const int share = (total - pair + kW2Pairs - 1) / kW2Pairs;   // entries this pair handles
  const bool busy = !A.mask_only && share > 0;
  if (busy) {
    int step = 0;
    const f16* xb = static_cast<const f16*>(A.x) + half * dh;
    XChunk<WT, DT_F16> xq[CPLH];
#pragma unroll
    for (int q = 0; q < CPLH; ++q) xq[q].load(xb + (size_t)(lane + q * WAVE) * EPC);
    const size_t rbytes = row_bytes(WT, d), hoff = row_bytes(WT, dh) * half;
    const int spr = d / 32, soff = half * (dh / 32);   // int4 scales per row, this half's first
    const char* wgb = static_cast<const char*>(A.w_gate) + hoff;
    const char* wub = static_cast<const char*>(A.w_up) + hoff;
    const char* wdb = static_cast<const char*>(A.w_down_t) + hoff;
#pragma unroll 1
    for (int k0 = 0; k0 < share; k0 += NJ) {
      int id[NJ];
      bool ok[NJ];
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        ok[jj] = k0 + jj < share;
        id[jj] = ok[jj] ? s_list[pair + kW2Pairs * (k0 + jj)] : 0;
      }
      // Every load of the step is issued before any is used: rows, biases and (int4) the raw
      // scales, the latter two from a valid neuron (id 0) for empty entries and dropped after.
      u32x4 wg[NJ][CPLH], wu[NJ][CPLH], wd[NJ][CPLH];
      f16 rsg[NJ][CPLH], rsu[NJ][CPLH], rsd[NJ][CPLH];
      float bj[NJ];
      const f16* sgp = A.gated ? A.s_gate : A.s_up;
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        bj[jj] = A.b[id[jj]];
#pragma unroll
        for (int q = 0; q < CPLH; ++q) {
          const int c = lane + q * WAVE;
          const size_t off = rbytes * id[jj];
          const bool g_ok = ok[jj] && A.gated;
          wg[jj][q] = g_ok ? ld_stream(reinterpret_cast<const u32x4*>(wgb + off) + c) : u32x4{0, 0, 0, 0};
          wu[jj][q] = ok[jj] ? ld_stream(reinterpret_cast<const u32x4*>(wub + off) + c) : u32x4{0, 0, 0, 0};
          wd[jj][q] = ok[jj] ? ld_stream(reinterpret_cast<const u32x4*>(wdb + off) + c) : u32x4{0, 0, 0, 0};
          if constexpr (WT == DT_Q4) {
            const size_t so = (size_t)id[jj] * spr + soff + c;
            rsg[jj][q] = sgp[so];
            rsu[jj][q] = A.s_up[so];
            rsd[jj][q] = A.s_down[so];
          }
        }
      }
      float sg[NJ][CPLH], su[NJ][CPLH], sd[NJ][CPLH];
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
        for (int q = 0; q < CPLH; ++q) {
          sg[jj][q] = (WT == DT_Q4 && ok[jj] && A.gated) ? (float)rsg[jj][q] : 1.f;
          su[jj][q] = (WT == DT_Q4 && ok[jj]) ? (float)rsu[jj][q] : 1.f;
          sd[jj][q] = (WT == DT_Q4 && ok[jj]) ? (float)rsd[jj][q] : 1.f;
        }
      const int slot = step & 1;
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        float pg = 0.f, pu = 0.f;
#pragma unroll
        for (int q = 0; q < CPLH; ++q) {
          if (A.gated) dot_chunk<WT, DT_F16>(pg, wg[jj][q], xq[q], sg[jj][q]);
          dot_chunk<WT, DT_F16>(pu, wu[jj][q], xq[q], su[jj][q]);
        }
        const float gh = A.gated ? wave_sum(pg) : 0.f;
        const float uh = wave_sum(pu);
        if (lane == 0) {
          s_gu[pair][slot][half][jj][0] = gh;
          s_gu[pair][slot][half][jj][1] = uh;
        }
      }
      // publish this wave's step, then wait for the partner's: the two-slot ring is safe
      // because a wave reuses a slot only after its partner has published the step after
      // the one that read it
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      ++step;
      if (lane == 0) __hip_atomic_store(&s_step[wave], step, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      while (__hip_atomic_load(&s_step[wave ^ 1], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < step)
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        if (!ok[jj]) continue;
        const float g = s_gu[pair][slot][0][jj][0] + s_gu[pair][slot][1][jj][0];
        const float u = s_gu[pair][slot][0][jj][1] + s_gu[pair][slot][1][jj][1];
        const float a = A.gated ? fmaxf(g + bj[jj], 0.f) * u : fmaxf(u + bj[jj], 0.f);
#pragma unroll
        for (int q = 0; q < CPLH; ++q) {
          float wf[EPC];
          Unpack<WT>::run(wd[jj][q], wf);
          const float as = a * sd[jj][q];
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[q][e] = fmaf(as, wf[e], acc[q][e]);
        }
      }
    }
  }

  // ---- the workgroup's mask bytes and partial of y ---------------------------------------------
  if ((int)threadIdx.x < u1 - u0) {
    const int bo = 8 * (int)threadIdx.x;
    reinterpret_cast<unsigned char*>(A.mask_words)[u0 + threadIdx.x] =
        (unsigned char)(s_bits[bo / 32] >> (bo % 32));
  }
  if (A.mask_only) return;
  // y halves in LDS: quad k (elements 4k .. 4k+3) of chunk c at k * (kCH + 1) + c, so the lanes
  // of a store touch consecutive 16-byte slots, and threads reading consecutive quads of a row
  // below land on different banks
  if (busy) {
#pragma unroll
    for (int q = 0; q < CPLH; ++q) {
      const int c = lane + q * WAVE;
#pragma unroll
      for (int k = 0; k < EPC / 4; ++k)
        s_y[wave][k * (kCH + 1) + c] = f32x4{acc[q][4 * k], acc[q][4 * k + 1], acc[q][4 * k + 2], acc[q][4 * k + 3]};
    }
    if (half == 0 && lane == 0) atomicOr(&s_busy, 1u << pair);
  }
  __syncthreads();
  const unsigned bmask = s_busy;
  float* dst = A.partial + (size_t)blockIdx.x * d;
  for (int g = threadIdx.x; g < 2 * kQH; g += blockDim.x) {   // quad g of the row
    const int hh = g / kQH, gq = g % kQH;                      // half, quad within it
    const int slot = (gq % (EPC / 4)) * (kCH + 1) + gq / (EPC / 4);
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    bool first = true;
#pragma unroll
    for (int p = 0; p < kW2Pairs; ++p) {
      if ((bmask >> p) & 1u) {
        v = first ? s_y[2 * p + hh][slot] : v + s_y[2 * p + hh][slot];
        first = false;
      }
    }
    *reinterpret_cast<f32x4*>(dst + 4 * g) = v;
  }
}

}  // namespace pik
