// Launchers of the one-token split path (k_act, then k_down).
#include <algorithm>

#include "kernels_split.h"

namespace pik {

namespace {

// Chosen by timing the variants on Llama2-70B, LLaMA-7B and Falcon-40B int4 shaped layers (MI355X):
constexpr int kNPW = 8;          // neurons per k_act wave: one mask byte (16 per wave: 4-25 % slower)
constexpr bool kXLds = true;     // k_act: x staged in LDS (in registers: 1 % slower, more VGPRs)
constexpr int kDnNT = 512;       // k_down: 8 waves per tile (4 waves: 6-35 % slower)
constexpr int kDnTiles = 256;    // k_down: about one tile per compute unit
// k_down chunks: each tile's own range of mask words, so no tile but (0, 0) scans the whole mask.
// Against equal counts of the global list this was 6 % faster on Llama2-70B (13.0 against
// 13.8 us), 3 % on Falcon-40B int4 and 1 % on LLaMA-7B, with the neurons' order random under the
// firing law.  A layout that packed the always-firing neurons into the first words would load
// the first chunks several times the mean (hot-first Llama2-70B: 42 us, not 15).
template <int WT> constexpr bool dn_local() { return true; }
// k_down rows per load batch (two batches in flight): 4 for both formats (fp16: 13.8 against
// 14.0 us with 8 on Llama2-70B, 7.9 against 8.2 on LLaMA-7B; int4: 12.0 against 14.5)
constexpr int kDnU = 4;

int epc_of(int wt) { return wt == DT_Q4 ? 32 : (wt == DT_F16 ? 8 : 4); }

// Chunks of 16 bytes per lane in a full weight row (0 if the row does not split evenly).
int row_cpl(int wt, int d) {
  const int per = WAVE * epc_of(wt);
  return d % per == 0 ? d / per : 0;
}

}  // namespace

int split_slices(int wt, int d) {
  const int sw = wt == DT_Q4 ? dn_slice_cols<DT_Q4>() : dn_slice_cols<DT_F16>();
  return (d + sw - 1) / sw;
}

bool split_supported(int wt, int at, int pt, int B, int d, int r, int n) {
  if (B != 1 || at != DT_F16 || (r > 0 && pt != DT_F16)) return false;
  // k_down addresses a weight matrix (and a, and int4 scales) through 32-bit buffer offsets
  if ((long long)n * (long long)row_bytes(wt, d) >= (1LL << 31)) return false;
  const int cpl = row_cpl(wt, d);
  bool ok = false;
  if (wt == DT_F16) ok = cpl >= 1 && cpl <= 16;   // d = 512 .. 8192 in steps of 512
  if (wt == DT_Q4) ok = cpl >= 1 && cpl <= 4;     // d = 2048 .. 8192 in steps of 2048
  return ok && split_slices(wt, d) <= kMaxDnSlices;
}

int split_chunks(int wt, int d) {
  // about kDnTiles down tiles, at most kMaxDnChunks partials per slice: the last tile of a slice
  // reads them all in one round of loads
  const int s = split_slices(wt, d);
  return std::max(1, std::min(kMaxDnChunks, (kDnTiles + s - 1) / s));
}

// Gated or not is a template argument: with it known, the compiler keeps the Llama2-70B-width
// kernel at 172 VGPRs instead of 211 and drops a branch around every row load (LLaMA-7B: 11.3
// against 11.8 us, Falcon-40B int4: 19.8 against 20.7).  Workgroup shape per row format, timed
// on each workload's shape:
//   fp16 gated, rows up to 4096 (LLaMA-7B)      8 waves, per-wave gathers (11.0 against 11.5 us
//                                               with 4)
//   fp16 gated, wider rows (Llama2-70B)         4 waves, per-wave gathers (8 waves: 29.0 against
//                                               28.5; dealt gathers: 29.0)
//   fp16 non-gated (OPT-30B)                    8 waves, per-wave gathers (16.6 against 17.0 with
//                                               4 waves dealt, 16.8 with 4 per wave)
//   int4 (Falcon-40B)                           4 waves, the selected neurons dealt to the waves
//                                               after a barrier (18.7 against 20.0 per wave)
template <int WT, int CPL, int GT> struct ActShape {
  static constexpr bool kDeal = WT == DT_Q4 && GT == 0;
  static constexpr int kWaves = (WT == DT_F16 && (GT == 0 || CPL <= 8)) ? 8 : 4;
};

template <int WT, int MODE, int GT>
static hipError_t act_cpl(const GroupArgs& a, float* abuf, int cpl, hipStream_t s) {
  const int waves = (a.n + kNPW - 1) / kNPW;
  switch (cpl) {
#define PIK_ACT(C)                                                                                                \
  case C: {                                                                                                        \
    using S = ActShape<WT, C, GT>;                                                                                \
    const dim3 grid((waves + S::kWaves - 1) / S::kWaves), block(S::kWaves * WAVE);                                \
    hipLaunchKernelGGL((k_act<WT, C, MODE, kNPW, kXLds, S::kWaves, GT, S::kDeal>), grid, block, 0, s, a, abuf);  \
    break;                                                                                                         \
  }
    PIK_ACT(1) PIK_ACT(2) PIK_ACT(3) PIK_ACT(4)
    default:
      if constexpr (WT == DT_F16) {
        switch (cpl) {
          PIK_ACT(5) PIK_ACT(6) PIK_ACT(7) PIK_ACT(8) PIK_ACT(9) PIK_ACT(10) PIK_ACT(11) PIK_ACT(12)
          PIK_ACT(13) PIK_ACT(14) PIK_ACT(15) PIK_ACT(16)
          default: return hipErrorInvalidValue;
        }
      } else {
        return hipErrorInvalidValue;
      }
#undef PIK_ACT
  }
  return hipGetLastError();
}

template <int WT, int GT>
static hipError_t act_mode(int mode, const GroupArgs& a, float* abuf, int cpl, hipStream_t s) {
  switch (mode) {
    case MODE_PRED: return act_cpl<WT, MODE_PRED, GT>(a, abuf, cpl, s);
    case MODE_EXACT: return act_cpl<WT, MODE_EXACT, GT>(a, abuf, cpl, s);
    case MODE_DENSE: return act_cpl<WT, MODE_DENSE, GT>(a, abuf, cpl, s);
    case MODE_LIST: return act_cpl<WT, MODE_LIST, GT>(a, abuf, cpl, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_act(int wt, int mode, const GroupArgs& a, float* abuf, hipStream_t s) {
  const int cpl = row_cpl(wt, a.d);
  if (wt == DT_F16) return a.gated ? act_mode<DT_F16, 1>(mode, a, abuf, cpl, s) : act_mode<DT_F16, 0>(mode, a, abuf, cpl, s);
  if (wt == DT_Q4) return a.gated ? act_mode<DT_Q4, 1>(mode, a, abuf, cpl, s) : act_mode<DT_Q4, 0>(mode, a, abuf, cpl, s);
  return hipErrorInvalidValue;
}

template <int WT>
static hipError_t down_mode(int mode, const DownArgs& D, dim3 grid, hipStream_t s) {
  constexpr int U = kDnU;
  const dim3 block(kDnNT);
  switch (mode) {
    case MODE_PRED: hipLaunchKernelGGL((k_down<WT, MODE_PRED, U, kDnNT, dn_local<WT>()>), grid, block, 0, s, D); break;
    case MODE_EXACT: hipLaunchKernelGGL((k_down<WT, MODE_EXACT, U, kDnNT, dn_local<WT>()>), grid, block, 0, s, D); break;
    case MODE_DENSE: hipLaunchKernelGGL((k_down<WT, MODE_DENSE, U, kDnNT, dn_local<WT>()>), grid, block, 0, s, D); break;
    case MODE_LIST: hipLaunchKernelGGL((k_down<WT, MODE_LIST, U, kDnNT, dn_local<WT>()>), grid, block, 0, s, D); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_down(int wt, int mode, const DownArgs& D, hipStream_t s) {
  // an index-list-only call (predict) runs one tile, which writes the list and count
  const dim3 grid = D.do_down ? dim3(split_slices(wt, D.d), D.chunks) : dim3(1, 1);
  if (wt == DT_F16) return down_mode<DT_F16>(mode, D, grid, s);
  if (wt == DT_Q4) return down_mode<DT_Q4>(mode, D, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace pik
