// Launchers of the batched matrix-core path.
#include "kernels_batch.h"

namespace pik {

bool batch_supported(int wt, int at, int pt, int B, int d, int r) {
  return B > 1 && B <= kMaxTokens && wt == DT_F16 && at == DT_F16 && (r == 0 || pt == DT_F16) && d % 128 == 0 &&
         r % 128 == 0;
}

bool batch_large_supported(int wt, int at, int B, int d) {
  return B > kMaxTokens && B <= kMaxBatchTokens && wt == DT_F16 && at == DT_F16 && d % 128 == 0;
}

int batch_tiles(int B) { return B <= 16 ? 1 : (B <= 32 ? 2 : 4); }

int batch_groups(int n) { return (n + kBG - 1) / kBG; }

int batch_down_chunks(int d) {
  const int slices = (d + kDW * kDCols - 1) / (kDW * kDCols);
  return (512 + slices - 1) / slices;   // about 512 down workgroups: two per CU, so one can multiply
                                        // while the other waits on its rows
}

namespace {

template <int TT>
hipError_t bgroup_tt(int mode, const GroupArgs& a, float* abuf, hipStream_t s) {
  const dim3 grid(batch_groups(a.n)), block(kBNW * WAVE);
  if constexpr (TT == 1) {
    switch (mode) {
      case MODE_PRED: hipLaunchKernelGGL((k_ffn_bgroup<MODE_PRED, 1>), grid, block, 0, s, a, abuf); break;
      case MODE_LIST: hipLaunchKernelGGL((k_ffn_bgroup<MODE_LIST, 1>), grid, block, 0, s, a, abuf); break;
      case MODE_EXACT: hipLaunchKernelGGL((k_ffn_bgroup<MODE_EXACT, 1>), grid, block, 0, s, a, abuf); break;
      case MODE_DENSE: hipLaunchKernelGGL((k_ffn_bgroup<MODE_DENSE, 1>), grid, block, 0, s, a, abuf); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (mode) {
      case MODE_EXACT: hipLaunchKernelGGL((k_ffn_bgroup<MODE_EXACT, TT>), grid, block, 0, s, a, abuf); break;
      case MODE_DENSE: hipLaunchKernelGGL((k_ffn_bgroup<MODE_DENSE, TT>), grid, block, 0, s, a, abuf); break;
      default: return hipErrorInvalidValue;   // more than 16 tokens: exact or dense only
    }
  }
  return hipGetLastError();
}

template <int TT>
hipError_t bdown_tt(int mode, const GroupArgs& a, const float* abuf, int chunks, hipStream_t s) {
  const dim3 grid((a.d + kDW * kDCols - 1) / (kDW * kDCols), chunks), block(kDW * WAVE);
  const f16* wd = static_cast<const f16*>(a.w_down_t);
  if (TT > 1 && mode != MODE_EXACT && mode != MODE_DENSE) return hipErrorInvalidValue;
  switch (mode) {
    case MODE_PRED:
      if constexpr (TT == 1)
        hipLaunchKernelGGL((k_ffn_bdown<MODE_PRED, 1>), grid, block, 0, s, abuf, wd, a.mask_words, nullptr, nullptr,
                           a.n, a.d, a.B, a.partial);
      break;
    case MODE_EXACT:
      hipLaunchKernelGGL((k_ffn_bdown<MODE_EXACT, TT>), grid, block, 0, s, abuf, wd, a.mask_words, nullptr, nullptr,
                         a.n, a.d, a.B, a.partial);
      break;
    case MODE_DENSE:
      hipLaunchKernelGGL((k_ffn_bdown<MODE_DENSE, TT>), grid, block, 0, s, abuf, wd, nullptr, nullptr, nullptr, a.n,
                         a.d, a.B, a.partial);
      break;
    case MODE_LIST:
      if constexpr (TT == 1)
        hipLaunchKernelGGL((k_ffn_bdown<MODE_LIST, 1>), grid, block, 0, s, abuf, wd, nullptr, a.list, a.list_count,
                           a.n, a.d, a.B, a.partial);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_bgroup(int mode, const GroupArgs& a, float* abuf, hipStream_t s) {
  switch (batch_tiles(a.B)) {
    case 1: return bgroup_tt<1>(mode, a, abuf, s);
    case 2: return bgroup_tt<2>(mode, a, abuf, s);
    default: return bgroup_tt<4>(mode, a, abuf, s);
  }
}

hipError_t launch_ffn_bdown(int mode, const GroupArgs& a, const float* abuf, int chunks, hipStream_t s) {
  switch (batch_tiles(a.B)) {
    case 1: return bdown_tt<1>(mode, a, abuf, chunks, s);
    case 2: return bdown_tt<2>(mode, a, abuf, chunks, s);
    default: return bdown_tt<4>(mode, a, abuf, chunks, s);
  }
}

}  // namespace pik
