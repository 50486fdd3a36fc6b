// Launchers of the batched matrix-core path.
#include "kernels_batch.h"

namespace pik {

bool batch_supported(int wt, int at, int pt, int B, int d, int r) {
  return B > 1 && B <= kMaxTokens && wt == DT_F16 && at == DT_F16 && (r == 0 || pt == DT_F16) && d % 128 == 0 &&
         r % 128 == 0;
}

int batch_groups(int n) { return (n + kBG - 1) / kBG; }

int batch_down_chunks(int d) {
  const int slices = (d + kDW * kDCols - 1) / (kDW * kDCols);
  return (512 + slices - 1) / slices;   // about 512 down workgroups: two per CU, so one can multiply
                                        // while the other waits on its rows
}

hipError_t launch_ffn_bgroup(int mode, const GroupArgs& a, float* abuf, hipStream_t s) {
  const dim3 grid(batch_groups(a.n)), block(kBNW * WAVE);
  switch (mode) {
    case MODE_PRED: hipLaunchKernelGGL((k_ffn_bgroup<MODE_PRED>), grid, block, 0, s, a, abuf); break;
    case MODE_EXACT: hipLaunchKernelGGL((k_ffn_bgroup<MODE_EXACT>), grid, block, 0, s, a, abuf); break;
    case MODE_DENSE: hipLaunchKernelGGL((k_ffn_bgroup<MODE_DENSE>), grid, block, 0, s, a, abuf); break;
    case MODE_LIST: hipLaunchKernelGGL((k_ffn_bgroup<MODE_LIST>), grid, block, 0, s, a, abuf); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_ffn_bdown(int mode, const GroupArgs& a, const float* abuf, int chunks, hipStream_t s) {
  const dim3 grid((a.d + kDW * kDCols - 1) / (kDW * kDCols), chunks), block(kDW * WAVE);
  const f16* wd = static_cast<const f16*>(a.w_down_t);
  switch (mode) {
    case MODE_PRED:
      hipLaunchKernelGGL((k_ffn_bdown<MODE_PRED>), grid, block, 0, s, abuf, wd, a.mask_words, nullptr, nullptr, a.n,
                         a.d, a.B, a.partial);
      break;
    case MODE_EXACT:
      hipLaunchKernelGGL((k_ffn_bdown<MODE_EXACT>), grid, block, 0, s, abuf, wd, a.mask_words, nullptr, nullptr, a.n,
                         a.d, a.B, a.partial);
      break;
    case MODE_DENSE:
      hipLaunchKernelGGL((k_ffn_bdown<MODE_DENSE>), grid, block, 0, s, abuf, wd, nullptr, nullptr, nullptr, a.n, a.d,
                         a.B, a.partial);
      break;
    case MODE_LIST:
      hipLaunchKernelGGL((k_ffn_bdown<MODE_LIST>), grid, block, 0, s, abuf, wd, nullptr, a.list, a.list_count, a.n,
                         a.d, a.B, a.partial);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pik
