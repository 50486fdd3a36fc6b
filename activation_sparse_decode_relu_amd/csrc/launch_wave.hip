// Launcher of the wave-independent one-token predicted kernel.
#include <algorithm>

#include "kernels_wave.h"

namespace pik {

bool wave_supported(int wt, int at, int pt, int mode, int B, int d) {
  return mode == MODE_PRED && B == 1 && wt == DT_F16 && at == DT_F16 && pt == DT_F16 && d % 512 == 0 && d >= 512 &&
         d <= 4096;
}

int wave_grid(int n) {
  const int units = (n + 7) / 8;
  const int need = (units + kWRows - 1) / kWRows;     // at most kWRows units (64 neurons) per workgroup
  return std::min(units, std::max(kWaveGridBase, need));
}

hipError_t launch_ffn_wave(const GroupArgs& a, hipStream_t s) {
  const int units = (a.n + 7) / 8;
  const dim3 grid(wave_grid(a.n)), block(kWWaves * WAVE);
  switch (a.d / 512) {
#define PIK_WAVE(C) \
  case C: hipLaunchKernelGGL((k_ffn_wave<C>), grid, block, 0, s, a, units); break;
    PIK_WAVE(1) PIK_WAVE(2) PIK_WAVE(3) PIK_WAVE(4) PIK_WAVE(5) PIK_WAVE(6) PIK_WAVE(7) PIK_WAVE(8)
#undef PIK_WAVE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pik
