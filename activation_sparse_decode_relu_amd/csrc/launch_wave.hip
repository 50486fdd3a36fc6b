// Launcher of the wave-independent one-token predicted kernel.
#include <algorithm>

#include "kernels_wave.h"

namespace pik {

// Wave pairs take fp16 layers wider than 4096 and int4 layers.
static bool wave_pairs(int wt, int d) { return wt == DT_Q4 || d > 4096; }

bool wave_supported(int wt, int at, int pt, int mode, int B, int d, int r) {
  if (mode != MODE_PRED || B != 1 || at != DT_F16 || pt != DT_F16) return false;
  if (wt == DT_F16 && d >= 512 && d <= 4096) return d % 512 == 0;
  // wave pairs: each wave holds half a row of d and takes half of r in one 16-byte chunk per lane
  if (r % 16 != 0 || r > 16 * WAVE) return false;
  if (wt == DT_F16) return d > 4096 && d <= 8192 && d % 1024 == 0;
  if (wt == DT_Q4) return d == 4096 || d == 8192;
  return false;
}

int wave_grid(int n, int d, int wt) {
  const int units = (n + 7) / 8;
  // at most kWRows units (64 neurons) per one-wave workgroup, kW2Units (128) per wave-pair one
  const int per = wave_pairs(wt, d) ? kW2Units : kWRows;
  return std::min(units, std::max(kWaveGridBase, (units + per - 1) / per));
}

hipError_t launch_ffn_wave(int wt, const GroupArgs& a, hipStream_t s) {
  const int units = (a.n + 7) / 8;
  const dim3 grid(wave_grid(a.n, a.d, wt));
  if (wt == DT_Q4) {
    const dim3 block(2 * kW2Pairs * WAVE);
    // one neuron per exchange step: a pair handles few selected neurons, and a step waits for all
    // of its neurons' rows (Falcon-40B shape: 42.0 us per layer-step, against 45.1 with four)
    if (a.d == 4096) hipLaunchKernelGGL((k_ffn_wave2<DT_Q4, 1, 1>), grid, block, 0, s, a, units);
    else if (a.d == 8192) hipLaunchKernelGGL((k_ffn_wave2<DT_Q4, 2, 1>), grid, block, 0, s, a, units);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (a.d > 4096) {
    const dim3 block(2 * kW2Pairs * WAVE);
    switch (a.d / 1024) {
#define PIK_WAVE2(C) \
  case C: hipLaunchKernelGGL((k_ffn_wave2<DT_F16, C, 1>), grid, block, 0, s, a, units); break;
      PIK_WAVE2(5) PIK_WAVE2(6) PIK_WAVE2(7) PIK_WAVE2(8)
#undef PIK_WAVE2
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const dim3 block(kWWaves * WAVE);
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
