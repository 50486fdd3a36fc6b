// Group kernel instances for int4 (group-32) weights.
#include "kernels_impl.h"

namespace pik {

#define PIK_GRP(W, AC, M, C, NWV) \
  hipLaunchKernelGGL((k_ffn_group<W, AC, NB, M, C, NWV>), dim3((a.n + a.G - 1) / a.G), dim3(a.nw * WAVE), 0, s, a)
#define PIK_GRP_NW(W, AC, M, C)                 \
  do {                                          \
    if (a.nw == 4) PIK_GRP(W, AC, M, C, 4);     \
    else PIK_GRP(W, AC, M, C, 8);               \
  } while (0)
#define PIK_GRP_C(W, AC, M)                      \
  do {                                           \
    if (cpl == 1) PIK_GRP_NW(W, AC, M, 1);       \
    else if (cpl == 2) PIK_GRP_NW(W, AC, M, 2);  \
    else PIK_GRP_NW(W, AC, M, 4);                \
  } while (0)
#define PIK_GRP_M(W, AC)                                       \
  do {                                                         \
    if (mode == MODE_PRED) PIK_GRP_C(W, AC, MODE_PRED);        \
    else if (mode == MODE_EXACT) PIK_GRP_C(W, AC, MODE_EXACT); \
    else if (mode == MODE_DENSE) PIK_GRP_C(W, AC, MODE_DENSE); \
    else PIK_GRP_C(W, AC, MODE_LIST);                          \
  } while (0)

hipError_t launch_ffn_group_q4(int at, int mode, const GroupArgs& a, int cpl, hipStream_t s) {
  return with_nb(a.B, [&](auto nbc) -> hipError_t {
    constexpr int NB = decltype(nbc)::value;
    if (at == DT_F16) PIK_GRP_M(DT_Q4, DT_F16);
    else PIK_GRP_M(DT_Q4, DT_F32);
    return hipGetLastError();
  });
}

}  // namespace pik
