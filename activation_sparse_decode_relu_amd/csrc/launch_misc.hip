// Host-side launchers: runtime dtypes -> template instances (small kernels here; the large
// group kernels in their own translation units).
#include "kernels_impl.h"

namespace pik {

namespace {
constexpr int kBlock = 256;
}  // namespace

int group_cpl(int wt, int d, int nw) {
  const int epc = wt == DT_F32 ? 4 : (wt == DT_F16 ? 8 : 32);
  const int nch = d / epc;
  const int cpw = (nch + nw - 1) / nw;
  return cpw <= 64 ? 1 : (cpw <= 128 ? 2 : (cpw <= 256 ? 4 : 0));
}

hipError_t launch_fill_u32(unsigned* p, int n, unsigned v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_u32, dim3((n + kBlock - 1) / kBlock), dim3(kBlock), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_pred_hidden(int pt, int at, const void* p1, const void* x, int d, int r, int B, float* h,
                              hipStream_t s) {
  if (B < 1 || B > kMaxTokens) return hipErrorInvalidValue;
  const dim3 grid((r + 3) / 4), block(kBlock);
  // Chunks of a row in flight per lane: one token, 8 (16 for rows wider than 4096, so a row is a
  // single round of loads); up to 4 tokens, 8; up to 16, 4 (x registers for 16 tokens).
  auto go = [&](auto nbc, auto uc) -> hipError_t {
    constexpr int NB = decltype(nbc)::value;
    constexpr int U = decltype(uc)::value;
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
  };
  using one = std::integral_constant<int, 1>;
  if (B == 1) return d > 4096 ? go(one{}, std::integral_constant<int, 16>{}) : go(one{}, std::integral_constant<int, 8>{});
  if (B <= 4) return go(std::integral_constant<int, 4>{}, std::integral_constant<int, 8>{});
  return go(std::integral_constant<int, 16>{}, std::integral_constant<int, 4>{});
}

hipError_t launch_ffn_group(int wt, int at, int mode, const GroupArgs& a, hipStream_t s) {
  if (a.G % 32 != 0 || a.G > kGMax || (a.nw != 4 && a.nw != 8) || a.G / a.nw > 32) return hipErrorInvalidValue;
  const int cpl = group_cpl(wt, a.d, a.nw);
  if (cpl == 0) return hipErrorInvalidValue;
  if (wt == DT_F16) return launch_ffn_group_f16(at, mode, a, cpl, s);
  if (wt == DT_F32) return launch_ffn_group_f32(at, mode, a, cpl, s);
  return launch_ffn_group_q4(at, mode, a, cpl, s);
}

// Every 16-byte unit of the buffer read once with streaming loads: each wave takes spans of
// 8 KB (8 loads of 64 lanes x 16 bytes in flight, each load one contiguous KB), the waves of the
// grid taking consecutive spans in turn.  On MI355X this sustains ~7.0 TB/s at 512-4096
// workgroups, where a grid-stride pattern (a wave's 8 loads far apart) reaches 5.2-6.6 TB/s.
// The words are summed (mod 2^32) so the reads cannot be dropped and their total can be checked.
__global__ __launch_bounds__(256) void k_read_probe(const u32x4* __restrict__ p, size_t n16,
                                                     unsigned* __restrict__ sums) {
  constexpr int kU = 8;
  const int lane = threadIdx.x & (WAVE - 1);
  const size_t wid = (size_t)blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE;
  const size_t nwv = (size_t)gridDim.x * (blockDim.x / WAVE);
  unsigned acc = 0u;
  for (size_t s0 = wid * WAVE * kU; s0 < n16; s0 += nwv * WAVE * kU) {
    u32x4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const size_t i = s0 + (size_t)u * WAVE + lane;
      v[u] = i < n16 ? ld_stream(p + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) acc += v[u].x + v[u].y + v[u].z + v[u].w;
  }
  __shared__ unsigned s_acc[256];
  s_acc[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned t = 0u;
    for (int k = 0; k < 256; ++k) t += s_acc[k];
    sums[blockIdx.x] = t;
  }
}

hipError_t launch_read_probe(const void* buf, size_t n16, unsigned* sums, int n_sums, hipStream_t s) {
  hipLaunchKernelGGL(k_read_probe, dim3(n_sums), dim3(kBlock), 0, s, static_cast<const u32x4*>(buf), n16, sums);
  return hipGetLastError();
}

hipError_t launch_finish(int ot, const float* partial, int ng, int B, int d, void* y,
                         const unsigned* mask_words, int mask_n, int iota_n, int* idx_out, int* count_out,
                         bool reduce, bool index_list, hipStream_t s) {
  const int ncol = reduce ? (d + 31) / 32 : 0;   // 32 columns per workgroup
  const int grid = ncol + (index_list ? 1 : 0);
  if (grid == 0) return hipSuccess;
  const dim3 g(grid, reduce ? B : 1);   // one row of column blocks per token
  if (ot == DT_F16)
    hipLaunchKernelGGL((k_finish<DT_F16>), g, dim3(kBlock), 0, s, partial, ng, B, d, y,
                       index_list ? mask_words : nullptr, mask_n, iota_n, idx_out, count_out, ncol);
  else
    hipLaunchKernelGGL((k_finish<DT_F32>), g, dim3(kBlock), 0, s, partial, ng, B, d, y,
                       index_list ? mask_words : nullptr, mask_n, iota_n, idx_out, count_out, ncol);
  return hipGetLastError();
}

}  // namespace pik
