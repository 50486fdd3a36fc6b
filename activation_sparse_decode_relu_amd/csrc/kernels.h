// Host-side launch interface of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace pik {

enum : int { GM_GATED = 0, GM_NONGATED = 1, GM_EXACT_GATED = 2 };
enum : int { ASRC_A = 0, ASRC_GRELU = 1 };

// Output columns owned by one down-projection workgroup.
int down_tile_width(int wt);

hipError_t launch_fill_u32(unsigned* p, int n, unsigned v, hipStream_t s);

hipError_t launch_pred_hidden(int pt, int at, const void* p1, const void* x, int d, int r, int B, float* h,
                              hipStream_t s);

hipError_t launch_rows_mask(int wt, int vt, const void* rows, const void* scales, const void* vec, int K, int n,
                            const float* bias, float thr, int B, float* vals_out,
                            unsigned long long* mask_words, unsigned* ticket, int* idx_out, int* count_out,
                            hipStream_t s);

hipError_t launch_gather(int wt, int at, int gm, const void* w_gate, const void* w_up, const void* s_gate,
                         const void* s_up, const float* bias, const float* g_ws, const void* x, int d, int n,
                         int B, const int* idx, const int* count, int dense, float* a_ws, int* iota_out,
                         int* count_out, int grid, hipStream_t s);

hipError_t launch_down(int wt, int ot, int asrc, const void* w_down_t, const void* s_down, const float* a_ws,
                       const float* g_ws, int d, int n, int B, const int* idx, const int* count, int dense,
                       int S, float* partial, unsigned* tickets, void* y, hipStream_t s);

}  // namespace pik
