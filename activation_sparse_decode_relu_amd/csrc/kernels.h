// Host-side launch interface of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace pik {

enum : int { MODE_PRED = 0, MODE_EXACT = 1, MODE_DENSE = 2, MODE_LIST = 3 };

constexpr int kMaxTokens = 16;        // one MFMA token tile: the predictor, vector and union paths
constexpr int kMaxBatchTokens = 64;   // the matrix-core path in exact and dense modes (four tiles)

// Everything one k_ffn_group launch reads and writes (passed by value).
struct GroupArgs {
  const void* w_gate;
  const void* w_up;
  const void* w_down_t;
  const _Float16* s_gate;
  const _Float16* s_up;
  const _Float16* s_down;
  const float* b;
  const void* p2;          // predictor second layer [n][r] (MODE_PRED)
  const float* b_p;        // predictor bias [n] (MODE_PRED)
  const float* h;          // predictor hidden [B][r] (MODE_PRED)
  const void* x;           // [B][d]
  const int* list;         // MODE_LIST: caller's ascending neuron ids
  const int* list_count;   // MODE_LIST: device int
  float* logits;           // MODE_PRED, optional: z [B][n]
  unsigned* mask_words;    // MODE_PRED / MODE_EXACT: [ceil(n/32)], bit b of word w = neuron 32w+b
  float* partial;          // [groups][B][d]
  float thr;
  int p_dtype, d, n, r, B, G, nw, gated, mask_only;
  const unsigned* hot_words;  // MODE_PRED, one-token split path, optional: bit i = neuron i always computed
};

// Chunks per lane of a wave's d-slice with nw waves per workgroup (1, 2 or 4), or 0 if d is too large.
int group_cpl(int wt, int d, int nw);

hipError_t launch_fill_u32(unsigned* p, int n, unsigned v, hipStream_t s);

hipError_t launch_pred_hidden(int pt, int at, const void* p1, const void* x, int d, int r, int B, float* h,
                              hipStream_t s);

hipError_t launch_ffn_group(int wt, int at, int mode, const GroupArgs& a, hipStream_t s);

// The batched matrix-core path (2..16 tokens with fp16 weights, activations and predictor, every
// mode; 17..64 tokens exact and dense): k_ffn_bgroup writes the mask words and
// a[neuron][16 batch_tiles(B)] (fp32) into abuf; k_ffn_bdown writes batch_down_chunks(d) partials
// of y.
bool batch_supported(int wt, int at, int pt, int B, int d, int r);
// 17 to 64 tokens (exact and dense modes): fp16 weights and activations, d a multiple of 128.
bool batch_large_supported(int wt, int at, int B, int d);
int batch_tiles(int B);   // 16-token tiles of a batch: 1, 2 or 4
int batch_groups(int n);
int batch_down_chunks(int d);
hipError_t launch_ffn_bgroup(int mode, const GroupArgs& a, float* abuf, hipStream_t s);
hipError_t launch_ffn_bdown(int mode, const GroupArgs& a, const float* abuf, int chunks, hipStream_t s);


// The one-token split path (fp16 activations, fp16 or int4 weights, fp16 predictor, batch 1):
// k_act writes the mask bits and a[neuron] (fp32) into abuf; k_down sums a * W_down^T rows over
// (column slice, list chunk) tiles, the last tile of each slice adding the chunks' partials into
// y, and writes the index list.
struct DownArgs {
  const float* abuf;        // a[neuron], fp32
  const void* w_down_t;     // [n][d] rows
  const _Float16* s_down;   // int4: fp16 [n][d/32]
  const unsigned* mask;     // MODE_PRED / MODE_EXACT
  const int* list;          // MODE_LIST
  const int* list_count;    // MODE_LIST
  float* partial;           // [chunks][d]
  unsigned* tickets;        // [slices * kTicketStride], zero between calls
  void* y;                  // [d] act dtype (fp16)
  int* idx_out;             // optional
  int* count_out;           // optional
  int n, d, chunks, do_down;
};
constexpr int kMaxDnChunks = 32;   // list chunks per column slice (partials the last tile adds)
constexpr int kTicketStride = 64;  // one ticket per 256 bytes: tickets of different slices share no line
constexpr int kMaxDnSlices = 16;   // column slices of the split path's widest rows (fp16, d = 8192)
bool split_supported(int wt, int at, int pt, int B, int d, int r, int n);
int split_slices(int wt, int d);
int split_chunks(int wt, int d);
hipError_t launch_act(int wt, int mode, const GroupArgs& a, float* abuf, hipStream_t s);
hipError_t launch_down(int wt, int mode, const DownArgs& D, hipStream_t s);

// Read-bandwidth probe: n16 16-byte units of buf, summed as 32-bit words (mod 2^32) into
// sums[n_sums], one sum per workgroup.
hipError_t launch_read_probe(const void* buf, size_t n16, unsigned* sums, int n_sums, hipStream_t s);

hipError_t launch_finish(int ot, const float* partial, int ng, int B, int d, void* y,
                         const unsigned* mask_words, int mask_n, int iota_n, int* idx_out, int* count_out,
                         bool reduce, bool index_list, hipStream_t s);

}  // namespace pik
