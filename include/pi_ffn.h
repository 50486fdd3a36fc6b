/*
 * pi_ffn.h -- C ABI of the activation-sparse ReLU FFN decode library (gfx950).
 *
 * One FFN layer of single-token (or small-batch) decode, computed only over the
 * neurons that fire:
 *
 *   FFN(x) = ReLU(x W_gate^T + b) (.) (x W_up^T) W_down          (gated)
 *   FFN(x) = ReLU(x W_up^T + b) W_down                          (non-gated)
 *
 * The FFN statement is the one in the PowerInfer paper explainer
 * (0h-n0.github.io, "PowerInfer - コンシューマGPUでの高速LLM推論エンジン"),
 * section "ニューロン活性化のべき乗則分布", FFN equation, with sigma = ReLU
 * (the ReLU-sparse models named on the PowerInfer project page, section
 * "サポートするモデル").  Which neurons are computed comes from one of three
 * masks: the activation predictor (same explainer, section "活性化予測器":
 * sigmoid(x W_p + b_p) > tau, here a rank-r two-layer ReLU MLP), the exact
 * ReLU support, or every neuron.  Only selected neurons are computed (same
 * explainer, section "GPU-CPUハイブリッドアーキテクチャ", inference flow; paper
 * summary gptget.net "PowerInfer: Fast Large Language Model Serving with a
 * Consumer-grade GPU", "Methodology": neuron-aware sparse operators).
 *
 * Conventions common to every call
 * --------------------------------
 * - Shapes: d = d_model, n = d_ffn, r = rank, B = tokens in the batch.
 * - Every matrix is neuron-major and row-contiguous: W_gate, W_up [n][d];
 *   the down projection is passed TRANSPOSED as W_downT [n][d], so row i holds
 *   neuron i's down weights.  P1 [r][d], P2 [n][r].  x and y are [B][d].
 * - dtypes: act (x, y) f32 or f16; weights f32, f16 or q4g32; predictor f32
 *   or f16; b and b_p are always f32.  All accumulation is f32.
 * - q4g32: each row is d/2 bytes, byte j holding element 2j in bits 0-3 and
 *   element 2j+1 in bits 4-7 as 4-bit two's complement; scales are fp16
 *   [n][d/32], one per 32 consecutive elements; value = q * s.
 * - A batch shares one mask: the union of the per-token masks.  Past 16 tokens
 *   (max_batch up to 64) that union covers most of a layer, so every row is read
 *   anyway: a PREDICTED call then runs as EXACT_RELU, without the predictor
 *   (pi_ffn_forward), and predict / forward_masked take at most 16 tokens.
 * - Index lists are int32, strictly ascending, unique; the count is one int32.
 *   Both live in device memory and are never copied to the host.
 * - Ownership: the caller allocates ALL device memory (weights, x, y, index
 *   buffers, workspace).  The library never allocates device memory; its only
 *   host allocation is the handle.  A handle borrows the weight and workspace
 *   pointers until pi_ffn_destroy.  (pi_ffn_forward_static works instead in a
 *   file-scope device array of the library, PI_FFN_STATIC_SCRATCH_BYTES per GPU.)
 * - Streams: calls only enqueue work on `stream` (a hipStream_t passed as
 *   void*, NULL = the null stream) and return without synchronising.  A
 *   handle is not safe for concurrent use from two streams: it shares its
 *   workspace between calls.  Handles whose calls are serialised on one
 *   stream may share one workspace (e.g. the layers of a model).
 * - Errors: every call returns a pi_status.  Arguments are validated on the
 *   host before anything is enqueued; PI_ERR_INVALID means nothing was
 *   enqueued.  PI_ERR_HIP reports a launch failure (or an earlier
 *   asynchronous fault surfacing at launch).  pi_last_error() returns a
 *   thread-local message for the last failing call on this thread.
 * - Pointers: weights, scales, biases, x, y and logits must be 16-byte
 *   aligned; index lists and counts 4-byte aligned.
 */
#ifndef PI_FFN_H
#define PI_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PI_FFN_ABI_VERSION 8

/* Bytes of the device scratch array pi_ffn_forward_static works in, one per GPU. */
#define PI_FFN_STATIC_SCRATCH_BYTES (16u << 20)

typedef enum pi_status {
  PI_OK = 0,
  PI_ERR_INVALID = 1,     /* bad argument; nothing enqueued */
  PI_ERR_WORKSPACE = 2,   /* workspace missing or smaller than pi_ffn_workspace_bytes */
  PI_ERR_HIP = 3,         /* HIP runtime error at launch */
  PI_ERR_UNSUPPORTED = 4  /* valid request the library does not implement */
} pi_status;

typedef enum pi_dtype { PI_F32 = 0, PI_F16 = 1, PI_Q4G32 = 2 } pi_dtype;

typedef enum pi_mask_mode {
  PI_MASK_PREDICTED = 0,  /* predictor mask, then the sparse operator            */
  PI_MASK_EXACT_RELU = 1, /* mask = {i : pre-activation > 0} from a dense pass    */
  PI_MASK_DENSE = 2       /* every neuron, no predictor                          */
} pi_mask_mode;

/* Kernels a profiling event pair can bracket (pi_ffn_profile_next). */
typedef enum pi_phase {
  PI_PHASE_PRED_HIDDEN = 0, /* h = ReLU(x P1^T)                                        */
  PI_PHASE_GROUP = 1,       /* the mask and the gate/up row gather with a = ReLU(g)*u:
                               one token (fp16 activations, fp16 or int4 rows): k_act;
                               2..64 tokens on the matrix cores: k_ffn_bgroup; otherwise
                               k_ffn_group, which also forms each group's partial y     */
  PI_PHASE_DOWN = 2,        /* the down projection over (column slice, neuron chunk)
                               tiles from the activations: one token, k_down (which also
                               sums the partials into y and writes the index list);
                               matrix-core batches, k_ffn_bdown                          */
  PI_PHASE_FINISH = 3,      /* fixed-order sum of the partials; index list (every path
                               but the one-token k_act / k_down path)                    */
  PI_PHASE_COUNT = 4
} pi_phase;

typedef struct pi_ffn_desc {
  int32_t d_model;   /* d: > 0, multiple of 64                                  */
  int32_t d_ffn;     /* n: > 0                                                  */
  int32_t rank;      /* r: predictor rank, 0 = no predictor, else multiple of 64 */
  int32_t gated;     /* 1 = gated (W_gate present), 0 = non-gated               */
  int32_t max_batch; /* 1..64: largest B any call will pass; above 16 only with
                        fp16 weights and activations and d a multiple of 128       */
  int32_t w_dtype;   /* pi_dtype of W_gate, W_up, W_downT                       */
  int32_t p_dtype;   /* PI_F32 or PI_F16: dtype of P1 and P2                     */
  int32_t act_dtype; /* PI_F32 or PI_F16: dtype of x and y                       */
  float tau;         /* predictor threshold on sigmoid(z), 0 < tau < 1          */
} pi_ffn_desc;

typedef struct pi_ffn_weights {
  const void* w_gate;   /* [n][d] (q4g32: [n][d/2] bytes); NULL iff non-gated   */
  const void* w_up;     /* [n][d]                                               */
  const void* w_down_t; /* [n][d], row i = neuron i's down weights              */
  const void* s_gate;   /* fp16 [n][d/32] iff q4g32 and gated, else NULL        */
  const void* s_up;     /* fp16 [n][d/32] iff q4g32, else NULL                  */
  const void* s_down;   /* fp16 [n][d/32] iff q4g32, else NULL                  */
  const float* b;       /* [n] bias on the gate (gated) or on up (non-gated)    */
  const void* p1;       /* [r][d] predictor first layer; NULL iff rank == 0     */
  const void* p2;       /* [n][r] predictor second layer; NULL iff rank == 0    */
  const float* b_p;     /* [n] predictor output bias; NULL iff rank == 0        */
} pi_ffn_weights;

typedef struct pi_ffn pi_ffn;

/* ABI version this library was built with (PI_FFN_ABI_VERSION). */
int32_t pi_ffn_abi_version(void);

/* Thread-local message of the last failing call on this thread ("" if none). */
const char* pi_last_error(void);

/* Bytes of device workspace a handle with this descriptor needs.  Host only. */
pi_status pi_ffn_workspace_bytes(const pi_ffn_desc* desc, size_t* bytes);

/*
 * Validate the descriptor and weights, bind them and the workspace to a new
 * handle, and clear the workspace's counters with a kernel on `stream`,
 * waiting for it before returning.  `workspace` is device memory of at least
 * pi_ffn_workspace_bytes(desc) bytes, 256-byte aligned.  The weights are one FFN layer
 * (paper explainer, section "ニューロン活性化のべき乗則分布", FFN equation) plus its predictor
 * (section "活性化予測器"), laid out as the conventions above state.
 */
pi_status pi_ffn_create(const pi_ffn_desc* desc, const pi_ffn_weights* weights,
                        void* workspace, size_t workspace_bytes, void* stream,
                        pi_ffn** out);

/* Release the handle (host memory only; borrowed device memory is untouched). */
pi_status pi_ffn_destroy(pi_ffn* h);

/*
 * Predictor and compaction alone: the activation predictor of the paper explainer, section
 * "活性化予測器" (sigmoid(x W_p + b_p) > tau, read as a rank-r two-layer ReLU MLP; sigmoid(z) > tau
 * is tested as z > log(tau/(1-tau))), and the list of neurons it selects, which the same page's
 * inference flow (section "GPU-CPUハイブリッドアーキテクチャ") computes next.  For x [B][d]:
 *   h = ReLU(x P1^T), z = h P2^T + b_p, selected_i = OR_t (z[t][i] > log(tau/(1-tau))),
 * and writes idx[0..count) = ascending selected neurons (capacity n), *count.
 * logits_dbg, if not NULL, receives z as f32 [B][n].  Requires rank > 0 and B <= 16
 * (PI_ERR_UNSUPPORTED above).
 */
pi_status pi_ffn_predict(pi_ffn* h, const void* x, int32_t batch, int32_t* idx,
                         int32_t* count, float* logits_dbg, void* stream);

/*
 * The whole step, the paper explainer's FFN equation (section "ニューロン活性化のべき乗則分布")
 * computed only over the neurons a mask selects (section "GPU-CPUハイブリッドアーキテクチャ",
 * inference flow; paper summary, "Methodology": neuron-aware sparse operators): mask (per
 * mask_mode: the predictor of section "活性化予測器", the exact ReLU support, or every neuron),
 * compaction, the gathered activation a = ReLU(g) (.) u over the selected neurons only, and
 * y[t] = sum over selected i of a[t][i] * W_downT[i], rounded once to act dtype.
 * idx_out (capacity n) and count_out, if not NULL, receive the index list.
 * With no neuron selected, y is +0.0.  Above 16 tokens a PREDICTED call runs as EXACT_RELU:
 * the union of the per-token masks covers most of the layer by then (the explainer's power-law
 * firing makes a few neurons fire for almost every token and the rest at random), so the
 * predictor would save no rows; idx is then the union of the exact ReLU supports.  Above 16
 * tokens the down projection also takes each a as two fp16 parts, hi = fp16(a) and
 * lo = fp16(a - hi), with exact products and f32 accumulation (about 22 of a's 24 bits); a
 * 32-neuron step holding an |a| of 2^15 or more keeps f32.
 */
pi_status pi_ffn_forward(pi_ffn* h, const void* x, int32_t batch, int32_t mask_mode,
                         void* y, int32_t* idx_out, int32_t* count_out, void* stream);

/*
 * The neuron-aware sparse operator alone (paper summary, "Methodology"; paper explainer, section
 * "GPU-CPUハイブリッドアーキテクチャ", inference flow step 2) on a caller-given list: idx[0..*count)
 * must be strictly ascending neuron ids in [0, n) (the list is read on the device and not
 * validated; an entry outside [0, n) contributes nothing), 0 <= *count <= n.  Computes the same
 * y as pi_ffn_forward for that list.  count == 0 writes +0.0.  B <= 16 (PI_ERR_UNSUPPORTED
 * above).
 */
pi_status pi_ffn_forward_masked(pi_ffn* h, const void* x, int32_t batch, const int32_t* idx,
                                const int32_t* count, void* y, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid it): pi_ffn_forward without a handle or a caller workspace.  It
 * works in a file-scope device array of PI_FFN_STATIC_SCRATCH_BYTES bytes, one per GPU, held
 * until the process ends, and allocates nothing (no hipMalloc, no host allocation).  desc and
 * weights are validated as by pi_ffn_create; a descriptor whose pi_ffn_workspace_bytes exceeds
 * PI_FFN_STATIC_SCRATCH_BYTES returns PI_ERR_WORKSPACE before anything is enqueued.  Every call
 * on one GPU shares that GPU's array, which keeps the last call's contents; the call clears what
 * must start at zero itself.  Calls that overlap on one GPU (two streams, or two threads) race
 * on the array and give wrong results: serialise them.  Otherwise as pi_ffn_forward.
 */
pi_status pi_ffn_forward_static(const pi_ffn_desc* desc, const pi_ffn_weights* weights, const void* x,
                                int32_t batch, int32_t mask_mode, void* y, int32_t* idx_out,
                                int32_t* count_out, void* stream);

/*
 * Measurement aid, not part of the FFN: reads `bytes` of device memory at buf once with
 * streaming 16-byte loads and writes the sum (mod 2^32) of the 32-bit words each of n_sums
 * workgroups read to sums[0..n_sums), so the reads cannot be dropped and their total can be
 * checked.  Timing it gives the read bandwidth this GPU sustains.  buf 16-byte aligned, bytes a
 * multiple of 16, 1 <= n_sums <= 65536.
 */
pi_status pi_probe_read(const void* buf, size_t bytes, uint32_t* sums, int32_t n_sums, void* stream);

/*
 * Hot set: declare the neurons of this handle's layer that are computed on every PREDICTED-mode
 * call whatever the predictor says; the predictor decides the rest, and the hot neurons' P2 rows
 * are never read.  The paper explainer's offline profiling (section "オフラインプロファイリング")
 * counts how often each neuron fires on calibration inputs and sorts the neurons by that count;
 * the project page ("コア技術原理") and the paper summary ("Key Results") describe the few hot
 * neurons that fire on almost every input.  The neurons stay where they are: moving the hot ones
 * to the front would give a few waves all of them.  hot_words is device memory, ceil(n / 32)
 * uint32 words, bit b of word w = neuron 32 w + b (bits of neurons >= n ignored), borrowed until
 * the next call of this function or pi_ffn_destroy; NULL clears the set.  PREDICTED mode then
 * selects hot neurons joined with {i : z_i > log(tau/(1-tau))}; predict() writes +inf as the hot
 * neurons' logits.  Other modes are unaffected.  A set needs rank > 0 and the one-token path
 * (max_batch 1, fp16 activations and predictor, fp16 rows with d a multiple of 512 up to 8192 or
 * int4 rows with d a multiple of 2048 up to 8192), else PI_ERR_UNSUPPORTED.  Host only; takes
 * effect from the next call.
 */
pi_status pi_ffn_set_hot(pi_ffn* h, const uint32_t* hot_words);

/*
 * Which kernels pi_ffn_forward(h, x, batch, mask_mode, ...) launches, for profiling and
 * byte accounting: bit p of *plan is set when phase p's kernel runs (pi_phase).  Host
 * only; enqueues nothing.  Returns PI_ERR_INVALID for a NULL handle or plan, a batch
 * outside [1, max_batch], an unknown mask mode, or PREDICTED without a predictor.
 */
pi_status pi_ffn_launch_plan(const pi_ffn* h, int32_t batch, int32_t mask_mode, uint32_t* plan);

/*
 * Profiling: arm a one-shot event pair.  The next launch of `phase`'s kernel
 * by this handle is bracketed by hipEventRecord(start_event) and
 * hipEventRecord(stop_event) on the launch stream; then the pair disarms.
 * The elapsed time covers the launch from dispatch to completion.  Meant for
 * eager calls: under stream capture HIP treats event records as capture
 * dependencies, not timed nodes.  Events are hipEvent_t passed as void*.
 * NULL events disarm.
 */
pi_status pi_ffn_profile_next(pi_ffn* h, int32_t phase, void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif

#endif /* PI_FFN_H */
