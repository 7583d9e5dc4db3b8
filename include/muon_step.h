/*
 * muon_step.h — C ABI of libmuonstep, one Muon optimizer step on one AMD
 * Instinct MI355X (gfx950) GPU.
 *
 * The step follows the DeepSpeed-Muon article ("DeepSpeed 集成 Muon 优化器实战：
 * 从正交化原理到 ZeRO 微调配置"):
 *   - section "什么是 Muon 优化器？": form the momentum from the gradient, then
 *     orthogonalise the momentum matrix by Newton-Schulz iterations, then update
 *     the weights with the result; 2D hidden weights only;
 *   - section "核心算子：牛顿-舒尔茨正交化内核": the quintic iteration with
 *     a = 3.4445, b = -4.7750, c = 2.0315, five steps ("standard", stable in
 *     bf16), the variant iterating on the small Gram matrix R = X X^T in fp16
 *     ("gram"), the method set {"standard", "gram"}, decoupled weight decay
 *     p *= 1 - lr*wd followed by p -= lr * update, and the Adam(W) fallback for
 *     parameters that are not 2D;
 *   - section "如何用 DeepSpeed 配置启用 Muon": defaults (Muon lr 0.02,
 *     momentum 0.95, ns_method "gram"; Adam lr 3e-4, betas (0.9, 0.95)).
 * The input layout is the DMuon owner's packed buffer ("Z2 与 Z3 模式", section on
 * the two packed-buffer lifecycles): all Muon-target matrices of one owner in
 * one contiguous buffer; here each matrix is row-major at an element offset.
 *
 * Per matrix (or per split block, see muon_matrix_t) the step computes
 *   M <- mu * M + G                                 (fp32 momentum, in place)
 *   Y  = M, transposed if it has more rows than columns
 *   X0 = Y / (||Y||_F + ns_eps)
 *   X  = NS(X0)  (ns_steps iterations; standard: A = X X^T,
 *                 B = a I + b A + c A A, X <- B X (= a X + b A X + c A A X);
 *                 gram: R = X0 X0^T, Q = a I + b R + c R R, P <- Q P,
 *                 R <- Q R Q, X = P X0)
 *   O  = X, transposed back
 *   p <- p * (1 - lr * weight_decay) - lr * O      (params, in place)
 *
 * Conventions for every entry point:
 *   - Device pointers are HIP device memory (for example torch CUDA tensors);
 *     host pointers are ordinary memory read during the call and not retained.
 *   - `stream` is a hipStream_t passed as void* (NULL: the default stream). All
 *     device work is enqueued on it asynchronously. No call allocates device
 *     memory, copies between host and device, or synchronises the host or the
 *     device (the profiling hooks below aside): a step's per-problem
 *     descriptors are written into the caller's workspace by a kernel on the
 *     stream, from the table passed as kernel arguments. Faults in device work
 *     surface at the caller's next synchronisation.
 *   - Return value: MUON_OK or one of the MUON_ERR_* codes below. Every argument
 *     check runs before the first launch, so a call that fails a check leaves
 *     every buffer unchanged. muon_last_error() gives a message for the last
 *     failing call on the calling thread.
 *   - The caller owns all device memory, including the workspace. The library
 *     keeps only host memory: the layout it derives from each distinct table
 *     (up to 1024 of them; the first call with one more drops them all,
 *     muon_release_plans() drops them on request).
 *   - Every call enqueues kernel launches only, so any call may be captured
 *     into a HIP graph (the profiling hooks below must be off while
 *     capturing). A replay reads the workspace given at capture time, which
 *     must then stay allocated and unused by other work.
 *   - Calls that share a workspace, or that update the same buffers, must be
 *     ordered by the caller (same stream, or events).
 */
#ifndef MUON_STEP_H
#define MUON_STEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. Invalid combinations raise errors, as the article's DeepSpeed
 * integration does for unsupported configurations. */
enum {
  MUON_OK = 0,
  MUON_ERR_NULL = 1,        /* a required pointer is NULL */
  MUON_ERR_BAD_METHOD = 2,  /* ns_method is neither STANDARD nor GRAM */
  MUON_ERR_BAD_SHAPE = 3,   /* rows/cols < 1, split_rows < 0 or not dividing rows,
                               split_cols < 0 or not dividing cols, n_entries < 0,
                               or a size beyond the limits below */
  MUON_ERR_RANGE = 4,       /* offset < 0 or offset + rows*cols > numel */
  MUON_ERR_OVERLAP = 5,     /* two entries overlap, or two buffers overlap */
  MUON_ERR_ALIGN = 6,       /* an offset not a multiple of 8 elements, or a buffer
                               pointer not 16-byte aligned */
  MUON_ERR_UNSUPPORTED = 7, /* a dtype combination that is not implemented (gram
                               with bf16 storage, bf16 params with a bf16 shadow or
                               in a partition holder's step, ...) */
  MUON_ERR_WORKSPACE = 8,   /* workspace smaller than muon_workspace_size() */
  MUON_ERR_HIP = 9,         /* a HIP runtime call or kernel launch failed */
  MUON_ERR_BAD_HYPER = 10   /* a non-finite hyperparameter, ns_steps outside
                               [1, 64], or AdamW step < 1 */
};

/* Element types. */
enum { MUON_DTYPE_F32 = 0, MUON_DTYPE_BF16 = 1, MUON_DTYPE_F16 = 2 };

/* Newton-Schulz methods (the article's NS_METHODS). */
enum { MUON_NS_STANDARD = 0, MUON_NS_GRAM = 1 };

/* Size limits: min(rows, cols) of a problem <= MUON_MAX_SHORT_SIDE,
 * max(rows, cols) <= MUON_MAX_LONG_SIDE; over a whole table, the sum of
 * rows * cols <= MUON_MAX_TABLE_ELEMENTS (2^36: 275 GB of fp32 parameters
 * alone, more than one GPU holds) and the problems (whole matrices plus split
 * blocks) <= MUON_MAX_PROBLEMS. Within them every launch grid of a step fits. */
#define MUON_MAX_SHORT_SIDE 16384
#define MUON_MAX_LONG_SIDE (1 << 24)
#define MUON_MAX_TABLE_ELEMENTS (1LL << 36)
#define MUON_MAX_PROBLEMS (1 << 24)

/* One Muon-target matrix inside the packed buffers. params, grads, momentum
 * (and update_out / bf16_shadow when given) share one layout: the matrix is
 * rows x cols, row-major, starting at element `offset` (the article recovers
 * each gradient with reshape(p.shape), i.e. row-major).
 * split_rows = 0 orthogonalises the whole matrix; split_rows = k > 0 cuts it
 * into rows/k blocks of k consecutive rows, each orthogonalised on its own with
 * its own norm (the "Muon Split" per-head orthogonalisation the article's TL;DR
 * mentions). split_cols = k > 0 cuts it the same way into cols/k blocks of k
 * consecutive columns: the per-head blocks of a projection whose input side
 * holds the heads, as an attention output projection (rows x cols, y = W x)
 * does. With both set the blocks are the split_rows x split_cols tiles, taken
 * row of blocks by row of blocks. A block is read and written in place, with
 * the matrix's row pitch (cols). */
typedef struct {
  int64_t offset;
  int64_t rows;
  int64_t cols;
  int64_t split_rows;
  int64_t split_cols;
} muon_matrix_t;

/* Hyperparameters of the Muon group. Fill with muon_default_hyper() first. */
typedef struct {
  float lr;            /* default 0.02 (the article's Muon default; muon_lr overrides lr) */
  float momentum;      /* default 0.95 */
  float weight_decay;  /* default 0.0 */
  float ns_a;          /* default 3.4445 */
  float ns_b;          /* default -4.7750 */
  float ns_c;          /* default 2.0315 */
  int32_t ns_steps;    /* default 5 */
  float ns_eps;        /* default 1e-7: X0 = Y / (||Y||_F + ns_eps) */
  int32_t ns_method;   /* MUON_NS_STANDARD | MUON_NS_GRAM; default GRAM */
  int32_t param_dtype; /* MUON_DTYPE_F32 (default: fp32 master weights) | BF16 (bf16
                          weights updated in place: p <- RNE_bf16(p * (1 - lr * wd)
                          - lr * O), computed in fp32) */
  int32_t grad_dtype;  /* MUON_DTYPE_BF16 (default) | F32 | F16 */
  int32_t ns_dtype;    /* storage/operand type of the iteration: standard F32 | BF16 |
                          F16; gram F32 | F16. Default F16 (the default method is
                          gram, which the article runs in fp16; it runs standard in
                          bf16). MFMA accumulation is fp32 in every case. */
} muon_hyper_t;

/* AdamW hyperparameters (the Adam group: adam_lr overrides lr). */
typedef struct {
  float lr;            /* default 3e-4 */
  float beta1;         /* default 0.9 */
  float beta2;         /* default 0.95 */
  float eps;           /* default 1e-10 (the article's default; its example config uses 1e-8) */
  float weight_decay;  /* default 0.0 */
  int32_t step;        /* t >= 1, used for bias correction */
  int32_t grad_dtype;  /* MUON_DTYPE_BF16 (default) | F32 | F16 */
} muon_adamw_hyper_t;

/* Fill *h with the defaults listed above. */
void muon_default_hyper(muon_hyper_t* h);
void muon_default_adamw_hyper(muon_adamw_hyper_t* h);

/* Bytes of device workspace that muon_step needs for this table and these
 * hyperparameters (validates the table like muon_step, without the buffer and
 * range checks). Host-only; no device work. The workspace holds the
 * per-problem descriptors (48 bytes per problem), the per-problem norms and
 * the tile-padded iterates of every shape group. */
int muon_workspace_size(const muon_matrix_t* table, int32_t n_entries,
                        const muon_hyper_t* h, size_t* bytes_out);

/* One Muon step over the packed buffers.
 *   params      device, param_dtype[numel] (float32, or bf16 as raw 16-bit
 *               words), updated in place (entries only).
 *   grads       device, grad_dtype[numel], read only.
 *   momentum    device, float32[numel], updated in place (entries only).
 *   numel       element count of each packed buffer.
 *   table       host, n_entries descriptors; entries must not overlap and each
 *               offset must be a multiple of 8 elements.
 *   h           host, hyperparameters.
 *   workspace   device, >= muon_workspace_size() bytes, 256-byte aligned; its
 *               contents on entry do not matter and are clobbered.
 *   update_out  optional device float32[numel]: receives O (entries only).
 *   bf16_shadow optional device bf16[numel] (raw 16-bit words): receives the
 *               round-to-nearest-even bf16 copy of the new params (entries only),
 *               the form an owner broadcasts. fp32 params only (bf16 params are
 *               that copy themselves: MUON_ERR_UNSUPPORTED).
 * Elements outside the entries are never written in any output. */
int muon_step(void* params, const void* grads, float* momentum, int64_t numel,
              const muon_matrix_t* table, int32_t n_entries, const muon_hyper_t* h,
              void* workspace, size_t workspace_bytes,
              float* update_out, uint16_t* bf16_shadow, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): muon_step with its
 * workspace taken from a device array inside the library, of
 * MUON_NOALLOC_WORKSPACE_BYTES bytes, one per GPU the library runs on, held
 * until the process ends. Arguments as in muon_step, without the workspace.
 * It calls no allocating routine. A table whose muon_workspace_size() exceeds
 * the array is refused with MUON_ERR_WORKSPACE before any device work. Every
 * call on one GPU uses that GPU's one array, whose contents do not matter on
 * entry: calls that may overlap on one GPU (other streams, other threads)
 * race on it, so the caller must order them (one stream, or events). */
#define MUON_NOALLOC_WORKSPACE_BYTES (64ull << 20)
int muon_step_noalloc(void* params, const void* grads, float* momentum, int64_t numel,
                      const muon_matrix_t* table, int32_t n_entries, const muon_hyper_t* h,
                      float* update_out, uint16_t* bf16_shadow, void* stream);

/* The part of one table entry that a parameter partition holds: elements
 * [lo, hi) of the matrix flattened in stored row-major order, found in the
 * partition from index param_offset on (element e at param_offset + e - lo).
 * lo == hi holds nothing (its param_offset is then ignored). */
typedef struct {
  int64_t lo;
  int64_t hi;
  int64_t param_offset;
} muon_window_t;

/* One Muon step for a holder of one flat parameter partition, whose matrices
 * may straddle the partition's boundaries. The DeepSpeed-Muon article (ZeRO
 * stage support section, on partition boundaries) gives every rank that holds
 * part of such a matrix the whole reduced gradient before the nonlinear
 * update: here the holder keeps the whole momentum of each listed matrix,
 * runs momentum and Newton-Schulz on the whole matrix, and updates only the
 * elements of its own window. Every holder of a matrix, given the same
 * gradient and momentum, computes the same momentum and the same update, so
 * the holders' windows together equal a muon_step of the whole matrix, bit
 * for bit.
 *   partition       device float32[partition_numel], updated in place
 *                   (window elements only); h->param_dtype must be F32
 *                   (MUON_ERR_UNSUPPORTED otherwise).
 *   grads, momentum, numel, table, h, workspace: as in muon_step (the table
 *                   describes the full-matrix layout of grads and momentum;
 *                   momentum is updated for every listed matrix in full).
 *   windows         host, one per table entry; windows must lie inside the
 *                   partition and must not share a partition element.
 *   update_out      optional device float32[numel] in the table's layout:
 *                   receives O for every element of every listed matrix.
 *   bf16_shadow     optional device bf16[partition_numel]: the bf16 copy of
 *                   the new partition elements (window elements only).
 * Workspace size: muon_workspace_size() of the same table. Errors as in
 * muon_step, plus MUON_ERR_RANGE for a window outside its matrix or the
 * partition, MUON_ERR_OVERLAP for windows sharing a partition element or a
 * partition that overlaps another buffer. Windows may start and end at any
 * element; runs of 8 elements whose partition index is a multiple of 8 take
 * the vector path, the rest a scalar one. */
int muon_step_window(float* partition, int64_t partition_numel, const void* grads, float* momentum,
                     int64_t numel, const muon_matrix_t* table, const muon_window_t* windows,
                     int32_t n_entries, const muon_hyper_t* h, void* workspace,
                     size_t workspace_bytes, float* update_out, uint16_t* bf16_shadow,
                     void* stream);

/* AdamW step over a flat buffer of non-2D parameters (the article's Adam
 * fallback, AdamW mode):
 *   m <- b1 m + (1-b1) g;  v <- b2 v + (1-b2) g^2;
 *   p <- p (1 - lr wd) - lr * (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps).
 * params, m, v: device float32[numel], updated in place; grads: device
 * grad_dtype[numel]. */
int adamw_step(float* params, const void* grads, float* m, float* v, int64_t numel,
               const muon_adamw_hyper_t* h, void* stream);

/* Pack n_entries device matrices into one packed buffer of `numel` elements:
 * srcs[i] (device, rows*cols elements of `dtype`, row-major) is copied bit for
 * bit to packed + table[i].offset. Elements of `packed` outside the entries are
 * not written. `srcs` is a host array of device pointers. The table is checked
 * as in muon_step (shapes, range, 8-element offset alignment, no overlap). */
int muon_pack(void* packed, int64_t numel, const void* const* srcs, const muon_matrix_t* table,
              int32_t n_entries, int32_t dtype, void* stream);

/* The inverse of muon_pack: dsts[i] <- packed + table[i].offset, bit for bit. */
int muon_unpack(void* const* dsts, const void* packed, int64_t numel, const muon_matrix_t* table,
                int32_t n_entries, int32_t dtype, void* stream);

/* ---- Owner planning (host only, no device work) --------------------------
 * DMuon ("Z2 与 Z3 模式") gives every Muon-target matrix one owner, which alone
 * runs its Newton-Schulz and keeps the authoritative copy; an owner packs all
 * of its matrices into one contiguous buffer for the broadcast, and under
 * DMuon-Z3 one layer's packed buffer at a time is resident. The pages do not
 * say how owners are chosen. muon_plan_owners balances the nominal
 * Newton-Schulz FLOPs of the owners greedily, largest first (LPT), and lays
 * each owner's matrices out in its packed buffer, layer by layer. */

/* One Muon-target matrix of the model: stored rows x cols (row-major),
 * split_rows and split_cols as in muon_matrix_t, and the index of the layer it
 * belongs to. */
typedef struct {
  int64_t rows;
  int64_t cols;
  int64_t split_rows;
  int32_t layer;
  int32_t reserved;  /* set to 0 */
  int64_t split_cols;
} muon_param_t;

/* Where a matrix went: its owner and its element offset in that owner's
 * packed buffer (a multiple of the planning alignment). */
typedef struct {
  int32_t owner;
  int32_t reserved;
  int64_t offset;
} muon_assign_t;

/* What one owner holds. */
typedef struct {
  int64_t numel;            /* packed buffer length in elements (gaps included):
                               what DMuon-Z2 keeps resident on this rank */
  int64_t max_layer_numel;  /* longest single-layer span of the packed buffer:
                               the DMuon-Z3 transient */
  int64_t ns_flops;         /* nominal Newton-Schulz FLOPs of the owned problems */
  int32_t n_matrices;
  int32_t reserved;
} muon_owner_t;

/* Nominal Newton-Schulz FLOPs of one problem with short side m and long side
 * n, counting 2 m k n per m x k by k x n product of the iteration as this
 * library runs it, for `steps` steps. Standard: per step X X^T, A A and B X,
 * i.e. steps (4 m^2 n + 2 m^3). Gram: R0 = X X^T and the final P X0
 * (4 m^2 n), per step Q = a I + b R + c R R (2 m^3), and for every step but
 * the first P <- Q P (2 m^3), for every step but the last R <- Q R Q
 * (4 m^3): 4 m^2 n + (8 steps - 6) m^3. Returns -1 for invalid input or on
 * int64 overflow. */
int64_t muon_ns_flops(int64_t m, int64_t n, int32_t ns_method, int32_t steps);

/* Assign n_params matrices to n_owners owners and lay out each owner's packed
 * buffer.
 *   Assignment: problems' FLOPs summed per matrix (muon_ns_flops over its
 *   split blocks); matrices taken in order of decreasing FLOPs (ties: more
 *   elements first, then lower index), each given to the owner with the
 *   least FLOPs so far (ties: lower owner index).
 *   Layout: each owner's matrices in order of (layer, index), each at the
 *   next multiple of `align` elements (align >= 8 and a multiple of 8), so
 *   each layer's matrices form one contiguous span.
 *   assign   host, n_params records (out).
 *   owners   host, n_owners records (out).
 * Errors: MUON_ERR_NULL, MUON_ERR_BAD_SHAPE (a shape muon_step would reject,
 * n_params < 0, n_owners < 1, layer < 0), MUON_ERR_ALIGN (bad align),
 * MUON_ERR_BAD_METHOD, MUON_ERR_BAD_HYPER (steps outside [1, 64]),
 * MUON_ERR_RANGE (int64 overflow). Nothing is written on error. */
int muon_plan_owners(const muon_param_t* params, int32_t n_params, int32_t n_owners,
                     int32_t ns_method, int32_t ns_steps, int64_t align,
                     muon_assign_t* assign, muon_owner_t* owners);

/* Elements sent per step on the shard group of n_ranks ranks, for P_M
 * Muon-target elements ("Z2 与 Z3 模式", section on per-step communication):
 * k (n_ranks - 1) / n_ranks * P_M with k = 2 for DMuon-Z2, 3 for DMuon-Z3,
 * 3 for Muon on FSDP2-Z2 without dedicated owners, 4 on FSDP2-Z3.
 *   zero_stage  2 or 3; dedicated 1 (DMuon) or 0 (no owners).
 * Multiply by the element size of the wire format for bytes. Returns a
 * negative value for invalid input. */
double muon_comm_elements(int64_t p_m, int32_t n_ranks, int32_t zero_stage, int32_t dedicated);

/* Message for the last failing call on this thread ("" if none). Valid until the
 * next call on this thread. */
const char* muon_last_error(void);

/* Drop the cached per-table host layouts (host memory only; no device work, no
 * synchronisation). Later calls rebuild them on demand. */
int muon_release_plans(void);

/* Kernel timing for measurement. Between muon_profile_begin() and
 * muon_profile_end(), every launch made by this library is bracketed with HIP
 * events on the stream it is launched on. muon_profile_end() waits for those
 * events and reports, per kernel kind, the number of launches and the summed
 * duration in milliseconds (at most `max_kinds` records). Not thread-safe
 * against concurrent muon_step calls on other threads. */
typedef struct {
  char name[48];
  int32_t launches;
  double total_ms;
} muon_kernel_stat_t;

int muon_profile_begin(void);
int muon_profile_end(muon_kernel_stat_t* out, int32_t max_kinds, int32_t* n_kinds_out);

/* Library version string. */
const char* muon_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MUON_STEP_H */
