/*
 * dmuon.h -- C ABI of the owner-side Muon step for MI355X (gfx950).
 *
 * The operation is the step that the DMuon Training Guide ("Step 4: Create
 * Optimizer") assigns to the owner of each dedicated matrix parameter:
 * momentum, then Newton-Schulz orthogonalisation, then the update.  The FAQ
 * ("Why isn't DMuon just ZeRO-1?") explains why it runs on whole (m, n)
 * matrices on one rank.  The hyperparameters and their defaults are the
 * Training Guide's dmuon.Muon arguments and its "Hyperparameter Guide" table:
 *   lr 0.02 (scaled per matrix by 0.2*sqrt(max(m, n))), momentum 0.95,
 *   nesterov true (NS input = grad + momentum*buf), ns_steps 5,
 *   weight_decay 0.0, ns_backend "gram" (default) or "direct".
 *
 * Conventions for every entry point:
 *   - Matrices are row-major and contiguous, rows x cols as stored.
 *   - Pointers named "device" are device memory of the current HIP device;
 *     the library reads and writes them only from kernels enqueued on
 *     `stream` (a hipStream_t; NULL is the default stream).  Host structs
 *     and arrays passed in are read before the call returns.
 *   - The caller owns every buffer, including the workspace.  No entry point
 *     allocates or frees device memory.  (The library keeps pinned host
 *     images of its launch tables, cached per workspace, plan and pointer
 *     set, and a shape-keyed plan cache; on each device it creates, once,
 *     one stream and a few events of its own, which a small batch uses to
 *     run two groups of matrices concurrently.)
 *   - Calls are asynchronous: results are visible to later work on `stream`.
 *     Calls that share a workspace must be ordered on one stream.  A call
 *     uploads its launch table into the workspace with a kernel that reads
 *     the pinned image when it runs, and a later call may refill that image,
 *     so these entry points must not be captured into a HIP graph for
 *     replay (dmuon_clip_grad_norm_noalloc, whose tables travel as kernel
 *     arguments, may be).
 *   - Return value: DMUON_OK, or a negative status.  Every argument check runs
 *     before the first launch, so on an error status nothing was modified.
 *     dmuon_last_error() gives a readable detail for the calling thread.
 *   - Gradient values are not checked: a NaN or Inf in one matrix's gradient
 *     propagates into that matrix only.
 *   - Threads: entry points may be called from several host threads; calls
 *     enqueued on different streams must use different workspaces.
 *   - Environment: DMUON_GEMM_TILE=128 or 256 forces the tile edge of the
 *     bf16 NS products (default: 256 for large batches, 128 otherwise), and
 *     DMUON_GEMM_TILE_F32=64 or 128 that of the fp32 ones (default: 128 for
 *     large batches, 64 otherwise); each changes the workspace size and the
 *     summation order, not the method.
 */
#ifndef DMUON_H
#define DMUON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DMUON_ABI_VERSION 1

/* status codes */
#define DMUON_OK                  0
#define DMUON_ERR_INVALID_ARG    (-1)  /* NULL pointer, bad size, bad hyperparameter */
#define DMUON_ERR_UNSUPPORTED    (-2)  /* dtype combination or device not supported   */
#define DMUON_ERR_WORKSPACE      (-3)  /* workspace NULL or smaller than required     */
#define DMUON_ERR_ALIASING       (-4)  /* two buffers overlap (the Training Guide's
                                          "Semantic Param Groups" rejects duplicate
                                          parameters the same way)                    */
#define DMUON_ERR_HIP            (-5)  /* a HIP runtime call or launch failed          */

typedef enum { DMUON_F32 = 0, DMUON_BF16 = 1 } dmuon_dtype_t;

/* Training Guide, Hyperparameter Guide table, ns_backend row. */
typedef enum { DMUON_NS_GRAM = 0, DMUON_NS_DIRECT = 1 } dmuon_ns_backend_t;

/* Arithmetic of the NS products: bf16 operands with fp32 accumulation, or
 * fp32 operands with fp32 accumulation. */
typedef enum { DMUON_NS_PREC_BF16 = 0, DMUON_NS_PREC_F32 = 1 } dmuon_ns_prec_t;

/* One owned matrix (the Training Guide's DedicatedParam, owner side). */
typedef struct {
  int64_t rows, cols;      /* as stored; both in 1 .. 2^22                        */
  void* param;             /* device, rows*cols of param_dtype, updated in place  */
  const void* grad;        /* device, rows*cols of grad_dtype; NULL skips the
                              matrix for this step (nothing of it is touched)     */
  float* momentum;         /* device, rows*cols fp32 momentum buffer, in/out;
                              zero before the first step                          */
  int32_t param_dtype;     /* dmuon_dtype_t */
  int32_t grad_dtype;      /* dmuon_dtype_t */
} dmuon_matrix_t;

/* Hyperparameters of one parameter group (Training Guide, Step 4 and the
 * Hyperparameter Guide table).  Use one call per group. */
typedef struct {
  double lr;               /* 0.02; the update is scaled by lr*0.2*sqrt(max(rows,cols)) */
  double momentum;         /* 0.95                                                 */
  int32_t nesterov;        /* 1: NS input = grad + momentum*buf (buf after its
                              update); 0: NS input = buf                          */
  int32_t ns_steps;        /* 5; 0..16                                             */
  double weight_decay;     /* 0.0; decoupled: W <- W*(1 - lr*weight_decay) first    */
  int32_t ns_backend;      /* dmuon_ns_backend_t, default DMUON_NS_GRAM            */
  int32_t ns_precision;    /* dmuon_ns_prec_t, default DMUON_NS_PREC_BF16          */
  const double* ns_coeffs; /* host; NULL: (3.4445, -4.7750, 2.0315) every step;
                              else ns_coeffs_len values: one (a, b, c) triple for
                              every step, or ns_steps triples (per-step table),
                              the dmuon.NewtonSchulz(...) custom-coefficient case */
  int32_t ns_coeffs_len;   /* 0, 3 or 3*ns_steps                                   */
  double eps;              /* 1e-7, added to the Frobenius norm of the NS input    */
} dmuon_hparams_t;

/* Fill *hp with the Training Guide's defaults (and eps 1e-7, bf16 NS). */
void dmuon_hparams_default(dmuon_hparams_t* hp);

/*
 * The whole step for a batch of n owned matrices (Training Guide, Step 4:
 * "momentum + NS + update, owner only"):
 *   buf <- momentum*buf + grad
 *   U   <- grad + momentum*buf  (nesterov) | buf
 *   X0  <- U / (||U||_F + eps), taken in the wide orientation (transposed
 *          when rows > cols)
 *   O   <- ns_steps Newton-Schulz iterations of X0 (direct or Gram form),
 *          oriented back to rows x cols
 *   W   <- W*(1 - lr*weight_decay) - lr*0.2*sqrt(max(rows,cols))*O, rounded
 *          once (to nearest even) to the parameter dtype.
 * Supported dtypes: param fp32 or bf16; grad fp32 or bf16; momentum fp32.
 * `workspace` (device, >= dmuon_step_workspace_size bytes, 256-byte aligned)
 * holds the NS intermediates; its contents on entry do not matter.
 * Matrices with the same shape need not be adjacent; each matrix is
 * independent of the others.  n == 0 is a no-op.
 */
size_t dmuon_step_workspace_size(const dmuon_matrix_t* mats, int32_t n,
                                 const dmuon_hparams_t* hp);
int dmuon_step(const dmuon_matrix_t* mats, int32_t n, const dmuon_hparams_t* hp,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * dmuon_step with the gradient clipping of the Training Guide ("Gradient
 * Clipping": the dedicated gradients are clipped after their reduce and
 * before momentum and Newton-Schulz) folded into the momentum pass: matrix
 * i's gradient is read as g * (*grad_scale[i]), the fp64 product rounded
 * once to the gradient's dtype -- the values dmuon_clip_grad_norm would
 * have written in place -- so that dmuon_clip_coefficients followed by this
 * call gives the bit-identical parameters and momenta of dmuon_clip_grad_norm
 * followed by dmuon_step, without the clip's read-and-write pass over the
 * gradients.  The gradients themselves are not modified.
 *   grad_scale  host array of n pointers, each to one double in device
 *               memory (e.g. into dmuon_clip_coefficients' coef_out), or
 *               NULL for a matrix that is not scaled; the array itself must
 *               not be NULL when n > 0
 * Everything else as dmuon_step (same workspace size).
 */
int dmuon_step_scaled(const dmuon_matrix_t* mats, int32_t n, const dmuon_hparams_t* hp,
                      const double* const* grad_scale, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * The momentum stage alone (the Hyperparameter Guide's momentum and nesterov
 * rows): updates every matrix's momentum buffer in place and writes the NS
 * input U of matrix i to ns_input[i] (device), dense and row-major in the wide
 * orientation: min(rows,cols) x max(rows,cols), i.e. transposed when
 * rows > cols, in ns_input_dtype (fp32 or bf16, rounded to nearest even).
 * sumsq (device, n doubles) receives sum(U*U) of the fp32 values before any
 * rounding.  The parameters are not read or written.  Matrices with a NULL
 * grad are skipped (their ns_input and sumsq entries are left untouched).
 * `workspace` (device, >= dmuon_momentum_workspace_size bytes) holds the
 * launch table and the per-block partial sums.
 */
size_t dmuon_momentum_workspace_size(const dmuon_matrix_t* mats, int32_t n);
int dmuon_momentum(const dmuon_matrix_t* mats, int32_t n, const dmuon_hparams_t* hp,
                   void* const* ns_input, int32_t ns_input_dtype, double* sumsq,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Newton-Schulz alone: out[i] = NS(in[i]) for n matrices of rows[i] x cols[i]
 * (host arrays), with in/out device buffers of io_dtype (fp32 or bf16) in the
 * stored orientation.  Uses hp->ns_steps, ns_backend, ns_precision,
 * ns_coeffs and eps; the momentum and update fields are ignored.
 * The backend "gram" runs the Gram form (FAQ, "What related work should I
 * cite?": Gram Newton-Schulz) on matrices with max(rows,cols) >= 2*min(rows,
 * cols) and the direct form on squarer ones, where the two cost the same and
 * the Gram form loses accuracy in bf16; dmuon_backend_info() states the rule.
 * in and out may be the same buffer.
 */
size_t dmuon_orthogonalize_workspace_size(const int64_t* rows, const int64_t* cols,
                                          int32_t n, const dmuon_hparams_t* hp);
int dmuon_orthogonalize(const void* const* in, void* const* out, const int64_t* rows,
                        const int64_t* cols, int32_t n, int32_t io_dtype,
                        const dmuon_hparams_t* hp, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * Newton-Schulz of matrices held as tensor-parallel shards (FAQ, "Does DMuon
 * work with Tensor Parallelism?": the Gram Newton-Schulz iteration of a TP
 * sharded matrix exchanges only Gram matrices, by all-reduce, whose size is
 * the square of the unsplit dimension).  On one device this runs every
 * shard's part of that scheme; the sum of the per-shard partial Gram
 * matrices stands in for the all-reduce.
 * Matrix i is mats[i].nshards contiguous blocks of one logical matrix U,
 * split along one dimension:
 *   split = 1: column blocks; every shard has the same rows d, U = [U_0 | U_1 | ...]
 *   split = 0: row blocks; every shard has the same cols d, U = [U_0; U_1; ...]
 * With X_i the shard with d as its rows (U_i, or U_i^T for row blocks) and
 * D the sum of the shards' other dimension:
 *   X0_i = X_i / (||U||_F + eps)       (||U||_F over all shards)
 *   Gram form (backend "gram" and D >= 2d): R = sum_i X0_i X0_i^T, the d x d
 *     iteration of dmuon_orthogonalize's Gram form, O_i = Q X0_i;
 *   direct form (otherwise): every iteration A = sum_i X_i X_i^T,
 *     B = bA + cA^2, X_i <- a X_i + B X_i;
 * and O_i is written to shards[s].out in the shard's stored orientation.
 * The result equals dmuon_orthogonalize of the joined matrix up to rounding
 * (the Gram sum adds the shards' rounded partial products).  d > D (a Gram
 * matrix over the longer side) is allowed and takes the direct form, at
 * the higher cost of its d x d products.  Shards of one matrix share the
 * d x d work; each shard's products run at its own size.
 *   mats       host array of n descriptors (n >= 0)
 *   shards     host array of nshards descriptors per matrix, in order along
 *              the split; in/out device, rows x cols row-major of io_dtype;
 *              out may equal in, outputs must not overlap anything else
 * Uses hp->ns_steps, ns_backend, ns_precision, ns_coeffs and eps.  n == 0
 * does nothing.  Errors as for dmuon_orthogonalize, plus INVALID_ARG for
 * nshards < 1, a split other than 0 or 1, or shards whose d differ.
 */
typedef struct {
  int64_t rows, cols;   /* this shard as stored, > 0 */
  const void* in;       /* device, rows*cols values of io_dtype */
  void* out;            /* device, rows*cols values of io_dtype; may equal in */
} dmuon_shard_t;

typedef struct {
  const dmuon_shard_t* shards;   /* host array of nshards */
  int32_t nshards;               /* >= 1 */
  int32_t split;                 /* 1: column blocks, 0: row blocks */
} dmuon_sharded_t;

size_t dmuon_orthogonalize_sharded_workspace_size(const dmuon_sharded_t* mats, int32_t n,
                                                  const dmuon_hparams_t* hp);
int dmuon_orthogonalize_sharded(const dmuon_sharded_t* mats, int32_t n, int32_t io_dtype,
                                const dmuon_hparams_t* hp, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * The update stage alone: W <- W*(1 - lr*weight_decay) -
 * lr*0.2*sqrt(max(rows,cols))*O for every matrix (Hyperparameter Guide, lr
 * row; weight_decay of Step 4), with O = update[i] (device, rows x cols as
 * stored, update_dtype fp32 or bf16).  Reads mats[i].param, rows, cols and
 * param_dtype only; grad and momentum are ignored.  `workspace` (device,
 * >= dmuon_apply_update_workspace_size bytes) holds the launch table.
 */
size_t dmuon_apply_update_workspace_size(int32_t n);
int dmuon_apply_update(const dmuon_matrix_t* mats, int32_t n, const void* const* update,
                       int32_t update_dtype, const dmuon_hparams_t* hp, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * Gradient clipping by the global p-norm (Training Guide, "Gradient
 * Clipping": the dedicated gradients are clipped after their reduce and
 * before momentum and Newton-Schulz, by default with global p-norm clipping;
 * "Fused CUDA clip for regular / Muon / AdamW": several gradient groups are
 * clipped in one pass, each with its own norm and coefficient).  Every
 * gradient belongs to one bucket; per bucket b:
 *   total_b = (sum over its gradients of sum |g|^p)^(1/p)   (p = +inf: max |g|)
 *   coef_b  = min(1, max_norm[b] / (total_b + 1e-6))
 *   each of its gradients *= coef_b in place (fp64 product, rounded once,
 *   to nearest-even, to the gradient's dtype); a bucket whose coefficient
 *   is exactly 1 is not written.
 * These are the semantics of PyTorch's clip_grad_norm_, which the same page
 * uses for the other parameters; the norm is accumulated in fp64.  A NaN or
 * Inf makes its bucket's total and coefficient non-finite and propagates
 * into that bucket's gradients only (no error).
 *   grads      host array of n descriptors (n >= 0); each grad is device
 *              memory of numel values, contiguous, any alignment
 *   max_norm   host array of nbuckets finite values >= 0
 *   norm_type  p > 0, or +inf
 *   total_norm device array of nbuckets doubles receiving total_b, or NULL
 *   workspace  device, >= dmuon_clip_workspace_size bytes, 256-byte aligned
 * Gradients must not overlap each other, the workspace or total_norm.
 * n == 0 does nothing (total_norm is not written).
 */
typedef struct {
  int64_t numel;    /* elements, > 0 */
  void* grad;       /* device, numel values of `dtype`, clipped in place */
  int32_t dtype;    /* DMUON_F32 or DMUON_BF16 */
  int32_t bucket;   /* 0 <= bucket < nbuckets */
} dmuon_grad_t;

size_t dmuon_clip_workspace_size(const dmuon_grad_t* grads, int32_t n, int32_t nbuckets);
int dmuon_clip_grad_norm(const dmuon_grad_t* grads, int32_t n, int32_t nbuckets,
                         const double* max_norm, double norm_type, double* total_norm,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * dmuon_clip_grad_norm for callers that cannot allocate device or pinned
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments and results as dmuon_clip_grad_norm,
 * without the workspace: the clip's scratch (gradient table, per-bucket block
 * ranges and max_norm values, one fp64 partial per 64 KB of gradient, the
 * per-bucket coefficients) lives in a device array the library holds on each
 * GPU until the process ends, DMUON_NOALLOC_SCRATCH_BYTES long (4 MiB: about
 * 30 GB of gradients with few buckets), and the table reaches it as the
 * arguments of small copy kernels.  The call allocates nothing (no hipMalloc,
 * hipHostMalloc, event or stream creation); its first call on a device looks
 * the array's address up once.
 * Errors as dmuon_clip_grad_norm, and DMUON_ERR_WORKSPACE, before any
 * launch, when the gradients need more scratch than the array holds
 * (dmuon_clip_workspace_size > DMUON_NOALLOC_SCRATCH_BYTES).
 * Every call on one GPU uses the same array: calls that overlap on one GPU
 * (on different streams, or enqueued from several threads without ordering)
 * race on it.  Calls in one stream are ordered and safe.
 */
#define DMUON_NOALLOC_SCRATCH_BYTES (4u << 20)
int dmuon_clip_grad_norm_noalloc(const dmuon_grad_t* grads, int32_t n, int32_t nbuckets,
                                 const double* max_norm, double norm_type, double* total_norm,
                                 void* stream);

/*
 * The clip's norms and coefficients without the scaling pass: coef_out
 * (device, nbuckets doubles, required) receives coef_b; the gradients are
 * only read.  For dmuon_step_scaled.  Arguments, workspace and errors as
 * dmuon_clip_grad_norm (coef_out must not overlap the other buffers);
 * n == 0 writes nothing.
 */
int dmuon_clip_coefficients(const dmuon_grad_t* grads, int32_t n, int32_t nbuckets,
                            const double* max_norm, double norm_type, double* total_norm,
                            double* coef_out, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * AdamW step of the symmetric (non-Muon) parameters (Training Guide, "Step 4:
 * Create Optimizer": the optimizer's second group runs standard AdamW, with
 * adamw_lr 1e-3, betas (0.9, 0.999), weight decay 0.01, eps 1e-8;
 * "Semantic Param Groups": per-group values), fused over every tensor of a
 * call.  For tensor i in group groups[tensors[i].group], at step t:
 *   m <- beta1 m + (1 - beta1) g
 *   v <- beta2 v + (1 - beta2) g^2
 *   p <- p (1 - lr wd) - lr (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
 * (PyTorch's AdamW without amsgrad), evaluated in fp32 with the group's
 * constants formed in fp64; a bf16 parameter is rounded once to nearest
 * even.  m and v are fp32 and start at zero (the caller zeroes them).
 *   tensors    host array of n descriptors; a NULL grad skips the tensor
 *   groups     host array of ngroups hyperparameter sets
 *   workspace  device, >= dmuon_adamw_workspace_size(n) bytes, 256-byte
 *              aligned (the launch table)
 * Errors (before any launch): INVALID_ARG for n < 0, ngroups < 1 with
 * n > 0, a group with a non-finite lr, eps or weight decay, eps < 0, a beta
 * outside [0, 1) or step < 1, a tensor with numel <= 0, a NULL param,
 * exp_avg or exp_avg_sq, or a group index out of range; UNSUPPORTED for a
 * dtype other than F32 or BF16; ALIASING when any two of the buffers
 * overlap; WORKSPACE when the workspace is too small.
 */
typedef struct {
  double lr, beta1, beta2, eps, weight_decay;
  int64_t step;          /* this call's step number, >= 1 */
} dmuon_adamw_group_t;

typedef struct {
  int64_t numel;
  void* param;           /* device, numel values of param_dtype, updated in place */
  const void* grad;      /* device, numel values of grad_dtype; NULL: tensor skipped */
  float* exp_avg;        /* device, numel fp32 (m), in/out */
  float* exp_avg_sq;     /* device, numel fp32 (v), in/out */
  int32_t param_dtype;   /* DMUON_F32 or DMUON_BF16 */
  int32_t grad_dtype;    /* DMUON_F32 or DMUON_BF16 */
  int32_t group;         /* index into groups */
  int32_t pad_;
} dmuon_adamw_tensor_t;

size_t dmuon_adamw_workspace_size(int32_t n);
int dmuon_adamw_step(const dmuon_adamw_tensor_t* tensors, int32_t n, const dmuon_adamw_group_t* groups,
                     int32_t ngroups, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Owner assignment (host only; FAQ, "Why isn't DMuon just ZeRO-1?": every
 * dedicated matrix has one owner rank that runs its whole step; Training
 * Guide, "Verify Parameter Assignment": the assignment is reported as loads
 * per rank and an imbalance).  Each of the n matrices (rows[i] x cols[i],
 * host arrays) gets a cost:
 *   DMUON_COST_NUMEL       rows*cols
 *   DMUON_COST_NS_NOMINAL  ns_steps*(4 m^2 n + 2 m^3), m = min, n = max
 *   DMUON_COST_ROOFLINE    seconds at the device peaks: the flops of the
 *                          products this library runs for the matrix (the
 *                          form hp->ns_backend picks; symmetric results
 *                          counted once) at 2516.6 TFLOP/s, plus 20 bytes per
 *                          element (bf16 param and grad, fp32 momentum, the
 *                          NS input and output) at 8 TB/s
 * then matrices are taken in decreasing cost (ties: lower index first) and
 * each goes to the least loaded rank (ties: lower rank).
 *   hp         host, for ns_steps and ns_backend; NULL: 5 and gram
 *   owner      host array of n ranks in 0..nranks-1 (required if n > 0)
 *   cost       host array of n costs, or NULL
 *   loads      host array of nranks summed costs, or NULL
 *   imbalance  host, max(load)/mean(load) - 1 (0 with no cost), or NULL
 * Returns INVALID_ARG for n < 0, nranks < 1, an unknown model or a shape
 * outside 1..2^24; nothing is written then.
 */
typedef enum {
  DMUON_COST_NUMEL = 0,
  DMUON_COST_NS_NOMINAL = 1,
  DMUON_COST_ROOFLINE = 2
} dmuon_cost_model_t;

int dmuon_assign_owners(const int64_t* rows, const int64_t* cols, int32_t n, int32_t nranks,
                        int32_t cost_model, const dmuon_hparams_t* hp, int32_t* owner,
                        double* cost, double* loads, double* imbalance);

/* Readable name of a status code (static storage). */
const char* dmuon_status_string(int status);

/* Detail of the last failing call on this thread ("" if none). */
const char* dmuon_last_error(void);

/* Kernels, tile shapes and the Gram/direct rule, as a static string (the
 * analog of the Training Guide's dmuon.get_ns_backend()). */
const char* dmuon_backend_info(void);

/*
 * Measurement hooks.  Between dmuon_profile_begin() and dmuon_profile_end(),
 * every kernel the library enqueues (from any entry point, on its stream) is
 * bracketed by a pair of HIP events.  dmuon_profile_end() waits for those
 * events and writes JSON into buf (as dmuon_plan_describe does): per kernel
 * kind the launch count, summed device time in ms ("ms"), the time covered
 * by the union of those launches' intervals ("wall_ms": less than "ms" when
 * launches on two streams overlap, as a small batch's two stream groups do),
 * and the algorithmic flops
 * and HBM bytes of those launches (flops of the NS products with the true,
 * unpadded sizes and symmetric products counted once; bytes that an ideal
 * kernel must move).  Returns the JSON length or a negative status.  Called
 * again with no profiling window open, it returns the last report (so a
 * caller can size a buffer first).
 * Profiling adds a few microseconds per launch; it is off by default.
 */
int dmuon_profile_begin(void);
int64_t dmuon_profile_end(char* buf, size_t buf_len);

/* Host-only: the launch plan dmuon_step would use for these shapes (NS form
 * per matrix, workspace bytes, launches and tile counts), written as JSON into
 * buf (NUL-terminated, truncated to buf_len).  Returns the full length needed
 * (excluding the NUL), or a negative status.  Touches no device. */
int64_t dmuon_plan_describe(const int64_t* rows, const int64_t* cols, int32_t n,
                            const dmuon_hparams_t* hp, char* buf, size_t buf_len);

#ifdef __cplusplus
}
#endif
#endif /* DMUON_H */
