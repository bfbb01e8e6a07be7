// Internal declarations of the dmuon library: launch-table records shared by
// host planning code and the gfx950 kernels, and the host-side launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/dmuon.h"

namespace dmuon {

enum : int32_t { DT_F32 = 0, DT_BF16 = 1 };

// Edge of the square element tile of the elementwise kernels.
constexpr int kEwTile = 64;
// Extra elements per row of every NS buffer (one 128-byte line in bf16).
constexpr int kPitchPad = 64;
constexpr int kEwThreads = 256;

// One matrix as seen by the elementwise kernels (momentum / load / update /
// store).  "Stored" is rows x cols as the caller holds it; "wide" is the
// min x max orientation the NS products use (the transpose when tall).
struct EwMat {
  int64_t rows, cols;        // stored shape
  const void* src;           // momentum: grad; load: the matrix to orthogonalise
  float* mom;                // momentum buffer (momentum mode), else null
  void* param;               // update: W, in place (param_dtype); store: output
  void* u_dst;               // momentum/load: U destination (wide), or null
  void* u_dst_t;             // momentum/load: U^T destination (wide_cols x wide_rows), or null
  const void* o_src;         // update/store: O source (wide)
  const double* gscale;      // momentum: if not null, the gradient is first
                             // scaled by *gscale (fp64 product rounded once to
                             // src_dtype, as gradient clipping writes it)
  int64_t ld_wide;           // leading dimension of the wide buffers (elements)
  int64_t ld_wide_t;         // leading dimension of the U^T buffer
  int32_t wide_rows;         // rows of the wide region to write (>= m; zero fill)
  int32_t wide_cols;         // cols of the wide region to write (>= n; zero fill)
  int32_t tall;              // rows > cols
  int32_t src_dtype;         // grad / load-source dtype
  int32_t wide_dtype;        // dtype of the wide buffer
  int32_t param_dtype;       // update: W dtype; store: output dtype
  int32_t scale_idx;         // update/store: multiply O by scale[scale_idx] if >= 0
  int32_t aligned;           // all rows of src / mom / param are 16-byte aligned
  int32_t user_index;        // position in the caller's array (per-matrix outputs)
  // shards of one tensor-parallel matrix: entries grp_first .. grp_first +
  // grp_count - 1 share one norm (grp_count 0: a matrix of its own)
  int32_t grp_first;
  int32_t grp_count;
  int32_t pad_;
  int64_t blk_wide;          // first block of this matrix over wide tiles
  int64_t blk_stored;        // first block of this matrix over stored tiles
  float lr_eff;              // lr * 0.2 * sqrt(max(rows, cols))
  float decay;               // 1 - lr * weight_decay
};

// One GEMM of a grouped launch: C[i][j] = alpha_eff * sum_k A[i][k] B[j][k]
// + beta_eff * Y[i][j] + gamma * [i == j < diag_limit], with
// alpha_eff = alpha * s^alpha_pow, beta_eff = beta * s^beta_pow and
// s = *scale (1 when scale is null).  A (M x K) and B (N x K) are row-major
// with K contiguous.  All extents are padded to whole tiles with zeros, so
// kernels do no bounds checks.
//   sym: the result is symmetric; only tiles with tm <= tn are computed and
//        the upper triangle is also written mirrored, so C is exactly
//        symmetric.
//   Ct:  if not null, C^T is also written there (N x M, ldct).
//   W:   if not null (the last product of a matrix in a step, bf16 kernel
//        and bf16 parameters only), C is not written; instead the parameter
//        is updated in place, W <- W*decay - lr_eff*O with O the product
//        rounded to bf16, evaluated in fp32 and rounded once to bf16.  W is rows x cols of the wide
//        orientation (w_m x w_n valid), or its transpose when w_tall; ldw is
//        its row pitch; w_vec: 16-byte accesses along W rows are aligned.
struct GemmTask {
  const void* A;
  const void* B;
  void* C;
  void* Ct;
  const void* Y;
  const float* scale;
  void* W;
  int64_t lda, ldb, ldc, ldct, ldy, ldw;
  int32_t K;
  int32_t tiles_m, tiles_n;
  int32_t sym;
  int32_t alpha_pow, beta_pow;
  int32_t diag_limit;
  int32_t w_m, w_n, w_dtype, w_tall, w_vec;
  float alpha, beta, gamma;
  float lr_eff, decay;
};

// One block of a grouped GEMM launch: which task and which output tile.
// Block b of a launch processes map[b]; the host orders the map so that the
// blocks the hardware sends to one XCD (b % 8 == x) cover a contiguous, 2-D
// blocked part of every task, sharing operand panels in that XCD's L2.
struct TileRef {
  int32_t task;
  uint16_t tm, tn;
};

// Number of XCDs that workgroups are dealt to round-robin, and the shape of
// the groups of tiles walked together inside a task (one group is as many
// 256-tiles as one XCD runs at once: 8 row panels by 4 column panels).
constexpr int kNumXcd = 8;
constexpr int kTileGroupRows = 8, kTileGroupCols = 4;

// One sum of the partial Gram matrices of a sharded matrix (the stand-in
// for their all-reduce across tensor-parallel ranks): dst = sum over
// parts[first_part .. first_part + count - 1], each edge x edge with row
// pitch ld, summed in fp32 in part order and rounded once.  edge is a
// multiple of kEwTile; block b of the launch covers one kEwTile x kEwTile
// tile of the entry whose blk_first is the last one <= b.
struct GramSum {
  void* dst;
  int64_t ld;
  int64_t blk_first;
  int32_t edge;
  int32_t first_part;
  int32_t count;
  int32_t pad_;
};

// One gradient of a clipping call.  The host orders the items by bucket, so
// each bucket's blocks form one contiguous range.
struct ClipItem {
  void* grad;          // in place
  int64_t numel;
  int64_t blk_first;   // first block of this gradient
  int32_t dtype;       // DT_F32 or DT_BF16
  int32_t bucket;
  int32_t aligned;     // grad is 16-byte aligned
  int32_t pad_;
};
constexpr int kClipThreads = 256;
constexpr int kClipFinalizeThreads = 1024;
constexpr int kClipChunkBytes = 65536;   // bytes of one gradient per block

// One tensor of a fused AdamW call, with its group's constants folded:
// decay = 1 - lr*wd, step_size = lr / (1 - beta1^t), inv_sqrt_bc2 =
// 1 / sqrt(1 - beta2^t) (all formed in fp64 on the host, rounded to fp32).
struct AdamItem {
  void* p;
  const void* g;
  float* m;
  float* v;
  int64_t numel;
  int64_t blk_first;     // first block of this tensor
  float decay, step_size, inv_sqrt_bc2, eps;
  float beta1, one_minus_beta1, beta2, one_minus_beta2;
  int32_t p_dtype, g_dtype;
  int32_t aligned;       // p, g, m and v all 16-byte aligned
  int32_t pad_;
};
constexpr int kAdamThreads = 256;
constexpr int kAdamChunk = 8192;   // elements of one tensor per block

// fp64 -> fp32 rounded to odd: truncate, then set the last bit when inexact.
// A value rounded to odd at 24 bits and then to nearest-even at 8 bits is the
// nearest-even rounding of the fp64 value itself (24 >= 2 * 8 + 2), so a bf16
// result formed this way is rounded once from the fp64 value.
__device__ __forceinline__ float f64_to_f32_round_odd(double d) {
  const float f = static_cast<float>(d);
  const double back = static_cast<double>(f);
  if (back == d) return f;
  uint32_t u = __float_as_uint(f);
  if (fabs(back) > fabs(d)) u -= 1;   // rounded away from zero: step back toward it
  return __uint_as_float(u | 1u);
}

// Records msg as the calling thread's last error (dmuon_last_error) and
// returns status; an empty message with no status clears it.
int set_last_error(int status, const std::string& msg);
inline void set_last_error(const char* msg) { set_last_error(0, msg); }

// ---- launchers (each enqueues one kernel on `stream`) ----------------------

// U = momentum / Nesterov (mode 0) or plain copy (mode 1) of every matrix into
// its wide buffer; partials[b] = sum of u^2 over block b.
// Copies `bytes` from a pinned host buffer to device memory with a kernel on
// `stream` (both 16-byte aligned).
hipError_t launch_table_copy(void* dst, const void* host_src, size_t bytes, hipStream_t stream);
hipError_t launch_momentum(const EwMat* mats_dev, int nmats, int64_t nblocks, int mode,
                           float mu, int nesterov, float* partials, hipStream_t stream);

// sumsq[i] = sum of matrix i's partials (fp64); scale[i] = 1/(sqrt(sumsq)+eps).
hipError_t launch_finalize(const EwMat* mats_dev, int nmats, int64_t nblocks,
                           const float* partials, double* sumsq, float* scale, double eps,
                           hipStream_t stream);

// mode 0: W <- W*decay - lr_eff*o_scale*O in place; mode 1: out <- o_scale*O.
hipError_t launch_gram_sum(const GramSum* sums_dev, int nsums, int64_t nblocks, const void* const* parts_dev,
                           int32_t dtype, hipStream_t stream);
hipError_t launch_adamw(const AdamItem* items_dev, int n, int64_t nblocks, hipStream_t stream);
hipError_t launch_update(const EwMat* mats_dev, int nmats, int64_t nblocks, int mode,
                         const float* scale, hipStream_t stream);

// Grouped NS products.  tile = 128 or 256 (bf16), 64 (fp32).
hipError_t launch_gemm_bf16(const GemmTask* tasks_dev, const TileRef* map_dev, int64_t ntiles,
                            int tile, hipStream_t stream);
hipError_t launch_gemm_f32(const GemmTask* tasks_dev, const TileRef* map_dev, int64_t ntiles,
                           int tile, hipStream_t stream);

// Gradient clipping: partials[b] = sum |g|^p (max |g| for p = inf) over
// block b; per bucket, total = the p-norm of its blocks' partials and
// coef = min(1, max_norm / (total + 1e-6)); then every gradient *= coef.
hipError_t launch_clip_norm(const ClipItem* items_dev, int n, int64_t nblocks, double p, double* partials,
                            hipStream_t stream);
hipError_t launch_clip_finalize(const int64_t* bucket_blocks_dev, int nbuckets, const double* max_norm_dev,
                                const double* partials, double p, double* total_out, double* coefs,
                                hipStream_t stream);
hipError_t launch_clip_scale(const ClipItem* items_dev, int n, int64_t nblocks, const double* coefs,
                             hipStream_t stream);

// Copies `bytes` (a multiple of 16) of host table to device `dst` (16-byte
// aligned) on `stream` as the arguments of small kernels, kArgChunkBytes per
// launch: no pinned buffer, no host-memory copy, nothing allocated.
constexpr int kArgChunkBytes = 2048;
hipError_t upload_by_kernel_args(void* dst, const void* host, size_t bytes, hipStream_t stream);

// dmuon_clip_grad_norm with the current device's scratch array
// (scratch_bytes long, its address from scratch_of_device, asked for once
// every host-side check has passed) as its workspace and its table uploaded
// by upload_by_kernel_args.
int clip_grad_norm_in_scratch(const dmuon_grad_t* grads, int32_t n, int32_t nbuckets, const double* max_norm,
                              double norm_type, double* total_norm, int (*scratch_of_device)(void**),
                              size_t scratch_bytes, void* stream);

// Tile edges of the grouped GEMM kernels.
constexpr int kTileBf16 = 128;
constexpr int kTileBf16Big = 256;
constexpr int kTileF32 = 64;
constexpr int kTileF32Big = 128;
// fp32 products use 128-tiles when the first NS stage has at least this many
// of them (two per CU, two waves of blocks), else 64-tiles.
constexpr int64_t kF32BigTileMinCount = 1024;
// 256-tiles are used when the first NS stage has at least this many of them
// and at least half of them belong to matrices kBigTileMinDim or more wide.
constexpr int64_t kBigTileMinCount = 128;
constexpr int64_t kBigTileMinDim = 2048;

}  // namespace dmuon
