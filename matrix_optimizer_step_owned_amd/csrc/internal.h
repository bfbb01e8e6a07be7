// Internal declarations of the dmuon library: launch-table records shared by
// host planning code and the gfx950 kernels, and the host-side launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace dmuon {

enum : int32_t { DT_F32 = 0, DT_BF16 = 1 };

// Edge of the square element tile of the elementwise kernels.
constexpr int kEwTile = 64;
constexpr int kEwThreads = 256;

// One matrix as seen by the elementwise kernels (momentum / load / update /
// store).  "Stored" is rows x cols as the caller holds it; "wide" is the
// min x max orientation the NS products use (the transpose when tall).
struct EwMat {
  int64_t rows, cols;        // stored shape
  const void* src;           // momentum: grad; load: the matrix to orthogonalise
  float* mom;                // momentum buffer (momentum mode), else null
  void* param;               // update: W, in place (param_dtype); store: output
  void* u_dst;               // momentum/load: U destination (wide)
  const void* o_src;         // update/store: O source (wide)
  int64_t ld_wide;           // leading dimension of the wide buffers (elements)
  int32_t wide_rows;         // rows of the wide region to write (>= m; zero fill)
  int32_t wide_cols;         // cols of the wide region to write (>= n; zero fill)
  int32_t tall;              // rows > cols
  int32_t src_dtype;         // grad / load-source dtype
  int32_t wide_dtype;        // dtype of the wide buffer
  int32_t param_dtype;       // update: W dtype; store: output dtype
  int32_t scale_idx;         // update/store: multiply O by scale[scale_idx] if >= 0
  int32_t aligned;           // all rows of src / mom / param are 16-byte aligned
  int32_t user_index;        // position in the caller's array (per-matrix outputs)
  int32_t pad_;
  int64_t blk_wide;          // first block of this matrix over wide tiles
  int64_t blk_stored;        // first block of this matrix over stored tiles
  float lr_eff;              // lr * 0.2 * sqrt(max(rows, cols))
  float decay;               // 1 - lr * weight_decay
};

// One GEMM of a grouped launch.  C = alpha_eff * (A . op(B)) + beta_eff * Y
// + gamma * I[i == j < diag_limit], with alpha_eff = alpha * s^alpha_pow and
// beta_eff = beta * s^beta_pow, s = *scale (1 when scale is null).
//   A: row-major, K contiguous (lda), rows = tiles_m * tile
//   op(B): NT kernels read B as row-major N x K (K contiguous);
//          NN kernels read B as row-major K x N (N contiguous).
// All extents are padded to whole tiles with zeros, so kernels do no bounds
// checks.  sym: the result is symmetric; only tiles with tm <= tn are
// computed and each is also written mirrored.
struct GemmTask {
  const void* A;
  const void* B;
  void* C;
  const void* Y;
  const float* scale;
  int64_t lda, ldb, ldc, ldy;
  int32_t K;
  int32_t tiles_m, tiles_n;
  int32_t sym;
  int32_t alpha_pow, beta_pow;
  int32_t diag_limit;
  int32_t tile_begin;        // index of this task's first tile in the launch
  float alpha, beta, gamma;
  int32_t pad_;
};

// ---- launchers (each enqueues one kernel on `stream`) ----------------------

// U = momentum / Nesterov (mode 0) or plain copy (mode 1) of every matrix into
// its wide buffer; partials[b] = sum of u^2 over block b.
hipError_t launch_momentum(const EwMat* mats_dev, int nmats, int64_t nblocks, int mode,
                           float mu, int nesterov, float* partials, hipStream_t stream);

// sumsq[i] = sum of matrix i's partials (fp64); scale[i] = 1/(sqrt(sumsq)+eps).
hipError_t launch_finalize(const EwMat* mats_dev, int nmats, int64_t nblocks,
                           const float* partials, double* sumsq, float* scale, double eps,
                           hipStream_t stream);

// mode 0: W <- W*decay - lr_eff*o_scale*O in place; mode 1: out <- o_scale*O.
hipError_t launch_update(const EwMat* mats_dev, int nmats, int64_t nblocks, int mode,
                         const float* scale, hipStream_t stream);

// Grouped NS products.  tile = 128 (bf16) or 64 (fp32).
enum class GemmKind { NT, NN };
hipError_t launch_gemm_bf16(GemmKind kind, const GemmTask* tasks_dev, int ntasks,
                            int64_t ntiles, int tile, hipStream_t stream);
hipError_t launch_gemm_f32(GemmKind kind, const GemmTask* tasks_dev, int ntasks,
                           int64_t ntiles, int tile, hipStream_t stream);

// Tile edge of the grouped GEMM kernels per precision.
constexpr int kTileBf16 = 128;
constexpr int kTileF32 = 64;

}  // namespace dmuon
