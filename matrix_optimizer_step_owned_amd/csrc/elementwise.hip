// HBM-bound elementwise kernels of the owner-side Muon step (gfx950).
//
//   momentum_kernel  buf <- mu*buf + g; U <- g + mu*buf (Nesterov) or buf,
//                    written in the wide orientation with zero padding, plus
//                    one partial sum of U^2 per block (DMuon Training Guide,
//                    Hyperparameter Guide: momentum and nesterov rows).
//   finalize_kernel  per-matrix fp64 sum of the partials and the NS input
//                    scale 1/(||U||_F + eps).
//   update_kernel    W <- W*(1 - lr*wd) - lr*0.2*sqrt(max(m,n))*O (lr row of
//                    the same table), or a plain store of O.
//
// Each block owns one 64 x 64 element tile of one matrix; a block finds its
// matrix by binary search over per-matrix first-block indices, so one launch
// covers a whole ragged batch.  Tall matrices go through a padded LDS tile so
// that both the stored-orientation and the wide-orientation accesses stay
// coalesced.  Arithmetic is fp32; bf16 results are rounded to nearest even.
#include "internal.h"

namespace dmuon {
namespace {

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float load1(const void* p, int64_t i, int dt) {
  return dt == DT_F32 ? static_cast<const float*>(p)[i]
                      : bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
}

__device__ __forceinline__ void store1(void* p, int64_t i, int dt, float v) {
  if (dt == DT_F32)
    static_cast<float*>(p)[i] = v;
  else
    static_cast<uint16_t*>(p)[i] = static_cast<uint16_t>(f32_to_bf16_bits(v));
}

// Four consecutive elements starting at i (i multiple of 4, base aligned).
__device__ __forceinline__ float4 load4(const void* p, int64_t i, int dt) {
  if (dt == DT_F32) return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
  const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
  return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                     __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
}

__device__ __forceinline__ void store4(void* p, int64_t i, int dt, float4 v) {
  if (dt == DT_F32) {
    *reinterpret_cast<float4*>(static_cast<float*>(p) + i) = v;
  } else {
    uint2 o;
    o.x = f32_to_bf16_bits(v.x) | (f32_to_bf16_bits(v.y) << 16);
    o.y = f32_to_bf16_bits(v.z) | (f32_to_bf16_bits(v.w) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p) + i) = o;
  }
}

// A gradient value scaled as gradient clipping writes it: the fp64 product,
// rounded once to the gradient's dtype.
__device__ __forceinline__ float scale_grad(float g, double c, int dt) {
  const double d = static_cast<double>(g) * c;
  if (dt == DT_F32) return static_cast<float>(d);
  return bf16_bits_to_f32(f32_to_bf16_bits(f64_to_f32_round_odd(d)));
}

__device__ __forceinline__ float get(const float4& v, int e) {
  return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}

__device__ __forceinline__ int find_mat(const EwMat* __restrict__ m, int n, int64_t b, bool stored) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    const int64_t s = stored ? m[mid].blk_stored : m[mid].blk_wide;
    if (s <= b) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Thread t of a block covers tile rows (t >> 4) + 16p, p = 0..3, and the four
// columns 4*(t & 15) .. +3.
constexpr int kRowsPerPass = kEwThreads / 16;
constexpr int kPasses = kEwTile / kRowsPerPass;

__global__ void __launch_bounds__(kEwThreads)
momentum_kernel(const EwMat* __restrict__ mats, int nmats, int mode, float mu, int nesterov,
                float* __restrict__ partials) {
  __shared__ float tile[kEwTile][kEwTile + 1];
  __shared__ float red[kEwThreads / 64];

  const int64_t b = blockIdx.x;
  const int mi = find_mat(mats, nmats, b, false);
  const EwMat M = mats[mi];
  const int64_t local = b - M.blk_wide;
  const int tiles_c = (M.wide_cols + kEwTile - 1) / kEwTile;
  const int64_t i0 = (local / tiles_c) * kEwTile;   // wide tile origin
  const int64_t j0 = (local % tiles_c) * kEwTile;
  const int64_t r0 = M.tall ? j0 : i0;                // stored tile origin
  const int64_t c0 = M.tall ? i0 : j0;

  const int t = threadIdx.x;
  const int lc = (t & 15) * 4;
  const int lr0 = t >> 4;

  float u[kPasses][4];
  float ss = 0.f;
  const bool full = M.aligned && r0 + kEwTile <= M.rows && c0 + kEwTile <= M.cols;
  const double gsc = M.gscale ? *M.gscale : 1.0;   // clipping coefficient, if fused
  const bool scaled = gsc != 1.0;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int64_t r = r0 + lr0 + kRowsPerPass * p;
    const int64_t base = r * M.cols + c0 + lc;
    if (full) {
      float4 g = load4(M.src, base, M.src_dtype);
      if (scaled) {
        g.x = scale_grad(g.x, gsc, M.src_dtype); g.y = scale_grad(g.y, gsc, M.src_dtype);
        g.z = scale_grad(g.z, gsc, M.src_dtype); g.w = scale_grad(g.w, gsc, M.src_dtype);
      }
      float4 uu;
      if (mode == 0) {
        const float4 m = *reinterpret_cast<const float4*>(M.mom + base);
        float4 mn;
        mn.x = fmaf(mu, m.x, g.x); mn.y = fmaf(mu, m.y, g.y);
        mn.z = fmaf(mu, m.z, g.z); mn.w = fmaf(mu, m.w, g.w);
        *reinterpret_cast<float4*>(M.mom + base) = mn;
        if (nesterov) {
          uu.x = fmaf(mu, mn.x, g.x); uu.y = fmaf(mu, mn.y, g.y);
          uu.z = fmaf(mu, mn.z, g.z); uu.w = fmaf(mu, mn.w, g.w);
        } else {
          uu = mn;
        }
      } else {
        uu = g;
      }
      u[p][0] = uu.x; u[p][1] = uu.y; u[p][2] = uu.z; u[p][3] = uu.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t c = c0 + lc + e;
        float v = 0.f;
        if (r < M.rows && c < M.cols) {
          const int64_t idx = r * M.cols + c;
          float g = load1(M.src, idx, M.src_dtype);
          if (scaled) g = scale_grad(g, gsc, M.src_dtype);
          if (mode == 0) {
            const float mn = fmaf(mu, M.mom[idx], g);
            M.mom[idx] = mn;
            v = nesterov ? fmaf(mu, mn, g) : mn;
          } else {
            v = g;
          }
        }
        u[p][e] = v;
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) ss = fmaf(u[p][e], u[p][e], ss);
  }

  // Write U (wide: wide_rows x wide_cols) and/or U^T (wide_cols x wide_rows).
  // One of the two is the stored orientation of this tile and is written
  // straight from registers; the other goes through the LDS tile.
  void* const direct_dst = M.tall ? M.u_dst_t : M.u_dst;
  void* const trans_dst = M.tall ? M.u_dst : M.u_dst_t;
  const int64_t direct_ld = M.tall ? M.ld_wide_t : M.ld_wide;
  const int64_t trans_ld = M.tall ? M.ld_wide : M.ld_wide_t;
  // extents (rows, cols) of the destinations and this tile's origin in them
  const int64_t d_rows = M.tall ? M.wide_cols : M.wide_rows, d_cols = M.tall ? M.wide_rows : M.wide_cols;
  const int64_t d_r0 = M.tall ? j0 : i0, d_c0 = M.tall ? i0 : j0;
  if (trans_dst) {
#pragma unroll
    for (int p = 0; p < kPasses; ++p)
#pragma unroll
      for (int e = 0; e < 4; ++e) tile[lr0 + kRowsPerPass * p][lc + e] = u[p][e];
  }
  if (direct_dst) {
    const bool dfull = (direct_ld % 4) == 0 && d_r0 + kEwTile <= d_rows && d_c0 + kEwTile <= d_cols;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int64_t i = d_r0 + lr0 + kRowsPerPass * p;
      const int64_t base = i * direct_ld + d_c0 + lc;
      if (dfull) {
        store4(direct_dst, base, M.wide_dtype, make_float4(u[p][0], u[p][1], u[p][2], u[p][3]));
      } else if (i < d_rows) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (d_c0 + lc + e < d_cols) store1(direct_dst, base + e, M.wide_dtype, u[p][e]);
      }
    }
  }
  if (trans_dst) {
    __syncthreads();
    // the transposed destination has extents (d_cols, d_rows), origin (d_c0, d_r0)
    const bool tfull = (trans_ld % 4) == 0 && d_c0 + kEwTile <= d_cols && d_r0 + kEwTile <= d_rows;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int64_t i = d_c0 + lr0 + kRowsPerPass * p;
      const int64_t base = i * trans_ld + d_r0 + lc;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = tile[lc + e][lr0 + kRowsPerPass * p];
      if (tfull) {
        store4(trans_dst, base, M.wide_dtype, make_float4(v[0], v[1], v[2], v[3]));
      } else if (i < d_cols) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (d_r0 + lc + e < d_rows) store1(trans_dst, base + e, M.wide_dtype, v[e]);
      }
    }
  }

  // block sum of U^2
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if ((t & 63) == 0) red[t >> 6] = ss;
  __syncthreads();
  if (t == 0) partials[b] = (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ void __launch_bounds__(256)
finalize_kernel(const EwMat* __restrict__ mats, int nmats, int64_t nblocks,
                const float* __restrict__ partials, double* __restrict__ sumsq,
                float* __restrict__ scale, double eps) {
  __shared__ double red[256];
  const int mi = blockIdx.x;
  // a shard of a sharded matrix sums the blocks of all its group's shards
  // (the same blocks in the same order for every member, so every shard
  // gets the identical scale)
  const int g0 = mats[mi].grp_count > 0 ? mats[mi].grp_first : mi;
  const int g1 = mats[mi].grp_count > 0 ? mats[mi].grp_first + mats[mi].grp_count : mi + 1;
  const int64_t b0 = mats[g0].blk_wide;
  const int64_t b1 = g1 < nmats ? mats[g1].blk_wide : nblocks;
  double acc = 0.0;
  for (int64_t b = b0 + threadIdx.x; b < b1; b += 256) acc += static_cast<double>(partials[b]);
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double v = red[0];
    if (sumsq) sumsq[mats[mi].user_index] = v;
    if (scale) scale[mi] = static_cast<float>(1.0 / (sqrt(v) + eps));
  }
}

__global__ void __launch_bounds__(kEwThreads)
update_kernel(const EwMat* __restrict__ mats, int nmats, int mode, const float* __restrict__ scale) {
  __shared__ float tile[kEwTile][kEwTile + 1];

  const int64_t b = blockIdx.x;
  const int mi = find_mat(mats, nmats, b, true);
  const EwMat M = mats[mi];
  const int64_t local = b - M.blk_stored;
  const int tiles_c = static_cast<int>((M.cols + kEwTile - 1) / kEwTile);
  const int64_t r0 = (local / tiles_c) * kEwTile;   // stored tile origin
  const int64_t c0 = (local % tiles_c) * kEwTile;

  const int t = threadIdx.x;
  const int lc = (t & 15) * 4;
  const int lr0 = t >> 4;
  const float osc = M.scale_idx >= 0 ? scale[M.scale_idx] : 1.0f;

  // O for the stored tile: o[p][e] = O(r0 + lr0 + 16p, c0 + lc + e)
  float o[kPasses][4];
  {
    // the wide buffer is read along its rows: wide (a, b) with
    // a = stored row (not tall) / stored col (tall)
    const int64_t a0 = M.tall ? c0 : r0;
    const int64_t bb0 = M.tall ? r0 : c0;
    const int64_t a_lim = M.tall ? M.cols : M.rows;
    const int64_t b_lim = M.tall ? M.rows : M.cols;
    const bool full = (M.ld_wide % 4) == 0 && a0 + kEwTile <= a_lim && bb0 + kEwTile <= b_lim;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int64_t a = a0 + lr0 + kRowsPerPass * p;
      const int64_t base = a * M.ld_wide + bb0 + lc;
      if (full) {
        const float4 v = load4(M.o_src, base, M.wide_dtype);
        o[p][0] = v.x; o[p][1] = v.y; o[p][2] = v.z; o[p][3] = v.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[p][e] = (a < a_lim && bb0 + lc + e < b_lim) ? load1(M.o_src, base + e, M.wide_dtype) : 0.f;
      }
    }
    if (M.tall) {
#pragma unroll
      for (int p = 0; p < kPasses; ++p)
#pragma unroll
        for (int e = 0; e < 4; ++e) tile[lr0 + kRowsPerPass * p][lc + e] = o[p][e];
      __syncthreads();
#pragma unroll
      for (int p = 0; p < kPasses; ++p)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[p][e] = tile[lc + e][lr0 + kRowsPerPass * p];
    }
  }

  const float step = M.lr_eff * osc;
  const bool full = M.aligned && r0 + kEwTile <= M.rows && c0 + kEwTile <= M.cols;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int64_t r = r0 + lr0 + kRowsPerPass * p;
    const int64_t base = r * M.cols + c0 + lc;
    if (full) {
      float4 res;
      if (mode == 0) {
        const float4 w = load4(M.param, base, M.param_dtype);
        res.x = fmaf(-step, o[p][0], w.x * M.decay);
        res.y = fmaf(-step, o[p][1], w.y * M.decay);
        res.z = fmaf(-step, o[p][2], w.z * M.decay);
        res.w = fmaf(-step, o[p][3], w.w * M.decay);
      } else {
        res = make_float4(osc * o[p][0], osc * o[p][1], osc * o[p][2], osc * o[p][3]);
      }
      store4(M.param, base, M.param_dtype, res);
    } else if (r < M.rows) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (c0 + lc + e >= M.cols) continue;
        float res;
        if (mode == 0)
          res = fmaf(-step, o[p][e], load1(M.param, base + e, M.param_dtype) * M.decay);
        else
          res = osc * o[p][e];
        store1(M.param, base + e, M.param_dtype, res);
      }
    }
  }
}

// Sum of partial Gram matrices (see GramSum).  Thread t covers tile rows
// (t >> 4) + 16p and the four columns 4*(t & 15) .. +3, as the other
// elementwise kernels; the parts are added in their order in fp32.
__global__ void __launch_bounds__(kEwThreads)
gram_sum_kernel(const GramSum* __restrict__ sums, int nsums, const void* const* __restrict__ parts,
                int32_t dtype) {
  const int64_t b = blockIdx.x;
  int lo = 0, hi = nsums - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (sums[mid].blk_first <= b) lo = mid; else hi = mid - 1;
  }
  const GramSum S = sums[lo];
  const int64_t local = b - S.blk_first;
  const int tiles = S.edge / kEwTile;
  const int64_t i0 = (local / tiles) * kEwTile, j0 = (local % tiles) * kEwTile;
  const int t = threadIdx.x;
  const int lc = (t & 15) * 4;
  const int lr0 = t >> 4;
  float acc[kPasses][4];
#pragma unroll
  for (int p = 0; p < kPasses; ++p)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[p][e] = 0.f;
  for (int q = 0; q < S.count; ++q) {
    const void* src = parts[S.first_part + q];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const float4 v = load4(src, (i0 + lr0 + kRowsPerPass * p) * S.ld + j0 + lc, dtype);
      acc[p][0] += v.x; acc[p][1] += v.y; acc[p][2] += v.z; acc[p][3] += v.w;
    }
  }
#pragma unroll
  for (int p = 0; p < kPasses; ++p)
    store4(S.dst, (i0 + lr0 + kRowsPerPass * p) * S.ld + j0 + lc, dtype,
           make_float4(acc[p][0], acc[p][1], acc[p][2], acc[p][3]));
}

}  // namespace

hipError_t launch_gram_sum(const GramSum* sums_dev, int nsums, int64_t nblocks, const void* const* parts_dev,
                           int32_t dtype, hipStream_t stream) {
  if (nblocks <= 0 || nsums <= 0) return hipSuccess;
  hipLaunchKernelGGL(gram_sum_kernel, dim3(static_cast<unsigned>(nblocks)), dim3(kEwThreads), 0, stream,
                     sums_dev, nsums, parts_dev, dtype);
  return hipGetLastError();
}

// Launch-table upload: the GPU reads the pinned host image directly (it is
// mapped into the device's address space) and writes the workspace, 16 bytes
// per lane, the last bytes one by one.  A kernel on the caller's stream
// keeps the upload on the compute queue, where waits on other streams are
// resolved on the GPU; a DMA copy behind such a wait was resolved on the host
// and blocked it.
__global__ void __launch_bounds__(256)
table_copy_kernel(const char* __restrict__ src, char* __restrict__ dst, int64_t bytes) {
  const int64_t n16 = bytes / 16;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(src)[i];
  if (blockIdx.x == 0 && threadIdx.x < bytes - n16 * 16) dst[n16 * 16 + threadIdx.x] = src[n16 * 16 + threadIdx.x];
}

hipError_t launch_table_copy(void* dst, const void* host_src, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  if (reinterpret_cast<uintptr_t>(dst) % 16 || reinterpret_cast<uintptr_t>(host_src) % 16) return hipErrorInvalidValue;
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  const unsigned blocks = static_cast<unsigned>(std::min<int64_t>(std::max<int64_t>((n16 + 255) / 256, 1), 1024));
  hipLaunchKernelGGL(table_copy_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const char*>(host_src),
                     static_cast<char*>(dst), static_cast<int64_t>(bytes));
  return hipGetLastError();
}

hipError_t launch_momentum(const EwMat* mats_dev, int nmats, int64_t nblocks, int mode, float mu,
                           int nesterov, float* partials, hipStream_t stream) {
  if (nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(momentum_kernel, dim3(static_cast<unsigned>(nblocks)), dim3(kEwThreads), 0,
                     stream, mats_dev, nmats, mode, mu, nesterov, partials);
  return hipGetLastError();
}

hipError_t launch_finalize(const EwMat* mats_dev, int nmats, int64_t nblocks, const float* partials,
                             double* sumsq, float* scale, double eps, hipStream_t stream) {
  if (nmats <= 0) return hipSuccess;
  hipLaunchKernelGGL(finalize_kernel, dim3(nmats), dim3(256), 0, stream, mats_dev, nmats, nblocks,
                     partials, sumsq, scale, eps);
  return hipGetLastError();
}

hipError_t launch_update(const EwMat* mats_dev, int nmats, int64_t nblocks, int mode,
                         const float* scale, hipStream_t stream) {
  if (nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(update_kernel, dim3(static_cast<unsigned>(nblocks)), dim3(kEwThreads), 0,
                     stream, mats_dev, nmats, mode, scale);
  return hipGetLastError();
}

}  // namespace dmuon
