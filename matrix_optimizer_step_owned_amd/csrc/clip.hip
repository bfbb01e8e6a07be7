// Gradient clipping by the global p-norm, per bucket (DMuon Training Guide,
// "Gradient Clipping" and "Fused CUDA clip for regular / Muon / AdamW"):
//   total_b = (sum over bucket b's gradients of sum |g|^p)^(1/p)
//             (p = inf: the largest |g|)
//   coef_b  = min(1, max_norm_b / (total_b + 1e-6))
//   g      <- g * coef_b in place: the product in fp64, rounded once (to nearest,
//             ties to even) to the gradient's dtype.
//
// Three launches, all HBM-bound:
//   clip_norm_kernel     one block per 64 KB chunk of a gradient: fp64 partial
//                        of sum |g|^p (or max |g|), wavefront shuffles + LDS;
//   clip_finalize_kernel one block per bucket: its blocks are contiguous (the
//                        host orders the gradients by bucket), so the total is
//                        a fixed-order fp64 tree sum; writes total and coef;
//   clip_scale_kernel    the same chunks: g *= coef; a chunk whose bucket's
//                        coefficient is exactly 1 is left untouched (no write).
#include "internal.h"

namespace dmuon {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
#define GLOBAL_AS __attribute__((address_space(1)))

// streaming 16-byte accesses: every byte is touched once per pass, so they
// carry the non-temporal hint (measured: the norm pass reads at ~7.0 TB/s
// with it, ~6.0 TB/s without)
__device__ __forceinline__ u32x4_t ld16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const GLOBAL_AS u32x4_t*>(reinterpret_cast<uintptr_t>(p)));
}
__device__ __forceinline__ void st16(void* p, u32x4_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<GLOBAL_AS u32x4_t*>(reinterpret_cast<uintptr_t>(p)));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// two fp64 products -> packed bf16 pair, each rounded once to nearest-even
__device__ __forceinline__ uint32_t pack2_from_f64(double a, double b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {f64_to_f32_round_odd(a), f64_to_f32_round_odd(b)};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// block -> gradient: the last item whose first block is <= b
__device__ __forceinline__ int find_item(const ClipItem* items, int n, int64_t b) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (items[mid].blk_first <= b) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// max that keeps a NaN once seen
__device__ __forceinline__ double nanmax(double a, double b) {
  if (a != a) return a;
  if (b != b) return b;
  return a > b ? a : b;
}

template <int P>  // 0: general p, 1: p = 1, 2: p = 2, 3: p = inf
__device__ __forceinline__ void accum(double& acc, float x, double p) {
  const double a = fabs(static_cast<double>(x));
  if constexpr (P == 1) acc += a;
  else if constexpr (P == 2) acc = fma(a, a, acc);
  else if constexpr (P == 3) acc = nanmax(acc, a);
  else acc += pow(a, p);
}

template <int P>
__device__ __forceinline__ double combine(double a, double b) {
  if constexpr (P == 3) return nanmax(a, b);
  else return a + b;
}

template <int P, int THREADS>
__device__ double block_reduce(double v, double* lds) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = combine<P>(v, __shfl_xor(v, off));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) lds[wave] = v;
  __syncthreads();
  double r = lds[0];
#pragma unroll
  for (int w = 1; w < THREADS / 64; ++w) r = combine<P>(r, lds[w]);
  return r;
}

template <int P>
__global__ void __launch_bounds__(kClipThreads)
clip_norm_kernel(const ClipItem* __restrict__ items, int n, double p, double* __restrict__ partials) {
  __shared__ double lds[kClipThreads / 64];
  const int64_t b = blockIdx.x;
  const ClipItem& it = items[find_item(items, n, b)];
  const int es = it.dtype == DT_BF16 ? 2 : 4;
  const int64_t per_chunk = kClipChunkBytes / es;
  const int64_t first = (b - it.blk_first) * per_chunk;
  const int64_t count = it.numel - first < per_chunk ? it.numel - first : per_chunk;
  const char* base = static_cast<const char*>(it.grad) + first * es;
  double acc = 0.0;
  if (it.aligned && count == per_chunk) {
    // 16 bytes per thread per pass
#pragma unroll 4
    for (int off = threadIdx.x * 16; off < kClipChunkBytes; off += kClipThreads * 16) {
      const u32x4_t v = ld16(base + off);
      if (it.dtype == DT_BF16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          accum<P>(acc, bf16_to_f32(v[e] & 0xffffu), p);
          accum<P>(acc, bf16_to_f32(v[e] >> 16), p);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) accum<P>(acc, __uint_as_float(v[e]), p);
      }
    }
  } else {
    for (int64_t i = threadIdx.x; i < count; i += kClipThreads) {
      const float x = it.dtype == DT_BF16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[i])
                                          : reinterpret_cast<const float*>(base)[i];
      accum<P>(acc, x, p);
    }
  }
  const double r = block_reduce<P, kClipThreads>(acc, lds);
  if (threadIdx.x == 0) partials[b] = r;
}

// one block per bucket; each thread keeps eight independent partial sums so
// that eight loads are in flight at once (the order is fixed, so the result
// is deterministic)
template <int P>
__global__ void __launch_bounds__(kClipFinalizeThreads)
clip_finalize_kernel(const int64_t* __restrict__ bucket_blocks, const double* __restrict__ max_norm,
                     const double* __restrict__ partials, double p, double* __restrict__ total_out,
                     double* __restrict__ coef_out) {
  __shared__ double lds[kClipFinalizeThreads / 64];
  const int bk = blockIdx.x;
  const int64_t lo = bucket_blocks[bk], hi = bucket_blocks[bk + 1];
  constexpr int kIlp = 8;
  double acc[kIlp];
#pragma unroll
  for (int u = 0; u < kIlp; ++u) acc[u] = 0.0;
  for (int64_t i = lo + threadIdx.x; i < hi; i += kIlp * kClipFinalizeThreads) {
#pragma unroll
    for (int u = 0; u < kIlp; ++u) {
      const int64_t j = i + int64_t(u) * kClipFinalizeThreads;
      if (j < hi) acc[u] = combine<P>(acc[u], partials[j]);
    }
  }
#pragma unroll
  for (int w = kIlp / 2; w > 0; w >>= 1)
#pragma unroll
    for (int u = 0; u < w; ++u) acc[u] = combine<P>(acc[u], acc[u + w]);
  const double s = block_reduce<P, kClipFinalizeThreads>(acc[0], lds);
  if (threadIdx.x == 0) {
    double total;
    if constexpr (P == 1 || P == 3) total = s;
    else if constexpr (P == 2) total = sqrt(s);
    else total = pow(s, 1.0 / p);
    const double c = max_norm[bk] / (total + 1e-6);
    const double coef = c >= 1.0 ? 1.0 : c;   // a NaN stays NaN
    if (total_out) total_out[bk] = total;
    coef_out[bk] = coef;
  }
}

__global__ void __launch_bounds__(kClipThreads)
clip_scale_kernel(const ClipItem* __restrict__ items, int n, const double* __restrict__ coefs) {
  const int64_t b = blockIdx.x;
  const ClipItem& it = items[find_item(items, n, b)];
  const double c = coefs[it.bucket];
  if (c == 1.0) return;
  const int es = it.dtype == DT_BF16 ? 2 : 4;
  const int64_t per_chunk = kClipChunkBytes / es;
  const int64_t first = (b - it.blk_first) * per_chunk;
  const int64_t count = it.numel - first < per_chunk ? it.numel - first : per_chunk;
  char* base = static_cast<char*>(it.grad) + first * es;
  if (it.aligned && count == per_chunk) {
#pragma unroll 4
    for (int off = threadIdx.x * 16; off < kClipChunkBytes; off += kClipThreads * 16) {
      u32x4_t v = ld16(base + off);
      if (it.dtype == DT_BF16) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = pack2_from_f64(static_cast<double>(bf16_to_f32(v[e] & 0xffffu)) * c,
                                static_cast<double>(bf16_to_f32(v[e] >> 16)) * c);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = __float_as_uint(static_cast<float>(static_cast<double>(__uint_as_float(v[e])) * c));
      }
      st16(base + off, v);
    }
  } else {
    for (int64_t i = threadIdx.x; i < count; i += kClipThreads) {
      if (it.dtype == DT_BF16) {
        uint16_t* q = reinterpret_cast<uint16_t*>(base) + i;
        const double x = static_cast<double>(bf16_to_f32(*q)) * c;
        *q = static_cast<uint16_t>(pack2_from_f64(x, 0.0) & 0xffffu);
      } else {
        float* q = reinterpret_cast<float*>(base) + i;
        *q = static_cast<float>(static_cast<double>(*q) * c);
      }
    }
  }
}

}  // namespace

namespace {
int clip_mode(double p) { return p == 1.0 ? 1 : p == 2.0 ? 2 : (p > 1e308) ? 3 : 0; }
}  // namespace

hipError_t launch_clip_norm(const ClipItem* items_dev, int n, int64_t nblocks, double p, double* partials,
                            hipStream_t stream) {
  if (nblocks <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(nblocks)), block(kClipThreads);
  switch (clip_mode(p)) {
    case 1: hipLaunchKernelGGL(clip_norm_kernel<1>, grid, block, 0, stream, items_dev, n, p, partials); break;
    case 2: hipLaunchKernelGGL(clip_norm_kernel<2>, grid, block, 0, stream, items_dev, n, p, partials); break;
    case 3: hipLaunchKernelGGL(clip_norm_kernel<3>, grid, block, 0, stream, items_dev, n, p, partials); break;
    default: hipLaunchKernelGGL(clip_norm_kernel<0>, grid, block, 0, stream, items_dev, n, p, partials); break;
  }
  return hipGetLastError();
}

hipError_t launch_clip_finalize(const int64_t* bucket_blocks_dev, int nbuckets, const double* max_norm_dev,
                                const double* partials, double p, double* total_out, double* coefs,
                                hipStream_t stream) {
  if (nbuckets <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(nbuckets)), block(kClipFinalizeThreads);
  switch (clip_mode(p)) {
    case 1: hipLaunchKernelGGL(clip_finalize_kernel<1>, grid, block, 0, stream, bucket_blocks_dev, max_norm_dev, partials, p, total_out, coefs); break;
    case 2: hipLaunchKernelGGL(clip_finalize_kernel<2>, grid, block, 0, stream, bucket_blocks_dev, max_norm_dev, partials, p, total_out, coefs); break;
    case 3: hipLaunchKernelGGL(clip_finalize_kernel<3>, grid, block, 0, stream, bucket_blocks_dev, max_norm_dev, partials, p, total_out, coefs); break;
    default: hipLaunchKernelGGL(clip_finalize_kernel<0>, grid, block, 0, stream, bucket_blocks_dev, max_norm_dev, partials, p, total_out, coefs); break;
  }
  return hipGetLastError();
}

hipError_t launch_clip_scale(const ClipItem* items_dev, int n, int64_t nblocks, const double* coefs,
                             hipStream_t stream) {
  if (nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(clip_scale_kernel, dim3(static_cast<unsigned>(nblocks)), dim3(kClipThreads), 0, stream,
                     items_dev, n, coefs);
  return hipGetLastError();
}

}  // namespace dmuon
