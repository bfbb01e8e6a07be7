// AdamW step of the symmetric (non-Muon) parameters (Training Guide, "Step 4:
// Create Optimizer": the second group runs standard AdamW; "Semantic Param
// Groups": per-group lr, betas, eps and weight decay), fused into one pass
// over every tensor of a call:
//   m <- beta1 m + (1 - beta1) g
//   v <- beta2 v + (1 - beta2) g^2
//   p <- p (1 - lr wd) - (lr / (1 - beta1^t)) m / (sqrt(v) / sqrt(1 - beta2^t) + eps)
// in fp32 with fp32 moments; a bf16 parameter is rounded once to nearest
// even.  HBM-bound: one block per 8192-element chunk of a tensor (binary
// search of the chunk's tensor), four elements per lane per pass, 16-byte
// non-temporal accesses when every stream of the tensor is 16-byte aligned.
#include "internal.h"

namespace dmuon {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
#define GLOBAL_AS __attribute__((address_space(1)))

template <class T>
__device__ __forceinline__ T ld_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const GLOBAL_AS T*>(reinterpret_cast<uintptr_t>(p)));
}
template <class T>
__device__ __forceinline__ void st_nt(void* p, T v) {
  __builtin_nontemporal_store(v, reinterpret_cast<GLOBAL_AS T*>(reinterpret_cast<uintptr_t>(p)));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

struct Upd {
  float p, m, v;
};

__device__ __forceinline__ Upd adam1(const AdamItem& it, float p, float g, float m, float v) {
  Upd r;
  r.m = fmaf(it.beta1, m, it.one_minus_beta1 * g);
  r.v = fmaf(it.beta2, v, it.one_minus_beta2 * (g * g));
  const float denom = fmaf(sqrtf(r.v), it.inv_sqrt_bc2, it.eps);
  r.p = fmaf(-it.step_size, r.m / denom, p * it.decay);
  return r;
}

__device__ __forceinline__ int find_item(const AdamItem* items, int n, int64_t b) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (items[mid].blk_first <= b) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ void __launch_bounds__(kAdamThreads)
adamw_kernel(const AdamItem* __restrict__ items, int n) {
  const int64_t b = blockIdx.x;
  const AdamItem it = items[find_item(items, n, b)];
  const int64_t first = (b - it.blk_first) * kAdamChunk;
  const int64_t count = it.numel - first < kAdamChunk ? it.numel - first : kAdamChunk;
  const bool pbf = it.p_dtype == DT_BF16, gbf = it.g_dtype == DT_BF16;
  char* pp = static_cast<char*>(it.p) + first * (pbf ? 2 : 4);
  const char* gp = static_cast<const char*>(it.g) + first * (gbf ? 2 : 4);
  float* mp = it.m + first;
  float* vp = it.v + first;
  if (it.aligned && count == kAdamChunk) {
#pragma unroll 2
    for (int e = threadIdx.x * 4; e < kAdamChunk; e += kAdamThreads * 4) {
      float p[4], g[4];
      if (pbf) {
        const u32x2_t w = ld_nt<u32x2_t>(pp + e * 2);
        p[0] = bf16_to_f32(w[0] & 0xffffu); p[1] = bf16_to_f32(w[0] >> 16);
        p[2] = bf16_to_f32(w[1] & 0xffffu); p[3] = bf16_to_f32(w[1] >> 16);
      } else {
        const f32x4_t w = ld_nt<f32x4_t>(pp + e * 4);
        p[0] = w[0]; p[1] = w[1]; p[2] = w[2]; p[3] = w[3];
      }
      if (gbf) {
        const u32x2_t w = ld_nt<u32x2_t>(gp + e * 2);
        g[0] = bf16_to_f32(w[0] & 0xffffu); g[1] = bf16_to_f32(w[0] >> 16);
        g[2] = bf16_to_f32(w[1] & 0xffffu); g[3] = bf16_to_f32(w[1] >> 16);
      } else {
        const f32x4_t w = ld_nt<f32x4_t>(gp + e * 4);
        g[0] = w[0]; g[1] = w[1]; g[2] = w[2]; g[3] = w[3];
      }
      const f32x4_t m = ld_nt<f32x4_t>(mp + e);
      const f32x4_t v = ld_nt<f32x4_t>(vp + e);
      f32x4_t mo, vo;
      float po[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const Upd u = adam1(it, p[k], g[k], m[k], v[k]);
        po[k] = u.p; mo[k] = u.m; vo[k] = u.v;
      }
      st_nt<f32x4_t>(mp + e, mo);
      st_nt<f32x4_t>(vp + e, vo);
      if (pbf) {
        const u32x2_t w = {pack_bf16x2(po[0], po[1]), pack_bf16x2(po[2], po[3])};
        st_nt<u32x2_t>(pp + e * 2, w);
      } else {
        const f32x4_t w = {po[0], po[1], po[2], po[3]};
        st_nt<f32x4_t>(pp + e * 4, w);
      }
    }
  } else {
    for (int64_t e = threadIdx.x; e < count; e += kAdamThreads) {
      const float p = pbf ? bf16_to_f32(reinterpret_cast<const uint16_t*>(pp)[e]) : reinterpret_cast<const float*>(pp)[e];
      const float g = gbf ? bf16_to_f32(reinterpret_cast<const uint16_t*>(gp)[e]) : reinterpret_cast<const float*>(gp)[e];
      const Upd u = adam1(it, p, g, mp[e], vp[e]);
      mp[e] = u.m;
      vp[e] = u.v;
      if (pbf)
        reinterpret_cast<uint16_t*>(pp)[e] = static_cast<uint16_t>(pack_bf16x2(u.p, 0.f) & 0xffffu);
      else
        reinterpret_cast<float*>(pp)[e] = u.p;
    }
  }
}

}  // namespace

hipError_t launch_adamw(const AdamItem* items_dev, int n, int64_t nblocks, hipStream_t stream) {
  if (nblocks <= 0 || n <= 0) return hipSuccess;
  hipLaunchKernelGGL(adamw_kernel, dim3(static_cast<unsigned>(nblocks)), dim3(kAdamThreads), 0, stream,
                     items_dev, n);
  return hipGetLastError();
}

}  // namespace dmuon
