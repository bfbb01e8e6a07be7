// Grouped Newton-Schulz products for gfx950.
//
// Every product of the NS iteration (direct form: A = X X^T, B = bA + cA^2,
// X <- aX + B X; Gram form: R = X X^T, P = aI + bA + cA^2, Q <- P Q,
// A <- (P A) P, O = Q X0) is one GemmTask.  A launch covers the same stage of
// every matrix in a ragged batch: block b finds its task by binary search over
// the tasks' first-tile indices.  Two operand forms are needed:
//   NT  C[i][j] = sum_k A[i][k] B[j][k]   -- X X^T and every m x m product
//        (all of them are polynomials in the Gram matrix, hence symmetric:
//        only tiles with tm <= tn run, and each is stored twice)
//   NN  C[i][j] = sum_k A[i][k] B[k][j]   -- the m x m by m x n products
// Epilogue: C = alpha_eff*acc + beta_eff*Y + gamma*I, with the per-matrix
// normalisation 1/(||U||+eps) folded into alpha/beta as a power of s.
//
// bf16 path: 128 x 128 x 64 block tiles, four waves of 64 x 64, each a 2 x 2
// grid of v_mfma_f32_32x32x16_bf16 with fp32 accumulators.  Both operands sit
// in LDS as [row][k] with 128-byte rows whose 16-byte chunks are XOR-swizzled
// by (row ^ row>>3) & 7, so the MFMA fragment reads (32 rows, one chunk) and
// the staging writes are bank-conflict free.  The NN B operand (k-major in
// HBM) is transposed in registers while staging: each thread loads a 4 x 8
// (k x n) block with four 16-byte loads and writes eight 8-byte k-runs.
// Global loads of tile k+1 are in flight while tile k is multiplied (register
// staging, two LDS buffers, one barrier per k step).
//
// fp32 path (the fp32 NS mode): 64 x 64 x 16 tiles, four waves of 32 x 32,
// v_mfma_f32_32x32x2f32, LDS held k-major.
#include "internal.h"

namespace dmuon {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Task and tile coordinates of block `tile`.
__device__ __forceinline__ void locate(const GemmTask* __restrict__ tasks, int ntasks, int tile,
                                       int& ti, int& tm, int& tn) {
  int lo = 0, hi = ntasks - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tasks[mid].tile_begin <= tile) lo = mid; else hi = mid - 1;
  }
  ti = lo;
  int local = tile - tasks[lo].tile_begin;
  const int tn_count = tasks[lo].tiles_n;
  if (tasks[lo].sym) {
    // upper triangle, row by row: row r holds tn_count - r tiles
    int r = 0, len = tn_count;
    while (local >= len) { local -= len; ++r; --len; }
    tm = r;
    tn = r + local;
  } else {
    tm = local / tn_count;
    tn = local - tm * tn_count;
  }
}

__device__ __forceinline__ float spow(float s, int p) { return p == 0 ? 1.f : p == 1 ? s : s * s; }

// ---------------------------------------------------------------------------
// bf16
// ---------------------------------------------------------------------------

constexpr int kBK = 64;  // k extent of one LDS tile (128 bytes of bf16 per row)

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
// byte offset of 16-byte chunk kc of row r of a [rows][64] bf16 tile
__device__ __forceinline__ int lds_off(int r, int kc) { return r * 128 + ((kc ^ swz(r)) << 4); }

__device__ __forceinline__ uint32_t dword_of(const uint4& v, int d) {
  return d < 2 ? (d == 0 ? v.x : v.y) : (d == 2 ? v.z : v.w);
}

// 16-byte loads through the global address space (the task pointers are
// generic; all of them point to device memory).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 gload16(const uint16_t* p) {
  const u32x4_t v = *reinterpret_cast<const __attribute__((address_space(1))) u32x4_t*>(
      reinterpret_cast<uintptr_t>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float4 gload16f(const float* p) {
  const f32x4_t v = *reinterpret_cast<const __attribute__((address_space(1))) f32x4_t*>(
      reinterpret_cast<uintptr_t>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

template <int BM, int BN, int WM, int WN, bool NN>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_bf16_kernel(const GemmTask* __restrict__ tasks, int ntasks) {
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int CA = BM * 8 / NT;                       // A chunks per thread
  constexpr int CB = NN ? (2 * BN / NT) : (BN * 8 / NT);  // NN: 4x8 blocks; NT: chunks
  static_assert(CA >= 1 && CB >= 1 && FM >= 1 && FN >= 1, "tile shape");
  constexpr int RB = NN ? 4 * CB : CB;

  __shared__ __attribute__((aligned(16))) char smem[2 * (BM + BN) * 128];
  char* const As = smem;
  char* const Bs = smem + 2 * BM * 128;

  int ti, tm, tn;
  locate(tasks, ntasks, blockIdx.x, ti, tm, tn);
  const GemmTask& T = tasks[ti];
  const int64_t lda = T.lda, ldb = T.ldb;
  const uint16_t* __restrict__ A = static_cast<const uint16_t*>(T.A) + int64_t(tm) * BM * lda;
  const uint16_t* __restrict__ B = NN ? static_cast<const uint16_t*>(T.B) + int64_t(tn) * BN
                                      : static_cast<const uint16_t*>(T.B) + int64_t(tn) * BN * ldb;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave / WN, wn = wave % WN;

  uint4 ra[CA];
  uint4 rb[RB];
  const int nk = T.K / kBK;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  for (int kt = 0; kt <= nk; ++kt) {
    // stage tile kt (loaded during the previous iteration) into LDS buffer kt&1
    if (kt > 0) {
      char* as = As + ((kt - 1) & 1) * BM * 128;
      char* bs = Bs + ((kt - 1) & 1) * BN * 128;
#pragma unroll
      for (int c = 0; c < CA; ++c) {
        const int chunk = t + NT * c;
        *reinterpret_cast<uint4*>(as + lds_off(chunk >> 3, chunk & 7)) = ra[c];
      }
      if constexpr (NN) {
#pragma unroll
        for (int q = 0; q < CB; ++q) {
          const int blk = t + NT * q;
          const int rest = blk >> 4;
          const int nb = (blk & 7) + 8 * (rest % (BN / 64));
          const int kb = 2 * (rest / (BN / 64)) + ((blk >> 3) & 1);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            // element n = 8nb + e of the four k rows 4kb .. 4kb+3
            const int sh = (e & 1) * 16;
            const uint32_t x0 = (dword_of(rb[4 * q + 0], e >> 1) >> sh) & 0xffffu;
            const uint32_t x1 = (dword_of(rb[4 * q + 1], e >> 1) >> sh) & 0xffffu;
            const uint32_t x2 = (dword_of(rb[4 * q + 2], e >> 1) >> sh) & 0xffffu;
            const uint32_t x3 = (dword_of(rb[4 * q + 3], e >> 1) >> sh) & 0xffffu;
            *reinterpret_cast<uint2*>(bs + lds_off(8 * nb + e, kb >> 1) + (kb & 1) * 8) =
                make_uint2(x0 | (x1 << 16), x2 | (x3 << 16));
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < CB; ++c) {
          const int chunk = t + NT * c;
          *reinterpret_cast<uint4*>(bs + lds_off(chunk >> 3, chunk & 7)) = rb[c];
        }
      }
      __syncthreads();
    }
    // issue the global loads of tile kt (consumed at the top of the next iteration)
    if (kt < nk) {
      const int k0 = kt * kBK;
#pragma unroll
      for (int c = 0; c < CA; ++c) {
        const int chunk = t + NT * c;
        ra[c] = gload16(A + int64_t(chunk >> 3) * lda + k0 + (chunk & 7) * 8);
      }
      if constexpr (NN) {
#pragma unroll
        for (int q = 0; q < CB; ++q) {
          const int blk = t + NT * q;
          const int rest = blk >> 4;
          const int nb = (blk & 7) + 8 * (rest % (BN / 64));
          const int kb = 2 * (rest / (BN / 64)) + ((blk >> 3) & 1);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            rb[4 * q + r] = gload16(B + int64_t(k0 + 4 * kb + r) * ldb + 8 * nb);
        }
      } else {
#pragma unroll
        for (int c = 0; c < CB; ++c) {
          const int chunk = t + NT * c;
          rb[c] = gload16(B + int64_t(chunk >> 3) * ldb + k0 + (chunk & 7) * 8);
        }
      }
    }
    // multiply tile kt-1 from LDS while tile kt is in flight
    if (kt > 0) {
      const char* as = As + ((kt - 1) & 1) * BM * 128;
      const char* bs = Bs + ((kt - 1) & 1) * BN * 128;
#pragma unroll
      for (int kk = 0; kk < kBK / 16; ++kk) {
        const int kc = kk * 2 + (lane >> 5);
        bf16x8_t fa[FM], fb[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
          fa[i] = *reinterpret_cast<const bf16x8_t*>(as + lds_off(wm * WTM + i * 32 + (lane & 31), kc));
#pragma unroll
        for (int j = 0; j < FN; ++j)
          fb[j] = *reinterpret_cast<const bf16x8_t*>(bs + lds_off(wn * WTN + j * 32 + (lane & 31), kc));
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
    }
  }

  // epilogue
  const float s = T.scale ? *T.scale : 1.f;
  const float alpha = T.alpha * spow(s, T.alpha_pow);
  const float beta = T.beta * spow(s, T.beta_pow);
  const float gamma = T.gamma;
  const int diag_limit = T.diag_limit;
  uint16_t* __restrict__ C = static_cast<uint16_t*>(T.C);
  const uint16_t* __restrict__ Y = static_cast<const uint16_t*>(T.Y);
  const int64_t ldc = T.ldc, ldy = T.ldy;
  // Symmetric results are made exactly symmetric: off-diagonal tiles are
  // stored and mirrored; diagonal tiles keep their upper triangle and mirror
  // it.  (Keeping a diagonal tile's own lower triangle, which differs from
  // the mirrored upper one by rounding wherever the factors do not commute
  // exactly, measurably degrades the bf16 Gram iteration.)
  const bool mirror = T.sym && tm != tn;
  const bool diag = T.sym && tm == tn;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = tn * BN + wn * WTN + j * 32 + (lane & 31);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row0 = tm * BM + wm * WTM + i * 32 + g * 8 + (lane >> 5) * 4;
        uint32_t h[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = row0 + r;
          float v = alpha * acc[i][j][g * 4 + r];
          if (Y) v = fmaf(beta, bf16_bits_to_f32(Y[int64_t(row) * ldy + col]), v);
          if (row == col && row < diag_limit) v += gamma;
          h[r] = f32_to_bf16_bits(v);
          if (!diag || row <= col) C[int64_t(row) * ldc + col] = static_cast<uint16_t>(h[r]);
        }
        if (mirror) {
          *reinterpret_cast<uint2*>(C + int64_t(col) * ldc + row0) =
              make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
        } else if (diag) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (row0 + r < col) C[int64_t(col) * ldc + row0 + r] = static_cast<uint16_t>(h[r]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32
// ---------------------------------------------------------------------------

constexpr int kF32Tile = 64;
constexpr int kF32BK = 16;
constexpr int kF32Pad = 4;

template <bool NN>
__global__ void __launch_bounds__(256)
gemm_f32_kernel(const GemmTask* __restrict__ tasks, int ntasks) {
  constexpr int BM = kF32Tile, BN = kF32Tile, BK = kF32BK;
  __shared__ __attribute__((aligned(16))) float As[2][BK][BM + kF32Pad];
  __shared__ __attribute__((aligned(16))) float Bs[2][BK][BN + kF32Pad];

  int ti, tm, tn;
  locate(tasks, ntasks, blockIdx.x, ti, tm, tn);
  const GemmTask& T = tasks[ti];
  const int64_t lda = T.lda, ldb = T.ldb;
  const float* __restrict__ A = static_cast<const float*>(T.A) + int64_t(tm) * BM * lda;
  const float* __restrict__ B = NN ? static_cast<const float*>(T.B) + int64_t(tn) * BN
                                   : static_cast<const float*>(T.B) + int64_t(tn) * BN * ldb;
  const int nk = T.K / BK;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // A (and NT B): thread t loads row t/4, k = 4*(t%4) .. +3
  const int arow = t >> 2, akc = (t & 3) * 4;
  // NN B: thread t loads k row t/16, n = 4*(t%16) .. +3
  const int bk = t >> 4, bnc = (t & 15) * 4;

  float4 ra = make_float4(0.f, 0.f, 0.f, 0.f), rb = ra;
  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;

  for (int kt = 0; kt <= nk; ++kt) {
    if (kt > 0) {
      const int buf = (kt - 1) & 1;
      As[buf][akc + 0][arow] = ra.x;
      As[buf][akc + 1][arow] = ra.y;
      As[buf][akc + 2][arow] = ra.z;
      As[buf][akc + 3][arow] = ra.w;
      if constexpr (NN) {
        *reinterpret_cast<float4*>(&Bs[buf][bk][bnc]) = rb;
      } else {
        Bs[buf][akc + 0][arow] = rb.x;
        Bs[buf][akc + 1][arow] = rb.y;
        Bs[buf][akc + 2][arow] = rb.z;
        Bs[buf][akc + 3][arow] = rb.w;
      }
      __syncthreads();
    }
    if (kt < nk) {
      const int k0 = kt * BK;
      ra = gload16f(A + int64_t(arow) * lda + k0 + akc);
      if constexpr (NN)
        rb = gload16f(B + int64_t(k0 + bk) * ldb + bnc);
      else
        rb = gload16f(B + int64_t(arow) * ldb + k0 + akc);
    }
    if (kt > 0) {
      const int cur = (kt - 1) & 1;
#pragma unroll
      for (int kk = 0; kk < BK / 2; ++kk) {
        const float a = As[cur][kk * 2 + (lane >> 5)][wm * 32 + (lane & 31)];
        const float b = Bs[cur][kk * 2 + (lane >> 5)][wn * 32 + (lane & 31)];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
      }
    }
  }

  const float s = T.scale ? *T.scale : 1.f;
  const float alpha = T.alpha * spow(s, T.alpha_pow);
  const float beta = T.beta * spow(s, T.beta_pow);
  const float gamma = T.gamma;
  const int diag_limit = T.diag_limit;
  float* __restrict__ C = static_cast<float*>(T.C);
  const float* __restrict__ Y = static_cast<const float*>(T.Y);
  const int64_t ldc = T.ldc, ldy = T.ldy;
  // exact symmetry as in the bf16 kernel
  const bool mirror = T.sym && tm != tn;
  const bool diag = T.sym && tm == tn;
  const int col = tn * BN + wn * 32 + (lane & 31);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int row0 = tm * BM + wm * 32 + g * 8 + (lane >> 5) * 4;
    float h[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row0 + r;
      float v = alpha * acc[g * 4 + r];
      if (Y) v = fmaf(beta, Y[int64_t(row) * ldy + col], v);
      if (row == col && row < diag_limit) v += gamma;
      h[r] = v;
      if (!diag || row <= col) C[int64_t(row) * ldc + col] = v;
    }
    if (mirror) {
      *reinterpret_cast<float4*>(C + int64_t(col) * ldc + row0) = make_float4(h[0], h[1], h[2], h[3]);
    } else if (diag) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (row0 + r < col) C[int64_t(col) * ldc + row0 + r] = h[r];
    }
  }
}

}  // namespace

hipError_t launch_gemm_bf16(GemmKind kind, const GemmTask* tasks_dev, int ntasks, int64_t ntiles,
                            int tile, hipStream_t stream) {
  if (ntiles <= 0) return hipSuccess;
  if (tile != 128) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(ntiles));
  if (kind == GemmKind::NT)
    hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, 2, 2, false>), grid, dim3(256), 0, stream,
                       tasks_dev, ntasks);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, 2, 2, true>), grid, dim3(256), 0, stream,
                       tasks_dev, ntasks);
  return hipGetLastError();
}

hipError_t launch_gemm_f32(GemmKind kind, const GemmTask* tasks_dev, int ntasks, int64_t ntiles,
                           int tile, hipStream_t stream) {
  if (ntiles <= 0) return hipSuccess;
  if (tile != kF32Tile) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(ntiles));
  if (kind == GemmKind::NT)
    hipLaunchKernelGGL((gemm_f32_kernel<false>), grid, dim3(256), 0, stream, tasks_dev, ntasks);
  else
    hipLaunchKernelGGL((gemm_f32_kernel<true>), grid, dim3(256), 0, stream, tasks_dev, ntasks);
  return hipGetLastError();
}

}  // namespace dmuon
