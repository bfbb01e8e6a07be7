// Grouped Newton-Schulz products for gfx950.
//
// Every product of the NS iteration is one GemmTask of the single form
//   C[i][j] = alpha_eff * sum_k A[i][k] B[j][k] + beta_eff * Y[i][j] + gamma*I
// with both operands K-contiguous:
//   direct form:  A = X X^T,  B = bA + c A A,  X' = aX + B X = NT(B, X^T)
//   Gram form:    R = X0 X0^T, P = aI + bA + cA A, Q <- P Q, T = P A,
//                 A <- T P, O = Q X0 = NT(Q, X0^T)
// (every m x m matrix is a polynomial in the Gram matrix, hence symmetric, so
// B A^T = B A; the m x n operand is kept in both orientations, X and X^T).
// Symmetric results run only the tiles with tm <= tn and store the upper
// triangle twice, which makes them exactly symmetric.
//
// A launch covers one stage of every matrix in a ragged batch: block b reads
// its task and output tile from a host-built map (XCD-aware and 2-D blocked
// for L2 reuse).
//
// bf16 kernel: BT x BT output tiles (BT = 256 or 128), four waves in a 2 x 2
// grid, each a (BT/2 x BT/2) block of v_mfma_f32_32x32x16_bf16 fragments with
// fp32 accumulators.  Operands stream through a four-stage LDS ring, 32 k per
// stage, filled by direct-to-LDS loads (global_load_lds_dwordx4: lane l of a
// wave writes bytes 16l..16l+15 of a 1 KB LDS block).  LDS rows are 64 bytes
// (four 16-byte chunks); chunk c of row r sits in slot c ^ (((r>>1)^(r>>2)) & 3),
// which the loads realise by choosing each lane's source address, and which
// makes the fragment reads (32 rows x one chunk per half-wave) bank-conflict
// free for any 16 consecutive rows (the LDS serves 16 lanes of a 128-bit
// read per cycle; a swizzle on bits 1..2 alone leaves rows r and r+8 in one
// bank, which the bank-conflict counter shows).  Loads run two stages ahead of the multiplies; fragment reads for the
// next half-stage are issued before the current half-stage's MFMAs, with one
// barrier per stage placed between its two halves.
//
// fp32 kernel (the fp32 NS mode): 64 x 64 x 16 tiles, four waves of 32 x 32,
// v_mfma_f32_32x32x2f32, register-staged k-major LDS.
#include <cstdlib>

#include "internal.h"

namespace dmuon {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ float spow(float s, int p) { return p == 0 ? 1.f : p == 1 ? s : s * s; }

// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Epilogue of one 32 x 32 accumulator fragment.  The lane holds column col and
// rows row0 + 8g + r (g, r = 0..3); row0 already carries the 4*(lane/32)
// offset.  mode 0: plain store; 1: store and mirror (off-diagonal symmetric
// tile); 2: diagonal symmetric tile (upper triangle stored and mirrored);
// 3: store, and store the transpose into Ct.
template <bool HAS_Y, typename OutT>
__device__ __forceinline__ void store_fragment(const f32x16_t& a, OutT* __restrict__ C, int64_t ldc,
                                               OutT* __restrict__ Ct, int64_t ldct,
                                               const OutT* __restrict__ Y, int64_t ldy, int row0,
                                               int col, float alpha, float beta, float gamma,
                                               int diag_limit, int mode) {
  constexpr bool BF = sizeof(OutT) == 2;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int rg = row0 + g * 8;
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = rg + r;
      float x = alpha * a[g * 4 + r];
      if constexpr (HAS_Y) {
        const OutT y = Y[int64_t(row) * ldy + col];
        float yf;
        if constexpr (BF) yf = bf16_bits_to_f32(y); else yf = y;
        x = fmaf(beta, yf, x);
      }
      x += (row == col && row < diag_limit) ? gamma : 0.f;
      v[r] = x;
    }
    OutT h[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (BF) h[r] = static_cast<OutT>(f32_to_bf16_bits(v[r])); else h[r] = v[r];
    }
    if (mode == 2) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (rg + r <= col) {
          C[int64_t(rg + r) * ldc + col] = h[r];
          C[int64_t(col) * ldc + rg + r] = h[r];
        }
      }
      continue;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) C[int64_t(rg + r) * ldc + col] = h[r];
    if (mode == 1 || mode == 3) {
      OutT* dst = mode == 1 ? C + int64_t(col) * ldc + rg : Ct + int64_t(col) * ldct + rg;
      if constexpr (BF) {
        *reinterpret_cast<uint2*>(dst) =
            make_uint2(uint32_t(h[0]) | (uint32_t(h[1]) << 16), uint32_t(h[2]) | (uint32_t(h[3]) << 16));
      } else {
        *reinterpret_cast<float4*>(dst) = make_float4(h[0], h[1], h[2], h[3]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16
// ---------------------------------------------------------------------------

constexpr int kStageK = 32;                     // k per LDS stage
constexpr int kRowBytes = kStageK * 2;          // 64
constexpr int kRowsPerLoad = 1024 / kRowBytes;  // rows filled by one wave-wide DMA load

// Column swizzle of the fp32 staging tile (row r, column c at r*BT + (c ^
// stage_swz(r))): conflict-free for the accumulator writes (32 columns of rows
// r and r+4 per instruction), the row reads (two aligned 16-byte pieces per
// 8 columns) and the column reads (16 row-groups x 4 columns).
__device__ __forceinline__ int stage_swz(int r) { return (((r >> 3) & 15) << 2) ^ (((r >> 2) & 1) << 5); }

__device__ __forceinline__ int slot_of(int row, int chunk) { return chunk ^ (((row >> 1) ^ (row >> 2)) & 3); }

template <int BT, int kStages>
__global__ void __launch_bounds__(256)
gemm_bf16_kernel(const GemmTask* __restrict__ tasks, const TileRef* __restrict__ map) {
  constexpr int WT = BT / 2;                       // wave tile edge
  constexpr int F = WT / 32;                       // fragments per wave edge
  constexpr int OPB = BT * kRowBytes;              // bytes of one operand in one stage
  constexpr int STB = 2 * OPB;                     // bytes of one stage
  constexpr int LOADS_PER_OP = BT / kRowsPerLoad;  // DMA loads per operand per stage
  constexpr int LOADS = 2 * LOADS_PER_OP / 4;      // DMA loads per wave per stage
  static_assert(LOADS >= 1 && (2 * LOADS_PER_OP) % 4 == 0, "tile");

  __shared__ __attribute__((aligned(1024))) char smem[kStages * STB];

  const TileRef ref = map[blockIdx.x];
  const int tm = ref.tm, tn = ref.tn;
  const GemmTask& T = tasks[ref.task];
  const int nk = T.K / kStageK;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // DMA sources: load q of this wave fills LDS block idx = wave + 4q of the
  // stage (blocks 0 .. LOADS_PER_OP-1: A rows, the rest: B rows); lane l
  // writes slot l%4 of row 16*block + l/4, which holds chunk slot^swizzle.
  const uint16_t* src[LOADS];
  int dst_off[LOADS];
#pragma unroll
  for (int q = 0; q < LOADS; ++q) {
    const int idx = wave + 4 * q;
    const bool is_b = idx >= LOADS_PER_OP;
    const int blk = is_b ? idx - LOADS_PER_OP : idx;
    const int row = blk * kRowsPerLoad + (lane >> 2);
    const int chunk = slot_of(row, lane & 3);
    const uint16_t* base = is_b ? static_cast<const uint16_t*>(T.B) + (int64_t(tn) * BT + row) * T.ldb
                                : static_cast<const uint16_t*>(T.A) + (int64_t(tm) * BT + row) * T.lda;
    src[q] = base + chunk * 8;
    dst_off[q] = (is_b ? OPB : 0) + blk * 1024;
  }

  // fragment read offsets (bytes within a stage) for the two k-halves
  int frag_off[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int r = lane & 31;
    frag_off[kk] = r * kRowBytes + slot_of(r, kk * 2 + (lane >> 5)) * 16;
  }

  f32x16_t acc[F][F];
#pragma unroll
  for (int i = 0; i < F; ++i)
#pragma unroll
    for (int j = 0; j < F; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // stage `data` of the operands into ring slot `slot % kStages`
  auto issue_stage = [&](int data, int slot) {
    char* st = smem + (slot % kStages) * STB;
#pragma unroll
    for (int q = 0; q < LOADS; ++q)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src[q] + data * kStageK),
                                       (LDS_AS void*)(st + dst_off[q]), 16, 0, 0);
  };
  auto read_frags = [&](int s, int kk, bf16x8_t (&fa)[F], bf16x8_t (&fb)[F]) {
    const char* st = smem + (s % kStages) * STB + frag_off[kk];
#pragma unroll
    for (int i = 0; i < F; ++i)
      fa[i] = *reinterpret_cast<const bf16x8_t*>(st + (wm * WT + i * 32) * kRowBytes);
#pragma unroll
    for (int j = 0; j < F; ++j)
      fb[j] = *reinterpret_cast<const bf16x8_t*>(st + OPB + (wn * WT + j * 32) * kRowBytes);
  };
  auto mfmas = [&](const bf16x8_t (&fa)[F], const bf16x8_t (&fb)[F]) {
#pragma unroll
    for (int i = 0; i < F; ++i)
#pragma unroll
      for (int j = 0; j < F; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };

  // The loop is branch-free: past the last stage, loads re-fetch the last
  // stage's data (in bounds) into buffers that are never read again, and the
  // fragment reads re-read the last stage, so every iteration issues the
  // same number of loads and the wait counts are constants.
  // prologue: stages 0 .. kStages-2 in flight, then stage 0 complete
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s) issue_stage(s < nk ? s : nk - 1, s);
  wait_vmcnt<LOADS * (kStages - 2)>();
  __builtin_amdgcn_s_barrier();

  // Instruction order is pinned with scheduling groups (the compiler would
  // otherwise sink each fragment read to just before its first use): the
  // in-order issue must never run out of independent MFMAs while loads and
  // LDS reads are issued.
  constexpr int kMfma = 0x008, kVmem = 0x010, kDsRead = 0x100;
  constexpr int NFRAG = 2 * F;          // fragment reads per half-stage
  constexpr int NMFMA = F * F;          // MFMAs per half-stage
  bf16x8_t fa0[F], fb0[F], fa1[F], fb1[F];
  read_frags(0, 0, fa0, fb0);
  for (int kt = 0; kt < nk; ++kt) {
    // phase A: first k-half of stage kt; the second half's fragments load
    read_frags(kt, 1, fa1, fb1);
    mfmas(fa0, fb0);
#pragma unroll
    for (int i = 0; i < NFRAG; ++i) {
      __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kMfma, NMFMA - NFRAG, 0);
    __builtin_amdgcn_sched_barrier(0);
    // stage kt+1 complete in this wave (kStages-3 later stages in flight),
    // then in every wave; all waves are past stage kt-1, whose buffer the
    // next load overwrites
    wait_vmcnt<LOADS * (kStages - 3)>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // phase B: second k-half of stage kt; loads for stage kt+kStages-1 and
    // the first-half fragments of stage kt+1 are issued in between
    const int ahead = kt + kStages - 1;
    issue_stage(ahead < nk ? ahead : nk - 1, ahead);
    read_frags(kt + 1 < nk ? kt + 1 : nk - 1, 0, fa0, fb0);
    mfmas(fa1, fb1);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      __builtin_amdgcn_sched_group_barrier(kVmem, 1, 1);
      __builtin_amdgcn_sched_group_barrier(kMfma, 1, 1);
    }
#pragma unroll
    for (int i = 0; i < NFRAG; ++i) {
      __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 1);
      if (LOADS + i < NMFMA) __builtin_amdgcn_sched_group_barrier(kMfma, 1, 1);
    }
    if (NMFMA > LOADS + NFRAG) __builtin_amdgcn_sched_group_barrier(kMfma, NMFMA - LOADS - NFRAG, 1);
    __builtin_amdgcn_sched_barrier(0);
  }
  // no load may still be writing this block's LDS when the block retires
  wait_vmcnt<0>();

  // Epilogue through LDS (the ring is free once the loads have drained): the
  // accumulators are staged in fp32, then written out with 16-byte,
  // row-contiguous stores -- C row by row, and the mirror (symmetric tiles)
  // or the transposed copy Ct column by column of the staged tile.
  __syncthreads();
  const float s = T.scale ? *T.scale : 1.f;
  const float alpha = T.alpha * spow(s, T.alpha_pow);
  const float beta = T.beta * spow(s, T.beta_pow);
  const float gamma = T.gamma;
  const int diag_limit = T.diag_limit;
  uint16_t* __restrict__ C = static_cast<uint16_t*>(T.C);
  uint16_t* __restrict__ Ct = static_cast<uint16_t*>(T.Ct);
  const uint16_t* __restrict__ Y = static_cast<const uint16_t*>(T.Y);
  const int64_t ldc = T.ldc, ldct = T.ldct, ldy = T.ldy;
  const int mode = T.sym ? (tm != tn ? 1 : 2) : (Ct ? 3 : 0);   // 0 plain, 1 mirror, 2 diagonal, 3 Ct
  uint16_t* const Tdst = mode == 3 ? Ct : C;
  const int64_t ldt = mode == 3 ? ldct : ldc;

  constexpr int RING = kStages * STB;
  constexpr int ROWS = RING >= BT * BT * 4 ? BT : WT;   // staged rows per pass
  static_assert(RING >= WT * BT * 4, "staging does not fit");
  constexpr int CPR = BT / 8;                           // 8-wide chunks per staged row
  constexpr int CH = ROWS / 8;                          // 8-long chunks per transposed row
  float* const stg = reinterpret_cast<float*>(smem);
  const int t = threadIdx.x;

  for (int pass = 0; pass < BT / ROWS; ++pass) {
    const int r_lo = pass * ROWS;
    if (pass > 0) __syncthreads();
    if (wm * WT >= r_lo && wm * WT < r_lo + ROWS) {
#pragma unroll
      for (int i = 0; i < F; ++i)
#pragma unroll
        for (int j = 0; j < F; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int r = wm * WT - r_lo + i * 32 + (lane >> 5) * 4 + g * 8 + rr;
              const int c = wn * WT + j * 32 + (lane & 31);
              stg[r * BT + (c ^ stage_swz(r))] = alpha * acc[i][j][g * 4 + rr];
            }
    }
    __syncthreads();

    // rows: thread t covers chunk t % CPR of staged rows t / CPR + (256 / CPR) k
#pragma unroll 4
    for (int k = 0; k < ROWS * CPR / 256; ++k) {
      const int lr = t / CPR + (256 / CPR) * k;
      const int c0 = (t % CPR) * 8;
      const int rt = r_lo + lr;                 // row within the tile
      const int64_t R = int64_t(tm) * BT + rt;  // row within C
      const int64_t C0 = int64_t(tn) * BT + c0;
      float* const lo = stg + lr * BT + ((c0 ^ stage_swz(lr)) & ~3);
      float* const hi = stg + lr * BT + (((c0 + 4) ^ stage_swz(lr)) & ~3);
      float4 a = *reinterpret_cast<const float4*>(lo);
      float4 b = *reinterpret_cast<const float4*>(hi);
      float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      if (Y) {
        const uint4 y = *reinterpret_cast<const uint4*>(Y + R * ldy + C0);
        const uint32_t yw[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          v[e] = fmaf(beta, bf16_bits_to_f32((yw[e >> 1] >> ((e & 1) * 16)) & 0xffffu), v[e]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] += (R == C0 + e && R < diag_limit) ? gamma : 0.f;
      if (mode != 0) {
        *reinterpret_cast<float4*>(lo) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(hi) = make_float4(v[4], v[5], v[6], v[7]);
      }
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = f32_to_bf16_bits(v[e]);
      uint16_t* dst = C + R * ldc + C0;
      if (mode != 2 || c0 >= rt) {
        *reinterpret_cast<uint4*>(dst) =
            make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
      } else if (c0 + 7 >= rt) {   // diagonal tile: upper triangle only
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (c0 + e >= rt) dst[e] = static_cast<uint16_t>(h[e]);
      }
    }

    // transposed: thread t covers chunk t % CH (8 staged rows) of staged
    // column t / CH + (256 / CH) k
    if (mode != 0) {
      __syncthreads();
#pragma unroll 4
      for (int k = 0; k < BT * CH / 256; ++k) {
        const int c = t / CH + (256 / CH) * k;   // column within the tile
        const int q = t % CH;
        const int r0 = 8 * q;                    // first staged row
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = f32_to_bf16_bits(stg[(r0 + i) * BT + (c ^ stage_swz(r0 + i))]);
        uint16_t* dst = Tdst + (int64_t(tn) * BT + c) * ldt + int64_t(tm) * BT + r_lo + r0;
        const int rt0 = r_lo + r0;               // tile row of element i = rt0 + i
        if (mode != 2 || rt0 + 7 < c) {
          *reinterpret_cast<uint4*>(dst) =
              make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
        } else if (rt0 < c) {      // diagonal tile: strict lower triangle only
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (rt0 + i < c) dst[i] = static_cast<uint16_t>(h[i]);
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

__device__ __forceinline__ float4 gload16f(const float* p) {
  const f32x4_t v = *reinterpret_cast<const __attribute__((address_space(1))) f32x4_t*>(
      reinterpret_cast<uintptr_t>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

__global__ void __launch_bounds__(256)
gemm_f32_kernel(const GemmTask* __restrict__ tasks, const TileRef* __restrict__ map) {
  constexpr int BM = kF32Tile, BN = kF32Tile, BK = kF32BK;
  __shared__ __attribute__((aligned(16))) float As[2][BK][BM + kF32Pad];
  __shared__ __attribute__((aligned(16))) float Bs[2][BK][BN + kF32Pad];

  const TileRef ref = map[blockIdx.x];
  const int tm = ref.tm, tn = ref.tn;
  const GemmTask& T = tasks[ref.task];
  const int64_t lda = T.lda, ldb = T.ldb;
  const float* __restrict__ A = static_cast<const float*>(T.A) + int64_t(tm) * BM * lda;
  const float* __restrict__ B = static_cast<const float*>(T.B) + int64_t(tn) * BN * ldb;
  const int nk = T.K / BK;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // thread t stages row t/4, k = 4*(t%4) .. +3 of both operands
  const int arow = t >> 2, akc = (t & 3) * 4;

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
      Bs[buf][akc + 0][arow] = rb.x;
      Bs[buf][akc + 1][arow] = rb.y;
      Bs[buf][akc + 2][arow] = rb.z;
      Bs[buf][akc + 3][arow] = rb.w;
      __syncthreads();
    }
    if (kt < nk) {
      const int k0 = kt * BK;
      ra = gload16f(A + int64_t(arow) * lda + k0 + akc);
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
  float* __restrict__ C = static_cast<float*>(T.C);
  float* __restrict__ Ct = static_cast<float*>(T.Ct);
  const float* __restrict__ Y = static_cast<const float*>(T.Y);
  const int mode = T.sym ? (tm != tn ? 1 : 2) : (Ct ? 3 : 0);
  const int row0 = tm * BM + wm * 32 + (lane >> 5) * 4;
  const int col = tn * BN + wn * 32 + (lane & 31);
  if (Y)
    store_fragment<true>(acc, C, T.ldc, Ct, T.ldct, Y, T.ldy, row0, col, alpha, beta, T.gamma,
                         T.diag_limit, mode);
  else
    store_fragment<false>(acc, C, T.ldc, Ct, T.ldct, Y, T.ldy, row0, col, alpha, beta, T.gamma,
                          T.diag_limit, mode);
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmTask* tasks_dev, const TileRef* map_dev, int64_t ntiles,
                            int tile, hipStream_t stream) {
  if (ntiles <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(ntiles));
  // ring depth: tuning knob for measurements (DMUON_GEMM_STAGES), default below
  static const int stages_env = [] {
    const char* v = std::getenv("DMUON_GEMM_STAGES");
    return v ? std::atoi(v) : 0;
  }();
  if (tile == 128) {
    if (stages_env == 8)
      hipLaunchKernelGGL((gemm_bf16_kernel<128, 8>), grid, dim3(256), 0, stream, tasks_dev, map_dev);
    else
      hipLaunchKernelGGL((gemm_bf16_kernel<128, 4>), grid, dim3(256), 0, stream, tasks_dev, map_dev);
  } else if (tile == 256) {
    if (stages_env == 4)
      hipLaunchKernelGGL((gemm_bf16_kernel<256, 4>), grid, dim3(256), 0, stream, tasks_dev, map_dev);
    else
      hipLaunchKernelGGL((gemm_bf16_kernel<256, 5>), grid, dim3(256), 0, stream, tasks_dev, map_dev);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmTask* tasks_dev, const TileRef* map_dev, int64_t ntiles,
                           int tile, hipStream_t stream) {
  if (ntiles <= 0) return hipSuccess;
  if (tile != kF32Tile) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_f32_kernel, dim3(static_cast<unsigned>(ntiles)), dim3(256), 0, stream,
                     tasks_dev, map_dev);
  return hipGetLastError();
}

}  // namespace dmuon
