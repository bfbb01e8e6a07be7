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
// grid, each a (BT/2 x BT/2) block with fp32 accumulators: 16 x 16 blocks of
// v_mfma_f32_16x16x32_bf16 for 256-tiles (under the power limit the
// smaller MFMA runs at a higher clock for the same flops), 32 x 32 blocks of
// v_mfma_f32_32x32x16_bf16 for 128-tiles.  Operands stream through a two-slot LDS ring of 64-k
// stages, filled by direct-to-LDS buffer loads (buffer_load_dwordx4 ... lds:
// lane l of a wave writes bytes 16l..16l+15 of a 1 KB LDS block; the base
// is a per-operand descriptor in scalar registers, the per-lane offsets are
// fixed).  An operand row of a
// stage is 128 bytes, one cache line; chunk c of row r sits in slot
// c ^ ((r >> 1) & 7), which the loads realise by choosing each lane's source
// address, so that a fragment read (16 rows x one 16-byte chunk per cycle)
// covers all 64 banks.  A stage runs as four k-quarters of 512 MFMA cycles
// per wave (32 16x16x32 or 16 32x32x16 MFMAs).  256-tiles hold a whole
// stage of fragments in registers (two 32-k steps): a stage's fragments are
// read within its first quarter and the quarter before, a
// barrier after that quarter frees its ring slot, and the loads of the stage
// two ahead go into the slot over the following four quarters, most of them
// in the two quarters without fragment reads; a second barrier after the
// third quarter makes the next stage visible (explicit wait counts, no
// fence, so the loads issued since stay in flight).  128-tiles interleave
// each quarter's MFMAs with the next quarter's reads, have one barrier per
// stage before its last quarter, and split the loads of the stage two ahead
// between that quarter and the next stage's first.  The last two stages are
// peeled so that nothing is loaded past the end.
// A diagonal tile of a product of a matrix with itself (A A, X X^T) loads its
// rows once: the B fragments are read from the A rows (a second instance of
// the loop, chosen per block).
// The epilogue stages the tile in the ring as bf16 and stores it row by row
// (and column by column for a mirror or a transposed copy) in 16-byte
// non-temporal pieces; a diagonal tile of a symmetric product is made
// exactly symmetric in LDS first.
//
// fp32 kernels (the fp32 NS mode): v_mfma_f32_32x32x2f32, register-staged
// k-major LDS, per-fragment epilogue; 64 x 64 x 16 tiles (four waves of
// 32 x 32) or 128 x 128 x 16 tiles (four waves of 64 x 64).
#include <cstdlib>
#include <type_traits>

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

constexpr int kStageK = 64;                     // k per LDS stage
constexpr int kRowBytes = kStageK * 2;          // 128: one cache line per row
constexpr int kRowsPerLoad = 1024 / kRowBytes;  // rows filled by one wave-wide DMA load

// Swizzle of the bf16 staging tile: 16-byte chunk c of staged row r sits at
// chunk c ^ stg_swz(r).  The staging writes (8 bytes of 32 consecutive rows
// per half-wave) then spread over 16 chunk positions, the row reads (16
// chunks of one row per 16 lanes) are a permutation, and the column reads
// (8 bytes of rows 8b + e, b = 0..15, per half-wave) hit 16 different chunk
// positions.
__device__ __forceinline__ int stg_swz(int r) { return (r ^ (r >> 3)) & 15; }

// Two fp32 values rounded to nearest-even bf16, packed (first in the low half).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
#define GLOBAL_AS __attribute__((address_space(1)))

// Global-address-space accesses (flat ones would also count against the LDS
// counter that the LDS-only barrier waits on), non-temporal: results and
// parameters pass through once, and kept in L2 they would push out the
// operand rows that neighbouring tiles are still reading.
__device__ __forceinline__ u32x4_t gload_u32x4(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const GLOBAL_AS u32x4_t*>(reinterpret_cast<uintptr_t>(p)));
}
__device__ __forceinline__ void gstore_u32x4(void* p, u32x4_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<GLOBAL_AS u32x4_t*>(reinterpret_cast<uintptr_t>(p)));
}
__device__ __forceinline__ float gload_f32(const float* p) {
  return *reinterpret_cast<const GLOBAL_AS float*>(reinterpret_cast<uintptr_t>(p));
}

// Workgroup barrier that orders LDS only: global stores already issued stay
// in flight (__syncthreads would wait for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Operand rows in LDS are 128 bytes (eight 16-byte chunks); chunk c of row r
// sits in slot c ^ ((r >> 1) & 7).  A fragment read (16 lanes of a 128-bit
// read per cycle: 16 consecutive rows, one chunk) then covers all 64 banks.
__device__ __forceinline__ int slot_of(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// Buffer descriptor of one operand slab (gfx9 raw buffer: 48-bit base, no
// stride, `bytes` in range, default format word); a lane whose offset is
// outside the range reads zeros.  Base and range are made wave-uniform so
// the descriptor lives in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t u = (uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32))))) << 32) |
                     uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(a))));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), static_cast<short>(0),
                                           __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
// Buffer load into LDS: lane l writes bytes 16l..16l+15 of the 1 KB block
// at `lds`, read from the descriptor's base + voffset.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rsrc, LDS_AS void* lds, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, lds, 16, voffset, 0, 0, 0);
}

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
  // everything the epilogue needs from the task, read before the main loop
  const float s_scale = T.scale ? gload_f32(T.scale) : 1.f;
  const float alpha = T.alpha * spow(s_scale, T.alpha_pow);
  const float beta = T.beta * spow(s_scale, T.beta_pow);
  const float gamma = T.gamma;
  const int diag_limit = T.diag_limit;
  uint16_t* const C = static_cast<uint16_t*>(T.C);
  uint16_t* const Ct = static_cast<uint16_t*>(T.Ct);
  const uint16_t* const Y = static_cast<const uint16_t*>(T.Y);
  const int64_t ldc = T.ldc, ldct = T.ldct, ldy = T.ldy;
  const int mode = T.sym ? (tm != tn ? 1 : 2) : (Ct ? 3 : 0);   // 0 plain, 1 mirror, 2 diagonal, 3 Ct
  // fused parameter update (the last product of a step; mode 0, bf16 W)
  uint16_t* const Wp = static_cast<uint16_t*>(T.W);
  const int64_t ldw = T.ldw;
  const int w_m = T.w_m, w_n = T.w_n, w_tall = T.w_tall, w_vec = T.w_vec;
  const float lr_eff = T.lr_eff, w_decay = T.decay;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // DMA sources: load q of this wave fills LDS block idx = wave + 4q of the
  // stage (blocks 0 .. LOADS_PER_OP-1: A rows, the rest: B rows); lane l
  // writes slot l%8 of row 8*block + l/8, which holds chunk slot^swizzle.
  // Each operand is read through a buffer descriptor based at the tile's
  // first row and the stage's first k (scalar registers, advanced per
  // stage) with a fixed 32-bit byte offset per lane and load, so issuing a
  // load costs no vector arithmetic; the range covers the BT rows of one
  // stage (dimensions up to 2^22 keep it below 2^31 bytes).
  const char* const a_base = static_cast<const char*>(T.A) + int64_t(tm) * BT * T.lda * 2;
  const char* const b_base = static_cast<const char*>(T.B) + int64_t(tn) * BT * T.ldb * 2;
  const int a_span = int((BT - 1) * T.lda * 2 + kRowBytes), b_span = int((BT - 1) * T.ldb * 2 + kRowBytes);
  uint32_t voff[LOADS];
  int dst_off[LOADS];
#pragma unroll
  for (int q = 0; q < LOADS; ++q) {
    const int idx = wave + 4 * q;
    const bool is_b = idx >= LOADS_PER_OP;
    const int blk = is_b ? idx - LOADS_PER_OP : idx;
    const int row = blk * kRowsPerLoad + (lane >> 3);
    const int chunk = slot_of(row, lane & 7);
    voff[q] = uint32_t(row * int(is_b ? T.ldb : T.lda) + chunk * 8) * 2u;
    dst_off[q] = (is_b ? OPB : 0) + blk * 1024;
  }

  // fragment read offsets (bytes within a stage) for the four k-quarters:
  // lanes 0-31 take chunk 2kq, lanes 32-63 chunk 2kq+1 of rows lane & 31
  // (the swizzle depends on the row bits below 16 only, so one offset serves
  // every 32-row fragment)
  int frag_off[4];
#pragma unroll
  for (int kq = 0; kq < 4; ++kq) {
    const int r = lane & 31;
    frag_off[kq] = r * kRowBytes + slot_of(r, kq * 2 + (lane >> 5)) * 16;
  }

  f32x16_t acc[F][F];
#pragma unroll
  for (int i = 0; i < F; ++i)
#pragma unroll
    for (int j = 0; j < F; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  // 256-tiles run v_mfma_f32_16x16x32_bf16 (the same flops for a quarter of
  // the accumulator traffic per instruction, which under the power limit
  // runs at a higher clock): F16 x F16 blocks of 16 x 16 per wave.  With the
  // B fragment first the lane holds row (lane & 15) of a block and, in
  // register r, column 4 (lane >> 4) + r.
  constexpr int F16 = WT / 16;
  f32x4_t acc16[F16][F16];
  if constexpr (BT == 256) {
#pragma unroll
    for (int i = 0; i < F16; ++i)
#pragma unroll
      for (int j = 0; j < F16; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc16[i][j][r] = 0.f;
  }
  // 16 x 16 x 32 fragment read offsets for the two 32-k steps of a stage:
  // lanes take row lane & 15, chunk 4t + (lane >> 4)
  int frag16_off[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int r = lane & 15;
    frag16_off[t] = r * kRowBytes + slot_of(r, 4 * t + (lane >> 4)) * 16;
  }

  auto read_frags = [&](int s, int kq, bf16x8_t (&fa)[F], bf16x8_t (&fb)[F], auto same) {
    constexpr int BOFF = decltype(same)::value ? 0 : OPB;
    const char* st = smem + (s % kStages) * STB + frag_off[kq];
#pragma unroll
    for (int i = 0; i < F; ++i)
      fa[i] = *reinterpret_cast<const bf16x8_t*>(st + (wm * WT + i * 32) * kRowBytes);
#pragma unroll
    for (int j = 0; j < F; ++j)
      fb[j] = *reinterpret_cast<const bf16x8_t*>(st + BOFF + (wn * WT + j * 32) * kRowBytes);
  };
  auto mfmas = [&](const bf16x8_t (&fa)[F], const bf16x8_t (&fb)[F]) {
#pragma unroll
    for (int i = 0; i < F; ++i)
#pragma unroll
      for (int j = 0; j < F; ++j)
        // B fragment first: the lane then holds row (lane & 31) of its
        // 32 x 32 block and, in register 4g + r, column 8g + 4(lane >> 5) + r
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
  };

  // Instruction order is pinned with scheduling groups (the compiler would
  // otherwise sink each fragment read to just before its first use): the
  // in-order issue must never run out of independent MFMAs while loads and
  // LDS reads are issued.
  constexpr int kMfma = 0x008, kVmem = 0x010, kDsRead = 0x100;
  constexpr int NFRAG = 2 * F;          // fragment reads per k-quarter
  constexpr int NMFMA = F * F;          // MFMAs per k-quarter
  bf16x8_t fa0[F], fb0[F], fa1[F], fb1[F];
  // one k-quarter: MFMAs on (fa, fb) while the next quarter's fragments load
  auto quarter = [&](int s, int kq_next, bf16x8_t (&na)[F], bf16x8_t (&nb)[F],
                     const bf16x8_t (&fa)[F], const bf16x8_t (&fb)[F], auto same) {
    read_frags(s, kq_next, na, nb, same);
    mfmas(fa, fb);
    // the reads go out two per MFMA over the first NFRAG/2 MFMAs, as early
    // as possible behind the first one
#pragma unroll
    for (int i = 0; i < NFRAG / 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kMfma, NMFMA - NFRAG / 2, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // Ring of two stages, 64 k each; stage kt's data sits in slot kt % 2.
  // 128-tiles (the 256-tile schedule follows below).
  // Per stage: quarters 0-2 run on fragments already in registers while the
  // next quarter's load; then one barrier, at which stage kt+1 has landed
  // (own loads counted, everyone's by the barrier) and every wave has
  // finished its LDS reads of stage kt; quarter 3 issues the reads of stage
  // kt+1's first quarter and the first part of stage kt+2's loads into stage
  // kt's slot, and quarter 0 of the next stage the rest, so that the loads'
  // LDS writes spread over two quarters.  The wait counts are constants: the
  // stage before the last issues no loads of a stage past the end, and the
  // last stage issues none and has no barrier.
  static_assert(kStages == 2, "two-slot ring");
  // loads of a stage issued in quarter 3 (the rest go in the next quarter 0)
  constexpr int LQ3 = LOADS / 2;
  constexpr int LQ0 = LOADS - LQ3;
  // part h of stage `data`'s loads into ring slot `slot % kStages`
  auto issue_part = [&](int data, int slot, int h) {
    char* st = smem + (slot % kStages) * STB;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_base + data * kRowBytes, a_span);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(b_base + data * kRowBytes, b_span);
#pragma unroll
    for (int q = h ? LQ3 : 0; q < (h ? LOADS : LQ3); ++q)
      buffer_load_lds16(q < LOADS_PER_OP / 4 ? ra : rb, (LDS_AS void*)(st + dst_off[q]), int(voff[q]));
  };
  // MFMAs of one quarter with the next quarter's reads and part of a stage's
  // loads interleaved; the reads come first in program order (the compiler
  // keeps LDS reads and direct-to-LDS loads in program order) and an MFMA
  // always goes first (its wait for this quarter's fragments must not also
  // cover a read of the next quarter issued ahead of it)
  auto pin_quarter_with_loads = [&](auto nloads) {
    constexpr int V = decltype(nloads)::value;
    // (instantiated for 256-tiles too, whose schedule is main_loop4; never run there)
    static_assert(BT != 128 || (NMFMA == 4 && NFRAG == 4 && (V == 4 || V == 0)), "schedule");
#pragma unroll
    for (int i = 0; i < 4; ++i) {                  // 4 MFMAs, 4 reads, 4 or 0 loads
      __builtin_amdgcn_sched_group_barrier(kMfma, 1, 1);
      __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 1);
      if constexpr (V > 0) __builtin_amdgcn_sched_group_barrier(kVmem, 1, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto main_loop = [&](auto same) {
  constexpr bool kSame = decltype(same)::value;
  issue_part(0, 0, 0);
  if constexpr (!kSame) issue_part(0, 0, 1);
  issue_part(nk > 1 ? 1 : 0, 1, 0);
  wait_vmcnt<LQ3>();
  __builtin_amdgcn_s_barrier();
  read_frags(0, 0, fa0, fb0, same);
  // One stage.  kLast: the last stage (no loads, no reads of a next stage,
  // no barrier); kNoAhead: the stage before it (no stage kt+2 to load).
  auto stage_step = [&](int kt, auto last, auto no_ahead) {
    constexpr bool kLast = decltype(last)::value, kNoAhead = decltype(no_ahead)::value;
    if constexpr (kLast) {
      quarter(kt, 1, fa1, fb1, fa0, fb0, same);
      quarter(kt, 2, fa0, fb0, fa1, fb1, same);
      quarter(kt, 3, fa1, fb1, fa0, fb0, same);
      mfmas(fa1, fb1);
      __builtin_amdgcn_sched_barrier(0);
    } else {
      // quarter 0, with the rest of stage kt+1's loads
      read_frags(kt, 1, fa1, fb1, same);
      if constexpr (kSame) {
        mfmas(fa0, fb0);
        pin_quarter_with_loads(std::integral_constant<int, 0>{});
      } else {
        issue_part(kt + 1, kt + 1, 1);
        mfmas(fa0, fb0);
        pin_quarter_with_loads(std::integral_constant<int, LQ0>{});
      }
      quarter(kt, 2, fa0, fb0, fa1, fb1, same);
      quarter(kt, 3, fa1, fb1, fa0, fb0, same);
      wait_vmcnt<0>();
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // quarter 3, with the first part of stage kt+2's loads
      read_frags(kt + 1, 0, fa0, fb0, same);
      if constexpr (kNoAhead) {
        mfmas(fa1, fb1);
        pin_quarter_with_loads(std::integral_constant<int, 0>{});
      } else {
        issue_part(kt + 2, kt + 2, 0);
        mfmas(fa1, fb1);
        pin_quarter_with_loads(std::integral_constant<int, LQ3>{});
      }
    }
  };
  int kt = 0;
  for (; kt + 2 < nk; ++kt) stage_step(kt, std::false_type{}, std::false_type{});
  if (kt + 1 < nk) stage_step(kt++, std::false_type{}, std::true_type{});
  stage_step(kt, std::true_type{}, std::false_type{});
  };
  // The wave of the lower-left quadrant of a diagonal tile of a symmetric
  // product computes nothing: that quadrant lies below the diagonal, and the
  // epilogue replaces it by the mirror of the upper one.  It issues its share
  // of the loads and meets every barrier, and leaves the LDS to the other
  // three waves' fragment reads.
  auto idle_loop = [&](auto same) {
    constexpr bool kSame = decltype(same)::value;
    issue_part(0, 0, 0);
    if constexpr (!kSame) issue_part(0, 0, 1);
    issue_part(nk > 1 ? 1 : 0, 1, 0);
    wait_vmcnt<LQ3>();
    __builtin_amdgcn_s_barrier();
    for (int kt = 0; kt + 1 < nk; ++kt) {
      if constexpr (!kSame) issue_part(kt + 1, kt + 1, 1);
      wait_vmcnt<0>();
      lds_barrier();
      if (kt + 2 < nk) issue_part(kt + 2, kt + 2, 0);
    }
  };

  // 256-tiles: a whole stage of fragments in registers, two barriers per
  // stage.  Fragment set t holds 32-k step t of a stage; a quarter is half a
  // step (32 MFMAs).  Stage s+1's step 0 is read during quarter 3 of stage s
  // (one read behind every second MFMA), its step 1 during its own quarter 0
  // (one behind each of the first sixteen MFMAs).
  // After quarter 0 a barrier frees the ring slot of stage s, and stage
  // s+2's 16 loads per wave go into it: 6 in quarter 1, 6 in quarter 2, 2 in
  // quarter 3, 2 in quarter 0 of stage s+1, evenly spaced within each
  // quarter.  After quarter 2 a second barrier makes stage s+1 visible: each
  // wave first waits for its own loads of that stage, the ones of stage s+2
  // issued since stay in flight.  Neither barrier carries a memory fence (a
  // fence would also wait for every direct-to-LDS load); the waits before
  // them are explicit.
  constexpr int LP1 = 6, LP2 = 6, LP3 = 2;       // loads per wave in quarters 1, 2, 3; the rest in quarter 0
  static_assert(BT != 256 || (LOADS == 16 && LP1 + LP2 + LP3 <= LOADS), "schedule");
  // load position p of a stage -> load q; A (q < 8) and B rows alternate, so
  // a diagonal tile of a matrix times itself (A rows only) splits its loads
  // over the four parts in the same proportion
  auto ord4 = [](int p) constexpr { return (p & 1) ? LOADS / 2 + (p >> 1) : (p >> 1); };
  auto plo4 = [](int h) constexpr { return h == 1 ? 0 : h == 2 ? LP1 : h == 3 ? LP1 + LP2 : LP1 + LP2 + LP3; };
  auto phi4 = [](int h) constexpr { return h == 1 ? LP1 : h == 2 ? LP1 + LP2 : h == 3 ? LP1 + LP2 + LP3 : LOADS; };
  // loads in part h (the quarter that issues them) of one stage
  auto pcount4 = [ord4, plo4, phi4](auto part, auto same) constexpr {
    constexpr int H = decltype(part)::value;
    int n = 0;
    for (int p = plo4(H); p < phi4(H); ++p) n += (!decltype(same)::value || ord4(p) < LOADS_PER_OP / 4) ? 1 : 0;
    return n;
  };
  // q of the l-th load of part h
  auto pq4 = [ord4, plo4, phi4](auto part, auto same, int l) constexpr {
    constexpr int H = decltype(part)::value;
    for (int p = plo4(H); p < phi4(H); ++p) {
      const bool ok = !decltype(same)::value || ord4(p) < LOADS_PER_OP / 4;
      if (ok && l-- == 0) return ord4(p);
    }
    return 0;
  };
  using Part0 = std::integral_constant<int, 0>;
  using Part1 = std::integral_constant<int, 1>;
  using Part2 = std::integral_constant<int, 2>;
  using Part3 = std::integral_constant<int, 3>;
  // part h of stage `data`'s loads into ring slot `slot`, back to back
  auto issue4 = [&](int data, int slot, auto part, auto same) {
    constexpr int N = pcount4(part, same);
    char* st = smem + (slot % kStages) * STB;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_base + data * kRowBytes, a_span);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(b_base + data * kRowBytes, b_span);
#pragma unroll
    for (int l = 0; l < N; ++l) {
      const int q = pq4(part, same, l);
      buffer_load_lds16(q < LOADS_PER_OP / 4 ? ra : rb, (LDS_AS void*)(st + dst_off[q]), int(voff[q]));
    }
  };
  // fragment set t holds 32-k step t of a stage: F16 A and F16 B blocks
  bf16x8_t fra[2][F16], frb[2][F16];
  // One quarter in a fixed instruction order: the 32 MFMAs of half h of the
  // step in set CS (A blocks 4h..4h+3 by every B block); behind every RS-th
  // of them one fragment read of the step RSET of the stage in ring slot
  // rs into set RSET (A blocks, then B blocks; none when RSET < 0); and the
  // loads of part h of stage ld_data, evenly spaced.  A scheduling barrier
  // after every MFMA keeps that order.
  auto q16 = [&](auto cs, auto half, auto rset, int rs, auto rstride, auto same, auto nloads, int ld_data,
                 auto part) {
    constexpr int CS = decltype(cs)::value, H = decltype(half)::value, RSET = decltype(rset)::value;
    constexpr int RS = decltype(rstride)::value, V = decltype(nloads)::value;
    constexpr int BOFF = decltype(same)::value ? 0 : OPB;
    constexpr int NM = F16 * F16 / 2;                // MFMAs per quarter
    const char* rst = smem + (rs % kStages) * STB + frag16_off[RSET < 0 ? 0 : RSET];
    char* ldst = smem + (ld_data % kStages) * STB;
    __amdgpu_buffer_rsrc_t ra, rb;
    if constexpr (V > 0) {
      ra = make_rsrc(a_base + ld_data * kRowBytes, a_span);
      rb = make_rsrc(b_base + ld_data * kRowBytes, b_span);
    }
    int l = 0;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int i = H * (F16 / 2) + m / F16, j = m % F16;
      // the MFMA in asm with the accumulator as a tied AGPR operand: each
      // accumulator stays in place (the builtin leaves the register
      // allocator shuffling the 64 four-register accumulators between AGPR
      // quads and VGPRs); it touches registers only
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc16[i][j]) : "v"(frb[CS][j]), "v"(fra[CS][i]));
      if constexpr (RSET >= 0) {
        if (m % RS == 0 && m / RS < 2 * F16) {
          const int r = m / RS;
          if (r < F16)
            fra[RSET][r] = *reinterpret_cast<const bf16x8_t*>(rst + (wm * WT + r * 16) * kRowBytes);
          else
            frb[RSET][r - F16] = *reinterpret_cast<const bf16x8_t*>(rst + BOFF + (wn * WT + (r - F16) * 16) * kRowBytes);
        }
      }
      if constexpr (V > 0) {
        if (((m + 1) * V) / NM > (m * V) / NM) {
          const int q = pq4(part, same, l);
          buffer_load_lds16(q < LOADS_PER_OP / 4 ? ra : rb, (LDS_AS void*)(ldst + dst_off[q]), int(voff[q]));
          ++l;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using Step0 = std::integral_constant<int, 0>;
  using Step1 = std::integral_constant<int, 1>;
  using NoSet = std::integral_constant<int, -1>;
  using NoLoads = std::integral_constant<int, 0>;
  using Half0 = std::integral_constant<int, 0>;
  using Half1 = std::integral_constant<int, 1>;
  using EveryMfma = std::integral_constant<int, 1>;
  using EverySecond = std::integral_constant<int, 2>;
  // s_waitcnt lgkmcnt(0), the other counters untouched (gfx9 encoding)
  auto wait_lgkm0 = []() { __builtin_amdgcn_s_waitcnt(0xC07F); };
  // workgroup barrier without a memory fence; the signal fences only keep
  // the compiler from moving memory accesses across it
  auto plain_barrier = []() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto main_loop4 = [&](auto same) {
    using S = decltype(same);
    constexpr int N0 = pcount4(Part0{}, S{});
    constexpr int N12 = pcount4(Part1{}, S{}) + pcount4(Part2{}, S{});
    // stage 0 whole and stage 1 but its quarter-0 part; a single stage
    // loads itself again into the other slot, harmlessly
    const int d1 = nk > 1 ? 1 : 0;
    issue4(0, 0, Part1{}, same); issue4(0, 0, Part2{}, same); issue4(0, 0, Part3{}, same); issue4(0, 0, Part0{}, same);
    issue4(d1, 1, Part1{}, same); issue4(d1, 1, Part2{}, same); issue4(d1, 1, Part3{}, same);
    wait_vmcnt<N12 + pcount4(Part3{}, S{})>();
    plain_barrier();
    // step 0 of stage 0 into set 0
    {
      const char* st = smem + frag16_off[0];
#pragma unroll
      for (int i = 0; i < F16; ++i) fra[0][i] = *reinterpret_cast<const bf16x8_t*>(st + (wm * WT + i * 16) * kRowBytes);
#pragma unroll
      for (int j = 0; j < F16; ++j)
        frb[0][j] = *reinterpret_cast<const bf16x8_t*>(st + (S::value ? 0 : OPB) + (wn * WT + j * 16) * kRowBytes);
    }
    __builtin_amdgcn_sched_barrier(0);
    auto stage16 = [&](int kt, auto last, auto no_ahead) {
      constexpr bool kLast = decltype(last)::value, kNoAhead = decltype(no_ahead)::value;
      if constexpr (kLast) {
        q16(Step0{}, Half0{}, Step1{}, kt, EveryMfma{}, same, NoLoads{}, 0, Part0{});
        q16(Step0{}, Half1{}, NoSet{}, 0, EveryMfma{}, same, NoLoads{}, 0, Part0{});
        q16(Step1{}, Half0{}, NoSet{}, 0, EveryMfma{}, same, NoLoads{}, 0, Part0{});
        q16(Step1{}, Half1{}, NoSet{}, 0, EveryMfma{}, same, NoLoads{}, 0, Part0{});
      } else {
        // quarter 0: reads of this stage's step 1, last loads of stage kt+1
        q16(Step0{}, Half0{}, Step1{}, kt, EveryMfma{}, same, std::integral_constant<int, N0>{}, kt + 1, Part0{});
        wait_lgkm0();
        plain_barrier();                             // ring slot kt is free
        if constexpr (kNoAhead) {
          q16(Step0{}, Half1{}, NoSet{}, 0, EveryMfma{}, same, NoLoads{}, 0, Part0{});
          q16(Step1{}, Half0{}, NoSet{}, 0, EveryMfma{}, same, NoLoads{}, 0, Part0{});
          wait_vmcnt<0>();
        } else {
          q16(Step0{}, Half1{}, NoSet{}, 0, EveryMfma{}, same, std::integral_constant<int, pcount4(Part1{}, S{})>{},
              kt + 2, Part1{});
          q16(Step1{}, Half0{}, NoSet{}, 0, EveryMfma{}, same, std::integral_constant<int, pcount4(Part2{}, S{})>{},
              kt + 2, Part2{});
          wait_vmcnt<N12>();
        }
        plain_barrier();                             // stage kt+1 has landed
        // quarter 3: reads of stage kt+1's step 0
        if constexpr (kNoAhead)
          q16(Step1{}, Half1{}, Step0{}, kt + 1, EverySecond{}, same, NoLoads{}, 0, Part0{});
        else
          q16(Step1{}, Half1{}, Step0{}, kt + 1, EverySecond{}, same,
              std::integral_constant<int, pcount4(Part3{}, S{})>{}, kt + 2, Part3{});
      }
    };
    int kt = 0;
    for (; kt + 2 < nk; ++kt) stage16(kt, std::false_type{}, std::false_type{});
    if (kt + 1 < nk) stage16(kt++, std::false_type{}, std::true_type{});
    stage16(kt, std::true_type{}, std::false_type{});
  };
  // the idle wave of a diagonal tile: the same loads, waits and barriers
  auto idle_loop4 = [&](auto same) {
    using S = decltype(same);
    constexpr int N12 = pcount4(Part1{}, S{}) + pcount4(Part2{}, S{});
    const int d1 = nk > 1 ? 1 : 0;
    issue4(0, 0, Part1{}, same); issue4(0, 0, Part2{}, same); issue4(0, 0, Part3{}, same); issue4(0, 0, Part0{}, same);
    issue4(d1, 1, Part1{}, same); issue4(d1, 1, Part2{}, same); issue4(d1, 1, Part3{}, same);
    wait_vmcnt<N12 + pcount4(Part3{}, S{})>();
    plain_barrier();
    for (int kt = 0; kt + 1 < nk; ++kt) {
      issue4(kt + 1, kt + 1, Part0{}, same);
      plain_barrier();
      if (kt + 2 < nk) {
        issue4(kt + 2, kt + 2, Part1{}, same);
        issue4(kt + 2, kt + 2, Part2{}, same);
        wait_vmcnt<N12>();
      } else {
        wait_vmcnt<0>();
      }
      plain_barrier();
      if (kt + 2 < nk) issue4(kt + 2, kt + 2, Part3{}, same);
    }
  };
  const bool idle = T.sym && tm == tn && wm == 1 && wn == 0;
  // a diagonal tile of a matrix times itself: one operand's rows serve both
  if constexpr (BT == 256) {
    if (T.A == T.B && tm == tn) {
      if (idle)
        idle_loop4(std::true_type{});
      else
        main_loop4(std::true_type{});
    } else if (idle) {
      idle_loop4(std::false_type{});
    } else {
      main_loop4(std::false_type{});
    }
  } else {
    if (T.A == T.B && tm == tn) {
      if (idle)
        idle_loop(std::true_type{});
      else
        main_loop(std::true_type{});
    } else if (idle) {
      idle_loop(std::false_type{});
    } else {
      main_loop(std::false_type{});
    }
  }
  // no load may still be writing this block's LDS when the block retires
  wait_vmcnt<0>();
  if constexpr (BT == 256) {
    // the compiler does not see the asm MFMAs' latency: wait states before
    // the epilogue reads their accumulators
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
  }

  // Epilogue.  The ring holds the finished tile as bf16, row-major, 16-byte
  // chunks swizzled per row (stg_swz).  Each lane scales its accumulators
  // (and adds beta*Y, which a Y tile first brings into the same place by
  // direct-to-LDS loads, and gamma on the diagonal), rounds them to bf16 in
  // pairs and writes 8 bytes per 4 columns.  C then leaves row by row in
  // 16-byte pieces; the mirror (symmetric tiles) or the transposed copy Ct
  // leaves column by column: a lane reads 4 columns of 8 rows (8 x 8 bytes)
  // and transposes them in registers into 4 pieces of 16 bytes.  Global
  // accesses use global (not flat) instructions and the barriers order LDS
  // only, so stores stay in flight until the block ends; LDS reads are
  // issued in batches ahead of their use.
  constexpr int RING = kStages * STB;
  static_assert(RING >= BT * BT * 2, "staging does not fit");
  constexpr int NCH = BT / 8;                    // 16-byte chunks per staged row
  constexpr int ROWB = BT * 2;                   // bytes per staged row
  char* const stg = smem;
  const int t = threadIdx.x;
  const int h = lane >> 5;
  constexpr int LPC = 2 * (BT / 8);              // lanes per column chunk of a block transpose
  constexpr int NTQ = BT * BT * 2 / 64 / 256;    // block transposes per thread

  // Fused parameter update (used at the end of the epilogue): a thread owns
  // 8 * WNB pieces of 8 values of W; piece pc of batch k is W row r from
  // column c on, taken from a staged tile row (wide W) or from a block
  // transpose of the staged tile (tall W).
  constexpr int NIT = BT * NCH / 256, WB = 8, QB = 2;
  constexpr int WNB = NIT / WB;
  static_assert(NIT % WB == 0 && NTQ % QB == 0 && NTQ / QB == WNB, "batches");
  const int w_chunk = t % NCH;
  const int64_t r_lim = w_tall ? w_n : w_m, c_lim = w_tall ? w_m : w_n;
  auto piece = [&](int k, int pc, int64_t& r, int64_t& c) {
    if (!w_tall) {
      const int row = t / NCH + (256 / NCH) * (k * WB + pc);
      r = int64_t(tm) * BT + row;
      c = int64_t(tn) * BT + w_chunk * 8;
    } else {
      const int tq = t + 256 * (k * QB + pc / 4);
      const int cc = tq / LPC, rb = (tq % LPC) >> 1, hf = tq & 1;
      r = int64_t(tn) * BT + 8 * cc + 4 * hf + (pc & 3);   // W row = tile column
      c = int64_t(tm) * BT + 8 * rb;                        // W columns = tile rows
    }
  };
  auto load_batch = [&](int k, u32x4_t (&w)[WB]) {
#pragma unroll
    for (int pc = 0; pc < WB; ++pc) {
      int64_t r, c;
      piece(k, pc, r, c);
      if (r < r_lim && c + 8 <= c_lim && w_vec) w[pc] = gload_u32x4(Wp + r * ldw + c);
    }
  };

  lds_barrier();                                 // every wave is done with the ring
  if (Y) {
    // Y tile into the staging layout: one 1 KB load covers 1024 / ROWB rows
    constexpr int RPL = 1024 / ROWB;
    constexpr int NLOAD = BT * ROWB / 1024 / 4;  // per wave
#pragma unroll
    for (int q = 0; q < NLOAD; ++q) {
      const int first = (wave + 4 * q) * RPL;
      const int row = first + lane / NCH;
      const int chunk = (lane % NCH) ^ stg_swz(row);
      __builtin_amdgcn_global_load_lds(
          static_cast<const void*>(Y + (int64_t(tm) * BT + row) * ldy + int64_t(tn) * BT + chunk * 8),
          (LDS_AS void*)(stg + first * ROWB), 16, 0, 0);
    }
    wait_vmcnt<0>();
    lds_barrier();
  }

  // scale, add, round and stage: fragment (i, j), register group g covers
  // row wm*WT + 32i + (lane & 31), columns wn*WT + 32j + 8g + 4(lane >> 5) + 0..3
  // (one instance with Y and one without, so no group carries a branch)
  auto stage_tile = [&](auto hy) {
    constexpr bool has_y = decltype(hy)::value;
    const bool add_gamma = tm == tn && gamma != 0.f && wm == wn;
#pragma unroll
    for (int i = 0; i < F; ++i) {
      const int row = wm * WT + i * 32 + (lane & 31);
      const int sw = stg_swz(row);
      char* const srow = stg + row * ROWB + h * 8;
      const bool diag_row = int64_t(tm) * BT + row < diag_limit;
#pragma unroll
      for (int j = 0; j < F; ++j) {
        uint2 y[4];
        if constexpr (has_y) {
#pragma unroll
          for (int g = 0; g < 4; ++g)
            y[g] = *reinterpret_cast<const uint2*>(srow + ((((wn * WT + j * 32) / 8 + g) ^ sw) << 4));
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = alpha * acc[i][j][4 * g + r];
          if constexpr (has_y) {
            v[0] = fmaf(beta, __uint_as_float(y[g].x << 16), v[0]);
            v[1] = fmaf(beta, __uint_as_float(y[g].x & 0xffff0000u), v[1]);
            v[2] = fmaf(beta, __uint_as_float(y[g].y << 16), v[2]);
            v[3] = fmaf(beta, __uint_as_float(y[g].y & 0xffff0000u), v[3]);
          }
          if (i == j && add_gamma) {             // wm == wn: the tile diagonal
#pragma unroll
            for (int r = 0; r < 4; ++r)
              v[r] += ((lane & 31) == 8 * g + 4 * h + r && diag_row) ? gamma : 0.f;
          }
          *reinterpret_cast<uint2*>(srow + ((((wn * WT + j * 32) / 8 + g) ^ sw) << 4)) =
              make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
        __builtin_amdgcn_sched_barrier(0);       // bounds the live accumulator copies
      }
    }
  };
  // 256-tiles: row wm*WT + 16i + (lane & 15), columns wn*WT + 16j + 4(lane >> 4) + 0..3
  auto stage_tile16 = [&](auto hy) {
    constexpr bool has_y = decltype(hy)::value;
    const bool add_gamma = tm == tn && gamma != 0.f && wm == wn;
    const int cq = lane >> 5;                    // chunk of the 8 columns within a 16-column block
#pragma unroll
    for (int i = 0; i < F16; ++i) {
      const int row = wm * WT + i * 16 + (lane & 15);
      const int sw = stg_swz(row);
      char* const srow = stg + row * ROWB + ((lane >> 4) & 1) * 8;
      const bool diag_row = int64_t(tm) * BT + row < diag_limit;
#pragma unroll
      for (int j = 0; j < F16; ++j) {
        char* const p = srow + ((((wn * WT + j * 16) / 8 + cq) ^ sw) << 4);
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = alpha * acc16[i][j][r];
        if constexpr (has_y) {
          const uint2 y = *reinterpret_cast<const uint2*>(p);
          v[0] = fmaf(beta, __uint_as_float(y.x << 16), v[0]);
          v[1] = fmaf(beta, __uint_as_float(y.x & 0xffff0000u), v[1]);
          v[2] = fmaf(beta, __uint_as_float(y.y << 16), v[2]);
          v[3] = fmaf(beta, __uint_as_float(y.y & 0xffff0000u), v[3]);
        }
        if (i == j && add_gamma) {               // wm == wn: the tile diagonal
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] += ((lane & 15) == 4 * (lane >> 4) + r && diag_row) ? gamma : 0.f;
        }
        *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
      __builtin_amdgcn_sched_barrier(0);         // bounds the live accumulator copies
    }
  };
  if constexpr (BT == 256) {
    if (Y)
      stage_tile16(std::true_type{});
    else
      stage_tile16(std::false_type{});
  } else {
    if (Y)
      stage_tile(std::true_type{});
    else
      stage_tile(std::false_type{});
  }
  lds_barrier();

  // 8 x 4 block transposes: lane tq takes rows 8rb..8rb+7 of columns
  // 8cc + 4hf + 0..3 of the staged tile and returns, for sc = 0..3, tile
  // column 8cc + 4hf + sc over those 8 rows as one 16-byte piece
  auto transpose_block = [&](int tq, int& cc, int& rb, int& hf, u32x4_t (&o)[4]) {
    cc = tq / LPC;
    rb = (tq % LPC) >> 1;
    hf = tq & 1;
    uint2 w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = 8 * rb + e;
      w[e] = *reinterpret_cast<const uint2*>(stg + row * ROWB + ((cc ^ stg_swz(row)) << 4) + hf * 8);
    }
#pragma unroll
    for (int sc = 0; sc < 4; ++sc) {
      const uint32_t sel = (sc & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
      for (int p2 = 0; p2 < 4; ++p2) {
        const uint32_t lo = (sc >> 1) ? w[2 * p2].y : w[2 * p2].x;
        const uint32_t hi = (sc >> 1) ? w[2 * p2 + 1].y : w[2 * p2 + 1].x;
        o[sc][p2] = __builtin_amdgcn_perm(hi, lo, sel);
      }
    }
  };

  // A diagonal tile of a symmetric product is made exactly symmetric in
  // LDS (every value below the diagonal replaced by its mirror above it),
  // then leaves like any other tile, row by row, with no mirror pass.
  if (mode == 2) {
#pragma unroll 2
    for (int q = 0; q < NTQ; ++q) {
      const int tq = t + 256 * q;
      if ((tq % LPC) >> 1 < tq / LPC) {          // row block above the column block
        int cc, rb, hf;
        u32x4_t o[4];
        transpose_block(tq, cc, rb, hf, o);
#pragma unroll
        for (int sc = 0; sc < 4; ++sc) {
          const int row = 8 * cc + 4 * hf + sc;  // destination: row `row`, chunk rb (below the diagonal)
          *reinterpret_cast<u32x4_t*>(stg + row * ROWB + ((rb ^ stg_swz(row)) << 4)) = o[sc];
        }
      }
    }
    // inside the 8 x 8 blocks on the diagonal, element by element
    for (int idx = t; idx < (BT / 8) * 64; idx += 256) {
      const int b = idx >> 6, i = (idx >> 3) & 7, j = idx & 7;
      if (i > j) {
        const int r = 8 * b + i, c = 8 * b + j;  // (r, c) below, (c, r) above
        const uint16_t v = *reinterpret_cast<const uint16_t*>(stg + c * ROWB + ((b ^ stg_swz(c)) << 4) + i * 2);
        *reinterpret_cast<uint16_t*>(stg + r * ROWB + ((b ^ stg_swz(r)) << 4) + j * 2) = v;
      }
    }
    lds_barrier();
  }

  // The last product of a step: the tile is O (rounded to bf16, staged);
  // instead of storing it, update the parameter: W <- W*decay - lr_eff*O in
  // fp32, rounded once, in W's stored orientation (row pieces of the staged
  // tile for a wide W, column pieces for a tall one).  Each thread owns
  // 8 * WNB pieces of 8 values; all its W loads go out at once once the tile
  // is staged (the accumulators are dead by then, so their registers are
  // free), then the pieces are updated batch by batch; pieces past W's edge
  // are skipped, and pieces at its edge (or on unaligned rows) go element by
  // element.
  if (Wp) {
    // eight values: o and w bf16 pairs -> the updated bf16 pairs (rounded
    // to nearest-even by the packed conversion, as the staging rounds)
    auto update8 = [&](const u32x4_t& o, const u32x4_t& w) {
      u32x4_t r;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float a0 = fmaf(-lr_eff, __uint_as_float(o[k] << 16), __uint_as_float(w[k] << 16) * w_decay);
        const float a1 = fmaf(-lr_eff, __uint_as_float(o[k] & 0xffff0000u),
                              __uint_as_float(w[k] & 0xffff0000u) * w_decay);
        r[k] = pack_bf16x2(a0, a1);
      }
      return r;
    };
    // the first cnt (< 8, or unaligned) values of a piece, one by one
    auto update_some = [&](const u32x4_t& o, uint16_t* wp, int cnt) {
      for (int e = 0; e < cnt; ++e) {
        const float of = __uint_as_float(((o[e >> 1] >> ((e & 1) * 16)) & 0xffffu) << 16);
        wp[e] = static_cast<uint16_t>(f32_to_bf16_bits(fmaf(-lr_eff, of, bf16_bits_to_f32(wp[e]) * w_decay)));
      }
    };
    auto run_batch = [&](int k, const u32x4_t (&w)[WB]) {
      u32x4_t ov[WB];
      if (!w_tall) {
#pragma unroll
        for (int pc = 0; pc < WB; ++pc) {
          const int row = t / NCH + (256 / NCH) * (k * WB + pc);
          ov[pc] = *reinterpret_cast<const u32x4_t*>(stg + row * ROWB + ((w_chunk ^ stg_swz(row)) << 4));
        }
      } else {
#pragma unroll
        for (int qq = 0; qq < QB; ++qq) {
          int cc, rb, hf;
          u32x4_t o4[4];
          transpose_block(t + 256 * (k * QB + qq), cc, rb, hf, o4);
#pragma unroll
          for (int sc = 0; sc < 4; ++sc) ov[qq * 4 + sc] = o4[sc];
        }
      }
#pragma unroll
      for (int pc = 0; pc < WB; ++pc) {
        int64_t r, c;
        piece(k, pc, r, c);
        if (r >= r_lim || c >= c_lim) continue;
        uint16_t* const wp = Wp + r * ldw + c;
        if (c + 8 <= c_lim && w_vec) {
          gstore_u32x4(wp, update8(ov[pc], w[pc]));
        } else {
          update_some(ov[pc], wp, static_cast<int>(c + 8 <= c_lim ? 8 : c_lim - c));
        }
      }
    };
    u32x4_t wall[WNB][WB];
#pragma unroll
    for (int k = 0; k < WNB; ++k) load_batch(k, wall[k]);
#pragma unroll
    for (int k = 0; k < WNB; ++k) run_batch(k, wall[k]);
    return;
  }

  // C, row by row: thread t covers chunk t % NCH of rows t / NCH + (256 / NCH) k
  {
    constexpr int NIT = BT * NCH / 256, BATCH = 4;
    const int chunk = t % NCH;
    const int c0 = chunk * 8;
    uint16_t* const cbase = C + (int64_t(tm) * BT) * ldc + int64_t(tn) * BT + c0;
#pragma unroll
    for (int k0 = 0; k0 < NIT; k0 += BATCH) {
      u32x4_t v[BATCH];
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        const int row = t / NCH + (256 / NCH) * (k0 + b);
        v[b] = *reinterpret_cast<const u32x4_t*>(stg + row * ROWB + ((chunk ^ stg_swz(row)) << 4));
      }
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        const int row = t / NCH + (256 / NCH) * (k0 + b);
        gstore_u32x4(cbase + int64_t(row) * ldc, v[b]);
      }
    }
  }

  // mirror (off-diagonal symmetric tiles) or Ct, column by column: tile
  // column c leaves as row c of the destination
  if (mode == 1 || mode == 3) {
    uint16_t* const Tdst = mode == 3 ? Ct : C;
    const int64_t ldt = mode == 3 ? ldct : ldc;
#pragma unroll 2
    for (int q = 0; q < NTQ; ++q) {
      int cc, rb, hf;
      u32x4_t o[4];
      transpose_block(t + 256 * q, cc, rb, hf, o);
#pragma unroll
      for (int sc = 0; sc < 4; ++sc) {
        const int col = 8 * cc + 4 * hf + sc;
        gstore_u32x4(Tdst + (int64_t(tn) * BT + col) * ldt + int64_t(tm) * BT + 8 * rb, o[sc]);
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

// 128 x 128 x 16 tiles for batches with enough work to fill the chip: four
// waves of 64 x 64 (2 x 2 fragments of 32 x 32), half the operand bytes per
// flop of the 64 tile, 32 MFMAs per wave per stage to cover the loads of the
// next stage, four blocks per CU.  Operands are staged through registers into
// k-major LDS rows of pitch BT + 2 words.  (Measured on 4096 plain tiles,
// K = 4096: 16-k stages 132 TFLOP/s, 32-k 127, 64-k 102; pitches BT + 2,
// BT + 4 and BT + 32 within 3 %; four blocks per CU instead of two +1.4 %,
// +2.4 % on 2080 symmetric tiles.)
constexpr int kF32BigTile = kTileF32Big;
constexpr int kF32BigBK = 16;
constexpr int kF32BigPitch = kF32BigTile + 2;

// (register budget for four waves per SIMD, so four blocks share a CU: the
// accumulators then live in VGPRs, 106 in all, no spills)
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4)))
gemm_f32_big_kernel(const GemmTask* __restrict__ tasks, const TileRef* __restrict__ map) {
  constexpr int BT = kF32BigTile, BK = kF32BigBK, LDP = kF32BigPitch;
  constexpr int KCH = BK / 4;                      // float4 chunks per operand row of a stage
  constexpr int RPP = 256 / KCH;                   // operand rows covered by one pass of the block
  constexpr int NLD = BT / RPP;                    // float4 loads per thread per operand per stage
  static_assert(BK % 4 == 0 && 256 % KCH == 0 && BT % RPP == 0 && NLD * RPP * KCH * 4 == BT * BK,
                "the block's loads cover the BT x BK operand slab exactly once");
  __shared__ __attribute__((aligned(16))) float As[2][BK][LDP];
  __shared__ __attribute__((aligned(16))) float Bs[2][BK][LDP];

  const TileRef ref = map[blockIdx.x];
  const int tm = ref.tm, tn = ref.tn;
  const GemmTask& T = tasks[ref.task];
  const int64_t lda = T.lda, ldb = T.ldb;
  const float* __restrict__ A = static_cast<const float*>(T.A) + int64_t(tm) * BT * lda;
  const float* __restrict__ B = static_cast<const float*>(T.B) + int64_t(tn) * BT * ldb;
  const int nk = T.K / BK;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // thread t stages rows t / KCH + RPP*i, k = 4*(t % KCH) .. +3 of both operands
  const int lrow = t / KCH, lk = (t % KCH) * 4;

  float4 ra[NLD], rb[NLD];
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  for (int kt = 0; kt <= nk; ++kt) {
    if (kt > 0) {
      const int buf = (kt - 1) & 1;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int row = lrow + RPP * i;
        As[buf][lk + 0][row] = ra[i].x; As[buf][lk + 1][row] = ra[i].y;
        As[buf][lk + 2][row] = ra[i].z; As[buf][lk + 3][row] = ra[i].w;
        Bs[buf][lk + 0][row] = rb[i].x; Bs[buf][lk + 1][row] = rb[i].y;
        Bs[buf][lk + 2][row] = rb[i].z; Bs[buf][lk + 3][row] = rb[i].w;
      }
      __syncthreads();
    }
    if (kt < nk) {
      const int k0 = kt * BK;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        ra[i] = gload16f(A + int64_t(lrow + RPP * i) * lda + k0 + lk);
        rb[i] = gload16f(B + int64_t(lrow + RPP * i) * ldb + k0 + lk);
      }
    }
    if (kt > 0) {
      const int cur = (kt - 1) & 1;
#pragma unroll
      for (int kk = 0; kk < BK / 2; ++kk) {
        const int k = kk * 2 + (lane >> 5);
        float a[2], b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) a[i] = As[cur][k][wm * 64 + i * 32 + (lane & 31)];
#pragma unroll
        for (int j = 0; j < 2; ++j) b[j] = Bs[cur][k][wn * 64 + j * 32 + (lane & 31)];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
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
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row0 = tm * BT + wm * 64 + i * 32 + (lane >> 5) * 4;
      const int col = tn * BT + wn * 64 + j * 32 + (lane & 31);
      if (Y)
        store_fragment<true>(acc[i][j], C, T.ldc, Ct, T.ldct, Y, T.ldy, row0, col, alpha, beta, T.gamma,
                             T.diag_limit, mode);
      else
        store_fragment<false>(acc[i][j], C, T.ldc, Ct, T.ldct, Y, T.ldy, row0, col, alpha, beta, T.gamma,
                              T.diag_limit, mode);
    }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmTask* tasks_dev, const TileRef* map_dev, int64_t ntiles,
                            int tile, hipStream_t stream) {
  if (ntiles <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(ntiles));
  // two 64-k stages: 128 KB of LDS at the 256 tile (one block per CU), 64 KB
  // at the 128 tile
  if (tile == 128) {
    hipLaunchKernelGGL((gemm_bf16_kernel<128, 2>), grid, dim3(256), 0, stream, tasks_dev, map_dev);
  } else if (tile == 256) {
    hipLaunchKernelGGL((gemm_bf16_kernel<256, 2>), grid, dim3(256), 0, stream, tasks_dev, map_dev);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmTask* tasks_dev, const TileRef* map_dev, int64_t ntiles,
                           int tile, hipStream_t stream) {
  if (ntiles <= 0) return hipSuccess;
  if (tile == kF32Tile) {
    hipLaunchKernelGGL(gemm_f32_kernel, dim3(static_cast<unsigned>(ntiles)), dim3(256), 0, stream,
                       tasks_dev, map_dev);
  } else if (tile == kF32BigTile) {
    hipLaunchKernelGGL(gemm_f32_big_kernel, dim3(static_cast<unsigned>(ntiles)), dim3(256), 0, stream,
                       tasks_dev, map_dev);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dmuon
