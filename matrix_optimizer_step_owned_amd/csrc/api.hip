// C-ABI entry points of the dmuon library: argument checks, the launch
// planner (grouping every matrix's NS products into one launch per stage),
// launch-table staging and the launch sequence.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <sstream>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/dmuon.h"
#include "internal.h"

namespace dmuon {
namespace {

// ---------------------------------------------------------------------------
// errors
// ---------------------------------------------------------------------------

thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

#define DMUON_HIP_TRY(expr)                                                              \
  do {                                                                                   \
    hipError_t e_ = (expr);                                                              \
    if (e_ != hipSuccess)                                                                \
      return fail(DMUON_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(e_));     \
  } while (0)

constexpr double kDefaultCoeffs[3] = {3.4445, -4.7750, 2.0315};
constexpr int kMaxNsSteps = 16;
constexpr int64_t kMaxDim = int64_t(1) << 22;   // tile coordinates are 16-bit
// the GEMM kernel's operand descriptors span 255 rows of the padded leading
// dimension plus one stage (and per-lane byte offsets are 32-bit)
static_assert(255 * kMaxDim * 2 + 128 < (int64_t(1) << 31), "operand descriptor range");
constexpr size_t kAlign = 256;

size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }
int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
size_t dtype_size(int32_t dt) { return dt == DT_F32 ? 4 : 2; }
bool dtype_ok(int32_t dt) { return dt == DT_F32 || dt == DT_BF16; }

// ---------------------------------------------------------------------------
// hyperparameters
// ---------------------------------------------------------------------------

struct Coeffs {
  std::vector<double> abc;  // 3 per step
};

int check_hparams(const dmuon_hparams_t* hp, bool need_momentum, Coeffs* out) {
  if (!hp) return fail(DMUON_ERR_INVALID_ARG, "hparams is NULL");
  if (hp->ns_steps < 0 || hp->ns_steps > kMaxNsSteps)
    return fail(DMUON_ERR_INVALID_ARG, "ns_steps must be in 0..16");
  if (hp->ns_backend != DMUON_NS_GRAM && hp->ns_backend != DMUON_NS_DIRECT)
    return fail(DMUON_ERR_INVALID_ARG, "ns_backend must be DMUON_NS_GRAM or DMUON_NS_DIRECT");
  if (hp->ns_precision != DMUON_NS_PREC_BF16 && hp->ns_precision != DMUON_NS_PREC_F32)
    return fail(DMUON_ERR_INVALID_ARG, "ns_precision must be BF16 or F32");
  if (!std::isfinite(hp->eps) || hp->eps < 0) return fail(DMUON_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (need_momentum) {
    if (!std::isfinite(hp->lr)) return fail(DMUON_ERR_INVALID_ARG, "lr must be finite");
    if (!std::isfinite(hp->momentum)) return fail(DMUON_ERR_INVALID_ARG, "momentum must be finite");
    if (!std::isfinite(hp->weight_decay)) return fail(DMUON_ERR_INVALID_ARG, "weight_decay must be finite");
  }
  const int K = hp->ns_steps;
  out->abc.clear();
  if (hp->ns_coeffs == nullptr) {
    if (hp->ns_coeffs_len != 0) return fail(DMUON_ERR_INVALID_ARG, "ns_coeffs_len set but ns_coeffs is NULL");
    for (int k = 0; k < K; ++k) out->abc.insert(out->abc.end(), kDefaultCoeffs, kDefaultCoeffs + 3);
  } else if (hp->ns_coeffs_len == 3) {
    for (int k = 0; k < K; ++k) out->abc.insert(out->abc.end(), hp->ns_coeffs, hp->ns_coeffs + 3);
  } else if (hp->ns_coeffs_len == 3 * K && K > 0) {
    out->abc.assign(hp->ns_coeffs, hp->ns_coeffs + 3 * K);
  } else {
    return fail(DMUON_ERR_INVALID_ARG, "ns_coeffs_len must be 3 or 3*ns_steps");
  }
  for (double v : out->abc)
    if (!std::isfinite(v)) return fail(DMUON_ERR_INVALID_ARG, "ns_coeffs must be finite");
  return DMUON_OK;
}

// ---------------------------------------------------------------------------
// plan
// ---------------------------------------------------------------------------

enum Form : int32_t { FORM_DIRECT = 0, FORM_GRAM = 1 };

// The Gram form pays off once the matrix is at least twice as wide as tall:
// it replaces 15 m^2 n + 5 m^3 multiply-adds (symmetric tiles) by
// 3 m^2 n + 17 m^3, and on near-square bf16 inputs its m x m iteration loses
// accuracy, so squarer matrices keep the direct form.
Form choose_form(int32_t backend, int64_t m, int64_t n) {
  if (backend == DMUON_NS_DIRECT) return FORM_DIRECT;
  return n >= 2 * m ? FORM_GRAM : FORM_DIRECT;
}

struct MatLayout {
  int64_t rows, cols, m, n, mp, np;
  int64_t pm, pn; // row pitches (elements) of the buffers whose rows hold mp / np values
  int64_t tile;   // GEMM tile edge of this matrix's products (mp, np are multiples)
  bool tall;      // the wide (m x n) orientation is the transpose of the stored one
  Form form;
  // byte offsets into the workspace (SIZE_MAX when unused); *t buffers hold
  // the transposes (n_pad x m_pad) of the m_pad x n_pad ones; r is a shard's
  // partial Gram matrix (sharded matrices of more than one shard only)
  size_t x0, x0t, x1, x1t, o, a, b, p, t, q0, q1, r;
  size_t out;  // where O is left
};

// One matrix of a call, or one shard of a sharded matrix.  The wide
// orientation is rows x cols, or its transpose when `tall`.
struct ShapeSpec {
  int64_t rows, cols;
  bool tall;
};

// Consecutive entries first .. first + count - 1 form one matrix: its shards
// share the wide row count d, and the matrix's wide column count is the sum
// of theirs (count 1: an ordinary matrix).
struct Group {
  int first, count;
  int64_t d, D;
  Form form;
};

// One GEMM as planned: pointers are workspace byte offsets.
struct Op {
  int mat;
  int tile;
  size_t A, B, C, Ct, Y;  // Ct, Y == SIZE_MAX: none
  int64_t lda, ldb, ldc, ldct, ldy;
  int64_t kr;             // true (unpadded) contraction length
  int32_t K, tiles_m, tiles_n, sym, alpha_pow, beta_pow, diag_limit;
  float alpha, beta, gamma;
  bool scaled;
  bool last;              // the product that yields the matrix's O
};

// One sum of partial Gram matrices, run after the GEMM launches of `stage`.
struct SumPlan {
  int stage;
  size_t dst;
  int64_t ld, edge;
  std::vector<size_t> parts;
};

struct Launch {
  int tile;
  int stage;
  int first;   // index into Plan::ops (sorted order)
  int count;
  int64_t tiles;
  int64_t map_first;  // index of this launch's first entry in Plan::tile_map
  int64_t alg_flops;  // true-size flops, symmetric products counted once
  int64_t alg_bytes;  // bytes an ideal kernel moves
};

struct Plan {
  std::string key;   // the plan cache key: shapes, groups, precision, backend, coefficients
  int n = 0;
  int32_t prec = 0;
  int ns_steps = 0;
  int tile = 0;
  std::vector<MatLayout> mats;
  std::vector<Group> groups;
  std::vector<Op> ops;            // grouped by launch
  std::vector<Launch> launches;
  std::vector<TileRef> tile_map;  // all launches' block -> (task, tile) maps
  std::vector<SumPlan> sums;      // ordered by stage
  int64_t sum_parts = 0;
  std::vector<int64_t> blk_wide, blk_stored;
  int64_t blocks_wide = 0, blocks_stored = 0;
  // workspace layout
  size_t off_ewmats = 0, off_tasks = 0, off_map = 0, off_sums = 0, off_sum_parts = 0;
  size_t off_partials = 0, off_sumsq = 0, off_scale = 0;
  size_t table_bytes = 0;   // EwMat[] + GemmTask[] + TileRef[] + GramSum[] + part pointers
  size_t ws_bytes = 0;
};

size_t kNone = SIZE_MAX;

// DMUON_GEMM_TILE=128|256 forces the bf16 tile edge and
// DMUON_GEMM_TILE_F32=64|128 the fp32 one (0: automatic choice).
int gemm_tile_override(int32_t prec) {
  const bool bf = prec == DMUON_NS_PREC_BF16;
  const char* v = std::getenv(bf ? "DMUON_GEMM_TILE" : "DMUON_GEMM_TILE_F32");
  if (!v) return 0;
  const int t = std::atoi(v);
  if (bf) return (t == kTileBf16 || t == kTileBf16Big) ? t : 0;
  return (t == kTileF32 || t == kTileF32Big) ? t : 0;
}

std::shared_ptr<Plan> build_plan(const std::vector<ShapeSpec>& shapes, const std::vector<Group>& groups_in,
                                 int32_t prec, int32_t backend, const Coeffs& cf, bool with_ns,
                                 int tile_override) {
  auto P = std::make_shared<Plan>();
  const int n = static_cast<int>(shapes.size());
  P->n = n;
  P->prec = prec;
  P->ns_steps = with_ns ? static_cast<int>(cf.abc.size() / 3) : 0;
  // Tile edge: fp32 products use 64.  bf16 products use 256 x 256 tiles
  // (half the LDS traffic per flop of 128 x 128) when the first (X X^T)
  // stage has at least half a wave of them and most of them come from wide
  // matrices (measured: a single 4096^2 matrix, 136 such tiles, runs 12 %
  // faster with them; sixteen 1024^2 matrices, 160 tiles of short K, 8 %
  // slower), and 128 otherwise; matrices narrower than 256 always use 128.
  // fp32 products: 128-tiles (half the operand bytes per flop of 64-tiles,
  // measured 18 % faster on a 4096^2 product) when the first stage has two
  // waves of them, else 64.
  int64_t big_tiles = 0, big_tiles_wide = 0, f32_big_tiles = 0;
  for (const ShapeSpec& s : shapes) {
    const int64_t m = s.tall ? s.cols : s.rows;
    const int64_t t = (m + kTileBf16Big - 1) / kTileBf16Big;
    big_tiles += t * (t + 1) / 2;
    if (m >= kBigTileMinDim) big_tiles_wide += t * (t + 1) / 2;
    const int64_t tf = (m + kTileF32Big - 1) / kTileF32Big;
    f32_big_tiles += tf * (tf + 1) / 2;
  }
  bool use_big = prec == DMUON_NS_PREC_BF16 && big_tiles >= kBigTileMinCount && 2 * big_tiles_wide >= big_tiles;
  if (prec == DMUON_NS_PREC_BF16 && tile_override != 0) use_big = tile_override == kTileBf16Big;
  bool f32_big = prec != DMUON_NS_PREC_BF16 && f32_big_tiles >= kF32BigTileMinCount;
  if (prec != DMUON_NS_PREC_BF16 && tile_override != 0) f32_big = tile_override == kTileF32Big;
  P->tile = prec == DMUON_NS_PREC_BF16 ? (use_big ? kTileBf16Big : kTileBf16)
                                       : (f32_big ? kTileF32Big : kTileF32);
  P->blk_wide.resize(n);
  P->blk_stored.resize(n);
  P->mats.resize(n);
  P->groups = groups_in;
  for (Group& g : P->groups) {
    g.d = shapes[g.first].tall ? shapes[g.first].cols : shapes[g.first].rows;
    g.D = 0;
    for (int i = g.first; i < g.first + g.count; ++i) g.D += shapes[i].tall ? shapes[i].rows : shapes[i].cols;
    g.form = choose_form(backend, g.d, g.D);
    for (int i = g.first; i < g.first + g.count; ++i) {
      MatLayout& L = P->mats[i];
      L.rows = shapes[i].rows;
      L.cols = shapes[i].cols;
      L.tall = shapes[i].tall;
      L.m = g.d;
      L.n = L.tall ? L.rows : L.cols;
      L.tile = prec == DMUON_NS_PREC_BF16 ? ((use_big && g.d >= 256) ? kTileBf16Big : kTileBf16)
                                          : ((f32_big && g.d >= kTileF32Big) ? kTileF32Big : kTileF32);
      L.mp = with_ns ? round_up(L.m, L.tile) : L.m;
      L.np = with_ns ? round_up(L.n, L.tile) : L.n;
      // one extra 128-byte line per row: rows of a power-of-two-like pitch
      // would otherwise start at the same offsets of the L2 channel
      // interleave, and a k-slice of a panel would land on a few channels
      L.pm = with_ns ? L.mp + kPitchPad : L.mp;
      L.pn = with_ns ? L.np + kPitchPad : L.np;
      L.form = g.form;
      L.x0 = L.x0t = L.x1 = L.x1t = L.o = L.a = L.b = L.p = L.t = L.q0 = L.q1 = L.r = L.out = kNone;
      P->blk_wide[i] = P->blocks_wide;
      P->blocks_wide += ((L.mp + kEwTile - 1) / kEwTile) * ((L.np + kEwTile - 1) / kEwTile);
      P->blk_stored[i] = P->blocks_stored;
      P->blocks_stored += ((L.rows + kEwTile - 1) / kEwTile) * ((L.cols + kEwTile - 1) / kEwTile);
    }
  }
  return P;  // buffers are laid out by layout_plan()
}

Op base_op(int mat, int64_t tile) {
  Op o{};
  o.mat = mat; o.tile = static_cast<int>(tile);
  o.Ct = kNone; o.Y = kNone; o.ldct = 0; o.ldy = 0;
  o.alpha = 1.f; o.beta = 0.f; o.gamma = 0.f; o.diag_limit = 0;
  o.alpha_pow = o.beta_pow = 0; o.scaled = false;
  return o;
}

// Symmetric d x d result A B^T of two row-major operands with leading
// dimension ldab and padded contraction length Kpad (true length kr).
Op sym_op(int mat, const MatLayout& G, size_t A, size_t B, size_t C, size_t Y, int64_t ldab, int64_t Kpad,
          int64_t kr) {
  Op o = base_op(mat, G.tile);
  o.A = A; o.B = B; o.C = C; o.Y = Y;
  o.lda = o.ldb = ldab; o.ldc = G.pm; o.ldy = G.pm;
  o.K = static_cast<int32_t>(Kpad); o.kr = kr;
  o.tiles_m = o.tiles_n = static_cast<int32_t>(G.mp / G.tile); o.sym = 1;
  return o;
}

// d x n_i result M . X of one matrix or shard S, where M is d x d and X^T
// (n_i x d) is stored.
Op left_op(int mat, const MatLayout& S, size_t M, size_t Xt, size_t C, size_t Ct) {
  Op o = base_op(mat, S.tile);
  o.A = M; o.B = Xt; o.C = C; o.Ct = Ct;
  o.lda = S.pm; o.ldb = S.pm; o.ldc = S.pn; o.ldct = S.pm;
  o.K = static_cast<int32_t>(S.mp); o.kr = S.m;
  o.tiles_m = static_cast<int32_t>(S.mp / S.tile);
  o.tiles_n = static_cast<int32_t>(S.np / S.tile);
  o.sym = 0;
  return o;
}

// Stage lists of the NS iteration, per group (kept on the group's first
// entry).  Every product is C = alpha * A B^T (+ beta Y + gamma I) with
// K-contiguous operands; the m x n operand of the left-multiplications comes
// from its transpose.  A group of several shards forms its Gram matrices as
// one partial product per shard followed by their sum (a SumPlan after that
// stage): once (Gram form) or every iteration (direct form); the d x d
// products run once per group and the left products once per shard.
void plan_ops(Plan& P, const Coeffs& cf, std::vector<std::vector<std::vector<Op>>>& stages) {
  const int K = P.ns_steps;
  stages.assign(P.n, {});
  P.sums.clear();
  for (const Group& g : P.groups) {
    const int f = g.first, e = g.first + g.count;
    MatLayout& G = P.mats[f];
    auto& st = stages[f];
    if (K == 0) {
      for (int i = f; i < e; ++i) P.mats[i].out = P.mats[i].x0;
      continue;
    }
    // the Gram products of every shard of stage `stage`, into A directly for
    // a single shard, else into the shards' partial buffers and then summed
    auto gram_products = [&](int stage, const size_t* xin, bool first) {
      std::vector<Op> ops;
      for (int i = f; i < e; ++i) {
        const MatLayout& S = P.mats[i];
        Op o = sym_op(i, G, xin[i - f], xin[i - f], g.count > 1 ? S.r : G.a, kNone, S.pn, S.np, S.n);
        if (first) { o.alpha_pow = 2; o.scaled = true; }
        ops.push_back(o);
      }
      if (g.count > 1) {
        SumPlan sp;
        sp.stage = stage; sp.dst = G.a; sp.ld = G.pm; sp.edge = G.mp;
        for (int i = f; i < e; ++i) sp.parts.push_back(P.mats[i].r);
        P.sums.push_back(sp);
      }
      return ops;
    };
    std::vector<size_t> x0(g.count), x0t(g.count), x1(g.count), x1t(g.count);
    for (int i = f; i < e; ++i) {
      x0[i - f] = P.mats[i].x0; x0t[i - f] = P.mats[i].x0t;
      x1[i - f] = P.mats[i].x1; x1t[i - f] = P.mats[i].x1t;
    }
    if (g.form == FORM_DIRECT) {
      const std::vector<size_t>* xb[2] = {&x0, &x1};
      const std::vector<size_t>* xtb[2] = {&x0t, &x1t};
      for (int k = 0; k < K; ++k) {
        const double a = cf.abc[3 * k], b = cf.abc[3 * k + 1], c = cf.abc[3 * k + 2];
        const std::vector<size_t>& xin = *xb[k % 2];
        const std::vector<size_t>& xin_t = *xtb[k % 2];
        const std::vector<size_t>& xout = *xb[(k + 1) % 2];
        const std::vector<size_t>& xout_t = *xtb[(k + 1) % 2];
        // A = s^2 X X^T (s folded in on the first step only)
        st.push_back(gram_products(static_cast<int>(st.size()), xin.data(), k == 0));
        // B = b A + c A A
        Op h = sym_op(f, G, G.a, G.a, G.b, G.a, G.pm, G.mp, G.m);
        h.alpha = static_cast<float>(c);
        h.beta = static_cast<float>(b);
        st.push_back({h});
        // X' = a X + B X, and X'^T for the next step's left product
        std::vector<Op> upd;
        for (int i = f; i < e; ++i) {
          const MatLayout& S = P.mats[i];
          Op u = left_op(i, S, G.b, xin_t[i - f], xout[i - f], k + 1 < K ? xout_t[i - f] : kNone);
          u.Y = xin[i - f]; u.ldy = S.pn;
          u.beta = static_cast<float>(a);
          u.alpha_pow = u.beta_pow = (k == 0) ? 1 : 0;
          u.scaled = (k == 0);
          u.last = k + 1 == K;
          upd.push_back(u);
        }
        st.push_back(upd);
      }
      for (int i = f; i < e; ++i) P.mats[i].out = (*xb[K % 2])[i - f];
    } else {
      // R = s^2 X0 X0^T, kept in A
      st.push_back(gram_products(0, x0.data(), true));
      const size_t qbuf[2] = {G.q0, G.q1};
      for (int k = 0; k < K; ++k) {
        const double a = cf.abc[3 * k], b = cf.abc[3 * k + 1], c = cf.abc[3 * k + 2];
        const size_t pk = (k == 0) ? G.q0 : G.p;   // P_0 is Q itself
        Op pp = sym_op(f, G, G.a, G.a, pk, G.a, G.pm, G.mp, G.m);
        pp.alpha = static_cast<float>(c);
        pp.beta = static_cast<float>(b);
        pp.gamma = static_cast<float>(a);
        pp.diag_limit = static_cast<int32_t>(G.m);
        st.push_back({pp});
        std::vector<Op> next;
        if (k >= 1) next.push_back(sym_op(f, G, pk, qbuf[(k - 1) % 2], qbuf[k % 2], kNone, G.pm, G.mp, G.m));  // Q <- P Q
        if (k + 1 < K) next.push_back(sym_op(f, G, pk, G.a, G.t, kNone, G.pm, G.mp, G.m));                     // T = P A
        if (!next.empty()) st.push_back(next);
        if (k + 1 < K) st.push_back({sym_op(f, G, G.t, pk, G.a, kNone, G.pm, G.mp, G.m)});                     // A = T P
      }
      std::vector<Op> fin;
      for (int i = f; i < e; ++i) {
        MatLayout& S = P.mats[i];
        Op o = left_op(i, S, qbuf[(K - 1) % 2], S.x0t, S.o, kNone);                                            // O = s Q X0
        o.alpha_pow = 1; o.scaled = true; o.last = true;
        fin.push_back(o);
        S.out = S.o;
      }
      st.push_back(fin);
    }
  }
  std::stable_sort(P.sums.begin(), P.sums.end(), [](const SumPlan& x, const SumPlan& y) { return x.stage < y.stage; });
}

int64_t op_tiles(const Op& o) {
  return o.sym ? int64_t(o.tiles_m) * (o.tiles_m + 1) / 2 : int64_t(o.tiles_m) * o.tiles_n;
}
// Output tiles of one product in the order one XCD walks them: groups of
// kTileGroupRows x kTileGroupCols tiles, group-row by group-row, so the tiles
// an XCD runs at once share their A and B panels; symmetric products keep
// tn >= tm only.
void op_tile_order(const Op& o, std::vector<std::pair<int, int>>& out) {
  out.clear();
  const int GR = kTileGroupRows, GC = kTileGroupCols;
  for (int bi = 0; bi < o.tiles_m; bi += GR)
    for (int bj = o.sym ? (bi / GC) * GC : 0; bj < o.tiles_n; bj += GC)
      for (int tm = bi; tm < std::min(bi + GR, o.tiles_m); ++tm)
        for (int tn = bj; tn < std::min(bj + GC, o.tiles_n); ++tn)
          if (!o.sym || tn >= tm) out.emplace_back(tm, tn);
}

// Block -> tile maps.  The hardware deals the blocks of a launch to the XCDs
// round-robin (block b runs on XCD b % 8), and each XCD has its own L2, so
// the blocks an XCD runs at once should be neighbouring tiles of one task.
// Tasks (longest k first, then largest) go whole to the XCD with the most
// room left; a task larger than that room is split, so every XCD's list is
// exactly as long as the number of blocks the hardware sends it and every
// XCD gets a like mix of short and long tasks.
void build_tile_maps(Plan& P) {
  P.tile_map.clear();
  std::vector<std::pair<int, int>> order;
  for (Launch& l : P.launches) {
    l.map_first = static_cast<int64_t>(P.tile_map.size());
    int64_t room[kNumXcd];
    for (int x = 0; x < kNumXcd; ++x) room[x] = l.tiles / kNumXcd + (x < l.tiles % kNumXcd ? 1 : 0);
    std::vector<int> idx(l.count);
    for (int j = 0; j < l.count; ++j) idx[j] = j;
    std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) {
      const Op& oa = P.ops[l.first + a];
      const Op& ob = P.ops[l.first + b];
      if (oa.K != ob.K) return oa.K > ob.K;
      return op_tiles(oa) > op_tiles(ob);
    });
    std::vector<std::vector<TileRef>> xl(kNumXcd);
    bool ok = true;
    for (int j : idx) {
      op_tile_order(P.ops[l.first + j], order);
      size_t pos = 0;
      while (pos < order.size()) {
        int x = 0;
        for (int y = 1; y < kNumXcd; ++y)
          if (room[y] > room[x]) x = y;
        if (room[x] <= 0) { ok = false; break; }
        const size_t take = std::min<size_t>(static_cast<size_t>(room[x]), order.size() - pos);
        for (size_t k = 0; k < take; ++k, ++pos)
          xl[x].push_back({j, static_cast<uint16_t>(order[pos].first), static_cast<uint16_t>(order[pos].second)});
        room[x] -= static_cast<int64_t>(take);
      }
      if (!ok) break;
    }
    for (int x = 0; x < kNumXcd; ++x) ok = ok && room[x] == 0;
    if (ok) {
      for (int64_t b = 0; b < l.tiles; ++b) P.tile_map.push_back(xl[b % kNumXcd][b / kNumXcd]);
    } else {
      // (cannot happen: the rooms add up to the tile count; a plain
      // task-by-task order keeps the map valid regardless)
      for (int j = 0; j < l.count; ++j) {
        op_tile_order(P.ops[l.first + j], order);
        for (auto& t : order)
          P.tile_map.push_back({j, static_cast<uint16_t>(t.first), static_cast<uint16_t>(t.second)});
      }
    }
  }
}

// Lay out workspace buffers and group ops into launches.
void layout_plan(Plan& P, const Coeffs& cf, bool with_ns) {
  const size_t es = P.prec == DMUON_NS_PREC_BF16 ? 2 : 4;
  // buffers: per group, its shards' own buffers, then the group's d x d ones
  size_t cur = 0;  // relative to the start of the matrix region
  const bool ns = with_ns && P.ns_steps > 0;
  for (const Group& g : P.groups) {
    for (int i = g.first; i < g.first + g.count; ++i) {
      MatLayout& L = P.mats[i];
      const size_t mn = align_up(size_t(L.mp) * L.pn * es);    // m x n, pitch pn
      const size_t mnt = align_up(size_t(L.np) * L.pm * es);   // n x m, pitch pm
      L.x0 = cur; cur += mn;
      if (!ns) continue;
      L.x0t = cur; cur += mnt;
      if (L.form == FORM_DIRECT) {
        L.x1 = cur; cur += mn;
        if (P.ns_steps > 1) { L.x1t = cur; cur += mnt; }
      } else {
        L.o = cur; cur += mn;
      }
      if (g.count > 1) { L.r = cur; cur += align_up(size_t(L.mp) * L.pm * es); }
    }
    if (!ns) continue;
    MatLayout& G = P.mats[g.first];
    const size_t mm = align_up(size_t(G.mp) * G.pm * es);    // d x d, pitch pm
    if (G.form == FORM_DIRECT) {
      G.a = cur; cur += mm;
      G.b = cur; cur += mm;
    } else {
      G.a = cur; cur += mm;
      G.p = cur; cur += mm;
      G.t = cur; cur += mm;
      G.q0 = cur; cur += mm;
      G.q1 = cur; cur += mm;
    }
  }
  const size_t mat_region = cur;

  std::vector<std::vector<std::vector<Op>>> stages;
  if (with_ns) plan_ops(P, cf, stages);
  else for (auto& L : P.mats) L.out = L.x0;

  // group: stage s, NT then NN; largest K first (LPT order)
  size_t max_st = 0;
  for (auto& st : stages) max_st = std::max(max_st, st.size());
  P.ops.clear();
  P.launches.clear();
  for (size_t s = 0; s < max_st; ++s) {
    // (the fp32 128-tile has the edge of the bf16 small tile: one plan holds
    // products of one precision only, so the edges below cover both)
    static_assert(kTileF32Big == kTileBf16, "tile edges");
    for (int tile : {kTileBf16Big, kTileBf16, kTileF32}) {
      std::vector<Op> group;
      for (auto& st : stages)
        if (s < st.size())
          for (auto& o : st[s])
            if (o.tile == tile) group.push_back(o);
      if (group.empty()) continue;
      std::stable_sort(group.begin(), group.end(), [](const Op& x, const Op& y) { return x.K > y.K; });
      Launch l{tile, static_cast<int>(s), static_cast<int>(P.ops.size()), static_cast<int>(group.size()),
               0, 0, 0, 0};
      const int64_t es = P.prec == DMUON_NS_PREC_BF16 ? 2 : 4;
      for (auto& o : group) {
        l.tiles += op_tiles(o);
        const MatLayout& L = P.mats[o.mat];
        const int64_t m = L.m, n = L.n;
        const bool has_y = o.Y != kNone;
        if (o.sym) {
          l.alg_flops += m * (m + 1) * o.kr;
          l.alg_bytes += es * (m * o.kr * (o.A == o.B ? 1 : 2) + (has_y ? m * m : 0) + m * m);
        } else {
          l.alg_flops += 2 * m * n * m;
          l.alg_bytes += es * (m * m + m * n + (has_y ? m * n : 0) + m * n * (o.Ct != kNone ? 2 : 1));
        }
      }
      P.ops.insert(P.ops.end(), group.begin(), group.end());
      P.launches.push_back(l);
    }
  }

  build_tile_maps(P);

  // workspace: [EwMat table][GemmTask table][tile maps][Gram sums][their
  // part pointers][partials][sumsq][scale][matrices]
  P.sum_parts = 0;
  for (const SumPlan& sp : P.sums) P.sum_parts += static_cast<int64_t>(sp.parts.size());
  size_t off = 0;
  P.off_ewmats = off;
  off += align_up(sizeof(EwMat) * std::max(P.n, 1));
  P.off_tasks = off;
  off += align_up(sizeof(GemmTask) * std::max<size_t>(P.ops.size(), 1));
  P.off_map = off;
  off += align_up(sizeof(TileRef) * std::max<size_t>(P.tile_map.size(), 1));
  P.off_sums = off;
  if (!P.sums.empty()) off += align_up(sizeof(GramSum) * P.sums.size());
  P.off_sum_parts = off;
  if (P.sum_parts > 0) off += align_up(sizeof(void*) * size_t(P.sum_parts));
  P.table_bytes = off;
  P.off_partials = off;
  off += align_up(sizeof(float) * std::max<int64_t>(P.blocks_wide, 1));
  P.off_sumsq = off;
  off += align_up(sizeof(double) * std::max(P.n, 1));
  P.off_scale = off;
  off += align_up(sizeof(float) * std::max(P.n, 1));
  for (auto& L : P.mats) {
    for (size_t* f : {&L.x0, &L.x0t, &L.x1, &L.x1t, &L.o, &L.a, &L.b, &L.p, &L.t, &L.q0, &L.q1, &L.r, &L.out})
      if (*f != kNone) *f += off;
  }
  for (auto& o : P.ops)
    for (size_t* f : {&o.A, &o.B, &o.C, &o.Ct, &o.Y})
      if (*f != kNone) *f += off;
  for (auto& sp : P.sums) {
    sp.dst += off;
    for (size_t& q : sp.parts) q += off;
  }
  P.ws_bytes = off + mat_region;
}

// ---------------------------------------------------------------------------
// plan cache
// ---------------------------------------------------------------------------

std::mutex g_plan_mu;
std::unordered_map<std::string, std::shared_ptr<Plan>> g_plans;

std::shared_ptr<Plan> get_plan(const std::vector<ShapeSpec>& shapes, const std::vector<Group>& groups,
                               int32_t prec, int32_t backend, const Coeffs& cf, bool with_ns) {
  std::string key;
  key.reserve(32 + shapes.size() * 24 + groups.size() * 8 + cf.abc.size() * 8);
  auto put = [&](const void* p, size_t n) { key.append(static_cast<const char*>(p), n); };
  const int tile_override = gemm_tile_override(prec);
  const int32_t hdr[4] = {prec, with_ns ? backend : -1, with_ns ? 1 : 0, tile_override};
  put(hdr, sizeof(hdr));
  const int64_t n = static_cast<int64_t>(shapes.size()), ng = static_cast<int64_t>(groups.size());
  put(&n, sizeof(n));
  put(&ng, sizeof(ng));
  for (const ShapeSpec& s : shapes) {
    const int64_t v[3] = {s.rows, s.cols, s.tall ? 1 : 0};
    put(v, sizeof(v));
  }
  for (const Group& g : groups) {
    const int32_t v[2] = {g.first, g.count};
    put(v, sizeof(v));
  }
  if (with_ns) put(cf.abc.data(), cf.abc.size() * sizeof(double));
  {
    std::lock_guard<std::mutex> lk(g_plan_mu);
    auto it = g_plans.find(key);
    if (it != g_plans.end()) return it->second;
  }
  auto P = build_plan(shapes, groups, prec, backend, cf, with_ns, tile_override);
  layout_plan(*P, cf, with_ns);
  P->key = key;
  std::lock_guard<std::mutex> lk(g_plan_mu);
  if (g_plans.size() > 256) g_plans.clear();
  g_plans.emplace(key, P);
  return P;
}

// The plan of independent whole matrices: each in its wide orientation
// (transposed when tall), one group each.
std::shared_ptr<Plan> get_plan(const std::vector<int64_t>& rows, const std::vector<int64_t>& cols,
                               int32_t prec, int32_t backend, const Coeffs& cf, bool with_ns) {
  std::vector<ShapeSpec> shapes(rows.size());
  std::vector<Group> groups(rows.size());
  for (size_t i = 0; i < rows.size(); ++i) {
    shapes[i] = {rows[i], cols[i], rows[i] > cols[i]};
    groups[i] = {static_cast<int>(i), 1, 0, 0, FORM_DIRECT};
  }
  return get_plan(shapes, groups, prec, backend, cf, with_ns);
}

// ---------------------------------------------------------------------------
// device check and launch-table staging
// ---------------------------------------------------------------------------

// Launch tables reach the device as one copy per call from a pinned host
// image.  An image depends only on what it was filled from (the plan and
// the caller's pointers and scalars, its `key`), so images are cached per
// device and never changed while cached: a call whose key matches an image
// enqueues the copy and nothing else, and any number of copies of one image
// may be in flight.  Every copy records an event; an image is refilled for
// another key only once all its events have completed, which the host
// queries without waiting.  The host blocks only when more than
// kMaxTableImages images on one device all still have copies in flight.
constexpr size_t kTableImagesKept = 16;
constexpr size_t kMaxTableImages = 64;

struct TableImage {
  std::string key;
  void* host = nullptr;   // pinned; `bytes` valid, `cap` allocated
  size_t cap = 0, bytes = 0;
  std::vector<hipEvent_t> pending;   // events behind copies not yet known complete
  uint64_t last_use = 0;
};

struct DeviceState {
  bool checked = false;
  bool ok = false;
  std::string arch;
  std::vector<std::unique_ptr<TableImage>> images;
  std::vector<hipEvent_t> free_events;
  uint64_t clock = 0;
};

std::mutex g_dev_mu;
std::map<int, DeviceState> g_dev;

int current_device_state(DeviceState** out) {
  int dev = 0;
  DMUON_HIP_TRY(hipGetDevice(&dev));
  DeviceState& d = g_dev[dev];
  if (!d.checked) {
    hipDeviceProp_t prop;
    DMUON_HIP_TRY(hipGetDeviceProperties(&prop, dev));
    d.arch = prop.gcnArchName;
    d.ok = d.arch.rfind("gfx950", 0) == 0;
    d.checked = true;
  }
  if (!d.ok) return fail(DMUON_ERR_UNSUPPORTED, "device arch " + d.arch + " is not gfx950");
  *out = &d;
  return DMUON_OK;
}

// Drops the image's completed events (returned to the pool); true when none
// is left in flight.
int retire_events(DeviceState& d, TableImage& im, bool* idle) {
  size_t k = 0;
  for (hipEvent_t e : im.pending) {
    const hipError_t q = hipEventQuery(e);
    if (q == hipSuccess) {
      d.free_events.push_back(e);
    } else if (q == hipErrorNotReady) {
      im.pending[k++] = e;
    } else {
      return fail(DMUON_ERR_HIP, std::string("hipEventQuery: ") + hipGetErrorString(q));
    }
  }
  im.pending.resize(k);
  *idle = k == 0;
  return DMUON_OK;
}

// Appends the object representation of trivially copyable values to a key.
struct KeyBuf {
  std::string s;
  template <class T>
  KeyBuf& put(const T& v) {
    s.append(reinterpret_cast<const char*>(&v), sizeof(T));
    return *this;
  }
  KeyBuf& put_str(const std::string& v) {
    put(v.size());
    s.append(v);
    return *this;
  }
};

// Copy `bytes` of launch table to device address `dst` on `stream`.  `key`
// must hold everything `fill` reads; `fill` writes the table into a zeroed
// host buffer and runs only when no cached image matches.
template <class Fill>
int stage_table(void* dst, size_t bytes, hipStream_t stream, const std::string& key, Fill fill) {
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DeviceState* d = nullptr;
  int st = current_device_state(&d);
  if (st != DMUON_OK) return st;
  KeyBuf full;
  full.put(dst).put(bytes).put_str(key);
  TableImage* im = nullptr;
  for (auto& p : d->images)
    if (p->bytes == bytes && p->key == full.s) { im = p.get(); break; }
  if (!im) {
    // an idle image to refill (least recently used first), else a new one
    std::vector<TableImage*> by_age;
    for (auto& p : d->images) by_age.push_back(p.get());
    std::sort(by_age.begin(), by_age.end(), [](const TableImage* a, const TableImage* b) {
      return a->last_use < b->last_use;
    });
    if (d->images.size() >= kTableImagesKept) {
      for (TableImage* c : by_age) {
        bool idle = false;
        st = retire_events(*d, *c, &idle);
        if (st != DMUON_OK) return st;
        if (idle) { im = c; break; }
      }
    }
    if (!im && d->images.size() >= kMaxTableImages) {
      // every image has a copy in flight: wait for the oldest
      im = by_age.front();
      for (hipEvent_t e : im->pending) {
        DMUON_HIP_TRY(hipEventSynchronize(e));
        d->free_events.push_back(e);
      }
      im->pending.clear();
    }
    if (!im) {
      d->images.push_back(std::make_unique<TableImage>());
      im = d->images.back().get();
    }
    if (im->cap < bytes) {
      if (im->host) DMUON_HIP_TRY(hipHostFree(im->host));
      im->host = nullptr;
      im->cap = 0;
      size_t cap = size_t(1) << 16;
      while (cap < bytes) cap <<= 1;
      DMUON_HIP_TRY(hipHostMalloc(&im->host, cap, hipHostMallocDefault));
      im->cap = cap;
    }
    im->key.clear();   // not a valid image until filled
    std::memset(im->host, 0, bytes);
    fill(static_cast<char*>(im->host));
    im->key = full.s;
    im->bytes = bytes;
  }
  im->last_use = ++d->clock;
  bool idle = false;
  st = retire_events(*d, *im, &idle);
  if (st != DMUON_OK) return st;
  hipEvent_t ev = nullptr;
  if (!d->free_events.empty()) {
    ev = d->free_events.back();
    d->free_events.pop_back();
  } else {
    DMUON_HIP_TRY(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
  }
  const hipError_t ce = launch_table_copy(dst, im->host, bytes, stream);
  if (ce != hipSuccess) {
    d->free_events.push_back(ev);
    return fail(DMUON_ERR_HIP, std::string("table copy: ") + hipGetErrorString(ce));
  }
  const hipError_t re = hipEventRecord(ev, stream);
  if (re != hipSuccess) {
    // the copy may be in flight with no event behind it: the buffer is left
    // allocated and no image refers to it any more
    im->host = nullptr;
    im->cap = im->bytes = 0;
    im->key.clear();
    d->free_events.push_back(ev);
    return fail(DMUON_ERR_HIP, std::string("table event: ") + hipGetErrorString(re));
  }
  im->pending.push_back(ev);
  return DMUON_OK;
}

int check_device() {
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DeviceState* d = nullptr;
  return current_device_state(&d);
}

// ---------------------------------------------------------------------------
// measurement hooks
// ---------------------------------------------------------------------------

enum ProfKind { PK_MOMENTUM, PK_FINALIZE, PK_GEMM_BF16, PK_GEMM_F32, PK_UPDATE,
                PK_CLIP_NORM, PK_CLIP_FINALIZE, PK_CLIP_SCALE, PK_GRAM_SUM, PK_ADAMW, PK_COUNT };
const char* const kProfNames[PK_COUNT] = {"momentum", "finalize", "gemm_bf16", "gemm_f32", "update",
                                          "clip_norm", "clip_finalize", "clip_scale", "gram_sum",
                                          "adamw"};

struct ProfRec {
  int kind;
  int64_t flops, bytes;
  hipEvent_t a, b;
};

std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof;

template <class F>
hipError_t prof_launch(int kind, int64_t flops, int64_t bytes, hipStream_t stream, F launch) {
  bool on;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    on = g_prof_on;
  }
  if (!on) return launch();
  hipEvent_t a = nullptr, b = nullptr;
  hipError_t e = hipEventCreate(&a);
  if (e == hipSuccess) e = hipEventCreate(&b);
  if (e == hipSuccess) e = hipEventRecord(a, stream);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  e = hipEventRecord(b, stream);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof.push_back({kind, flops, bytes, a, b});
  return e;
}

// ---------------------------------------------------------------------------
// validation helpers
// ---------------------------------------------------------------------------

struct Range {
  uintptr_t lo, hi;
  std::string what;
};

int check_overlaps(std::vector<Range>& r) {
  std::sort(r.begin(), r.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  for (size_t i = 1; i < r.size(); ++i)
    if (r[i].lo < r[i - 1].hi)
      return fail(DMUON_ERR_ALIASING, r[i - 1].what + " overlaps " + r[i].what);
  return DMUON_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

float lr_eff_of(double lr, int64_t rows, int64_t cols) {
  return static_cast<float>(lr * 0.2 * std::sqrt(static_cast<double>(std::max(rows, cols))));
}

// Where the last product of a matrix updates its parameter instead of
// leaving O in the workspace (dmuon_step with bf16 products).
struct FusedUpdate {
  void* param;
  int32_t dtype;
  float lr_eff, decay;
};

void fill_tasks(const Plan& P, char* ws_base, GemmTask* out, const FusedUpdate* fused = nullptr) {
  auto ptr = [&](size_t off) -> void* { return off == kNone ? nullptr : ws_base + off; };
  for (const Launch& l : P.launches) {
    for (int j = 0; j < l.count; ++j) {
      const Op& o = P.ops[l.first + j];
      GemmTask& t = out[l.first + j];
      t.A = ptr(o.A);
      t.B = ptr(o.B);
      t.C = ptr(o.C);
      t.Ct = ptr(o.Ct);
      t.Y = ptr(o.Y);
      t.scale = o.scaled ? reinterpret_cast<const float*>(ws_base + P.off_scale) + o.mat : nullptr;
      t.lda = o.lda; t.ldb = o.ldb; t.ldc = o.ldc; t.ldct = o.ldct; t.ldy = o.ldy;
      t.K = o.K; t.tiles_m = o.tiles_m; t.tiles_n = o.tiles_n; t.sym = o.sym;
      t.alpha_pow = o.alpha_pow; t.beta_pow = o.beta_pow; t.diag_limit = o.diag_limit;
      t.alpha = o.alpha; t.beta = o.beta; t.gamma = o.gamma;
      if (fused && o.last) {
        const MatLayout& L = P.mats[o.mat];
        const FusedUpdate& f = fused[o.mat];
        t.W = f.param;
        t.ldw = L.cols;
        t.w_m = static_cast<int32_t>(L.m);
        t.w_n = static_cast<int32_t>(L.n);
        t.w_dtype = f.dtype;
        t.w_tall = L.tall ? 1 : 0;
        t.w_vec = (L.cols % 8 == 0) && (reinterpret_cast<uintptr_t>(f.param) % 16 == 0);   // 8 bf16 = 16 bytes
        t.lr_eff = f.lr_eff;
        t.decay = f.decay;
      }
    }
  }
  if (!P.tile_map.empty())
    std::memcpy(reinterpret_cast<char*>(out) + (P.off_map - P.off_tasks), P.tile_map.data(),
                sizeof(TileRef) * P.tile_map.size());
  // Gram sums: entries of one stage are contiguous; blk_first counts from
  // the first entry of that stage (one launch per stage)
  GramSum* sums = reinterpret_cast<GramSum*>(reinterpret_cast<char*>(out) + (P.off_sums - P.off_tasks));
  void** parts = reinterpret_cast<void**>(reinterpret_cast<char*>(out) + (P.off_sum_parts - P.off_tasks));
  int32_t part = 0;
  int64_t blk = 0;
  for (size_t j = 0; j < P.sums.size(); ++j) {
    const SumPlan& sp = P.sums[j];
    if (j == 0 || P.sums[j - 1].stage != sp.stage) blk = 0;
    GramSum& g = sums[j];
    g.dst = ws_base + sp.dst;
    g.ld = sp.ld;
    g.blk_first = blk;
    g.edge = static_cast<int32_t>(sp.edge);
    g.first_part = part;
    g.count = static_cast<int32_t>(sp.parts.size());
    for (size_t q : sp.parts) parts[part++] = ws_base + q;
    blk += (sp.edge / kEwTile) * (sp.edge / kEwTile);
  }
}

// The GEMM launches in stage order; after the last launch of a stage, the
// Gram sums planned for that stage (sharded matrices only).
int run_gemms(const Plan& P, char* ws, hipStream_t stream) {
  const GemmTask* tasks = reinterpret_cast<const GemmTask*>(ws + P.off_tasks);
  const TileRef* map = reinterpret_cast<const TileRef*>(ws + P.off_map);
  const GramSum* sums = reinterpret_cast<const GramSum*>(ws + P.off_sums);
  const void* const* parts = reinterpret_cast<const void* const*>(ws + P.off_sum_parts);
  const bool bf = P.prec == DMUON_NS_PREC_BF16;
  const int64_t es = bf ? 2 : 4;
  size_t next_sum = 0;
  for (size_t li = 0; li < P.launches.size(); ++li) {
    const Launch& l = P.launches[li];
    hipError_t e = prof_launch(bf ? PK_GEMM_BF16 : PK_GEMM_F32, l.alg_flops, l.alg_bytes, stream, [&] {
      return bf ? launch_gemm_bf16(tasks + l.first, map + l.map_first, l.tiles, l.tile, stream)
                : launch_gemm_f32(tasks + l.first, map + l.map_first, l.tiles, l.tile, stream);
    });
    if (e != hipSuccess) return fail(DMUON_ERR_HIP, std::string("GEMM launch: ") + hipGetErrorString(e));
    const bool stage_end = li + 1 == P.launches.size() || P.launches[li + 1].stage != l.stage;
    if (!stage_end) continue;
    size_t end = next_sum;
    int64_t blocks = 0, bytes = 0;
    while (end < P.sums.size() && P.sums[end].stage == l.stage) {
      const SumPlan& sp = P.sums[end];
      const int64_t tiles = (sp.edge / kEwTile) * (sp.edge / kEwTile);
      blocks += tiles;
      bytes += es * sp.edge * sp.edge * int64_t(sp.parts.size() + 1);
      ++end;
    }
    if (end == next_sum) continue;
    e = prof_launch(PK_GRAM_SUM, 0, bytes, stream, [&] {
      return launch_gram_sum(sums + next_sum, static_cast<int>(end - next_sum), blocks, parts,
                             bf ? DT_BF16 : DT_F32, stream);
    });
    if (e != hipSuccess) return fail(DMUON_ERR_HIP, std::string("Gram sum launch: ") + hipGetErrorString(e));
    next_sum = end;
  }
  return DMUON_OK;
}

int check_matrix_fields(const dmuon_matrix_t& m, int i, bool need_grad_mom) {
  char buf[160];
  if (m.rows <= 0 || m.cols <= 0) {
    std::snprintf(buf, sizeof buf, "matrix %d: rows and cols must be > 0", i);
    return fail(DMUON_ERR_INVALID_ARG, buf);
  }
  if (m.rows > kMaxDim || m.cols > kMaxDim) {
    std::snprintf(buf, sizeof buf, "matrix %d: dimension above 2^22", i);
    return fail(DMUON_ERR_INVALID_ARG, buf);
  }
  if (!dtype_ok(m.param_dtype) || !dtype_ok(m.grad_dtype)) {
    std::snprintf(buf, sizeof buf, "matrix %d: dtype must be DMUON_F32 or DMUON_BF16", i);
    return fail(DMUON_ERR_UNSUPPORTED, buf);
  }
  if (need_grad_mom && m.momentum == nullptr) {
    std::snprintf(buf, sizeof buf, "matrix %d: momentum is NULL", i);
    return fail(DMUON_ERR_INVALID_ARG, buf);
  }
  return DMUON_OK;
}

std::string mat_name(const char* what, int i) { return std::string(what) + "[" + std::to_string(i) + "]"; }

}  // namespace
}  // namespace dmuon

namespace dmuon {
int set_last_error(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}
}  // namespace dmuon

using namespace dmuon;

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

extern "C" {

void dmuon_hparams_default(dmuon_hparams_t* hp) {
  if (!hp) return;
  hp->lr = 0.02;
  hp->momentum = 0.95;
  hp->nesterov = 1;
  hp->ns_steps = 5;
  hp->weight_decay = 0.0;
  hp->ns_backend = DMUON_NS_GRAM;
  hp->ns_precision = DMUON_NS_PREC_BF16;
  hp->ns_coeffs = nullptr;
  hp->ns_coeffs_len = 0;
  hp->eps = 1e-7;
}

const char* dmuon_status_string(int status) {
  switch (status) {
    case DMUON_OK: return "ok";
    case DMUON_ERR_INVALID_ARG: return "invalid argument";
    case DMUON_ERR_UNSUPPORTED: return "unsupported dtype or device";
    case DMUON_ERR_WORKSPACE: return "workspace missing or too small";
    case DMUON_ERR_ALIASING: return "buffers overlap";
    case DMUON_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* dmuon_last_error(void) { return g_last_error.c_str(); }

const char* dmuon_backend_info(void) {
  // built from the constants the planner and the launchers use
  static const std::string info = [] {
    std::ostringstream os;
    os << "{\"arch\": \"gfx950\", "
       << "\"ns_gemm_bf16\": {\"kernel\": \"gemm_bf16_kernel\", \"tiles\": [" << kTileBf16 << ", " << kTileBf16Big
       << "], \"waves\": 4, \"mfma\": {\"" << kTileBf16 << "\": \"v_mfma_f32_32x32x16_bf16\", \""
       << kTileBf16Big << "\": \"v_mfma_f32_16x16x32_bf16\"}, \"accumulate\": \"f32\", "
       << "\"stage_k\": 64, \"lds_stages\": 2, \"operand_loads\": \"buffer_load_dwordx4 to LDS\", "
       << "\"big_tile_rule\": {\"min_first_stage_tiles\": " << kBigTileMinCount
       << ", \"min_wide_share\": 0.5, \"wide_min_dim\": " << kBigTileMinDim
       << ", \"min_matrix_dim\": " << kTileBf16Big << "}, "
       << "\"products\": \"NT (K-contiguous operands); symmetric results as upper-triangle tiles "
          "stored with their mirror\"}, "
       << "\"ns_gemm_f32\": {\"kernel\": \"gemm_f32_kernel / gemm_f32_big_kernel\", \"tiles\": [" << kTileF32
       << ", " << kTileF32Big << "], \"waves\": 4, \"mfma\": \"v_mfma_f32_32x32x2f32\", \"stage_k\": 16, "
       << "\"big_tile_rule\": {\"min_first_stage_tiles\": " << kF32BigTileMinCount
       << ", \"min_matrix_dim\": " << kTileF32Big << "}}, "
       << "\"tile_override_env\": {\"bf16\": \"DMUON_GEMM_TILE\", \"f32\": \"DMUON_GEMM_TILE_F32\"}, "
       << "\"elementwise\": {\"tile\": " << kEwTile << ", \"threads\": " << kEwThreads
       << ", \"sum_of_squares\": \"wave shuffles, fp64 per-matrix finish\"}, "
       << "\"gram_rule\": {\"gram_form_when_n_at_least_m_times\": 2}}";
    return os.str();
  }();
  return info.c_str();
}

}  // extern "C"

// ---- two stream groups for small batches -------------------------------------

namespace dmuon {
namespace {

// A batch whose first NS stage has fewer than kSplitMaxTiles tiles of 256
// leaves most of the chip idle in every launch (fewer than three waves, and
// long-K tiles next to short ones); such a batch (bf16 products, two or more
// matrices) runs as two groups of matrices, balanced by their NS flops, each with its
// own launches, the second on a stream of the library's own that forks from
// and joins back into the caller's stream, provided the two groups' loads
// are within kSplitMaxImbalance of each other.  The launch tails of one
// group then overlap the other group's work.  Measured per step (50 queued
// steps): one 3B decoder layer 4.06 -> 3.66 ms (its best split is 1.25:1 in
// flops); two, four, eight and sixteen equal matrices 4-16 % faster; three
// and five equal matrices (2:1 and 3:2 splits) 7 % and 3 % slower, hence the
// balance condition; on larger batches two concurrent launch streams were
// 5-7 % slower, so they keep one.
constexpr int64_t kSplitMaxTiles = 768;
constexpr int kStreamGroups = 2;
constexpr double kSplitMaxImbalance = 1.4;    // heaviest group's NS flops over the lightest's

struct SplitPlan {
  std::vector<std::vector<int>> groups;          // positions in the active list
  std::vector<std::shared_ptr<Plan>> plans;
  std::vector<size_t> ws_off;
  size_t ws_bytes = 0;
};

// Flops of one matrix's NS products with K iterations, symmetric results
// counted once (the measure the stream groups balance): the standard form
// runs X X^T (m^2 n), B (m^3) and B X (2 m^2 n) per iteration; the Gram form
// R (m^2 n), 4K - 3 products of m x m matrices (m^3 each) and O (2 m^2 n).
double ns_cost(int64_t rows, int64_t cols, int32_t backend, int K) {
  const double m = double(std::min(rows, cols)), n = double(std::max(rows, cols));
  if (K == 0) return m * n;
  if (choose_form(backend, static_cast<int64_t>(m), static_cast<int64_t>(n)) == FORM_DIRECT)
    return K * (3.0 * m * m * n + m * m * m);
  return 3.0 * m * m * n + (4.0 * K - 3.0) * m * m * m;
}

// Groups of the active matrices (rows/cols in active order): one group, or
// two balanced ones when the batch is small.
std::vector<std::vector<int>> stream_groups(const std::vector<int64_t>& rows, const std::vector<int64_t>& cols,
                                            int32_t prec, int32_t backend, int K) {
  const int n = static_cast<int>(rows.size());
  std::vector<std::vector<int>> g(1);
  for (int i = 0; i < n; ++i) g[0].push_back(i);
  if (n < 2 || prec != DMUON_NS_PREC_BF16) return g;
  int64_t tiles = 0;
  for (int i = 0; i < n; ++i) {
    const int64_t t = (std::min(rows[i], cols[i]) + kTileBf16Big - 1) / kTileBf16Big;
    tiles += t * (t + 1) / 2;
  }
  if (tiles >= kSplitMaxTiles) return g;
  std::vector<int> order(n);
  for (int i = 0; i < n; ++i) order[i] = i;
  auto cost = [&](int i) { return ns_cost(rows[i], cols[i], backend, K); };
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return cost(a) > cost(b); });
  const int G = std::min(kStreamGroups, n);
  std::vector<std::vector<int>> gs(G);
  std::vector<double> load(G, 0.0);
  for (int i : order) {
    int k = 0;
    for (int j = 1; j < G; ++j)
      if (load[j] < load[k]) k = j;
    gs[k].push_back(i);
    load[k] += cost(i);
  }
  // an uneven split (three or five equal matrices) leaves one stream idle
  // for a large part of every stage and was measured slower than one stream
  const auto mm = std::minmax_element(load.begin(), load.end());
  if (*mm.second > kSplitMaxImbalance * *mm.first) return g;
  for (auto& v : gs) std::sort(v.begin(), v.end());
  return gs;
}

SplitPlan split_plan(const std::vector<int64_t>& rows, const std::vector<int64_t>& cols, int32_t prec,
                     int32_t backend, const Coeffs& cf) {
  SplitPlan S;
  S.groups = stream_groups(rows, cols, prec, backend, static_cast<int>(cf.abc.size() / 3));
  for (const auto& g : S.groups) {
    std::vector<int64_t> r, c;
    for (int i : g) { r.push_back(rows[i]); c.push_back(cols[i]); }
    S.plans.push_back(get_plan(r, c, prec, backend, cf, true));
    S.ws_off.push_back(S.ws_bytes);
    S.ws_bytes += align_up(S.plans.back()->ws_bytes);
  }
  return S;
}

// The library's own streams on each device (one per group after the first)
// and the events that fork them from, and join them back into, the caller's
// stream (a wait takes an event's latest record at the time of the call, so
// the same events serve every call).
struct SideStreams {
  hipStream_t stream[kStreamGroups - 1] = {};
  hipEvent_t fork = nullptr;
  hipEvent_t join[kStreamGroups - 1] = {};
};
std::mutex g_side_mu;
std::map<int, SideStreams> g_side;

int side_streams(SideStreams** out) {
  int dev = 0;
  DMUON_HIP_TRY(hipGetDevice(&dev));
  SideStreams& s = g_side[dev];
  if (!s.fork) {
    for (int k = 0; k < kStreamGroups - 1; ++k) {
      if (!s.stream[k]) DMUON_HIP_TRY(hipStreamCreateWithFlags(&s.stream[k], hipStreamNonBlocking));
      if (!s.join[k]) DMUON_HIP_TRY(hipEventCreateWithFlags(&s.join[k], hipEventDisableTiming));
    }
    DMUON_HIP_TRY(hipEventCreateWithFlags(&s.fork, hipEventDisableTiming));
  }
  *out = &s;
  return DMUON_OK;
}

// Runs run_group(g, stream) for every group: group 0 on the caller's stream,
// group g > 0 on the library's stream g - 1, between a fork and a join event.
template <class Run>
int run_groups(const SplitPlan& S, hipStream_t stream, Run run_group) {
  if (S.groups.size() == 1) return run_group(0, stream);
  std::lock_guard<std::mutex> lk(g_side_mu);
  SideStreams* side = nullptr;
  int st = side_streams(&side);
  if (st) return st;
  const int G = static_cast<int>(S.groups.size());
  DMUON_HIP_TRY(hipEventRecord(side->fork, stream));
  for (int g = 1; g < G; ++g) DMUON_HIP_TRY(hipStreamWaitEvent(side->stream[g - 1], side->fork, 0));
  st = run_group(0, stream);
  for (int g = 1; g < G && !st; ++g) st = run_group(g, side->stream[g - 1]);
  // the caller's stream waits for every group's stream whatever happened above
  hipError_t ej = hipSuccess;
  for (int g = 1; g < G; ++g) {
    hipError_t r = hipEventRecord(side->join[g - 1], side->stream[g - 1]);
    if (r == hipSuccess) r = hipStreamWaitEvent(stream, side->join[g - 1], 0);
    if (r != hipSuccess && ej == hipSuccess) ej = r;
  }
  if (st) return st;
  if (ej != hipSuccess) return fail(DMUON_ERR_HIP, std::string("stream join: ") + hipGetErrorString(ej));
  return DMUON_OK;
}

}  // namespace
}  // namespace dmuon

extern "C" {

// ---- dmuon_step ------------------------------------------------------------

static int step_prepare(const dmuon_matrix_t* mats, int32_t n, const dmuon_hparams_t* hp,
                        Coeffs* cf, std::vector<int>* active, SplitPlan* plan) {
  if (n < 0) return fail(DMUON_ERR_INVALID_ARG, "n < 0");
  if (n > 0 && !mats) return fail(DMUON_ERR_INVALID_ARG, "mats is NULL");
  int st = check_hparams(hp, true, cf);
  if (st) return st;
  std::vector<int64_t> rows, cols;
  for (int i = 0; i < n; ++i) {
    st = check_matrix_fields(mats[i], i, true);
    if (st) return st;
    if (!mats[i].param) return fail(DMUON_ERR_INVALID_ARG, mat_name("param", i) + " is NULL");
    if (!mats[i].grad) continue;
    active->push_back(i);
    rows.push_back(mats[i].rows);
    cols.push_back(mats[i].cols);
  }
  if (!active->empty()) *plan = split_plan(rows, cols, hp->ns_precision, hp->ns_backend, *cf);
  return DMUON_OK;
}

size_t dmuon_step_workspace_size(const dmuon_matrix_t* mats, int32_t n, const dmuon_hparams_t* hp) {
  Coeffs cf;
  std::vector<int> active;
  SplitPlan plan;
  if (step_prepare(mats, n, hp, &cf, &active, &plan) != DMUON_OK) return 0;
  return active.empty() ? 0 : plan.ws_bytes;
}

// One group of a step (the matrices active[g[j]]) with its plan, in its
// part of the workspace, on `stream`.
static int step_group(const dmuon_matrix_t* mats, const std::vector<int>& active, const std::vector<int>& grp,
                      const dmuon_hparams_t* hp, const double* const* grad_scale, const Plan& P, char* ws,
                      hipStream_t stream);

static int step_impl(const dmuon_matrix_t* mats, int32_t n, const dmuon_hparams_t* hp,
                     const double* const* grad_scale, void* workspace, size_t workspace_bytes, void* stream_) {
  g_last_error.clear();
  Coeffs cf;
  std::vector<int> active;
  SplitPlan S;
  int st = step_prepare(mats, n, hp, &cf, &active, &S);
  if (st) return st;
  if (active.empty()) return DMUON_OK;
  if (!workspace || workspace_bytes < S.ws_bytes) {
    char buf[128];
    std::snprintf(buf, sizeof buf, "workspace needs %zu bytes, got %zu", S.ws_bytes, workspace_bytes);
    return fail(DMUON_ERR_WORKSPACE, buf);
  }
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(DMUON_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  std::vector<Range> ranges;
  for (int i : active) {
    const dmuon_matrix_t& m = mats[i];
    const size_t ne = size_t(m.rows) * m.cols;
    auto add = [&](const void* p, size_t bytes, const char* what) {
      const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
      ranges.push_back({lo, lo + bytes, mat_name(what, i)});
    };
    add(m.param, ne * dtype_size(m.param_dtype), "param");
    add(m.grad, ne * dtype_size(m.grad_dtype), "grad");
    add(m.momentum, ne * 4, "momentum");
  }
  ranges.push_back({reinterpret_cast<uintptr_t>(workspace),
                    reinterpret_cast<uintptr_t>(workspace) + S.ws_bytes, "workspace"});
  st = check_overlaps(ranges);
  if (st) return st;
  st = check_device();
  if (st) return st;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  return run_groups(S, stream, [&](size_t g, hipStream_t s) {
    return step_group(mats, active, S.groups[g], hp, grad_scale, *S.plans[g],
                      static_cast<char*>(workspace) + S.ws_off[g], s);
  });
}

static int step_group(const dmuon_matrix_t* mats, const std::vector<int>& active_all, const std::vector<int>& grp,
                      const dmuon_hparams_t* hp, const double* const* grad_scale, const Plan& P, char* ws,
                      hipStream_t stream) {
  std::vector<int> active(grp.size());
  for (size_t j = 0; j < grp.size(); ++j) active[j] = active_all[grp[j]];
  int st = DMUON_OK;
  const int32_t wide_dt = hp->ns_precision == DMUON_NS_PREC_BF16 ? DT_BF16 : DT_F32;
  const float decay = static_cast<float>(1.0 - hp->lr * hp->weight_decay);
  // with bf16 products and bf16 parameters the last product of each matrix
  // updates the parameter itself (no O in the workspace, no separate update
  // pass); a batch with any fp32 parameter takes the update pass
  bool fuse_update = P.prec == DMUON_NS_PREC_BF16 && P.ns_steps > 0;
  for (int j = 0; j < P.n && fuse_update; ++j) fuse_update = mats[active[j]].param_dtype == DT_BF16;
  std::vector<FusedUpdate> fused(fuse_update ? P.n : 0);
  for (size_t j = 0; j < fused.size(); ++j) {
    const dmuon_matrix_t& m = mats[active[j]];
    fused[j] = {m.param, m.param_dtype, lr_eff_of(hp->lr, m.rows, m.cols), decay};
  }
  KeyBuf key;
  key.put_str("step").put_str(P.key).put(hp->lr).put(hp->weight_decay);
  for (int j = 0; j < P.n; ++j) {
    key.put(mats[active[j]]);
    key.put(grad_scale ? grad_scale[active[j]] : nullptr);
  }
  st = stage_table(ws, P.table_bytes, stream, key.s, [&](char* host) {
    EwMat* em = reinterpret_cast<EwMat*>(host + P.off_ewmats);
    for (int j = 0; j < P.n; ++j) {
      const dmuon_matrix_t& m = mats[active[j]];
      const MatLayout& L = P.mats[j];
      EwMat& e = em[j];
      e.rows = m.rows; e.cols = m.cols;
      e.src = m.grad; e.mom = m.momentum; e.param = m.param;
      e.u_dst = ws + L.x0; e.o_src = ws + L.out;
      e.u_dst_t = L.x0t != kNone ? ws + L.x0t : nullptr; e.ld_wide_t = L.pm;
      e.ld_wide = L.pn; e.wide_rows = static_cast<int32_t>(L.mp); e.wide_cols = static_cast<int32_t>(L.np);
      e.tall = L.tall; e.src_dtype = m.grad_dtype; e.wide_dtype = wide_dt; e.param_dtype = m.param_dtype;
      e.scale_idx = P.ns_steps == 0 ? j : -1;
      e.aligned = (m.cols % 4 == 0) && aligned16(m.grad) && aligned16(m.momentum) && aligned16(m.param);
      e.user_index = j;
      e.blk_wide = P.blk_wide[j]; e.blk_stored = P.blk_stored[j];
      e.lr_eff = lr_eff_of(hp->lr, m.rows, m.cols);
      e.decay = decay;
      e.gscale = grad_scale ? grad_scale[active[j]] : nullptr;
    }
    fill_tasks(P, ws, reinterpret_cast<GemmTask*>(host + P.off_tasks), fuse_update ? fused.data() : nullptr);
  });
  if (st) return st;
  const EwMat* em_dev = reinterpret_cast<const EwMat*>(ws + P.off_ewmats);
  float* partials = reinterpret_cast<float*>(ws + P.off_partials);
  float* scale = reinterpret_cast<float*>(ws + P.off_scale);
  double* sumsq = reinterpret_cast<double*>(ws + P.off_sumsq);
  int64_t mom_bytes = 0, upd_bytes = 0;
  for (int j = 0; j < P.n; ++j) {
    const dmuon_matrix_t& m = mats[active[j]];
    const int64_t ne = m.rows * m.cols;
    // gradient in, momentum in and out, the NS input out (twice when its
    // transpose is kept as well)
    const int64_t outs = P.mats[j].x0t != kNone ? 2 : 1;
    mom_bytes += ne * (int64_t(dtype_size(m.grad_dtype)) + 8 + outs * int64_t(dtype_size(wide_dt)));
    upd_bytes += ne * (2 * int64_t(dtype_size(m.param_dtype)) + int64_t(dtype_size(wide_dt)));
  }
  DMUON_HIP_TRY(prof_launch(PK_MOMENTUM, 0, mom_bytes, stream, [&] {
    return launch_momentum(em_dev, P.n, P.blocks_wide, 0, static_cast<float>(hp->momentum),
                           hp->nesterov ? 1 : 0, partials, stream);
  }));
  DMUON_HIP_TRY(prof_launch(PK_FINALIZE, 0, P.blocks_wide * 4, stream, [&] {
    return launch_finalize(em_dev, P.n, P.blocks_wide, partials, sumsq, scale, hp->eps, stream);
  }));
  st = run_gemms(P, ws, stream);
  if (st) return st;
  if (fuse_update) return DMUON_OK;
  DMUON_HIP_TRY(prof_launch(PK_UPDATE, 0, upd_bytes, stream, [&] {
    return launch_update(em_dev, P.n, P.blocks_stored, 0, scale, stream);
  }));
  return DMUON_OK;
}

int dmuon_step(const dmuon_matrix_t* mats, int32_t n, const dmuon_hparams_t* hp, void* workspace,
               size_t workspace_bytes, void* stream) {
  return step_impl(mats, n, hp, nullptr, workspace, workspace_bytes, stream);
}

int dmuon_step_scaled(const dmuon_matrix_t* mats, int32_t n, const dmuon_hparams_t* hp,
                      const double* const* grad_scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (n > 0 && !grad_scale) {
    g_last_error = "grad_scale is NULL";
    return DMUON_ERR_INVALID_ARG;
  }
  return step_impl(mats, n, hp, grad_scale, workspace, workspace_bytes, stream);
}

// ---- dmuon_momentum --------------------------------------------------------

size_t dmuon_momentum_workspace_size(const dmuon_matrix_t* mats, int32_t n) {
  if (n <= 0 || !mats) return 0;
  std::vector<int64_t> rows, cols;
  for (int i = 0; i < n; ++i)
    if (mats[i].grad && mats[i].rows > 0 && mats[i].cols > 0) {
      rows.push_back(mats[i].rows);
      cols.push_back(mats[i].cols);
    }
  if (rows.empty()) return 0;
  Coeffs cf;
  auto P = get_plan(rows, cols, DMUON_NS_PREC_F32, 0, cf, false);
  return P->off_sumsq;  // tables and partials only
}

int dmuon_momentum(const dmuon_matrix_t* mats, int32_t n, const dmuon_hparams_t* hp,
                   void* const* ns_input, int32_t ns_input_dtype, double* sumsq, void* workspace,
                   size_t workspace_bytes, void* stream_) {
  g_last_error.clear();
  if (n < 0) return fail(DMUON_ERR_INVALID_ARG, "n < 0");
  if (n > 0 && (!mats || !ns_input || !sumsq)) return fail(DMUON_ERR_INVALID_ARG, "mats, ns_input or sumsq is NULL");
  if (!hp) return fail(DMUON_ERR_INVALID_ARG, "hparams is NULL");
  if (!std::isfinite(hp->momentum)) return fail(DMUON_ERR_INVALID_ARG, "momentum must be finite");
  if (!dtype_ok(ns_input_dtype)) return fail(DMUON_ERR_UNSUPPORTED, "ns_input_dtype must be F32 or BF16");
  std::vector<int> active;
  std::vector<int64_t> rows, cols;
  for (int i = 0; i < n; ++i) {
    int st = check_matrix_fields(mats[i], i, true);
    if (st) return st;
    if (!mats[i].grad) continue;
    if (!ns_input[i]) return fail(DMUON_ERR_INVALID_ARG, mat_name("ns_input", i) + " is NULL");
    active.push_back(i);
    rows.push_back(mats[i].rows);
    cols.push_back(mats[i].cols);
  }
  if (active.empty()) return DMUON_OK;
  Coeffs cf;
  auto plan = get_plan(rows, cols, DMUON_NS_PREC_F32, 0, cf, false);
  const Plan& P = *plan;
  const size_t need = P.off_sumsq;
  if (!workspace || workspace_bytes < need) return fail(DMUON_ERR_WORKSPACE, "workspace too small");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(DMUON_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  std::vector<Range> ranges;
  for (int i : active) {
    const dmuon_matrix_t& m = mats[i];
    const size_t ne = size_t(m.rows) * m.cols;
    auto add = [&](const void* p, size_t bytes, const char* what) {
      const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
      ranges.push_back({lo, lo + bytes, mat_name(what, i)});
    };
    add(m.grad, ne * dtype_size(m.grad_dtype), "grad");
    add(m.momentum, ne * 4, "momentum");
    add(ns_input[i], ne * dtype_size(ns_input_dtype), "ns_input");
  }
  ranges.push_back({reinterpret_cast<uintptr_t>(sumsq), reinterpret_cast<uintptr_t>(sumsq) + 8 * size_t(n), "sumsq"});
  ranges.push_back({reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + need, "workspace"});
  int st = check_overlaps(ranges);
  if (st) return st;
  st = check_device();
  if (st) return st;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  char* ws = static_cast<char*>(workspace);
  KeyBuf key;
  key.put_str("momentum").put_str(P.key).put(ns_input_dtype);
  for (int j = 0; j < P.n; ++j) key.put(mats[active[j]]).put(ns_input[active[j]]).put(active[j]);
  st = stage_table(ws, P.off_ewmats + sizeof(EwMat) * P.n, stream, key.s, [&](char* host) {
    EwMat* em = reinterpret_cast<EwMat*>(host + P.off_ewmats);
    for (int j = 0; j < P.n; ++j) {
      const dmuon_matrix_t& m = mats[active[j]];
      const MatLayout& L = P.mats[j];
      EwMat& e = em[j];
      e.rows = m.rows; e.cols = m.cols;
      e.src = m.grad; e.mom = m.momentum; e.param = nullptr;
      e.u_dst = ns_input[active[j]]; e.o_src = nullptr;
      e.u_dst_t = nullptr; e.ld_wide_t = 0;
      e.ld_wide = L.n; e.wide_rows = static_cast<int32_t>(L.m); e.wide_cols = static_cast<int32_t>(L.n);
      e.tall = L.tall; e.src_dtype = m.grad_dtype; e.wide_dtype = ns_input_dtype; e.param_dtype = m.param_dtype;
      e.scale_idx = -1;
      e.aligned = (m.cols % 4 == 0) && aligned16(m.grad) && aligned16(m.momentum);
      e.user_index = active[j];
      e.blk_wide = P.blk_wide[j]; e.blk_stored = P.blk_stored[j];
      e.lr_eff = 0.f; e.decay = 1.f;
    }
  });
  if (st) return st;
  const EwMat* em_dev = reinterpret_cast<const EwMat*>(ws + P.off_ewmats);
  float* partials = reinterpret_cast<float*>(ws + P.off_partials);
  DMUON_HIP_TRY(launch_momentum(em_dev, P.n, P.blocks_wide, 0, static_cast<float>(hp->momentum),
                                hp->nesterov ? 1 : 0, partials, stream));
  DMUON_HIP_TRY(launch_finalize(em_dev, P.n, P.blocks_wide, partials, sumsq, nullptr, 0.0, stream));
  return DMUON_OK;
}

// ---- dmuon_orthogonalize -----------------------------------------------------

static int ortho_prepare(const int64_t* rows, const int64_t* cols, int32_t n, const dmuon_hparams_t* hp,
                         Coeffs* cf, std::shared_ptr<Plan>* plan) {
  if (n < 0) return fail(DMUON_ERR_INVALID_ARG, "n < 0");
  if (n > 0 && (!rows || !cols)) return fail(DMUON_ERR_INVALID_ARG, "rows or cols is NULL");
  int st = check_hparams(hp, false, cf);
  if (st) return st;
  for (int i = 0; i < n; ++i)
    if (rows[i] <= 0 || cols[i] <= 0 || rows[i] > kMaxDim || cols[i] > kMaxDim)
      return fail(DMUON_ERR_INVALID_ARG, "matrix " + std::to_string(i) + ": bad shape");
  if (n == 0) return DMUON_OK;
  *plan = get_plan(std::vector<int64_t>(rows, rows + n), std::vector<int64_t>(cols, cols + n),
                   hp->ns_precision, hp->ns_backend, *cf, true);
  return DMUON_OK;
}

// The split plan of an orthogonalize call (the same grouping as dmuon_step).
static int ortho_split(const int64_t* rows, const int64_t* cols, int32_t n, const dmuon_hparams_t* hp,
                       Coeffs* cf, SplitPlan* S) {
  std::shared_ptr<Plan> unused;
  int st = ortho_prepare(rows, cols, n, hp, cf, &unused);
  if (st || n == 0) return st;
  *S = split_plan(std::vector<int64_t>(rows, rows + n), std::vector<int64_t>(cols, cols + n), hp->ns_precision,
                  hp->ns_backend, *cf);
  return DMUON_OK;
}

size_t dmuon_orthogonalize_workspace_size(const int64_t* rows, const int64_t* cols, int32_t n,
                                          const dmuon_hparams_t* hp) {
  Coeffs cf;
  SplitPlan S;
  if (ortho_split(rows, cols, n, hp, &cf, &S) != DMUON_OK || n == 0) return 0;
  return S.ws_bytes;
}

int dmuon_orthogonalize(const void* const* in, void* const* out, const int64_t* rows, const int64_t* cols,
                        int32_t n, int32_t io_dtype, const dmuon_hparams_t* hp, void* workspace,
                        size_t workspace_bytes, void* stream_) {
  g_last_error.clear();
  Coeffs cf;
  SplitPlan S;
  int st = ortho_split(rows, cols, n, hp, &cf, &S);
  if (st) return st;
  if (n == 0) return DMUON_OK;
  if (!in || !out) return fail(DMUON_ERR_INVALID_ARG, "in or out is NULL");
  if (!dtype_ok(io_dtype)) return fail(DMUON_ERR_UNSUPPORTED, "io_dtype must be F32 or BF16");
  if (!workspace || workspace_bytes < S.ws_bytes) {
    char buf[128];
    std::snprintf(buf, sizeof buf, "workspace needs %zu bytes, got %zu", S.ws_bytes, workspace_bytes);
    return fail(DMUON_ERR_WORKSPACE, buf);
  }
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(DMUON_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  std::vector<Range> outs, ins;
  const uintptr_t wlo = reinterpret_cast<uintptr_t>(workspace);
  for (int i = 0; i < n; ++i) {
    if (!in[i] || !out[i]) return fail(DMUON_ERR_INVALID_ARG, "in[" + std::to_string(i) + "] or out is NULL");
    const size_t bytes = size_t(rows[i]) * cols[i] * dtype_size(io_dtype);
    const uintptr_t o = reinterpret_cast<uintptr_t>(out[i]), s = reinterpret_cast<uintptr_t>(in[i]);
    outs.push_back({o, o + bytes, mat_name("out", i)});
    ins.push_back({s, s + bytes, mat_name("in", i)});
  }
  {
    std::vector<Range> r = outs;
    r.push_back({wlo, wlo + S.ws_bytes, "workspace"});
    st = check_overlaps(r);
    if (st) return st;
    for (int i = 0; i < n; ++i) {
      if (ins[i].lo < wlo + S.ws_bytes && wlo < ins[i].hi) return fail(DMUON_ERR_ALIASING, ins[i].what + " overlaps workspace");
      for (int j = 0; j < n; ++j) {
        if (i == j) {
          if (ins[i].lo != outs[i].lo && ins[i].lo < outs[i].hi && outs[i].lo < ins[i].hi)
            return fail(DMUON_ERR_ALIASING, ins[i].what + " partially overlaps " + outs[i].what);
        } else if (ins[i].lo < outs[j].hi && outs[j].lo < ins[i].hi) {
          return fail(DMUON_ERR_ALIASING, ins[i].what + " overlaps " + outs[j].what);
        }
      }
    }
  }
  st = check_device();
  if (st) return st;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const int32_t wide_dt = hp->ns_precision == DMUON_NS_PREC_BF16 ? DT_BF16 : DT_F32;
  return run_groups(S, stream, [&](size_t g, hipStream_t gs) -> int {
    const Plan& P = *S.plans[g];
    const std::vector<int>& grp = S.groups[g];
    char* ws = static_cast<char*>(workspace) + S.ws_off[g];
    KeyBuf key;
    key.put_str("orthogonalize").put_str(P.key).put(io_dtype);
    for (int j = 0; j < P.n; ++j) key.put(in[grp[j]]).put(out[grp[j]]);
    int rc = stage_table(ws, P.table_bytes, gs, key.s, [&](char* host) {
      EwMat* em = reinterpret_cast<EwMat*>(host + P.off_ewmats);
      for (int j = 0; j < P.n; ++j) {
        const int i = grp[j];
        const MatLayout& L = P.mats[j];
        EwMat& e = em[j];
        e.rows = rows[i]; e.cols = cols[i];
        e.src = in[i]; e.mom = nullptr; e.param = out[i];
        e.u_dst = ws + L.x0; e.o_src = ws + L.out;
        e.u_dst_t = L.x0t != kNone ? ws + L.x0t : nullptr; e.ld_wide_t = L.pm;
        e.ld_wide = L.pn; e.wide_rows = static_cast<int32_t>(L.mp); e.wide_cols = static_cast<int32_t>(L.np);
        e.tall = L.tall; e.src_dtype = io_dtype; e.wide_dtype = wide_dt; e.param_dtype = io_dtype;
        e.scale_idx = P.ns_steps == 0 ? j : -1;
        e.aligned = (cols[i] % 4 == 0) && aligned16(in[i]) && aligned16(out[i]);
        e.user_index = j;
        e.blk_wide = P.blk_wide[j]; e.blk_stored = P.blk_stored[j];
        e.lr_eff = 0.f; e.decay = 1.f;
      }
      fill_tasks(P, ws, reinterpret_cast<GemmTask*>(host + P.off_tasks));
    });
    if (rc) return rc;
    const EwMat* em_dev = reinterpret_cast<const EwMat*>(ws + P.off_ewmats);
    float* partials = reinterpret_cast<float*>(ws + P.off_partials);
    float* scale = reinterpret_cast<float*>(ws + P.off_scale);
    double* sumsq = reinterpret_cast<double*>(ws + P.off_sumsq);
    DMUON_HIP_TRY(launch_momentum(em_dev, P.n, P.blocks_wide, 1, 0.f, 0, partials, gs));
    DMUON_HIP_TRY(launch_finalize(em_dev, P.n, P.blocks_wide, partials, sumsq, scale, hp->eps, gs));
    rc = run_gemms(P, ws, gs);
    if (rc) return rc;
    DMUON_HIP_TRY(launch_update(em_dev, P.n, P.blocks_stored, 1, scale, gs));
    return DMUON_OK;
  });
}

// ---- dmuon_orthogonalize_sharded ----------------------------------------------

static int sharded_prepare(const dmuon_sharded_t* mats, int32_t n, const dmuon_hparams_t* hp, Coeffs* cf,
                           std::shared_ptr<Plan>* plan) {
  if (n < 0) return fail(DMUON_ERR_INVALID_ARG, "n < 0");
  if (n > 0 && !mats) return fail(DMUON_ERR_INVALID_ARG, "mats is NULL");
  int st = check_hparams(hp, false, cf);
  if (st) return st;
  std::vector<ShapeSpec> shapes;
  std::vector<Group> groups;
  for (int i = 0; i < n; ++i) {
    const dmuon_sharded_t& M = mats[i];
    const std::string name = mat_name("mats", i);
    if (M.nshards < 1) return fail(DMUON_ERR_INVALID_ARG, name + ".nshards must be >= 1");
    if (M.split != 0 && M.split != 1) return fail(DMUON_ERR_INVALID_ARG, name + ".split must be 0 or 1");
    if (!M.shards) return fail(DMUON_ERR_INVALID_ARG, name + ".shards is NULL");
    if (shapes.size() + size_t(M.nshards) > size_t(1) << 30)
      return fail(DMUON_ERR_INVALID_ARG, "too many shards");
    groups.push_back({static_cast<int>(shapes.size()), M.nshards, 0, 0, FORM_DIRECT});
    int64_t d = -1;
    for (int s = 0; s < M.nshards; ++s) {
      const dmuon_shard_t& S = M.shards[s];
      if (S.rows <= 0 || S.cols <= 0 || S.rows > kMaxDim || S.cols > kMaxDim)
        return fail(DMUON_ERR_INVALID_ARG, name + ".shards[" + std::to_string(s) + "]: bad shape");
      const int64_t dd = M.split == 1 ? S.rows : S.cols;
      if (d >= 0 && dd != d)
        return fail(DMUON_ERR_INVALID_ARG, name + ".shards[" + std::to_string(s) +
                                               "]: the unsplit dimension differs from shard 0's");
      d = dd;
      shapes.push_back({S.rows, S.cols, M.split == 0});
    }
  }
  if (n == 0) return DMUON_OK;
  *plan = get_plan(shapes, groups, hp->ns_precision, hp->ns_backend, *cf, true);
  return DMUON_OK;
}

size_t dmuon_orthogonalize_sharded_workspace_size(const dmuon_sharded_t* mats, int32_t n,
                                                  const dmuon_hparams_t* hp) {
  Coeffs cf;
  std::shared_ptr<Plan> plan;
  if (sharded_prepare(mats, n, hp, &cf, &plan) != DMUON_OK || n == 0) return 0;
  return plan->ws_bytes;
}

int dmuon_orthogonalize_sharded(const dmuon_sharded_t* mats, int32_t n, int32_t io_dtype,
                                const dmuon_hparams_t* hp, void* workspace, size_t workspace_bytes,
                                void* stream_) {
  g_last_error.clear();
  Coeffs cf;
  std::shared_ptr<Plan> plan;
  int st = sharded_prepare(mats, n, hp, &cf, &plan);
  if (st) return st;
  if (n == 0) return DMUON_OK;
  if (!dtype_ok(io_dtype)) return fail(DMUON_ERR_UNSUPPORTED, "io_dtype must be F32 or BF16");
  const Plan& P = *plan;
  if (!workspace || workspace_bytes < P.ws_bytes) {
    char buf[128];
    std::snprintf(buf, sizeof buf, "workspace needs %zu bytes, got %zu", P.ws_bytes, workspace_bytes);
    return fail(DMUON_ERR_WORKSPACE, buf);
  }
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(DMUON_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  // the shards in plan order, with the index of their matrix
  std::vector<const dmuon_shard_t*> sh;
  std::vector<int> owner;
  for (int i = 0; i < n; ++i)
    for (int s = 0; s < mats[i].nshards; ++s) {
      sh.push_back(&mats[i].shards[s]);
      owner.push_back(i);
    }
  std::vector<Range> outs, ins;
  const uintptr_t wlo = reinterpret_cast<uintptr_t>(workspace);
  for (size_t j = 0; j < sh.size(); ++j) {
    const std::string name = mat_name("mats", owner[j]) + ".shards[" +
                             std::to_string(j - size_t(P.groups[owner[j]].first)) + "]";
    if (!sh[j]->in || !sh[j]->out) return fail(DMUON_ERR_INVALID_ARG, name + ": in or out is NULL");
    const size_t bytes = size_t(sh[j]->rows) * sh[j]->cols * dtype_size(io_dtype);
    const uintptr_t o = reinterpret_cast<uintptr_t>(sh[j]->out), i = reinterpret_cast<uintptr_t>(sh[j]->in);
    outs.push_back({o, o + bytes, name + ".out"});
    ins.push_back({i, i + bytes, name + ".in"});
  }
  {
    std::vector<Range> r = outs;
    r.push_back({wlo, wlo + P.ws_bytes, "workspace"});
    st = check_overlaps(r);
    if (st) return st;
    for (size_t i = 0; i < ins.size(); ++i) {
      if (ins[i].lo < wlo + P.ws_bytes && wlo < ins[i].hi) return fail(DMUON_ERR_ALIASING, ins[i].what + " overlaps workspace");
      for (size_t j = 0; j < outs.size(); ++j) {
        if (i == j) {
          if (ins[i].lo != outs[i].lo && ins[i].lo < outs[i].hi && outs[i].lo < ins[i].hi)
            return fail(DMUON_ERR_ALIASING, ins[i].what + " partially overlaps " + outs[i].what);
        } else if (ins[i].lo < outs[j].hi && outs[j].lo < ins[i].hi) {
          return fail(DMUON_ERR_ALIASING, ins[i].what + " overlaps " + outs[j].what);
        }
      }
    }
  }
  st = check_device();
  if (st) return st;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  char* ws = static_cast<char*>(workspace);
  const int32_t wide_dt = hp->ns_precision == DMUON_NS_PREC_BF16 ? DT_BF16 : DT_F32;
  KeyBuf key;
  key.put_str("sharded").put_str(P.key).put(io_dtype);
  for (size_t j = 0; j < sh.size(); ++j) key.put(*sh[j]).put(owner[j]);
  st = stage_table(ws, P.table_bytes, stream, key.s, [&](char* host) {
    EwMat* em = reinterpret_cast<EwMat*>(host + P.off_ewmats);
    for (int j = 0; j < P.n; ++j) {
      const MatLayout& L = P.mats[j];
      const dmuon_shard_t& S = *sh[j];
      const Group& g = P.groups[owner[j]];
      EwMat& e = em[j];
      e.rows = S.rows; e.cols = S.cols;
      e.src = S.in; e.mom = nullptr; e.param = S.out;
      e.u_dst = ws + L.x0; e.o_src = ws + L.out;
      e.u_dst_t = L.x0t != kNone ? ws + L.x0t : nullptr; e.ld_wide_t = L.pm;
      e.ld_wide = L.pn; e.wide_rows = static_cast<int32_t>(L.mp); e.wide_cols = static_cast<int32_t>(L.np);
      e.tall = L.tall; e.src_dtype = io_dtype; e.wide_dtype = wide_dt; e.param_dtype = io_dtype;
      e.scale_idx = P.ns_steps == 0 ? j : -1;
      e.aligned = (S.cols % 4 == 0) && aligned16(S.in) && aligned16(S.out);
      e.user_index = owner[j];
      e.grp_first = g.first; e.grp_count = g.count;
      e.blk_wide = P.blk_wide[j]; e.blk_stored = P.blk_stored[j];
      e.lr_eff = 0.f; e.decay = 1.f;
    }
    fill_tasks(P, ws, reinterpret_cast<GemmTask*>(host + P.off_tasks));
  });
  if (st) return st;
  const EwMat* em_dev = reinterpret_cast<const EwMat*>(ws + P.off_ewmats);
  float* partials = reinterpret_cast<float*>(ws + P.off_partials);
  float* scale = reinterpret_cast<float*>(ws + P.off_scale);
  double* sumsq = reinterpret_cast<double*>(ws + P.off_sumsq);
  int64_t load_bytes = 0, store_bytes = 0;
  for (int j = 0; j < P.n; ++j) {
    const int64_t ne = sh[j]->rows * sh[j]->cols;
    const int64_t outs_n = P.mats[j].x0t != kNone ? 2 : 1;
    load_bytes += ne * (int64_t(dtype_size(io_dtype)) + outs_n * int64_t(dtype_size(wide_dt)));
    store_bytes += ne * (int64_t(dtype_size(io_dtype)) + int64_t(dtype_size(wide_dt)));
  }
  DMUON_HIP_TRY(prof_launch(PK_MOMENTUM, 0, load_bytes, stream, [&] {
    return launch_momentum(em_dev, P.n, P.blocks_wide, 1, 0.f, 0, partials, stream);
  }));
  DMUON_HIP_TRY(prof_launch(PK_FINALIZE, 0, P.blocks_wide * 4, stream, [&] {
    return launch_finalize(em_dev, P.n, P.blocks_wide, partials, sumsq, scale, hp->eps, stream);
  }));
  st = run_gemms(P, ws, stream);
  if (st) return st;
  DMUON_HIP_TRY(prof_launch(PK_UPDATE, 0, store_bytes, stream, [&] {
    return launch_update(em_dev, P.n, P.blocks_stored, 1, scale, stream);
  }));
  return DMUON_OK;
}

// ---- dmuon_apply_update -----------------------------------------------------

// ---------------------------------------------------------------------------
// gradient clipping
// ---------------------------------------------------------------------------

namespace {
struct ClipLayout {
  size_t off_items, off_bucket_blocks, off_max_norm, off_partials, off_coefs, total;
  int64_t blocks;
};

ClipLayout clip_layout(const dmuon_grad_t* grads, int32_t n, int32_t nbuckets) {
  ClipLayout L{};
  L.blocks = 0;
  for (int i = 0; i < n; ++i) {
    const int64_t bytes = grads[i].numel * int64_t(dtype_size(grads[i].dtype));
    L.blocks += (bytes + kClipChunkBytes - 1) / kClipChunkBytes;
  }
  size_t cur = 0;
  L.off_items = cur; cur = align_up(cur + sizeof(ClipItem) * size_t(n));
  L.off_bucket_blocks = cur; cur = align_up(cur + sizeof(int64_t) * size_t(nbuckets + 1));
  L.off_max_norm = cur; cur = align_up(cur + sizeof(double) * size_t(nbuckets));
  L.off_partials = cur; cur = align_up(cur + sizeof(double) * size_t(L.blocks));
  L.off_coefs = cur; cur = align_up(cur + sizeof(double) * size_t(nbuckets));
  L.total = cur;
  return L;
}
}  // namespace

size_t dmuon_clip_workspace_size(const dmuon_grad_t* grads, int32_t n, int32_t nbuckets) {
  if (n <= 0 || nbuckets <= 0 || !grads) return 0;
  for (int i = 0; i < n; ++i)
    if (grads[i].numel <= 0 || !dtype_ok(grads[i].dtype)) return 0;
  return clip_layout(grads, n, nbuckets).total;
}

// noalloc: the workspace is the library's scratch array (dmuon_clip_grad_norm_noalloc);
// then the table goes up as kernel arguments and no event is created.
static int clip_impl(const dmuon_grad_t* grads, int32_t n, int32_t nbuckets, const double* max_norm,
                     double norm_type, double* total_norm, double* coef_out, void* workspace,
                     size_t workspace_bytes, void* stream_, bool noalloc = false,
                     int (*scratch_of_device)(void**) = nullptr) {
  g_last_error.clear();
  if (n < 0) return fail(DMUON_ERR_INVALID_ARG, "n < 0");
  if (nbuckets <= 0) return fail(DMUON_ERR_INVALID_ARG, "nbuckets must be >= 1");
  if (n > 0 && !grads) return fail(DMUON_ERR_INVALID_ARG, "grads is NULL");
  if (!max_norm) return fail(DMUON_ERR_INVALID_ARG, "max_norm is NULL");
  if (!(norm_type > 0.0)) return fail(DMUON_ERR_INVALID_ARG, "norm_type must be > 0 (or +inf)");
  for (int b = 0; b < nbuckets; ++b)
    if (!std::isfinite(max_norm[b]) || max_norm[b] < 0.0)
      return fail(DMUON_ERR_INVALID_ARG, "max_norm[" + std::to_string(b) + "] must be finite and >= 0");
  std::vector<Range> ranges;
  for (int i = 0; i < n; ++i) {
    const dmuon_grad_t& g = grads[i];
    if (!g.grad) return fail(DMUON_ERR_INVALID_ARG, mat_name("grads", i) + ".grad is NULL");
    if (g.numel <= 0) return fail(DMUON_ERR_INVALID_ARG, mat_name("grads", i) + ".numel must be > 0");
    if (!dtype_ok(g.dtype)) return fail(DMUON_ERR_UNSUPPORTED, mat_name("grads", i) + ".dtype must be F32 or BF16");
    if (g.bucket < 0 || g.bucket >= nbuckets)
      return fail(DMUON_ERR_INVALID_ARG, mat_name("grads", i) + ".bucket out of range");
    const uintptr_t p = reinterpret_cast<uintptr_t>(g.grad);
    ranges.push_back({p, p + size_t(g.numel) * dtype_size(g.dtype), mat_name("grads", i)});
  }
  if (n == 0) return DMUON_OK;
  const ClipLayout L = clip_layout(grads, n, nbuckets);
  if (noalloc && L.total > workspace_bytes) {
    char buf[192];
    std::snprintf(buf, sizeof buf,
                  "these gradients need %zu bytes of clip scratch; the allocation-free entry point holds %zu",
                  L.total, workspace_bytes);
    return fail(DMUON_ERR_WORKSPACE, buf);
  }
  if (noalloc) {
    // every host-side check has passed: now the current device's scratch
    const int sst = scratch_of_device(&workspace);
    if (sst != DMUON_OK) return sst;
  }
  if (!workspace || workspace_bytes < L.total) return fail(DMUON_ERR_WORKSPACE, "workspace too small");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(DMUON_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  ranges.push_back({reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + L.total,
                    "workspace"});
  if (total_norm)
    ranges.push_back({reinterpret_cast<uintptr_t>(total_norm),
                      reinterpret_cast<uintptr_t>(total_norm) + sizeof(double) * size_t(nbuckets), "total_norm"});
  if (coef_out)
    ranges.push_back({reinterpret_cast<uintptr_t>(coef_out),
                      reinterpret_cast<uintptr_t>(coef_out) + sizeof(double) * size_t(nbuckets), "coef_out"});
  int st = check_overlaps(ranges);
  if (st) return st;
  st = check_device();
  if (st) return st;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  char* ws = static_cast<char*>(workspace);
  // gradients ordered by bucket (stable), so each bucket's blocks are contiguous
  std::vector<int> order(n);
  for (int i = 0; i < n; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return grads[a].bucket < grads[b].bucket; });
  auto fill = [&](char* host) {
    ClipItem* items = reinterpret_cast<ClipItem*>(host + L.off_items);
    int64_t* bb = reinterpret_cast<int64_t*>(host + L.off_bucket_blocks);
    double* mx = reinterpret_cast<double*>(host + L.off_max_norm);
    int64_t blk = 0;
    int k = 0;
    for (int b = 0; b <= nbuckets; ++b) {
      while (k < n && grads[order[k]].bucket < b) {
        const dmuon_grad_t& g = grads[order[k]];
        ClipItem& it = items[k];
        it.grad = g.grad; it.numel = g.numel; it.blk_first = blk; it.dtype = g.dtype; it.bucket = g.bucket;
        it.aligned = aligned16(g.grad);
        blk += (g.numel * int64_t(dtype_size(g.dtype)) + kClipChunkBytes - 1) / kClipChunkBytes;
        ++k;
      }
      bb[b] = blk;
    }
    for (int b = 0; b < nbuckets; ++b) mx[b] = max_norm[b];
  };
  const ClipItem* items_dev = reinterpret_cast<const ClipItem*>(ws + L.off_items);
  double* partials = reinterpret_cast<double*>(ws + L.off_partials);
  double* coefs = coef_out ? coef_out : reinterpret_cast<double*>(ws + L.off_coefs);
  if (noalloc) {
    // the table is written in full here: nothing in the scratch has to
    // start at zero (every partial and coefficient is written by a kernel)
    thread_local std::vector<char> host;
    if (host.size() < L.off_partials) host.resize(L.off_partials);
    std::memset(host.data(), 0, L.off_partials);
    fill(host.data());
    DMUON_HIP_TRY(upload_by_kernel_args(ws, host.data(), L.off_partials, stream));
    DMUON_HIP_TRY(launch_clip_norm(items_dev, n, L.blocks, norm_type, partials, stream));
    DMUON_HIP_TRY(launch_clip_finalize(reinterpret_cast<const int64_t*>(ws + L.off_bucket_blocks), nbuckets,
                                       reinterpret_cast<const double*>(ws + L.off_max_norm), partials, norm_type,
                                       total_norm, coefs, stream));
    DMUON_HIP_TRY(launch_clip_scale(items_dev, n, L.blocks, coefs, stream));
    return DMUON_OK;
  }
  KeyBuf key;
  key.put_str("clip").put(n).put(nbuckets);
  for (int i = 0; i < n; ++i) key.put(grads[i]);
  for (int b = 0; b < nbuckets; ++b) key.put(max_norm[b]);
  st = stage_table(ws, L.off_partials, stream, key.s, fill);
  if (st) return st;
  int64_t bytes = 0;
  for (int i = 0; i < n; ++i) bytes += grads[i].numel * int64_t(dtype_size(grads[i].dtype));
  DMUON_HIP_TRY(prof_launch(PK_CLIP_NORM, 0, bytes, stream, [&] {
    return launch_clip_norm(items_dev, n, L.blocks, norm_type, partials, stream);
  }));
  DMUON_HIP_TRY(prof_launch(PK_CLIP_FINALIZE, 0, L.blocks * 8, stream, [&] {
    return launch_clip_finalize(reinterpret_cast<const int64_t*>(ws + L.off_bucket_blocks), nbuckets,
                                reinterpret_cast<const double*>(ws + L.off_max_norm), partials, norm_type,
                                total_norm, coefs, stream);
  }));
  if (coef_out) return DMUON_OK;   // the coefficients are the result; nothing is scaled
  DMUON_HIP_TRY(prof_launch(PK_CLIP_SCALE, 0, 2 * bytes, stream, [&] {
    return launch_clip_scale(items_dev, n, L.blocks, coefs, stream);
  }));
  return DMUON_OK;
}

}  // extern "C"

namespace dmuon {
int clip_grad_norm_in_scratch(const dmuon_grad_t* grads, int32_t n, int32_t nbuckets, const double* max_norm,
                              double norm_type, double* total_norm, int (*scratch_of_device)(void**),
                              size_t scratch_bytes, void* stream) {
  return clip_impl(grads, n, nbuckets, max_norm, norm_type, total_norm, nullptr, nullptr, scratch_bytes, stream,
                   true, scratch_of_device);
}
}  // namespace dmuon

extern "C" {

int dmuon_clip_grad_norm(const dmuon_grad_t* grads, int32_t n, int32_t nbuckets, const double* max_norm,
                         double norm_type, double* total_norm, void* workspace, size_t workspace_bytes,
                         void* stream) {
  return clip_impl(grads, n, nbuckets, max_norm, norm_type, total_norm, nullptr, workspace, workspace_bytes,
                   stream);
}

int dmuon_clip_coefficients(const dmuon_grad_t* grads, int32_t n, int32_t nbuckets, const double* max_norm,
                            double norm_type, double* total_norm, double* coef_out, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (!coef_out) {
    g_last_error = "coef_out is NULL";
    return DMUON_ERR_INVALID_ARG;
  }
  return clip_impl(grads, n, nbuckets, max_norm, norm_type, total_norm, coef_out, workspace, workspace_bytes,
                   stream);
}

// ---- dmuon_adamw_step --------------------------------------------------------

size_t dmuon_adamw_workspace_size(int32_t n) { return n <= 0 ? 0 : align_up(sizeof(AdamItem) * size_t(n)); }

int dmuon_adamw_step(const dmuon_adamw_tensor_t* tensors, int32_t n, const dmuon_adamw_group_t* groups,
                     int32_t ngroups, void* workspace, size_t workspace_bytes, void* stream_) {
  g_last_error.clear();
  if (n < 0) return fail(DMUON_ERR_INVALID_ARG, "n < 0");
  if (n == 0) return DMUON_OK;
  if (!tensors) return fail(DMUON_ERR_INVALID_ARG, "tensors is NULL");
  if (ngroups < 1 || !groups) return fail(DMUON_ERR_INVALID_ARG, "ngroups must be >= 1 and groups non-NULL");
  for (int k = 0; k < ngroups; ++k) {
    const dmuon_adamw_group_t& G = groups[k];
    const std::string name = mat_name("groups", k);
    if (!std::isfinite(G.lr) || !std::isfinite(G.weight_decay))
      return fail(DMUON_ERR_INVALID_ARG, name + ": lr and weight_decay must be finite");
    if (!std::isfinite(G.eps) || G.eps < 0) return fail(DMUON_ERR_INVALID_ARG, name + ": eps must be finite and >= 0");
    if (!(G.beta1 >= 0 && G.beta1 < 1) || !(G.beta2 >= 0 && G.beta2 < 1))
      return fail(DMUON_ERR_INVALID_ARG, name + ": betas must be in [0, 1)");
    if (G.step < 1) return fail(DMUON_ERR_INVALID_ARG, name + ": step must be >= 1");
  }
  std::vector<int> active;
  std::vector<Range> ranges;
  for (int i = 0; i < n; ++i) {
    const dmuon_adamw_tensor_t& T = tensors[i];
    const std::string name = mat_name("tensors", i);
    if (T.numel <= 0) return fail(DMUON_ERR_INVALID_ARG, name + ".numel must be > 0");
    if (!T.param || !T.exp_avg || !T.exp_avg_sq)
      return fail(DMUON_ERR_INVALID_ARG, name + ": param, exp_avg and exp_avg_sq must be non-NULL");
    if (!dtype_ok(T.param_dtype) || !dtype_ok(T.grad_dtype))
      return fail(DMUON_ERR_UNSUPPORTED, name + ": dtypes must be F32 or BF16");
    if (T.group < 0 || T.group >= ngroups) return fail(DMUON_ERR_INVALID_ARG, name + ".group out of range");
    if (!T.grad) continue;
    active.push_back(i);
    auto add = [&](const void* p, size_t bytes, const char* what) {
      const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
      ranges.push_back({lo, lo + bytes, name + "." + what});
    };
    const size_t ne = size_t(T.numel);
    add(T.param, ne * dtype_size(T.param_dtype), "param");
    add(T.grad, ne * dtype_size(T.grad_dtype), "grad");
    add(T.exp_avg, ne * 4, "exp_avg");
    add(T.exp_avg_sq, ne * 4, "exp_avg_sq");
  }
  if (active.empty()) return DMUON_OK;
  const size_t need = align_up(sizeof(AdamItem) * active.size());
  if (!workspace || workspace_bytes < need) return fail(DMUON_ERR_WORKSPACE, "workspace too small");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(DMUON_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  ranges.push_back({reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + need,
                    "workspace"});
  int st = check_overlaps(ranges);
  if (st) return st;
  st = check_device();
  if (st) return st;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  int64_t blocks = 0, bytes = 0;
  KeyBuf key;
  key.put_str("adamw").put(ngroups);
  for (int i : active) key.put(tensors[i]);
  for (int k = 0; k < ngroups; ++k) key.put(groups[k]);
  st = stage_table(workspace, need, stream, key.s, [&](char* host) {
    AdamItem* items = reinterpret_cast<AdamItem*>(host);
    for (size_t j = 0; j < active.size(); ++j) {
      const dmuon_adamw_tensor_t& T = tensors[active[j]];
      const dmuon_adamw_group_t& G = groups[T.group];
      AdamItem& it = items[j];
      it.p = T.param; it.g = T.grad; it.m = T.exp_avg; it.v = T.exp_avg_sq;
      it.numel = T.numel;
      it.blk_first = blocks;
      const double t = static_cast<double>(G.step);
      const double bc1 = 1.0 - std::pow(G.beta1, t), bc2 = 1.0 - std::pow(G.beta2, t);
      it.decay = static_cast<float>(1.0 - G.lr * G.weight_decay);
      it.step_size = static_cast<float>(G.lr / bc1);
      it.inv_sqrt_bc2 = static_cast<float>(1.0 / std::sqrt(bc2));
      it.eps = static_cast<float>(G.eps);
      it.beta1 = static_cast<float>(G.beta1);
      it.one_minus_beta1 = static_cast<float>(1.0 - G.beta1);
      it.beta2 = static_cast<float>(G.beta2);
      it.one_minus_beta2 = static_cast<float>(1.0 - G.beta2);
      it.p_dtype = T.param_dtype; it.g_dtype = T.grad_dtype;
      it.aligned = aligned16(T.param) && aligned16(T.grad) && aligned16(T.exp_avg) && aligned16(T.exp_avg_sq);
      blocks += (T.numel + kAdamChunk - 1) / kAdamChunk;
      bytes += T.numel * (2 * int64_t(dtype_size(T.param_dtype)) + int64_t(dtype_size(T.grad_dtype)) + 16);
    }
  });
  if (st) return st;
  const AdamItem* items_dev = static_cast<const AdamItem*>(workspace);
  const int na = static_cast<int>(active.size());
  DMUON_HIP_TRY(prof_launch(PK_ADAMW, 0, bytes, stream, [&] { return launch_adamw(items_dev, na, blocks, stream); }));
  return DMUON_OK;
}

size_t dmuon_apply_update_workspace_size(int32_t n) {
  return n <= 0 ? 0 : align_up(sizeof(EwMat) * n);
}

int dmuon_apply_update(const dmuon_matrix_t* mats, int32_t n, const void* const* update, int32_t update_dtype,
                       const dmuon_hparams_t* hp, void* workspace, size_t workspace_bytes, void* stream_) {
  g_last_error.clear();
  if (n < 0) return fail(DMUON_ERR_INVALID_ARG, "n < 0");
  if (n == 0) return DMUON_OK;
  if (!mats || !update) return fail(DMUON_ERR_INVALID_ARG, "mats or update is NULL");
  if (!hp) return fail(DMUON_ERR_INVALID_ARG, "hparams is NULL");
  if (!std::isfinite(hp->lr) || !std::isfinite(hp->weight_decay))
    return fail(DMUON_ERR_INVALID_ARG, "lr and weight_decay must be finite");
  if (!dtype_ok(update_dtype)) return fail(DMUON_ERR_UNSUPPORTED, "update_dtype must be F32 or BF16");
  const size_t need = dmuon_apply_update_workspace_size(n);
  if (!workspace || workspace_bytes < need) return fail(DMUON_ERR_WORKSPACE, "workspace too small");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(DMUON_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  std::vector<Range> ranges;
  std::vector<int64_t> blk(n);
  int64_t blocks = 0;
  for (int i = 0; i < n; ++i) {
    const dmuon_matrix_t& m = mats[i];
    int st = check_matrix_fields(m, i, false);
    if (st) return st;
    if (!m.param || !update[i]) return fail(DMUON_ERR_INVALID_ARG, mat_name("param/update", i) + " is NULL");
    const size_t ne = size_t(m.rows) * m.cols;
    const uintptr_t p = reinterpret_cast<uintptr_t>(m.param), u = reinterpret_cast<uintptr_t>(update[i]);
    ranges.push_back({p, p + ne * dtype_size(m.param_dtype), mat_name("param", i)});
    ranges.push_back({u, u + ne * dtype_size(update_dtype), mat_name("update", i)});
    blk[i] = blocks;
    blocks += ((m.rows + kEwTile - 1) / kEwTile) * ((m.cols + kEwTile - 1) / kEwTile);
  }
  ranges.push_back({reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + need, "workspace"});
  int st = check_overlaps(ranges);
  if (st) return st;
  st = check_device();
  if (st) return st;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  char* ws = static_cast<char*>(workspace);
  const float decay = static_cast<float>(1.0 - hp->lr * hp->weight_decay);
  KeyBuf key;
  key.put_str("apply_update").put(update_dtype).put(hp->lr).put(hp->weight_decay);
  for (int j = 0; j < n; ++j) key.put(mats[j]).put(update[j]);
  st = stage_table(ws, sizeof(EwMat) * n, stream, key.s, [&](char* host) {
    EwMat* em = reinterpret_cast<EwMat*>(host);
    for (int j = 0; j < n; ++j) {
      const dmuon_matrix_t& m = mats[j];
      EwMat& e = em[j];
      e.rows = m.rows; e.cols = m.cols;
      e.src = nullptr; e.mom = nullptr; e.param = m.param;
      e.u_dst = nullptr; e.o_src = update[j];
      e.u_dst_t = nullptr; e.ld_wide_t = 0;
      e.ld_wide = m.cols; e.wide_rows = static_cast<int32_t>(m.rows); e.wide_cols = static_cast<int32_t>(m.cols);
      e.tall = 0; e.src_dtype = update_dtype; e.wide_dtype = update_dtype; e.param_dtype = m.param_dtype;
      e.scale_idx = -1;
      e.aligned = (m.cols % 4 == 0) && aligned16(m.param);
      e.user_index = j;
      e.blk_wide = 0; e.blk_stored = blk[j];
      e.lr_eff = lr_eff_of(hp->lr, m.rows, m.cols);
      e.decay = decay;
    }
  });
  if (st) return st;
  DMUON_HIP_TRY(launch_update(reinterpret_cast<const EwMat*>(ws), n, blocks, 0, nullptr, stream));
  return DMUON_OK;
}

// ---- measurement hooks -------------------------------------------------------

int dmuon_profile_begin(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = true;
  return DMUON_OK;
}

int64_t dmuon_profile_end(char* buf, size_t buf_len) {
  std::vector<ProfRec> recs;
  bool was_on;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    was_on = g_prof_on;
    g_prof_on = false;
    recs.swap(g_prof);
  }
  static std::string last_report = "{\"kernels\": {}}";
  if (!was_on && recs.empty()) {
    // no profiling window open: hand out the last report again
    if (buf && buf_len) {
      const size_t k = std::min(buf_len - 1, last_report.size());
      std::memcpy(buf, last_report.data(), k);
      buf[k] = '\0';
    }
    return static_cast<int64_t>(last_report.size());
  }
  int64_t count[PK_COUNT] = {}, flops[PK_COUNT] = {}, bytes[PK_COUNT] = {};
  double ms[PK_COUNT] = {};
  // every launch's interval against the window's first event (events on
  // different streams of one device share a clock); the union of a kind's
  // intervals is its wall time when launches on two streams overlap
  std::vector<std::pair<double, double>> spans[PK_COUNT];
  int status = DMUON_OK;
  for (auto& r : recs) {
    float t = 0.f, t0 = 0.f;
    if (status == DMUON_OK) {
      hipError_t e = hipEventSynchronize(r.b);
      if (e == hipSuccess) e = hipEventSynchronize(recs.front().a);
      if (e == hipSuccess) e = hipEventElapsedTime(&t, r.a, r.b);
      if (e == hipSuccess) e = hipEventElapsedTime(&t0, recs.front().a, r.a);
      if (e != hipSuccess) status = fail(DMUON_ERR_HIP, std::string("profile events: ") + hipGetErrorString(e));
    }
    count[r.kind] += 1;
    ms[r.kind] += t;
    flops[r.kind] += r.flops;
    bytes[r.kind] += r.bytes;
    spans[r.kind].emplace_back(double(t0), double(t0) + double(t));
  }
  for (auto& r : recs) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  if (status != DMUON_OK) return status;
  double wall[PK_COUNT] = {};
  for (int k = 0; k < PK_COUNT; ++k) {
    auto& v = spans[k];
    std::sort(v.begin(), v.end());
    double lo = 0.0, hi = -1.0;
    for (auto& iv : v) {
      if (iv.first > hi) {
        if (hi > lo) wall[k] += hi - lo;
        lo = iv.first;
        hi = iv.second;
      } else {
        hi = std::max(hi, iv.second);
      }
    }
    if (hi > lo) wall[k] += hi - lo;
  }
  std::ostringstream os;
  os.precision(9);
  os << "{\"kernels\": {";
  bool first = true;
  for (int k = 0; k < PK_COUNT; ++k) {
    if (!count[k]) continue;
    os << (first ? "" : ", ") << "\"" << kProfNames[k] << "\": {\"launches\": " << count[k]
       << ", \"ms\": " << ms[k] << ", \"wall_ms\": " << wall[k] << ", \"flops\": " << flops[k]
       << ", \"bytes\": " << bytes[k] << "}";
    first = false;
  }
  os << "}}";
  last_report = os.str();
  if (buf && buf_len) {
    const size_t k = std::min(buf_len - 1, last_report.size());
    std::memcpy(buf, last_report.data(), k);
    buf[k] = '\0';
  }
  return static_cast<int64_t>(last_report.size());
}

// ---- plan description (host only) -------------------------------------------

int64_t dmuon_plan_describe(const int64_t* rows, const int64_t* cols, int32_t n, const dmuon_hparams_t* hp,
                            char* buf, size_t buf_len) {
  g_last_error.clear();
  Coeffs cf;
  std::shared_ptr<Plan> plan;
  int st = ortho_prepare(rows, cols, n, hp, &cf, &plan);
  if (st) return st;
  std::ostringstream os;
  os << "{\"n\": " << n;
  if (n > 0) {
    const Plan& P = *plan;
    os << ", \"tile\": " << P.tile << ", \"ns_steps\": " << P.ns_steps
       << ", \"workspace_bytes\": " << P.ws_bytes
       << ", \"elementwise_blocks\": {\"wide\": " << P.blocks_wide << ", \"stored\": " << P.blocks_stored << "}"
       << ", \"matrices\": [";
    for (int i = 0; i < P.n; ++i) {
      const MatLayout& L = P.mats[i];
      os << (i ? ", " : "") << "{\"rows\": " << L.rows << ", \"cols\": " << L.cols
         << ", \"form\": \"" << (L.form == FORM_GRAM ? "gram" : "direct") << "\""
         << ", \"tall\": " << (L.tall ? "true" : "false") << ", \"tile\": " << L.tile
         << ", \"m_pad\": " << L.mp << ", \"n_pad\": " << L.np << "}";
    }
    // every launch's map must hit each output tile once, and give XCD x
    // exactly the blocks b < tiles with b % 8 == x
    bool map_ok = P.tile_map.size() == [&] { size_t t = 0; for (auto& l : P.launches) t += l.tiles; return t; }();
    for (const Launch& l : P.launches) {
      std::vector<std::vector<char>> seen(l.count);
      for (int j = 0; j < l.count; ++j) {
        const Op& o = P.ops[l.first + j];
        seen[j].assign(size_t(o.tiles_m) * o.tiles_n, 0);
      }
      for (int64_t b = 0; b < l.tiles && map_ok; ++b) {
        const TileRef r = P.tile_map[l.map_first + b];
        if (r.task < 0 || r.task >= l.count) { map_ok = false; break; }
        const Op& o = P.ops[l.first + r.task];
        if (r.tm >= o.tiles_m || r.tn >= o.tiles_n || (o.sym && r.tn < r.tm)) { map_ok = false; break; }
        char& c = seen[r.task][size_t(r.tm) * o.tiles_n + r.tn];
        if (c) { map_ok = false; break; }
        c = 1;
      }
    }
    os << "], \"tile_map_valid\": " << (map_ok ? "true" : "false");
    // the groups dmuon_step / dmuon_orthogonalize run on two streams (one
    // group: a single launch sequence)
    const auto groups = stream_groups(std::vector<int64_t>(rows, rows + n), std::vector<int64_t>(cols, cols + n),
                                      hp->ns_precision, hp->ns_backend, P.ns_steps);
    os << ", \"stream_groups\": [";
    for (size_t g = 0; g < groups.size(); ++g) {
      os << (g ? ", " : "") << "[";
      for (size_t k = 0; k < groups[g].size(); ++k) os << (k ? ", " : "") << groups[g][k];
      os << "]";
    }
    os << "], \"launches\": [";
    for (size_t j = 0; j < P.launches.size(); ++j) {
      const Launch& l = P.launches[j];
      int64_t flops = 0;
      int64_t kmax = 0, kmin = INT64_MAX;
      for (int q = 0; q < l.count; ++q) {
        const Op& o = P.ops[l.first + q];
        flops += 2 * op_tiles(o) * o.tile * o.tile * o.K;
        kmax = std::max<int64_t>(kmax, o.K);
        kmin = std::min<int64_t>(kmin, o.K);
      }
      int nsym = 0;
      for (int q = 0; q < l.count; ++q) nsym += P.ops[l.first + q].sym;
      os << (j ? ", " : "") << "{\"sym_tasks\": " << nsym << ", \"left_tasks\": " << (l.count - nsym)
         << ", \"tile\": " << l.tile << ", \"tasks\": " << l.count << ", \"tiles\": " << l.tiles
         << ", \"k_max\": " << kmax << ", \"k_min\": " << kmin << ", \"flops\": " << flops << "}";
    }
    os << "]";
  }
  os << "}";
  const std::string s = os.str();
  if (buf && buf_len) {
    const size_t k = std::min(buf_len - 1, s.size());
    std::memcpy(buf, s.data(), k);
    buf[k] = '\0';
  }
  return static_cast<int64_t>(s.size());
}

}  // extern "C"
