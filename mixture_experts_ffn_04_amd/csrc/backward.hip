// Backward of the layer: gradients of sum(out * dout) with the selection held
// at the forward's indices.
//
// [SF1033] = SpecForge PR #1033 "MoE FFN for DFlash-family drafts: the
// module", "Router" section (forward returns scores, indices, weights; the
// weights gather the unshifted scores, renormalise with the 1e-20 guard and
// scale).  [SF1073] = SpecForge PR #1073 "MoE drafts: DeepSeek-V4.1's own
// DSpark draft (stacked on #1035)": the expert bias shifts the picks, never
// the weights; clamped SwiGLU; the V4.1 port's output and every gradient are
// compared.  [SGL48763] = sglang PR #48763: sigmoid-gated shared expert.
//
// Plan (the forward in reverse; fp32 arithmetic, bf16 inputs widened exactly):
//   1. stable permutation: rows of each expert in slot order (so every sum
//      over an expert's rows has a fixed order), row -> token, row -> weight
//   2. routing weights per slot from the forward's scores (as the forward)
//   3. pre = x Wgu^T (+ b), h = SwiGLU(pre)           grouped GEMM, elementwise
//   4. gd = dout Wd  (so dh = w gd and dout . y = gd . h + dout . b_down)
//   5. dweights, dpre = SwiGLU'(pre, w gd)           elementwise, row dots
//   6. dx_rows = dpre Wgu; dWd = sum_r (w dout)^T h; dWgu = sum_r dpre^T x;
//      expert bias gradients by ordered row sums
//   7. the shared expert the same way over all tokens, with its gate
//   8. router: d weights -> d scores (renormalisation) -> d logits (score
//      function) -> dgate = dl^T x, drouter_bias = sum_t dl, dx += dl gate
//   9. dx = sum_k dx_rows (k order) + shared + router + gate terms
// One generic grouped GEMM on the bf16 matrix cores (128 x 128 tiles staged
// in LDS, fixed k order per output) serves every contraction through operand
// descriptors; fp32 operands enter as exact pairs of bf16 numbers (hi + lo),
// so the products carry at most a few 2^-18 of relative error.  The three
// expert products, when experts hold few rows, run instead on the fp32
// matrix cores in 16-row tiles of one wave that read their operands straight
// from memory, with the reduction split into fixed chunks whose partial
// results a separate pass sums in chunk order, so the result does not depend
// on scheduling.
#include <algorithm>
#include <type_traits>

#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kSkinnyRows = 16;

// expert ids index memory: keep them in range whatever the caller passed
__device__ __forceinline__ int clamp_id(int e, int E) { return min(max(e, 0), E - 1); }

__device__ __forceinline__ float ld_elem(const void *p, int bf16, size_t i) {
  return bf16 ? bf16_to_f32(static_cast<const uint16_t *>(p)[i]) : static_cast<const float *>(p)[i];
}

// Element (i, k) of an operand, i = row of the output (A) or column (B).
// kmajor = 0: element at row(i) * ld + k; kmajor = 1: at row(k) * ld + i.
// The "row" index runs along i (kmajor 0) or k (kmajor 1); it is offset by
// the group's first row when token_rows is set, mapped through gather and
// scaled by scale[] when those are given.  Weight operands use gstride: the
// group's matrix starts at group * gstride.
struct GOp {
  const void *p;
  int bf16, kmajor, token_rows, vec;  // vec: the base and every row start are 16-byte aligned
  long ld, gstride;
  const int32_t *gather;
  const float *scale;
};

// C[m, n] = sum_k A(m, k) B(n, k) for each group.
//   mode 0: one group of M x N x K.
//   mode 1: group e has counts[e] rows (M), row base offsets[e]; the row tiles
//           of all groups are listed by mtile_prefix (tiles of the kernel's
//           row height); C rows are the global rows.  With ksplit > 1, chunk
//           z of kchunk reduction steps writes its partial product to
//           C + z * split_stride.
//   mode 2: group e has counts[e] reduction steps (K), row base offsets[e];
//           C of group e starts at e * cgstride.  Groups with no rows write 0.
struct GGemm {
  GOp A, B;
  float *C;
  long ldc, cgstride;
  int M, N, K, mode, E;
  const int32_t *counts, *offsets, *mtile_prefix;
  int ksplit, kchunk;
  long split_stride;
  int vec;  // both operands read as whole 16-byte runs (vec_runs)
};

// Reads of one operand in runs of eight elements along its contiguous
// direction: (i, k..k+7) when KM = 0 (row-major), (i..i+7, k) when KM = 1
// (k-major).  Elements outside [0, ni) x [0, nk) read as 0.  Every access is
// made at a clamped in-bounds address and masked afterwards, so the code has
// no branches around loads and the next slice's loads stay in flight while
// the current one is multiplied.  VEC: every run is whole or empty (the run
// dimension is a multiple of 8, rows start on 16-byte boundaries), and is
// read with 16-byte loads.
template <int KM, int BF, bool VEC>
struct Runs {
  // the "row" of a run is i (KM = 0, fixed per thread) or k (KM = 1)
  size_t base;  // element offset of the row
  float sc;
  bool ok;
  // a row's source (through gather) and scale: fetched ahead of the loads
  // that use them when the row changes from slice to slice (k-major)
  struct Ix {
    long src;
    float sc;
    bool ok;
  };
  __device__ __forceinline__ static Ix fetch(const GOp &o, int row, int nrow, int r0) {
    Ix x;
    x.ok = row < nrow;
    const int rix = (o.token_rows ? r0 : 0) + (x.ok ? row : nrow - 1);
    x.src = o.gather ? o.gather[rix] : rix;
    x.sc = o.scale ? o.scale[rix] : 1.f;
    return x;
  }
  __device__ __forceinline__ void set(const GOp &o, const Ix &x, int grp) {
    ok = x.ok;
    base = (size_t)grp * o.gstride + (size_t)x.src * o.ld;
    sc = x.sc;
  }
  __device__ __forceinline__ void set_row(const GOp &o, int row, int nrow, int grp, int r0) {
    set(o, fetch(o, row, nrow, r0), grp);
  }
  // issue(): the loads of one run, kept raw; finish(): decode, scale and
  // mask.  Between the two the loads stay in flight.
  struct Raw {
    uint32_t w[8];
    uint32_t on;  // bit q: element q is in range
    float sc;
  };
  __device__ __forceinline__ void issue(const GOp &o, int run0, int runn, Raw &r) const {
    r.sc = sc;
    if constexpr (VEC) {
      const bool on = ok && run0 < runn;
      r.on = on ? 0xffu : 0u;
      const size_t at = base + (on ? run0 : runn - 8);
      if constexpr (BF) {
        const u32x4_t u = load16(static_cast<const uint16_t *>(o.p) + at);
#pragma unroll
        for (int q = 0; q < 4; ++q) r.w[q] = u[q];
      } else {
        const u32x4_t *f = reinterpret_cast<const u32x4_t *>(static_cast<const float *>(o.p) + at);
        const u32x4_t a = f[0], b = f[1];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          r.w[q] = a[q];
          r.w[4 + q] = b[q];
        }
      }
    } else {
      r.on = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const bool on = ok && run0 + q < runn;
        r.on |= on ? 1u << q : 0u;
        r.w[q] = __float_as_uint(ld_elem(o.p, BF, base + (on ? run0 + q : 0)));
      }
    }
  }
  __device__ __forceinline__ static void finish(const Raw &r, float (&v)[8]) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      float x;
      if constexpr (VEC && BF) x = bf16_to_f32(q & 1 ? r.w[q >> 1] >> 16 : r.w[q >> 1] & 0xffffu);
      else x = __uint_as_float(r.w[q]);
      v[q] = (r.on >> q) & 1 ? x * r.sc : 0.f;
    }
  }
};

// ---- contractions on the bf16 matrix cores ----------------------------------
// C[m, n] = sum_k A(m, k) B(n, k) with v_mfma_f32_32x32x16_bf16: bf16 operand
// products are exact in fp32 and summed in fp32.  An operand that is bf16 in
// memory (and not scaled) enters as it is; an fp32 (or scaled) operand v is
// split into two bf16 numbers hi = rne(v), lo = rne(v - hi), which hold v to
// 2^-18 of its size, and the product takes the passes hi.hi, lo.hi (A split),
// hi.lo (B split); the lo.lo term (2^-18 of the product) is dropped.  So each
// product carries a relative error of a few 2^-18 at most, far below the
// rounding of the fp32 sums over the reduction.
//
// Tile 128 x 128 with 256 threads; four waves of 64 x 64 (2 x 2 fragments of
// 32 x 32); 32-deep reduction slices staged in LDS as bf16 planes (hi, and lo
// for a split operand) of [row][k] with an XOR swizzle of the 16-byte chunks
// (row r, chunk c at r * 4 + (c ^ (r / 4) % 4)), so the 32 rows of a fragment
// read and the 16 rows of a row-major store hit distinct banks.  The next
// slice's global loads are in flight while the current slice is multiplied.
// The weight-gradient products reduce over an expert's rows only (a hundred
// or so at T*K/E of that size), a few slices per tile, so each tile's first
// loads are exposed: three workgroups per CU (registers held to 168 per lane
// in the 16-byte-run forms, without spills) overlap them.
constexpr int kMT = 128;  // output tile rows and columns of the matrix-core kernel
constexpr int kMK = 32;   // reduction slice

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef float f32x16v __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16v mfma32(u32x4_t a, u32x4_t b, f32x16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8v, a), __builtin_bit_cast(bf16x8v, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ int munit(int row, int ch) { return row * 4 + (ch ^ ((row >> 2) & 3)); }

template <int AF, int BF, bool VEC>
__global__ __launch_bounds__(256, VEC ? 3 : 2) void grouped_gemm_mfma(GGemm g) {
  constexpr int AK = AF & 1, BK = BF & 1;
  constexpr int NT = 256;
  constexpr int NR = kMT * kMK / 8 / NT;  // 8-element runs per thread, operand and slice (2)
  constexpr int PU = kMT * 4;             // 16-byte units of one plane
  // LDS planes: A hi, A lo, B hi, B lo
  __shared__ u32x4_t lds[4 * PU];
  u32x4_t *Ah = lds, *Al = lds + PU, *Bh = lds + 2 * PU, *Bl = lds + 3 * PU;
  const bool asplit = !(AF >> 1) || g.A.scale, bsplit = !(BF >> 1) || g.B.scale;

  int grp = 0, m0, M, K, r0 = 0;
  const int n0 = blockIdx.x * kMT;
  if (g.mode == 0) {
    m0 = blockIdx.y * kMT;
    M = g.M;
    K = g.K;
  } else if (g.mode == 1) {
    const int q = blockIdx.y;
    if (q >= g.mtile_prefix[g.E]) return;
    int lo = 0, hi = g.E;  // mtile_prefix[lo] <= q < mtile_prefix[lo + 1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (g.mtile_prefix[mid] <= q) lo = mid;
      else hi = mid;
    }
    grp = lo;
    m0 = (q - g.mtile_prefix[lo]) * kMT;
    M = g.counts[lo];
    K = g.K;
    r0 = g.offsets[lo];
  } else {
    const int mtiles = (g.M + kMT - 1) / kMT;
    grp = blockIdx.y / mtiles;
    m0 = (blockIdx.y - grp * mtiles) * kMT;
    M = g.M;
    K = g.counts[grp];
    r0 = g.offsets[grp];
  }
  if (m0 >= M || n0 >= g.N) return;  // whole workgroup leaves together

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, lh = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;
  // Run u of a thread: row-major operand: row (tid + 256 u) / 4, chunk
  // tid % 4; k-major operand: 8 rows from (tid % 16) * 8 at k = 2 (tid / 16) + u,
  // so a thread's two runs pair up k and k + 1 for each row (4-byte stores).
  auto place = [&](int u, bool kmajor, int &i, int &k) {
    if (kmajor) {
      i = (tid & 15) * 8;
      k = 2 * (tid >> 4) + u;
    } else {
      i = (tid + NT * u) >> 2;
      k = (tid & 3) * 8;
    }
  };
  int ai[NR], ak[NR], bi[NR], bk[NR];
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    place(u, AK, ai[u], ak[u]);
    place(u, BK, bi[u], bk[u]);
  }
  using RA = Runs<AK, (AF >> 1), VEC>;
  using RB = Runs<BK, (BF >> 1), VEC>;
  RA ra_[NR];
  RB rb_[NR];
  if constexpr (!AK) {
#pragma unroll
    for (int u = 0; u < NR; ++u) ra_[u].set_row(g.A, m0 + ai[u], M, grp, r0);
  }
  if constexpr (!BK) {
#pragma unroll
    for (int u = 0; u < NR; ++u) rb_[u].set_row(g.B, n0 + bi[u], g.N, grp, r0);
  }
  typename RA::Raw ra[NR];
  typename RB::Raw rb[NR];
  // Slice s of nsl (indices past the end load the last slice again: every
  // iteration issues the same loads, so the compiler's wait counts stay
  // exact).  A k-major operand's rows change with the slice; their sources
  // and scales (a gather and a scale load each) are fetched one slice ahead
  // of the data loads that use them, and issued before those data loads:
  // waiting for the indices (the addresses of the next slice) then leaves
  // the data loads in flight.
  const int nsl = (K + kMK - 1) / kMK;
  typename RA::Ix ixa[NR];
  typename RB::Ix ixb[NR];
  auto fetch_ix = [&](int sl) {
    const int k0 = min(sl, nsl - 1) * kMK;
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      if constexpr (AK) ixa[u] = RA::fetch(g.A, k0 + ak[u], K, r0);
      if constexpr (BK) ixb[u] = RB::fetch(g.B, k0 + bk[u], K, r0);
    }
  };
  auto set_bases = [&]() {  // k-major rows of the slice whose indices are in ixa / ixb
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      if constexpr (AK) ra_[u].set(g.A, ixa[u], grp);
      if constexpr (BK) rb_[u].set(g.B, ixb[u], grp);
    }
  };
  auto issue_data = [&](int sl) {
    const int k0 = min(sl, nsl - 1) * kMK;
#pragma unroll
    for (int u = 0; u < NR; ++u) {
      if constexpr (AK) ra_[u].issue(g.A, m0 + ai[u], M, ra[u]);
      else ra_[u].issue(g.A, k0 + ak[u], K, ra[u]);
      if constexpr (BK) rb_[u].issue(g.B, n0 + bi[u], g.N, rb[u]);
      else rb_[u].issue(g.B, k0 + bk[u], K, rb[u]);
    }
  };
  // One operand's runs of a slice -> its LDS planes.  Exact bf16 operands
  // (stored as bf16, not scaled, whole 16-byte runs) go in as their raw
  // words; the others are split into (hi, lo) pairs with the paired
  // conversion (round to nearest even).  k-major runs pair up k and k + 1
  // for each row (one 4-byte store per row and plane); row-major runs are
  // one row's 8 consecutive k (one 16-byte store per plane).
  auto stash = [&](auto R, auto vecbf, const auto (&raw)[NR], const int (&ri)[NR], const int (&rk)[NR],
                   bool kmajor, bool split, u32x4_t *H, u32x4_t *L) {
    using RT = decltype(R);
    if constexpr (decltype(vecbf)::value) {
      if (!split) {
        if (kmajor) {
          const int k = rk[0];
          const uint32_t m0 = raw[0].on ? 0xffffffffu : 0u, m1 = raw[1].on ? 0xffffffffu : 0u;
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            // element q of run k (low half) and of run k + 1 (high half)
            const uint32_t w0 = raw[0].w[q >> 1] & m0, w1 = raw[1].w[q >> 1] & m1;
            const uint32_t d = __builtin_amdgcn_perm(w1, w0, q & 1 ? 0x07060302u : 0x05040100u);
            reinterpret_cast<uint32_t *>(H)[munit(ri[0] + q, k >> 3) * 4 + ((k & 7) >> 1)] = d;
          }
        } else {
#pragma unroll
          for (int u = 0; u < NR; ++u) {
            const uint32_t m = raw[u].on ? 0xffffffffu : 0u;
            H[munit(ri[u], rk[u] >> 3)] =
                u32x4_t{raw[u].w[0] & m, raw[u].w[1] & m, raw[u].w[2] & m, raw[u].w[3] & m};
          }
        }
        return;
      }
    }
    float v[NR][8];
#pragma unroll
    for (int u = 0; u < NR; ++u) RT::finish(raw[u], v[u]);
    // (a, b) -> packed bf16 hi pair and lo pair, hi + lo = (a, b) to 2^-18
    auto split2 = [](float a, float b, uint32_t &hp, uint32_t &lp) {
      hp = pack_bf16x2(a, b);
      lp = pack_bf16x2(a - bf16_lo(hp), b - bf16_hi(hp));
    };
    if (kmajor) {
      const int k = rk[0];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        uint32_t hp, lp;
        split2(v[0][q], v[1][q], hp, lp);
        const int off = munit(ri[0] + q, k >> 3) * 4 + ((k & 7) >> 1);  // dword within the plane
        reinterpret_cast<uint32_t *>(H)[off] = hp;
        if (split) reinterpret_cast<uint32_t *>(L)[off] = lp;
      }
    } else {
#pragma unroll
      for (int u = 0; u < NR; ++u) {
        uint32_t hp[4], lp[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) split2(v[u][2 * q], v[u][2 * q + 1], hp[q], lp[q]);
        const int un = munit(ri[u], rk[u] >> 3);
        H[un] = u32x4_t{hp[0], hp[1], hp[2], hp[3]};
        if (split) L[un] = u32x4_t{lp[0], lp[1], lp[2], lp[3]};
      }
    }
  };

  f32x16v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  if (nsl > 0) {
    fetch_ix(0);
    set_bases();
    fetch_ix(1);
    issue_data(0);
  }
  for (int sl = 0; sl < nsl; ++sl) {
    stash(RA{}, std::bool_constant<VEC && (AF >> 1)>{}, ra, ai, ak, AK, asplit, Ah, Al);
    stash(RB{}, std::bool_constant<VEC && (BF >> 1)>{}, rb, bi, bk, BK, bsplit, Bh, Bl);
    __syncthreads();
    set_bases();       // slice sl + 1
    fetch_ix(sl + 2);
    issue_data(sl + 1);
#pragma unroll
    for (int kk = 0; kk < kMK / 16; ++kk) {
      const int ch = 2 * kk + lh;
      u32x4_t a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = Ah[munit(wm * 64 + i * 32 + l32, ch)];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = Bh[munit(wn * 64 + j * 32 + l32, ch)];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
      if (asplit) {
        u32x4_t al[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) al[i] = Al[munit(wm * 64 + i * 32 + l32, ch)];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(al[i], b[j], acc[i][j]);
      }
      if (bsplit) {
        u32x4_t bl[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) bl[j] = Bl[munit(wn * 64 + j * 32 + l32, ch)];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[i], bl[j], acc[i][j]);
      }
    }
    __syncthreads();
  }

  // lane l holds column l % 32 of each fragment and rows 8 (e / 4) + 4 (l / 32) + e % 4
  float *C = g.C + (g.mode == 2 ? (size_t)grp * g.cgstride : 0);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + j * 32 + l32;
    if (n >= g.N) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
        if (m >= M) continue;
        float *dst = C + (g.mode == 1 ? (size_t)(r0 + m) : (size_t)m) * g.ldc + n;
        // weight gradients are written once and not read back here: stream them
        if (g.mode == 2) __builtin_nontemporal_store(acc[i][j][e], dst);
        else *dst = acc[i][j][e];
      }
    }
  }
}


// ---- expert products with few rows on the fp32 matrix cores -----------------
// v_mfma_f32_16x16x4f32 takes fp32 operands and sums fp32 products in fp32,
// the arithmetic of the multiply-add path.  Lane l supplies A(l % 16, k = l /
// 16) and B(k = l / 16, col l % 16) and holds C(4 (l / 16) + i, col l % 16).
// Which reduction index and which output column a lane's operands stand for
// is ours to choose, as long as A and B agree:
//   B k-major: each lane loads 8 consecutive columns at one k (16 bytes);
//   product q of a 4-deep substep gives output column n0 + 8 (l % 16) + q.
//   A wave computes 16 rows x 128 columns in 32-deep steps (8 substeps).
//   B row-major: each lane loads 16 consecutive k of one column (a whole
//   32-byte run, so a 16-lane row group reads whole 128-byte lines); product
//   r of column block c takes k = k0 + 16 (l / 16) + r and gives column
//   n0 + 16 c + l % 16.  A wave computes 16 rows x 64 columns in 64-deep steps.
// The next step's loads are in flight while the current step multiplies.
// Loads go to clamped in-bounds addresses and are masked at use.
template <int BKM>
struct SkinnyShape {
  static constexpr int cols = BKM ? 128 : 64, step = BKM ? 32 : 64;
  static constexpr int nacc = 8 * (BKM ? 1 : 0) + 4 * (BKM ? 0 : 1);  // accumulators (16 x 16 each)
};

__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 16-byte load of element offset `at` of a bf16 (BF) or f32 array
template <int BF>
__device__ __forceinline__ u32x4_t ld16(const void *p, size_t at) {
  return BF ? load16(static_cast<const uint16_t *>(p) + at) : load16(static_cast<const float *>(p) + at);
}

template <int BKM, int ABF, int BBF>
struct SkinnyStage {
  // k-major B: 8 substeps x 8 elements; A: 8 single elements (raw words)
  // row-major B: 4 column blocks x 16 elements; A: 16 elements
  static constexpr int nb = BKM ? 8 : 4, bw = (BKM ? 8 : 16) / (BBF ? 2 : 1);
  static constexpr int aw = BKM ? 8 : 16 / (ABF ? 2 : 1);
  uint32_t b[nb][bw];
  uint32_t a[aw];
  uint32_t bon, aon;  // in-range bits
};

template <int BKM, int ABF, int BBF>
__global__ __launch_bounds__(64) void skinny_mfma_f32(GGemm g) {
  using Sh = SkinnyShape<BKM>;
  const int q = blockIdx.y;
  if (q >= g.mtile_prefix[g.E]) return;
  int lo = 0, hi = g.E;  // mtile_prefix[lo] <= q < mtile_prefix[lo + 1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (g.mtile_prefix[mid] <= q) lo = mid;
    else hi = mid;
  }
  const int grp = lo, M = g.counts[grp], r0 = g.offsets[grp];
  const int m0 = (q - g.mtile_prefix[grp]) * kSkinnyRows, n0 = blockIdx.x * Sh::cols;
  if (m0 >= M || n0 >= g.N) return;
  const int kbeg = blockIdx.z * g.kchunk;
  const int kend = g.ksplit > 1 ? min(g.K, kbeg + g.kchunk) : g.K;
  const int l = threadIdx.x, lr = l & 15, lk = l >> 4;
  const GOp &A = g.A, &B = g.B;
  // this lane's A row (token rows of the group, maybe gathered and scaled)
  const bool aok = m0 + lr < M;
  const int arix = (A.token_rows ? r0 : 0) + (aok ? m0 + lr : M - 1);
  const size_t abase = (size_t)(A.gather ? A.gather[arix] : arix) * A.ld;
  const float asc = A.scale ? A.scale[arix] : 1.f;
  const size_t bgrp = (size_t)grp * B.gstride;
  using Stage = SkinnyStage<BKM, ABF, BBF>;
  auto load = [&](int k0, Stage &st) {
    st.bon = st.aon = 0;
    if constexpr (BKM) {
      const int n = n0 + 8 * lr;
      const bool nok = n < g.N;  // whole runs: n + 8 <= N
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int k = k0 + 4 * s + lk;
        const bool on = nok && k < kend;
        st.bon |= on ? 1u << s : 0u;
        const size_t at = bgrp + (size_t)(on ? k : kend - 1) * B.ld + (on ? n : g.N - 8);
        const u32x4_t w0 = ld16<BBF>(B.p, at);
#pragma unroll
        for (int j = 0; j < 4; ++j) st.b[s][j] = w0[j];
        if constexpr (!BBF) {
          const u32x4_t w1 = ld16<BBF>(B.p, at + 4);
#pragma unroll
          for (int j = 0; j < 4; ++j) st.b[s][4 + j] = w1[j];
        }
        const bool aon = aok && k < kend;
        st.aon |= aon ? 1u << s : 0u;
        const size_t ai = abase + (aon ? k : kend - 1);
        st.a[s] = ABF ? static_cast<const uint16_t *>(A.p)[ai] : __float_as_uint(static_cast<const float *>(A.p)[ai]);
      }
    } else {
      // two 8-runs per lane: k0 + 16 lk + 8 h, h = 0, 1 (whole runs: each in
      // range or not)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = k0 + 16 * lk + 8 * h;
        const bool kok = k < kend;
        const size_t kc = kok ? k : kend - 8;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int n = n0 + 16 * c + lr;
          const bool on = kok && n < g.N;
          st.bon |= on ? 1u << (2 * c + h) : 0u;
          const size_t at = bgrp + (size_t)(n < g.N ? n : g.N - 1) * B.ld + kc;
          const u32x4_t w0 = ld16<BBF>(B.p, at);
          constexpr int hw = BBF ? 4 : 8;  // words per 8-run
#pragma unroll
          for (int j = 0; j < 4; ++j) st.b[c][h * hw + j] = w0[j];
          if constexpr (!BBF) {
            const u32x4_t w1 = ld16<BBF>(B.p, at + 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) st.b[c][h * hw + 4 + j] = w1[j];
          }
        }
        const bool aon = aok && kok;
        st.aon |= aon ? 1u << h : 0u;
        const u32x4_t w0 = ld16<ABF>(A.p, abase + kc);
        constexpr int hw = ABF ? 4 : 8;
#pragma unroll
        for (int j = 0; j < 4; ++j) st.a[h * hw + j] = w0[j];
        if constexpr (!ABF) {
          const u32x4_t w1 = ld16<ABF>(A.p, abase + kc + 4);
#pragma unroll
          for (int j = 0; j < 4; ++j) st.a[h * hw + 4 + j] = w1[j];
        }
      }
    }
  };
  // element e of a run of raw words, widened
  auto elem = [](const uint32_t *w, int e, auto bf) -> float {
    if constexpr (decltype(bf)::value) return bf16_to_f32(e & 1 ? w[e >> 1] >> 16 : w[e >> 1] & 0xffffu);
    else return __uint_as_float(w[e]);
  };
  using BBf = std::integral_constant<bool, BBF != 0>;
  using ABf = std::integral_constant<bool, ABF != 0>;
  f32x4_t acc[Sh::nacc];
#pragma unroll
  for (int c = 0; c < Sh::nacc; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const Stage &st) {
    if constexpr (BKM) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const float a = (st.aon >> s) & 1 ? (ABF ? bf16_to_f32(st.a[s]) : __uint_as_float(st.a[s])) * asc : 0.f;
        const bool bon = (st.bon >> s) & 1;
#pragma unroll
        for (int qn = 0; qn < 8; ++qn) acc[qn] = mfma_f32(a, bon ? elem(st.b[s], qn, BBf{}) : 0.f, acc[qn]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int h = r >> 3;
        const float a = (st.aon >> h) & 1 ? elem(st.a, r, ABf{}) * asc : 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[c] = mfma_f32(a, (st.bon >> (2 * c + h)) & 1 ? elem(st.b[c], r, BBf{}) : 0.f, acc[c]);
      }
    }
  };
  if (kbeg < kend) {  // the clamped addresses need kend >= 8
    // the scheduling barriers keep each step's loads ahead of the previous
    // step's products (the scheduler would otherwise sink them next to their
    // uses and leave nothing in flight)
    constexpr int S = Sh::step;
    Stage st0, st1;
    load(kbeg, st0);
    for (int k0 = kbeg; k0 < kend; k0 += 2 * S) {
      load(k0 + S, st1);  // masked when past the end
      __builtin_amdgcn_sched_barrier(0);
      compute(st0);
      __builtin_amdgcn_sched_barrier(0);
      load(k0 + 2 * S, st0);
      __builtin_amdgcn_sched_barrier(0);
      compute(st1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float *C = g.C + (size_t)blockIdx.z * g.split_stride;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + 4 * lk + i;
    if (m >= M) continue;
    float *row = C + (size_t)(r0 + m) * g.ldc;
    if constexpr (BKM) {
      const int n = n0 + 8 * lr;
      if (n < g.N) {
        *reinterpret_cast<f32x4_t *>(row + n) = f32x4_t{acc[0][i], acc[1][i], acc[2][i], acc[3][i]};
        *reinterpret_cast<f32x4_t *>(row + n + 4) = f32x4_t{acc[4][i], acc[5][i], acc[6][i], acc[7][i]};
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int n = n0 + 16 * c + lr;
        if (n < g.N) row[n] = acc[c][i];
      }
    }
  }
}

// C[r, :] = sum over z in order of P[z][r, :], for the rows * n outputs
__global__ void split_sum(const float *P, float *C, size_t n, long stride, int S) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float s = P[i];
  for (int z = 1; z < S; ++z) s += P[(size_t)z * stride + i];
  C[i] = s;
}

unsigned blocks(size_t n, int per) { return (unsigned)((n + per - 1) / per); }

// Few rows per expert: the expert products are weight streams; 16-row tiles
// waste less work than 64-row ones.
bool skinny_rows(int rows, int E) { return rows <= 32 * E; }

// Reduction chunks for a skinny expert product whose waves cover `cols`
// columns: enough (row tile, column tile, chunk) waves to keep the weight
// stream busy (about kWaves, assuming the rows spread over min(rows, E)
// experts), chunks of whole 64-deep steps and at least 128 deep, at most 32.
struct SplitPlan {
  int S, chunk;
};
SplitPlan split_plan(int rows, int E, int N, int K, int cols) {
  const long tiles = (long)((N + cols - 1) / cols) * std::max(1, std::min(rows, E)) *
                     ((std::max(1, rows / std::max(E, 1)) + kSkinnyRows - 1) / kSkinnyRows);
  constexpr long kWaves = 4096;
  int S = (int)std::min<long>(32, std::max<long>(1, (kWaves + tiles - 1) / tiles));
  S = std::max(1, std::min(S, K / 128));
  const int chunk = ((K + S - 1) / S + 63) / 64 * 64;
  return SplitPlan{chunk > 0 ? (K + chunk - 1) / chunk : 1, chunk};
}

// ---- 1. stable permutation --------------------------------------------------
// One workgroup of 1024 threads; wave w owns the slot range [w L, (w+1) L).
// Per-wave histograms give each wave its first row inside every expert; each
// wave then ranks its slots in slot order (ballots over 64-slot chunks), so
// the rows of an expert are its slots in increasing order.
constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / 64;

// Expert counts -> counts, offsets and the tile prefix (exclusive offsets
// returned for tid < E).  One workgroup of kPermThreads; `total` is the
// expert's count (tid < E), 0 elsewhere.
__device__ __forceinline__ int perm_scan(const BackwardArgs &a, int total, int (*wsum)[2]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tiles = tid < a.E ? (total + a.tile_rows - 1) / a.tile_rows : 0;
  int v0 = total, v1 = tiles;  // inclusive scans of (count, tiles) over experts
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int p0 = __shfl_up(v0, off, 64), p1 = __shfl_up(v1, off, 64);
    if (lane >= off) {
      v0 += p0;
      v1 += p1;
    }
  }
  if (lane == 63) {
    wsum[wave][0] = v0;
    wsum[wave][1] = v1;
  }
  __syncthreads();
  for (int w = 0; w < wave; ++w) {
    v0 += wsum[w][0];
    v1 += wsum[w][1];
  }
  if (tid < a.E) {
    a.counts[tid] = total;
    a.offsets[tid] = v0 - total;
    a.mtile_prefix[tid + 1] = v1;
    if (tid == 0) a.mtile_prefix[0] = 0;
    if (tid == a.E - 1) a.offsets[a.E] = v0;
  }
  return v0 - total;
}

// Rows of the 64 slots [c0, c0 + 64) ∩ [.., s1) of one wavefront, in slot
// order within each expert: base[e] is the wave's first row of expert e
// (LDS) and advances past the wave's slots of e.
__device__ __forceinline__ void perm_rank_chunk(const BackwardArgs &a, int c0, int s1, int *base) {
  const int lane = threadIdx.x & 63;
  const int s = c0 + lane;
  const bool valid = s < s1;
  const int id = valid ? clamp_id(a.indices[s], a.E) : -1;
  uint64_t left = __ballot(valid);
  while (left) {
    const int leader = __ffsll((unsigned long long)left) - 1;
    const int lid = __builtin_amdgcn_readlane(id, leader);
    const uint64_t m = __ballot(valid && id == lid);
    if (valid && id == lid) {
      const int row = base[lid] + __popcll(m & ((1ull << lane) - 1ull));
      a.row_slot[row] = s;
      a.row_token[row] = s / a.K;
      a.row_expert[row] = lid;
      a.slot_row[s] = row;
    }
    left &= ~m;
    if (lane == leader) base[lid] += __popcll(m);
  }
}

// Stable expert-sorted order of the slots (rows of an expert in slot order),
// one workgroup: each wave counts and ranks a contiguous range of slots.
__global__ __launch_bounds__(kPermThreads) void stable_permute(BackwardArgs a) {
  extern __shared__ int hist[];  // [kPermWaves][E]: counts, then each wave's first row
  __shared__ int wsum[kPermWaves][2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = a.T * a.K;
  const int L = (n + kPermWaves - 1) / kPermWaves;
  for (int i = tid; i < kPermWaves * a.E; i += kPermThreads) hist[i] = 0;
  __syncthreads();
  const int s0 = wave * L, s1 = min(n, s0 + L);
  for (int s = s0 + lane; s < s1; s += 64) atomicAdd(&hist[wave * a.E + clamp_id(a.indices[s], a.E)], 1);
  __syncthreads();
  int total = 0;
  if (tid < a.E) {  // each wave's first row within the expert
    for (int w = 0; w < kPermWaves; ++w) {
      const int c = hist[w * a.E + tid];
      hist[w * a.E + tid] = total;
      total += c;
    }
  }
  const int off = perm_scan(a, total, wsum);
  if (tid < a.E)
    for (int w = 0; w < kPermWaves; ++w) hist[w * a.E + tid] += off;
  __syncthreads();
  for (int c0 = s0; c0 < s1; c0 += 64) perm_rank_chunk(a, c0, s1, hist + wave * a.E);
}

// The same order for many slots, in three launches over blocks of
// kPermThreads slots: (1) each block's expert counts; (2) one workgroup:
// counts, offsets, tile prefix and each block's first row per expert (the
// blocks in slot order); (3) each block ranks its slots, a wave per 64.
__global__ __launch_bounds__(kPermThreads) void perm_block_counts(BackwardArgs a) {
  extern __shared__ int h[];  // [E]
  const int tid = threadIdx.x, n = a.T * a.K;
  for (int i = tid; i < a.E; i += kPermThreads) h[i] = 0;
  __syncthreads();
  const int s = blockIdx.x * kPermThreads + tid;
  if (s < n) atomicAdd(&h[clamp_id(a.indices[s], a.E)], 1);
  __syncthreads();
  for (int i = tid; i < a.E; i += kPermThreads) a.blk[(size_t)blockIdx.x * a.E + i] = h[i];
}

__global__ __launch_bounds__(kPermThreads) void perm_block_scan(BackwardArgs a, int nb) {
  __shared__ int wsum[kPermWaves][2];
  const int tid = threadIdx.x;
  int *col = a.blk + tid;  // this expert's count of each block, E apart
  int total = 0;
  if (tid < a.E)
    for (int b = 0; b < nb; ++b) total += col[(size_t)b * a.E];
  const int off = perm_scan(a, total, wsum);
  if (tid < a.E) {  // each block's first row of the expert, in batches of loads
    int run = off;
    for (int b0 = 0; b0 < nb; b0 += 8) {
      int c[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = b0 + j < nb ? col[(size_t)(b0 + j) * a.E] : 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (b0 + j < nb) col[(size_t)(b0 + j) * a.E] = run;
        run += c[j];
      }
    }
  }
}

__global__ __launch_bounds__(kPermThreads) void perm_block_rank(BackwardArgs a) {
  extern __shared__ int hist[];  // [kPermWaves][E]: counts, then each wave's first row
  const int tid = threadIdx.x, wave = tid >> 6;
  const int n = a.T * a.K;
  for (int i = tid; i < kPermWaves * a.E; i += kPermThreads) hist[i] = 0;
  __syncthreads();
  const int s = blockIdx.x * kPermThreads + tid;
  if (s < n) atomicAdd(&hist[wave * a.E + clamp_id(a.indices[s], a.E)], 1);
  __syncthreads();
  if (tid < a.E) {
    int base = a.blk[(size_t)blockIdx.x * a.E + tid];
    for (int w = 0; w < kPermWaves; ++w) {
      const int c = hist[w * a.E + tid];
      hist[w * a.E + tid] = base;
      base += c;
    }
  }
  __syncthreads();
  const int c0 = blockIdx.x * kPermThreads + wave * 64;
  perm_rank_chunk(a, c0, n, hist + wave * a.E);
}

// ---- 2. routing weights per slot (the forward's arithmetic) ------------------
__global__ void slot_weights(BackwardArgs a) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= a.T) return;
  float tot = 0.f;
  for (int k = 0; k < a.K; ++k) tot += a.scores[(size_t)t * a.E + clamp_id(a.indices[t * a.K + k], a.E)];
  for (int k = 0; k < a.K; ++k) {
    const float s = a.scores[(size_t)t * a.E + clamp_id(a.indices[t * a.K + k], a.E)];
    a.slot_w[t * a.K + k] = a.norm ? (s / (tot + 1e-20f)) * a.route_scale : s * a.route_scale;
  }
}

__global__ void rows_weight(BackwardArgs a) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < a.T * a.K) a.row_w[r] = a.slot_w[a.row_slot[r]];
}

// ---- 3. SwiGLU (and the pre-activation bias) --------------------------------
// pre [rows, 2I] gets the per-group bias added in place; h [rows, I].
// group = row_expert[r] (routed) or 0 (shared: one group, no bias).
__global__ void swiglu_fwd(float *pre, float *h, const int32_t *row_group, const void *bias, int bias_bf16,
                           int rows, int I, float limit, int act) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)rows * I) return;
  const size_t r = i / I, j = i - r * I;
  float g = pre[r * 2 * I + j], u = pre[r * 2 * I + I + j];
  if (bias) {
    const size_t e = row_group ? (size_t)row_group[r] : 0;
    g += ld_elem(bias, bias_bf16, e * 2 * I + j);
    u += ld_elem(bias, bias_bf16, e * 2 * I + I + j);
    pre[r * 2 * I + j] = g;
    pre[r * 2 * I + I + j] = u;
  }
  h[i] = swiglu_exact(g, u, limit, act);
}

// ---- 5. dpre = SwiGLU'(pre, w * gd) -------------------------------------------
// With s = sigma(a g') (a = 1, or 1.702 for swigluoai): d/dg' (g' s) =
// s (1 + a g' (1 - s)), times u' (or u' + 1); d/du' = g' s.  The clamp cuts
// the gradient where it binds (it passes on the boundary itself).
__global__ void swiglu_bwd(const float *pre, const float *gd, const float *row_scale, float *dpre, int rows, int I,
                           float limit, int act) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)rows * I) return;
  const size_t r = i / I, j = i - r * I;
  const float g = pre[r * 2 * I + j], u = pre[r * 2 * I + I + j];
  const float dh = (row_scale ? row_scale[r] : 1.f) * gd[i];
  const float gc = clamp_hi(g, limit), uc = clamp_sym(u, limit);
  const float al = act ? kOaiAlpha : 1.f;
  const float sg = 1.f / (1.f + expf(-al * gc));
  const float glu = gc * sg, dglu = sg * (1.f + al * gc * (1.f - sg));
  const float lin = act ? uc + 1.f : uc;
  dpre[r * 2 * I + j] = g <= limit ? dh * lin * dglu : 0.f;
  dpre[r * 2 * I + I + j] = (u >= -limit && u <= limit) ? dh * glu : 0.f;
}

// Row dot products, one wavefront per row, lanes strided then a fixed
// butterfly: out[r] = sum_i a[r, i] * b[r, i] (+ sum_h dout[tok(r), h] *
// bias[group(r), h] when bias is set).
__global__ void row_dots(const float *a, const float *b, int rows, int n, const void *dout, int dout_bf16,
                         const int32_t *row_token, const int32_t *row_group, const void *bias, int bias_bf16, int H,
                         float *out, const int32_t *out_index) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= rows) return;
  float s = 0.f;
  for (int i = lane; i < n; i += 64) s = fmaf(a[(size_t)r * n + i], b[(size_t)r * n + i], s);
  if (bias) {
    const size_t t = row_token ? (size_t)row_token[r] : (size_t)r, e = row_group ? (size_t)row_group[r] : 0;
    for (int h = lane; h < H; h += 64)
      s = fmaf(ld_elem(dout, dout_bf16, t * H + h), ld_elem(bias, bias_bf16, e * H + h), s);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane == 0) out[out_index ? out_index[r] : r] = s;
}

// ---- expert bias gradients: ordered sums over each expert's rows ------------
// db_down[e, h] = sum_r w_r dout[tok(r), h]; db_gate_up[e, j] = sum_r dpre[r, j]
__global__ void bias_grads(BackwardArgs a) {
  const int e = blockIdx.y;
  const int r0 = a.offsets[e], n = a.counts[e];
  const int H = a.H, I2 = 2 * a.I;
  for (int c = blockIdx.x * blockDim.x + threadIdx.x; c < H + I2; c += gridDim.x * blockDim.x) {
    float s = 0.f;
    if (c < H) {
      for (int r = r0; r < r0 + n; ++r)
        s = fmaf(a.row_w[r], ld_elem(a.dout, a.act_bf16, (size_t)a.row_token[r] * H + c), s);
      if (a.g.db_down) a.g.db_down[(size_t)e * H + c] = s;
    } else {
      const int j = c - H;
      for (int r = r0; r < r0 + n; ++r) s += a.dpre[(size_t)r * I2 + j];
      if (a.g.db_gate_up) a.g.db_gate_up[(size_t)e * I2 + j] = s;
    }
  }
}

// ---- 7. shared-expert gate: gamma, d gamma -> dz ------------------------------
// gamma_t = sigmoid(x_t . sh_gate) (the forward's gate, f32 dot in a fixed
// order); dz_t = (dout_t . sh_t) gamma (1 - gamma), dout_t . sh_t being
// gd_s[t] . h_s[t] (row_dots into dgam)
__global__ void shared_gamma(BackwardArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (t >= a.T) return;
  float s = 0.f;
  for (int h = lane; h < a.H; h += 64)
    s = fmaf(ld_elem(a.x, a.act_bf16, (size_t)t * a.H + h), ld_elem(a.sh_gate, a.act_bf16, h), s);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane == 0) a.gamma[t] = 1.f / (1.f + expf(-s));
}

__global__ void shared_dz(BackwardArgs a) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= a.T) return;
  const float g = a.gamma[t];
  a.dz[t] = a.dgam[t] * g * (1.f - g);
}

// ---- 8. router: d weights -> d scores -> d logits ----------------------------
// w_k = rs s_k / (S + eps): ds_j = rs dw_j / D - rs (sum_k dw_k s_k) / D^2,
// D = S + eps (or ds_j = rs dw_j without renormalisation).  Scores:
// softmax dl = s (ds - sum ds s); sigmoid ds s (1 - s); sqrt(softplus):
// ds sigma(l) / (2 s) with sigma(l) = 1 - exp(-softplus(l)) = 1 - exp(-s^2).
__global__ void router_bwd(BackwardArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (t >= a.T) return;
  const float *s = a.scores + (size_t)t * a.E;
  // selected scores and their d weights (K <= 16: every lane holds all)
  float S = 0.f, dws = 0.f;
  for (int k = 0; k < a.K; ++k) {
    const float sk = s[clamp_id(a.indices[t * a.K + k], a.E)];
    S += sk;
    dws = fmaf(a.dweights[t * a.K + k], sk, dws);
  }
  const float D = S + 1e-20f;
  float dot = 0.f;  // softmax: sum_e ds_e s_e (ds is zero off the selection)
  for (int k = 0; k < a.K; ++k) {
    const int e = clamp_id(a.indices[t * a.K + k], a.E);
    const float dw = a.dweights[t * a.K + k];
    const float ds = a.norm ? a.route_scale * dw / D - a.route_scale * dws / (D * D) : a.route_scale * dw;
    dot = fmaf(ds, s[e], dot);
  }
  for (int e = lane; e < a.E; e += 64) {
    float ds = 0.f;
    for (int k = 0; k < a.K; ++k)
      if (clamp_id(a.indices[t * a.K + k], a.E) == e) {
        const float dw = a.dweights[t * a.K + k];
        ds = a.norm ? a.route_scale * dw / D - a.route_scale * dws / (D * D) : a.route_scale * dw;
      }
    const float se = s[e];
    float dl;
    if (a.score_fn == 0) dl = se * (ds - dot);
    else if (a.score_fn == 1) dl = ds * se * (1.f - se);
    else dl = se > 0.f ? ds * (1.f - expf(-se * se)) / (2.f * se) : 0.f;
    a.dl[(size_t)t * a.E + e] = dl;
  }
}

// Column sums out[c] = sum_r w[r] m[r, c] (w = 1 when null) of a [rows, cols]
// matrix, f32 or bf16, in a fixed order and over many workgroups: the rows
// are cut into nch chunks; a workgroup of 4 x 64 threads takes 64 columns
// of one chunk, thread q summing rows q, q + 4, ... of it, and the four
// partial sums are added in q order (col_partials); then each column's
// chunk sums are added in chunk order (col_finish).  Used for
// drouter_bias[e] = sum_t dl[t, e] and dsh_gate[h] = sum_t dz[t] x[t, h].
constexpr int kColChunksMax = 64;

__global__ __launch_bounds__(256) void col_partials(const void *m, int bf16, const float *w, int rows, int cols,
                                                    int chunk, float *part) {
  __shared__ float red[4][64];
  const int l = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + l;
  const int r0 = blockIdx.y * chunk, r1 = min(rows, r0 + chunk);
  float s = 0.f;
  if (c < cols) {
    if (w) {
      for (int r = r0 + q; r < r1; r += 4) s = fmaf(w[r], ld_elem(m, bf16, (size_t)r * cols + c), s);
    } else {
      for (int r = r0 + q; r < r1; r += 4) s += ld_elem(m, bf16, (size_t)r * cols + c);
    }
  }
  red[q][l] = s;
  __syncthreads();
  if (q == 0 && c < cols) part[(size_t)blockIdx.y * cols + c] = ((red[0][l] + red[1][l]) + red[2][l]) + red[3][l];
}

__global__ void col_finish(const float *part, int nch, int cols, float *out) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= cols) return;
  float s = 0.f;
  for (int k = 0; k < nch; ++k) s += part[(size_t)k * cols + c];
  out[c] = s;
}

hipError_t column_sums(const void *m, int bf16, const float *w, int rows, int cols, float *part, float *out,
                       hipStream_t st) {
  const int nch = std::max(1, std::min(kColChunksMax, (rows + 63) / 64));
  const int chunk = (rows + nch - 1) / nch;
  hipLaunchKernelGGL(col_partials, dim3((cols + 63) / 64, nch), dim3(256), 0, st, m, bf16, w, rows, cols, chunk,
                     part);
  hipLaunchKernelGGL(col_finish, dim3(blocks(cols, 256)), dim3(256), 0, st, part, nch, cols, out);
  return hipGetLastError();
}

// ---- 9. dx --------------------------------------------------------------------
__global__ void dx_combine(BackwardArgs a) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)a.T * a.H) return;
  const size_t t = i / a.H, h = i - t * a.H;
  float s = 0.f;
  for (int k = 0; k < a.K; ++k) s += a.dx_rows[(size_t)a.slot_row[t * a.K + k] * a.H + h];
  if (a.dx_sh) s += a.dx_sh[i];
  s += a.dx_router[i];
  if (a.dz && a.sh_gate) s = fmaf(a.dz[t], ld_elem(a.sh_gate, a.act_bf16, h), s);
  a.g.dx[i] = s;
}

template <int AF, int BF>
void launch_mfma(const GGemm &g, dim3 grid, hipStream_t st) {
  if (g.vec) hipLaunchKernelGGL((grouped_gemm_mfma<AF, BF, true>), grid, dim3(256), 0, st, g);
  else hipLaunchKernelGGL((grouped_gemm_mfma<AF, BF, false>), grid, dim3(256), 0, st, g);
}
template <int AF>
void launch_b(const GGemm &g, dim3 grid, hipStream_t st) {
  switch (g.B.kmajor | g.B.bf16 << 1) {
    case 0: launch_mfma<AF, 0>(g, grid, st); break;
    case 1: launch_mfma<AF, 1>(g, grid, st); break;
    case 2: launch_mfma<AF, 2>(g, grid, st); break;
    default: launch_mfma<AF, 3>(g, grid, st); break;
  }
}
void launch_gemm(const GGemm &g, dim3 grid, hipStream_t st) {
  switch (g.A.kmajor | g.A.bf16 << 1) {
    case 0: launch_b<0>(g, grid, st); break;
    case 1: launch_b<1>(g, grid, st); break;
    case 2: launch_b<2>(g, grid, st); break;
    default: launch_b<3>(g, grid, st); break;
  }
}

// Whole 16-byte runs: both operands aligned, and the dimension each one runs
// along (k for a row-major operand, its rows for a k-major one) a multiple of
// 8.  The reduction length of a K-grouped product is only known on the device:
// there the operands must be k-major.
bool vec_runs(const GGemm &g) {
  auto one = [&](const GOp &o, int rows) {
    const int run = o.kmajor ? rows : (g.mode == 2 ? 1 : g.K);
    return o.vec && run % 8 == 0;
  };
  // rows of A in the row-grouped product vary by group
  return one(g.A, g.mode == 1 ? 1 : g.M) && one(g.B, g.N) && (g.ksplit <= 1 || g.kchunk % 8 == 0);
}

// Large tiles on the matrix cores, no split.  rows: M (mode 0), the rows of
// all groups together (mode 1), or each group's M (mode 2).
hipError_t gemm(GGemm g, int rows, hipStream_t st) {
  if (rows <= 0 || g.N <= 0) return hipSuccess;
  g.ksplit = 1; g.kchunk = 0; g.split_stride = 0;
  g.vec = vec_runs(g) ? 1 : 0;
  int grid_rows = (rows + kMT - 1) / kMT;
  if (g.mode == 1) grid_rows += g.E;  // a partial tile per group at most
  if (g.mode == 2) grid_rows *= g.E;
  launch_gemm(g, dim3((g.N + kMT - 1) / kMT, grid_rows), st);
  return hipGetLastError();
}

// The 16-row matrix-core kernel takes whole 16-byte runs, a row-major A, a
// plain weight operand B (no gather, scale or token rows) and 16-byte aligned
// output rows (the partial-product buffer is aligned).  Operands that pass
// the entry point's checks always qualify.
bool skinny_ok(GGemm g, const float *part) {
  g.ksplit = 1;
  return vec_runs(g) && !g.A.kmajor && !g.B.gather && !g.B.scale && !g.B.token_rows && g.ldc % 4 == 0 &&
         (reinterpret_cast<uintptr_t>(g.C) & 15) == 0 && (reinterpret_cast<uintptr_t>(part) & 15) == 0;
}

// Expert products (mode 1) over `rows` rows.  Skinny: 16-row tiles on the
// fp32 matrix cores, the reduction split as split_plan() says, the chunks'
// partial products in `part` and summed in chunk order into C.  Otherwise
// 128-row tiles on the bf16 matrix cores.
hipError_t expert_gemm(GGemm g, int rows, bool skinny, float *part, hipStream_t st) {
  if (!skinny) return gemm(g, rows, st);
  if (rows <= 0 || g.N <= 0) return hipSuccess;
  g.ksplit = 1;
  g.vec = vec_runs(g) ? 1 : 0;  // 1: skinny_ok() held
  const int cols = g.B.kmajor ? SkinnyShape<1>::cols : SkinnyShape<0>::cols;
  const SplitPlan sp = split_plan(rows, g.E, g.N, g.K, cols);
  float *C = g.C;
  g.ksplit = sp.S; g.kchunk = sp.chunk;
  g.split_stride = (long)rows * g.ldc;
  if (sp.S > 1) g.C = part;
  const dim3 grid((g.N + cols - 1) / cols, (rows + kSkinnyRows - 1) / kSkinnyRows + g.E, sp.S);
  switch (g.B.kmajor | g.A.bf16 << 1 | g.B.bf16 << 2) {
    case 0: hipLaunchKernelGGL((skinny_mfma_f32<0, 0, 0>), grid, dim3(64), 0, st, g); break;
    case 1: hipLaunchKernelGGL((skinny_mfma_f32<1, 0, 0>), grid, dim3(64), 0, st, g); break;
    case 2: hipLaunchKernelGGL((skinny_mfma_f32<0, 1, 0>), grid, dim3(64), 0, st, g); break;
    case 3: hipLaunchKernelGGL((skinny_mfma_f32<1, 1, 0>), grid, dim3(64), 0, st, g); break;
    case 4: hipLaunchKernelGGL((skinny_mfma_f32<0, 0, 1>), grid, dim3(64), 0, st, g); break;
    case 5: hipLaunchKernelGGL((skinny_mfma_f32<1, 0, 1>), grid, dim3(64), 0, st, g); break;
    case 6: hipLaunchKernelGGL((skinny_mfma_f32<0, 1, 1>), grid, dim3(64), 0, st, g); break;
    default: hipLaunchKernelGGL((skinny_mfma_f32<1, 1, 1>), grid, dim3(64), 0, st, g); break;
  }
  if (sp.S > 1) {
    const size_t n = (size_t)rows * g.ldc;
    hipLaunchKernelGGL(split_sum, dim3(blocks(n, 256)), dim3(256), 0, st, part, C, n, g.split_stride, sp.S);
  }
  return hipGetLastError();
}

GOp op(const void *p, bool bf16, bool kmajor, long ld, long gstride = 0, bool token_rows = false,
       const int32_t *gather = nullptr, const float *scale = nullptr) {
  // 16-byte runs need the base, every row start and every group start on a
  // 16-byte boundary
  const long per = bf16 ? 8 : 4;
  const bool vec = (reinterpret_cast<uintptr_t>(p) & 15) == 0 && ld % per == 0 && gstride % per == 0;
  return GOp{p, bf16 ? 1 : 0, kmajor ? 1 : 0, token_rows ? 1 : 0, vec ? 1 : 0, ld, gstride, gather, scale};
}

}  // namespace

size_t backward_layout(int T, int K, int E, int H, int I, int Is, BackwardArgs *a, char *ws) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char *p = ws ? ws + off : nullptr;
    off += (bytes + 255) & ~(size_t)255;
    return p;
  };
  const size_t rows = (size_t)T * K;
  BackwardArgs b{};
  b.row_slot = reinterpret_cast<int32_t *>(take(rows * 4));
  b.row_token = reinterpret_cast<int32_t *>(take(rows * 4));
  b.row_expert = reinterpret_cast<int32_t *>(take(rows * 4));
  b.slot_row = reinterpret_cast<int32_t *>(take(rows * 4));
  b.counts = reinterpret_cast<int32_t *>(take((size_t)E * 4));
  b.offsets = reinterpret_cast<int32_t *>(take((size_t)(E + 1) * 4));
  b.mtile_prefix = reinterpret_cast<int32_t *>(take((size_t)(E + 1) * 4));
  b.blk = reinterpret_cast<int32_t *>(take((rows + kPermThreads - 1) / kPermThreads * (size_t)E * 4));
  b.slot_w = reinterpret_cast<float *>(take(rows * 4));
  b.row_w = reinterpret_cast<float *>(take(rows * 4));
  b.pre = reinterpret_cast<float *>(take(rows * 2 * I * 4));
  b.hact = reinterpret_cast<float *>(take(rows * I * 4));
  b.gd = reinterpret_cast<float *>(take(rows * I * 4));
  b.dpre = reinterpret_cast<float *>(take(rows * 2 * I * 4));
  b.dx_rows = reinterpret_cast<float *>(take(rows * H * 4));
  b.dweights = reinterpret_cast<float *>(take(rows * 4));
  b.dl = reinterpret_cast<float *>(take((size_t)T * E * 4));
  b.colpart = reinterpret_cast<float *>(take((size_t)kColChunksMax * std::max(H, E) * 4));
  if (skinny_rows((int)rows, E)) {
    size_t part = 0;
    const int nk[3][2] = {{2 * I, H}, {I, H}, {H, 2 * I}};  // pre, gd, dx_rows
    const int cols[3] = {SkinnyShape<0>::cols, SkinnyShape<1>::cols, SkinnyShape<1>::cols};  // B layouts
    for (int i = 0; i < 3; ++i) {
      const SplitPlan sp = split_plan((int)rows, E, nk[i][0], nk[i][1], cols[i]);
      if (sp.S > 1) part = std::max(part, (size_t)sp.S * rows * nk[i][0] * 4);
    }
    b.part = reinterpret_cast<float *>(take(part));
  }
  b.dx_router = reinterpret_cast<float *>(take((size_t)T * H * 4));
  if (Is > 0) {
    b.pre_s = reinterpret_cast<float *>(take((size_t)T * 2 * Is * 4));
    b.hact_s = reinterpret_cast<float *>(take((size_t)T * Is * 4));
    b.gd_s = reinterpret_cast<float *>(take((size_t)T * Is * 4));
    b.dpre_s = reinterpret_cast<float *>(take((size_t)T * 2 * Is * 4));
    b.dx_sh = reinterpret_cast<float *>(take((size_t)T * H * 4));
    b.gamma = reinterpret_cast<float *>(take((size_t)T * 4));
    b.dgam = reinterpret_cast<float *>(take((size_t)T * 4));
    b.dz = reinterpret_cast<float *>(take((size_t)T * 4));
  }
  if (a) {
    // keep the caller's inputs, outputs and sizes; fill in the scratch
    BackwardArgs c = *a;
    c.row_slot = b.row_slot; c.row_token = b.row_token; c.row_expert = b.row_expert; c.slot_row = b.slot_row;
    c.counts = b.counts; c.offsets = b.offsets; c.mtile_prefix = b.mtile_prefix; c.blk = b.blk; c.part = b.part;
    c.slot_w = b.slot_w; c.row_w = b.row_w; c.pre = b.pre; c.hact = b.hact; c.gd = b.gd; c.dpre = b.dpre;
    c.dx_rows = b.dx_rows; c.dweights = b.dweights; c.dl = b.dl; c.colpart = b.colpart; c.dx_router = b.dx_router;
    c.pre_s = b.pre_s; c.hact_s = b.hact_s; c.gd_s = b.gd_s; c.dpre_s = b.dpre_s; c.dx_sh = b.dx_sh;
    c.gamma = b.gamma; c.dgam = b.dgam; c.dz = b.dz;
    if (!c.sh_gate) c.dz = nullptr;
    *a = c;
  }
  return off;
}

hipError_t launch_backward(const BackwardArgs &a, hipStream_t st) {
#define BW_TRY(x)                         \
  do {                                    \
    const hipError_t e_ = (x);            \
    if (e_ != hipSuccess) return e_;      \
  } while (0)
  const int T = a.T, K = a.K, E = a.E, H = a.H, I = a.I, Is = a.Is;
  const int rows = T * K;
  const bool ab = a.act_bf16, wb = a.w_bf16;
  const float lim = a.limit;

  // the three expert products: pre = x_rows Wgu^T, gd = dout_rows Wd,
  // dx_rows = dpre Wgu
  GGemm g1{}, g2{}, g3{};
  for (GGemm *g : {&g1, &g2, &g3}) {
    g->mode = 1; g->E = E; g->counts = a.counts; g->offsets = a.offsets; g->mtile_prefix = a.mtile_prefix;
  }
  g1.A = op(a.x, ab, false, H, 0, true, a.row_token);
  g1.B = op(a.w_gate_up, wb, false, H, (long)2 * I * H);
  g1.C = a.pre; g1.ldc = 2 * I; g1.N = 2 * I; g1.K = H;
  g2.A = op(a.dout, ab, false, H, 0, true, a.row_token);
  g2.B = op(a.w_down, wb, true, I, (long)H * I);
  g2.C = a.gd; g2.ldc = I; g2.N = I; g2.K = H;
  g3.A = op(a.dpre, false, false, 2 * I, 0, true);
  g3.B = op(a.w_gate_up, wb, true, H, (long)2 * I * H);
  g3.C = a.dx_rows; g3.ldc = H; g3.N = H; g3.K = 2 * I;
  const bool skinny = skinny_rows(rows, E) && skinny_ok(g1, a.part) && skinny_ok(g2, a.part) && skinny_ok(g3, a.part);
  // 1-2. permutation and weights
  BackwardArgs pa = a;
  pa.tile_rows = skinny ? kSkinnyRows : kMT;
  const int nb = (rows + kPermThreads - 1) / kPermThreads;
  if (nb <= 1) {
    hipLaunchKernelGGL(stable_permute, dim3(1), dim3(kPermThreads), (size_t)kPermWaves * E * 4, st, pa);
  } else {
    hipLaunchKernelGGL(perm_block_counts, dim3(nb), dim3(kPermThreads), (size_t)E * 4, st, pa);
    hipLaunchKernelGGL(perm_block_scan, dim3(1), dim3(kPermThreads), 0, st, pa, nb);
    hipLaunchKernelGGL(perm_block_rank, dim3(nb), dim3(kPermThreads), (size_t)kPermWaves * E * 4, st, pa);
  }
  BW_TRY(hipGetLastError());
  hipLaunchKernelGGL(slot_weights, dim3(blocks(T, 256)), dim3(256), 0, st, a);
  hipLaunchKernelGGL(rows_weight, dim3(blocks(rows, 256)), dim3(256), 0, st, a);
  BW_TRY(hipGetLastError());

  // 3. pre = x_rows Wgu^T, h = SwiGLU(pre + b)
  BW_TRY(expert_gemm(g1, rows, skinny, a.part, st));
  hipLaunchKernelGGL(swiglu_fwd, dim3(blocks((size_t)rows * I, 256)), dim3(256), 0, st, a.pre, a.hact, a.row_expert,
                     a.b_gate_up, ab ? 1 : 0, rows, I, lim, a.act);
  // 4. gd = dout_rows Wd
  BW_TRY(expert_gemm(g2, rows, skinny, a.part, st));
  // 5. dweights (slot order) and dpre
  hipLaunchKernelGGL(row_dots, dim3(blocks(rows, 4)), dim3(256), 0, st, a.gd, a.hact, rows, I, a.dout, ab ? 1 : 0,
                     a.row_token, a.row_expert, a.b_down, ab ? 1 : 0, H, a.dweights, a.row_slot);
  hipLaunchKernelGGL(swiglu_bwd, dim3(blocks((size_t)rows * I, 256)), dim3(256), 0, st, a.pre, a.gd, a.row_w, a.dpre,
                     rows, I, lim, a.act);
  BW_TRY(hipGetLastError());
  // 6. dx_rows = dpre Wgu; dWd = sum_r (w dout)^T h; dWgu = sum_r dpre^T x
  BW_TRY(expert_gemm(g3, rows, skinny, a.part, st));
  GGemm w{};
  w.mode = 2; w.E = E; w.counts = a.counts; w.offsets = a.offsets;
  w.A = op(a.dout, ab, true, H, 0, true, a.row_token, a.row_w);
  w.B = op(a.hact, false, true, I, 0, true);
  w.C = a.g.dw_down; w.ldc = I; w.cgstride = (long)H * I; w.M = H; w.N = I;
  BW_TRY(gemm(w, H, st));
  w.A = op(a.dpre, false, true, 2 * I, 0, true);
  w.B = op(a.x, ab, true, H, 0, true, a.row_token);
  w.C = a.g.dw_gate_up; w.ldc = H; w.cgstride = (long)2 * I * H; w.M = 2 * I; w.N = H;
  BW_TRY(gemm(w, 2 * I, st));
  if (a.g.db_down || a.g.db_gate_up) {
    hipLaunchKernelGGL(bias_grads, dim3(blocks(H + 2 * I, 256), E), dim3(256), 0, st, a);
    BW_TRY(hipGetLastError());
  }

  // 7. shared expert over all tokens (gamma = 1 when ungated)
  if (Is > 0) {
    GGemm s{};
    s.mode = 0; s.M = T;
    s.A = op(a.x, ab, false, H);
    s.B = op(a.sh_gate_up, ab, false, H);
    s.C = a.pre_s; s.ldc = 2 * Is; s.N = 2 * Is; s.K = H;
    BW_TRY(gemm(s, T, st));
    hipLaunchKernelGGL(swiglu_fwd, dim3(blocks((size_t)T * Is, 256)), dim3(256), 0, st, a.pre_s, a.hact_s,
                       (const int32_t *)nullptr, (const void *)nullptr, 0, T, Is, lim, a.act);
    s.A = op(a.dout, ab, false, H);
    s.B = op(a.sh_down, ab, true, Is);
    s.C = a.gd_s; s.ldc = Is; s.N = Is; s.K = H;
    BW_TRY(gemm(s, T, st));
    const float *gam = nullptr;
    if (a.sh_gate) {
      hipLaunchKernelGGL(shared_gamma, dim3(blocks(T, 4)), dim3(256), 0, st, a);
      hipLaunchKernelGGL(row_dots, dim3(blocks(T, 4)), dim3(256), 0, st, a.gd_s, a.hact_s, T, Is, (const void *)nullptr,
                         0, (const int32_t *)nullptr, (const int32_t *)nullptr, (const void *)nullptr, 0, H, a.dgam,
                         (const int32_t *)nullptr);
      hipLaunchKernelGGL(shared_dz, dim3(blocks(T, 256)), dim3(256), 0, st, a);
      BW_TRY(hipGetLastError());
      gam = a.gamma;
    }
    hipLaunchKernelGGL(swiglu_bwd, dim3(blocks((size_t)T * Is, 256)), dim3(256), 0, st, a.pre_s, a.gd_s, gam, a.dpre_s,
                       T, Is, lim, a.act);
    s.A = op(a.dpre_s, false, false, 2 * Is);
    s.B = op(a.sh_gate_up, ab, true, H);
    s.C = a.dx_sh; s.ldc = H; s.N = H; s.K = 2 * Is;
    BW_TRY(gemm(s, T, st));
    s.M = H; s.K = T;
    s.A = op(a.dout, ab, true, H, 0, false, nullptr, gam);
    s.B = op(a.hact_s, false, true, Is);
    s.C = a.g.dsh_down; s.ldc = Is; s.N = Is;
    BW_TRY(gemm(s, H, st));
    s.M = 2 * Is;
    s.A = op(a.dpre_s, false, true, 2 * Is);
    s.B = op(a.x, ab, true, H);
    s.C = a.g.dsh_gate_up; s.ldc = H; s.N = H;
    BW_TRY(gemm(s, 2 * Is, st));
    if (a.sh_gate) BW_TRY(column_sums(a.x, ab ? 1 : 0, a.dz, T, H, a.colpart, a.g.dsh_gate, st));
  }

  // 8. router
  hipLaunchKernelGGL(router_bwd, dim3(blocks(T, 4)), dim3(256), 0, st, a);
  BW_TRY(hipGetLastError());
  GGemm r{};
  r.mode = 0;
  r.M = E; r.N = H; r.K = T;
  r.A = op(a.dl, false, true, E);
  r.B = op(a.x, ab, true, H);
  r.C = a.g.dgate; r.ldc = H;
  BW_TRY(gemm(r, E, st));
  r.M = T; r.N = H; r.K = E;
  r.A = op(a.dl, false, false, E);
  r.B = op(a.gate_w, ab, true, H);
  r.C = a.dx_router; r.ldc = H;
  BW_TRY(gemm(r, T, st));
  if (a.g.drouter_bias) BW_TRY(column_sums(a.dl, 0, nullptr, T, E, a.colpart, a.g.drouter_bias, st));

  // 9. dx
  hipLaunchKernelGGL(dx_combine, dim3(blocks((size_t)T * H, 256)), dim3(256), 0, st, a);
  return hipGetLastError();
#undef BW_TRY
}

}  // namespace moe
