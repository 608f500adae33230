// Newton-Schulz orthogonalisation (a2-a5) on CDNA4 matrix cores.
//
// One iteration is three products ("NVIDIA Megatron..." article, paragraph
// 「分散モード」): A = X X^T, B = b A + c A A, X' = a X + B X.  The first two
// are symmetric rank-k products (paragraph 「SYRK と融合された all-reduce」):
// only tiles on or below the diagonal are computed, and each off-diagonal
// tile is also stored mirrored, so A and B are full symmetric matrices.
//
// Working layout: X is [batch][s][l] with s <= l (a tall momentum is
// transposed once by the normalisation kernel), A and B are [batch][s][s];
// s and l are padded to multiples of MUON_NS_PAD with zeros, and zeros stay
// zeros through every product, so the GEMM kernels never test bounds.
//
// GEMM kernel: C = alpha * P Q^T (+ beta * Z) where P's rows and Q's rows
// are contiguous along k ("NT"), or Q is given k-major ("NN", the B X
// product).  Tiles are staged in LDS as 128-byte rows (64 bf16 / 32 fp32
// along k) with an XOR swizzle of the 16-byte chunks so that both the tile
// stores and the MFMA fragment reads are free of bank conflicts; the NN
// loader transposes 8x8 (bf16) or 4x4 (fp32) blocks in registers so that its
// LDS tile has the same k-contiguous layout.  bf16 uses
// v_mfma_f32_32x32x16_bf16, fp32 uses v_mfma_f32_32x32x2f32; both accumulate
// in fp32.
#include <math.h>

#include <algorithm>
#include <cmath>
#include <vector>

#include "common.h"
#include "gemm.h"

namespace muon {

// one launch of sign_pack for evenly spaced equal problems (elementwise.hip)
int sign_pack_runs(const void* U, int u_dtype, int64_t numel, int64_t count, int64_t strideU, uint64_t* bits,
                   int64_t stride_bits, hipStream_t st);

int sumsq_strided(const void* M, int m_dtype, int64_t len, int64_t count, int64_t stride, float* out,
                  void* partials, hipStream_t stream);

namespace {

using gemm::EPI_AXPBY;
using gemm::EPI_FINAL;
using gemm::EPI_STORE;
using gemm::GemmArgs;

// ---------------------------------------------------------------------------
// a2: X0 = pad(orient(M)) * scale, scale = 1/sqrt(sumsq) (0 for a zero matrix).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float frobenius_scale(const float* sumsq, int64_t b, int64_t stride) {
  const double ss = static_cast<double>(sumsq[b * stride]);
  return ss == 0.0 ? 0.0f : static_cast<float>(1.0 / sqrt(ss));
}

// Wide matrix (rows <= cols): one thread writes 8 consecutive entries of a
// working row; with `vec` (cols and the batch stride multiples of 8) full
// groups are read and written as vectors.
template <typename TM, typename TX>
__global__ __launch_bounds__(256) void normalize_kernel(const TM* __restrict__ M, int64_t strideM,
                                                       int64_t rows, int64_t cols,
                                                       const float* __restrict__ sumsq,
                                                       int64_t stride_sumsq, TX* __restrict__ X,
                                                       int64_t sp, int64_t lp, int vec) {
  const int64_t b = blockIdx.y;
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t per_row = lp / 8;
  if (t >= sp * per_row) return;
  const int64_t i = t / per_row, j0 = (t % per_row) * 8;
  const float scale = frobenius_scale(sumsq, b, stride_sumsq);
  const TM* src = M + b * strideM + i * cols + j0;
  TX* dst = X + b * sp * lp + i * lp + j0;
  float v[8];
  if (i < rows && j0 + 8 <= cols && vec) {
    Vec8<TM>::load(src, v);
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] *= scale;
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = (i < rows && j0 + q < cols) ? to_f32(src[q]) * scale : 0.0f;
  }
  Vec8<TX>::store(dst, v);
}

// Tall matrix (rows > cols): X0 = M^T, transposed through LDS one 64 x 64 tile
// at a time so that both the reads (along M's rows) and the writes (along
// X's rows) are coalesced.  With VEC (cols and strideM multiples of 8, M
// 16-byte aligned) every lane moves 8 consecutive entries per access: M in
// whole 8-entry groups, each inside or outside the matrix; X's rows are
// padded to multiples of 256, so its 8-entry groups are always whole.
template <typename TM, typename TX, bool VEC>
__global__ __launch_bounds__(256) void normalize_tall_kernel(const TM* __restrict__ M, int64_t strideM,
                                                            int64_t rows, int64_t cols,
                                                            const float* __restrict__ sumsq,
                                                            int64_t stride_sumsq, TX* __restrict__ X,
                                                            int64_t sp, int64_t lp) {
  __shared__ float tile[64][65];
  const int64_t b = blockIdx.z;
  const int64_t i0 = int64_t(blockIdx.y) * 64;   // X rows = M columns
  const int64_t j0 = int64_t(blockIdx.x) * 64;   // X columns = M rows
  const float scale = frobenius_scale(sumsq, b, stride_sumsq);
  const TM* Mb = M + b * strideM;
  TX* Xb = X + b * sp * lp;
  if constexpr (VEC) {
    // thread t: row t / 8 (+ 32) of the tile, entries 8 (t % 8) .. + 7
    const int q = threadIdx.x & 7, r0 = threadIdx.x >> 3;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = r0 + 32 * h;
      const int64_t mr = j0 + r, mc = i0 + 8 * q;
      float v[8];
      if (mr < rows && mc < cols) {
        Vec8<TM>::load(Mb + mr * cols + mc, v);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[r][8 * q + e] = v[e] * scale;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = r0 + 32 * h;   // X row i0 + r, columns j0 + 8 q .. + 7
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = tile[8 * q + e][r];
      Vec8<TX>::store(Xb + (i0 + r) * lp + j0 + 8 * q, v);
    }
  } else {
    const int c = threadIdx.x & 63;
    for (int r = threadIdx.x >> 6; r < 64; r += 4) {
      const int64_t mr = j0 + r, mc = i0 + c;
      tile[r][c] = (mr < rows && mc < cols) ? to_f32(Mb[mr * cols + mc]) * scale : 0.0f;
    }
    __syncthreads();
    for (int r = threadIdx.x >> 6; r < 64; r += 4) Xb[(i0 + r) * lp + j0 + c] = from_f32<TX>(tile[c][r]);
  }
}

// steps == 0: U = X0 (un-padded, original orientation)
template <typename TX, typename TU>
__global__ __launch_bounds__(256) void emit_kernel(const TX* __restrict__ X, int64_t sp, int64_t lp,
                                                  int64_t rows, int64_t cols, TU* __restrict__ U,
                                                  int64_t strideU) {
  const int64_t b = blockIdx.y;
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t >= rows * cols) return;
  const int64_t r = t / cols, c = t % cols;
  const bool tall = rows > cols;
  const int64_t i = tall ? c : r, j = tall ? r : c;
  U[b * strideU + t] = from_f32<TU>(to_f32(X[b * sp * lp + i * lp + j]));
}

// ---------------------------------------------------------------------------
// Launch helpers
// ---------------------------------------------------------------------------
// bf16 products run the DMA-pipelined kernel with a 4-stage LDS ring.  Tile
// choice (measured on MI355X with the batched workloads' matrix sets): 256 x
// 256 tiles of 8 waves (64 x 128 each) for B X with K >= 1024 and for
// symmetric products with a side of at least 1024 (or a contraction long
// enough to split, K >= 8192); 128 x 128 tiles (8 waves of 32 x 64)
// otherwise: there a 256 x 256 grid leaves most CUs idle (a 768 side: 6 tiles
// per matrix) and prologue and epilogue weigh more than the smaller tiles'
// lower reuse.  128 x 1024^2: 4.96 -> 4.36 ms per orthogonalisation call;
// GPT-2-small layer set: 3.02 -> 2.30 ms, and 2.26 ms with the 128 x 128
// tiles on 8 waves instead of 4.  fp32 products (small,
// latency-bound workloads) use the register-staged kernel.
//
// The 256 x 256-tile symmetric products may split their work units
// (gemm::Split) when given scratch: long contractions whose n_p^2 units fit
// one round of the CUs.
constexpr bool big_tiles(bool syrk, int64_t K, int64_t M) { return syrk ? (M >= 1024 || K >= 8192) : K >= 1024; }

// B X on 256 x 256 tiles: when the last round of tiles would leave at least
// half of the CUs idle and those tiles form whole column strips, the strips
// run as a second launch of 128 x 256 tiles (twice the tiles at half the work
// each), so that round fills the CUs.  4096 x 14336: 768 tiles (three
// rounds of 256 CUs), then 256 tiles of 128 x 256 over the last 2048 columns.
template <int EPI>
int launch_apply_big(const GemmArgs& g, int64_t batch, hipStream_t st) {
  const gemm::Scratch none{nullptr, 0};
  const int64_t TM = g.M / 256, TN = g.N / 256, T = TM * TN;
  const int64_t cus = batch == 1 ? gemm::device_cus() : 0;
  int64_t ct = 0;   // 256-column strips run as 128 x 256 tiles
  if (cus > 0 && TM > 0) {
    const int64_t r = T % cus;
    if (r > 0 && 2 * r <= cus && r % TM == 0 && r / TM < TN) ct = r / TM;
  }
  if (ct == 0) return gemm::launch_dma<256, 256, 64, 128, 4, false, true, EPI>(g, batch, st, none);
  const int64_t n1 = (TN - ct) * 256;
  GemmArgs g1 = g;
  g1.ld = g.N;
  g1.N = n1;
  GemmArgs g2 = g;
  g2.ld = g.N;
  g2.N = ct * 256;
  g2.col0 = n1;
  g2.Q = static_cast<const bf16_t*>(g.Q) + n1;
  if (g.Z) g2.Z = static_cast<const bf16_t*>(g.Z) + n1;
  if (g.C) g2.C = static_cast<bf16_t*>(g.C) + n1;
  if (g.Zl) g2.Zl = static_cast<const bf16_t*>(g.Zl) + n1;
  if (g.Cl) g2.Cl = static_cast<bf16_t*>(g.Cl) + n1;
  // one launch when the whole-tile count keeps the XCD grouping (batch is 1 here)
  const int64_t whole = TM * (TN - ct);
  if (whole > 0 && whole % gemm::kXcds == 0) return gemm::launch_apply_mixed<EPI>(g1, g2, st);
  int status = gemm::launch_dma<256, 256, 64, 128, 4, false, true, EPI>(g1, batch, st, none);
  if (status != MUON_OK) return status;
  return gemm::launch_dma<128, 256, 64, 64, 4, false, true, EPI>(g2, batch, st, none);
}

// bf16 symmetric product with the addend (the polynomial) as column halves
// and diagonal lower halves: when its n_p^2 units per batch entry fit one
// round of the CUs (4096: 256 units for 256 CUs, against 136 whole tiles).
bool syrk_halves_fit(const GemmArgs& g, int64_t batch) {
  const int64_t np = g.M / 256, cus = gemm::device_cus();
  return np >= 2 && g.M % 256 == 0 && cus > 0 && np * np * batch <= cus;
}

template <typename T, bool SYRK, bool NN, int EPI>
int launch_gemm(const GemmArgs& g, int64_t batch, hipStream_t st, const gemm::Scratch& sc) {
  if constexpr (sizeof(T) == 2) {
    if constexpr (NN && !SYRK)
      if (big_tiles(SYRK, g.K, g.M)) return launch_apply_big<EPI>(g, batch, st);
    if constexpr (SYRK && EPI == EPI_AXPBY)
      if (big_tiles(SYRK, g.K, g.M) && syrk_halves_fit(g, batch)) return gemm::launch_syrk_halves<EPI>(g, batch, st);
    if (big_tiles(SYRK, g.K, g.M)) return gemm::launch_dma<256, 256, 64, 128, 4, SYRK, NN, EPI>(g, batch, st, sc);
    // 8 waves of 32 x 64: two per SIMD, and two workgroups per CU (74 KB of LDS each)
    return gemm::launch_dma<128, 128, 32, 64, 4, SYRK, NN, EPI>(g, batch, st, gemm::Scratch{nullptr, 0});
  } else {
    return gemm::launch<T, 128, 128, 64, 64, SYRK, NN, EPI>(g, batch, st);
  }
}

// Scratch that the bf16 products of one iteration on [batch][s][l] may use:
// the Gram's split plan (the polynomial, a contraction of s <= 4096 whenever
// n_p^2 units fit one round, never splits).
size_t split_scratch_bound(int64_t s, int64_t l, int64_t batch) {
  return gemm::split_scratch_bytes(gemm::plan_split<256, 256, true>(s, s, l, batch, 0).split_tiles, 256, 256);
}

__global__ __launch_bounds__(256) void zero_ints_kernel(int* __restrict__ p, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) p[i] = 0;
}

int zero_counters(void* base, int64_t n, hipStream_t st) {
  if (n <= 0) return MUON_OK;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
  launch_kernel(zero_ints_kernel, dim3(blocks), dim3(256), 0, st, static_cast<int*>(base), n);
  return launch_status();
}

// Frobenius scaling folded into the first iteration (bf16 only): the raw
// momentum M stands in for X0 = M / ||M||_F, the Gram is scaled by 1/sumsq
// and the product with M by 1/sqrt(sumsq).
struct Fold {
  const float* sumsq;     // null: X is already normalised
  int64_t stride_sumsq;
  int64_t strideX;        // batch stride of X (0: s * l)
};

template <typename T>
int gram_t(const void* X, void* A, int64_t s, int64_t l, int64_t batch, hipStream_t st,
           const gemm::Scratch& sc, const Fold& fold = Fold{}) {
  GemmArgs g{};
  g.P = X; g.Q = X; g.Z = nullptr; g.C = A;
  g.M = s; g.N = s; g.K = l;
  g.strideP = g.strideQ = fold.strideX ? fold.strideX : s * l; g.strideC = s * s;
  g.alpha = 1.0f; g.beta = 0.0f;
  g.scale_sumsq = fold.sumsq; g.stride_sumsq = fold.stride_sumsq; g.scale_mode = 1;
  return launch_gemm<T, true, false, EPI_STORE>(g, batch, st, sc);
}

template <typename T>
int poly_t(const void* A, void* B, int64_t s, int64_t batch, float b, float c, hipStream_t st,
           const gemm::Scratch& sc) {
  GemmArgs g{};
  g.P = A; g.Q = A; g.Z = A; g.C = B;
  g.M = s; g.N = s; g.K = s;
  g.strideP = g.strideQ = g.strideZ = g.strideC = s * s;
  g.alpha = c; g.beta = b;
  return launch_gemm<T, true, false, EPI_AXPBY>(g, batch, st, sc);
}

// Residual of X (bf16 products): X_lo_in, when set, is added to the addend
// a X; X_lo_out, when set, receives the rounding residual of the stored X'
// (not with final_out).  They may be one buffer.
template <typename T>
int apply_t(const void* B, const void* X, void* Xout, int64_t s, int64_t l, int64_t batch, float a,
            float alpha, hipStream_t st, const gemm::Scratch& sc, const GemmArgs* final_out,
            const Fold& fold = Fold{}, const GemmArgs* signs = nullptr, const void* X_lo_in = nullptr,
            void* X_lo_out = nullptr) {
  GemmArgs g{};
  if (final_out) g = *final_out;
  if (signs) {
    g.bits = signs->bits;
    g.bits_rows = signs->bits_rows;
    g.bits_cols = signs->bits_cols;
    g.stride_bits = signs->stride_bits;
  }
  g.P = B; g.Q = X; g.Z = X; g.C = Xout;
  g.Zl = X_lo_in;
  g.Cl = final_out ? nullptr : X_lo_out;
  g.M = s; g.N = l; g.K = s;
  g.strideP = s * s; g.strideQ = g.strideZ = fold.strideX ? fold.strideX : s * l; g.strideC = s * l;
  g.alpha = alpha; g.beta = a;
  g.scale_sumsq = fold.sumsq; g.stride_sumsq = fold.stride_sumsq; g.scale_mode = 2;
  if (final_out) return launch_gemm<T, false, true, EPI_FINAL>(g, batch, st, sc);
  return launch_gemm<T, false, true, EPI_AXPBY>(g, batch, st, sc);
}

template <typename TM, typename TX>
int normalize_t(const void* M, int64_t strideM, int64_t rows, int64_t cols, const float* sumsq,
                int64_t stride_sumsq, void* X, int64_t sp, int64_t lp, int64_t batch, hipStream_t st) {
  if (sp == 0 || lp == 0 || batch == 0) return MUON_OK;
  if (rows > cols) {
    const bool vec = cols % 8 == 0 && strideM % 8 == 0 && aligned16(M);
    auto kern = vec ? normalize_tall_kernel<TM, TX, true> : normalize_tall_kernel<TM, TX, false>;
    launch_kernel(kern, dim3(lp / 64, sp / 64, batch), dim3(256), 0, st, static_cast<const TM*>(M), strideM, rows,
                  cols, sumsq, stride_sumsq, static_cast<TX*>(X), sp, lp);
  } else {
    const int64_t blocks = (sp * (lp / 8) + 255) / 256;
    const int vec = cols % 8 == 0 && strideM % 8 == 0;
    launch_kernel(normalize_kernel<TM, TX>, dim3(blocks, batch), dim3(256), 0, st, 
        static_cast<const TM*>(M), strideM, rows, cols, sumsq, stride_sumsq, static_cast<TX*>(X), sp, lp,
        vec);
  }
  return launch_status();
}

int normalize_dispatch(const void* M, int m_dtype, int64_t strideM, int64_t rows, int64_t cols,
                       const float* sumsq, int64_t stride_sumsq, void* X, int precision, int64_t sp,
                       int64_t lp, int64_t batch, hipStream_t st) {
  if (precision == MUON_BF16) {
    if (m_dtype == MUON_BF16)
      return normalize_t<bf16_t, bf16_t>(M, strideM, rows, cols, sumsq, stride_sumsq, X, sp, lp, batch, st);
    return normalize_t<float, bf16_t>(M, strideM, rows, cols, sumsq, stride_sumsq, X, sp, lp, batch, st);
  }
  if (m_dtype == MUON_BF16)
    return normalize_t<bf16_t, float>(M, strideM, rows, cols, sumsq, stride_sumsq, X, sp, lp, batch, st);
  return normalize_t<float, float>(M, strideM, rows, cols, sumsq, stride_sumsq, X, sp, lp, batch, st);
}

template <typename TX>
int emit_t(const void* X, int64_t sp, int64_t lp, int64_t rows, int64_t cols, void* U, int u_dtype,
           int64_t strideU, int64_t batch, hipStream_t st) {
  const int64_t blocks = (rows * cols + 255) / 256;
  if (blocks == 0 || batch == 0) return MUON_OK;
  if (u_dtype == MUON_BF16)
    launch_kernel(emit_kernel<TX, bf16_t>, dim3(blocks, batch), dim3(256), 0, st, 
        static_cast<const TX*>(X), sp, lp, rows, cols, static_cast<bf16_t*>(U), strideU);
  else
    launch_kernel(emit_kernel<TX, float>, dim3(blocks, batch), dim3(256), 0, st, 
        static_cast<const TX*>(X), sp, lp, rows, cols, static_cast<float*>(U), strideU);
  return launch_status();
}

// ---------------------------------------------------------------------------
// Problem grouping: problems of equal shape and dtypes (in any order) are
// sorted by the address of M; runs of them whose M, U and sumsq pointers
// advance by a constant stride become one batched run.
// ---------------------------------------------------------------------------
struct Run {
  int count;
  const void* M;
  void* U;                 // null: only the signs are written
  const float* sumsq;
  uint64_t* bits;          // packed signs of U, or null
  int64_t rows, cols, sp, lp;
  int m_dtype, u_dtype;
  bool has_sumsq;
  int64_t strideM, strideU, stride_sumsq;  // elements
  int64_t stride_bits;                     // words
};

int64_t pad_to(int64_t x) { return (x + MUON_NS_PAD - 1) / MUON_NS_PAD * MUON_NS_PAD; }

bool same_kind(const muon_ns_problem& a, const muon_ns_problem& b) {
  return a.rows == b.rows && a.cols == b.cols && a.m_dtype == b.m_dtype && a.u_dtype == b.u_dtype &&
         (a.sumsq != nullptr) == (b.sumsq != nullptr) && (a.U != nullptr) == (b.U != nullptr) &&
         (a.bits != nullptr) == (b.bits != nullptr);
}

bool kind_less(const muon_ns_problem& a, const muon_ns_problem& b) {
  if (a.rows != b.rows) return a.rows < b.rows;
  if (a.cols != b.cols) return a.cols < b.cols;
  if (a.m_dtype != b.m_dtype) return a.m_dtype < b.m_dtype;
  if (a.u_dtype != b.u_dtype) return a.u_dtype < b.u_dtype;
  if ((a.sumsq != nullptr) != (b.sumsq != nullptr)) return a.sumsq == nullptr;
  if ((a.U != nullptr) != (b.U != nullptr)) return a.U == nullptr;
  if ((a.bits != nullptr) != (b.bits != nullptr)) return a.bits == nullptr;
  return reinterpret_cast<uintptr_t>(a.M) < reinterpret_cast<uintptr_t>(b.M);
}

int64_t diff_elems(const void* a, const void* b, size_t es) {
  const int64_t d = reinterpret_cast<const char*>(b) - reinterpret_cast<const char*>(a);
  if (d <= 0 || d % static_cast<int64_t>(es) != 0) return -1;
  return d / static_cast<int64_t>(es);
}

// stride of an optional pointer: both null gives 0 (no stride needed)
int64_t diff_opt(const void* a, const void* b, size_t es) {
  if (!a && !b) return 0;
  if (!a || !b) return -1;
  return diff_elems(a, b, es);
}

std::vector<Run> make_runs(const muon_ns_problem* probs, int count) {
  std::vector<muon_ns_problem> p(probs, probs + count);
  std::stable_sort(p.begin(), p.end(), kind_less);
  std::vector<Run> runs;
  int i = 0;
  while (i < count) {
    Run r{};
    r.count = 1;
    r.M = p[i].M; r.U = p[i].U; r.sumsq = p[i].sumsq; r.bits = p[i].bits;
    r.rows = p[i].rows; r.cols = p[i].cols;
    r.sp = pad_to(std::min(r.rows, r.cols));
    r.lp = pad_to(std::max(r.rows, r.cols));
    r.m_dtype = p[i].m_dtype; r.u_dtype = p[i].u_dtype;
    r.has_sumsq = p[i].sumsq != nullptr;
    r.strideM = r.strideU = r.rows * r.cols;
    r.stride_sumsq = 1;
    r.stride_bits = (r.rows * r.cols + 63) / 64;
    if (i + 1 < count && same_kind(p[i], p[i + 1])) {
      const int64_t sm = diff_elems(p[i].M, p[i + 1].M, dtype_size(r.m_dtype));
      const int64_t su = diff_opt(p[i].U, p[i + 1].U, dtype_size(r.u_dtype));
      const int64_t ss = r.has_sumsq ? diff_elems(p[i].sumsq, p[i + 1].sumsq, sizeof(float)) : 1;
      const int64_t sb = diff_opt(p[i].bits, p[i + 1].bits, sizeof(uint64_t));
      if (sm > 0 && su >= 0 && ss > 0 && sb >= 0) {
        int j = i + 1;
        while (j < count && same_kind(p[j - 1], p[j]) &&
               diff_elems(p[j - 1].M, p[j].M, dtype_size(r.m_dtype)) == sm &&
               diff_opt(p[j - 1].U, p[j].U, dtype_size(r.u_dtype)) == su &&
               (!r.has_sumsq || diff_elems(p[j - 1].sumsq, p[j].sumsq, sizeof(float)) == ss) &&
               diff_opt(p[j - 1].bits, p[j].bits, sizeof(uint64_t)) == sb)
          ++j;
        r.count = j - i;
        r.strideM = sm; r.strideU = su; r.stride_sumsq = ss;
        if (sb > 0) r.stride_bits = sb;
      }
    }
    runs.push_back(r);
    i += r.count;
  }
  return runs;
}

// bf16 products need a short side of at least kBf16MinSide.  Below it the
// rounding of B = bA + cA^2 alone puts 1.8e-2 to 2.4e-2 of relative error on a
// Gaussian 37 x 300 or 16 x 128 momentum (with or without residuals), so such
// problems run on the fp32 products; at these sizes they take microseconds
// either way.  From 96 up, Gaussian inputs stay at or below 1.4e-2.
constexpr int64_t kBf16MinSide = 96;

// the precision a problem's products actually run in
int run_precision(int64_t rows, int64_t cols, int precision) {
  return precision == MUON_BF16 && std::min(rows, cols) < kBf16MinSide ? MUON_F32 : precision;
}

struct RunLayout {
  size_t x0, x1, xl, a, b, sumsq, partials, total;
};

RunLayout layout_of(const Run& r, int requested) {
  const int precision = run_precision(r.rows, r.cols, requested);
  const size_t es = precision == MUON_BF16 ? 2 : 4;
  const size_t n = static_cast<size_t>(r.count);
  RunLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += round_up(bytes, 256); return o; };
  L.x0 = take(n * r.sp * r.lp * es);
  L.x1 = take(n * r.sp * r.lp * es);
  L.xl = take(precision == MUON_BF16 ? n * r.sp * r.lp * es : 0);
  L.a = take(n * r.sp * r.sp * es);
  L.b = take(n * r.sp * r.sp * es);
  L.sumsq = take(r.has_sumsq ? 0 : n * sizeof(float));
  size_t part = 0;
  if (!r.has_sumsq) {
    const int64_t len = r.rows * r.cols;
    part = r.strideM == len ? muon_momentum_workspace_bytes(len * r.count, r.count)
                            : muon_momentum_workspace_bytes(len, 1);
  }
  L.partials = take(part);
  L.total = off;
  return L;
}

// bf16 momentum already in the working layout (wide, sides multiples of
// MUON_NS_PAD, 16-byte aligned rows): no normalisation pass is needed
bool folds_normalisation(const Run& r, int precision) {
  return precision == MUON_BF16 && r.m_dtype == MUON_BF16 && r.rows <= r.cols &&
         r.rows % MUON_NS_PAD == 0 && r.cols % MUON_NS_PAD == 0 && r.strideM % 8 == 0;
}

// bf16 products: the outputs X_1 .. X_k of the first k iterations keep a bf16
// residual beside X (X + X_lo holds X to about 16 significant bits), which the
// next iteration adds to its addend a X.  Rounding X costs the most while the
// singular values are small: there the iteration grows them about a-fold,
// noise included, and the noise that rounding puts on the small directions is
// large next to them.  With the residual, the rounding error of X enters the
// next iterate through the slope of B X alone, p'(x) - a, instead of the whole
// slope p'(x) of x -> p(x) = a x + b x^3 + c x^5; that pays while p'(x) stays
// above a / 2, and costs a little once the singular values near the point
// where the iteration flattens out (for the quintic p'(x) falls to a / 2 at
// x = 0.365).
// k is the larger of two counts.  The first follows the typical normalised
// singular value of a well-conditioned s-row matrix, 1/sqrt(s), through p
// while it stays below the first x > 0 with p'(x) <= a / 2.  The second is
// steps - 2: an ill-conditioned momentum has directions far below the typical
// value that keep growing for most of the iterations.  Measured against the
// fp64 iteration (bf16 stage calls, short sides 768 to 4096), three residuals
// hold spectra over three decades, a rank-s/8 matrix plus noise of 1e-2 or
// 1e-3, and a two-level spectrum at 5.5e-3 to 9.9e-3, where two residuals
// reach 2.8e-2 and one 8.6e-2; on Gaussian and heavy-tailed inputs three cost
// at most 15% over two (7.8e-3 to 1.1e-2).  Quintic, 5 steps: k = 3; cubic:
// 4 (all but the last).
int residual_iterations(int64_t s, float a, float b, float c, int steps) {
  if (!(a > 0.0f) || steps < 2 || s < 1) return 0;
  const double A = a, B = b, C = c;
  auto p = [&](double x) { return x * (A + x * x * (B + C * x * x)); };
  auto slope = [&](double x) { return A + x * x * (3.0 * B + 5.0 * C * x * x); };
  double xstar = HUGE_VAL;
  for (int i = 1; i <= 4000; ++i) {
    const double x = 1e-3 * i;
    if (slope(x) <= 0.5 * A) {
      xstar = x;
      break;
    }
  }
  double x = 1.0 / std::sqrt(static_cast<double>(s));
  int k = 0;
  while (k < steps - 1) {
    x = p(x);
    if (!(x > 0.0 && x < xstar)) break;
    ++k;
  }
  return std::max(k, steps - 2);
}

// signs from the last product's epilogue: bf16 products, U not transposed,
// whole 64-bit words per row of U
bool fuses_signs(int64_t rows, int64_t cols, int precision, int steps) {
  return run_precision(rows, cols, precision) == MUON_BF16 && steps > 0 && rows <= cols && cols % 64 == 0;
}

bool valid_problem(const muon_ns_problem& p) {
  return p.rows > 0 && p.cols > 0 && p.M && (p.U || p.bits);
}

// The workspace of ns_orthogonalize starts with the split scratch shared by
// every product of every run (its counters are cleared once per call and
// each launch leaves them clear), followed by the largest run's buffers.
struct SplitRegion {
  size_t bytes;
};

SplitRegion split_region(const std::vector<Run>& runs, int precision) {
  // the counter block (with the error word ns_workspace_status reads) is
  // always there, also when nothing splits
  SplitRegion R{gemm::kSplitCounterBytes};
  if (precision != MUON_BF16) return R;
  for (const Run& r : runs)
    if (run_precision(r.rows, r.cols, precision) == MUON_BF16)
      R.bytes = std::max(R.bytes, round_up(split_scratch_bound(r.sp, r.lp, r.count), 256));
  return R;
}

// packed signs of every U of a run whose signs were not fused into its last
// product: one sign_pack over the whole run when its directions lie back to
// back and each starts a fresh 64-bit word with its words back to back too
// (the words are then those of the concatenation), else one per problem
int pack_run_signs(const Run& r, hipStream_t st) {
  if (!r.bits) return MUON_OK;
  const size_t es = dtype_size(r.u_dtype);
  const int64_t n = r.rows * r.cols;
  if (r.count > 1 && r.strideU == n && n % 64 == 0 && r.stride_bits == n / 64)
    return sign_pack(r.U, r.u_dtype, n * r.count, r.bits, st);
  // evenly spaced problems (a layer set's matrices of one shape): one launch
  if (r.count > 1 && sign_pack_runs(r.U, r.u_dtype, n, r.count, r.strideU, r.bits, r.stride_bits, st) == MUON_OK)
    return MUON_OK;
  for (int k = 0; k < r.count; ++k) {
    const int status = sign_pack(static_cast<const char*>(r.U) + k * r.strideU * es, r.u_dtype,
                                 r.rows * r.cols, r.bits + k * r.stride_bits, st);
    if (status != MUON_OK) return status;
  }
  return MUON_OK;
}

size_t runs_bytes(const std::vector<Run>& runs, int precision) {
  size_t need = 0;
  for (const Run& r : runs) need = std::max(need, layout_of(r, precision).total);
  return need;
}

// One run of equal-shape problems: normalisation (unless folded), `steps`
// iterations, and the signs; `ws` holds the run's buffers (layout_of), `sc`
// the split scratch of the lane it runs on.
int run_one(const Run& r, char* ws, const gemm::Scratch& sc, int precision, float a, float b, float c, int steps,
            hipStream_t st) {
  const RunLayout L = layout_of(r, precision);
  const int prec = run_precision(r.rows, r.cols, precision);
  const float* sumsq = r.sumsq;
  int64_t stride_sumsq = r.stride_sumsq;
  int status;
  if (!r.has_sumsq) {
    float* out = reinterpret_cast<float*>(ws + L.sumsq);
    status = sumsq_strided(r.M, r.m_dtype, r.rows * r.cols, r.count, r.strideM, out,
                           ws + L.partials, st);
    if (status != MUON_OK) return status;
    sumsq = out;
    stride_sumsq = 1;
  }
  void* X[2] = {ws + L.x0, ws + L.x1};
  void* A = ws + L.a;
  void* B = ws + L.b;
  // a bf16, wide, pad-free momentum is its own (unnormalised) X0: the first
  // iteration reads M and folds the Frobenius scale into its epilogues
  const bool fold_norm = folds_normalisation(r, prec) && steps > 0;
  if (!fold_norm) {
    status = normalize_dispatch(r.M, r.m_dtype, r.strideM, r.rows, r.cols, sumsq, stride_sumsq, X[0],
                                prec, r.sp, r.lp, r.count, st);
    if (status != MUON_OK) return status;
  }
  if (steps == 0) {
    status = prec == MUON_BF16
                 ? emit_t<bf16_t>(X[0], r.sp, r.lp, r.rows, r.cols, r.U, r.u_dtype, r.strideU, r.count, st)
                 : emit_t<float>(X[0], r.sp, r.lp, r.rows, r.cols, r.U, r.u_dtype, r.strideU, r.count, st);
    if (status == MUON_OK) status = pack_run_signs(r, st);
    if (status != MUON_OK) return status;
    return MUON_OK;
  }
  GemmArgs fin{};
  fin.U = r.U;
  fin.strideU = r.strideU;
  fin.s_valid = std::min(r.rows, r.cols);
  fin.l_valid = std::max(r.rows, r.cols);
  fin.u_dtype = r.u_dtype;
  fin.transpose_out = r.rows > r.cols;
  const bool fused_signs = r.bits && fuses_signs(r.rows, r.cols, precision, steps);
  if (fused_signs) {
    fin.bits = r.bits;
    fin.bits_rows = r.rows;
    fin.bits_cols = r.cols;
    fin.stride_bits = r.stride_bits;
  }
  const int kres = prec == MUON_BF16 ? residual_iterations(std::min(r.rows, r.cols), a, b, c, steps) : 0;
  for (int it = 0; it < steps; ++it) {
    const bool first_folded = fold_norm && it == 0;
    const void* Xc = first_folded ? r.M : X[it & 1];
    void* Xn = X[(it + 1) & 1];
    const bool last = it + 1 == steps;
    const Fold fold = first_folded ? Fold{sumsq, stride_sumsq, r.strideM} : Fold{};
    if (prec == MUON_BF16) {
      // c != 0: X' = a X + (bA + cA^2) X;  c == 0: X' = a X + b A X
      status = gram_t<bf16_t>(Xc, A, r.sp, r.lp, r.count, st, sc, fold);
      if (status == MUON_OK && c != 0.0f) status = poly_t<bf16_t>(A, B, r.sp, r.count, b, c, st, sc);
      // the residual buffer is read and rewritten in place (entry by entry, by one lane)
      void* Xlo = ws + L.xl;
      const bool lo_in = it >= 1 && it <= kres;
      const bool lo_out = it < kres && !last;
      // signs only (no direction wanted): the last product is the kernel of the
      // other iterations with no output but the packed signs
      const bool signs_only = last && r.U == nullptr;
      if (status == MUON_OK)
        status = apply_t<bf16_t>(c != 0.0f ? B : A, Xc, signs_only ? nullptr : Xn, r.sp, r.lp, r.count, a,
                                 c != 0.0f ? 1.0f : b, st, sc, last && !signs_only ? &fin : nullptr, fold,
                                 signs_only ? &fin : nullptr, lo_in ? Xlo : nullptr, lo_out ? Xlo : nullptr);
    } else {
      status = gram_t<float>(Xc, A, r.sp, r.lp, r.count, st, sc);
      if (status == MUON_OK && c != 0.0f) status = poly_t<float>(A, B, r.sp, r.count, b, c, st, sc);
      if (status == MUON_OK)
        status = apply_t<float>(c != 0.0f ? B : A, Xc, Xn, r.sp, r.lp, r.count, a, c != 0.0f ? 1.0f : b,
                                st, sc, last ? &fin : nullptr);
    }
    if (status != MUON_OK) return status;
  }
  if (!fused_signs) {
    status = pack_run_signs(r, st);
    if (status != MUON_OK) return status;
  }
  return MUON_OK;
}

// Runs of different shapes (a layer set) go to lanes, the caller's stream and
// up to three streams of the library's, forked from and joined back into the
// caller's stream with events: the small launches of one run then fill the
// CUs that another run's tails and ramps leave idle.  Measured on the
// GPT-2-small set (four runs on two streams): 2.15 -> 2.0 ms; on three and four
// streams it ran 2% and 5% slower than on two (these products fill the CUs
// better than Dion's, and more runs at once share the caches).  Each lane has
// its own run buffers and split scratch; lane 0's are sized for every run, so
// all runs can also go to lane 0 alone (when a stream or the events cannot be
// had).
#ifndef MUON_NS_LANES
#define MUON_NS_LANES 2
#endif
constexpr int kNsLanes = MUON_NS_LANES;
static_assert(kNsLanes >= 1 && kNsLanes <= kLibStreams + 1, "one library stream per extra lane");

// relative cost of a run (its products' multiply-adds per iteration)
double run_cost(const Run& r) {
  const double s = static_cast<double>(r.sp), l = static_cast<double>(r.lp);
  return static_cast<double>(r.count) * (s * s * l + s * s * s + 2.0 * s * s * l);
}

struct LanePlan {
  int lanes = 1;
  std::vector<int> lane;                // lane of each run
  size_t split[kNsLanes] = {};          // split scratch of each lane (counters first)
  size_t bufs[kNsLanes] = {};           // run buffers of each lane
  size_t split_off(int l) const {
    size_t o = 0;
    for (int i = 0; i < l; ++i) o += split[i];
    return o;
  }
  size_t bufs_off(int l) const {
    size_t o = split_off(kNsLanes);
    for (int i = 0; i < l; ++i) o += bufs[i];
    return o;
  }
  size_t total() const { return bufs_off(kNsLanes); }
};

// Workspace: [split scratch 0][split scratch 1] .. [run buffers 0][run buffers 1] ..
// Runs are placed largest first on the lane with the least work so far.
LanePlan plan_lanes(const std::vector<Run>& runs, int precision) {
  LanePlan P;
  P.lane.assign(runs.size(), 0);
  P.split[0] = split_region(runs, precision).bytes;
  P.bufs[0] = runs_bytes(runs, precision);
  P.lanes = static_cast<int>(std::min<size_t>(kNsLanes, runs.size()));
  if (P.lanes < 2) {
    P.lanes = 1;
    return P;
  }
  std::vector<size_t> order(runs.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(),
                   [&](size_t x, size_t y) { return run_cost(runs[x]) > run_cost(runs[y]); });
  double load[kNsLanes] = {};
  for (size_t i : order) {
    int l = 0;
    for (int j = 1; j < P.lanes; ++j)
      if (load[j] < load[l]) l = j;
    P.lane[i] = l;
    load[l] += run_cost(runs[i]);
  }
  for (int l = 1; l < P.lanes; ++l) {
    std::vector<Run> mine;
    for (size_t i = 0; i < runs.size(); ++i)
      if (P.lane[i] == l) mine.push_back(runs[i]);
    P.split[l] = split_region(mine, precision).bytes;
    P.bufs[l] = runs_bytes(mine, precision);
  }
  return P;
}

}  // namespace
}  // namespace muon

using namespace muon;

extern "C" {

size_t ns_workspace_bytes(const muon_ns_problem* probs, int count, int precision) {
  if (!probs || count <= 0 || (precision != MUON_F32 && precision != MUON_BF16)) return 0;
  for (int i = 0; i < count; ++i)
    if (!valid_problem(probs[i])) return 0;
  return plan_lanes(make_runs(probs, count), precision).total();
}

int ns_orthogonalize(const muon_ns_problem* probs, int count, float a, float b, float c, int steps,
                     int precision, void* workspace, size_t ws_bytes, void* stream) {
  if (count < 0 || steps < 0) return MUON_EINVAL;
  if (count == 0) return MUON_OK;
  if (!probs) return MUON_EINVAL;
  if (precision != MUON_F32 && precision != MUON_BF16) return MUON_EDTYPE;
  for (int i = 0; i < count; ++i) {
    const muon_ns_problem& p = probs[i];
    if (!valid_problem(p)) return MUON_EINVAL;
    if (!valid_dtype(p.m_dtype) || !valid_dtype(p.u_dtype)) return MUON_EDTYPE;
    if (!p.U && !fuses_signs(p.rows, p.cols, precision, steps)) return MUON_EINVAL;
    if (!aligned16(p.M) || (p.U && !aligned16(p.U))) return MUON_EALIGN;
    if (reinterpret_cast<uintptr_t>(p.bits) % 8 != 0) return MUON_EALIGN;
  }
  const std::vector<Run> runs = make_runs(probs, count);
  const LanePlan P = plan_lanes(runs, precision);
  if (!workspace || ws_bytes < P.total()) return MUON_EWORKSPACE;
  if (!aligned16(workspace)) return MUON_EALIGN;

  hipStream_t st = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(workspace);
  // bf16 products may split (a symmetric product with one tile row needs no
  // scratch: its only unit is the diagonal lower half).  Every lane reports a
  // wait that runs out in lane 0's error word, the one ns_workspace_status reads.
  int* error_word = reinterpret_cast<int*>(base) + gemm::kSplitCounters;
  const bool bf16 = precision == MUON_BF16;
  gemm::Scratch sc[kNsLanes];
  char* bufs[kNsLanes];
  for (int l = 0; l < kNsLanes; ++l) {
    sc[l] = gemm::Scratch{bf16 ? base + P.split_off(l) : nullptr, P.split[l], l > 0 ? error_word : nullptr};
    bufs[l] = base + P.bufs_off(l);
  }
  // arrival counters and the error word start at zero on every call
  for (int l = 0; l < P.lanes; ++l) {
    const int status = zero_counters(base + P.split_off(l), gemm::kSplitWords, st);
    if (status != MUON_OK) return status;
  }
  // the lanes' streams, forked from the caller's; with any of them or the
  // events missing, every run goes to the caller's stream
  int lanes = P.lanes;
  hipStream_t lane_st[kNsLanes] = {st};
  hipEvent_t ev[kNsLanes] = {};   // the fork, then the joins of lanes 1 ..
  for (int l = 1; l < lanes; ++l)
    if ((lane_st[l] = lane_stream(l - 1)) == nullptr) lanes = 1;
  if (lanes > 1 && (!lane_events(ev, lanes) || hipEventRecord(ev[0], st) != hipSuccess)) lanes = 1;
  int forked = 1;   // lanes 1 .. forked - 1 wait on the fork (and are joined below)
  for (int l = 1; l < lanes; ++l, ++forked)
    if (hipStreamWaitEvent(lane_st[l], ev[0], 0) != hipSuccess) break;
  if (forked < lanes) lanes = 1;
  int status = MUON_OK;
  for (size_t i = 0; i < runs.size() && status == MUON_OK; ++i) {
    const int l = lanes > 1 ? P.lane[i] : 0;
    status = run_one(runs[i], bufs[l], sc[l], precision, a, b, c, steps, lane_st[l]);
  }
  for (int l = 1; l < forked; ++l)
    if ((hipEventRecord(ev[l], lane_st[l]) != hipSuccess || hipStreamWaitEvent(st, ev[l], 0) != hipSuccess) &&
        status == MUON_OK)
      status = MUON_ELAUNCH;
  return status;
}

int ns_workspace_status(const void* workspace, size_t ws_bytes, void* stream) {
  if (!workspace || ws_bytes < gemm::kSplitCounterBytes) return MUON_EINVAL;
  if (!aligned16(workspace)) return MUON_EALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int word = 0;
  const char* src = static_cast<const char*>(workspace) + gemm::kSplitCounters * sizeof(int);
  if (hipMemcpyAsync(&word, src, sizeof(int), hipMemcpyDeviceToHost, st) != hipSuccess) return MUON_ELAUNCH;
  if (hipStreamSynchronize(st) != hipSuccess) return MUON_ELAUNCH;
  return word != 0 ? MUON_ESPLIT : MUON_OK;
}

int ns_bf16_min_side(void) { return static_cast<int>(kBf16MinSide); }

int ns_residual_iterations(int64_t rows, int64_t cols, float a, float b, float c, int steps, int precision) {
  if (rows <= 0 || cols <= 0 || steps < 0) return MUON_EINVAL;
  if (precision != MUON_F32 && precision != MUON_BF16) return MUON_EDTYPE;
  return run_precision(rows, cols, precision) == MUON_BF16 ? residual_iterations(std::min(rows, cols), a, b, c, steps)
                                                            : 0;
}

int muon_set_split_wait_limit(int polls) {
  if (polls < 0) return MUON_EINVAL;
  gemm::split_spin_limit().store(polls, std::memory_order_relaxed);
  return MUON_OK;
}

int muon_get_split_wait_limit(void) { return gemm::split_spin_limit().load(std::memory_order_relaxed); }

static bool stage_dims_ok(int64_t s, int64_t l, int64_t batch) {
  return s > 0 && l > 0 && batch >= 0 && s % MUON_NS_PAD == 0 && l % MUON_NS_PAD == 0 && s <= l;
}

int ns_normalize(const void* M, int m_dtype, int64_t rows, int64_t cols, int64_t batch,
                 const float* sumsq, void* X0, int precision, void* stream) {
  if (rows <= 0 || cols <= 0 || batch < 0) return MUON_EINVAL;
  if (!valid_dtype(m_dtype)) return MUON_EDTYPE;
  if (precision != MUON_F32 && precision != MUON_BF16) return MUON_EDTYPE;
  if (batch == 0) return MUON_OK;
  if (!M || !sumsq || !X0) return MUON_EINVAL;
  if (!aligned16(M) || !aligned16(X0)) return MUON_EALIGN;
  const int64_t sp = pad_to(std::min(rows, cols)), lp = pad_to(std::max(rows, cols));
  return normalize_dispatch(M, m_dtype, rows * cols, rows, cols, sumsq, 1, X0, precision, sp, lp,
                            batch, static_cast<hipStream_t>(stream));
}

size_t ns_stage_workspace_bytes(int64_t s, int64_t l, int64_t batch, int precision) {
  if (!stage_dims_ok(s, l, batch) || precision != MUON_BF16) return 0;
  return split_scratch_bound(s, l, batch);
}

// scratch of a stage call: null (no splitting) or at least
// ns_stage_workspace_bytes, 16-byte aligned
static int stage_scratch(void* workspace, size_t ws_bytes, int64_t s, int64_t l, int64_t batch,
                         int precision, gemm::Scratch& sc) {
  sc = gemm::Scratch{nullptr, 0};
  if (!workspace || precision != MUON_BF16) return MUON_OK;
  if (ws_bytes < split_scratch_bound(s, l, batch)) return MUON_EWORKSPACE;
  if (!aligned16(workspace)) return MUON_EALIGN;
  sc = gemm::Scratch{static_cast<char*>(workspace), ws_bytes};
  return MUON_OK;
}

int ns_gram(const void* X, void* A, int64_t s, int64_t l, int64_t batch, int precision,
            const float* sumsq, void* workspace, size_t ws_bytes, void* stream) {
  if (!stage_dims_ok(s, l, batch)) return MUON_EINVAL;
  if (precision != MUON_F32 && precision != MUON_BF16) return MUON_EDTYPE;
  if (sumsq && precision != MUON_BF16) return MUON_EDTYPE;
  if (batch == 0) return MUON_OK;
  if (!X || !A) return MUON_EINVAL;
  if (!aligned16(X) || !aligned16(A)) return MUON_EALIGN;
  gemm::Scratch sc;
  const int status = stage_scratch(workspace, ws_bytes, s, l, batch, precision, sc);
  if (status != MUON_OK) return status;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return precision == MUON_BF16 ? gram_t<bf16_t>(X, A, s, l, batch, st, sc, Fold{sumsq, 1, 0})
                                : gram_t<float>(X, A, s, l, batch, st, sc);
}

int ns_poly(const void* A, void* B, int64_t s, int64_t batch, float b, float c, int precision,
            void* workspace, size_t ws_bytes, void* stream) {
  if (!stage_dims_ok(s, s, batch)) return MUON_EINVAL;
  if (precision != MUON_F32 && precision != MUON_BF16) return MUON_EDTYPE;
  if (batch == 0) return MUON_OK;
  if (!A || !B) return MUON_EINVAL;
  if (!aligned16(A) || !aligned16(B)) return MUON_EALIGN;
  gemm::Scratch sc;
  const int status = stage_scratch(workspace, ws_bytes, s, s, batch, precision, sc);
  if (status != MUON_OK) return status;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return precision == MUON_BF16 ? poly_t<bf16_t>(A, B, s, batch, b, c, st, sc)
                                : poly_t<float>(A, B, s, batch, b, c, st, sc);
}

int ns_apply(const void* B, const void* X, const void* X_lo, void* Xout, void* Xout_lo, int64_t s,
             int64_t l, int64_t batch, float a, float alpha, int precision, const float* sumsq,
             void* workspace, size_t ws_bytes, void* stream) {
  if (!stage_dims_ok(s, l, batch)) return MUON_EINVAL;
  if (precision != MUON_F32 && precision != MUON_BF16) return MUON_EDTYPE;
  if ((sumsq || X_lo || Xout_lo) && precision != MUON_BF16) return MUON_EDTYPE;
  if (batch == 0) return MUON_OK;
  if (!B || !X || !Xout) return MUON_EINVAL;
  if (!aligned16(B) || !aligned16(X) || !aligned16(Xout)) return MUON_EALIGN;
  if ((X_lo && !aligned16(X_lo)) || (Xout_lo && !aligned16(Xout_lo))) return MUON_EALIGN;
  gemm::Scratch sc;
  const int status = stage_scratch(workspace, ws_bytes, s, l, batch, precision, sc);
  if (status != MUON_OK) return status;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return precision == MUON_BF16
             ? apply_t<bf16_t>(B, X, Xout, s, l, batch, a, alpha, st, sc, nullptr, Fold{sumsq, 1, 0},
                               nullptr, X_lo, Xout_lo)
             : apply_t<float>(B, X, Xout, s, l, batch, a, alpha, st, sc, nullptr);
}

int ns_apply_signs(const void* B, const void* X, const void* X_lo, void* Xout, uint64_t* bits, int64_t s,
                   int64_t l, int64_t batch, float a, float alpha, int precision, const float* sumsq,
                   void* workspace, size_t ws_bytes, void* stream) {
  if (!stage_dims_ok(s, l, batch)) return MUON_EINVAL;
  if (precision != MUON_BF16) return MUON_EDTYPE;
  if (batch == 0) return MUON_OK;
  if (!B || !X || !bits) return MUON_EINVAL;
  if (!aligned16(B) || !aligned16(X) || (Xout && !aligned16(Xout))) return MUON_EALIGN;
  if (X_lo && !aligned16(X_lo)) return MUON_EALIGN;
  if (reinterpret_cast<uintptr_t>(bits) % 8 != 0) return MUON_EALIGN;
  gemm::Scratch sc;
  const int status = stage_scratch(workspace, ws_bytes, s, l, batch, precision, sc);
  if (status != MUON_OK) return status;
  GemmArgs signs{};
  signs.bits = bits;
  signs.bits_rows = s;
  signs.bits_cols = l;
  signs.stride_bits = s * l / 64;
  return apply_t<bf16_t>(B, X, Xout, s, l, batch, a, alpha, static_cast<hipStream_t>(stream), sc, nullptr,
                         Fold{sumsq, 1, 0}, &signs, X_lo, nullptr);
}

}  // extern "C"
