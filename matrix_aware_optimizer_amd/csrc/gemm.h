// Matrix-core GEMM used by the Newton-Schulz products (gfx950, wave64).
//
//   C = alpha * P Q^T (+ beta * Z)          P, Q rows contiguous along k ("NT")
//   C = alpha * P Q   (+ beta * Z)          Q given k-major: [K][N] ("NN")
//
// The symmetric products (the Gram X X^T and A A for symmetric A) run NT
// with P = Q over the lower-triangle tiles only; every off-diagonal tile is
// stored twice (at (i,j) and mirrored at (j,i)), so the output is the full
// symmetric matrix.
//
// Structure of one workgroup (BM x BN output tile, (BM/WM) x (BN/WN) waves):
//  * k advances in LDS tiles of 128 bytes per row (64 bf16 / 32 fp32); two
//    LDS stages: while the waves multiply stage s, the next k-tile travels
//    global -> registers, and is written to stage s^1 before the one barrier
//    of the iteration.
//  * LDS rows hold 8 chunks of 16 bytes; chunk c of row r sits at slot
//    c ^ ((r ^ (r >> 3)) & 7), which keeps both the tile stores (8 lanes per
//    row) and the fragment reads (32 consecutive rows) free of bank
//    conflicts.
//  * The NN operand is read as E x E blocks (E = 8 bf16 / 4 fp32 per 16 bytes)
//    of [k][n] and transposed in registers, so its LDS tile has the same
//    k-contiguous rows as the NT operands.
//  * Fragments: lane l holds row (l % 32) and k-group (l / 32) of a 32 x 32
//    tile; bf16 issues v_mfma_f32_32x32x16_bf16, fp32 four
//    v_mfma_f32_32x32x2f32, both accumulating in fp32.
//  * Workgroup ids are spread round-robin over the 8 XCDs by the dispatcher;
//    they are remapped so each XCD gets a contiguous range of tiles, ordered
//    in groups of GROUP_M tile rows so that concurrently running tiles share
//    operand strips in that XCD's L2.
#pragma once

#include <algorithm>
#include <type_traits>
#include <utility>

#include "common.h"

namespace muon {
namespace gemm {

constexpr int kRowBytes = 128;
constexpr int kXcds = 8;
#ifndef MUON_GEMM_INTERLEAVE
#define MUON_GEMM_INTERLEAVE 1
#endif
#ifndef MUON_GEMM_LGKM_SPLIT
#define MUON_GEMM_LGKM_SPLIT 1
#endif
constexpr int kGroupM = 8;

template <typename T> struct Mfma;
template <> struct Mfma<bf16_t> {
  static constexpr int kElems = 8;  // elements per 16 bytes
  __device__ __forceinline__ static void mma(const u32x4_t& a, const u32x4_t& b, f32x16_t& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  static constexpr int kElems = 4;
  __device__ __forceinline__ static void mma(const u32x4_t& a, const u32x4_t& b, f32x16_t& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  }
};

// byte offset of 16-byte chunk `chunk` (0..7) of LDS tile row `row`
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

enum Epi { EPI_STORE = 0, EPI_AXPBY = 1, EPI_FINAL = 2 };

// Work units of the bf16 DMA kernel.  SPLIT_NONE: one workgroup per tile.
// SPLIT_SYRK (long symmetric products whose n_p^2 units fit one round of the
// CUs, n_p = M / BM): every off-diagonal tile runs as two K halves and every
// diagonal tile as one unit that computes only its lower half, n_p^2 units of
// about half a tile each instead of n_p (n_p + 1) / 2 whole tiles, which
// would leave the other CUs idle.  SPLIT_DIAG: unit v is the lower half of
// diagonal tile v.  SPLIT_TRI (symmetric products over several rounds of the
// CUs): the n_p (n_p - 1) / 2 off-diagonal tiles whole, row by row, then the n_p
// diagonal tiles as lower halves, so no unit computes the upper half of a
// diagonal tile (the same unit count as whole tiles, less work).
enum Split { SPLIT_NONE = 0, SPLIT_SYRK = 1, SPLIT_DIAG = 2, SPLIT_TRI = 3 };
#ifndef MUON_SYRK_TRI
#define MUON_SYRK_TRI 1
#endif
constexpr bool kSyrkTri = MUON_SYRK_TRI != 0;
#ifndef MUON_SYRK_HALF_ORDER
#define MUON_SYRK_HALF_ORDER 1
#endif
constexpr bool kSyrkHalfOrder = MUON_SYRK_HALF_ORDER != 0;
// default bound on the polls of the second K half waiting for the first
// one's partial (each poll sleeps ~128 cycles; the first half never needs
// more than microseconds, the bound only keeps a wait from outliving its
// cause).  A wait that runs out sets the scratch's error word and leaves the
// tile unwritten; the host reads the word back (ns_workspace_status).
constexpr int kSplitSpinLimit = 1 << 22;

struct GemmArgs {
  const void* P;  // rows of the left operand, k-contiguous, ld = K
  const void* Q;  // NT: rows of the right operand (k-contiguous, ld = K); NN: [K][N]
  const void* Z;  // epilogue addend [M][N] (ld = N), may be null
  void* C;        // output [M][N] (ld = N)
  // bf16 residuals (B X products only): the addend is Z + Zl when Zl is set,
  // and Cl receives C's rounding residual bf16(v - bf16(v)), so that C + Cl
  // carries v to about 16 significant bits.  Same layout as Z and C.  Each
  // entry of Zl is read by the lane that writes the same entry of Cl, so Zl
  // and Cl may be one buffer.
  const void* Zl;
  void* Cl;
  int64_t M, N, K;
  int64_t strideP, strideQ, strideZ, strideC;  // batch strides (elements)
  float alpha, beta;                           // C = alpha*acc + beta*Z (Z unread if beta == 0)
  // Frobenius scaling folded into the first iteration: with scale_sumsq set,
  // alpha and beta of batch entry b are multiplied by f(sumsq[b * stride]),
  // f = 1/ss (scale_mode 1, the Gram of M) or 1/sqrt(ss) (scale_mode 2, the
  // product with M), and f = 0 for ss == 0
  const float* scale_sumsq;
  int64_t stride_sumsq;
  int scale_mode;
  // EPI_FINAL: write U instead of C, un-padded (s_valid x l_valid of the
  // working layout) and transposed back when the momentum was tall.
  void* U;
  int64_t strideU;
  int64_t s_valid, l_valid;
  int u_dtype;
  int transpose_out;
  // work units (Split): the two halves of a split tile each store an fp32
  // partial tile; the second to finish (counted by an arrival counter) adds
  // the other's and runs the epilogue
  // Row stride (elements) of Q for NN, Z and C; 0 means N.  A launch may
  // cover columns [col0, col0 + N) of a wider output: its Q, Z and C point at
  // column col0, and col0 places the columns of U (EPI_FINAL).
  int64_t ld;
  int64_t col0;
  // Optional packed signs of the stored output (non-symmetric products): bit
  // (r, c) of a bits_rows x bits_cols row-major matrix (bits_cols a multiple
  // of 64) is bit (r * bits_cols + c) % 64 of word (r * bits_cols + c) / 64,
  // batch entries stride_bits words apart.  For EPI_FINAL the matrix is U
  // (not transposed), else the launch's full output.  C (EPI_AXPBY) or U
  // (EPI_FINAL) may then be null, and only the signs are written.
  uint64_t* bits;
  int64_t bits_rows, bits_cols, stride_bits;
  int split_mode;
  float* partials;       // (split tiles) x BM x BN fp32: the first-arriving half's
  int* counters;         // one per split tile: zero on entry, left zero
  int* split_error;      // set to 1 by a second half whose wait ran out
  int spin_limit;        // polls of that wait
};

template <typename T, int BM_, int BN_, int WM_, int WN_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int E = Mfma<T>::kElems;
  static constexpr int BK = kRowBytes / sizeof(T);  // k per LDS tile
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int NT = WAVES_M * WAVES_N * kWave;
  static constexpr int FM = WM / 32, FN = WN / 32;  // 32x32 fragments per wave
  static constexpr int KSTEPS = BK / (2 * E);       // fragment reads per LDS tile
  static constexpr int A_CHUNKS = BM * 8 / NT;      // 16-byte loads per thread
  static constexpr int B_CHUNKS = BN * 8 / NT;
  static constexpr int NN_BLOCKS = (BK / E) * (BN / E);
  static constexpr int NN_PER_T = (NN_BLOCKS + NT - 1) / NT;
  static constexpr int STAGE_BYTES = (BM + BN) * kRowBytes;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
  static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile/threads mismatch");
};

__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t nblocks) {
  const int64_t full = nblocks / kXcds * kXcds;
  if (bid >= full) return bid;
  return (bid % kXcds) * (full / kXcds) + bid / kXcds;
}

template <typename T, int BM, int BN, int WM, int WN, bool SYRK, bool NN, int EPI>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void gemm_kernel(GemmArgs g) {
  using C_ = Tile<T, BM, BN, WM, WN>;
  constexpr int E = C_::E, BK = C_::BK, NT = C_::NT, FM = C_::FM, FN = C_::FN;
  static_assert(!SYRK || BM == BN, "symmetric products need square tiles");
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t batch = blockIdx.y;

  // ---- tile coordinates ----
  int64_t tm, tn;
  if (SYRK) {
    const int64_t T_ = g.M / BM;
    const int64_t t = xcd_remap(blockIdx.x, T_ * (T_ + 1) / 2);
    int64_t ti = static_cast<int64_t>((sqrt(8.0 * double(t) + 1.0) - 1.0) * 0.5);
    while ((ti + 1) * (ti + 2) / 2 <= t) ++ti;
    while (ti * (ti + 1) / 2 > t) --ti;
    tm = ti;
    tn = t - ti * (ti + 1) / 2;
  } else {
    const int64_t TM = g.M / BM, TN = g.N / BN;
    const int64_t t = xcd_remap(blockIdx.x, TM * TN);
    const int64_t per_group = int64_t(kGroupM) * TN;
    const int64_t first_m = (t / per_group) * kGroupM;
    const int64_t gsize = min(TM - first_m, int64_t(kGroupM));
    const int64_t r = t % per_group;
    tm = first_m + r % gsize;
    tn = r / gsize;
  }
  const int64_t m0 = tm * BM, n0 = tn * BN;

  const T* P = static_cast<const T*>(g.P) + batch * g.strideP;
  const T* Q = static_cast<const T*>(g.Q) + batch * g.strideQ;

  // ---- global -> register staging ----
  u32x4_t ra[C_::A_CHUNKS];
  u32x4_t rb[NN ? C_::NN_PER_T * E : C_::B_CHUNKS];

  auto load_tiles = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < C_::A_CHUNKS; ++i) {
      const int c = tid + i * NT;
      ra[i] = *reinterpret_cast<const u32x4_t*>(P + (m0 + (c >> 3)) * g.K + k0 + (c & 7) * E);
    }
    if (!NN) {
#pragma unroll
      for (int i = 0; i < C_::B_CHUNKS; ++i) {
        const int c = tid + i * NT;
        rb[i] = *reinterpret_cast<const u32x4_t*>(Q + (n0 + (c >> 3)) * g.K + k0 + (c & 7) * E);
      }
    } else {
#pragma unroll
      for (int i = 0; i < C_::NN_PER_T; ++i) {
        const int blk = tid + i * NT;
        if (blk < C_::NN_BLOCKS) {
          const int nb = blk % (BN / E), kb = blk / (BN / E);
#pragma unroll
          for (int r = 0; r < E; ++r)
            rb[i * E + r] =
                *reinterpret_cast<const u32x4_t*>(Q + (k0 + kb * E + r) * g.N + n0 + nb * E);
        }
      }
    }
  };

  auto store_tiles = [&](char* stage) {
    char* sA = stage;
    char* sB = stage + BM * kRowBytes;
#pragma unroll
    for (int i = 0; i < C_::A_CHUNKS; ++i) {
      const int c = tid + i * NT;
      *reinterpret_cast<u32x4_t*>(sA + lds_off(c >> 3, c & 7)) = ra[i];
    }
    if (!NN) {
#pragma unroll
      for (int i = 0; i < C_::B_CHUNKS; ++i) {
        const int c = tid + i * NT;
        *reinterpret_cast<u32x4_t*>(sB + lds_off(c >> 3, c & 7)) = rb[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < C_::NN_PER_T; ++i) {
        const int blk = tid + i * NT;
        if (blk < C_::NN_BLOCKS) {
          const int nb = blk % (BN / E), kb = blk / (BN / E);
          const u32x4_t* in = rb + i * E;
          if (sizeof(T) == 2) {
            // in[r] holds k = kb*8 + r for n = nb*8 + 0..7 (two per dword);
            // column e of the 8x8 block becomes the 8 k-values of row n.
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int d = e >> 1;
              uint32_t w[4];
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const uint32_t lo = in[2 * j][d], hi = in[2 * j + 1][d];
                w[j] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
              }
              u32x4_t o;
              o.x = w[0]; o.y = w[1]; o.z = w[2]; o.w = w[3];
              *reinterpret_cast<u32x4_t*>(sB + lds_off(nb * 8 + e, kb)) = o;
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              u32x4_t o;
              o.x = in[0][e]; o.y = in[1][e]; o.z = in[2][e]; o.w = in[3][e];
              *reinterpret_cast<u32x4_t*>(sB + lds_off(nb * 4 + e, kb)) = o;
            }
          }
        }
      }
    }
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int wm0 = (wave / C_::WAVES_N) * WM;
  const int wn0 = (wave % C_::WAVES_N) * WN;
  const int frow = lane & 31, fgrp = lane >> 5;

  const int64_t KT = g.K / BK;
  load_tiles(0);
  store_tiles(lds);
  __syncthreads();
  for (int64_t kt = 0; kt < KT; ++kt) {
    char* cur = lds + (kt & 1) * C_::STAGE_BYTES;
    char* nxt = lds + ((kt + 1) & 1) * C_::STAGE_BYTES;
    if (kt + 1 < KT) load_tiles((kt + 1) * BK);
    const char* sA = cur;
    const char* sB = cur + BM * kRowBytes;
#pragma unroll
    for (int ks = 0; ks < C_::KSTEPS; ++ks) {
      const int chunk = ks * 2 + fgrp;
      u32x4_t fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        fa[i] = *reinterpret_cast<const u32x4_t*>(sA + lds_off(wm0 + i * 32 + frow, chunk));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        fb[j] = *reinterpret_cast<const u32x4_t*>(sB + lds_off(wn0 + j * 32 + frow, chunk));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) Mfma<T>::mma(fa[i], fb[j], acc[i][j]);
    }
    if (kt + 1 < KT) store_tiles(nxt);
    __syncthreads();
  }

  // ---- epilogue ----
  // 32x32 accumulator layout: value v of lane l is row 8*(v/4) + 4*(l/32) +
  // (v%4), column l%32 of the fragment.
  T* C = static_cast<T*>(g.C) + batch * g.strideC;
  const T* Z = static_cast<const T*>(g.Z) + batch * g.strideZ;
  const bool mirror = SYRK && (tm != tn);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t col = n0 + wn0 + j * 32 + frow;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row0 = m0 + wm0 + i * 32 + 8 * q + 4 * fgrp;
        float out[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = acc[i][j][4 * q + r] * g.alpha;
          if (EPI != EPI_STORE && g.beta != 0.0f) v = fmaf(g.beta, to_f32(Z[(row0 + r) * g.N + col]), v);
          out[r] = v;
        }
        if (EPI == EPI_FINAL) {
          if (col < g.l_valid) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int64_t row = row0 + r;
              if (row < g.s_valid) {
                const int64_t idx = g.transpose_out ? col * g.s_valid + row : row * g.l_valid + col;
                if (g.u_dtype == MUON_BF16)
                  static_cast<bf16_t*>(g.U)[batch * g.strideU + idx] = f32_to_bf16(out[r]);
                else
                  static_cast<float*>(g.U)[batch * g.strideU + idx] = out[r];
              }
            }
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) C[(row0 + r) * g.N + col] = from_f32<T>(out[r]);
          if (mirror) {
            // the four consecutive rows are four consecutive entries of row `col`
            T* dst = C + col * g.N + row0;
            if (sizeof(T) == 2) {
              const uint32_t w0 = uint32_t(from_f32<bf16_t>(out[0])) | (uint32_t(from_f32<bf16_t>(out[1])) << 16);
              const uint32_t w1 = uint32_t(from_f32<bf16_t>(out[2])) | (uint32_t(from_f32<bf16_t>(out[3])) << 16);
              *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
            } else {
              *reinterpret_cast<float4*>(dst) = make_float4(out[0], out[1], out[2], out[3]);
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 kernel with global -> LDS DMA (global_load_lds_dwordx4) and an
// S-stage LDS ring.  k advances 32 at a time (two 32x32x16 MFMA steps).
//
// LDS layouts (16-byte chunks, XOR-swizzled; both chosen by measuring the
// SQ_LDS_BANK_CONFLICT counter on MI355X for the exact access patterns below,
// where they read zero conflicts):
//  * k-contiguous operand rows (P, and Q for NT): 64 bytes = 4 chunks per
//    row; chunk c of row r sits at slot c ^ ((r >> 2) & 3).
//  * k-major Q tile for NN ([k][n], n contiguous): rows of 2*BN bytes; chunk
//    c of row r sits at slot c ^ (4 * (r & 3)), so the four rows one
//    transposing read touches are 64 bytes apart within 256 bytes.
// One DMA instruction moves 1 KB (64 lanes x 16 bytes) to consecutive LDS
// bytes; each lane picks the global chunk whose swizzled slot is its own.
//
// NN fragments come from ds_read_tr16_b64: within each 16-lane group, lane i
// receives element (i % 4) of the 8-byte chunks addressed by lanes
// 4j + i/4 (j = 0..3).  Pointing lane 4j + q at row k0 + j, columns
// n0 + 4q .. n0 + 4q + 3 hands lane i the four k-values of column n0 + i:
// two such reads (rows k0.., k0+4..) make one 8-deep MFMA operand.
//
// Pipeline per k-step of 32 (iteration `it`, stage it % S resident):
//   fragments (it, 0) are in registers;  read fragments (it, 1);  MFMA (it, 0);
//   wait until this wave's DMA for stage it+1 landed; s_barrier (all waves'
//   DMA landed, and every wave is done reading stage it-1);  DMA stage
//   it+S-1 into the slot of stage it-1;  read fragments (it+1, 0);  MFMA (it, 1).
// __syncthreads() is not used inside the loop: its fence would wait for every
// DMA in flight, including the stages being prefetched.
// ---------------------------------------------------------------------------
template <int BM_, int BN_, int WM_, int WN_, int S_, bool NN_>
struct DmaTile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, S = S_;
  static constexpr int BK = 32;
  static constexpr int W = (BM / WM) * (BN / WN);
  static constexpr int NT = W * kWave;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int P_BYTES = BM * 64;
  static constexpr int Q_BYTES = NN_ ? BK * BN * 2 : BN * 64;
  static constexpr int STAGE_BYTES = P_BYTES + Q_BYTES;
  // epilogue staging: per wave one 32-row slab of fp32 accumulators; the row
  // pitch WN + 8 floats puts the two half-waves' rows 128 bytes apart in the
  // banks
  static constexpr int LDW = WN + 8;
  static constexpr int EPI_BYTES = W * 32 * LDW * 4;
  static constexpr int LDS_BYTES = (S * STAGE_BYTES > EPI_BYTES) ? S * STAGE_BYTES : EPI_BYTES;
  static constexpr int P_DMA = P_BYTES / 1024 / W;   // DMA instructions per wave and stage
  static constexpr int Q_DMA = Q_BYTES / 1024 / W;
  static constexpr int D = P_DMA + Q_DMA;
  static_assert(P_BYTES % (1024 * W) == 0 && Q_BYTES % (1024 * W) == 0, "DMA split");
  static_assert(S >= 3 && D * (S - 3) <= 63, "vmcnt range");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS capacity");
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gbl_void_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 lds_bf16x4_t;

__device__ __forceinline__ int krow_off(int r, int c) {  // k-contiguous rows, 64 B
  return r * 64 + ((c ^ ((r >> 2) & 3)) << 4);
}
// slot of chunk c in row k of the [k][n] tile
__device__ __forceinline__ int nrow_slot(int c, int k) { return c ^ (4 * (k & 3)); }

// Wait for every LDS read of this wave (s_waitcnt lgkmcnt(0), vmcnt and
// expcnt left open).  Placed where the reads it covers were issued a whole
// k-step earlier, it costs nothing and keeps the compiler from placing a
// conservative wait after the next, freshly issued reads.
__device__ __forceinline__ void lds_reads_done() {
#if MUON_GEMM_LGKM_SPLIT
  __builtin_amdgcn_s_waitcnt(0xC07F);
#endif
}

template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// 16 bytes per lane from global memory to LDS bytes [lds_addr + 16 * lane).
// Written as inline asm so the compiler's wait-count pass does not see an LDS
// write it cannot tell apart from the stage being read (it would then drain
// every DMA in flight before each fragment read); ordering is explicit here:
// wait_vm_barrier() is the only consumer-side synchronisation.
// M0 is reserved by the compiler; these kernels contain no other M0 user (no
// LDS-DMA builtins, no relative register indexing, no messages -- checked in
// the generated assembly), so setting it here cannot disturb compiled code.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g),
               "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ u32x4_t read_tr_pair(const char* base0, const char* base1) {
  const lds_bf16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) lds_bf16x4_t*)base0);
  const lds_bf16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) lds_bf16x4_t*)base1);
  uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
  u32x4_t r;
  r.x = ua.x; r.y = ua.y; r.z = ub.x; r.w = ub.y;
  return r;
}

// tile index within one batch entry -> (tile row, tile column): the lower
// triangle for symmetric products, else groups of kGroupM tile rows walked
// column by column
template <int BM, int BN, bool SYRK>
__device__ __forceinline__ void tile_coords(const GemmArgs& g, int64_t t, int64_t& tm, int64_t& tn) {
  if (SYRK) {
    int64_t ti = static_cast<int64_t>((sqrt(8.0 * double(t) + 1.0) - 1.0) * 0.5);
    while ((ti + 1) * (ti + 2) / 2 <= t) ++ti;
    while (ti * (ti + 1) / 2 > t) --ti;
    tm = ti;
    tn = t - ti * (ti + 1) / 2;
  } else {
    const int64_t TM = g.M / BM, TN = g.N / BN;
    const int64_t per_group = int64_t(kGroupM) * TN;
    const int64_t first_m = (t / per_group) * kGroupM;
    const int64_t gsize = min(TM - first_m, int64_t(kGroupM));
    const int64_t r = t % per_group;
    tm = first_m + r % gsize;
    tn = r / gsize;
  }
}

// The lower half of a 256 x 256 diagonal tile of a symmetric product in
// 32 x 32 blocks, spread so that every SIMD gets 9 of the 36 blocks (waves
// w and w + 4 share a SIMD).  Waves 0-3 take the 128 x 128 block below the
// tile's diagonal as four 64 x 64 quads; waves 4-7 take the lower halves of
// the two 128 x 128 diagonal blocks, five 32 x 32 blocks each.  P = Q for
// these tiles, so one LDS operand serves both sides of every product: a
// wave reads NF fragment rows and multiplies the pairs (IA[b], IB[b]).
template <int PAT> struct DiagPattern;
template <> struct DiagPattern<0> {   // quad: rows {a0, a1} x cols {b0, b1}
  static constexpr int NF = 4, NB = 4;
  static constexpr int IA[NB] = {0, 0, 1, 1}, IB[NB] = {2, 3, 2, 3};
};
template <> struct DiagPattern<1> {   // rows {96, 0, 32, 64}: blocks (3,0) (3,1) (3,2) (3,3) (0,0)
  static constexpr int NF = 4, NB = 5;
  static constexpr int IA[NB] = {0, 0, 0, 0, 1}, IB[NB] = {1, 2, 3, 0, 1};
};
template <> struct DiagPattern<2> {   // rows {64, 0, 32}: blocks (2,0) (2,1) (2,2) (1,0) (1,1)
  static constexpr int NF = 3, NB = 5;
  static constexpr int IA[NB] = {0, 0, 0, 2, 2}, IB[NB] = {1, 2, 0, 1, 2};
};

// Off-diagonal tile t (0 <= t < n_p (n_p - 1) / 2) of a lower triangle of n_p
// tile rows, in the order of the split Gram's units: blocks of 8 tile columns,
// and within a block row by row (rows i > j).  The XCD-grouped launch hands
// each XCD 32 consecutive units, all of one K half: a column block then
// reads its few row panels (the block's columns and the rows it spans) over
// one K range in step, and the XCD's L2 serves the repeats.  Modelled per
// XCD at 4096 (16 tile rows): 77% of the panel reads are repeats, against 62%
// for tile rows with both halves side by side.
__device__ __forceinline__ void syrk_offdiag_tile(int64_t np, int64_t t, int64_t& ti, int64_t& tj) {
  for (int64_t j0 = 0;; j0 += 8) {
    const int64_t j1 = min(j0 + 8, np - 1);   // columns [j0, j1) of this block
    for (int64_t i = j0 + 1; i < np; ++i) {
      const int64_t c = min(i, j1) - j0;      // tiles of row i in the block
      if (t < c) {
        ti = i;
        tj = j0 + t;
        return;
      }
      t -= c;
    }
  }
}

// Sign bit of a stored value: 1 iff !(u < 0) on its encoding (+0, -0 and NaN
// give 1), the rule of the 1-bit packing.
__device__ __forceinline__ uint32_t nonneg_bf16(bf16_t h) { return !(h > 0x8000u && h <= 0xff80u); }
__device__ __forceinline__ uint32_t nonneg_f32(uint32_t u) { return !(u > 0x80000000u && u <= 0xff800000u); }

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), in order.
template <typename F, int... I>
__device__ __forceinline__ void static_for_seq(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

// Value of lane i - SH of the same 16-lane DPP row, 0 where that lane lies
// before the row's first lane.
template <int SH>
__device__ __forceinline__ uint32_t row_shr_or(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x110 | SH, 0xf, 0xf, true));
}

// Column of slab element (row, col) in the epilogue's LDS slab: the column is
// XOR-swizzled by the row's group of four (bits 3 and up), which keeps 4-column
// groups contiguous for 16-byte accesses and spreads the transposed reads
// (four rows 4c..4c+3 at one column, eight columns per instruction) over the
// banks.  MASK = 7 for slabs of 64 or more columns, 3 for 32.
template <int MASK>
__device__ __forceinline__ int slab_col(int row, int col) {
  return col ^ (((row >> 2) & MASK) << 3);
}

// Epilogue scalars of batch entry `batch`: C = alpha * acc + beta * Z, with the
// folded Frobenius scale (1/sumsq for the Gram of M, 1/sqrt(sumsq) for the
// product with M, 0 for a zero matrix)
__device__ __forceinline__ void epilogue_scale(const GemmArgs& g, int64_t batch, float& alpha, float& beta) {
  alpha = g.alpha;
  beta = g.beta;
  if (g.scale_sumsq != nullptr) {
    const double ss = static_cast<double>(g.scale_sumsq[batch * g.stride_sumsq]);
    const float f = ss == 0.0 ? 0.0f : static_cast<float>(g.scale_mode == 1 ? 1.0 / ss : 1.0 / sqrt(ss));
    alpha *= f;
    beta *= f;
  }
}

// One work unit (workgroup `bid` of the launch's unit list) of a product; the
// kernels below are thin wrappers, so that one launch can hold units of two
// tile shapes.
// `bid` is the unit's index within its batch entry `batch`, already in the
// XCD-grouped order (the kernels below remap the launch's flat workgroup
// index once, over all batch entries).
template <int BM, int BN, int WM, int WN, int S, bool SYRK, bool NN, int EPI>
__device__ __forceinline__ void gemm_dma_unit(const GemmArgs& g, const int64_t bid, const int64_t batch,
                                              char* lds) {
  using C_ = DmaTile<BM, BN, WM, WN, S, NN>;
  constexpr int FM = C_::FM, FN = C_::FN, BK = C_::BK;
  // symmetric products: square tiles, or (HALVES) the column halves of the
  // off-diagonal square tiles of a BM-tiled lower triangle
  constexpr bool HALVES = SYRK && BN * 2 == BM;
  static_assert(!SYRK || ((BM == BN || HALVES) && !NN), "symmetric products are NT with square or half tiles");
  static_assert(WN >= 64, "the epilogue slab swizzle (slab_col<7>) needs 64 or more columns per wave");
  // split units exist only in the 256 x 256-tile Gram (the one long symmetric
  // product); the other instantiations carry none of their code
  constexpr bool SPLITS = SYRK && EPI == EPI_STORE && BM == 256 && C_::W == 8;
  // lower-half diagonal units (the split Gram's, and SPLIT_DIAG launches)
  constexpr bool DIAGS = SYRK && BM == 256 && BN == 256 && C_::W == 8;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keeps DMA addresses scalar
  const int wm0 = (wave / (BN / WN)) * WM;
  const int wn0 = (wave % (BN / WN)) * WN;
  const int frow = lane & 31, fgrp = lane >> 5;
  const int64_t KT = g.K / BK;

  // ---- work unit: a whole tile, one K half of a tile, or a diagonal lower half ----
  int64_t tm, tn;
  int64_t kb = 0, ke = KT;      // k-tiles of this unit
  int64_t sidx = -1;            // split tile index (K halves only)
  int half = 0;
  bool diag_half = false;
  const int64_t tiles = SYRK ? (g.M / BM) * (g.M / BM + 1) / 2 : (g.M / BM) * (g.N / BN);
  if (SPLITS && g.split_mode == SPLIT_SYRK && kSyrkHalfOrder) {
    // n_p^2 units per batch entry: the first K halves of the T = n_p (n_p - 1) / 2
    // off-diagonal tiles, then their second halves, then the lower halves of
    // the n_p diagonal tiles (syrk_offdiag_tile gives the tile order)
    const int64_t np = g.M / BM, T = np * (np - 1) / 2;
    const int64_t v = bid;
    if (v < 2 * T) {
      half = v >= T ? 1 : 0;
      const int64_t t = v - half * T;
      syrk_offdiag_tile(np, t, tm, tn);
      sidx = batch * T + t;
    } else {
      tm = tn = v - 2 * T;
      diag_half = true;
    }
  } else if (SPLITS && g.split_mode == SPLIT_SYRK) {
    // n_p^2 units per batch entry: tile row i holds units [i^2, (i+1)^2): the two
    // K halves of tiles (i, 0..i-1), then the lower half of diagonal tile (i, i)
    const int64_t np = g.M / BM;
    const int64_t v = bid;
    int64_t i = static_cast<int64_t>(sqrt(double(v)));
    while (i * i > v) --i;
    while ((i + 1) * (i + 1) <= v) ++i;
    const int64_t w = v - i * i;
    tm = i;
    if (w == 2 * i) {
      tn = i;
      diag_half = true;
    } else {
      tn = w >> 1;
      half = static_cast<int>(w & 1);
      sidx = batch * (np * (np - 1) / 2) + i * (i - 1) / 2 + tn;
    }
  } else if (DIAGS && g.split_mode == SPLIT_DIAG) {
    // unit v: the lower half of diagonal tile v
    tm = tn = bid;
    diag_half = true;
  } else if (DIAGS && g.split_mode == SPLIT_TRI) {
    // units [0, n_p (n_p - 1) / 2): off-diagonal tile (i, j), j < i, row by row;
    // then the lower half of diagonal tile v - n_p (n_p - 1) / 2
    const int64_t np = g.M / BM, noff = np * (np - 1) / 2;
    if (bid < noff) {
      int64_t i = static_cast<int64_t>((1.0 + sqrt(1.0 + 8.0 * double(bid))) * 0.5);
      while (i * (i - 1) / 2 > bid) --i;
      while ((i + 1) * i / 2 <= bid) ++i;
      tm = i;
      tn = bid - i * (i - 1) / 2;
    } else {
      tm = tn = bid - noff;
      diag_half = true;
    }
  } else if (HALVES) {
    // n_p (n_p - 1) units per batch entry: unit v is column half v & 1 of
    // off-diagonal tile t = v >> 1 = i (i - 1) / 2 + j (row i, column j < i);
    // both halves of a tile are neighbours in the XCD-grouped order
    const int64_t np = g.M / BM;
    const int64_t v = bid;
    const int64_t t = v >> 1;
    int64_t i = static_cast<int64_t>((1.0 + sqrt(1.0 + 8.0 * double(t))) * 0.5);
    while (i * (i - 1) / 2 > t) --i;
    while ((i + 1) * i / 2 <= t) ++i;
    tm = i;
    tn = 2 * (t - i * (i - 1) / 2) + (v & 1);   // in units of BN columns
  } else {
    tile_coords<BM, BN, SYRK>(g, bid, tm, tn);
  }
  if (sidx >= 0) {
    kb = half ? KT / 2 : 0;
    ke = half ? KT : KT / 2;
  }
  // the decode is uniform across the workgroup: keep it in scalar registers so
  // the k loop bound and the tile addresses stay scalar
  tm = __builtin_amdgcn_readfirstlane(static_cast<int>(tm));
  tn = __builtin_amdgcn_readfirstlane(static_cast<int>(tn));
  kb = __builtin_amdgcn_readfirstlane(static_cast<int>(kb));
  ke = __builtin_amdgcn_readfirstlane(static_cast<int>(ke));
  sidx = __builtin_amdgcn_readfirstlane(static_cast<int>(sidx));
  half = __builtin_amdgcn_readfirstlane(half);
  diag_half = __builtin_amdgcn_readfirstlane(static_cast<int>(diag_half)) != 0;
  const int64_t nk = ke - kb;
  const int64_t m0 = tm * BM, n0 = tn * BN;

  // ---- DMA sources: tile origin plus a 32-bit per-lane offset (elements) ----
  const bf16_t* Pt = static_cast<const bf16_t*>(g.P) + batch * g.strideP + m0 * g.K + kb * BK;
  const bf16_t* Qt = static_cast<const bf16_t*>(g.Q) + batch * g.strideQ +
                     (NN ? n0 + kb * BK * g.ld : n0 * g.K + kb * BK);
  // P (and NT Q): block b covers rows 16b..16b+15; lane -> row 16b + lane/4, slot lane%4
  uint32_t p_off[C_::P_DMA], q_off[C_::Q_DMA];
#pragma unroll
  for (int i = 0; i < C_::P_DMA; ++i) {
    const int r = 16 * (wave * C_::P_DMA + i) + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    p_off[i] = uint32_t(r) * uint32_t(g.K) + c * 8;
  }
#pragma unroll
  for (int i = 0; i < C_::Q_DMA; ++i) {
    const int b = wave * C_::Q_DMA + i;
    if (!NN) {
      const int r = 16 * b + (lane >> 2);
      const int c = (lane & 3) ^ ((r >> 2) & 3);
      q_off[i] = uint32_t(r) * uint32_t(g.K) + c * 8;
    } else {
      constexpr int ROW_CHUNKS = BN / 8;           // 16-byte chunks per k-row
      constexpr int ROWS_PER_BLOCK = 64 / ROW_CHUNKS;
      const int r = ROWS_PER_BLOCK * b + lane / ROW_CHUNKS;
      const int c = nrow_slot(lane % ROW_CHUNKS, r);   // the slot is an involution
      q_off[i] = uint32_t(r) * uint32_t(g.ld) + c * 8;
    }
  }
  const uint32_t lds_base =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)lds));

  // stages live at byte offsets 0, STAGE_BYTES, ..., (S-1) STAGE_BYTES of the
  // ring; the loops advance offsets incrementally (no modulo by S per k-step)
  auto ring_next = [](uint32_t o) {
    o += C_::STAGE_BYTES;
    return o == uint32_t(S * C_::STAGE_BYTES) ? 0u : o;
  };
  auto issue_p = [&](int64_t kt, uint32_t off) {
    const uint32_t st = lds_base + off;
    const bf16_t* pk = Pt + kt * BK;
#pragma unroll
    for (int q = 0; q < C_::P_DMA; ++q) dma16(pk + p_off[q], st + (wave * C_::P_DMA + q) * 1024);
  };
  auto issue_stage = [&](int64_t kt, uint32_t off) {
    issue_p(kt, off);
    const uint32_t st = lds_base + off;
    const bf16_t* qk = NN ? Qt + kt * BK * g.ld : Qt + kt * BK;
#pragma unroll
    for (int q = 0; q < C_::Q_DMA; ++q)
      dma16(qk + q_off[q], st + C_::P_BYTES + (wave * C_::Q_DMA + q) * 1024);
  };

  if constexpr (DIAGS) {
    if (diag_half) {
      // ---- lower half of a diagonal tile: P = Q, only P is staged ----
      auto body = [&](auto pat_c) {
        constexpr int PAT = decltype(pat_c)::value;
        using DP = DiagPattern<PAT>;
        constexpr int NF = DP::NF, NB = DP::NB;
        int rows[NF];   // tile-relative first row of each fragment row-block
        if constexpr (PAT == 0) {
          const int qr = wave >> 1, qc = wave & 1;
          rows[0] = 128 + 64 * qr; rows[1] = 160 + 64 * qr; rows[2] = 64 * qc; rows[3] = 64 * qc + 32;
        } else {
          const int base = wave >= 6 ? 128 : 0;
          if constexpr (PAT == 1) {
            rows[0] = base + 96; rows[1] = base; rows[2] = base + 32; rows[3] = base + 64;
          } else {
            rows[0] = base + 64; rows[1] = base; rows[2] = base + 32;
          }
        }
        f32x16_t dacc[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int v = 0; v < 16; ++v) dacc[b][v] = 0.0f;
        u32x4_t f[2][NF];
        auto read = [&](const char* st, int ks, u32x4_t (&fr)[NF]) {
          const int chunk = 2 * ks + fgrp;
#pragma unroll
          for (int r = 0; r < NF; ++r)
            fr[r] = *reinterpret_cast<const u32x4_t*>(st + krow_off(rows[r] + frow, chunk));
        };
        auto mma = [&](const u32x4_t (&fr)[NF]) {
#pragma unroll
          for (int b = 0; b < NB; ++b) Mfma<bf16_t>::mma(fr[DP::IA[b]], fr[DP::IB[b]], dacc[b]);
        };
        auto interleave = [&]() {
#pragma unroll
          for (int i = 0; i < (NF > NB ? NF : NB); ++i) {
            if (i < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (i < NB) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          }
        };
        constexpr int D = C_::P_DMA;
#pragma unroll
        for (int s = 0; s < S - 1; ++s)
          if (s < nk) issue_p(s, uint32_t(s) * C_::STAGE_BYTES);
        if (nk >= S - 1) wait_vm_barrier<D * (S - 2)>();
        else wait_vm_barrier<0>();
        read(lds, 0, f[0]);
        int64_t it = 0;
        uint32_t o_cur = 0, o_iss = uint32_t(S - 1) * C_::STAGE_BYTES;
        for (; it < nk - (S - 1); ++it) {
          const uint32_t o_nxt = ring_next(o_cur);
          lds_reads_done();
          read(lds + o_cur, 1, f[1]);
          mma(f[0]);
          interleave();
          wait_vm_barrier<D * (S - 3)>();
          issue_p(it + S - 1, o_iss);
          lds_reads_done();
          read(lds + o_nxt, 0, f[0]);
          mma(f[1]);
          interleave();
          o_cur = o_nxt;
          o_iss = ring_next(o_iss);
        }
        for (; it < nk; ++it) {
          const uint32_t o_nxt = ring_next(o_cur);
          read(lds + o_cur, 1, f[1]);
          mma(f[0]);
          if (it + 1 < nk) {
            wait_vm_barrier<0>();
            read(lds + o_nxt, 0, f[0]);
          }
          mma(f[1]);
          o_cur = o_nxt;
        }
        // epilogue: each 32 x 32 block through a per-wave LDS slab; off-diagonal
        // blocks are also stored mirrored
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // the ring is free
        const bool use_z = EPI != EPI_STORE && g.beta != 0.0f;
        float alpha, beta;
        epilogue_scale(g, batch, alpha, beta);
        bf16_t* C = static_cast<bf16_t*>(g.C) + batch * g.strideC;
        const bf16_t* Z = static_cast<const bf16_t*>(g.Z) + batch * g.strideZ;
        constexpr int LDB = 36;
        float* wl = reinterpret_cast<float*>(lds) + wave * 32 * LDB;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int ra = rows[DP::IA[b]], rb = rows[DP::IB[b]];
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int row = 8 * (v >> 2) + 4 * fgrp + (v & 3);
            wl[row * LDB + slab_col<3>(row, frow)] = dacc[b][v];
          }
          uint2 zr[4];
          if (use_z) {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const int q = lane + 64 * p, row = q >> 3, c4 = q & 7;
              zr[p] = *reinterpret_cast<const uint2*>(Z + (m0 + ra + row) * g.ld + n0 + rb + 4 * c4);
            }
          }
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int q = lane + 64 * p, row = q >> 3, c4 = q & 7;
            const float4 a = *reinterpret_cast<const float4*>(wl + row * LDB + slab_col<3>(row, 4 * c4));
            float o[4] = {a.x * alpha, a.y * alpha, a.z * alpha, a.w * alpha};
            if (use_z) {
              o[0] = fmaf(beta, __uint_as_float(zr[p].x << 16), o[0]);
              o[1] = fmaf(beta, __uint_as_float(zr[p].x & 0xffff0000u), o[1]);
              o[2] = fmaf(beta, __uint_as_float(zr[p].y << 16), o[2]);
              o[3] = fmaf(beta, __uint_as_float(zr[p].y & 0xffff0000u), o[3]);
            }
            const uint32_t w0 = uint32_t(f32_to_bf16(o[0])) | (uint32_t(f32_to_bf16(o[1])) << 16);
            const uint32_t w1 = uint32_t(f32_to_bf16(o[2])) | (uint32_t(f32_to_bf16(o[3])) << 16);
            *reinterpret_cast<uint2*>(C + (m0 + ra + row) * g.ld + n0 + rb + 4 * c4) = make_uint2(w0, w1);
            if (ra != rb) *reinterpret_cast<float4*>(wl + row * LDB + slab_col<3>(row, 4 * c4)) = make_float4(o[0], o[1], o[2], o[3]);
          }
          if (ra != rb) {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const int q = lane + 64 * p, mr = q >> 3, c4 = q & 7;
              float o[4];
#pragma unroll
              for (int t = 0; t < 4; ++t) o[t] = wl[(4 * c4 + t) * LDB + slab_col<3>(4 * c4 + t, mr)];
              const uint32_t w0 = uint32_t(f32_to_bf16(o[0])) | (uint32_t(f32_to_bf16(o[1])) << 16);
              const uint32_t w1 = uint32_t(f32_to_bf16(o[2])) | (uint32_t(f32_to_bf16(o[3])) << 16);
              *reinterpret_cast<uint2*>(C + (n0 + rb + mr) * g.ld + m0 + ra + 4 * c4) = make_uint2(w0, w1);
            }
          }
        }
      };
      if (wave < 4) body(std::integral_constant<int, 0>{});
      else if (wave & 1) body(std::integral_constant<int, 2>{});
      else body(std::integral_constant<int, 1>{});
      return;
    }
  }

  auto read_frags = [&](const char* st, int ks, u32x4_t (&fa)[FM], u32x4_t (&fb)[FN]) {
    const int chunk = 2 * ks + fgrp;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      fa[i] = *reinterpret_cast<const u32x4_t*>(st + krow_off(wm0 + i * 32 + frow, chunk));
    if (!NN) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
        fb[j] = *reinterpret_cast<const u32x4_t*>(st + C_::P_BYTES + krow_off(wn0 + j * 32 + frow, chunk));
    } else {
      const int gi = lane & 15, G = lane >> 4;
      const int k0 = ks * 16 + 8 * (G >> 1) + (gi >> 2);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = wn0 + j * 32 + 16 * (G & 1) + 4 * (gi & 3);   // first of 4 columns
        const int c = col >> 3, half = (col & 7) * 2;                    // chunk, byte in chunk
        const char* b0 = st + C_::P_BYTES + k0 * (BN * 2) + (nrow_slot(c, k0) << 4) + half;
        const int k1 = k0 + 4;
        const char* b1 = st + C_::P_BYTES + k1 * (BN * 2) + (nrow_slot(c, k1) << 4) + half;
        fb[j] = read_tr_pair(b0, b1);
      }
    }
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  u32x4_t fa[2][FM], fb[2][FN];
  auto mma_all = [&](const u32x4_t (&a)[FM], const u32x4_t (&b)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) Mfma<bf16_t>::mma(a[i], b[j], acc[i][j]);
  };

  // Ask the scheduler to alternate one LDS fragment read with one MFMA, so
  // the reads for the next k-step run under the current MFMAs.
  auto interleave = [&]() {
    constexpr int NDS = FM + (NN ? 2 * FN : FN), NMF = FM * FN;
#if MUON_GEMM_INTERLEAVE == 1
#pragma unroll
    for (int i = 0; i < (NDS > NMF ? NDS : NMF); ++i) {
      if (i < NDS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (i < NMF) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
#elif MUON_GEMM_INTERLEAVE == 2
    // two reads per MFMA over the first MFMAs, then MFMAs only, so the last
    // reads have several MFMAs' time to land before the next k-step uses them
    static_assert(NDS % 2 == 0, "reads come in pairs");
    constexpr int PAIRS = NDS / 2;
#pragma unroll
    for (int i = 0; i < PAIRS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    if (NMF > PAIRS) __builtin_amdgcn_sched_group_barrier(0x008, NMF - PAIRS, 0);
#endif
  };

  // prologue: stages 0 .. S-2 in flight, stage 0 resident
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nk) issue_stage(s, uint32_t(s) * C_::STAGE_BYTES);
  if (nk >= S - 1) wait_vm_barrier<C_::D * (S - 2)>();
  else wait_vm_barrier<0>();
  read_frags(lds, 0, fa[0], fb[0]);
  int64_t it = 0;
  uint32_t o_cur = 0, o_iss = uint32_t(S - 1) * C_::STAGE_BYTES;   // stages it and it + S - 1
  // steady state (branch-free, so the compiler's LDS wait counts stay exact):
  // stages it+1 .. it+S-2 are in flight on entry, stage it+S-1 is issued here
  for (; it < nk - (S - 1); ++it) {
    const uint32_t o_nxt = ring_next(o_cur);
    lds_reads_done();
    read_frags(lds + o_cur, 1, fa[1], fb[1]);
    mma_all(fa[0], fb[0]);
    interleave();
    wait_vm_barrier<C_::D * (S - 3)>();
    issue_stage(it + S - 1, o_iss);
    lds_reads_done();
    read_frags(lds + o_nxt, 0, fa[0], fb[0]);
    mma_all(fa[1], fb[1]);
    interleave();
    o_cur = o_nxt;
    o_iss = ring_next(o_iss);
  }
  // drain: nothing left to issue
  for (; it < nk; ++it) {
    const uint32_t o_nxt = ring_next(o_cur);
    read_frags(lds + o_cur, 1, fa[1], fb[1]);
    mma_all(fa[0], fb[0]);
    if (it + 1 < nk) {
      wait_vm_barrier<0>();
      read_frags(lds + o_nxt, 0, fa[0], fb[0]);
    }
    mma_all(fa[1], fb[1]);
    o_cur = o_nxt;
  }

  // ---- K halves: both halves store their fp32 partial tile, then count in;
  // the second to arrive adds the other half (for two terms the sum does not
  // depend on the order) and runs the epilogue, then clears the counter.
  // The partials move as device-coherent relaxed atomic stores and loads
  // (global_store / global_load with sc1: written through, and read past, the
  // per-XCD L2), so no L2 write-back or invalidation is needed; the
  // vmcnt(0) wait puts every partial store before the counter increment, and
  // the loads are issued only after the increment has returned ----
  if constexpr (SPLITS) if (sidx >= 0) {
    // The tile's arrival counter (zero on entry): each half adds 1 when its
    // k-loop is done.  The first to arrive stores its fp32 partial tile as
    // device-coherent relaxed atomic stores (global_store sc1, written
    // through past the per-XCD L2), waits for them (vmcnt(0)), adds 2 and
    // leaves; the count then reaches 4 once both have arrived and the partial
    // is in memory.  The second waits for 4, reads the partial with coherent
    // loads, adds it (two terms: the order does not change the sum), clears
    // the counter and runs the epilogue.  The first half depends on no other
    // workgroup after its loop, so the wait ends; it is also bounded.
    __shared__ int split_arrival;   // only this instantiation holds it: the others may use all 160 KB
    constexpr int PER_WAVE = FM * FN * 4 * kWave;   // 16-byte pieces per wave
    typedef unsigned long long u64_t;
    u64_t* part = reinterpret_cast<u64_t*>(g.partials + sidx * int64_t(BM * BN)) + 2 * (wave * PER_WAVE + lane);
    if (tid == 0)
      split_arrival = __hip_atomic_fetch_add(g.counters + sidx, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (split_arrival == 0) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int o = 2 * ((i * FN + j) * 4 + q) * kWave;
            const u64_t lo = (u64_t(__float_as_uint(acc[i][j][4 * q + 1])) << 32) | __float_as_uint(acc[i][j][4 * q]);
            const u64_t hi = (u64_t(__float_as_uint(acc[i][j][4 * q + 3])) << 32) | __float_as_uint(acc[i][j][4 * q + 2]);
            __hip_atomic_store(part + o, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(part + o + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's partial stores are done
      __syncthreads();
      if (tid == 0) __hip_atomic_fetch_add(g.counters + sidx, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;   // the other half finishes the tile
    }
    __shared__ int split_ready;
    if (tid == 0) {
      int ready = 0;
      for (int spin = 0; spin < g.spin_limit; ++spin) {
        // an agent-scope atomic load observes the agent-scope adds to the
        // same word (the compiler emits a coherent sc1 load, and turns an
        // add of zero into the same load)
        if (__hip_atomic_load(g.counters + sidx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 4) {
          ready = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      split_ready = ready;
      // the wait ran out: report it and leave the tile (and its counter) alone
      if (!ready) __hip_atomic_store(g.split_error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!split_ready) return;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int o = 2 * ((i * FN + j) * 4 + q) * kWave;
          const u64_t lo = __hip_atomic_load(part + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const u64_t hi = __hip_atomic_load(part + o + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          acc[i][j][4 * q] += __uint_as_float(static_cast<uint32_t>(lo));
          acc[i][j][4 * q + 1] += __uint_as_float(static_cast<uint32_t>(lo >> 32));
          acc[i][j][4 * q + 2] += __uint_as_float(static_cast<uint32_t>(hi));
          acc[i][j][4 * q + 3] += __uint_as_float(static_cast<uint32_t>(hi >> 32));
        }
    if (tid == 0) __hip_atomic_store(g.counters + sidx, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- epilogue, staged through LDS one 32-row slab at a time ----
  // 32x32 accumulator layout: value v of lane l is row 8*(v/4) + 4*(l/32) +
  // (v%4), column l%32 of the fragment.  Staging turns the column-per-lane
  // layout into 4-column chunks per lane, so the addend Z is read with one
  // 8-byte load per chunk, all issued before any is used, and the outputs
  // are written as 8-byte chunks; a second pass over the staged values writes
  // the mirrored tile (symmetric products) or the transposed U (final
  // iteration of a tall matrix).
  bf16_t* C = static_cast<bf16_t*>(g.C) + batch * g.strideC;
  const bf16_t* Z = static_cast<const bf16_t*>(g.Z) + batch * g.strideZ;
  const bool mirror = SYRK && (HALVES || tm != tn);
  const bool second_pass = mirror || (EPI == EPI_FINAL && g.transpose_out);
  const bool use_z = EPI != EPI_STORE && g.beta != 0.0f;
  // B X products: the addend's residual, and the output's residual
  const bool use_zl = !SYRK && use_z && g.Zl != nullptr;
  const bool write_cl = !SYRK && EPI == EPI_AXPBY && g.Cl != nullptr;
  const bf16_t* Zl = static_cast<const bf16_t*>(g.Zl) + batch * g.strideZ;
  bf16_t* Cl = static_cast<bf16_t*>(g.Cl) + batch * g.strideC;
  float alpha, beta;
  epilogue_scale(g, batch, alpha, beta);
  constexpr int LDW = C_::LDW;
  constexpr int CPR = WN / 4;                 // 4-column chunks per slab row
  constexpr int NP = 32 * CPR / 64;           // chunks per lane and slab
  constexpr int NP2 = WN * 8 / 64;            // transposed chunks per lane and slab
  // The addend of slab i + 1 is loaded while slab i is staged and written
  // (double-buffered registers), and slab 0's before the barrier below, so
  // its latency is not paid once per slab.
  constexpr int RPP = 64 / CPR;               // slab rows per chunk index
  static_assert(64 % CPR == 0, "a lane keeps its column across chunks");
  const int rb = lane / CPR, cc = lane % CPR;
  // EPI_FINAL: 4-entry chunks of U are whole and aligned when its row length is
  // a multiple of 4 (all chunk columns are multiples of 4)
  const bool u_vec = EPI == EPI_FINAL && g.l_valid % 4 == 0;
  uint2 zbuf[2][NP];
  auto load_z = [&](int i, uint2 (&dst)[NP]) __attribute__((always_inline)) {
    const bf16_t* zrow = Z + (m0 + wm0 + i * 32 + rb) * g.ld + n0 + wn0 + 4 * cc;
#pragma unroll
    for (int p = 0; p < NP; ++p) dst[p] = *reinterpret_cast<const uint2*>(zrow + int64_t(p * RPP) * g.ld);
  };
  if (use_z) load_z(0, zbuf[0]);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // the ring is free
  float* wl = reinterpret_cast<float*>(lds) + wave * 32 * LDW;
  // one 32-row slab per accumulator row block; expanded at compile time (the
  // unroller gives up on bodies this large, and the accumulators must keep
  // constant indices to stay in registers)
  auto slab = [&](auto I_) __attribute__((always_inline)) {
    constexpr int i = decltype(I_)::value;
    const int64_t r0 = m0 + wm0 + i * 32, c0 = n0 + wn0;
    // chunk p of a lane: slab row rb + p * RPP, columns 4 cc .. 4 cc + 3 (the
    // column does not depend on p, so addresses advance by a uniform stride)
    const int64_t gcol = c0 + 4 * cc;
    // the addend's residual (only some iterations carry one): loaded per slab,
    // issued before the accumulators go to LDS so that store hides its latency
    uint2 zl[NP];
    if constexpr (!SYRK) {
      if (use_zl) {
        const bf16_t* zlrow = Zl + (r0 + rb) * g.ld + gcol;
#pragma unroll
        for (int p = 0; p < NP; ++p) zl[p] = *reinterpret_cast<const uint2*>(zlrow + int64_t(p * RPP) * g.ld);
      }
    }
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        {
          const int row = 8 * (v >> 2) + 4 * fgrp + (v & 3);
          wl[row * LDW + slab_col<7>(row, j * 32 + frow)] = acc[i][j][v];
        }
    if constexpr (i + 1 < FM)
      if (use_z) load_z(i + 1, zbuf[(i + 1) & 1]);
    const uint2 (&zr)[NP] = zbuf[i & 1];
    bf16_t* crow = C + (r0 + rb) * g.ld + gcol;
    bf16_t* clrow = Cl + (r0 + rb) * g.ld + gcol;
    auto pass1 = [&](auto SG_) __attribute__((always_inline)) {
      constexpr bool SG = decltype(SG_)::value;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int row = rb + p * RPP;
        float4 a = *reinterpret_cast<const float4*>(wl + row * LDW + slab_col<7>(row, 4 * cc));
        float o[4] = {a.x * alpha, a.y * alpha, a.z * alpha, a.w * alpha};
        if constexpr (!SYRK) {
          if (use_zl) {
            o[0] = fmaf(beta, __uint_as_float(zl[p].x << 16), o[0]);
            o[1] = fmaf(beta, __uint_as_float(zl[p].x & 0xffff0000u), o[1]);
            o[2] = fmaf(beta, __uint_as_float(zl[p].y << 16), o[2]);
            o[3] = fmaf(beta, __uint_as_float(zl[p].y & 0xffff0000u), o[3]);
          }
        }
        if (use_z) {
          o[0] = fmaf(beta, __uint_as_float(zr[p].x << 16), o[0]);
          o[1] = fmaf(beta, __uint_as_float(zr[p].x & 0xffff0000u), o[1]);
          o[2] = fmaf(beta, __uint_as_float(zr[p].y << 16), o[2]);
          o[3] = fmaf(beta, __uint_as_float(zr[p].y & 0xffff0000u), o[3]);
        }
        const int64_t grow = r0 + row;
        if constexpr (SG) {
          // sign bits of the stored values (bit 1 iff !(u < 0) on the stored
          // encoding, as sign_pack tests it).  A 16-lane DPP row holds 64
          // consecutive columns of one row, 4 per lane: each lane places its
          // nibble in the word's low or high half, an OR-scan over the row
          // (shifts 1, 2, 4, 8) gathers the word in the row's last lane.
          const bool f32_out = EPI == EPI_FINAL && g.u_dtype == MUON_F32;
          uint32_t nib = 0;
#pragma unroll
          for (int t = 0; t < 4; ++t)
            nib |= (f32_out ? nonneg_f32(__float_as_uint(o[t])) : nonneg_bf16(f32_to_bf16(o[t]))) << t;
          const int rl = lane & 15;
          uint32_t lo = rl < 8 ? nib << (4 * rl) : 0u;
          uint32_t hi = rl < 8 ? 0u : nib << (4 * (rl - 8));
          lo |= row_shr_or<1>(lo); hi |= row_shr_or<1>(hi);
          lo |= row_shr_or<2>(lo); hi |= row_shr_or<2>(hi);
          lo |= row_shr_or<4>(lo); hi |= row_shr_or<4>(hi);
          lo |= row_shr_or<8>(lo); hi |= row_shr_or<8>(hi);
          if (rl == 15 && grow < g.bits_rows && g.col0 + gcol < g.bits_cols)
            *reinterpret_cast<uint2*>(g.bits + batch * g.stride_bits + (grow * g.bits_cols + g.col0 + gcol) / 64) =
                make_uint2(lo, hi);
        }
        if (EPI == EPI_FINAL) {
          if (g.U != nullptr && !g.transpose_out && grow < g.s_valid) {
            const int64_t idx = batch * g.strideU + grow * g.l_valid + g.col0 + gcol;
            if (u_vec) {
              // whole chunk inside U, 8- (bf16) or 16-byte (fp32) aligned
              if (g.col0 + gcol < g.l_valid) {
                if (g.u_dtype == MUON_BF16) {
                  const uint32_t w0 = uint32_t(f32_to_bf16(o[0])) | (uint32_t(f32_to_bf16(o[1])) << 16);
                  const uint32_t w1 = uint32_t(f32_to_bf16(o[2])) | (uint32_t(f32_to_bf16(o[3])) << 16);
                  *reinterpret_cast<uint2*>(static_cast<bf16_t*>(g.U) + idx) = make_uint2(w0, w1);
                } else {
                  *reinterpret_cast<float4*>(static_cast<float*>(g.U) + idx) = make_float4(o[0], o[1], o[2], o[3]);
                }
              }
            } else {
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                if (g.col0 + gcol + t < g.l_valid) {
                  if (g.u_dtype == MUON_BF16) static_cast<bf16_t*>(g.U)[idx + t] = f32_to_bf16(o[t]);
                  else static_cast<float*>(g.U)[idx + t] = o[t];
                }
              }
            }
          }
        } else if (SYRK || g.C != nullptr) {
          bf16_t h[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) h[t] = f32_to_bf16(o[t]);
          const uint32_t w0 = uint32_t(h[0]) | (uint32_t(h[1]) << 16);
          const uint32_t w1 = uint32_t(h[2]) | (uint32_t(h[3]) << 16);
          *reinterpret_cast<uint2*>(crow + int64_t(p * RPP) * g.ld) = make_uint2(w0, w1);
          if constexpr (!SYRK) {
            if (write_cl) {
              bf16_t r[4];
#pragma unroll
              for (int t = 0; t < 4; ++t) r[t] = f32_to_bf16(o[t] - bf16_to_f32(h[t]));
              const uint32_t l0 = uint32_t(r[0]) | (uint32_t(r[1]) << 16);
              const uint32_t l1 = uint32_t(r[2]) | (uint32_t(r[3]) << 16);
              *reinterpret_cast<uint2*>(clrow + int64_t(p * RPP) * g.ld) = make_uint2(l0, l1);
            }
          }
        }
        if (second_pass) *reinterpret_cast<float4*>(wl + row * LDW + slab_col<7>(row, 4 * cc)) = make_float4(o[0], o[1], o[2], o[3]);
      }
    };
    if constexpr (!SYRK && WN % 64 == 0) {
      if (g.bits != nullptr) pass1(std::true_type{});
      else pass1(std::false_type{});
    } else {
      pass1(std::false_type{});
    }
    if (second_pass) {
      // mirrored / transposed: row c0 + mr receives slab rows 4*c4 .. 4*c4+3
#pragma unroll
      for (int p = 0; p < NP2; ++p) {
        const int q = lane + 64 * p, mr = q / 8, c4 = q % 8;
        float o[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) o[t] = wl[(4 * c4 + t) * LDW + slab_col<7>(4 * c4 + t, mr)];
        const int64_t orow = c0 + mr, ocol = r0 + 4 * c4;
        if (EPI == EPI_FINAL) {
          if (g.U != nullptr && g.col0 + orow < g.l_valid) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              if (ocol + t < g.s_valid) {
                const int64_t idx = batch * g.strideU + (g.col0 + orow) * g.s_valid + ocol + t;
                if (g.u_dtype == MUON_BF16) static_cast<bf16_t*>(g.U)[idx] = f32_to_bf16(o[t]);
                else static_cast<float*>(g.U)[idx] = o[t];
              }
            }
          }
        } else {
          const uint32_t w0 = uint32_t(f32_to_bf16(o[0])) | (uint32_t(f32_to_bf16(o[1])) << 16);
          const uint32_t w1 = uint32_t(f32_to_bf16(o[2])) | (uint32_t(f32_to_bf16(o[3])) << 16);
          *reinterpret_cast<uint2*>(C + orow * g.ld + ocol) = make_uint2(w0, w1);
        }
      }
    }
  };
  static_for<FM>(slab);
}

// Workgroups are dispatched round-robin over the 8 XCDs by their flat index.
// The flat index over all (batch entry, unit) pairs is remapped so that each
// XCD runs a contiguous range of them: whole batch entries, or neighbouring
// tiles of one entry, whose operand panels then meet in that XCD's L2.  (With
// the batch as a second grid dimension, every small matrix's tiles were dealt
// to all 8 XCDs, and each L2 held panels of every matrix: 128 matrices of
// 1024^2 ran their products at a 42-46% L2 hit rate.)
__device__ __forceinline__ void flat_unit(int64_t units, int64_t nbatch, int64_t& batch, int64_t& bid) {
  const int64_t u = xcd_remap(blockIdx.x, units * nbatch);
  batch = __builtin_amdgcn_readfirstlane(static_cast<int>(u / units));
  bid = __builtin_amdgcn_readfirstlane(static_cast<int>(u % units));
}

template <int BM, int BN, int WM, int WN, int S, bool SYRK, bool NN, int EPI>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void gemm_dma_kernel(GemmArgs g, int64_t units,
                                                                              int64_t nbatch) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  int64_t batch, bid;
  flat_unit(units, nbatch, batch, bid);
  gemm_dma_unit<BM, BN, WM, WN, S, SYRK, NN, EPI>(g, bid, batch, lds);
}

// B X whose last round runs as 128 x 256 column strips, in one launch:
// workgroups [0, n1) take the 256 x 256 tiles of g1, the others the strips
// of g2, so a CU starts its strip as soon as its last whole tile is done
// instead of after the slowest tile of the chip and a second launch.  n1 is a
// multiple of the XCD count, so both parts keep their XCD-grouped tile order.
template <int EPI>
__global__ __launch_bounds__(512) void gemm_apply_mixed_kernel(GemmArgs g1, GemmArgs g2, int64_t n1,
                                                               int64_t n2) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int64_t b = blockIdx.x;
  if (b < n1) gemm_dma_unit<256, 256, 64, 128, 4, false, true, EPI>(g1, xcd_remap(b, n1), 0, lds);
  else gemm_dma_unit<128, 256, 64, 64, 4, false, true, EPI>(g2, xcd_remap(b - n1, n2), 0, lds);
}

// A symmetric product as n_p^2 units per batch entry (n_p = M / 256), one
// round when they fit the CUs: workgroups [0, n1 = n_p (n_p - 1)) take the
// column halves (256 x 128) of the off-diagonal 256 x 256 tiles, the other
// n_p the lower halves of the diagonal tiles.  No unit depends on another.
template <int EPI>
__global__ __launch_bounds__(512) void gemm_syrk_halves_kernel(GemmArgs gh, GemmArgs gd, int64_t n1,
                                                               int64_t units, int64_t nbatch) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  int64_t batch, b;
  flat_unit(units, nbatch, batch, b);
  if (b < n1) gemm_dma_unit<256, 128, 64, 64, 4, true, false, EPI>(gh, b, batch, lds);
  else gemm_dma_unit<256, 256, 64, 128, 4, true, false, EPI>(gd, b - n1, batch, lds);
}

// Number of workgroups of one batch entry.
template <int BM, int BN, bool SYRK>
inline int64_t tiles_of(const GemmArgs& g) {
  if (SYRK) {
    const int64_t t = g.M / BM;
    return t * (t + 1) / 2;
  }
  return (g.M / BM) * (g.N / BN);
}

// The dynamic LDS limit is an attribute of the kernel on the current device:
// set it once per device (`configured` holds one bit per device).  Setting it
// twice is harmless, so threads that race here only repeat the call.
template <typename K>
int set_lds_limit(K kern, int bytes, std::atomic<uint64_t>& configured) {
  const uint64_t bit = device_bit(current_device());
  if (bit == 0 || !(configured.load(std::memory_order_acquire) & bit)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess)
      return MUON_ELAUNCH;
    configured.fetch_or(bit, std::memory_order_release);
  }
  return MUON_OK;
}

template <typename T, int BM, int BN, int WM, int WN, bool SYRK, bool NN, int EPI>
int launch(const GemmArgs& g, int64_t batch, hipStream_t st) {
  using C_ = Tile<T, BM, BN, WM, WN>;
  const int64_t blocks = tiles_of<BM, BN, SYRK>(g);
  if (blocks == 0 || batch == 0) return MUON_OK;
  if (g.bits != nullptr) return MUON_EINVAL;   // sign bits: DMA kernel only
  auto kern = gemm_kernel<T, BM, BN, WM, WN, SYRK, NN, EPI>;
  static std::atomic<uint64_t> configured{0};   // devices with the LDS limit set
  if (set_lds_limit(kern, C_::LDS_BYTES, configured) != MUON_OK) return MUON_ELAUNCH;
  launch_kernel(kern, dim3(blocks, batch), dim3(C_::NT), C_::LDS_BYTES, st, g);
  return launch_status();
}

// ---------------------------------------------------------------------------
// Split planning (host).  The scratch of a split launch is a fixed block of
// kSplitCounters int arrival counters, then one fp32 BM x BN partial tile
// per split tile (written by the first K half to finish).  Every plan has at most kSplitCounters split tiles
// (SPLIT_SYRK: n_p (n_p - 1) / 2 * batch < n_p^2 * batch / 2 <= 128), so one
// scratch serves launches of any shape without its counters moving.
// ---------------------------------------------------------------------------
constexpr int64_t kSplitMaxUnits = 256;   // SPLIT_SYRK: at most this many units per launch
// SPLIT_SYRK only for contractions of at least this many 32-wide k-tiles:
// measured on MI355X, the Gram of 4096 x 14336 (448 k-tiles) gains a fifth
// while the 4096^3 polynomial product (128 k-tiles) does not gain, the
// exchange of the halves costing as much as the idle CUs
constexpr int64_t kSplitMinKTiles = 256;
constexpr int64_t kSplitCounters = 128;
// the counter block: kSplitCounters arrival counters, then the error word
// (int index kSplitCounters), padded to 1 KB
constexpr int64_t kSplitWords = kSplitCounters + 1;
constexpr size_t kSplitCounterBytes = 1024;
static_assert(kSplitWords * sizeof(int) <= kSplitCounterBytes, "counter block");

// polls of a split wait, set for the process (tests lower it to drive the
// give-up path with every kernel still exiting normally)
inline std::atomic<int>& split_spin_limit() {
  static std::atomic<int> limit{kSplitSpinLimit};
  return limit;
}

struct SplitPlan {
  int mode;
  int64_t units;         // workgroups per batch entry
  int64_t split_tiles;   // split tiles of the whole launch
};

struct Scratch {         // caller-provided split scratch (base == nullptr: no splitting)
  char* base;
  size_t bytes;
  int* error = nullptr;  // the error word a wait that runs out sets (null: the one after base's counters)
};

inline size_t split_scratch_bytes(int64_t split_tiles, int bm, int bn) {
  if (split_tiles <= 0) return 0;
  return kSplitCounterBytes + static_cast<size_t>(split_tiles) * bm * bn * sizeof(float);
}

// cus > 0: the plan for a device with that many CUs (one 256 x 256-tile
// workgroup per CU).  cus == 0: the largest plan any device can get, which
// sizes the scratch.
template <int BM, int BN, bool SYRK>
SplitPlan plan_split(int64_t M, int64_t N, int64_t K, int64_t batch, int64_t cus) {
  const int64_t tiles = SYRK ? (M / BM) * (M / BM + 1) / 2 : (M / BM) * (N / BN);
  SplitPlan p{SPLIT_NONE, tiles, 0};
  if (!SYRK || BM != 256 || K / 32 < kSplitMinKTiles || tiles == 0 || batch <= 0) return p;
  const int64_t np = M / BM;
  const int64_t limit = cus > 0 ? std::min(cus, kSplitMaxUnits) : kSplitMaxUnits;
  if (np * np * batch <= limit) p = SplitPlan{SPLIT_SYRK, np * np, np * (np - 1) / 2 * batch};
  return p;
}

// compute units of the current device (cached per device)
inline int64_t device_cus() {
  static std::atomic<int> cache[kMaxTrackedDevices];   // 0 = not yet queried
  const int dev = current_device();
  if (dev < 0) return 0;
  if (dev < kMaxTrackedDevices) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < kMaxTrackedDevices && n > 0) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <int BM, int BN, int WM, int WN, int S, bool SYRK, bool NN, int EPI>
int launch_dma(GemmArgs g, int64_t batch, hipStream_t st, const Scratch& sc) {
  using C_ = DmaTile<BM, BN, WM, WN, S, NN>;
  const int64_t tpb = tiles_of<BM, BN, SYRK>(g);
  if (tpb == 0 || batch == 0) return MUON_OK;
  // sign bits come from 16-lane groups that each hold 64 columns of one row
  if (g.bits != nullptr && (SYRK || WN % 64 != 0 || g.bits_cols % 64 != 0)) return MUON_EINVAL;
  int64_t grid = tpb;
  if (g.ld == 0) g.ld = g.N;
  g.split_mode = SPLIT_NONE;
  // only the instantiation that carries the split units may be given a split plan
  constexpr bool SPLITS = SYRK && EPI == EPI_STORE && BM == 256 && C_::W == 8;
  if (SPLITS && sc.base != nullptr) {
    const int64_t cus = device_cus();
    const SplitPlan p = cus > 0 ? plan_split<BM, BN, SYRK>(g.M, g.N, g.K, batch, cus)
                                : SplitPlan{SPLIT_NONE, tpb, 0};
    if (p.mode != SPLIT_NONE) {
      if (sc.bytes < split_scratch_bytes(p.split_tiles, BM, BN) || p.split_tiles > kSplitCounters)
        return MUON_EWORKSPACE;
      g.split_mode = p.mode;
      g.counters = reinterpret_cast<int*>(sc.base);
      g.split_error = sc.error != nullptr ? sc.error : g.counters + kSplitCounters;
      g.spin_limit = split_spin_limit().load(std::memory_order_relaxed);
      g.partials = reinterpret_cast<float*>(sc.base + kSplitCounterBytes);
      grid = p.units;
    }
  }
  // several rounds of whole symmetric tiles: diagonal tiles as lower halves
  constexpr bool DIAGS = SYRK && BM == 256 && BN == 256 && C_::W == 8;
  if (DIAGS && kSyrkTri && g.split_mode == SPLIT_NONE && g.M / BM >= 2) {
    const int64_t cus = device_cus();
    if (cus > 0 && tpb * batch > cus) g.split_mode = SPLIT_TRI;
  }
  auto kern = gemm_dma_kernel<BM, BN, WM, WN, S, SYRK, NN, EPI>;
  static std::atomic<uint64_t> configured{0};   // devices with the LDS limit set
  if (set_lds_limit(kern, C_::LDS_BYTES, configured) != MUON_OK) return MUON_ELAUNCH;
  if (grid * batch > INT32_MAX) return MUON_EINVAL;
  launch_kernel(kern, dim3(grid * batch), dim3(C_::NT), C_::LDS_BYTES, st, g, grid, batch);
  return launch_status();
}

// The mixed launch above: g1 covers the first n1 = tiles of 256 x 256, g2 the
// strips; both already carry their row stride, column offset and pointers.
template <int EPI>
int launch_apply_mixed(GemmArgs g1, GemmArgs g2, hipStream_t st) {
  using A_ = DmaTile<256, 256, 64, 128, 4, true>;
  using B_ = DmaTile<128, 256, 64, 64, 4, true>;
  const int64_t n1 = tiles_of<256, 256, false>(g1), n2 = tiles_of<128, 256, false>(g2);
  if (n1 % kXcds != 0) return MUON_EINVAL;
  if (g1.bits != nullptr && (g1.bits_cols % 64 != 0 || g2.bits_cols % 64 != 0)) return MUON_EINVAL;
  g1.split_mode = g2.split_mode = SPLIT_NONE;
  constexpr int lds_bytes = A_::LDS_BYTES > B_::LDS_BYTES ? A_::LDS_BYTES : B_::LDS_BYTES;
  auto kern = gemm_apply_mixed_kernel<EPI>;
  static std::atomic<uint64_t> configured{0};
  if (set_lds_limit(kern, lds_bytes, configured) != MUON_OK) return MUON_ELAUNCH;
  launch_kernel(kern, dim3(n1 + n2, 1), dim3(512), lds_bytes, st, g1, g2, n1, n2);
  return launch_status();
}

// The halves launch above for g (a symmetric product on 256 x 256 tiles,
// M a multiple of 512).
template <int EPI>
int launch_syrk_halves(GemmArgs g, int64_t batch, hipStream_t st) {
  using H_ = DmaTile<256, 128, 64, 64, 4, false>;
  using D_ = DmaTile<256, 256, 64, 128, 4, false>;
  const int64_t np = g.M / 256;
  if (np < 2 || g.M % 256 != 0 || g.N != g.M || batch == 0) return MUON_EINVAL;
  if (g.ld == 0) g.ld = g.N;
  GemmArgs gh = g, gd = g;
  gh.split_mode = SPLIT_NONE;
  gd.split_mode = SPLIT_DIAG;
  const int64_t n1 = np * (np - 1);
  constexpr int lds_bytes = H_::LDS_BYTES > D_::LDS_BYTES ? H_::LDS_BYTES : D_::LDS_BYTES;
  auto kern = gemm_syrk_halves_kernel<EPI>;
  static std::atomic<uint64_t> configured{0};
  if (set_lds_limit(kern, lds_bytes, configured) != MUON_OK) return MUON_ELAUNCH;
  if ((n1 + np) * batch > INT32_MAX) return MUON_EINVAL;
  launch_kernel(kern, dim3((n1 + np) * batch), dim3(512), lds_bytes, st, gh, gd, n1, n1 + np, batch);
  return launch_status();
}

}  // namespace gemm
}  // namespace muon
