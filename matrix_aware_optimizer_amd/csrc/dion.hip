// Dion step on the GPU (the Dion page's algorithm: a low-rank power iteration
// with error feedback).  Per weight matrix X (m x n, fp32) with momentum M,
// gradient G and the previous right factor Q (n x r):
//
//   B = M + G                                (in place in M)
//   P = orth(B Q)                            (thin QR factor, Cholesky-QR twice)
//   R = B^T P
//   M = B - (1 - mu) P R^T                   (error feedback)
//   Q = ColumnNormalize(R)
//   X = X - eta P Q^T
//
// These products are skinny (r <= 192 against m, n of a few thousand) and
// small, so they run in fp32 on one tiled kernel with arbitrary element
// strides (the transposes are strides, never copies).  orth(P): the Gram
// P^T P is factored L L^T in LDS by one workgroup per matrix, L is inverted
// in place, and P <- P L^-T; the second pass restores orthogonality lost to
// fp32 rounding.  A column whose Gram-Schmidt residual (the Cholesky pivot)
// is at most 1e-4 of its own norm counts as dependent and is zeroed, and so
// is every column after the first min(m, n) independent ones (the rank bound
// of B Q, which the fp32 Gram's rounding could not show at that tolerance).
#include <algorithm>
#include <vector>

#include "common.h"

namespace muon {
namespace {

constexpr int kDionMaxRank = MUON_DION_MAX_RANK;
constexpr float kDependentTol = 1e-4f;

// ---------------------------------------------------------------------------
// C[b](i,j) = alpha * sum_k A[b](i,k) B[b](k,j) + beta * Z[b](i,j)
// A(i,k) = A[b*sA + i*a_i + k*a_k], B(k,j) = B[b*sB + k*b_k + j*b_j];
// C and Z row-major with their own leading dimensions (Z may alias C).
// ---------------------------------------------------------------------------
struct DGemm {
  const float* A;
  int64_t sA, a_i, a_k;
  const float* B;
  int64_t sB, b_k, b_j;
  const float* Z;
  int64_t sZ, ldz;
  float* C;
  int64_t sC, ldc;
  int64_t M, N, K;
  float alpha, beta;
  // dion_gemm_dma48_kernel only: the left operand is A + A2 (each sum rounded
  // once to fp32), A2 with A's element strides and batch stride sA2, and the
  // sum is written to Aout (A's strides and batch stride), whose entries this
  // product alone reads
  const float* A2 = nullptr;
  int64_t sA2 = 0;
  float* Aout = nullptr;
};

// the exact sum of two fp32 values rounded once to fp32
__device__ __forceinline__ float add_once(float a, float b) {
  return static_cast<float>(static_cast<double>(a) + static_cast<double>(b));
}

constexpr int kDT = 64;        // output tile
constexpr int kDK = 32;        // k per LDS tile
constexpr int kDPitch = 96;    // LDS row pitch (floats): the two k-rows an MFMA operand read
                               // touches land 32 banks apart

// One operand tile (64 rows of the output dimension x 32 of k, stored k-major
// in LDS) per thread: 8 elements.  When the operand is contiguous along k
// (CK: 4 threads per row, 8 k each) or along the output dimension (4 x 8 per
// k-row), the 8 elements are two 16-byte loads; a group that leaves the
// matrix falls back to guarded scalar loads.  `vec` (checked on the host:
// contiguous dimension stride 1, the other stride and the batch stride
// multiples of 4, 16-byte aligned base) enables the 16-byte loads.
struct TileLoad {
  const float* base;   // this batch entry
  int64_t s_out, s_k;  // element strides along the output dimension and along k
  int64_t n_out, K;    // extents
  bool ck;             // contiguous along k
  bool vec;
  __device__ __forceinline__ void fetch(int tid, int64_t o0, int64_t k0, float (&r)[8]) const {
    int oo, kk;       // first element of this thread's group of 8 (along the contiguous dim)
    if (ck) { oo = tid >> 2; kk = (tid & 3) * 8; } else { kk = tid >> 3; oo = (tid & 7) * 8; }
    const int64_t go = o0 + oo, gk = k0 + kk;
    const float* ptr = base + go * s_out + gk * s_k;
    const bool full = ck ? (go < n_out && gk + 8 <= K) : (gk < K && go + 8 <= n_out);
    if (vec && full) {
      const float4 x = *reinterpret_cast<const float4*>(ptr);
      const float4 y = *reinterpret_cast<const float4*>(ptr + 4);
      r[0] = x.x; r[1] = x.y; r[2] = x.z; r[3] = x.w; r[4] = y.x; r[5] = y.y; r[6] = y.z; r[7] = y.w;
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int64_t o = ck ? go : go + q, k = ck ? gk + q : gk;
        r[q] = (o < n_out && k < K) ? base[o * s_out + k * s_k] : 0.0f;
      }
    }
  }
  __device__ __forceinline__ void store(int tid, float (&r)[8], float (*T)[kDPitch]) const {
    int oo, kk;
    if (ck) { oo = tid >> 2; kk = (tid & 3) * 8; } else { kk = tid >> 3; oo = (tid & 7) * 8; }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (ck) T[kk + q][oo] = r[q];
      else T[kk][oo + q] = r[q];
    }
  }
};

// The tile is computed on fp32 matrix cores: wave w owns the 32 x 32 quarter
// (w / 2, w % 2) and issues v_mfma_f32_32x32x2f32 over k, lane l supplying
// A(row l % 32, k + l / 32) and B(k + l / 32, column l % 32); accumulator
// value v of lane l is row 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32.
// The next k-tile is fetched into registers while the current one is used.
// Split k: with `splits` > 1, blockIdx.z = batch * splits + s covers the
// k-tiles of range s and writes its raw sums to part[s][b] (M x N row-major);
// reduce_kernel adds the ranges in order and applies alpha, beta.
__global__ __launch_bounds__(256) void dion_gemm_kernel(DGemm g, int splits, float* part, int a_vec, int b_vec) {
  __shared__ __attribute__((aligned(16))) float As[kDK][kDPitch];
  __shared__ __attribute__((aligned(16))) float Bs[kDK][kDPitch];
  const int64_t b = blockIdx.z / splits;
  const int sp = blockIdx.z % splits;
  const int64_t i0 = int64_t(blockIdx.y) * kDT, j0 = int64_t(blockIdx.x) * kDT;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wi = (wave >> 1) * 32, wj = (wave & 1) * 32;
  const TileLoad la{g.A + b * g.sA, g.a_i, g.a_k, g.M, g.K, g.a_k == 1, a_vec != 0};
  const TileLoad lb{g.B + b * g.sB, g.b_j, g.b_k, g.N, g.K, g.b_k == 1, b_vec != 0};
  const int64_t ktiles = (g.K + kDK - 1) / kDK;
  const int64_t kt0 = ktiles * sp / splits, kt1 = ktiles * (sp + 1) / splits;
  f32x16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  float ra[8], rb[8];
  if (kt0 < kt1) {
    la.fetch(tid, i0, kt0 * kDK, ra);
    lb.fetch(tid, j0, kt0 * kDK, rb);
  }
  for (int64_t kt = kt0; kt < kt1; ++kt) {
    la.store(tid, ra, As);
    lb.store(tid, rb, Bs);
    __syncthreads();
    if (kt + 1 < kt1) {
      la.fetch(tid, i0, (kt + 1) * kDK, ra);
      lb.fetch(tid, j0, (kt + 1) * kDK, rb);
    }
#pragma unroll
    for (int k = 0; k < kDK; k += 2) {
      const float a = As[k + (lane >> 5)][wi + (lane & 31)];
      const float bb = Bs[k + (lane >> 5)][wj + (lane & 31)];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bb, acc, 0, 0, 0);
    }
    __syncthreads();
  }
  const int64_t col = j0 + wj + (lane & 31);
  if (splits > 1) {
    float* Pp = part + (int64_t(sp) * gridDim.z / splits + b) * g.M * g.N;
    if (col < g.N) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = i0 + wi + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < g.M) Pp[row * g.N + col] = acc[v];
      }
    }
    return;
  }
  float* C = g.C + b * g.sC;
  const float* Z = g.Z ? g.Z + b * g.sZ : nullptr;
  if (col < g.N) {
    // all 16 addend values are loaded before the first store: Z may be C
    // itself (the in-place updates), and a lane reads only the entries it
    // writes, so no store can change a value another lane still has to read.
    // Interleaved, each load would wait for the store before it.
    float z[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t row = i0 + wi + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      z[v] = (g.beta != 0.0f && row < g.M) ? Z[row * g.ldz + col] : 0.0f;
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t row = i0 + wi + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (row >= g.M) continue;
      float o = g.alpha * acc[v];
      if (g.beta != 0.0f) o = fmaf(g.beta, z[v], o);
      C[row * g.ldc + col] = o;
    }
  }
}

// ---------------------------------------------------------------------------
// The same product with its operands staged by global -> LDS DMA
// (global_load_lds_dwordx4: 16 bytes per lane straight into LDS, no register
// round trip) in an S-stage ring, so S - 1 k-tiles are in flight while one is
// multiplied.  Used when both operands allow 16-byte chunks: stride 1 along
// one dimension, the other strides multiples of 4 floats, 16-byte aligned
// base, and the chunked extent (k for a k-contiguous operand, the output
// dimension otherwise) a multiple of 4.
//
// An operand tile (64 of the output dimension x 32 of k, 8 KB) is 512 chunks;
// DMA instruction i of wave w fills chunks [64 (2 w + i), +64), one per lane.
//  * k-contiguous operand ("ck"): LDS rows of 32 k (128 bytes) per output
//    index o, chunk c (k = 4c .. 4c + 3) of row o at slot c ^ (o & 7).  A
//    lane reads 4 k-values of one row with ds_read_b128; the 8 lanes of a
//    read group touch 8 different slots, so all 32 banks.
//  * output-contiguous operand ("co"): LDS rows of 64 o (256 bytes) per k,
//    unswizzled; a half-wave reads 32 consecutive floats of one row.
// k-values are paired across the two half-waves of v_mfma_f32_32x32x2f32 as
// (k, k + 4) within each 8-deep group, so a ck lane's ds_read_b128 feeds 4
// MFMAs; a co lane reads the matching row for each MFMA.
// Chunks past the contraction (k >= K) load from a 16 KB page of zeros in the
// workspace (spread over it by slot and workgroup), so both operands are zero
// there and the tail adds nothing; chunks past the output dimension load a
// clamped valid chunk, whose products land only in rows or columns that are
// never stored.
// The waits are explicit: each wave issues exactly 4 DMA instructions per
// k-tile, so while S - 2 younger stages are in flight s_waitcnt vmcnt(4 (S -
// 2)) means its chunks of the oldest stage have landed, and the s_barrier
// after it means every wave's have; the last S - 1 iterations issue nothing
// and wait for everything.
// ---------------------------------------------------------------------------
// Tile (x, y, z) of a DMA product's workgroup.  Workgroups go to the 8 XCDs
// round-robin by their flat index (x fastest); the flat index is remapped so
// that each XCD takes a contiguous range of tiles, and the tiles that share a
// row panel of the left operand (consecutive x: B Q's rank-wide row at rank
// 96 or 192) meet in one XCD's L2 instead of being read from memory by
// several.
#ifndef MUON_DION_XCD
#define MUON_DION_XCD 1
#endif
struct DTile {
  int64_t x, y, z;
};
__device__ __forceinline__ DTile dion_tile() {
  const int64_t X = gridDim.x, Y = gridDim.y;
  const int64_t n = X * Y * int64_t(gridDim.z);
  int64_t t = blockIdx.x + X * (blockIdx.y + Y * int64_t(blockIdx.z));
  if (MUON_DION_XCD) {
    const int64_t full = n / 8 * 8;
    if (t < full) t = (t % 8) * (full / 8) + t / 8;
  }
  return DTile{t % X, (t / X) % Y, t / (X * Y)};
}

constexpr int kDmaTileBytes = kDT * kDK * 4;   // one operand tile: 8 KB
constexpr int kZeroPageFloats = 4096;          // the workspace's page of zeros: 16 KB

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane from global memory to LDS bytes [lds_addr + 16 lane).  M0
// is set here and used by nothing else in the kernel (no other LDS-DMA, no
// relative register indexing, no messages).
__device__ __forceinline__ void dion_dma16(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g),
               "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void dion_wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// the slot of chunk c in row o of a half tile is c ^ half_swizzle(o)
__device__ __forceinline__ int half_swizzle(int o) { return (o + (o >> 2)) & 3; }

struct DmaOperand {
  const float* base;     // this batch entry
  int64_t s_out, s_k;    // element strides along the output dimension and along k
  int64_t n_out, K;
  // global address of the chunk that LDS chunk slot p of the tile at (o0, k0) holds
  template <bool CK>
  __device__ __forceinline__ const float* chunk(int p, int64_t o0, int64_t k0, const float* zero, int zspread) const {
    int64_t o, k;
    if constexpr (CK) {
      const int row = p >> 3, c = (p & 7) ^ (row & 7);
      o = o0 + row;
      k = k0 + 4 * c;
      if (o >= n_out) o = n_out - 1;
    } else {
      k = k0 + (p >> 4);
      o = o0 + 4 * (p & 15);
      if (o >= n_out) o = n_out - 4;
    }
    // past the contraction: a chunk of the zero page, spread over its 16 KB by
    // slot and workgroup so that the tail reads of many workgroups do not all
    // land on the same few cache lines
    return k < K ? base + o * s_out + k * s_k : zero + 4 * ((p + 67 * zspread) & (kZeroPageFloats / 4 - 1));
  }
  // a half tile of a k-contiguous operand: 16 k-values (64 bytes) per output
  // index, chunk c of index o at slot c ^ ((o + o / 4) % 4), so that the eight
  // rows one 16-byte read phase touches fall in distinct banks
  __device__ __forceinline__ const float* chunk16(int p, int64_t o0, int64_t k0, const float* zero,
                                                  int zspread) const {
    const int row = p >> 2, c = (p & 3) ^ half_swizzle(row);
    int64_t o = o0 + row;
    if (o >= n_out) o = n_out - 1;
    const int64_t k = k0 + 4 * c;
    return k < K ? base + o * s_out + k * s_k : zero + 4 * ((p + 67 * zspread) & (kZeroPageFloats / 4 - 1));
  }
};

template <int S, bool ACK, bool BCK, bool ZPRE>
__global__ __launch_bounds__(256) void dion_gemm_dma_kernel(DGemm g, int splits, float* part, const float* zero) {
  extern __shared__ __attribute__((aligned(16))) char dsm[];
  const DTile T = dion_tile();
  const int64_t b = T.z / splits;
  const int sp = static_cast<int>(T.z % splits);
  const int64_t i0 = T.y * kDT, j0 = T.x * kDT;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wi = (wave >> 1) * 32, wj = (wave & 1) * 32;
  const int half = lane >> 5, l32 = lane & 31;
  const DmaOperand oa{g.A + b * g.sA, g.a_i, g.a_k, g.M, g.K};
  const DmaOperand ob{g.B + b * g.sB, g.b_j, g.b_k, g.N, g.K};
  const int64_t ktiles = (g.K + kDK - 1) / kDK;
  const int64_t kt0 = ktiles * sp / splits, kt1 = ktiles * (sp + 1) / splits;
  const int nk = static_cast<int>(kt1 - kt0);
  const uint32_t lds0 =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)dsm));
  const int zspread = static_cast<int>((T.x + 3 * T.y + 5 * T.z) & 63);
  // stage s: A tile at s * 16 KB, B tile 8 KB after it
  auto issue = [&](int stage, int64_t kt) __attribute__((always_inline)) {
    const int64_t k0 = kt * kDK;
    const uint32_t sa = lds0 + stage * 2 * kDmaTileBytes, sb = sa + kDmaTileBytes;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int slot0 = 64 * (2 * wave + i);
      // beyond the last k-tile: dummies from the zero page (k0 >= K)
      dion_dma16(oa.chunk<ACK>(slot0 + lane, i0, k0, zero, zspread), sa + 16 * slot0);
      dion_dma16(ob.chunk<BCK>(slot0 + lane, j0, k0, zero, zspread + 1), sb + 16 * slot0);
    }
  };
  f32x16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  // the first S - 1 stages (those past the range are not issued; the waits
  // below count only issued ones)
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nk) issue(s, kt0 + s);
  // ZPRE (an addend and no split): the addend is read before the contraction,
  // so its latency overlaps the k-loop (the m x n updates have a short k and a
  // full tile of addend each).  Z may be C itself: every lane reads only the
  // entries it writes, and reads them all before its first store.
  const int64_t col = j0 + wj + l32;
  const float* Z = g.Z ? g.Z + b * g.sZ : nullptr;
  float z[16];
  auto load_z = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t row = i0 + wi + 8 * (v >> 2) + 4 * half + (v & 3);
      z[v] = (g.beta != 0.0f && row < g.M && col < g.N) ? Z[row * g.ldz + col] : 0.0f;
    }
  };
  if constexpr (ZPRE) load_z();
  for (int it = 0; it < nk; ++it) {
    // steady state: S - 2 younger stages are in flight behind the one needed;
    // in the last S - 1 iterations nothing is issued any more, so wait for all
    if (it + S - 1 < nk) {
      dion_wait_vm_barrier<4 * (S - 2)>();
      issue((it + S - 1) % S, kt0 + it + S - 1);
    } else {
      dion_wait_vm_barrier<0>();
    }
    const char* ta = dsm + (it % S) * 2 * kDmaTileBytes;
    const char* tb = ta + kDmaTileBytes;
#pragma unroll
    for (int gk = 0; gk < 4; ++gk) {
      float av[4], bv[4];
      if constexpr (ACK) {
        const int row = wi + l32, c = 2 * gk + half;
        const float4 v = *reinterpret_cast<const float4*>(ta + row * 128 + ((c ^ (row & 7)) << 4));
        av[0] = v.x; av[1] = v.y; av[2] = v.z; av[3] = v.w;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          av[j] = *reinterpret_cast<const float*>(ta + ((8 * gk + j + 4 * half) * kDT + wi + l32) * 4);
      }
      if constexpr (BCK) {
        const int row = wj + l32, c = 2 * gk + half;
        const float4 v = *reinterpret_cast<const float4*>(tb + row * 128 + ((c ^ (row & 7)) << 4));
        bv[0] = v.x; bv[1] = v.y; bv[2] = v.z; bv[3] = v.w;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bv[j] = *reinterpret_cast<const float*>(tb + ((8 * gk + j + 4 * half) * kDT + wj + l32) * 4);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[j], bv[j], acc, 0, 0, 0);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // every stage has landed
  if (splits > 1) {
    float* Pp = part + (int64_t(sp) * gridDim.z / splits + b) * g.M * g.N;
    if (col < g.N) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = i0 + wi + 8 * (v >> 2) + 4 * half + (v & 3);
        if (row < g.M) Pp[row * g.N + col] = acc[v];
      }
    }
    return;
  }
  float* C = g.C + b * g.sC;
  if constexpr (!ZPRE) load_z();
  if (col < g.N) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t row = i0 + wi + 8 * (v >> 2) + 4 * half + (v & 3);
      if (row >= g.M) continue;
      float o = g.alpha * acc[v];
      if (g.beta != 0.0f) o = fmaf(g.beta, z[v], o);
      C[row * g.ldc + col] = o;
    }
  }
}

// A 64 x 16 NB output tile on 16 x 16 blocks: NB = 3 for output widths that
// are multiples of 48 but not of 64 (rank 48 or 96, where 64-wide tiles would
// compute a quarter or a third of padding), and one tile as wide as the output
// (NB = r / 16) for B Q with B = M + G formed in the product.  Wave w owns rows
// 16 w .. 16 w + 15 and all 16 NB columns as NB blocks on
// v_mfma_f32_16x16x4f32: lane l supplies A(16 w + l % 16, k) and B(k, 16 j +
// l % 16) for the product's k-slot l / 16 and holds rows 4 (l / 16) .. + 3 of
// column l % 16.  Operands are staged as in dion_gemm_dma_kernel, B as
// ceil(16 NB / 64) tiles of 64 output indices (indices past the tile's width
// are loaded, clamped at the edge, and not used).  In each 16-deep k group g,
// k-slot q of product t (t = 0..3) is k = 16 g + 4 q + t, so a k-contiguous
// lane's 16-byte read feeds four products.
//
// KD16: stages of 16 k-values (half tiles, 4 KB per operand: k-contiguous ones
// in 64-byte rows, see DmaOperand::chunk16; the others as the first 16 k-rows
// of the 32-deep layout), for a ring of more, smaller stages.  The k ranges
// and the order of the products over k are those of 32-deep stages.
template <int S, int NB, bool ACK, bool BCK, bool ADDA, bool KD16 = false>
__global__ __launch_bounds__(256) void dion_gemm_dma48_kernel(DGemm g, int splits, float* part,
                                                              const float* zero) {
  constexpr int kW = 16 * NB, kSub = (kW + kDT - 1) / kDT;   // tile width, B tiles per stage
  constexpr int KD = KD16 ? 16 : kDK;                          // k-values per stage
  constexpr int kTB = KD16 ? kDmaTileBytes / 2 : kDmaTileBytes;   // bytes per operand tile
  constexpr int kSlots = KD16 ? 1 : 2;                         // DMA instructions per operand tile and wave
  extern __shared__ __attribute__((aligned(16))) char dsm[];
  const DTile T = dion_tile();
  const int64_t b = T.z / splits;
  const int sp = static_cast<int>(T.z % splits);
  const int64_t i0 = T.y * kDT, j0 = T.x * kW;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, q = lane >> 4;
  const int arow = 16 * wave + li;   // the tile row this lane supplies
  const DmaOperand oa{g.A + b * g.sA, g.a_i, g.a_k, g.M, g.K};
  const DmaOperand ob{g.B + b * g.sB, g.b_j, g.b_k, g.N, g.K};
  // ADDA: A's second term, staged like A (a third tile per stage)
  const DmaOperand oa2{ADDA ? g.A2 + b * g.sA2 : nullptr, g.a_i, g.a_k, g.M, g.K};
  constexpr int kTiles = 1 + kSub + (ADDA ? 1 : 0);   // A, the B tiles, A2
  const int64_t ktiles = (g.K + kDK - 1) / kDK;
  const int64_t kt0 = ktiles * sp / splits, kt1 = ktiles * (sp + 1) / splits;
  const int nk = static_cast<int>(kt1 - kt0) * (kDK / KD);   // stages of this range
  const int64_t kbase = kt0 * kDK;                           // its first k
  const uint32_t lds0 =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)dsm));
  const int zspread = static_cast<int>((T.x + 3 * T.y + 5 * T.z) & 63);
  // a k-contiguous operand's chunk in a half tile, else the 32-deep layout's
  auto chunk_of = [&](const DmaOperand& o, auto ck, int p, int64_t o0, int64_t k0, int zs)
      __attribute__((always_inline)) {
    constexpr bool CK = decltype(ck)::value;
    if constexpr (KD16 && CK) return o.chunk16(p, o0, k0, zero, zs);
    else return o.template chunk<CK>(p, o0, k0, zero, zs);
  };
  auto issue = [&](int stage, int it) __attribute__((always_inline)) {
    const int64_t k0 = kbase + int64_t(it) * KD;
    const uint32_t sa = lds0 + stage * kTiles * kTB, sb = sa + kTB;
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
      const int slot0 = 64 * (kSlots * wave + i);
      dion_dma16(chunk_of(oa, std::integral_constant<bool, ACK>{}, slot0 + lane, i0, k0, zspread), sa + 16 * slot0);
#pragma unroll
      for (int t = 0; t < kSub; ++t)
        dion_dma16(chunk_of(ob, std::integral_constant<bool, BCK>{}, slot0 + lane, j0 + kDT * t, k0, zspread + 1 + t),
                   sb + t * kTB + 16 * slot0);
      if constexpr (ADDA)
        dion_dma16(chunk_of(oa2, std::integral_constant<bool, ACK>{}, slot0 + lane, i0, k0, zspread + 5),
                   sb + kSub * kTB + 16 * slot0);
    }
  };
  // ADDA: the lane that reads an entry of A + A2 (one lane per entry: a wave
  // owns its 16 rows, and k-slot q reads chunk 4 g + q) writes it to Aout
  float* aout = ADDA ? g.Aout + b * g.sA + (i0 + arow) * g.a_i : nullptr;
  const bool arow_in = i0 + arow < g.M;
  f32x4_t acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nk) issue(s, s);
  for (int it = 0; it < nk; ++it) {
    if (it + S - 1 < nk) {
      dion_wait_vm_barrier<kSlots * kTiles * (S - 2)>();
      issue((it + S - 1) % S, it + S - 1);
    } else {
      dion_wait_vm_barrier<0>();
    }
    const char* ta = dsm + (it % S) * kTiles * kTB;
    const char* tb = ta + kTB;
#pragma unroll
    for (int gk = 0; gk < KD / 16; ++gk) {
      float av[4];
      if constexpr (ACK) {
        const int c = 4 * gk + q;
        const int o = KD16 ? arow * 64 + ((c ^ half_swizzle(arow)) << 4) : arow * 128 + ((c ^ (arow & 7)) << 4);
        const float4 v = *reinterpret_cast<const float4*>(ta + o);
        av[0] = v.x; av[1] = v.y; av[2] = v.z; av[3] = v.w;
        if constexpr (ADDA) {
          const float4 w = *reinterpret_cast<const float4*>(tb + kSub * kTB + o);
          av[0] = add_once(av[0], w.x); av[1] = add_once(av[1], w.y);
          av[2] = add_once(av[2], w.z); av[3] = add_once(av[3], w.w);
          const int64_t k = kbase + int64_t(it) * KD + 4 * c;
          if (arow_in && k < g.K)
            *reinterpret_cast<float4*>(aout + k) = make_float4(av[0], av[1], av[2], av[3]);
        }
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          av[t] = *reinterpret_cast<const float*>(ta + ((16 * gk + 4 * q + t) * kDT + arow) * 4);
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int bcol = (16 * j) % kDT + li;        // index within its B tile
        const char* tbj = tb + (16 * j / kDT) * kTB;   // the B tile holding block j
        float bv[4];
        if constexpr (BCK) {
          const int c = 4 * gk + q;
          const int o = KD16 ? bcol * 64 + ((c ^ half_swizzle(bcol)) << 4) : bcol * 128 + ((c ^ (bcol & 7)) << 4);
          const float4 v = *reinterpret_cast<const float4*>(tbj + o);
          bv[0] = v.x; bv[1] = v.y; bv[2] = v.z; bv[3] = v.w;
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            bv[t] = *reinterpret_cast<const float*>(tbj + ((16 * gk + 4 * q + t) * kDT + bcol) * 4);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[t], bv[t], acc[j], 0, 0, 0);
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // every stage has landed
  float* Pp = splits > 1 ? part + (int64_t(sp) * gridDim.z / splits + b) * g.M * g.N : nullptr;
  float* C = g.C + b * g.sC;
  const float* Z = g.Z ? g.Z + b * g.sZ : nullptr;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int64_t col = j0 + 16 * j + li;
    if (col >= g.N) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t row = i0 + 16 * wave + 4 * q + v;
      if (row >= g.M) continue;
      if (Pp != nullptr) {
        Pp[row * g.N + col] = acc[j][v];
      } else {
        float o = g.alpha * acc[j][v];
        if (g.beta != 0.0f) o = fmaf(g.beta, Z[row * g.ldz + col], o);
        C[row * g.ldc + col] = o;
      }
    }
  }
}

// Both rank-r updates of one step in one pass over the m x n tiles:
//   M <- M + alpha_m * P R^T   (error feedback, alpha_m = -(1 - mu))
//   X <- X + alpha_x * P Q^T   (alpha_x = -eta)
// P (m x r), R and Q (n x r) row-major, every operand k-contiguous.  A
// workgroup stages P's, R's and Q's tiles side by side in the DMA ring (three
// 8 KB tiles per stage), reads its tiles of M and X before the contraction,
// and runs the two products from one P fragment each; each product, and
// each output value, is computed as by dion_gemm_dma_kernel alone.
struct DUpdate2 {
  const float* P;
  int64_t sP, ldp;
  const float* R;
  int64_t sR, ldr;
  const float* Q;
  int64_t sQ, ldq;
  float* M;
  int64_t sM, ldm;
  float* X;
  int64_t sX, ldx;
  int64_t m, n, r;
  float alpha_m, alpha_x;
  float beta;   // 1: the addend's factor, a run-time value as in dion_gemm_dma_kernel, so that
                // alpha * acc and its sum with the addend round as they do there
};

// HALF (r = 16 or 48: one whole k-tile at most, then the 16-deep tail): the
// whole tile in one 24 KB stage and the tail in a 12 KB half stage of 64-byte
// rows, both issued at once; 36 KB of LDS, so four workgroups share a CU.
// The addends are read once the whole tile has landed, under its products.
//
// KD16: every stage 16 k-values deep (half tiles, 12 KB a stage), S of them,
// for the ranks HALF does not take; the addends are read first, so every wait
// counts only the stages' copies.  The order of the products over k is that
// of 32-deep stages.
template <int S, bool TAIL16, bool HALF, bool KD16 = false>
__global__ __launch_bounds__(256) void dion_update2_kernel(DUpdate2 u, const float* zero) {
  extern __shared__ __attribute__((aligned(16))) char dsm[];
  const DTile T = dion_tile();
  const int64_t b = T.z;
  const int64_t i0 = T.y * kDT, j0 = T.x * kDT;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wi = (wave >> 1) * 32, wj = (wave & 1) * 32;
  const int half = lane >> 5, l32 = lane & 31;
  const DmaOperand op{u.P + b * u.sP, u.ldp, 1, u.m, u.r};
  const DmaOperand orr{u.R + b * u.sR, u.ldr, 1, u.n, u.r};
  const DmaOperand oq{u.Q + b * u.sQ, u.ldq, 1, u.n, u.r};
  const int nk = static_cast<int>((u.r + kDK - 1) / kDK);
  const uint32_t lds0 =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)dsm));
  const int zspread = static_cast<int>((T.x + 3 * T.y + 5 * T.z) & 63);
  // stage s: P's tile, R's 8 KB after it, Q's after that (6 DMA instructions
  // per wave)
  auto issue = [&](int stage, int64_t kt) __attribute__((always_inline)) {
    const int64_t k0 = kt * kDK;
    const uint32_t sa = lds0 + stage * 3 * kDmaTileBytes;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int slot0 = 64 * (2 * wave + i);
      dion_dma16(op.chunk<true>(slot0 + lane, i0, k0, zero, zspread), sa + 16 * slot0);
      dion_dma16(orr.chunk<true>(slot0 + lane, j0, k0, zero, zspread + 1), sa + kDmaTileBytes + 16 * slot0);
      dion_dma16(oq.chunk<true>(slot0 + lane, j0, k0, zero, zspread + 2), sa + 2 * kDmaTileBytes + 16 * slot0);
    }
  };
  constexpr int kHalfBytes = kDmaTileBytes / 2;
  // the half stage after the whole one: P's, R's and Q's 4 KB (3 DMA
  // instructions per wave)
  auto issue_half = [&](int64_t kt) __attribute__((always_inline)) {
    const int64_t k0 = kt * kDK;
    const uint32_t sa = lds0 + 3 * kDmaTileBytes + 16 * 64 * wave;
    dion_dma16(op.chunk16(64 * wave + lane, i0, k0, zero, zspread), sa);
    dion_dma16(orr.chunk16(64 * wave + lane, j0, k0, zero, zspread + 1), sa + kHalfBytes);
    dion_dma16(oq.chunk16(64 * wave + lane, j0, k0, zero, zspread + 2), sa + 2 * kHalfBytes);
  };
  // KD16: stage s of the ring holds P's, R's and Q's half tiles of 16-deep
  // step `it` (3 DMA instructions per wave)
  auto issue16 = [&](int stage, int it) __attribute__((always_inline)) {
    const int64_t k0 = int64_t(it) * 16;
    const uint32_t sa = lds0 + stage * 3 * kHalfBytes + 16 * 64 * wave;
    dion_dma16(op.chunk16(64 * wave + lane, i0, k0, zero, zspread), sa);
    dion_dma16(orr.chunk16(64 * wave + lane, j0, k0, zero, zspread + 1), sa + kHalfBytes);
    dion_dma16(oq.chunk16(64 * wave + lane, j0, k0, zero, zspread + 2), sa + 2 * kHalfBytes);
  };
  f32x16_t am, ax;
#pragma unroll
  for (int v = 0; v < 16; ++v) am[v] = ax[v] = 0.0f;
  if constexpr (HALF) {
    if (nk == 2) issue(0, 0);
    issue_half(nk - 1);
    if (nk == 2) dion_wait_vm_barrier<3>();   // the whole tile has landed; the half stage may be in flight
  } else if constexpr (!KD16) {
#pragma unroll
    for (int s = 0; s < S - 1; ++s)
      if (s < nk) issue(s, s);
  }
  // the addends (this lane's entries of M and X), read before the products
  const int64_t col = j0 + wj + l32;
  float* Mb = u.M + b * u.sM;
  float* Xb = u.X + b * u.sX;
  float zm[16], zx[16];
  // this lane's first row of M and X; its other rows at uniform offsets
  const int64_t row0 = i0 + wi + 4 * half;
  const float* mrow = Mb + row0 * u.ldm + col;
  const float* xrow = Xb + row0 * u.ldx + col;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int dr = 8 * (v >> 2) + (v & 3);
    const bool in = row0 + dr < u.m && col < u.n;
    zm[v] = in ? mrow[dr * u.ldm] : 0.0f;
    zx[v] = in ? xrow[dr * u.ldx] : 0.0f;
  }
  const int nk16 = static_cast<int>((u.r + 15) / 16);
  if constexpr (KD16) {
#pragma unroll
    for (int s = 0; s < S - 1; ++s)
      if (s < nk16) issue16(s, s);
  }
  // the products of k-tile `it` over its first G 8-deep groups
  auto mma = [&](int it, auto groups) __attribute__((always_inline)) {
    constexpr int G = decltype(groups)::value;
    const char* ta = dsm + (it % S) * 3 * kDmaTileBytes;
    const char* tr = ta + kDmaTileBytes;
    const char* tq = tr + kDmaTileBytes;
#pragma unroll
    for (int gk = 0; gk < G; ++gk) {
      const int c = 2 * gk + half;
      const int ra = wi + l32, rb = wj + l32;
      const float4 a = *reinterpret_cast<const float4*>(ta + ra * 128 + ((c ^ (ra & 7)) << 4));
      const float4 br = *reinterpret_cast<const float4*>(tr + rb * 128 + ((c ^ (rb & 7)) << 4));
      const float4 bq = *reinterpret_cast<const float4*>(tq + rb * 128 + ((c ^ (rb & 7)) << 4));
      am = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, br.x, am, 0, 0, 0);
      am = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, br.y, am, 0, 0, 0);
      am = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, br.z, am, 0, 0, 0);
      am = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, br.w, am, 0, 0, 0);
      ax = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, bq.x, ax, 0, 0, 0);
      ax = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, bq.y, ax, 0, 0, 0);
      ax = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, bq.z, ax, 0, 0, 0);
      ax = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, bq.w, ax, 0, 0, 0);
    }
  };
  // the products of one half tile (16 k-values in 64-byte rows) at ta
  auto mma_half = [&](const char* ta) __attribute__((always_inline)) {
    const char* tr = ta + kHalfBytes;
    const char* tq = tr + kHalfBytes;
    const int ra = wi + l32, rb = wj + l32;
#pragma unroll
    for (int gk = 0; gk < 2; ++gk) {
      const int c = 2 * gk + half;
      const float4 a = *reinterpret_cast<const float4*>(ta + ra * 64 + ((c ^ ((ra + (ra >> 2)) & 3)) << 4));
      const float4 br = *reinterpret_cast<const float4*>(tr + rb * 64 + ((c ^ ((rb + (rb >> 2)) & 3)) << 4));
      const float4 bq = *reinterpret_cast<const float4*>(tq + rb * 64 + ((c ^ ((rb + (rb >> 2)) & 3)) << 4));
      am = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, br.x, am, 0, 0, 0);
      am = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, br.y, am, 0, 0, 0);
      am = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, br.z, am, 0, 0, 0);
      am = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, br.w, am, 0, 0, 0);
      ax = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, bq.x, ax, 0, 0, 0);
      ax = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, bq.y, ax, 0, 0, 0);
      ax = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, bq.z, ax, 0, 0, 0);
      ax = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, bq.w, ax, 0, 0, 0);
    }
  };
  if constexpr (HALF) {
    if (nk == 2) mma(0, std::integral_constant<int, 4>{});
    dion_wait_vm_barrier<0>();
    mma_half(dsm + 3 * kDmaTileBytes);
  }
  if constexpr (KD16) {
    for (int it = 0; it < nk16; ++it) {
      if (it + S - 1 < nk16) {
        dion_wait_vm_barrier<3 * (S - 2)>();
        issue16((it + S - 1) % S, it + S - 1);
      } else {
        dion_wait_vm_barrier<0>();
      }
      mma_half(dsm + (it % S) * 3 * kHalfBytes);
    }
  }
  // TAIL16: the contraction ends 16 into its last k-tile (r = 48, 80, ...),
  // whose last two 8-deep groups hold only the zero page's zeros
  const int full = HALF || KD16 ? 0 : TAIL16 ? nk - 1 : nk;
  for (int it = 0; it < full; ++it) {
    if (it + S - 1 < nk) {
      dion_wait_vm_barrier<6 * (S - 2)>();
      issue((it + S - 1) % S, it + S - 1);
    } else {
      dion_wait_vm_barrier<0>();
    }
    mma(it, std::integral_constant<int, 4>{});
  }
  if constexpr (TAIL16 && !HALF && !KD16) {
    if (full >= 0) {
      dion_wait_vm_barrier<0>();
      mma(full, std::integral_constant<int, 2>{});
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // every stage has landed
  if (col < u.n) {
    float* mw = Mb + row0 * u.ldm + col;
    float* xw = Xb + row0 * u.ldx + col;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int dr = 8 * (v >> 2) + (v & 3);
      if (row0 + dr >= u.m) continue;
      mw[dr * u.ldm] = fmaf(u.beta, zm[v], u.alpha_m * am[v]);
      xw[dr * u.ldx] = fmaf(u.beta, zx[v], u.alpha_x * ax[v]);
    }
  }
}

// the zero page the DMA kernel's tail chunks read (16 KB)
__global__ __launch_bounds__(256) void zero_page_kernel(float* z) { z[blockIdx.x * 256 + threadIdx.x] = 0.0f; }

// C[b](i,j) = alpha * sum_s part[s][b](i,j) + beta * Z[b](i,j), ranges added in order
__global__ __launch_bounds__(256) void reduce_kernel(DGemm g, int splits, const float* __restrict__ part,
                                                    int64_t batch) {
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t per = g.M * g.N;
  if (t >= batch * per) return;
  const int64_t b = t / per, e = t % per, i = e / g.N, j = e % g.N;
  float sum = 0.0f;
  for (int s = 0; s < splits; ++s) sum += part[(int64_t(s) * batch + b) * per + e];
  float v = g.alpha * sum;
  if (g.beta != 0.0f) v = fmaf(g.beta, g.Z[b * g.sZ + i * g.ldz + j], v);
  g.C[b * g.sC + i * g.ldc + j] = v;
}

// reduce_kernel on four consecutive entries of a row per thread (N, the
// leading dimensions and batch strides multiples of 4, 16-byte aligned bases):
// each entry summed and scaled as there
__global__ __launch_bounds__(256) void reduce4_kernel(DGemm g, int splits, const float* __restrict__ part,
                                                     int64_t batch) {
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t per = g.M * g.N;
  if (4 * t >= batch * per) return;
  const int64_t b = 4 * t / per, e = 4 * t % per, i = e / g.N, j = e % g.N;
  float4 sum = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int s = 0; s < splits; ++s) {
    const float4 v = *reinterpret_cast<const float4*>(part + (int64_t(s) * batch + b) * per + e);
    sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
  }
  float4 o = make_float4(g.alpha * sum.x, g.alpha * sum.y, g.alpha * sum.z, g.alpha * sum.w);
  if (g.beta != 0.0f) {
    const float4 z = *reinterpret_cast<const float4*>(g.Z + b * g.sZ + i * g.ldz + j);
    o = make_float4(fmaf(g.beta, z.x, o.x), fmaf(g.beta, z.y, o.y), fmaf(g.beta, z.z, o.z), fmaf(g.beta, z.w, o.w));
  }
  *reinterpret_cast<float4*>(g.C + b * g.sC + i * g.ldc + j) = o;
}

// ---------------------------------------------------------------------------
// Linv[b] = L^-1 with G[b] = L L^T (r x r, lower triangle of G read).  One
// workgroup per matrix, on 16 x 16 blocks in LDS (size padded to a multiple
// of 16 with an identity block; row pitch rp + 1).  Dependent columns
// (pivot^2 <= tol^2 * G_jj, G_jj the diagonal of G, or a real column after
// the first cap independent ones) get a zero column in L;
// L^-1 is then the inverse over the independent indices, with zero rows and
// columns at the dependent ones.
//
// Cholesky, left-looking by block column J: the panel (rows >= 16 J) takes
// the products of the earlier block columns; one wave factors the diagonal
// block and inverts it in registers (lane i owns row i, other rows reach it
// through readlane); the rows below are multiplied by the transposed inverse.
// Inverse: with W_IK = D_I L_IK (D_I the inverse of diagonal block I), block
// (I, J) of L^-1 is -sum_{J <= K < I} W_IK X_KJ, computed one block diagonal
// at a time.  X is stored transposed in the upper triangle (D_I^T on the
// diagonal), so each entry is one dot product of two LDS rows.
// ---------------------------------------------------------------------------
constexpr int kCb = 16, kCbMax = kDionMaxRank / kCb;

__device__ __forceinline__ float from_lane(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

#ifndef MUON_CHOL_THREADS
#define MUON_CHOL_THREADS 512
#endif
constexpr int kCholThreads = MUON_CHOL_THREADS;   // threads of the factorisation's workgroup
constexpr int kCholWaves = kCholThreads / 64;
__global__ __launch_bounds__(kCholThreads) void chol_inv_kernel(const float* __restrict__ G, int64_t sG,
                                                      float* __restrict__ Linv, int64_t sL, int r, int cap) {
  extern __shared__ float sm[];
  const int nb = (r + kCb - 1) / kCb, rp = nb * kCb, ld = rp + 1;
  float* S = sm;                 // rp x ld
  float* g0 = sm + rp * ld;      // diagonal of G
  const float* Gb = G + int64_t(blockIdx.x) * sG;
  const int tid = threadIdx.x;
  // G (row-major r x r, 16-byte aligned rows when r % 4 == 0) into S, eight
  // loads in flight per thread; the padding is an identity block
  if (r % 4 == 0) {
    const int q = r / 4, n4 = r * q;
    for (int e0 = 0; e0 < n4; e0 += kCholThreads * 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * kCholThreads + tid;
        v[u] = reinterpret_cast<const float4*>(Gb)[e < n4 ? e : 0];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * kCholThreads + tid;
        if (e < n4) {
          const int i = e / q, k = 4 * (e % q);
          float* d = S + i * ld + k;
          d[0] = k <= i ? v[u].x : 0.0f;
          d[1] = k + 1 <= i ? v[u].y : 0.0f;
          d[2] = k + 2 <= i ? v[u].z : 0.0f;
          d[3] = k + 3 <= i ? v[u].w : 0.0f;
        }
      }
    }
  } else {
    const int n = r * r;
    for (int e0 = 0; e0 < n; e0 += kCholThreads * 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * kCholThreads + tid;
        v[u] = Gb[e < n ? e : 0];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * kCholThreads + tid;
        if (e < n) {
          const int i = e / r, k = e % r;
          S[i * ld + k] = k <= i ? v[u] : 0.0f;
        }
      }
    }
  }
  for (int e = tid; e < rp * rp - r * r; e += kCholThreads) {
    // padding rows r.. (all columns), then columns r.. of rows < r
    const int pr = (rp - r) * rp;
    const int i = e < pr ? r + e / rp : (e - pr) / (rp - r), k = e < pr ? e % rp : r + (e - pr) % (rp - r);
    S[i * ld + k] = i == k ? 1.0f : 0.0f;
  }
  __syncthreads();
  for (int i = tid; i < rp; i += kCholThreads) g0[i] = S[i * ld + i];   // read before the first factorisation

  int kept = 0;   // the factoring wave's count of independent columns so far
  for (int J = 0; J < nb; ++J) {
    const int c0 = J * kCb;
    if (J > 0) {
      // panel: A(i, c0 + k) -= sum_{m < c0} L(i, m) L(c0 + k, m), lower part,
      // on fp32 matrix cores: wave w takes the 16-row blocks J + w, J + w + W,
      // ... (W waves); v_mfma_f32_16x16x4f32 with lane l supplying L(16 ib + l % 16,
      // m + l / 16) and L(c0 + l % 16, m + l / 16), and holding result rows
      // 4 (l / 16) .. + 3 of column l % 16
      const int wave = tid >> 6, lane = tid & 63, li = lane & 15, lk = lane >> 4;
      for (int ib = J + wave; ib < nb; ib += kCholWaves) {
        f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
        const float* ar = S + (kCb * ib + li) * ld + lk;
        const float* br = S + (c0 + li) * ld + lk;
        for (int m = 0; m < c0; m += kCb) {   // c0 is a multiple of 16: four MFMAs per pass
          float a4[4], b4[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            a4[q] = ar[m + 4 * q];
            b4[q] = br[m + 4 * q];
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[q], b4[q], acc, 0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = kCb * ib + 4 * lk + v;
          if (ib > J || li <= 4 * lk + v) S[row * ld + c0 + li] -= acc[v];
        }
      }
    }
    __syncthreads();
    if (tid < 64) {
      // diagonal block: factor, then invert; lane i < 16 holds row i
      const int lane = tid, row = c0 + (lane & (kCb - 1));
      float a[kCb], x[kCb], acc[kCb];
#pragma unroll
      for (int c = 0; c < kCb; ++c) a[c] = S[row * ld + c0 + c];
      const float g = g0[row];
      // the factor's step k and row k of D = L_JJ^-1 in one pass: row k of D
      // needs only columns <= k of L, final after step k, so the two chains
      // are independent from there and interleave:
      // D(k, c) = (delta_kc - sum_{m<k} L(k, m) D(m, c)) / l_kk
      float own_inv = 0.0f;
#pragma unroll
      for (int c = 0; c < kCb; ++c) x[c] = acc[c] = 0.0f;
#pragma unroll
      for (int k = 0; k < kCb; ++k) {
        const float d = from_lane(a[k], k);
        const bool room = c0 + k >= r || kept < cap;   // a real column past the rank bound is dependent
        const bool ok = room && d > 0.0f && d > kDependentTol * kDependentTol * from_lane(g, k);
        // the hardware square root and reciprocal (1 ulp each), computed
        // unconditionally: this chain of uniform operations is the factor's
        // critical path, and the correctly rounded forms take several times
        // as many dependent instructions
        const float sq = __builtin_amdgcn_sqrtf(fmaxf(d, 0.0f));
        const float piv = ok ? sq : 0.0f;
        const float inv = ok ? __builtin_amdgcn_rcpf(sq) : 0.0f;
        kept += piv > 0.0f ? 1 : 0;
        // selects, not branches: lane k keeps the pivot, the others scale
        own_inv = lane == k ? inv : own_inv;
        a[k] = lane == k ? piv : a[k] * inv;
#pragma unroll
        for (int m = k + 1; m < kCb; ++m) a[m] = fmaf(-a[k], from_lane(a[k], m), a[m]);
#pragma unroll
        for (int c = 0; c <= k; ++c) x[c] = lane == k ? ((c == k ? 1.0f : 0.0f) - acc[c]) * own_inv : x[c];
#pragma unroll
        for (int c = 0; c <= k; ++c) acc[c] = fmaf(a[k], from_lane(x[c], k), acc[c]);
      }
      if (lane < kCb) {
#pragma unroll
        for (int c = 0; c < kCb; ++c) S[(c0 + c) * ld + c0 + lane] = x[c];   // D^T
      }
    }
    __syncthreads();
    // rows below: L(i, c0 + k) = sum_m A(i, c0 + m) D(k, m), the block row times
    // D^T (the diagonal block of S holds D^T, zero above D's diagonal), on fp32
    // matrix cores: wave w takes the 16-row blocks J + 1 + w, J + 1 + w + W,
    // ...; lane l supplies A(16 ib + l % 16, c0 + 4 q + l / 16) and D^T(4 q +
    // l / 16, l % 16) for pass q and holds rows 4 (l / 16) .. + 3 of column
    // l % 16.  A wave reads its block row before it writes it.
    {
      const int wave = tid >> 6, lane = tid & 63, li = lane & 15, lk = lane >> 4;
      for (int ib = J + 1 + wave; ib < nb; ib += kCholWaves) {
        float a4[4], b4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          a4[q] = S[(kCb * ib + li) * ld + c0 + 4 * q + lk];
          b4[q] = S[(c0 + 4 * q + lk) * ld + c0 + li];
        }
        f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[q], b4[q], acc, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v) S[(kCb * ib + 4 * lk + v) * ld + c0 + li] = acc[v];
      }
    }
    __syncthreads();
  }

  // W_IK = D_I L_IK for every block left of the diagonal, one column per thread
  const int nw = kCb * nb * (nb - 1) / 2;
  for (int w = tid; w < nw; w += kCholThreads) {
    int I = 1;
    while (kCb * I * (I + 1) / 2 <= w) ++I;
    const int col = w - kCb * I * (I - 1) / 2, r0 = kCb * I;
    float v[kCb];
#pragma unroll
    for (int m = 0; m < kCb; ++m) v[m] = S[(r0 + m) * ld + col];
#pragma unroll
    for (int i = 0; i < kCb; ++i) {
      float o = 0.0f;
#pragma unroll
      for (int m = 0; m <= i; ++m) o = fmaf(S[(r0 + m) * ld + r0 + i], v[m], o);
      S[(r0 + i) * ld + col] = o;
    }
  }
  __syncthreads();
  // X_IJ(i, j) = -sum_{16 J <= c < 16 I} S(16 I + i, c) S(16 J + j, c), stored at S(16 J + j, 16 I + i)
  for (int d = 1; d < nb; ++d) {
    // block (J + d, J) on fp32 matrix cores, one wave per block (J = w, w + W,
    // ...): lane l supplies S(16 I + l % 16, c + l / 16) and S(16 J + l % 16,
    // c + l / 16) and holds rows 4 (l / 16) .. + 3 of column l % 16
    const int wave = tid >> 6, lane = tid & 63, li = lane & 15, lk = lane >> 4;
    for (int J = wave; J < nb - d; J += kCholWaves) {
      const int I = J + d;
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
      const float* ar = S + (kCb * I + li) * ld + lk;
      const float* br = S + (kCb * J + li) * ld + lk;
      for (int c = kCb * J; c < kCb * I; c += kCb) {   // four MFMAs per pass
        float a4[4], b4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          a4[q] = ar[c + 4 * q];
          b4[q] = br[c + 4 * q];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[q], b4[q], acc, 0, 0, 0);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) S[(kCb * J + li) * ld + kCb * I + 4 * lk + v] = -acc[v];
    }
    __syncthreads();
  }
  float* Lb = Linv + int64_t(blockIdx.x) * sL;
  for (int e = tid; e < r * r; e += kCholThreads) {
    const int i = e / r, k = e % r;
    Lb[e] = k <= i ? S[k * ld + i] : 0.0f;
  }
}

// Q[b] = R[b] with every column divided by its norm (zero columns stay zero);
// R and Q row-major n x r.  Two passes over chunks of `rows_per` rows, one
// workgroup per (chunk, matrix): colsq_kernel writes each chunk's column sums
// of squares (four interleaved partial sums per column: sum k takes the rows
// i0 + k, i0 + k + 4, ... of the chunk's whole groups of four, sum 0 also the
// rows after them; the chunk's sum is (s0 + s1) + (s2 + s3)), and
// colscale_kernel adds the chunks' sums in chunk order -- the same order in
// every workgroup -- and scales its chunk.
__global__ __launch_bounds__(256) void colsq_kernel(const float* __restrict__ R, int64_t sR,
                                                   float* __restrict__ part, int64_t n, int r,
                                                   int64_t rows_per, int64_t nch) {
  __shared__ float sums[4][kDionMaxRank];
  const int64_t b = blockIdx.y, ch = blockIdx.x;
  const int64_t i0 = ch * rows_per, i1 = min(n, i0 + rows_per);
  const int64_t whole = i0 + (i1 - i0) / 4 * 4;   // end of the whole groups of four rows
  const float* Rb = R + b * sR;
  // thread (k, c), k = e / r: partial sum k of column c (4 r threads' work)
  for (int e = threadIdx.x; e < 4 * r; e += 256) {
    const int k = e / r, c = e % r;
    float acc = 0.0f;
    int64_t i = i0 + k;
    for (; i + 12 < whole; i += 16) {   // four rows of this sum in flight
      const float v0 = Rb[i * r + c], v1 = Rb[(i + 4) * r + c];
      const float v2 = Rb[(i + 8) * r + c], v3 = Rb[(i + 12) * r + c];
      acc = fmaf(v0, v0, acc);
      acc = fmaf(v1, v1, acc);
      acc = fmaf(v2, v2, acc);
      acc = fmaf(v3, v3, acc);
    }
    for (; i < whole; i += 4) acc = fmaf(Rb[i * r + c], Rb[i * r + c], acc);
    if (k == 0)
      for (i = whole; i < i1; ++i) acc = fmaf(Rb[i * r + c], Rb[i * r + c], acc);
    sums[k][c] = acc;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < r; c += 256)
    part[(b * nch + ch) * r + c] = (sums[0][c] + sums[1][c]) + (sums[2][c] + sums[3][c]);
}

__global__ __launch_bounds__(256) void colscale_kernel(const float* __restrict__ R, int64_t sR,
                                                      const float* __restrict__ part, float* __restrict__ Q,
                                                      int64_t sQ, int64_t n, int r, int64_t rows_per,
                                                      int64_t nch) {
  __shared__ float inv[kDionMaxRank];
  const int64_t b = blockIdx.y, ch = blockIdx.x;
  for (int c = threadIdx.x; c < r; c += 256) {
    // the chunks' sums added in chunk order, eight loads in flight at a time
    float t = 0.0f;
    const float* pc = part + b * nch * r + c;
    int64_t q = 0;
    for (; q + 8 <= nch; q += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = pc[(q + u) * r];
#pragma unroll
      for (int u = 0; u < 8; ++u) t += v[u];
    }
    for (; q < nch; ++q) t += pc[q * r];
    const float nrm = sqrtf(t);
    inv[c] = nrm > 0.0f ? 1.0f / nrm : 0.0f;
  }
  __syncthreads();
  // thread t: column group t % groups (4 columns when rows are 16-byte
  // aligned, else 1), rows t / groups, t / groups + 256 / groups, ...
  const int64_t i0 = ch * rows_per, i1 = min(n, i0 + rows_per);
  const float* Rb = R + b * sR;
  float* Qb = Q + b * sQ;
  const bool vec = r % 4 == 0 && sQ % 4 == 0 && sR % 4 == 0;
  const int groups = vec ? r / 4 : r, step = 256 / groups;
  const int t = threadIdx.x, g = t % groups;
  if (t >= groups * step) return;
  if (vec) {
    const float4 w = make_float4(inv[4 * g], inv[4 * g + 1], inv[4 * g + 2], inv[4 * g + 3]);
    for (int64_t i = i0 + t / groups; i < i1; i += step) {
      const float4 v = *reinterpret_cast<const float4*>(Rb + i * r + 4 * g);
      *reinterpret_cast<float4*>(Qb + i * r + 4 * g) = make_float4(v.x * w.x, v.y * w.y, v.z * w.z, v.w * w.w);
    }
  } else {
    for (int64_t i = i0 + t / groups; i < i1; i += step) Qb[i * r + g] = Rb[i * r + g] * inv[g];
  }
}

// M[b] <- round_fp32(M[b] + G[b]) (the exact sum of two fp32 values rounded
// once), len entries per matrix; 4 entries per thread when len and the batch
// strides are multiples of 4 (the bases are 16-byte aligned)

__global__ __launch_bounds__(256) void add_kernel(float* __restrict__ M, int64_t sM,
                                                 const float* __restrict__ G, int64_t sG, int64_t len, int vec) {
  const int64_t b = blockIdx.y;
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  float* m = M + b * sM;
  const float* g = G + b * sG;
  if (vec) {
    if (4 * t >= len) return;
    float4 x = *reinterpret_cast<const float4*>(m + 4 * t);
    const float4 y = *reinterpret_cast<const float4*>(g + 4 * t);
    x = make_float4(add_once(x.x, y.x), add_once(x.y, y.y), add_once(x.z, y.z), add_once(x.w, y.w));
    *reinterpret_cast<float4*>(m + 4 * t) = x;
  } else {
    if (t >= len) return;
    m[t] = add_once(m[t], g[t]);
  }
}

// k ranges per output tile: about kSplitTarget workgroups,
// at least 256 of k per range, at most 16 ranges
// 48-wide output tiles (dion_gemm_dma48_kernel) for widths that are multiples
// of 48 but not of 64, when the operands can be staged by DMA
bool use48(int64_t N) { return N % 48 == 0 && N % kDT != 0; }

// output widths one fused-add workgroup spans (16 x 16 blocks per wave row)
bool fused_width(int64_t N) { return N == 48 || N == 64 || N == 96 || N == 128 || N == 192; }
#ifndef MUON_DION_FUSED_ADD_MAX_RANK
#define MUON_DION_FUSED_ADD_MAX_RANK 192
#endif
constexpr int kFusedAddMaxRank = MUON_DION_FUSED_ADD_MAX_RANK;   // ranks whose B Q forms B = M + G

// workgroups a split product aims for: 512 measured 1-2% faster than 1024 at
// every rank (the four streams' products share the chip), and fixed, so that a
// run's k ranges do not depend on what else shares the call
constexpr int64_t kSplitTarget = 512;
int gemm_splits(int64_t M, int64_t N, int64_t K, int64_t batch, bool w48 = false) {
  const int64_t blocks = (w48 ? N / 48 : (N + kDT - 1) / kDT) * ((M + kDT - 1) / kDT) * batch;
  int64_t s = (kSplitTarget + blocks - 1) / blocks;
  s = std::min<int64_t>(s, std::max<int64_t>(1, K / 256));
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(s, 16)));
}

size_t gemm_part_bytes(int64_t M, int64_t N, int64_t K, int64_t batch) {
  // the larger of the two tile widths' split counts (the width is chosen per
  // product, from whether its operands can be staged by DMA)
  const int s = std::max(gemm_splits(M, N, K, batch), use48(N) ? gemm_splits(M, N, K, batch, true) : 1);
  return s > 1 ? static_cast<size_t>(s) * batch * M * N * 4 : 0;
}

#ifndef MUON_DION_STAGES
#define MUON_DION_STAGES 2
#endif
constexpr int kDionStages = MUON_DION_STAGES;   // DMA ring depth (16 KB per stage)
#ifndef MUON_DION_UPDATE2_HALF
#define MUON_DION_UPDATE2_HALF 1
#endif
constexpr bool kUpdate2Half = MUON_DION_UPDATE2_HALF;   // r = 16, 48: the tail in a half stage
// the other ranks' fused updates on 16-deep stages, kUpdate2Stages16 of them
#ifndef MUON_DION_UPDATE2_KD16
#define MUON_DION_UPDATE2_KD16 1
#endif
#ifndef MUON_DION_UPDATE2_STAGES16
#define MUON_DION_UPDATE2_STAGES16 3
#endif
constexpr bool kUpdate2KD16 = MUON_DION_UPDATE2_KD16;
constexpr int kUpdate2Stages16 = MUON_DION_UPDATE2_STAGES16;
// B Q with B = M + G formed in it at rank 192: 16-deep stages, kAddStages of
// them (2% faster there; 1-4% slower at ranks 48 and 96, which keep 32)
#ifndef MUON_DION_ADD_KD16
#define MUON_DION_ADD_KD16 1
#endif
#ifndef MUON_DION_ADD_STAGES
#define MUON_DION_ADD_STAGES 3
#endif
constexpr bool kAddKD16 = MUON_DION_ADD_KD16;
constexpr int kAddStages = MUON_DION_ADD_STAGES;

// an operand the DMA kernel can stage: 16-byte chunks along its contiguous
// dimension (k when s_k == 1, else the output dimension), whole chunks only
bool dma_operand_ok(const float* p, int64_t s_batch, int64_t s_out, int64_t s_k, int64_t n_out, int64_t K) {
  if (!aligned16(p) || s_batch % 4 != 0) return false;
  if (s_k == 1) return s_out % 4 == 0 && K % 4 == 0;
  return s_out == 1 && s_k % 4 == 0 && n_out % 4 == 0;
}

template <bool ACK, bool BCK>
void launch_dma(const DGemm& g, dim3 grid, int splits, float* part, const float* zero, hipStream_t st) {
  const uint32_t lds = kDionStages * 2 * kDmaTileBytes;
  // only k-contiguous operands with an addend (the m x n updates) read it first
  if constexpr (ACK && BCK) {
    if (splits == 1 && g.beta != 0.0f) {
      launch_kernel(dion_gemm_dma_kernel<kDionStages, true, true, true>, grid, dim3(256), lds, st, g, splits, part,
                    zero);
      return;
    }
  }
  launch_kernel(dion_gemm_dma_kernel<kDionStages, ACK, BCK, false>, grid, dim3(256), lds, st, g, splits, part, zero);
}

// the sum of a product's k ranges (part: splits x batch x M x N)
void launch_reduce(const DGemm& g, int splits, const float* part, int64_t batch, hipStream_t st) {
  const int64_t n = batch * g.M * g.N;
  const bool vec = g.N % 4 == 0 && g.ldc % 4 == 0 && g.sC % 4 == 0 && aligned16(g.C) && aligned16(part) &&
                   (g.beta == 0.0f || (g.ldz % 4 == 0 && g.sZ % 4 == 0 && aligned16(g.Z)));
  if (vec)
    launch_kernel(reduce4_kernel, dim3((n / 4 + 255) / 256), dim3(256), 0, st, g, splits, part, batch);
  else
    launch_kernel(reduce_kernel, dim3((n + 255) / 256), dim3(256), 0, st, g, splits, part, batch);
}

// zero: the workspace's zero page (NULL keeps every product on the
// register-staged kernel)
int dgemm(const float* A, int64_t sA, int64_t a_i, int64_t a_k, const float* B, int64_t sB, int64_t b_k,
          int64_t b_j, const float* Z, int64_t sZ, int64_t ldz, float* C, int64_t sC, int64_t ldc,
          int64_t M, int64_t N, int64_t K, float alpha, float beta, int64_t batch, float* part,
          const float* zero, hipStream_t st, const float* A2 = nullptr, int64_t sA2 = 0, float* Aout = nullptr) {
  DGemm g{A, sA, a_i, a_k, B, sB, b_k, b_j, Z, sZ, ldz, C, sC, ldc, M, N, K, alpha, beta, A2, sA2, Aout};
  const bool dma = zero && dma_operand_ok(A, sA, a_i, a_k, M, K) && dma_operand_ok(B, sB, b_j, b_k, N, K);
  // A + A2 written back to Aout: one column tile as wide as the output (every
  // entry of A read by one workgroup) and a k-contiguous A
  if (A2 && !(dma && fused_width(N) && a_k == 1 && Aout && dma_operand_ok(A2, sA2, a_i, a_k, M, K)))
    return MUON_EINVAL;
  if (A2) {
    // ranges per product as for 64-wide tiles, so that the split-k buffer
    // sized for those holds these
    const int splits = N == 48 ? gemm_splits(M, N, K, batch, true) : gemm_splits(M, N, K, batch);
    const dim3 grid(1, (M + kDT - 1) / kDT, batch * splits);
    const bool bck = b_k == 1;
    // the 192-wide tile on 16-deep stages (kAddStages half stages), the
    // others on the 32-deep ring
    auto go = [&](auto kern, int nb, bool kd16) {
      const uint32_t stages = kd16 ? kAddStages : kDionStages;
      const uint32_t lds = stages * (2 + (16 * nb + kDT - 1) / kDT) * (kDmaTileBytes / (kd16 ? 2 : 1));
      launch_kernel(kern, grid, dim3(256), lds, st, g, splits, part, zero);
    };
    constexpr int S = kDionStages, SA = kAddStages;
    constexpr bool H = kAddKD16;
    switch (N) {
      case 48: bck ? go(dion_gemm_dma48_kernel<S, 3, true, true, true>, 3, false)
                   : go(dion_gemm_dma48_kernel<S, 3, true, false, true>, 3, false); break;
      case 64: bck ? go(dion_gemm_dma48_kernel<S, 4, true, true, true>, 4, false)
                   : go(dion_gemm_dma48_kernel<S, 4, true, false, true>, 4, false); break;
      case 96: bck ? go(dion_gemm_dma48_kernel<S, 6, true, true, true>, 6, false)
                   : go(dion_gemm_dma48_kernel<S, 6, true, false, true>, 6, false); break;
      case 128: bck ? go(dion_gemm_dma48_kernel<S, 8, true, true, true>, 8, false)
                    : go(dion_gemm_dma48_kernel<S, 8, true, false, true>, 8, false); break;
      default: bck ? go(dion_gemm_dma48_kernel<H ? SA : S, 12, true, true, true, H>, 12, H)
                   : go(dion_gemm_dma48_kernel<H ? SA : S, 12, true, false, true, H>, 12, H); break;
    }
    if (splits > 1) launch_reduce(g, splits, part, batch, st);
    return launch_status();
  }
  if (dma && use48(N)) {
    const int splits = gemm_splits(M, N, K, batch, true);
    const dim3 grid(N / 48, (M + kDT - 1) / kDT, batch * splits);
    const uint32_t lds = kDionStages * 2 * kDmaTileBytes;
    auto go = [&](auto kern) { launch_kernel(kern, grid, dim3(256), lds, st, g, splits, part, zero); };
    const bool ack = a_k == 1, bck = b_k == 1;
    if (ack && bck) go(dion_gemm_dma48_kernel<kDionStages, 3, true, true, false>);
    else if (ack) go(dion_gemm_dma48_kernel<kDionStages, 3, true, false, false>);
    else if (bck) go(dion_gemm_dma48_kernel<kDionStages, 3, false, true, false>);
    else go(dion_gemm_dma48_kernel<kDionStages, 3, false, false, false>);
    if (splits > 1) launch_reduce(g, splits, part, batch, st);
    return launch_status();
  }
  const int splits = gemm_splits(M, N, K, batch);
  const dim3 grid((N + kDT - 1) / kDT, (M + kDT - 1) / kDT, batch * splits);
  if (dma) {
    const bool ack = a_k == 1, bck = b_k == 1;
    if (ack && bck) launch_dma<true, true>(g, grid, splits, part, zero, st);
    else if (ack) launch_dma<true, false>(g, grid, splits, part, zero, st);
    else if (bck) launch_dma<false, true>(g, grid, splits, part, zero, st);
    else launch_dma<false, false>(g, grid, splits, part, zero, st);
  } else {
    // 16-byte operand loads: contiguous dimension stride 1, every other stride a
    // multiple of 4 floats, aligned base
    auto vec_ok = [](const float* p, int64_t s_batch, int64_t s_a, int64_t s_b) {
      return aligned16(p) && (s_a == 1 || s_b == 1) && s_batch % 4 == 0 && (s_a == 1 ? s_b : s_a) % 4 == 0;
    };
    const int a_vec = vec_ok(A, sA, a_i, a_k), b_vec = vec_ok(B, sB, b_k, b_j);
    launch_kernel(dion_gemm_kernel, grid, dim3(256), 0, st, g, splits, part, a_vec, b_vec);
  }
  if (splits > 1) launch_reduce(g, splits, part, batch, st);
  return launch_status();
}

// ---------------------------------------------------------------------------
// Grouping: consecutive problems of one shape whose M, G, X and Q advance by
// constant strides run batched.
// ---------------------------------------------------------------------------
struct DRun {
  int first, count;
  int64_t m, n;
  int64_t sM, sG, sX, sQ;   // batch strides (elements)
};

int64_t stride_of(const void* a, const void* b) {
  const int64_t d = reinterpret_cast<const char*>(b) - reinterpret_cast<const char*>(a);
  return (d > 0 && d % 4 == 0) ? d / 4 : -1;
}

// problems are taken in order of (rows, cols, address of M), so matrices of
// one shape interleaved with others (a layer set) still batch
std::vector<muon_dion_problem> dion_sorted(const muon_dion_problem* probs, int count) {
  std::vector<muon_dion_problem> p(probs, probs + count);
  std::stable_sort(p.begin(), p.end(), [](const muon_dion_problem& a, const muon_dion_problem& b) {
    if (a.rows != b.rows) return a.rows < b.rows;
    if (a.cols != b.cols) return a.cols < b.cols;
    return reinterpret_cast<uintptr_t>(a.M) < reinterpret_cast<uintptr_t>(b.M);
  });
  return p;
}

std::vector<DRun> dion_runs(const muon_dion_problem* p, int count) {
  std::vector<DRun> runs;
  int i = 0;
  while (i < count) {
    DRun r{i, 1, p[i].rows, p[i].cols, 0, 0, 0, 0};   // strides unused for a single problem
    if (i + 1 < count && p[i + 1].rows == r.m && p[i + 1].cols == r.n) {
      const int64_t sM = stride_of(p[i].M, p[i + 1].M), sG = stride_of(p[i].G, p[i + 1].G);
      const int64_t sX = stride_of(p[i].X, p[i + 1].X), sQ = stride_of(p[i].Q, p[i + 1].Q);
      if (sM > 0 && sG > 0 && sX > 0 && sQ > 0) {
        int j = i + 1;
        while (j < count && p[j].rows == r.m && p[j].cols == r.n &&
               stride_of(p[j - 1].M, p[j].M) == sM && stride_of(p[j - 1].G, p[j].G) == sG &&
               stride_of(p[j - 1].X, p[j].X) == sX && stride_of(p[j - 1].Q, p[j].Q) == sQ)
          ++j;
        r.count = j - i;
        r.sM = sM; r.sG = sG; r.sX = sX; r.sQ = sQ;
      }
    }
    runs.push_back(r);
    i += r.count;
  }
  return runs;
}

// Lanes: the caller's stream and up to three of the library's streams,
// forked from and joined back into the caller's with events, one lane per run
// up to that count.  Runs are placed largest first on the lane with the least
// work so far, and each lane takes the stages below over its own runs.  The
// launches that leave most CUs idle (the factorisation's one workgroup per
// matrix, the r x r Grams, the split-k reductions, the column norms) then run
// beside the other lanes' products.
#ifndef MUON_DION_LANES
#define MUON_DION_LANES 4
#endif
constexpr int kDionLanes = MUON_DION_LANES;
static_assert(kDionLanes >= 1 && kDionLanes <= kLibStreams + 1, "one library stream per extra lane");

// Workspace: every run keeps its own P (twice) and R, since the stages run
// over all runs of a lane in turn; the Grams and their inverse factors sit in
// two arrays, lane by lane, so each lane factors its matrices in one launch;
// each lane has a split-k partial buffer for its products (lane 0's is sized
// for every run, so all runs can also go to lane 0 alone, when a stream or
// the events cannot be had).
struct DLayout {
  std::vector<size_t> p0, p1, R;
  std::vector<int> lane;        // lane of each run
  std::vector<int64_t> slot;    // first matrix of each run in the Gram and factor arrays
  int64_t lane_mats[kDionLanes] = {};
  int lanes = 1;
  size_t gram = 0, linv = 0, part[kDionLanes] = {}, zero = 0, total = 0;
};

size_t run_part_bytes(const DRun& r, int rank) {
  return std::max({gemm_part_bytes(r.m, rank, r.n, r.count), gemm_part_bytes(rank, rank, r.m, r.count),
                   gemm_part_bytes(r.m, rank, rank, r.count), gemm_part_bytes(r.n, rank, r.m, r.count),
                   gemm_part_bytes(r.m, r.n, rank, r.count)});
}

DLayout dion_layout(const std::vector<DRun>& runs, int count, int rank) {
  const size_t rk = static_cast<size_t>(rank);
  DLayout L{};
  L.lane.assign(runs.size(), 0);
  L.lanes = static_cast<int>(std::min<size_t>(kDionLanes, runs.size()));
  if (L.lanes > 1) {
    // every product of a run moves or multiplies in proportion to its m n
    std::vector<size_t> order(runs.size());
    for (size_t i = 0; i < order.size(); ++i) order[i] = i;
    auto cost = [&](size_t i) { return static_cast<double>(runs[i].count) * runs[i].m * runs[i].n; };
    std::stable_sort(order.begin(), order.end(), [&](size_t x, size_t y) { return cost(x) > cost(y); });
    double load[kDionLanes] = {};
    for (size_t i : order) {
      int l = 0;
      for (int j = 1; j < L.lanes; ++j)
        if (load[j] < load[l]) l = j;
      L.lane[i] = l;
      load[l] += cost(i);
    }
  }
  L.slot.assign(runs.size(), 0);
  int64_t slots = 0;
  for (int l = 0; l < L.lanes; ++l)
    for (size_t k = 0; k < runs.size(); ++k)
      if (L.lane[k] == l) {
        L.slot[k] = slots;
        slots += runs[k].count;
        L.lane_mats[l] += runs[k].count;
      }
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += round_up(bytes, 256); return o; };
  size_t part[kDionLanes] = {};
  for (size_t k = 0; k < runs.size(); ++k) {
    const DRun& r = runs[k];
    const size_t b = static_cast<size_t>(r.count);
    L.p0.push_back(take(b * r.m * rk * 4));
    L.p1.push_back(take(b * r.m * rk * 4));
    L.R.push_back(take(b * r.n * rk * 4));
    const size_t pb = run_part_bytes(r, rank);
    part[0] = std::max(part[0], pb);
    if (L.lane[k] > 0) part[L.lane[k]] = std::max(part[L.lane[k]], pb);
  }
  L.gram = take(static_cast<size_t>(count) * rk * rk * 4);
  L.linv = take(static_cast<size_t>(count) * rk * rk * 4);
  for (int l = 0; l < kDionLanes; ++l) L.part[l] = take(part[l]);
  L.zero = take(kZeroPageFloats * sizeof(float));
  L.total = off;
  return L;
}

// Launch limits of the products' tile grids: at most 65535 row tiles of 64
// (grid y), 16 k ranges times the batch in grid z, and fewer than 2^32
// workgroups in one launch.  The largest grids are the m x n outputs and the
// m x rank outputs split 16 ways.
constexpr int64_t kDionMaxSide = 65535 * kDT, kDionMaxCount = 65535 / 16;

bool dion_valid(const muon_dion_problem& p, int count) {
  if (!(p.rows > 0 && p.cols > 0 && p.M && p.G && p.X && p.Q)) return false;
  if (p.rows > kDionMaxSide || p.cols > kDionMaxSide || count > kDionMaxCount) return false;
  const int64_t tm = (p.rows + kDT - 1) / kDT, tn = (p.cols + kDT - 1) / kDT;
  return std::max<int64_t>(tn, 48) * tm * count < (int64_t(1) << 32) &&
         std::max<int64_t>(tm, 48) * tn * count < (int64_t(1) << 32);
}

// The LDS limit of the factorisation kernel, raised per device to the largest
// request so far (a raced update only repeats the attribute call).
int set_chol_lds(int bytes) {
  static std::atomic<int> configured[kMaxTrackedDevices];   // bytes set, per device
  const int dev = current_device();
  const bool tracked = dev >= 0 && dev < kMaxTrackedDevices;
  if (!tracked || bytes > configured[dev].load(std::memory_order_acquire)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(chol_inv_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess)
      return MUON_ELAUNCH;
    if (tracked) {
      int cur = configured[dev].load(std::memory_order_relaxed);
      while (bytes > cur && !configured[dev].compare_exchange_weak(cur, bytes, std::memory_order_release)) {
      }
    }
  }
  return MUON_OK;
}

// One call's state shared by both lanes.
struct DionCall {
  const std::vector<DRun>* runs;
  const std::vector<muon_dion_problem>* sorted;
  const DLayout* L;
  char* ws;
  int rank, chol_lds;
  float mu, eta;
  const float* zero;   // the DMA products' zero page (null: register-staged products)
};

// Stage `stage` of Dion's step for the runs `ids` of one lane, on stream st:
//   0     B = M + G in place, and P = B Q
//   1-3   first orthonormalisation pass: the Grams P^T P, their factorisation
//         (one launch over the lane's nmat matrices from slot0), P <- P L^-T
//   4-6   the second pass, back into P's first buffer
//   7     R = B^T P, Q = ColumnNormalize(R), then the error feedback and the X
//         update (one pass over the m x n tiles where both fit the DMA kernel)
constexpr int kDionStagesPerCall = 8;

int dion_stage(const DionCall& C, int stage, const std::vector<int>& ids, float* part, int64_t slot0,
               int64_t nmat, hipStream_t st) {
  const DLayout& L = *C.L;
  const int64_t r = C.rank;
  float* Gm = reinterpret_cast<float*>(C.ws + L.gram);
  float* Li = reinterpret_cast<float*>(C.ws + L.linv);
  auto Pbuf = [&](size_t k, int which) {
    return reinterpret_cast<float*>(C.ws + (which == 0 ? L.p0[k] : L.p1[k]));
  };
  const float* zp = C.zero;
  int status = MUON_OK;
  if (stage == 0) {
    for (int k : ids) {
      const DRun& run = (*C.runs)[k];
      const muon_dion_problem& p = (*C.sorted)[run.first];
      float* M = static_cast<float*>(p.M);
      const float* G = static_cast<const float*>(p.G);
      const float* Q = static_cast<const float*>(p.Q);
      const int64_t m = run.m, n = run.n, b = run.count, mn = m * n;
      // B = M + G formed by B Q as it stages M and G, and written back to M
      // there, instead of by a pass of its own (one column tile as wide as the
      // rank reads each entry of M once)
      const bool fused = zp != nullptr && fused_width(r) && r <= kFusedAddMaxRank &&
                         dma_operand_ok(M, run.sM, n, 1, m, n) &&
                         dma_operand_ok(G, run.sG, n, 1, m, n) && dma_operand_ok(Q, run.sQ, 1, r, r, n);
      if (!fused) {
        const int vec = mn % 4 == 0 && run.sM % 4 == 0 && run.sG % 4 == 0;
        const int64_t threads = vec ? mn / 4 : mn;
        launch_kernel(add_kernel, dim3((threads + 255) / 256, b), dim3(256), 0, st, M, run.sM, G, run.sG, mn, vec);
        if ((status = launch_status()) != MUON_OK) return status;
      }
      status = dgemm(M, run.sM, n, 1, Q, run.sQ, r, 1, nullptr, 0, 0, Pbuf(k, 0), m * r, r, m, r, n, 1.0f, 0.0f, b,
                     part, zp, st, fused ? G : nullptr, run.sG, fused ? M : nullptr);
      if (status != MUON_OK) return status;
    }
    return MUON_OK;
  }
  if (stage <= 6) {
    const int pass = (stage - 1) / 3, step = (stage - 1) % 3;
    if (step == 0) {
      for (int k : ids) {
        const DRun& run = (*C.runs)[k];
        const float* P = Pbuf(k, pass);
        status = dgemm(P, run.m * r, 1, r, P, run.m * r, r, 1, nullptr, 0, 0, Gm + L.slot[k] * r * r, r * r, r,
                       r, r, run.m, 1.0f, 0.0f, run.count, part, zp, st);
        if (status != MUON_OK) return status;
      }
    } else if (step == 1) {
      // P = B Q has rank at most min(m, n): a run whose side is below the rank
      // factors on its own with that bound, the others in one launch
      bool bounded = false;
      for (int k : ids) bounded = bounded || std::min((*C.runs)[k].m, (*C.runs)[k].n) < r;
      if (!bounded && nmat > 0) {
        launch_kernel(chol_inv_kernel, dim3(nmat), dim3(kCholThreads), C.chol_lds, st, Gm + slot0 * r * r, r * r,
                      Li + slot0 * r * r, r * r, C.rank, C.rank);
        status = launch_status();
      }
      for (int k : ids) {
        if (!bounded) break;
        const DRun& run = (*C.runs)[k];
        const int cap = static_cast<int>(std::min<int64_t>({run.m, run.n, r}));
        launch_kernel(chol_inv_kernel, dim3(run.count), dim3(kCholThreads), C.chol_lds, st, Gm + L.slot[k] * r * r,
                      r * r, Li + L.slot[k] * r * r, r * r, C.rank, cap);
        if ((status = launch_status()) != MUON_OK) return status;
      }
    } else {
      for (int k : ids) {
        const DRun& run = (*C.runs)[k];
        status = dgemm(Pbuf(k, pass), run.m * r, r, 1, Li + L.slot[k] * r * r, r * r, 1, r, nullptr, 0, 0,
                       Pbuf(k, 1 - pass), run.m * r, r, run.m, r, r, 1.0f, 0.0f, run.count, part, zp, st);
        if (status != MUON_OK) return status;
      }
    }
    return status;
  }
  for (int k : ids) {
    const DRun& run = (*C.runs)[k];
    const muon_dion_problem& p = (*C.sorted)[run.first];
    float* M = static_cast<float*>(p.M);
    float* X = static_cast<float*>(p.X);
    float* Q = static_cast<float*>(p.Q);
    float* R = reinterpret_cast<float*>(C.ws + L.R[k]);
    const float* Pf = Pbuf(k, 0);      // two passes: back in buffer 0
    const int64_t m = run.m, n = run.n, b = run.count;
    status = dgemm(M, run.sM, 1, n, Pf, m * r, r, 1, nullptr, 0, 0, R, n * r, r, n, r, m, 1.0f, 0.0f, b, part, zp, st);
    if (status != MUON_OK) return status;
    // the two rank-r updates in one pass when their products would each run
    // unsplit on the DMA kernel (the error feedback then waits for the column
    // norms, on which it does not depend)
    const bool both = zp != nullptr && !use48(n) && gemm_splits(m, n, r, b) == 1 &&
                      dma_operand_ok(Pf, m * r, r, 1, m, r) && dma_operand_ok(R, n * r, r, 1, n, r) &&
                      dma_operand_ok(Q, run.sQ, r, 1, n, r);
    if (!both) {
      status = dgemm(Pf, m * r, r, 1, R, n * r, 1, r, M, run.sM, n, M, run.sM, n, m, n, r, -(1.0f - C.mu), 1.0f, b,
                     part, zp, st);
      if (status != MUON_OK) return status;
    }
    {
      // chunks of at least 64 rows and at most m chunks, so the partial sums
      // (b x chunks x r) fit in P's second buffer, free after the two passes
      const int64_t rows_per = std::max<int64_t>(64, (n + m - 1) / m);
      const int64_t nch = (n + rows_per - 1) / rows_per;
      float* cpart = Pbuf(k, 1);
      launch_kernel(colsq_kernel, dim3(nch, b), dim3(256), 0, st, R, n * r, cpart, n, C.rank, rows_per, nch);
      launch_kernel(colscale_kernel, dim3(nch, b), dim3(256), 0, st, R, n * r, cpart, Q, run.sQ, n, C.rank,
                    rows_per, nch);
    }
    if ((status = launch_status()) != MUON_OK) return status;
    if (both) {
      const DUpdate2 u{Pf, m * r, r, R, n * r, r, Q, run.sQ, r, M, run.sM, n, X, run.sX, n, m, n, r,
                       -(1.0f - C.mu), -C.eta, 1.0f};
      const dim3 grid((n + kDT - 1) / kDT, (m + kDT - 1) / kDT, b);
      const uint32_t lds = kDionStages * 3 * kDmaTileBytes;
      if (r % kDK == 16 && r <= kDK + 16 && kUpdate2Half)
        launch_kernel(dion_update2_kernel<kDionStages, true, true>, grid, dim3(256), 9 * kDmaTileBytes / 2, st, u,
                      zp);
      else if (kUpdate2KD16)
        launch_kernel(dion_update2_kernel<kUpdate2Stages16, false, false, true>, grid, dim3(256),
                      kUpdate2Stages16 * 3 * kDmaTileBytes / 2, st, u, zp);
      else if (r % kDK == 16)
        launch_kernel(dion_update2_kernel<kDionStages, true, false>, grid, dim3(256), lds, st, u, zp);
      else launch_kernel(dion_update2_kernel<kDionStages, false, false>, grid, dim3(256), lds, st, u, zp);
      status = launch_status();
    } else {
      status = dgemm(Pf, m * r, r, 1, Q, run.sQ, 1, r, X, run.sX, n, X, run.sX, n, m, n, r, -C.eta, 1.0f, b, part,
                     zp, st);
    }
    if (status != MUON_OK) return status;
  }
  return MUON_OK;
}

}  // namespace
}  // namespace muon

using namespace muon;

extern "C" {

size_t dion_workspace_bytes(const muon_dion_problem* probs, int count, int rank) {
  if (!probs || count <= 0 || rank < 1 || rank > kDionMaxRank) return 0;
  for (int i = 0; i < count; ++i)
    if (!dion_valid(probs[i], count)) return 0;
  const std::vector<muon_dion_problem> sorted = dion_sorted(probs, count);
  return dion_layout(dion_runs(sorted.data(), count), count, rank).total;
}

int dion_step(const muon_dion_problem* probs, int count, int rank, float mu, float eta, void* workspace,
              size_t ws_bytes, void* stream) {
  if (count < 0 || rank < 1 || rank > kDionMaxRank) return MUON_EINVAL;
  if (count == 0) return MUON_OK;
  if (!probs) return MUON_EINVAL;
  for (int i = 0; i < count; ++i) {
    if (!dion_valid(probs[i], count)) return MUON_EINVAL;
    if (!aligned16(probs[i].M) || !aligned16(probs[i].G) || !aligned16(probs[i].X) ||
        !aligned16(probs[i].Q))
      return MUON_EALIGN;
  }
  const std::vector<muon_dion_problem> sorted = dion_sorted(probs, count);
  const std::vector<DRun> runs = dion_runs(sorted.data(), count);
  const DLayout L = dion_layout(runs, count, rank);
  if (!workspace || ws_bytes < L.total) return MUON_EWORKSPACE;
  if (!aligned16(workspace)) return MUON_EALIGN;
  const int rp = (rank + kCb - 1) / kCb * kCb;
  const int lds = (rp * (rp + 1) + rp) * 4;
  if (set_chol_lds(lds) != MUON_OK) return MUON_ELAUNCH;

  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
#ifndef MUON_DION_DMA
#define MUON_DION_DMA 1
#endif
  // the DMA products' zero page, cleared on every call (the workspace's
  // contents on entry do not matter)
  float* zp = MUON_DION_DMA ? reinterpret_cast<float*>(ws + L.zero) : nullptr;
  if (zp) {
    launch_kernel(zero_page_kernel, dim3(kZeroPageFloats / 256), dim3(256), 0, st, zp);
    const int status = launch_status();
    if (status != MUON_OK) return status;
  }
  const DionCall C{&runs, &sorted, &L, ws, rank, lds, mu, eta, zp};
  // the lanes' streams, forked from the caller's; with any of them or the
  // events missing, every run goes to the caller's stream
  int lanes = L.lanes;
  hipStream_t lane_st[kDionLanes] = {st};
  hipEvent_t ev[kDionLanes] = {};   // the fork, then the joins of lanes 1 ..
  for (int l = 1; l < lanes; ++l)
    if ((lane_st[l] = lane_stream(l - 1)) == nullptr) lanes = 1;
  if (lanes > 1 && (!lane_events(ev, lanes) || hipEventRecord(ev[0], st) != hipSuccess)) lanes = 1;
  int forked = 1;   // lanes 1 .. forked - 1 wait on the fork (and are joined below)
  for (int l = 1; l < lanes; ++l, ++forked)
    if (hipStreamWaitEvent(lane_st[l], ev[0], 0) != hipSuccess) break;
  if (forked < lanes) lanes = 1;
  std::vector<int> ids[kDionLanes];
  int64_t mats[kDionLanes] = {}, slot0[kDionLanes] = {};
  for (int l = 0; l < L.lanes; ++l)   // lane by lane: the order of the Gram slots
    for (size_t k = 0; k < runs.size(); ++k)
      if (L.lane[k] == l) ids[lanes > 1 ? l : 0].push_back(static_cast<int>(k));
  if (lanes > 1) {
    for (int l = 0; l < lanes; ++l) mats[l] = L.lane_mats[l];
    for (int l = 1; l < lanes; ++l) slot0[l] = slot0[l - 1] + mats[l - 1];
  } else {
    mats[0] = count;
  }
  // the lanes' launches are enqueued stage by stage, so all start at once
  int status = MUON_OK;
  for (int stage = 0; stage < kDionStagesPerCall && status == MUON_OK; ++stage)
    for (int l = 0; l < lanes && status == MUON_OK; ++l)
      status = dion_stage(C, stage, ids[l], reinterpret_cast<float*>(ws + L.part[l]), slot0[l], mats[l], lane_st[l]);
  for (int l = 1; l < forked; ++l)
    if ((hipEventRecord(ev[l], lane_st[l]) != hipSuccess || hipStreamWaitEvent(st, ev[l], 0) != hipSuccess) &&
        status == MUON_OK)
      status = MUON_ELAUNCH;
  return status;
}

}  // extern "C"
