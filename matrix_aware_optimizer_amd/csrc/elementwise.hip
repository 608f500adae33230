// HBM-bound kernels of the step: momentum EMA with per-matrix sum of squares
// (a1), sign + 1-bit packing (a6), majority vote (a7) and the update (a8).
//
// Every kernel streams its operands once with 16-byte vector accesses
// (8 bf16 or 4 fp32 per access, consecutive lanes on consecutive addresses)
// and keeps all arithmetic in registers.  Reductions use a fixed order so
// identical inputs give bit-identical outputs.
#include "common.h"

namespace muon {
namespace {

// ---------------------------------------------------------------------------
// a1: momentum EMA + per-segment sum of squares.
// A block owns a chunk of kChunk consecutive entries.  The chunk's part inside
// segment s is the "piece" (block b, segment s); its partial sum goes to
// partials[b + s], an index that is unique for every non-empty piece.
// ---------------------------------------------------------------------------
constexpr int kThreads = 256;
constexpr int kIters = 2;
constexpr int64_t kChunk = int64_t(kThreads) * 8 * kIters;  // 4096 entries

struct SegMap {
  const int64_t* offs;  // device offsets [nseg+1], or null for uniform segments
  int64_t uniform;      // segment length when offs is null
  int nseg;
  __device__ __forceinline__ int64_t at(int s) const {
    return offs ? offs[s] : int64_t(s) * uniform;
  }
};

// beta*m + alpha*g rounded once: both products of fp32 values are exact in
// fp64, the fp64 fma rounds their sum once, then it is rounded to fp32.
__device__ __forceinline__ float ema(float beta, float m, float alpha, float g) {
  return static_cast<float>(fma(static_cast<double>(beta), static_cast<double>(m),
                                static_cast<double>(alpha) * static_cast<double>(g)));
}

__device__ __forceinline__ double block_sum(double v, double* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x == 0)
    for (int i = 0; i < kThreads / kWave; ++i) t += red[i];
  __syncthreads();
  return t;
}

template <typename TM, typename TG, bool UPDATE, bool SUMS>
__global__ __launch_bounds__(kThreads) void momentum_kernel(TM* __restrict__ M,
                                                           const TG* __restrict__ G,
                                                           int64_t numel, SegMap seg,
                                                           float beta, float alpha,
                                                           double* __restrict__ partials) {
  const int64_t c0 = int64_t(blockIdx.x) * kChunk;
  const int64_t c1 = min(numel, c0 + kChunk);
  float vals[kIters][8];
  if (c1 - c0 == kChunk) {
    // full chunk: every load is issued before any arithmetic
    float g[kIters][8];
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int64_t e0 = c0 + int64_t(it) * (kThreads * 8) + threadIdx.x * 8;
      Vec8<TM>::load(M + e0, vals[it]);
      if (UPDATE) Vec8<TG>::load(G + e0, g[it]);
    }
    if (UPDATE) {
#pragma unroll
      for (int it = 0; it < kIters; ++it) {
        const int64_t e0 = c0 + int64_t(it) * (kThreads * 8) + threadIdx.x * 8;
#pragma unroll
        for (int q = 0; q < 8; ++q) vals[it][q] = ema(beta, vals[it][q], alpha, g[it][q]);
        Vec8<TM>::store(M + e0, vals[it]);
        // the stored value is what the norm must see
#pragma unroll
        for (int q = 0; q < 8; ++q) vals[it][q] = to_f32(from_f32<TM>(vals[it][q]));
      }
    }
  } else {
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int64_t e0 = c0 + int64_t(it) * (kThreads * 8) + threadIdx.x * 8;
    if (e0 + 8 <= c1) {
      float m[8];
      Vec8<TM>::load(M + e0, m);
      if (UPDATE) {
        float g[8];
        Vec8<TG>::load(G + e0, g);
#pragma unroll
        for (int q = 0; q < 8; ++q) m[q] = ema(beta, m[q], alpha, g[q]);
        Vec8<TM>::store(M + e0, m);
        // the stored value is what the norm must see
#pragma unroll
        for (int q = 0; q < 8; ++q) m[q] = to_f32(from_f32<TM>(m[q]));
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) vals[it][q] = m[q];
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        float m = 0.0f;
        if (e0 + q < c1) {
          m = to_f32(M[e0 + q]);
          if (UPDATE) {
            const TM st = from_f32<TM>(ema(beta, m, alpha, to_f32(G[e0 + q])));
            M[e0 + q] = st;
            m = to_f32(st);
          }
        }
        vals[it][q] = m;
      }
    }
  }
  }
  if (!SUMS) return;

  __shared__ double red[kThreads / kWave];
  __shared__ int s_first;
  if (threadIdx.x == 0) {
    // largest s with offset(s) <= c0; that segment contains entry c0
    int lo = 0, hi = seg.nseg - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (seg.at(mid) <= c0) lo = mid; else hi = mid - 1;
    }
    s_first = lo;
  }
  __syncthreads();
  for (int s = s_first; s < seg.nseg; ++s) {
    const int64_t s0 = seg.at(s), s1 = seg.at(s + 1);
    if (s0 >= c1) break;
    const int64_t p0 = max(c0, s0), p1 = min(c1, s1);
    if (p0 >= p1) continue;
    double acc = 0.0;
    if (p0 == c0 && p1 == c1) {   // the chunk lies inside one segment (entries past numel are 0)
#pragma unroll
      for (int it = 0; it < kIters; ++it)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc = fma(double(vals[it][q]), double(vals[it][q]), acc);
    } else {
#pragma unroll
      for (int it = 0; it < kIters; ++it) {
        const int64_t e0 = c0 + int64_t(it) * (kThreads * 8) + threadIdx.x * 8;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const double v = vals[it][q];
          if (e0 + q >= p0 && e0 + q < p1) acc = fma(v, v, acc);
        }
      }
    }
    const double tot = block_sum(acc, red);
    if (threadIdx.x == 0) partials[blockIdx.x + s] = tot;
  }
}

// One block of kReduceThreads per segment adds that segment's piece partials
// in a fixed order: thread t adds entries b0 + t, b0 + t + kReduceThreads, ...
// in that order, with kReduceLoads loads in flight, then the block sum runs
// in a fixed butterfly order.  A segment of one 4096 x 14336 matrix has 14336
// partials: one pass of loads per thread.
constexpr int kReduceThreads = 1024;
constexpr int kReduceLoads = 16;

__global__ __launch_bounds__(kReduceThreads) void segment_reduce_kernel(const double* __restrict__ partials,
                                                                       SegMap seg, int64_t nchunks,
                                                                       float* __restrict__ out) {
  __shared__ double red[kReduceThreads / kWave];
  const int s = blockIdx.x;
  const int64_t s0 = seg.at(s), s1 = seg.at(s + 1);
  double acc = 0.0;
  if (s1 > s0 && s0 >= 0) {
    // clamped so that offsets beyond numel cannot index past the partials
    const int64_t b0 = s0 / kChunk, b1 = min((s1 - 1) / kChunk, nchunks - 1);
    for (int64_t b = b0 + threadIdx.x; b <= b1; b += int64_t(kReduceLoads) * kReduceThreads) {
      double x[kReduceLoads];
#pragma unroll
      for (int j = 0; j < kReduceLoads; ++j) {
        const int64_t i = b + int64_t(j) * kReduceThreads;
        x[j] = i <= b1 ? partials[i + s] : 0.0;
      }
#pragma unroll
      for (int j = 0; j < kReduceLoads; ++j) acc += x[j];
    }
  }
  acc = wave_sum(acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int i = 0; i < kReduceThreads / kWave; ++i) t += red[i];
    out[s] = static_cast<float>(t);
  }
}

template <typename TM, typename TG, bool UPDATE>
int launch_momentum(TM* M, const TG* G, int64_t numel, SegMap seg, float beta, float alpha,
                    float* sumsq_out, double* partials, hipStream_t stream) {
  const int64_t nchunks = (numel + kChunk - 1) / kChunk;
  if (nchunks == 0 && !(sumsq_out && seg.nseg > 0)) return MUON_OK;  // nothing to launch
  if (nchunks > 0) {
    if (sumsq_out)
      launch_kernel(momentum_kernel<TM, TG, UPDATE, true>, dim3(nchunks), dim3(kThreads), 0, stream, 
          M, G, numel, seg, beta, alpha, partials);
    else
      launch_kernel(momentum_kernel<TM, TG, UPDATE, false>, dim3(nchunks), dim3(kThreads), 0, stream, 
          M, G, numel, seg, beta, alpha, partials);
  }
  if (sumsq_out && seg.nseg > 0)
    launch_kernel(segment_reduce_kernel, dim3(seg.nseg), dim3(kReduceThreads), 0, stream, partials, seg, nchunks,
                                                                          sumsq_out);
  return launch_status();
}

// ---------------------------------------------------------------------------
// a6: sign + pack.  Each lane turns 8 consecutive entries into one byte of
// bits; eight neighbouring lanes merge their bytes into one 64-bit word with
// three shuffles, and every eighth lane stores it.  The test "u < 0" is done
// on the encoding (sign bit set, magnitude non-zero, not NaN), so it is exact
// for subnormals whatever the float mode.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t nonneg_bit(bf16_t h) {
  return !(h > 0x8000u && h <= 0xff80u);
}
__device__ __forceinline__ uint32_t nonneg_bit(uint32_t u) {
  return !(u > 0x80000000u && u <= 0xff800000u);
}

template <typename T> struct SignByte;
template <> struct SignByte<bf16_t> {
  __device__ __forceinline__ static uint32_t full(const bf16_t* p) {
    const uint4 r = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
    uint32_t byte = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      byte |= nonneg_bit(static_cast<bf16_t>(w[i] & 0xffffu)) << (2 * i);
      byte |= nonneg_bit(static_cast<bf16_t>(w[i] >> 16)) << (2 * i + 1);
    }
    return byte;
  }
  __device__ __forceinline__ static uint32_t one(const bf16_t* p) { return nonneg_bit(*p); }
};
template <> struct SignByte<float> {
  __device__ __forceinline__ static uint32_t full(const float* p) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    const uint4 b = *reinterpret_cast<const uint4*>(p + 4);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t byte = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) byte |= nonneg_bit(w[i]) << i;
    return byte;
  }
  __device__ __forceinline__ static uint32_t one(const float* p) {
    return nonneg_bit(*reinterpret_cast<const uint32_t*>(p));
  }
};

// A block packs kPackGroups groups of kThreads * 8 entries; each lane tests
// its 8 entries of every group (all loads first), then the groups are merged
// and stored one after another.
constexpr int kPackGroups = 4;
constexpr int64_t kPackBlock = int64_t(kPackGroups) * kThreads * 8;   // entries per block

template <typename T>
__global__ __launch_bounds__(kThreads) void sign_pack_kernel(const T* __restrict__ U, int64_t numel,
                                                            uint64_t* __restrict__ bits,
                                                            int64_t nwords, int64_t strideU, int64_t stride_bits) {
  // grid y: equal problems strideU elements and stride_bits words apart
  U += int64_t(blockIdx.y) * strideU;
  bits += int64_t(blockIdx.y) * stride_bits;
  const int64_t base = int64_t(blockIdx.x) * kPackBlock + threadIdx.x * 8;
  uint32_t byte[kPackGroups];
  if (int64_t(blockIdx.x + 1) * kPackBlock <= numel) {
#pragma unroll
    for (int g = 0; g < kPackGroups; ++g) byte[g] = SignByte<T>::full(U + base + g * (kThreads * 8));
  } else {
#pragma unroll
    for (int g = 0; g < kPackGroups; ++g) {
      const int64_t e0 = base + g * (kThreads * 8);
      byte[g] = 0;
      if (e0 + 8 <= numel) {
        byte[g] = SignByte<T>::full(U + e0);
      } else {
        for (int q = 0; q < 8; ++q)
          if (e0 + q < numel) byte[g] |= SignByte<T>::one(U + e0 + q) << q;
      }
    }
  }
#pragma unroll
  for (int g = 0; g < kPackGroups; ++g) {
    uint32_t v = byte[g];
    v |= static_cast<uint32_t>(__shfl_down(static_cast<int>(v), 1, kWave)) << 8;
    v |= static_cast<uint32_t>(__shfl_down(static_cast<int>(v), 2, kWave)) << 16;
    const uint32_t hi = static_cast<uint32_t>(__shfl_down(static_cast<int>(v), 4, kWave));
    if ((threadIdx.x & 7) == 0) {
      const int64_t w = (base + g * (kThreads * 8)) >> 6;
      if (w < nwords) bits[w] = static_cast<uint64_t>(v) | (static_cast<uint64_t>(hi) << 32);
    }
  }
}

// ---------------------------------------------------------------------------
// a7: majority vote.  A bit-sliced counter (NB planes of 64 bits) adds the M
// buffers' words; the result is compared with ceil(M/2) plane by plane.
// ---------------------------------------------------------------------------
template <int NB, typename W>
__device__ __forceinline__ void counter_add(W (&cnt)[NB], W x) {
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const W carry = cnt[i] & x;
    cnt[i] ^= x;
    x = carry;
  }
}

// bit set where the per-bit count is >= thr (thr < 2^NB)
template <int NB, typename W>
__device__ __forceinline__ W counter_ge(const W (&cnt)[NB], int thr) {
  W gt = 0, eq = ~W(0);
#pragma unroll
  for (int i = NB - 1; i >= 0; --i) {
    if ((thr >> i) & 1) {
      eq &= cnt[i];
    } else {
      gt |= eq & cnt[i];
      eq &= ~cnt[i];
    }
  }
  return gt | eq;
}

// The workers' words are loaded kVoteChunk at a time: loads past M are not
// issued and add zero, so all loads of a chunk are in flight before the
// first counter add (a loop that added each word as it arrived waited on the
// loads one after another).
constexpr int kVoteChunk = 8;

// One lane per word.
template <int NB>
__global__ __launch_bounds__(kThreads) void vote_kernel(const uint64_t* __restrict__ bits, int M,
                                                       int64_t nwords, uint64_t* __restrict__ out) {
  const int64_t w = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (w >= nwords) return;
  uint64_t cnt[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) cnt[i] = 0;
  for (int k = 0; k < M; k += kVoteChunk) {
    uint64_t x[kVoteChunk];
#pragma unroll
    for (int j = 0; j < kVoteChunk; ++j) x[j] = k + j < M ? bits[int64_t(k + j) * nwords + w] : 0ull;
#pragma unroll
    for (int j = 0; j < kVoteChunk; ++j) counter_add<NB>(cnt, x[j]);
  }
  out[w] = counter_ge<NB>(cnt, (M + 1) >> 1);
}

// 16-byte accesses with the nontemporal hint: every word is touched once, so
// the caches need not keep it (measured 4-8% faster for the vote than plain
// loads and stores, warm or cold).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream(uint4* p, uint4 x) {
  const u32x4_t v = {x.x, x.y, x.z, x.w};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

// Two words per 16-byte access when every buffer row is 16-byte aligned (an
// even word count); a lane handles kVotePairs such pairs, kThreads pairs
// apart, so consecutive lanes stay on consecutive addresses.  Same
// arithmetic per word.
constexpr int kVotePairs = 1;

template <int NB>
__global__ __launch_bounds__(kThreads) void vote2_kernel(const uint4* __restrict__ bits, int M,
                                                        int64_t npairs, uint4* __restrict__ out) {
  const int64_t t0 = int64_t(blockIdx.x) * (kThreads * kVotePairs) + threadIdx.x;
  uint64_t c[kVotePairs][2][NB];
#pragma unroll
  for (int p = 0; p < kVotePairs; ++p)
#pragma unroll
    for (int i = 0; i < NB; ++i) c[p][0][i] = c[p][1][i] = 0;
  auto add = [&](int p, const uint4 x) {
    counter_add<NB>(c[p][0], static_cast<uint64_t>(x.x) | (static_cast<uint64_t>(x.y) << 32));
    counter_add<NB>(c[p][1], static_cast<uint64_t>(x.z) | (static_cast<uint64_t>(x.w) << 32));
  };
  for (int k = 0; k < M; k += kVoteChunk) {
    uint4 x[kVoteChunk][kVotePairs];
#pragma unroll
    for (int j = 0; j < kVoteChunk; ++j)
#pragma unroll
      for (int p = 0; p < kVotePairs; ++p) {
        const int64_t t = t0 + int64_t(p) * kThreads;
        x[j][p] = t < npairs && k + j < M ? load_stream(bits + int64_t(k + j) * npairs + t) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
    for (int j = 0; j < kVoteChunk; ++j)
#pragma unroll
      for (int p = 0; p < kVotePairs; ++p) add(p, x[j][p]);
  }
#pragma unroll
  for (int p = 0; p < kVotePairs; ++p) {
    const int64_t t = t0 + int64_t(p) * kThreads;
    if (t >= npairs) continue;
    const uint64_t v0 = counter_ge<NB>(c[p][0], (M + 1) >> 1), v1 = counter_ge<NB>(c[p][1], (M + 1) >> 1);
    store_stream(out + t, make_uint4(static_cast<uint32_t>(v0), static_cast<uint32_t>(v0 >> 32),
                                     static_cast<uint32_t>(v1), static_cast<uint32_t>(v1 >> 32)));
  }
}

// ---------------------------------------------------------------------------
// a8: update, and the fused vote + update.  A lane updates 8 consecutive
// weights with one byte of vote bits.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void update8(T* __restrict__ W, int64_t e0, int64_t numel, uint32_t byte,
                                        float eta) {
  if (e0 + 8 <= numel) {
    float v[8];
    Vec8<T>::load(W + e0, v);
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = ((byte >> q) & 1u) ? v[q] - eta : v[q] + eta;
    Vec8<T>::store(W + e0, v);
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (e0 + q < numel) {
        const float x = to_f32(W[e0 + q]);
        W[e0 + q] = from_f32<T>(((byte >> q) & 1u) ? x - eta : x + eta);
      }
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void update_kernel(T* __restrict__ W, int64_t numel,
                                                         const uint8_t* __restrict__ vote,
                                                         float eta) {
  const int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t e0 = t * 8;
  if (e0 >= numel) return;
  update8<T>(W, e0, numel, vote[t], eta);
}

// The workers' vote bytes are loaded a chunk at a time as in the vote, and
// the lane's weights before them.

template <typename T, int NB>
__device__ __forceinline__ uint32_t vote_byte(const uint8_t* __restrict__ bits, int M, int64_t nbytes,
                                              int64_t t) {
  uint32_t cnt[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) cnt[i] = 0;
  // the first chunk outside the loop: a loop's head waits for every load in
  // flight, the caller's weights included
  auto chunk = [&](int k) {
    uint32_t x[kVoteChunk];
#pragma unroll
    for (int j = 0; j < kVoteChunk; ++j) x[j] = k + j < M ? bits[int64_t(k + j) * nbytes + t] : 0u;
#pragma unroll
    for (int j = 0; j < kVoteChunk; ++j) counter_add<NB>(cnt, x[j]);
  };
  chunk(0);
  for (int k = kVoteChunk; k < M; k += kVoteChunk) chunk(k);
  return counter_ge<NB>(cnt, (M + 1) >> 1) & 0xffu;
}

template <typename T, int NB>
__global__ __launch_bounds__(kThreads) void vote_update_kernel(T* __restrict__ W, int64_t numel,
                                                              const uint8_t* __restrict__ bits,
                                                              int M, int64_t nbytes, float eta) {
  const int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t e0 = t * 8;
  if (e0 >= numel) return;
  if (e0 + 8 > numel) {      // the ragged tail
    update8<T>(W, e0, numel, vote_byte<T, NB>(bits, M, nbytes, t), eta);
    return;
  }
  // the lane's 8 weights are loaded raw first and converted only after the
  // vote, so their load stays in flight with the vote's
  constexpr int NV = sizeof(T) * 8 / 16;      // 16-byte vectors: 1 (bf16) or 2 (fp32)
  uint4 raw[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) raw[i] = reinterpret_cast<const uint4*>(W + e0)[i];
  const uint32_t byte = vote_byte<T, NB>(bits, M, nbytes, t);
  float v[8];
  if constexpr (sizeof(T) == 2) {
    const uint32_t w[4] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      v[4 * i] = __uint_as_float(raw[i].x);
      v[4 * i + 1] = __uint_as_float(raw[i].y);
      v[4 * i + 2] = __uint_as_float(raw[i].z);
      v[4 * i + 3] = __uint_as_float(raw[i].w);
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) v[q] = ((byte >> q) & 1u) ? v[q] - eta : v[q] + eta;
  Vec8<T>::store(W + e0, v);
}

// ---------------------------------------------------------------------------
// int8 exchange format: signs as int8 +-1, their SUM over the workers, and
// the local threshold of the sum packed to bits.
// ---------------------------------------------------------------------------
constexpr int kInt8PerLane = 16;

template <typename T>
__global__ __launch_bounds__(kThreads) void sign_int8_kernel(const T* __restrict__ U, int64_t numel,
                                                            int8_t* __restrict__ S) {
  const int64_t e0 = (int64_t(blockIdx.x) * kThreads + threadIdx.x) * kInt8PerLane;
  if (e0 >= numel) return;
  if (e0 + kInt8PerLane <= numel) {
    // bit q of the two bytes of entries is 1 for +1; byte = 0x01 (+1) or 0xff (-1)
    const uint32_t lo = SignByte<T>::full(U + e0), hi = SignByte<T>::full(U + e0 + 8);
    const uint32_t bitsv = lo | (hi << 8);
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t v = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) v |= (((bitsv >> (4 * d + b)) & 1u) ? 0x01u : 0xffu) << (8 * b);
      w[d] = v;
    }
    *reinterpret_cast<uint4*>(S + e0) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    for (int q = 0; e0 + q < numel; ++q) S[e0 + q] = SignByte<T>::one(U + e0 + q) ? int8_t(1) : int8_t(-1);
  }
}

// per-byte addition modulo 256 of four int8 lanes packed in a word: exact
// for sums that fit int8
__device__ __forceinline__ uint32_t add_bytes(uint32_t a, uint32_t b) {
  return ((a & 0x7f7f7f7fu) + (b & 0x7f7f7f7fu)) ^ ((a ^ b) & 0x80808080u);
}
__device__ __forceinline__ uint4 add_bytes(uint4 a, uint4 b) {
  return make_uint4(add_bytes(a.x, b.x), add_bytes(a.y, b.y), add_bytes(a.z, b.z), add_bytes(a.w, b.w));
}

// rows of 16-byte multiples: 16 sums per lane, rows read kVoteChunk at a
// time as in the vote (absent rows add zero)
__global__ __launch_bounds__(kThreads) void sum_int8_kernel(const uint4* __restrict__ S, int M,
                                                           int64_t nvec, uint4* __restrict__ out) {
  const int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (t >= nvec) return;
  uint4 acc = make_uint4(0, 0, 0, 0);
  for (int k = 0; k < M; k += kVoteChunk) {
    uint4 x[kVoteChunk];
#pragma unroll
    for (int j = 0; j < kVoteChunk; ++j) x[j] = k + j < M ? load_stream(S + int64_t(k + j) * nvec + t) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < kVoteChunk; ++j) acc = add_bytes(acc, x[j]);
  }
  out[t] = acc;
}

// any length: one sum per lane
__global__ __launch_bounds__(kThreads) void sum_int8_bytes_kernel(const int8_t* __restrict__ S, int M,
                                                                 int64_t numel, int8_t* __restrict__ out) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= numel) return;
  int acc = 0;
  for (int k = 0; k < M; ++k) acc += S[int64_t(k) * numel + i];
  out[i] = static_cast<int8_t>(acc);
}

// bit i = 1 iff sum[i] >= 0; 16 sums per lane (one 16-byte load), four lanes
// per 64-bit word
__device__ __forceinline__ uint32_t nonneg_nibble(uint32_t x) {   // 4 int8 lanes -> 4 bits
  const uint32_t sgn = ((x >> 7) & 1u) | ((x >> 14) & 2u) | ((x >> 21) & 4u) | ((x >> 28) & 8u);
  return ~sgn & 0xfu;
}

__global__ __launch_bounds__(kThreads) void threshold_pack_kernel(const int8_t* __restrict__ sum,
                                                                 int64_t numel, uint64_t* __restrict__ bits,
                                                                 int64_t nwords) {
  const int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t e0 = t * 16;
  uint32_t v = 0;
  if (e0 + 16 <= numel) {
    const uint4 x = *reinterpret_cast<const uint4*>(sum + e0);
    v = nonneg_nibble(x.x) | (nonneg_nibble(x.y) << 4) | (nonneg_nibble(x.z) << 8) |
        (nonneg_nibble(x.w) << 12);
  } else {
    for (int q = 0; q < 16; ++q)
      if (e0 + q < numel) v |= (sum[e0 + q] >= 0 ? 1u : 0u) << q;
  }
  v |= static_cast<uint32_t>(__shfl_down(static_cast<int>(v), 1, kWave)) << 16;
  const uint32_t hi = static_cast<uint32_t>(__shfl_down(static_cast<int>(v), 2, kWave));
  if ((threadIdx.x & 3) == 0) {
    const int64_t w = e0 >> 6;
    if (w < nwords) bits[w] = static_cast<uint64_t>(v) | (static_cast<uint64_t>(hi) << 32);
  }
}

// ---------------------------------------------------------------------------
// Local re-orthogonalisation of the vote: the vote bits as a +-1 matrix, and
// the dense update W <- W - eta * U.
// ---------------------------------------------------------------------------
// 16 entries (two bytes of bits) per lane
constexpr int kUnpackPerLane = 8;   // entries (vote bits) per lane: 8, 16 or 32 (8 measured fastest)

template <typename T>
__global__ __launch_bounds__(kThreads) void unpack_signs_kernel(const uint8_t* __restrict__ bits,
                                                               int64_t numel, T* __restrict__ out) {
  const int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t e0 = t * kUnpackPerLane;
  if (e0 >= numel) return;
  if (e0 + kUnpackPerLane <= numel) {
    // one load of the lane's kUnpackPerLane vote bits, then groups of 8 outputs
    uint32_t bw;
    if constexpr (kUnpackPerLane == 8) bw = bits[t];
    else if constexpr (kUnpackPerLane == 16) bw = *reinterpret_cast<const uint16_t*>(bits + 2 * t);
    else bw = *reinterpret_cast<const uint32_t*>(bits + 4 * t);
#pragma unroll
    for (int g = 0; g < kUnpackPerLane / 8; ++g) {
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = ((bw >> (8 * g + q)) & 1u) ? 1.0f : -1.0f;
      Vec8<T>::store(out + e0 + 8 * g, v);
    }
  } else {
    for (int q = 0; e0 + q < numel; ++q)
      out[e0 + q] = from_f32<T>(((bits[(e0 + q) >> 3] >> ((e0 + q) & 7)) & 1u) ? 1.0f : -1.0f);
  }
}

// W, eta and U are fp32 values: eta * U is exact in fp64, the fp64
// difference is rounded once, then to fp32 (and bf16 for bf16 storage)
__device__ __forceinline__ float dense_step(float w, float eta, float u) {
  return static_cast<float>(static_cast<double>(w) - static_cast<double>(eta) * static_cast<double>(u));
}

template <typename TW, typename TU>
__global__ __launch_bounds__(kThreads) void update_dense_kernel(TW* __restrict__ W, int64_t numel,
                                                               const TU* __restrict__ U, float eta) {
  const int64_t e0 = (int64_t(blockIdx.x) * kThreads + threadIdx.x) * 8;
  if (e0 >= numel) return;
  if (e0 + 8 <= numel) {
    float w[8], u[8];
    Vec8<TW>::load(W + e0, w);
    Vec8<TU>::load(U + e0, u);
#pragma unroll
    for (int q = 0; q < 8; ++q) w[q] = dense_step(w[q], eta, u[q]);
    Vec8<TW>::store(W + e0, w);
  } else {
    for (int q = 0; e0 + q < numel; ++q)
      W[e0 + q] = from_f32<TW>(dense_step(to_f32(W[e0 + q]), eta, to_f32(U[e0 + q])));
  }
}

int planes_for(int M) {
  int nb = 1;
  while ((1 << nb) <= M) ++nb;
  return nb;
}

template <template <int> class F, typename... Args>
int dispatch_planes(int nb, Args... args) {
  switch (nb) {
    case 1: return F<1>::run(args...);
    case 2: return F<2>::run(args...);
    case 3: return F<3>::run(args...);
    case 4: return F<4>::run(args...);
    case 5: return F<5>::run(args...);
    case 6: return F<6>::run(args...);
    case 7: return F<7>::run(args...);
    case 8: return F<8>::run(args...);
    case 9: return F<9>::run(args...);
    case 10: return F<10>::run(args...);
    default: return MUON_EINVAL;
  }
}

template <int NB> struct VoteLaunch {
  static int run(const uint64_t* bits, int M, int64_t nwords, uint64_t* out, hipStream_t st) {
    if (nwords % 2 == 0) {
      const int64_t npairs = nwords / 2;
      const int64_t blocks = (npairs + kThreads * kVotePairs - 1) / (kThreads * kVotePairs);
      launch_kernel(vote2_kernel<NB>, dim3(blocks), dim3(kThreads), 0, st, reinterpret_cast<const uint4*>(bits), M,
                                                                 npairs, reinterpret_cast<uint4*>(out));
    } else {
      const int64_t blocks = (nwords + kThreads - 1) / kThreads;
      launch_kernel(vote_kernel<NB>, dim3(blocks), dim3(kThreads), 0, st, bits, M, nwords, out);
    }
    return launch_status();
  }
};

template <int NB> struct VoteUpdateLaunch {
  static int run(void* W, int w_dtype, int64_t numel, const uint64_t* bits, int M, int64_t nwords,
                 float eta, hipStream_t st) {
    const int64_t blocks = ((numel + 7) / 8 + kThreads - 1) / kThreads;
    const uint8_t* b8 = reinterpret_cast<const uint8_t*>(bits);
    if (w_dtype == MUON_BF16)
      launch_kernel(vote_update_kernel<bf16_t, NB>, dim3(blocks), dim3(kThreads), 0, st, 
          static_cast<bf16_t*>(W), numel, b8, M, nwords * 8, eta);
    else
      launch_kernel(vote_update_kernel<float, NB>, dim3(blocks), dim3(kThreads), 0, st, 
          static_cast<float*>(W), numel, b8, M, nwords * 8, eta);
    return launch_status();
  }
};

}  // namespace

// Sum of squares of `count` equal matrices of `len` entries spaced `stride`
// entries apart (the normalisation's norm when the caller supplies none).
// partials needs muon_momentum_workspace_bytes(len * count, count) bytes when
// stride == len, else muon_momentum_workspace_bytes(len, 1) bytes.
int sumsq_strided(const void* M, int m_dtype, int64_t len, int64_t count, int64_t stride,
                  float* out, void* partials, hipStream_t stream) {
  double* part = static_cast<double*>(partials);
  if (stride == len) {
    SegMap seg{nullptr, len, static_cast<int>(count)};
    if (m_dtype == MUON_BF16)
      return launch_momentum<bf16_t, bf16_t, false>(static_cast<bf16_t*>(const_cast<void*>(M)),
                                                     nullptr, len * count, seg, 1.f, 0.f, out,
                                                     part, stream);
    return launch_momentum<float, float, false>(static_cast<float*>(const_cast<void*>(M)), nullptr,
                                                len * count, seg, 1.f, 0.f, out, part, stream);
  }
  for (int64_t i = 0; i < count; ++i) {
    SegMap seg{nullptr, len, 1};
    const size_t es = dtype_size(m_dtype);
    void* Mi = static_cast<char*>(const_cast<void*>(M)) + i * stride * es;
    int st;
    if (m_dtype == MUON_BF16)
      st = launch_momentum<bf16_t, bf16_t, false>(static_cast<bf16_t*>(Mi), nullptr, len, seg,
                                                  1.f, 0.f, out + i, part, stream);
    else
      st = launch_momentum<float, float, false>(static_cast<float*>(Mi), nullptr, len, seg, 1.f,
                                                0.f, out + i, part, stream);
    if (st != MUON_OK) return st;
  }
  return MUON_OK;
}

}  // namespace muon

// ---------------------------------------------------------------------------
// Fixed scratch of muon_momentum_noalloc: the per-piece partial sums of the
// norms (the buffer muon_momentum takes as its workspace), 4 MiB on every
// device the library runs on, held until the process ends.  Host code never
// passes `scratch` itself to a kernel (on the host it only names the symbol):
// it passes the device address looked up once per device below.
// ---------------------------------------------------------------------------
static constexpr int64_t kScratchDoubles = int64_t(1) << 19;
static __device__ __align__(256) double scratch[kScratchDoubles];

namespace muon {
namespace {

// Device address of the current device's copy of `scratch`, looked up with
// that device current on its first use and kept per device (ordinals past the
// tracked range look it up on every call).
int scratch_address(double** out) {
  static std::atomic<uintptr_t> cache[kMaxTrackedDevices];
  const int dev = current_device();
  if (dev < 0) return MUON_ELAUNCH;
  if (dev < kMaxTrackedDevices) {
    const uintptr_t cached = cache[dev].load(std::memory_order_acquire);
    if (cached != 0) {
      *out = reinterpret_cast<double*>(cached);
      return MUON_OK;
    }
  }
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return MUON_ELAUNCH;
  if (dev < kMaxTrackedDevices) cache[dev].store(reinterpret_cast<uintptr_t>(ptr), std::memory_order_release);
  *out = static_cast<double*>(ptr);
  return MUON_OK;
}

}  // namespace
}  // namespace muon

using namespace muon;

namespace muon {
// sign_pack of `count` problems of numel entries each, strideU entries and
// stride_bits words apart, in one launch (a run of ns_orthogonalize whose
// signs are packed after the iteration).  Each problem's words are its own:
// a last partial word holds zeros past numel.  U and every problem's U
// 16-byte aligned, bits 8-byte aligned; MUON_EALIGN otherwise.
int sign_pack_runs(const void* U, int u_dtype, int64_t numel, int64_t count, int64_t strideU, uint64_t* bits,
                   int64_t stride_bits, hipStream_t st) {
  if (!numel_ok(numel) || count < 0 || count > 65535 || strideU < 0 || stride_bits < 0) return MUON_EINVAL;
  if (!valid_dtype(u_dtype)) return MUON_EDTYPE;
  if (numel == 0 || count == 0) return MUON_OK;
  if (!U || !bits) return MUON_EINVAL;
  if (!aligned16(U) || (strideU * int64_t(dtype_size(u_dtype))) % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(bits) & 7u) != 0)
    return MUON_EALIGN;
  const int64_t nwords = (numel + 63) / 64;
  const int64_t blocks = (numel + kPackBlock - 1) / kPackBlock;
  if (u_dtype == MUON_BF16)
    launch_kernel(sign_pack_kernel<bf16_t>, dim3(blocks, count), dim3(kThreads), 0, st,
                  static_cast<const bf16_t*>(U), numel, bits, nwords, strideU, stride_bits);
  else
    launch_kernel(sign_pack_kernel<float>, dim3(blocks, count), dim3(kThreads), 0, st,
                  static_cast<const float*>(U), numel, bits, nwords, strideU, stride_bits);
  return launch_status();
}
}  // namespace muon

extern "C" {

size_t muon_momentum_workspace_bytes(int64_t numel, int nseg) {
  if (!numel_ok(numel) || nseg < 0) return 0;
  const int64_t nchunks = (numel + kChunk - 1) / kChunk;
  return round_up(static_cast<size_t>(nchunks + nseg + 1) * sizeof(double), 256);
}

int muon_momentum(void* M, int m_dtype, const void* G, int g_dtype, int64_t numel,
                  const int64_t* seg_offsets, int nseg, float beta, float alpha, float* sumsq_out,
                  void* workspace, size_t ws_bytes, void* stream) {
  if (!numel_ok(numel)) return MUON_EINVAL;
  if (!valid_dtype(m_dtype) || !valid_dtype(g_dtype)) return MUON_EDTYPE;
  if (numel > 0 && (!M || !G)) return MUON_EINVAL;
  if (numel > 0 && (!aligned16(M) || !aligned16(G))) return MUON_EALIGN;
  if (sumsq_out) {
    if (nseg < 1 || !seg_offsets) return MUON_EINVAL;
    if (!aligned16(seg_offsets)) return MUON_EALIGN;
    if (!workspace || ws_bytes < muon_momentum_workspace_bytes(numel, nseg)) return MUON_EWORKSPACE;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  SegMap seg{seg_offsets, 0, sumsq_out ? nseg : 0};
  double* part = static_cast<double*>(workspace);
  if (m_dtype == MUON_BF16 && g_dtype == MUON_BF16)
    return launch_momentum<bf16_t, bf16_t, true>(static_cast<bf16_t*>(M), static_cast<const bf16_t*>(G),
                                                 numel, seg, beta, alpha, sumsq_out, part, st);
  if (m_dtype == MUON_BF16 && g_dtype == MUON_F32)
    return launch_momentum<bf16_t, float, true>(static_cast<bf16_t*>(M), static_cast<const float*>(G),
                                                numel, seg, beta, alpha, sumsq_out, part, st);
  if (m_dtype == MUON_F32 && g_dtype == MUON_BF16)
    return launch_momentum<float, bf16_t, true>(static_cast<float*>(M), static_cast<const bf16_t*>(G),
                                                numel, seg, beta, alpha, sumsq_out, part, st);
  return launch_momentum<float, float, true>(static_cast<float*>(M), static_cast<const float*>(G),
                                             numel, seg, beta, alpha, sumsq_out, part, st);
}

int muon_momentum_noalloc(void* M, int m_dtype, const void* G, int g_dtype, int64_t numel,
                          const int64_t* seg_offsets, int nseg, float beta, float alpha,
                          float* sumsq_out, void* stream) {
  if (!numel_ok(numel)) return MUON_EINVAL;
  if (!valid_dtype(m_dtype) || !valid_dtype(g_dtype)) return MUON_EDTYPE;
  if (numel > 0 && (!M || !G)) return MUON_EINVAL;
  if (numel > 0 && (!aligned16(M) || !aligned16(G))) return MUON_EALIGN;
  double* part = nullptr;
  if (sumsq_out) {
    if (nseg < 1 || !seg_offsets) return MUON_EINVAL;
    if (!aligned16(seg_offsets)) return MUON_EALIGN;
    if (muon_momentum_workspace_bytes(numel, nseg) > size_t(kScratchDoubles) * sizeof(double))
      return MUON_ESCRATCH;
    const int status = scratch_address(&part);
    if (status != MUON_OK) return status;
  }
  // the partials need no clearing: the reduction reads only pieces this call wrote
  return muon_momentum(M, m_dtype, G, g_dtype, numel, seg_offsets, nseg, beta, alpha, sumsq_out, part,
                       size_t(kScratchDoubles) * sizeof(double), stream);
}

int sign_pack(const void* U, int u_dtype, int64_t numel, uint64_t* bits, void* stream) {
  if (!numel_ok(numel)) return MUON_EINVAL;
  if (!valid_dtype(u_dtype)) return MUON_EDTYPE;
  if (numel == 0) return MUON_OK;
  if (!U || !bits) return MUON_EINVAL;
  if (!aligned16(U) || !aligned16(bits)) return MUON_EALIGN;
  const int64_t nwords = (numel + 63) / 64;
  const int64_t blocks = (numel + kPackBlock - 1) / kPackBlock;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (u_dtype == MUON_BF16)
    launch_kernel(sign_pack_kernel<bf16_t>, dim3(blocks), dim3(kThreads), 0, st, static_cast<const bf16_t*>(U),
                                                                      numel, bits, nwords, 0, 0);
  else
    launch_kernel(sign_pack_kernel<float>, dim3(blocks), dim3(kThreads), 0, st, static_cast<const float*>(U),
                                                                     numel, bits, nwords, 0, 0);
  return launch_status();
}


int majority_vote(const uint64_t* bits, int M, int64_t nwords, uint64_t* out, void* stream) {
  if (nwords < 0 || nwords > MUON_MAX_NUMEL / 64 || M < 1 || M > MUON_MAX_VOTERS) return MUON_EINVAL;
  if (nwords == 0) return MUON_OK;
  if (!bits || !out) return MUON_EINVAL;
  if (!aligned16(bits) || !aligned16(out)) return MUON_EALIGN;
  return dispatch_planes<VoteLaunch>(planes_for(M), bits, M, nwords, out,
                                     static_cast<hipStream_t>(stream));
}

int apply_update(void* W, int w_dtype, int64_t numel, const uint64_t* vote_bits, float eta,
                 void* stream) {
  if (!numel_ok(numel)) return MUON_EINVAL;
  if (!valid_dtype(w_dtype)) return MUON_EDTYPE;
  if (numel == 0) return MUON_OK;
  if (!W || !vote_bits) return MUON_EINVAL;
  if (!aligned16(W) || !aligned16(vote_bits)) return MUON_EALIGN;
  const int64_t blocks = ((numel + 7) / 8 + kThreads - 1) / kThreads;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint8_t* v8 = reinterpret_cast<const uint8_t*>(vote_bits);
  if (w_dtype == MUON_BF16)
    launch_kernel(update_kernel<bf16_t>, dim3(blocks), dim3(kThreads), 0, st, static_cast<bf16_t*>(W), numel,
                                                                   v8, eta);
  else
    launch_kernel(update_kernel<float>, dim3(blocks), dim3(kThreads), 0, st, static_cast<float*>(W), numel, v8,
                                                                  eta);
  return launch_status();
}

int vote_and_update(void* W, int w_dtype, int64_t numel, const uint64_t* bits, int M, float eta,
                    void* stream) {
  if (!numel_ok(numel) || M < 1 || M > MUON_MAX_VOTERS) return MUON_EINVAL;
  if (!valid_dtype(w_dtype)) return MUON_EDTYPE;
  if (numel == 0) return MUON_OK;
  if (!W || !bits) return MUON_EINVAL;
  if (!aligned16(W) || !aligned16(bits)) return MUON_EALIGN;
  const int64_t nwords = (numel + 63) / 64;
  return dispatch_planes<VoteUpdateLaunch>(planes_for(M), W, w_dtype, numel, bits, M, nwords, eta,
                                           static_cast<hipStream_t>(stream));
}

const char* muon_status_string(int status) {
  switch (status) {
    case MUON_OK: return "ok";
    case MUON_EINVAL: return "invalid argument (null pointer or bad size)";
    case MUON_EDTYPE: return "unsupported dtype or precision";
    case MUON_EALIGN: return "device pointer not 16-byte aligned";
    case MUON_EWORKSPACE: return "workspace missing or too small";
    case MUON_ELAUNCH: return "kernel launch failed";
    case MUON_ESPLIT:
      return "a split product's second half gave up waiting for the first: its tile was not written";
    case MUON_ESCRATCH:
      return "the problem needs more than the fixed scratch of the allocation-free entry point";
    default: return "unknown status";
  }
}

int muon_version(void) { return 200; }

int muon_time_next_launch(void* start_event, void* stop_event) {
  pending_launch_events() = LaunchEvents{static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event)};
  return MUON_OK;
}


int sign_int8(const void* U, int u_dtype, int64_t numel, int8_t* S, void* stream) {
  if (!numel_ok(numel)) return MUON_EINVAL;
  if (!valid_dtype(u_dtype)) return MUON_EDTYPE;
  if (numel == 0) return MUON_OK;
  if (!U || !S) return MUON_EINVAL;
  if (!aligned16(U) || !aligned16(S)) return MUON_EALIGN;
  const int64_t lanes = (numel + kInt8PerLane - 1) / kInt8PerLane;
  const int64_t blocks = (lanes + kThreads - 1) / kThreads;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (u_dtype == MUON_BF16)
    launch_kernel(sign_int8_kernel<bf16_t>, dim3(blocks), dim3(kThreads), 0, st, static_cast<const bf16_t*>(U), numel, S);
  else
    launch_kernel(sign_int8_kernel<float>, dim3(blocks), dim3(kThreads), 0, st, static_cast<const float*>(U), numel, S);
  return launch_status();
}

int sum_int8(const int8_t* S, int M, int64_t numel, int8_t* out, void* stream) {
  if (!numel_ok(numel) || M < 1 || M > MUON_INT8_MAX_VOTERS) return MUON_EINVAL;
  if (numel == 0) return MUON_OK;
  if (!S || !out) return MUON_EINVAL;
  if (!aligned16(S) || !aligned16(out)) return MUON_EALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (numel % 16 == 0) {
    const int64_t nvec = numel / 16;
    launch_kernel(sum_int8_kernel, dim3((nvec + kThreads - 1) / kThreads), dim3(kThreads), 0, st, 
        reinterpret_cast<const uint4*>(S), M, nvec, reinterpret_cast<uint4*>(out));
  } else {
    launch_kernel(sum_int8_bytes_kernel, dim3((numel + kThreads - 1) / kThreads), dim3(kThreads), 0, st, S, M, numel, out);
  }
  return launch_status();
}

int threshold_pack(const int8_t* sum, int64_t numel, uint64_t* bits, void* stream) {
  if (!numel_ok(numel)) return MUON_EINVAL;
  if (numel == 0) return MUON_OK;
  if (!sum || !bits) return MUON_EINVAL;
  if (!aligned16(sum) || !aligned16(bits)) return MUON_EALIGN;
  const int64_t nwords = (numel + 63) / 64;
  const int64_t blocks = (nwords * 4 + kThreads - 1) / kThreads;
  launch_kernel(threshold_pack_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream), 
      sum, numel, bits, nwords);
  return launch_status();
}

int unpack_signs(const uint64_t* bits, int64_t numel, void* out, int out_dtype, void* stream) {
  if (!numel_ok(numel)) return MUON_EINVAL;
  if (!valid_dtype(out_dtype)) return MUON_EDTYPE;
  if (numel == 0) return MUON_OK;
  if (!bits || !out) return MUON_EINVAL;
  if (!aligned16(bits) || !aligned16(out)) return MUON_EALIGN;
  const int64_t blocks = ((numel + kUnpackPerLane - 1) / kUnpackPerLane + kThreads - 1) / kThreads;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint8_t* b8 = reinterpret_cast<const uint8_t*>(bits);
  if (out_dtype == MUON_BF16)
    launch_kernel(unpack_signs_kernel<bf16_t>, dim3(blocks), dim3(kThreads), 0, st, b8, numel, static_cast<bf16_t*>(out));
  else
    launch_kernel(unpack_signs_kernel<float>, dim3(blocks), dim3(kThreads), 0, st, b8, numel, static_cast<float*>(out));
  return launch_status();
}

int apply_update_dense(void* W, int w_dtype, int64_t numel, const void* U, int u_dtype, float eta,
                       void* stream) {
  if (!numel_ok(numel)) return MUON_EINVAL;
  if (!valid_dtype(w_dtype) || !valid_dtype(u_dtype)) return MUON_EDTYPE;
  if (numel == 0) return MUON_OK;
  if (!W || !U) return MUON_EINVAL;
  if (!aligned16(W) || !aligned16(U)) return MUON_EALIGN;
  const int64_t blocks = ((numel + 7) / 8 + kThreads - 1) / kThreads;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (w_dtype == MUON_BF16 && u_dtype == MUON_BF16)
    launch_kernel(update_dense_kernel<bf16_t, bf16_t>, dim3(blocks), dim3(kThreads), 0, st, 
        static_cast<bf16_t*>(W), numel, static_cast<const bf16_t*>(U), eta);
  else if (w_dtype == MUON_BF16)
    launch_kernel(update_dense_kernel<bf16_t, float>, dim3(blocks), dim3(kThreads), 0, st, 
        static_cast<bf16_t*>(W), numel, static_cast<const float*>(U), eta);
  else if (u_dtype == MUON_BF16)
    launch_kernel(update_dense_kernel<float, bf16_t>, dim3(blocks), dim3(kThreads), 0, st, 
        static_cast<float*>(W), numel, static_cast<const bf16_t*>(U), eta);
  else
    launch_kernel(update_dense_kernel<float, float>, dim3(blocks), dim3(kThreads), 0, st, 
        static_cast<float*>(W), numel, static_cast<const float*>(U), eta);
  return launch_status();
}

}  // extern "C"
