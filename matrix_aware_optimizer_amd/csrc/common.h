// Shared device helpers for libmuon (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "muon.h"

namespace muon {

typedef unsigned short bf16_t;  // bfloat16 bit pattern in memory

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Host-side one-time set-up is tracked per device (ordinals 0..63) with
// atomics, so host threads may call concurrently and each device gets its own
// kernel attributes.  A device past 63 simply repeats the set-up every call.
constexpr int kMaxTrackedDevices = 64;

inline int current_device() {
  int dev = -1;
  return hipGetDevice(&dev) == hipSuccess ? dev : -1;
}

// Bit of `dev` in a per-device set, or 0 when the ordinal is not tracked.
inline uint64_t device_bit(int dev) {
  return dev >= 0 && dev < kMaxTrackedDevices ? uint64_t(1) << dev : 0;
}

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float -> bfloat16, round to nearest, ties to even; NaN stays a quiet NaN.
// Round to nearest even; a NaN keeps its sign and top payload bits and is
// made quiet.  Written as a select, not a branch: in a wave's epilogue a
// branch per conversion costs an exec-mask save and restore each time.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t quiet = (u >> 16) | 0x40u;
  return static_cast<bf16_t>((u & 0x7fffffffu) > 0x7f800000u ? quiet : rounded);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static float to_f32(float v) { return v; }
  __device__ __forceinline__ static float from_f32(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  __device__ __forceinline__ static float to_f32(bf16_t v) { return bf16_to_f32(v); }
  __device__ __forceinline__ static bf16_t from_f32(float v) { return f32_to_bf16(v); }
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return bf16_to_f32(v); }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

// ---------------------------------------------------------------------------
// 8-element vector access (16 B for bf16, 2 x 16 B for fp32).
// ---------------------------------------------------------------------------
template <typename T> struct Vec8;
template <> struct Vec8<bf16_t> {
  __device__ __forceinline__ static void load(const bf16_t* p, float v[8]) {
    uint4 r = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static void store(bf16_t* p, const float v[8]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f32_to_bf16(v[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16(v[2 * i + 1])) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};
template <> struct Vec8<float> {
  __device__ __forceinline__ static void load(const float* p, float v[8]) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ static void store(float* p, const float v[8]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
};

// Wave-wide sum of a double with a fixed butterfly order (deterministic).
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// An element count the elementwise calls accept (0 .. MUON_MAX_NUMEL).
inline bool numel_ok(int64_t n) { return n >= 0 && n <= MUON_MAX_NUMEL; }
inline bool valid_dtype(int d) { return d == MUON_F32 || d == MUON_BF16; }
inline size_t dtype_size(int d) { return d == MUON_F32 ? 4 : 2; }
inline size_t round_up(size_t x, size_t m) { return (x + m - 1) / m * m; }

// Timing events for the next kernel this host thread launches through the
// library (set by muon_time_next_launch): that launch records them at the
// kernel's start and end (hipExtLaunchKernelGGL), then they are forgotten.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
inline LaunchEvents& pending_launch_events() {
  static thread_local LaunchEvents ev;
  return ev;
}

// Every kernel of the library is launched here.
template <typename... KArgs, typename... Args>
inline void launch_kernel(void (*kern)(KArgs...), dim3 grid, dim3 block, uint32_t lds, hipStream_t st,
                          Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  LaunchEvents& pending = pending_launch_events();
  if (pending.start != nullptr || pending.stop != nullptr) {
    const LaunchEvents ev = pending;
    pending = LaunchEvents{};
    hipExtLaunchKernelGGL(kern, grid, block, lds, st, ev.start, ev.stop, 0, static_cast<KArgs>(args)...);
  } else {
    kern<<<grid, block, lds, st>>>(static_cast<KArgs>(args)...);
  }
}

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MUON_OK : MUON_ELAUNCH;
}

// The library's own streams on the current device (default priority, not
// synchronising with the null stream; stream i for i < kLibStreams), created
// on first use; null if one cannot be created.  Host threads share them; each
// call orders its own work with its own events.
constexpr int kLibStreams = 3;
inline hipStream_t lane_stream(int i = 0) {
  static std::mutex mu;
  static hipStream_t streams[kMaxTrackedDevices][kLibStreams] = {};
  const int dev = current_device();
  if (dev < 0 || dev >= kMaxTrackedDevices || i < 0 || i >= kLibStreams) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (streams[dev][i] == nullptr) {
    hipStream_t st = nullptr;
    if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return nullptr;
    streams[dev][i] = st;
  }
  return streams[dev][i];
}

// n events of this host thread on the current device (n <= kLibStreams + 1:
// a fork and one join per library stream), created on first use and kept (a
// wait takes the event's last record at the time it is enqueued, so reusing
// them call after call is safe).
inline bool lane_events(hipEvent_t* ev, int n) {
  static thread_local hipEvent_t events[kMaxTrackedDevices][kLibStreams + 1] = {};
  const int dev = current_device();
  if (dev < 0 || dev >= kMaxTrackedDevices || n < 0 || n > kLibStreams + 1) return false;
  for (int i = 0; i < n; ++i) {
    hipEvent_t& e = events[dev][i];
    if (e == nullptr && hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) {
      e = nullptr;
      return false;
    }
    ev[i] = e;
  }
  return true;
}

// The fork and join events of one second stream.
inline bool fork_join_events(hipEvent_t& fork, hipEvent_t& join) {
  hipEvent_t ev[2];
  if (!lane_events(ev, 2)) return false;
  fork = ev[0];
  join = ev[1];
  return true;
}

}  // namespace muon
