// Achievable-peak probes: what this part sustains on the two resources the
// attention kernels are bound by, measured with the simplest kernels that can
// reach them, so that a kernel's rate can be read against both the published
// peak and what the chip delivers under its own clocks and power limit.
//  * MFMA: chains of independent v_mfma_f32_32x32x16_bf16 (the instruction of
//    the anchor and the projections) on register operands, no memory traffic;
//  * HBM: a read of 16-byte words (XOR-folded) and a copy, four 16-byte accesses
//    in flight per thread, the copy with ordinary or non-temporal accesses (the
//    apply streams with non-temporal ones).  A block covers 4 x 256 consecutive
//    words per pass (a thread's four words one block-width apart) and the grid
//    strides over the buffer, so every block streams contiguous memory.
// Each kernel stores to its one-float sink only under a condition that the
// data practically never meets, which keeps the compiler from dropping the work.
#include <algorithm>

#include "ha_device.h"
#include "ha_launch.h"

namespace ha {

namespace {

constexpr int kProbeChains = 4;  // independent accumulators per wave
constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 4;          // 16-byte words in flight per thread
constexpr int64_t kStreamBlocks = 4096;   // 16 blocks per CU

__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  // small multiples of 1/16 (exact in bf16): sums stay far below fp32 overflow
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(static_cast<float>((lane + i) & 7) * 0.0625f);
    b[i] = static_cast<__bf16>(static_cast<float>((3 * lane + i) & 7) * 0.0625f);
  }
  f32x16 acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  if (s == -1.0f) sink[0] = s;  // the sums are non-negative
}

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// word u of the pass starting at i0 is i0 + u * kStreamThreads
__global__ __launch_bounds__(kStreamThreads) void probe_read_kernel(const u32x4* __restrict__ src, int64_t n,
                                                                    float* sink) {
  constexpr int64_t span = static_cast<int64_t>(kStreamThreads) * kStreamUnroll;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * span;
  uint32_t x = 0;
  for (int64_t i0 = static_cast<int64_t>(blockIdx.x) * span + threadIdx.x; i0 < n; i0 += stride) {
    if (i0 + (kStreamUnroll - 1) * kStreamThreads < n) {
      u32x4 v[kStreamUnroll];
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) v[u] = src[i0 + u * kStreamThreads];
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) x ^= fold(v[u]);
    } else {
      for (int u = 0; u < kStreamUnroll; ++u)
        if (i0 + u * kStreamThreads < n) x ^= fold(src[i0 + u * kStreamThreads]);
    }
  }
  if (x == 0x9e3779b9u) sink[0] = static_cast<float>(x);
}

template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  return *p;
}

template <bool NT>
__device__ __forceinline__ void st(u32x4* p, u32x4 v) {
  if constexpr (NT) {
    __builtin_nontemporal_store(v, p);
  } else {
    *p = v;
  }
}

template <bool NT>
__global__ __launch_bounds__(kStreamThreads) void probe_copy_kernel(const u32x4* __restrict__ src,
                                                                    u32x4* __restrict__ dst, int64_t n) {
  constexpr int64_t span = static_cast<int64_t>(kStreamThreads) * kStreamUnroll;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * span;
  for (int64_t i0 = static_cast<int64_t>(blockIdx.x) * span + threadIdx.x; i0 < n; i0 += stride) {
    if (i0 + (kStreamUnroll - 1) * kStreamThreads < n) {
      u32x4 v[kStreamUnroll];
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) v[u] = ld<NT>(src + i0 + u * kStreamThreads);
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) st<NT>(dst + i0 + u * kStreamThreads, v[u]);
    } else {
      for (int u = 0; u < kStreamUnroll; ++u)
        if (i0 + u * kStreamThreads < n) st<NT>(dst + i0 + u * kStreamThreads, ld<NT>(src + i0 + u * kStreamThreads));
    }
  }
}

unsigned stream_grid(int64_t n) {
  constexpr int64_t span = static_cast<int64_t>(kStreamThreads) * kStreamUnroll;
  return static_cast<unsigned>(std::min(kStreamBlocks, std::max<int64_t>(1, (n + span - 1) / span)));
}

}  // namespace

double probe_mfma_flops(int blocks, int iters) {
  // 4 waves per block, kProbeChains MFMAs per iteration, 2 * 32 * 32 * 16 flop each
  return static_cast<double>(blocks) * 4.0 * kProbeChains * static_cast<double>(iters) * 2.0 * 32 * 32 * 16;
}

hipError_t launch_probe_mfma(int blocks, int iters, float* sink, hipStream_t s) {
  probe_mfma_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(iters, sink);
  return hipGetLastError();
}

hipError_t launch_probe_read(const void* src, size_t bytes, float* sink, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(bytes / 16);
  if (n == 0) return hipSuccess;
  probe_read_kernel<<<dim3(stream_grid(n)), dim3(kStreamThreads), 0, s>>>(static_cast<const u32x4*>(src), n, sink);
  return hipGetLastError();
}

hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, bool nontemporal, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(bytes / 16);
  if (n == 0) return hipSuccess;
  const dim3 grid(stream_grid(n)), block(kStreamThreads);
  if (nontemporal)
    probe_copy_kernel<true><<<grid, block, 0, s>>>(static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n);
  else
    probe_copy_kernel<false><<<grid, block, 0, s>>>(static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n);
  return hipGetLastError();
}

}  // namespace ha
