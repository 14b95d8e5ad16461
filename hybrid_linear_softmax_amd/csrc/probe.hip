// Achievable-peak probes: what this part sustains on the two resources the
// attention kernels are bound by, measured with the simplest kernels that can
// reach them, so that a kernel's rate can be read against both the published
// peak and what the chip delivers under its own clocks and power limit.
//  * MFMA: chains of independent v_mfma_f32_32x32x16_bf16 (the instruction of
//    the anchor and the projections) on register operands, no memory traffic,
//    on constant operands and on operands that change with every instruction;
//  * HBM: a read of 16-byte words (XOR-folded) and a copy, four 16-byte accesses
//    in flight per thread, the copy with ordinary or non-temporal accesses (the
//    apply streams with non-temporal ones).  A block covers 4 x 256 consecutive
//    words per pass (a thread's four words one block-width apart) and the grid
//    strides over the buffer, so every block streams contiguous memory.
//  * issue overlap: whether one SIMD runs the anchor's softmax VALU work (fused
//    multiply-add, exp2, bf16 pack, dot2 row sum) while MFMAs execute, within a
//    wave and between waves.  One block per CU (its LDS reservation keeps a
//    second one off), 1 or 2 waves per SIMD; the caller times the MFMA-only,
//    VALU-only and mixed runs and compares.
// Each kernel stores to its one-float sink only under a condition that the
// data practically never meets, which keeps the compiler from dropping the work.
#include <algorithm>

#include "ha_device.h"
#include "ha_launch.h"
#include "../../include/ha_probe.h"

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

// The same chains on operands that change with every instruction: each lane
// holds 8 operand pairs of pseudo-random bf16 (random sign and mantissa,
// magnitudes 0.5 to 4, the range of the attention inputs' larger values) and
// cycles through them, so the multipliers' inputs toggle as they do on real
// data.  A matrix core's power depends on that toggling: on constant operands
// the part holds its top clock under the power limit, on data like this it
// may not.
__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

__global__ __launch_bounds__(256) void probe_mfma_data_kernel(int iters, float* sink) {
  constexpr int kSets = 8;
  const uint32_t seed = (blockIdx.x * 256u + threadIdx.x) * 0x9e3779b9u;
  bf16x8 a[kSets], b[kSets];
#pragma unroll
  for (int k = 0; k < kSets; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t ha = probe_hash(seed + 16u * k + i);
      const uint32_t hb = probe_hash(seed + 16u * k + 8 + i);
      // sign bit, exponent 126..128 (0.5 <= |x| < 4), 7 mantissa bits
      a[k][i] = __builtin_bit_cast(__bf16, static_cast<uint16_t>((ha & 0x807fu) | ((126u + (ha >> 16) % 3u) << 7)));
      b[k][i] = __builtin_bit_cast(__bf16, static_cast<uint16_t>((hb & 0x807fu) | ((126u + (hb >> 16) % 3u) << 7)));
    }
  f32x16 acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  static_assert(kSets == 2 * kProbeChains, "two rounds of the chains per pass over the sets");
  for (int it = 0; it + 2 <= iters; it += 2) {
#pragma unroll
    for (int k = 0; k < kSets; ++k)
      acc[k % kProbeChains] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], b[k], acc[k % kProbeChains], 0, 0, 0);
  }
  if (iters & 1) {
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], b[c], acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  if (s != s) sink[0] = s;  // finite operands: the sum is never NaN
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

// Overlap probe.  Per round: the MFMA part is kProbeChains independent 32x32x16
// bf16 MFMAs on VGPR accumulators (as the anchor's), the VALU part the anchor's
// instructions for 8 probabilities (8 fused multiply-adds and 8 exp2, 4 bf16
// pair packs, 4 dot2 row-sum steps) plus one add that moves the maximum they
// are taken against, so that no round is loop-invariant; BOTH interleaves one
// MFMA with a quarter of the VALU part (the anchor's logit phase: per MFMA two
// fused multiply-adds, two exp2, a pack and a dot2).
constexpr int kOverlapLds = 96 * 1024;  // more than half a CU's LDS: one block per CU

template <int MODE>
__global__ __launch_bounds__(512) void probe_overlap_kernel(int iters, float* sink) {
  extern __shared__ int reserve[];
  const int lane = threadIdx.x & 63;
  bool do_mfma = MODE == HA_PROBE_OVERLAP_MFMA || MODE == HA_PROBE_OVERLAP_BOTH;
  bool do_valu = MODE == HA_PROBE_OVERLAP_VALU || MODE == HA_PROBE_OVERLAP_BOTH;
  if constexpr (MODE == HA_PROBE_OVERLAP_SPLIT) {
    // roles by placement, not by wave index: the first wave of each SIMD (SIMD
    // id from the HW_ID register, bits 5:4) takes the VALU part, the rest MFMA
    if (threadIdx.x < 4) reserve[threadIdx.x] = 0;
    __syncthreads();
    const int simd = static_cast<int>((__builtin_amdgcn_s_getreg(4 | (0 << 6) | (31 << 11)) >> 4) & 3);
    int slot = 0;
    if (lane == 0) slot = atomicAdd(&reserve[simd], 1);
    slot = __shfl(slot, 0);
    do_valu = slot == 0;
    do_mfma = !do_valu;
  }
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
  // logit-like inputs, a scale and a running maximum (scaled) as in the
  // anchor: the maximum grows by 2^-20 a round, so the probabilities stay in
  // (0, 1] and every sum finite up to the largest iters
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = 0.01f * static_cast<float>(lane + e);
  const float c = 0.12752977f;
  float mc = 0.75f;
  float rowsum = 0.f;
  const bf16x2 one = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  auto valu_quarter = [&](int k) {
    if (k == 0) {
      mc += 0x1p-20f;
      asm volatile("" : "+v"(mc));
    }
    const float p0 = __builtin_amdgcn_exp2f(fmaf(x[2 * k], c, -mc));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(x[2 * k + 1], c, -mc));
    const uint32_t pk = pack_bf16(p0, p1);
    rowsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), one, rowsum, false);
    asm volatile("" : "+v"(rowsum));
  };
  if constexpr (MODE == HA_PROBE_OVERLAP_SPLIT) {
    if (do_mfma) {
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int k = 0; k < kProbeChains; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
    } else {
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int k = 0; k < 4; ++k) valu_quarter(k);
    }
  } else {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (do_mfma) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
        if (do_valu) valu_quarter(k);
      }
    }
  }
  float r = rowsum;
#pragma unroll
  for (int e = 0; e < 8; ++e) r += x[e];
#pragma unroll
  for (int k = 0; k < kProbeChains; ++k)
#pragma unroll
    for (int q = 0; q < 16; ++q) r += acc[k][q];
  if (r == -1.0f) sink[0] = r;  // every term is non-negative
}

template <int MODE>
hipError_t launch_overlap_mode(int blocks, int threads, int iters, float* sink, hipStream_t s) {
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(probe_overlap_kernel<MODE>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kOverlapLds);
  if (e != hipSuccess) return e;
  probe_overlap_kernel<MODE><<<dim3(static_cast<unsigned>(blocks)), dim3(threads), kOverlapLds, s>>>(iters, sink);
  return hipGetLastError();
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

hipError_t launch_probe_mfma_data(int blocks, int iters, float* sink, hipStream_t s) {
  probe_mfma_data_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(iters, sink);
  return hipGetLastError();
}

hipError_t launch_probe_overlap(int mode, int waves_per_simd, int blocks, int iters, float* sink, hipStream_t s) {
  const int threads = 256 * waves_per_simd;
  switch (mode) {
    case HA_PROBE_OVERLAP_MFMA: return launch_overlap_mode<HA_PROBE_OVERLAP_MFMA>(blocks, threads, iters, sink, s);
    case HA_PROBE_OVERLAP_VALU: return launch_overlap_mode<HA_PROBE_OVERLAP_VALU>(blocks, threads, iters, sink, s);
    case HA_PROBE_OVERLAP_BOTH: return launch_overlap_mode<HA_PROBE_OVERLAP_BOTH>(blocks, threads, iters, sink, s);
    case HA_PROBE_OVERLAP_SPLIT: return launch_overlap_mode<HA_PROBE_OVERLAP_SPLIT>(blocks, threads, iters, sink, s);
    default: return hipErrorInvalidValue;
  }
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
