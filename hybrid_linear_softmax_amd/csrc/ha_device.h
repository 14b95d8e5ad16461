// Device helpers shared by the gfx950 kernels: bf16 packing, the ReLU feature
// map on packed bf16, the sigmoid gate and MFMA operand types.
#pragma once
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace ha {

typedef uint16_t bf16_t;  // bfloat16 storage
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Streaming 16-byte accesses for data a kernel touches exactly once (the apply
// kernel's Q, G and O): non-temporal loads and stores.  On this part a
// read-two-write-one stream runs ~10 % faster this way; a read-only stream
// (the KV-state reduction) runs slower, so it keeps plain loads.
__device__ __forceinline__ uint4 load_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store_stream(void* p, uint4 v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}

// phi = ReLU on two bf16 packed in a dword: a bf16 is negative exactly when its
// bit pattern is negative as an int16, so a packed signed max with 0 zeroes the
// negative halves (and -0) and keeps the rest.
__device__ __forceinline__ uint32_t relu2(uint32_t w) {
  s16x2 v = __builtin_bit_cast(s16x2, w);
  const s16x2 zero = {0, 0};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(v, zero));
}

__device__ __forceinline__ uint4 relu8(uint4 w) {
  return make_uint4(relu2(w.x), relu2(w.y), relu2(w.z), relu2(w.w));
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats to two bf16 (round to nearest even), packed lo | hi << 16.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 r;
  r.x = (__bf16)lo;
  r.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Logistic gate 1 / (1 + exp(-x)); 0 at -inf, 1 at +inf.
__device__ __forceinline__ float gate_fast(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}
__device__ __forceinline__ float gate_exact(float x) { return 1.0f / (1.0f + expf(-x)); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// 4 tokens x 8 features (4 rows of 8 packed bf16) -> 8 features x 4 tokens:
// out[f] = { token0[f] | token1[f] << 16, token2[f] | token3[f] << 16 }.
__device__ __forceinline__ void transpose4x8(const uint4 (&in)[4], uint2 (&out)[8]) {
  const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&in[0]);
  const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&in[1]);
  const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&in[2]);
  const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&in[3]);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    out[2 * p] = make_uint2((r0[p] & 0xffffu) | (r1[p] << 16), (r2[p] & 0xffffu) | (r3[p] << 16));
    out[2 * p + 1] = make_uint2((r0[p] >> 16) | (r1[p] & 0xffff0000u), (r2[p] >> 16) | (r3[p] & 0xffff0000u));
  }
}

// Block index remap so that consecutive logical tiles run on the same XCD
// (blocks are dispatched round-robin over the 8 XCDs); tiles of one (b, h) then
// share that XCD's L2 while they stream the same keys.
__device__ __forceinline__ int64_t xcd_remap(int64_t i, int64_t total) {
  const int64_t per = total / 8;
  if (i >= per * 8) return i;
  return (i % 8) * per + i / 8;
}

}  // namespace ha
