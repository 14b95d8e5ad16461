// Block attention residuals (AttnRes; SANA-Video 2.0 summary page, section 03;
// review page, sections 1 and 3; news item): summaries of completed blocks are
// routed into later linear layers.  Per token, the input of such a layer is a
// softmax mixture over candidates v_0 .. v_{M} (the completed summaries, then
// the current stream):
//   score_m = w . v_m / rms(v_m) / sqrt(C),  rms(v) = sqrt(mean(v^2) + eps),
//   h = sum_m softmax_m(score) v_m.
// HBM-bound, one wave per token.  bf16 rows of up to 6,144 features take a
// single pass: a lane keeps its 16-byte chunks of a candidate row in registers
// (the next candidate's already loading), scores the row (w . v and v . v,
// reduced over the wave) and folds it into an online softmax -- running
// maximum, denominator and accumulator, rescaled when the maximum rises -- so
// every candidate row is read once.  Other rows (float32, wider bf16) take two
// passes: the scores first, then the weighted sum, re-reading the rows (from L2:
// they were just read).
#include <type_traits>

#include "ha_device.h"
#include "ha_launch.h"

namespace ha {

namespace {

constexpr int kMaxCand = 64;

template <typename T>
__device__ __forceinline__ void ld8(const T* p, float (&v)[8]) {
  if constexpr (std::is_same<T, float>::value) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    v[0] = bf_lo(u.x); v[1] = bf_hi(u.x); v[2] = bf_lo(u.y); v[3] = bf_hi(u.y);
    v[4] = bf_lo(u.z); v[5] = bf_hi(u.z); v[6] = bf_lo(u.w); v[7] = bf_hi(u.w);
  }
}

template <typename T>
__device__ __forceinline__ void st8(T* p, const float (&v)[8]) {
  if constexpr (std::is_same<T, float>::value) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]),
                                              pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7]));
  }
}

// candidate m of token t: summaries[m] for m < M, x for m == M
template <typename T>
__global__ __launch_bounds__(256) void attnres_mix_kernel(const T* __restrict__ summaries, int M,
                                                          const T* __restrict__ x, const float* __restrict__ w,
                                                          T* __restrict__ h, int64_t tokens, int C, float eps) {
  __shared__ float sScore[4][kMaxCand];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t tok = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (tok >= tokens) return;   // a whole wave: no barrier below
  const int nch = C / 8;
  auto row = [&](int m) -> const T* {
    return (m < M ? summaries + static_cast<int64_t>(m) * tokens * C : x) + tok * C;
  };
  const float inv_c = 1.0f / static_cast<float>(C);
  const float inv_sqrt_c = rsqrtf(static_cast<float>(C));
  float mx = -INFINITY;
  for (int m = 0; m <= M; ++m) {
    const T* v = row(m);
    float dot = 0.f, ss = 0.f;
    for (int ch = lane; ch < nch; ch += 64) {
      float a[8];
      ld8(v + 8 * ch, a);
      const float4 w0 = *reinterpret_cast<const float4*>(w + 8 * ch);
      const float4 w1 = *reinterpret_cast<const float4*>(w + 8 * ch + 4);
      dot = fmaf(a[0], w0.x, dot); dot = fmaf(a[1], w0.y, dot);
      dot = fmaf(a[2], w0.z, dot); dot = fmaf(a[3], w0.w, dot);
      dot = fmaf(a[4], w1.x, dot); dot = fmaf(a[5], w1.y, dot);
      dot = fmaf(a[6], w1.z, dot); dot = fmaf(a[7], w1.w, dot);
#pragma unroll
      for (int k = 0; k < 8; ++k) ss = fmaf(a[k], a[k], ss);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      dot += __shfl_xor(dot, o);
      ss += __shfl_xor(ss, o);
    }
    const float sc = dot * rsqrtf(ss * inv_c + eps) * inv_sqrt_c;
    mx = fmaxf(mx, sc);
    if (lane == 0) sScore[wave][m] = sc;
  }
  __builtin_amdgcn_wave_barrier();
  float den = 0.f;
  for (int m = 0; m <= M; ++m) den += __expf(sScore[wave][m] - mx);
  const float inv = 1.0f / den;
  for (int ch = lane; ch < nch; ch += 64) {
    float acc[8] = {};
    for (int m = 0; m <= M; ++m) {
      const float a_m = __expf(sScore[wave][m] - mx) * inv;
      float v[8];
      ld8(row(m) + 8 * ch, v);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = fmaf(a_m, v[k], acc[k]);
    }
    st8(h + tok * C + 8 * ch, acc);
  }
}

// bf16 single pass for C <= 512 CPL (see the header of this file): a lane owns
// chunks lane + 64 i (i < CPL) of every row; rows end mid-lane-range when C is
// not a multiple of 512 (those chunks load zeros and are not stored).
template <int CPL>
__global__ __launch_bounds__(256) void attnres_mix_bf16_1pass(const bf16_t* __restrict__ summaries, int M,
                                                              const bf16_t* __restrict__ x,
                                                              const float* __restrict__ w, bf16_t* __restrict__ h,
                                                              int64_t tokens, int C, float eps) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t tok = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (tok >= tokens) return;   // a whole wave
  const int nch = C / 8;
  auto row = [&](int m) -> const bf16_t* {
    return (m < M ? summaries + static_cast<int64_t>(m) * tokens * C : x) + tok * C;
  };
  auto load = [&](u32x4 (&r)[CPL], int m) {
    const bf16_t* v = row(m);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int ch = lane + 64 * i;
      r[i] = ch < nch ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v + 8 * ch)) : u32x4{0, 0, 0, 0};
    }
  };
  auto unpack = [](const u32x4& u, float (&a)[8]) {
    a[0] = bf_lo(u.x); a[1] = bf_hi(u.x); a[2] = bf_lo(u.y); a[3] = bf_hi(u.y);
    a[4] = bf_lo(u.z); a[5] = bf_hi(u.z); a[6] = bf_lo(u.w); a[7] = bf_hi(u.w);
  };
  const float inv_c = 1.0f / static_cast<float>(C);
  const float inv_sqrt_c = rsqrtf(static_cast<float>(C));
  float acc[CPL][8];
#pragma unroll
  for (int i = 0; i < CPL; ++i)
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[i][k] = 0.f;
  float mx = -INFINITY, den = 0.f;
  u32x4 cur[CPL], nxt[CPL];
  load(nxt, 0);
  for (int m = 0; m <= M; ++m) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) cur[i] = nxt[i];
    if (m < M) load(nxt, m + 1);
    float dot = 0.f, ss = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int ch = lane + 64 * i;
      if (ch < nch) {
        float a[8];
        unpack(cur[i], a);
        const float4 w0 = *reinterpret_cast<const float4*>(w + 8 * ch);
        const float4 w1 = *reinterpret_cast<const float4*>(w + 8 * ch + 4);
        dot = fmaf(a[0], w0.x, dot); dot = fmaf(a[1], w0.y, dot);
        dot = fmaf(a[2], w0.z, dot); dot = fmaf(a[3], w0.w, dot);
        dot = fmaf(a[4], w1.x, dot); dot = fmaf(a[5], w1.y, dot);
        dot = fmaf(a[6], w1.z, dot); dot = fmaf(a[7], w1.w, dot);
#pragma unroll
        for (int k = 0; k < 8; ++k) ss = fmaf(a[k], a[k], ss);
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      dot += __shfl_xor(dot, o);
      ss += __shfl_xor(ss, o);
    }
    const float sc = dot * rsqrtf(ss * inv_c + eps) * inv_sqrt_c;
    const float m_new = fmaxf(mx, sc);
    const float scale = __expf(mx - m_new);   // 0 for the first candidate (mx = -inf)
    const float p = __expf(sc - m_new);
    den = fmaf(den, scale, p);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      // unpack again rather than keep the scoring loop's 8 floats per chunk
      // alive across the reduction (two VALU operations per pair, and about
      // 8 CPL fewer registers)
      asm volatile("" : "+v"(cur[i]));
      float a[8];
      unpack(cur[i], a);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[i][k] = fmaf(acc[i][k], scale, p * a[k]);
    }
    mx = m_new;
  }
  const float inv = 1.0f / den;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int ch = lane + 64 * i;
    if (ch < nch) {
      float o[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = acc[i][k] * inv;
      st8(h + tok * C + 8 * ch, o);
    }
  }
}

template <int CPL>
void launch_1pass(const void* summaries, int M, const void* x, const float* w, void* h, int64_t tokens, int C,
                  float eps, hipStream_t s) {
  attnres_mix_bf16_1pass<CPL><<<dim3(static_cast<unsigned>((tokens + 3) / 4)), dim3(256), 0, s>>>(
      static_cast<const bf16_t*>(summaries), M, static_cast<const bf16_t*>(x), w, static_cast<bf16_t*>(h), tokens,
      C, eps);
}

}  // namespace

int attnres_max_candidates() { return kMaxCand; }

hipError_t launch_attnres_mix(bool bf16, const void* summaries, int M, const void* x, const float* w, void* h,
                              int64_t tokens, int C, float eps, hipStream_t s) {
  if (tokens == 0) return hipSuccess;
  if (bf16) {
    // 16-byte chunks per lane of the single pass: the smallest instantiated
    // count that covers the row
    const int per_lane = (C / 8 + 63) / 64;
    switch (per_lane) {
      case 1: launch_1pass<1>(summaries, M, x, w, h, tokens, C, eps, s); return hipGetLastError();
      case 2: launch_1pass<2>(summaries, M, x, w, h, tokens, C, eps, s); return hipGetLastError();
      case 3: launch_1pass<3>(summaries, M, x, w, h, tokens, C, eps, s); return hipGetLastError();
      case 4: launch_1pass<4>(summaries, M, x, w, h, tokens, C, eps, s); return hipGetLastError();
      case 5: case 6: launch_1pass<6>(summaries, M, x, w, h, tokens, C, eps, s); return hipGetLastError();
      case 7: case 8: launch_1pass<8>(summaries, M, x, w, h, tokens, C, eps, s); return hipGetLastError();
      case 9: case 10: launch_1pass<10>(summaries, M, x, w, h, tokens, C, eps, s); return hipGetLastError();
      case 11: case 12: launch_1pass<12>(summaries, M, x, w, h, tokens, C, eps, s); return hipGetLastError();
      default: break;   // wider rows: the two-pass kernel below
    }
  }
  const dim3 grid(static_cast<unsigned>((tokens + 3) / 4)), block(256);
  if (bf16)
    attnres_mix_kernel<bf16_t><<<grid, block, 0, s>>>(static_cast<const bf16_t*>(summaries), M,
                                                      static_cast<const bf16_t*>(x), w, static_cast<bf16_t*>(h),
                                                      tokens, C, eps);
  else
    attnres_mix_kernel<float><<<grid, block, 0, s>>>(static_cast<const float*>(summaries), M,
                                                     static_cast<const float*>(x), w, static_cast<float*>(h),
                                                     tokens, C, eps);
  return hipGetLastError();
}

}  // namespace ha
