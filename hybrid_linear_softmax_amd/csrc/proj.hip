// Projections of the attention block around the hybrid group (SANA-Video 2.0
// review page, section 3: the hybrid attention inside the DiT blocks of the
// compiled forward; summary page, section 03):
//   proj_in:  [Q | K | V | G] = x W_in^T, x: [B, N, C], W_in: [4C, C], each
//             C-wide block split into H heads of d features -> [B, H, N, d];
//   proj_out: x_out = x + concat_h(O) W_out^T, O: [B, H, N, d], W_out: [C, C].
// Both are dense contractions over C, run on the bf16 MFMA with float32
// accumulation.
//
// bf16 kernel: one block = 256 output features x 256 tokens, 8 waves (2 along
// features x 4 along tokens, 128 x 64 each), K in steps of 64.
//  * the product is taken transposed, out^T = W x^T: the MFMA A operand is a
//    weight row, the B operand a token row, both contiguous along C, so both
//    LDS tiles are read the same way, and a lane's accumulator holds four
//    consecutive output features of one token -- an 8-byte store in either
//    epilogue (the head scatter of proj_in, the residual add of proj_out);
//  * proj_out reads its token rows straight out of O's [B, H, N, d] layout: a
//    64-wide K step lies inside one head, so a row is 128 contiguous bytes;
//  * tiles past M tokens or the last feature clamp their load rows to the last
//    valid row (valid memory, results never stored), so no load is predicated;
//  * global loads of the next K step are in flight during the MFMAs of the
//    current one; LDS is double buffered with one barrier per step;
//  * tiles are ordered in groups of 4 token tiles x all feature tiles and the
//    order is split into 8 contiguous ranges, one per XCD, so the blocks that
//    run together on one XCD share token rows and weight rows in its L2.
#include "ha_device.h"
#include "ha_launch.h"

namespace ha {

namespace {

constexpr int kTF = 256;   // output features per block
constexpr int kTM = 256;   // tokens per block
constexpr int kTK = 64;    // K per step
constexpr int kGroupM = 4; // token tiles per ordering group
constexpr int kLP = kTK + 8;  // LDS pitch (elements) of a 64-wide row

struct ProjShape {
  int64_t M;      // tokens B * N
  int64_t Nf;     // output features (4C or C)
  int64_t K;      // C
  int64_t N;      // tokens per batch item
  int64_t H;
  int d;
  int64_t nt_f, nt_m, total;
};

__device__ __forceinline__ void tile_of(int64_t t, const ProjShape& p, int64_t& tf, int64_t& tm) {
  const int64_t g = t / (kGroupM * p.nt_f);
  const int64_t gm = min((int64_t)kGroupM, p.nt_m - g * kGroupM);
  const int64_t idx = t - g * kGroupM * p.nt_f;
  tf = idx / gm;
  tm = g * kGroupM + idx % gm;
}

// MODE 0: proj_in, X = x [M, K], outputs scattered into out[0..3] = Q, K, V, G.
// MODE 1: proj_out, X = O [B, H, N, d] read as [M, K], out[0] = resid + X W^T;
// out0 may be resid itself (each element is read, then written, by one lane).
template <int MODE>
__global__ __launch_bounds__(512, 1) void proj_bf16(const bf16_t* __restrict__ X,
                                                    const bf16_t* __restrict__ W,
                                                    bf16_t* out0, bf16_t* __restrict__ out1,
                                                    bf16_t* __restrict__ out2, bf16_t* __restrict__ out3,
                                                    const bf16_t* resid, ProjShape p) {
  __shared__ __attribute__((aligned(16))) bf16_t sW[2][kTF * kLP];
  __shared__ __attribute__((aligned(16))) bf16_t sX[2][kTM * kLP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int wf = wave >> 2;  // 128-feature half
  const int wt = wave & 3;   // 64-token quarter
  int64_t tf, tm;
  tile_of(xcd_remap(blockIdx.x, p.total), p, tf, tm);
  const int64_t f0 = tf * kTF, m0 = tm * kTM;

  // rows this thread loads: r = (tid + 512 i) / 8, 16-byte chunk kc = tid % 8
  const int kc = tid & 7;
  int64_t xrow[4], wrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 64 * i;
    const int64_t m = min(m0 + r, p.M - 1);
    if (MODE == 0) {
      xrow[i] = m * p.K;
    } else {
      const int64_t b = m / p.N, n = m - b * p.N;
      xrow[i] = (b * p.H * p.N + n) * p.d;
    }
    wrow[i] = min(f0 + r, p.Nf - 1) * p.K;
  }
  auto xcol = [&](int64_t k0) -> int64_t {
    if (MODE == 0) return k0 + 8 * kc;
    return (k0 / p.d) * p.N * p.d + (k0 % p.d) + 8 * kc;
  };
  u32x4 xr[4], wr[4];
  auto load = [&](int64_t k0) {
    const int64_t xc = xcol(k0), wc = k0 + 8 * kc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xr[i] = *reinterpret_cast<const u32x4*>(X + xrow[i] + xc);
      wr[i] = *reinterpret_cast<const u32x4*>(W + wrow[i] + wc);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 64 * i;
      *reinterpret_cast<u32x4*>(&sX[buf][r * kLP + 8 * kc]) = xr[i];
      *reinterpret_cast<u32x4*>(&sW[buf][r * kLP + 8 * kc]) = wr[i];
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int fi = 0; fi < 4; ++fi)
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[fi][ti][r] = 0.f;

  const int64_t nk = p.K / kTK;
  load(0);
  store(0);
  __syncthreads();
  for (int64_t ks = 0; ks < nk; ++ks) {
    const int buf = static_cast<int>(ks & 1);
    // unconditional (the last step re-reads its own slice into the idle
    // buffer): a conditional load keeps the prefetch registers in scratch
    load(min(ks + 1, nk - 1) * kTK);
    __builtin_amdgcn_sched_barrier(0);  // issue the loads before the MFMAs
#pragma unroll
    for (int kk = 0; kk < kTK / 16; ++kk) {
      bf16x8 a[4], bx[2];
#pragma unroll
      for (int fi = 0; fi < 4; ++fi)
        a[fi] = *reinterpret_cast<const bf16x8*>(&sW[buf][(128 * wf + 32 * fi + l32) * kLP + 16 * kk + 8 * h]);
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
        bx[ti] = *reinterpret_cast<const bf16x8*>(&sX[buf][(64 * wt + 32 * ti + l32) * kLP + 16 * kk + 8 * h]);
#pragma unroll
      for (int fi = 0; fi < 4; ++fi)
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
          acc[fi][ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[fi], bx[ti], acc[fi][ti], 0, 0, 0);
    }
    store(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds features f .. f+3 of token m for each (fi, ti, g)
  const int64_t C = MODE == 0 ? p.K : p.Nf;
#pragma unroll
  for (int ti = 0; ti < 2; ++ti) {
    const int64_t m = m0 + 64 * wt + 32 * ti + l32;
    if (m >= p.M) continue;
    const int64_t b = m / p.N, n = m - b * p.N;
#pragma unroll
    for (int fi = 0; fi < 4; ++fi)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t f = f0 + 128 * wf + 32 * fi + 8 * g + 4 * h;
        if (f >= p.Nf) continue;
        const float v0 = acc[fi][ti][4 * g + 0], v1 = acc[fi][ti][4 * g + 1];
        const float v2 = acc[fi][ti][4 * g + 2], v3 = acc[fi][ti][4 * g + 3];
        if (MODE == 0) {
          const int64_t t = f / C, fc = f - t * C;
          const int64_t hh = fc / p.d, e = fc - hh * p.d;
          bf16_t* dst = t == 0 ? out0 : t == 1 ? out1 : t == 2 ? out2 : out3;
          *reinterpret_cast<uint2*>(dst + ((b * p.H + hh) * p.N + n) * p.d + e) =
              make_uint2(pack_bf16(v0, v1), pack_bf16(v2, v3));
        } else {
          const int64_t off = m * C + f;
          const uint2 rv = *reinterpret_cast<const uint2*>(resid + off);
          *reinterpret_cast<uint2*>(out0 + off) =
              make_uint2(pack_bf16(bf_lo(rv.x) + v0, bf_hi(rv.x) + v1), pack_bf16(bf_lo(rv.y) + v2, bf_hi(rv.y) + v3));
        }
      }
  }
}

// Plain float32 projections: 64 x 64 output tile per block of 256 threads,
// 4 x 4 outputs per thread, K through LDS in steps of 16.
template <int MODE>
__global__ __launch_bounds__(256) void proj_f32(const float* __restrict__ X, const float* __restrict__ W,
                                                float* out0, float* __restrict__ out1,
                                                float* __restrict__ out2, float* __restrict__ out3,
                                                const float* resid, ProjShape p) {
  __shared__ float sX[64][17];
  __shared__ float sW[64][17];
  const int tid = threadIdx.x;
  const int64_t nt_f = (p.Nf + 63) / 64;
  const int64_t tm = blockIdx.x / nt_f, tf = blockIdx.x % nt_f;
  const int64_t m0 = tm * 64, f0 = tf * 64;
  const int tx = tid & 15, ty = tid >> 4;  // features 4 tx.., tokens 4 ty..
  float acc[4][4] = {};
  auto xaddr = [&](int64_t m, int64_t k) -> int64_t {
    if (MODE == 0) return m * p.K + k;
    const int64_t b = m / p.N, n = m - b * p.N;
    return ((b * p.H + k / p.d) * p.N + n) * p.d + k % p.d;
  };
  for (int64_t k0 = 0; k0 < p.K; k0 += 16) {
    for (int e = tid; e < 64 * 16; e += 256) {
      const int r = e / 16, c = e % 16;
      const int64_t m = m0 + r, f = f0 + r, k = k0 + c;
      sX[r][c] = (m < p.M && k < p.K) ? X[xaddr(m, k)] : 0.f;
      sW[r][c] = (f < p.Nf && k < p.K) ? W[f * p.K + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 16; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(sX[4 * ty + i][c], sW[4 * tx + j][c], acc[i][j]);
    __syncthreads();
  }
  const int64_t C = MODE == 0 ? p.K : p.Nf;
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + 4 * ty + i;
    if (m >= p.M) continue;
    const int64_t b = m / p.N, n = m - b * p.N;
    for (int j = 0; j < 4; ++j) {
      const int64_t f = f0 + 4 * tx + j;
      if (f >= p.Nf) continue;
      if (MODE == 0) {
        const int64_t t = f / C, fc = f - t * C;
        float* dst = t == 0 ? out0 : t == 1 ? out1 : t == 2 ? out2 : out3;
        dst[((b * p.H + fc / p.d) * p.N + n) * p.d + fc % p.d] = acc[i][j];
      } else {
        out0[m * C + f] = resid[m * C + f] + acc[i][j];
      }
    }
  }
}

ProjShape shape(int64_t B, int64_t H, int64_t N, int d, bool in) {
  ProjShape p{};
  const int64_t C = H * d;
  p.M = B * N;
  p.Nf = in ? 4 * C : C;
  p.K = C;
  p.N = N;
  p.H = H;
  p.d = d;
  p.nt_f = (p.Nf + kTF - 1) / kTF;
  p.nt_m = (p.M + kTM - 1) / kTM;
  p.total = p.nt_f * p.nt_m;
  return p;
}

template <int MODE>
hipError_t launch_proj(bool bf16, const void* X, const void* W, void* o0, void* o1, void* o2, void* o3,
                       const void* resid, int64_t B, int64_t H, int64_t N, int d, hipStream_t s) {
  const ProjShape p = shape(B, H, N, d, MODE == 0);
  if (p.M == 0 || p.K == 0) return hipSuccess;
  if (bf16) {
    proj_bf16<MODE><<<dim3(static_cast<unsigned>(p.total)), dim3(512), 0, s>>>(
        static_cast<const bf16_t*>(X), static_cast<const bf16_t*>(W), static_cast<bf16_t*>(o0),
        static_cast<bf16_t*>(o1), static_cast<bf16_t*>(o2), static_cast<bf16_t*>(o3),
        static_cast<const bf16_t*>(resid), p);
  } else {
    const int64_t blocks = ((p.M + 63) / 64) * ((p.Nf + 63) / 64);
    proj_f32<MODE><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(
        static_cast<const float*>(X), static_cast<const float*>(W), static_cast<float*>(o0),
        static_cast<float*>(o1), static_cast<float*>(o2), static_cast<float*>(o3),
        static_cast<const float*>(resid), p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_proj_in(bool bf16, const void* x, const void* W_in, void* Q, void* K, void* V, void* G,
                          int64_t B, int64_t H, int64_t N, int d, hipStream_t s) {
  return launch_proj<0>(bf16, x, W_in, Q, K, V, G, nullptr, B, H, N, d, s);
}

hipError_t launch_proj_out(bool bf16, const void* O, const void* W_out, const void* x, void* x_out,
                           int64_t B, int64_t H, int64_t N, int d, hipStream_t s) {
  return launch_proj<1>(bf16, O, W_out, x_out, nullptr, nullptr, nullptr, x, B, H, N, d, s);
}

}  // namespace ha
