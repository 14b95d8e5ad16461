// Backward pass of the gated linear layer (the model is trained from scratch:
// SANA-Video 2.0 review page, section 3; the layer: summary page, section 03).
// Per head, with phi = ReLU, s = sigmoid(g), n = phi(q) S, den = phi(q).z + eps,
// a = n / den, o = s * a and an upstream gradient dO:
//   dG = dO a s (1 - s)     da = dO s     dn = da / den     dden = -(da . a) / den
//   dS = sum_i phi(q_i)^T dn_i            dz = sum_i dden_i phi(q_i)
//   dQ = (dn S^T + dden z) [q > 0]        dK = (v dS^T + dz) [k > 0]     dV = phi(k) dS
// Six passes, all streaming tokens once:
//   1. S, z (the forward's split-N state reduction, also keeping S as bf16 hi/lo
//      in both orientations);
//   2. per token: n on the MFMA, then dG, dn (bf16) and dden;
//   3. dS, dz: the same state reduction on (phi(Q), dn) with the z sum weighted
//      by dden;
//   4-6. per token: dQ, dV, dK, each one d x d product on the MFMA with a fused
//      epilogue.
// Passes 2 and 4-6 share one kernel: a 64-token tile of X times a d x d matrix
// held by each wave as bf16 hi + lo MFMA B operands in registers (as the
// forward apply does), the product staged through LDS so that the epilogue
// reads and writes whole token rows with 16-byte accesses.
#include "ha_device.h"
#include "ha_launch.h"

namespace ha {

namespace {

constexpr int kTok = 64;
enum : int { kEpiN = 0, kEpiDQ = 1, kEpiDV = 2, kEpiDK = 3 };

__device__ __forceinline__ float pos(float x) { return x > 0.f ? 1.f : 0.f; }

// out[t][j] = sum_a X'[t][a] M[a][j], M given as Mt[j][a] = hi + lo (bf16), X' = phi(X)
// for kEpiN and kEpiDV.  Epilogues:
//   kEpiN : vec = z, E1 = G, E2 = dO -> out1 = dG, out2 = dn, rowout = dden
//   kEpiDQ: vec = z, E1 = Q, rowv = dden -> out1 = (acc + dden z) [Q > 0]
//   kEpiDV:                   -> out1 = acc
//   kEpiDK: vec = dz, E1 = K  -> out1 = (acc + dz) [K > 0]
// Two blocks per CU at least: the compiler keeps every epilogue within 256
// registers (the n-pass epilogue took 268, which left one block per CU).
template <int D, int EPI>
__global__ __launch_bounds__(256, 2) void tgemm_bf16(const bf16_t* __restrict__ X,
                                                  const bf16_t* __restrict__ Mt_hi,
                                                  const bf16_t* __restrict__ Mt_lo,
                                                  const float* __restrict__ vec,
                                                  const bf16_t* __restrict__ E1,
                                                  const bf16_t* __restrict__ E2,
                                                  const float* __restrict__ rowv,
                                                  bf16_t* __restrict__ out1, bf16_t* __restrict__ out2,
                                                  float* __restrict__ rowout, int64_t N,
                                                  int64_t tiles_per_block, int64_t blocks_per_head,
                                                  float eps) {
  constexpr bool PHI = EPI == kEpiN || EPI == kEpiDV;
  constexpr bool HAS_E1 = EPI != kEpiDV;
  constexpr bool HAS_E2 = EPI == kEpiN;
  constexpr bool HAS_VEC = EPI != kEpiDV;
  constexpr int XP = D + 8;
  constexpr int NP = D + 4;
  constexpr int FG = D / 8;
  constexpr int CH = kTok * FG / 256;
  constexpr int NB = D / 64;
  constexpr int KS = D / 32;
  __shared__ __attribute__((aligned(16))) bf16_t sX[kTok * XP];
  __shared__ __attribute__((aligned(16))) float sNum[kTok * NP];
  __shared__ float sDen[kTok];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c16 = lane & 15;
  const int kq = lane >> 4;
  const int64_t bh = blockIdx.x / blocks_per_head;
  const int64_t blk = blockIdx.x % blocks_per_head;
  const int64_t base = bh * N * D;

  bf16x8 bhi[NB][KS], blo[NB][KS];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int j = wave * (D / 4) + 16 * nb + c16;
      const int64_t off = bh * D * D + j * D + 32 * s + 8 * kq;
      bhi[nb][s] = as_bf16x8(*reinterpret_cast<const uint4*>(Mt_hi + off));
      blo[nb][s] = as_bf16x8(*reinterpret_cast<const uint4*>(Mt_lo + off));
    }
  const int fg = tid % FG;
  float vf[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) vf[k] = HAS_VEC ? vec[bh * D + 8 * fg + k] : 0.f;

  // block blk of a head takes its tiles blk, blk + B, blk + 2B, ... (B blocks
  // per head): the blocks in flight sweep the head's rows as one front
  const int64_t ntiles = (N + kTok - 1) / kTok;
  const int64_t tstride = blocks_per_head;

  uint4 xv[CH], e1v[CH], e2v[CH];
  auto load_tile = [&](int64_t t) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int64_t tok = t * kTok + (tid + 256 * i) / FG;
      const bool ok = t < ntiles && tok < N;
      const int64_t off = base + tok * D + 8 * fg;
      xv[i] = ok ? *reinterpret_cast<const uint4*>(X + off) : make_uint4(0, 0, 0, 0);
      e1v[i] = (HAS_E1 && ok) ? *reinterpret_cast<const uint4*>(E1 + off) : make_uint4(0, 0, 0, 0);
      e2v[i] = (HAS_E2 && ok) ? *reinterpret_cast<const uint4*>(E2 + off) : make_uint4(0, 0, 0, 0);
    }
  };
  load_tile(blk);
  for (int64_t t = blk; t < ntiles; t += tstride) {
    const int64_t tok0 = t * kTok;
    uint4 e1c[CH], e2c[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int row = (tid + 256 * i) / FG;
      const uint4 x = PHI ? relu8(xv[i]) : xv[i];
      e1c[i] = e1v[i];
      e2c[i] = e2v[i];
      if (EPI == kEpiN) {
        float dp = bf_lo(x.x) * vf[0];
        dp = fmaf(bf_hi(x.x), vf[1], dp);
        dp = fmaf(bf_lo(x.y), vf[2], dp);
        dp = fmaf(bf_hi(x.y), vf[3], dp);
        dp = fmaf(bf_lo(x.z), vf[4], dp);
        dp = fmaf(bf_hi(x.z), vf[5], dp);
        dp = fmaf(bf_lo(x.w), vf[6], dp);
        dp = fmaf(bf_hi(x.w), vf[7], dp);
#pragma unroll
        for (int m = 1; m < FG; m <<= 1) dp += __shfl_xor(dp, m);
        if (fg == 0) sDen[row] = dp + eps;
      }
      *reinterpret_cast<uint4*>(sX + row * XP + 8 * fg) = x;
    }
    __syncthreads();
    load_tile(t + tstride);
#pragma unroll
    for (int mb = 0; mb < kTok / 16; ++mb) {
      f32x4 acc[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(sX + (16 * mb + c16) * XP + 32 * s + 8 * kq);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bhi[nb][s], acc[nb], 0, 0, 0);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, blo[nb][s], acc[nb], 0, 0, 0);
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sNum[(16 * mb + 4 * kq + r) * NP + wave * (D / 4) + 16 * nb + c16] = acc[nb][r];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int row = (tid + 256 * i) / FG;
      const int64_t tok = tok0 + row;
      if (tok < N) {
        const float4 n0 = *reinterpret_cast<const float4*>(sNum + row * NP + 8 * fg);
        const float4 n1 = *reinterpret_cast<const float4*>(sNum + row * NP + 8 * fg + 4);
        const float acc8[8] = {n0.x, n0.y, n0.z, n0.w, n1.x, n1.y, n1.z, n1.w};
        const int64_t off = base + tok * D + 8 * fg;
        const uint32_t e1w[4] = {e1c[i].x, e1c[i].y, e1c[i].z, e1c[i].w};
        const uint32_t e2w[4] = {e2c[i].x, e2c[i].y, e2c[i].z, e2c[i].w};
        float r8[8], r8b[8];
        if (EPI == kEpiN) {
          const float inv = __builtin_amdgcn_rcpf(sDen[row]);
          float p = 0.f;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float g = (k & 1) ? bf_hi(e1w[k / 2]) : bf_lo(e1w[k / 2]);
            const float dout = (k & 1) ? bf_hi(e2w[k / 2]) : bf_lo(e2w[k / 2]);
            const float a = acc8[k] * inv;
            const float sg = gate_fast(g);
            const float da = dout * sg;
            r8[k] = da * a * (1.f - sg);   // dG
            r8b[k] = da * inv;             // dn
            p = fmaf(da, a, p);
          }
#pragma unroll
          for (int m = 1; m < FG; m <<= 1) p += __shfl_xor(p, m);
          if (fg == 0) rowout[bh * N + tok] = -p * inv;
          *reinterpret_cast<uint4*>(out2 + off) =
              make_uint4(pack_bf16(r8b[0], r8b[1]), pack_bf16(r8b[2], r8b[3]),
                         pack_bf16(r8b[4], r8b[5]), pack_bf16(r8b[6], r8b[7]));
        } else if (EPI == kEpiDQ) {
          const float dd = rowv[bh * N + tok];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float q = (k & 1) ? bf_hi(e1w[k / 2]) : bf_lo(e1w[k / 2]);
            r8[k] = fmaf(dd, vf[k], acc8[k]) * pos(q);
          }
        } else if (EPI == kEpiDV) {
#pragma unroll
          for (int k = 0; k < 8; ++k) r8[k] = acc8[k];
        } else {
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float kk = (k & 1) ? bf_hi(e1w[k / 2]) : bf_lo(e1w[k / 2]);
            r8[k] = (acc8[k] + vf[k]) * pos(kk);
          }
        }
        *reinterpret_cast<uint4*>(out1 + off) =
            make_uint4(pack_bf16(r8[0], r8[1]), pack_bf16(r8[2], r8[3]),
                       pack_bf16(r8[4], r8[5]), pack_bf16(r8[6], r8[7]));
      }
    }
    __syncthreads();
  }
}

// Plain float32 version: 16 tokens per tile, thread (row, column slice), M read
// through the caches: element (a, j) at M[a * D + j], or M[j * D + a] when TRANS.
template <int D, int EPI, bool TRANS>
__global__ __launch_bounds__(256) void tgemm_f32(const float* __restrict__ X, const float* __restrict__ M,
                                                 const float* __restrict__ vec,
                                                 const float* __restrict__ E1,
                                                 const float* __restrict__ E2,
                                                 const float* __restrict__ rowv,
                                                 float* __restrict__ out1, float* __restrict__ out2,
                                                 float* __restrict__ rowout, int64_t N,
                                                 int64_t tiles_per_block, int64_t blocks_per_head,
                                                 float eps) {
  constexpr bool PHI = EPI == kEpiN || EPI == kEpiDV;
  constexpr int T = 16;
  __shared__ float sX[T * D];
  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x / blocks_per_head;
  const int64_t blk = blockIdx.x % blocks_per_head;
  const int64_t base = bh * N * D;
  const float* Mh = M + bh * D * D;
  const float* vh = vec != nullptr ? vec + bh * D : nullptr;
  const int row = tid >> 4, tj = tid & 15;
  const int64_t ntiles = (N + T - 1) / T;
  const int64_t tb = blk * tiles_per_block;
  const int64_t te = min(ntiles, tb + tiles_per_block);
  for (int64_t t = tb; t < te; ++t) {
    const int64_t tok0 = t * T;
    __syncthreads();
    for (int e = tid; e < T * D; e += 256) {
      const int64_t tok = tok0 + e / D;
      const float x = tok < N ? X[base + tok * D + e % D] : 0.f;
      sX[e] = PHI ? fmaxf(x, 0.f) : x;
    }
    __syncthreads();
    const int64_t tok = tok0 + row;
    const bool ok = tok < N;   // uniform over the 16 lanes of a row
    float den = 1.f;
    if (EPI == kEpiN) {
      den = 0.f;
#pragma unroll 8
      for (int a = 0; a < D; ++a) den = fmaf(sX[row * D + a], vh[a], den);
      den += eps;
    }
    float p = 0.f;
#pragma unroll 1
    for (int y = 0; y < D / 16; ++y) {
      const int j = tj + 16 * y;
      float acc = 0.f;
#pragma unroll 8
      for (int a = 0; a < D; ++a) acc = fmaf(sX[row * D + a], TRANS ? Mh[j * D + a] : Mh[a * D + j], acc);
      if (!ok) continue;
      const int64_t off = base + tok * D + j;
      if (EPI == kEpiN) {
        const float a = acc / den;
        const float sg = gate_exact(E1[off]);
        const float da = E2[off] * sg;
        out1[off] = da * a * (1.f - sg);
        out2[off] = da / den;
        p = fmaf(da, a, p);
      } else if (EPI == kEpiDQ) {
        out1[off] = fmaf(rowv[bh * N + tok], vh[j], acc) * pos(E1[off]);
      } else if (EPI == kEpiDV) {
        out1[off] = acc;
      } else {
        out1[off] = (acc + vh[j]) * pos(E1[off]);
      }
    }
    if (EPI == kEpiN) {
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) p += __shfl_xor(p, m);
      if (ok && tj == 0) rowout[bh * N + tok] = -p / den;
    }
  }
}

struct Grid {
  int64_t tpb, bph;
};

Grid token_grid(int64_t BH, int64_t N, int tile) {
  const int64_t ntiles = (N + tile - 1) / tile;
  int64_t bph = (2048 + BH - 1) / BH;
  if (bph > ntiles) bph = ntiles;
  const int64_t tpb = (ntiles + bph - 1) / bph;
  return Grid{tpb, (ntiles + tpb - 1) / tpb};
}

template <int EPI>
hipError_t launch_tgemm(bool bf16, int d, const void* X, const uint16_t* Mt_hi, const uint16_t* Mt_lo,
                        const float* M, bool trans, const float* vec, const void* E1, const void* E2,
                        const float* rowv, void* out1, void* out2, float* rowout, int64_t BH, int64_t N,
                        float eps, hipStream_t s) {
  const Grid g = token_grid(BH, N, bf16 ? kTok : 16);
  const dim3 grid(static_cast<unsigned>(BH * g.bph)), block(256);
  if (bf16) {
    auto go = [&](auto kern) {
      kern<<<grid, block, 0, s>>>(static_cast<const bf16_t*>(X), Mt_hi, Mt_lo, vec,
                                  static_cast<const bf16_t*>(E1), static_cast<const bf16_t*>(E2), rowv,
                                  static_cast<bf16_t*>(out1), static_cast<bf16_t*>(out2), rowout, N, g.tpb,
                                  g.bph, eps);
    };
    if (d == 128)
      go(tgemm_bf16<128, EPI>);
    else
      go(tgemm_bf16<64, EPI>);
  } else {
    auto go = [&](auto kern) {
      kern<<<grid, block, 0, s>>>(static_cast<const float*>(X), M, vec, static_cast<const float*>(E1),
                                  static_cast<const float*>(E2), rowv, static_cast<float*>(out1),
                                  static_cast<float*>(out2), rowout, N, g.tpb, g.bph, eps);
    };
    if (d == 128)
      trans ? go(tgemm_f32<128, EPI, true>) : go(tgemm_f32<128, EPI, false>);
    else
      trans ? go(tgemm_f32<64, EPI, true>) : go(tgemm_f32<64, EPI, false>);
  }
  return hipGetLastError();
}

}  // namespace

LinearBwdWs linear_bwd_ws(int64_t BH, int64_t N, int d, bool bf16) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  const KvSplit sp = kv_split(BH, N);
  const size_t dd = static_cast<size_t>(d) * d;
  const size_t hsz = static_cast<size_t>(BH) * dd * sizeof(uint16_t);
  const size_t fsz = static_cast<size_t>(BH) * dd * sizeof(float);
  const size_t vsz = static_cast<size_t>(BH) * d * sizeof(float);
  LinearBwdWs L{};
  size_t off = 0;
  L.part = off;
  off += up(static_cast<size_t>(BH) * sp.chunks * (dd + d) * sizeof(float));
  L.S = off;
  off += up(fsz);
  L.z = off;
  off += up(vsz);
  L.dS = off;
  off += up(fsz);
  L.dz = off;
  off += up(vsz);
  for (size_t* h : {&L.St_hi, &L.St_lo, &L.S_hi, &L.S_lo, &L.dSt_hi, &L.dSt_lo, &L.dS_hi, &L.dS_lo}) {
    *h = off;
    if (bf16) off += up(hsz);
  }
  L.dn = off;
  off += up(static_cast<size_t>(BH) * N * d * (bf16 ? 2u : 4u));
  L.dden = off;
  off += up(static_cast<size_t>(BH) * N * sizeof(float));
  L.total = off;
  return L;
}

hipError_t launch_linear_backward(bool bf16, int d, const void* Q, const void* K, const void* V,
                                  const void* G, const void* dO, void* dQ, void* dK, void* dV, void* dG,
                                  int64_t BH, int64_t N, float eps, void* ws, hipStream_t s) {
  if (BH == 0 || N == 0) return hipSuccess;
  const LinearBwdWs L = linear_bwd_ws(BH, N, d, bf16);
  char* w = static_cast<char*>(ws);
  auto f = [&](size_t o) { return reinterpret_cast<float*>(w + o); };
  auto h = [&](size_t o) { return reinterpret_cast<uint16_t*>(w + o); };
  float *part = f(L.part), *S = f(L.S), *z = f(L.z), *dS = f(L.dS), *dz = f(L.dz), *dden = f(L.dden);
  void* dn = w + L.dn;
  const KvSplit sp = kv_split(BH, N);
  hipError_t e;
  // 1. S, z
  if ((e = launch_kv_partials(bf16, d, K, V, part, BH, N, sp, s)) != hipSuccess) return e;
  if ((e = launch_kv_reduce(bf16, d, part, S, z, h(L.St_hi), h(L.St_lo), BH, sp.chunks, s, h(L.S_hi),
                            h(L.S_lo))) != hipSuccess)
    return e;
  // 2. n = phi(Q) S -> dG, dn, dden
  if ((e = launch_tgemm<kEpiN>(bf16, d, Q, h(L.St_hi), h(L.St_lo), S, false, z, G, dO, nullptr, dG, dn,
                               dden, BH, N, eps, s)) != hipSuccess)
    return e;
  // 3. dS = phi(Q)^T dn, dz = sum dden phi(Q)
  if ((e = launch_kv_partials(bf16, d, Q, dn, part, BH, N, sp, s, dden)) != hipSuccess) return e;
  if ((e = launch_kv_reduce(bf16, d, part, dS, dz, h(L.dSt_hi), h(L.dSt_lo), BH, sp.chunks, s,
                            h(L.dS_hi), h(L.dS_lo))) != hipSuccess)
    return e;
  // 4. dQ = (dn S^T + dden z) [Q > 0]
  if ((e = launch_tgemm<kEpiDQ>(bf16, d, dn, h(L.S_hi), h(L.S_lo), S, true, z, Q, nullptr, dden, dQ,
                                nullptr, nullptr, BH, N, eps, s)) != hipSuccess)
    return e;
  // 5. dV = phi(K) dS
  if ((e = launch_tgemm<kEpiDV>(bf16, d, K, h(L.dSt_hi), h(L.dSt_lo), dS, false, nullptr, nullptr, nullptr,
                                nullptr, dV, nullptr, nullptr, BH, N, eps, s)) != hipSuccess)
    return e;
  // 6. dK = (V dS^T + dz) [K > 0]
  return launch_tgemm<kEpiDK>(bf16, d, V, h(L.dS_hi), h(L.dS_lo), dS, true, dz, K, nullptr, nullptr, dK,
                              nullptr, nullptr, BH, N, eps, s);
}

}  // namespace ha
