// Gated softmax anchor (SANA-Video 2.0 summary page, section 03; review page,
// section 1): o_i = sigmoid(g_i) * sum_j softmax_j(q_i . k_j / sqrt(d)) v_j over
// all N tokens of the (batch, head), without materialising the N x N logits:
// key blocks stream through LDS and an online maximum and sum per query row
// rescale the running output (the flash-attention recurrence).
//
// bf16 kernel, one block = 128 queries of one (b, h), 4 waves x 32 queries:
//  * logits are computed transposed, S^T = K Q^T, with the 32x32x16 bf16 MFMA:
//    the A operand is a K row from LDS, the B operand the wave's Q rows, held in
//    registers.  A lane's accumulator then holds 16 keys of ONE query, so the
//    row maximum and sum are mostly lane-local (one exchange with lane ^ 32);
//  * the probabilities P^T stay in registers and feed the PV MFMA directly as
//    its B operand (O^T += V^T P^T).  The key order that the accumulator layout
//    gives each lane is matched by storing V^T in LDS with bits 2 and 3 of the
//    key index swapped inside every 16-key group;
//  * V is transposed on the way into LDS (4 keys x 8 features per thread);
//  * the next key block's loads are issued before the current block's MFMAs.
#include "ha_device.h"
#include "ha_launch.h"

namespace ha {

namespace {

constexpr int kBr = 128;  // queries per block
constexpr int kBc = 64;   // keys per iteration
constexpr float kLog2e = 1.4426950408889634f;

// LDS column of key k (0..63 inside a key block) in the V^T tile.
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~15) | ((k & 4) << 1) | ((k & 8) >> 1) | (k & 3);
}

template <int D>
__global__ __launch_bounds__(256, 2) void anchor_bf16(const bf16_t* __restrict__ Q,
                                                      const bf16_t* __restrict__ K,
                                                      const bf16_t* __restrict__ V,
                                                      const bf16_t* __restrict__ G,
                                                      bf16_t* __restrict__ O, int64_t N,
                                                      int64_t qblocks, int64_t total, float c) {
  constexpr int KP = D + 8;              // LDS pitch of K rows (elements)
  constexpr int VP = kBc + 8;            // LDS pitch of V^T rows (elements)
  constexpr int FG = D / 8;              // 16-byte groups per row
  constexpr int KCH = kBc * FG / 256;    // K chunks per thread per block
  constexpr int VSUB = (kBc / 4) * FG;   // V sub-tiles (4 keys x 8 features) per block
  constexpr int KS = D / 16;             // k-steps of the logit MFMA
  constexpr int RB = D / 32;             // 32-feature row blocks of O^T
  __shared__ __attribute__((aligned(16))) bf16_t sK[kBc * KP];
  __shared__ __attribute__((aligned(16))) bf16_t sVt[D * VP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int64_t id = xcd_remap(blockIdx.x, total);
  const int64_t bh = id / qblocks;
  const int64_t q0 = (id % qblocks) * kBr + 32 * wave;
  const int64_t base = bh * N * D;
  const int64_t qrow = q0 + l32;

  bf16x8 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    qf[s] = as_bf16x8(qrow < N ? *reinterpret_cast<const uint4*>(Q + base + qrow * D + 16 * s + 8 * h)
                               : make_uint4(0, 0, 0, 0));

  // loads of one key block into registers
  const bool v_loader = tid < VSUB;
  const int v_fg = tid % FG, v_m = tid / FG;
  uint4 kreg[KCH], vreg[4];
  auto load_block = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int cidx = tid + 256 * i;
      const int64_t key = k0 + cidx / FG;
      kreg[i] = key < N ? *reinterpret_cast<const uint4*>(K + base + key * D + 8 * (cidx % FG))
                        : make_uint4(0, 0, 0, 0);
    }
    if (v_loader) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t key = k0 + 4 * v_m + r;
        vreg[r] = key < N ? *reinterpret_cast<const uint4*>(V + base + key * D + 8 * v_fg)
                          : make_uint4(0, 0, 0, 0);
      }
    }
  };

  f32x16 o[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[rb][r] = 0.f;
  float m = -INFINITY;  // running max of the raw logits of this lane's query
  float lsum = 0.f;     // running sum of this lane's probabilities (half the keys)

  const int64_t nkb = (N + kBc - 1) / kBc;
  load_block(0);
  for (int64_t kb = 0; kb < nkb; ++kb) {
    const int64_t k0 = kb * kBc;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int cidx = tid + 256 * i;
      *reinterpret_cast<uint4*>(sK + (cidx / FG) * KP + 8 * (cidx % FG)) = kreg[i];
    }
    if (v_loader) {
      uint2 tr[8];
      transpose4x8(vreg, tr);
      const int pos = vt_pos(4 * v_m);
#pragma unroll
      for (int f = 0; f < 8; ++f) *reinterpret_cast<uint2*>(sVt + (8 * v_fg + f) * VP + pos) = tr[f];
    }
    __syncthreads();
    if (kb + 1 < nkb) load_block(k0 + kBc);

    // S^T for 64 keys x 32 queries: two 32x32 blocks
    f32x16 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[t][r] = 0.f;
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sK + (32 * t + l32) * KP + 16 * st + 8 * h);
        s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[st], s[t], 0, 0, 0);
      }
    }
    if (k0 + kBc > N) {  // ragged last block: keys >= N get -inf
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t key = k0 + 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
          if (key >= N) s[t][r] = -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f((m - m_new) * c);
    const float mc = m_new * c;
    m = m_new;
    float ps = 0.f;
    bf16x8 pf[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          p[j] = __builtin_amdgcn_exp2f(fmaf(s[t][8 * tt + j], c, -mc));
          ps += p[j];
        }
        uint4 pk;
        pk.x = pack_bf16(p[0], p[1]);
        pk.y = pack_bf16(p[2], p[3]);
        pk.z = pack_bf16(p[4], p[5]);
        pk.w = pack_bf16(p[6], p[7]);
        pf[t][tt] = as_bf16x8(pk);
      }
    lsum = fmaf(lsum, alpha, ps);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) o[rb][r] *= alpha;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const bf16x8 vf =
              *reinterpret_cast<const bf16x8*>(sVt + (32 * rb + l32) * VP + 32 * t + 16 * tt + 8 * h);
          o[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[t][tt], o[rb], 0, 0, 0);
        }
    }
  }

  const float l = lsum + __shfl_xor(lsum, 32);
  const float inv = __builtin_amdgcn_rcpf(l);
  if (qrow < N) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int f0 = 32 * rb + 8 * g4 + 4 * h;
        const int64_t off = base + qrow * D + f0;
        const uint2 gv = *reinterpret_cast<const uint2*>(G + off);
        uint2 ov;
        ov.x = pack_bf16(gate_fast(bf_lo(gv.x)) * (o[rb][4 * g4 + 0] * inv),
                         gate_fast(bf_hi(gv.x)) * (o[rb][4 * g4 + 1] * inv));
        ov.y = pack_bf16(gate_fast(bf_lo(gv.y)) * (o[rb][4 * g4 + 2] * inv),
                         gate_fast(bf_hi(gv.y)) * (o[rb][4 * g4 + 3] * inv));
        *reinterpret_cast<uint2*>(O + off) = ov;
      }
  }
}

// Plain float32 anchor: two lanes per query (each half of d), 64 queries per
// block, 32-key blocks in LDS, online softmax per key block.
template <int D>
__global__ __launch_bounds__(128) void anchor_f32(const float* __restrict__ Q,
                                                  const float* __restrict__ K,
                                                  const float* __restrict__ V,
                                                  const float* __restrict__ G,
                                                  float* __restrict__ O, int64_t N,
                                                  int64_t qblocks, float scale) {
  constexpr int BQ = 64, BK = 32, HD = D / 2;
  __shared__ float sK[BK][D];
  __shared__ float sV[BK][D];
  const int tid = threadIdx.x;
  const int half = tid & 1;
  const int64_t bh = blockIdx.x / qblocks;
  const int64_t qrow = (blockIdx.x % qblocks) * BQ + (tid >> 1);
  const int64_t base = bh * N * D;
  float q[HD], acc[HD];
#pragma unroll
  for (int e = 0; e < HD; ++e) {
    q[e] = qrow < N ? Q[base + qrow * D + half * HD + e] : 0.f;
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int64_t k0 = 0; k0 < N; k0 += BK) {
    __syncthreads();
    for (int e = tid; e < BK * D; e += 128) {
      const int64_t key = k0 + e / D;
      sK[e / D][e % D] = key < N ? K[base + key * D + e % D] : 0.f;
      sV[e / D][e % D] = key < N ? V[base + key * D + e % D] : 0.f;
    }
    __syncthreads();
    float sc[BK];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < BK; ++j) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < HD; ++e) part = fmaf(q[e], sK[j][half * HD + e], part);
      part += __shfl_xor(part, 1);
      sc[j] = k0 + j < N ? part * scale : -INFINITY;
      mx = fmaxf(mx, sc[j]);
    }
    const float m_new = fmaxf(m, mx);
    const float alpha = expf(m - m_new);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < HD; ++e) acc[e] *= alpha;
#pragma unroll
    for (int j = 0; j < BK; ++j) {
      const float p = expf(sc[j] - m_new);
      l += p;
#pragma unroll
      for (int e = 0; e < HD; ++e) acc[e] = fmaf(p, sV[j][half * HD + e], acc[e]);
    }
    m = m_new;
  }
  if (qrow < N) {
#pragma unroll
    for (int e = 0; e < HD; ++e) {
      const int64_t off = base + qrow * D + half * HD + e;
      O[off] = gate_exact(G[off]) * (acc[e] / l);
    }
  }
}

}  // namespace

hipError_t launch_anchor(bool bf16, int d, const void* Q, const void* K, const void* V,
                         const void* G, void* O, int64_t BH, int64_t N, hipStream_t s) {
  if (BH == 0 || N == 0) return hipSuccess;
  if (bf16) {
    const int64_t qb = (N + kBr - 1) / kBr;
    const int64_t total = BH * qb;
    const float c = kLog2e / sqrtf(static_cast<float>(d));
    const bf16_t* q = static_cast<const bf16_t*>(Q);
    const bf16_t* k = static_cast<const bf16_t*>(K);
    const bf16_t* v = static_cast<const bf16_t*>(V);
    const bf16_t* g = static_cast<const bf16_t*>(G);
    bf16_t* o = static_cast<bf16_t*>(O);
    const dim3 grid(static_cast<unsigned>(total)), block(256);
    if (d == 128)
      anchor_bf16<128><<<grid, block, 0, s>>>(q, k, v, g, o, N, qb, total, c);
    else
      anchor_bf16<64><<<grid, block, 0, s>>>(q, k, v, g, o, N, qb, total, c);
  } else {
    const int64_t qb = (N + 63) / 64;
    const float scale = 1.0f / sqrtf(static_cast<float>(d));
    const float* q = static_cast<const float*>(Q);
    const float* k = static_cast<const float*>(K);
    const float* v = static_cast<const float*>(V);
    const float* g = static_cast<const float*>(G);
    float* o = static_cast<float*>(O);
    const dim3 grid(static_cast<unsigned>(BH * qb)), block(128);
    if (d == 128)
      anchor_f32<128><<<grid, block, 0, s>>>(q, k, v, g, o, N, qb, scale);
    else
      anchor_f32<64><<<grid, block, 0, s>>>(q, k, v, g, o, N, qb, scale);
  }
  return hipGetLastError();
}

}  // namespace ha
