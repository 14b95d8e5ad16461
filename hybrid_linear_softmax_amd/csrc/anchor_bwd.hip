// Backward pass of the gated softmax anchor (the model is trained from scratch:
// SANA-Video 2.0 review page, section 3; the anchor: summary page, section 03).
// With s = sigmoid(g), P = softmax(Q K^T / sqrt(d)), a = P V, o = s * a, an
// upstream gradient dO and the forward's per-query log-sum-exp L:
//   da = dO * s,   dG = dO * o * (1 - s),   D_i = da_i . a_i = dO_i . o_i,
//   P_ij = exp(q_i . k_j / sqrt(d) - L_i),  dP_ij = da_i . v_j,
//   dS_ij = P_ij (dP_ij - D_i),
//   dQ = dS K / sqrt(d),   dK = dS^T Q / sqrt(d),   dV = P^T da.
// Three kernels: an elementwise pre-pass (dG, da in the I/O dtype, D in
// float32), then dQ with queries resident (the forward's structure: S^T = K Q^T
// so that a lane's accumulator holds keys of one query, and dS^T feeds the
// dQ^T product as its B operand straight from registers), then dK and dV with
// keys resident (S = Q K^T, so a lane holds queries of one key and P, dS feed
// the dV^T and dK^T products).  Q^T, da^T and K^T tiles are written to LDS
// with bits 2 and 3 of the row index swapped inside each 16-row group: the
// order in which an MFMA accumulator lists its rows.  No atomics: dQ, dK and
// dV are each owned by one block, so results are reproducible.
#include <type_traits>

#include "ha_device.h"
#include "ha_launch.h"

namespace ha {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int perm16(int k) {
  return (k & ~15) | ((k & 4) << 1) | ((k & 8) >> 1) | (k & 3);
}

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}

// ------------------------------------------------------------------ pre-pass
template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]) {
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
__device__ __forceinline__ void store8(T* p, const float (&v)[8]) {
  if constexpr (std::is_same<T, float>::value) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]),
                                              pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7]));
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void sm_bwd_pre(const T* __restrict__ O, const T* __restrict__ dO,
                                                  const T* __restrict__ G, T* __restrict__ dG,
                                                  T* __restrict__ da, float* __restrict__ Dv, int64_t rows) {
  constexpr int FG = D / 8;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t row = e / FG;
  const int fg = static_cast<int>(e % FG);
  const bool ok = row < rows;   // the same for the FG consecutive lanes of a row
  float o[8] = {}, d[8] = {}, g[8] = {};
  const int64_t off = row * D + 8 * fg;
  if (ok) {
    load8(O + off, o);
    load8(dO + off, d);
    load8(G + off, g);
  }
  float p = 0.f, rg[8], ra[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    p = fmaf(d[k], o[k], p);
    const float sg = std::is_same<T, float>::value ? gate_exact(g[k]) : gate_fast(g[k]);
    rg[k] = d[k] * o[k] * (1.f - sg);
    ra[k] = d[k] * sg;
  }
#pragma unroll
  for (int m = 1; m < FG; m <<= 1) p += __shfl_xor(p, m);
  if (ok) {
    store8(dG + off, rg);
    store8(da + off, ra);
    if (fg == 0) Dv[row] = p;
  }
}

// ------------------------------------------------------------------ bf16 dQ
// 8 waves x 32 queries per block, 64-key steps.  Per step: S^T and dP^T
// (keys x queries) on the 32x32x16 MFMA with the wave's Q and da rows as
// register-resident B operands, then dQ^T += K^T dS^T.  K and V tiles come
// straight from global memory into a double-buffered LDS ring (the next tile
// loads during the current step's MFMAs), in unpadded rows whose 16-byte
// chunk c sits in slot c ^ (row mod chunks per row).

// 16 bytes per lane from a buffer straight into LDS at dst + 16 lane (dst
// wave-uniform).  A device function: a target builtin inside a kernel lambda
// can make the host compilation drop the kernel's launch stub.
__device__ __forceinline__ void dq_tile_to_lds16(__amdgpu_buffer_rsrc_t r, bf16_t* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, static_cast<int>(voff), 0, 0, 0);
}

// barrier that waits for this wave's LDS accesses only: the direct tile loads
// in flight (counted by vmcnt) are waited for explicitly where they are needed
__device__ __forceinline__ void dq_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <int D>
__global__ __launch_bounds__(512) void sm_bwd_dq_bf16(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K,
                                                      const bf16_t* __restrict__ V, const bf16_t* __restrict__ da,
                                                      const float* __restrict__ lse, const float* __restrict__ Dv,
                                                      bf16_t* __restrict__ dQ, int64_t N, int64_t qblocks,
                                                      float c) {
  constexpr int NT = 512, BK = 64, BQ = 256;
  constexpr int TP = BK + 8, FG = D / 8;
  constexpr int KS = D / 16, RB = D / 32;
  constexpr int TSUB = (BK / 4) * FG;    // 4-key x 8-feature sub-tiles of the K^T transpose
  constexpr int TILE = BK * D;           // elements of one K or V tile
  constexpr int RPL = 64 / FG;           // rows per 1 KB load
  constexpr int NLD = TILE / 512 / (NT / 64);  // 1 KB loads per wave per tile
  static_assert(NLD * (NT / 64) * 512 == TILE, "tile split over the waves");
  // two buffers as separate arrays, so that the loads into one are seen not to
  // alias the reads of the other
  __shared__ __attribute__((aligned(1024))) bf16_t sK0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16_t sV0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16_t sK1[TILE];
  __shared__ __attribute__((aligned(1024))) bf16_t sV1[TILE];
  __shared__ __attribute__((aligned(16))) bf16_t sKt[D * TP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  // plain dispatch order: the blocks in flight cover one (b, h) across all
  // XCDs, which measured faster here than one head per XCD (xcd_remap)
  const int64_t id = blockIdx.x;
  const int64_t bh = id / qblocks;
  const int64_t qrow = (id % qblocks) * BQ + 32 * wave + l32;
  const int64_t base = bh * N * D;
  const uint32_t head_bytes = static_cast<uint32_t>(N * D * 2);
  const __amdgpu_buffer_rsrc_t rK =
      __builtin_amdgcn_make_buffer_rsrc((void*)(K + base), (short)0, (int)head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rV =
      __builtin_amdgcn_make_buffer_rsrc((void*)(V + base), (short)0, (int)head_bytes, 0x00020000);

  bf16x8 qf[KS], af[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const bool ok = qrow < N;
    qf[s] = as_bf16x8(ok ? *reinterpret_cast<const uint4*>(Q + base + qrow * D + 16 * s + 8 * h) : make_uint4(0, 0, 0, 0));
    af[s] = as_bf16x8(ok ? *reinterpret_cast<const uint4*>(da + base + qrow * D + 16 * s + 8 * h) : make_uint4(0, 0, 0, 0));
  }
  const float l2 = qrow < N ? lse[bh * N + qrow] * kLog2e : 0.f;
  const float Dq = qrow < N ? Dv[bh * N + qrow] : 0.f;
  f32x16 dq[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[rb][r] = 0.f;

  // load j of this wave fills rows RPL (NLD wave + j) .. + RPL - 1 of a tile;
  // lane L fills row RPL (NLD wave + j) + L / FG, slot L % FG, with the row's
  // chunk (L % FG) ^ (row mod FG).  Rows past N read zeros.
  uint32_t voff[NLD];
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    const int row = RPL * (NLD * wave + j) + lane / FG;
    voff[j] = static_cast<uint32_t>(row * (D * 2) + (((lane % FG) ^ (row & (FG - 1))) * 16));
  }
  auto load_tile = [&](int64_t kb, bf16_t* tK, bf16_t* tV) {
    const uint32_t t0 = static_cast<uint32_t>(kb * BK * (D * 2));
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      dq_tile_to_lds16(rK, tK + 512 * (NLD * wave + j), t0 + voff[j]);
      dq_tile_to_lds16(rV, tV + 512 * (NLD * wave + j), t0 + voff[j]);
    }
  };
  const int sw = l32 & (FG - 1);   // chunk swizzle of this lane's fragment rows

  const int64_t nkb = (N + BK - 1) / BK;
  load_tile(0, sK0, sV0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile 0 is in LDS
  __syncthreads();
  // MASKED: the block may hold keys past N (only the last one does); the other
  // steps skip the per-logit key test
  auto step = [&](int64_t kb, const bf16_t* sK, const bf16_t* sV, bf16_t* nK, bf16_t* nV, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    const int64_t k0 = kb * BK;
    if (tid < TSUB) {   // K^T: 4 keys x 8 features per thread
      // keys 4 m .. 4 m + 3 with m = tid mod 16 (16 distinct m per 16 lanes: the
      // transposed 8-byte writes hit distinct slots); the feature group is
      // XOR-ed with lane bits 1-2 so that 8 neighbouring lanes, which share the
      // chunk swizzle of rows 4 m + j two by two, read distinct 16-byte slots
      const int m = tid % (BK / 4);
      const int fg = (tid / (BK / 4)) ^ (((tid >> 1) & 1) | (((tid >> 2) & 1) << 1));
      uint4 r[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 4 * m + j;
        r[j] = *reinterpret_cast<const uint4*>(&sK[row * D + 8 * (fg ^ (row & (FG - 1)))]);
      }
      const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&r[0]);
      const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&r[1]);
      const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&r[2]);
      const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&r[3]);
      const int pos = perm16(4 * m);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        *reinterpret_cast<uint2*>(&sKt[(8 * fg + 2 * p) * TP + pos]) =
            make_uint2(__builtin_amdgcn_perm(r1[p], r0[p], 0x05040100u), __builtin_amdgcn_perm(r3[p], r2[p], 0x05040100u));
        *reinterpret_cast<uint2*>(&sKt[(8 * fg + 2 * p + 1) * TP + pos]) =
            make_uint2(__builtin_amdgcn_perm(r1[p], r0[p], 0x07060302u), __builtin_amdgcn_perm(r3[p], r2[p], 0x07060302u));
      }
    }
    // the next tile loads into the other buffer (last read in the previous step)
    if (kb + 1 < nkb) load_tile(kb + 1, nK, nV);
    dq_barrier();
    // valid keys of this block, less this lane's accumulator row offset 4 h
    const int limh = static_cast<int>(min((int64_t)BK, N - k0)) - 4 * h;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x16 s, dp;
      // dP accumulates onto -D of the lane's query: the MFMAs return dP - D
#pragma unroll
      for (int r = 0; r < 16; ++r) { s[r] = 0.f; dp[r] = -Dq; }
      bf16x8 fk[2], fv[2];
      auto frag = [&](int st, int b) {
        const int off = (32 * t + l32) * D + 8 * ((2 * st + h) ^ sw);
        fk[b] = *reinterpret_cast<const bf16x8*>(&sK[off]);
        fv[b] = *reinterpret_cast<const bf16x8*>(&sV[off]);
      };
      frag(0, 0);
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        if (st + 1 < KS) frag(st + 1, (st + 1) & 1);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fk[st & 1], qf[st], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fv[st & 1], af[st], dp, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(s[r], c, -l2));
        const float p = (!MASKED || 32 * t + 8 * (r >> 2) + (r & 3) < limh) ? e : 0.f;
        ds[r] = p * dp[r];
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        uint4 pk;
        pk.x = pack_bf16(ds[8 * tt + 0], ds[8 * tt + 1]); pk.y = pack_bf16(ds[8 * tt + 2], ds[8 * tt + 3]);
        pk.z = pack_bf16(ds[8 * tt + 4], ds[8 * tt + 5]); pk.w = pack_bf16(ds[8 * tt + 6], ds[8 * tt + 7]);
        const bf16x8 dsf = as_bf16x8(pk);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const bf16x8 kt = *reinterpret_cast<const bf16x8*>(&sKt[(32 * rb + l32) * TP + 32 * t + 16 * tt + 8 * h]);
          dq[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt, dsf, dq[rb], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next tile is in LDS
    dq_barrier();                        // and everyone is done with this one and K^T
  };
  using NoMask = std::integral_constant<bool, false>;
  using Mask = std::integral_constant<bool, true>;
  // blocks 0 .. nfull - 1 hold 64 valid keys; the last steps (at most two,
  // including the ragged block) take the masked body
  const int64_t nfull = N / BK;
  int64_t kb = 0;
  for (; kb + 2 <= nfull; kb += 2) {
    step(kb, sK0, sV0, sK1, sV1, NoMask{});
    step(kb + 1, sK1, sV1, sK0, sV0, NoMask{});
  }
  for (; kb < nkb; kb += 2) {
    step(kb, sK0, sV0, sK1, sV1, Mask{});
    if (kb + 1 < nkb) step(kb + 1, sK1, sV1, sK0, sV0, Mask{});
  }
  if (qrow < N) {
    const float scale = c / kLog2e;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int f0 = 32 * rb + 8 * g4 + 4 * h;
        *reinterpret_cast<uint2*>(dQ + base + qrow * D + f0) =
            make_uint2(pack_bf16(dq[rb][4 * g4 + 0] * scale, dq[rb][4 * g4 + 1] * scale),
                       pack_bf16(dq[rb][4 * g4 + 2] * scale, dq[rb][4 * g4 + 3] * scale));
      }
  }
}

// ------------------------------------------------------------------ bf16 dK, dV
// 8 waves: waves w and w + 4 own the same 32 keys (the block's 128 K and V rows
// sit in LDS for the whole kernel) and take the two 32-query halves of every
// 64-query step, so each SIMD runs two waves; their dK, dV accumulators are
// added once at the end.  Per step: S and dP (queries x keys), then
// dV^T += da^T P and dK^T += Q^T dS.  The next step's Q and da rows are loaded
// into registers during the current step's MFMAs and written to LDS, row-major
// and transposed, straight from those registers.
template <int D>
__global__ __launch_bounds__(512, 1) void sm_bwd_dkv_bf16(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K,
                                                          const bf16_t* __restrict__ V, const bf16_t* __restrict__ da,
                                                          const float* __restrict__ lse, const float* __restrict__ Dv,
                                                          bf16_t* __restrict__ dK, bf16_t* __restrict__ dV, int64_t N,
                                                          int64_t kblocks, float c) {
  constexpr int NT = 512, BQ = 64, BKW = 128;
  constexpr int KP = D + 8, TP = BQ + 8, FG = D / 8;
  constexpr int KCHW = BKW * FG / NT;
  constexpr int KS = D / 16, RB = D / 32;
  constexpr int TSUB = (BQ / 4) * FG;   // 4-query x 8-feature sub-tiles per tensor (<= 256)
  constexpr int OFF_K = 0;
  constexpr int OFF_V = OFF_K + BKW * KP * 2;
  constexpr int OFF_Q = OFF_V + BKW * KP * 2;
  constexpr int OFF_A = OFF_Q + BQ * KP * 2;
  constexpr int OFF_QT = OFF_A + BQ * KP * 2;
  constexpr int OFF_AT = OFF_QT + D * TP * 2;
  constexpr int OFF_L = OFF_AT + D * TP * 2;
  constexpr int OFF_D = OFF_L + BQ * 4;
  constexpr int LDS = OFF_D + BQ * 4;
  static_assert(4 * RB * 16 * 64 * 4 <= LDS, "the pair reduction reuses the tiles' LDS");
  __shared__ __attribute__((aligned(16))) char lds[LDS];
  bf16_t* sKw = reinterpret_cast<bf16_t*>(lds + OFF_K);
  bf16_t* sVw = reinterpret_cast<bf16_t*>(lds + OFF_V);
  bf16_t* sQ = reinterpret_cast<bf16_t*>(lds + OFF_Q);
  bf16_t* sA = reinterpret_cast<bf16_t*>(lds + OFF_A);
  bf16_t* sQt = reinterpret_cast<bf16_t*>(lds + OFF_QT);
  bf16_t* sAt = reinterpret_cast<bf16_t*>(lds + OFF_AT);
  float* sL = reinterpret_cast<float*>(lds + OFF_L);
  float* sD = reinterpret_cast<float*>(lds + OFF_D);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int kw = wave & 3;   // 32-key group
  const int th = wave >> 2;  // 32-query half of each step
  // plain dispatch order: the blocks in flight cover one (b, h) across all
  // XCDs, which measured faster here than one head per XCD (xcd_remap)
  const int64_t id = blockIdx.x;
  const int64_t bh = id / kblocks;
  const int64_t kbase = (id % kblocks) * BKW;
  const int64_t krow = kbase + 32 * kw + l32;
  const int64_t base = bh * N * D;
  const uint32_t head_bytes = static_cast<uint32_t>(N * D * 2);
  const __amdgpu_buffer_rsrc_t rK =
      __builtin_amdgcn_make_buffer_rsrc((void*)(K + base), (short)0, (int)head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rV =
      __builtin_amdgcn_make_buffer_rsrc((void*)(V + base), (short)0, (int)head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rQ =
      __builtin_amdgcn_make_buffer_rsrc((void*)(Q + base), (short)0, (int)head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rA =
      __builtin_amdgcn_make_buffer_rsrc((void*)(da + base), (short)0, (int)head_bytes, 0x00020000);

#pragma unroll
  for (int i = 0; i < KCHW; ++i) {
    const int cidx = tid + NT * i;
    const uint32_t off = static_cast<uint32_t>((kbase + cidx / FG) * (D * 2) + (cidx % FG) * 16);
    *reinterpret_cast<uint4*>(&sKw[(cidx / FG) * KP + 8 * (cidx % FG)]) = buffer_load16(rK, off);
    *reinterpret_cast<uint4*>(&sVw[(cidx / FG) * KP + 8 * (cidx % FG)]) = buffer_load16(rV, off);
  }
  f32x16 dk[RB], dv[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dk[rb][r] = 0.f; dv[rb][r] = 0.f; }

  // each thread stages a sub-tile of the next query step's Q or da rows
  const int sub = tid & 255;
  const bool loader = sub < TSUB;
  // waves 0-3 fetch Q, waves 4-7 da: the choice is taken from a wave-uniform
  // value so that the buffer descriptor stays in scalar registers (chosen per
  // lane, it made the compiler wrap every load in a loop over the distinct
  // descriptors of the wave)
  const bool is_a = __builtin_amdgcn_readfirstlane(wave) >= 4;
  // this thread's sub-tile: 4 query rows 4 sm .. 4 sm + 3, features 8 sfg ..
  // 8 sfg + 7.  LDS writes go 8 lanes (16-byte writes) or 16 lanes (8-byte
  // writes) at a time with banks repeating every 128 bytes; 16-byte reads see
  // a wider window (a column swizzle of the transposed tile, conflict-free for
  // 16-lane groups, made its reads conflict).  Lane l = b0 .. b5 of the
  // tensor's wave w' takes sm = l mod 16 and sfg = (b1 ^ b4) + 2 (b2 ^ b5) + 4 w':
  //  * transposed writes: any 16 neighbouring lanes hold 16 distinct sm, i.e.
  //    16 distinct 8-byte slots of the feature row (the row pitch is a
  //    multiple of 16 bytes, so sfg does not move the slot);
  //  * row-major writes: row 4 sm + j, chunk sfg lands on 16-byte slot
  //    (4 sm + j + sfg) mod 8 (the row pitch is 16 bytes past a multiple of 128),
  //    and over any 8 neighbouring lanes 4 b0 + (b1 ^ b4) + 2 (b2 ^ b5) takes all
  //    8 values;
  //  * a wave still reads 64 contiguous bytes of each of 16 rows per load.
  // Both kinds of commit write are then conflict-free, and the tiles keep the
  // layout their readers expect.  (The previous map, 8 sm x 2 sfg per 16 lanes
  // with half the threads' rows rotated, had both kinds collide two ways: half
  // of the commit's LDS cycles were bank conflicts.)
  const int ll = sub & 63;
  const int sm = ll & 15;
  const int sfg = (((ll >> 1) ^ (ll >> 4)) & 1) | ((((ll >> 2) ^ (ll >> 5)) & 1) << 1) | (4 * (sub >> 6));
  const __amdgpu_buffer_rsrc_t rsrc = is_a ? rA : rQ;
  bf16_t* dst_row = is_a ? sA : sQ;
  bf16_t* dst_t = is_a ? sAt : sQt;
  // rows 4 sm .. 4 sm + 3: one lane offset, the step in the scalar offset
  const int offA = 4 * sm * (D * 2) + sfg * 16;
  bf16_t* rowA = dst_row + 4 * sm * KP + 8 * sfg;
  uint4 pre[4];
  // lse and D of the next step's queries, as loaded: they are first used at the
  // commit, so the loads stay in flight during the step's MFMAs (scaling lse
  // right after its load made the compiler wait there for all of the wave's
  // loads of the step, the Q/da rows included).  Past N they read as 0.
  float preL = 0.f, preD = 0.f;
  int preQ = 0;
  const __amdgpu_buffer_rsrc_t rL =
      __builtin_amdgcn_make_buffer_rsrc((void*)(lse + bh * N), (short)0, (int)(N * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t rD =
      __builtin_amdgcn_make_buffer_rsrc((void*)(Dv + bh * N), (short)0, (int)(N * 4), 0x00020000);
  auto fetch = [&](int64_t q0) {
    if (loader) {
      const int soff = static_cast<int>(q0 * (D * 2));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pre[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, offA + j * (D * 2), soff, 0));
    }
    if (tid < BQ) {
      preQ = static_cast<int>(q0) + tid;
      preL = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rL, preQ * 4, 0, 0));
      preD = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rD, preQ * 4, 0, 0));
    }
  };
  auto commit = [&]() {
    if (loader) {
      const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&pre[0]);
      const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&pre[1]);
      const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&pre[2]);
      const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&pre[3]);
      const int pos = perm16(4 * sm);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        *reinterpret_cast<uint2*>(&dst_t[(8 * sfg + 2 * p) * TP + pos]) =
            make_uint2(__builtin_amdgcn_perm(r1[p], r0[p], 0x05040100u), __builtin_amdgcn_perm(r3[p], r2[p], 0x05040100u));
        *reinterpret_cast<uint2*>(&dst_t[(8 * sfg + 2 * p + 1) * TP + pos]) =
            make_uint2(__builtin_amdgcn_perm(r1[p], r0[p], 0x07060302u), __builtin_amdgcn_perm(r3[p], r2[p], 0x07060302u));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4*>(rowA + j * KP) = pre[j];
    }
    if (tid < BQ) {
      // a query past N contributes nothing: P = exp2(s c - inf) = 0
      sL[tid] = preQ < N ? preL * kLog2e : INFINITY;
      sD[tid] = -preD;
    }
  };

  // column of this lane's transposed-tile fragments: queries 32 th + 8 h
  const int tcol = 32 * th + 8 * h;
  const int64_t nqb = (N + BQ - 1) / BQ;
  fetch(0);
  for (int64_t qb = 0; qb < nqb; ++qb) {
    __syncthreads();   // every wave is done with the previous step's tiles
    commit();
    __syncthreads();
    fetch((qb + 1 < nqb ? qb + 1 : qb) * BQ);   // in flight during the MFMAs
    const int t = th;
    f32x16 s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
    // dP accumulates onto -D of its rows (sD holds -D), so the MFMAs return
    // dP - D and dS needs one multiply per element
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 D4 = *reinterpret_cast<const float4*>(&sD[32 * t + 8 * g + 4 * h]);
      dp[4 * g + 0] = D4.x; dp[4 * g + 1] = D4.y; dp[4 * g + 2] = D4.z; dp[4 * g + 3] = D4.w;
    }
    // S and dP with each k-slice's fragments read one slice ahead
    bf16x8 fq[2], fa[2], fk[2], fv[2];
    auto frag = [&](int st, int b) {
      fq[b] = *reinterpret_cast<const bf16x8*>(&sQ[(32 * t + l32) * KP + 16 * st + 8 * h]);
      fa[b] = *reinterpret_cast<const bf16x8*>(&sA[(32 * t + l32) * KP + 16 * st + 8 * h]);
      fk[b] = *reinterpret_cast<const bf16x8*>(&sKw[(32 * kw + l32) * KP + 16 * st + 8 * h]);
      fv[b] = *reinterpret_cast<const bf16x8*>(&sVw[(32 * kw + l32) * KP + 16 * st + 8 * h]);
    };
    frag(0, 0);
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      if (st + 1 < KS) frag(st + 1, (st + 1) & 1);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fq[st & 1], fk[st & 1], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[st & 1], fv[st & 1], dp, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    float p[16], ds[16];
    auto probs = [&](int g) {  // P and dS of accumulator rows 4 g .. 4 g + 3
      const float4 L4 = *reinterpret_cast<const float4*>(&sL[32 * t + 8 * g + 4 * h]);
      const float Lr[4] = {L4.x, L4.y, L4.z, L4.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * g + j;
        p[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c, -Lr[j]));
        ds[r] = p[r] * dp[r];
      }
    };
    // the second half's P and dS are computed in the shadow of the first
    // half's dV/dK MFMAs (pinned there by the empty asm statements)
    probs(0);
    probs(1);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      uint4 pk, dk4;
      pk.x = pack_bf16(p[8 * tt + 0], p[8 * tt + 1]); pk.y = pack_bf16(p[8 * tt + 2], p[8 * tt + 3]);
      pk.z = pack_bf16(p[8 * tt + 4], p[8 * tt + 5]); pk.w = pack_bf16(p[8 * tt + 6], p[8 * tt + 7]);
      dk4.x = pack_bf16(ds[8 * tt + 0], ds[8 * tt + 1]); dk4.y = pack_bf16(ds[8 * tt + 2], ds[8 * tt + 3]);
      dk4.z = pack_bf16(ds[8 * tt + 4], ds[8 * tt + 5]); dk4.w = pack_bf16(ds[8 * tt + 6], ds[8 * tt + 7]);
      const bf16x8 pf = as_bf16x8(pk), dsf = as_bf16x8(dk4);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const bf16x8 at = *reinterpret_cast<const bf16x8*>(&sAt[(32 * rb + l32) * TP + tcol + 16 * tt]);
        const bf16x8 qt = *reinterpret_cast<const bf16x8*>(&sQt[(32 * rb + l32) * TP + tcol + 16 * tt]);
        dv[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(at, pf, dv[rb], 0, 0, 0);
        dk[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qt, dsf, dk[rb], 0, 0, 0);
        if (tt == 0 && rb < 2) {
          probs(2 + rb);
#pragma unroll
          for (int u = 0; u < 4; ++u) asm volatile("" : "+v"(p[8 + 4 * rb + u]), "+v"(ds[8 + 4 * rb + u]));
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }
  // add the two halves' accumulators: waves 4..7 hand theirs to waves 0..3
  // through LDS (the tiles are no longer needed), dK then dV
  float* red = reinterpret_cast<float*>(lds);
  const float scale = c / kLog2e;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    __syncthreads();
    if (th == 1)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[((kw * RB + rb) * 16 + r) * 64 + lane] = which == 0 ? dk[rb][r] : dv[rb][r];
    __syncthreads();
    if (th == 0 && krow < N) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          float v[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 4 * g4 + j;
            const float own = which == 0 ? dk[rb][r] : dv[rb][r];
            v[j] = (own + red[((kw * RB + rb) * 16 + r) * 64 + lane]) * (which == 0 ? scale : 1.f);
          }
          const int f0 = 32 * rb + 8 * g4 + 4 * h;
          *reinterpret_cast<uint2*>((which == 0 ? dK : dV) + base + krow * D + f0) =
              make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
        }
    }
  }
}

// ------------------------------------------------------------------ float32
// Plain VALU versions: a row (query for dQ, key for dK/dV) is split over
// D / 16 consecutive lanes, 16 features each; dot products are reduced over
// those lanes.  The other side's rows are read through the caches.
template <int D>
__global__ __launch_bounds__(256) void sm_bwd_dq_f32(const float* __restrict__ Q, const float* __restrict__ K,
                                                     const float* __restrict__ V, const float* __restrict__ da,
                                                     const float* __restrict__ lse, const float* __restrict__ Dv,
                                                     float* __restrict__ dQ, int64_t N, int64_t total_rows,
                                                     float scale) {
  constexpr int FS = D / 16;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  // lanes past the last row still run the loop (for the shuffles) on row 0
  const bool ok = e / FS < total_rows;
  const int64_t row = ok ? e / FS : 0;
  const int64_t bh = row / N, qi = row % N;
  const int sl = static_cast<int>(e % FS);
  const int64_t base = bh * N * D;
  float q[16], a[16], acc[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    q[k] = ok ? Q[base + qi * D + 16 * sl + k] : 0.f;
    a[k] = ok ? da[base + qi * D + 16 * sl + k] : 0.f;
    acc[k] = 0.f;
  }
  const float L = ok ? lse[bh * N + qi] : 0.f;
  const float Dq = ok ? Dv[bh * N + qi] : 0.f;
  for (int64_t j = 0; j < N; ++j) {
    const float* kr = K + base + j * D + 16 * sl;
    const float* vr = V + base + j * D + 16 * sl;
    float sp = 0.f, dp = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      sp = fmaf(q[k], kr[k], sp);
      dp = fmaf(a[k], vr[k], dp);
    }
#pragma unroll
    for (int m = 1; m < FS; m <<= 1) {
      sp += __shfl_xor(sp, m);
      dp += __shfl_xor(dp, m);
    }
    const float ds = expf(sp * scale - L) * (dp - Dq);
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] = fmaf(ds, kr[k], acc[k]);
  }
  if (ok)
#pragma unroll
    for (int k = 0; k < 16; ++k) dQ[base + qi * D + 16 * sl + k] = acc[k] * scale;
}

template <int D>
__global__ __launch_bounds__(256) void sm_bwd_dkv_f32(const float* __restrict__ Q, const float* __restrict__ K,
                                                      const float* __restrict__ V, const float* __restrict__ da,
                                                      const float* __restrict__ lse, const float* __restrict__ Dv,
                                                      float* __restrict__ dK, float* __restrict__ dV, int64_t N,
                                                      int64_t total_rows, float scale) {
  constexpr int FS = D / 16;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const bool ok = e / FS < total_rows;
  const int64_t row = ok ? e / FS : 0;
  const int64_t bh = row / N, kj = row % N;
  const int sl = static_cast<int>(e % FS);
  const int64_t base = bh * N * D;
  float kk[16], vv[16], ak[16], av[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    kk[k] = ok ? K[base + kj * D + 16 * sl + k] : 0.f;
    vv[k] = ok ? V[base + kj * D + 16 * sl + k] : 0.f;
    ak[k] = 0.f;
    av[k] = 0.f;
  }
  for (int64_t i = 0; i < N; ++i) {
    const float* qr = Q + base + i * D + 16 * sl;
    const float* ar = da + base + i * D + 16 * sl;
    float sp = 0.f, dp = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      sp = fmaf(qr[k], kk[k], sp);
      dp = fmaf(ar[k], vv[k], dp);
    }
#pragma unroll
    for (int m = 1; m < FS; m <<= 1) {
      sp += __shfl_xor(sp, m);
      dp += __shfl_xor(dp, m);
    }
    const float p = expf(sp * scale - lse[bh * N + i]);
    const float ds = p * (dp - Dv[bh * N + i]);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      av[k] = fmaf(p, ar[k], av[k]);
      ak[k] = fmaf(ds, qr[k], ak[k]);
    }
  }
  if (ok)
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      dK[base + kj * D + 16 * sl + k] = ak[k] * scale;
      dV[base + kj * D + 16 * sl + k] = av[k];
    }
}

template <typename T>
hipError_t launch_pre(int d, const void* O, const void* dO, const void* G, void* dG, void* da, float* Dv,
                      int64_t rows, hipStream_t s) {
  const int64_t threads = rows * (d / 8);
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256)), block(256);
  auto go = [&](auto kern) {
    kern<<<grid, block, 0, s>>>(static_cast<const T*>(O), static_cast<const T*>(dO), static_cast<const T*>(G),
                                static_cast<T*>(dG), static_cast<T*>(da), Dv, rows);
  };
  if (d == 128)
    go(sm_bwd_pre<T, 128>);
  else
    go(sm_bwd_pre<T, 64>);
  return hipGetLastError();
}

}  // namespace

size_t softmax_bwd_ws(int64_t BH, int64_t N, int d, bool bf16) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  return up(static_cast<size_t>(BH) * N * d * (bf16 ? 2u : 4u)) + up(static_cast<size_t>(BH) * N * sizeof(float));
}

hipError_t launch_softmax_backward(bool bf16, int d, const void* Q, const void* K, const void* V,
                                   const void* G, const void* O, const void* dO, const float* lse,
                                   void* dQ, void* dK, void* dV, void* dG, int64_t BH, int64_t N,
                                   void* ws, hipStream_t s) {
  if (BH == 0 || N == 0) return hipSuccess;
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  char* w = static_cast<char*>(ws);
  void* da = w;
  float* Dv = reinterpret_cast<float*>(w + up(static_cast<size_t>(BH) * N * d * (bf16 ? 2u : 4u)));
  hipError_t e = bf16 ? launch_pre<bf16_t>(d, O, dO, G, dG, da, Dv, BH * N, s)
                      : launch_pre<float>(d, O, dO, G, dG, da, Dv, BH * N, s);
  if (e != hipSuccess) return e;
  const float c = kLog2e / sqrtf(static_cast<float>(d));
  if (bf16) {
    const bf16_t* q = static_cast<const bf16_t*>(Q);
    const bf16_t* k = static_cast<const bf16_t*>(K);
    const bf16_t* v = static_cast<const bf16_t*>(V);
    const bf16_t* a = static_cast<const bf16_t*>(da);
    const int64_t qb = (N + 255) / 256, tq = BH * qb;
    const int64_t kb = (N + 127) / 128, tk = BH * kb;
    if (d == 128) {
      sm_bwd_dq_bf16<128><<<dim3(static_cast<unsigned>(tq)), dim3(512), 0, s>>>(q, k, v, a, lse, Dv,
                                                                                 static_cast<bf16_t*>(dQ), N, qb, c);
      sm_bwd_dkv_bf16<128><<<dim3(static_cast<unsigned>(tk)), dim3(512), 0, s>>>(
          q, k, v, a, lse, Dv, static_cast<bf16_t*>(dK), static_cast<bf16_t*>(dV), N, kb, c);
    } else {
      sm_bwd_dq_bf16<64><<<dim3(static_cast<unsigned>(tq)), dim3(512), 0, s>>>(q, k, v, a, lse, Dv,
                                                                                static_cast<bf16_t*>(dQ), N, qb, c);
      sm_bwd_dkv_bf16<64><<<dim3(static_cast<unsigned>(tk)), dim3(512), 0, s>>>(
          q, k, v, a, lse, Dv, static_cast<bf16_t*>(dK), static_cast<bf16_t*>(dV), N, kb, c);
    }
  } else {
    const float* q = static_cast<const float*>(Q);
    const float* k = static_cast<const float*>(K);
    const float* v = static_cast<const float*>(V);
    const float* a = static_cast<const float*>(da);
    const float scale = 1.0f / sqrtf(static_cast<float>(d));
    const int64_t threads = BH * N * (d / 16);
    const dim3 grid(static_cast<unsigned>((threads + 255) / 256)), block(256);
    if (d == 128) {
      sm_bwd_dq_f32<128><<<grid, block, 0, s>>>(q, k, v, a, lse, Dv, static_cast<float*>(dQ), N, BH * N, scale);
      sm_bwd_dkv_f32<128><<<grid, block, 0, s>>>(q, k, v, a, lse, Dv, static_cast<float*>(dK),
                                                 static_cast<float*>(dV), N, BH * N, scale);
    } else {
      sm_bwd_dq_f32<64><<<grid, block, 0, s>>>(q, k, v, a, lse, Dv, static_cast<float*>(dQ), N, BH * N, scale);
      sm_bwd_dkv_f32<64><<<grid, block, 0, s>>>(q, k, v, a, lse, Dv, static_cast<float*>(dK),
                                                static_cast<float*>(dV), N, BH * N, scale);
    }
  }
  return hipGetLastError();
}

}  // namespace ha
