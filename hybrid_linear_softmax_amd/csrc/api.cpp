// C ABI of libhybrid_attn.so: argument validation (host only, before any HIP
// call) and the launch sequence of each entry point.
#include <stdint.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "../../include/ha_probe.h"
#include "../../include/hybrid_attn.h"
#include "ha_launch.h"

namespace {

struct Problem {
  int64_t B, H, N, d, BH;
  bool bf16;
  size_t tensor_bytes;  // bytes of one [B, H, N, d] tensor
};

int check_shape(int B, int H, int64_t N, int d, int dtype, Problem* p) {
  if (dtype != HA_BF16 && dtype != HA_F32) return HA_EUNSUPPORTED;
  if (d != 64 && d != 128) return HA_EUNSUPPORTED;
  if (B < 0 || H < 0 || N < 0) return HA_EINVAL;
  if (N > HA_MAX_N) return HA_EINVAL;
  const int64_t BH = static_cast<int64_t>(B) * H;
  if (BH > HA_MAX_BH) return HA_EINVAL;
  p->B = B;
  p->H = H;
  p->N = N;
  p->d = d;
  p->BH = BH;
  p->bf16 = dtype == HA_BF16;
  p->tensor_bytes = static_cast<size_t>(BH) * static_cast<size_t>(N) * static_cast<size_t>(d) *
                    (p->bf16 ? 2u : 4u);
  return HA_OK;
}

bool misaligned(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) != 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Null, alignment and aliasing checks of n_in inputs and one output.
int check_buffers(const void* const* in, int n_in, size_t in_bytes, const void* out,
                  size_t out_bytes) {
  for (int i = 0; i < n_in; ++i)
    if (in[i] == nullptr) return HA_EINVAL;
  if (out == nullptr) return HA_EINVAL;
  for (int i = 0; i < n_in; ++i)
    if (misaligned(in[i])) return HA_EALIGN;
  if (misaligned(out)) return HA_EALIGN;
  for (int i = 0; i < n_in; ++i)
    if (overlaps(in[i], in_bytes, out, out_bytes)) return HA_EINVAL;
  return HA_OK;
}

// The linear layer's workspace: present, large enough, aligned, and disjoint
// from the n tensors of the call (t[i] spanning t_bytes[i] bytes).
int check_workspace(const Problem& p, const void* ws, size_t ws_bytes, const void* const* t,
                    const size_t* t_bytes, int n) {
  const size_t need = ha::linear_ws(p.BH, p.N, static_cast<int>(p.d), p.bf16).total;
  if (ws == nullptr || ws_bytes < need) return HA_EWORKSPACE;
  if (misaligned(ws)) return HA_EALIGN;
  for (int i = 0; i < n; ++i)
    if (overlaps(ws, need, t[i], t_bytes[i])) return HA_EINVAL;
  return HA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? HA_OK : HA_EHIP; }

// One linear layer on validated arguments.  events (optional, four): recorded
// before pass 1 of the state reduction, after it, after pass 2, after the apply.
int run_linear(const Problem& p, const void* Q, const void* K, const void* V, const void* G,
               void* O, void* ws, hipStream_t s, hipEvent_t const* events = nullptr) {
  auto mark = [&](int i) { return events == nullptr || hipEventRecord(events[i], s) == hipSuccess; };
  const int d = static_cast<int>(p.d);
  const ha::LinearWs L = ha::linear_ws(p.BH, p.N, d, p.bf16);
  char* w = static_cast<char*>(ws);
  float* part = reinterpret_cast<float*>(w + L.part);
  float* S = reinterpret_cast<float*>(w + L.S);
  float* z = reinterpret_cast<float*>(w + L.z);
  uint16_t* hi = reinterpret_cast<uint16_t*>(w + L.St_hi);
  uint16_t* lo = reinterpret_cast<uint16_t*>(w + L.St_lo);
  const ha::KvSplit sp = ha::kv_split(p.BH, p.N);
  if (!mark(0)) return HA_EHIP;
  hipError_t e = ha::launch_kv_partials(p.bf16, d, K, V, part, p.BH, p.N, sp, s);
  if (e != hipSuccess || !mark(1)) return HA_EHIP;
  e = ha::launch_kv_reduce(p.bf16, d, part, S, z, hi, lo, p.BH, sp.chunks, s);
  if (e != hipSuccess || !mark(2)) return HA_EHIP;
  e = ha::launch_apply(p.bf16, d, Q, G, O, S, z, hi, lo, p.BH, p.N, HA_LINEAR_EPS, s);
  if (e != hipSuccess || !mark(3)) return HA_EHIP;
  return HA_OK;
}

// Null, alignment and aliasing checks of inputs and outputs of different
// sizes: no output may overlap an input or another output.
int check_io(const void* const* in, const size_t* in_bytes, int n_in, void* const* out,
             const size_t* out_bytes, int n_out) {
  for (int i = 0; i < n_in; ++i)
    if (in[i] == nullptr) return HA_EINVAL;
  for (int i = 0; i < n_out; ++i)
    if (out[i] == nullptr) return HA_EINVAL;
  for (int i = 0; i < n_in; ++i)
    if (misaligned(in[i])) return HA_EALIGN;
  for (int i = 0; i < n_out; ++i)
    if (misaligned(out[i])) return HA_EALIGN;
  for (int j = 0; j < n_out; ++j) {
    for (int i = 0; i < n_in; ++i)
      if (overlaps(in[i], in_bytes[i], out[j], out_bytes[j])) return HA_EINVAL;
    for (int i = 0; i < j; ++i)
      if (overlaps(out[i], out_bytes[i], out[j], out_bytes[j])) return HA_EINVAL;
  }
  return HA_OK;
}

// Device workspace of the attention block: Q, K, V, G, O of one sub-layer,
// then the linear layer's workspace (256-byte aligned pieces).
struct BlockWs {
  size_t q, k, v, g, o, lin, lin_bytes, total;
};

BlockWs block_ws(const Problem& p) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  BlockWs w{};
  size_t off = 0;
  w.q = off;
  off += up(p.tensor_bytes);
  w.k = off;
  off += up(p.tensor_bytes);
  w.v = off;
  off += up(p.tensor_bytes);
  w.g = off;
  off += up(p.tensor_bytes);
  w.o = off;
  off += up(p.tensor_bytes);
  w.lin = off;
  w.lin_bytes = ha::linear_ws(p.BH, p.N, static_cast<int>(p.d), p.bf16).total;
  off += w.lin_bytes;
  w.total = off;
  return w;
}

size_t weight_bytes(const Problem& p, int64_t rows) {
  const int64_t C = p.H * p.d;
  return static_cast<size_t>(rows) * static_cast<size_t>(C) * (p.bf16 ? 2u : 4u);
}

}  // namespace

namespace ha {

LinearWs linear_ws(int64_t BH, int64_t N, int d, bool bf16) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  const KvSplit sp = kv_split(BH, N);
  const size_t dd = static_cast<size_t>(d) * d;
  LinearWs L{};
  size_t off = 0;
  L.part = off;
  off += up(static_cast<size_t>(BH) * sp.chunks * (dd + d) * sizeof(float));
  L.S = off;
  off += up(static_cast<size_t>(BH) * dd * sizeof(float));
  L.z = off;
  off += up(static_cast<size_t>(BH) * d * sizeof(float));
  L.St_hi = off;
  if (bf16) off += up(static_cast<size_t>(BH) * dd * sizeof(uint16_t));
  L.St_lo = off;
  if (bf16) off += up(static_cast<size_t>(BH) * dd * sizeof(uint16_t));
  L.total = off;
  return L;
}

}  // namespace ha

extern "C" {

HA_API const char* hybrid_attn_strerror(int status) {
  switch (status) {
    case HA_OK: return "success";
    case HA_EINVAL: return "invalid argument (size, null pointer, or an output or workspace overlapping another buffer)";
    case HA_EUNSUPPORTED: return "unsupported head dimension or dtype (d must be 64 or 128; dtype bf16 or f32)";
    case HA_EALIGN: return "pointer not 16-byte aligned";
    case HA_EWORKSPACE: return "workspace missing or smaller than hybrid_attn_workspace_bytes()";
    case HA_EHIP: return "HIP kernel launch or event record failed";
    default: return "unknown status";
  }
}

HA_API size_t hybrid_attn_workspace_bytes(int B, int H, int64_t N, int d, ha_dtype dtype) {
  Problem p;
  if (check_shape(B, H, N, d, dtype, &p) != HA_OK || p.BH == 0) return 0;
  return ha::linear_ws(p.BH, p.N, d, p.bf16).total;
}

HA_API int hybrid_attn_kv_state(const void* K, const void* V, float* S, float* z, int B, int H,
                                int64_t N, int d, ha_dtype dtype, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  Problem p;
  int st = check_shape(B, H, N, d, dtype, &p);
  if (st != HA_OK) return st;
  if (p.BH == 0) return HA_OK;
  const size_t s_bytes = static_cast<size_t>(p.BH) * d * d * sizeof(float);
  const size_t z_bytes = static_cast<size_t>(p.BH) * d * sizeof(float);
  if (S == nullptr || z == nullptr) return HA_EINVAL;
  if (p.N > 0) {
    const void* in[2] = {K, V};
    st = check_buffers(in, 2, p.tensor_bytes, S, s_bytes);
    if (st != HA_OK) return st;
    st = check_buffers(in, 2, p.tensor_bytes, z, z_bytes);
    if (st != HA_OK) return st;
  } else if (misaligned(S) || misaligned(z)) {
    return HA_EALIGN;
  }
  if (overlaps(S, s_bytes, z, z_bytes)) return HA_EINVAL;
  {
    const void* t[4] = {K, V, S, z};
    const size_t tb[4] = {p.tensor_bytes, p.tensor_bytes, s_bytes, z_bytes};
    st = check_workspace(p, workspace, workspace_bytes, t, tb, 4);
    if (st != HA_OK) return st;
  }

  const ha::LinearWs L = ha::linear_ws(p.BH, p.N, d, p.bf16);
  char* w = static_cast<char*>(workspace);
  float* part = reinterpret_cast<float*>(w + L.part);
  const ha::KvSplit sp = ha::kv_split(p.BH, p.N);
  hipError_t e = ha::launch_kv_partials(p.bf16, d, K, V, part, p.BH, p.N, sp, stream);
  if (e != hipSuccess) return HA_EHIP;
  // the exported state is float32 only: no bf16 split needed here
  e = ha::launch_kv_reduce(false, d, part, S, z, nullptr, nullptr, p.BH, sp.chunks, stream);
  return hip_status(e);
}

HA_API int hybrid_attn_linear(const void* Q, const void* K, const void* V, const void* G, void* O,
                              int B, int H, int64_t N, int d, ha_dtype dtype, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  Problem p;
  int st = check_shape(B, H, N, d, dtype, &p);
  if (st != HA_OK) return st;
  if (p.BH == 0 || p.N == 0) return HA_OK;
  const void* in[4] = {Q, K, V, G};
  st = check_buffers(in, 4, p.tensor_bytes, O, p.tensor_bytes);
  if (st != HA_OK) return st;
  const void* t[5] = {Q, K, V, G, O};
  const size_t tb[5] = {p.tensor_bytes, p.tensor_bytes, p.tensor_bytes, p.tensor_bytes, p.tensor_bytes};
  st = check_workspace(p, workspace, workspace_bytes, t, tb, 5);
  if (st != HA_OK) return st;
  return run_linear(p, Q, K, V, G, O, workspace, stream);
}

HA_API int hybrid_attn_linear_timed(const void* Q, const void* K, const void* V, const void* G, void* O,
                                    int B, int H, int64_t N, int d, ha_dtype dtype, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream, hipEvent_t const events[4]) {
  if (events == nullptr) return HA_EINVAL;
  for (int i = 0; i < 4; ++i)
    if (events[i] == nullptr) return HA_EINVAL;
  Problem p;
  int st = check_shape(B, H, N, d, dtype, &p);
  if (st != HA_OK) return st;
  if (p.BH == 0 || p.N == 0) return HA_OK;
  const void* in[4] = {Q, K, V, G};
  st = check_buffers(in, 4, p.tensor_bytes, O, p.tensor_bytes);
  if (st != HA_OK) return st;
  const void* t[5] = {Q, K, V, G, O};
  const size_t tb[5] = {p.tensor_bytes, p.tensor_bytes, p.tensor_bytes, p.tensor_bytes, p.tensor_bytes};
  st = check_workspace(p, workspace, workspace_bytes, t, tb, 5);
  if (st != HA_OK) return st;
  return run_linear(p, Q, K, V, G, O, workspace, stream, events);
}

HA_API int hybrid_attn_softmax(const void* Q, const void* K, const void* V, const void* G, void* O,
                               int B, int H, int64_t N, int d, ha_dtype dtype, hipStream_t stream) {
  Problem p;
  int st = check_shape(B, H, N, d, dtype, &p);
  if (st != HA_OK) return st;
  if (p.BH == 0 || p.N == 0) return HA_OK;
  const void* in[4] = {Q, K, V, G};
  st = check_buffers(in, 4, p.tensor_bytes, O, p.tensor_bytes);
  if (st != HA_OK) return st;
  return hip_status(ha::launch_anchor(p.bf16, d, Q, K, V, G, O, p.BH, p.N, stream));
}

HA_API int hybrid_attn_softmax_blocksparse(const void* Q, const void* K, const void* V, const void* G,
                                           void* O, int B, int H, int64_t N, int d, ha_dtype dtype,
                                           const int32_t* block_offsets, const int32_t* block_indices,
                                           int64_t num_indices, hipStream_t stream) {
  static_assert(HA_SPARSE_BLOCK_Q == ha::kSparseBlockQ && HA_SPARSE_BLOCK_K == ha::kSparseBlockK,
                "pattern block sizes");
  Problem p;
  int st = check_shape(B, H, N, d, dtype, &p);
  if (st != HA_OK) return st;
  if (p.BH == 0 || p.N == 0) return HA_OK;
  const void* in[4] = {Q, K, V, G};
  st = check_buffers(in, 4, p.tensor_bytes, O, p.tensor_bytes);
  if (st != HA_OK) return st;
  // list positions are 32-bit byte offsets inside the kernel: fewer than 2^30 entries
  if (block_offsets == nullptr || num_indices < 0 || num_indices >= (int64_t{1} << 30)) return HA_EINVAL;
  if (block_indices == nullptr && num_indices > 0) return HA_EINVAL;
  if ((reinterpret_cast<uintptr_t>(block_offsets) & 3u) || (reinterpret_cast<uintptr_t>(block_indices) & 3u))
    return HA_EALIGN;
  const size_t off_bytes = static_cast<size_t>((p.N + HA_SPARSE_BLOCK_Q - 1) / HA_SPARSE_BLOCK_Q + 1) * 4u;
  if (overlaps(block_offsets, off_bytes, O, p.tensor_bytes) ||
      (num_indices > 0 && overlaps(block_indices, static_cast<size_t>(num_indices) * 4u, O, p.tensor_bytes)))
    return HA_EINVAL;
  return hip_status(ha::launch_anchor(p.bf16, d, Q, K, V, G, O, p.BH, p.N, stream, block_offsets,
                                      block_indices, num_indices));
}

HA_API int hybrid_attn_group_timed(const void* Q4, const void* K4, const void* V4, const void* G4,
                                   void* O4, int B, int H, int64_t N, int d, ha_dtype dtype,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream,
                                   hipEvent_t const events[5]) {
  Problem p;
  int st = check_shape(B, H, N, d, dtype, &p);
  if (st != HA_OK) return st;
  if (events != nullptr)
    for (int i = 0; i < 5; ++i)
      if (events[i] == nullptr) return HA_EINVAL;
  if (p.BH == 0 || p.N == 0) return HA_OK;
  const size_t group_bytes = 4 * p.tensor_bytes;
  const void* in[4] = {Q4, K4, V4, G4};
  st = check_buffers(in, 4, group_bytes, O4, group_bytes);
  if (st != HA_OK) return st;
  const void* t[5] = {Q4, K4, V4, G4, O4};
  const size_t tb[5] = {group_bytes, group_bytes, group_bytes, group_bytes, group_bytes};
  st = check_workspace(p, workspace, workspace_bytes, t, tb, 5);
  if (st != HA_OK) return st;

  int kinds[4];
  hybrid_attn_group_schedule(kinds);
  if (events != nullptr && hipEventRecord(events[0], stream) != hipSuccess) return HA_EHIP;
  for (int l = 0; l < 4; ++l) {
    const size_t off = static_cast<size_t>(l) * p.tensor_bytes;
    const char* q = static_cast<const char*>(Q4) + off;
    const char* k = static_cast<const char*>(K4) + off;
    const char* v = static_cast<const char*>(V4) + off;
    const char* g = static_cast<const char*>(G4) + off;
    char* o = static_cast<char*>(O4) + off;
    if (kinds[l] == 0)
      st = run_linear(p, q, k, v, g, o, workspace, stream);
    else
      st = hip_status(ha::launch_anchor(p.bf16, d, q, k, v, g, o, p.BH, p.N, stream));
    if (st != HA_OK) return st;
    if (events != nullptr && hipEventRecord(events[l + 1], stream) != hipSuccess) return HA_EHIP;
  }
  return HA_OK;
}

HA_API int hybrid_attn_group(const void* Q4, const void* K4, const void* V4, const void* G4, void* O4,
                             int B, int H, int64_t N, int d, ha_dtype dtype, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  return hybrid_attn_group_timed(Q4, K4, V4, G4, O4, B, H, N, d, dtype, workspace, workspace_bytes,
                                 stream, nullptr);
}

HA_API size_t hybrid_attn_linear_backward_workspace_bytes(int B, int H, int64_t N, int d, ha_dtype dtype) {
  Problem p;
  if (check_shape(B, H, N, d, dtype, &p) != HA_OK || p.BH == 0) return 0;
  return ha::linear_bwd_ws(p.BH, p.N, d, p.bf16).total;
}

HA_API int hybrid_attn_linear_backward(const void* Q, const void* K, const void* V, const void* G,
                                       const void* dO, void* dQ, void* dK, void* dV, void* dG, int B,
                                       int H, int64_t N, int d, ha_dtype dtype, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  Problem p;
  int st = check_shape(B, H, N, d, dtype, &p);
  if (st != HA_OK) return st;
  if (p.BH == 0 || p.N == 0) return HA_OK;
  const void* in[5] = {Q, K, V, G, dO};
  const size_t in_bytes[5] = {p.tensor_bytes, p.tensor_bytes, p.tensor_bytes, p.tensor_bytes, p.tensor_bytes};
  void* out[4] = {dQ, dK, dV, dG};
  const size_t out_bytes[4] = {p.tensor_bytes, p.tensor_bytes, p.tensor_bytes, p.tensor_bytes};
  st = check_io(in, in_bytes, 5, out, out_bytes, 4);
  if (st != HA_OK) return st;
  const size_t need = ha::linear_bwd_ws(p.BH, p.N, d, p.bf16).total;
  if (workspace == nullptr || workspace_bytes < need) return HA_EWORKSPACE;
  if (misaligned(workspace)) return HA_EALIGN;
  for (int i = 0; i < 5; ++i)
    if (overlaps(workspace, need, in[i], in_bytes[i])) return HA_EINVAL;
  for (int i = 0; i < 4; ++i)
    if (overlaps(workspace, need, out[i], out_bytes[i])) return HA_EINVAL;
  return hip_status(ha::launch_linear_backward(p.bf16, d, Q, K, V, G, dO, dQ, dK, dV, dG, p.BH, p.N,
                                               HA_LINEAR_EPS, workspace, stream));
}

HA_API int hybrid_attn_softmax_lse(const void* Q, const void* K, const void* V, const void* G, void* O,
                                   float* lse, int B, int H, int64_t N, int d, ha_dtype dtype,
                                   hipStream_t stream) {
  Problem p;
  int st = check_shape(B, H, N, d, dtype, &p);
  if (st != HA_OK) return st;
  if (p.BH == 0 || p.N == 0) return HA_OK;
  const void* in[4] = {Q, K, V, G};
  const size_t in_bytes[4] = {p.tensor_bytes, p.tensor_bytes, p.tensor_bytes, p.tensor_bytes};
  void* out[2] = {O, lse};
  const size_t out_bytes[2] = {p.tensor_bytes, static_cast<size_t>(p.BH) * p.N * sizeof(float)};
  st = check_io(in, in_bytes, 4, out, out_bytes, 2);
  if (st != HA_OK) return st;
  return hip_status(ha::launch_anchor(p.bf16, d, Q, K, V, G, O, p.BH, p.N, stream, nullptr, nullptr, 0, lse));
}

HA_API size_t hybrid_attn_softmax_backward_workspace_bytes(int B, int H, int64_t N, int d, ha_dtype dtype) {
  Problem p;
  if (check_shape(B, H, N, d, dtype, &p) != HA_OK || p.BH == 0) return 0;
  return ha::softmax_bwd_ws(p.BH, p.N, d, p.bf16);
}

HA_API int hybrid_attn_softmax_backward(const void* Q, const void* K, const void* V, const void* G,
                                        const void* O, const void* dO, const float* lse, void* dQ, void* dK,
                                        void* dV, void* dG, int B, int H, int64_t N, int d, ha_dtype dtype,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Problem p;
  int st = check_shape(B, H, N, d, dtype, &p);
  if (st != HA_OK) return st;
  if (p.BH == 0 || p.N == 0) return HA_OK;
  const size_t tb = p.tensor_bytes, lb = static_cast<size_t>(p.BH) * p.N * sizeof(float);
  const void* in[7] = {Q, K, V, G, O, dO, lse};
  const size_t in_bytes[7] = {tb, tb, tb, tb, tb, tb, lb};
  void* out[4] = {dQ, dK, dV, dG};
  const size_t out_bytes[4] = {tb, tb, tb, tb};
  st = check_io(in, in_bytes, 7, out, out_bytes, 4);
  if (st != HA_OK) return st;
  const size_t need = ha::softmax_bwd_ws(p.BH, p.N, d, p.bf16);
  if (workspace == nullptr || workspace_bytes < need) return HA_EWORKSPACE;
  if (misaligned(workspace)) return HA_EALIGN;
  for (int i = 0; i < 7; ++i)
    if (overlaps(workspace, need, in[i], in_bytes[i])) return HA_EINVAL;
  for (int i = 0; i < 4; ++i)
    if (overlaps(workspace, need, out[i], out_bytes[i])) return HA_EINVAL;
  return hip_status(ha::launch_softmax_backward(p.bf16, d, Q, K, V, G, O, dO, lse, dQ, dK, dV, dG, p.BH,
                                                p.N, workspace, stream));
}

HA_API int hybrid_attn_proj_in(const void* x, const void* W_in, void* Q, void* K, void* V, void* G,
                               int B, int H, int64_t N, int d, ha_dtype dtype, hipStream_t stream) {
  Problem p;
  int st = check_shape(B, H, N, d, dtype, &p);
  if (st != HA_OK) return st;
  if (p.BH == 0 || p.N == 0) return HA_OK;
  const int64_t C = p.H * p.d;
  const void* in[2] = {x, W_in};
  const size_t in_bytes[2] = {p.tensor_bytes, weight_bytes(p, 4 * C)};
  void* out[4] = {Q, K, V, G};
  const size_t out_bytes[4] = {p.tensor_bytes, p.tensor_bytes, p.tensor_bytes, p.tensor_bytes};
  st = check_io(in, in_bytes, 2, out, out_bytes, 4);
  if (st != HA_OK) return st;
  return hip_status(ha::launch_proj_in(p.bf16, x, W_in, Q, K, V, G, p.B, p.H, p.N, d, stream));
}

HA_API int hybrid_attn_proj_out(const void* O, const void* W_out, const void* x, void* x_out, int B, int H,
                                int64_t N, int d, ha_dtype dtype, hipStream_t stream) {
  Problem p;
  int st = check_shape(B, H, N, d, dtype, &p);
  if (st != HA_OK) return st;
  if (p.BH == 0 || p.N == 0) return HA_OK;
  const int64_t C = p.H * p.d;
  // x_out may be x itself; otherwise it must not overlap x
  const bool in_place = x_out == x;
  const void* in[3] = {O, W_out, x};
  const size_t in_bytes[3] = {p.tensor_bytes, weight_bytes(p, C), p.tensor_bytes};
  void* out[1] = {x_out};
  const size_t out_bytes[1] = {p.tensor_bytes};
  st = check_io(in, in_bytes, in_place ? 2 : 3, out, out_bytes, 1);
  if (st != HA_OK) return st;
  if (in_place && (x == nullptr || misaligned(x))) return x == nullptr ? HA_EINVAL : HA_EALIGN;
  return hip_status(ha::launch_proj_out(p.bf16, O, W_out, x, x_out, p.B, p.H, p.N, d, stream));
}

HA_API size_t hybrid_attn_block_workspace_bytes(int B, int H, int64_t N, int d, ha_dtype dtype) {
  Problem p;
  if (check_shape(B, H, N, d, dtype, &p) != HA_OK || p.BH == 0) return 0;
  return block_ws(p).total;
}

HA_API int hybrid_attn_block(const void* x, const void* W_in4, const void* W_out4, void* x_out, int B,
                             int H, int64_t N, int d, ha_dtype dtype, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  Problem p;
  int st = check_shape(B, H, N, d, dtype, &p);
  if (st != HA_OK) return st;
  if (p.BH == 0 || p.N == 0) return HA_OK;
  const int64_t C = p.H * p.d;
  const size_t win_bytes = weight_bytes(p, 4 * C), wout_bytes = weight_bytes(p, C);
  const bool in_place = x_out == x;
  const void* in[3] = {W_in4, W_out4, x};
  const size_t in_bytes[3] = {4 * win_bytes, 4 * wout_bytes, p.tensor_bytes};
  void* out[1] = {x_out};
  const size_t out_bytes[1] = {p.tensor_bytes};
  st = check_io(in, in_bytes, in_place ? 2 : 3, out, out_bytes, 1);
  if (st != HA_OK) return st;
  if (in_place && (x == nullptr || misaligned(x))) return x == nullptr ? HA_EINVAL : HA_EALIGN;
  const BlockWs L = block_ws(p);
  if (workspace == nullptr || workspace_bytes < L.total) return HA_EWORKSPACE;
  if (misaligned(workspace)) return HA_EALIGN;
  for (int i = 0; i < 3; ++i)
    if (overlaps(workspace, L.total, in[i], in_bytes[i])) return HA_EINVAL;
  if (overlaps(workspace, L.total, x_out, p.tensor_bytes)) return HA_EINVAL;

  char* w = static_cast<char*>(workspace);
  void *q = w + L.q, *k = w + L.k, *v = w + L.v, *g = w + L.g, *o = w + L.o, *lin = w + L.lin;
  int kinds[4];
  hybrid_attn_group_schedule(kinds);
  for (int l = 0; l < 4; ++l) {
    const void* xin = l == 0 ? x : x_out;
    const char* wi = static_cast<const char*>(W_in4) + static_cast<size_t>(l) * win_bytes;
    const char* wo = static_cast<const char*>(W_out4) + static_cast<size_t>(l) * wout_bytes;
    st = hip_status(ha::launch_proj_in(p.bf16, xin, wi, q, k, v, g, p.B, p.H, p.N, d, stream));
    if (st != HA_OK) return st;
    if (kinds[l] == 0)
      st = run_linear(p, q, k, v, g, o, lin, stream);
    else
      st = hip_status(ha::launch_anchor(p.bf16, d, q, k, v, g, o, p.BH, p.N, stream));
    if (st != HA_OK) return st;
    st = hip_status(ha::launch_proj_out(p.bf16, o, wo, xin, x_out, p.B, p.H, p.N, d, stream));
    if (st != HA_OK) return st;
  }
  return HA_OK;
}

HA_API int hybrid_attn_attnres_mix(const void* summaries, int M, const void* x, const float* w, void* h,
                                   int B, int64_t N, int C, ha_dtype dtype, hipStream_t stream) {
  if (dtype != HA_BF16 && dtype != HA_F32) return HA_EUNSUPPORTED;
  if (C <= 0 || C % 8 != 0) return HA_EUNSUPPORTED;
  if (B < 0 || N < 0 || N > HA_MAX_N || M < 0 || M > HA_ATTNRES_MAX_SUMMARIES) return HA_EINVAL;
  static_assert(HA_ATTNRES_MAX_SUMMARIES < 64, "candidate scores fit the kernel's table");
  const int64_t tokens = static_cast<int64_t>(B) * N;
  if (tokens == 0) return HA_OK;
  const size_t row_bytes = static_cast<size_t>(tokens) * C * (dtype == HA_BF16 ? 2u : 4u);
  if (M > 0 && summaries == nullptr) return HA_EINVAL;
  const void* in[3] = {x, w, M > 0 ? summaries : x};
  const size_t in_bytes[3] = {row_bytes, static_cast<size_t>(C) * sizeof(float), M * row_bytes};
  void* out[1] = {h};
  const size_t out_bytes[1] = {row_bytes};
  int st = check_io(in, in_bytes, M > 0 ? 3 : 2, out, out_bytes, 1);
  if (st != HA_OK) return st;
  return hip_status(ha::launch_attnres_mix(dtype == HA_BF16, summaries, M, x, w, h, tokens, C, HA_RMS_EPS, stream));
}

HA_API size_t hybrid_attn_block_routed_workspace_bytes(int B, int H, int64_t N, int d, ha_dtype dtype) {
  Problem p;
  if (check_shape(B, H, N, d, dtype, &p) != HA_OK || p.BH == 0) return 0;
  return block_ws(p).total + ((p.tensor_bytes + 255) & ~static_cast<size_t>(255));
}

HA_API int hybrid_attn_block_routed(const void* x, const void* summaries, int M, const float* w_route,
                                    const void* W_in4, const void* W_out4, void* x_out, int B, int H, int64_t N,
                                    int d, ha_dtype dtype, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  Problem p;
  int st = check_shape(B, H, N, d, dtype, &p);
  if (st != HA_OK) return st;
  if (M < 0 || M > HA_ATTNRES_MAX_SUMMARIES) return HA_EINVAL;
  if (p.BH == 0 || p.N == 0) return HA_OK;
  const int64_t C = p.H * p.d;
  const size_t win_bytes = weight_bytes(p, 4 * C), wout_bytes = weight_bytes(p, C);
  const bool in_place = x_out == x;
  if (M > 0 && summaries == nullptr) return HA_EINVAL;
  const void* in[5] = {W_in4, W_out4, w_route, M > 0 ? summaries : W_in4, x};
  const size_t in_bytes[5] = {4 * win_bytes, 4 * wout_bytes, static_cast<size_t>(4 * C) * sizeof(float),
                              M * p.tensor_bytes, p.tensor_bytes};
  void* out[1] = {x_out};
  const size_t out_bytes[1] = {p.tensor_bytes};
  // x may lie inside the summaries (read-only both); x_out may be x itself
  const int n_in = in_place ? 4 : 5;
  st = check_io(in, in_bytes, n_in, out, out_bytes, 1);
  if (st != HA_OK) return st;
  if (in_place && (x == nullptr || misaligned(x))) return x == nullptr ? HA_EINVAL : HA_EALIGN;
  const BlockWs L = block_ws(p);
  const size_t need = L.total + ((p.tensor_bytes + 255) & ~static_cast<size_t>(255));
  if (workspace == nullptr || workspace_bytes < need) return HA_EWORKSPACE;
  if (misaligned(workspace)) return HA_EALIGN;
  for (int i = 0; i < 5; ++i)
    if ((i < 4 || !in_place) && overlaps(workspace, need, in[i], in_bytes[i])) return HA_EINVAL;
  if (overlaps(workspace, need, x_out, p.tensor_bytes)) return HA_EINVAL;

  char* w = static_cast<char*>(workspace);
  void *q = w + L.q, *k = w + L.k, *v = w + L.v, *g = w + L.g, *o = w + L.o, *lin = w + L.lin;
  void* hbuf = w + L.total;
  int kinds[4];
  hybrid_attn_group_schedule(kinds);
  for (int l = 0; l < 4; ++l) {
    const void* xin = l == 0 ? x : x_out;
    const char* wi = static_cast<const char*>(W_in4) + static_cast<size_t>(l) * win_bytes;
    const char* wo = static_cast<const char*>(W_out4) + static_cast<size_t>(l) * wout_bytes;
    const void* src = xin;
    if (kinds[l] == 0) {
      st = hip_status(ha::launch_attnres_mix(p.bf16, summaries, M, xin, w_route + l * C, hbuf, p.B * p.N,
                                             static_cast<int>(C), HA_RMS_EPS, stream));
      if (st != HA_OK) return st;
      src = hbuf;
    }
    st = hip_status(ha::launch_proj_in(p.bf16, src, wi, q, k, v, g, p.B, p.H, p.N, d, stream));
    if (st != HA_OK) return st;
    if (kinds[l] == 0)
      st = run_linear(p, q, k, v, g, o, lin, stream);
    else
      st = hip_status(ha::launch_anchor(p.bf16, d, q, k, v, g, o, p.BH, p.N, stream));
    if (st != HA_OK) return st;
    st = hip_status(ha::launch_proj_out(p.bf16, o, wo, xin, x_out, p.B, p.H, p.N, d, stream));
    if (st != HA_OK) return st;
  }
  return HA_OK;
}

HA_API int hybrid_attn_group_schedule(int kinds[4]) {
  if (kinds == nullptr) return HA_EINVAL;
  static const int schedule[4] = {0, 0, 0, 1};
  memcpy(kinds, schedule, sizeof(schedule));
  return HA_OK;
}

HA_API double hybrid_attn_probe_mfma_flops(int blocks, int iters) {
  if (blocks < 1 || blocks > HA_PROBE_MAX_BLOCKS || iters < 1 || iters > HA_PROBE_MAX_ITERS) return 0.0;
  return ha::probe_mfma_flops(blocks, iters);
}

HA_API int hybrid_attn_probe_mfma(int blocks, int iters, float* sink, hipStream_t stream) {
  if (sink == nullptr || blocks < 1 || blocks > HA_PROBE_MAX_BLOCKS || iters < 1 || iters > HA_PROBE_MAX_ITERS)
    return HA_EINVAL;
  return hip_status(ha::launch_probe_mfma(blocks, iters, sink, stream));
}

HA_API int hybrid_attn_probe_mfma_data(int blocks, int iters, float* sink, hipStream_t stream) {
  if (sink == nullptr || blocks < 1 || blocks > HA_PROBE_MAX_BLOCKS || iters < 1 || iters > HA_PROBE_MAX_ITERS)
    return HA_EINVAL;
  return hip_status(ha::launch_probe_mfma_data(blocks, iters, sink, stream));
}

HA_API int hybrid_attn_probe_overlap(int mode, int waves_per_simd, int blocks, int iters, float* sink,
                                     hipStream_t stream) {
  if (sink == nullptr || blocks < 1 || blocks > HA_PROBE_MAX_BLOCKS || iters < 1 || iters > HA_PROBE_MAX_ITERS)
    return HA_EINVAL;
  if (mode < HA_PROBE_OVERLAP_MFMA || mode > HA_PROBE_OVERLAP_SPLIT) return HA_EINVAL;
  if (waves_per_simd != 1 && waves_per_simd != 2) return HA_EINVAL;
  if (mode == HA_PROBE_OVERLAP_SPLIT && waves_per_simd != 2) return HA_EINVAL;
  return hip_status(ha::launch_probe_overlap(mode, waves_per_simd, blocks, iters, sink, stream));
}

HA_API int hybrid_attn_probe_read(const void* src, size_t bytes, float* sink, hipStream_t stream) {
  if (src == nullptr || sink == nullptr) return HA_EINVAL;
  if (misaligned(src) || bytes % 16 != 0) return HA_EALIGN;
  return hip_status(ha::launch_probe_read(src, bytes, sink, stream));
}

HA_API int hybrid_attn_probe_copy(const void* src, void* dst, size_t bytes, int nontemporal, hipStream_t stream) {
  if (src == nullptr || dst == nullptr || overlaps(src, bytes, dst, bytes)) return HA_EINVAL;
  if (misaligned(src) || misaligned(dst) || bytes % 16 != 0) return HA_EALIGN;
  return hip_status(ha::launch_probe_copy(src, dst, bytes, nontemporal != 0, stream));
}

}  // extern "C"
