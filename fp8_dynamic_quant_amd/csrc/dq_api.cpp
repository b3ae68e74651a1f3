// C ABI of libdq: argument checks on the host, then asynchronous launches on the caller's stream.
// Every check runs before any HIP call, so a rejected call enqueues nothing and needs no GPU.
#include "../../include/dq.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "dq_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxElems = int64_t(1) << 47;
constexpr int64_t kMaxLinearK = int64_t(1) << 24;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [a, a + na) and [b, b + nb) overlap (byte ranges, empty ranges never overlap).
bool overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
  if (na == 0 || nb == 0 || a == nullptr || b == nullptr) return false;
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return DQ_OK;
  g_last_hip_error = static_cast<int>(e);
  return DQ_ERR_HIP;
}

int check_quantize(const void* x, int64_t R, int64_t K, const void* q, const float* scale) {
  if (R < 0 || R > kMaxDim || K < 8 || K > kMaxDim || (K % 8) != 0) return DQ_ERR_SHAPE;
  if (R > 0 && K > kMaxElems / R) return DQ_ERR_SHAPE;
  if (R == 0) return DQ_OK;
  if (!x || !q || !scale) return DQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(q) || !aligned16(scale)) return DQ_ERR_ALIGN;
  const uint64_t n = static_cast<uint64_t>(R) * static_cast<uint64_t>(K);
  if (overlap(q, n, x, 2 * n) || overlap(scale, 4 * static_cast<uint64_t>(R), x, 2 * n) ||
      overlap(scale, 4 * static_cast<uint64_t>(R), q, n))
    return DQ_ERR_ALIAS;
  return DQ_OK;
}

int quantize_rows(const void* x, int64_t R, int64_t K, void* q, float* scale, void* stream) {
  const int st = check_quantize(x, R, K, q, scale);
  if (st != DQ_OK || R == 0) return st;
  return hip_status(dq::launch_quantize_rows(static_cast<const uint16_t*>(x), R, K,
                                             static_cast<uint8_t*>(q), scale,
                                             static_cast<hipStream_t>(stream)));
}

// Sizes of dq_linear_fp8 (shared with the workspace size query).
int check_linear_shape(int64_t M, int64_t K, int64_t N) {
  // K < 2^24 keeps a 256-row tile of an operand inside one 32-bit buffer range
  if (M < 0 || M > kMaxDim || K < 128 || K >= kMaxLinearK || (K % 128) != 0 || N < 64 ||
      N > kMaxDim || (N % 64) != 0)
    return DQ_ERR_SHAPE;
  if ((M > 0 && K > kMaxElems / M) || K > kMaxElems / N || (M > 0 && N > kMaxElems / M))
    return DQ_ERR_SHAPE;
  // tile-steps are counted in 32-bit integers on the device
  if (dq::linear_units(M, K, N) >= (int64_t(1) << 31)) return DQ_ERR_SHAPE;
  return DQ_OK;
}

}  // namespace

extern "C" {

int dq_quantize_fp8(const void* x, int64_t M, int64_t K, void* q, float* scale, void* stream) {
  return quantize_rows(x, M, K, q, scale, stream);
}

int dq_quantize_weight_fp8(const void* w, int64_t N, int64_t K, void* qw, float* w_scale,
                           void* stream) {
  return quantize_rows(w, N, K, qw, w_scale, stream);
}

}  // extern "C"

namespace {

// Everything dq_linear_fp8 checks, for the workspace range [workspace, + workspace_bytes) (NULL:
// none). Returns DQ_OK, or the status to return with nothing enqueued.
int check_linear_args(const void* q, const float* scale, int64_t M, int64_t K, const void* qw,
                      const float* w_scale, int64_t N, const void* bias, int epilogue,
                      const void* gate, const void* residual, const void* out,
                      const void* workspace, uint64_t workspace_bytes) {
  const int shape = check_linear_shape(M, K, N);
  if (shape != DQ_OK) return shape;
  if (epilogue != DQ_EPI_BIAS && epilogue != DQ_EPI_GELU_TANH &&
      epilogue != DQ_EPI_GATED_RESIDUAL)
    return DQ_ERR_EPILOGUE;
  const bool gated = epilogue == DQ_EPI_GATED_RESIDUAL;
  if (gated && (!gate || !residual)) return DQ_ERR_EPILOGUE;
  if (M == 0) return DQ_OK;
  if (!q || !scale || !qw || !w_scale || !out) return DQ_ERR_NULL;
  if (!aligned16(q) || !aligned16(scale) || !aligned16(qw) || !aligned16(w_scale) ||
      !aligned16(out) || (bias && !aligned16(bias)) || (gated && !aligned16(gate)) ||
      (gated && !aligned16(residual)))
    return DQ_ERR_ALIGN;
  const uint64_t m = static_cast<uint64_t>(M), k = static_cast<uint64_t>(K),
                 n = static_cast<uint64_t>(N);
  const uint64_t out_bytes = 2 * m * n;
  if (workspace) {
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return DQ_ERR_WORKSPACE;
    const uint64_t wb = workspace_bytes;
    if (overlap(workspace, wb, q, m * k) || overlap(workspace, wb, scale, 4 * m) ||
        overlap(workspace, wb, qw, n * k) || overlap(workspace, wb, w_scale, 4 * n) ||
        overlap(workspace, wb, bias, bias ? 2 * n : 0) ||
        (gated && overlap(workspace, wb, gate, 2 * n)) ||
        (gated && overlap(workspace, wb, residual, out_bytes)) ||
        overlap(workspace, wb, out, out_bytes))
      return DQ_ERR_ALIAS;
  }
  if (overlap(out, out_bytes, q, m * k) || overlap(out, out_bytes, scale, 4 * m) ||
      overlap(out, out_bytes, qw, n * k) || overlap(out, out_bytes, w_scale, 4 * n) ||
      overlap(out, out_bytes, bias, bias ? 2 * n : 0) ||
      (gated && overlap(out, out_bytes, gate, 2 * n)))
    return DQ_ERR_ALIAS;
  if (gated && residual != out && overlap(out, out_bytes, residual, out_bytes)) return DQ_ERR_ALIAS;
  return DQ_OK;
}

}  // namespace

extern "C" {

int dq_linear_fp8(const void* q, const float* scale, int64_t M, int64_t K, const void* qw,
                  const float* w_scale, int64_t N, const void* bias, int epilogue,
                  const void* gate, const void* residual, void* out, void* workspace,
                  uint64_t workspace_bytes, void* stream) {
  const int st = check_linear_args(q, scale, M, K, qw, w_scale, N, bias, epilogue, gate, residual,
                                   out, workspace, workspace_bytes);
  if (st != DQ_OK || M == 0) return st;
  const bool gated = epilogue == DQ_EPI_GATED_RESIDUAL;
  return hip_status(dq::launch_linear(
      static_cast<const uint8_t*>(q), scale, M, K, static_cast<const uint8_t*>(qw), w_scale, N,
      static_cast<const uint16_t*>(bias), epilogue,
      gated ? static_cast<const uint16_t*>(gate) : nullptr,
      gated ? static_cast<const uint16_t*>(residual) : nullptr, static_cast<uint16_t*>(out),
      workspace, workspace ? workspace_bytes : 0, static_cast<hipStream_t>(stream)));
}

// Checks of dq_linear_fp8_segmented; on success *M_out is the total row count.
static int check_segmented(const void* q, const float* scale, int64_t K, int64_t nseg,
                           const int64_t* seg_rows, const void* const* qw,
                           const float* const* w_scale, int64_t N, const void* const* bias,
                           int epilogue, const void* const* gate, const void* residual,
                           const void* out, const void* workspace, uint64_t workspace_bytes,
                           int64_t* M_out) {
  if (nseg < 1 || nseg > dq::kMaxSegments) return DQ_ERR_SHAPE;
  if (!seg_rows || !qw || !w_scale || !bias) return DQ_ERR_NULL;
  int64_t M = 0, tiles_m = 0;
  for (int64_t i = 0; i < nseg; ++i) {
    if (seg_rows[i] < 0 || seg_rows[i] > kMaxDim - M) return DQ_ERR_SHAPE;
    M += seg_rows[i];
    tiles_m += (seg_rows[i] + dq::kTileM - 1) / dq::kTileM;
  }
  const int shape = check_linear_shape(M, K, N);
  if (shape != DQ_OK) return shape;
  if (tiles_m * ((N + dq::kTileN - 1) / dq::kTileN) * (K / dq::kStepK) >= (int64_t(1) << 31))
    return DQ_ERR_SHAPE;
  if (epilogue != DQ_EPI_BIAS && epilogue != DQ_EPI_GELU_TANH &&
      epilogue != DQ_EPI_GATED_RESIDUAL)
    return DQ_ERR_EPILOGUE;
  const bool gated = epilogue == DQ_EPI_GATED_RESIDUAL;
  if (gated && (!gate || !residual)) return DQ_ERR_EPILOGUE;
  *M_out = M;
  if (M == 0) return DQ_OK;
  // every segment's weight, scales, bias and gate with the shared row-indexed tensors, as
  // dq_linear_fp8 checks them
  for (int64_t i = 0; i < nseg; ++i) {
    if (gated && !gate[i]) return DQ_ERR_EPILOGUE;
    const int st = check_linear_args(q, scale, M, K, qw[i], w_scale[i], N, bias[i], epilogue,
                                     gated ? gate[i] : nullptr, residual, out, workspace,
                                     workspace_bytes);
    if (st != DQ_OK) return st;
  }
  return DQ_OK;
}

int dq_linear_fp8_segmented(const void* q, const float* scale, int64_t K, int64_t nseg,
                            const int64_t* seg_rows, const void* const* qw,
                            const float* const* w_scale, int64_t N, const void* const* bias,
                            int epilogue, const void* const* gate, const void* residual,
                            void* out, void* workspace, uint64_t workspace_bytes, void* stream) {
  int64_t M = 0;
  const int st = check_segmented(q, scale, K, nseg, seg_rows, qw, w_scale, N, bias, epilogue,
                                 gate, residual, out, workspace, workspace_bytes, &M);
  if (st != DQ_OK || M == 0) return st;
  const bool gated = epilogue == DQ_EPI_GATED_RESIDUAL;
  const uint8_t* w[dq::kMaxSegments];
  const float* ws[dq::kMaxSegments];
  const uint16_t* b[dq::kMaxSegments];
  const uint16_t* g[dq::kMaxSegments];
  for (int64_t i = 0; i < nseg; ++i) {
    w[i] = static_cast<const uint8_t*>(qw[i]);
    ws[i] = w_scale[i];
    b[i] = static_cast<const uint16_t*>(bias[i]);
    g[i] = gated ? static_cast<const uint16_t*>(gate[i]) : nullptr;
  }
  return hip_status(dq::launch_linear_segmented(
      static_cast<const uint8_t*>(q), scale, nseg, seg_rows, K, w, ws, N, b, epilogue, g,
      gated ? static_cast<const uint16_t*>(residual) : nullptr, static_cast<uint16_t*>(out),
      workspace, workspace ? workspace_bytes : 0, static_cast<hipStream_t>(stream)));
}

uint64_t dq_linear_fp8_segmented_workspace_size(int64_t nseg, const int64_t* seg_rows, int64_t K,
                                                int64_t N) {
  if (nseg < 1 || nseg > dq::kMaxSegments || !seg_rows) return 0;
  int64_t M = 0;
  for (int64_t i = 0; i < nseg; ++i) {
    if (seg_rows[i] < 0 || seg_rows[i] > kMaxDim - M) return 0;
    M += seg_rows[i];
  }
  if (check_linear_shape(M, K, N) != DQ_OK) return 0;
  return dq::linear_segmented_workspace_bytes(nseg, seg_rows, K, N);
}

int dq_linear_fp8_noalloc(const void* q, const float* scale, int64_t M, int64_t K,
                          const void* qw, const float* w_scale, int64_t N, const void* bias,
                          int epilogue, const void* gate, const void* residual, void* out,
                          void* stream) {
  const int st = check_linear_args(q, scale, M, K, qw, w_scale, N, bias, epilogue, gate, residual,
                                   out, nullptr, 0);
  if (st != DQ_OK || M == 0) return st;
  const bool gated = epilogue == DQ_EPI_GATED_RESIDUAL;
  return hip_status(dq::launch_linear_noalloc(
      static_cast<const uint8_t*>(q), scale, M, K, static_cast<const uint8_t*>(qw), w_scale, N,
      static_cast<const uint16_t*>(bias), epilogue,
      gated ? static_cast<const uint16_t*>(gate) : nullptr,
      gated ? static_cast<const uint16_t*>(residual) : nullptr, static_cast<uint16_t*>(out),
      static_cast<hipStream_t>(stream)));
}

int dq_layernorm_modulate_quantize_fp8(const void* x, int64_t M, int64_t K, const void* mod_scale,
                                       const void* mod_shift, float eps, void* y_out, void* q,
                                       float* scale, void* stream) {
  if (M < 0 || M > kMaxDim || K < 8 || K > dq::kMaxModulateK || (K % 8) != 0) return DQ_ERR_SHAPE;
  if (!std::isfinite(eps) || !(eps > 0.0f)) return DQ_ERR_VALUE;
  if (M == 0) return DQ_OK;
  if (!x || !mod_scale || !mod_shift || !q || !scale) return DQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(mod_scale) || !aligned16(mod_shift) || !aligned16(q) ||
      !aligned16(scale) || (y_out && !aligned16(y_out)))
    return DQ_ERR_ALIGN;
  const uint64_t n = static_cast<uint64_t>(M) * static_cast<uint64_t>(K);
  const uint64_t kb = 2 * static_cast<uint64_t>(K), sb = 4 * static_cast<uint64_t>(M);
  const uint64_t yb = y_out ? 2 * n : 0;
  // outputs against inputs, then outputs against each other
  const void* ins[3] = {x, mod_scale, mod_shift};
  const uint64_t in_bytes[3] = {2 * n, kb, kb};
  for (int i = 0; i < 3; ++i) {
    if (overlap(y_out, yb, ins[i], in_bytes[i]) || overlap(q, n, ins[i], in_bytes[i]) ||
        overlap(scale, sb, ins[i], in_bytes[i]))
      return DQ_ERR_ALIAS;
  }
  if (overlap(y_out, yb, q, n) || overlap(y_out, yb, scale, sb) || overlap(q, n, scale, sb))
    return DQ_ERR_ALIAS;
  return hip_status(dq::launch_ln_modulate_quantize(
      static_cast<const uint16_t*>(x), M, K, static_cast<const uint16_t*>(mod_scale),
      static_cast<const uint16_t*>(mod_shift), eps, static_cast<uint16_t*>(y_out),
      static_cast<uint8_t*>(q), scale, static_cast<hipStream_t>(stream)));
}

int dq_linear_qkv_fp8(const void* q, const float* scale, int64_t M, int64_t K, const void* qw,
                      const float* w_scale, int64_t heads, const void* bias, const void* norm_qk,
                      const float* rope_cos, const float* rope_sin, float eps, void* out_q,
                      void* out_k, void* out_v, void* workspace, uint64_t workspace_bytes,
                      void* stream) {
  if (heads < 1 || heads > kMaxDim / (3 * dq::kHeadDim)) return DQ_ERR_SHAPE;
  const int64_t N = 3 * heads * dq::kHeadDim;
  const int shape = check_linear_shape(M, K, N);
  if (shape != DQ_OK) return shape;
  if (!std::isfinite(eps) || !(eps > 0.0f)) return DQ_ERR_VALUE;
  if (M == 0) return DQ_OK;
  if (!q || !scale || !qw || !w_scale || !norm_qk || !rope_cos || !rope_sin || !out_q || !out_k ||
      !out_v)
    return DQ_ERR_NULL;
  if (!aligned16(q) || !aligned16(scale) || !aligned16(qw) || !aligned16(w_scale) ||
      (bias && !aligned16(bias)) || !aligned16(norm_qk) || !aligned16(rope_cos) ||
      !aligned16(rope_sin) || !aligned16(out_q) || !aligned16(out_k) || !aligned16(out_v))
    return DQ_ERR_ALIGN;
  const uint64_t m = static_cast<uint64_t>(M), k = static_cast<uint64_t>(K),
                 n = static_cast<uint64_t>(N);
  const uint64_t rope_bytes = m * static_cast<uint64_t>(dq::kHeadDim / 2) * 4;
  const void* ins[8] = {q, scale, qw, w_scale, bias, norm_qk, rope_cos, rope_sin};
  const uint64_t in_bytes[8] = {m * k, 4 * m, n * k, 4 * n, bias ? 2 * n : 0,
                                4 * static_cast<uint64_t>(dq::kHeadDim), rope_bytes, rope_bytes};
  const uint64_t ob = 2 * m * (n / 3);  // one of the three outputs
  void* outs[3] = {out_q, out_k, out_v};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 8; ++i)
      if (overlap(outs[o], ob, ins[i], in_bytes[i])) return DQ_ERR_ALIAS;
    for (int o2 = o + 1; o2 < 3; ++o2)
      if (overlap(outs[o], ob, outs[o2], ob)) return DQ_ERR_ALIAS;
  }
  if (workspace) {
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return DQ_ERR_WORKSPACE;
    for (int i = 0; i < 8; ++i)
      if (overlap(workspace, workspace_bytes, ins[i], in_bytes[i])) return DQ_ERR_ALIAS;
    for (int o = 0; o < 3; ++o)
      if (overlap(workspace, workspace_bytes, outs[o], ob)) return DQ_ERR_ALIAS;
  }
  return hip_status(dq::launch_linear_qkv(
      static_cast<const uint8_t*>(q), scale, M, K, static_cast<const uint8_t*>(qw), w_scale,
      heads, static_cast<const uint16_t*>(bias), static_cast<const uint16_t*>(norm_qk), rope_cos,
      rope_sin, eps, static_cast<uint16_t*>(out_q), static_cast<uint16_t*>(out_k),
      static_cast<uint16_t*>(out_v), workspace, workspace ? workspace_bytes : 0,
      static_cast<hipStream_t>(stream)));
}

int dq_linear_qkv_fp8_attn(const void* q, const float* scale, int64_t M, int64_t K, const void* qw,
                           const float* w_scale, int64_t heads, const void* bias,
                           const void* norm_qk, const float* rope_cos, const float* rope_sin,
                           float eps, void* q8, float* q_scale, void* k8, float* k_scale, void* vt8,
                           float* v_scale, void* workspace, uint64_t workspace_bytes,
                           void* stream) {
  if (heads < 1 || heads > kMaxDim / (3 * dq::kHeadDim)) return DQ_ERR_SHAPE;
  const int64_t N = 3 * heads * dq::kHeadDim;
  const int shape = check_linear_shape(M, K, N);
  if (shape != DQ_OK) return shape;
  if (M % 16 != 0) return DQ_ERR_SHAPE;  // the transposed value rows: 16-byte chunks of tokens
  if (!std::isfinite(eps) || !(eps > 0.0f)) return DQ_ERR_VALUE;
  if (M == 0) return DQ_OK;
  if (!q || !scale || !qw || !w_scale || !norm_qk || !rope_cos || !rope_sin || !q8 || !q_scale ||
      !k8 || !k_scale || !vt8 || !v_scale)
    return DQ_ERR_NULL;
  if (!aligned16(q) || !aligned16(scale) || !aligned16(qw) || !aligned16(w_scale) ||
      (bias && !aligned16(bias)) || !aligned16(norm_qk) || !aligned16(rope_cos) ||
      !aligned16(rope_sin) || !aligned16(q8) || !aligned16(q_scale) || !aligned16(k8) ||
      !aligned16(k_scale) || !aligned16(vt8) || !aligned16(v_scale))
    return DQ_ERR_ALIGN;
  const uint64_t m = static_cast<uint64_t>(M), k = static_cast<uint64_t>(K),
                 n = static_cast<uint64_t>(N);
  const uint64_t rows = m * static_cast<uint64_t>(heads);  // head rows of each output
  const uint64_t rope_bytes = m * static_cast<uint64_t>(dq::kHeadDim / 2) * 4;
  const void* ins[8] = {q, scale, qw, w_scale, bias, norm_qk, rope_cos, rope_sin};
  const uint64_t in_bytes[8] = {m * k, 4 * m, n * k, 4 * n, bias ? 2 * n : 0,
                                4 * static_cast<uint64_t>(dq::kHeadDim), rope_bytes, rope_bytes};
  void* outs[6] = {q8, q_scale, k8, k_scale, vt8, v_scale};
  const uint64_t cb = rows * dq::kHeadDim;
  const uint64_t out_bytes[6] = {cb, 4 * rows, cb, 4 * rows, cb, 4 * rows};
  for (int o = 0; o < 6; ++o) {
    for (int i = 0; i < 8; ++i)
      if (overlap(outs[o], out_bytes[o], ins[i], in_bytes[i])) return DQ_ERR_ALIAS;
    for (int o2 = o + 1; o2 < 6; ++o2)
      if (overlap(outs[o], out_bytes[o], outs[o2], out_bytes[o2])) return DQ_ERR_ALIAS;
  }
  if (workspace) {
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return DQ_ERR_WORKSPACE;
    for (int i = 0; i < 8; ++i)
      if (overlap(workspace, workspace_bytes, ins[i], in_bytes[i])) return DQ_ERR_ALIAS;
    for (int o = 0; o < 6; ++o)
      if (overlap(workspace, workspace_bytes, outs[o], out_bytes[o])) return DQ_ERR_ALIAS;
  }
  return hip_status(dq::launch_linear_qkv_q8(
      static_cast<const uint8_t*>(q), scale, M, K, static_cast<const uint8_t*>(qw), w_scale,
      heads, static_cast<const uint16_t*>(bias), static_cast<const uint16_t*>(norm_qk), rope_cos,
      rope_sin, eps, static_cast<uint8_t*>(q8), q_scale, static_cast<uint8_t*>(k8), k_scale,
      static_cast<uint8_t*>(vt8), v_scale, workspace, workspace ? workspace_bytes : 0,
      static_cast<hipStream_t>(stream)));
}

// Sizes of the attention entry points: 1 <= S < 2^24 with S % 16 == 0 (or an empty problem),
// 0 <= H < 65536, H S 128 < 2^47.
static int check_attention_shape(int64_t H, int64_t S) {
  if (H < 0 || H >= 65536 || S < 0 || S >= (int64_t(1) << 24) || (S % 16) != 0) return DQ_ERR_SHAPE;
  if (H > 0 && S > kMaxElems / (H * dq::kHeadDim)) return DQ_ERR_SHAPE;
  return DQ_OK;
}

int dq_quantize_v_fp8(const void* v, int64_t H, int64_t S, void* vt, float* v_scale,
                      void* stream) {
  const int shape = check_attention_shape(H, S);
  if (shape != DQ_OK) return shape;
  if (H == 0 || S == 0) return DQ_OK;
  if (!v || !vt || !v_scale) return DQ_ERR_NULL;
  if (!aligned16(v) || !aligned16(vt) || !aligned16(v_scale)) return DQ_ERR_ALIGN;
  const uint64_t n = static_cast<uint64_t>(H) * static_cast<uint64_t>(S) * dq::kHeadDim;
  const uint64_t sb = 4 * static_cast<uint64_t>(H) * static_cast<uint64_t>(S);
  if (overlap(vt, n, v, 2 * n) || overlap(v_scale, sb, v, 2 * n) || overlap(vt, n, v_scale, sb))
    return DQ_ERR_ALIAS;
  return hip_status(dq::launch_quantize_v(static_cast<const uint16_t*>(v), H, S,
                                          static_cast<uint8_t*>(vt), v_scale,
                                          static_cast<hipStream_t>(stream)));
}

int dq_attention_fp8(const void* q, const float* q_scale, const void* k, const float* k_scale,
                     const void* vt, const float* v_scale, int64_t H, int64_t S, void* out,
                     void* workspace, uint64_t workspace_bytes, int64_t max_workgroups,
                     void* stream) {
  const int shape = check_attention_shape(H, S);
  if (shape != DQ_OK) return shape;
  if (max_workgroups < 0) return DQ_ERR_VALUE;
  if (H == 0 || S == 0) return DQ_OK;
  if (!q || !q_scale || !k || !k_scale || !vt || !v_scale || !out) return DQ_ERR_NULL;
  if (!aligned16(q) || !aligned16(q_scale) || !aligned16(k) || !aligned16(k_scale) ||
      !aligned16(vt) || !aligned16(v_scale) || !aligned16(out))
    return DQ_ERR_ALIGN;
  const uint64_t n = static_cast<uint64_t>(H) * static_cast<uint64_t>(S) * dq::kHeadDim;
  const uint64_t sb = 4 * static_cast<uint64_t>(H) * static_cast<uint64_t>(S);
  const void* ins[6] = {q, q_scale, k, k_scale, vt, v_scale};
  const uint64_t in_bytes[6] = {n, sb, n, sb, n, sb};
  for (int i = 0; i < 6; ++i)
    if (overlap(out, 2 * n, ins[i], in_bytes[i])) return DQ_ERR_ALIAS;
  if (workspace) {
    const uint64_t need = dq::attention_workspace_bytes(H, S);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 || workspace_bytes < need)
      return DQ_ERR_WORKSPACE;
    for (int i = 0; i < 6; ++i)
      if (overlap(workspace, need, ins[i], in_bytes[i])) return DQ_ERR_ALIAS;
    if (overlap(workspace, need, out, 2 * n)) return DQ_ERR_ALIAS;
  }
  return hip_status(dq::launch_attention(
      static_cast<const uint8_t*>(q), q_scale, static_cast<const uint8_t*>(k), k_scale,
      static_cast<const uint8_t*>(vt), v_scale, H, S, static_cast<uint16_t*>(out), workspace,
      max_workgroups, static_cast<hipStream_t>(stream)));
}

int dq_quantize_mx_fp8(const void* x, int64_t M, int64_t K, void* q, void* scales,
                       void* stream) {
  if (M < 0 || M > kMaxDim || K < 32 || K > kMaxDim || (K % 32) != 0) return DQ_ERR_SHAPE;
  if (M > 0 && K > kMaxElems / M) return DQ_ERR_SHAPE;
  if (M == 0) return DQ_OK;
  if (!x || !q || !scales) return DQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(q)) return DQ_ERR_ALIGN;
  const uint64_t n = static_cast<uint64_t>(M) * static_cast<uint64_t>(K);
  if (overlap(q, n, x, 2 * n) || overlap(scales, n / 32, x, 2 * n) ||
      overlap(scales, n / 32, q, n))
    return DQ_ERR_ALIAS;
  return hip_status(dq::launch_quantize_mx(static_cast<const uint16_t*>(x), M, K,
                                           static_cast<uint8_t*>(q),
                                           static_cast<uint8_t*>(scales),
                                           static_cast<hipStream_t>(stream)));
}

int dq_linear_mx_fp8(const void* qa, const void* sa, int64_t M, int64_t K, const void* qw,
                     const void* sw, int64_t N, const void* bias, int epilogue, void* out,
                     void* stream) {
  const int shape = check_linear_shape(M, K, N);
  if (shape != DQ_OK) return shape;
  if (epilogue != DQ_EPI_BIAS && epilogue != DQ_EPI_GELU_TANH) return DQ_ERR_EPILOGUE;
  // the block-scaled limit on output tiles
  if (((M + 255) / 256) * ((N + 255) / 256) >= (int64_t(1) << 23)) return DQ_ERR_SHAPE;
  if (M == 0) return DQ_OK;
  if (!qa || !sa || !qw || !sw || !out) return DQ_ERR_NULL;
  if (!aligned16(qa) || !aligned16(qw) || !aligned16(out) || (bias && !aligned16(bias)) ||
      (reinterpret_cast<uintptr_t>(sa) & 3u) != 0 || (reinterpret_cast<uintptr_t>(sw) & 3u) != 0)
    return DQ_ERR_ALIGN;
  const uint64_t m = static_cast<uint64_t>(M), k = static_cast<uint64_t>(K),
                 n = static_cast<uint64_t>(N);
  const uint64_t out_bytes = 2 * m * n;
  if (overlap(out, out_bytes, qa, m * k) || overlap(out, out_bytes, sa, m * k / 32) ||
      overlap(out, out_bytes, qw, n * k) || overlap(out, out_bytes, sw, n * k / 32) ||
      overlap(out, out_bytes, bias, bias ? 2 * n : 0))
    return DQ_ERR_ALIAS;
  return hip_status(dq::launch_linear_mx(
      static_cast<const uint8_t*>(qa), static_cast<const uint8_t*>(sa), M, K,
      static_cast<const uint8_t*>(qw), static_cast<const uint8_t*>(sw), N,
      static_cast<const uint16_t*>(bias), epilogue == DQ_EPI_GELU_TANH ? 1 : 0,
      static_cast<uint16_t*>(out), static_cast<hipStream_t>(stream)));
}

int dq_quantize_mxfp4(const void* x, int64_t M, int64_t K, void* q, void* scales, void* stream) {
  if (M < 0 || M > kMaxDim || K < 32 || K > kMaxDim || (K % 32) != 0) return DQ_ERR_SHAPE;
  if (M > 0 && K > kMaxElems / M) return DQ_ERR_SHAPE;
  if (M == 0) return DQ_OK;
  if (!x || !q || !scales) return DQ_ERR_NULL;
  if (!aligned16(x) || !aligned16(q)) return DQ_ERR_ALIGN;
  const uint64_t n = static_cast<uint64_t>(M) * static_cast<uint64_t>(K);
  if (overlap(q, n / 2, x, 2 * n) || overlap(scales, n / 32, x, 2 * n) ||
      overlap(scales, n / 32, q, n / 2))
    return DQ_ERR_ALIAS;
  return hip_status(dq::launch_quantize_mxfp4(static_cast<const uint16_t*>(x), M, K,
                                              static_cast<uint8_t*>(q),
                                              static_cast<uint8_t*>(scales),
                                              static_cast<hipStream_t>(stream)));
}

// The checks of one MXFP4 segment (its weight, scales, bias and gate) with the shared
// row-indexed tensors, over all M rows.
static int check_mxfp4_args(const void* qa, const void* sa, int64_t M, int64_t K, const void* qw,
                            const void* sw, int64_t N, const void* bias, int epilogue,
                            const void* gate, const void* residual, const void* out) {
  const int shape = check_linear_shape(M, K, N);
  if (shape != DQ_OK) return shape;
  if ((K % 256) != 0) return DQ_ERR_SHAPE;  // a K step is 128 bytes of codes: 256 values
  if (epilogue != DQ_EPI_BIAS && epilogue != DQ_EPI_GELU_TANH &&
      epilogue != DQ_EPI_GATED_RESIDUAL)
    return DQ_ERR_EPILOGUE;
  const bool gated = epilogue == DQ_EPI_GATED_RESIDUAL;
  if (gated && (!gate || !residual)) return DQ_ERR_EPILOGUE;
  if (((M + 255) / 256) * ((N + 255) / 256) >= (int64_t(1) << 23)) return DQ_ERR_SHAPE;
  if (M == 0) return DQ_OK;
  if (!qa || !sa || !qw || !sw || !out) return DQ_ERR_NULL;
  if (!aligned16(qa) || !aligned16(qw) || !aligned16(out) || (bias && !aligned16(bias)) ||
      (gated && !aligned16(gate)) || (gated && !aligned16(residual)) ||
      (reinterpret_cast<uintptr_t>(sa) & 7u) != 0 || (reinterpret_cast<uintptr_t>(sw) & 7u) != 0)
    return DQ_ERR_ALIGN;
  const uint64_t m = static_cast<uint64_t>(M), k = static_cast<uint64_t>(K),
                 n = static_cast<uint64_t>(N);
  const uint64_t out_bytes = 2 * m * n;
  if (overlap(out, out_bytes, qa, m * k / 2) || overlap(out, out_bytes, sa, m * k / 32) ||
      overlap(out, out_bytes, qw, n * k / 2) || overlap(out, out_bytes, sw, n * k / 32) ||
      overlap(out, out_bytes, bias, bias ? 2 * n : 0) ||
      (gated && overlap(out, out_bytes, gate, 2 * n)))
    return DQ_ERR_ALIAS;
  if (gated && residual != out && overlap(out, out_bytes, residual, out_bytes)) return DQ_ERR_ALIAS;
  return DQ_OK;
}

int dq_linear_mxfp4_segmented(const void* qa, const void* sa, int64_t K, int64_t nseg,
                              const int64_t* seg_rows, const void* const* qw,
                              const void* const* sw, int64_t N, const void* const* bias,
                              int epilogue, const void* const* gate, const void* residual,
                              void* out, void* stream) {
  if (nseg < 1 || nseg > dq::kMaxSegments) return DQ_ERR_SHAPE;
  if (!seg_rows || !qw || !sw || !bias) return DQ_ERR_NULL;
  int64_t M = 0, tiles_m = 0;
  for (int64_t i = 0; i < nseg; ++i) {
    if (seg_rows[i] < 0 || seg_rows[i] > kMaxDim - M) return DQ_ERR_SHAPE;
    M += seg_rows[i];
    tiles_m += (seg_rows[i] + dq::kTileM - 1) / dq::kTileM;
  }
  const bool gated = epilogue == DQ_EPI_GATED_RESIDUAL;
  if (gated && !gate) return DQ_ERR_EPILOGUE;
  for (int64_t i = 0; i < nseg; ++i) {
    if (gated && !gate[i]) return DQ_ERR_EPILOGUE;
    const int st = check_mxfp4_args(qa, sa, M, K, qw[i], sw[i], N, bias[i], epilogue,
                                     gated ? gate[i] : nullptr, residual, out);
    if (st != DQ_OK) return st;
  }
  if (tiles_m * ((N + dq::kTileN - 1) / dq::kTileN) >= (int64_t(1) << 23)) return DQ_ERR_SHAPE;
  if (M == 0) return DQ_OK;
  const uint8_t* w[dq::kMaxSegments];
  const uint8_t* ws[dq::kMaxSegments];
  const uint16_t* b[dq::kMaxSegments];
  const uint16_t* g[dq::kMaxSegments];
  for (int64_t i = 0; i < nseg; ++i) {
    w[i] = static_cast<const uint8_t*>(qw[i]);
    ws[i] = static_cast<const uint8_t*>(sw[i]);
    b[i] = static_cast<const uint16_t*>(bias[i]);
    g[i] = gated ? static_cast<const uint16_t*>(gate[i]) : nullptr;
  }
  return hip_status(dq::launch_linear_mxfp4_segmented(
      static_cast<const uint8_t*>(qa), static_cast<const uint8_t*>(sa), nseg, seg_rows, K, w, ws,
      N, b, epilogue, g, static_cast<const uint16_t*>(residual), static_cast<uint16_t*>(out),
      static_cast<hipStream_t>(stream)));
}

int dq_linear_mxfp4(const void* qa, const void* sa, int64_t M, int64_t K, const void* qw,
                    const void* sw, int64_t N, const void* bias, int epilogue, const void* gate,
                    const void* residual, void* out, void* stream) {
  const void* w[1] = {qw};
  const void* s[1] = {sw};
  const void* b[1] = {bias};
  const void* g[1] = {gate};
  const int64_t rows[1] = {M};
  return dq_linear_mxfp4_segmented(qa, sa, K, 1, rows, w, s, N, b, epilogue, g, residual, out,
                                   stream);
}

uint64_t dq_attention_fp8_workspace_size(int64_t H, int64_t S) {
  if (check_attention_shape(H, S) != DQ_OK) return 0;
  return dq::attention_workspace_bytes(H, S);
}

uint64_t dq_linear_fp8_workspace_size(int64_t M, int64_t K, int64_t N) {
  if (check_linear_shape(M, K, N) != DQ_OK) return 0;
  return dq::linear_workspace_bytes(M, K, N);
}

const char* dq_status_string(int status) {
  switch (status) {
    case DQ_OK: return "ok";
    case DQ_ERR_NULL: return "a required pointer is NULL";
    case DQ_ERR_SHAPE: return "a size is out of range or breaks a multiple-of rule";
    case DQ_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case DQ_ERR_ALIAS: return "an output overlaps an input";
    case DQ_ERR_EPILOGUE: return "unknown epilogue, or gate/residual missing for the gated one";
    case DQ_ERR_HIP: return "a HIP runtime call failed";
    case DQ_ERR_WORKSPACE: return "workspace not 256-byte aligned";
    case DQ_ERR_VALUE: return "a scalar argument is out of range";
    default: return "unknown status";
  }
}

int dq_last_hip_error(void) { return g_last_hip_error; }

int dq_abi_version(void) { return 11; }

}  // extern "C"
