// Internal declarations shared by the host layer and the kernel launchers of libdq.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace dq {

// Per-row FP8 quantization of a bf16 [R, K] matrix (activations per token, weights per output
// channel). Arguments are already validated. Returns the launch status.
hipError_t launch_quantize_rows(const uint16_t* x, int64_t R, int64_t K, uint8_t* q, float* scale,
                                hipStream_t stream);

// LayerNorm (no affine) + modulation + per-row FP8 quantization of a bf16 [R, K] matrix,
// K <= kMaxModulateK. y (bf16 [R, K]) is stored when non-null. Arguments are already validated.
constexpr int64_t kMaxModulateK = 8192;
hipError_t launch_ln_modulate_quantize(const uint16_t* x, int64_t R, int64_t K,
                                       const uint16_t* mod_scale, const uint16_t* mod_shift,
                                       float eps, uint16_t* y, uint8_t* q, float* scale,
                                       hipStream_t stream);

// ---------------------------------------------------------------------------------------------
// GEMM work split, shared by the size query (host only, no GPU needed) and the launchers.
//   tile = 256 x 256 outputs; step = 128 of K.
// With a workspace, the tiles left over after the full rounds of whole tiles may be cut into
// up to kMaxSplits parts along K (see gemm_fp8.hip). Workspace layout:
//   [0, kCounterBytes)                      one arrival counter per left-over tile (at most
//                                           kMaxCutTiles), zero between calls
//   [kCounterBytes, + parts * kPartialBytes) one 256 x 256 fp32 partial tile per part
// The counters sit at the same place for every problem, so one workspace serves calls of any
// size in turn; only they must hold zeros (the partial tiles are written before they are read).
// ---------------------------------------------------------------------------------------------
constexpr int64_t kTileM = 256, kTileN = 256, kStepK = 128;
constexpr int64_t kMaxParts = 1024;
constexpr int64_t kMaxSplits = 8;
constexpr int64_t kMaxCutTiles = 1024;
constexpr uint64_t kCounterBytes = 4 * kMaxCutTiles;
constexpr uint64_t kPartialBytes = kTileM * kTileN * 4;

inline int64_t linear_tiles(int64_t M, int64_t N) {
  return ((M + kTileM - 1) / kTileM) * ((N + kTileN - 1) / kTileN);
}
inline int64_t linear_units(int64_t M, int64_t K, int64_t N) {
  return linear_tiles(M, N) * (K / kStepK);
}

// Workspace bytes of the schedule the launcher picks for an M x K -> N problem on the current
// device when its workspace is unbounded: 0 when it cuts no tile, else kCounterBytes plus one
// partial tile per part. A smaller workspace makes the launcher pick the best schedule that
// fits in it.
uint64_t linear_workspace_bytes(int64_t M, int64_t K, int64_t N);

// FP8 GEMM + fused epilogue. Arguments are already validated; `workspace` is NULL or holds
// `workspace_bytes` bytes (counters zero). Returns the launch status.
hipError_t launch_linear(const uint8_t* q, const float* scale, int64_t M, int64_t K,
                         const uint8_t* qw, const float* w_scale, int64_t N, const uint16_t* bias,
                         int epilogue, const uint16_t* gate, const uint16_t* residual,
                         uint16_t* out, void* workspace, uint64_t workspace_bytes,
                         hipStream_t stream);

// The GEMM over nseg <= kMaxSegments row segments of q (seg_rows, a host array; segment s is
// rows [sum of seg_rows[< s], + seg_rows[s]) of q, scale, residual and out) each with its own
// weight, scales, bias and gate (host arrays of device pointers), in one launch. Arguments are
// already validated.
constexpr int64_t kMaxSegments = 4;
hipError_t launch_linear_segmented(const uint8_t* q, const float* scale, int64_t nseg,
                                   const int64_t* seg_rows, int64_t K,
                                   const uint8_t* const* qw, const float* const* w_scale,
                                   int64_t N, const uint16_t* const* bias, int epilogue,
                                   const uint16_t* const* gate, const uint16_t* residual,
                                   uint16_t* out, void* workspace, uint64_t workspace_bytes,
                                   hipStream_t stream);
// linear_workspace_bytes for a segmented problem.
uint64_t linear_segmented_workspace_bytes(int64_t nseg, const int64_t* seg_rows, int64_t K,
                                          int64_t N);

// The same GEMM with the library's own device scratch (kNoAllocScratchBytes per device, held
// until the process ends) in place of a caller workspace: nothing is allocated.
constexpr uint64_t kNoAllocParts = 128;
constexpr uint64_t kNoAllocScratchBytes = kCounterBytes + kNoAllocParts * kPartialBytes;
hipError_t launch_linear_noalloc(const uint8_t* q, const float* scale, int64_t M, int64_t K,
                                 const uint8_t* qw, const float* w_scale, int64_t N,
                                 const uint16_t* bias, int epilogue, const uint16_t* gate,
                                 const uint16_t* residual, uint16_t* out, hipStream_t stream);

// FP8 GEMM with the QKV epilogue: N = 3 heads kHeadDim; query and key RMS-normalized per head
// (weights norm_qk [2][kHeadDim]) and rotated pairwise by rope_cos/sin [M][kHeadDim / 2]; outputs
// out_q/k/v [heads][M][kHeadDim]. Arguments are already validated.
constexpr int64_t kHeadDim = 128;
hipError_t launch_linear_qkv(const uint8_t* q, const float* scale, int64_t M, int64_t K,
                             const uint8_t* qw, const float* w_scale, int64_t heads,
                             const uint16_t* bias, const uint16_t* norm_qk, const float* rope_cos,
                             const float* rope_sin, float eps, uint16_t* out_q, uint16_t* out_k,
                             uint16_t* out_v, void* workspace, uint64_t workspace_bytes,
                             hipStream_t stream);
// launch_linear_qkv with every output as E4M3 codes and one scale per head row [heads, M]:
// queries and keys [heads, M, 128], values transposed [heads, 128, M] (M % 16 == 0).
hipError_t launch_linear_qkv_q8(const uint8_t* q, const float* scale, int64_t M, int64_t K,
                                const uint8_t* qw, const float* w_scale, int64_t heads,
                                const uint16_t* bias, const uint16_t* norm_qk,
                                const float* rope_cos, const float* rope_sin, float eps,
                                uint8_t* q8, float* q_scale, uint8_t* k8, float* k_scale,
                                uint8_t* vt8, float* v_scale, void* workspace,
                                uint64_t workspace_bytes, hipStream_t stream);

// FP8 attention (attention.hip). S % 16 == 0 and 1 <= S, H.
//   launch_quantize_v: v bf16 [H, S, kHeadDim] -> codes transposed [H, kHeadDim, S], scales [H, S]
//   launch_attention:  q, k codes [H, S, kHeadDim] and scales [H, S], v as above ->
//                      out bf16 [S, H, kHeadDim]; workspace NULL or at least
//                      attention_workspace_bytes(H, S) bytes (zero before first use), max_workgroups
//                      0 (two per compute unit) or a lower cap
hipError_t launch_quantize_v(const uint16_t* v, int64_t H, int64_t S, uint8_t* vt, float* sv,
                             hipStream_t stream);
hipError_t launch_attention(const uint8_t* q8, const float* sq, const uint8_t* k8, const float* sk,
                            const uint8_t* vt8, const float* sv, int64_t H, int64_t S,
                            uint16_t* out, void* workspace, int64_t max_workgroups,
                            hipStream_t stream);
uint64_t attention_workspace_bytes(int64_t H, int64_t S);

// Block-scaled (MX) FP8 (gemm_mx.hip): E4M3 codes with one E8M0 scale byte per 32 values along K.
//   launch_quantize_mx: x bf16 [R, K] (K % 32 == 0) -> codes [R, K], scale bytes [R, K / 32]
//   launch_linear_mx:   codes and scale bytes of A [M, K] and W [N, K] (K % 128 == 0,
//                       N % 64 == 0), bias bf16 [N] or null, epilogue 0 bias / 1 GELU-tanh ->
//                       out bf16 [M, N]
hipError_t launch_quantize_mx(const uint16_t* x, int64_t R, int64_t K, uint8_t* q, uint8_t* scale,
                              hipStream_t stream);
hipError_t launch_linear_mx(const uint8_t* qa, const uint8_t* sa, int64_t M, int64_t K,
                            const uint8_t* qw, const uint8_t* sw, int64_t N, const uint16_t* bias,
                            int epilogue, uint16_t* out, hipStream_t stream);

// Block-scaled FP4 (MXFP4): E2M1 codes, two per byte (element 2j in the low nibble of byte j),
// with one E8M0 scale byte per 32 values along K.
//   launch_quantize_mxfp4: x bf16 [R, K] (K % 32 == 0) -> codes [R, K / 2], scales [R, K / 32]
//   launch_linear_mxfp4_segmented: codes [M, K / 2] and scales of A over nseg row segments, each
//                          with its own W codes [N, K / 2], scales, bias (or null) and gate
//                          (K % 256 == 0, N % 64 == 0); epilogue 0 bias / 1 GELU-tanh / 2 gated
//                          residual -> out bf16 [M, N]
hipError_t launch_quantize_mxfp4(const uint16_t* x, int64_t R, int64_t K, uint8_t* q,
                                 uint8_t* scale, hipStream_t stream);
hipError_t launch_linear_mxfp4_segmented(const uint8_t* qa, const uint8_t* sa, int64_t nseg,
                                         const int64_t* seg_rows, int64_t K,
                                         const uint8_t* const* qw, const uint8_t* const* sw,
                                         int64_t N, const uint16_t* const* bias, int epilogue,
                                         const uint16_t* const* gate, const uint16_t* residual,
                                         uint16_t* out, hipStream_t stream);
hipError_t launch_linear_mxfp4(const uint8_t* qa, const uint8_t* sa, int64_t M, int64_t K,
                               const uint8_t* qw, const uint8_t* sw, int64_t N,
                               const uint16_t* bias, int epilogue, uint16_t* out,
                               hipStream_t stream);

}  // namespace dq
