/*
 * dq.h -- C ABI of libdq: FP8 (OCP E4M3) dynamically quantized linear layers for AMD MI355X
 * (gfx950).
 *
 * The operation is the dynamically quantized linear layer of a FLUX-style diffusion
 * transformer:
 *   - weights and activations are brought to FP8 at run time so that the 8-bit matrix units do
 *     the GEMM (page "Solucion de WaveSpeed para Acelerar la Generacion de Imagenes
 *     FLUX.1-dev", section "Cuantizacion Dinamica FP8");
 *   - the model keeps bf16 tensors around an FP8 compute core (page "WaveSpeedAI X DataCrunch:
 *     Inferencia de Imagenes FLUX en Tiempo Real en B200", section "Marco de Inferencia
 *     Propietario": mixed BF16/FP8 precision);
 *   - the GEMM carries its epilogue fused (page "Accelerarea generarii de imagini cu FLUX 3
 *     Image Klein pe GPU-urile Blackwell NVIDIA", the paragraph after "Tabelul 1" on GEMMs with
 *     fused epilogues);
 *   - no host round trips and memory planned ahead of time (page "WaveSpeedAI X DataCrunch",
 *     section "Marco de Inferencia Propietario"): every call is asynchronous on the caller's
 *     stream, and the library allocates nothing.
 *
 * Readings taken where the pages are silent: one scale per row (token of x, output channel of
 * W); OCP E4M3 (largest finite 448); scale = amax / 448 and each code = E4M3(x / scale), both
 * divisions correctly rounded in fp32, rounding to nearest with ties to the even code and
 * saturation at +-448; an all-zero row gets scale 0 and signed-zero codes.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, owned by the caller, row-major and contiguous,
 *     16-byte aligned. bf16 tensors are passed as raw 16-bit storage, FP8 tensors as raw bytes.
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued on it and the call
 *     returns without waiting; nothing is allocated, freed or synchronized.
 *   - Arguments are checked on the host before anything is enqueued. On a failed check the call
 *     returns a nonzero DQ_ERR_* code and enqueues nothing. A failed kernel launch returns
 *     DQ_ERR_HIP and the HIP error code can be read with dq_last_hip_error(). Faults inside a
 *     kernel surface at the caller's next synchronization, as for any HIP kernel.
 *   - Calls are thread-safe; the library keeps no per-call state (a workspace passed to
 *     dq_linear_fp8 is the caller's, see there).
 *   - M = 0 is valid and enqueues nothing.
 */
#ifndef DQ_H
#define DQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum {
  DQ_OK = 0,
  DQ_ERR_NULL = 1,      /* a required pointer is NULL */
  DQ_ERR_SHAPE = 2,     /* a size is negative, too large, or breaks a multiple-of rule */
  DQ_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned */
  DQ_ERR_ALIAS = 4,     /* an output overlaps an input (other than out == residual) */
  DQ_ERR_EPILOGUE = 5,  /* unknown epilogue, or gate/residual missing for the gated one */
  DQ_ERR_HIP = 6,       /* a HIP runtime call failed; see dq_last_hip_error() */
  DQ_ERR_WORKSPACE = 7, /* workspace not 256-byte aligned */
  DQ_ERR_VALUE = 8      /* a scalar argument is out of range (eps <= 0, or not finite) */
};

/* Epilogues of dq_linear_fp8 (v = acc * scale[m] * w_scale[n] + bias[n]). */
enum {
  DQ_EPI_BIAS = 0,           /* out = bf16(v) */
  DQ_EPI_GELU_TANH = 1,      /* out = bf16(0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3)))) */
  DQ_EPI_GATED_RESIDUAL = 2  /* out = bf16(residual[m,n] + gate[n] * v) */
};

/*
 * dq_quantize_fp8 -- per-token dynamic FP8 quantization of activations.
 * Follows "Cuantizacion Dinamica FP8" (page "Solucion de WaveSpeed para Acelerar la Generacion
 * de Imagenes FLUX.1-dev"): scales are recomputed from the live tensor on every call.
 *
 *   x      bf16 [M, K]   input activations (read only)
 *   q      uint8 [M, K]  output E4M3 codes
 *   scale  float [M]     output per-row scale: scale[m] = fl32(max_k |x[m,k]| / 448)
 *   q[m,k] = E4M3_RNE_SAT(fl32(x[m,k] / scale[m])); a zero row gives scale 0 and codes 0x00/0x80
 *   (the sign bit of each x).
 * Requirements: 0 <= M < 2^31, 8 <= K < 2^31, K % 8 == 0, M*K < 2^47, x/q/scale 16-byte
 * aligned, q and scale not overlapping x or each other. Inputs must be finite (NaN/Inf inputs
 * give unspecified codes).
 */
int dq_quantize_fp8(const void* x, int64_t M, int64_t K, void* q, float* scale, void* stream);

/*
 * dq_quantize_weight_fp8 -- per-output-channel FP8 quantization of a weight W [N, K]
 * (row n = output channel n). The same arithmetic as dq_quantize_fp8, applied once when a
 * weight is loaded; the result (qw, w_scale) is what dq_linear_fp8 consumes.
 *
 *   w        bf16 [N, K]   weight (read only)
 *   qw       uint8 [N, K]  output E4M3 codes
 *   w_scale  float [N]     output per-channel scale
 * Requirements as dq_quantize_fp8 with M replaced by N.
 */
int dq_quantize_weight_fp8(const void* w, int64_t N, int64_t K, void* qw, float* w_scale,
                           void* stream);

/*
 * dq_linear_fp8 -- W8A8 GEMM with the dequant / bias / activation epilogue fused.
 * The GEMM with a fused epilogue follows the page "Accelerarea generarii de imagini cu FLUX 3
 * Image Klein pe GPU-urile Blackwell NVIDIA" (paragraph after "Tabelul 1").
 *
 *   q         uint8 [M, K]   activation codes (from dq_quantize_fp8)
 *   scale     float [M]      activation scales
 *   qw        uint8 [N, K]   weight codes (from dq_quantize_weight_fp8), K-contiguous
 *   w_scale   float [N]      weight scales
 *   bias      bf16 [N]       or NULL (= zero bias)
 *   epilogue  DQ_EPI_*
 *   gate      bf16 [N]       required iff epilogue == DQ_EPI_GATED_RESIDUAL, else ignored
 *   residual  bf16 [M, N]    required iff epilogue == DQ_EPI_GATED_RESIDUAL, else ignored;
 *                            may be the same pointer as out (in-place residual update)
 *   out       bf16 [M, N]    output
 *   workspace                NULL (workspace_bytes ignored), or workspace_bytes bytes of device
 *                            memory, 256-byte aligned, overlapping no other argument, whose
 *                            first 4096 bytes hold zeros (see below)
 *   acc[m,n] = sum_k dec(q[m,k]) * dec(qw[n,k]) accumulated by the FP8 matrix units into fp32;
 *   v = acc * scale[m] * w_scale[n] + bias[n], then the epilogue, rounded once to bf16 (nearest
 *   even).
 *
 * Work split: the output is cut into 256 x 256 tiles and each tile's K range into steps of 128.
 * Without a workspace every workgroup computes whole tiles. With one, the tiles left over after
 * the full rounds of whole tiles (one tile per compute unit per round) may each be cut along K
 * into 2 to 8 equal parts, when a cost model of the device says that is faster: each part is
 * summed in fp32 into the workspace and the last part of a tile to finish adds them up (in a
 * fixed order, so the result does not depend on timing) and applies the epilogue.
 * Workspace layout: bytes [0, 4096) are one arrival counter per cut tile, at the same place for
 * every problem; they must hold zeros before the first use, and every call that completes
 * leaves them at zero again, so one zero fill at allocation is enough and one workspace serves
 * calls of any size in turn. The 256 KiB partial tiles follow. workspace_bytes is a budget: the
 * library picks the fastest schedule whose partial tiles fit in it, so a workspace of
 * dq_linear_fp8_workspace_size(M, K, N) bytes gives the schedule it prefers, and a smaller one
 * (or none) a schedule that needs no more. Calls that may run concurrently (other streams,
 * overlapping graph nodes) must not share a workspace.
 *
 * Requirements: 0 <= M < 2^31, 128 <= K < 2^24 with K % 128 == 0, 64 <= N < 2^31 with
 * N % 64 == 0, all tensor pointers 16-byte aligned, out overlapping no input except
 * out == residual.
 */
int dq_linear_fp8(const void* q, const float* scale, int64_t M, int64_t K, const void* qw,
                  const float* w_scale, int64_t N, const void* bias, int epilogue,
                  const void* gate, const void* residual, void* out, void* workspace,
                  uint64_t workspace_bytes, void* stream);

/*
 * dq_linear_fp8_segmented -- dq_linear_fp8 over a token sequence made of row segments that each
 * have their own weight, in one launch. FLUX-dev is a hybrid of multimodal and parallel
 * transformer blocks (page "WaveSpeedAI X DataCrunch: Inferencia de Imagenes FLUX en Tiempo Real
 * en B200", section "FLUX-Dev"); the reading taken for its multimodal (double-stream) blocks is
 * the public architecture's: text and image tokens form one joint sequence for attention, but
 * every linear layer has one weight for the text tokens and another for the image tokens. One
 * call runs both: the text stream's few tiles then fill the compute units the image stream's
 * last round leaves idle, instead of running as a separate, mostly idle launch.
 *
 *   q, scale   uint8 [M, K] codes and float [M] scales of the whole sequence (dq_quantize_fp8
 *              quantizes each row on its own, so one call covers every segment)
 *   nseg       1 <= nseg <= 4 segments; seg_rows[s] >= 0 (HOST array) is the row count of
 *              segment s: rows [seg_rows[0] + ... + seg_rows[s - 1], + seg_rows[s]); M is their
 *              sum
 *   qw[s], w_scale[s], bias[s], gate[s]  HOST arrays of nseg DEVICE pointers: segment s's
 *              weight codes [N, K], scales [N], bias [N] (NULL = zero), gate [N] (required iff
 *              gated; gate itself may be NULL otherwise)
 *   epilogue, residual, out, workspace, workspace_bytes  as dq_linear_fp8, over all M rows
 * Row m of out is exactly what dq_linear_fp8 gives for that row with its segment's weight (a
 * tile never spans two segments).
 * Requirements: as dq_linear_fp8 for M, K, N and every segment's tensors; the preferred
 * workspace size is dq_linear_fp8_segmented_workspace_size(nseg, seg_rows, K, N).
 */
int dq_linear_fp8_segmented(const void* q, const float* scale, int64_t K, int64_t nseg,
                            const int64_t* seg_rows, const void* const* qw,
                            const float* const* w_scale, int64_t N, const void* const* bias,
                            int epilogue, const void* const* gate, const void* residual,
                            void* out, void* workspace, uint64_t workspace_bytes, void* stream);

/*
 * dq_linear_fp8_segmented_workspace_size -- dq_linear_fp8_workspace_size for a segmented call
 * (0 for invalid sizes).
 */
uint64_t dq_linear_fp8_segmented_workspace_size(int64_t nseg, const int64_t* seg_rows, int64_t K,
                                                int64_t N);

/*
 * dq_linear_fp8_noalloc -- dq_linear_fp8 for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). The same
 * arguments without a workspace, the same result, and no hipMalloc, hipFree or allocating
 * library call: in place of a caller workspace the K-cut schedule uses the library's own device
 * scratch, a static array of 4096 + 128 * 256 KiB bytes (32 MiB + 4 KiB) that each GPU the
 * library runs on holds until the process ends. The scratch bounds the schedule, not the
 * problem: a problem whose preferred cut would need more than the scratch holds runs the best
 * schedule that fits (whole tiles or narrow halves need none), so every size dq_linear_fp8
 * accepts is accepted and every size it rejects is rejected with the same status. Before a call
 * that cuts tiles the scratch's arrival counters are cleared by a small kernel on `stream`.
 * All calls on one GPU share its scratch: calls that may overlap on one GPU (several streams,
 * several host threads, overlapping graph nodes) race and must be serialized by the caller.
 */
int dq_linear_fp8_noalloc(const void* q, const float* scale, int64_t M, int64_t K,
                          const void* qw, const float* w_scale, int64_t N, const void* bias,
                          int epilogue, const void* gate, const void* residual, void* out,
                          void* stream);

/*
 * dq_linear_qkv_fp8 -- the attention input projection: the W8A8 GEMM of dq_linear_fp8 with an
 * epilogue that splits the output into queries, keys and values, normalizes queries and keys per
 * head and applies the rotary position embedding, all before the single rounding to bf16.
 * The page "Accelerarea generarii de imagini cu FLUX 3 Image Klein pe GPU-urile Blackwell NVIDIA"
 * names this fused epilogue (query/key/value projections with query/key normalization and
 * rotary position embeddings, in its paragraph on the PrimsTS GEMMs); it gives no formula, and
 * the reading taken is the FLUX-style attention input:
 *
 *   v[m, n] = acc[m, n] * scale[m] * w_scale[n] + bias[n],  n < N = 3 * heads * 128: the query,
 *             key and value of `heads` heads of 128 channels, in that order
 *   query / key head row r (128 channels):  r' = r / sqrt(mean(r^2) + eps) * norm_qk[0 / 1][:]
 *   then each channel pair (2i, 2i + 1):    (a, b) -> (cos a - sin b, sin a + cos b),
 *                                           cos = rope_cos[m, i], sin = rope_sin[m, i]
 *   value head rows unchanged
 *   out_q / out_k / out_v [head, m, c] = bf16 of the result (nearest even), head-major
 *
 *   q, scale, qw, w_scale  as dq_linear_fp8 (N = 3 * heads * 128)
 *   bias        bf16 [N] or NULL (= zero bias)
 *   norm_qk     bf16 [2][128]  query then key RMS-norm weights
 *   rope_cos    float [M][64]  cosine of the angle of token m and channel pair i
 *   rope_sin    float [M][64]  its sine
 *   eps         float          added to the mean square; finite and > 0 (else DQ_ERR_VALUE)
 *   out_q, out_k, out_v  bf16 [heads][M][128] each
 *   workspace, workspace_bytes  as dq_linear_fp8 (its preferred size is
 *                               dq_linear_fp8_workspace_size(M, K, N))
 *
 * Everything after the contraction is fp32; the head's mean square is summed in fp32.
 * Requirements: as dq_linear_fp8 for M, K and N = 3 * heads * 128 with 1 <= heads; every pointer
 * 16-byte aligned; no output overlapping an input, another output or the workspace.
 */
int dq_linear_qkv_fp8(const void* q, const float* scale, int64_t M, int64_t K, const void* qw,
                      const float* w_scale, int64_t heads, const void* bias, const void* norm_qk,
                      const float* rope_cos, const float* rope_sin, float eps, void* out_q,
                      void* out_k, void* out_v, void* workspace, uint64_t workspace_bytes,
                      void* stream);

/*
 * dq_linear_qkv_fp8_attn -- dq_linear_qkv_fp8 with every output leaving as the FP8 operands of
 * dq_attention_fp8: E4M3 codes with one scale per head row, written by the GEMM's epilogue in
 * place of the bf16 outputs. The fused query/key/value epilogue (page "Accelerarea generarii de
 * imagini cu FLUX 3 Image Klein pe GPU-urile Blackwell NVIDIA", its paragraph on the PrimsTS
 * GEMMs) meets the pages' FP8 attention (page "Optimizacion de la inferencia de FLUX 3 Image
 * Klein en GPUs NVIDIA Blackwell", section "Como funciona": query, key and value held in FP8);
 * the reading taken is that the handoff equals the unfused path exactly:
 *
 *   q8, q_scale = dq_quantize_fp8 of the bf16 queries dq_linear_qkv_fp8 gives, as
 *                 [heads * M] rows of 128 (codes [heads][M][128], scales [heads][M]);
 *   k8, k_scale   the same for the keys;
 *   vt8, v_scale  dq_quantize_v_fp8 of its bf16 values (codes transposed [heads][128][M],
 *                 scales [heads][M])
 *
 * so every code and scale is bit-identical to dq_linear_qkv_fp8 followed by those quantizers.
 * Other arguments, requirements and errors as dq_linear_qkv_fp8, and M % 16 == 0 (else
 * DQ_ERR_SHAPE; dq_attention_fp8 asks the same of S); all six outputs 16-byte aligned and
 * overlapping no input, no other output and no workspace.
 */
int dq_linear_qkv_fp8_attn(const void* q, const float* scale, int64_t M, int64_t K, const void* qw,
                           const float* w_scale, int64_t heads, const void* bias,
                           const void* norm_qk, const float* rope_cos, const float* rope_sin,
                           float eps, void* q8, float* q_scale, void* k8, float* k_scale, void* vt8,
                           float* v_scale, void* workspace, uint64_t workspace_bytes,
                           void* stream);

/*
 * dq_quantize_v_fp8 -- per-(head, token) FP8 quantization of attention values, codes written
 * transposed for dq_attention_fp8.
 *
 *   v        bf16 [H, S, 128]   values, one row of 128 channels per (head, token)
 *   vt       uint8 [H, 128, S]  E4M3 codes, keys contiguous per channel
 *   v_scale  float [H, S]       per-row scales
 *   Codes and scales of each row are exactly those of dq_quantize_fp8 on that row.
 * Queries and keys need no special form: dq_quantize_fp8 on the [H * S, 128] view gives their
 * codes [H, S, 128] and scales [H, S].
 * Requirements: 0 <= H < 65536, 0 <= S < 2^24 with S % 16 == 0, pointers 16-byte aligned, no
 * overlap. Inputs must be finite.
 */
int dq_quantize_v_fp8(const void* v, int64_t H, int64_t S, void* vt, float* v_scale,
                      void* stream);

/*
 * dq_attention_fp8 -- attention over FP8 queries, keys and values, one head at a time:
 *
 *   t[i, j] = (dec(q_i) q_scale_i) . (dec(k_j) k_scale_j) / sqrt(128)
 *   o_i     = sum_j softmax_j(t[i, :]) v_scale_j dec(v_j)          (no mask: every token sees all)
 *
 * The pages treat FP8 attention as the next lever after the quantized GEMMs (page "Accelerarea
 * generarii de imagini cu FLUX 3 Image Klein pe GPU-urile Blackwell NVIDIA": attention is about
 * 60 % of the DiT's time at 2048 x 2048; page "Optimizacion de la inferencia de FLUX 3 Image
 * Klein en GPUs NVIDIA Blackwell", section "Como funciona": query, key and value in FP8). They do
 * not write it out; the reading taken quantizes each (head, token) row as the linear layer's
 * activations, multiplies queries by keys on the FP8 matrix units (fp32 accumulation), keeps the
 * softmax in fp32 (base 2, online over blocks of keys) and rounds each weight times its value
 * scale to bf16 for a bf16 matrix product with the decoded values (exact in bf16).
 *
 *   q, k      uint8 [H, S, 128]  codes;  q_scale, k_scale  float [H, S]
 *   vt        uint8 [H, 128, S]  codes (from dq_quantize_v_fp8);  v_scale  float [H, S]
 *   out       bf16 [S, H, 128]   token-major (row s holds the H heads' outputs in order)
 *   workspace           NULL (workspace_bytes ignored), or device memory of at least
 *                       dq_attention_fp8_workspace_size(H, S) bytes, 256-byte aligned, overlapping
 *                       no other argument
 *   max_workgroups      0 for the default (one workgroup per compute unit, all resident at
 *                       once), or a lower cap on the workgroups launched
 *
 * Work split: a tile is 384 queries of one head against all S keys, in blocks of 64 keys. When
 * there are no more tiles than workgroups, each workgroup computes one tile. Otherwise, without a
 * workspace each workgroup computes a contiguous run of whole tiles; with one, the tiles' key
 * blocks are dealt out in equal contiguous runs, so a tile may be cut between two neighbouring
 * workgroups: the part that finishes first stores its unnormalized fp32 result and (running
 * max, sum) in the workspace (both do when they finish together), and the part that finishes
 * second merges the two in a fixed order (the result does not depend on timing; it can differ
 * in the last bits from an uncut run). The workspace must
 * hold zeros before its first use; every call that completes leaves its counters at zero, so one
 * zero fill at allocation is enough, and one workspace serves calls of any size up to the one it
 * was sized for. Calls that may run concurrently must not share a workspace.
 * Requirements: as dq_quantize_v_fp8; out overlapping no input; max_workgroups >= 0
 * (DQ_ERR_VALUE otherwise).
 */
int dq_attention_fp8(const void* q, const float* q_scale, const void* k, const float* k_scale,
                     const void* vt, const float* v_scale, int64_t H, int64_t S, void* out,
                     void* workspace, uint64_t workspace_bytes, int64_t max_workgroups,
                     void* stream);

/*
 * dq_quantize_mx_fp8 -- block-scaled (MX) FP8 quantization: every 32 consecutive values of a row
 * share one power-of-two scale.
 *
 * The pages run the linears in NVFP4 on Blackwell, a format with a shared scale per small block
 * (page "Accelerarea generarii de imagini cu FLUX 3 Image Klein pe GPU-urile Blackwell NVIDIA",
 * its paragraph on NVFP4 against BF16). The block format gfx950's matrix units execute is the
 * OCP Microscaling one; its definition with E4M3 elements is the one taken:
 *   shared exponent e = floor(log2(max |x| of the block)) - 8, clamped to [-127, 127]
 *                       (-127 for an all-zero block);
 *   q = E4M3 nearest to x / 2^e (ties to even), magnitudes past 448 saturating to 448;
 *   scale byte = e + 127 (E8M0).
 *
 *   x       bf16 [M, K]       row-major; 32 <= K < 2^31, K % 32 == 0, M K < 2^47
 *   q       uint8 [M, K]      codes
 *   scales  uint8 [M, K / 32] scale bytes, row-major
 * x and q 16-byte aligned; no overlap. Inputs must be finite.
 */
int dq_quantize_mx_fp8(const void* x, int64_t M, int64_t K, void* q, void* scales, void* stream);

/*
 * dq_linear_mx_fp8 -- the block-scaled linear layer on gfx950's scaled FP8 matrix instruction:
 *
 *   y[m, n] = sum over blocks b of 2^(ea[m, b] + ew[n, b]) sum_{k in b} dec(qa[m, k]) dec(qw[n, k])
 *   out[m, n] = bf16(epilogue(y[m, n] + bias[n]))      accumulation in fp32, one rounding
 *
 *   qa, sa   codes [M, K] and scale bytes [M, K / 32] of the activations (dq_quantize_mx_fp8)
 *   qw, sw   codes [N, K] and scale bytes [N, K / 32] of the weights (the same routine)
 *   bias     bf16 [N] or NULL;  epilogue DQ_EPI_BIAS or DQ_EPI_GELU_TANH
 *   out      bf16 [M, N]
 * Requirements: as dq_linear_fp8 (128 <= K < 2^24, K % 128 == 0, N % 64 == 0); codes, bias and
 * out 16-byte aligned, scale arrays 4-byte aligned; out overlapping no input; fewer than 2^23
 * output tiles of 256 x 256 (DQ_ERR_SHAPE otherwise).
 */
int dq_linear_mx_fp8(const void* qa, const void* sa, int64_t M, int64_t K, const void* qw,
                     const void* sw, int64_t N, const void* bias, int epilogue, void* out,
                     void* stream);

/*
 * dq_quantize_mxfp4 -- block-scaled FP4 (MXFP4) quantization: every 32 consecutive values of a
 * row share one power-of-two scale, each value is a 4-bit E2M1 code.
 *
 * The pages run FLUX 3 Image Klein's linears with 4-bit weights and activations and a shared
 * scale per small block (NVFP4, page "Accelerarea generarii de imagini cu FLUX 3 Image Klein pe
 * GPU-urile Blackwell NVIDIA", its paragraph on NVFP4 against BF16; page "Optimizacion de la
 * inferencia de FLUX 3 Image Klein en GPUs NVIDIA Blackwell", section "Como funciona"). The
 * 4-bit block format gfx950's matrix units execute is OCP MX with E2M1 elements (magnitudes
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7, sign in bit 3); its definition is the one taken:
 *   shared exponent e = floor(log2(max |x| of the block)) - 2, clamped to [-127, 127]
 *                       (-127 for an all-zero block);
 *   q = E2M1 nearest to x / 2^e (ties to the even code), magnitudes past 6 saturating to 6,
 *       the sign kept (also when the value rounds to zero);
 *   scale byte = e + 127 (E8M0).
 *
 *   x       bf16 [M, K]       row-major; 32 <= K < 2^31, K % 32 == 0, M K < 2^47
 *   q       uint8 [M, K / 2]  two codes per byte: element 2j in the low nibble of byte j
 *   scales  uint8 [M, K / 32] scale bytes, row-major
 * x and q 16-byte aligned; no overlap. Inputs must be finite.
 */
int dq_quantize_mxfp4(const void* x, int64_t M, int64_t K, void* q, void* scales, void* stream);

/*
 * dq_linear_mxfp4 -- the MXFP4 linear layer on gfx950's scaled matrix instruction with 4-bit
 * operands (twice the rate of its FP8 form):
 *
 *   y[m, n] = sum over blocks b of 2^(ea[m, b] + ew[n, b]) sum_{k in b} dec(qa[m, k]) dec(qw[n, k])
 *   v[m, n] = y[m, n] + bias[n]                          accumulation in fp32
 *   out[m, n] = bf16(v)                                  DQ_EPI_BIAS
 *             = bf16(gelu_tanh(v))                       DQ_EPI_GELU_TANH
 *             = bf16(residual[m, n] + gate[n] v)         DQ_EPI_GATED_RESIDUAL
 *
 *   qa, sa   codes [M, K / 2] and scale bytes [M, K / 32] of the activations (dq_quantize_mxfp4)
 *   qw, sw   codes [N, K / 2] and scale bytes [N, K / 32] of the weights (the same routine)
 *   bias     bf16 [N] or NULL;  gate bf16 [N] and residual bf16 [M, N] for the gated epilogue
 *            (ignored otherwise); out bf16 [M, N], which may be the residual itself
 * Requirements: 256 <= K < 2^24, K % 256 == 0, N % 64 == 0, fewer than 2^23 output tiles of
 * 256 x 256 (DQ_ERR_SHAPE otherwise); codes, bias, gate, residual and out 16-byte aligned, scale
 * arrays 8-byte aligned; out overlapping no input but the residual.
 */
int dq_linear_mxfp4(const void* qa, const void* sa, int64_t M, int64_t K, const void* qw,
                    const void* sw, int64_t N, const void* bias, int epilogue, const void* gate,
                    const void* residual, void* out, void* stream);

/*
 * dq_linear_mxfp4_segmented -- dq_linear_mxfp4 over a sequence of up to 4 row segments, each with
 * its own weight, in one launch: the MXFP4 form of dq_linear_fp8_segmented (a double-stream
 * block's text and image tokens, page "WaveSpeedAI X DataCrunch: Inferencia de Imagenes FLUX en
 * Tiempo Real en B200", section "FLUX-Dev").
 *
 *   qa, sa     codes [M, K / 2] and scale bytes [M, K / 32] of the whole sequence
 *   nseg       1 <= nseg <= 4; seg_rows[s] >= 0 (HOST array): the row count of segment s, M
 *              their sum
 *   qw[s], sw[s], bias[s], gate[s]  HOST arrays of nseg DEVICE pointers: segment s's codes
 *              [N, K / 2], scale bytes [N, K / 32], bias [N] (NULL = zero), gate [N] (gated only)
 *   epilogue, residual, out  as dq_linear_mxfp4, over all M rows
 * Row m of out is exactly what dq_linear_mxfp4 gives for that row with its segment's weight.
 */
int dq_linear_mxfp4_segmented(const void* qa, const void* sa, int64_t K, int64_t nseg,
                              const int64_t* seg_rows, const void* const* qw,
                              const void* const* sw, int64_t N, const void* const* bias,
                              int epilogue, const void* const* gate, const void* residual,
                              void* out, void* stream);

/*
 * dq_attention_fp8_workspace_size -- bytes of workspace dq_attention_fp8 may use for H heads of
 * S tokens, or 0 if the sizes break its requirements: 4 KiB of counters plus two 198 KiB partial
 * results per workgroup boundary, for at most min(H ceil(S / 384), 256) workgroups (at most
 * about 99 MiB). Needs no GPU.
 */
uint64_t dq_attention_fp8_workspace_size(int64_t H, int64_t S);

/*
 * dq_linear_fp8_workspace_size -- bytes of workspace the schedule dq_linear_fp8 (and
 * dq_linear_qkv_fp8, with N = 3 * heads * 128) prefers for an M x K -> N problem on the current
 * device: 0 when that schedule cuts no tile (then no workspace is needed), else 4096 bytes of
 * counters plus 256 KiB per part of the cut tiles. Returns 0 for sizes dq_linear_fp8 rejects.
 * It queries the current device's compute unit count (256 when no device is visible).
 */
uint64_t dq_linear_fp8_workspace_size(int64_t M, int64_t K, int64_t N);

/*
 * dq_layernorm_modulate_quantize_fp8 -- a DiT block's LayerNorm and modulation folded into the
 * per-token FP8 quantization of the next linear's input, in one pass over x:
 *
 *   n[m, k] = (x[m, k] - mean_m) / sqrt(var_m + eps)      mean, (biased) variance over k
 *   y[m, k] = bf16( n[m, k] * (1 + mod_scale[k]) + mod_shift[k] )
 *   scale[m], q[m, :] = per-row FP8 quantization of y, exactly as dq_quantize_fp8
 *
 * This is the kernel fusion that the page "Solucion de WaveSpeed para Acelerar la Generacion de
 * Imagenes FLUX.1-dev" lists among the fixes for high per-image latency (its lists of bottlenecks
 * and of the engine's innovations). The pages do not write the normalization out; the reading
 * taken is the FLUX-style block's: LayerNorm without learned weight or bias (eps = 1e-6 there)
 * and per-channel shift and scale from the block's modulation. The statistics and y are computed
 * in fp32 and y is rounded to bf16 (nearest even), the activation the unfused step would store;
 * the codes are a function of that bf16 y.
 *
 *   x          bf16 [M, K]  hidden states, one token per row
 *   mod_scale  bf16 [K]     per-channel modulation scale (y uses 1 + mod_scale)
 *   mod_shift  bf16 [K]     per-channel modulation shift
 *   eps        float        added to the variance; finite and > 0 (else DQ_ERR_VALUE: a row
 *                           of equal values would give 0/0)
 *   y_out      bf16 [M, K]  the modulated activation, or NULL to skip storing it
 *   q          uint8 [M, K] codes;  scale  fp32 [M] per-token scales (as dq_quantize_fp8)
 *
 * Requirements: 0 <= M < 2^31, 8 <= K <= 8192 with K % 8 == 0 (a row stays in registers), all
 * pointers 16-byte aligned, no output (y_out, q, scale) overlapping an input or another output.
 * Inputs must be finite and every modulated value must lie in bf16's finite range (the codes
 * are unspecified otherwise). M = 0 enqueues nothing.
 */
int dq_layernorm_modulate_quantize_fp8(const void* x, int64_t M, int64_t K, const void* mod_scale,
                                       const void* mod_shift, float eps, void* y_out, void* q,
                                       float* scale, void* stream);

/* Static English text for a status code (never NULL). */
const char* dq_status_string(int status);

/* The hipError_t behind the most recent DQ_ERR_HIP returned on the calling thread (0 if none). */
int dq_last_hip_error(void);

/* ABI version of this header (currently 11). */
int dq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DQ_H */
