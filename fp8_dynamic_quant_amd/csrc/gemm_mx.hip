// Block-scaled (MX) quantizers for gfx950: activations and weights in E4M3 (or E2M1) with one
// power-of-two scale (an E8M0 byte) per 32 values along K, multiplied by gfx950's scaled matrix
// instruction, which applies each operand's block scale itself.
//
// The pages run the linears in NVFP4 on Blackwell, a format with a shared scale per small block
// (page "Accelerarea generarii de imagini cu FLUX 3 Image Klein pe GPU-urile Blackwell NVIDIA",
// its paragraph on NVFP4 against BF16; page "Optimizacion de la inferencia de FLUX 3 Image Klein
// en GPUs NVIDIA Blackwell", section "Como funciona"). The block format gfx950 executes is the
// OCP Microscaling one; its definition with E4M3 elements is the one taken here:
//   shared exponent of a block = floor(log2(amax)) - 8, clamped to [-127, 127] (all-zero: -127),
//   element = E4M3 nearest (ties to even) to x / 2^shared, saturating at 448,
//   scale byte = shared + 127.
//
// quant_mx_rows: a thread takes 8 values (16 bytes) at a time, four chunks in flight; the 4
// threads of a block are a DPP quad.
// The block's amax is a bf16, so floor(log2(amax)) is its exponent field minus 127 (a zero or
// subnormal amax has field 0 and clamps to -127): the scale byte is max(field - 8, 0). x / 2^shared
// is a product by a power of two, exact in fp32 (below 2^-126 it may round, far under half of
// E4M3's smallest step), clamped to +-448 and converted by the hardware's nearest-even
// conversion.
//
// The block-scaled GEMM runs on the ping-pong kernel of gemm_fp8.hip in its MX mode: each K
// step's copy batches also bring the 4 scale bytes (one dword) of every A and B row, and the
// scaled instruction applies them. That instruction takes the 64 codes of a row in two blocks of
// 32: the first four registers of lanes l and l + 32 (the same row) make up the first block, the
// last four the second, and the first block is scaled by lane l's scale, the second by lane
// l + 32's (measured: with codes [32 (l >> 5), +32) in lane l, as for the unscaled instruction,
// codes 16-31 took the second block's scale). So lane l takes the 16-code chunks 4h + (l >> 5)
// and 4h + 2 + (l >> 5) of K half h, and the row's scale dword shifted right by 8 (l >> 5), whose
// byte 2h (the instruction's byte select) is then the scale of block 2h + (l >> 5).
#include "dq_internal.h"

namespace dq {
namespace {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------------------------
// quantizer
// ---------------------------------------------------------------------------------------------

__device__ __forceinline__ uint32_t absmax_pair(uint32_t acc, uint32_t w) {
  const u16x2 a = __builtin_bit_cast(u16x2, acc);
  const u16x2 b = __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}

// Two dwords of bf16 (4 values) times y, clamped to +-448, as four E4M3 codes.
__device__ __forceinline__ uint32_t encode4(uint32_t w0, uint32_t w1, float y) {
  float v[4] = {__uint_as_float(w0 << 16), __uint_as_float(w0 & 0xFFFF0000u),
                __uint_as_float(w1 << 16), __uint_as_float(w1 & 0xFFFF0000u)};
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = fminf(fmaxf(v[i] * y, -448.0f), 448.0f);
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], r, true);
  return (uint32_t)r;
}

// Thread t of a workgroup takes the 16-byte chunks u = 1024 b + 256 i + t, i = 0..3 (four loads
// in flight, non-temporal: x is read once); the 4 threads of an MX block are a DPP quad. A
// workgroup steps through chunk groups b = blockIdx.x, + gridDim.x, ... (at most kMaxGroups
// workgroups, so that any size fits a dispatch's 32-bit work-item count).
constexpr int kQuantUnroll = 4;
constexpr int64_t kMaxGroups = int64_t(1) << 20;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) quant_mx_rows(const uint16_t* __restrict__ x, int64_t n8,
                                                     uint8_t* __restrict__ q,
                                                     uint8_t* __restrict__ scale) {
  for (int64_t grp = blockIdx.x; grp * (256 * kQuantUnroll) < n8; grp += gridDim.x) {
    const int64_t base = grp * (256 * kQuantUnroll) + threadIdx.x;
    uint4 v[kQuantUnroll];
#pragma unroll
    for (int i = 0; i < kQuantUnroll; ++i) {
      const int64_t t = base + 256 * i;  // n8 is a multiple of 4: a quad is live or not as a whole
      if (t < n8) {
        const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x) + t);
        v[i] = make_uint4(r[0], r[1], r[2], r[3]);
      } else {
        v[i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int i = 0; i < kQuantUnroll; ++i) {
      const int64_t t = base + 256 * i;
      uint32_t mx = absmax_pair(absmax_pair(absmax_pair(absmax_pair(0u, v[i].x), v[i].y), v[i].z),
                                v[i].w);
      uint32_t m = (mx & 0xFFFFu) > (mx >> 16) ? (mx & 0xFFFFu) : (mx >> 16);
      uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false);
      m = m > o ? m : o;
      o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false);
      m = m > o ? m : o;
      if (t >= n8) continue;
      const uint32_t field = (m >> 7) & 0xFFu;            // bf16 exponent field of the block amax
      const uint32_t byte = field > 8u ? field - 8u : 0u;  // shared + 127
      const float y = __uint_as_float((254u - byte) << 23);  // 2^-shared (byte <= 246 for bf16)
      reinterpret_cast<uint2*>(q)[t] =
          make_uint2(encode4(v[i].x, v[i].y, y), encode4(v[i].z, v[i].w, y));
      if ((threadIdx.x & 3) == 0) scale[t >> 2] = (uint8_t)byte;
    }
  }
}

// MXFP4: the same blocks with E2M1 elements. Shared exponent floor(log2(amax)) - 2, so the scale
// byte is max(field - 2, 0); x / 2^shared is again a product by a power of two (values it pushes
// below fp32's range are under a quarter, E2M1's rounding point to zero, and keep their sign).
// The hardware's packed FP4 conversion rounds to the nearest E2M1 value with ties to even,
// saturates at 6 and keeps the sign of zero: it is used with scale 1 on the scaled values (it
// agrees bit for bit with that definition on every bf16 value, measured). Two codes per byte,
// element 2j in the low nibble of byte j: a thread's 8 values give one dword of codes.
template <int J>
__device__ __forceinline__ uint32_t cvt_fp4_pair(uint32_t r, uint32_t w, float y) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __uint_as_float(w << 16) * y,
                                                  __uint_as_float(w & 0xFFFF0000u) * y, 1.0f, J);
}

__global__ void __launch_bounds__(256) quant_mx4_rows(const uint16_t* __restrict__ x, int64_t n8,
                                                      uint32_t* __restrict__ q,
                                                      uint8_t* __restrict__ scale) {
  for (int64_t grp = blockIdx.x; grp * (256 * kQuantUnroll) < n8; grp += gridDim.x) {
    const int64_t base = grp * (256 * kQuantUnroll) + threadIdx.x;
    uint4 v[kQuantUnroll];
#pragma unroll
    for (int i = 0; i < kQuantUnroll; ++i) {
      const int64_t t = base + 256 * i;  // n8 is a multiple of 4: a quad is live or not as a whole
      if (t < n8) {
        const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x) + t);
        v[i] = make_uint4(r[0], r[1], r[2], r[3]);
      } else {
        v[i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int i = 0; i < kQuantUnroll; ++i) {
      const int64_t t = base + 256 * i;
      uint32_t mx = absmax_pair(absmax_pair(absmax_pair(absmax_pair(0u, v[i].x), v[i].y), v[i].z),
                                v[i].w);
      uint32_t m = (mx & 0xFFFFu) > (mx >> 16) ? (mx & 0xFFFFu) : (mx >> 16);
      uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false);
      m = m > o ? m : o;
      o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false);
      m = m > o ? m : o;
      if (t >= n8) continue;
      const uint32_t field = (m >> 7) & 0xFFu;            // bf16 exponent field of the block amax
      const uint32_t byte = field > 2u ? field - 2u : 0u;  // shared + 127
      const float y = __uint_as_float((254u - byte) << 23);  // 2^-shared (byte <= 252 for bf16)
      uint32_t r = cvt_fp4_pair<0>(0u, v[i].x, y);
      r = cvt_fp4_pair<1>(r, v[i].y, y);
      r = cvt_fp4_pair<2>(r, v[i].z, y);
      r = cvt_fp4_pair<3>(r, v[i].w, y);
      q[t] = r;
      if ((threadIdx.x & 3) == 0) scale[t >> 2] = (uint8_t)byte;
    }
  }
}

}  // namespace

hipError_t launch_quantize_mxfp4(const uint16_t* x, int64_t R, int64_t K, uint8_t* q,
                                 uint8_t* scale, hipStream_t stream) {
  const int64_t n8 = R * K / 8;
  if (n8 == 0) return hipSuccess;
  const int64_t per_wg = 256 * kQuantUnroll;
  const int64_t groups = (n8 + per_wg - 1) / per_wg;
  hipLaunchKernelGGL(quant_mx4_rows, dim3((unsigned)(groups < kMaxGroups ? groups : kMaxGroups)),
                     dim3(256), 0, stream, x, n8, reinterpret_cast<uint32_t*>(q), scale);
  return hipGetLastError();
}

hipError_t launch_quantize_mx(const uint16_t* x, int64_t R, int64_t K, uint8_t* q, uint8_t* scale,
                              hipStream_t stream) {
  const int64_t n8 = R * K / 8;
  if (n8 == 0) return hipSuccess;
  const int64_t per_wg = 256 * kQuantUnroll;
  const int64_t groups = (n8 + per_wg - 1) / per_wg;
  hipLaunchKernelGGL(quant_mx_rows, dim3((unsigned)(groups < kMaxGroups ? groups : kMaxGroups)),
                     dim3(256), 0, stream, x, n8, q, scale);
  return hipGetLastError();
}

}  // namespace dq
