// Per-row dynamic FP8 (OCP E4M3) quantization for gfx950.
//
// One wavefront owns one row. Each lane loads its share of the row as 16-byte chunks (8 bf16)
// straight into registers, so the row is read from HBM exactly once:
//   1. amax: |bf16| compares like its 15 magnitude bits read as an unsigned integer (finite
//      inputs), so the running max is a packed 16-bit integer max; then a wavefront butterfly.
//   2. scale = amax / 448 (IEEE division, correctly rounded).
//   3. code = E4M3(fl32(x / scale)), then the hardware conversion v_cvt_pk_fp8_f32, which rounds
//      to nearest-even into OCP E4M3. That conversion does not saturate (inputs above 464
//      become NaN), but x / scale <= 448 (1 + 2^-23) whenever the scale is a normal fp32, which
//      rounds to 448. The quotient is not formed by a division per element but by Markstein's
//      correction of a reciprocal product (Muller et al., Handbook of Floating-Point
//      Arithmetic, division by FMA): y = fl32(1 / scale) once per row, q = fl32(x y),
//      r = fma(-q, scale, x) (exact), q' = fma(r, y, q). For every bf16 amax with a normal
//      scale and every bf16 |x| <= amax, E4M3(q') == E4M3(fl32(x / scale)); this was checked
//      by exhaustion over all 531,921,744 such pairs, with rows whose amax is below 2^-60
//      working on x 2^64 and scale 2^64 (the same quotient, and no subnormal residual). The
//      chain is odd in x, except that x = -0 gives +0, so the result takes the sign of x.
//      Rows with a subnormal scale divide per element and clamp the quotient to +-448.
//   4. An all-zero row stores scale 0 and copies each sign bit into its code.
// Codes leave as 8-byte stores (one per 16-byte input chunk), consecutive lanes on consecutive
// addresses. The scheme follows the dynamic FP8 quantization of weights and activations on the
// page "Solucion de WaveSpeed para Acelerar la Generacion de Imagenes FLUX.1-dev", section
// "Cuantizacion Dinamica FP8", with one scale per row.
#include "dq_internal.h"
#include "e4m3_codec.h"

namespace dq {
namespace {

using namespace codec;

__device__ __forceinline__ uint32_t wave_max(uint32_t m) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t o = (uint32_t)__shfl_xor((int)m, off, 64);
    m = m > o ? m : o;
  }
  return m;
}


typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16 bytes of x, read once: a non-temporal load, so the stream of activations does not push the
// codes (which the GEMM reads next) and the weights out of the caches.
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(r[0], r[1], r[2], r[3]);
}

// Workgroups of a row-group grid: at most this many are launched and each steps through row
// groups b, b + gridDim.x, ..., so that any row count fits the 32-bit work-item count of a
// dispatch.
constexpr int64_t kMaxRowGroups = int64_t(1) << 20;

// Register-resident version: WPR waves share a row (4 / WPR rows per 256-thread workgroup); lane
// l of the row's wave p holds chunks 64 p + l + 64 WPR i, i < NCH, loaded once. Each wave takes
// its chunks' magnitude max; with WPR > 1 the row's waves combine theirs through LDS (two
// buffers, so one barrier per row group suffices).
template <int NCH, int WPR>
__global__ void __launch_bounds__(256) quant_rows_reg(const uint16_t* __restrict__ x, int R, int K,
                                                      uint8_t* __restrict__ q,
                                                      float* __restrict__ scale) {
  constexpr int kRows = 4 / WPR;
  __shared__ uint32_t smax[2][4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rl = w / WPR, part = w % WPR;
  const int C = K >> 3;
  int it = 0;
  for (int64_t grp = blockIdx.x; grp * kRows < R; grp += gridDim.x, ++it) {
    const int64_t row = grp * kRows + rl;
    const bool live = row < R;
    const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)(live ? row : 0) * (size_t)K);
    uint2* qr = reinterpret_cast<uint2*>(q + (size_t)(live ? row : 0) * (size_t)K);
    uint4 v[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = part * 64 + lane + 64 * WPR * i;
      v[i] = (live && c < C) ? load_nt(xr + c) : make_uint4(0u, 0u, 0u, 0u);
    }
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < NCH; ++i) mx = absmax4(mx, v[i]);
    uint32_t m = (mx & 0xFFFFu) > (mx >> 16) ? (mx & 0xFFFFu) : (mx >> 16);
    m = wave_max(m);
    if (WPR > 1) {
      if (lane == 0) smax[it & 1][w] = m;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < WPR; ++j) {
        const uint32_t o = smax[it & 1][rl * WPR + j];
        m = m > o ? m : o;
      }
    }
    m = __builtin_amdgcn_readfirstlane(m);
    if (!live) continue;
    const float amax = __uint_as_float(m << 16);
    const float s = amax / kE4M3Max;
    if (lane == 0 && part == 0) scale[row] = s;
    if (m == 0) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = part * 64 + lane + 64 * WPR * i;
        if (c < C) qr[c] = signs8(v[i]);
      }
    } else if (s < kFltMinNormal) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = part * 64 + lane + 64 * WPR * i;
        if (c < C) qr[c] = encode8<1, false>(v[i], s, 0.0f);
      }
    } else if (amax < kTinyAmax) {
      const float ss = s * 0x1p64f;
      const float y = 1.0f / ss;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = part * 64 + lane + 64 * WPR * i;
        if (c < C) qr[c] = encode8<0, true>(v[i], ss, y);
      }
    } else {
      const float y = 1.0f / s;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = part * 64 + lane + 64 * WPR * i;
        if (c < C) qr[c] = encode8<0, false>(v[i], s, y);
      }
    }
  }
}

// One row, any K: two passes over it (the second pass usually hits in L2).
__device__ __forceinline__ void quant_row_loop(const uint16_t* __restrict__ x, int64_t row, int K,
                                               uint8_t* __restrict__ q, float* __restrict__ scale,
                                               int lane) {
  const int C = K >> 3;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)row * (size_t)K);
  uint2* qr = reinterpret_cast<uint2*>(q + (size_t)row * (size_t)K);
  uint32_t mx = 0;
  for (int c = lane; c < C; c += 64) mx = absmax4(mx, xr[c]);
  uint32_t m = (mx & 0xFFFFu) > (mx >> 16) ? (mx & 0xFFFFu) : (mx >> 16);
  m = __builtin_amdgcn_readfirstlane(wave_max(m));
  const float amax = __uint_as_float(m << 16);
  const float s = amax / kE4M3Max;
  if (lane == 0) scale[row] = s;
  if (m == 0) {
    for (int c = lane; c < C; c += 64) qr[c] = signs8(xr[c]);
  } else if (s < kFltMinNormal) {
    for (int c = lane; c < C; c += 64) qr[c] = encode8<1, false>(xr[c], s, 0.0f);
  } else if (amax < kTinyAmax) {
    const float ss = s * 0x1p64f;
    const float y = 1.0f / ss;
    for (int c = lane; c < C; c += 64) qr[c] = encode8<0, true>(xr[c], ss, y);
  } else {
    const float y = 1.0f / s;
    for (int c = lane; c < C; c += 64) qr[c] = encode8<0, false>(xr[c], s, y);
  }
}

__global__ void __launch_bounds__(256) quant_rows_loop(const uint16_t* __restrict__ x, int R, int K,
                                                       uint8_t* __restrict__ q,
                                                       float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < R;
       row += (int64_t)gridDim.x * 4)
    quant_row_loop(x, row, K, q, scale, lane);
}

// ---------------------------------------------------------------------------------------------
// LayerNorm + modulation + quantization of one row per wave (the row stays in registers)
// ---------------------------------------------------------------------------------------------

// Wave-wide reductions without LDS round trips: DPP moves combine lanes inside each 16-lane row
// (quad_perm swaps of 1 and 2 lanes, then the half-row and row mirrors), after which every lane of
// a row holds the same row total; the four row totals are read into scalar registers and combined
// in a fixed order, so every lane returns the same value.
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float row_sum16(float v) {
  v += __builtin_bit_cast(float, dpp<0xB1>(__builtin_bit_cast(int, v)));   // lanes ^ 1
  v += __builtin_bit_cast(float, dpp<0x4E>(__builtin_bit_cast(int, v)));   // lanes ^ 2
  v += __builtin_bit_cast(float, dpp<0x141>(__builtin_bit_cast(int, v)));  // half-row mirror
  v += __builtin_bit_cast(float, dpp<0x140>(__builtin_bit_cast(int, v)));  // row mirror
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t m) {
  m = umax(m, (uint32_t)dpp<0xB1>((int)m));
  m = umax(m, (uint32_t)dpp<0x4E>((int)m));
  m = umax(m, (uint32_t)dpp<0x141>((int)m));
  m = umax(m, (uint32_t)dpp<0x140>((int)m));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)m, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)m, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)m, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)m, 48);
  return umax(umax(r0, r1), umax(r2, r3));
}

typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){a, b}, bf2v));
}

// y for one 8-value chunk: (((x - mean0) - c) rstd) (1 + s) + t, rounded to bf16.
__device__ __forceinline__ uint4 modulate8(uint4 v, uint4 ms, uint4 mt, float mean0, float c,
                                           float rstd) {
  const uint32_t xv[4] = {v.x, v.y, v.z, v.w};
  const uint32_t sv[4] = {ms.x, ms.y, ms.z, ms.w};
  const uint32_t tv[4] = {mt.x, mt.y, mt.z, mt.w};
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float n0 = ((bf16_lo(xv[j]) - mean0) - c) * rstd;
    const float n1 = ((bf16_hi(xv[j]) - mean0) - c) * rstd;
    const float y0 = __builtin_fmaf(n0, 1.0f + bf16_lo(sv[j]), bf16_lo(tv[j]));
    const float y1 = __builtin_fmaf(n1, 1.0f + bf16_hi(sv[j]), bf16_hi(tv[j]));
    o[j] = pack2_bf16(y0, y1);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// One row per wave, four rows per workgroup; lane l holds chunks l, l + 64, ... of its row (NCH
// per lane, K <= 512 NCH). The workgroup's four rows share one copy of the modulation vectors in
// LDS. Every sum is fp32: each lane adds
// its values in order, then wave_sum.
//   1. mean0 = (sum of the row) / K. Its rounding error grows with |mean|, so
//   2. with e = x - mean0 (exact for x near mean0), c = (sum of e) / K and
//      var = (sum of e^2) / K - c^2, both sums in one pass: c is tiny next to the row's spread,
//      so nothing cancels, and d = e - c is accurate relative to the spread rather than to |mean|
//      (rows with a large common offset keep their variance); rstd = 1 / sqrt(var + eps), IEEE;
//   3. y = (d rstd) (1 + s) + t with one fma, rounded to bf16 in place of x;
//   4. the bf16 row y is quantized exactly as quant_rows_reg does (amax, scale, codes).
// Waves past the last row still take part in the workgroup barrier and store nothing.
template <int NCH, bool kStoreY>
__global__ void __launch_bounds__(256) ln_mod_quant_rows(
    const uint16_t* __restrict__ x, int R, int K, const uint16_t* __restrict__ mscale,
    const uint16_t* __restrict__ mshift, float eps, uint16_t* __restrict__ y,
    uint8_t* __restrict__ q, float* __restrict__ scale) {
  constexpr int kFill = (64 * NCH + 255) / 256;  // chunks of each vector per thread
  __shared__ uint4 smod[2][256 * kFill];
  const int lane = threadIdx.x & 63;
  const int C = K >> 3;
  // The modulation vectors go straight to LDS (16 bytes per lane, lane l of wave w at slot
  // 256 f + 64 w + l), issued before the first row's loads; they serve every row group the
  // workgroup takes. Slots past the row read chunk 0 and are never used.
  {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int f = 0; f < kFill; ++f) {
      const int c = threadIdx.x + 256 * f < C ? threadIdx.x + 256 * f : 0;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint4*>(mscale) + c,
                                       (__attribute__((address_space(3))) void*)&smod[0][256 * f + 64 * w],
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint4*>(mshift) + c,
                                       (__attribute__((address_space(3))) void*)&smod[1][256 * f + 64 * w],
                                       16, 0, 0);
    }
  }
  bool first = true;
  for (int64_t grp = blockIdx.x; grp * 4 < R; grp += gridDim.x) {
    const int64_t row = grp * 4 + (threadIdx.x >> 6);
    const bool live = row < R;
    const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)(live ? row : 0) * (size_t)K);
    uint4 v[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane + 64 * i;
      v[i] = (live && c < C) ? load_nt(xr + c) : make_uint4(0u, 0u, 0u, 0u);
    }
    // 1. first mean (chunks past the row are zeros and add nothing)
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) sum = (sum + bf16_lo(w[j])) + bf16_hi(w[j]);
    }
    const float mean0 = wave_sum(sum) / (float)K;
    // 2. correction and variance, over the row's own values only (chunks past it give e = 0)
    float es = 0.0f, ss = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const float m = lane + 64 * i < C ? mean0 : 0.0f;
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float e0 = bf16_lo(w[j]) - m, e1 = bf16_hi(w[j]) - m;
        es = (es + e0) + e1;
        ss = __builtin_fmaf(e0, e0, ss);
        ss = __builtin_fmaf(e1, e1, ss);
      }
    }
    const float corr = wave_sum(es) / (float)K;
    const float m2 = wave_sum(ss) / (float)K;
    const float var = __builtin_fmaxf(__builtin_fmaf(-corr, corr, m2), 0.0f);
    const float rstd = 1.0f / __builtin_sqrtf(var + eps);
    if (first) {                           // the same for every wave of the workgroup
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies have landed
      __syncthreads();                     // and every other wave's
      first = false;
    }
    // 3. y in bf16, in place of x
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane + 64 * i;
      if (c < C) v[i] = modulate8(v[i], smod[0][c], smod[1][c], mean0, corr, rstd);
    }
    if (!live) continue;
    if (kStoreY) {
      uint4* yr = reinterpret_cast<uint4*>(y + (size_t)row * (size_t)K);
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = lane + 64 * i;
        if (c < C) yr[c] = v[i];
      }
    }
    // 4. per-row quantization of the bf16 y (chunks past the row are zeros)
    uint2* qr = reinterpret_cast<uint2*>(q + (size_t)row * (size_t)K);
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < NCH; ++i) mx = absmax4(mx, v[i]);
    uint32_t m = (mx & 0xFFFFu) > (mx >> 16) ? (mx & 0xFFFFu) : (mx >> 16);
    m = wave_max_dpp(m);
    const float amax = __uint_as_float(m << 16);
    const float s = amax / kE4M3Max;
    if (lane == 0) scale[row] = s;
    if (m == 0) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = lane + 64 * i;
        if (c < C) qr[c] = signs8(v[i]);
      }
    } else if (s < kFltMinNormal) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = lane + 64 * i;
        if (c < C) qr[c] = encode8<1, false>(v[i], s, 0.0f);
      }
    } else if (amax < kTinyAmax) {
      const float ss2 = s * 0x1p64f;
      const float yy = 1.0f / ss2;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = lane + 64 * i;
        if (c < C) qr[c] = encode8<0, true>(v[i], ss2, yy);
      }
    } else {
      const float yy = 1.0f / s;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = lane + 64 * i;
        if (c < C) qr[c] = encode8<0, false>(v[i], s, yy);
      }
    }
  }
}

// Rows of at most 128 values (16 chunks): four rows per wave, one 16-lane DPP row each (lane
// l & 15 holds chunk l & 15 of row 4 (wave index) + (l >> 4)), so no lane idles. The scale and
// the codes are exactly quant_rows_reg's.
__global__ void __launch_bounds__(256) quant_rows_small(const uint16_t* __restrict__ x, int R,
                                                        int K, uint8_t* __restrict__ q,
                                                        float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, C = K >> 3;
  for (int64_t grp = blockIdx.x; grp * 16 < R; grp += gridDim.x) {
    const int64_t row = (grp * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
    const bool live = row < R && c < C;
    const uint4 v = live ? load_nt(reinterpret_cast<const uint4*>(x + (size_t)row * (size_t)K) + c)
                         : make_uint4(0u, 0u, 0u, 0u);
    uint32_t mx = absmax4(0u, v);
    uint32_t m = (mx & 0xFFFFu) > (mx >> 16) ? (mx & 0xFFFFu) : (mx >> 16);
    m = umax(m, (uint32_t)dpp<0xB1>((int)m));
    m = umax(m, (uint32_t)dpp<0x4E>((int)m));
    m = umax(m, (uint32_t)dpp<0x141>((int)m));
    m = umax(m, (uint32_t)dpp<0x140>((int)m));
    if (row >= R) continue;
    const float amax = __uint_as_float(m << 16);
    const float s = amax / kE4M3Max;
    if (c == 0) scale[row] = s;
    if (c >= C) continue;
    uint2 code;
    if (m == 0) {
      code = signs8(v);
    } else if (s < kFltMinNormal) {
      code = encode8<1, false>(v, s, 0.0f);
    } else if (amax < kTinyAmax) {
      const float ss = s * 0x1p64f;
      code = encode8<0, true>(v, ss, 1.0f / ss);
    } else {
      code = encode8<0, false>(v, s, 1.0f / s);
    }
    reinterpret_cast<uint2*>(q + (size_t)row * (size_t)K)[c] = code;
  }
}

// Workgroups for `groups` row groups: one per group, at most kMaxRowGroups.
inline dim3 group_grid(int64_t groups) {
  return dim3((unsigned)(groups < kMaxRowGroups ? groups : kMaxRowGroups));
}

template <int NCH>
hipError_t launch_lnmq(const uint16_t* x, int R, int K, const uint16_t* ms, const uint16_t* mt,
                       float eps, uint16_t* y, uint8_t* q, float* scale, hipStream_t st) {
  const dim3 grid = group_grid(((int64_t)R + 3) / 4);
  if (y)
    hipLaunchKernelGGL((ln_mod_quant_rows<NCH, true>), grid, dim3(256), 0, st, x, R, K, ms, mt,
                       eps, y, q, scale);
  else
    hipLaunchKernelGGL((ln_mod_quant_rows<NCH, false>), grid, dim3(256), 0, st, x, R, K, ms, mt,
                       eps, y, q, scale);
  return hipGetLastError();
}

template <int NCH, int WPR>
hipError_t launch_reg(const uint16_t* x, int R, int K, uint8_t* q, float* scale, hipStream_t st) {
  constexpr int kRows = 4 / WPR;
  hipLaunchKernelGGL((quant_rows_reg<NCH, WPR>), group_grid(((int64_t)R + kRows - 1) / kRows),
                     dim3(256), 0, st, x, R, K, q, scale);
  return hipGetLastError();
}

}  // namespace

// Rows of up to 128 values: four rows per wave. Otherwise one, two or four waves per row (a
// row's 16-byte chunks spread over 64, 128 or 256 lanes, at most 8 per lane up to 8192 values,
// 16 up to 32768), so that each lane keeps few chunks in flight and every row of a large launch
// is resident at once (measured: 4608 x 15360 in 38 us with four waves per row, 48 us with one);
// longer rows take two passes.
hipError_t launch_quantize_rows(const uint16_t* x, int64_t R, int64_t K, uint8_t* q, float* scale,
                                hipStream_t stream) {
  if (R == 0) return hipSuccess;
  const int r = (int)R, k = (int)K;
  const int64_t C = K / 8;  // 16-byte chunks per row
  if (K <= 128) {
    hipLaunchKernelGGL(quant_rows_small, group_grid((R + 15) / 16), dim3(256), 0, stream, x, r, k,
                       q, scale);
    return hipGetLastError();
  }
  if (C <= 64) return launch_reg<1, 1>(x, r, k, q, scale, stream);
  if (C <= 128) return launch_reg<2, 1>(x, r, k, q, scale, stream);
  if (C <= 256) return launch_reg<4, 1>(x, r, k, q, scale, stream);
  if (C <= 384) return launch_reg<3, 2>(x, r, k, q, scale, stream);
  if (C <= 512) return launch_reg<4, 2>(x, r, k, q, scale, stream);
  if (C <= 768) return launch_reg<6, 2>(x, r, k, q, scale, stream);
  if (C <= 1024) return launch_reg<8, 2>(x, r, k, q, scale, stream);
  if (C <= 1536) return launch_reg<6, 4>(x, r, k, q, scale, stream);
  if (C <= 2048) return launch_reg<8, 4>(x, r, k, q, scale, stream);
  if (C <= 3072) return launch_reg<12, 4>(x, r, k, q, scale, stream);
  if (C <= 4096) return launch_reg<16, 4>(x, r, k, q, scale, stream);
  hipLaunchKernelGGL(quant_rows_loop, group_grid((R + 3) / 4), dim3(256), 0, stream, x, r, k, q,
                     scale);
  return hipGetLastError();
}

hipError_t launch_ln_modulate_quantize(const uint16_t* x, int64_t R, int64_t K,
                                       const uint16_t* mod_scale, const uint16_t* mod_shift,
                                       float eps, uint16_t* y, uint8_t* q, float* scale,
                                       hipStream_t stream) {
  if (R == 0) return hipSuccess;
  const int r = (int)R, k = (int)K;
  const int64_t nch = (K / 8 + 63) / 64;  // 16-byte chunks per lane; K <= 8192 gives <= 16
  if (nch <= 1) return launch_lnmq<1>(x, r, k, mod_scale, mod_shift, eps, y, q, scale, stream);
  if (nch <= 2) return launch_lnmq<2>(x, r, k, mod_scale, mod_shift, eps, y, q, scale, stream);
  if (nch <= 4) return launch_lnmq<4>(x, r, k, mod_scale, mod_shift, eps, y, q, scale, stream);
  if (nch <= 6) return launch_lnmq<6>(x, r, k, mod_scale, mod_shift, eps, y, q, scale, stream);
  if (nch <= 8) return launch_lnmq<8>(x, r, k, mod_scale, mod_shift, eps, y, q, scale, stream);
  if (nch <= 12) return launch_lnmq<12>(x, r, k, mod_scale, mod_shift, eps, y, q, scale, stream);
  return launch_lnmq<16>(x, r, k, mod_scale, mod_shift, eps, y, q, scale, stream);
}

}  // namespace dq
