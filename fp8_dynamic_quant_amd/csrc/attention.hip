// FP8 attention for gfx950: o = softmax(q k^T / sqrt(128)) v per head, over queries, keys and
// values quantized to OCP E4M3 with one scale per (head, token) row.
//
// The pages count quantized attention as the main lever once the linears are in FP8 (page
// "Accelerarea generarii de imagini cu FLUX 3 Image Klein pe GPU-urile Blackwell NVIDIA": attention
// is about 60 % of the DiT's GPU time at 2048 x 2048, with FP8 attention as the remedy; page
// "Optimizacion de la inferencia de FLUX 3 Image Klein en GPUs NVIDIA Blackwell", section "Como
// funciona": query, key and value held in FP8).
//
// Layouts: q, k codes [H, S, 128] and scales [H, S]; v codes transposed, [H, 128, S] (keys
// contiguous per channel, the order the P V matrix product reads), scales [H, S]; the output
// [S, H, 128] bf16, token-major (the input layout of the projection after attention).
//
// quant_v_t: one workgroup quantizes 64 tokens of one head (4 lanes per token, the row scale as
// dq_quantize_fp8 computes it, the same encoder) and writes the codes transposed through LDS.
//
// attn_fp8: one workgroup (4 waves) takes 128 queries of one head; wave w owns 32 of them and
// keeps their codes in registers. Keys come in blocks of 64, double-buffered in LDS:
//   * K codes by global -> LDS copies (16 bytes per lane), 16-byte chunk c of key row r stored
//     at slot c ^ ((r >> 1) & 7) so that 16 rows read at one offset hit 16 different slots;
//   * V codes through registers, decoded once per workgroup to bf16 (exact: every E4M3 value is
//     a bf16 value), stored [channel][key] with the same swizzle;
//   * the blocks' key and value scales.
// Per block and wave:
//   1. logits: 2 x 2 FP8 matrix ops (32 keys x 32 queries x 64 channels each, keys as the
//      first operand), so lane l holds query l & 31 and keys 8 g + 4 (l >> 5) + j;
//   2. online softmax in base 2: t = s sk_j (sq_i log2(e) / sqrt(128)); the row max takes the
//      lane and its partner l ^ 32; the running max m (and with it the output and the sum,
//      rescaled by 2^(m - m')) moves only when a block's max exceeds it by more than 8, so the
//      rescale is rare after the first blocks; p = 2^(t - m) <= 2^8; keys past S are masked;
//   3. P V: p sv_j rounded to bf16 becomes the second operand of 16 bf16 matrix ops (32
//      channels x 32 queries x 16 keys) after one half swap between partner lanes (the
//      logits' layout holds keys 0-3 and 8-11 of a 16-key chunk in the lower lane, 4-7 and 12-15
//      in the upper one; the operand wants 0-7 and 8-15);
// so the output accumulates transposed, [channel][query], 64 registers per lane. One workgroup
// barrier per block. At the end o / sum goes to bf16 and leaves as 16-byte stores.
#include "dq_internal.h"
#include "e4m3_codec.h"

#include <type_traits>

namespace dq {
namespace {

using namespace codec;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 bf8v __attribute__((ext_vector_type(8)));
typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));

constexpr int kD = kHeadDim;   // 128 channels per head
constexpr int kQB = 128;       // queries per workgroup
constexpr int kKB = 64;        // keys per block

// ---------------------------------------------------------------------------------------------
// value quantization, transposed
// ---------------------------------------------------------------------------------------------

// Wave w takes tokens 16 w + (l >> 2) of the tile; lane l holds channels [32 (l & 3), +32).
__global__ void __launch_bounds__(256) quant_v_t(const uint16_t* __restrict__ v, int S,
                                                 uint8_t* __restrict__ vt, float* __restrict__ sv) {
  constexpr int kRow = 80;  // bytes per channel row of the tile (64 tokens + padding, 16-aligned)
  __shared__ __attribute__((aligned(16))) uint8_t tile[kD * kRow];
  const int h = blockIdx.y, t0 = blockIdx.x * 64;
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int tl = 16 * w + (l >> 2), cg = l & 3;
  const int t = t0 + tl;
  const bool live = t < S;
  const uint4* src =
      reinterpret_cast<const uint4*>(v + ((size_t)h * (size_t)S + (size_t)(live ? t : 0)) * kD) +
      cg * 4;
  uint4 x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = live ? src[i] : make_uint4(0u, 0u, 0u, 0u);
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) mx = absmax4(mx, x[i]);
  uint32_t m = (mx & 0xFFFFu) > (mx >> 16) ? (mx & 0xFFFFu) : (mx >> 16);
  // the token's 4 lanes are a DPP quad
  uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false);
  m = m > o ? m : o;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false);
  m = m > o ? m : o;
  const float amax = __uint_as_float(m << 16);
  const float s = amax / kE4M3Max;
  uint2 c[4];
  if (m == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = signs8(x[i]);
  } else if (s < kFltMinNormal) {
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = encode8<1, false>(x[i], s, 0.0f);
  } else if (amax < kTinyAmax) {
    const float ss = s * 0x1p64f;
    const float y = 1.0f / ss;
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = encode8<0, true>(x[i], ss, y);
  } else {
    const float y = 1.0f / s;
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = encode8<0, false>(x[i], s, y);
  }
  if (cg == 0 && live) sv[(size_t)h * (size_t)S + t] = s;
  // channel 32 cg + 8 i + b of token tl -> tile[channel][tl]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t d[2] = {c[i].x, c[i].y};
#pragma unroll
    for (int b = 0; b < 8; ++b)
      tile[(32 * cg + 8 * i + b) * kRow + tl] = (uint8_t)(d[b >> 2] >> (8 * (b & 3)));
  }
  __syncthreads();
  // thread: channel tid >> 1, tokens 32 (tid & 1) + [0, 32) as two 16-byte chunks
  const int ch = threadIdx.x >> 1, hf = threadIdx.x & 1;
  uint8_t* dst = vt + ((size_t)h * kD + ch) * (size_t)S + t0 + 32 * hf;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (t0 + 32 * hf + 16 * i + 16 <= S)
      *reinterpret_cast<uint4*>(dst + 16 * i) =
          *reinterpret_cast<const uint4*>(tile + ch * kRow + 32 * hf + 16 * i);
  }
}

// ---------------------------------------------------------------------------------------------
// attention
// ---------------------------------------------------------------------------------------------

struct AttnArgs {
  const uint8_t* q8;   // [H, S, 128]
  const float* sq;     // [H, S]
  const uint8_t* k8;   // [H, S, 128]
  const float* sk;     // [H, S]
  const uint8_t* vt8;  // [H, 128, S]
  const float* sv;     // [H, S]
  uint16_t* out;       // [S, H, 128]
  int H, S;
  float c;             // log2(e) / sqrt(128)
};

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){a, b}, bf2v));
}

// Exchange a's value in lanes 32..63 with b's value in lanes 0..31.
__device__ __forceinline__ void swap_halves(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}
__device__ __forceinline__ void swap_halves(float& a, float& b) {
  uint32_t x = __float_as_uint(a), y = __float_as_uint(b);
  swap_halves(x, y);
  a = __uint_as_float(x);
  b = __uint_as_float(y);
}

// Key block kb (64 rows of 128 bytes) into an LDS stage: wave w fills 16-byte slots
// [128 w, 128 w + 128) with two copies; slot n is row n >> 3, position n & 7, which holds chunk
// (n & 7) ^ key(row). Rows past S read row S - 1 (their logits are masked).
__device__ __forceinline__ void copy_keys(const AttnArgs& a, int h, int kb, uint8_t* stage,
                                          int w, int l) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int n = w * 128 + i * 64 + l;
    const int r = n >> 3, p = n & 7;
    const int key = kb * kKB + r < a.S ? kb * kKB + r : a.S - 1;
    const uint8_t* src = a.k8 + ((size_t)h * (size_t)a.S + (size_t)key) * kD + swz(r, p) * 16;
    __builtin_amdgcn_global_load_lds(
        src, (__attribute__((address_space(3))) void*)(stage + (w * 128 + i * 64) * 16), 16, 0,
        0);
  }
}

// Value codes of block kb: thread tid takes channel tid >> 1, keys 32 (tid & 1) + [0, 32).
// S is a multiple of 16, so a 16-key chunk is either inside the sequence or past it (zeros).
__device__ __forceinline__ void load_values(const AttnArgs& a, int h, int kb, int tid,
                                            uint4 (&vr)[2]) {
  const int ch = tid >> 1, k0 = kb * kKB + 32 * (tid & 1);
  const uint8_t* row = a.vt8 + ((size_t)h * kD + ch) * (size_t)a.S;
#pragma unroll
  for (int i = 0; i < 2; ++i)
    vr[i] = k0 + 16 * i < a.S ? *reinterpret_cast<const uint4*>(row + k0 + 16 * i)
                              : make_uint4(0u, 0u, 0u, 0u);
}

// 8 codes (two dwords) -> 8 bf16: gfx950's scaled conversion, two codes per instruction, at
// scale 1 (exact; checked on the hardware for every code and both halves of a dword).
template <bool kHi>
__device__ __forceinline__ uint32_t decode2(uint32_t d) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d, 1.0f, kHi));
}
__device__ __forceinline__ uint4 decode8(uint32_t d0, uint32_t d1) {
  return make_uint4(decode2<false>(d0), decode2<true>(d0), decode2<false>(d1), decode2<true>(d1));
}

// The decoded values into an LDS stage, [channel][key] bf16, 128-byte rows, swizzled.
__device__ __forceinline__ void store_values(uint8_t* stage, int tid, const uint4 (&vr)[2]) {
  const int ch = tid >> 1, hf = tid & 1;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t d[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int chunk = 4 * hf + 2 * i + j;  // 8 keys = 16 bytes
      *reinterpret_cast<uint4*>(stage + ch * 128 + swz(ch, chunk) * 16) =
          decode8(d[2 * j], d[2 * j + 1]);
    }
  }
}

// Two waves per SIMD: without the bound the compiler spends 280 registers (one wave per SIMD);
// asking for three spills to scratch and measured slower.
__global__ void __launch_bounds__(256, 2) attn_fp8(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t sK[2][kKB * kD];      // 2 x 8 KiB codes
  __shared__ __attribute__((aligned(1024))) uint8_t sV[2][kD * kKB * 2];  // 2 x 16 KiB bf16
  __shared__ __attribute__((aligned(16))) float sSK[2][kKB];
  __shared__ __attribute__((aligned(16))) float sSV[2][kKB];
  const int h = blockIdx.y, q0 = blockIdx.x * kQB;
  const int tid = threadIdx.x, l = tid & 63, hi = l >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = a.S;
  const int qi = q0 + 32 * w + (l & 31);
  const bool qlive = qi < S;

  // this lane's query: channels [64 dh + 32 hi, +32) for the two 64-channel halves
  v8i qf[2];
  {
    const uint8_t* qrow = a.q8 + ((size_t)h * (size_t)S + (size_t)(qlive ? qi : 0)) * kD;
#pragma unroll
    for (int dh = 0; dh < 2; ++dh)
      qf[dh] = qlive ? *reinterpret_cast<const v8i*>(qrow + 64 * dh + 32 * hi) : (v8i){};
  }
  const float sqc = qlive ? a.sq[(size_t)h * (size_t)S + qi] * a.c : 0.0f;

  const int nblk = (S + kKB - 1) / kKB;
  // block 0 into stage 0
  {
    copy_keys(a, h, 0, sK[0], w, l);
    uint4 vr[2];
    load_values(a, h, 0, tid, vr);
    store_values(sV[0], tid, vr);
    if (tid < kKB) sSK[0][tid] = tid < S ? a.sk[(size_t)h * (size_t)S + tid] : 0.0f;
    else if (tid < 2 * kKB) sSV[0][tid - kKB] = tid - kKB < S ? a.sv[(size_t)h * (size_t)S + tid - kKB] : 0.0f;
  }

  float m = -__builtin_inff(), lsum = 0.0f;
  v16f o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = (v16f){};

  // One key block; kTail marks the last block when S is not a multiple of 64 (the only one whose
  // keys past S must take no weight), a separate instance so that full blocks carry no masking.
  auto step = [&](const int kb, auto tail_tag) {
    constexpr bool tail = decltype(tail_tag)::value;
    const int st = kb & 1;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's key copies of block kb
    __syncthreads();                     // every wave's copies and stores of block kb
    const bool more = kb + 1 < nblk;
    uint4 vr[2];
    float scn = 0.0f;
    if (more) {
      copy_keys(a, h, kb + 1, sK[st ^ 1], w, l);
      load_values(a, h, kb + 1, tid, vr);
      const int j = (kb + 1) * kKB + (tid & (kKB - 1));
      if (tid < 2 * kKB && j < S) scn = (tid < kKB ? a.sk : a.sv)[(size_t)h * (size_t)S + j];
    }
    // 1. logits, [key][query]
    v16f s[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      s[kh] = (v16f){};
      const int r = 32 * kh + (l & 31);
#pragma unroll
      for (int dh = 0; dh < 2; ++dh) {
        const int c0 = 4 * dh + 2 * hi;
        const uint4 lo = *reinterpret_cast<const uint4*>(sK[st] + r * kD + swz(r, c0) * 16);
        const uint4 up = *reinterpret_cast<const uint4*>(sK[st] + r * kD + swz(r, c0 + 1) * 16);
        const v8i kf = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                             (int)up.x, (int)up.y, (int)up.z, (int)up.w};
        s[kh] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf[dh], s[kh], 0, 0, 0, 0, 0,
                                                                0);
      }
    }
    // 2. softmax in base 2: u = s sk, t = u sqc (sqc >= 0, so max t = sqc max u); the running
    //    max m moves only when a block's max exceeds it by more than 8 (weights stay <= 2^8,
    //    harmless in fp32 and bf16), and the rescale runs only when some lane of the wave moved
    v16f (&u)[2] = s;  // u = s sk, in place
    float mxu = -__builtin_inff();
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 sk4 = *reinterpret_cast<const float4*>(&sSK[st][32 * kh + 8 * g + 4 * hi]);
        const float skv[4] = {sk4.x, sk4.y, sk4.z, sk4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) u[kh][4 * g + j] *= skv[j];
      }
    if constexpr (tail) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kb * kKB + 32 * kh + 8 * (v >> 2) + 4 * hi + (v & 3);
          if (key < S) mxu = fmaxf(mxu, u[kh][v]);
        }
    } else {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int v = 0; v < 16; ++v) mxu = fmaxf(mxu, u[kh][v]);
    }
    {
      float a0 = mxu, b0 = mxu;
      swap_halves(a0, b0);
      mxu = fmaxf(a0, b0);
    }
    const float mx = mxu * sqc;
    const bool move = mx > m + 8.0f;
    if (__builtin_amdgcn_ballot_w64(move) != 0) {
      const float mn = move ? mx : m;
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] *= alpha;
      m = mn;
    }
    float ps = 0.0f;
    uint32_t pk[2][4][2];  // bf16 pairs of p sv: [kh][g][j pair]
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 sv4 = *reinterpret_cast<const float4*>(&sSV[st][32 * kh + 8 * g + 4 * hi]);
        const float svv[4] = {sv4.x, sv4.y, sv4.z, sv4.w};
        float p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          p[j] = __builtin_amdgcn_exp2f(fmaf(u[kh][4 * g + j], sqc, -m));
          if constexpr (tail)
            if (kb * kKB + 32 * kh + 8 * g + 4 * hi + j >= S) p[j] = 0.0f;
          ps += p[j];
        }
        pk[kh][g][0] = pack_bf16(p[0] * svv[0], p[1] * svv[1]);
        pk[kh][g][1] = pack_bf16(p[2] * svv[2], p[3] * svv[3]);
      }
    {
      float a0 = ps, b0 = ps;
      swap_halves(a0, b0);
      ps = a0 + b0;
    }
    lsum += ps;
    // 3. P V
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int kh = kc >> 1, c2 = kc & 1;
      uint32_t x0 = pk[kh][2 * c2][0], x1 = pk[kh][2 * c2][1];
      uint32_t y0 = pk[kh][2 * c2 + 1][0], y1 = pk[kh][2 * c2 + 1][1];
      swap_halves(x0, y0);
      swap_halves(x1, y1);
      const bf8v pb = __builtin_bit_cast(bf8v, make_uint4(x0, x1, y0, y1));
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int r = 32 * db + (l & 31);
        const bf8v vf = *reinterpret_cast<const bf8v*>(sV[st] + r * 128 + swz(r, 2 * kc + hi) * 16);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, o[db], 0, 0, 0);
      }
    }
    if (more) {
      store_values(sV[st ^ 1], tid, vr);
      if (tid < kKB) sSK[st ^ 1][tid] = scn;
      else if (tid < 2 * kKB) sSV[st ^ 1][tid - kKB] = scn;
    }
  };
  const int nfull = S / kKB;
  for (int kb = 0; kb < nfull; ++kb) step(kb, std::false_type{});
  if (nfull < nblk) step(nfull, std::true_type{});

  // o / sum, [channel][query] -> out[query][h][channel]
  const float inv = 1.0f / lsum;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int gp = 0; gp < 2; ++gp) {
      float v0[4], v1[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v0[j] = o[db][(2 * gp) * 4 + j] * inv;
        v1[j] = o[db][(2 * gp + 1) * 4 + j] * inv;
        swap_halves(v0[j], v1[j]);
      }
      const uint4 ov = make_uint4(pack_bf16(v0[0], v0[1]), pack_bf16(v0[2], v0[3]),
                                  pack_bf16(v1[0], v1[1]), pack_bf16(v1[2], v1[3]));
      if (qlive)
        *reinterpret_cast<uint4*>(a.out + ((size_t)qi * (size_t)a.H + h) * kD + 32 * db + 16 * gp +
                                  8 * hi) = ov;
    }
}

}  // namespace

hipError_t launch_quantize_v(const uint16_t* v, int64_t H, int64_t S, uint8_t* vt, float* sv,
                             hipStream_t stream) {
  if (H == 0 || S == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_v_t, dim3((unsigned)((S + 63) / 64), (unsigned)H), dim3(256), 0, stream,
                     v, (int)S, vt, sv);
  return hipGetLastError();
}

hipError_t launch_attention(const uint8_t* q8, const float* sq, const uint8_t* k8, const float* sk,
                            const uint8_t* vt8, const float* sv, int64_t H, int64_t S,
                            uint16_t* out, hipStream_t stream) {
  if (H == 0 || S == 0) return hipSuccess;
  AttnArgs a;
  a.q8 = q8;
  a.sq = sq;
  a.k8 = k8;
  a.sk = sk;
  a.vt8 = vt8;
  a.sv = sv;
  a.out = out;
  a.H = (int)H;
  a.S = (int)S;
  a.c = 1.4426950408889634f / 11.313708498984761f;  // log2(e) / sqrt(128)
  hipLaunchKernelGGL(attn_fp8, dim3((unsigned)((S + kQB - 1) / kQB), (unsigned)H), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace dq
