// Block-scaled (MX) FP8 linear layer for gfx950: activations and weights in E4M3 with one
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
// gemm_mx: a workgroup of 8 waves computes a 256 x 256 output tile in K steps of 128. Each step,
// the A and W tiles (256 rows x 128 codes each) and one dword of block scales per row (the
// step's four blocks) go straight from global memory into one of two LDS stages; a code row is
// stored as 8 chunks of 16 bytes, chunk c of row r at slot c ^ ((r >> 1) & 7), so that 16 rows
// read at one offset hit 16 different banks. Wave w computes rows 128 (w & 1) + [0, 128) by
// columns 64 (w >> 1) + [0, 64) with 4 x 2 blocks of the 32 x 32 x 64 scaled FP8 instruction per
// K half (weights as the first operand). The scaled instruction takes the 64 codes of a row in
// two blocks of 32: the first four registers of lanes l and l + 32 (the same row) make up the
// first block, the last four the second, and the first block is scaled by lane l's scale, the
// second by lane l + 32's (measured: with codes [32 (l >> 5), +32) in lane l, as for the
// unscaled instruction, codes 16-31 took the second block's scale). So lane l loads the 16-code
// chunks 4h + (l >> 5) and 4h + 2 + (l >> 5) of K half h, and the row's scale dword shifted right
// by 8 (l >> 5), whose byte 2h (the instruction's byte select) is then the scale of block
// 2h + (l >> 5). The epilogue adds the bias, applies the activation, rounds to bf16 and stores 8
// consecutive columns per lane after a half swap.
#include "dq_internal.h"

namespace dq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kBlk = 32;                           // values per MX block
constexpr int kTM = 256, kTN = 256, kTK = 128;     // output tile and K step
constexpr int kThreads = 512;
constexpr int kTileBytes = kTM * kTK;              // 32 KiB of codes per operand per stage
constexpr int kStageBytes = 2 * kTileBytes + 4 * (kTM + kTN);  // codes, then scale dwords
constexpr int kGroupM = 8;                         // tile rows per group in the tile order

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

// ---------------------------------------------------------------------------------------------
// GEMM
// ---------------------------------------------------------------------------------------------

struct MxArgs {
  const uint8_t* qa;     // [M, K] activation codes
  const uint8_t* sa;     // [M, K / 32] their scale bytes
  const uint8_t* qw;     // [N, K] weight codes
  const uint8_t* sw;     // [N, K / 32]
  const uint16_t* bias;  // bf16 [N] or null
  uint16_t* out;         // bf16 [M, N]
  int M, N, K;
  int tiles_m, tiles_n;
};

// Raw buffer descriptor over `bytes` bytes from `base`: reads past the end give zeros.
__device__ __forceinline__ v4i buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return (v4i){__builtin_amdgcn_readfirstlane((int)(uint32_t)b),
               __builtin_amdgcn_readfirstlane((int)((uint32_t)(b >> 32) & 0xFFFFu)),
               __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// 16 (or 4) bytes per lane from global memory straight into LDS at lds_base + 16 (4) * lane;
// the uniform LDS base travels in M0, saved and restored around the copy. The compiler does not
// see these as memory operations: the kernel waits for them itself (vmcnt) before its barrier.
__device__ __forceinline__ void copy16(v4i rsrc, uint32_t voff, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(lds_base)
      : "memory");
}
__device__ __forceinline__ void copy4(v4i rsrc, uint32_t voff, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "buffer_load_dword %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(lds_base)
      : "memory");
}

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){a, b}, bf2v));
}

// Exchange a's value in lanes 32..63 with b's value in lanes 0..31.
__device__ __forceinline__ void swap_halves(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// 0.5 v (1 + tanh(u)), u = sqrt(2/pi) (v + 0.044715 v^3), written as v / (1 + 2^(-2 u log2 e)).
__device__ __forceinline__ float gelu_tanh(float v) {
  constexpr float k0 = 2.3022082f;  // 2 sqrt(2/pi) / ln 2
  const float qq = fmaf(v * v, -k0 * 0.044715f, -k0);
  return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(qq * v));
}

template <int EPI>
__global__ void __launch_bounds__(kThreads, 1) gemm_mx(MxArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kStageBytes];
  const int tid = threadIdx.x, l = tid & 63, hi = l >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w & 1, wn = w >> 1;

  // tile of this workgroup: XCD-contiguous renumbering, then groups of kGroupM tile rows
  const int G = gridDim.x;
  const int t = (G & 7) == 0 ? (int)(blockIdx.x & 7u) * (G >> 3) + (int)(blockIdx.x >> 3)
                             : (int)blockIdx.x;
  const int per_group = kGroupM * a.tiles_n;
  const int first = (t / per_group) * kGroupM;
  const int gsz = a.tiles_m - first < kGroupM ? a.tiles_m - first : kGroupM;
  const int tm = first + (t % per_group) % gsz, tn = (t % per_group) / gsz;
  const int m0 = tm * kTM, n0 = tn * kTN;
  const uint32_t K = (uint32_t)a.K, KB = K / kBlk;
  const int rows_a = a.M - m0 < kTM ? a.M - m0 : kTM;
  const int rows_w = a.N - n0 < kTN ? a.N - n0 : kTN;
  const v4i rs_qa = buffer_rsrc(a.qa + (size_t)m0 * K, (uint32_t)rows_a * K);
  const v4i rs_qw = buffer_rsrc(a.qw + (size_t)n0 * K, (uint32_t)rows_w * K);
  // scale dwords: waves 0-3 copy the A rows', waves 4-7 the W rows'
  const v4i rs_sc = w < 4 ? buffer_rsrc(a.sa + (size_t)m0 * KB, (uint32_t)rows_a * KB)
                          : buffer_rsrc(a.sw + (size_t)n0 * KB, (uint32_t)rows_w * KB);
  // copy addressing: code slot n = 512 i + tid is row n >> 3, position n & 7
  const int crow = tid >> 3, cpos = tid & 7;  // + 64 i rows for copy i
  uint32_t coff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = crow + 64 * i;
    coff[i] = (uint32_t)r * K + (uint32_t)swz(r, cpos) * 16u;
  }
  const uint32_t soff = (uint32_t)(tid & (kTM - 1)) * KB;
  const uint32_t lds0 = lds_addr(lds);
  auto issue = [&](int k, int stage) {
    const uint32_t st = lds0 + (uint32_t)(stage * kStageBytes);
    const uint32_t kk = (uint32_t)k * kTK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t dst = st + (uint32_t)((512 * i + 64 * w) * 16);
      copy16(rs_qa, coff[i] + kk, __builtin_amdgcn_readfirstlane(dst));
      copy16(rs_qw, coff[i] + kk, __builtin_amdgcn_readfirstlane(dst + kTileBytes));
    }
    copy4(rs_sc, soff + (uint32_t)k * 4u,
          __builtin_amdgcn_readfirstlane(st + 2u * kTileBytes + (uint32_t)(256 * w)));
  };

  v16f acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (v16f){};

  const int nk = (int)(K / kTK);
  issue(0, 0);
  for (int k = 0; k < nk; ++k) {
    const uint8_t* st = lds + (k & 1) * kStageBytes;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies of step k
    __syncthreads();                     // everyone's copies of step k; step k - 1 read by all
    if (k + 1 < nk) issue(k + 1, (k + 1) & 1);
    const uint32_t* sc = reinterpret_cast<const uint32_t*>(st + 2 * kTileBytes);
    uint32_t sa4[4], sw2[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) sa4[i] = sc[wm * 128 + 32 * i + (l & 31)] >> (8 * hi);
#pragma unroll
    for (int i = 0; i < 2; ++i) sw2[i] = sc[kTM + wn * 64 + 32 * i + (l & 31)] >> (8 * hi);
    // both K halves' fragments first (their reads overlap), then the 16 matrix ops
    v8i fa[2][4], fw[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c0 = 4 * h + hi;  // chunks c0 (registers 0-3) and c0 + 2 (registers 4-7)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 128 + 32 * i + (l & 31);
        const uint4 lo = *reinterpret_cast<const uint4*>(st + r * kTK + swz(r, c0) * 16);
        const uint4 up = *reinterpret_cast<const uint4*>(st + r * kTK + swz(r, c0 + 2) * 16);
        fa[h][i] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                         (int)up.x, (int)up.y, (int)up.z, (int)up.w};
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wn * 64 + 32 * i + (l & 31);
        const uint8_t* wt = st + kTileBytes;
        const uint4 lo = *reinterpret_cast<const uint4*>(wt + r * kTK + swz(r, c0) * 16);
        const uint4 up = *reinterpret_cast<const uint4*>(wt + r * kTK + swz(r, c0 + 2) * 16);
        fw[h][i] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                         (int)up.x, (int)up.y, (int)up.z, (int)up.w};
      }
    }
    // the byte select (2h) is an immediate of the instruction
#pragma unroll
    for (int bn = 0; bn < 2; ++bn)
#pragma unroll
      for (int bm = 0; bm < 4; ++bm)
        acc[bn][bm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            fw[0][bn], fa[0][bm], acc[bn][bm], 0, 0, 0, (int)sw2[bn], 0, (int)sa4[bm]);
#pragma unroll
    for (int bn = 0; bn < 2; ++bn)
#pragma unroll
      for (int bm = 0; bm < 4; ++bm)
        acc[bn][bm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            fw[1][bn], fa[1][bm], acc[bn][bm], 0, 0, 2, (int)sw2[bn], 2, (int)sa4[bm]);
  }

  // epilogue: lane holds output row m (its column in the instruction's layout) and columns
  // 32 bn + 8 g + 4 hi + j of the wave's 64. The four 16-byte stores that cover a row's 64
  // columns (one 128-byte line) are issued back to back.
  float bv[2][2][8];
#pragma unroll
  for (int bn = 0; bn < 2; ++bn)
#pragma unroll
    for (int gp = 0; gp < 2; ++gp) {
      const int n = n0 + wn * 64 + 32 * bn + 16 * gp + 8 * hi;
      if (a.bias && n < a.N) {
        const uint4 b4 = *reinterpret_cast<const uint4*>(a.bias + n);
        const uint32_t bw[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bv[bn][gp][2 * j] = __uint_as_float(bw[j] << 16);
          bv[bn][gp][2 * j + 1] = __uint_as_float(bw[j] & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) bv[bn][gp][j] = 0.0f;
      }
    }
  // N is a multiple of 64: a wave's 64 columns are all in or all out
  if (n0 + wn * 64 < a.N) {
#pragma unroll
    for (int bm = 0; bm < 4; ++bm) {
      const int m = m0 + wm * 128 + 32 * bm + (l & 31);
#pragma unroll
      for (int bn = 0; bn < 2; ++bn)
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
          const int n = n0 + wn * 64 + 32 * bn + 16 * gp + 8 * hi;
          float v0[4], v1[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v0[j] = acc[bn][bm][(2 * gp) * 4 + j];
            v1[j] = acc[bn][bm][(2 * gp + 1) * 4 + j];
            swap_halves(v0[j], v1[j]);
          }
          float y[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            y[j] += bv[bn][gp][j];
            if (EPI == 1) y[j] = gelu_tanh(y[j]);
          }
          if (m < a.M)
            *reinterpret_cast<uint4*>(a.out + (size_t)m * (size_t)a.N + n) =
                make_uint4(pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]), pack_bf16(y[4], y[5]),
                           pack_bf16(y[6], y[7]));
        }
    }
  }
}

}  // namespace

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

hipError_t launch_linear_mx(const uint8_t* qa, const uint8_t* sa, int64_t M, int64_t K,
                            const uint8_t* qw, const uint8_t* sw, int64_t N, const uint16_t* bias,
                            int epilogue, uint16_t* out, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  MxArgs a;
  a.qa = qa;
  a.sa = sa;
  a.qw = qw;
  a.sw = sw;
  a.bias = bias;
  a.out = out;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.tiles_m = (int)((M + kTM - 1) / kTM);
  a.tiles_n = (int)((N + kTN - 1) / kTN);
  const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
  if (epilogue == 1)
    hipLaunchKernelGGL(gemm_mx<1>, dim3((unsigned)tiles), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(gemm_mx<0>, dim3((unsigned)tiles), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dq
