// FP8 (OCP E4M3) x FP8 GEMM with the dequant / bias / activation epilogue fused, for gfx950.
//
//   out[m, n] = epi( (sum_k dec(q[m, k]) dec(qw[n, k])) * scale[m] * w_scale[n] + bias[n] )
//
// Both operands are K-contiguous ("TN"), which is the operand layout the CDNA4 matrix cores
// read, so no transposition happens anywhere.
//
// Work decomposition (one workgroup = 4 wavefronts = 256 threads, one per SIMD):
//   * workgroup tile 256 (M) x 256 (N), K consumed 128 bytes at a time;
//   * each K step stages the A tile (256 x 128 B) and the B tile (256 x 128 B) in LDS, double
//     buffered (2 x 64 KiB); global loads for step k+1 are in flight while step k computes;
//   * LDS rows are 128 B; the 16-byte chunk c of row r is stored at chunk position c ^ (r & 7),
//     so the 8 lanes that read 8 consecutive rows at the same K offset hit 8 different chunks;
//   * wavefront (wm, wn) owns a 128 x 128 sub-tile: 4 x 4 blocks of 32 x 32 computed with
//     V_MFMA_F32_32X32X64_F8F6F4, 2 instructions per block per K step, fp32 accumulators;
//   * the weight fragment is the instruction's first operand and the activation fragment the
//     second, so each lane ends up holding 4 consecutive output columns of one output row:
//     the epilogue stores 4 bf16 (8 bytes) per lane per group.
//   * tiles are numbered so that the workgroups resident on one XCD (hardware dispatch sends
//     workgroup i to XCD i mod 8) cover a compact block of output tiles, and share A and B
//     panels in that XCD's L2.
//
// The FP8 GEMM with a fused epilogue follows the page "Accelerarea generarii de imagini cu
// FLUX 3 Image Klein pe GPU-urile Blackwell NVIDIA" (paragraph after "Tabelul 1"); the 8-bit
// matrix units fed with dynamically quantized weights and activations follow the page
// "Solucion de WaveSpeed para Acelerar la Generacion de Imagenes FLUX.1-dev", section
// "Cuantizacion Dinamica FP8".
#include "dq_internal.h"

namespace dq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256, kBK = 128;
constexpr int kThreads = 256;
constexpr int kStageBytes = (kBM + kBN) * kBK;  // 64 KiB
constexpr int kGroupM = 4;                      // tile rows per group in the tile order

enum { EPI_BIAS = 0, EPI_GELU_TANH = 1, EPI_GATED_RESIDUAL = 2 };

struct EpiArgs {
  const float* sa;           // [M]
  const float* sw;           // [N]
  const uint16_t* bias;      // [N] or null
  const uint16_t* gate;      // [N]
  const uint16_t* residual;  // [M, N]
  uint16_t* out;             // [M, N]
};

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kBK + ((chunk ^ (row & 7)) << 4);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// 0.5 v (1 + tanh(u)) = v / (1 + exp(-2u)), u = sqrt(2/pi) (v + 0.044715 v^3).
__device__ __forceinline__ float gelu_tanh(float v) {
  const float u = 0.7978845608028654f * fmaf(0.044715f * v, v * v, v);
  return v / (1.0f + __expf(-2.0f * u));
}

template <int EPI>
__device__ __forceinline__ void epilogue_store(const v16f (&acc)[4][4], const EpiArgs& ea, int M,
                                               int N, int mbase, int nbase, int lane) {
#pragma unroll
  for (int bm = 0; bm < 4; ++bm) {
    const int m = mbase + bm * 32 + (lane & 31);
    if (m >= M) continue;
    const float sam = ea.sa[m];
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = nbase + bn * 32 + g * 8 + (lane >> 5) * 4;
        if (n >= N) continue;
        const float4 swv = *reinterpret_cast<const float4*>(ea.sw + n);
        float b[4] = {0.f, 0.f, 0.f, 0.f};
        if (ea.bias) {
          const uint2 bb = *reinterpret_cast<const uint2*>(ea.bias + n);
          b[0] = bf16_to_f32(bb.x & 0xFFFFu);
          b[1] = bf16_to_f32(bb.x >> 16);
          b[2] = bf16_to_f32(bb.y & 0xFFFFu);
          b[3] = bf16_to_f32(bb.y >> 16);
        }
        const float swa[4] = {swv.x, swv.y, swv.z, swv.w};
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v = fmaf(acc[bn][bm][g * 4 + j] * sam, swa[j], b[j]);
          if (EPI == EPI_GELU_TANH) {
            y[j] = gelu_tanh(v);
          } else {
            y[j] = v;
          }
        }
        const size_t off = (size_t)m * (size_t)N + (size_t)n;
        if (EPI == EPI_GATED_RESIDUAL) {
          const uint2 gg = *reinterpret_cast<const uint2*>(ea.gate + n);
          const uint2 rr = *reinterpret_cast<const uint2*>(ea.residual + off);
          y[0] = fmaf(bf16_to_f32(gg.x & 0xFFFFu), y[0], bf16_to_f32(rr.x & 0xFFFFu));
          y[1] = fmaf(bf16_to_f32(gg.x >> 16), y[1], bf16_to_f32(rr.x >> 16));
          y[2] = fmaf(bf16_to_f32(gg.y & 0xFFFFu), y[2], bf16_to_f32(rr.y & 0xFFFFu));
          y[3] = fmaf(bf16_to_f32(gg.y >> 16), y[3], bf16_to_f32(rr.y >> 16));
        }
        uint2 o;
        o.x = f32_to_bf16(y[0]) | (f32_to_bf16(y[1]) << 16);
        o.y = f32_to_bf16(y[2]) | (f32_to_bf16(y[3]) << 16);
        *reinterpret_cast<uint2*>(ea.out + off) = o;
      }
    }
  }
}

// One K step on a staged pair of tiles: 2 x (4 + 4 fragment reads, 16 MFMAs) per wavefront.
__device__ __forceinline__ void mma_stage(const uint8_t* __restrict__ st, v16f (&acc)[4][4],
                                          const int (&fr_off)[2][2], int wm, int wn) {
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    v8i fb[4], fa[4];
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) {
      const uint8_t* base = st + kBM * kBK + (wn * 128 + bn * 32) * kBK;
      const uint4 lo = *reinterpret_cast<const uint4*>(base + fr_off[kh][0]);
      const uint4 hi = *reinterpret_cast<const uint4*>(base + fr_off[kh][1]);
      fb[bn] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int bm = 0; bm < 4; ++bm) {
      const uint8_t* base = st + (wm * 128 + bm * 32) * kBK;
      const uint4 lo = *reinterpret_cast<const uint4*>(base + fr_off[kh][0]);
      const uint4 hi = *reinterpret_cast<const uint4*>(base + fr_off[kh][1]);
      fa[bm] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int bn = 0; bn < 4; ++bn)
#pragma unroll
      for (int bm = 0; bm < 4; ++bm)
        acc[bn][bm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[bn], fa[bm], acc[bn][bm],
                                                                       0, 0, 0, 0, 0, 0);
  }
}

typedef __attribute__((address_space(3))) void* lptr_t;

// Raw buffer descriptor over `bytes` bytes from `base`; loads past the end return zeros (or
// leave their LDS slot untouched) and never fault.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Wait until this wavefront's global->LDS copies have landed (vmcnt = 0; lgkm/exp unchanged).
__device__ __forceinline__ void wait_lds_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Global -> LDS without registers: each buffer_load_dwordx4 ... lds of a wavefront fills 1 KiB
// of LDS (8 rows of 128 B); lane l lands in slot l, i.e. row l >> 3, chunk position l & 7, so
// it fetches the global chunk (l & 7) ^ (row & 7) of that row. Wavefront w fills rows
// [64 w, 64 w + 64) of both tiles with 8 + 8 instructions.
__device__ __forceinline__ void stage_load(uint8_t* __restrict__ st, __amdgpu_buffer_rsrc_t ra,
                                           __amdgpu_buffer_rsrc_t rb, uint32_t voff, uint32_t K,
                                           int wave) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t off = voff + (uint32_t)j * 8u * K;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lptr_t)(st + (wave * 64 + j * 8) * kBK), 16, off,
                                             0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rb, (lptr_t)(st + kBM * kBK + (wave * 64 + j * 8) * kBK), 16, off, 0, 0, 0);
  }
}

template <int EPI>
__global__ void __launch_bounds__(kThreads) gemm_fp8_256x256(const uint8_t* __restrict__ A,
                                                             const uint8_t* __restrict__ B, int M,
                                                             int N, int K, EpiArgs ea, int tilesM,
                                                             int tilesN) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[kStageBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- tile index: contiguous tile ranges per XCD, grouped order inside ----
  const int T = tilesM * tilesN;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, loc = bid >> 3;
  const int per = T >> 3, rem = T & 7;
  const int t = xcd * per + (xcd < rem ? xcd : rem) + loc;
  const int per_group = kGroupM * tilesN;
  const int grp = t / per_group;
  const int first_m = grp * kGroupM;
  const int gsz = (tilesM - first_m) < kGroupM ? (tilesM - first_m) : kGroupM;
  const int tin = t - grp * per_group;
  const int tm = first_m + tin % gsz;
  const int tn = tin / gsz;
  const int m0 = tm * kBM, n0 = tn * kBN;

  // ---- per-tile buffer descriptors: rows past M (N) are out of range ----
  const uint32_t rowsA = (uint32_t)(M - m0 < kBM ? M - m0 : kBM);
  const uint32_t rowsB = (uint32_t)(N - n0 < kBN ? N - n0 : kBN);
  const __amdgpu_buffer_rsrc_t rsA = buffer_rsrc(A + (size_t)m0 * (size_t)K, rowsA * (uint32_t)K);
  const __amdgpu_buffer_rsrc_t rsB = buffer_rsrc(B + (size_t)n0 * (size_t)K, rowsB * (uint32_t)K);
  const uint32_t voff0 =
      (uint32_t)(wave * 64 + (lane >> 3)) * (uint32_t)K + (uint32_t)(((lane & 7) ^ ((lane >> 3) & 7)) * 16);

  // ---- LDS -> fragment offsets ----
  // lane reads row (lane & 31) of a 32-row block, bytes [32 (lane >> 5) + 64 kh, +32)
  int fr_off[2][2];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int h = 0; h < 2; ++h) fr_off[kh][h] = swz(lane & 31, kh * 4 + (lane >> 5) * 2 + h);

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (v16f){};

  const int nk = K / kBK;
  const uint32_t uK = (uint32_t)K;
  stage_load(lds0, rsA, rsB, voff0, uK, wave);
  wait_lds_dma();
  __syncthreads();
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    stage_load(lds1, rsA, rsB, voff0 + (uint32_t)(kt + 1) * kBK, uK, wave);
    mma_stage(lds0, acc, fr_off, wm, wn);
    wait_lds_dma();
    __syncthreads();
    if (kt + 2 < nk) stage_load(lds0, rsA, rsB, voff0 + (uint32_t)(kt + 2) * kBK, uK, wave);
    mma_stage(lds1, acc, fr_off, wm, wn);
    wait_lds_dma();
    __syncthreads();
  }
  if (kt < nk) mma_stage(lds0, acc, fr_off, wm, wn);  // odd number of K steps

  epilogue_store<EPI>(acc, ea, M, N, m0 + wm * 128, n0 + wn * 128, lane);
}

template <int EPI>
hipError_t launch_epi(const uint8_t* q, int M, int K, const uint8_t* qw, int N, const EpiArgs& ea,
                      hipStream_t stream) {
  const int tilesM = (M + kBM - 1) / kBM;
  const int tilesN = (N + kBN - 1) / kBN;
  const int T = tilesM * tilesN;
  hipLaunchKernelGGL(gemm_fp8_256x256<EPI>, dim3(T), dim3(kThreads), 0, stream, q, qw, M,
                     N, K, ea, tilesM, tilesN);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear(const uint8_t* q, const float* scale, int64_t M, int64_t K,
                         const uint8_t* qw, const float* w_scale, int64_t N, const uint16_t* bias,
                         int epilogue, const uint16_t* gate, const uint16_t* residual,
                         uint16_t* out, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  EpiArgs ea{scale, w_scale, bias, gate, residual, out};
  const int m = (int)M, k = (int)K, n = (int)N;
  switch (epilogue) {
    case EPI_BIAS: return launch_epi<EPI_BIAS>(q, m, k, qw, n, ea, stream);
    case EPI_GELU_TANH: return launch_epi<EPI_GELU_TANH>(q, m, k, qw, n, ea, stream);
    default: return launch_epi<EPI_GATED_RESIDUAL>(q, m, k, qw, n, ea, stream);
  }
}

}  // namespace dq
