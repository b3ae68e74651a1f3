// FP8 (OCP E4M3) x FP8 GEMM with the dequant / bias / activation epilogue fused, for gfx950.
//
//   out[m, n] = epi( (sum_k dec(q[m, k]) dec(qw[n, k])) * scale[m] * w_scale[n] + bias[n] )
//
// Both operands are K-contiguous ("TN"), the operand layout the CDNA4 matrix cores read.
//
// Work decomposition (one workgroup = 4 wavefronts = 256 threads, one per SIMD):
//   * workgroup tile 256 (M) x 256 (N); K is consumed 128 bytes per step;
//   * a step's A tile (256 x 128 B) and B tile (256 x 128 B) are copied global -> LDS by
//     buffer_load_dwordx4 ... lds (no registers involved); one instruction moves 8 rows x 128 B,
//     i.e. whole 128-byte lines (copies touching half lines run at half the rate);
//   * two 64 KiB LDS buffers: the copy of step s+2 is issued right after the barrier that retires
//     the last fragment reads of step s, so each copy has a whole step to land;
//   * LDS rows are 128 B; 16-byte chunk c of row r sits at chunk position c ^ (r & 7), so the 8
//     lanes that read 8 consecutive rows at one K offset hit 8 different chunks (no conflicts);
//   * wavefront (wm, wn) owns a 128 x 128 sub-tile: 4 x 4 blocks of 32 x 32 computed with
//     V_MFMA_F32_32X32X64_F8F6F4, fp32 accumulators; the fragments of the next 64-wide K half are
//     read into a second register set while the MFMAs of the current half run, two LDS reads
//     issued under each of the first eight MFMAs;
//   * the weight fragment is the instruction's first operand, so a lane holds 4 consecutive
//     output columns per 8-column group; lanes l and l + 32 then swap halves (v_permlane32_swap)
//     so that each lane owns 8 consecutive columns: residual loads and bf16 stores are 16 bytes;
//   * tiles are numbered so that the workgroups on one XCD (hardware dispatch sends workgroup i
//     to XCD i mod 8) cover one contiguous range of tiles, walked 4 tile rows at a time, and
//     share A and B panels in that XCD's L2.
// The copies are issued from inline assembly so that the compiler does not serialize the LDS
// fragment reads behind them; every wait on them is explicit (s_waitcnt vmcnt).
//
// The FP8 GEMM with a fused epilogue follows the page "Accelerarea generarii de imagini cu
// FLUX 3 Image Klein pe GPU-urile Blackwell NVIDIA" (paragraph after "Tabelul 1"); the 8-bit
// matrix units fed with dynamically quantized weights and activations follow the page
// "Solucion de WaveSpeed para Acelerar la Generacion de Imagenes FLUX.1-dev", section
// "Cuantizacion Dinamica FP8".
#include "dq_internal.h"

namespace dq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256, kBK = 128;
constexpr int kThreads = 256;
constexpr int kStageBytes = (kBM + kBN) * kBK;  // 64 KiB
constexpr int kGroupM = 4;                      // tile rows per group in the tile order

enum { EPI_BIAS = 0, EPI_GELU_TANH = 1, EPI_GATED_RESIDUAL = 2 };

struct Params {
  const uint8_t* A;          // q  [M, K]
  const uint8_t* B;          // qw [N, K]
  const float* sa;           // [M]
  const float* sw;           // [N]
  const uint16_t* bias;      // [N] or null
  const uint16_t* gate;      // [N] (gated only)
  const uint16_t* residual;  // [M, N] (gated only; may equal out)
  uint16_t* out;             // [M, N]
  int M, N, K, tilesM, tilesN;
};

// ---------------------------------------------------------------------------------------------
// memory helpers
// ---------------------------------------------------------------------------------------------

// Raw buffer descriptor over `bytes` bytes from `base`; accesses past the end read zero and
// never fault. The fields are uniform, so they live in scalar registers.
__device__ __forceinline__ v4i buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return (v4i){__builtin_amdgcn_readfirstlane((int)(uint32_t)b),
               __builtin_amdgcn_readfirstlane((int)((uint32_t)(b >> 32) & 0xFFFFu)),
               __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}

// 16 bytes per lane from global memory straight into LDS at lds_base + 16 * lane. The LDS base
// (uniform) travels in M0, which is saved and restored around the copy.
__device__ __forceinline__ void copy_to_lds(v4i rsrc, uint32_t voff, uint32_t lds_base) {
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

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// All copies of this wavefront have landed (vmcnt = 0; lgkm and exp counters untouched).
__device__ __forceinline__ void wait_copies() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// At most 16 copies of this wavefront still in flight.
__device__ __forceinline__ void wait_copies_16() { __builtin_amdgcn_s_waitcnt(0x4F70); }

// This wavefront's LDS reads done, then the workgroup barrier. The lgkmcnt wait goes through
// the builtin so that the compiler's own wait bookkeeping sees it; the asm is a compiler-level
// memory barrier as well.
__device__ __forceinline__ void barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("s_barrier" ::: "memory");
}

// ---------------------------------------------------------------------------------------------
// main loop pieces
// ---------------------------------------------------------------------------------------------

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kBK + ((chunk ^ (row & 7)) << 4);
}

// Wavefront w copies rows [64 w, 64 w + 64) of both tiles of one step: 8 + 8 instructions of
// 8 rows x 128 B each. Lane l lands in LDS slot l of its 1 KiB block (row l >> 3, chunk
// position l & 7), so it fetches global chunk (l & 7) ^ (row & 7).
__device__ __forceinline__ void stage_copy(uint8_t* st, v4i ra, v4i rb, uint32_t voff, uint32_t K,
                                           int wave) {
  const uint32_t la = lds_addr(st) + (uint32_t)(wave * 64 * kBK);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t off = voff + (uint32_t)(j * 8) * K;
    copy_to_lds(ra, off, __builtin_amdgcn_readfirstlane(la + j * 1024));
    copy_to_lds(rb, off, __builtin_amdgcn_readfirstlane(la + kBM * kBK + j * 1024));
  }
}

struct Frags {
  v8i a[4];
  v8i b[4];
};

// Fragments of K half h (64 bytes) of one staged step: lane l reads row l & 31 of each 32-row
// block, bytes [64 h + 32 (l >> 5), +32) -- the same K positions for A and B.
__device__ __forceinline__ void read_frags(const uint8_t* st, Frags& f, int h, int wm, int wn,
                                           int lane) {
  const int r = lane & 31;
  const int c0 = h * 4 + (lane >> 5) * 2;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint8_t* bb = st + kBM * kBK + (wn * 128 + i * 32) * kBK;
    const uint4 lo = *reinterpret_cast<const uint4*>(bb + swz(r, c0));
    const uint4 hi = *reinterpret_cast<const uint4*>(bb + swz(r, c0 + 1));
    f.b[i] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                   (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    const uint8_t* ab = st + (wm * 128 + i * 32) * kBK;
    const uint4 lo2 = *reinterpret_cast<const uint4*>(ab + swz(r, c0));
    const uint4 hi2 = *reinterpret_cast<const uint4*>(ab + swz(r, c0 + 1));
    f.a[i] = (v8i){(int)lo2.x, (int)lo2.y, (int)lo2.z, (int)lo2.w,
                   (int)hi2.x, (int)hi2.y, (int)hi2.z, (int)hi2.w};
  }
}

__device__ __forceinline__ void mma16(const Frags& f, v16f (&acc)[4][4]) {
#pragma unroll
  for (int bn = 0; bn < 4; ++bn)
#pragma unroll
    for (int bm = 0; bm < 4; ++bm)
      acc[bn][bm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[bn], f.a[bm], acc[bn][bm],
                                                                     0, 0, 0, 0, 0, 0);
}

// Schedule: two LDS fragment reads under each of the first eight MFMAs, then the other eight.
__device__ __forceinline__ void reads_under_mfma() {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
}

// ---------------------------------------------------------------------------------------------
// epilogue
// ---------------------------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// 0.5 v (1 + tanh(u)) = v / (1 + exp(-2u)), u = sqrt(2/pi) (v + 0.044715 v^3); the exponential
// as exp2 of -2 sqrt(2/pi) log2(e) v (1 + 0.044715 v^2). Relative error a few fp32 ulps.
__device__ __forceinline__ float gelu_tanh(float v) {
  constexpr float k0 = 2.3022082f;  // 2 sqrt(2/pi) / ln 2
  const float q = fmaf(v * v, -k0 * 0.044715f, -k0);
  const float e = __builtin_amdgcn_exp2f(q * v);
  return v * __builtin_amdgcn_rcpf(1.0f + e);
}

// Exchange a's value in lanes 32..63 with b's value in lanes 0..31.
__device__ __forceinline__ void swap_halves(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// The tile's scales, bias and gate are staged in LDS (one round trip for the workgroup). Then,
// per pair of 8-column groups, each lane computes v for its 4 + 4 columns, swaps halves with
// its partner lane (l <-> l + 32) so that it holds 8 consecutive columns of one group, applies
// the activation or the gated residual there, and stores 16 bytes.
template <int EPI>
__device__ __forceinline__ void epilogue(const v16f (&acc)[4][4], const Params& p, int m0, int n0,
                                         int wm, int wn, int lane, const float* s_sa,
                                         const float* s_sw, const uint16_t* s_b,
                                         const uint16_t* s_g) {
  const int hi = lane >> 5;
#pragma unroll
  for (int bm = 0; bm < 4; ++bm) {
    const int ml = wm * 128 + bm * 32 + (lane & 31);
    const int m = m0 + ml;
    const float sam = s_sa[ml];
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) {
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        float v[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int g = gp * 2 + h;
          const int nl = wn * 128 + bn * 32 + g * 8 + hi * 4;
          const float4 swv = *reinterpret_cast<const float4*>(s_sw + nl);
          const uint2 bb = *reinterpret_cast<const uint2*>(s_b + nl);
          v[h][0] = fmaf(acc[bn][bm][g * 4 + 0] * sam, swv.x, bf16_lo(bb.x));
          v[h][1] = fmaf(acc[bn][bm][g * 4 + 1] * sam, swv.y, bf16_hi(bb.x));
          v[h][2] = fmaf(acc[bn][bm][g * 4 + 2] * sam, swv.z, bf16_lo(bb.y));
          v[h][3] = fmaf(acc[bn][bm][g * 4 + 3] * sam, swv.w, bf16_hi(bb.y));
        }
        // Before: lane l < 32 holds columns [0, 4) of group 2gp in v[0] and of group 2gp+1 in
        // v[1]; lane l + 32 holds columns [4, 8) of both. After the swap lane l owns group 2gp
        // (v[0] = columns 0-3, v[1] = columns 4-7) and lane l + 32 owns group 2gp + 1.
#pragma unroll
        for (int j = 0; j < 4; ++j) swap_halves(v[0][j], v[1][j]);
        const int nl = wn * 128 + bn * 32 + (gp * 2 + hi) * 8;
        const int n = n0 + nl;
        float y[8] = {v[0][0], v[0][1], v[0][2], v[0][3], v[1][0], v[1][1], v[1][2], v[1][3]};
        if (EPI == EPI_GELU_TANH) {
#pragma unroll
          for (int j = 0; j < 8; ++j) y[j] = gelu_tanh(y[j]);
        }
        const bool live = m < p.M && n < p.N;
        const size_t off = (size_t)m * (size_t)p.N + (size_t)n;
        if (EPI == EPI_GATED_RESIDUAL) {
          const uint4 gg = *reinterpret_cast<const uint4*>(s_g + nl);
          uint4 rr = make_uint4(0u, 0u, 0u, 0u);
          if (live) rr = *reinterpret_cast<const uint4*>(p.residual + off);
          const uint32_t gw[4] = {gg.x, gg.y, gg.z, gg.w};
          const uint32_t rw[4] = {rr.x, rr.y, rr.z, rr.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            y[2 * j] = fmaf(bf16_lo(gw[j]), y[2 * j], bf16_lo(rw[j]));
            y[2 * j + 1] = fmaf(bf16_hi(gw[j]), y[2 * j + 1], bf16_hi(rw[j]));
          }
        }
        uint4 o;
        o.x = f32_to_bf16(y[0]) | (f32_to_bf16(y[1]) << 16);
        o.y = f32_to_bf16(y[2]) | (f32_to_bf16(y[3]) << 16);
        o.z = f32_to_bf16(y[4]) | (f32_to_bf16(y[5]) << 16);
        o.w = f32_to_bf16(y[6]) | (f32_to_bf16(y[7]) << 16);
        if (live) *reinterpret_cast<uint4*>(p.out + off) = o;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// kernel
// ---------------------------------------------------------------------------------------------

__device__ __forceinline__ void tile_origin(const Params& p, int& m0, int& n0) {
  const int T = p.tilesM * p.tilesN;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, loc = bid >> 3;
  const int per = T >> 3, rem = T & 7;
  const int t = xcd * per + (xcd < rem ? xcd : rem) + loc;
  const int per_group = kGroupM * p.tilesN;
  const int grp = t / per_group;
  const int first_m = grp * kGroupM;
  const int gsz = (p.tilesM - first_m) < kGroupM ? (p.tilesM - first_m) : kGroupM;
  const int tin = t - grp * per_group;
  m0 = (first_m + tin % gsz) * kBM;
  n0 = (tin / gsz) * kBN;
}

template <int EPI>
__global__ void __launch_bounds__(kThreads) gemm_fp8_256x256(Params p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kStageBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  int m0, n0;
  tile_origin(p, m0, n0);

  // per-tile descriptors: rows past M (N) are out of range and read as zero
  const uint32_t rowsA = (uint32_t)(p.M - m0 < kBM ? p.M - m0 : kBM);
  const uint32_t rowsB = (uint32_t)(p.N - n0 < kBN ? p.N - n0 : kBN);
  const v4i rsA = buffer_rsrc(p.A + (size_t)m0 * (size_t)p.K, rowsA * (uint32_t)p.K);
  const v4i rsB = buffer_rsrc(p.B + (size_t)n0 * (size_t)p.K, rowsB * (uint32_t)p.K);
  const int lr = lane >> 3;
  const uint32_t voff0 =
      (uint32_t)(wave * 64 + lr) * (uint32_t)p.K + (uint32_t)(((lane & 7) ^ (lr & 7)) * 16);
  const uint32_t uK = (uint32_t)p.K;
  const int nk = p.K / kBK;

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (v16f){};
  Frags f0, f1;

  stage_copy(lds, rsA, rsB, voff0, uK, wave);
  if (nk > 1) {
    stage_copy(lds + kStageBytes, rsA, rsB, voff0 + kBK, uK, wave);
    wait_copies_16();  // step 0 landed, step 1 may still be in flight
  } else {
    wait_copies();
  }
  barrier();
  read_frags(lds, f0, 0, wm, wn, lane);

  int s = 0;
  for (; s + 1 < nk; ++s) {
    uint8_t* cur = lds + (s & 1) * kStageBytes;
    uint8_t* nxt = lds + ((s + 1) & 1) * kStageBytes;
    read_frags(cur, f1, 1, wm, wn, lane);  // MMA on K half (s, 0) while reading (s, 1)
    mma16(f0, acc);
    reads_under_mfma();
    wait_copies();                         // step s + 1 landed (the only copy in flight)
    barrier();                             // for every wavefront; step s fully read
    if (s + 2 < nk) stage_copy(cur, rsA, rsB, voff0 + (uint32_t)(s + 2) * kBK, uK, wave);
    read_frags(nxt, f0, 0, wm, wn, lane);  // MMA on K half (s, 1) while reading (s + 1, 0)
    mma16(f1, acc);
    reads_under_mfma();
  }
  read_frags(lds + (s & 1) * kStageBytes, f1, 1, wm, wn, lane);
  mma16(f0, acc);
  reads_under_mfma();
  mma16(f1, acc);

  // epilogue parameters of this tile, staged in the (now free) LDS
  barrier();
  float* s_sa = reinterpret_cast<float*>(lds);
  float* s_sw = s_sa + kBM;
  uint16_t* s_b = reinterpret_cast<uint16_t*>(s_sw + kBN);
  uint16_t* s_g = s_b + kBN;
  {
    const int m = m0 + tid, n = n0 + tid;
    s_sa[tid] = m < p.M ? p.sa[m] : 0.f;
    s_sw[tid] = n < p.N ? p.sw[n] : 0.f;
    s_b[tid] = (p.bias && n < p.N) ? p.bias[n] : (uint16_t)0;
    if (EPI == EPI_GATED_RESIDUAL) s_g[tid] = n < p.N ? p.gate[n] : (uint16_t)0;
  }
  __syncthreads();
  epilogue<EPI>(acc, p, m0, n0, wm, wn, lane, s_sa, s_sw, s_b, s_g);
}

template <int EPI>
hipError_t launch_epi(const Params& p, hipStream_t stream) {
  const int T = p.tilesM * p.tilesN;
  hipLaunchKernelGGL(gemm_fp8_256x256<EPI>, dim3(T), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear(const uint8_t* q, const float* scale, int64_t M, int64_t K,
                         const uint8_t* qw, const float* w_scale, int64_t N, const uint16_t* bias,
                         int epilogue, const uint16_t* gate, const uint16_t* residual,
                         uint16_t* out, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  Params p;
  p.A = q;
  p.B = qw;
  p.sa = scale;
  p.sw = w_scale;
  p.bias = bias;
  p.gate = gate;
  p.residual = residual;
  p.out = out;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.tilesM = (p.M + kBM - 1) / kBM;
  p.tilesN = (p.N + kBN - 1) / kBN;
  switch (epilogue) {
    case EPI_BIAS: return launch_epi<EPI_BIAS>(p, stream);
    case EPI_GELU_TANH: return launch_epi<EPI_GELU_TANH>(p, stream);
    default: return launch_epi<EPI_GATED_RESIDUAL>(p, stream);
  }
}

}  // namespace dq
