// FP8 (OCP E4M3) x FP8 GEMM with the dequant / bias / activation epilogue fused, for gfx950.
//
//   out[m, n] = epi( (sum_k dec(q[m, k]) dec(qw[n, k])) * scale[m] * w_scale[n] + bias[n] )
//
// Both operands are K-contiguous ("TN"), the operand layout the CDNA4 matrix cores read.
//
// Work decomposition
//   * output tiles of 256 x 256, K consumed 128 bytes per step; a "unit" is one step of one tile;
//   * a persistent grid of G <= (compute units) workgroups taking work items round-robin
//     (workgroup v takes items v, v + G, ...), so the workgroups of an XCD hold neighbouring
//     items, step through K together and share A and B slices in L2. The items are the tiles of
//     the full rounds (T - T mod G of them), then the T mod G tiles left over. When the
//     left-over tiles fit on half the compute units they run as two 256 x 128 halves each, in a
//     second launch of the kernel built for that width (one wave then owns 128 x 32). With a
//     workspace the left-over tiles may instead be cut along K into s equal parts (s divides the
//     step count; the host picks by counting steps), the parts ordered so that neighbouring
//     workgroups hold neighbouring tiles at the same K range: the last round then keeps the
//     compute units busy. The parts of a cut tile are summed in fp32 through the workspace by
//     the part that finishes last (an arrival counter per tile; no workgroup ever waits for
//     another), in part order, so the result does not depend on timing; parts travel with
//     device-coherent (sc1) loads and stores, so no cache flush is needed;
//   * workgroups are numbered so that the ones on one XCD (hardware dispatch sends workgroup b to
//     XCD b mod 8) get consecutive numbers, hence neighbouring tiles, and tiles are walked 4 tile
//     rows at a time, so an XCD's L2 serves the A and B panels its compute units share.
//
// Inside a workgroup (8 wavefronts, two per SIMD: waves w and w + 4 share a SIMD)
//   * wave (g, q), g = w >> 2, q = w & 3, owns a 128 (M) x 64 (N) sub-tile: 4 x 2 blocks of
//     32 x 32 from V_MFMA_F32_32X32X64_F8F6F4, fp32 accumulators;
//   * group 1 runs one phase behind group 0, and every phase ends at a workgroup barrier, so in
//     each phase one wave per SIMD issues 8 MFMAs (one 64-deep K half) while the other reads its
//     next fragments from LDS (ping-pong);
//   * each step's A tile (256 x 128 B) and B tile (256 x 128 B) go global -> LDS through
//     buffer_load_dwordx4 ... lds (no registers involved), one instruction moving 8 rows x 128 B
//     (whole 128-byte lines), in four batches of 16 KiB, one per phase, each issued by that
//     phase's reading wave after its LDS reads. Two stages: the A rows and group 1's B rows of
//     step s + 1 go into the stage step s - 1 used, group 0's B rows of step s + 2 into the stage
//     of step s once group 0 has read them, so every batch has two to four phases to land. A
//     wave waits for its own batches (all but its last one) before the barrier that precedes
//     their first reader. Issuing a phase's copies in one burst, or working out the next step
//     with integer divisions, held the reading wave past the MFMAs of its phase;
//   * LDS rows are 128 B; 16-byte chunk c of row r sits at position c ^ ((r >> 1) & 7). A
//     ds_read_b128 serves 16 lanes at a time, here 16 consecutive rows at one K offset, and with
//     this key they land in 16 different 16-byte slots of a 256-byte bank period (no conflicts);
//   * the weight fragment is the MFMA's first operand, so a lane holds 4 consecutive output
//     columns per 8-column group; lanes l and l + 32 swap halves (v_permlane32_swap) so that each
//     lane owns 8 consecutive columns: residual loads and bf16 stores are 16 bytes;
//   * the tile's scales, bias and gate are copied to LDS with the first step of each share part.
// The copies are issued from inline assembly so that the compiler does not serialize LDS reads
// behind them; every wait on them is explicit (s_waitcnt vmcnt).
//
// The FP8 GEMM with a fused epilogue follows the page "Accelerarea generarii de imagini cu
// FLUX 3 Image Klein pe GPU-urile Blackwell NVIDIA" (paragraph after "Tabelul 1"); the 8-bit
// matrix units fed with dynamically quantized weights and activations follow the page
// "Solucion de WaveSpeed para Acelerar la Generacion de Imagenes FLUX.1-dev", section
// "Cuantizacion Dinamica FP8".
#include "dq_internal.h"
#include "e4m3_codec.h"

#include <atomic>
#include <mutex>

namespace dq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 256, kBN = 256, kBK = 128;
constexpr int kThreads = 512;
constexpr int kStageBytes = (kBM + kBN) * kBK;  // 64 KiB: A tile, then B tile
constexpr int kParamBytes = 4096;               // sa f32[256] | sw f32[256] | bias | gate (1 KiB each)
constexpr int kParamBufs = 3;                   // part i of a share uses buffer i % 3
constexpr int kGroupM = 4;                      // tile rows per group in the tile order
constexpr int kPartFloats = kBM * kBN;
constexpr int kMaxSeg = (int)kMaxSegments;      // row segments with their own weights

enum { EPI_BIAS = 0, EPI_GELU_TANH = 1, EPI_GATED_RESIDUAL = 2, EPI_QKV = 3,
       EPI_MX_BIAS = 4, EPI_MX_GELU_TANH = 5, EPI_MX_GATED = 6,
       EPI_MX4_BIAS = 7, EPI_MX4_GELU_TANH = 8, EPI_MX4_GATED = 9,
       EPI_QKV_Q8 = 10,    // the QKV epilogue with its outputs leaving as E4M3 codes
       EPI_MXG_BIAS = 11, EPI_MXG_GELU_TANH = 12,    // MX FP8 with grouped scale copies
       EPI_MX4G_BIAS = 13, EPI_MX4G_GELU_TANH = 14, EPI_MX4G_GATED = 15 };  // and MX FP4

// Block-scaled (MX) operands: E4M3 codes with one E8M0 scale byte per 32 values along K. Each
// K step then also stages the 4 scale bytes (one dword) of every A and B row of the tile, after
// the codes of the stage: for each group of 32 tile rows (A rows, then B rows) a 256-byte slot
// whose first 128 bytes hold the 32 rows' dwords (a copy instruction moves 64 lanes' dwords and
// its upper 32 lanes fill the rest with zeros, so no lane needs to be switched off).
// With FP4 (E2M1) elements (EPI_MX4_*) the operands are two codes per byte, so a step of 128 bytes
// per row is 256 values along K and its 8 scale bytes are two dwords per row: lanes 0-31 of the
// copy move the first dword of 32 rows, lanes 32-63 the second, filling the whole slot.
//
// Grouped scale copies (EPI_MXG_*, E4M3 elements, K steps per tile a multiple of 4): the 4 scale
// bytes of a row for 4 consecutive K steps are 16 contiguous bytes of the [M, K / 32] scale
// matrix, so every fourth step one 16-byte copy per lane moves the next 4 steps' scales of 64 rows,
// two copies per wave of group 0 (its A rows 64 q + [0, 64), and the 64 B rows of its batches 2
// and 3) instead of one 4-byte copy per batch and step. They go into one of two 8 KiB group
// buffers (A rows [0, 4 KiB) at 16 bytes a row, then wave q's B copy at 4 KiB + 1 KiB q), the
// group's index parity choosing the buffer; with every item a multiple of 4 steps long, group j
// holds steps [4 j, 4 j + 4) of the workgroup's sequence and rides on group 0's batch 1 of step
// 4 j (issued in step 4 j - 1, waited for at its end), three steps after the last reader of the
// buffer's previous group. (Issuing it a step earlier measured no faster.) With E2M1 elements
// (EPI_MX4G_*, K steps a multiple of 2) a row's 16 bytes are the 8 scale bytes of 2 steps, so a
// group is 2 steps and the buffer's previous group was last read one step before the copy.
constexpr int kScaleBytes = 4096;
constexpr int kGroupBytes = 16384;
__host__ __device__ constexpr bool is_mxg(int epi) {
  return epi == EPI_MXG_BIAS || epi == EPI_MXG_GELU_TANH;
}
__host__ __device__ constexpr bool is_mx4g(int epi) {
  return epi >= EPI_MX4G_BIAS && epi <= EPI_MX4G_GATED;
}
__host__ __device__ constexpr bool is_mx(int epi) {
  return (epi >= EPI_MX_BIAS && epi <= EPI_MX4_GATED) || is_mxg(epi) || is_mx4g(epi);
}
__host__ __device__ constexpr bool is_qkv(int epi) { return epi == EPI_QKV || epi == EPI_QKV_Q8; }
// 0: per-row scales; 1: MX with E4M3 elements; 2: MX with E2M1 elements; 3 and 4: MX with E4M3
// and with E2M1 elements and grouped scale copies
__host__ __device__ constexpr int mx_kind(int epi) {
  return epi >= EPI_MX4_BIAS && epi <= EPI_MX4_GATED ? 2 : is_mxg(epi) ? 3 : is_mx4g(epi) ? 4
       : is_mx(epi) ? 1 : 0;
}
__host__ __device__ constexpr bool mx_fp4(int mx) { return mx == 2 || mx == 4; }
__host__ __device__ constexpr bool mx_grouped(int mx) { return mx == 3 || mx == 4; }
// K steps per scale group (grouped kinds)
__host__ __device__ constexpr int group_steps(int mx) { return mx == 4 ? 2 : 4; }
// The output step after dequantization: EPI_BIAS, EPI_GELU_TANH, EPI_GATED_RESIDUAL (or EPI_QKV)
__host__ __device__ constexpr int act_of(int epi) {
  return is_qkv(epi) ? EPI_QKV : epi < EPI_MX_BIAS ? epi
       : is_mxg(epi) ? epi - EPI_MXG_BIAS : is_mx4g(epi) ? epi - EPI_MX4G_BIAS
       : (epi - EPI_MX_BIAS) % 3;
}
// Scales staged with each step's codes (MX kinds 1 and 2)
__host__ __device__ constexpr bool step_scales(int epi) {
  return mx_kind(epi) == 1 || mx_kind(epi) == 2;
}
__host__ __device__ constexpr int stage_bytes(int epi) {
  return kStageBytes + (step_scales(epi) ? kScaleBytes : 0);
}
// Copy instructions per batch: four of codes, plus one of scales with per-step scale copies. (The
// grouped copies are the last instructions of batch 1, which no wait leaves in flight.)
__host__ __device__ constexpr int batch_ops(int epi) { return step_scales(epi) ? 5 : 4; }

// Arguments of the QKV epilogue only. They are read where they are used (the epilogue and the
// parameter copy), through qkv_args(), so that they do not sit in scalar registers through the
// MFMA loop (where they would be spilled).
struct QkvArgs {
  const uint16_t* norm_qk;   // [2][128] query then key RMS-norm weights
  const float* rope_cos;     // [M, 64]
  const float* rope_sin;     // [M, 64]
  uint16_t* out_q;           // [heads, M, 128] each; EPI_QKV_Q8: codes (bytes), the values'
  uint16_t* out_k;           // transposed, [heads, 128, M]
  uint16_t* out_v;
  float* scale_q;            // EPI_QKV_Q8 only: [heads, M], the scale of each head row
  float* scale_k;
  float* scale_v;
  float eps;
  int heads;
};

// Row segments: rows [row0[s], row0[s + 1]) of q, scale, residual and out use the weight of
// segment s. A segment's tile rows are its own (a tile never spans two segments): segment s
// owns tile rows [trow0[s], trow0[s + 1]). Read where used, through seg_args().
struct SegArgs {
  const uint8_t* B[kMaxSeg];       // qw [N, K] of each segment
  const float* sw[kMaxSeg];        // [N]
  const uint16_t* bias[kMaxSeg];   // [N] or null
  const uint16_t* gate[kMaxSeg];   // [N] (gated only)
  int row0[kMaxSeg + 1];
  int trow0[kMaxSeg + 1];
  int nseg;
};

struct Params {
  const uint8_t* A;          // q  [M, K]
  const float* sa;           // [M]
  const uint16_t* residual;  // [M, N] (gated only; may equal out)
  uint16_t* out;             // [M, N]
  uint32_t* flags;           // [left-over tiles] arrival counters (cut tiles only)
  float* part;               // [parts][256 * 256] partial tiles (cut tiles only)
  uint32_t part_bytes;       // bytes of the partial tiles
  const uint8_t* mxa;        // MX only: A's scale bytes [M, K / 32] (B's: in seg.sw, per segment)
  int M, N, K, tilesM, tilesN, nk, tiles;
  int dp_tiles;              // tiles of full rounds run by this launch (a multiple of the grid)
  int tail0;                 // first left-over tile
  int tail_tiles;            // left-over tiles run by this launch
  int splits;                // parts per left-over tile (1: not cut)
  int part_steps;            // nk / splits
  int narrow;                // 1: each left-over tile runs as two 256 x 128 halves (not cut)
  QkvArgs qkv;               // QKV epilogue only (N = 3 heads 128); read through qkv_args()
  SegArgs seg;               // per-segment weights and rows; read through seg_args()
};

// The kernel's own copy of Params.qkv, read from the kernel argument segment at the point of
// use: the empty asm hides where the pointer comes from, so the loads stay where they are.
__device__ __forceinline__ QkvArgs qkv_args() {
  typedef const __attribute__((address_space(4))) Params* KParams;
  KParams kp = (KParams)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(kp));
  QkvArgs a;
  a.norm_qk = kp->qkv.norm_qk;
  a.rope_cos = kp->qkv.rope_cos;
  a.rope_sin = kp->qkv.rope_sin;
  a.out_q = kp->qkv.out_q;
  a.out_k = kp->qkv.out_k;
  a.out_v = kp->qkv.out_v;
  a.scale_q = kp->qkv.scale_q;
  a.scale_k = kp->qkv.scale_k;
  a.scale_v = kp->qkv.scale_v;
  a.eps = kp->qkv.eps;
  a.heads = kp->qkv.heads;
  return a;
}

typedef const __attribute__((address_space(4))) SegArgs* KSeg;

// The kernel's own copy of Params.seg, in the kernel argument segment (scalar loads at the point
// of use, as for qkv_args()).
__device__ __forceinline__ KSeg seg_args() {
  typedef const __attribute__((address_space(4))) Params* KParams;
  KParams kp = (KParams)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(kp));
  return &kp->seg;
}

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

// 4 bytes per lane from global memory straight into LDS at lds_base + 4 * lane (64 lanes: 256
// bytes). Any 4-byte aligned source works.
__device__ __forceinline__ void copy_to_lds_b32(v4i rsrc, uint32_t voff, uint32_t lds_base) {
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

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// All vector memory operations of this wavefront done (vmcnt = 0; lgkm and exp untouched).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// All but the last N (one batch: 4, or 5 in MX mode) vector memory operations of this wavefront
// done (vmcnt <= N). Memory operations of one wavefront are counted off in the order they were
// issued.
template <int N>
__device__ __forceinline__ void wait_vmem_but() { __builtin_amdgcn_s_waitcnt(0x0F70 | N); }

// Phase boundary: this wavefront's LDS reads done, then the workgroup barrier. No instruction
// is scheduled across it (the MFMAs of a phase must stay in their phase).
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ int swz_key(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kBK + ((chunk ^ swz_key(row)) << 4);
}

// ---------------------------------------------------------------------------------------------
// schedule: shares, tiles, contributors
// ---------------------------------------------------------------------------------------------

// Workgroup v's items: n_dp whole tiles v, v + G, ... of the full rounds, then n_parts items
// u = v, v + G, ... of the left-over tiles: either parts (part u: tile tail0 + u % tail_tiles,
// steps [j part_steps, (j + 1) part_steps), j = u / tail_tiles) or, with narrow, halves (half
// u & 1, columns [128 (u & 1), + 128), of tile tail0 + (u >> 1)).
struct Work {
  int n_dp, n_parts;
};

__device__ __forceinline__ Work work_of(const Params& p, int v, int G) {
  Work w;
  w.n_dp = p.dp_tiles / G;
  const int P = p.narrow ? 2 * p.tail_tiles : p.tail_tiles * p.splits;
  w.n_parts = v < P ? (P - v + G - 1) / G : 0;
  return w;
}

// A position in a workgroup's sequence of steps: work item `item`, its tile t, its part of a
// cut tile (-1: not cut), its half of a narrow tile (-1: full width), the K step k and the
// item's end step kend. Moving one step on costs an increment; the divisions happen once per
// item.
struct Cursor {
  int item, t, cut, half, k, kend;
};

template <int NB>
__device__ __forceinline__ void cursor_item(const Params& p, const Work& w, int v, int G,
                                            Cursor& c) {
  c.cut = -1;
  c.half = -1;
  c.k = 0;
  c.kend = p.nk;
  if (c.item < w.n_dp) {
    c.t = v + c.item * G;
  } else if (NB == 1) {  // a launch of narrow halves
    const int u = v + (c.item - w.n_dp) * G;
    c.t = p.tail0 + (u >> 1);
    c.half = u & 1;
  } else {
    const int part = v + (c.item - w.n_dp) * G;
    const int j = part / p.tail_tiles;
    c.t = p.tail0 + (part - j * p.tail_tiles);
    if (p.splits > 1) c.cut = part;
    c.k = j * p.part_steps;
    c.kend = c.k + p.part_steps;
  }
}

// The next step; past the last one the cursor keeps its tile (and is not used).
template <int NB>
__device__ __forceinline__ void cursor_next(const Params& p, const Work& w, int v, int G,
                                            Cursor& c) {
  if (++c.k == c.kend) {
    ++c.item;
    if (c.item < w.n_dp + w.n_parts) cursor_item<NB>(p, w, v, G, c);
  }
}

// Geometry of a work item: its origin, the end of its row segment and the segment.
struct Geo {
  int m0, n0, mend, s;
};

// Tile t: tile rows are walked kGroupM at a time (every column of a group of tile rows, then the
// next group); tile row tr belongs to the last segment whose first tile row is <= tr.
__device__ __forceinline__ Geo tile_geo(const Params& p, int t) {
  const int per_group = kGroupM * p.tilesN;
  const int grp = t / per_group;
  const int first_m = grp * kGroupM;
  const int gsz = (p.tilesM - first_m) < kGroupM ? (p.tilesM - first_m) : kGroupM;
  const int tin = t - grp * per_group;
  const int tr = first_m + tin % gsz;
  const KSeg sg = seg_args();
  int s = 0;
  for (int i = 1; i < sg->nseg; ++i)
    if (tr >= sg->trow0[i]) s = i;
  Geo g;
  g.s = s;
  g.m0 = sg->row0[s] + (tr - sg->trow0[s]) * kBM;
  g.mend = sg->row0[s + 1];
  g.n0 = (tin / gsz) * kBN;
  return g;
}

// Tile t, or its 128-column half (half >= 0, narrow launches only).
template <int NB>
__device__ __forceinline__ Geo item_geo(const Params& p, int t, int half) {
  Geo g = tile_geo(p, t);
  if (NB == 1) g.n0 += half * (kBN / 2);
  return g;
}

struct TileDesc {
  Geo g;  // origin of the tile (of the half, in a narrow launch), segment end, segment
  v4i rsA, rsB;
  v4i rsSA, rsSB;  // MX only: the tile rows' scale bytes
};

// Descriptors of a tile or of one half of it: rows past the segment end (columns past N) are out
// of range and read as zero (a half entirely past N has an empty B range).
template <int NB, int MX>
__device__ __forceinline__ TileDesc tile_desc(const Params& p, int t, int half) {
  TileDesc d;
  d.g = item_geo<NB>(p, t, half);
  const int m0 = d.g.m0, n0 = d.g.n0;
  const int width = NB == 1 ? kBN / 2 : kBN;
  const int rb = p.N - n0 < width ? p.N - n0 : width;
  const uint32_t rowsA = (uint32_t)(d.g.mend - m0 < kBM ? d.g.mend - m0 : kBM);
  const uint32_t rowsB = (uint32_t)(rb > 0 ? rb : 0);
  d.rsA = buffer_rsrc(p.A + (size_t)m0 * (size_t)p.K, rowsA * (uint32_t)p.K);
  d.rsB = buffer_rsrc(seg_args()->B[d.g.s] + (size_t)(rb > 0 ? n0 : 0) * (size_t)p.K,
                      rowsB * (uint32_t)p.K);
  if (MX) {
    // scale bytes per row: K / 32 values; p.K counts bytes, two values each with FP4. A
    // segment's weight scale bytes sit where its per-channel scales would.
    const uint32_t kb = (uint32_t)p.K / (mx_fp4(MX) ? 16u : 32u);
    const uint8_t* sw = reinterpret_cast<const uint8_t*>(seg_args()->sw[d.g.s]);
    d.rsSA = buffer_rsrc(p.mxa + (size_t)m0 * kb, rowsA * kb);
    d.rsSB = buffer_rsrc(sw + (size_t)(rb > 0 ? n0 : 0) * kb, rowsB * kb);
  }
  return d;
}

// ---------------------------------------------------------------------------------------------
// copies
// ---------------------------------------------------------------------------------------------

// One copy batch: 32 rows (4 blocks of 8 rows x 128 B) of one operand of step k into stage st,
// one instruction per block. The batches of a step, for wave q of the copying group:
//   0: A rows 64q + [0, 32)            1: A rows 64q + [32, 64)
//   2: B rows that group 1 reads: 128 (q >> 1) + 64 + 32 (q & 1) + [0, 32)
//   3: B rows that group 0 reads: 128 (q >> 1) + 32 (q & 1) + [0, 32)
// B rows sit in LDS at their tile row. In a narrow (256 x 128) tile group 0 reads tile rows
// [0, 32) and [64, 96), group 1 rows [32, 64) and [96, 128); they sit at LDS rows [0, 64) and
// [64, 128), inside the rows each group reads in a full tile, so that either kind of step can
// follow the other in a stage. A narrow B batch has 16 rows per wave (tile rows
// 64 (q >> 1) + 32 [group 1] + 16 (q & 1) + [0, 16), LDS rows 64 [group 1] + 16 q + [0, 16));
// its two other instructions copy from an empty range into rows no narrow step reads (group 0:
// [128, 192), group 1: [192, 256)), so that every batch is four instructions.
// Lane l lands in LDS slot l of a block (row l >> 3, position l & 7), so it fetches global chunk
// (l & 7) ^ key(row); every block starts 16 LDS rows after a multiple of 16 plus 8 for odd
// blocks, so the key depends only on l >> 3 and on the parity of the block (odd blocks add dodd
// to the offset). A batch with `live` false copies from an empty range: its instructions still
// run (keeping the count of outstanding copies fixed) and write zeros into a region nobody
// reads any more.
struct Batch {
  v4i rs01, rs23;        // blocks 0-1 and 2-3
  uint32_t off0, lds01, lds23;
  v4i rsS;               // MX only: the batch's 32 rows' scale dwords of step k (lanes 0-31)
  uint32_t soff, slds;
  // grouped scale copies (MX kind 3, a batch given a group buffer for a step that starts a group):
  // the offsets of this lane's 16 bytes for the A and the B copy, and their LDS places
  bool grp;
  v4i rsGA, rsGB;
  uint32_t goA, goB, gldsA, gldsB;
};

template <int NB, int MX>
__device__ __forceinline__ Batch batch_of(const TileDesc& d, uint32_t K, int k, uint8_t* st,
                                          uint32_t vlane, int q, int which, bool live,
                                          uint8_t* gbuf = nullptr) {
  Batch b;
  const uint32_t base = lds_addr(st);
  int grow, lrow;
  if (which < 2) {
    grow = lrow = q * 64 + which * 32;
    b.rs01 = d.rsA;
  } else {
    b.rs01 = d.rsB;
    if (NB == 2) {
      grow = lrow = (q >> 1) * 128 + (q & 1) * 32 + (which == 2 ? 64 : 0);
    } else {
      grow = (q >> 1) * 64 + (q & 1) * 16 + (which == 2 ? 32 : 0);
      lrow = (which == 2 ? 64 : 0) + q * 16;
    }
  }
  if (!live) b.rs01[2] = 0;
  b.rs23 = b.rs01;
  const uint32_t region = base + (which < 2 ? 0u : (uint32_t)(kBM * kBK));
  b.lds01 = region + (uint32_t)(lrow * kBK);
  b.lds23 = b.lds01 + 2048u;
  if (NB == 1 && which >= 2) {  // narrow: blocks 2-3 are empty copies into unread rows
    b.rs23[2] = 0;
    b.lds23 = region + (uint32_t)(((which == 2 ? 192 : 128) + q * 16) * kBK);
  }
  b.off0 = (uint32_t)grow * K + vlane + (uint32_t)k * kBK;
  if (MX) {
    // lane i < n fetches the dword of tile row grow + i, the other lanes read past the range;
    // n = 32 rows per slot, or 16 for the B rows of a narrow half (16 per batch there). With
    // FP4 elements lane 32 + i fetches the same row's second dword of the step.
    const bool n16 = NB == 1 && which >= 2;
    b.rsS = which < 2 ? d.rsSA : d.rsSB;
    if (!live) b.rsS[2] = 0;
    const uint32_t lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const uint32_t n = n16 ? 16u : 32u;
    if (MX == 2) {
      const uint32_t kb = K / 16u, r = lane & 31u;
      b.soff = r < n ? ((uint32_t)grow + r) * kb + (uint32_t)k * 8u + (lane >> 5) * 4u
                     : 0xFFFFFFF0u;
    } else {
      const uint32_t kb = K / 32u;
      b.soff = lane < n ? ((uint32_t)grow + lane) * kb + (uint32_t)k * 4u : 0xFFFFFFF0u;
    }
    b.slds = base + (uint32_t)kStageBytes + (which < 2 ? 0u : 2048u) +
             (uint32_t)(n16 ? grow >> 4 : grow >> 5) * 256u;
  }
  if (mx_grouped(MX)) {
    b.grp = live && gbuf != nullptr && k % group_steps(MX) == 0;
    b.rsGA = d.rsSA;
    b.rsGB = d.rsSB;
    if (b.grp) {
      // lane L: A tile row 64 q + L; B tile row (q >> 1) 128 + (L >> 5) 64 + (q & 1) 32 + (L & 31)
      // in a full tile (batch 3's rows, then batch 2's), in a narrow half lanes L < 32 take
      // (q >> 1) 64 + ((L >> 4) & 1) 32 + (q & 1) 16 + (L & 15) and the others read past the
      // range (zeros into bytes no reader reads)
      const uint32_t lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
      // scale bytes per row and per step: 4 (E4M3; p.K counts values), 8 (E2M1; p.K counts bytes)
      const uint32_t kb = K / (MX == 4 ? 16u : 32u), kstep = MX == 4 ? 8u : 4u, qq = (uint32_t)q;
      const uint32_t ra = 64u * qq + lane;
      uint32_t rb;
      bool okb = true;
      if (NB == 2) {
        rb = (qq >> 1) * 128u + (lane >> 5) * 64u + (qq & 1u) * 32u + (lane & 31u);
      } else {
        rb = (qq >> 1) * 64u + ((lane >> 4) & 1u) * 32u + (qq & 1u) * 16u + (lane & 15u);
        okb = lane < 32u;
      }
      b.goA = ra * kb + (uint32_t)k * kstep;
      b.goB = okb ? rb * kb + (uint32_t)k * kstep : 0x80000000u;
      b.gldsA = lds_addr(gbuf) + qq * 1024u;
      b.gldsB = b.gldsA + 4096u;
    }
  }
  return b;
}

// The scale dwords of a batch (MX): lanes 0-31 one row each (no branch: see batch_of).
__device__ __forceinline__ void copy_scales(const Batch& b) {
  copy_to_lds_b32(b.rsS, b.soff, __builtin_amdgcn_readfirstlane(b.slds));
}

// Grouped scale copies of a group-0 wave: its A rows' and its B rows' next 4 steps (see above).
__device__ __forceinline__ v4i uniform_rsrc(v4i r) {
  return (v4i){__builtin_amdgcn_readfirstlane(r[0]), __builtin_amdgcn_readfirstlane(r[1]),
               __builtin_amdgcn_readfirstlane(r[2]), __builtin_amdgcn_readfirstlane(r[3])};
}
__device__ __forceinline__ void copy_group_a(const Batch& b) {
  copy_to_lds(uniform_rsrc(b.rsGA), b.goA, __builtin_amdgcn_readfirstlane(b.gldsA));
}
__device__ __forceinline__ void copy_group_b(const Batch& b) {
  copy_to_lds(uniform_rsrc(b.rsGB), b.goB, __builtin_amdgcn_readfirstlane(b.gldsB));
}

__device__ __forceinline__ void copy_block(const Batch& b, uint32_t K, uint32_t dodd, int j) {
  copy_to_lds(j < 2 ? b.rs01 : b.rs23, b.off0 + (uint32_t)(j * 8) * K + ((j & 1) ? dodd : 0u),
              __builtin_amdgcn_readfirstlane((j < 2 ? b.lds01 : b.lds23) +
                                             (uint32_t)((j & 1) * 1024)));
}

template <int NB, int MX>
__device__ __forceinline__ void copy_batch(const TileDesc& d, uint32_t K, int k, uint8_t* st,
                                           uint32_t vlane, uint32_t dodd, int q, int which,
                                           uint8_t* gbuf = nullptr) {
  const Batch b = batch_of<NB, MX>(d, K, k, st, vlane, q, which, true, gbuf);
#pragma unroll
  for (int j = 0; j < 4; ++j) copy_block(b, K, dodd, j);
  if (MX == 1 || MX == 2) copy_scales(b);
  if (mx_grouped(MX) && b.grp) {
    copy_group_a(b);
    copy_group_b(b);
  }
}

// The tile's epilogue parameters into param buffer pb, one copy per group-0 wave (q).
template <int EPI>
__device__ __forceinline__ void copy_params(const Params& p, const TileDesc& d, uint8_t* pb, int q,
                                            int lane) {
  const int m0 = d.g.m0;
  int n0 = d.g.n0;
  const uint32_t lp = __builtin_amdgcn_readfirstlane(lds_addr(pb) + (uint32_t)(q * 1024));
  const uint32_t lo = (uint32_t)lane * 16u;
  const uint32_t rows = (uint32_t)(d.g.mend - m0 < kBM ? d.g.mend - m0 : kBM);
  const KSeg sg = seg_args();
  const int s = d.g.s;
  // columns of this tile that exist: none for a narrow half that lies past N
  const int nc = p.N - n0 < kBN ? p.N - n0 : kBN;
  const uint32_t cols = (uint32_t)(nc > 0 ? nc : 0);
  if (nc <= 0) n0 = 0;
  if (is_mx(EPI) && q < 2) {
    // block-scaled operands carry their scales with the codes: only bias and gate are copied
  } else if (q == 0) {
    // a segment may start at any row, so the scales move 4 bytes per lane (4 x 64 of them)
    const v4i rs = buffer_rsrc(p.sa + m0, rows * 4u);
#pragma unroll
    for (int j = 0; j < 4; ++j) copy_to_lds_b32(rs, (uint32_t)(j * 256 + lane * 4), lp + j * 256u);
  } else if (q == 1) {
    copy_to_lds(buffer_rsrc(sg->sw[s] + n0, cols * 4u), lo, lp);
  } else if (q == 2) {
    const uint16_t* bias = sg->bias[s];
    copy_to_lds(buffer_rsrc(bias + n0, bias ? cols * 2u : 0u), lo, lp);
  } else if (act_of(EPI) == EPI_GATED_RESIDUAL) {
    copy_to_lds(buffer_rsrc(sg->gate[s] + n0, cols * 2u), lo, lp);
  } else if (is_qkv(EPI)) {
    copy_to_lds(buffer_rsrc(qkv_args().norm_qk, 512u), lo, lp);
  }
}

// ---------------------------------------------------------------------------------------------
// fragments and MFMA
// ---------------------------------------------------------------------------------------------

struct Frags {
  v8i a[4];  // rows wm * 128 + 32 i + (lane & 31) of the A tile
  v8i b[2];  // B rows: full tile wn * 64 + 32 i + (lane & 31); narrow tile only b[0]
  uint32_t sa[4], sb[2];  // MX only: those rows' scale dwords, shifted right by 8 (lane >> 5)
                          // (with FP4 elements: the dword of the K half read)
};

// Fragments of K half h (64 bytes) of one staged step: lane l reads row l & 31 of each 32-row
// block, bytes [64 h + 32 (l >> 5), +32) -- the same K positions for A and B. NB is the number
// of 32-column blocks per wave: 2 in a full tile; 1 in a narrow one, whose block (tile rows
// 32 wn + [0, 32)) sits at LDS rows 64 g + 32 (q & 1) + [0, 32).
// In MX mode the scaled instruction takes a row's 64 codes as two blocks of 32, registers 0-3 of
// lanes l and l + 32 holding the first block and registers 4-7 the second: lane l reads chunks
// 4 h + (l >> 5) and 4 h + 2 + (l >> 5) (16 codes each), and with K half 0 the rows' scale
// dwords, of which the instruction selects byte 2 h. With FP4 elements the same two chunks are
// the operands of two instructions (64 values each: registers 0-3 of lanes l and l + 32 the
// first, registers 4-7 the second), and each K half reads the rows' dword of its 4 blocks, of
// which the two instructions select bytes 0 and 2.
// With grouped scale copies gb is the step's group buffer plus the step's place in its rows'
// 16 bytes: 4 (step mod 4) with E4M3 elements, 8 (step mod 2) with E2M1 (whose K halves read the
// two dwords there).
template <int NB, int MX>
__device__ __forceinline__ void read_frags(const uint8_t* st, Frags& f, int h, int wm, int wn,
                                           int lane, const uint8_t* gb = nullptr) {
  const int r = lane & 31;
  const int c0 = MX ? h * 4 + (lane >> 5) : h * 4 + (lane >> 5) * 2;
  const int dc = MX ? 2 : 1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint8_t* ab = st + (wm * 128 + i * 32) * kBK;
    const uint4 lo = *reinterpret_cast<const uint4*>(ab + swz(r, c0));
    const uint4 hi = *reinterpret_cast<const uint4*>(ab + swz(r, c0 + dc));
    f.a[i] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                   (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
  // for NB == 1: 32 wn = 64 (q & 1) + 32 g, stored at 64 g + 32 (q & 1)
  const int b0 = NB == 2 ? wn * 64 : (wn & 1) * 64 + (wn >> 1) * 32;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const uint8_t* bb = st + kBM * kBK + (b0 + i * 32) * kBK;
    const uint4 lo = *reinterpret_cast<const uint4*>(bb + swz(r, c0));
    const uint4 hi = *reinterpret_cast<const uint4*>(bb + swz(r, c0 + dc));
    f.b[i] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                   (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
  if (mx_grouped(MX) && (MX == 4 || h == 0)) {
    // A tile row ra at 16 ra; B tile row rb in the copy of wave
    // 2 (rb >> 7) + ((rb >> 5) & 1), lane ((rb >> 6) & 1) 32 + (rb & 31) (full tile), or of wave
    // 2 (rb >> 6) + ((rb >> 4) & 1), lane ((rb >> 5) & 1) 16 + (rb & 15) (narrow half)
    const int sh = 8 * (lane >> 5);
    if (MX == 4) gb += 4 * h;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      f.sa[i] = *reinterpret_cast<const uint32_t*>(gb + (wm * 128 + i * 32 + r) * 16) >> sh;
    if (NB == 2) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int rb = b0 + i * 32 + r;
        const int wq = 2 * (rb >> 7) + ((rb >> 5) & 1), l = ((rb >> 6) & 1) * 32 + (rb & 31);
        f.sb[i] = *reinterpret_cast<const uint32_t*>(gb + 4096 + wq * 1024 + l * 16) >> sh;
      }
    } else {
      const int rb = 32 * wn + r;
      const int wq = 2 * (rb >> 6) + ((rb >> 4) & 1), l = ((rb >> 5) & 1) * 16 + (rb & 15);
      f.sb[0] = *reinterpret_cast<const uint32_t*>(gb + 4096 + wq * 1024 + l * 16) >> sh;
    }
  }
  if ((MX == 1 || MX == 2) && (MX == 2 || h == 0)) {  // 256-byte slots (A rows from 0, B from 2048)
    const uint32_t* sc = reinterpret_cast<const uint32_t*>(st + kStageBytes);
    const int sh = 8 * (lane >> 5);
    const int hd = MX == 2 ? 32 * h : 0;  // FP4: the K half's dword sits 32 dwords further
#pragma unroll
    for (int i = 0; i < 4; ++i) f.sa[i] = sc[64 * (wm * 4 + i) + hd + r] >> sh;
    if (NB == 2) {  // a slot per 32 rows
#pragma unroll
      for (int i = 0; i < NB; ++i) f.sb[i] = sc[512 + 64 * ((b0 >> 5) + i) + hd + r] >> sh;
    } else {        // narrow half: the wave's B rows are tile rows 32 wn + [0, 32), 16 per slot
      const int tr = 32 * wn + r;
      f.sb[0] = sc[512 + 64 * (tr >> 4) + hd + (tr & 15)] >> sh;
    }
  }
}

// One pass of the MFMAs of a K half over the wave's blocks; with E2M1 operands pass P (0 or 1)
// takes fragment registers 4P .. 4P + 3 and scale byte 2P. The first pass issues the batch's
// copies: one after each of its first four MFMAs (a copy instruction waits for the vector memory
// unit to take it, which here overlaps the matrix unit's work instead of holding up the next
// phase), and the scale copy after the fifth (grouped scale copies: after the sixth and seventh).
template <int NB, int MX, int H, int P>
__device__ __forceinline__ void mma_pass(const Frags& f, v16f (&acc)[NB][4], const Batch& b,
                                         uint32_t K, uint32_t dodd) {
#pragma unroll
  for (int bn = 0; bn < NB; ++bn)
#pragma unroll
    for (int bm = 0; bm < 4; ++bm) {
      if (mx_fp4(MX)) {
        const v8i bv = P == 0 ? f.b[bn]
                              : __builtin_shufflevector(f.b[bn], f.b[bn], 4, 5, 6, 7, 0, 1, 2, 3);
        const v8i av = P == 0 ? f.a[bm]
                              : __builtin_shufflevector(f.a[bm], f.a[bm], 4, 5, 6, 7, 0, 1, 2, 3);
        acc[bn][bm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            bv, av, acc[bn][bm], 4, 4, 2 * P, (int)f.sb[bn], 2 * P, (int)f.sa[bm]);
      } else if (MX) {
        acc[bn][bm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            f.b[bn], f.a[bm], acc[bn][bm], 0, 0, 2 * H, (int)f.sb[bn], 2 * H, (int)f.sa[bm]);
      } else {
        acc[bn][bm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            f.b[bn], f.a[bm], acc[bn][bm], 0, 0, 0, 0, 0, 0);
      }
      if (P == 0 && bn == 0) copy_block(b, K, dodd, bm);
      if ((MX == 1 || MX == 2) && P == 0 && bn == NB - 1 && bm == 0) copy_scales(b);
      if (mx_grouped(MX) && P == 0 && b.grp && bn == NB - 1 && bm == 1) copy_group_a(b);
      if (mx_grouped(MX) && P == 0 && b.grp && bn == NB - 1 && bm == 2) copy_group_b(b);
      __builtin_amdgcn_sched_barrier(0);
    }
}

// The MFMAs of one K half (8, or 4 in a narrow tile; twice as many with E2M1 operands, all
// blocks' first instructions before the second ones, so that none waits for the accumulator of
// the one before) with the copies of batch b.
template <int NB, int MX, int H>
__device__ __forceinline__ void mma8_copy(const Frags& f, v16f (&acc)[NB][4], const Batch& b,
                                          uint32_t K, uint32_t dodd) {
  mma_pass<NB, MX, H, 0>(f, acc, b, K, dodd);
  if constexpr (mx_fp4(MX)) mma_pass<NB, MX, H, 1>(f, acc, b, K, dodd);
}

// ---------------------------------------------------------------------------------------------
// epilogue
// ---------------------------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> packed bf16, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, bf2));
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

// Per pair of 8-column groups, each lane computes v for its 4 + 4 columns, swaps halves with its
// partner lane (l <-> l + 32) so that it holds 8 consecutive columns of one group, applies the
// activation or the gated residual there, and stores 16 bytes.
template <int EPI, int NB>
__device__ __forceinline__ void epilogue(const v16f (&acc)[NB][4], const Params& p, int m0, int n0,
                                         int mend, int wm, int wn, int lane, const uint8_t* pb) {
  const float* s_sa = reinterpret_cast<const float*>(pb);
  const float* s_sw = reinterpret_cast<const float*>(pb + 1024);
  const uint16_t* s_b = reinterpret_cast<const uint16_t*>(pb + 2048);
  const uint16_t* s_g = reinterpret_cast<const uint16_t*>(pb + 3072);
  const int hi = lane >> 5;
#pragma unroll
  for (int bm = 0; bm < 4; ++bm) {
    const int ml = wm * 128 + bm * 32 + (lane & 31);
    const int m = m0 + ml;
    const float sam = s_sa[ml];
#pragma unroll
    for (int bn = 0; bn < NB; ++bn) {
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        float v[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int g = gp * 2 + h;
          const int nl = wn * 32 * NB + bn * 32 + g * 8 + hi * 4;
          const float4 swv = *reinterpret_cast<const float4*>(s_sw + nl);
          const uint2 bb = *reinterpret_cast<const uint2*>(s_b + nl);
          if (is_mx(EPI)) {  // the block scales were applied by the matrix instruction
            v[h][0] = acc[bn][bm][g * 4 + 0] + bf16_lo(bb.x);
            v[h][1] = acc[bn][bm][g * 4 + 1] + bf16_hi(bb.x);
            v[h][2] = acc[bn][bm][g * 4 + 2] + bf16_lo(bb.y);
            v[h][3] = acc[bn][bm][g * 4 + 3] + bf16_hi(bb.y);
          } else {
            v[h][0] = fmaf(acc[bn][bm][g * 4 + 0] * sam, swv.x, bf16_lo(bb.x));
            v[h][1] = fmaf(acc[bn][bm][g * 4 + 1] * sam, swv.y, bf16_hi(bb.x));
            v[h][2] = fmaf(acc[bn][bm][g * 4 + 2] * sam, swv.z, bf16_lo(bb.y));
            v[h][3] = fmaf(acc[bn][bm][g * 4 + 3] * sam, swv.w, bf16_hi(bb.y));
          }
        }
        // Before: lane l < 32 holds columns [0, 4) of group 2gp in v[0] and of group 2gp+1 in
        // v[1]; lane l + 32 holds columns [4, 8) of both. After the swap lane l owns group 2gp
        // (v[0] = columns 0-3, v[1] = columns 4-7) and lane l + 32 owns group 2gp + 1.
#pragma unroll
        for (int j = 0; j < 4; ++j) swap_halves(v[0][j], v[1][j]);
        const int nl = wn * 32 * NB + bn * 32 + (gp * 2 + hi) * 8;
        const int n = n0 + nl;
        float y[8] = {v[0][0], v[0][1], v[0][2], v[0][3], v[1][0], v[1][1], v[1][2], v[1][3]};
        if (act_of(EPI) == EPI_GELU_TANH) {
#pragma unroll
          for (int j = 0; j < 8; ++j) y[j] = gelu_tanh(y[j]);
        }
        const bool live = m < mend && n < p.N;
        const size_t off = (size_t)m * (size_t)p.N + (size_t)n;
        if (act_of(EPI) == EPI_GATED_RESIDUAL) {
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
        o.x = pack_bf16(y[0], y[1]);
        o.y = pack_bf16(y[2], y[3]);
        o.z = pack_bf16(y[4], y[5]);
        o.w = pack_bf16(y[6], y[7]);
        if (live) *reinterpret_cast<uint4*>(p.out + off) = o;
      }
    }
  }
}

// QKV epilogue. The output row holds the query, key and value of `heads` heads of 128 channels
// (in that order). v = acc sa sw + bias as in the plain epilogue; query and key channels are then
// divided by their head's root mean square (over the head's 128 channels, plus eps) and scaled by
// the query or key weight, and each channel pair (2i, 2i + 1) is turned by the token's angle:
//   (a, b) -> (cos a - sin b, sin a + cos b),  cos, sin = rope_cos/sin[m, i];
// value channels pass through. Every output goes head-major, out[(head M + m) 128 + channel],
// rounded once to bf16.
// A wave's columns lie inside one head, but a head spans several waves (2 with NB = 2, 4 with
// NB = 1) of both groups, which the caller has aligned. A first pass turns the accumulators into
// v in place and writes each row's sum of squares over the wave's columns to `scratch` (4 KiB,
// [wn][256 rows]); after one workgroup barrier, which every wave reaches, each wave adds its
// head's sums in wave order, so all waves of a head use the same bits, and finishes from v.
// The rotary cosines and sines a lane needs for one unit (row block bm, column block bn): 4
// pairs per gp, through a buffer descriptor whose range is empty for value columns (those loads
// read zeros and touch no memory).
__device__ __forceinline__ void rope_load(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs,
                                          int bm, int bn, int lane, int dw, v4i (&c)[2],
                                          v4i (&sn)[2]) {
  const uint32_t row_off = (uint32_t)(bm * 32 + (lane & 31)) * 256u;
#pragma unroll
  for (int gp = 0; gp < 2; ++gp) {
    const uint32_t off =
        row_off + (uint32_t)((dw + bn * 32 + (gp * 2 + (lane >> 5)) * 8) >> 1) * 4u;
    c[gp] = __builtin_amdgcn_raw_buffer_load_b128(rc, off, 0, 0);
    sn[gp] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
  }
}

template <int NB, bool kQ8>
__device__ __forceinline__ void epilogue_qkv(v16f (&acc)[NB][4], const Params& p, int m0,
                                             int n0, int wm, int wn, int lane, const uint8_t* pb,
                                             float* scratch, uint32_t* qscr) {
  const float* s_sa = reinterpret_cast<const float*>(pb);
  const float* s_sw = reinterpret_cast<const float*>(pb + 1024);
  const uint16_t* s_b = reinterpret_cast<const uint16_t*>(pb + 2048);
  const uint16_t* s_w = reinterpret_cast<const uint16_t*>(pb + 3072);
  const int hi = lane >> 5;
  const QkvArgs qa = qkv_args();
  const int HD = qa.heads * 128;
  const int nw = n0 + wn * 32 * NB;            // this wave's first column (uniform)
  const int region = nw / HD;                  // 0 query, 1 key, 2 value, 3: past N
  const int head = (nw - region * HD) >> 7;
  const int dw = (nw - region * HD) & 127;     // channel of that column inside its head
  const bool normed = region < 2;
  // v for 4 + 4 columns of 8-column groups 2 gp and 2 gp + 1 (before the half swap)
  auto dequant = [&](int bm, int bn, int gp, float (&v)[2][4]) {
    const float sam = s_sa[wm * 128 + bm * 32 + (lane & 31)];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int g = gp * 2 + h;
      const int nl = wn * 32 * NB + bn * 32 + g * 8 + hi * 4;
      const float4 swv = *reinterpret_cast<const float4*>(s_sw + nl);
      const uint2 bb = *reinterpret_cast<const uint2*>(s_b + nl);
      v[h][0] = fmaf(acc[bn][bm][g * 4 + 0] * sam, swv.x, bf16_lo(bb.x));
      v[h][1] = fmaf(acc[bn][bm][g * 4 + 1] * sam, swv.y, bf16_hi(bb.x));
      v[h][2] = fmaf(acc[bn][bm][g * 4 + 2] * sam, swv.z, bf16_lo(bb.y));
      v[h][3] = fmaf(acc[bn][bm][g * 4 + 3] * sam, swv.w, bf16_hi(bb.y));
    }
  };
  // first pass: v into the accumulator registers, and the per-row sums of squares
#pragma unroll
  for (int bm = 0; bm < 4; ++bm) {
    float ss = 0.0f;
#pragma unroll
    for (int bn = 0; bn < NB; ++bn)
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        float v[2][4];
        dequant(bm, bn, gp, v);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[bn][bm][(gp * 2 + h) * 4 + j] = v[h][j];
            ss = fmaf(v[h][j], v[h][j], ss);
          }
      }
    if (normed) {
      // lanes l and l + 32 hold the two halves of the row's columns: lower + upper in both
      float lo_s = ss, up_s = ss;
      swap_halves(lo_s, up_s);
      const float row_ss = lo_s + up_s;
      if (hi == 0) scratch[wn * 256 + wm * 128 + bm * 32 + lane] = row_ss;
    }
  }
  // the rotary table rows of this wave's 128 rows (256 bytes each), through descriptors that
  // end at row M (rows past it read zeros; they are computed, never stored); block 0's loads
  // fly across the barrier, block bm + 1's while block bm is worked on
  const int mw = m0 + wm * 128;
  const int rows_w = p.M - mw < 128 ? (p.M - mw > 0 ? p.M - mw : 0) : 128;
  const int tab_bytes = normed ? rows_w * 256 : 0;
  const size_t tab0 = (size_t)(mw < p.M ? mw : 0) * 64;
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(qa.rope_cos + tab0), (short)0, tab_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsn = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(qa.rope_sin + tab0), (short)0, tab_bytes, 0x00020000);
  // units (bm, bn) in order; each prefetches the next unit's tables
  v4i cc[2], ss4[2];
  rope_load(rc, rsn, 0, 0, lane, dw, cc, ss4);
  phase_barrier();  // every wave's sums are in LDS
#pragma unroll
  for (int bm = 0; bm < 4; ++bm) {
    const int ml = wm * 128 + bm * 32 + (lane & 31);
    const int m = m0 + ml;
    float rr = 1.0f;
    if (normed) {
      float t;
      if (NB == 2) {
        const int w0 = wn & ~1;
        t = scratch[w0 * 256 + ml] + scratch[(w0 + 1) * 256 + ml];
      } else {
        t = ((scratch[ml] + scratch[256 + ml]) + scratch[512 + ml]) + scratch[768 + ml];
      }
      rr = 1.0f / __builtin_sqrtf(fmaf(t, 1.0f / 128.0f, qa.eps));
    }
    uint32_t amx = 0;  // kQ8: packed maxima of |bf16| over this lane's query or key outputs
#pragma unroll
    for (int bn = 0; bn < NB; ++bn) {
      const int nu = bm * NB + bn + 1;  // next unit
      v4i cn[2], sn4[2];
      if (nu < 4 * NB) rope_load(rc, rsn, nu / NB, nu % NB, lane, dw, cn, sn4);
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        float v[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int j = 0; j < 4; ++j) v[h][j] = acc[bn][bm][(gp * 2 + h) * 4 + j];
#pragma unroll
        for (int j = 0; j < 4; ++j) swap_halves(v[0][j], v[1][j]);
        const int d = dw + bn * 32 + (gp * 2 + hi) * 8;  // channel of y[0] inside the head
        float y[8] = {v[0][0], v[0][1], v[0][2], v[0][3], v[1][0], v[1][1], v[1][2], v[1][3]};
        if (normed) {
          const uint4 ww = *reinterpret_cast<const uint4*>(s_w + region * 128 + d);
          const uint32_t wv[4] = {ww.x, ww.y, ww.z, ww.w};
          const v4i c = cc[gp], sn = ss4[gp];
          const float cs[4] = {__int_as_float(c[0]), __int_as_float(c[1]), __int_as_float(c[2]),
                               __int_as_float(c[3])};
          const float sv[4] = {__int_as_float(sn[0]), __int_as_float(sn[1]),
                               __int_as_float(sn[2]), __int_as_float(sn[3])};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float a = (y[2 * j] * rr) * bf16_lo(wv[j]);
            const float b = (y[2 * j + 1] * rr) * bf16_hi(wv[j]);
            y[2 * j] = fmaf(cs[j], a, -(sv[j] * b));
            y[2 * j + 1] = fmaf(sv[j], a, cs[j] * b);
          }
        }
        uint4 o;
        o.x = pack_bf16(y[0], y[1]);
        o.y = pack_bf16(y[2], y[3]);
        o.z = pack_bf16(y[4], y[5]);
        o.w = pack_bf16(y[6], y[7]);
        if (kQ8 && region < 3) {
          // the bf16 results wait in the accumulator registers for the head row's scale
          acc[bn][bm][gp * 8 + 0] = __uint_as_float(o.x);
          acc[bn][bm][gp * 8 + 1] = __uint_as_float(o.y);
          acc[bn][bm][gp * 8 + 2] = __uint_as_float(o.z);
          acc[bn][bm][gp * 8 + 3] = __uint_as_float(o.w);
          amx = codec::absmax4(amx, o);
        } else if (m < p.M && region < 3) {
          uint16_t* out = region == 0 ? qa.out_q : region == 1 ? qa.out_k : qa.out_v;
          *reinterpret_cast<uint4*>(out + ((size_t)head * (size_t)p.M + (size_t)m) * 128 + d) = o;
        }
      }
      if (nu < 4 * NB) {
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
          cc[gp] = cn[gp];
          ss4[gp] = sn4[gp];
        }
      }
    }
    if (kQ8 && region < 3) {
      // the row's maximum over this wave's columns (lanes l and l + 32 hold its two halves)
      const uint32_t m16 = (amx & 0xFFFFu) > (amx >> 16) ? (amx & 0xFFFFu) : (amx >> 16);
      // (through the float form of the half swap, which moves the bits unchanged)
      float a0 = __uint_as_float(m16), a1 = a0;
      swap_halves(a0, a1);
      const uint32_t o16 = __float_as_uint(a0) > __float_as_uint(a1) ? __float_as_uint(a0)
                                                                     : __float_as_uint(a1);
      if (hi == 0) qscr[wn * 256 + ml] = o16;
    }
  }
  if constexpr (kQ8) {
    // Queries, keys and values to E4M3 with one scale per head row, exactly as dq_quantize_fp8
    // (and, for the values, dq_quantize_v_fp8) encode those bf16 rows: the row's |max| over the
    // head's waves, scale = amax / 448, then the quantizer's encoder on each group of 8 values.
    phase_barrier();  // every wave's row maxima are in LDS (every wave reaches it)
    if (region < 3) {
      uint8_t* codes = reinterpret_cast<uint8_t*>(region == 0 ? qa.out_q
                                                  : region == 1 ? qa.out_k : qa.out_v);
      float* scales = region == 0 ? qa.scale_q : region == 1 ? qa.scale_k : qa.scale_v;
      // values: this wave's 1 KiB of LDS for turning 32 rows x 32 channels of codes around
      uint8_t* vtile = reinterpret_cast<uint8_t*>(qscr + 1024) + (wm * 4 + wn) * 1024;
      const int w0 = NB == 2 ? (wn & ~1) : (wn & ~3);
#pragma unroll
      for (int bm = 0; bm < 4; ++bm) {
        const int ml = wm * 128 + bm * 32 + (lane & 31);
        const int m = m0 + ml;
        uint32_t mx = 0;
#pragma unroll
        for (int i = 0; i < 4 / NB; ++i) {
          const uint32_t o = qscr[(w0 + i) * 256 + ml];
          mx = mx > o ? mx : o;
        }
        const float amax = __uint_as_float(mx << 16);
        const float sc = amax / codec::kE4M3Max;
        float ss = sc, y = 0.0f;
        const int kind = mx == 0 ? 0 : sc < codec::kFltMinNormal ? 1
                                     : amax < codec::kTinyAmax ? 2 : 3;
        if (kind == 2) {
          ss = sc * 0x1p64f;
          y = 1.0f / ss;
        } else if (kind == 3) {
          y = 1.0f / sc;
        }
        const bool live = m < p.M;
        const size_t row = (size_t)head * (size_t)p.M + (size_t)(live ? m : 0);
        if (live && hi == 0 && wn == w0) scales[row] = sc;
#pragma unroll
        for (int bn = 0; bn < NB; ++bn) {
          uint2 c[2];
#pragma unroll
          for (int gp = 0; gp < 2; ++gp) {
            const uint4 v = make_uint4(__float_as_uint(acc[bn][bm][gp * 8 + 0]),
                                       __float_as_uint(acc[bn][bm][gp * 8 + 1]),
                                       __float_as_uint(acc[bn][bm][gp * 8 + 2]),
                                       __float_as_uint(acc[bn][bm][gp * 8 + 3]));
            if (kind == 0)
              c[gp] = codec::signs8(v);
            else if (kind == 1)
              c[gp] = codec::encode8<1, false>(v, sc, 0.0f);
            else if (kind == 2)
              c[gp] = codec::encode8<0, true>(v, ss, y);
            else
              c[gp] = codec::encode8<0, false>(v, sc, y);
          }
          if (region < 2) {  // queries and keys: [head row][channel]
#pragma unroll
            for (int gp = 0; gp < 2; ++gp) {
              const int d = dw + bn * 32 + (gp * 2 + hi) * 8;
              if (live) *reinterpret_cast<uint2*>(codes + row * 128 + d) = c[gp];
            }
          } else {
            // values: [head][channel][token]. The 32 rows x 32 channels of codes go into the
            // wave's LDS tile as [channel][row] bytes, and come back as 16 rows of one channel
            // per lane, a 16-byte store (M is a multiple of 16, so a chunk is all in or out)
#pragma unroll
            for (int gp = 0; gp < 2; ++gp)
#pragma unroll
              for (int i = 0; i < 8; ++i) {
                const int cl = (gp * 2 + hi) * 8 + i;
                const uint32_t w = i < 4 ? c[gp].x : c[gp].y;
                vtile[cl * 32 + (lane & 31)] = (uint8_t)(w >> (8 * (i & 3)));
              }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's tile is written
            const int cl = lane >> 1, half = lane & 1;
            const uint4 t = *reinterpret_cast<const uint4*>(vtile + cl * 32 + half * 16);
            const int mt = m0 + wm * 128 + bm * 32 + half * 16;  // first row of the chunk
            if (mt < p.M)
              *reinterpret_cast<uint4*>(
                  codes + ((size_t)head * 128 + (size_t)(dw + bn * 32 + cl)) * (size_t)p.M +
                  (size_t)mt) = t;
            __builtin_amdgcn_s_waitcnt(0xC07F);  // (the tile is read before it is written again)
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// split tiles
// ---------------------------------------------------------------------------------------------

// Partial tiles live in one region addressed through one buffer descriptor; their loads
// and stores carry the device-coherence bit (sc1), so they are seen across XCDs without
// flushing or invalidating caches.
constexpr int kCoherent = 16;  // sc1

// A wave's 128 accumulators into partial tile `slot` (byte offset): wave-major, then 4-register
// groups, then lanes, so that every store moves 1 KiB contiguous.
__device__ __forceinline__ void store_part(const v16f (&acc)[2][4], __amdgpu_buffer_rsrc_t rs,
                                           uint32_t slot, int wave, int lane) {
  const uint32_t base = slot + (uint32_t)(wave * 32 * 64 + lane) * 16u;
#pragma unroll
  for (int g4 = 0; g4 < 32; ++g4) {
    const int blk = g4 >> 2, e = (g4 & 3) * 4;
    const v16f& a = acc[blk >> 2][blk & 3];
    const v4i x = (v4i){__float_as_int(a[e]), __float_as_int(a[e + 1]), __float_as_int(a[e + 2]),
                        __float_as_int(a[e + 3])};
    __builtin_amdgcn_raw_buffer_store_b128(x, rs, base + (uint32_t)g4 * 1024u, 0, kCoherent);
  }
}

// acc (+)= partial tile `slot`, sixteen 4-register groups in flight at a time (the fragment
// registers are free here), so a partial costs two memory round trips per wave.
template <bool FIRST>
__device__ __forceinline__ void add_part(v16f (&acc)[2][4], __amdgpu_buffer_rsrc_t rs,
                                         uint32_t slot, int wave, int lane) {
  const uint32_t base = slot + (uint32_t)(wave * 32 * 64 + lane) * 16u;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    v4i x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      x[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, base + (uint32_t)(c * 16 + i) * 1024u, 0,
                                                   kCoherent);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int g4 = c * 16 + i;
      const int blk = g4 >> 2, e = (g4 & 3) * 4;
      v16f& a = acc[blk >> 2][blk & 3];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float y = __int_as_float(x[i][j]);
        a[e + j] = FIRST ? y : a[e + j] + y;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Byte offset of the partial tile of part p.
__device__ __forceinline__ uint32_t part_slot(int p) {
  return (uint32_t)p * (uint32_t)(kPartFloats * 4);
}

// Part `part` of left-over tile t is in acc (both groups are done with its MFMAs). Store it and
// count its arrival. The last part to arrive loads all parts of the tile, in part order, into
// acc and clears the tile's counter for the next call; it returns true and the caller applies
// the epilogue.
__device__ bool finish_split(v16f (&acc)[2][4], const Params& p, int t, int part, int wave,
                             int lane, int* s_last) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      p.part, 0, (int)p.part_bytes, 0x00020000);
  store_part(acc, rs, part_slot(part), wave, lane);
  wait_vmem();
  phase_barrier();  // every wave's part is stored
  if (threadIdx.x == 0) {
    const uint32_t old =
        __hip_atomic_fetch_add(p.flags + (t - p.tail0), 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    *s_last = old == (uint32_t)(p.splits - 1);
  }
  phase_barrier();
  if (!*s_last) return false;
  const int tt = t - p.tail0;
  for (int j = 0; j < p.splits; ++j) {
    const uint32_t slot = part_slot(j * p.tail_tiles + tt);
    if (j == 0)
      add_part<true>(acc, rs, slot, wave, lane);
    else
      add_part<false>(acc, rs, slot, wave, lane);
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(p.flags + (t - p.tail0), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// ---------------------------------------------------------------------------------------------
// kernel
// ---------------------------------------------------------------------------------------------

__device__ __forceinline__ bool same_tile(const Cursor& a, const Cursor& b) {
  return a.t == b.t && a.half == b.half;
}

// NB = 2: whole tiles and cut parts; NB = 1: the narrow halves of left-over tiles.
template <int EPI, int NB>
__global__ void __launch_bounds__(kThreads) gemm_fp8_pp(Params p) {
  constexpr int MX = mx_kind(EPI);
  constexpr int kStage = stage_bytes(EPI);
  constexpr int kOps = batch_ops(EPI);
  // (EPI_QKV_Q8: 4 KiB more for the rows' absolute maxima exchanged between the waves of a head,
  // and 1 KiB per wave for turning value codes around)
  constexpr int kQ8Bytes = EPI == EPI_QKV_Q8 ? 4096 + 8 * 1024 : 0;
  // (grouped scale copies: the two group buffers)
  constexpr int kGrpBytes = mx_grouped(MX) ? kGroupBytes : 0;
  constexpr int GS = group_steps(MX);
  __shared__ __attribute__((aligned(1024)))
  uint8_t lds[2 * kStage + kParamBufs * kParamBytes + kQ8Bytes + kGrpBytes];
  __shared__ int s_last;
  uint8_t* pbuf = lds + 2 * kStage;
  uint32_t* qscr = reinterpret_cast<uint32_t*>(pbuf + kParamBufs * kParamBytes);
  uint8_t* gbase = pbuf + kParamBufs * kParamBytes + kQ8Bytes;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wave >> 2, q = wave & 3;
  const int wm = q >> 1, wn = (q & 1) * 2 + g;
  const int G = gridDim.x;
  const int b = blockIdx.x;
  const int v = (G & 7) == 0 ? (b & 7) * (G >> 3) + (b >> 3) : b;
  const int nk = p.nk;
  const Work w = work_of(p, v, G);
  const int nsteps = w.n_dp * nk + w.n_parts * p.part_steps;
  if (nsteps == 0) return;  // more workgroups than items (the whole workgroup leaves)
  const uint32_t uK = (uint32_t)p.K;

  // copy addressing of this lane: row (lane >> 3) of an 8-row block, chunk position lane & 7
  const int r = lane >> 3;
  const uint32_t cE = (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
  const uint32_t cO = (uint32_t)((lane & 7) ^ (((r >> 1) + 4) & 7));
  const uint32_t vlane = (uint32_t)r * uK + cE * 16u;
  const uint32_t dodd = (cO - cE) * 16u;  // added (mod 2^32) in odd blocks

  // Pipeline. Step S is read from stage S & 1 in four phases; group 1 runs one phase behind
  // group 0, so in every phase one wave per SIMD reads fragments and the other issues its MFMAs
  // together with one copy batch (4 instructions):
  //   phase A: G0 reads K half 0 of S   | G1 MFMAs (half 1 of S - 1) + batch 0 of S + 1
  //   phase B: G1 reads K half 0 of S   | G0 MFMAs (half 0 of S)     + batch 1 of S + 1
  //   phase C: G0 reads K half 1 of S   | G1 MFMAs (half 0 of S)     + batch 2 of S + 1
  //   phase D: G1 reads K half 1 of S   | G0 MFMAs (half 1 of S)     + batch 3 of S + 2
  // Stage (S + 1) & 1 is free from phase A of S (step S - 1 was read by the end of D of S - 1);
  // group 0's B rows of stage S & 1 are free from phase D of S (G0 read them in A and C), so
  // batch 3 runs one step ahead. Each wave waits for its own batches before the barrier that
  // precedes their first reader: G1 at the end of D (batch 0), G0 at the end of D (batch 1, and
  // batch 3 of the step before), G1 at the end of A (batch 2); every batch has two to four
  // phases to land.
  Cursor c1, c2;  // steps S + 1 and S + 2
  TileDesc d1, d2;
  {
    Cursor c0;
    c0.item = 0;
    cursor_item<NB>(p, w, v, G, c0);
    const TileDesc d0 = tile_desc<NB, MX>(p, c0.t, c0.half);
    if (g == 0) {
      copy_batch<NB, MX>(d0, uK, c0.k, lds, vlane, dodd, q, 0);
      copy_batch<NB, MX>(d0, uK, c0.k, lds, vlane, dodd, q, 1, gbase);
      copy_params<EPI>(p, d0, pbuf, q, lane);
    } else {
      copy_batch<NB, MX>(d0, uK, c0.k, lds, vlane, dodd, q, 2);
      copy_batch<NB, MX>(d0, uK, c0.k, lds, vlane, dodd, q, 3);
    }
    c1 = c0;
    cursor_next<NB>(p, w, v, G, c1);
    d1 = same_tile(c1, c0) ? d0 : tile_desc<NB, MX>(p, c1.t, c1.half);
    c2 = c1;
    cursor_next<NB>(p, w, v, G, c2);
    d2 = same_tile(c2, c1) ? d1 : tile_desc<NB, MX>(p, c2.t, c2.half);
  }
  wait_vmem();
  phase_barrier();
  // batch 3 of step 1 (G0, as in phase D of step -1) and batch 0 of step 1 (G1, as in its
  // MFMA phase of step -1), then group 1 falls one phase behind
  if (nsteps > 1)
    copy_batch<NB, MX>(d1, uK, c1.k, lds + kStage, vlane, dodd, q, g == 0 ? 3 : 0);
  if (g == 1) phase_barrier();

  Frags f;
  int S = 0;     // steps done; step S is in stage S & 1
  int part = 0;  // items done; item i's parameters are in buffer i % 3
  Cursor c;
  c.item = 0;
  cursor_item<NB>(p, w, v, G, c);
  while (S < nsteps) {
    const int t = c.t, half = c.half, cutp = c.cut, len = c.kend - c.k;
    v16f acc[NB][4];
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = (v16f){};
    for (int j = 0; j < len; ++j, ++S) {
      uint8_t* st = lds + (S & 1) * kStage;
      uint8_t* st1 = lds + ((S + 1) & 1) * kStage;
      const bool has1 = S + 1 < nsteps, has2 = S + 2 < nsteps;
      const bool starts = has1 && (j + 1 == len);  // step S + 1 begins the next item
      // reads of K half 0 (G0: phase A, G1: phase B)
      const uint8_t* gb = gbase + ((S / GS) & 1) * 8192 + (S % GS) * (16 / GS);
      read_frags<NB, MX>(st, f, 0, wm, wn, lane, gb);
      phase_barrier();
      // MFMAs of K half 0 with batch g + 1 of step S + 1 (G0: phase B, G1: phase C)
      // (grouped scale copies: G0's batch 1 also carries the scales of the group step S + 1 starts)
      mma8_copy<NB, MX, 0>(f, acc,
                           batch_of<NB, MX>(d1, uK, c1.k, st1, vlane, q, g + 1, has1,
                                            mx_grouped(MX) && g == 0
                                                ? gbase + (((S + 1) / GS) & 1) * 8192
                                                : nullptr),
                           uK, dodd);
      phase_barrier();
      // reads of K half 1 (G0: phase C, G1: phase D); G0 starts the next item's parameters,
      // G1 waits for its batch 0 of step S + 1
      read_frags<NB, MX>(st, f, 1, wm, wn, lane, gb);
      if (g == 0) {
        if (starts)
          copy_params<EPI>(p, d1, pbuf + ((part + 1) % kParamBufs) * kParamBytes, q, lane);
      } else {
        if (has1) wait_vmem_but<kOps>(); else wait_vmem();
      }
      phase_barrier();
      // MFMAs of K half 1 (G0: phase D, G1: phase A of S + 1) with batch 3 (G0) or 0 (G1) of
      // step S + 2, into this stage; the cursors move on meanwhile; then every wave waits for
      // all but that batch
      mma8_copy<NB, MX, 1>(f, acc, batch_of<NB, MX>(d2, uK, c2.k, st, vlane, q, g == 0 ? 3 : 0, has2), uK,
                    dodd);
      c1 = c2;
      d1 = d2;
      cursor_next<NB>(p, w, v, G, c2);
      if (!same_tile(c2, c1) && S + 3 < nsteps) d2 = tile_desc<NB, MX>(p, c2.t, c2.half);
      wait_vmem_but<kOps>();
      phase_barrier();
    }
    const Geo gi = item_geo<NB>(p, t, half);
    const int m0 = gi.m0, n0 = gi.n0;
    const uint8_t* pb = pbuf + (part % kParamBufs) * kParamBytes;
    // the QKV epilogue exchanges sums between the groups, so like a cut tile it first aligns
    // them; its scratch is the parameter buffer of the item after next (free until then)
    float* scratch = reinterpret_cast<float*>(pbuf + ((part + 2) % kParamBufs) * kParamBytes);
    if constexpr (NB == 2) {
      const bool cut = cutp >= 0;
      const bool align = cut || is_qkv(EPI);
      bool write = true;
      if (align && g == 0) phase_barrier();  // group 1's last MFMAs of this item are done
      if (cut) write = finish_split(acc, p, t, cutp, wave, lane, &s_last);
      if (write) {
        if constexpr (is_qkv(EPI))
          epilogue_qkv<2, EPI == EPI_QKV_Q8>(acc, p, m0, n0, wm, wn, lane, pb, scratch, qscr);
        else
          epilogue<EPI, 2>(acc, p, m0, n0, gi.mend, wm, wn, lane, pb);
      }
      if (align && g == 1) phase_barrier();  // back to one phase behind
    } else {
      if constexpr (is_qkv(EPI)) {
        if (g == 0) phase_barrier();
        epilogue_qkv<1, EPI == EPI_QKV_Q8>(acc, p, m0, n0, wm, wn, lane, pb, scratch, qscr);
        if (g == 1) phase_barrier();
      } else {
        epilogue<EPI, 1>(acc, p, m0, n0, gi.mend, wm, wn, lane, pb);
      }
    }
    ++part;
    ++c.item;
    if (c.item < w.n_dp + w.n_parts) cursor_item<NB>(p, w, v, G, c);
  }
  if (g == 0) phase_barrier();  // matches group 1's extra barrier
  wait_vmem();                  // the empty batches of the last two steps
}

template <int EPI>
hipError_t launch_epi(const Params& p, int grid, int narrow_grid, hipStream_t stream) {
  if (grid > 0) {
    Params a = p;
    if (narrow_grid > 0) a.tail_tiles = 0;  // the halves run in the second launch
    a.narrow = 0;
    hipLaunchKernelGGL((gemm_fp8_pp<EPI, 2>), dim3(grid), dim3(kThreads), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (narrow_grid > 0) {
    Params b = p;
    b.dp_tiles = 0;
    b.narrow = 1;
    hipLaunchKernelGGL((gemm_fp8_pp<EPI, 1>), dim3(narrow_grid), dim3(kThreads), 0, stream, b);
    return hipGetLastError();
  }
  return hipSuccess;
}

// Compute units of the current device, queried once per device.
int compute_units() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = __atomic_load_n(&cached[dev], __ATOMIC_RELAXED);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    __atomic_store_n(&cached[dev], n, __ATOMIC_RELAXED);
  }
  return n;
}

}  // namespace

// The schedule of one problem: full rounds of whole tiles (one per compute unit per round), then
// the T mod G tiles left over, run whole, as narrow halves in a second launch, or cut along K.
struct Plan {
  int64_t grid = 0;        // workgroups of the launch of whole tiles / parts (0: none)
  int64_t narrow_grid = 0; // workgroups of the launch of narrow halves (0: none)
  int64_t dp_tiles = 0, left = 0, splits = 1;
  int narrow = 0;
  uint64_t workspace = 0;  // workspace bytes the plan uses
};

// Chosen by counting steps of the last round:
//   whole tiles: nk steps;
//   narrow halves (when all halves fit on the device at once): a 256 x 128 half moves 3/4 of
//     a tile's operand bytes for half its MFMAs and takes about kNarrow of a tile's time;
//   cut into s parts along K (s divides nk, s <= 8), when the parts' partial tiles fit in
//     `budget` bytes of workspace: the last round takes ceil(left s / G) parts of nk / s steps
//     per workgroup, every part stores a 256 x 256 fp32 partial tile and the part that
//     finishes a tile loads the s - 1 others; a partial tile moves at the compute unit's share
//     of HBM bandwidth (at most about 60 GB/s for one unit, 5.6 TB/s for the chip; one step is
//     about 1.5 us on a busy chip). A cut must win by 20 %.
static Plan choose_plan(int64_t tilesM, int64_t K, int64_t N, int64_t cus, uint64_t budget) {
  Plan pl;
  const int64_t tiles = tilesM * ((N + kBN - 1) / kBN), nk = K / kBK;
  pl.grid = tiles < cus ? tiles : cus;
  const int64_t rounds = tiles / cus;
  pl.dp_tiles = rounds * cus;
  pl.left = tiles - pl.dp_tiles;
  const int64_t left = pl.left;
  if (left > 0) {
    constexpr double kNarrow = 0.7, kStepUs = 1.5, kUnitGBs = 60.0, kChipGBs = 5600.0;
    double best = (double)nk;
    if (2 * left <= cus && kNarrow * nk < best) {
      best = kNarrow * nk;
      pl.narrow = 1;
    }
    if (left <= kMaxCutTiles) {
      double best_cut = 0.8 * best;
      for (int64_t s = 2; s <= kMaxSplits; ++s) {
        if (nk % s != 0 || left * s > kMaxParts) continue;
        if (kCounterBytes + (uint64_t)(left * s) * kPartialBytes > budget) continue;
        const int64_t active = left * s < cus ? left * s : cus;
        const double unit_gbs = kChipGBs / (double)active < kUnitGBs
                                    ? kChipGBs / (double)active
                                    : kUnitGBs;
        const double part_steps_cost = (double)kPartialBytes / (unit_gbs * 1e3) / kStepUs;
        const double per_unit = (double)((left * s + active - 1) / active);
        const double cost = per_unit * ((double)(nk / s) + part_steps_cost) +
                            (double)(s - 1) * part_steps_cost;
        if (cost < best_cut) {
          best_cut = cost;
          pl.splits = s;
          pl.narrow = 0;
        }
      }
    }
    if (pl.dp_tiles == 0 && !pl.narrow) {
      const int64_t items = left * pl.splits;
      pl.grid = items < cus ? items : cus;
    }
  }
  if (pl.narrow) {
    pl.narrow_grid = 2 * left;
    pl.grid = pl.dp_tiles > 0 ? cus : 0;
  }
  if (pl.splits > 1) pl.workspace = kCounterBytes + (uint64_t)(left * pl.splits) * kPartialBytes;
  return pl;
}

// Sizes and schedule into a Params whose pointers and segments are set, then the launches.
static hipError_t schedule_and_launch(Params& p, int64_t M, int64_t K, int64_t N, int epilogue,
                                      void* workspace, uint64_t workspace_bytes,
                                      hipStream_t stream) {
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.tilesM = p.seg.trow0[p.seg.nseg];
  p.tilesN = (int)((N + kBN - 1) / kBN);
  p.nk = (int)(K / kBK);
  p.tiles = p.tilesM * p.tilesN;
  const Plan pl = choose_plan(p.tilesM, K, N, compute_units(), workspace ? workspace_bytes : 0);
  p.dp_tiles = (int)pl.dp_tiles;
  p.tail0 = (int)pl.dp_tiles;
  p.tail_tiles = (int)pl.left;
  p.splits = (int)pl.splits;
  p.part_steps = (int)(p.nk / pl.splits);
  p.narrow = pl.narrow;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  p.flags = pl.splits > 1 ? reinterpret_cast<uint32_t*>(ws) : nullptr;
  p.part = pl.splits > 1 ? reinterpret_cast<float*>(ws + kCounterBytes) : nullptr;
  p.part_bytes = pl.splits > 1 ? (uint32_t)(pl.workspace - kCounterBytes) : 0u;
  const int g = (int)pl.grid, ng = (int)pl.narrow_grid;
  switch (epilogue) {
    case EPI_BIAS: return launch_epi<EPI_BIAS>(p, g, ng, stream);
    case EPI_GELU_TANH: return launch_epi<EPI_GELU_TANH>(p, g, ng, stream);
    case EPI_QKV: return launch_epi<EPI_QKV>(p, g, ng, stream);
    case EPI_QKV_Q8: return launch_epi<EPI_QKV_Q8>(p, g, ng, stream);
    case EPI_MX_BIAS: return launch_epi<EPI_MX_BIAS>(p, g, ng, stream);
    case EPI_MX_GELU_TANH: return launch_epi<EPI_MX_GELU_TANH>(p, g, ng, stream);
    case EPI_MXG_BIAS: return launch_epi<EPI_MXG_BIAS>(p, g, ng, stream);
    case EPI_MXG_GELU_TANH: return launch_epi<EPI_MXG_GELU_TANH>(p, g, ng, stream);
    case EPI_MX4_BIAS: return launch_epi<EPI_MX4_BIAS>(p, g, ng, stream);
    case EPI_MX4_GELU_TANH: return launch_epi<EPI_MX4_GELU_TANH>(p, g, ng, stream);
    case EPI_MX4_GATED: return launch_epi<EPI_MX4_GATED>(p, g, ng, stream);
    case EPI_MX4G_BIAS: return launch_epi<EPI_MX4G_BIAS>(p, g, ng, stream);
    case EPI_MX4G_GELU_TANH: return launch_epi<EPI_MX4G_GELU_TANH>(p, g, ng, stream);
    case EPI_MX4G_GATED: return launch_epi<EPI_MX4G_GATED>(p, g, ng, stream);
    default: return launch_epi<EPI_GATED_RESIDUAL>(p, g, ng, stream);
  }
}

// Row segments of nseg sizes (host array) into p.seg's rows and tile rows; the caller sets the
// per-segment pointers. Returns the total number of rows.
static int64_t set_segments(Params& p, int64_t nseg, const int64_t* rows) {
  p.seg.nseg = (int)nseg;
  int64_t r = 0, tr = 0;
  for (int64_t i = 0; i < nseg; ++i) {
    p.seg.row0[i] = (int)r;
    p.seg.trow0[i] = (int)tr;
    r += rows[i];
    tr += (rows[i] + kBM - 1) / kBM;
  }
  p.seg.row0[nseg] = (int)r;
  p.seg.trow0[nseg] = (int)tr;
  return r;
}

uint64_t linear_workspace_bytes(int64_t M, int64_t K, int64_t N) {
  if (M == 0) return 0;
  return choose_plan((M + kBM - 1) / kBM, K, N, compute_units(), ~uint64_t(0)).workspace;
}

uint64_t linear_segmented_workspace_bytes(int64_t nseg, const int64_t* rows, int64_t K,
                                          int64_t N) {
  int64_t tiles_m = 0;
  for (int64_t i = 0; i < nseg; ++i) tiles_m += (rows[i] + kBM - 1) / kBM;
  if (tiles_m == 0) return 0;
  return choose_plan(tiles_m, K, N, compute_units(), ~uint64_t(0)).workspace;
}

hipError_t launch_linear(const uint8_t* q, const float* scale, int64_t M, int64_t K,
                         const uint8_t* qw, const float* w_scale, int64_t N, const uint16_t* bias,
                         int epilogue, const uint16_t* gate, const uint16_t* residual,
                         uint16_t* out, void* workspace, uint64_t workspace_bytes,
                         hipStream_t stream) {
  return launch_linear_segmented(q, scale, 1, &M, K, &qw, &w_scale, N, &bias, epilogue, &gate,
                                 residual, out, workspace, workspace_bytes, stream);
}

hipError_t launch_linear_segmented(const uint8_t* q, const float* scale, int64_t nseg,
                                   const int64_t* seg_rows, int64_t K,
                                   const uint8_t* const* qw, const float* const* w_scale,
                                   int64_t N, const uint16_t* const* bias, int epilogue,
                                   const uint16_t* const* gate, const uint16_t* residual,
                                   uint16_t* out, void* workspace, uint64_t workspace_bytes,
                                   hipStream_t stream) {
  Params p{};
  const int64_t M = set_segments(p, nseg, seg_rows);
  if (M == 0) return hipSuccess;
  p.A = q;
  p.sa = scale;
  p.residual = residual;
  p.out = out;
  for (int64_t i = 0; i < nseg; ++i) {
    p.seg.B[i] = qw[i];
    p.seg.sw[i] = w_scale[i];
    p.seg.bias[i] = bias[i];
    p.seg.gate[i] = gate[i];
  }
  return schedule_and_launch(p, M, K, N, epilogue, workspace, workspace_bytes, stream);
}

// Block-scaled (MX) linear: the same kernel in MX mode (no workspace, so the left-over tiles of
// the last round run whole or as narrow halves, never cut).
hipError_t launch_linear_mx(const uint8_t* qa, const uint8_t* sa, int64_t M, int64_t K,
                            const uint8_t* qw, const uint8_t* sw, int64_t N, const uint16_t* bias,
                            int epilogue, uint16_t* out, hipStream_t stream) {
  Params p{};
  if (set_segments(p, 1, &M) == 0) return hipSuccess;
  p.A = qa;
  p.out = out;
  p.mxa = sa;
  p.seg.B[0] = qw;
  p.seg.sw[0] = reinterpret_cast<const float*>(sw);
  p.seg.bias[0] = bias;
  // grouped scale copies when every item's K steps come in whole groups of 4
  const bool grouped = (K / kBK) % 4 == 0;
  const int epi = grouped ? (epilogue == 1 ? EPI_MXG_GELU_TANH : EPI_MXG_BIAS)
                          : (epilogue == 1 ? EPI_MX_GELU_TANH : EPI_MX_BIAS);
  return schedule_and_launch(p, M, K, N, epi, nullptr,
                             0, stream);
}

// MXFP4 linear over row segments with their own weights: the same kernel in MX mode with E2M1
// operands. p.K counts bytes (K / 2), so a K step of 128 bytes per row covers 256 values and 8
// scale bytes.
hipError_t launch_linear_mxfp4_segmented(const uint8_t* qa, const uint8_t* sa, int64_t nseg,
                                         const int64_t* seg_rows, int64_t K,
                                         const uint8_t* const* qw, const uint8_t* const* sw,
                                         int64_t N, const uint16_t* const* bias, int epilogue,
                                         const uint16_t* const* gate, const uint16_t* residual,
                                         uint16_t* out, hipStream_t stream) {
  Params p{};
  const int64_t M = set_segments(p, nseg, seg_rows);
  if (M == 0) return hipSuccess;
  p.A = qa;
  p.mxa = sa;
  p.residual = residual;
  p.out = out;
  for (int64_t i = 0; i < nseg; ++i) {
    p.seg.B[i] = qw[i];
    p.seg.sw[i] = reinterpret_cast<const float*>(sw[i]);
    p.seg.bias[i] = bias[i];
    p.seg.gate[i] = gate[i];
  }
  // grouped scale copies when every item's K steps (256 values each) come in pairs
  const bool grouped = (K / 2 / kBK) % 2 == 0;
  const int epi = grouped ? (epilogue == 1 ? EPI_MX4G_GELU_TANH
                             : epilogue == 2 ? EPI_MX4G_GATED : EPI_MX4G_BIAS)
                          : (epilogue == 1 ? EPI_MX4_GELU_TANH
                             : epilogue == 2 ? EPI_MX4_GATED : EPI_MX4_BIAS);
  return schedule_and_launch(p, M, K / 2, N, epi, nullptr, 0, stream);
}

// ---------------------------------------------------------------------------------------------
// allocation-free entry: the library's own scratch in place of a caller workspace
// ---------------------------------------------------------------------------------------------

// The scratch: arrival counters, then room for kNoAllocParts partial tiles. Every GPU the
// library runs on holds its own copy until the process ends; all calls on one GPU share it.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

// Clears the arrival counters before a call that cuts tiles (a call cut short elsewhere could
// have left them nonzero): a fill kernel, so that a captured graph holds no memset node.
namespace {
__global__ void __launch_bounds__(256) clear_counters(uint32_t* c, int n) {
  for (int i = threadIdx.x; i < n; i += 256) c[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
}  // namespace

// The device address of the current device's scratch, looked up once per device (with that
// device current) and kept. The array's name is only a host-side stand-in for it.
static hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (ptr == nullptr) {
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (ptr == nullptr) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return hipSuccess;
}

hipError_t launch_linear_noalloc(const uint8_t* q, const float* scale, int64_t M, int64_t K,
                                 const uint8_t* qw, const float* w_scale, int64_t N,
                                 const uint16_t* bias, int epilogue, const uint16_t* gate,
                                 const uint16_t* residual, uint16_t* out, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  void* ws = nullptr;
  hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  if (choose_plan((M + kBM - 1) / kBM, K, N, compute_units(), kNoAllocScratchBytes).splits > 1) {
    hipLaunchKernelGGL(clear_counters, dim3(1), dim3(256), 0, stream,
                       static_cast<uint32_t*>(ws), (int)kMaxCutTiles);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_linear(q, scale, M, K, qw, w_scale, N, bias, epilogue, gate, residual, out, ws,
                       kNoAllocScratchBytes, stream);
}

hipError_t launch_linear_qkv(const uint8_t* q, const float* scale, int64_t M, int64_t K,
                             const uint8_t* qw, const float* w_scale, int64_t heads,
                             const uint16_t* bias, const uint16_t* norm_qk, const float* rope_cos,
                             const float* rope_sin, float eps, uint16_t* out_q, uint16_t* out_k,
                             uint16_t* out_v, void* workspace, uint64_t workspace_bytes,
                             hipStream_t stream) {
  if (M == 0) return hipSuccess;
  Params p{};
  set_segments(p, 1, &M);
  p.A = q;
  p.sa = scale;
  p.seg.B[0] = qw;
  p.seg.sw[0] = w_scale;
  p.seg.bias[0] = bias;
  p.qkv.norm_qk = norm_qk;
  p.qkv.rope_cos = rope_cos;
  p.qkv.rope_sin = rope_sin;
  p.qkv.out_q = out_q;
  p.qkv.out_k = out_k;
  p.qkv.out_v = out_v;
  p.qkv.eps = eps;
  p.qkv.heads = (int)heads;
  return schedule_and_launch(p, M, K, 3 * heads * 128, EPI_QKV, workspace, workspace_bytes,
                             stream);
}

hipError_t launch_linear_qkv_q8(const uint8_t* q, const float* scale, int64_t M, int64_t K,
                                const uint8_t* qw, const float* w_scale, int64_t heads,
                                const uint16_t* bias, const uint16_t* norm_qk,
                                const float* rope_cos, const float* rope_sin, float eps,
                                uint8_t* q8, float* q_scale, uint8_t* k8, float* k_scale,
                                uint8_t* vt8, float* v_scale, void* workspace,
                                uint64_t workspace_bytes, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  Params p{};
  set_segments(p, 1, &M);
  p.A = q;
  p.sa = scale;
  p.seg.B[0] = qw;
  p.seg.sw[0] = w_scale;
  p.seg.bias[0] = bias;
  p.qkv.norm_qk = norm_qk;
  p.qkv.rope_cos = rope_cos;
  p.qkv.rope_sin = rope_sin;
  p.qkv.out_q = reinterpret_cast<uint16_t*>(q8);
  p.qkv.out_k = reinterpret_cast<uint16_t*>(k8);
  p.qkv.out_v = reinterpret_cast<uint16_t*>(vt8);
  p.qkv.scale_q = q_scale;
  p.qkv.scale_k = k_scale;
  p.qkv.scale_v = v_scale;
  p.qkv.eps = eps;
  p.qkv.heads = (int)heads;
  return schedule_and_launch(p, M, K, 3 * heads * 128, EPI_QKV_Q8, workspace, workspace_bytes,
                             stream);
}

}  // namespace dq
