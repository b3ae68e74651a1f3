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
// attn_fp8: a tile is 384 queries of one head; a workgroup (12 waves, one per compute unit)
// works on one tile at a time, wave w owning 32 of its queries with their codes in registers
// (the work split across workgroups is described at the kernel). Keys come in blocks of 64,
// double-buffered in LDS:
//   * K codes by global -> LDS copies (16 bytes per lane), 16-byte chunk c of key row r stored
//     at slot c ^ ((r >> 1) & 7) so that 16 rows read at one offset hit 16 different slots;
//   * V codes through registers, decoded once per workgroup to bf16 (exact: every E4M3 value is
//     a bf16 value), stored [channel][key] with the same swizzle, the keys of each 16-key group
//     in the order the logits leave them (0-3, 8-11, 4-7, 12-15);
//   * the blocks' key and value scales.
// Per block and wave:
//   1. logits: 2 x 2 FP8 matrix ops (32 keys x 32 queries x 64 channels each, keys as the
//      first operand), so lane l holds query l & 31 and keys 8 g + 4 (l >> 5) + j;
//   2. online softmax in base 2: t = s sk_j (sq_i log2(e) / sqrt(128)); the row max takes the
//      lane and its partner l ^ 32; the running max m (and with it the output and the sum,
//      rescaled by 2^(m - m')) moves only when a block's max exceeds it by more than 8, so the
//      rescale is rare after the first blocks; p = 2^(t - m) <= 2^8; keys past S are masked.
//      The weights are first formed against m as it stands: when every lane's sum of them stays
//      within 2^8 the max would not have moved and is not taken (the common case); otherwise
//      the logits are formed again and the block goes the way just described;
//   3. P V: p sv_j rounded to bf16 becomes the second operand of 16 bf16 matrix ops (32
//      channels x 32 queries x 16 keys) as the lanes hold it (the logits' layout holds keys 0-3
//      and 8-11 of a 16-key group in the lower lane of a query, 4-7 and 12-15 in the upper one,
//      and the values are stored in that order);
// so the output accumulates transposed, [channel][query], 64 registers per lane, and each lane
// keeps the sum of its own keys' weights (the lane pair's two sums are added at the end). One
// workgroup barrier per block. At the end o / sum goes to bf16 and leaves as 16-byte stores.
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
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

constexpr int kD = kHeadDim;   // 128 channels per head
constexpr int kWaves = 12;     // wavefronts per workgroup, three per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kQB = 32 * kWaves;  // queries per workgroup (32 per wave)
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
  uint8_t* ws;         // split schedule: arrival counters, then partial results (else unused)
  uint32_t ws_bytes;
  int H, S;
  int qtiles;          // ceil(S / 128): query tiles per head
  int nblk;            // ceil(S / 64): key blocks per tile
  int split;           // 1: workgroups take runs of key blocks, cutting tiles; 0: whole tiles
  float c;             // log2(e) / sqrt(128)
};

// Split schedule. The workspace opens with one arrival counter per workgroup boundary, then two
// partial results per boundary for the tile cut there (side 0: its first key blocks, side 1: its
// last ones). A partial holds, per wave and lane, the 64 unnormalized output sums as 16-byte
// groups (lane minor), then (m, sum) of the lane (the sum of its own keys' weights).
constexpr int kMaxGroups = 256;
constexpr uint32_t kFlagBytes = 4096;  // kMaxGroups counters, padded
constexpr uint32_t kPartBytes = kThreads * (64 + 2) * 4;
constexpr int kCoherent = 16;  // sc1: loads and stores coherent across XCDs

__device__ __forceinline__ uint32_t part_offset(int boundary, int side) {
  return kFlagBytes + (uint32_t)(2 * boundary + side) * kPartBytes;
}

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){a, b}, bf2v));
}

// Lane n of each row of 16 lanes, to every lane of that row (DPP row_newbcast; folded into the
// multiply that uses it).
template <int N>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               0x150 + N, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_bcast(float v, int n) {  // n a constant after unrolling
  switch (n) {
    case 0: return row_bcast<0>(v);
    case 1: return row_bcast<1>(v);
    case 2: return row_bcast<2>(v);
    case 3: return row_bcast<3>(v);
    case 4: return row_bcast<4>(v);
    case 5: return row_bcast<5>(v);
    case 6: return row_bcast<6>(v);
    case 7: return row_bcast<7>(v);
    case 8: return row_bcast<8>(v);
    case 9: return row_bcast<9>(v);
    case 10: return row_bcast<10>(v);
    case 11: return row_bcast<11>(v);
    case 12: return row_bcast<12>(v);
    case 13: return row_bcast<13>(v);
    case 14: return row_bcast<14>(v);
    default: return row_bcast<15>(v);
  }
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

// One key block of one head: the row index h S + key0 of its first key, and key0 (the
// addresses follow from these, so a block takes three scalar registers, not nine).
struct Blk {
  size_t tok;
  int key0;
};

__device__ __forceinline__ Blk block_at(const AttnArgs& a, int h, int kb) {
  return Blk{(size_t)h * (size_t)a.S + (size_t)kb * kKB, kb * kKB};
}
__device__ __forceinline__ Blk next_block(Blk b) { return Blk{b.tok + kKB, b.key0 + kKB}; }

// A block of key or value codes is 8 KiB: the first kMoveThreads threads move it, 16 bytes each.
constexpr int kMoveThreads = kKB * kD / 16;

// A key block (64 rows of 128 bytes) into an LDS stage, one 16-byte copy per thread of waves
// 0-7: wave w fills slots [64 w, 64 w + 64); slot n is row n >> 3, position n & 7, which holds
// chunk (n & 7) ^ key(row). Rows past S read row S - 1 (their logits are masked).
__device__ __forceinline__ void copy_keys(const AttnArgs& a, const Blk& b, uint8_t* stage, int w,
                                          int l) {
  if (w >= kMoveThreads / 64) return;
  const int S = a.S;
  const int n = w * 64 + l;
  const int r = n >> 3, p = n & 7;
  const int row = b.key0 + r < S ? r : S - 1 - b.key0;
  const uint8_t* src = a.k8 + b.tok * kD + row * kD + swz(r, p) * 16;
  __builtin_amdgcn_global_load_lds(
      src, (__attribute__((address_space(3))) void*)(stage + w * 64 * 16), 16, 0, 0);
}

// Value codes of a block: thread tid takes channel tid >> 2, keys 16 (tid & 3) + [0, 16); vrow
// is that row offset, (tid >> 2) S + 16 (tid & 3). S is a multiple of 16, so the 16 keys are
// either inside the sequence or past it (zeros).
// Threads past kMoveThreads load nothing.
// Buffer loads with a 32-bit lane offset off a block-uniform base: a 64-bit address per lane
// would be formed once outside the loop and spilled.
__device__ __forceinline__ uint4 load_values(const AttnArgs& a, const Blk& b, int tid, uint32_t vrow) {
  const uint8_t* v = a.vt8 + (b.tok - (size_t)b.key0) * kD + b.key0;  // channel 0, first key
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(v), 0, 0x7FFFFFFF, 0x00020000);
  if (tid < kMoveThreads && b.key0 + 16 * (tid & 3) < a.S)
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, vrow, 0, 0));
  return make_uint4(0u, 0u, 0u, 0u);
}

// The block's key scale (threads 0-63) or value scale (threads 64-127) of key tid & 63, 0 past S.
__device__ __forceinline__ float load_scale(const AttnArgs& a, const Blk& b, int tid) {
  const int j = tid & (kKB - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave 0: key scales, 1: values
  const float* base = (w == 0 ? a.sk : a.sv) + b.tok;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, 0x7FFFFFFF, 0x00020000);
  if (tid < 2 * kKB && b.key0 + j < a.S)
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, 4u * j, 0, 0));
  return 0.0f;
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

// The decoded values into an LDS stage, [channel][key] bf16, 128-byte rows, swizzled. Within
// each 16-key group the keys are stored in the order the logits leave them in a lane pair: keys
// 0-3 and 8-11 (held by the lower lane of a query) in the first 16 bytes, 4-7 and 12-15 in the
// second, so the weights enter the P V matrix op without an exchange between lanes.
__device__ __forceinline__ void store_values(uint8_t* stage, int tid, const uint4 vr) {
  if (tid >= kMoveThreads) return;
  const int ch = tid >> 2, q = tid & 3;
  const uint32_t d[4] = {vr.x, vr.y, vr.z, vr.w};  // keys 16 q + 4 i + [0, 4) in d[i]
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int chunk = 2 * q + j;  // 8 keys = 16 bytes
    *reinterpret_cast<uint4*>(stage + ch * 128 + swz(ch, chunk) * 16) = decode8(d[j], d[j + 2]);
  }
}

// One workgroup of 12 waves per compute unit (three per SIMD; the bound keeps the registers
// within what three waves may hold). Several smaller workgroups on a unit ran unevenly: the waves
// of the one dispatched first win the issue arbitration and finish early, and the others then
// run at lower throughput.
//
// Schedule: the (tile, key block) units, tile-major (tile = head * qtiles + query tile), are cut
// into gridDim.x contiguous runs, one per workgroup: runs of whole tiles, or with a workspace
// (split = 1) runs of equal length that may start or end inside a tile. A run is then a piece A
// (the last blocks of a tile begun by the previous run), a piece B (the first blocks of a tile
// that the next run finishes) and whole tiles; it takes A, then B, then the whole tiles, so both
// cut tiles are settled early. Every run holds at least one whole tile's length of units, so a
// tile is cut at most once. A cut piece stores its unnormalized result and counts its arrival
// (unless it sees the other part in already); the second to arrive adds the other's result to its
// own in a fixed order (side 0 first), so the output does not depend on which arrives first, and
// zeroes the counter for the next call.
__global__ void __launch_bounds__(kThreads, 1) attn_fp8(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t sK[2][kKB * kD];      // 2 x 8 KiB codes
  __shared__ __attribute__((aligned(1024))) uint8_t sV[2][kD * kKB * 2];  // 2 x 16 KiB bf16
  __shared__ __attribute__((aligned(16))) float sSC[2][2][kKB];  // [stage][key, value][key]
  __shared__ int s_last;
  const int tid = threadIdx.x, l = tid & 63, hi = l >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = a.S, nb = a.nblk;

  // This workgroup's run. Consecutive workgroup ids go round-robin over the 8 XCDs; renumbering
  // gives each XCD a contiguous stretch of runs, so its L2 serves the keys of few heads.
  const int G = gridDim.x;
  const int g = (G & 7) == 0 ? (int)(blockIdx.x & 7u) * (G >> 3) + (int)(blockIdx.x >> 3)
                             : (int)blockIdx.x;
  const int64_t T = (int64_t)a.H * a.qtiles;
  int64_t u0, u1;
  if (a.split) {
    u0 = T * nb * g / G;
    u1 = T * nb * (g + 1) / G;
  } else {
    u0 = T * g / G * nb;
    u1 = T * (g + 1) / G * nb;
  }
  const int tA = (int)(u0 / nb), kA = (int)(u0 % nb);  // piece A: blocks [kA, nb) of tile tA
  const int tB = (int)(u1 / nb), kB = (int)(u1 % nb);  // piece B: blocks [0, kB) of tile tB
  const int tF = kA > 0 ? tA + 1 : tA;                 // whole tiles [tF, tB)
  const int npieces = 2 + (tB - tF);
  // piece p (0: A, 1: B, 2 + i: whole tile tF + i) -> tile and block range; false if empty
  auto piece = [&](int p, int& t, int& k0, int& k1) -> bool {
    if (p == 0) {
      t = tA, k0 = kA, k1 = nb;
      return kA > 0;
    }
    if (p == 1) {
      t = tB, k0 = 0, k1 = kB;
      return kB > 0;
    }
    t = tF + p - 2, k0 = 0, k1 = nb;
    return true;
  };
  auto next_piece = [&](int p, int& t, int& k0, int& k1) -> int {
    for (++p; p < npieces; ++p)
      if (piece(p, t, k0, k1)) break;
    return p;
  };

  // per-wave state of the current tile
  v8i qf[2];
  float sqc = 0.0f, m = 0.0f, lsum = 0.0f;
  int qi = 0;
  bool qlive = false;
  v16f o[4];
  auto start_tile = [&](int t) {
    const int h = t / a.qtiles, q0 = (t - h * a.qtiles) * kQB;
    qi = q0 + 32 * w + (l & 31);
    qlive = qi < S;
    // this lane's query: channels [64 dh + 32 hi, +32) for the two 64-channel halves
    const uint8_t* qrow = a.q8 + ((size_t)h * (size_t)S + (size_t)(qlive ? qi : 0)) * kD;
#pragma unroll
    for (int dh = 0; dh < 2; ++dh)
      qf[dh] = qlive ? *reinterpret_cast<const v8i*>(qrow + 64 * dh + 32 * hi) : (v8i){};
    sqc = qlive ? a.sq[(size_t)h * (size_t)S + qi] * a.c : 0.0f;
    m = -__builtin_inff();
    lsum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (v16f){};
  };

  // One key block of head h in stage st; the block (hn, kbn) goes into the other stage when
  // `more`. kTail marks the last block when S is not a multiple of 64 (the only one whose keys
  // past S must take no weight), a separate instance so that full blocks carry no masking.
  // (32 bits: S < 2^24, so 127 S + 48 < 2^31. Formed again in each step from a copy of tid
  // that the compiler cannot see through: else it is kept, spilled and reloaded.)
  auto value_row = [&]() -> uint32_t {
    int t = tid;
    asm volatile("" : "+v"(t));
    return (uint32_t)((t >> 2) & (kD - 1)) * (uint32_t)S + 16u * (t & 3);
  };
  auto step = [&](const int kb, const int st, const bool more, const Blk& bn, auto tail_tag) {
    constexpr bool tail = decltype(tail_tag)::value;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's key copies of block kb
    __syncthreads();                     // every wave's copies and stores of block kb
    uint4 vr = make_uint4(0u, 0u, 0u, 0u);
    float scn = 0.0f;
    if (more) {
      vr = load_values(a, bn, tid, value_row());
      scn = load_scale(a, bn, tid);
    }
    // 1. logits, [key][query]. The next block's key copies into the other stage are issued only
    //    after this block's key fragments are read: the compiler cannot tell the two stages of
    //    sK apart and would otherwise wait for the copies before the first read.
    auto read_keys = [&](v8i (&kf)[2][2]) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const int r = 32 * kh + (l & 31);
#pragma unroll
        for (int dh = 0; dh < 2; ++dh) {
          const int c0 = 4 * dh + 2 * hi;
          const uint4 lo = *reinterpret_cast<const uint4*>(sK[st] + r * kD + swz(r, c0) * 16);
          const uint4 up =
              *reinterpret_cast<const uint4*>(sK[st] + r * kD + swz(r, c0 + 1) * 16);
          kf[kh][dh] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                             (int)up.x, (int)up.y, (int)up.z, (int)up.w};
        }
      }
    };
    auto logits = [&](const v8i (&kf)[2][2], v16f (&s)[2]) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        s[kh] = (v16f){};
#pragma unroll
        for (int dh = 0; dh < 2; ++dh)
          s[kh] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf[kh][dh], qf[dh], s[kh], 0,
                                                                  0, 0, 0, 0, 0);
      }
    };
    // 2. softmax in base 2: u = s sk, t = u sqc (sqc >= 0, so max t = sqc max u). The block's
    //    scales come in one 16-byte read per lane: lane 16 r + n holds the key (n < 8) or value
    //    (n >= 8) scales of keys 32 kh + 8 g + 4 (r >> 1) + [0, 4), with kh = (n >> 2) & 1 and
    //    g = n & 3, i.e. the four keys that lanes of half r >> 1 hold in register group (kh, g);
    //    a row broadcast from lane n of the row hands them to every lane.
    auto read_scales = [&](float (&sc)[4]) {
      const float4 sc4 = *reinterpret_cast<const float4*>(
          &sSC[st][(l >> 3) & 1][32 * ((l >> 2) & 1) + 8 * (l & 3) + 4 * hi]);
      sc[0] = sc4.x, sc[1] = sc4.y, sc[2] = sc4.z, sc[3] = sc4.w;
    };
    auto scale_keys = [&](v16f (&u)[2], const float (&sc)[4]) {  // u = s sk, in place
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
#pragma unroll
          for (int j = 0; j < 4; ++j) u[kh][4 * gq + j] *= row_bcast(sc[j], 4 * kh + gq);
    };
    // p = 2^(u sqc - mn) (0 for keys past S), times the value scale, into bf16 pairs [kh][gq][j
    // pair]; returns the sum of this lane's p (the partner lane l ^ 32 holds the query's other
    // keys; the two partial sums are added when the tile ends).
    auto weights = [&](const v16f (&u)[2], const float (&sc)[4], float mn,
                       uint32_t (&pk)[2][4][2]) -> float {
      float ps = 0.0f;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          float p[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            p[j] = __builtin_amdgcn_exp2f(fmaf(u[kh][4 * gq + j], sqc, -mn));
            if constexpr (tail)
              if (kb * kKB + 32 * kh + 8 * gq + 4 * hi + j >= S) p[j] = 0.0f;
            ps += p[j];
          }
          const int n = 8 + 4 * kh + gq;
          pk[kh][gq][0] = pack_bf16(p[0] * row_bcast(sc[0], n), p[1] * row_bcast(sc[1], n));
          pk[kh][gq][1] = pack_bf16(p[2] * row_bcast(sc[2], n), p[3] * row_bcast(sc[3], n));
        }
      return ps;
    };
    // The running max m moves only when a block's max exceeds it by more than 8 (weights stay
    // <= 2^8, harmless in fp32 and bf16); the output is rescaled only when some lane of the
    // wave moved, which is rare after the first blocks. The weights are first formed against m
    // as it stands: when every lane's sum stays within 2^8 (so does each weight) the max would
    // not have moved and is not needed. Otherwise (the first block of a tile, a new max) the
    // block max is taken and the weights are formed once more, by the same code.
    auto new_max = [&](const v16f (&u)[2]) -> float {
      float mxu = -__builtin_inff();
      asm volatile("" : "+v"(mxu));  // (keeps the max on the path that needs it)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          if constexpr (tail) {
            const int key = kb * kKB + 32 * kh + 8 * (v >> 2) + 4 * hi + (v & 3);
            if (key < S) mxu = fmaxf(mxu, u[kh][v]);
          } else {
            mxu = fmaxf(mxu, u[kh][v]);
          }
        }
      float a0 = mxu, b0 = mxu;
      swap_halves(a0, b0);
      const float mx = fmaxf(a0, b0) * sqc;
      return mx > m + 8.0f ? mx : m;
    };
    // One pass of the block's logits and weights; a second pass (rare: see above) forms the
    // logits again from the keys still in this stage, takes the max and then the weights.
    uint32_t pk[2][4][2];
    float mn = m, ps;
    bool again = false;
#pragma nounroll
    for (;;) {
      v16f s[2];
      // The key fragments and the scales are read before the next block's key copies are
      // issued: the compiler does not tell the LDS arrays apart from the copies' target and
      // would make any later LDS read wait for every outstanding load (those copies, and the
      // next block's values and scales, issued at the top of the step).
      float sc[4];
      {
        v8i kf[2][2];
        read_keys(kf);
        read_scales(sc);
        if (more && !again) copy_keys(a, bn, sK[st ^ 1], w, l);
        logits(kf, s);
      }
      scale_keys(s, sc);
      if (again) mn = new_max(s);
      ps = weights(s, sc, mn, pk);
      // (the packed weights are pinned here: else the compiler moves their products out of the
      // loop, away from the scales' row broadcasts that they would fold in, and keeps the 32
      // fp32 weights alive instead of 16 packed pairs)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) asm volatile("" : "+v"(pk[kh][gq][0]), "+v"(pk[kh][gq][1]));
      if (again || __builtin_amdgcn_ballot_w64(!(ps <= 256.0f)) == 0) break;
      again = true;
      asm volatile("" ::: "memory");  // (the second pass reads the keys and scales again)
    }
    if (again) {
      // rescale by 2^(m - m') (2^0 = 1 where the max holds)
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      lsum = lsum * alpha + ps;
      if (__builtin_amdgcn_ballot_w64(mn != m) != 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] *= alpha;
      }
      m = mn;
    } else {
      lsum += ps;
    }
    // 3. P V: the weights of keys [16 kc, +16) as the lanes hold them (the values are stored in
    //    that key order)
    bf8v pb[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int kh = kc >> 1, c2 = kc & 1;
      pb[kc] = __builtin_bit_cast(bf8v, make_uint4(pk[kh][2 * c2][0], pk[kh][2 * c2][1],
                                                   pk[kh][2 * c2 + 1][0], pk[kh][2 * c2 + 1][1]));
    }
    // The value fragments of one 16-key group (four reads) are in flight while the matrix ops
    // of the previous group run: left to itself the compiler reads one fragment at a time,
    // each matrix op waiting for its read.
    auto read_values = [&](int kc, bf8v (&vf)[4]) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int r = 32 * db + (l & 31);
        vf[db] = *reinterpret_cast<const bf8v*>(sV[st] + r * 128 + swz(r, 2 * kc + hi) * 16);
      }
    };
    bf8v vf[2][4];
    read_values(0, vf[0]);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      if (kc < 3) read_values(kc + 1, vf[(kc + 1) & 1]);
      if (kc == 0)  // DS reads: this group's and the next one's, then the next one's only
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      else if (kc < 3)
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int db = 0; db < 4; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[kc & 1][db], pb[kc], o[db], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // matrix ops
    }
    if (more) {
      store_values(sV[st ^ 1], tid, vr);
      if (tid < 2 * kKB) sSC[st ^ 1][tid >> 6][tid & (kKB - 1)] = scn;
    }
  };

  // A cut piece: store this workgroup's part, count it; the second part to arrive loads the
  // other, adds the two and returns true (it then writes the output). Side 0 (a run's piece B,
  // taken after its piece A) usually arrives second, so it first looks whether side 1 is in
  // already and then skips storing its own part.
  auto settle_cut = [&](int boundary, int side) -> bool {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(a.ws, 0, (int)a.ws_bytes, 0x00020000);
    const uint32_t lane_off = (uint32_t)(w * 64 + l) * 16u;
    uint32_t* flags = reinterpret_cast<uint32_t*>(a.ws);
    bool in = false;  // the other part is stored and counted
    if (side == 0) {
      if (tid == 0)
        s_last = __hip_atomic_load(flags + boundary, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT) == 1u;
      __syncthreads();
      in = s_last;
      __syncthreads();  // s_last is written again below
    }
    if (!in) {
      const uint32_t base = part_offset(boundary, side);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 x = make_float4(o[db][4 * q4], o[db][4 * q4 + 1], o[db][4 * q4 + 2],
                                       o[db][4 * q4 + 3]);
          __builtin_amdgcn_raw_buffer_store_b128(
              __builtin_bit_cast(v4u, x), rs,
              base + (uint32_t)(4 * db + q4) * (kThreads * 16u) + lane_off, 0, kCoherent);
        }
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, make_float2(m, lsum)), rs,
                                            base + kThreads * 256u + (uint32_t)(w * 64 + l) * 8u, 0,
                                            kCoherent);
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the part is stored
      __syncthreads();
      if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(flags + boundary, 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        s_last = old == 1u;
      }
      __syncthreads();
      if (!s_last) return false;
    }
    const uint32_t base = part_offset(boundary, side ^ 1);
    v4u x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      x[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, base + (uint32_t)i * (kThreads * 16u) + lane_off, 0,
                                                   kCoherent);
    const v2u ml = __builtin_amdgcn_raw_buffer_load_b64(
        rs, base + kThreads * 256u + (uint32_t)(w * 64 + l) * 8u, 0, kCoherent);
    const float m_o = __uint_as_float(ml[0]), l_o = __uint_as_float(ml[1]);
    // side 0 is always the first operand of the sum
    const float m0 = side == 0 ? m : m_o, m1 = side == 0 ? m_o : m;
    const float mn = fmaxf(m0, m1);
    const float a0 = __builtin_amdgcn_exp2f(m0 - mn), a1 = __builtin_amdgcn_exp2f(m1 - mn);
    const float l0 = side == 0 ? lsum : l_o, l1 = side == 0 ? l_o : lsum;
    lsum = fmaf(l0, a0, __fmul_rn(l1, a1));
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float other = __uint_as_float(x[4 * db + (e >> 2)][e & 3]);
        const float v0 = side == 0 ? o[db][e] : other, v1 = side == 0 ? other : o[db][e];
        o[db][e] = fmaf(v0, a0, __fmul_rn(v1, a1));
      }
    if (tid == 0)
      __hip_atomic_store(flags + boundary, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
  };

  // o / sum, [channel][query] -> out[query][h][channel]
  auto write_out = [&](int h) {
    float s0 = lsum, s1 = lsum;  // the query's sum: this lane's keys and its partner's
    swap_halves(s0, s1);
    const float inv = 1.0f / (s0 + s1);
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
          *reinterpret_cast<uint4*>(a.out + ((size_t)qi * (size_t)a.H + h) * kD + 32 * db +
                                    16 * gp + 8 * hi) = ov;
      }
  };

  int t, k0, k1;
  int p = piece(0, t, k0, k1) ? 0 : next_piece(0, t, k0, k1);
  if (p >= npieces) return;  // an empty run (the host never launches one)
  // the run's first block into stage 0
  Blk bc = block_at(a, t / a.qtiles, k0);
  {
    copy_keys(a, bc, sK[0], w, l);
    store_values(sV[0], tid, load_values(a, bc, tid, value_row()));
    const float sc = load_scale(a, bc, tid);
    if (tid < 2 * kKB) sSC[0][tid >> 6][tid & (kKB - 1)] = sc;
  }
  int st = 0;
  const int nfull = S / kKB;  // blocks without keys past S; block nfull (if any) is the last
  for (;;) {
    start_tile(t);
    const int h = t / a.qtiles;
    int tn = t, k0n = 0, k1n = 0;
    const int pn = next_piece(p, tn, k0n, k1n);
    // the block after kb: the next one of this piece, else the first of the next piece
    auto after = [&](int kb, bool& more) -> Blk {
      const bool last = kb + 1 == k1;
      more = !last || pn < npieces;
      return !last ? next_block(bc) : block_at(a, more ? tn / a.qtiles : 0, k0n);
    };
    // full blocks, then (kept out of the loop so that the two instances do not meet in one
    // loop body) the partial last block
    const int kfull = k1 < nfull ? k1 : nfull;
    for (int kb = k0; kb < kfull; ++kb) {
      bool more;
      const Blk bn = after(kb, more);
      step(kb, st, more, bn, std::false_type{});
      bc = bn;
      st ^= 1;
    }
    if (k1 > nfull) {
      bool more;
      const Blk bn = after(nfull, more);
      step(nfull, st, more, bn, std::true_type{});
      bc = bn;
      st ^= 1;
    }
    // p == 0 is piece A (side 1 of boundary g), p == 1 piece B (side 0 of boundary g + 1)
    if (p >= 2 || settle_cut(p == 0 ? g : g + 1, p == 0 ? 1 : 0)) write_out(h);
    if (pn >= npieces) break;
    p = pn, t = tn, k0 = k0n, k1 = k1n;
  }
}

// Compute units of the current device, queried once per device.
int device_compute_units() {
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

hipError_t launch_quantize_v(const uint16_t* v, int64_t H, int64_t S, uint8_t* vt, float* sv,
                             hipStream_t stream) {
  if (H == 0 || S == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_v_t, dim3((unsigned)((S + 63) / 64), (unsigned)H), dim3(256), 0, stream,
                     v, (int)S, vt, sv);
  return hipGetLastError();
}

hipError_t launch_attention(const uint8_t* q8, const float* sq, const uint8_t* k8, const float* sk,
                            const uint8_t* vt8, const float* sv, int64_t H, int64_t S,
                            uint16_t* out, void* workspace, int64_t max_workgroups,
                            hipStream_t stream) {
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
  a.qtiles = (int)((S + kQB - 1) / kQB);
  a.nblk = (int)((S + kKB - 1) / kKB);
  a.c = 1.4426950408889634f / 11.313708498984761f;  // log2(e) / sqrt(128)
  const int64_t tiles = H * a.qtiles;
  int64_t cap = device_compute_units();  // one workgroup per compute unit
  if (max_workgroups > 0 && max_workgroups < cap) cap = max_workgroups;
  if (workspace && cap > kMaxGroups) cap = kMaxGroups;
  const int64_t grid = tiles < cap ? tiles : cap;
  a.split = workspace != nullptr && tiles > grid;
  a.ws = static_cast<uint8_t*>(workspace);
  a.ws_bytes = a.split ? (uint32_t)attention_workspace_bytes(H, S) : 0u;
  hipLaunchKernelGGL(attn_fp8, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

uint64_t attention_workspace_bytes(int64_t H, int64_t S) {
  const int64_t tiles = H * ((S + kQB - 1) / kQB);
  const int64_t groups = tiles < kMaxGroups ? tiles : kMaxGroups;
  return kFlagBytes + 2 * (uint64_t)groups * kPartBytes;
}

}  // namespace dq
