// Absorbed MLA attention over the latent cache (gfx950).
//
// Scores come straight from the cached latents: for query row (token, head)
// the score of cache row i is q[h] . row_i over the full 576-wide row
// (latent part against q_lat = c_Q W_UQK[h], RoPE part against q_pe[h]);
// the output is the latent-space head output o_lat[h] = softmax . C[:, :d_L]
// (pages "Multi-Head Latent Attention (MLA)", section "Two merges are where
// the compute win comes from"; "How DeepSeek Rewrote the Transformer",
// "The short version").
//
// Work decomposition: every (sequence, query token) pair is a "virtual
// sequence" whose visible rows are 0 .. kv_len - n_q + j.  Its rows are cut
// into 32-token tiles; the concatenated tile list is split evenly over G
// work-groups (one per CU).  A work-group walks its tile range, and for
// each virtual sequence it touches runs an online softmax over the tiles it
// owns.  Whole sequences are normalised and written to o_lat directly; a
// sequence cut by a work-group boundary leaves one (O, LSE) partial per
// piece, combined afterwards with a log-sum-exp merge.
//
// Inside a work-group (4 waves, all 128 heads of the sequence):
//   * 32-token tiles are DMA'd global -> LDS (global_load_lds, 16 B/lane)
//     through a 3-stage ring.  A tile is stored as 9 column blocks of 64
//     latent/rope values (128 B per row) with a 16-byte-chunk XOR swizzle;
//     wave w DMAs rows 8w..8w+7 of every block, so its per-lane source
//     offset is one register plus immediates.  Rows past the visible length
//     are DMA'd from a zero buffer, never from the cache.
//   * Score phase: wave w owns heads 32w..32w+31; S^T[32 tokens x 32 heads]
//     = tile . q^T on 32x32x16 bf16 MFMA, q held in registers for the whole
//     segment; online-softmax statistics per head (lanes l and l^32 share a
//     head); P goes to LDS in bf16.
//   * PV phase: wave w owns latent columns [128w, 128w+128) for all 128
//     heads: O[128 x 128] (AGPRs) += P[128 x 32] . tile[32 x 128-col slice];
//     each tile column is read from LDS by exactly one wave.
#include <math.h>

#include <climits>
#include <type_traits>

#include "mla_common.h"
#include "mla_internal.h"

namespace mla {

static __device__ __attribute__((aligned(16))) unsigned char g_zero_rows[64 * 16];

#define MLA_CONST_PTR(p) ((const __attribute__((address_space(4))) int32_t*)(p))

typedef float f32x16 __attribute__((ext_vector_type(16)));

// 32x32 MFMA of the attention kernel.  Lane l holds A[l%32][(l/32)*KPL + j],
// B[(l/32)*KPL + j][l%32] and D[8*(r/4) + 4*(l/32) + r%4][l%32], r < 16.
//
// bf16: the 128 x 128 fp32 O block of a wave fills all 256 AGPRs, so the
// MFMAs are issued through inline asm with explicit register classes: the
// score chain accumulates in VGPRs (its result feeds VALU code), the O
// tiles in AGPRs.  The asm is volatile, so LDS loads stay where the source
// puts them (the loops below prefetch operands a fixed distance ahead).
// The compiler's hazard tracking does not see into asm, so each asm carries
// the wait states its consumers need:
//   * a VALU-written B operand needs 2 wait states before an MFMA reads it;
//   * an MFMA result needs >= 18 wait states before VALU or copies read it
//     (24 are issued: s_nop 15 + s_nop 7);
//   * back-to-back MFMAs accumulating into the same registers need none.
template <typename T>
struct Mfma32;
template <>
struct Mfma32<__bf16> {
  static constexpr int KB = 16, KPL = 8;
  using frag = bf16x8;
  // s = a.b (fresh accumulator in VGPRs)
  __device__ static inline f32x16 first(frag a, frag b) {
    f32x16 d;
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
    return d;
  }
  // s += a.b, VGPR accumulator
  __device__ static inline void acc_v(f32x16& s, frag a, frag b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(a), "v"(b));
  }
  // s += a.b, last of a chain: the result is readable by VALU afterwards
  __device__ static inline void acc_v_last(f32x16& s, frag a, frag b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 15\n\ts_nop 7" : "+v"(s) : "v"(a), "v"(b));
  }
  // o += a.b, AGPR accumulator; b was just assembled by VALU code
  __device__ static inline void acc_a_fresh_b(f32x16& o, frag a, frag b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(a), "v"(b));
  }
  __device__ static inline void acc_a(f32x16& o, frag a, frag b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(a), "v"(b));
  }
  __device__ static inline frag zero() { return Mfma<__bf16>::zero(); }
};
template <>
struct Mfma32<float> {
  static constexpr int KB = 2, KPL = 1;
  using frag = float;
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline f32x16 first(frag a, frag b) { return mma(a, b, f32x16{}); }
  __device__ static inline void acc_v(f32x16& s, frag a, frag b) { s = mma(a, b, s); }
  __device__ static inline void acc_v_last(f32x16& s, frag a, frag b) { s = mma(a, b, s); }
  __device__ static inline void acc_a_fresh_b(f32x16& o, frag a, frag b) { o = mma(a, b, o); }
  __device__ static inline void acc_a(f32x16& o, frag a, frag b) { o = mma(a, b, o); }
  __device__ static inline frag zero() { return 0.0f; }
};

// o[r] *= al[r] for an AGPR-resident accumulator tile, one element at a
// time through a scratch VGPR (keeps the tile in place).
__device__ inline void o_scale_tile(f32x16& o, const float (&al)[16]) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float e = o[r], t;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(e), "=&v"(t)
                 : "v"(al[r]));
    o[r] = e;
  }
}

// Wait states between the last asm MFMA into the O block and any other
// access to it (rescale, final read); a no-op for compiler-issued MFMAs.
template <typename T, int NTH, int NCT>
__device__ inline void o_settle(f32x16 (&O)[NTH][NCT]) {
  if constexpr (sizeof(T) == 2 && NTH == 4 && NCT == 4) {
    asm volatile("s_nop 15\n\ts_nop 7"
                 : "+a"(O[0][0]), "+a"(O[0][1]), "+a"(O[0][2]), "+a"(O[0][3]), "+a"(O[1][0]), "+a"(O[1][1]),
                   "+a"(O[1][2]), "+a"(O[1][3]), "+a"(O[2][0]), "+a"(O[2][1]), "+a"(O[2][2]), "+a"(O[2][3]),
                   "+a"(O[3][0]), "+a"(O[3][1]), "+a"(O[3][2]), "+a"(O[3][3]));
  }
}

template <typename T_, int HP_, int NW_, int DL_, int DR_, int NSTAGE_, bool CNT_ = false, bool E4_ = false>
struct AttnCfg {
  // cache rows read by one stream only: non-temporal tile loads
  static constexpr bool CNT = CNT_;
  // cache rows are E4M3 codes with per-row scales: tiles are DMA'd into a
  // two-slot staging ring and converted into the bf16 tile slots
  static constexpr bool E4 = E4_;
  using T = T_;
  using F = Mfma32<T>;
  static constexpr int HP = HP_, NW = NW_, DL = DL_, DR = DR_, R = DL_ + DR_;
  static constexpr int ES = (int)sizeof(T);
  static constexpr int TILE = 32;
  static constexpr int NSTAGE = NSTAGE_;
  static constexpr int NTHR = NW * 64;
  static constexpr int NTH = HP / 32;        // 32-head tiles
  static constexpr int KB = F::KB, KPL = F::KPL;
  static constexpr int RK = R / KB;          // score k-steps over one row
  static constexpr int PV_KS = TILE / KB;    // PV k-steps over one tile
  static constexpr int CPW = DL / NW;        // latent columns per wave (PV phase)
  static constexpr int NCT = CPW / 32;       // 32-column tiles per wave
  static constexpr int ROW_BYTES = R * ES;
  static constexpr int ROW_CHUNKS = ROW_BYTES / 16;
  // column-block layout with swizzle (bf16, 64-value blocks, 128-col slices)
  static constexpr bool FAST = (ES == 2) && (ROW_CHUNKS % 8 == 0) && (CPW % 64 == 0) && (NW == 4);
  static constexpr int BLOCK_BYTES = TILE * 128;
  static constexpr int TILE_BYTES = TILE * ROW_BYTES;
  static constexpr int NINST = TILE_BYTES / 1024;
  static constexpr int PSTR = TILE + 16 / ES;
  // FAST: the last QL 64-wide column blocks of q sit in LDS ([block][head]
  // rows of 128 B, swizzled like the tiles); the rest stays in registers
  static constexpr int QL = FAST ? 2 : 0;
  static constexpr int RKQ = RK - QL * 4;  // q fragments held in registers
  static constexpr int OFF_Q = NSTAGE * TILE_BYTES;
  static constexpr int Q_BLOCK_BYTES = HP * 128;
  static constexpr int OFF_P = OFF_Q + QL * Q_BLOCK_BYTES;
  static constexpr int OFF_ALPHA = OFF_P + HP * PSTR * ES;
  static constexpr int OFF_M = OFF_ALPHA + HP * 4;
  static constexpr int OFF_L = OFF_M + HP * 4;
  static constexpr int OFF_FLAG = OFF_L + HP * 4;
  // E4M3 staging slot: TILE rows of R codes, then 256 B of scales (one per
  // lane of the scale load, rows past the tile read as 0) and 256 B that
  // the padding load of a wave without a block of its own writes
  static constexpr int E4_TILE = TILE * R;
  static constexpr int E4_BLOCKS = E4_TILE / 1024;
  static constexpr int E4_STAGE = E4_TILE + 512;
  static constexpr int E4_LOADS = (E4_BLOCKS + 2 + NW - 1) / NW;  // DMA instructions per tile and wave
  static constexpr int OFF_E4 = (OFF_FLAG + NTH * 4 + 15) & ~15;
  static constexpr int LDS_BYTES = E4 ? OFF_E4 + 2 * E4_STAGE : OFF_FLAG + NTH * 4;
  static_assert(NTH == NW, "one 32-head tile per wave in the score phase");
  static_assert(R % KB == 0 && TILE % KB == 0, "whole MFMA k-steps");
  static_assert(TILE_BYTES % 1024 == 0 && NINST % NW == 0, "tile must be whole 1 KB DMA blocks per wave");
  static_assert(DL % (NW * 32) == 0, "latent columns must split evenly over waves");
  static_assert(ROW_BYTES % 16 == 0, "rows must be whole 16 B chunks");
  static_assert(!FAST || NINST == 4 * (ROW_CHUNKS / 8), "FAST: 4 DMA blocks per column block");
  static_assert(!E4 || (FAST && NSTAGE == 2 && E4_TILE % 1024 == 0 && E4_LOADS * NW == E4_BLOCKS + 2),
                "E4M3: bf16 FAST layout, two bf16 slots, whole 1 KB code blocks plus the scale and padding loads");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// 128 heads per work-group: 4 waves x 32 heads (score phase), 4 waves x 128
// latent columns (PV phase); the fp32 O accumulators (128 x 512) fill the
// AGPRs of the four waves.
using CfgBf16 = AttnCfg<__bf16, 128, 4, 512, 64, 3>;
using CfgBf16Nt = AttnCfg<__bf16, 128, 4, 512, 64, 3, true>;
using CfgE4 = AttnCfg<__bf16, 128, 4, 512, 64, 2, false, true>;
using CfgE4Nt = AttnCfg<__bf16, 128, 4, 512, 64, 2, true, true>;
using CfgF32 = AttnCfg<float, 32, 1, 32, 8, 3>;

// Softmax statistics are only rebased when a head's running max grows by
// more than this (log2 units); P stays <= 2^8, exact in bf16 and fp32.
constexpr float kRescaleSlack = 8.0f;

// 16-byte-chunk swizzle inside a 128-byte block row: logical chunk c of
// tile row r sits at chunk c ^ swz(r).  Measured on gfx950 (8 waves per CU,
// ds_read_b128 of a 16x16x32 or 32x32x16 fragment: 16 consecutive rows, one
// logical chunk per 16 lanes): swz(r) = r & 7 reads at 252 B/clk per CU, the
// LDS peak, while a swizzle that spreads the 16 rows over the two bank
// halves by row parity ((r >> 1) & 1 in bit 2) conflicts two ways (135
// B/clk).  The transposing PV reads run at ~87 B/clk under either.
__device__ inline int swz(int r) { return r & 7; }

// Byte offset of logical chunk c of row r in a 128-byte-row block.
__device__ inline int tile_chunk(int r, int c) { return r * 128 + 16 * (c ^ swz(r)); }

// Byte offset of element e of tile row r in an LDS stage.
template <class C>
__device__ inline int lds_off(int r, int e) {
  const int byte = e * C::ES;
  if constexpr (C::FAST) {
    const int c = byte >> 4;
    return (c >> 3) * C::BLOCK_BYTES + r * 128 + (((c & 7) ^ swz(r)) << 4) + (byte & 15);
  } else {
    return r * C::ROW_BYTES + byte;
  }
}

__device__ inline float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Raw buffer resource over [base, base + bytes): loads past the end return
// zeros.  Word 3 selects 32-bit data format (raw untyped access).
// The arguments must be wave-uniform; they are pinned to scalar registers.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p), hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void* b = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(b, (short)0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// Buffer-load DMA of this lane's 16 bytes of column blocks KK .. N-1 of a
// tile (block kk lands 4 KB further in LDS and starts 128 bytes further in
// the row).  The 128-byte step goes in the scalar offset: the instruction's
// immediate offset would move the LDS destination as well, and a per-block
// vector offset costs a register per block.
template <int KK, int N, int CP>
__device__ inline void dma_column_blocks(__amdgpu_buffer_rsrc_t rsrc, unsigned char* stage, int wave, int dma_off) {
  if constexpr (KK < N) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, MLA_LDS_PTR(stage + (wave + 4 * KK) * 1024), 16, dma_off,
                                             KK * 128, 0, CP);
    dma_column_blocks<KK + 1, N, CP>(rsrc, stage, wave, dma_off);
  }
}

// DMA one 32-row tile into an LDS stage with buffer loads whose record
// count is the tile's visible bytes: rows at or past `vis`, a page id
// outside the pool (which also raises error bit 2), and a tile past the end
// of the segment (`live` false) all read as zeros.  Every call issues the same NINST / NW loads per wave,
// so the pipeline can wait on a constant count.
// Buffer record of tile k (page lookup, visible bytes), as issue_tile uses.
template <class C>
__device__ inline __amdgpu_buffer_rsrc_t tile_rsrc(const AttnArgs& a, int b, int k, int vis, int lane, bool live) {
  const int t0 = k * C::TILE;
  const unsigned char* gbase = reinterpret_cast<const unsigned char*>(a.pool);
  bool ok = live;
  if (live) {
    if (a.paged) {
      const int pg = MLA_CONST_PTR(a.page_table)[(size_t)b * a.max_pages + t0 / a.page_size];
      ok = (pg >= 0) && (pg < a.n_pages);
      if (!ok && lane == 0) atomicOr(a.err, 2);  // flagged, then read as zeros
      gbase += ((size_t)(ok ? pg : 0) * a.page_size + (t0 % a.page_size)) * (size_t)C::ROW_BYTES;
    } else {
      gbase += ((size_t)b * a.s_max + t0) * (size_t)C::ROW_BYTES;
    }
  }
  const int nbytes = ok ? min(max(vis - t0, 0), C::TILE) * C::ROW_BYTES : 0;
  return make_rsrc(gbase, nbytes);
}

// Column block KK of a FAST tile (see issue_tile), for loads issued one at a
// time between other work.
template <class C, int KK>
__device__ inline void dma_block(__amdgpu_buffer_rsrc_t rsrc, unsigned char* stage, int wave, int dma_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, MLA_LDS_PTR(stage + (wave + 4 * KK) * 1024), 16, dma_off, KK * 128,
                                           0, C::CNT ? 2 : 0);
}

template <class C>
__device__ inline void issue_tile(const AttnArgs& a, unsigned char* stage, int b, int k, int vis, int wave,
                                  int lane, int dma_off, bool live) {
  const int t0 = k * C::TILE;
  const unsigned char* gbase = reinterpret_cast<const unsigned char*>(a.pool);
  bool ok = live;
  if (live) {
    if (a.paged) {
      const int pg = MLA_CONST_PTR(a.page_table)[(size_t)b * a.max_pages + t0 / a.page_size];
      ok = (pg >= 0) && (pg < a.n_pages);
      if (!ok && lane == 0) atomicOr(a.err, 2);  // flagged, then read as zeros
      gbase += ((size_t)(ok ? pg : 0) * a.page_size + (t0 % a.page_size)) * (size_t)C::ROW_BYTES;
    } else {
      gbase += ((size_t)b * a.s_max + t0) * (size_t)C::ROW_BYTES;
    }
  }
  const int nbytes = ok ? min(max(vis - t0, 0), C::TILE) * C::ROW_BYTES : 0;
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(gbase, nbytes);
  if constexpr (C::FAST) {
    // wave w fills rows 8w + lane/8 of every column block; dma_off holds the
    // lane's row and swizzled chunk, block k adds 128 B in global memory.
    // When every cache row is read by one stream only (one query token, all
    // heads in one work-group: C::CNT) the loads are non-temporal (cache
    // policy 2); with several query tokens per sequence the tiles are
    // re-read by the other streams and stay cacheable.
    dma_column_blocks<0, C::NINST / C::NW, C::CNT ? 2 : 0>(rsrc, stage, wave, dma_off);
  } else {
    // row-major rows; 16-byte chunk p of the tile goes to LDS byte 16 p
#pragma unroll
    for (int kk = 0; kk < C::NINST / C::NW; ++kk) {
      const int in = wave + kk * C::NW;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, MLA_LDS_PTR(stage + in * 1024), 16, (in * 64 + lane) * 16, 0, 0,
                                               0);
    }
  }
}

// E4M3 cache: DMA one 32-row tile of codes (contiguous R-byte rows, one
// 1 KB block per load) and its 32 scales into a staging slot.  Wave w takes
// blocks w, w + NW, ...; the last two load slots are the scales and a
// padding load into the slot's spare 256 B, so that every wave issues
// E4_LOADS loads.  Rows at or past `vis`, a page outside the pool (error
// bit 2) and a dead tile read as zeros, as in issue_tile.
// Buffer records of an E4M3 tile's codes and scales (page lookup and
// visible rows), and load i of a wave (see issue_tile_e4).
struct E4Rsrc {
  __amdgpu_buffer_rsrc_t codes, scales;
};
template <class C>
__device__ inline E4Rsrc e4_rsrc(const AttnArgs& a, int b, int k, int vis, int lane, bool live) {
  const int t0 = k * C::TILE;
  size_t row0 = 0;
  bool ok = live;
  if (live) {
    if (a.paged) {
      const int pg = MLA_CONST_PTR(a.page_table)[(size_t)b * a.max_pages + t0 / a.page_size];
      ok = (pg >= 0) && (pg < a.n_pages);
      if (!ok && lane == 0) atomicOr(a.err, 2);
      row0 = (size_t)(ok ? pg : 0) * a.page_size + (t0 % a.page_size);
    } else {
      row0 = (size_t)b * a.s_max + t0;
    }
  }
  const int rows = ok ? min(max(vis - t0, 0), C::TILE) : 0;
  return E4Rsrc{make_rsrc(reinterpret_cast<const unsigned char*>(a.pool) + row0 * C::R, rows * C::R),
                make_rsrc(a.scales + row0, rows * 4)};
}
template <class C>
__device__ inline void e4_load(const E4Rsrc& r, unsigned char* st, int wave, int lane, int i) {
  constexpr int CP = C::CNT ? 2 : 0;
  const int j = wave + C::NW * i;  // wave-uniform
  if (j < C::E4_BLOCKS)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.codes, MLA_LDS_PTR(st + j * 1024), 16, lane * 16, j * 1024, 0, CP);
  else if (j == C::E4_BLOCKS)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r.scales, MLA_LDS_PTR(st + C::E4_TILE), 4, lane * 4, 0, 0, CP);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(g_zero_rows, 0), MLA_LDS_PTR(st + C::E4_TILE + 256), 4, 0, 0,
                                             0, 0);
}

template <class C>
__device__ inline void issue_tile_e4(const AttnArgs& a, unsigned char* st, int b, int k, int vis, int wave, int lane,
                                     bool live) {
  const E4Rsrc r = e4_rsrc<C>(a, b, k, vis, lane, live);
#pragma unroll
  for (int i = 0; i < C::E4_LOADS; ++i) e4_load<C>(r, st, wave, lane, i);
}

// Converts a staged E4M3 tile into a bf16 tile slot (FAST layout), 16 codes
// per thread and item; code * scale is exact in
// bf16 for the power-of-two scales the library writes.  The conversion is
// v_cvt_scalef32_pk_bf16_fp8 (two codes of the selected 16-bit half, times
// the fp32 scale, to two bf16), written in one asm block per chunk: the
// compiler's builtin for it keeps only the first result of each pair (it
// copies the low bf16 over the high one), while the instruction itself
// gives the format's value for all 256 codes (checked against
// torch.float8_e4m3fn on this hardware).  The block's inputs come from LDS
// loads (waited for by the compiler before the asm) and its trailing
// s_nop leaves wait states before any consumer of the results.
// Items k0 .. k0 + N - 1 of this thread: all loaded, then converted.
template <class C, int N>
__device__ inline void convert_items_e4(const unsigned char* __restrict__ st, unsigned char* __restrict__ tb, int tid,
                                        int k0) {
  constexpr int ITEMS_PER_BLOCK = C::TILE * 4;
  constexpr int ITEMS = C::E4_TILE / 16;
  const float* sc = reinterpret_cast<const float*>(st + C::E4_TILE);
  uint4 w[N];
  float s[N];
  int off[N];
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const int it = min(tid + (k0 + k) * C::NTHR, ITEMS - 1);  // the tail repeats the last item (same value, same place)
    const int blk = it / ITEMS_PER_BLOCK, rem = it - blk * ITEMS_PER_BLOCK;
    const int r = rem >> 2, e0 = blk * 64 + (rem & 3) * 16;
    w[k] = *reinterpret_cast<const uint4*>(st + r * C::R + e0);
    s[k] = sc[r];
    off[k] = lds_off<C>(r, e0);
  }
#pragma unroll
  for (int k = 0; k < N; ++k) {
    uint32_t o0, o1, o2, o3, o4, o5, o6, o7;
    asm volatile(
        "v_cvt_scalef32_pk_bf16_fp8 %0, %8, %12\n\t"
        "v_cvt_scalef32_pk_bf16_fp8 %1, %8, %12 op_sel:[1,0,0]\n\t"
        "v_cvt_scalef32_pk_bf16_fp8 %2, %9, %12\n\t"
        "v_cvt_scalef32_pk_bf16_fp8 %3, %9, %12 op_sel:[1,0,0]\n\t"
        "v_cvt_scalef32_pk_bf16_fp8 %4, %10, %12\n\t"
        "v_cvt_scalef32_pk_bf16_fp8 %5, %10, %12 op_sel:[1,0,0]\n\t"
        "v_cvt_scalef32_pk_bf16_fp8 %6, %11, %12\n\t"
        "v_cvt_scalef32_pk_bf16_fp8 %7, %11, %12 op_sel:[1,0,0]\n\t"
        "s_nop 1"
        : "=&v"(o0), "=&v"(o1), "=&v"(o2), "=&v"(o3), "=&v"(o4), "=&v"(o5), "=&v"(o6), "=&v"(o7)
        : "v"(w[k].x), "v"(w[k].y), "v"(w[k].z), "v"(w[k].w), "v"(s[k]));
    // e0 + 8 is the next 16-byte chunk of the same block row
    *reinterpret_cast<uint4*>(tb + off[k]) = make_uint4(o0, o1, o2, o3);
    *reinterpret_cast<uint4*>(tb + (off[k] ^ 16)) = make_uint4(o4, o5, o6, o7);
  }
}

// Item = (column block, row, 16-code quarter of the block): consecutive
// lanes take the four quarters of consecutive rows of one block, so a
// wave's bf16 stores stay inside one block (rows 128 B apart, chunks
// swizzled) and its staging reads walk rows R bytes apart.  A thread's
// items are loaded a few at a time before they are converted (two LDS
// round trips per tile instead of one per item, within the registers the
// kernel leaves free).
template <class C>
__device__ inline void convert_tile_e4(const unsigned char* __restrict__ st, unsigned char* __restrict__ tb, int tid) {
  constexpr int ITEMS = C::E4_TILE / 16;
  constexpr int PER = (ITEMS + C::NTHR - 1) / C::NTHR;
  static_assert(ITEMS == (C::R / 64) * C::TILE * 4, "whole 64-column blocks");
  constexpr int FIRST = (PER + 1) / 2;
  convert_items_e4<C, FIRST>(st, tb, tid, 0);
  convert_items_e4<C, PER - FIRST>(st, tb, tid, FIRST);
}

// DMA the trailing QL column blocks of q for this wave's 32 heads into LDS
// (swizzled 128-byte rows, one per head); heads past H read as zeros.
template <class C>
__device__ inline void issue_q_tail(const AttnArgs& a, unsigned char* smem, int v, int h_base, int wave, int lane) {
  using T = typename C::T;
  const int h0 = h_base + wave * 32;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(
      reinterpret_cast<const T*>(a.q) + ((size_t)v * a.H + min(h0, a.H)) * C::R, max(min(a.H - h0, 32), 0) * C::ROW_BYTES);
#pragma unroll
  for (int qb = 0; qb < C::QL; ++qb)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int r = 8 * i4 + (lane >> 3);  // head row within the wave
      const int c = (lane & 7) ^ swz(r);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, MLA_LDS_PTR(smem + C::OFF_Q + qb * C::Q_BLOCK_BYTES + wave * 4096 + i4 * 1024),
                                               16, r * C::ROW_BYTES + ((C::RKQ / 4 + qb) * 64 + c * 8) * C::ES, 0, 0, 0);
    }
}

// One 32-token tile of a segment: issue the DMA of a later tile into
// `dma_stage`, then the score phase, online softmax and PV phase on `tb`.
// The LDS pointers are restrict-qualified: within one call the stage being
// filled, the stage being read and the P / alpha buffers never overlap, which
// lets the compiler's wait insertion keep the DMA of later tiles in flight
// (the DMA of this tile was waited for explicitly before the call).
template <class C>
__device__ __forceinline__ void tile_step(const AttnArgs& a, unsigned char* __restrict__ dma_stage,
                                          const unsigned char* __restrict__ tb, typename C::T* __restrict__ p_s,
                                          const unsigned char* __restrict__ q_s, float* __restrict__ alpha_s,
                                          int* __restrict__ flag_s, bool issue,
                                          int b, int k_issue, int tok0, int vis, int i, int wave, int lane,
                                          int dma_off, const int (&s_base)[4], const int (&tr_base)[2][2],
                                          const typename C::F::frag (&qf)[C::RKQ], float& m_run, float& l_run,
                                          f32x16 (&O)[C::NTH][C::NCT],
                                          const unsigned char* __restrict__ conv_src = nullptr,
                                          unsigned char* __restrict__ conv_dst = nullptr) {
  using T = typename C::T;
  using F = typename C::F;
  using frag = typename F::frag;
  const int hi = lane >> 5, l32 = lane & 31;
  // DMA of the tile NSTAGE-1 ahead.  FAST bf16 tiles: the buffer record
  // (and the page lookup) now, the nine loads spread over the score MFMAs,
  // one every four k-steps: issued back to back, the four waves' 36 loads
  // held each wave for ~600 clocks while the address unit drained them.
  // (E4M3 tiles the same way: the code and scale records now, the loads
  // of the staging slot spread over the first k-steps.)
  constexpr bool SPREAD = C::FAST && !C::E4;
  __amdgpu_buffer_rsrc_t dma_rsrc;
  E4Rsrc e4r;
  if constexpr (C::E4)
    e4r = e4_rsrc<C>(a, b, k_issue, vis, lane, issue);
  else if constexpr (SPREAD)
    dma_rsrc = tile_rsrc<C>(a, b, k_issue, vis, lane, issue);
  else
    issue_tile<C>(a, dma_stage, b, k_issue, vis, wave, lane, dma_off, issue);

  // ---- S^T[32 tokens x 32 heads] = tile . q^T (one MFMA chain) --------
  auto a_frag = [&](int kb) -> frag {
    if constexpr (C::FAST) {
      return *reinterpret_cast<const frag*>(tb + s_base[kb & 3] + (kb >> 2) * C::BLOCK_BYTES);
    } else {
      return *reinterpret_cast<const frag*>(tb + lds_off<C>(l32, kb * C::KB + hi * C::KPL));
    }
  };
  // q^T fragment kb: registers, or the LDS copy of the trailing blocks
  auto b_frag = [&](int kb) -> frag {
    if constexpr (C::QL > 0) {
      if (kb >= C::RKQ) return *reinterpret_cast<const frag*>(q_s + (kb / 4 - C::RKQ / 4) * C::Q_BLOCK_BYTES + s_base[kb & 3]);
    }
    return qf[kb < C::RKQ ? kb : 0];
  };
  // operands are fetched SD k-steps ahead of their MFMA
  constexpr int SD = 4;
  frag ring_a[SD], ring_b[SD];
#pragma unroll
  for (int kb = 0; kb < SD; ++kb) {
    ring_a[kb] = a_frag(kb);
    if (kb >= C::RKQ) ring_b[kb] = b_frag(kb);
  }
  f32x16 s0;
#pragma unroll
  for (int kb = 0; kb < C::RK; ++kb) {
    const frag av = ring_a[kb % SD];
    const frag bv = kb >= C::RKQ ? ring_b[kb % SD] : qf[kb < C::RKQ ? kb : 0];
    if (kb + SD < C::RK) {
      ring_a[kb % SD] = a_frag(kb + SD);
      if (kb + SD >= C::RKQ) ring_b[kb % SD] = b_frag(kb + SD);
    }
    if (kb == 0)
      s0 = F::first(av, bv);
    else if (kb + 1 < C::RK)
      F::acc_v(s0, av, bv);
    else
      F::acc_v_last(s0, av, bv);
    if constexpr (C::E4) {
      static_assert(!C::E4 || C::RK >= 4 * C::E4_LOADS, "one load per four k-steps");
      if (kb % 4 == 2 && kb / 4 < C::E4_LOADS) e4_load<C>(e4r, dma_stage, wave, lane, kb / 4);
    }
    if constexpr (SPREAD) {
      static_assert(!SPREAD || C::RK >= 4 * (C::NINST / C::NW), "one load per four k-steps");
      if (kb % 4 == 2) {
        switch (kb / 4) {
          case 0: dma_block<C, 0>(dma_rsrc, dma_stage, wave, dma_off); break;
          case 1: dma_block<C, 1>(dma_rsrc, dma_stage, wave, dma_off); break;
          case 2: dma_block<C, 2>(dma_rsrc, dma_stage, wave, dma_off); break;
          case 3: dma_block<C, 3>(dma_rsrc, dma_stage, wave, dma_off); break;
          case 4: dma_block<C, 4>(dma_rsrc, dma_stage, wave, dma_off); break;
          case 5: dma_block<C, 5>(dma_rsrc, dma_stage, wave, dma_off); break;
          case 6: dma_block<C, 6>(dma_rsrc, dma_stage, wave, dma_off); break;
          case 7: dma_block<C, 7>(dma_rsrc, dma_stage, wave, dma_off); break;
          case 8: dma_block<C, 8>(dma_rsrc, dma_stage, wave, dma_off); break;
          default: break;
        }
      }
    }
  }

  // ---- online softmax for head (wave*32 + l32) over the 32 tokens -------
  // register r of this lane holds token 8*(r/4) + 4*hi + r%4
  const int hl = wave * 32 + l32;
  float x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = s0[r] * a.scale_log2;
  if (tok0 + C::TILE > vis) {  // uniform: only the last tile of a sequence is ragged
    const int lim = vis - tok0 - 4 * hi;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (8 * (r >> 2) + (r & 3) >= lim) x[r] = -INFINITY;
  }
  float mloc = x[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mloc = fmaxf(mloc, x[r]);
  mloc = max_xor32(mloc);
  const bool rebase = mloc > m_run + kRescaleSlack;
  float alpha = 1.f;
  if (rebase) {
    alpha = __builtin_amdgcn_exp2f(m_run - mloc);
    m_run = mloc;
  }
  float psum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    x[r] = __builtin_amdgcn_exp2f(x[r] - m_run);
    psum += x[r];
  }
  psum = sum_xor32(psum);
  l_run = l_run * alpha + psum;
  {
    // P[head][token]: this lane's tokens 8*q4 + 4*hi + (0..3) are contiguous
    T* prow = p_s + (size_t)hl * C::PSTR + 4 * hi;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      if constexpr (C::ES == 2) {
        T v4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v4[u] = from_f32<T>(x[4 * q4 + u]);
        *reinterpret_cast<uint2*>(prow + 8 * q4) = *reinterpret_cast<const uint2*>(v4);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) prow[8 * q4 + u] = from_f32<T>(x[4 * q4 + u]);
      }
    }
  }
  if (hi == 0) alpha_s[hl] = alpha;
  const bool any = __any(rebase);
  if (lane == 0) flag_s[wave] = any ? 1 : 0;
  // E4M3: the codes of the next tile (DMA'd a step ago) are in for every
  // wave behind this barrier; only this step's DMA may be in flight
  if constexpr (C::E4) vm_wait<C::E4_LOADS>();
  lds_barrier();

  // ---- PV: O[all heads][this wave's columns] += P . tile ----------------
  if (i > 0) {
    int anyf = 0;
#pragma unroll
    for (int ht = 0; ht < C::NTH; ++ht) anyf |= flag_s[ht];
    if (__builtin_amdgcn_readfirstlane(anyf)) {
      o_settle<T>(O);
#pragma unroll
      for (int ht = 0; ht < C::NTH; ++ht) {
        // O row of register r: head ht*32 + 8*(r/4) + 4*hi + r%4
        float al[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 a4 = *reinterpret_cast<const float4*>(alpha_s + ht * 32 + 8 * q4 + 4 * hi);
          al[4 * q4 + 0] = a4.x;
          al[4 * q4 + 1] = a4.y;
          al[4 * q4 + 2] = a4.z;
          al[4 * q4 + 3] = a4.w;
        }
#pragma unroll
        for (int ct = 0; ct < C::NCT; ++ct) {
          if constexpr (C::ES == 2) {
            o_scale_tile(O[ht][ct], al);
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) O[ht][ct][r] *= al[r];
          }
        }
      }
      o_settle<T>(O);
    }
  }
  if constexpr (C::FAST) {
    // B operand of (ks, ct): 8 rows x 1 column per lane, read with two
    // transposing LDS loads (ds_read_b64_tr_b16).  In each 16-lane group the
    // instruction hands lane i element i%4 of the 8-byte rows addressed by
    // lanes i/4 + 4j (j = 0..3); lane s of the group therefore addresses row
    // kbase + s/4, columns nbase + 4(s%4) .. +3, and lane i receives rows
    // kbase..kbase+3 of column nbase + i.  tr_base holds those addresses.
    // The loads of the next column tile are issued before the MFMAs of the
    // current one.
    typedef short v4s __attribute__((ext_vector_type(4)));
    auto b_load = [&](int ks, int ct, v4s (&bb)[2]) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
        bb[h2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<__attribute__((address_space(3))) v4s*>(
            MLA_LDS_PTR(tb + tr_base[ct & 1][h2] + (ct >> 1) * C::BLOCK_BYTES + ks * 16 * 128)));
    };
    v4s bb[2];
    b_load(0, 0, bb);
#pragma unroll
    for (int ks = 0; ks < C::PV_KS; ++ks) {
      frag pa[C::NTH];
#pragma unroll
      for (int ht = 0; ht < C::NTH; ++ht)
        pa[ht] = *reinterpret_cast<const frag*>(p_s + (size_t)(ht * 32 + l32) * C::PSTR + ks * C::KB + hi * C::KPL);
#pragma unroll
      for (int ct = 0; ct < C::NCT; ++ct) {
        const frag bfr = __builtin_bit_cast(frag, bb);
        if (ct + 1 < C::NCT)
          b_load(ks, ct + 1, bb);
        else if (ks + 1 < C::PV_KS)
          b_load(ks + 1, 0, bb);
#pragma unroll
        for (int ht = 0; ht < C::NTH; ++ht) F::acc_a(O[ht][ct], pa[ht], bfr);
      }
    }
  } else {
    // generic layout: one element per lane and k (KPL == 1 for fp32)
#pragma unroll
    for (int ks = 0; ks < C::PV_KS; ++ks) {
      frag pa[C::NTH];
#pragma unroll
      for (int ht = 0; ht < C::NTH; ++ht)
        pa[ht] = *reinterpret_cast<const frag*>(p_s + (size_t)(ht * 32 + l32) * C::PSTR + ks * C::KB + hi * C::KPL);
#pragma unroll
      for (int ct = 0; ct < C::NCT; ++ct) {
        frag bfr;
        if constexpr (C::KPL == 1) {
          bfr = *reinterpret_cast<const T*>(tb + lds_off<C>(ks * C::KB + hi, wave * C::CPW + ct * 32 + l32));
        } else {
#pragma unroll
          for (int j = 0; j < C::KPL; ++j)
            bfr[j] = *reinterpret_cast<const T*>(tb + lds_off<C>(ks * C::KB + hi * C::KPL + j, wave * C::CPW + ct * 32 + l32));
        }
        F::acc_a_fresh_b(O[0][ct], pa[0], bfr);
#pragma unroll
        for (int ht = 1; ht < C::NTH; ++ht) F::acc_a(O[ht][ct], pa[ht], bfr);
      }
    }
  }
  // E4M3: convert the next tile into the other bf16 slot (its tile was
  // finished a step ago); the next step's barrier publishes it
  if constexpr (C::E4) convert_tile_e4<C>(conv_src, conv_dst, wave * 64 + lane);
}

template <class C>
__global__ __launch_bounds__(C::NTHR, 1) void attn_split_kernel(AttnArgs a) {
  using T = typename C::T;
  using F = typename C::F;
  using frag = typename F::frag;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5, l32 = lane & 31;
  const int G = gridDim.x;
  // XCD-aware order: the hardware deals blocks round-robin over 8 XCDs, so
  // logical ranges are assigned such that neighbours share an XCD's L2.
  const int w = ((G & 7) == 0) ? ((int)(blockIdx.x & 7) * (G >> 3) + (int)(blockIdx.x >> 3)) : (int)blockIdx.x;
  // work-group record: tile range and the first stream it touches
  const auto wr = MLA_CONST_PTR(a.wrec) + 8 * w;
  const int g0 = wr[0], g1 = wr[1];
  if (g0 >= g1) return;
  int u = wr[2], tb0 = wr[3], tb1 = wr[4], vis = wr[5];

  float* alpha_s = reinterpret_cast<float*>(smem + C::OFF_ALPHA);
  float* m_s = reinterpret_cast<float*>(smem + C::OFF_M);
  float* l_s = reinterpret_cast<float*>(smem + C::OFF_L);
  int* flag_s = reinterpret_cast<int*>(smem + C::OFF_FLAG);
  T* p_s = reinterpret_cast<T*>(smem + C::OFF_P);

  // Lane-constant offsets (closed forms of lds_off, FAST layout):
  //   dma_off      : global offset of this lane's 16 B in its wave's DMA rows
  //   s_base[u]    : score-phase A fragment, k-step kb with kb%4 == u
  //   tr_base[t][h]: transposing PV read of column tile ct (t = ct&1), rows
  //                  16ks + 8(g>>1) + 4h + s/4 (g = lane/16, s = lane%16)
  int dma_off = 0, s_base[4] = {0, 0, 0, 0}, tr_base[2][2] = {{0, 0}, {0, 0}};
  if constexpr (C::FAST) {
    const int r = 8 * wave + (lane >> 3);
    dma_off = r * C::ROW_BYTES + 16 * ((lane & 7) ^ swz(r));
#pragma unroll
    for (int u = 0; u < 4; ++u) s_base[u] = l32 * 128 + 16 * ((2 * u + hi) ^ swz(l32));
    const int g = lane >> 4, sl = lane & 15;
    const int c_low = 2 * (g & 1) + ((sl & 3) >> 1);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
        tr_base[t][h2] = 2 * wave * C::BLOCK_BYTES + tile_chunk(8 * (g >> 1) + 4 * h2 + (sl >> 2), 4 * t + c_low) +
                         8 * (sl & 1);
  }

  constexpr int n_loads = C::NINST / C::NW;  // DMA instructions per tile and wave

  int gcur = g0;
  while (gcur < g1) {
    if (tb1 <= gcur) {  // next stream (an empty one has tb0 == tb1)
      ++u;
      const auto sr = MLA_CONST_PTR(a.srec) + 4 * u;
      tb0 = sr[0];
      tb1 = sr[1];
      vis = sr[2];
      continue;
    }
    const int k0 = gcur - tb0, k1 = min(g1, tb1) - tb0;
    const bool whole = (k0 == 0) && (k1 == tb1 - tb0);
    const int cnt = k1 - k0;
    const int v = u / a.n_hg, hgrp = u - v * a.n_hg;
    const int h_base = hgrp * C::HP;
    const int b = v / a.n_q;

    // tile 0 first, then q, then the other prologue tiles: the wait before
    // tile 0 then also covers q, and later tiles stay in flight
    unsigned char* e4_stage = smem + C::OFF_E4;  // E4M3 staging slots (E4 only)
    if constexpr (C::E4)
      issue_tile_e4<C>(a, e4_stage, b, k0, vis, wave, lane, true);
    else
      issue_tile<C>(a, smem, b, k0, vis, wave, lane, dma_off, true);
    asm volatile("" ::: "memory");  // keep the issue order: tile 0, q, tile 1
    // q^T fragments of this wave's 32 heads: the first RKQ k-steps in
    // registers, the trailing QL column blocks DMA'd into LDS (same
    // swizzled 128-byte row layout as the tiles, one row per head).  Heads
    // past H read the zero buffer.
    frag qf[C::RKQ];
    {
      const int h = h_base + wave * 32 + l32;
      const T* qp = (h < a.H) ? reinterpret_cast<const T*>(a.q) + ((size_t)v * a.H + h) * C::R + hi * C::KPL
                              : reinterpret_cast<const T*>(g_zero_rows) + hi * C::KPL;
#pragma unroll
      for (int kb = 0; kb < C::RKQ; ++kb) qf[kb] = load_frag<T>(qp + kb * C::KB);
      if constexpr (C::QL > 0) issue_q_tail<C>(a, smem, v, h_base, wave, lane);
    }
    asm volatile("" ::: "memory");
    if constexpr (C::E4) {
      issue_tile_e4<C>(a, e4_stage + C::E4_STAGE, b, k0 + 1, vis, wave, lane, 1 < cnt);
    } else {
      for (int s = 1; s < C::NSTAGE - 1; ++s)
        issue_tile<C>(a, smem + s * C::TILE_BYTES, b, k0 + s, vis, wave, lane, dma_off, s < cnt);
    }

    float m_run = -1e30f, l_run = 0.f;
    f32x16 O[C::NTH][C::NCT];
#pragma unroll
    for (int ht = 0; ht < C::NTH; ++ht)
#pragma unroll
      for (int ct = 0; ct < C::NCT; ++ct) O[ht][ct] = f32x16{};

    if constexpr (C::E4) {
      // codes of tile 0 (and q) are in, tile 1 in flight: convert tile 0
      vm_wait<C::E4_LOADS>();
      lds_barrier();
      convert_tile_e4<C>(e4_stage, smem, tid);
    }
    auto step = [&](int i) {
      if constexpr (C::E4) {
        // tile i was converted into bf16 slot i % 2 at the end of the last
        // step; the DMA of tile i + 2 goes into the staging slot of tile i
        // (converted then too), and tile i + 1 is converted at the end
        lds_barrier();
        tile_step<C>(a, e4_stage + (i % 2) * C::E4_STAGE, smem + (i % 2) * C::TILE_BYTES, p_s,
                     smem + C::OFF_Q + wave * 4096, alpha_s, flag_s, i + 2 < cnt, b, k0 + i + 2, (k0 + i) * C::TILE,
                     vis, i, wave, lane, dma_off, s_base, tr_base, qf, m_run, l_run, O,
                     e4_stage + ((i + 1) % 2) * C::E4_STAGE, smem + ((i + 1) % 2) * C::TILE_BYTES);
      } else {
        // tiles i+1 .. i+NSTAGE-2 may stay in flight (zero-filled past the end)
        vm_wait<(C::NSTAGE - 2) * n_loads>();
        lds_barrier();
        tile_step<C>(a, smem + ((i + C::NSTAGE - 1) % C::NSTAGE) * C::TILE_BYTES, smem + (i % C::NSTAGE) * C::TILE_BYTES,
                     p_s, smem + C::OFF_Q + wave * 4096, alpha_s, flag_s, i + C::NSTAGE - 1 < cnt, b,
                     k0 + i + C::NSTAGE - 1, (k0 + i) * C::TILE, vis, i, wave, lane, dma_off, s_base, tr_base, qf,
                     m_run, l_run, O);
      }
    };
    // tile 0 is peeled: the compiler's wait for the q registers then lands
    // in front of its first use (leaving the DMA of tile 1 in flight)
    // instead of in front of the loop
    step(0);
    for (int i = 1; i < cnt; ++i) step(i);

    // ---- finalise the segment ----------------------------------------
    o_settle<T>(O);
    if (hi == 0) {
      m_s[wave * 32 + l32] = m_run;
      l_s[wave * 32 + l32] = l_run;
    }
    lds_barrier();
    const int pid = w + u;  // partial slot of this (work-group, stream) piece
    {
      // this lane's O elements: head ht*32 + 8*q4 + 4*hi + rr, column
      // wave*CPW + ct*32 + l32; one base pointer, compile-time offsets
      float* base = whole ? a.o_lat + ((size_t)v * a.H + h_base) * C::DL : a.part_o + (size_t)pid * C::HP * C::DL;
      base += (size_t)(4 * hi) * C::DL + wave * C::CPW + l32;
#pragma unroll
      for (int ht = 0; ht < C::NTH; ++ht) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 l4 = *reinterpret_cast<const float4*>(l_s + ht * 32 + 8 * q4 + 4 * hi);
          const float inv[4] = {1.f / l4.x, 1.f / l4.y, 1.f / l4.z, 1.f / l4.w};
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int hl0 = ht * 32 + 8 * q4 + rr;
            if (h_base + hl0 + 4 * hi >= a.H) continue;
#pragma unroll
            for (int ct = 0; ct < C::NCT; ++ct) base[hl0 * C::DL + ct * 32] = O[ht][ct][4 * q4 + rr] * inv[rr];
          }
        }
      }
    }
    {
      const int hl = wave * 32 + l32;
      if (hi == 0 && h_base + hl < a.H) {
        const float lse2 = m_run + __log2f(l_run);
        if (whole) {
          if (a.lse) a.lse[(size_t)v * a.H + h_base + hl] = lse2 * 0.69314718055994531f;
        } else {
          a.part_lse[(size_t)pid * C::HP + hl] = lse2;
        }
      }
    }
    lds_barrier();
    gcur = tb0 + k1;
  }
}

constexpr int kPlanThreads = 256;

// Inclusive prefix sum over the plan block (4 waves); *total gets the sum.
__device__ inline int plan_scan(int v, int* wsum, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(v, off, 64);
    if (lane >= off) v += y;
  }
  if (lane == 63) wsum[wv] = v;
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < kPlanThreads / 64; ++k) {
    pre += k < wv ? wsum[k] : 0;
    tot += wsum[k];
  }
  __syncthreads();
  *total = tot;
  return v + pre;
}

__device__ inline int plan_max(int v, int* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
  if (lane == 0) wsum[wv] = v;
  __syncthreads();
  int m = wsum[0];
#pragma unroll
  for (int k = 1; k < kPlanThreads / 64; ++k) m = max(m, wsum[k]);
  __syncthreads();
  return m;
}

// Work plan (one block).  Streams u = v * n_hg + head group are cut into
// 32-token tiles; every work-group gets a contiguous range of the
// concatenated tile list.  Three ways to cut it:
//   * even: per0 = ceil(T / G) tiles each; ranges may span stream ends, so a
//     work-group can run several segments (each costs a q load, a pipeline
//     fill and a 256 KB partial write);
//   * aligned: every stream is cut into chunks of `per` tiles with
//     per = max(per0, ceil(T / (G - nz))) (nz: streams with tiles), which
//     gives at most T / per + nz <= G chunks; one segment per work-group;
//   * balanced: ranges of equal cost, tiles + kSegCost x stream starts
//     (stream records staged in LDS only).
// The one whose busiest work-group costs least in (tiles + kSegCost x
// segments) is used; kSegCost is the measured cost of a segment in tiles
// (per-work-group timestamps, 64 streams of 16-512 tiles: 4.6 k clocks per
// tile, 26 k per segment).  Outputs: srec[u] = {first tile, end tile, visible rows, 0},
// wfl[u] = {first, last work-group} (-1 for an invalid length), wrec[w] =
// {g0, g1, first stream, its srec}.  Invalid lengths get no tiles and raise
// error bit 4 (page ids are checked where the split kernel follows them).
constexpr int kSegCost = 6;

__global__ __launch_bounds__(kPlanThreads) void attn_plan_kernel(AttnArgs a, int cap) {
  constexpr int kLdsU = 2048;  // stream records staged in LDS up to this many streams
  __shared__ int wsum[kPlanThreads / 64];
  __shared__ int hist[1024];
  __shared__ int sx[kLdsU], sy[kLdsU];
  __shared__ int xs[kLdsU];    // starts of the streams with tiles, in order (balanced cut)
  __shared__ int gb[1025];     // balanced cut: work-group w gets tiles [gb[w], gb[w + 1])
  __shared__ int jb[1025];     // ... and tile gb[w] lies in stream piece jb[w]
  const int tid = threadIdx.x;
  const int U = a.U, G = a.G, n_q = a.n_q, n_hg = a.n_hg;
  const bool staged = U <= kLdsU;
  auto rec = [&](int u) -> int2 {
    if (staged) return make_int2(sx[u], sy[u]);
    const int4 r = reinterpret_cast<const int4*>(a.srec)[u];
    return make_int2(r.x, r.y);
  };
  // tile prefix sums and per-stream records
  int carry = 0, nz = 0;
  for (int base = 0; base < U; base += kPlanThreads) {
    const int u = base + tid;
    int cnt = 0, vis = 0;
    if (u < U) {
      const int v = u / n_hg, b = v / n_q, j = v - b * n_q;
      const int L = a.kv_len[b];
      if (L < n_q || L > cap) {
        if (j == 0 && u % n_hg == 0) atomicOr(a.err, 4);
      } else {
        vis = L - n_q + j + 1;
        cnt = (vis + 31) / 32;
      }
    }
    int tot, tot_nz;
    const int inc = plan_scan(cnt, wsum, &tot);
    const int inz = plan_scan(cnt > 0, wsum, &tot_nz);
    if (u < U) {
      reinterpret_cast<int4*>(a.srec)[u] = make_int4(carry + inc - cnt, carry + inc, vis, 0);
      if (staged) {
        sx[u] = carry + inc - cnt;
        sy[u] = carry + inc;
        if (cnt > 0) xs[nz + inz - 1] = carry + inc - cnt;
      }
    }
    carry += tot;
    nz += tot_nz;
  }
  const int T = carry;
  const int per0 = max(1, (T + G - 1) / G);
  for (int w = tid; w < G; w += kPlanThreads) hist[w] = 0;
  __syncthreads();  // srec visible to the whole block

  // even cut: streams starting strictly inside a work-group's range add a
  // segment to it; aligned cut: chunk counts for per0 .. per0 + 7
  for (int u = tid; u < U; u += kPlanThreads) {
    const int2 r = rec(u);
    if (r.y > r.x && r.x % per0) atomicAdd(&hist[r.x / per0], 1);
  }
  __syncthreads();
  int hmax = 0;
  for (int w = tid; w < G; w += kPlanThreads) hmax = max(hmax, hist[w]);
  const int smax = 1 + plan_max(hmax, wsum);
  // chunks(per) <= T / per + nz, so this per yields at most G chunks
  const int per = G > nz ? max(per0, (T + (G - nz) - 1) / (G - nz)) : 0;
  // balanced cut.  Entering stream piece j (the j-th stream with tiles,
  // tiles [xs[j], xs[j + 1])) costs kSegCost, each tile 1: the cumulative
  // cost is F = xs[j] + kSegCost (j + 1) + (g - xs[j]) inside piece j, and
  // its entry step spans [xs[j] + kSegCost j, xs[j] + kSegCost (j + 1)).
  // Boundary w sits where F reaches w FT / G (FT = T + kSegCost nz): at
  // xs[j] when that falls in piece j's entry step, else inside the piece.
  // One thread per boundary finds its piece, the last j with
  // xs[j] + kSegCost j <= w FT / G, and jb[w] records the piece that holds
  // tile gb[w].
  // Skipped when a lower bound on its cost would not beat the other cuts:
  // the mean FT / G, and with more than two work-groups per piece FT / G
  // plus one segment (some work-group then holds no stream start; checked
  // on random stream mixes).
  const long long cost_even = (long long)per0 + (long long)kSegCost * smax;
  const long long cost_al = per > 0 ? (long long)per + kSegCost : LLONG_MAX;
  const long long FT = (long long)T + (long long)kSegCost * nz;
  const long long bal_lb = G > 2 * nz ? FT / G + kSegCost : (FT + G - 1) / G;
  long long cost_bal = LLONG_MAX;
  if (staged && G <= 1024 && nz > 0 && bal_lb + kSegCost / 2 <= min(cost_even, cost_al)) {
    const bool narrow = FT * G < (1LL << 31);  // 32-bit division suffices
    for (int w = tid; w <= G; w += kPlanThreads) {
      if (w == G) {
        gb[w] = T;
        jb[w] = nz;
        continue;
      }
      const long long t = narrow ? (long long)(w * (int)FT / G) : (long long)w * FT / G;
      int lo = 0, hi = nz;  // xs[0] + 0 = 0 <= t
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((long long)xs[mid] + (long long)kSegCost * mid <= t) lo = mid; else hi = mid;
      }
      const long long x0 = xs[lo], x1 = lo + 1 < nz ? xs[lo + 1] : T;
      const long long f_in = x0 + (long long)kSegCost * (lo + 1);
      gb[w] = (int)(t < f_in ? x0 : min(x1, x0 + (t - f_in)));
      jb[w] = lo;
    }
    __syncthreads();
    int cmax = 0;
    for (int w = tid; w < G; w += kPlanThreads) {
      const int g0 = gb[w], g1 = gb[w + 1];
      if (g1 > g0) {
        // pieces holding tiles g0 and g1 - 1 (g1 at a piece start ends the previous one)
        const int j0 = jb[w], j1 = (jb[w + 1] < nz && g1 == xs[jb[w + 1]]) || jb[w + 1] == nz ? jb[w + 1] - 1 : jb[w + 1];
        cmax = max(cmax, g1 - g0 + kSegCost * (j1 - j0 + 1));
      }
    }
    cost_bal = plan_max(cmax, wsum);
  }
  // (the balanced cut only when it saves at least half a segment: it may
  // cut more streams than the others, and a close call is within the
  // model's error)
  // (cost_even is finite; cost_bal is LLONG_MAX when the cut was not computed)
  const bool balanced = cost_bal <= min(cost_even, cost_al) - kSegCost / 2;
  const bool aligned = !balanced && cost_al <= cost_even;

  // work-group records
  for (int w = tid; w < G; w += kPlanThreads) {
    int* wr = a.wrec + 8 * w;
    int g0 = 0, g1 = 0, u0 = 0;
    int4 r = make_int4(0, 0, 0, 0);
    if (balanced ? gb[w + 1] > gb[w] : (!aligned && w * per0 < T)) {
      g0 = balanced ? gb[w] : w * per0;
      g1 = balanced ? gb[w + 1] : min(g0 + per0, T);
      int lo = 0, hi = U;  // last stream with start <= g0 (and tiles)
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (rec(mid).x <= g0) lo = mid; else hi = mid;
      }
      u0 = lo;
      while (rec(u0).y <= g0) ++u0;  // skip empty streams
      r = reinterpret_cast<const int4*>(a.srec)[u0];
    }
    wr[0] = g0; wr[1] = g1; wr[2] = u0; wr[3] = r.x; wr[4] = r.y; wr[5] = r.z; wr[6] = 0; wr[7] = 0;
  }
  __syncthreads();
  int chunk_base = 0;
  for (int base = 0; base < U; base += kPlanThreads) {
    const int u = base + tid;
    int4 r = make_int4(0, 0, 0, 0);
    if (u < U) {
      const int2 xy = rec(u);
      r = make_int4(xy.x, xy.y, 0, 0);
    }
    const int nch = aligned ? (r.y - r.x + per - 1) / per : 0;
    int tot;
    const int c0 = chunk_base + plan_scan(nch, wsum, &tot) - nch;
    chunk_base += tot;
    if (u < U) {
      if (aligned && staged) xs[u] = c0;  // first chunk of stream u (xs is free again)
      int2 f = make_int2(-1, -1);
      if (r.y > r.x) {
        if (aligned) {
          f = make_int2(c0, c0 + nch - 1);
          if (!staged) {
            const int vis = reinterpret_cast<const int4*>(a.srec)[u].z;
            for (int c = 0; c < nch; ++c) {
              int* wr = a.wrec + 8 * (c0 + c);
              wr[0] = r.x + c * per; wr[1] = min(r.x + (c + 1) * per, r.y); wr[2] = u;
              wr[3] = r.x; wr[4] = r.y; wr[5] = vis;
            }
          }
        } else if (balanced) {
          // last work-group whose range starts at or before the stream's
          // first / last tile (empty ranges sit before the one that holds it)
          auto wg_of = [&](int g) {
            int lo = 0, hi = G;  // largest w with gb[w] <= g
            while (hi - lo > 1) {
              const int mid = (lo + hi) >> 1;
              if (gb[mid] <= g) lo = mid; else hi = mid;
            }
            return lo;
          };
          f = make_int2(wg_of(r.x), wg_of(r.y - 1));
        } else {
          f = make_int2(r.x / per0, (r.y - 1) / per0);
        }
      }
      reinterpret_cast<int2*>(a.wfl)[u] = f;
    }
  }
  if (aligned && staged) {
    // chunk records, one thread per work-group: its stream is the last one
    // whose first chunk is at or before it (a stream without chunks shares
    // its first-chunk index with the next stream, so it is never the last)
    __syncthreads();
    for (int w = tid; w < chunk_base; w += kPlanThreads) {
      int lo = 0, hi = U;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (xs[mid] <= w) lo = mid; else hi = mid;
      }
      const int c = w - xs[lo];
      const int vis = reinterpret_cast<const int4*>(a.srec)[lo].z;
      int* wr = a.wrec + 8 * w;
      wr[0] = sx[lo] + c * per; wr[1] = min(sx[lo] + (c + 1) * per, sy[lo]); wr[2] = lo;
      wr[3] = sx[lo]; wr[4] = sy[lo]; wr[5] = vis;
    }
  }
}

// Log-sum-exp merge of the pieces of every stream that was cut by a
// work-group boundary: lse = log2 sum_s 2^lse_s, o = sum_s 2^(lse_s - lse) O_s.
// Block = (stream, HPB heads of its group); each thread owns 4 columns.
template <int HP, int DL>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  constexpr int TPH = DL / 4;  // threads per head (4 columns each)
  constexpr int HPB = 256 / TPH;  // heads per block
  constexpr int CH = 16;          // pieces whose O values are held in registers at once
  const int u = blockIdx.x, tid = threadIdx.x;
  const int v = u / a.n_hg, hgrp = u - v * a.n_hg;
  const int hl = blockIdx.y * HPB + tid / TPH;  // head within the group
  const int h = hgrp * HP + hl;                 // global head
  const int c0 = (tid % TPH) * 4;
  if (hl >= HP || h >= a.H) return;
  const int2 fl = reinterpret_cast<const int2*>(a.wfl)[u];
  const int wf = fl.x, wl = fl.y;
  float* dst = a.o_lat + ((size_t)v * a.H + h) * DL + c0;
  if (wf < 0) {  // invalid length: flagged by the plan kernel; poison the output
    *reinterpret_cast<float4*>(dst) = make_float4(NAN, NAN, NAN, NAN);
    if (a.lse && c0 == 0) a.lse[(size_t)v * a.H + h] = NAN;
    return;
  }
  if (wf == wl) return;  // written whole by the split kernel
  const int n = wl - wf + 1;
  const float* pl = a.part_lse + (size_t)(wf + u) * HP + hl;             // piece s at pl[s * HP]
  const float* src = a.part_o + ((size_t)(wf + u) * HP + hl) * DL + c0;  // piece s at src[s * HP * DL]
  // Loads are issued CH pieces at a time (O values and LSEs together), so a
  // chunk costs one memory round trip.  Pass 1 forms the total LSE with a
  // running max; pass 2 weights the O values (the first chunk stays in
  // registers from pass 1).  Only the chunk's real pieces are loaded (n is
  // uniform over the block: scalar branches); the rest take LSE -inf.
  float4 x[CH];
  float lv[CH];
  auto load_chunk = [&](int base, bool with_o) {
#pragma unroll
    for (int s = 0; s < CH; ++s) {
      if (base + s < n) {
        lv[s] = pl[(size_t)(base + s) * HP];
        if (with_o) x[s] = *reinterpret_cast<const float4*>(src + (size_t)(base + s) * HP * DL);
      } else {
        lv[s] = -INFINITY;
      }
    }
  };
  load_chunk(0, true);
  float mx = -INFINITY, sum = 0.f;
  for (int base = 0; base < n; base += CH) {
    if (base > 0) load_chunk(base, false);
    float cm = -INFINITY;
#pragma unroll
    for (int s = 0; s < CH; ++s) cm = fmaxf(cm, lv[s]);  // at least one real piece
    const float nm = fmaxf(mx, cm);
    float cs = 0.f;
#pragma unroll
    for (int s = 0; s < CH; ++s) cs += (base + s < n) ? exp2f(lv[s] - nm) : 0.f;
    sum = sum * exp2f(mx - nm) + cs;
    mx = nm;
  }
  const float L = mx + log2f(sum);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int base = 0; base < n; base += CH) {
    if (base > 0 || n > CH) load_chunk(base, true);
#pragma unroll
    for (int s = 0; s < CH; ++s) {
      if (base + s < n) {
        const float wgt = exp2f(lv[s] - L);
        acc.x += wgt * x[s].x;
        acc.y += wgt * x[s].y;
        acc.z += wgt * x[s].z;
        acc.w += wgt * x[s].w;
      }
    }
  }
  *reinterpret_cast<float4*>(dst) = acc;
  if (a.lse && c0 == 0) a.lse[(size_t)v * a.H + h] = L * 0.69314718055994531f;
}

int attn_supported(bool bf16, int H, int d_latent, int d_rope) {
  if (bf16) return H >= 1 && H <= 1024 && d_latent == CfgBf16::DL && d_rope == CfgBf16::DR;
  return H >= 1 && H <= 1024 && d_latent == CfgF32::DL && d_rope == CfgF32::DR;
}

int attn_head_group(bool bf16) { return bf16 ? CfgBf16::HP : CfgF32::HP; }

int attn_tile() { return 32; }

size_t attn_sched_ints(int U, int G) { return 6 * (size_t)U + 8 * (size_t)G; }

template <class C>
static hipError_t launch_attn_t(const AttnArgs& a, hipStream_t s) {
  if (hipError_t e = ensure_lds_limit<&attn_split_kernel<C>>(C::LDS_BYTES); e != hipSuccess) return e;
  const int cap = a.paged ? a.max_pages * a.page_size : a.s_max;
  hipLaunchKernelGGL(attn_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a, cap);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_split_kernel<C>, dim3(a.G), dim3(C::NTHR), C::LDS_BYTES, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int hpb = 256 / (C::DL / 4);
  hipLaunchKernelGGL((attn_merge_kernel<C::HP, C::DL>), dim3(a.U, (C::HP + hpb - 1) / hpb), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a_in, bool bf16, hipStream_t s) {
  AttnArgs a = a_in;
  a.n_hg = (a.H + attn_head_group(bf16) - 1) / attn_head_group(bf16);
  a.U = a.V * a.n_hg;
  if (a.G < 8 || a.G > 1024) return hipErrorInvalidValue;
  // plan storage: wrec [8G] | srec [4U] | wfl [2U]
  a.wrec = a.sched;
  a.srec = a.wrec + 8 * a.G;
  a.wfl = a.srec + 4 * a.U;
  if (!bf16) return a.e4m3 ? hipErrorInvalidValue : launch_attn_t<CfgF32>(a, s);
  // one query token and one head group: every cache row is read by one
  // stream only, so its tiles are loaded non-temporally
  const bool nt = a.n_q == 1 && a.n_hg == 1;
  if (a.e4m3) return nt ? launch_attn_t<CfgE4Nt>(a, s) : launch_attn_t<CfgE4>(a, s);
  return nt ? launch_attn_t<CfgBf16Nt>(a, s) : launch_attn_t<CfgBf16>(a, s);
}

// ===========================================================================
// Expanded-form chunked prefill (bf16, d_nope = d_v = 128, d_rope = 64).
//
// For long query chunks the scores are cheaper against per-head keys than
// against the 576-wide latents: every cached latent is up-projected once to
// k[h] = c W_UK[h] (128) and v[h] = c W_UV[h] (128) (GEMMs, outside this
// kernel), and each head runs causal softmax attention with 192-wide keys
// (k[h] | the shared RoPE key of the cache row) and 128-wide values (page
// "How DeepSeek Rewrote the Transformer", sections 03-04: queries, keys,
// values and the causal mask per head; page "Multi-Head Latent Attention
// (MLA)", "The construction": per-head keys and values are up-projections
// of the latent).
//
// A work-group takes 128 queries of one (sequence, head); wave w owns
// queries 32w..32w+31 and needs nothing from the other waves except the
// shared key/value tiles:
//   * 32-key tiles go global -> LDS by buffer-load DMA through a 3-stage
//     ring, as five 64-column blocks (k[h] 0-63, 64-127, k_pe, v[h] 0-63,
//     64-127) of 128-byte rows with the decode kernel's chunk swizzle;
//   * S^T[32 keys x 32 queries] = K_tile . Q^T (12 MFMAs, Q in registers):
//     a lane holds one query, so the online softmax is in-lane plus one
//     permlane32 exchange;
//   * O^T[128 dims x 32 queries] += V_tile^T . P^T: the B operand (P^T) is
//     the score registers rounded to bf16, the A operand four transposing
//     LDS reads per 32 dims; the lane again holds one query, so rescaling
//     and the final normalisation are per lane.
// ===========================================================================
constexpr int kFaTile = 32;
constexpr int kFaBlk = kFaTile * 128;     // one 64-column block of a tile
constexpr int kFaStage = 5 * kFaBlk;      // K 0-63 | K 64-127 | k_pe | V 0-63 | V 64-127
constexpr int kFaNst = 3;
constexpr int kFaOStr = 128 * 2 + 16;     // O staging row: 128 bf16 + pad
constexpr int kFaLds = kFaNst * kFaStage > 4 * 32 * kFaOStr ? kFaNst * kFaStage : 4 * 32 * kFaOStr;

bool prefill_supported(bool bf16, int d_nope, int d_rope, int d_v) {
  return bf16 && d_nope == 128 && d_rope == 64 && d_v == 128;
}

// One 32-key tile of the prefill: the DMA of a later tile into `dma_st`,
// then (if any key of the tile is visible to the wave) scores, online
// softmax and the PV update from `tb`.  Both stage pointers are restrict:
// within one call the stage being filled and the stage being read never
// overlap, which lets the compiler's wait insertion keep the DMA in flight
// while the tile is read.  The fragments of each phase are read from LDS
// before its MFMAs.
template <class Issue>
__device__ __forceinline__ void prefill_tile(const PrefillArgs& a, const Issue& issue, unsigned char* __restrict__ dma_st,
                                             const unsigned char* __restrict__ tb, int it_issue, int k0, bool live,
                                             int wave_q0, int qpos, int hi, const int (&s_base)[4],
                                             const int (&trb)[2][2], const bf16x8 (&qf)[12], float& m_run,
                                             float& l_run, f32x16 (&O)[4]) {
  issue(it_issue, dma_st);
  if (!live) return;  // every key of the tile is after this wave's queries
  // ---- S^T = K . Q^T -----------------------------------------------------
  bf16x8 ka[12];
#pragma unroll
  for (int kb = 0; kb < 12; ++kb) ka[kb] = *reinterpret_cast<const bf16x8*>(tb + (kb >> 2) * kFaBlk + s_base[kb & 3]);
  __builtin_amdgcn_sched_barrier(0);  // keep the twelve reads ahead of the chain
  // Wave priority: the softmax runs raised, everything else at base, so
  // while one wave's MFMAs occupy the SIMD's matrix unit the other wave's
  // softmax issues first (measured on the V3 expanded step: 2.08 -> 2.045 ms
  // with the reads and DMA raised as well, 2.02 ms with the softmax alone;
  // raising the MFMA sections instead changed nothing).
  f32x16 s = f32x16{};
  __builtin_amdgcn_s_setprio(0);
#pragma unroll
  for (int kb = 0; kb < 12; ++kb) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kb], qf[kb], s, 0, 0, 0);
  __builtin_amdgcn_s_setprio(2);
  // ---- online softmax for this lane's query (register r: key k0 + 8(r/4) + 4hi + r%4)
  float x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = s[r];
  if (k0 + kFaTile - 1 > wave_q0) {  // uniform: the tile reaches past the wave's first query
    const int lim = qpos - k0 - 4 * hi;  // visible: 8(r/4) + r%4 <= lim
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (8 * (r >> 2) + (r & 3) > lim) x[r] = -INFINITY;
  }
  float mraw = x[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mraw = fmaxf(mraw, x[r]);
  const float mloc = max_xor32(mraw) * a.scale_log2;
  if (mloc > m_run + kRescaleSlack) {
    const float alpha = __builtin_amdgcn_exp2f(m_run - mloc);
    m_run = mloc;
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) O[dt][r] *= alpha;
  }
  float psum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    x[r] = __builtin_amdgcn_exp2f(fmaf(x[r], a.scale_log2, -m_run));
    psum += x[r];
  }
  l_run += sum_xor32(psum);
  bf16x8 pf[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int j = 0; j < 8; ++j) pf[ks][j] = (__bf16)x[8 * ks + j];
  __builtin_amdgcn_s_setprio(0);
  // ---- O^T += V^T . P^T ----------------------------------------------------
  typedef short v4s __attribute__((ext_vector_type(4)));
  v4s vv[4][2][2];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
        vv[dt][ks][h2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<__attribute__((address_space(3))) v4s*>(
            MLA_LDS_PTR(const_cast<unsigned char*>(tb) + (3 + (dt >> 1)) * kFaBlk + trb[dt & 1][h2] + ks * 16 * 128)));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv[dt][ks]), pf[ks], O[dt], 0, 0, 0);
}

__global__ __launch_bounds__(256, 2) void prefill_attn_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hi = lane >> 5, l32 = lane & 31;
  // Work-groups are handed to the eight XCDs round-robin by linear id.  The
  // query blocks of one (sequence, head) read the same keys and values, so
  // they are renumbered to run together on one XCD and share its L2.
  int qb, h, b;
  {
    const int gx = gridDim.x, gy = gridDim.y, T = gx * gy * gridDim.z;
    const int id = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
    const int L = (T & 7) ? id : (id & 7) * (T >> 3) + (id >> 3);
    qb = L % gx;
    h = (L / gx) % gy;
    b = L / (gx * gy);
  }
  const int t0 = qb * 128;
  const int kvl = a.kv_len[b];
  const int tw = t0 + 32 * wave;  // first query of this wave
  const int t = tw + l32;         // this lane's query
  const bool qv = t < a.n_q;
  const size_t orow = (size_t)(b * a.n_q + t) * a.H + h;  // output row of (query, head)
  if (kvl < a.n_q || kvl > a.s_max) {
    // the sequence's length is unusable: flag it, poison its outputs
    if (threadIdx.x == 0) atomicOr(a.err, 4);
    if (qv && hi == 0) {
      __bf16* o = reinterpret_cast<__bf16*>(a.vo) + orow * 128;
      for (int d = 0; d < 128; ++d) o[d] = (__bf16)__builtin_nanf("");
      if (a.lse) a.lse[orow] = __builtin_nanf("");
    }
    return;
  }
  const int S = kvl - a.n_q;                        // rows before the chunk
  const int t_last = min(t0 + 127, a.n_q - 1);
  const int kend = S + t_last + 1;                  // keys [0, kend) for this block
  const int ntiles = (kend + kFaTile - 1) / kFaTile;
  const int wave_kend = tw < a.n_q ? S + min(tw + 31, a.n_q - 1) + 1 : 0;  // keys this wave needs
  const int qpos = S + t;                           // keys 0 .. qpos are visible to this lane

  // Q^T fragments (B operand): query t, dims 16 kb + 8 hi .. +7
  bf16x8 qf[12];
  {
    const __bf16* qp = reinterpret_cast<const __bf16*>(a.qe) + (qv ? orow : (size_t)h) * 192 + 8 * hi;
#pragma unroll
    for (int kb = 0; kb < 12; ++kb) qf[kb] = qv ? load_frag<__bf16>(qp + 16 * kb) : Mfma<__bf16>::zero();
  }

  // DMA: wave w fills rows 8w + lane/8 of each block; the lane's LDS slot is
  // physical chunk lane%8 of its row, i.e. logical chunk c
  const int dr = 8 * wave + (lane >> 3);
  const int dc = (lane & 7) ^ swz(dr);
  const int kv_row_bytes = a.H * 256;
  auto issue = [&](int it, unsigned char* st) {
    const int k0 = it * kFaTile;
    const int rows = it < ntiles ? min(kFaTile, kend - k0) : 0;
    const size_t r0 = (size_t)b * a.s_max + k0;
    const __amdgpu_buffer_rsrc_t rk =
        make_rsrc(reinterpret_cast<const __bf16*>(a.ke) + (r0 * a.H + h) * 128, rows * kv_row_bytes);
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc(reinterpret_cast<const __bf16*>(a.ve) + (r0 * a.H + h) * 128, rows * kv_row_bytes);
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(reinterpret_cast<const __bf16*>(a.pool) + r0 * 576 + 512, rows * 1152);
    const int ko = dr * kv_row_bytes + dc * 16;
    unsigned char* w0 = st + wave * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, MLA_LDS_PTR(w0 + 0 * kFaBlk), 16, ko, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, MLA_LDS_PTR(w0 + 1 * kFaBlk), 16, ko + 128, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rp, MLA_LDS_PTR(w0 + 2 * kFaBlk), 16, dr * 1152 + dc * 16, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, MLA_LDS_PTR(w0 + 3 * kFaBlk), 16, ko, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, MLA_LDS_PTR(w0 + 4 * kFaBlk), 16, ko + 128, 0, 0, 0);
  };
  constexpr int kLoads = 5;  // DMA instructions per tile and wave

  // lane-constant LDS offsets: score A fragments (key row l32, chunk pair
  // 2u + hi of a block) and the transposing V reads (rows 16 ks + 4 hi +
  // 8 h2 + s/4 of column tile t, s = lane%16)
  int s_base[4], trb[2][2];
#pragma unroll
  for (int u = 0; u < 4; ++u) s_base[u] = l32 * 128 + 16 * ((2 * u + hi) ^ swz(l32));
  {
    const int g = lane >> 4, sl = lane & 15;
    const int c_low = 2 * (g & 1) + ((sl & 3) >> 1);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
        trb[tt][h2] = tile_chunk(4 * hi + 8 * h2 + (sl >> 2), 4 * tt + c_low) + 8 * (sl & 1);
  }

  issue(0, smem);
  issue(1, smem + kFaStage);
  float m_run = -1e30f, l_run = 0.f;
  f32x16 O[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) O[dt] = f32x16{};

  for (int it = 0; it < ntiles; ++it) {
    vm_wait<(kFaNst - 2) * kLoads>();
    lds_barrier();
    prefill_tile(a, issue, smem + ((it + 2) % kFaNst) * kFaStage, smem + (it % kFaNst) * kFaStage, it + 2,
                 it * kFaTile, it * kFaTile < wave_kend, S + tw, qpos, hi, s_base, trb, qf, m_run, l_run, O);
  }

  // ---- finalise: normalise, stage [32 queries][128 dims] per wave, store rows
  vm_wait<0>();  // the DMA issued past the last tile (zeros) may still land in the ring
  lds_barrier();
  const float inv = 1.f / l_run;
  unsigned char* ost = smem + wave * 32 * kFaOStr;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      __bf16 v4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v4[u] = (__bf16)(O[dt][4 * q4 + u] * inv);
      *reinterpret_cast<uint2*>(ost + l32 * kFaOStr + (32 * dt + 8 * q4 + 4 * hi) * 2) =
          *reinterpret_cast<const uint2*>(v4);
    }
  lds_barrier();
  for (int i = lane; i < 32 * 16; i += 64) {
    const int qr = i >> 4, ch = i & 15, tq = tw + qr;
    if (tq < a.n_q)
      *reinterpret_cast<uint4*>(reinterpret_cast<__bf16*>(a.vo) + ((size_t)(b * a.n_q + tq) * a.H + h) * 128 + ch * 8) =
          *reinterpret_cast<const uint4*>(ost + qr * kFaOStr + ch * 16);
  }
  if (qv && hi == 0 && a.lse) a.lse[orow] = (m_run + __log2f(l_run)) * 0.69314718055994531f;
}

hipError_t launch_prefill_attention(const PrefillArgs& a, hipStream_t s) {
  if (hipError_t e = ensure_lds_limit<&prefill_attn_kernel>(kFaLds); e != hipSuccess) return e;
  hipLaunchKernelGGL(prefill_attn_kernel, dim3((a.n_q + 127) / 128, a.H, a.B), dim3(256), kFaLds, s, a);
  return hipGetLastError();
}

}  // namespace mla
