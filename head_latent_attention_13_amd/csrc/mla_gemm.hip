// Weight-streaming GEMM, its epilogues (RoPE, cache append) and the one-time
// weight absorption for the MLA library (gfx950).
//
// Decode-time projections multiply a few token rows (M = batch * new tokens)
// by a large weight, so they are bound by streaming the weight from HBM.
// Weights are stored in the packed fragment order of mla_common.h: one
// MFMA B fragment is one contiguous 1 KB block (bf16), so every wave-wide
// weight load is a single fully coalesced 16 B-per-lane access.
#include <algorithm>

#include "mla_common.h"
#include "mla_internal.h"

namespace mla {

// --------------------------------------------------------------------------
// Epilogue of one column pair (n, n+1) of output row m, given final sums.
// Pairs keep a RoPE rotation (pairs (2j, 2j+1) of the rope part) in-thread.
// --------------------------------------------------------------------------
template <typename T>
__device__ inline void epi_pair(const EpiArgs& e, int m, int n, float v0, float v1) {
  if (m >= e.M || n >= e.N) return;
  const bool has1 = n + 1 < e.N;
  if (e.mode == EPI_F32) {
    float* y = reinterpret_cast<float*>(e.out) + (size_t)m * e.N + n;
    if (has1) {
      *reinterpret_cast<float2*>(y) = make_float2(v0, v1);
    } else {
      y[0] = v0;
    }
    return;
  }
  if (e.mode == EPI_STORE_T) {
    T* y = reinterpret_cast<T*>(e.out) + (size_t)m * e.N + n;
    y[0] = from_f32<T>(v0);
    if (has1) y[1] = from_f32<T>(v1);
    return;
  }
  const int b = m / e.n_q, t = m - b * e.n_q;
  const bool q = e.mode == EPI_Q;
  // column within its group (EPI_Q) or within one cache row (EPI_APPEND)
  const int f = n % (q ? e.qg_cols : e.row), rope0 = q ? e.rope_from : e.d_latent;
  const int pos = q ? e.kv_len[b] - e.n_q + t : e.pos[b] + t;
  if (f >= rope0) {
    float c, s;
    rope_cos_sin(pos, (f - rope0) >> 1, e.d_rope, e.rope_base, &c, &s);
    const float a0 = v0, a1 = v1;
    v0 = a0 * c - a1 * s;
    v1 = a0 * s + a1 * c;
  }
  if (q) {
    T* y = reinterpret_cast<T*>(e.out) + (size_t)m * e.q_ld + e.q_off + (size_t)(n / e.qg_cols) * e.qg_stride + f;
    y[0] = from_f32<T>(v0);
    y[1] = from_f32<T>(v1);
    return;
  }
  // EPI_APPEND: N == row; write into the cache slot of position pos.
  T* dst;
  if (e.paged) {
    const int cap = e.max_pages * e.page_size;
    if (pos < 0 || pos >= cap) {
      if (n == 0) atomicOr(e.err, 1);
      return;
    }
    const int pg = e.page_table[(size_t)b * e.max_pages + pos / e.page_size];
    if (pg < 0 || pg >= e.n_pages) {
      if (n == 0) atomicOr(e.err, 2);
      return;
    }
    dst = reinterpret_cast<T*>(e.pool) + ((size_t)pg * e.page_size + pos % e.page_size) * e.row;
  } else {
    if (pos < 0 || pos >= e.s_max) {
      if (n == 0) atomicOr(e.err, 1);
      return;
    }
    dst = reinterpret_cast<T*>(e.pool) + ((size_t)b * e.s_max + pos) * e.row;
  }
  dst[n] = from_f32<T>(v0);
  dst[n + 1] = from_f32<T>(v1);
}

// XCD-aware block order: the hardware deals work-groups round-robin over the
// 8 XCDs (each with its own L2), so physical block b runs on XCD b % 8.
// Logical block (b % 8) * (T / 8) + b / 8 gives every XCD a contiguous range
// of the (x fastest, then y, then z) logical order: one XCD then holds one
// K slice (or two) of the A operand instead of all of them.
struct BlockXYZ {
  int x, y, z;
};
__device__ inline BlockXYZ xcd_block() {
  const int gx = gridDim.x, gy = gridDim.y, T = gx * gy * gridDim.z;
  const int b = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  const int L = (T & 7) ? b : (b & 7) * (T >> 3) + (b >> 3);
  return BlockXYZ{L % gx, (L / gx) % gy, L / (gx * gy)};
}

struct GemmArgs {
  const void* A;
  int lda;
  const void* Wp;
  int kblocks, ntiles, Np, ksplit, kb_per_split;
  int a_gtiles, a_gstride;  // A column groups (0: none)
  float* part;
  EpiArgs e;
  const int32_t* row_len;   // needed rows per group of row_group rows (NULL: all)
  int row_group;
};

// Whether any row of [m0, m1) is needed: row m of group b = m / row_group
// is needed when m - b * row_group < row_len[b] (clamped to [0, row_group]).
// Uniform across the block (scalar loads of the group lengths).
__device__ inline bool rows_needed(const GemmArgs& g, int m0, int m1) {
  if (!g.row_len) return true;
  const int G = g.row_group;
  for (int b = m0 / G; b * G < m1; ++b) {
    const int lim = min(max(g.row_len[b], 0), G);
    if (max(m0 - b * G, 0) < lim) return true;
  }
  return false;
}

// --------------------------------------------------------------------------
// Streamed-weight GEMM with the epilogue fused when the K range is not split
// (see mla_internal.h).  With ksplit > 1 the block writes its fp32 slice of
// the tile and splitk_epilogue_kernel finishes the sum in a second launch
// (no cross-work-group fences: the kernel boundary orders the slices).
// --------------------------------------------------------------------------
template <typename T, typename TA, int MT, int NT, int KSW>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  using F = Mfma<T>;
  using frag = typename F::frag;
  constexpr int KB = F::KB, KPL = F::KPL, FR = 64 * KPL;
  constexpr int NGW = 4 / KSW;                 // column groups per block
  constexpr int ROWS = MT * 16, COLS = NGW * NT * 16;
  __shared__ float red[KSW][ROWS][COLS];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int M = g.e.M;
  const BlockXYZ blk = xcd_block();
  const int col0 = blk.x * COLS;                                       // first column of the block tile
  const int nt0 = blk.x * NGW * NT + (KSW == 1 ? wave * NT : 0);
  const int mt0 = blk.y * MT;
  const int ks = blk.z;
  if (!rows_needed(g, mt0 * 16, min((mt0 + MT) * 16, M))) return;  // whole block
  int kb0 = ks * g.kb_per_split;
  int kb1 = min(kb0 + g.kb_per_split, g.kblocks);
  if (KSW > 1) {  // this wave's share of the slice
    const int len = kb1 - kb0, per = (len + KSW - 1) / KSW;
    kb0 = min(kb0 + wave * per, kb1);
    kb1 = min(kb0 + per, kb1);
  }

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int ni = 0; ni < NT; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  const TA* ap[MT];
  bool aval[MT];
  // A column group of this wave's tiles (they never straddle two groups)
  const size_t a_col = g.a_gtiles ? (size_t)(nt0 / g.a_gtiles) * g.a_gstride : 0;
#pragma unroll
  for (int mi = 0; mi < MT; ++mi) {
    const int m = (mt0 + mi) * 16 + (lane & 15);
    aval[mi] = m < M;
    ap[mi] = reinterpret_cast<const TA*>(g.A) + (size_t)(aval[mi] ? m : 0) * (size_t)g.lda + a_col + (lane >> 4) * KPL;
  }
  // k-block-major packed weights: tile nt at k-block kb is fragment kb*ntiles + nt
  const size_t kb_stride = (size_t)g.ntiles * FR;
  const T* wp[NT];
#pragma unroll
  for (int ni = 0; ni < NT; ++ni) {
    const int nt = min(nt0 + ni, g.ntiles - 1);
    wp[ni] = reinterpret_cast<const T*>(g.Wp) + (size_t)nt * FR + lane * KPL;
  }

  // Weights are read exactly once: non-temporal loads (a read-once stream
  // reaches a higher HBM rate that way, and does not evict the A operand,
  // re-read by every column block, from L2).
  constexpr bool kStreamW = sizeof(frag) == 16;
  auto load_b = [&](frag (&b)[NT], int kb) {
#pragma unroll
    for (int ni = 0; ni < NT; ++ni) {
      if constexpr (kStreamW) {
        typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
        b[ni] = __builtin_bit_cast(
            frag, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(wp[ni] + (size_t)kb * kb_stride)));
      } else {
        b[ni] = *reinterpret_cast<const frag*>(wp[ni] + (size_t)kb * kb_stride);
      }
    }
  };
  auto load_a = [&](frag (&a)[MT], int kb) {
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      if constexpr (sizeof(TA) == sizeof(T)) {
        a[mi] = load_frag<T>(reinterpret_cast<const T*>(ap[mi]) + kb * KB);
      } else {
        a[mi] = load_frag_from_f32<T>(reinterpret_cast<const float*>(ap[mi]) + kb * KB);
      }
      if (!aval[mi]) a[mi] = F::zero();
    }
  };
  auto mma_all = [&](const frag (&a)[MT], const frag (&b)[NT]) {
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int ni = 0; ni < NT; ++ni) acc[mi][ni] = F::mma(a[mi], b[ni], acc[mi][ni]);
  };
  // Software pipeline over groups of U k-blocks with two register buffers:
  // the loads of group i+1 are issued before the MFMAs of group i, so the
  // weight stream never drains between groups.
  constexpr int U = (12 / (NT + MT)) > 1 ? (12 / (NT + MT)) : 1;
  auto load_group = [&](frag (&b)[U][NT], frag (&a)[U][MT], int kb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      load_b(b[u], kb + u);
      load_a(a[u], kb + u);
    }
  };
  auto mma_group = [&](const frag (&b)[U][NT], const frag (&a)[U][MT]) {
#pragma unroll
    for (int u = 0; u < U; ++u) mma_all(a[u], b[u]);
  };
  int kb = kb0;
  if (kb + U <= kb1) {
    frag b0[U][NT], a0[U][MT], b1[U][NT], a1[U][MT];
    load_group(b0, a0, kb);
    for (;;) {
      const bool n1 = kb + 2 * U <= kb1;
      if (n1) load_group(b1, a1, kb + U);
      mma_group(b0, a0);
      kb += U;
      if (!n1) break;
      const bool n2 = kb + 2 * U <= kb1;
      if (n2) load_group(b0, a0, kb + U);
      mma_group(b1, a1);
      kb += U;
      if (!n2) break;
    }
  }
  for (; kb < kb1; ++kb) {
    frag b[NT], a[MT];
    load_b(b, kb);
    load_a(a, kb);
    mma_all(a, b);
  }

  // ---- combine the block tile in LDS -----------------------------------
  {
    const int slot = KSW > 1 ? wave : 0;
    const int cbase = KSW > 1 ? 0 : wave * NT * 16;
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int ni = 0; ni < NT; ++ni)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          red[slot][mi * 16 + 4 * (lane >> 4) + i][cbase + ni * 16 + (lane & 15)] = acc[mi][ni][i];
  }
  __syncthreads();
  constexpr int PAIRS = ROWS * COLS / 2;
  const int row0 = mt0 * 16;
  for (int p = threadIdx.x; p < PAIRS; p += 256) {
    const int r = p / (COLS / 2), c = (p % (COLS / 2)) * 2;
    const int m = row0 + r, n = col0 + c;
    if (m >= M || n >= g.Np) continue;
    float v0 = 0.f, v1 = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < KSW; ++s2) {
      v0 += red[s2][r][c];
      v1 += red[s2][r][c + 1];
    }
    if (g.ksplit == 1) {
      epi_pair<T>(g.e, m, n, v0, v1);
    } else {
      *reinterpret_cast<float2*>(g.part + ((size_t)ks * M + m) * g.Np + n) = make_float2(v0, v1);
    }
  }
}

// --------------------------------------------------------------------------
// LDS-tiled GEMM for more than 16 rows (batched decode, chunked prefill).
//
// Block tile BM x BN = (64 MTW) x (64 NTW); 4 waves in a 2 x 2 grid, wave
// (wm, wn) computes rows [32 MTW wm, +32 MTW) x columns [32 NTW wn, +32 NTW)
// with v_mfma_f32_32x32x16_bf16.  A stage covers SKB k-blocks (32 k each):
//   A: BM rows x 32 SKB k of TA, row-major, 16-byte chunk c of row r stored
//      at chunk c ^ swz_a(r) (conflict-free 16-lane ds_read_b128 passes);
//   W: the BN/16 packed 1 KB fragments of each k-block, in fragment order.
// Both are DMA'd with buffer loads (rows past M and n-tiles past the weight
// read as zeros) through a 3-stage ring, two stages in flight.
// A 32x32x16 B operand is read straight from the packed 16-column
// fragments: lane l takes column tile (l%32)/16, rows 8 (l/32) + 16 ks.
// Every MFMA reads (MTW + NTW) / (MTW NTW) KB of operands from LDS, so the
// large-M configuration uses 128 x 128 wave tiles (0.5 KB per MFMA) to stay
// clear of the LDS bandwidth.
// --------------------------------------------------------------------------
// An unsplit K of at most this many k-blocks counts as short (ring choice)
constexpr int kShortSlice = 64;

template <typename TA, int MTW, int NTW, int SKB_, int NSTAGE_ = 3, bool WNT_ = false>
struct TiledCfg {
  static constexpr bool WNT = WNT_;                  // weights read once: non-temporal DMA
  static constexpr int BM = 64 * MTW, BN = 64 * NTW;
  static constexpr int SKB = SKB_;                   // k-blocks (32 k) per stage
  static constexpr int ESA = (int)sizeof(TA);
  static constexpr int ROWB = SKB * 32 * ESA;        // A bytes per row per stage
  static constexpr int CPR = ROWB / 16;              // 16-byte chunks per A row
  static constexpr int A_BYTES = BM * ROWB;
  static constexpr int NTB = BN / 16;                // packed n-tiles per block
  static constexpr int B_BYTES = SKB * NTB * 1024;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int NSTAGE = NSTAGE_;             // ring stages, NSTAGE - 1 in flight
  static constexpr int A_INST = A_BYTES / 1024, B_INST = SKB * NTB;
  static constexpr int LOADS = (A_INST + B_INST) / 4;  // DMA instructions per wave per stage
  // RoPE epilogue: half the block tile in fp32, rows padded by 16 bytes,
  // then per-row positions / cache offsets (12 B per row)
  static constexpr int TS = BN + 4;
  static constexpr int ROW_META = BM / 2 * TS * 4;
  static constexpr int EPI_TOTAL = ROW_META + BM * 12;
  static constexpr int LDS = NSTAGE * STAGE > EPI_TOTAL ? NSTAGE * STAGE : EPI_TOTAL;
  static_assert(A_INST % 4 == 0 && B_INST % 4 == 0, "whole DMA instructions per wave");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

__device__ inline int swz_a(int r, int cpr) {
  // 64-byte rows: 4 rows per 256 bytes, rows r and r+4 differ in the chunk;
  // 128-byte rows alternate bank halves: permute the 8 same-parity rows of a
  // 16-row group; 256-byte rows all start on bank 0: spread 16 rows over 16 chunks
  return cpr == 4 ? ((r >> 2) & 3) : cpr == 8 ? ((((r >> 1) & 1) << 2) | ((r >> 2) & 3)) : (r & 15);
}

__device__ inline __amdgpu_buffer_rsrc_t gemm_rsrc(const void* base, long bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p), hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  const int n = (int)(bytes > 0x7fffffffL ? 0x7fffffffL : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0,
                                           __builtin_amdgcn_readfirstlane(n), 0x00020000);
}

// DMA of stage `kb` (first k-block of the stage) into `st`; live == false
// (past the slice) loads zeros.  Every wave issues C::LOADS instructions;
// instruction u of a wave is one of its A rows-group loads (u < A_INST/4) or
// one of its packed W fragments.
template <class C>
struct TiledDma {
  unsigned char* st;
  int m0, nt0, kb;
  bool live;
};
template <class C>
__device__ inline TiledDma<C> tiled_dma(const GemmArgs&, unsigned char* st, int m0, int nt0, int kb, bool live) {
  return TiledDma<C>{st, m0, nt0, kb, live};
}
// (Not a template: the tile constants come in as arguments and fold at the
// inlined call sites.)
__device__ inline void tiled_dma_load(const GemmArgs& g, unsigned char* st, int m0, int nt0, int kb, bool live, int u,
                                      int wave, int lane, int a_inst, int rowb, int esa, int ntb, int a_bytes,
                                      bool wnt) {
  const int aw = a_inst / 4, cpr = rowb / 16;
  if (u < aw) {
    // A: rows m0.., k from kb*32; the record count stops at row M (zeros below)
    const long a_rows = live ? (long)max(g.e.M - m0, 0) : 0;
    const size_t a_col = g.a_gtiles ? (size_t)(nt0 / g.a_gtiles) * g.a_gstride : 0;  // A column group
    const __amdgpu_buffer_rsrc_t ra =
        gemm_rsrc(reinterpret_cast<const unsigned char*>(g.A) + ((size_t)m0 * g.lda + a_col + (size_t)kb * 32) * esa,
                  a_rows * g.lda * esa);
    const int i = wave + 4 * u;
    const int r = i * (1024 / rowb) + lane / cpr, pc = lane % cpr;
    const int c = pc ^ swz_a(r, cpr);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, MLA_LDS_PTR(st + i * 1024), 16, r * g.lda * esa + c * 16, 0, 0, 0);
  } else {
    // W: fragment (kb + j, nt0 + t) -> B region slot j * NTB + t
    const __amdgpu_buffer_rsrc_t rw = gemm_rsrc(g.Wp, live ? (long)g.kblocks * g.ntiles * 1024 : 0);
    const int i = wave + 4 * (u - aw);
    const int j = i / ntb, t = i % ntb;
    const int nt = nt0 + t;
    const int off = nt < g.ntiles ? (int)((((long)(kb + j) * g.ntiles) + nt) * 1024) + lane * 16 : 0x7ffffff0;
    // (cache policy 2 = non-temporal: a stream read once reaches a higher
    // HBM rate and does not displace A from L2)
    if (wnt)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, MLA_LDS_PTR(st + a_bytes + i * 1024), 16, off, 0, 0, 2);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, MLA_LDS_PTR(st + a_bytes + i * 1024), 16, off, 0, 0, 0);
  }
}
template <class C>
__device__ inline void tiled_dma_one(const GemmArgs& g, const TiledDma<C>& d, int u, int wave, int lane) {
  tiled_dma_load(g, d.st, d.m0, d.nt0, d.kb, d.live, u, wave, lane, C::A_INST, C::ROWB, C::ESA, C::NTB, C::A_BYTES,
                 C::WNT);
}
template <class C>
__device__ inline void tiled_issue(const GemmArgs& g, unsigned char* st, int m0, int nt0, int kb, bool live, int wave,
                                   int lane) {
  const TiledDma<C> d = tiled_dma<C>(g, st, m0, nt0, kb, live);
#pragma unroll
  for (int u = 0; u < C::LOADS; ++u) tiled_dma_one<C>(g, d, u, wave, lane);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename TA, int MTW, int NTW, int SKB, int NS, bool WNT>
__global__ __launch_bounds__(256, 1) void gemm_tiled_kernel(GemmArgs g) {
  using C = TiledCfg<TA, MTW, NTW, SKB, NS, WNT>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  // row blocks vary fastest: blocks running together share their weight
  // columns (each W tile is fetched once) while A, M rows deep, stays cached
  const BlockXYZ blk = xcd_block();
  const int m0 = blk.x * C::BM, nt0 = blk.y * C::NTB;
  const int ks = blk.z;
  if (!rows_needed(g, m0, min(m0 + C::BM, g.e.M))) return;  // whole block, before any DMA
  const int kb0 = ks * g.kb_per_split, kb1 = min(kb0 + g.kb_per_split, g.kblocks);
  const int nst = (kb1 - kb0 + C::SKB - 1) / C::SKB;  // stages in this slice

  f32x16 acc[MTW][NTW];
#pragma unroll
  for (int i = 0; i < MTW; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[i][j] = f32x16{};

  // lane-constant LDS offsets
  int a_off[MTW][2];  // [tile][chunk parity within the 16-k step]
#pragma unroll
  for (int i = 0; i < MTW; ++i) {
    const int r = (wm * MTW + i) * 32 + (lane & 31);
#pragma unroll
    for (int h = 0; h < 2; ++h) a_off[i][h] = r * C::ROWB;  // chunk added per k-step
  }
  const int a_row = lane & 31, a_hi = lane >> 5;
  int b_off[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j)
    b_off[j] = C::A_BYTES + ((wn * NTW + j) * 2 + ((lane & 31) >> 4)) * 1024 + ((lane & 15) + 16 * a_hi) * 16;

  // Fragments of 16-k step q of a stage (q = 2 kbl + k2).
  auto load_a = [&](const unsigned char* __restrict__ st, int q, bf16x8 (&af)[MTW]) {
    const int kbl = q >> 1, k2 = q & 1;
#pragma unroll
    for (int i = 0; i < MTW; ++i) {
      const int r = (wm * MTW + i) * 32 + a_row;
      if constexpr (C::ESA == 2) {
        const int c = (kbl * 4 + k2 * 2 + a_hi) ^ swz_a(r, C::CPR);
        af[i] = *reinterpret_cast<const bf16x8*>(st + a_off[i][0] + c * 16);
      } else {
        const int c0 = (kbl * 8 + k2 * 4 + a_hi * 2) ^ swz_a(r, C::CPR);
        const int c1 = (kbl * 8 + k2 * 4 + a_hi * 2 + 1) ^ swz_a(r, C::CPR);
        const float4 x0 = *reinterpret_cast<const float4*>(st + a_off[i][0] + c0 * 16);
        const float4 x1 = *reinterpret_cast<const float4*>(st + a_off[i][0] + c1 * 16);
        af[i][0] = (__bf16)x0.x; af[i][1] = (__bf16)x0.y; af[i][2] = (__bf16)x0.z; af[i][3] = (__bf16)x0.w;
        af[i][4] = (__bf16)x1.x; af[i][5] = (__bf16)x1.y; af[i][6] = (__bf16)x1.z; af[i][7] = (__bf16)x1.w;
      }
    }
  };
  auto load_b = [&](const unsigned char* __restrict__ st, int q, bf16x8 (&bf)[NTW]) {
    const int kbl = q >> 1, k2 = q & 1;
#pragma unroll
    for (int j = 0; j < NTW; ++j)
      bf[j] = *reinterpret_cast<const bf16x8*>(st + b_off[j] + kbl * C::NTB * 1024 + k2 * 32 * 16);
  };
  // One stage: the fragments of all its 16-k steps are read first, then
  // the MFMAs run (one LDS round trip per stage instead of one per step;
  // the scheduling barriers keep the compiler from re-serialising the reads
  // behind the MFMAs that use them).
  // (The DMA of a later stage is issued between the MFMAs: issued back to
  // back the loads would stall the wave on the address unit's queue.)
  auto compute = [&](const unsigned char* __restrict__ st, int nkb, const TiledDma<C>& dma) {
    constexpr int NQ = 2 * C::SKB;
    constexpr int NMF = NQ * MTW * NTW;
    const int nq = 2 * min(nkb, C::SKB);
    bf16x8 af[NQ][MTW], bf[NQ][NTW];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      if (q < nq) {
        load_a(st, q, af[q]);
        load_b(st, q, bf[q]);
      }
    }
    int mf = 0, issued = 0;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
#pragma unroll
      for (int i = 0; i < MTW; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
          if (q < nq) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[q][j], af[q][i], acc[i][j], 0, 0, 0);
          ++mf;
          // DMA instruction u goes after MFMA (u + 1) * NMF / LOADS
          while (issued < C::LOADS && mf * C::LOADS >= (issued + 1) * NMF) {
            tiled_dma_one<C>(g, dma, issued, wave, lane);
            ++issued;
          }
        }
    }
  };

  if constexpr (C::NSTAGE >= 4) {
    // Pipelined ring: while the MFMAs of 16-k step q run, the fragments of
    // step q + 1 are read from LDS into the registers step q + 1 used last
    // time (after the last step of a stage: step 0 of the next stage), and
    // the DMA of stage s + NSTAGE - 1 is spread over the MFMAs, so LDS
    // reads overlap the matrix work.  Stage s + 1 has to be in LDS when
    // stage s starts: NSTAGE - 3 stages stay in flight behind it.
    constexpr int NQ = 2 * C::SKB;
    constexpr int NMF = MTW * NTW;       // MFMAs per 16-k step
    constexpr int NRD = MTW + NTW;       // fragment reads per 16-k step
    bf16x8 af[NQ][MTW], bf[NQ][NTW];
    auto read_one = [&](const unsigned char* __restrict__ st, int q, int u) __attribute__((always_inline)) {
      const int kbl = q >> 1, k2 = q & 1;
      if (u < MTW) {
        const int rr = (wm * MTW + u) * 32 + a_row;
        if constexpr (C::ESA == 2) {
          const int c = (kbl * 4 + k2 * 2 + a_hi) ^ swz_a(rr, C::CPR);
          af[q][u] = *reinterpret_cast<const bf16x8*>(st + a_off[u][0] + c * 16);
        } else {
          const int c0 = (kbl * 8 + k2 * 4 + a_hi * 2) ^ swz_a(rr, C::CPR);
          const int c1 = (kbl * 8 + k2 * 4 + a_hi * 2 + 1) ^ swz_a(rr, C::CPR);
          const float4 x0 = *reinterpret_cast<const float4*>(st + a_off[u][0] + c0 * 16);
          const float4 x1 = *reinterpret_cast<const float4*>(st + a_off[u][0] + c1 * 16);
          bf16x8 v;
          v[0] = (__bf16)x0.x; v[1] = (__bf16)x0.y; v[2] = (__bf16)x0.z; v[3] = (__bf16)x0.w;
          v[4] = (__bf16)x1.x; v[5] = (__bf16)x1.y; v[6] = (__bf16)x1.z; v[7] = (__bf16)x1.w;
          af[q][u] = v;
        }
      } else {
        const int j = u - MTW;
        bf[q][j] = *reinterpret_cast<const bf16x8*>(st + b_off[j] + kbl * C::NTB * 1024 + k2 * 32 * 16);
      }
    };
    // One stage: cur = its ring slot, nxt = the next stage's slot (read by
    // the last step), dst = the slot the DMA fills; three distinct slots.
    // (Every stage is whole: slices are a multiple of SKB k-blocks, checked
    // at launch.  Reads are unconditional: a slot past the slice holds stale
    // data that no MFMA uses.)
    auto stage = [&](const unsigned char* __restrict__ cur, const unsigned char* __restrict__ nxt,
                     unsigned char* __restrict__ dst, int kb_dma, bool dma_live) __attribute__((always_inline)) {
      const TiledDma<C> dma = tiled_dma<C>(g, dst, m0, nt0, kb_dma, dma_live);
      int issued = 0;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const bool last = q + 1 == NQ;
        int rds = 0, mf = 0;
#pragma unroll
        for (int i = 0; i < MTW; ++i)
#pragma unroll
          for (int j = 0; j < NTW; ++j) {
            // the step's reads over its first half of MFMAs
            while (rds < NRD && 2 * mf * NRD >= rds * NMF) {
              read_one(last ? nxt : cur, last ? 0 : q + 1, rds);
              ++rds;
            }
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[q][j], af[q][i], acc[i][j], 0, 0, 0);
            ++mf;
            const int done = q * NMF + mf;
            while (issued < C::LOADS && done * C::LOADS >= (issued + 1) * NQ * NMF) {
              tiled_dma_one<C>(g, dma, issued, wave, lane);
              ++issued;
            }
          }
        while (rds < NRD) {
          read_one(last ? nxt : cur, last ? 0 : q + 1, rds);
          ++rds;
        }
      }
    };
    for (int s2 = 0; s2 < C::NSTAGE - 1; ++s2)
      tiled_issue<C>(g, smem + s2 * C::STAGE, m0, nt0, kb0 + s2 * C::SKB, s2 < nst, wave, lane);
    vm_wait<(C::NSTAGE - 2) * C::LOADS>();
    lds_barrier();
#pragma unroll
    for (int u = 0; u < NRD; ++u) read_one(smem, 0, u);
    for (int s2 = 0; s2 < nst; ++s2) {
      vm_wait<(C::NSTAGE - 3) * C::LOADS>();
      lds_barrier();
      unsigned char* cur = smem + (s2 % C::NSTAGE) * C::STAGE;
      unsigned char* nxt = smem + ((s2 + 1) % C::NSTAGE) * C::STAGE;
      unsigned char* dst = smem + ((s2 + C::NSTAGE - 1) % C::NSTAGE) * C::STAGE;
      const int kb_dma = kb0 + (s2 + C::NSTAGE - 1) * C::SKB;
      const bool dma_live = s2 + C::NSTAGE - 1 < nst;
      stage(cur, nxt, dst, kb_dma, dma_live);
    }
  } else {
    for (int s2 = 0; s2 < C::NSTAGE - 1; ++s2)
      tiled_issue<C>(g, smem + s2 * C::STAGE, m0, nt0, kb0 + s2 * C::SKB, s2 < nst, wave, lane);
    for (int s2 = 0; s2 < nst; ++s2) {
      vm_wait<(C::NSTAGE - 2) * C::LOADS>();
      lds_barrier();
      const TiledDma<C> dma = tiled_dma<C>(g, smem + ((s2 + C::NSTAGE - 1) % C::NSTAGE) * C::STAGE, m0, nt0,
                                           kb0 + (s2 + C::NSTAGE - 1) * C::SKB, s2 + C::NSTAGE - 1 < nst);
      compute(smem + (s2 % C::NSTAGE) * C::STAGE, min(C::SKB, kb1 - kb0 - s2 * C::SKB), dma);
    }
  }
  vm_wait<0>();
  lds_barrier();

  // ---- epilogue -----------------------------------------------------------
  // The MFMAs take the weight fragment as their first operand, so the
  // accumulators hold the transposed tile: lane l of tile (i, j) holds row
  // (its row base) + l % 32 and, in registers 4u .. 4u + 3, the four
  // consecutive columns 8u + 4 (l / 32) .. + 3 of the tile, written to LDS
  // as one 16-byte store (rows padded by 16 bytes, so a wave's 32 rows fall
  // in distinct banks).  The block tile goes through LDS one half of its
  // rows at a time; each thread then owns one chunk of 8 consecutive
  // columns, read back as 32 bytes and stored as 16 (bf16) or 32 (fp32)
  // contiguous bytes, so a wave's store covers 1-2 KB of a row.
  // Per-row values are looked up once per block into LDS (a load per row
  // in the store loop would expose a memory round trip): the token position
  // (RoPE) and, when appending, the element offset of the destination cache
  // row (-1: no valid slot).
  const EpiArgs& e = g.e;
  float* tile = reinterpret_cast<float*>(smem);
  int* row_pos = reinterpret_cast<int*>(smem + C::ROW_META);
  long long* row_dst = reinterpret_cast<long long*>(smem + C::ROW_META + C::BM * 4);
  const int mode = g.ksplit > 1 ? -1 : e.mode;  // -1: fp32 partial slice
  const bool rope_mode = mode == EPI_Q || mode == EPI_APPEND;
  if (rope_mode) {
    for (int r = threadIdx.x; r < C::BM; r += 256) {
      const int m = m0 + r;
      int pos = 0;
      long long dst = -1;
      if (m < e.M) {
        const int b = m / e.n_q, t = m - b * e.n_q;
        pos = (mode == EPI_Q) ? e.kv_len[b] - e.n_q + t : e.pos[b] + t;
        if (mode == EPI_APPEND) {
          if (e.paged) {
            if (pos < 0 || pos >= e.max_pages * e.page_size) {
              atomicOr(e.err, 1);
            } else {
              const int pg = e.page_table[(size_t)b * e.max_pages + pos / e.page_size];
              if (pg < 0 || pg >= e.n_pages)
                atomicOr(e.err, 2);
              else
                dst = ((long long)pg * e.page_size + pos % e.page_size) * e.row;
            }
          } else if (pos < 0 || pos >= e.s_max) {
            atomicOr(e.err, 1);
          } else {
            dst = ((long long)b * e.s_max + pos) * e.row;
          }
        }
      }
      row_pos[r] = pos;
      row_dst[r] = dst;
    }
  }
  constexpr int HM = C::BM / 2;       // rows per half: the rows of the waves with wm == half
  constexpr int CPR = C::BN / 8;      // 8-column chunks per block row
  constexpr int RSTEP = 256 / CPR;    // rows advanced per thread iteration
  const int cc = threadIdx.x % CPR, r_first = threadIdx.x / CPR;
  const int n = nt0 * 16 + 8 * cc;    // first column of this thread's chunk
  const bool qm = mode == EPI_Q;
  // Per column pair p of the chunk (rope modes): rotation frequency in
  // revolutions per position (0: not a rope column) and the destination
  // column (EPI_Q maps the column through its groups)
  double rev[4] = {0.0, 0.0, 0.0, 0.0};
  size_t dcol[4] = {0, 0, 0, 0};
  bool q_contig = false;  // the 8 destination columns are consecutive (EPI_Q)
  if (rope_mode) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int nn = n + 2 * p;
      if (nn >= e.N) break;
      const int f = nn % (qm ? e.qg_cols : e.row), rope0 = qm ? e.rope_from : e.d_latent;
      if (f >= rope0)
        rev[p] = exp2(-(2.0 * (double)((f - rope0) >> 1) / (double)e.d_rope) * log2((double)e.rope_base)) *
                 0.15915494309189535;
      dcol[p] = qm ? (size_t)e.q_off + (size_t)(nn / e.qg_cols) * e.qg_stride + f : (size_t)nn;
    }
    q_contig = qm && n + 7 < e.N && n / e.qg_cols == (n + 7) / e.qg_cols;
  }
  // (angle reduced to (-1/2, 1/2] revolutions in fp64, then the hardware
  // sine / cosine, whose argument is in revolutions)
  auto rotate = [&](int pos, double rv, float& x, float& y) {
    double a = (double)pos * rv;
    a -= rint(a);
    const float rf = (float)a;
    const float c = __builtin_amdgcn_cosf(rf), sn = __builtin_amdgcn_sinf(rf);
    const float a0 = x, a1 = y;
    x = a0 * c - a1 * sn;
    y = a0 * sn + a1 * c;
  };
  auto bf2 = [](float x, float y) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 t = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(uint32_t, t);
  };
  const int nlim = mode == -1 ? g.Np : e.N;  // columns that exist in the destination
  const int ldo = mode == -1 ? g.Np : e.N;   // its row stride (fp32 / bf16 plain outputs)
  const bool whole = n + 7 < nlim;           // all 8 columns of the chunk exist
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wm == half) {
#pragma unroll
      for (int i = 0; i < MTW; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int row = i * 32 + a_row;
            const int col = (wn * NTW + j) * 32 + 8 * u + 4 * a_hi;
            *reinterpret_cast<float4*>(tile + row * C::TS + col) =
                make_float4(acc[i][j][4 * u], acc[i][j][4 * u + 1], acc[i][j][4 * u + 2], acc[i][j][4 * u + 3]);
          }
    }
    __syncthreads();
    const int mlim = e.M - (m0 + half * HM);  // rows of this half that exist
    if (n < nlim) {
      for (int r = r_first; r < HM && r < mlim; r += RSTEP) {
        const float4 lo = *reinterpret_cast<const float4*>(tile + r * C::TS + 8 * cc);
        const float4 hi = *reinterpret_cast<const float4*>(tile + r * C::TS + 8 * cc + 4);
        float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        const int rb = half * HM + r;
        const size_t m = (size_t)(m0 + rb);
        if (mode == -1 || mode == EPI_F32) {
          float* y = (mode == -1 ? g.part + (size_t)ks * e.M * g.Np : reinterpret_cast<float*>(e.out)) + m * ldo + n;
          if (whole && (ldo & 3) == 0) {
            reinterpret_cast<float4*>(y)[0] = lo;
            reinterpret_cast<float4*>(y)[1] = hi;
          } else {
#pragma unroll
            for (int c = 0; c < 8; ++c)
              if (n + c < nlim) y[c] = v[c];
          }
        } else if (mode == EPI_STORE_T) {
          __bf16* y = reinterpret_cast<__bf16*>(e.out) + m * ldo + n;
          if (whole && (ldo & 7) == 0) {
            *reinterpret_cast<uint4*>(y) = make_uint4(bf2(v[0], v[1]), bf2(v[2], v[3]), bf2(v[4], v[5]), bf2(v[6], v[7]));
          } else {
#pragma unroll
            for (int c = 0; c < 8; ++c)
              if (n + c < nlim) y[c] = (__bf16)v[c];
          }
        } else {
          // EPI_Q / EPI_APPEND: rotate the rope pairs, then one 16-byte
          // store when the 8 destination columns are consecutive and
          // aligned, else a store per pair
          const int pos = row_pos[rb];
          __bf16* base;
          if (qm) {
            base = reinterpret_cast<__bf16*>(e.out) + m * e.q_ld;
          } else {
            const long long d = row_dst[rb];
            if (d < 0) continue;
            base = reinterpret_cast<__bf16*>(e.pool) + d;
          }
#pragma unroll
          for (int p = 0; p < 4; ++p)
            if (rev[p] != 0.0) rotate(pos, rev[p], v[2 * p], v[2 * p + 1]);
          const bool contig = qm ? q_contig : whole;
          if (contig && ((reinterpret_cast<uintptr_t>(base + dcol[0])) & 15) == 0) {
            *reinterpret_cast<uint4*>(base + dcol[0]) =
                make_uint4(bf2(v[0], v[1]), bf2(v[2], v[3]), bf2(v[4], v[5]), bf2(v[6], v[7]));
          } else {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const int nn = n + 2 * p;
              if (nn >= e.N) break;
              if (nn + 1 < e.N)
                *reinterpret_cast<uint32_t*>(base + dcol[p]) = bf2(v[2 * p], v[2 * p + 1]);
              else
                base[dcol[p]] = (__bf16)v[2 * p];
            }
          }
        }
      }
    }
    __syncthreads();
  }
}

// Sum of the K slices in slice order (deterministic), then the epilogue.
template <typename T>
__global__ __launch_bounds__(256) void splitk_epilogue_kernel(GemmArgs g) {
  const int pairs = g.Np / 2;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)g.e.M * pairs) return;
  const int m = (int)(idx / pairs);
  const int n = (int)(idx % pairs) * 2;
  if (!rows_needed(g, m, m + 1)) return;  // its slices were not written
  // slices are loaded CH at a time (one memory round trip per chunk) and
  // summed in slice order
  constexpr int CH = 8;
  float v0 = 0.f, v1 = 0.f;
  for (int base = 0; base < g.ksplit; base += CH) {
    float2 p[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j)
      p[j] = *reinterpret_cast<const float2*>(g.part + ((size_t)min(base + j, g.ksplit - 1) * g.e.M + m) * g.Np + n);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      if (base + j < g.ksplit) {
        v0 += p[j].x;
        v1 += p[j].y;
      }
    }
  }
  epi_pair<T>(g.e, m, n, v0, v1);
}

static int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Column-tile counts per wave instantiated for the decode path (16 tiles
// per wave, one wave per SIMD, measured slower than 10 in every split
// tried for the output projection; 1 only for one-tile A column groups).
static const int kDecodeNT[] = {1, 2, 4, 5, 8, 9, 10};

GemmPlan plan_gemm(int M, int K, int N, bool bf16, bool a_f32, int n_cu, int a_gtiles, int a_gstride,
                   size_t part_cap) {
  GemmPlan g{};
  g.M = M; g.K = K; g.N = N;
  g.a_gtiles = a_gtiles; g.a_gstride = a_gstride;
  // with A column groups, the n-tiles a wave (or tiled block) covers must
  // lie inside one group
  auto fits = [&](int tiles) { return a_gtiles == 0 || a_gtiles % tiles == 0; };
  g.KB = bf16 ? Mfma<__bf16>::KB : Mfma<float>::KB;
  g.Kp = ceil_div(K, g.KB) * g.KB;
  g.Np = ceil_div(N, 16) * 16;
  g.kblocks = g.Kp / g.KB;
  g.ntiles = g.Np / 16;
  const int mtiles = ceil_div(std::max(M, 1), 16);
  // Cost model for a weight-streaming kernel (units: 1 KB fragments): the
  // busiest CU streams ceil(blocks / CUs) blocks of (cols + A) * kb_per_split
  // fragments; fewer than two narrow blocks per CU leave too few loads in
  // flight (measured: wide blocks, 10 column tiles per wave, do best at one
  // block per CU);
  // every K slice beyond the first adds an fp32 partial round trip and a
  // second launch.
  double best = 1e300;
  long best_blocks = 0;
  auto consider = [&](int MT, int NT, int KSW) {
    if (!fits(NT) || (NT == 1 && a_gtiles != 1)) return;  // one-tile waves only for one-tile groups
    const int cols = (4 / KSW) * NT;
    const int gx = ceil_div(g.ntiles, cols), gy = ceil_div(mtiles, MT);
    const int ksmax = std::max(1, g.kblocks / (2 * KSW));
    for (int ks = 1; ks <= ksmax; ++ks) {
      const int kbs = ceil_div(g.kblocks, ks);
      if (ceil_div(g.kblocks, kbs) != ks) continue;
      if (ks > 1 && (double)ks * M * g.Np * 4.0 > (double)part_cap) continue;  // partials must fit
      const long blocks = (long)gx * gy * ks;
      // per k-block a block streams `cols` weight fragments; an fp32 A
      // operand (the output projection's, large and re-read by every column
      // block) adds its fragments too, once per wave covering the k-block
      const double a_kb = a_f32 ? 2.0 * MT * (KSW == 1 ? 4 : 1) : 0.0;
      double cost = (double)((blocks + n_cu - 1) / n_cu) * (cols + a_kb) * kbs;
      if (blocks < n_cu) cost *= 1.6;
      else if (blocks < 2L * n_cu && NT < 8) cost *= 1.25;  // narrow blocks: few loads in flight
      if (ks > 1) cost += 2.0 * ks * M * g.Np * 4.0 / 1024.0 / n_cu + 100.0;
      if (cost < best * 0.999 || (cost <= best * 1.001 && blocks < best_blocks)) {
        best = cost;
        best_blocks = blocks;
        g.MT = MT; g.NT = NT; g.KSW = KSW; g.gx = gx; g.gy = gy; g.ksplit = ks; g.kb_per_split = kbs;
      }
    }
  };
  g.tiled = 0;
  // 256 x 256 tiles (16 n-tiles per block), one k-block per stage
  const bool big = M >= 256 && g.ntiles >= 64 && fits(16);
  if (bf16 && M > 16 && (big || g.kblocks % 2 == 0) && fits(8)) {
    // LDS-tiled kernel: 64 x 128 tiles up to 64 rows, 128 x 128 up to 255,
    // 256 x 256 above (one k-block per stage, slices a multiple of a stage)
    g.tiled = 1;
    g.MT = big ? 4 : (M > 64 ? 2 : 1);
    g.NT = big ? 4 : 2;
    g.KSW = 1;
    const int skb = big ? 1 : 2;
    const int BM = 64 * g.MT, NTB = 4 * g.NT;
    g.gx = ceil_div(g.ntiles, NTB);
    g.gy = ceil_div(M, BM);
    const long blocks0 = (long)g.gx * g.gy;
    int ks = 1;
    if (big) {
      // 256 x 256 tiles (one block per CU) only split K when there are
      // fewer blocks than about 0.8 CUs
      const long want = (long)(0.8 * n_cu);
      if (blocks0 < want) ks = (int)std::min<long>((want + blocks0 - 1) / blocks0, std::max(1, g.kblocks / 4));
      while (ks > 1 && (double)ks * M * g.Np * 4.0 > (double)part_cap) --ks;  // partials must fit
    } else {
      // Blocks run in rounds of n_cu * occ resident blocks (occ from the
      // LDS ring); every round costs the streaming time of one block, a
      // sparse last round as much as a full one.  Each K slice adds an fp32
      // partial round trip.  A larger split must save 5% to be taken.
      const int lds = a_f32 ? (g.MT == 2 ? TiledCfg<float, 2, 2, 2>::LDS : TiledCfg<float, 1, 2, 2, 4>::LDS)
                            : (g.MT == 2 ? TiledCfg<__bf16, 2, 2, 2, 4>::LDS : TiledCfg<__bf16, 1, 2, 2, 4>::LDS);
      const long slots = (long)n_cu * std::max(1, std::min(2, 160 * 1024 / lds));
      const double kb_bytes = BM * 32.0 * (a_f32 ? 4 : 2) + NTB * 1024.0;  // one block, one k-block
      double best_cost = 1e300;
      for (int k = 1; k <= std::max(1, g.kblocks / (2 * skb)); ++k) {
        const int kbs = ceil_div(ceil_div(g.kblocks, k), skb) * skb;
        if (ceil_div(g.kblocks, kbs) != k) continue;
        if (k > 1 && (double)k * M * g.Np * 4.0 > (double)part_cap) continue;  // partials must fit
        const long rounds = (blocks0 * k + slots - 1) / slots;
        double cost = (double)rounds * kbs;  // k-blocks streamed by the busiest slot
        // (partials: written, read back by a second launch; weighted double)
        if (k > 1) cost += 2.0 * (double)k * M * g.Np * 8.0 / ((double)slots * kb_bytes);
        if (cost < best_cost * 0.95) {
          best_cost = cost;
          ks = k;
        }
      }
    }
    int kbs = ceil_div(g.kblocks, ks);
    kbs = ceil_div(kbs, skb) * skb;
    g.kb_per_split = kbs;
    g.ksplit = ceil_div(g.kblocks, kbs);
  } else if (mtiles <= 4) {
    // up to 64 rows: the block's waves split K; the LDS tile (4 x rows x
    // cols fp32) stays within 64 KB
    const int MT = mtiles == 1 ? 1 : (mtiles == 2 ? 2 : 4);
    for (int nt : kDecodeNT)
      if (MT * nt <= 16) consider(MT, nt, 4);
  } else {
    consider(4, 4, 1);
  }
  if (!g.tiled && best == 1e300) g.tiled = -1;  // no configuration fits the A column groups
  g.part_bytes = g.ksplit > 1 ? (size_t)g.ksplit * (size_t)M * (size_t)g.Np * sizeof(float) : 0;
  return g;
}

template <typename T, typename TA, int MT, int NT, int KSW>
static hipError_t launch_gemm_t(const GemmPlan& g, const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((gemm_kernel<T, TA, MT, NT, KSW>), dim3(g.gx, g.gy, g.ksplit), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || g.ksplit == 1) return e;
  const long total = (long)g.M * (g.Np / 2);
  hipLaunchKernelGGL(splitk_epilogue_kernel<T>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename TA, int MTW, int NTW, int SKB, int NS = 3, bool WNT = false>
static hipError_t launch_tiled_t(const GemmPlan& g, const GemmArgs& a, hipStream_t s) {
  using C = TiledCfg<TA, MTW, NTW, SKB, NS, WNT>;
  // the pipelined ring (four slots or more) runs whole stages only
  if (NS >= 4 && (g.kblocks % SKB != 0 || g.kb_per_split % SKB != 0)) return hipErrorInvalidValue;
  if (hipError_t e = ensure_lds_limit<&gemm_tiled_kernel<TA, MTW, NTW, SKB, NS, WNT>>(C::LDS); e != hipSuccess)
    return e;
  hipLaunchKernelGGL((gemm_tiled_kernel<TA, MTW, NTW, SKB, NS, WNT>), dim3(g.gy, g.gx, g.ksplit), dim3(256), C::LDS, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || g.ksplit == 1) return e;
  const long total = (long)g.M * (g.Np / 2);
  hipLaunchKernelGGL(splitk_epilogue_kernel<__bf16>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename TA>
static hipError_t launch_tiled_sel(const GemmPlan& g, const GemmArgs& a, hipStream_t s) {
  // Four ring slots (the pipelined loop) wherever they fit in LDS: every
  // bf16-A tile and the 64-row fp32-A tile; the larger fp32-A tiles keep
  // three slots and the read-then-compute loop.
  // With bf16 A and one row block the weights are read once: non-temporal
  // weight DMA (measured slower with the fp32-A kernel, so not used there)
  if constexpr (sizeof(TA) == 4) {
    if (g.MT == 4) return launch_tiled_t<TA, 4, 4, 1>(g, a, s);
    return g.MT == 2 ? launch_tiled_t<TA, 2, 2, 2>(g, a, s) : launch_tiled_t<TA, 1, 2, 2, 4>(g, a, s);
  } else {
    if (g.MT == 4) return launch_tiled_t<TA, 4, 4, 1, 4>(g, a, s);
    // 64-row blocks over an unsplit short K: the 3-slot ring, which fits
    // two blocks per CU (the fill and the epilogue of one hide under the
    // other; measured better for a 1536-deep query projection, worse for
    // the long output-projection slices)
    const bool short_slice = g.MT == 1 && g.ksplit == 1 && g.kb_per_split <= kShortSlice;
    if (g.gy == 1) {
      if (short_slice) return launch_tiled_t<TA, 1, 2, 2, 3, true>(g, a, s);
      return g.MT == 2 ? launch_tiled_t<TA, 2, 2, 2, 4, true>(g, a, s) : launch_tiled_t<TA, 1, 2, 2, 4, true>(g, a, s);
    }
    if (short_slice) return launch_tiled_t<TA, 1, 2, 2, 3>(g, a, s);
    return g.MT == 2 ? launch_tiled_t<TA, 2, 2, 2, 4>(g, a, s) : launch_tiled_t<TA, 1, 2, 2, 4>(g, a, s);
  }
}

template <typename T, typename TA>
static hipError_t launch_gemm_sel(const GemmPlan& g, const GemmArgs& a, hipStream_t s) {
  if (g.KSW == 4 && g.MT == 1) {
    switch (g.NT) {
      case 1: return launch_gemm_t<T, TA, 1, 1, 4>(g, a, s);
      case 2: return launch_gemm_t<T, TA, 1, 2, 4>(g, a, s);
      case 4: return launch_gemm_t<T, TA, 1, 4, 4>(g, a, s);
      case 5: return launch_gemm_t<T, TA, 1, 5, 4>(g, a, s);
      case 8: return launch_gemm_t<T, TA, 1, 8, 4>(g, a, s);
      case 9: return launch_gemm_t<T, TA, 1, 9, 4>(g, a, s);
      default: return launch_gemm_t<T, TA, 1, 10, 4>(g, a, s);
    }
  }
  if (g.KSW == 4 && g.MT == 2) {
    switch (g.NT) {
      case 2: return launch_gemm_t<T, TA, 2, 2, 4>(g, a, s);
      case 4: return launch_gemm_t<T, TA, 2, 4, 4>(g, a, s);
      case 5: return launch_gemm_t<T, TA, 2, 5, 4>(g, a, s);
      default: return launch_gemm_t<T, TA, 2, 8, 4>(g, a, s);
    }
  }
  if (g.KSW == 4) {
    return g.NT == 2 ? launch_gemm_t<T, TA, 4, 2, 4>(g, a, s) : launch_gemm_t<T, TA, 4, 4, 4>(g, a, s);
  }
  return launch_gemm_t<T, TA, 4, 4, 1>(g, a, s);
}

// fp32 -> bf16, rounded to nearest even: the rounding the fp32-A kernels
// apply to each A fragment, so a GEMM over the converted copy is the same
// computation.  8 values (32 B in, 16 B out) per thread and step.
__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float* __restrict__ x, __bf16* __restrict__ y, long n8) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n8; i += (long)gridDim.x * 256) {
    const float4 u = reinterpret_cast<const float4*>(x)[2 * i], w = reinterpret_cast<const float4*>(x)[2 * i + 1];
    bf16x8 v;
    v[0] = (__bf16)u.x; v[1] = (__bf16)u.y; v[2] = (__bf16)u.z; v[3] = (__bf16)u.w;
    v[4] = (__bf16)w.x; v[5] = (__bf16)w.y; v[6] = (__bf16)w.z; v[7] = (__bf16)w.w;
    reinterpret_cast<bf16x8*>(y)[i] = v;
  }
}

hipError_t launch_f32_to_bf16(const float* x, void* y, size_t n, hipStream_t s) {
  if (n % 8 || (reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) % 16) return hipErrorInvalidValue;
  if (n == 0) return hipSuccess;
  const long n8 = (long)(n / 8);
  const unsigned blocks = (unsigned)std::min<long>((n8 + 255) / 256, 4096L);
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3(blocks), dim3(256), 0, s, x, reinterpret_cast<__bf16*>(y), n8);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmPlan& g, bool bf16, bool a_f32, const void* A, int lda, const void* Wp, float* part,
                       const EpiArgs& e, hipStream_t s, const int32_t* row_len, int row_group) {
  if (g.tiled < 0) return hipErrorInvalidConfiguration;
  if (row_len && row_group <= 0) return hipErrorInvalidValue;
  GemmArgs a{};
  a.row_len = row_len;
  a.row_group = row_group;
  a.A = A;
  a.lda = lda;
  a.Wp = Wp;
  a.kblocks = g.kblocks;
  a.ntiles = g.ntiles;
  a.Np = g.Np;
  a.ksplit = g.ksplit;
  a.kb_per_split = g.kb_per_split;
  a.a_gtiles = g.a_gtiles;
  a.a_gstride = g.a_gstride;
  a.part = part;
  a.e = e;
  a.e.M = g.M;
  a.e.N = g.N;
  if (bf16 && g.tiled) return a_f32 ? launch_tiled_sel<float>(g, a, s) : launch_tiled_sel<__bf16>(g, a, s);
  if (bf16) {
    return a_f32 ? launch_gemm_sel<__bf16, float>(g, a, s) : launch_gemm_sel<__bf16, __bf16>(g, a, s);
  }
  return launch_gemm_sel<float, float>(g, a, s);
}

// --------------------------------------------------------------------------
// Factored query projection for up to 16 rows in one launch (after c_Q).
// Block (head h, half j): phase A computes q_nope[h] = c_Q W_UQ[h] (all
// 128 columns) together with half j of c_Q W_QR[h] (32 of 64 columns), the
// four waves splitting K = d_q_latent and summing through LDS; q_nope is
// rounded to bf16 into LDS (the rounding the unfused form applies when it
// stores q_nope) and the q_pe half is rotated and stored.  Phase B computes
// half j of q_lat[h] = q_nope[h] W_UK[h]^T (256 of 512 columns, K = 128),
// each wave owning four 16-column tiles, staged through LDS into 16-byte
// stores.  The two halves of a head are placed on one XCD (physical block
// b runs on XCD b % 8), so the second read of W_UQ[h] is served by its L2.
// --------------------------------------------------------------------------
constexpr int kQfDn = 128, kQfDr = 64, kQfDl = 512;

bool q_fused_supported(bool bf16, int M, int d_nope, int d_rope, int d_latent, int d_q_latent) {
  return bf16 && M >= 1 && M <= 16 && d_nope == kQfDn && d_rope == kQfDr && d_latent == kQfDl &&
         d_q_latent > 0 && d_q_latent % 32 == 0;
}

__global__ __launch_bounds__(256) void q_fused_kernel(QFusedArgs a) {
  using F = Mfma<__bf16>;
  using frag = F::frag;
  constexpr int NTA = kQfDn / 16 + kQfDr / 32;  // phase A column tiles: 8 of q_nope, 2 of q_pe
  constexpr int NTB = kQfDl / 2 / 16 / 4;       // phase B column tiles per wave
  constexpr int KBB = kQfDn / 32;               // phase B k-blocks
  constexpr int QS = kQfDn + 8;                 // q_nope row stride in LDS (bf16, padded)
  constexpr int OS = kQfDl / 2 + 4;             // phase B staging row stride (fp32)
  constexpr int R = kQfDl + kQfDr;              // q row width per head
  __shared__ float red[4][16][NTA * 16];
  __shared__ __attribute__((aligned(16))) __bf16 qn_s[16 * QS];
  static_assert(16 * OS <= 4 * 16 * NTA * 16, "phase B staging fits the reduction buffer");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int bid = blockIdx.x, xcd = bid & 7, slot = bid >> 3;
  const int j = slot & 1, h = xcd + 8 * (slot >> 1);
  if (h >= a.H) return;
  const int M = a.M;
  const int row = lane & 15, kq = 8 * (lane >> 4);
  const bool rv = row < M;

  // ---- phase A: K split over the waves ------------------------------------
  const int KBA = a.d_q_latent / 32;
  const int per = (KBA + 3) / 4;
  const int kb0 = min(wave * per, KBA), kb1 = min(kb0 + per, KBA);
  const __bf16* ap = reinterpret_cast<const __bf16*>(a.cq) + (size_t)(rv ? row : 0) * a.d_q_latent + kq;
  const size_t ntu = (size_t)a.H * (kQfDn / 16), ntr = (size_t)a.H * (kQfDr / 16);
  const __bf16* wu = reinterpret_cast<const __bf16*>(a.w_uq) + (size_t)h * (kQfDn / 16) * 512 + lane * 8;
  const __bf16* wr = reinterpret_cast<const __bf16*>(a.w_qr) + ((size_t)h * (kQfDr / 16) + 2 * j) * 512 + lane * 8;
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  auto wload = [](const __bf16* p) {
    return __builtin_bit_cast(frag, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
  };
  auto load = [&](frag (&bf)[NTA], frag& af, int kb) {
#pragma unroll
    for (int t = 0; t < kQfDn / 16; ++t) bf[t] = wload(wu + ((size_t)kb * ntu + t) * 512);
#pragma unroll
    for (int t = 0; t < kQfDr / 32; ++t) bf[kQfDn / 16 + t] = wload(wr + ((size_t)kb * ntr + t) * 512);
    af = rv ? load_frag<__bf16>(ap + kb * 32) : F::zero();
  };
  f32x4 acc[NTA];
#pragma unroll
  for (int t = 0; t < NTA; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](const frag (&bf)[NTA], const frag& af) {
#pragma unroll
    for (int t = 0; t < NTA; ++t) acc[t] = F::mma(af, bf[t], acc[t]);
  };
  {
    // two register buffers: the loads of k-block kb + 1 are in flight
    // while the MFMAs of kb run
    frag b0[NTA], b1[NTA], a0, a1;
    int kb = kb0;
    if (kb < kb1) load(b0, a0, kb);
    while (kb < kb1) {
      if (kb + 1 < kb1) load(b1, a1, kb + 1);
      mma(b0, a0);
      if (++kb >= kb1) break;
      if (kb + 1 < kb1) load(b0, a0, kb + 1);
      mma(b1, a1);
      ++kb;
    }
  }
#pragma unroll
  for (int t = 0; t < NTA; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][4 * (lane >> 4) + i][t * 16 + (lane & 15)] = acc[t][i];
  // phase B weights do not depend on q_nope: in flight across the reduction
  const size_t ntk = (size_t)a.H * (kQfDl / 16);
  const __bf16* wk = reinterpret_cast<const __bf16*>(a.w_ukt) +
                     ((size_t)h * (kQfDl / 16) + j * (kQfDl / 32) + wave * NTB) * 512 + lane * 8;
  frag wb[KBB][NTB];
#pragma unroll
  for (int kb = 0; kb < KBB; ++kb)
#pragma unroll
    for (int t = 0; t < NTB; ++t) wb[kb][t] = wload(wk + ((size_t)kb * ntk + t) * 512);
  __syncthreads();
  // sums in wave order; q_nope -> bf16 LDS rows, q_pe pairs rotated and stored
  for (int e = threadIdx.x; e < 16 * NTA * 8; e += 256) {
    const int r = e / (NTA * 8), c = (e % (NTA * 8)) * 2;
    float v0 = red[0][r][c], v1 = red[0][r][c + 1];
#pragma unroll
    for (int w2 = 1; w2 < 4; ++w2) {
      v0 += red[w2][r][c];
      v1 += red[w2][r][c + 1];
    }
    if (c < kQfDn) {
      qn_s[r * QS + c] = (__bf16)v0;
      qn_s[r * QS + c + 1] = (__bf16)v1;
    } else if (r < M) {
      const int f = 32 * j + (c - kQfDn);  // column within q_pe (even)
      const int b = r / a.n_q, t = r - b * a.n_q;
      float cs, sn;
      rope_cos_sin(a.kv_len[b] - a.n_q + t, f >> 1, kQfDr, a.rope_base, &cs, &sn);
      __bf16* y = reinterpret_cast<__bf16*>(a.q) + ((size_t)r * a.H + h) * R + kQfDl + f;
      y[0] = (__bf16)(v0 * cs - v1 * sn);
      y[1] = (__bf16)(v0 * sn + v1 * cs);
    }
  }
  __syncthreads();

  // ---- phase B: half j of q_nope[h] W_UK[h]^T -----------------------------
  f32x4 accb[NTB];
#pragma unroll
  for (int t = 0; t < NTB; ++t) accb[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < KBB; ++kb) {
    const frag af = *reinterpret_cast<const frag*>(qn_s + row * QS + kb * 32 + kq);
#pragma unroll
    for (int t = 0; t < NTB; ++t) accb[t] = F::mma(af, wb[kb][t], accb[t]);
  }
  float* ost = &red[0][0][0];  // [16][OS] fp32 (the reduction buffer is free)
#pragma unroll
  for (int t = 0; t < NTB; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) ost[(4 * (lane >> 4) + i) * OS + (wave * NTB + t) * 16 + (lane & 15)] = accb[t][i];
  __syncthreads();
  for (int e = threadIdx.x; e < 16 * (kQfDl / 2 / 8); e += 256) {
    const int r = e / (kQfDl / 2 / 8), ch = e % (kQfDl / 2 / 8);
    if (r >= M) continue;
    const float4 lo = *reinterpret_cast<const float4*>(ost + r * OS + 8 * ch);
    const float4 hi = *reinterpret_cast<const float4*>(ost + r * OS + 8 * ch + 4);
    bf16x8 v;
    v[0] = (__bf16)lo.x; v[1] = (__bf16)lo.y; v[2] = (__bf16)lo.z; v[3] = (__bf16)lo.w;
    v[4] = (__bf16)hi.x; v[5] = (__bf16)hi.y; v[6] = (__bf16)hi.z; v[7] = (__bf16)hi.w;
    *reinterpret_cast<bf16x8*>(reinterpret_cast<__bf16*>(a.q) + ((size_t)r * a.H + h) * R + j * (kQfDl / 2) + 8 * ch) = v;
  }
}

hipError_t launch_q_fused(const QFusedArgs& a, hipStream_t s) {
  if (a.M < 1 || a.M > 16 || a.H < 1 || a.d_q_latent % 32 != 0) return hipErrorInvalidValue;
  // two blocks per head, heads dealt 8 at a time over the XCDs
  const int blocks = 16 * ((a.H + 7) / 8);
  hipLaunchKernelGGL(q_fused_kernel, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// Weight absorption (one-time).
//
// Packed outputs (K x N logical, see mla_common.h):
//   P_KV : K = d_model, N = R            [W_DKV | W_KR]
//   P_DQ : K = d_model, N = d_LQ         W_DQ
//   P_QC : K = d_LQ,    N = H * R        per head h: [W_UQ[h] W_UK[h]^T | W_QR[h]]
//   P_O  : K = H * d_L, N = d_model      row h*d_L + c: (W_UV[h] W_O[h])[c]
// --------------------------------------------------------------------------
// PACK_PLAIN: element (k, n) of a row-major source with row stride `ld`;
// PACK_UKT: W_UK[c, h, k] at (k, n = h*d_L + c) (the factored key weight,
// transposed per head).
enum PackMode { PACK_KV = 0, PACK_DQ = 1, PACK_QC = 2, PACK_O = 3, PACK_PLAIN = 4, PACK_UKT = 5 };

template <typename T>
__global__ __launch_bounds__(256) void pack_kernel(AbsorbArgs a, int mode, int K, int N, int Kp, int Np, T* out,
                                                   const T* plain, long ld) {
  using F = Mfma<T>;
  const size_t total = (size_t)Kp * Np;
  const size_t p = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= total) return;
  // invert packed_index: p = ((kb * NTT + nt) * 64 + lane) * KPL + j
  const int j = (int)(p % F::KPL);
  const size_t q = p / F::KPL;
  const int lane = (int)(q % 64);
  const size_t r = q / 64;
  const int ntt = Np / 16;
  const int nt = (int)(r % ntt);
  const int kb = (int)(r / ntt);
  const int n = nt * 16 + (lane & 15);
  const int k = kb * F::KB + (lane >> 4) * F::KPL + j;
  const T* src = nullptr;
  size_t off = 0;
  bool zero = (k >= K) || (n >= N);
  const int R = a.d_latent + a.d_rope;
  if (!zero) {
    switch (mode) {
      case PACK_KV:
        if (n < a.d_latent) { src = (const T*)a.W_DKV; off = (size_t)k * a.d_latent + n; }
        else { src = (const T*)a.W_KR; off = (size_t)k * a.d_rope + (n - a.d_latent); }
        break;
      case PACK_DQ:
        src = (const T*)a.W_DQ; off = (size_t)k * a.d_q_latent + n;
        break;
      case PACK_QC: {
        const int h = n / R, f = n % R;
        if (f < a.d_latent) return;  // written by the product kernel
        src = (const T*)a.W_QR; off = ((size_t)k * a.H + h) * a.d_rope + (f - a.d_latent);
        break;
      }
      case PACK_PLAIN:
        src = plain; off = (size_t)k * ld + n;
        break;
      case PACK_UKT: {
        const int h = n / a.d_latent, c = n % a.d_latent;
        src = (const T*)a.W_UK; off = ((size_t)c * a.H + h) * a.d_nope + k;
        break;
      }
      default:
        return;  // PACK_O: product kernel writes every in-range element
    }
  }
  out[p] = zero ? from_f32<T>(0.f) : src[off];
}

// out(h, r, c) = sum_d A(h, r, d) * B(h, d, c), fp32 accumulate on MFMA.
// A(h, r, d) = Ab[h*a_hs + r*a_rs + d*a_ds]; B(h, d, c) = Bb[h*b_hs + d*b_ds + c*b_cs].
// Written to packed (k = h*k_hs + r, n = h*n_hs + c).
struct ProdArgs {
  const void* Ab; long a_hs, a_rs, a_ds;
  const void* Bb; long b_hs, b_ds, b_cs;
  int H, rows, cols, kd;
  int k_hs, n_hs, Np;   // Np: padded column count of the packed output
  void* out;
};

template <typename T>
__global__ __launch_bounds__(256) void absorb_product_kernel(ProdArgs p) {
  using F = Mfma<T>;
  const int lane = threadIdx.x & 63;
  const int rt_n = (p.rows + 15) / 16, ct_n = (p.cols + 15) / 16;
  const long tile = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= (long)p.H * rt_n * ct_n) return;
  const int ct = (int)(tile % ct_n);
  const int rt = (int)((tile / ct_n) % rt_n);
  const int h = (int)(tile / ((long)ct_n * rt_n));
  const T* Ab = reinterpret_cast<const T*>(p.Ab) + (long)h * p.a_hs;
  const T* Bb = reinterpret_cast<const T*>(p.Bb) + (long)h * p.b_hs;
  const int r = rt * 16 + (lane & 15), c = ct * 16 + (lane & 15);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int d0 = 0; d0 < p.kd; d0 += F::KB) {
    typename F::frag af, bfr;
    if constexpr (F::KPL == 1) {
      const int d = d0 + (lane >> 4);
      af = (r < p.rows && d < p.kd) ? (float)Ab[(long)r * p.a_rs + (long)d * p.a_ds] : 0.f;
      bfr = (c < p.cols && d < p.kd) ? (float)Bb[(long)d * p.b_ds + (long)c * p.b_cs] : 0.f;
    } else {
#pragma unroll
      for (int j = 0; j < F::KPL; ++j) {
        const int d = d0 + (lane >> 4) * F::KPL + j;
        af[j] = (r < p.rows && d < p.kd) ? Ab[(long)r * p.a_rs + (long)d * p.a_ds] : (T)0.f;
        bfr[j] = (c < p.cols && d < p.kd) ? Bb[(long)d * p.b_ds + (long)c * p.b_cs] : (T)0.f;
      }
    }
    acc = F::mma(af, bfr, acc);
  }
  T* out = reinterpret_cast<T*>(p.out);
  const int cc = ct * 16 + (lane & 15);
  if (cc >= p.cols) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = rt * 16 + 4 * (lane >> 4) + i;
    if (rr < p.rows)
      out[packed_index(h * p.k_hs + rr, h * p.n_hs + cc, p.Np, F::KB, F::KPL)] = from_f32<T>(acc[i]);
  }
}

// Per-head products for bf16 weights with K = 128 and 64-divisible sides, one
// 64 x 64 output tile of one head per work-group: A (rows x 128, k
// contiguous) and B (read as columns x 128, k contiguous in LDS: W_UK[h]
// is stored that way, W_O[h] is stored k-major and transposed on its way
// into LDS) are staged with 16-byte loads; each wave takes 16 rows and
// four 16-column tiles through the same 16x16x32 MFMAs, in the same k
// order, as absorb_product_kernel, so the products are bit-identical; the
// tile goes back through LDS column-major and leaves as whole 1 KB packed
// fragments (16 bytes per lane).
constexpr int kAbK = 128, kAbT = 64, kAbS = kAbK + 8;  // LDS row stride (bf16), padded

// Shapes, strides (in elements) and pointers the tiled kernel's 16-byte
// accesses need; anything else takes absorb_product_kernel.
static bool absorb_tiled_ok(const ProdArgs& p, bool b_kmajor) {
  auto a16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  const bool b_ok = b_kmajor ? (p.b_ds % 8 == 0 && p.b_cs == 1) : (p.b_cs % 8 == 0 && p.b_ds == 1);
  return p.kd == kAbK && p.rows % kAbT == 0 && p.cols % kAbT == 0 && p.k_hs % 32 == 0 && p.n_hs % 16 == 0 &&
         p.a_ds == 1 && p.a_rs % 8 == 0 && p.a_hs % 8 == 0 && p.b_hs % 8 == 0 && b_ok && a16(p.Ab) && a16(p.Bb) &&
         a16(p.out);
}

template <bool B_KMAJOR>
__global__ __launch_bounds__(256) void absorb_tile_kernel(ProdArgs p) {
  using F = Mfma<__bf16>;
  __shared__ __attribute__((aligned(16))) __bf16 as[kAbT * kAbS];
  __shared__ __attribute__((aligned(16))) __bf16 bs[kAbT * kAbS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ct_n = p.cols / kAbT, rt_n = p.rows / kAbT;
  const int ct = blockIdx.x % ct_n, rt = (blockIdx.x / ct_n) % rt_n, h = blockIdx.x / (ct_n * rt_n);
  const int r0 = rt * kAbT, c0 = ct * kAbT;
  const __bf16* Ab = reinterpret_cast<const __bf16*>(p.Ab) + (long)h * p.a_hs;
  const __bf16* Bb = reinterpret_cast<const __bf16*>(p.Bb) + (long)h * p.b_hs;
  // A rows r0.. (k contiguous): 64 rows x 16 chunks of 8
  for (int q = tid; q < kAbT * (kAbK / 8); q += 256) {
    const int r = q / (kAbK / 8), ch = q % (kAbK / 8);
    *reinterpret_cast<bf16x8*>(as + r * kAbS + 8 * ch) =
        *reinterpret_cast<const bf16x8*>(Ab + (long)(r0 + r) * p.a_rs + 8 * ch);
  }
  if constexpr (!B_KMAJOR) {
    // B column c at Bb[c * b_cs + d] (k contiguous)
    for (int q = tid; q < kAbT * (kAbK / 8); q += 256) {
      const int c = q / (kAbK / 8), ch = q % (kAbK / 8);
      *reinterpret_cast<bf16x8*>(bs + c * kAbS + 8 * ch) =
          *reinterpret_cast<const bf16x8*>(Bb + (long)(c0 + c) * p.b_cs + 8 * ch);
    }
  } else {
    // B row d at Bb[d * b_ds + c] (columns contiguous): transposed into LDS
    for (int q = tid; q < kAbK * (kAbT / 8); q += 256) {
      const int d = q / (kAbT / 8), cc = q % (kAbT / 8);
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(Bb + (long)d * p.b_ds + c0 + 8 * cc);
#pragma unroll
      for (int j = 0; j < 8; ++j) bs[(8 * cc + j) * kAbS + d] = v[j];
    }
  }
  __syncthreads();
  f32x4 acc[kAbT / 16];
#pragma unroll
  for (int t = 0; t < kAbT / 16; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int rl = 16 * wave + (lane & 15), kq = 8 * (lane >> 4);
#pragma unroll
  for (int ks = 0; ks < kAbK / 32; ++ks) {
    const bf16x8 af = *reinterpret_cast<const bf16x8*>(as + rl * kAbS + 32 * ks + kq);
#pragma unroll
    for (int t = 0; t < kAbT / 16; ++t) {
      const bf16x8 bf = *reinterpret_cast<const bf16x8*>(bs + (16 * t + (lane & 15)) * kAbS + 32 * ks + kq);
      acc[t] = F::mma(af, bf, acc[t]);
    }
  }
  __syncthreads();
  // column-major tile in the A buffer: element (r, c) at as[c * kAbS + r]
#pragma unroll
  for (int t = 0; t < kAbT / 16; ++t) {
    __bf16 v4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v4[i] = (__bf16)acc[t][i];
    *reinterpret_cast<uint2*>(as + (16 * t + (lane & 15)) * kAbS + 16 * wave + 4 * (lane >> 4)) =
        *reinterpret_cast<const uint2*>(v4);
  }
  __syncthreads();
  // packed fragments (k-block kb, column tile nt): lane l holds rows
  // 32 kb + 8 (l / 16) .. + 7 of column 16 nt + l % 16
  __bf16* out = reinterpret_cast<__bf16*>(p.out);
  const long kb0 = ((long)h * p.k_hs + r0) / 32, nt0 = ((long)h * p.n_hs + c0) / 16;
  for (int f = wave; f < (kAbT / 32) * (kAbT / 16); f += 4) {
    const int kb = f / (kAbT / 16), nt = f % (kAbT / 16);
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(as + (16 * nt + (lane & 15)) * kAbS + 32 * kb + kq);
    *reinterpret_cast<bf16x8*>(out + (((kb0 + kb) * (long)(p.Np / 16) + nt0 + nt) * 64 + lane) * 8) = v;
  }
}

template <typename T>
static hipError_t launch_product(const ProdArgs& p, bool b_kmajor, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    if (absorb_tiled_ok(p, b_kmajor)) {
      const unsigned blocks = (unsigned)((long)p.H * (p.rows / kAbT) * (p.cols / kAbT));
      if (b_kmajor)
        hipLaunchKernelGGL(absorb_tile_kernel<true>, dim3(blocks), dim3(256), 0, s, p);
      else
        hipLaunchKernelGGL(absorb_tile_kernel<false>, dim3(blocks), dim3(256), 0, s, p);
      return hipGetLastError();
    }
  }
  const long tiles = (long)p.H * ceil_div(p.rows, 16) * ceil_div(p.cols, 16);
  hipLaunchKernelGGL(absorb_product_kernel<T>, dim3((unsigned)((tiles + 3) / 4)), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <typename T>
static hipError_t pack_one(const AbsorbArgs& a, int mode, int K, int N, void* out, const void* plain, long ld,
                           hipStream_t s) {
  using F = Mfma<T>;
  const int Kp = ceil_div(K, F::KB) * F::KB, Np = ceil_div(N, 16) * 16;
  const size_t total = (size_t)Kp * Np;
  hipLaunchKernelGGL(pack_kernel<T>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a, mode, K, N, Kp, Np,
                     reinterpret_cast<T*>(out), reinterpret_cast<const T*>(plain), ld);
  return hipGetLastError();
}

// Factored form: the raw factors, repacked (no products).
template <typename T>
static hipError_t pack_factored_t(const AbsorbArgs& a, hipStream_t s) {
  const int R = a.d_latent + a.d_rope;
  hipError_t e;
  if ((e = pack_one<T>(a, PACK_KV, a.d_model, R, a.P_KV, nullptr, 0, s)) != hipSuccess) return e;
  if ((e = pack_one<T>(a, PACK_DQ, a.d_model, a.d_q_latent, a.P_DQ, nullptr, 0, s)) != hipSuccess) return e;
  if ((e = pack_one<T>(a, PACK_PLAIN, a.d_q_latent, a.H * a.d_nope, a.P_UQ, a.W_UQ, (long)a.H * a.d_nope, s)))
    return e;
  if ((e = pack_one<T>(a, PACK_PLAIN, a.d_q_latent, a.H * a.d_rope, a.P_QR, a.W_QR, (long)a.H * a.d_rope, s)))
    return e;
  if ((e = pack_one<T>(a, PACK_UKT, a.d_nope, a.H * a.d_latent, a.P_UKT, nullptr, 0, s)) != hipSuccess) return e;
  if ((e = pack_one<T>(a, PACK_PLAIN, a.d_latent, a.H * a.d_nope, a.P_UK, a.W_UK, (long)a.H * a.d_nope, s)))
    return e;
  if ((e = pack_one<T>(a, PACK_PLAIN, a.d_latent, a.H * a.d_v, a.P_UV, a.W_UV, (long)a.H * a.d_v, s)))
    return e;
  return pack_one<T>(a, PACK_PLAIN, a.H * a.d_v, a.d_model, a.P_WO, a.W_O, (long)a.d_model, s);
}

template <typename T>
static hipError_t absorb_t(const AbsorbArgs& a, hipStream_t s) {
  using F = Mfma<T>;
  const int R = a.d_latent + a.d_rope;
  struct M { int mode, K, N; void* out; } mats[4] = {
      {PACK_KV, a.d_model, R, a.P_KV},
      {PACK_DQ, a.d_model, a.d_q_latent, a.P_DQ},
      {PACK_QC, a.d_q_latent, a.H * R, a.P_QC},
      {PACK_O, a.H * a.d_latent, a.d_model, a.P_O},
  };
  for (auto& mt : mats) {
    const int Kp = ceil_div(mt.K, F::KB) * F::KB, Np = ceil_div(mt.N, 16) * 16;
    const size_t total = (size_t)Kp * Np;
    // PACK_O only has padding to fill; the product kernel writes the rest.
    if (mt.mode == PACK_O && Kp == mt.K && Np == mt.N) continue;
    hipLaunchKernelGGL(pack_kernel<T>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a, mt.mode,
                       mt.K, mt.N, Kp, Np, reinterpret_cast<T*>(mt.out), nullptr, 0L);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // W_UQK[h] = W_UQ[h] W_UK[h]^T : rows d_LQ, cols d_L, reduce over d_nope
  {
    ProdArgs p{};
    p.Ab = a.W_UQ; p.a_hs = a.d_nope; p.a_rs = (long)a.H * a.d_nope; p.a_ds = 1;
    p.Bb = a.W_UK; p.b_hs = a.d_nope; p.b_ds = 1; p.b_cs = (long)a.H * a.d_nope;
    p.H = a.H; p.rows = a.d_q_latent; p.cols = a.d_latent; p.kd = a.d_nope;
    p.k_hs = 0; p.n_hs = R; p.Np = ceil_div(a.H * R, 16) * 16; p.out = a.P_QC;
    hipError_t err = launch_product<T>(p, false, s);
    if (err != hipSuccess) return err;
  }
  // W_UVO[h] = W_UV[h] W_O[h] : rows d_L, cols d_model, reduce over d_v
  {
    ProdArgs p{};
    p.Ab = a.W_UV; p.a_hs = a.d_v; p.a_rs = (long)a.H * a.d_v; p.a_ds = 1;
    p.Bb = a.W_O; p.b_hs = (long)a.d_v * a.d_model; p.b_ds = a.d_model; p.b_cs = 1;
    p.H = a.H; p.rows = a.d_latent; p.cols = a.d_model; p.kd = a.d_v;
    p.k_hs = a.d_latent; p.n_hs = 0; p.Np = ceil_div(a.d_model, 16) * 16; p.out = a.P_O;
    hipError_t err = launch_product<T>(p, true, s);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t launch_absorb(const AbsorbArgs& a, bool bf16, hipStream_t s) {
  if (a.factored) return bf16 ? pack_factored_t<__bf16>(a, s) : pack_factored_t<float>(a, s);
  return bf16 ? absorb_t<__bf16>(a, s) : absorb_t<float>(a, s);
}

}  // namespace mla
