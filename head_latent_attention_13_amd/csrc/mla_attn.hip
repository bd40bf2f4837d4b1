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
// Inside a work-group (8 waves for 128 heads):
//   * 32-token tiles are DMA'd global -> LDS (global_load_lds, 16 B/lane)
//     through a 3-stage ring, with a 16-byte-chunk XOR swizzle so MFMA
//     operand reads are bank-conflict free.  Rows past the visible length
//     are DMA'd from a zero buffer, never from the cache.
//   * S phase: wave w owns heads 16w..16w+15; S^T[32 tokens x 16 heads] =
//     tile . q^T on MFMA (q held in registers for the whole segment);
//     online-softmax statistics per head with cross-lane reductions; P is
//     written to LDS in bf16.
//   * PV phase: wave w owns latent columns [64w, 64w+64) for all 128 heads;
//     O[128 x 64] += P[128 x 32] . tile[32 x 64-col slice] on MFMA.  Each
//     tile column is read from LDS by exactly one wave.
#include <math.h>

#include "mla_common.h"
#include "mla_internal.h"

namespace mla {

static __device__ __attribute__((aligned(16))) unsigned char g_zero_rows[64 * 16];

#define MLA_CONST_PTR(p) ((const __attribute__((address_space(4))) int32_t*)(p))

template <typename T_, int HP_, int NW_, int DL_, int DR_, int NSTAGE_>
struct AttnCfg {
  using T = T_;
  using F = Mfma<T>;
  // HP = heads handled by one work-group (one head group)
  static constexpr int HP = HP_, NW = NW_, DL = DL_, DR = DR_, R = DL_ + DR_;
  static constexpr int ES = (int)sizeof(T);
  static constexpr int TILE = 32;
  static constexpr int NSTAGE = NSTAGE_;
  static constexpr int NTHR = NW * 64;
  static constexpr int NHT = HP / 16;        // head tiles
  static constexpr int HTW = NHT / NW;       // head tiles per wave in the score phase
  static constexpr int KB = F::KB, KPL = F::KPL;
  static constexpr int RK = R / KB;          // MFMA k-steps over one row
  static constexpr int CPW = DL / NW;        // latent columns per wave in the PV phase
  static constexpr int NCT = CPW / 16;
  static constexpr int ROW_BYTES = R * ES;
  static constexpr int ROW_CHUNKS = ROW_BYTES / 16;
  static constexpr bool SWZ = (ROW_CHUNKS % 8) == 0;
  // closed-form swizzled offsets (bf16 rows, 4 chunks per k-step, 64-column slices)
  static constexpr bool FAST = SWZ && KPL == 8 && (CPW % 64) == 0;
  static constexpr int TILE_BYTES = TILE * ROW_BYTES;
  static constexpr int NINST = TILE_BYTES / 1024;
  static constexpr int PSTR = TILE + 16 / ES;
  static constexpr int PV_KS = TILE / KB;
  static constexpr int OFF_P = NSTAGE * TILE_BYTES;
  static constexpr int OFF_ALPHA = OFF_P + HP * PSTR * ES;
  static constexpr int OFF_M = OFF_ALPHA + HP * 4;
  static constexpr int OFF_L = OFF_M + HP * 4;
  static constexpr int OFF_FLAG = OFF_L + HP * 4;
  static constexpr int LDS_BYTES = OFF_FLAG + NHT * 4;
  static_assert(R % KB == 0, "row width must be a multiple of the MFMA k");
  static_assert(TILE_BYTES % 1024 == 0, "tile must be whole 1 KB DMA blocks");
  static_assert(NINST % NW == 0, "DMA blocks must split evenly over waves");
  static_assert(NHT % NW == 0, "head tiles must split evenly over waves");
  static_assert(DL % (NW * 16) == 0, "latent columns must split evenly over waves");
  static_assert(TILE % KB == 0, "tile must be whole MFMA k-steps");
  static_assert(ROW_BYTES % 16 == 0, "rows must be whole 16 B chunks");
};

// One work-group = one head group of 64 heads: 4 waves x 16 heads in the
// score phase, 4 waves x 128 latent columns in the PV phase (O: 64 x 512
// fp32 = 128 accumulator registers per lane).  Both head groups of a tile
// range run on the same XCD, so each tile is fetched from HBM once.
using CfgBf16 = AttnCfg<__bf16, 64, 4, 512, 64, 3>;
using CfgF32 = AttnCfg<float, 16, 1, 32, 8, 3>;

// Softmax statistics are only rebased when a head's running max grows by
// more than this (log2 units); P stays <= 2^8, exact in bf16 and fp32.
constexpr float kRescaleSlack = 8.0f;

// 16-byte-chunk swizzle of a tile row: logical chunk c of row r sits at
// chunk c ^ swz(r).  Rows 8g+j of the four lane groups of a transposed PV
// read, and the 8 rows of one ds_read_b128 pass of the score phase, land in
// distinct banks.
__device__ inline int swz(int r) { return (r ^ ((r >> 3) << 1)) & 7; }

template <class C>
__device__ inline int lds_off(int r, int e) {
  const int byte = e * C::ES;
  int chunk = byte >> 4;
  if constexpr (C::SWZ) chunk ^= swz(r);
  return r * C::ROW_BYTES + (chunk << 4) + (byte & 15);
}

// max / sum with the lanes 16 and 32 apart (gfx950 permlane swaps, no LDS)
__device__ inline float max_xor16_32(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_xor16_32(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline void vm_wait_rt(int n) {
  switch (n) {
    case 0: vm_wait<0>(); break;
    case 1: vm_wait<1>(); break;
    case 2: vm_wait<2>(); break;
    case 3: vm_wait<3>(); break;
    case 4: vm_wait<4>(); break;
    case 5: vm_wait<5>(); break;
    case 6: vm_wait<6>(); break;
    case 7: vm_wait<7>(); break;
    case 8: vm_wait<8>(); break;
    case 9: vm_wait<9>(); break;
    case 10: vm_wait<10>(); break;
    case 11: vm_wait<11>(); break;
    case 12: vm_wait<12>(); break;
    case 16: vm_wait<16>(); break;
    case 18: vm_wait<18>(); break;
    default: vm_wait<0>(); break;
  }
}

// DMA one 32-row tile into an LDS stage.  Every wave issues the same number
// of load instructions on every call, so the per-wave vmcnt bookkeeping of
// the pipeline is exact.  Rows at or past `vis` (and rows of a page id
// outside the pool) are DMA'd from a zero buffer instead of the cache.
template <class C>
__device__ inline void issue_tile(const AttnArgs& a, unsigned char* stage, int b, int k, int vis, int wave,
                                  int lane) {
  const int t0 = k * C::TILE;
  const unsigned char* gbase;
  bool ok = true;
  if (a.paged) {
    const int pg = MLA_CONST_PTR(a.page_table)[(size_t)b * a.max_pages + t0 / a.page_size];
    ok = (pg >= 0) && (pg < a.n_pages);
    gbase = reinterpret_cast<const unsigned char*>(a.pool) +
            ((size_t)(ok ? pg : 0) * a.page_size + (t0 % a.page_size)) * (size_t)C::ROW_BYTES;
  } else {
    gbase = reinterpret_cast<const unsigned char*>(a.pool) + ((size_t)b * a.s_max + t0) * (size_t)C::ROW_BYTES;
  }
#pragma unroll
  for (int inst = 0; inst < C::NINST / C::NW; ++inst) {
    const int in = wave + inst * C::NW;
    const int p = in * 64 + lane;
    const int r = p / C::ROW_CHUNKS, s = p % C::ROW_CHUNKS;
    const int c = C::SWZ ? (s ^ swz(r)) : s;
    const bool valid = ok && (t0 + r < vis);
    const void* src =
        valid ? (const void*)(gbase + r * C::ROW_BYTES + c * 16) : (const void*)(g_zero_rows + lane * 16);
    __builtin_amdgcn_global_load_lds(src, MLA_LDS_PTR(stage + in * 1024), 16, 0, 0);
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
                                          float* __restrict__ alpha_s, int* __restrict__ flag_s, bool issue,
                                          int b, int k_issue, int tok0, int vis, int i, int wave, int lane,
                                          const int (&s_base)[2][2], const int (&v_base)[4][2],
                                          const typename C::F::frag (&qf)[C::HTW][C::RK], float (&m_run)[C::HTW],
                                          float (&l_run)[C::HTW], f32x4 (&O)[C::NHT][C::NCT]) {
  using T = typename C::T;
  using F = typename C::F;
  using frag = typename F::frag;
  const int g = lane >> 4, l16 = lane & 15;
  if (issue) issue_tile<C>(a, dma_stage, b, k_issue, vis, wave, lane);

  // ---- S^T[32 tokens x 16 heads] = tile . q^T, per head tile ----------
  // two accumulators per sub-tile (even / odd k-steps): four independent
  // MFMA chains in flight
  f32x4 sacc[C::HTW][2][2];
#pragma unroll
  for (int ht = 0; ht < C::HTW; ++ht)
#pragma unroll
    for (int u = 0; u < 2; ++u) sacc[ht][u][0] = sacc[ht][u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < C::RK; ++kb) {
    frag a0, a1;
    if constexpr (C::FAST) {
      a0 = *reinterpret_cast<const frag*>(tb + s_base[0][kb & 1] + 128 * (kb >> 1));
      a1 = *reinterpret_cast<const frag*>(tb + s_base[1][kb & 1] + 128 * (kb >> 1));
    } else {
      const int e = kb * C::KB + g * C::KPL;
      a0 = *reinterpret_cast<const frag*>(tb + lds_off<C>(l16, e));
      a1 = *reinterpret_cast<const frag*>(tb + lds_off<C>(16 + l16, e));
    }
#pragma unroll
    for (int ht = 0; ht < C::HTW; ++ht) {
      sacc[ht][0][kb & 1] = F::mma(a0, qf[ht][kb], sacc[ht][0][kb & 1]);
      sacc[ht][1][kb & 1] = F::mma(a1, qf[ht][kb], sacc[ht][1][kb & 1]);
    }
  }

  // ---- online softmax over this tile's 32 tokens, per head ------------
  const bool tail = tok0 + C::TILE > vis;  // uniform: only the last tile is ragged
#pragma unroll
  for (int ht = 0; ht < C::HTW; ++ht) {
    const int hl = (wave * C::HTW + ht) * 16 + l16;  // head within the group
    float x[8];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      x[ii] = (sacc[ht][0][0][ii] + sacc[ht][0][1][ii]) * a.scale_log2;
      x[4 + ii] = (sacc[ht][1][0][ii] + sacc[ht][1][1][ii]) * a.scale_log2;
    }
    if (tail) {
      const int lim = vis - tok0 - 4 * g;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        if (ii >= lim) x[ii] = -INFINITY;
        if (16 + ii >= lim) x[4 + ii] = -INFINITY;
      }
    }
    float mloc = x[0];
#pragma unroll
    for (int ii = 1; ii < 8; ++ii) mloc = fmaxf(mloc, x[ii]);
    mloc = max_xor16_32(mloc);
    const bool rebase = mloc > m_run[ht] + kRescaleSlack;
    float alpha = 1.f;
    if (rebase) {
      alpha = __builtin_amdgcn_exp2f(m_run[ht] - mloc);
      m_run[ht] = mloc;
    }
    float psum = 0.f, pv[8];
#pragma unroll
    for (int ii = 0; ii < 8; ++ii) {
      pv[ii] = __builtin_amdgcn_exp2f(x[ii] - m_run[ht]);
      psum += pv[ii];
    }
    psum = sum_xor16_32(psum);
    l_run[ht] = l_run[ht] * alpha + psum;
    T* prow = p_s + (size_t)hl * C::PSTR;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      prow[4 * g + ii] = from_f32<T>(pv[ii]);
      prow[16 + 4 * g + ii] = from_f32<T>(pv[4 + ii]);
    }
    if (g == 0) alpha_s[hl] = alpha;
    const bool any = __any(rebase);
    if (lane == 0) flag_s[wave * C::HTW + ht] = any ? 1 : 0;
  }
  lds_barrier();

  // ---- PV: O[group heads][this wave's columns] += P . tile ------------
  if (i > 0) {
#pragma unroll
    for (int ht = 0; ht < C::NHT; ++ht) {
      if (__builtin_amdgcn_readfirstlane(flag_s[ht])) {
        const float4 a4 = *reinterpret_cast<const float4*>(alpha_s + ht * 16 + 4 * g);
#pragma unroll
        for (int ct = 0; ct < C::NCT; ++ct) {
          O[ht][ct][0] *= a4.x;
          O[ht][ct][1] *= a4.y;
          O[ht][ct][2] *= a4.z;
          O[ht][ct][3] *= a4.w;
        }
      }
    }
  }
#pragma unroll
  for (int ks = 0; ks < C::PV_KS; ++ks) {
    frag pa[C::NHT];
#pragma unroll
    for (int ht = 0; ht < C::NHT; ++ht)
      pa[ht] = *reinterpret_cast<const frag*>(p_s + (size_t)(ht * 16 + l16) * C::PSTR + ks * C::KB + g * C::KPL);
#pragma unroll
    for (int ct = 0; ct < C::NCT; ++ct) {
      frag bfr;
      if constexpr (C::FAST) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          bfr[jj] = *reinterpret_cast<const T*>(tb + v_base[(ct & 3) ^ (jj >> 1)][jj & 1] + jj * C::ROW_BYTES +
                                                128 * (ct >> 2));
      } else if constexpr (C::KPL == 1) {
        bfr = *reinterpret_cast<const T*>(tb + lds_off<C>(ks * C::KB + g, wave * C::CPW + ct * 16 + l16));
      } else {
#pragma unroll
        for (int jj = 0; jj < C::KPL; ++jj)
          bfr[jj] = *reinterpret_cast<const T*>(
              tb + lds_off<C>(ks * C::KB + g * C::KPL + jj, wave * C::CPW + ct * 16 + l16));
      }
#pragma unroll
      for (int ht = 0; ht < C::NHT; ++ht) O[ht][ct] = F::mma(pa[ht], bfr, O[ht][ct]);
    }
  }
}

template <class C>
__global__ __launch_bounds__(C::NTHR, 1) void attn_split_kernel(AttnArgs a) {
  using T = typename C::T;
  using F = typename C::F;
  using frag = typename F::frag;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, l16 = lane & 15;
  const int G = gridDim.x;
  // XCD-aware order: the hardware deals blocks round-robin over 8 XCDs, so
  // logical ranges are assigned such that neighbours share an XCD's L2.
  const int w = ((G & 7) == 0) ? ((int)(blockIdx.x & 7) * (G >> 3) + (int)(blockIdx.x >> 3)) : (int)blockIdx.x;
  const int U = a.U;  // streams = (virtual sequence, head group) pairs
  const int Ttot = MLA_CONST_PTR(a.tile_off)[U];
  const int per = (Ttot + G - 1) / G;
  const int g0 = w * per;
  const int g1 = min(g0 + per, Ttot);
  if (g0 >= g1) return;

  float* alpha_s = reinterpret_cast<float*>(smem + C::OFF_ALPHA);
  float* m_s = reinterpret_cast<float*>(smem + C::OFF_M);
  float* l_s = reinterpret_cast<float*>(smem + C::OFF_L);
  int* flag_s = reinterpret_cast<int*>(smem + C::OFF_FLAG);
  T* p_s = reinterpret_cast<T*>(smem + C::OFF_P);

  // lane-constant LDS offsets (see the swizzle in issue_tile)
  // s_base[sub-tile][k-step parity]: row l16 (+16) reads logical chunk
  // 4*kb + g; v_base[t][p]: rows 8g+j of the transposed PV read, with
  // t = (ct & 3) ^ (j >> 1) and p = j & 1 (closed forms of lds_off)
  int s_base[2][2] = {{0, 0}, {0, 0}}, v_base[4][2] = {{0, 0}, {0, 0}, {0, 0}, {0, 0}};
  if constexpr (C::FAST) {
    const int hb = l16 >> 3;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int r = l16 + 16 * sub;
#pragma unroll
      for (int par = 0; par < 2; ++par) s_base[sub][par] = r * C::ROW_BYTES + 16 * ((par * 4 + g) ^ swz(r));
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int par = 0; par < 2; ++par)
        v_base[t][par] = g * 8 * C::ROW_BYTES + 16 * wave * (C::CPW / 8) + 16 * ((2 * (t ^ g) + (hb ^ par)) & 7) +
                         2 * (l16 & 7);
  }

  // first stream holding tile g0
  int lo = 0, hi = U;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (MLA_CONST_PTR(a.tile_off)[mid] <= g0) lo = mid; else hi = mid;
  }
  constexpr int n_loads = C::NINST / C::NW;  // DMA instructions per tile and wave

  int u = lo, gcur = g0;
  while (gcur < g1) {
    const int tb0 = MLA_CONST_PTR(a.tile_off)[u], tb1 = MLA_CONST_PTR(a.tile_off)[u + 1];
    if (tb1 <= gcur) { ++u; continue; }
    const int k0 = gcur - tb0, k1 = min(g1, tb1) - tb0;
    const bool whole = (k0 == 0) && (k1 == tb1 - tb0);
    const int cnt = k1 - k0;
    const int v = u / a.n_hg, hgrp = u - v * a.n_hg;
    const int h_base = hgrp * C::HP;
    const int b = v / a.n_q, jq = v - b * a.n_q;
    const int vis = MLA_CONST_PTR(a.kv_len)[b] - a.n_q + jq + 1;

    vm_wait<0>();
    // q^T fragments of this wave's head tiles, kept in registers
    frag qf[C::HTW][C::RK];
#pragma unroll
    for (int ht = 0; ht < C::HTW; ++ht) {
      const int h = h_base + (wave * C::HTW + ht) * 16 + l16;
      const T* qp = reinterpret_cast<const T*>(a.q) + ((size_t)v * a.H + min(h, a.H - 1)) * C::R + g * C::KPL;
#pragma unroll
      for (int kb = 0; kb < C::RK; ++kb) {
        qf[ht][kb] = load_frag<T>(qp + kb * C::KB);
        if (h >= a.H) qf[ht][kb] = F::zero();
      }
    }
    for (int s = 0; s < C::NSTAGE - 1 && s < cnt; ++s)
      issue_tile<C>(a, smem + s * C::TILE_BYTES, b, k0 + s, vis, wave, lane);

    float m_run[C::HTW], l_run[C::HTW];
#pragma unroll
    for (int ht = 0; ht < C::HTW; ++ht) {
      m_run[ht] = -1e30f;
      l_run[ht] = 0.f;
    }
    f32x4 O[C::NHT][C::NCT];
#pragma unroll
    for (int ht = 0; ht < C::NHT; ++ht)
#pragma unroll
      for (int ct = 0; ct < C::NCT; ++ct) O[ht][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int i = 0; i < cnt; ++i) {
      const int st = i % C::NSTAGE;
      vm_wait_rt(min(C::NSTAGE - 2, cnt - 1 - i) * n_loads);
      lds_barrier();
      const bool issue = i + C::NSTAGE - 1 < cnt;
      tile_step<C>(a, smem + ((i + C::NSTAGE - 1) % C::NSTAGE) * C::TILE_BYTES, smem + st * C::TILE_BYTES, p_s,
                   alpha_s, flag_s, issue, b, k0 + i + C::NSTAGE - 1, (k0 + i) * C::TILE, vis, i, wave, lane,
                   s_base, v_base, qf, m_run, l_run, O);
    }

    // ---- finalise the segment ----------------------------------------
#pragma unroll
    for (int ht = 0; ht < C::HTW; ++ht) {
      const int hl = (wave * C::HTW + ht) * 16 + l16;
      if (g == 0) {
        m_s[hl] = m_run[ht];
        l_s[hl] = l_run[ht];
      }
    }
    lds_barrier();
    const int pid = w + u;  // partial slot of this (work-group, stream) piece
#pragma unroll
    for (int ht = 0; ht < C::NHT; ++ht) {
      const float4 l4 = *reinterpret_cast<const float4*>(l_s + ht * 16 + 4 * g);
      const float inv[4] = {1.f / l4.x, 1.f / l4.y, 1.f / l4.z, 1.f / l4.w};
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int hl = ht * 16 + 4 * g + ii;
        if (h_base + hl >= a.H) continue;
        float* dst = whole ? a.o_lat + ((size_t)v * a.H + h_base + hl) * C::DL
                           : a.part_o + ((size_t)pid * C::HP + hl) * C::DL;
#pragma unroll
        for (int ct = 0; ct < C::NCT; ++ct) dst[wave * C::CPW + ct * 16 + l16] = O[ht][ct][ii] * inv[ii];
      }
    }
#pragma unroll
    for (int ht = 0; ht < C::HTW; ++ht) {
      const int hl = (wave * C::HTW + ht) * 16 + l16;
      if (g == 0 && h_base + hl < a.H) {
        const float lse2 = m_run[ht] + __log2f(l_run[ht]);
        if (whole) {
          if (a.lse) a.lse[(size_t)v * a.H + h_base + hl] = lse2 * 0.69314718055994531f;
        } else {
          a.part_lse[(size_t)pid * C::HP + hl] = lse2;
        }
      }
    }
    lds_barrier();
    gcur = tb0 + k1;
    ++u;
  }
}

// Prefix sum of 32-token tiles over the streams u = v * n_hg + head group
// (one block).  Invalid lengths get no tiles and raise error bit 4.
__global__ __launch_bounds__(1024) void attn_plan_kernel(const int32_t* __restrict__ kv_len, int n_q, int n_hg, int U,
                                                        int cap, int32_t* __restrict__ tile_off,
                                                        int32_t* __restrict__ err, const int32_t* __restrict__ table,
                                                        int page_size, int max_pages, int n_pages) {
  __shared__ int buf[1024];
  __shared__ int carry;
  const int tid = threadIdx.x;
  // page ids the split kernel will follow must lie inside the pool (it
  // reads zeros instead of a bad page; this raises error bit 2)
  if (table) {
    const int B = U / (n_hg * n_q);
    for (long i = tid; i < (long)B * max_pages; i += 1024) {
      const int b = (int)(i / max_pages), p = (int)(i % max_pages);
      const int L = kv_len[b];
      if (L >= n_q && L <= cap && p < (L + page_size - 1) / page_size) {
        const int pg = table[i];
        if (pg < 0 || pg >= n_pages) atomicOr(err, 2);
      }
    }
  }
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < U; base += 1024) {
    const int u = base + tid;
    int cnt = 0;
    if (u < U) {
      const int v = u / n_hg;
      const int b = v / n_q, j = v - b * n_q;
      const int L = kv_len[b];
      if (L < n_q || L > cap) {
        if (j == 0 && u % n_hg == 0) atomicOr(err, 4);
      } else {
        cnt = (L - n_q + j + 1 + 31) / 32;
      }
    }
    buf[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int add = tid >= off ? buf[tid - off] : 0;
      __syncthreads();
      buf[tid] += add;
      __syncthreads();
    }
    if (u < U) tile_off[u] = carry + buf[tid] - cnt;
    __syncthreads();
    if (tid == 1023) carry += buf[1023];
    __syncthreads();
  }
  if (tid == 0) tile_off[U] = carry;
}

// Log-sum-exp merge of the pieces of every stream that was cut by a
// work-group boundary: lse = log2 sum_s 2^lse_s, o = sum_s 2^(lse_s - lse) O_s.
// Block = (stream, HPB heads of its group); each thread owns 4 columns.
template <int HP, int DL>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  constexpr int TPH = DL / 4;                      // threads per head
  constexpr int HPB = 256 / TPH;                   // heads per block
  constexpr int MAXS = 32;
  __shared__ float wts[HPB][MAXS];
  __shared__ float lse_s[HPB];
  const int u = blockIdx.x, tid = threadIdx.x;
  const int v = u / a.n_hg, hgrp = u - v * a.n_hg;
  const int r = tid / TPH;                         // head slot in the block
  const int hl = blockIdx.y * HPB + r;             // head within the group
  const int h = hgrp * HP + hl;                    // global head
  const int c0 = (tid % TPH) * 4;
  const bool active = (hl < HP) && (h < a.H);
  const int G = a.G;
  const int Ttot = a.tile_off[a.U];
  const int per = (Ttot + G - 1) / G;
  const int t0 = a.tile_off[u], t1 = a.tile_off[u + 1];
  if (t1 == t0) {  // invalid length: flagged by the plan kernel; poison the output
    if (active) {
      *reinterpret_cast<float4*>(a.o_lat + ((size_t)v * a.H + h) * DL + c0) = make_float4(NAN, NAN, NAN, NAN);
      if (a.lse && c0 == 0) a.lse[(size_t)v * a.H + h] = NAN;
    }
    return;
  }
  const int wf = t0 / per, wl = (t1 - 1) / per;
  if (wf == wl) return;  // written whole by the split kernel
  const int n = wl - wf + 1;
  if (tid % TPH == 0 && active) {
    const float* pl = a.part_lse + (size_t)(wf + u) * HP + hl;   // piece s at pl[s * HP]
    float mx = -INFINITY;
    for (int s = 0; s < n; ++s) mx = fmaxf(mx, pl[(size_t)s * HP]);
    float sum = 0.f;
    for (int s = 0; s < n; ++s) sum += exp2f(pl[(size_t)s * HP] - mx);
    const float L = mx + log2f(sum);
    lse_s[r] = L;
    for (int s = 0; s < n && s < MAXS; ++s) wts[r][s] = exp2f(pl[(size_t)s * HP] - L);
    if (a.lse) a.lse[(size_t)v * a.H + h] = L * 0.69314718055994531f;
  }
  __syncthreads();
  if (!active) return;
  const float* src = a.part_o + ((size_t)(wf + u) * HP + hl) * DL + c0;  // piece s at src[s * HP * DL]
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < n; ++s) {
    const float wgt = (s < MAXS) ? wts[r][s] : exp2f(a.part_lse[(size_t)(wf + s + u) * HP + hl] - lse_s[r]);
    const float4 x = *reinterpret_cast<const float4*>(src + (size_t)s * HP * DL);
    acc.x += wgt * x.x;
    acc.y += wgt * x.y;
    acc.z += wgt * x.z;
    acc.w += wgt * x.w;
  }
  *reinterpret_cast<float4*>(a.o_lat + ((size_t)v * a.H + h) * DL + c0) = acc;
}

int attn_supported(bool bf16, int H, int d_latent, int d_rope) {
  if (bf16) return H >= 1 && H <= 1024 && d_latent == CfgBf16::DL && d_rope == CfgBf16::DR;
  return H >= 1 && H <= 1024 && d_latent == CfgF32::DL && d_rope == CfgF32::DR;
}

int attn_head_group(bool bf16) { return bf16 ? CfgBf16::HP : CfgF32::HP; }

int attn_tile() { return 32; }

template <class C>
static hipError_t launch_attn_t(const AttnArgs& a, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_split_kernel<C>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int cap = a.paged ? a.max_pages * a.page_size : a.s_max;
  hipLaunchKernelGGL(attn_plan_kernel, dim3(1), dim3(1024), 0, s, a.kv_len, a.n_q, a.n_hg, a.U, cap, a.tile_off,
                     a.err, a.paged ? a.page_table : nullptr, a.page_size, a.max_pages, a.n_pages);
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
  return bf16 ? launch_attn_t<CfgBf16>(a, s) : launch_attn_t<CfgF32>(a, s);
}

}  // namespace mla
