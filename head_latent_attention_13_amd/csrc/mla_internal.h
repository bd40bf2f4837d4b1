// Host-side interfaces between the C ABI (mla_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

// ---------------------------------------------------------------- GEMM ----
// y[M][N] = A[M][K] * W[K][N] with W in the packed fragment layout, followed
// by an epilogue (store / RoPE / cache append).  Two kernels:
//   streaming (M <= 16, decode): one block computes MT*16 rows x NT*16
//     columns over one K slice; its 4 waves split the slice and are summed
//     through LDS;
//   tiled (M > 16, bf16): a block computes BM x BN = 64*MT x 64*NT with 4
//     waves in a 2 x 2 grid of 32x32x16 MFMA sub-tiles; A and W tiles are
//     DMA'd into LDS through a 3-stage ring.
// With ksplit > 1 slices, each block leaves an fp32 partial tile in the
// workspace and a second kernel sums the slices in order and applies the
// epilogue.
// A may be read in column groups: the n-tiles [g*a_gtiles, (g+1)*a_gtiles)
// take their A operand from columns g*a_gstride .. of A (a per-head product
// packed as one wide matrix); a block never straddles two groups.
enum EpiMode { EPI_F32 = 0, EPI_STORE_T = 1, EPI_Q = 2, EPI_APPEND = 3 };

struct EpiArgs {
  int mode;
  int M, N;
  void* out;            // EPI_F32: float[M][N]; EPI_STORE_T: T[M][N]; EPI_Q: see below
  // RoPE (EPI_Q, EPI_APPEND)
  int d_latent, d_rope, row;   // row = d_latent + d_rope (EPI_APPEND: the cache row)
  // EPI_Q: column n is element f = n % qg_cols of group n / qg_cols; it is
  // stored to out[m * q_ld + q_off + (n / qg_cols) * qg_stride + f] and
  // rotated (pairs f, f+1 counted from rope_from) when f >= rope_from
  int qg_cols, qg_stride, q_off, q_ld, rope_from;
  float rope_base;
  int n_q;
  const int32_t* kv_len;       // EPI_Q: query t of sequence b sits at kv_len[b]-n_q+t
  const int32_t* pos;          // EPI_APPEND: token t of sequence b sits at pos[b]+t
  // cache (EPI_APPEND)
  void* pool;
  const int32_t* page_table;
  int paged, page_size, n_pages, max_pages, s_max;
  int32_t* err;
};

struct GemmPlan {
  int M, K, N;       // logical sizes
  int Kp, Np;        // padded sizes of the packed weight
  int KB;            // k per MFMA (32 bf16, 4 fp32)
  int kblocks, ntiles;
  int MT, NT, KSW;
  int tiled;         // 1: LDS-tiled kernel (MT, NT = 32x32 tiles per wave)
  int gx, gy;        // blocks over columns / rows
  int ksplit, kb_per_split;
  size_t part_bytes; // fp32 partial tiles (ksplit > 1)
  int a_gtiles;      // A column groups (0: none): n-tiles per group ...
  int a_gstride;     // ... and A column offset per group
};

// a_f32: the A operand is fp32 (converted to bf16 fragments in the kernel).
// a_gtiles / a_gstride: A column groups (0: none).  part_cap: the most bytes
// the fp32 split-K partials may take (K splits that need more are not
// considered; an unsplit plan needs none).  Returns a plan with tiled == -1
// when no kernel configuration fits the groups.
GemmPlan plan_gemm(int M, int K, int N, bool bf16, bool a_f32, int n_cu, int a_gtiles = 0, int a_gstride = 0,
                   size_t part_cap = SIZE_MAX);

// fp32 -> bf16 copy (round to nearest even); n a multiple of 8, both
// pointers 16-byte aligned.
hipError_t launch_f32_to_bf16(const float* x, void* y, size_t n, hipStream_t s);

// A is T (a_f32 == false) or fp32 (a_f32 == true); Wp is T.
// row_len / row_group: rows m with m % row_group >= row_len[m / row_group]
// (clamped to [0, row_group]) are not needed: blocks holding only such rows
// return at once and leave their output rows unwritten (NULL: every row).
hipError_t launch_gemm(const GemmPlan& g, bool bf16, bool a_f32, const void* A, int lda, const void* Wp, float* part,
                       const EpiArgs& e, hipStream_t s,
                       const int32_t* row_len = nullptr, int row_group = 0);

// Factored query projection after c_Q, in one launch, for up to 16 rows
// (bf16; d_nope = 128, d_rope = 64, d_latent = 512, d_q_latent a multiple
// of 32): per head h, q_nope = c_Q W_UQ[h] rounded to bf16, then
// q[m][h] = [q_nope W_UK[h]^T | RoPE(c_Q W_QR[h])].  The weights are the
// packed factors of the absorbed buffer (W_UQ: K = d_q_latent, N = H*128;
// W_QR: N = H*64; W_UK^T: K = 128, N = H*512).
struct QFusedArgs {
  const void* cq;         // [M][d_q_latent] bf16
  const void* w_uq;
  const void* w_qr;
  const void* w_ukt;
  void* q;                // [M][H][576] bf16
  const int32_t* kv_len;  // query t of sequence b sits at kv_len[b] - n_q + t
  int M, n_q, H, d_q_latent;
  float rope_base;
};
bool q_fused_supported(bool bf16, int M, int d_nope, int d_rope, int d_latent, int d_q_latent);
hipError_t launch_q_fused(const QFusedArgs& a, hipStream_t s);

// ------------------------------------------------------------- absorb ----
struct AbsorbArgs {
  int d_model, H, d_latent, d_q_latent, d_nope, d_rope, d_v;
  const void *W_DQ, *W_UQ, *W_QR, *W_DKV, *W_KR, *W_UK, *W_UV, *W_O;
  void *P_KV, *P_DQ, *P_QC, *P_O;   // packed outputs (merged form: all four)
  int factored;                      // factored form: P_KV, P_DQ and these five
  void *P_UQ, *P_QR, *P_UKT, *P_UK, *P_UV, *P_WO;
};
hipError_t launch_absorb(const AbsorbArgs& a, bool bf16, hipStream_t s);

// ------------------------------------------------------- cache store ----
// Rows [M][R] fp32 into the cache slots of positions pos[b] + t (m = b*n_q+t),
// RoPE'd first (columns d_latent.., append path) when `rope` is set: bf16
// (RNE) or fp32 rows, or E4M3 codes with one power-of-two scale per row.
struct StoreArgs {
  const float* rows;
  const int32_t* pos;
  int M, n_q, R, d_latent, d_rope;
  int rope;
  float rope_base;
  int format;             // 0: dtype rows, 1: E4M3 codes + scales
  int bf16;               // dtype rows: bf16 (1) or fp32 (0)
  void* pool;
  float* scales;
  const int32_t* page_table;
  int paged, page_size, n_pages, max_pages, s_max;
  int32_t* err;           // bit 1: position outside the cache, bit 2: page id outside the pool
};
hipError_t launch_cache_store(const StoreArgs& a, hipStream_t s);

// ---------------------------------------------------------- attention ----
struct AttnArgs {
  const void* q;               // [V][H][R]
  const void* pool;
  const int32_t* page_table;
  int paged, page_size, n_pages, max_pages, s_max;
  const int32_t* kv_len;
  int B, n_q, H, V;
  int n_hg, U;                 // head groups per query row; streams U = V * n_hg (set by the launcher)
  // work plan (written by the plan kernel), carved out of `sched`:
  int32_t* sched;              // plan storage, attn_sched_ints(U, G) ints
  int32_t* wrec;               // [G][8] {g0, g1, first stream u, srec[u] (3), 0, 0}
  int32_t* srec;               // [U][4] {first tile, end tile, visible rows, 0}
  int32_t* wfl;                // [U][2] first / last work-group of stream u (-1: invalid length)
  float* o_lat;                // [V][H][d_latent]
  float* lse;                  // [V][H] natural-log LSE of scaled scores, or null
  float* part_o;               // [(G+U)][head group][d_latent], slot w + u
  float* part_lse;             // [(G+U)][head group]
  int32_t* err;
  float scale_log2;            // softmax scale * log2(e)
  int G;                       // attention work-groups
  int e4m3;                    // cache rows are E4M3 codes with per-row scales
  const float* scales;         // their scales, laid out like the rows
};

int attn_supported(bool bf16, int H, int d_latent, int d_rope);
int attn_head_group(bool bf16);  // heads per attention work-group
int attn_tile();
size_t attn_sched_ints(int U, int G);  // ints of plan storage for U streams, G work-groups
hipError_t launch_attention(const AttnArgs& a, bool bf16, hipStream_t s);

// ------------------------------------------------ expanded-form prefill ----
// Causal attention of n_q new query tokens per sequence over per-head keys
// and values up-projected from the latent cache (bf16; d_nope = d_v = 128,
// d_rope = 64).  Query row m = b*n_q + t sits at position kv_len[b]-n_q+t and
// sees keys 0 .. that position.
struct PrefillArgs {
  const void* qe;         // [B*n_q][H][192] bf16: q_nope | RoPE'd q_pe
  const void* ke;         // [B*s_max][H*128] bf16: c_i W_UK[h]
  const void* ve;         // [B*s_max][H*128] bf16: c_i W_UV[h]
  const void* pool;       // [B][s_max][576] bf16 contiguous cache (k_pe at 512..575)
  const int32_t* kv_len;  // [B]
  int B, n_q, H, s_max;
  float scale_log2;       // softmax scale * log2(e)
  void* vo;               // [B*n_q][H*128] bf16 out: softmax . V per head
  float* lse;             // [B*n_q][H] out or null (natural log)
  int32_t* err;           // bit 4: kv_len outside [n_q, s_max]
};
bool prefill_supported(bool bf16, int d_nope, int d_rope, int d_v);
hipError_t launch_prefill_attention(const PrefillArgs& a, hipStream_t s);

}  // namespace mla
