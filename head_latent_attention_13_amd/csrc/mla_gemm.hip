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
// GEMM: part[ks][m][n] = sum_{k in slice ks} A[m][k] * W[k][n]
// Block = 4 waves; wave -> one n-group (NT tiles of 16 columns), all MT
// m-tiles of the block's m-group, one K slice.
// --------------------------------------------------------------------------
template <typename T, typename TA, int MT, int NT>
__global__ __launch_bounds__(256) void gemm_stream_kernel(
    const TA* __restrict__ A, int lda, int M, const T* __restrict__ Wp, int kblocks, int ntiles,
    int kb_per_split, float* __restrict__ part, int Np) {
  using F = Mfma<T>;
  constexpr int KB = F::KB, KPL = F::KPL, FR = 64 * KPL;
  const int lane = threadIdx.x & 63;
  const int ng = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nt0 = ng * NT;
  if (nt0 >= ntiles) return;
  const int mt0 = blockIdx.y * MT;
  const int ks = blockIdx.z;
  const int kb0 = ks * kb_per_split;
  const int kb1 = min(kb0 + kb_per_split, kblocks);

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int ni = 0; ni < NT; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  const TA* ap[MT];
  bool aval[MT];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi) {
    const int m = (mt0 + mi) * 16 + (lane & 15);
    aval[mi] = m < M;
    ap[mi] = A + (size_t)(aval[mi] ? m : 0) * (size_t)lda + (lane >> 4) * KPL;
  }
  const T* wp[NT];
#pragma unroll
  for (int ni = 0; ni < NT; ++ni) {
    const int nt = min(nt0 + ni, ntiles - 1);
    wp[ni] = Wp + (size_t)nt * (size_t)kblocks * FR + lane * KPL;
  }

#pragma unroll 2
  for (int kb = kb0; kb < kb1; ++kb) {
    typename F::frag b[NT];
#pragma unroll
    for (int ni = 0; ni < NT; ++ni) b[ni] = load_frag<T>(wp[ni] + (size_t)kb * FR);
    typename F::frag a[MT];
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      if constexpr (sizeof(TA) == sizeof(T)) {
        a[mi] = load_frag<T>(reinterpret_cast<const T*>(ap[mi]) + kb * KB);
      } else {
        a[mi] = load_frag_from_f32<T>(reinterpret_cast<const float*>(ap[mi]) + kb * KB);
      }
      if (!aval[mi]) a[mi] = F::zero();
    }
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int ni = 0; ni < NT; ++ni) acc[mi][ni] = F::mma(a[mi], b[ni], acc[mi][ni]);
  }

#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int ni = 0; ni < NT; ++ni) {
      const int nt = nt0 + ni;
      if (nt >= ntiles) continue;
      const int n = nt * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = (mt0 + mi) * 16 + 4 * (lane >> 4) + i;
        if (m < M) part[((size_t)ks * M + m) * Np + n] = acc[mi][ni][i];
      }
    }
}

static int ceil_div(int a, int b) { return (a + b - 1) / b; }

GemmPlan plan_gemm(int M, int K, int N, bool bf16, int n_cu) {
  GemmPlan g{};
  g.M = M; g.K = K; g.N = N;
  g.KB = bf16 ? Mfma<__bf16>::KB : Mfma<float>::KB;
  g.Kp = ceil_div(K, g.KB) * g.KB;
  g.Np = ceil_div(N, 16) * 16;
  g.kblocks = g.Kp / g.KB;
  g.ntiles = g.Np / 16;
  g.NT = g.ntiles >= 64 ? 8 : 2;
  const int mtiles = ceil_div(std::max(M, 1), 16);
  g.MT = mtiles >= 4 ? 4 : (mtiles >= 2 ? 2 : 1);
  g.ngroups = ceil_div(g.ntiles, g.NT);
  g.mgroups = ceil_div(mtiles, g.MT);
  // Enough waves to keep every SIMD streaming (about 8 per CU), but keep
  // each K slice at least 16 blocks long so partial sums stay small.
  const long target = (long)n_cu * 8;
  const long base = (long)g.ngroups * g.mgroups;
  int ks = (int)std::max(1L, target / std::max(base, 1L));
  ks = std::min(ks, std::max(1, g.kblocks / 16));
  g.kb_per_split = ceil_div(g.kblocks, ks);
  g.ksplit = ceil_div(g.kblocks, g.kb_per_split);
  g.part_bytes = (size_t)g.ksplit * (size_t)M * (size_t)g.Np * sizeof(float);
  return g;
}

template <typename T, typename TA, int MT, int NT>
static hipError_t launch_gemm_t(const GemmPlan& g, const void* A, int lda, const void* Wp, float* part,
                                hipStream_t s) {
  dim3 grid(ceil_div(g.ngroups, 4), g.mgroups, g.ksplit);
  hipLaunchKernelGGL((gemm_stream_kernel<T, TA, MT, NT>), grid, dim3(256), 0, s,
                     reinterpret_cast<const TA*>(A), lda, g.M, reinterpret_cast<const T*>(Wp), g.kblocks,
                     g.ntiles, g.kb_per_split, part, g.Np);
  return hipGetLastError();
}

template <typename T, typename TA>
static hipError_t launch_gemm_mt(const GemmPlan& g, const void* A, int lda, const void* Wp, float* part,
                                 hipStream_t s) {
  if (g.NT == 8) {
    switch (g.MT) {
      case 1: return launch_gemm_t<T, TA, 1, 8>(g, A, lda, Wp, part, s);
      case 2: return launch_gemm_t<T, TA, 2, 8>(g, A, lda, Wp, part, s);
      default: return launch_gemm_t<T, TA, 4, 8>(g, A, lda, Wp, part, s);
    }
  }
  switch (g.MT) {
    case 1: return launch_gemm_t<T, TA, 1, 2>(g, A, lda, Wp, part, s);
    case 2: return launch_gemm_t<T, TA, 2, 2>(g, A, lda, Wp, part, s);
    default: return launch_gemm_t<T, TA, 4, 2>(g, A, lda, Wp, part, s);
  }
}

hipError_t launch_gemm(const GemmPlan& g, bool bf16, bool a_f32, const void* A, int lda, const void* Wp,
                       float* part, hipStream_t s) {
  if (bf16) {
    return a_f32 ? launch_gemm_mt<__bf16, float>(g, A, lda, Wp, part, s)
                 : launch_gemm_mt<__bf16, __bf16>(g, A, lda, Wp, part, s);
  }
  return launch_gemm_mt<float, float>(g, A, lda, Wp, part, s);
}

// --------------------------------------------------------------------------
// Epilogue: sum the K slices, then store / rotate / append.
// One thread per column pair (n, n+1) so a RoPE pair is handled in-thread.
// --------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void epilogue_kernel(EpiArgs e) {
  const int pairs = e.Np / 2;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)e.M * pairs) return;
  const int m = (int)(idx / pairs);
  const int n = (int)(idx % pairs) * 2;
  if (n >= e.N) return;
  float v0 = 0.f, v1 = 0.f;
  for (int ks = 0; ks < e.ksplit; ++ks) {
    const float2 p = *reinterpret_cast<const float2*>(e.part + ((size_t)ks * e.M + m) * e.Np + n);
    v0 += p.x;
    v1 += p.y;
  }
  const bool has1 = n + 1 < e.N;
  if (e.mode == EPI_F32) {
    float* y = reinterpret_cast<float*>(e.out) + (size_t)m * e.N + n;
    y[0] = v0;
    if (has1) y[1] = v1;
    return;
  }
  if (e.mode == EPI_STORE_T) {
    T* y = reinterpret_cast<T*>(e.out) + (size_t)m * e.N + n;
    y[0] = from_f32<T>(v0);
    if (has1) y[1] = from_f32<T>(v1);
    return;
  }
  const int b = m / e.n_q, t = m - b * e.n_q;
  const int f = n % e.row;  // column within one head's (latent | rope) row
  int pos;
  if (e.mode == EPI_Q) {
    pos = e.kv_len[b] - e.n_q + t;
  } else {
    pos = e.pos[b] + t;
  }
  if (f >= e.d_latent) {
    float c, s;
    rope_cos_sin(pos, (f - e.d_latent) >> 1, e.d_rope, e.rope_base, &c, &s);
    const float a0 = v0, a1 = v1;
    v0 = a0 * c - a1 * s;
    v1 = a0 * s + a1 * c;
  }
  if (e.mode == EPI_Q) {
    T* y = reinterpret_cast<T*>(e.out) + (size_t)m * e.N + n;
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

hipError_t launch_epilogue(const EpiArgs& e, bool bf16, hipStream_t s) {
  const long total = (long)e.M * (e.Np / 2);
  const int blocks = (int)((total + 255) / 256);
  if (bf16)
    hipLaunchKernelGGL(epilogue_kernel<__bf16>, dim3(blocks), dim3(256), 0, s, e);
  else
    hipLaunchKernelGGL(epilogue_kernel<float>, dim3(blocks), dim3(256), 0, s, e);
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
enum PackMode { PACK_KV = 0, PACK_DQ = 1, PACK_QC = 2, PACK_O = 3 };

template <typename T>
__global__ __launch_bounds__(256) void pack_kernel(AbsorbArgs a, int mode, int K, int N, int Kp, int Np, T* out) {
  using F = Mfma<T>;
  const size_t total = (size_t)Kp * Np;
  const size_t p = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= total) return;
  // invert packed_index: p = ((nt * KBLK + kb) * 64 + lane) * KPL + j
  const int j = (int)(p % F::KPL);
  const size_t q = p / F::KPL;
  const int lane = (int)(q % 64);
  const size_t r = q / 64;
  const int kblk = Kp / F::KB;
  const int kb = (int)(r % kblk);
  const int nt = (int)(r / kblk);
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
  int k_hs, n_hs, Kp;
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
      out[packed_index(h * p.k_hs + rr, h * p.n_hs + cc, p.Kp, F::KB, F::KPL)] = from_f32<T>(acc[i]);
  }
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
                       mt.K, mt.N, Kp, Np, reinterpret_cast<T*>(mt.out));
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // W_UQK[h] = W_UQ[h] W_UK[h]^T : rows d_LQ, cols d_L, reduce over d_nope
  {
    ProdArgs p{};
    p.Ab = a.W_UQ; p.a_hs = a.d_nope; p.a_rs = (long)a.H * a.d_nope; p.a_ds = 1;
    p.Bb = a.W_UK; p.b_hs = a.d_nope; p.b_ds = 1; p.b_cs = (long)a.H * a.d_nope;
    p.H = a.H; p.rows = a.d_q_latent; p.cols = a.d_latent; p.kd = a.d_nope;
    p.k_hs = 0; p.n_hs = R; p.Kp = ceil_div(a.d_q_latent, F::KB) * F::KB; p.out = a.P_QC;
    const long tiles = (long)a.H * ceil_div(p.rows, 16) * ceil_div(p.cols, 16);
    hipLaunchKernelGGL(absorb_product_kernel<T>, dim3((unsigned)((tiles + 3) / 4)), dim3(256), 0, s, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // W_UVO[h] = W_UV[h] W_O[h] : rows d_L, cols d_model, reduce over d_v
  {
    ProdArgs p{};
    p.Ab = a.W_UV; p.a_hs = a.d_v; p.a_rs = (long)a.H * a.d_v; p.a_ds = 1;
    p.Bb = a.W_O; p.b_hs = (long)a.d_v * a.d_model; p.b_ds = a.d_model; p.b_cs = 1;
    p.H = a.H; p.rows = a.d_latent; p.cols = a.d_model; p.kd = a.d_v;
    p.k_hs = a.d_latent; p.n_hs = 0; p.Kp = ceil_div(a.H * a.d_latent, F::KB) * F::KB; p.out = a.P_O;
    const long tiles = (long)a.H * ceil_div(p.rows, 16) * ceil_div(p.cols, 16);
    hipLaunchKernelGGL(absorb_product_kernel<T>, dim3((unsigned)((tiles + 3) / 4)), dim3(256), 0, s, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t launch_absorb(const AbsorbArgs& a, bool bf16, hipStream_t s) {
  return bf16 ? absorb_t<__bf16>(a, s) : absorb_t<float>(a, s);
}

}  // namespace mla
