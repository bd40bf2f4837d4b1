// Shared device helpers for the MLA library (gfx950 / CDNA4).
//
// MFMA fragment conventions (16x16 output tiles, 64-lane wavefront):
//   A operand  : lane l holds A[row = l % 16][k = (l / 16) * KPL + j], j < KPL
//   B operand  : lane l holds B[k = (l / 16) * KPL + j][col = l % 16]
//   C/D        : lane l holds D[row = 4 * (l / 16) + i][col = l % 16], i < 4
// bf16: v_mfma_f32_16x16x32_bf16 (K = 32 per instruction, KPL = 8)
// fp32: v_mfma_f32_16x16x4_f32   (K = 4 per instruction,  KPL = 1)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define MLA_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

template <typename T>
struct Mfma;

template <>
struct Mfma<__bf16> {
  static constexpr int KB = 32;   // k per instruction
  static constexpr int KPL = 8;   // k elements held per lane
  using frag = bf16x8;
  __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline frag zero() {
    frag z;
#pragma unroll
    for (int j = 0; j < 8; ++j) z[j] = (__bf16)0.0f;
    return z;
  }
};

template <>
struct Mfma<float> {
  static constexpr int KB = 4;
  static constexpr int KPL = 1;
  using frag = float;
  __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline frag zero() { return 0.0f; }
};

// Load KPL consecutive elements as one A/B fragment.
template <typename T>
__device__ inline typename Mfma<T>::frag load_frag(const T* p);
template <>
__device__ inline bf16x8 load_frag<__bf16>(const __bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
template <>
__device__ inline float load_frag<float>(const float* p) {
  return *p;
}

// Fragment of type T from fp32 source (converted with round-to-nearest-even).
template <typename T>
__device__ inline typename Mfma<T>::frag load_frag_from_f32(const float* p);
template <>
__device__ inline bf16x8 load_frag_from_f32<__bf16>(const float* p) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  bf16x8 r;
  r[0] = (__bf16)a.x; r[1] = (__bf16)a.y; r[2] = (__bf16)a.z; r[3] = (__bf16)a.w;
  r[4] = (__bf16)b.x; r[5] = (__bf16)b.y; r[6] = (__bf16)b.z; r[7] = (__bf16)b.w;
  return r;
}
template <>
__device__ inline float load_frag_from_f32<float>(const float* p) {
  return *p;
}

template <typename T>
__device__ inline T from_f32(float v) { return (T)v; }

// ------------------------------------------------------------------------
// Packed ("fragment-ordered") weight layout used by every streamed weight.
//
// A logical row-major matrix W[K][N] (y = x W) is stored as
//   [Kp/KB][ceil(N/16)][64 lanes][KPL]       Kp = roundup(K, KB)
// so that the B-operand fragment of one MFMA (16 columns x KB rows) is one
// contiguous 64*KPL-element block: lane l holds W[kb*KB + (l/16)*KPL + j]
// [nt*16 + l%16].  Fragments are k-block-major: the fragments of adjacent
// column tiles at one k-block are adjacent, so a wave that owns NT
// neighbouring tiles reads one contiguous NT-fragment run per k-block.
// Padding (rows >= K, columns >= N) is zero.
// ------------------------------------------------------------------------
__host__ __device__ inline size_t packed_index(int k, int n, int Np, int KB, int KPL) {
  const int nt = n >> 4, kb = k / KB, kk = k - kb * KB;
  const int lane = (n & 15) + 16 * (kk / KPL), j = kk % KPL;
  return ((size_t)kb * (size_t)(Np / 16) + (size_t)nt) * (size_t)(64 * KPL) + (size_t)(lane * KPL + j);
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ inline void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// LDS-only workgroup barrier: completes this wave's LDS traffic first.
__device__ inline void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// RoPE angle for pair j at integer position pos, built in fp64 so that
// positions up to ~1e5 keep full fp32 accuracy after sin/cos.
__device__ inline void rope_cos_sin(int pos, int j, int d_rope, float base, float* c, float* s) {
  const double theta = exp2(-(2.0 * (double)j / (double)d_rope) * log2((double)base));
  double sd, cd;
  sincos((double)pos * theta, &sd, &cd);
  *c = (float)cd;
  *s = (float)sd;
}

// Raises kernel K's dynamic LDS limit to `bytes` on the current device, once
// per device (the attribute is per device; setting it twice is harmless, so
// concurrent first calls only repeat it).  Devices beyond 64 set it on every
// call.
template <auto K>
inline hipError_t ensure_lds_limit(int bytes) {
  static std::atomic<uint64_t> done{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t{1} << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(K), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}
