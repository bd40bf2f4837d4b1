// Cache store: given fp32 rows into the cache slots of their positions, as
// bf16 / fp32 rows or as E4M3 codes with one power-of-two scale per row.
//
// E4M3 (OCP e4m3fn) row quantiser: k is the smallest integer >= -126 with
// amax <= 448 * 2^k, read off the binary exponent of the row's fp32 amax
// (amax = f 2^e, f in [0.5, 1): k = e - 9 when f <= 0.875, since
// 448 = 0.875 * 2^9, else e - 8), so the decision is an exact comparison;
// the row is multiplied by 2^-k (exact) and each value rounded to the
// nearest code, ties to even, by the hardware conversion (values at most
// 448 in magnitude, where it follows the format exactly).  The cache then
// holds codes and 2^k; code * 2^k is exactly a bf16 value.
#include <math.h>

#include "mla_common.h"
#include "mla_internal.h"

namespace mla {

namespace {

// One wave per row: lane l takes column pairs l, l + 64, ... (RoPE pairs
// never straddle two lanes: d_latent is even).
__global__ __launch_bounds__(64) void cache_store_kernel(StoreArgs a) {
  const int m = blockIdx.x, lane = threadIdx.x;
  if (m >= a.M) return;
  const int b = m / a.n_q, t = m - b * a.n_q;
  const int pos = a.pos[b] + t;
  long long slot = -1;
  if (a.paged) {
    if (pos < 0 || pos >= a.max_pages * a.page_size) {
      if (lane == 0) atomicOr(a.err, 1);
    } else {
      const int pg = a.page_table[(size_t)b * a.max_pages + pos / a.page_size];
      if (pg < 0 || pg >= a.n_pages) {
        if (lane == 0) atomicOr(a.err, 2);
      } else {
        slot = (long long)pg * a.page_size + pos % a.page_size;
      }
    }
  } else if (pos < 0 || pos >= a.s_max) {
    if (lane == 0) atomicOr(a.err, 1);
  } else {
    slot = (long long)b * a.s_max + pos;
  }
  if (slot < 0) return;  // uniform over the wave
  const int pairs = a.R / 2;
  constexpr int MAXP = 8;  // pairs per lane: R <= 1024
  float2 v[MAXP];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < MAXP; ++i) {
    const int p = lane + 64 * i;
    v[i] = make_float2(0.f, 0.f);
    if (p < pairs) {
      v[i] = *reinterpret_cast<const float2*>(a.rows + (size_t)m * a.R + 2 * p);
      if (a.rope && 2 * p >= a.d_latent) {
        float c, sn;
        rope_cos_sin(pos, p - a.d_latent / 2, a.d_rope, a.rope_base, &c, &sn);
        const float x0 = v[i].x, x1 = v[i].y;
        v[i].x = x0 * c - x1 * sn;
        v[i].y = x0 * sn + x1 * c;
      }
      amax = fmaxf(amax, fmaxf(fabsf(v[i].x), fabsf(v[i].y)));
    }
  }
  unsigned char* row = reinterpret_cast<unsigned char*>(a.pool);
  if (a.format == 1) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    int e = 0;
    const float f = frexpf(amax, &e);
    int k = (f <= 0.875f) ? e - 9 : e - 8;
    if (k < -126) k = -126;
    if (!(amax > 0.f) || !isfinite(amax)) k = 0;  // zero row: scale 1; non-finite values give NaN codes
    const float inv = ldexpf(1.f, -k);
    row += slot * a.R;
#pragma unroll
    for (int i = 0; i < MAXP; ++i) {
      const int p = lane + 64 * i;
      if (p < pairs) {
        const unsigned w = __builtin_amdgcn_cvt_pk_fp8_f32(v[i].x * inv, v[i].y * inv, 0, false);
        *reinterpret_cast<uint16_t*>(row + 2 * p) = (uint16_t)(w & 0xFFFF);
      }
    }
    if (lane == 0) a.scales[slot] = ldexpf(1.f, k);
  } else if (a.bf16) {
    __bf16* r = reinterpret_cast<__bf16*>(row) + slot * a.R;
#pragma unroll
    for (int i = 0; i < MAXP; ++i) {
      const int p = lane + 64 * i;
      if (p < pairs) {
        r[2 * p] = (__bf16)v[i].x;
        r[2 * p + 1] = (__bf16)v[i].y;
      }
    }
  } else {
    float* r = reinterpret_cast<float*>(row) + slot * a.R;
#pragma unroll
    for (int i = 0; i < MAXP; ++i) {
      const int p = lane + 64 * i;
      if (p < pairs) *reinterpret_cast<float2*>(r + 2 * p) = v[i];
    }
  }
}

}  // namespace

hipError_t launch_cache_store(const StoreArgs& a, hipStream_t s) {
  if (a.R <= 0 || a.R > 1024 || (a.R & 1) || (a.d_latent & 1)) return hipErrorInvalidValue;
  if (a.M <= 0) return hipSuccess;
  hipLaunchKernelGGL(cache_store_kernel, dim3(a.M), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
