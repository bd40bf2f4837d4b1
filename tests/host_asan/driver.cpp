// Host-side paths of the MLA library under AddressSanitizer: sizing and
// layout queries, workspace fits and every argument check that returns
// before anything is enqueued.  No GPU work is launched (device addresses
// below are placeholders that the checks never dereference).
#include <initializer_list>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mla.h"

static int failures = 0;

static void expect(bool ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "FAILED: %s (%s)\n", what, mla_last_error());
    ++failures;
  }
}

static mla_dims dims(int d_model, int H, int dl, int dq, int dn, int dr, int dv, int dtype, int form) {
  mla_dims d;
  memset(&d, 0, sizeof d);
  d.d_model = d_model; d.n_heads = H; d.d_latent = dl; d.d_q_latent = dq; d.d_nope = dn; d.d_rope = dr;
  d.d_v = dv; d.dtype = dtype; d.rope_base = 10000.f; d.softmax_scale = 0.f; d.weight_form = form;
  return d;
}

static void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }

int main() {
  printf("%s\n", mla_version());
  for (int s = -6; s <= 1; ++s) expect(mla_status_str(s) != nullptr, "status string");

  const mla_dims shapes[] = {
      dims(5120, 128, 512, 1536, 128, 64, 128, MLA_BF16, MLA_WEIGHTS_MERGED),
      dims(5120, 128, 512, 1536, 128, 64, 128, MLA_BF16, MLA_WEIGHTS_FACTORED),
      dims(7168, 128, 512, 1536, 128, 64, 128, MLA_BF16, MLA_WEIGHTS_FACTORED),
      dims(64, 4, 32, 48, 16, 8, 16, MLA_F32, MLA_WEIGHTS_MERGED),
      dims(64, 4, 32, 48, 16, 8, 16, MLA_F32, MLA_WEIGHTS_FACTORED),
  };
  for (const mla_dims& d : shapes) {
    size_t off[4], sz[4], total = 0;
    expect(mla_absorbed_layout(&d, off, sz, &total) == MLA_OK && total > 0, "absorbed layout");
    for (int b : {1, 3, 16, 20, 23, 64}) {
      for (int nq : {1, 7, 64, 1024}) {
        size_t ws = 0;
        const int st = mla_workspace_size(&d, b, nq, &ws);
        if (st == MLA_ERR_UNSUPPORTED) {
          // a shape the size query refuses is refused by the check as well
          expect(mla_workspace_check(&d, b, nq, (size_t)1 << 40) == MLA_ERR_UNSUPPORTED, "check agrees with size");
          continue;
        }
        expect(st == MLA_OK && ws > 0, "workspace size");
        expect(mla_workspace_check(&d, b, nq, ws) == MLA_OK, "sized workspace fits");
        // fewer rows on the same workspace fit; far fewer bytes do not
        expect(mla_workspace_check(&d, (b + 1) / 2, nq, ws) == MLA_OK, "smaller call fits");
        expect(mla_workspace_check(&d, b, nq, 1024) == MLA_ERR_WORKSPACE, "tiny workspace refused");
      }
    }
  }
  const mla_dims v3 = shapes[2];
  size_t pf = 0;
  expect(mla_prefill_workspace_size(&v3, 2, 1024, 5120, &pf) == MLA_OK && pf > 0, "prefill workspace size");
  expect(mla_prefill_workspace_check(&v3, 2, 1024, 5120, pf) == MLA_OK, "prefill workspace fits");
  expect(mla_prefill_workspace_check(&v3, 2, 1024, 5120, pf / 2) == MLA_ERR_WORKSPACE, "prefill tiny workspace");

  // argument checks (no launch)
  const mla_dims d = shapes[0];
  mla_dims bad = d;
  bad.d_rope = 63;
  size_t n = 0;
  expect(mla_workspace_size(&bad, 16, 1, &n) == MLA_ERR_INVALID_ARG, "odd d_rope");
  expect(mla_workspace_size(nullptr, 16, 1, &n) == MLA_ERR_INVALID_ARG, "null dims");
  expect(mla_workspace_size(&d, 0, 1, &n) == MLA_ERR_INVALID_ARG, "zero batch");
  mla_cache c;
  memset(&c, 0, sizeof c);
  c.pool = P(0x1000);
  c.s_max = 4097;
  expect(mla_decode(&d, P(0x1000), nullptr, (const int32_t*)P(0x2000), 16, 1, &c, (float*)P(0x3000), nullptr,
                    P(0x100000), (size_t)1 << 40, nullptr) == MLA_ERR_INVALID_ARG, "null x");
  expect(mla_decode(&d, P(0x1000), P(0x1002), (const int32_t*)P(0x2000), 16, 1, &c, (float*)P(0x3000), nullptr,
                    P(0x100000), (size_t)1 << 40, nullptr) == MLA_ERR_INVALID_ARG, "misaligned x");
  expect(mla_attention(&d, P(0x1000), (const int32_t*)P(0x2000), 16, 1, &c, (float*)P(0x3000), nullptr,
                       P(0x100000), 1024, nullptr) == MLA_ERR_WORKSPACE, "small workspace");
  mla_cache e4 = c;
  e4.row_format = MLA_ROWS_E4M3;
  expect(mla_attention(&d, P(0x1000), (const int32_t*)P(0x2000), 16, 1, &e4, (float*)P(0x3000), nullptr,
                       P(0x100000), (size_t)1 << 40, nullptr) == MLA_ERR_INVALID_ARG, "E4M3 without scales");
  e4.row_format = 9;
  expect(mla_attention(&d, P(0x1000), (const int32_t*)P(0x2000), 16, 1, &e4, (float*)P(0x3000), nullptr,
                       P(0x100000), (size_t)1 << 40, nullptr) == MLA_ERR_INVALID_ARG, "unknown row format");
  mla_cache paged = c;
  paged.page_table = (const int32_t*)P(0x2000);
  paged.page_size = 48;
  paged.n_pages = 10;
  paged.max_pages_per_seq = 4;
  expect(mla_attention(&d, P(0x1000), (const int32_t*)P(0x2000), 16, 1, &paged, (float*)P(0x3000), nullptr,
                       P(0x100000), (size_t)1 << 40, nullptr) == MLA_ERR_INVALID_ARG, "page size not /32");
  expect(mla_attention_noalloc(&d, P(0x1000), (const int32_t*)P(0x2000), 1, 400, &c, (float*)P(0x3000), nullptr,
                               nullptr, nullptr) == MLA_ERR_WORKSPACE, "no-alloc beyond the scratch");
  expect(mla_cache_store_rows(&d, (const float*)P(0x1000), (const int32_t*)P(0x2000), 4, 1, &c, P(0x100000), 128,
                              nullptr) == MLA_ERR_WORKSPACE, "store needs the error word");
  const mla_dims f32 = shapes[3];
  mla_cache e4s = c;
  e4s.row_format = MLA_ROWS_E4M3;
  e4s.scales = (float*)P(0x4000);
  expect(mla_attention(&f32, P(0x1000), (const int32_t*)P(0x2000), 1, 1, &e4s, (float*)P(0x3000), nullptr,
                       P(0x100000), (size_t)1 << 40, nullptr) == MLA_ERR_UNSUPPORTED, "E4M3 on an fp32 layer");
  expect(mla_prefill_expanded(&v3, P(0x1000), P(0x2000), (const int32_t*)P(0x3000), 2, 8, &e4s, (float*)P(0x4000),
                              nullptr, P(0x100000), (size_t)1 << 40, nullptr) != MLA_OK, "expanded prefill on E4M3");
  printf("host checks: %d failures\n", failures);
  return failures ? 1 : 0;
}
