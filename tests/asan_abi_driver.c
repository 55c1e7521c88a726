/* Host driver for the AddressSanitizer build of the C-ABI validation layer.
 *
 * Calls every entry point of dg.h on its argument, configuration and handle
 * checks -- the paths that run on the host before any device work, so it runs
 * without a GPU -- and checks each returned status.  Built and run by
 * tests/test_host_asan.py against a libdg whose dg_api.cpp host code carries
 * AddressSanitizer; an out-of-bounds access, use after free or double free on
 * these paths aborts the run.  Prints "ASAN_DRIVER_OK n" after n checks. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dg.h"

static int n_checks = 0, n_fail = 0;

static void expect(int got, int want, const char* what) {
  ++n_checks;
  if (got != want) {
    ++n_fail;
    fprintf(stderr, "FAIL %s: status %d, expected %d (%s)\n", what, got, want, dg_last_error());
  } else if (want != DG_OK && dg_last_error()[0] == '\0') {
    ++n_fail;
    fprintf(stderr, "FAIL %s: no error text\n", what);
  }
}

static dg_config tiny(void) {
  dg_config c;
  memset(&c, 0, sizeof(c));
  c.n_layers = 1; c.d_model = 256; c.n_q_heads = 4; c.n_kv_heads = 4; c.head_dim = 64;
  c.n_experts = 8; c.ffn_hidden = 512; c.top_k = 2; c.vocab = 2048; c.canvas_len = 256;
  c.dtype = DG_DTYPE_BF16; c.self_cond = 1; c.rope_theta = 10000.f; c.rms_eps = 1e-6f;
  return c;
}

/* dg_model_create on a config with one field changed; the weight pointers are
 * all null, so a config that passes its checks still fails (DG_ERR_ARG). */
static int create_with(dg_config c) {
  const void* w[64];
  memset(w, 0, sizeof(w));
  dg_model* m = (dg_model*)0x1;
  int n = dg_weight_count(&c);
  int st = dg_model_create(&c, w, n > 0 && n <= 64 ? n : 0, &m);
  if (m != NULL) {
    ++n_fail;
    fprintf(stderr, "FAIL a failed dg_model_create left *out set\n");
  }
  return st;
}

int main(void) {
  dg_config c;
  /* configuration checks, one field at a time */
#define CASE(field, value, code)            \
  c = tiny();                               \
  c.field = value;                          \
  expect(create_with(c), code, #field " = " #value);
  CASE(n_layers, 0, DG_ERR_ARG)
  CASE(d_model, 100, DG_ERR_UNSUPPORTED)
  CASE(d_model, 1280, DG_ERR_UNSUPPORTED)
  CASE(d_model, 8192, DG_ERR_UNSUPPORTED)
  CASE(head_dim, 96, DG_ERR_UNSUPPORTED)
  CASE(n_kv_heads, 3, DG_ERR_ARG)
  CASE(n_q_heads, 0, DG_ERR_ARG)
  CASE(n_experts, 0, DG_ERR_UNSUPPORTED)
  CASE(n_experts, 129, DG_ERR_UNSUPPORTED)
  CASE(top_k, 0, DG_ERR_UNSUPPORTED)
  CASE(top_k, 9, DG_ERR_UNSUPPORTED)
  CASE(ffn_hidden, 100, DG_ERR_UNSUPPORTED)
  CASE(vocab, 1000, DG_ERR_UNSUPPORTED)
  CASE(vocab, 262208, DG_ERR_UNSUPPORTED)
  CASE(canvas_len, 0, DG_ERR_UNSUPPORTED)
  CASE(canvas_len, 257, DG_ERR_UNSUPPORTED)
  CASE(dtype, 7, DG_ERR_ARG)
  CASE(rope_theta, 0.f, DG_ERR_ARG)
  CASE(rms_eps, -1.f, DG_ERR_ARG)
  CASE(expert_dtype, 9, DG_ERR_ARG)
  CASE(expert_dtype, DG_DTYPE_FP8_E4M3, DG_ERR_UNSUPPORTED)   /* d_model 256: not a multiple of 512 */
  CASE(head_dtype, 9, DG_ERR_ARG)
#undef CASE
  c = tiny();
  c.dtype = DG_DTYPE_F32;
  c.head_dtype = DG_DTYPE_FP8_E4M3;
  expect(create_with(c), DG_ERR_UNSUPPORTED, "FP8 head on an fp32 model");
  c = tiny();
  expect(create_with(c), DG_ERR_ARG, "valid config, null weight pointers");
  {
    const void* w[64];
    memset(w, 0, sizeof(w));
    dg_model* m = NULL;
    expect(dg_model_create(&c, w, 3, &m), DG_ERR_ARG, "wrong weight count");
    expect(dg_model_create(NULL, w, 3, &m), DG_ERR_ARG, "null config");
    expect(dg_model_create(&c, NULL, dg_weight_count(&c), &m), DG_ERR_ARG, "null weight array");
    expect(dg_model_create(&c, w, dg_weight_count(&c), NULL), DG_ERR_ARG, "null out");
  }
  expect(dg_weight_count(NULL), -1, "dg_weight_count(NULL)");
  ++n_checks;
  if (dg_weight_count(&c) != 2 + 1 + 10 * c.n_layers) {
    ++n_fail;
    fprintf(stderr, "FAIL dg_weight_count\n");
  }

  /* null handles on every call that takes one */
  {
    void* p = NULL;
    size_t b = 0;
    uint64_t seeds[1] = {1};
    dg_sampler_params sp = {0.8f, 0.4f, 0.1f, 0.05f, 12, DG_STOP_NONE, 0};
    expect(dg_model_view(NULL, 0, 0, &p, &b), DG_ERR_ARG, "dg_model_view(NULL)");
    expect(dg_state_bytes(NULL, 1, 512, &b), DG_ERR_ARG, "dg_state_bytes(NULL)");
    expect(dg_state_init(NULL, NULL, 0, 1, 512, NULL), DG_ERR_ARG, "dg_state_init(NULL)");
    expect(dg_state_ctx_len(NULL), -1, "dg_state_ctx_len(NULL)");
    expect(dg_state_canvas_index(NULL), -1, "dg_state_canvas_index(NULL)");
    expect(dg_state_view(NULL, 0, &p, &b), DG_ERR_ARG, "dg_state_view(NULL)");
    expect(dg_init_canvas(NULL, NULL, seeds, NULL), DG_ERR_ARG, "dg_init_canvas(NULL)");
    expect(dg_encode_prompt(NULL, NULL, 4, NULL), DG_ERR_ARG, "dg_encode_prompt(NULL)");
    expect(dg_denoise_step(NULL, NULL, 0, &sp, seeds, NULL, NULL, NULL, NULL, NULL, NULL, NULL), DG_ERR_ARG,
           "dg_denoise_step(NULL)");
    expect(dg_sample_logits(NULL, NULL, 0, &sp, seeds, NULL, NULL, NULL, NULL, NULL, NULL), DG_ERR_ARG,
           "dg_sample_logits(NULL)");
    expect(dg_sample_commit(NULL, NULL, NULL, NULL, NULL, 0, &sp, seeds, NULL, NULL, NULL, NULL), DG_ERR_ARG,
           "dg_sample_commit(NULL)");
    expect(dg_commit_canvas_to_kv(NULL, NULL, NULL, NULL), DG_ERR_ARG, "dg_commit_canvas_to_kv(NULL)");
    expect(dg_run_canvas(NULL, NULL, &sp, seeds, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, 1, 0, NULL, NULL),
           DG_ERR_ARG, "dg_run_canvas(NULL)");
    expect(dg_corrupt_forward_loss(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL), DG_ERR_ARG,
           "dg_corrupt_forward_loss(NULL)");
    expect(dg_profile_enable(NULL, 1), DG_ERR_ARG, "dg_profile_enable(NULL)");
    expect(dg_profile_read(NULL, NULL, NULL), DG_ERR_ARG, "dg_profile_read(NULL)");
    dg_model_destroy(NULL);
    dg_state_destroy(NULL);
  }

  /* the allocation-free sampler's checks (never dereferences the fake buffers) */
  {
    void* fake = (void*)16;
    uint64_t seeds[1] = {1};
    dg_sampler_params sp = {0.8f, 0.4f, 0.1f, 0.05f, 12, DG_STOP_NONE, 0};
#define STATIC(rows, vocab, canvas, cidx, step) \
  dg_sample_logits_static((const float*)fake, rows, vocab, canvas, cidx, step, &sp, seeds, (float*)fake, \
                          (int32_t*)fake, (int32_t*)fake, (float*)fake, NULL)
    expect(STATIC(256, 4096, 256, 0, 12), DG_ERR_ARG, "static sampler: step past the budget");
    expect(STATIC(100, 4096, 256, 0, 0), DG_ERR_ARG, "static sampler: rows not whole canvases");
    expect(STATIC(256, 1000, 256, 0, 0), DG_ERR_UNSUPPORTED, "static sampler: vocabulary");
    expect(STATIC(256 * 129, 4096, 256, 0, 0), DG_ERR_UNSUPPORTED, "static sampler: requests");
    expect(STATIC(512, 262144, 256, 0, 0), DG_ERR_CAPACITY, "static sampler: scratch");
    expect(STATIC(256, 4096, 256, -1, 0), DG_ERR_ARG, "static sampler: canvas index");
    sp.top_k = 8;
    expect(STATIC(256, 4096, 256, 0, 0), DG_ERR_UNSUPPORTED, "static sampler: top_k");
    sp.top_k = 0;
    sp.max_steps = 0;
    expect(STATIC(256, 4096, 256, 0, 0), DG_ERR_ARG, "static sampler: max_steps");
#undef STATIC
  }

  if (n_fail) {
    fprintf(stderr, "%d of %d checks failed\n", n_fail, n_checks);
    return 1;
  }
  printf("ASAN_DRIVER_OK %d\n", n_checks);
  return 0;
}
