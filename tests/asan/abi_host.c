/* Host-side checks of the C ABI, run against a build of the library whose host
 * code is compiled with AddressSanitizer.  Every call here must be rejected
 * by the library's argument checks before it touches a device, so the program
 * needs no GPU: it exercises the validation paths and the error-message
 * formatting for heap or stack misuse.  Exit status = number of failed
 * expectations. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "flashmap.h"

static int failures = 0;

static void expect(int ok, const char* what) {
  if (!ok) {
    ++failures;
    fprintf(stderr, "FAILED: %s (last error: \"%s\")\n", what, fm_last_error());
  }
}

static void expect_status(fm_status got, fm_status want, const char* what) {
  char buf[256];
  snprintf(buf, sizeof buf, "%s: status %d, expected %d", what, (int)got, (int)want);
  expect(got == want, buf);
  if (want != FM_OK) expect(fm_last_error()[0] != '\0', "a failed call leaves a message");
}

static fm_config base_config(void) {
  fm_config c;
  memset(&c, 0, sizeof c);
  c.K = 16;
  c.V = 1024;
  c.d = 256;
  c.L = 2;
  c.n_heads = 4;
  c.mlp_mult = 4;
  c.H = 512;
  c.n_ctx_layers = 5;
  c.C_max = 64;
  c.max_branches = 1;
  c.max_new = 16;
  c.max_steps = 1;
  c.dtype = FM_F32;
  c.max_requests = 1;
  return c;
}

int main(void) {
  /* ---- configurations */
  fm_config c = base_config();
  const size_t n = fm_workspace_bytes(&c);
  expect(n > 0, "valid configuration has a workspace size");
  expect(fm_workspace_bytes(NULL) == 0, "NULL configuration");
  {
    fm_config bad[12];
    int i = 0;
    for (i = 0; i < 12; ++i) bad[i] = base_config();
    bad[0].K = 8;
    bad[1].d = 200;
    bad[2].n_heads = 3;
    bad[3].V = 10;
    bad[4].max_branches = 5;
    bad[5].n_ctx_layers = 4;
    bad[6].max_steps = 0;
    bad[7].d = 8192;
    bad[7].n_heads = 64;
    bad[8].dtype = (fm_dtype)7;
    bad[9].max_new = 17;
    bad[10].max_requests = 2;
    bad[10].max_branches = 4;
    bad[11].C_max = -1;
    for (i = 0; i < 12; ++i) {
      char what[64];
      snprintf(what, sizeof what, "invalid configuration %d is rejected", i);
      expect(fm_workspace_bytes(&bad[i]) == 0, what);
      expect(strlen(fm_last_error()) > 0, "the rejection has a message");
    }
  }
  /* a long run of failures must keep the message buffer consistent */
  {
    int i = 0;
    fm_config big = base_config();
    for (i = 0; i < 1000; ++i) {
      big.V = 17 + i;
      (void)fm_workspace_bytes(&big);
    }
  }

  /* ---- handle creation: every argument check fires before any device call */
  {
    fm_handle* h = NULL;
    void* fake = (void*)(uintptr_t)0x100000; /* never dereferenced */
    expect_status(fm_create(NULL, fake, n, 0, &h), FM_EINVAL, "fm_create(NULL config)");
    expect_status(fm_create(&c, fake, n, 0, NULL), FM_EINVAL, "fm_create(NULL out)");
    expect_status(fm_create(&c, NULL, n, 0, &h), FM_EINVAL, "fm_create(NULL workspace)");
    expect_status(fm_create(&c, (char*)fake + 4, n, 0, &h), FM_EINVAL, "fm_create(misaligned workspace)");
    expect_status(fm_create(&c, fake, n, -1, &h), FM_EINVAL, "fm_create(negative device)");
    expect_status(fm_create(&c, fake, n - 1, 0, &h), FM_ECAPACITY, "fm_create(workspace too small)");
    expect(h == NULL, "no handle after a failed create");
    fm_destroy(NULL);
  }

  /* ---- stateless greedy verify */
  {
    void* d = (void*)(uintptr_t)0x200000;
    expect_status(fm_verify(NULL, FM_BF16, 1, 16, 100, NULL, NULL, NULL, NULL, NULL), FM_EINVAL,
                  "fm_verify(NULL)");
    expect_status(fm_verify(d, FM_BF16, 0, 16, 100, d, d, d, d, NULL), FM_EINVAL, "fm_verify(B = 0)");
    expect_status(fm_verify(d, FM_BF16, 65, 16, 100, d, d, d, d, NULL), FM_EINVAL, "fm_verify(B = 65)");
    expect_status(fm_verify(d, FM_BF16, 1, 65, 100, d, d, d, d, NULL), FM_EINVAL, "fm_verify(K = 65)");
    expect_status(fm_verify(d, FM_BF16, 1, 16, 0, d, d, d, d, NULL), FM_EINVAL, "fm_verify(V = 0)");
    expect_status(fm_verify(d, (fm_dtype)7, 1, 16, 100, d, d, d, d, NULL), FM_EINVAL, "fm_verify(dtype)");
    expect_status(fm_verify((char*)d + 1, FM_BF16, 1, 16, 100, d, d, d, d, NULL), FM_EINVAL,
                  "fm_verify(misaligned logits)");
  }

  /* ---- the no-allocation verifier rejects what its static scratch cannot hold */
  {
    void* d = (void*)(uintptr_t)0x300000;
    float* f = (float*)d;
    int32_t* i32 = (int32_t*)d;
    expect_status(fm_verify_sample_noalloc(d, FM_BF16, 1, 16, 100, f, f, i32, 0.f, 1, i32, i32, NULL), FM_EINVAL,
                  "noalloc(temperature 0)");
    expect_status(fm_verify_sample_noalloc(d, FM_BF16, 1, 8, 100, f, f, i32, 1.f, 1, i32, i32, NULL), FM_EINVAL,
                  "noalloc(K = 8)");
    expect_status(fm_verify_sample_noalloc(d, FM_BF16, 5, 16, 100, f, f, i32, 1.f, 1, i32, i32, NULL), FM_ECAPACITY,
                  "noalloc(B = 5)");
  }

  /* ---- every handle call with a NULL handle */
  {
    void* d = (void*)(uintptr_t)0x400000;
    int32_t* i32 = (int32_t*)d;
    float* f = (float*)d;
    const int n_new[4] = {1, 1, 1, 1};
    const float times[2] = {0.f, 1.f};
    fm_weights w;
    memset(&w, 0, sizeof w);
    expect_status(fm_set_weights(NULL, &w), FM_EINVAL, "fm_set_weights(NULL handle)");
    expect_status(fm_set_schedule(NULL, times, 1, NULL), FM_EINVAL, "fm_set_schedule(NULL handle)");
    expect_status(fm_context_append(NULL, d, 1, NULL), FM_EINVAL, "fm_context_append(NULL handle)");
    expect_status(fm_context_truncate(NULL, 0, NULL), FM_EINVAL, "fm_context_truncate(NULL handle)");
    expect_status(fm_context_sync(NULL, NULL), FM_EINVAL, "fm_context_sync(NULL handle)");
    expect_status(fm_context_append_req(NULL, 0, d, 1, NULL), FM_EINVAL, "fm_context_append_req(NULL handle)");
    expect_status(fm_context_truncate_req(NULL, 0, 0, NULL), FM_EINVAL, "fm_context_truncate_req(NULL handle)");
    expect(fm_context_length(NULL) == -1, "fm_context_length(NULL handle)");
    expect(fm_context_length_req(NULL, 0) == -1, "fm_context_length_req(NULL handle)");
    expect_status(fm_draft(NULL, d, 1, NULL, 0, i32, NULL, NULL, NULL), FM_EINVAL, "fm_draft(NULL handle)");
    expect_status(fm_draft_sample(NULL, d, 1, NULL, 0, 1.f, 7, i32, f, f, NULL), FM_EINVAL,
                  "fm_draft_sample(NULL handle)");
    expect_status(fm_draft_batch(NULL, d, 4, d, n_new, i32, NULL, NULL), FM_EINVAL, "fm_draft_batch(NULL handle)");
    expect_status(fm_verify_greedy(NULL, d, FM_BF16, 1, i32, i32, i32, i32, NULL), FM_EINVAL,
                  "fm_verify_greedy(NULL handle)");
    expect_status(fm_verify_sample(NULL, d, FM_BF16, 1, f, f, i32, 1.f, 7, i32, i32, NULL), FM_EINVAL,
                  "fm_verify_sample(NULL handle)");
    expect_status(fm_set_probe(NULL, FM_PROBE_NONE, NULL, NULL), FM_EINVAL, "fm_set_probe(NULL handle)");
    {
      const uint64_t seeds[4] = {1, 2, 3, 4};
      expect_status(fm_draft_batch_sample(NULL, d, 4, d, n_new, 1.f, seeds, i32, f, f, NULL), FM_EINVAL,
                    "fm_draft_batch_sample(NULL handle)");
      expect_status(fm_draft_batch_sample(NULL, d, 4, d, n_new, 0.f, seeds, i32, f, f, NULL), FM_EINVAL,
                    "fm_draft_batch_sample(temperature 0)");
      expect_status(fm_draft_batch_sample(NULL, d, 4, d, n_new, 1.f, NULL, i32, f, f, NULL), FM_EINVAL,
                    "fm_draft_batch_sample(NULL seeds)");
      expect_status(fm_verify_sample_batch(NULL, d, FM_BF16, 4, f, f, i32, 1.f, seeds, i32, i32, NULL), FM_EINVAL,
                    "fm_verify_sample_batch(NULL handle)");
    }
  }

  if (failures == 0) printf("abi_host: all checks passed\n");
  return failures;
}
