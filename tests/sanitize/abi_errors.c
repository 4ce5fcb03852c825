/* Host-only driver of the C ABI, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer together with the library's host layer (api.cpp)
 * and stand-in launchers (launch_stubs.cpp) that run nothing on a device.
 * It drives every argument-validation path of every entry point (all of them
 * return before any device call), the workspace-size queries, the error
 * names, the profiling record, and the SpaCO chunk selector, whose choices it
 * prints as "select k t seed : i0 i1 ..." lines for the test to compare with
 * the oracle's selector. Prints "ok <checks>" and exits 0 when every check
 * holds. */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "chunk_attn.h"

static int checks = 0, fails = 0;
#define EXPECT(cond)                                                                         \
  do {                                                                                       \
    ++checks;                                                                                \
    if (!(cond)) {                                                                           \
      ++fails;                                                                               \
      printf("FAIL line %d: %s (last error: %s)\n", __LINE__, #cond, chunk_attn_last_error()); \
    }                                                                                        \
  } while (0)

#define FAKE ((void*)0x10000) /* 16-byte aligned, never dereferenced */
#define MIS ((void*)0x10008)

static chunk_attn_desc base(void) {
  chunk_attn_desc d = {1, 4, 2, 128, 1024, 256, 0, 512, 256, 1.0f, CA_BF16};
  return d;
}

static int fwd(const chunk_attn_desc* d, void* q, void* v) {
  return chunk_attn_fwd(d, q, FAKE, v, FAKE, (float*)FAKE, NULL, 0, NULL);
}

static int bwd(const chunk_attn_desc* d, void* ws, size_t ws_bytes, float gs, void* dq) {
  return chunk_attn_bwd(d, FAKE, FAKE, FAKE, FAKE, (const float*)FAKE, FAKE, gs, (float*)dq, (float*)FAKE,
                        (float*)FAKE, ws, ws_bytes, NULL);
}

static void descriptor_errors(void) {
  chunk_attn_desc d;
  const int n = 13;
  for (int i = 0; i < n; ++i) {
    d = base();
    int want = CA_ERR_SHAPE;
    switch (i) {
      case 0: d.dtype = 7; want = CA_ERR_DTYPE; break;
      case 1: d.head_dim = 96; want = CA_ERR_UNSUPPORTED; break;
      case 2: d.head_dim = 256; want = CA_ERR_UNSUPPORTED; break;
      case 3: d.n_q_heads = 6; d.n_kv_heads = 4; break;
      case 4: d.n_kv_heads = 0; break;
      case 5: d.batch = 0; break;
      case 6: d.chunk_len = 0; break;
      case 7: d.chunk_start = 900; break;
      case 8: d.q_row_offset = 1; break;
      case 9: d.chunk_start = -1; break;
      case 10: d.softmax_scale = NAN; break;
      case 11: d.softmax_scale = INFINITY; break;
      case 12: d.batch = 65535; d.n_q_heads = 65535; d.n_kv_heads = 1; break;
    }
    EXPECT(fwd(&d, FAKE, FAKE) == want);
    EXPECT(bwd(&d, FAKE, 1 << 20, 1.0f, FAKE) == want);
    EXPECT(chunk_attn_bwd_noalloc(&d, FAKE, FAKE, FAKE, FAKE, (const float*)FAKE, FAKE, 1.0f, (float*)FAKE,
                                  (float*)FAKE, (float*)FAKE, NULL) == want);
    EXPECT(chunk_attn_workspace_size(&d, CA_OP_BWD) == 0);
    EXPECT(strlen(chunk_attn_last_error()) > 0);
  }
}

static void pointer_and_workspace_errors(void) {
  chunk_attn_desc d = base();
  EXPECT(fwd(NULL, FAKE, FAKE) == CA_ERR_NULL);
  EXPECT(fwd(&d, NULL, FAKE) == CA_ERR_NULL);
  EXPECT(fwd(&d, FAKE, MIS) == CA_ERR_ALIGN);
  EXPECT(bwd(&d, FAKE, 1 << 20, 1.0f, MIS) == CA_ERR_ALIGN);
  EXPECT(bwd(&d, FAKE, 1 << 20, NAN, FAKE) == CA_ERR_SHAPE);
  const size_t need = chunk_attn_workspace_size(&d, CA_OP_BWD_MIN);
  EXPECT(need >= 4 * 4 * 256 && need % 256 == 0);
  EXPECT(chunk_attn_workspace_size(&d, CA_OP_FWD) == 0);
  EXPECT(chunk_attn_workspace_size(&d, CA_OP_BWD) >= need);
  EXPECT(chunk_attn_workspace_size(&d, 99) == 0);
  EXPECT(chunk_attn_workspace_size(NULL, CA_OP_BWD) == 0);
  EXPECT(bwd(&d, NULL, 0, 1.0f, FAKE) == CA_ERR_WORKSPACE);
  EXPECT(bwd(&d, FAKE, need - 1, 1.0f, FAKE) == CA_ERR_WORKSPACE);
  EXPECT(bwd(&d, MIS, need, 1.0f, FAKE) == CA_ERR_ALIGN);
  /* the allocation-free backward: rows beyond its static scratch */
  chunk_attn_desc big = base();
  big.n_q_heads = 64;
  big.n_kv_heads = 8;
  big.q_capacity = big.kv_capacity = 32768;
  big.chunk_start = 0;
  big.chunk_len = 32768;
  EXPECT(chunk_attn_bwd_noalloc(&big, FAKE, FAKE, FAKE, FAKE, (const float*)FAKE, FAKE, 1.0f, (float*)FAKE,
                                (float*)FAKE, (float*)FAKE, NULL) == CA_ERR_WORKSPACE);
  EXPECT(chunk_attn_bwd_noalloc(&d, FAKE, FAKE, FAKE, FAKE, (const float*)FAKE, FAKE, 1.0f, (float*)MIS,
                                (float*)FAKE, (float*)FAKE, NULL) == CA_ERR_ALIGN);
}

static void accumulate_and_sparse_errors(void) {
  float* F = (float*)FAKE;
  EXPECT(prefix_grad_accumulate(NULL, F, 1, 1, 8, 8, 64, 4, 1.0f, NULL) == CA_ERR_NULL);
  EXPECT(prefix_grad_accumulate((float*)MIS, F, 1, 1, 8, 8, 64, 4, 1.0f, NULL) == CA_ERR_ALIGN);
  EXPECT(prefix_grad_accumulate(F, F, 1, 1, 8, 8, 64, 9, 1.0f, NULL) == CA_ERR_SHAPE);
  EXPECT(prefix_grad_accumulate(F, F, 1, 1, 8, 8, 6, 4, 1.0f, NULL) == CA_ERR_SHAPE);
  EXPECT(prefix_grad_accumulate(F, F, 0, 1, 8, 8, 64, 4, 1.0f, NULL) == CA_ERR_SHAPE);
  chunk_attn_desc d = base();
  d.chunk_start = 0;
  d.chunk_len = 128;
  d.q_capacity = 1024;
  int32_t sel[16];
  const size_t ws = 1 << 20;
#define SPARSE(seq, t, selp, wsb) \
  sparse_chunk_bwd(&d, seq, t, 0, FAKE, FAKE, FAKE, FAKE, F, FAKE, F, F, F, selp, FAKE, wsb, NULL)
  EXPECT(SPARSE(1024, 9, sel, ws) == CA_ERR_SHAPE); /* t > k = 8 */
  EXPECT(SPARSE(1024, 0, sel, ws) == CA_ERR_SHAPE);
  EXPECT(SPARSE(2048, 2, sel, ws) == CA_ERR_SHAPE); /* past the capacities */
  EXPECT(SPARSE(1024, 2, NULL, ws) == CA_ERR_NULL);
  EXPECT(SPARSE(1024, 2, sel, 16) == CA_ERR_WORKSPACE);
#undef SPARSE
}

static void sweep_errors(void) {
  chunk_attn_desc d = base();
  d.chunk_start = 0;
  d.chunk_len = 128;
  d.q_capacity = 1024;
  float* F = (float*)FAKE;
  EXPECT(chunked_fwd_sweep(NULL, 1024, FAKE, FAKE, FAKE, FAKE, F, NULL) == CA_ERR_NULL);
  EXPECT(chunked_fwd_sweep(&d, 0, FAKE, FAKE, FAKE, FAKE, F, NULL) == CA_ERR_SHAPE);
  EXPECT(chunked_fwd_sweep(&d, 1025, FAKE, FAKE, FAKE, FAKE, F, NULL) == CA_ERR_SHAPE);
  EXPECT(chunked_fwd_sweep(&d, 1024, FAKE, MIS, FAKE, FAKE, F, NULL) == CA_ERR_ALIGN);
#define BS(seq, gs, wsp, wsb) chunked_bwd_sweep(&d, seq, FAKE, FAKE, FAKE, FAKE, F, FAKE, gs, F, F, F, wsp, wsb, NULL)
  EXPECT(BS(2048, 1.0f, FAKE, 1 << 20) == CA_ERR_SHAPE);
  EXPECT(BS(1024, INFINITY, FAKE, 1 << 20) == CA_ERR_SHAPE);
  EXPECT(BS(1024, 1.0f, NULL, 0) == CA_ERR_WORKSPACE);
  EXPECT(BS(1024, 1.0f, FAKE, 16) == CA_ERR_WORKSPACE);
#undef BS
}

static void selector(void) {
  static const int32_t ks[] = {1, 2, 3, 4, 5, 16, 17, 64, 129};
  static const uint64_t seeds[] = {0ull, 1ull, 12345ull, 9223372036854775815ull, 18446744073709551615ull};
  int32_t out[129];
  for (size_t a = 0; a < sizeof ks / sizeof ks[0]; ++a) {
    const int32_t k = ks[a];
    const int32_t ts[] = {1, 2, k / 3 > 0 ? k / 3 : 1, k};
    for (int b = 0; b < 4; ++b) {
      if (ts[b] > k) continue;
      for (size_t c = 0; c < sizeof seeds / sizeof seeds[0]; ++c) {
        EXPECT(chunk_select(k, ts[b], seeds[c], out) == CA_OK);
        printf("select %d %d %llu :", k, ts[b], (unsigned long long)seeds[c]);
        for (int i = 0; i < ts[b]; ++i) printf(" %d", out[i]);
        printf("\n");
      }
    }
  }
  EXPECT(chunk_select(4, 5, 0, out) == CA_ERR_SHAPE);
  EXPECT(chunk_select(4, 0, 0, out) == CA_ERR_SHAPE);
  EXPECT(chunk_select(0, 1, 0, out) == CA_ERR_SHAPE);
  EXPECT(chunk_select(4, 1, 0, NULL) == CA_ERR_NULL);
}

static void projection_stack_head_errors(void) {
  chunk_attn_desc d = base();
  float* F = (float*)FAKE;
  EXPECT(qkv_proj_bwd_workspace_size(&d, 256) > 0);
  EXPECT(qkv_proj_bwd_workspace_size(&d, 96) == 0);
  EXPECT(qkv_proj_bwd_workspace_size(NULL, 256) == 0);
#define PB(dm, hcap, h, wsp, wsb) \
  qkv_proj_bwd(&d, dm, hcap, 512, h, FAKE, FAKE, FAKE, F, F, F, F, F, F, F, wsp, wsb, NULL)
  EXPECT(PB(256, 1024, FAKE, NULL, 0) == CA_ERR_WORKSPACE);
  EXPECT(PB(96, 1024, FAKE, FAKE, 1 << 26) == CA_ERR_SHAPE);
  EXPECT(PB(256, 700, FAKE, FAKE, 1 << 26) == CA_ERR_SHAPE);
  EXPECT(PB(256, 1024, NULL, FAKE, 1 << 26) == CA_ERR_NULL);
#undef PB
  EXPECT(qkv_proj_weights_t_bytes(&d, 256) > 0);
  EXPECT(qkv_proj_weights_t_bytes(NULL, 256) == 0);
  EXPECT(qkv_proj_weights_t(&d, 96, FAKE, FAKE, FAKE, FAKE, NULL) == CA_ERR_SHAPE);
  EXPECT(qkv_proj_weights_t(&d, 256, FAKE, FAKE, FAKE, NULL, NULL) == CA_ERR_NULL);
  EXPECT(qkv_proj_weights_t(NULL, 256, FAKE, FAKE, FAKE, FAKE, NULL) == CA_ERR_NULL);
  {
    chunk_attn_desc f = base();
    f.dtype = CA_F32;
    EXPECT(qkv_proj_weights_t(&f, 256, FAKE, FAKE, FAKE, FAKE, NULL) == CA_ERR_DTYPE);
  }
#define PBW(wt, wsp, wsb) \
  qkv_proj_bwd_wt(&d, 256, 1024, 512, FAKE, FAKE, FAKE, FAKE, wt, F, F, F, F, F, F, F, wsp, wsb, NULL)
  EXPECT(PBW(NULL, FAKE, 1 << 26) == CA_ERR_NULL);
  EXPECT(PBW(MIS, FAKE, 1 << 26) == CA_ERR_ALIGN);
  EXPECT(PBW(FAKE, NULL, 0) == CA_ERR_WORKSPACE);
#undef PBW
  EXPECT(qkv_proj_fwd(&d, 96, 1024, 512, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL) == CA_ERR_SHAPE);
  EXPECT(qkv_proj_fwd(&d, 256, 1024, 512, FAKE, FAKE, MIS, FAKE, FAKE, FAKE, FAKE, NULL) == CA_ERR_ALIGN);

  chunk_attn_desc s = base();
  s.chunk_start = 0;
  s.chunk_len = 128;
  s.q_capacity = 128;
  s.n_q_heads = 2;
  s.n_kv_heads = 1;
  spaco_layer lay[2];
  for (int i = 0; i < 2; ++i) {
    lay[i].wq = lay[i].wk = lay[i].wv = FAKE;
    lay[i].k_cache = lay[i].v_cache = FAKE;
    lay[i].dk_acc = lay[i].dv_acc = lay[i].dwq = lay[i].dwk = lay[i].dwv = F;
  }
  int32_t ch[3] = {0, 3, 5};
  const size_t need = spaco_stack_workspace_size(&s, 2);
  EXPECT(need > 0);
  EXPECT(spaco_stack_workspace_size(&s, 0) == 0);
#define SB(seq, L, layers, chunks, n, factor, wsb) \
  spaco_stack_backward(&s, seq, L, layers, FAKE, F, F, 1024, chunks, n, factor, FAKE, wsb, NULL)
  EXPECT(SB(1024, 0, lay, ch, 3, 2.0f, need) == CA_ERR_SHAPE);
  EXPECT(SB(1024, 2, NULL, ch, 3, 2.0f, need) == CA_ERR_NULL);
  EXPECT(SB(1024, 2, lay, ch, 3, 2.0f, need - 1) == CA_ERR_WORKSPACE);
  EXPECT(SB(1024, 2, lay, ch, 3, NAN, need) == CA_ERR_SHAPE);
  EXPECT(SB(1024, 2, lay, ch, 9, 2.0f, need) == CA_ERR_SHAPE);
  int32_t bad[3] = {0, 8, 5}, rep[3] = {1, 3, 1};
  EXPECT(SB(1024, 2, lay, bad, 3, 2.0f, need) == CA_ERR_SHAPE);
  EXPECT(SB(1024, 2, lay, rep, 3, 2.0f, need) == CA_ERR_SHAPE);
  EXPECT(SB(2048, 2, lay, ch, 3, 2.0f, need) == CA_ERR_SHAPE);
  lay[1].dwk = NULL;
  EXPECT(SB(1024, 2, lay, ch, 3, 2.0f, need) == CA_ERR_NULL);
#undef SB
  EXPECT(spaco_stack_forward(&s, 1024, 2, lay, FAKE, 1024, FAKE, need - 1, NULL) == CA_ERR_WORKSPACE);

  lm_head_desc h = {1, 1024, 256, 1024, CA_BF16};
  const size_t hneed = lm_head_sft_workspace_size(&h, 100);
  EXPECT(hneed > 0);
  lm_head_desc hv = h;
  hv.vocab = 1000;
  EXPECT(lm_head_sft_workspace_size(&hv, 100) == 0);
  EXPECT(lm_head_sft_workspace_size(&h, 0) == 0);
#define HP(dd, rs, rows, labels, scale, wsb) \
  lm_head_sft_partition(dd, rs, rows, FAKE, FAKE, FAKE, labels, NULL, scale, F, F, F, FAKE, wsb, NULL)
  lm_head_desc hf = h;
  hf.dtype = CA_F32;
  EXPECT(HP(&hf, 0, 100, (const int32_t*)FAKE, 1.0f, hneed) == CA_ERR_UNSUPPORTED);
  EXPECT(HP(&h, 1000, 100, (const int32_t*)FAKE, 1.0f, hneed) == CA_ERR_SHAPE);
  EXPECT(HP(&h, 0, 0, (const int32_t*)FAKE, 1.0f, hneed) == CA_ERR_SHAPE);
  EXPECT(HP(&h, 0, 100, NULL, 1.0f, hneed) == CA_ERR_NULL);
  EXPECT(HP(&h, 0, 100, (const int32_t*)MIS, 1.0f, hneed) == CA_ERR_ALIGN);
  EXPECT(HP(&h, 0, 100, (const int32_t*)FAKE, 1.0f, hneed - 1) == CA_ERR_WORKSPACE);
  EXPECT(HP(&h, 0, 100, (const int32_t*)FAKE, INFINITY, hneed) == CA_ERR_SHAPE);
#undef HP
  EXPECT(lm_head_transpose(NULL, FAKE, FAKE, NULL) == CA_ERR_NULL);
  EXPECT(lm_head_transpose(&hv, FAKE, FAKE, NULL) == CA_ERR_SHAPE);
  float loss = 0.f, c = 0.f;
  EXPECT(lm_head_dpo_finish(&h, 100, F, 0.f, 0.f, 0.1f, F, F, &loss, &c, NULL) == CA_ERR_SHAPE);
  lm_head_desc h2 = h;
  h2.batch = 2;
  EXPECT(lm_head_dpo_finish(&h2, 100, F, 0.f, 0.f, 0.1f, F, F, NULL, &c, NULL) == CA_ERR_NULL);
}

static void names_and_profiling(void) {
  const int codes[] = {CA_OK, CA_ERR_NULL, CA_ERR_SHAPE, CA_ERR_DTYPE, CA_ERR_ALIGN, CA_ERR_WORKSPACE,
                       CA_ERR_UNSUPPORTED, CA_ERR_HIP};
  for (int i = 0; i < 8; ++i) EXPECT(strlen(chunk_attn_strerror(codes[i])) > 0);
  EXPECT(strcmp(chunk_attn_strerror(-99), "unknown error") == 0);
  int64_t n = -1;
  double ms = -1.0;
  EXPECT(chunk_attn_profile_start() == CA_OK);
  EXPECT(chunk_attn_profile_select(1u << CA_KERNEL_FWD) == CA_OK);
  EXPECT(chunk_attn_profile_stop() == CA_OK);
  EXPECT(chunk_attn_profile_read(CA_KERNEL_DKDV, &n, &ms) == CA_OK && n == 0 && ms == 0.0);
  EXPECT(chunk_attn_profile_read(CA_KERNEL_COUNT, &n, &ms) == CA_ERR_SHAPE);
  EXPECT(chunk_attn_profile_read(-1, &n, &ms) == CA_ERR_SHAPE);
  EXPECT(chunk_attn_profile_read(CA_KERNEL_FWD, NULL, &ms) == CA_ERR_NULL);
}

int main(void) {
  descriptor_errors();
  pointer_and_workspace_errors();
  accumulate_and_sparse_errors();
  sweep_errors();
  selector();
  projection_stack_head_errors();
  names_and_profiling();
  if (fails) {
    printf("%d of %d checks failed\n", fails, checks);
    return 1;
  }
  printf("ok %d\n", checks);
  return 0;
}
