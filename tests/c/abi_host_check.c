/* A plain C caller of the library: no Python, no torch. Creates plans for the layer's
 * shapes, and checks that argument errors are reported before any device work (these calls
 * need no GPU). Exit status 0 when every check holds; the first failing check is printed. */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "sparse_attn.h"

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s (last error: %s)\n", \
              __LINE__, #cond, sparse_attn_last_error());             \
      return 1;                                                       \
    }                                                                 \
  } while (0)

static sa_params layer(int ratio, int key_dtype, int kv_dtype) {
  sa_params p;
  memset(&p, 0, sizeof p);
  p.num_heads = 64;
  p.latent_dim = 512;
  p.window = 128;
  p.topk = 512;
  p.idx_heads = 16;
  p.idx_dim = 128;
  p.block = 8;
  p.cand_blocks = 2048;
  p.ratio = ratio;
  p.idx_key_dtype = key_dtype;
  p.softmax_scale = 1.0f / sqrtf(512.0f);
  p.max_queries = 128;
  p.max_compressed = 65536;
  p.kv_dtype = kv_dtype;
  return p;
}

int main(void) {
  sa_plan* plan = NULL;
  size_t ws = 0;
  for (int kd = 0; kd <= 2; ++kd) {
    for (int kv = 0; kv <= 2; ++kv) {
      sa_params p = layer(2, kd, kv);
      CHECK(sparse_attn_plan(&p, &plan, &ws) == SA_OK);
      CHECK(plan != NULL && ws > 0);
      CHECK(sparse_attn_last_error()[0] == '\0');
      sparse_attn_plan_destroy(plan);
      plan = NULL;
    }
  }
  /* unsupported shapes and values are refused with a message */
  sa_params bad = layer(3, 0, 0);
  CHECK(sparse_attn_plan(&bad, &plan, &ws) == SA_EUNSUPPORTED && plan == NULL);
  CHECK(strlen(sparse_attn_last_error()) > 0);
  bad = layer(2, 0, 0);
  bad.num_heads = 32;
  CHECK(sparse_attn_plan(&bad, &plan, &ws) == SA_EUNSUPPORTED);
  bad = layer(2, 0, 7);
  CHECK(sparse_attn_plan(&bad, &plan, &ws) == SA_EUNSUPPORTED);

  /* calls with missing arguments return SA_EINVAL before touching the device */
  sa_params p = layer(2, 1, 0);
  CHECK(sparse_attn_plan(&p, &plan, &ws) == SA_OK);
  CHECK(indexer_score(plan, NULL, NULL, NULL, NULL, NULL, 0, NULL, 0, NULL) == SA_EINVAL);
  CHECK(select_topk(plan, NULL, NULL, 0, NULL, 0, NULL, NULL, NULL, 0, NULL) == SA_EINVAL);
  CHECK(sparse_attn_fwd(plan, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == SA_EINVAL);
  CHECK(sparse_attn_compress(plan, NULL, 1024, NULL, 1024, NULL, NULL, 512, 4, NULL) == SA_EINVAL);
  CHECK(sparse_attn_compress_codes(plan, NULL, 1024, NULL, 1024, NULL, NULL, 512, NULL, 4, 4, NULL) ==
        SA_EUNSUPPORTED);
  sparse_attn_plan_destroy(plan);
  printf("abi host checks ok\n");
  return 0;
}
