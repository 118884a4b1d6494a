/* A plain C caller of the whole path on the GPU: no Python and no torch,
 * only the HIP runtime's C API for device memory and a stream.
 *
 *   step_c <inputs.bin> <outputs.bin>
 *
 * inputs.bin (little-endian): int32 header {R, B, Hq, Hkv, D, capacity,
 * qkv dtype (cpdec_dtype), chunk_tokens}, then q [B][Hq][D], K [R][B][Hkv][cap][D],
 * V (same) as 16-bit words, then lens [R][B] int32.
 *
 * The program sizes one workspace for both attention entry points, clears it
 * once, runs cpdec_cp_decode twice on it (the counter region must be zero
 * after each call), then cpdec_attn_partial + cpdec_lse_merge into a second
 * set of outputs, then cpdec_cp_decode_noalloc (no workspace) into a third,
 * and writes {o_part fp32, lse_part, out 16-bit, lse_out} of the first call,
 * of the second call, of the two-call form and of the allocation-free step
 * to outputs.bin. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "cpdec.h"

#define HIP_OK(x)                                                                   \
  do {                                                                              \
    hipError_t e_ = (x);                                                            \
    if (e_ != hipSuccess) {                                                         \
      fprintf(stderr, "%s failed: %s (line %d)\n", #x, hipGetErrorString(e_), __LINE__); \
      return 1;                                                                     \
    }                                                                               \
  } while (0)
#define CPDEC_OK_(x)                                                                \
  do {                                                                              \
    cpdec_status s_ = (x);                                                          \
    if (s_ != CPDEC_OK) {                                                           \
      fprintf(stderr, "%s failed: %s (line %d)\n", #x, cpdec_status_string(s_), __LINE__); \
      return 1;                                                                     \
    }                                                                               \
  } while (0)

typedef struct {
  void* o_part;
  float* lse_part;
  void* out;
  float* lse_out;
} outputs;

static int alloc_outputs(outputs* o, size_t n_opart, size_t n_lsep, size_t n_out, size_t n_lse) {
  HIP_OK(hipMalloc(&o->o_part, n_opart * 4));
  HIP_OK(hipMalloc((void**)&o->lse_part, n_lsep * 4));
  HIP_OK(hipMalloc(&o->out, n_out * 2));
  HIP_OK(hipMalloc((void**)&o->lse_out, n_lse * 4));
  return 0;
}

static int write_outputs(FILE* f, const outputs* o, size_t n_opart, size_t n_lsep, size_t n_out,
                         size_t n_lse) {
  const size_t bytes = n_opart * 4 + n_lsep * 4 + n_out * 2 + n_lse * 4;
  char* h = (char*)malloc(bytes);
  if (!h) return 1;
  char* p = h;
  HIP_OK(hipMemcpy(p, o->o_part, n_opart * 4, hipMemcpyDeviceToHost)); p += n_opart * 4;
  HIP_OK(hipMemcpy(p, o->lse_part, n_lsep * 4, hipMemcpyDeviceToHost)); p += n_lsep * 4;
  HIP_OK(hipMemcpy(p, o->out, n_out * 2, hipMemcpyDeviceToHost)); p += n_out * 2;
  HIP_OK(hipMemcpy(p, o->lse_out, n_lse * 4, hipMemcpyDeviceToHost));
  const int ok = fwrite(h, 1, bytes, f) == bytes;
  free(h);
  return ok ? 0 : 1;
}

static int counters_zero(const void* ws, int* zero) {
  unsigned char* h = (unsigned char*)malloc(CPDEC_STEP_COUNTER_BYTES);
  if (!h) return 1;
  HIP_OK(hipMemcpy(h, ws, CPDEC_STEP_COUNTER_BYTES, hipMemcpyDeviceToHost));
  *zero = 1;
  for (size_t i = 0; i < CPDEC_STEP_COUNTER_BYTES; ++i)
    if (h[i]) *zero = 0;
  free(h);
  return 0;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s inputs.bin outputs.bin\n", argv[0]);
    return 2;
  }
  FILE* fin = fopen(argv[1], "rb");
  if (!fin) { perror(argv[1]); return 1; }
  int32_t hdr[8];
  if (fread(hdr, 4, 8, fin) != 8) { fprintf(stderr, "short header\n"); return 1; }
  const int R = hdr[0], B = hdr[1], Hq = hdr[2], Hkv = hdr[3], D = hdr[4], cap = hdr[5];
  const size_t n_q = (size_t)B * Hq * D;
  const size_t n_shard = (size_t)B * Hkv * cap * D;
  const size_t n_kv = (size_t)R * n_shard;
  const size_t n_lens = (size_t)R * B;
  uint16_t* hq = (uint16_t*)malloc(n_q * 2);
  uint16_t* hk = (uint16_t*)malloc(n_kv * 2);
  uint16_t* hv = (uint16_t*)malloc(n_kv * 2);
  int32_t* hl = (int32_t*)malloc(n_lens * 4);
  if (!hq || !hk || !hv || !hl) { fprintf(stderr, "out of host memory\n"); return 1; }
  if (fread(hq, 2, n_q, fin) != n_q || fread(hk, 2, n_kv, fin) != n_kv ||
      fread(hv, 2, n_kv, fin) != n_kv || fread(hl, 4, n_lens, fin) != n_lens) {
    fprintf(stderr, "short input file\n");
    return 1;
  }
  fclose(fin);

  cpdec_attn_desc d;
  memset(&d, 0, sizeof d);
  d.batch = B; d.num_q_heads = Hq; d.num_kv_heads = Hkv; d.head_dim = D; d.num_shards = R;
  d.kv_capacity = cap;
  d.kv_stride_token = D; d.kv_stride_head = (int64_t)cap * D; d.kv_stride_batch = (int64_t)Hkv * cap * D;
  d.sm_scale = 0.f;
  d.qkv_dtype = (cpdec_dtype)hdr[6];
  d.opart_dtype = CPDEC_F32;
  d.chunk_tokens = hdr[7];

  void *q, *k, *v;
  int32_t* lens;
  HIP_OK(hipMalloc(&q, n_q * 2));
  HIP_OK(hipMalloc(&k, n_kv * 2));
  HIP_OK(hipMalloc(&v, n_kv * 2));
  HIP_OK(hipMalloc((void**)&lens, n_lens * 4));
  HIP_OK(hipMemcpy(q, hq, n_q * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(k, hk, n_kv * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(v, hv, n_kv * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(lens, hl, n_lens * 4, hipMemcpyHostToDevice));

  const void* ks[CPDEC_MAX_SHARDS];
  const void* vs[CPDEC_MAX_SHARDS];
  if (R < 1 || R > CPDEC_MAX_SHARDS) { fprintf(stderr, "bad shard count\n"); return 1; }
  for (int r = 0; r < R; ++r) {
    ks[r] = (const uint16_t*)k + (size_t)r * n_shard;
    vs[r] = (const uint16_t*)v + (size_t)r * n_shard;
  }

  const size_t n_opart = (size_t)R * B * Hq * D, n_lsep = (size_t)R * B * Hq;
  const size_t n_out = (size_t)B * Hq * D, n_lse = (size_t)B * Hq;
  outputs step1, step2, two, na;
  if (alloc_outputs(&step1, n_opart, n_lsep, n_out, n_lse) ||
      alloc_outputs(&step2, n_opart, n_lsep, n_out, n_lse) ||
      alloc_outputs(&two, n_opart, n_lsep, n_out, n_lse) ||
      alloc_outputs(&na, n_opart, n_lsep, n_out, n_lse))
    return 1;

  // one workspace serves both attention entry points
  size_t ws_bytes = cpdec_step_workspace_bytes(&d);
  const size_t ws_attn = cpdec_attn_workspace_bytes(&d);
  if (ws_attn > ws_bytes) ws_bytes = ws_attn;
  if (ws_bytes < CPDEC_STEP_COUNTER_BYTES) { fprintf(stderr, "workspace query failed\n"); return 1; }
  void* ws;
  HIP_OK(hipMalloc(&ws, ws_bytes));
  int32_t launches = 0;
  CPDEC_OK_(cpdec_step_plan(&d, &launches));

  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));
  CPDEC_OK_(cpdec_workspace_clear(ws, CPDEC_STEP_COUNTER_BYTES, s));
  int zero1 = 0, zero2 = 0;
  CPDEC_OK_(cpdec_cp_decode(&d, q, ks, vs, lens, step1.o_part, step1.lse_part, step1.out,
                            step1.lse_out, ws, ws_bytes, s));
  HIP_OK(hipStreamSynchronize(s));
  if (counters_zero(ws, &zero1)) return 1;
  CPDEC_OK_(cpdec_cp_decode(&d, q, ks, vs, lens, step2.o_part, step2.lse_part, step2.out,
                            step2.lse_out, ws, ws_bytes, s));
  HIP_OK(hipStreamSynchronize(s));
  if (counters_zero(ws, &zero2)) return 1;
  CPDEC_OK_(cpdec_attn_partial(&d, q, ks, vs, lens, two.o_part, two.lse_part, ws, ws_bytes, s));
  CPDEC_OK_(cpdec_lse_merge(two.o_part, two.lse_part, R, (int64_t)B * Hq, D, CPDEC_F32,
                            d.qkv_dtype, two.out, two.lse_out, s));
  HIP_OK(hipStreamSynchronize(s));
  if (!zero1 || !zero2) { fprintf(stderr, "counter region not zero after a call\n"); return 1; }
  // the same step with the library's static scratch: no workspace from the caller
  CPDEC_OK_(cpdec_cp_decode_noalloc(&d, q, ks, vs, lens, na.o_part, na.lse_part, na.out,
                                    na.lse_out, s));
  HIP_OK(hipStreamSynchronize(s));

  FILE* fout = fopen(argv[2], "wb");
  if (!fout) { perror(argv[2]); return 1; }
  if (write_outputs(fout, &step1, n_opart, n_lsep, n_out, n_lse) ||
      write_outputs(fout, &step2, n_opart, n_lsep, n_out, n_lse) ||
      write_outputs(fout, &two, n_opart, n_lsep, n_out, n_lse) ||
      write_outputs(fout, &na, n_opart, n_lsep, n_out, n_lse)) {
    fprintf(stderr, "writing outputs failed\n");
    return 1;
  }
  fclose(fout);
  HIP_OK(hipStreamDestroy(s));
  printf("step_c ok: %d launch(es) per step, workspace %zu bytes\n", launches, ws_bytes);
  return 0;
}
