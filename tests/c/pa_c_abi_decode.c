/* A plain C caller of the library's C-ABI (include/pa.h): no Python, no
 * torch. Reads one decode problem from raw files in a directory, copies it to
 * device memory it allocates with hipMalloc, builds the work list in a
 * workspace of pa_workspace_bytes, decodes on a stream of its own, checks
 * the device status, and writes the output back as raw bf16 bits.
 *
 * Files in DIR (all little-endian):
 *   dims.txt   the thirteen pa_dims fields in declaration order, then q_len
 *              is repeated (as the decode's argument), then the softmax
 *              scale and the kv scale mode
 *   q.bin      bf16 bits [batch, q_len, num_q_heads, head_dim]
 *   k.bin, v.bin   cache bytes [num_pages, num_kv_heads, page_size, head_dim]
 *   bt.bin     int32 [batch, max_pages_per_seq]
 *   ctx.bin    int32 [batch]
 *   scales.bin float32 K/V scales (absent for bf16 caches)
 * Writes DIR/out.bin (bf16 bits, the shape of q) and prints one line:
 * "status <device status> grid <workgroups> variant <instantiation>".
 * Exit code 0 on success; any library or HIP error prints pa_last_error()
 * and exits 1. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "pa.h"

static void* read_file(const char* dir, const char* name, size_t* size) {
  char path[4096];
  snprintf(path, sizeof(path), "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  fseek(f, 0, SEEK_END);
  long n = ftell(f);
  fseek(f, 0, SEEK_SET);
  void* buf = malloc(n > 0 ? (size_t)n : 1);
  if (!buf || fread(buf, 1, (size_t)n, f) != (size_t)n) {
    fclose(f);
    free(buf);
    return NULL;
  }
  fclose(f);
  *size = (size_t)n;
  return buf;
}

static int die(const char* what, int rc) {
  fprintf(stderr, "%s failed: %d (%s) %s\n", what, rc, pa_status_string(rc), pa_last_error());
  return 1;
}

static int hip_die(const char* what, hipError_t e) {
  fprintf(stderr, "%s failed: %s\n", what, hipGetErrorString(e));
  return 1;
}

/* host buffer -> new device buffer of the same size */
static void* to_device(const void* host, size_t n) {
  void* d = NULL;
  if (hipMalloc(&d, n ? n : 16) != hipSuccess) return NULL;
  if (n && hipMemcpy(d, host, n, hipMemcpyHostToDevice) != hipSuccess) return NULL;
  return d;
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s DIR\n", argv[0]);
    return 2;
  }
  const char* dir = argv[1];
  char path[4096];
  snprintf(path, sizeof(path), "%s/dims.txt", dir);
  FILE* f = fopen(path, "r");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", path);
    return 2;
  }
  pa_dims dims;
  int32_t q_len = 0, mode = 0;
  float scale = 0.f;
  int32_t* fields = &dims.batch;
  int nread = 0;
  for (int i = 0; i < 13; ++i) nread += fscanf(f, "%d", &fields[i]);
  nread += fscanf(f, "%d %f %d", &q_len, &scale, &mode);
  fclose(f);
  if (nread != 16) {
    fprintf(stderr, "%s: expected 16 numbers, read %d\n", path, nread);
    return 2;
  }

  size_t nq, nk, nv, nbt, nctx, nsc = 0;
  void* hq = read_file(dir, "q.bin", &nq);
  void* hk = read_file(dir, "k.bin", &nk);
  void* hv = read_file(dir, "v.bin", &nv);
  void* hbt = read_file(dir, "bt.bin", &nbt);
  void* hctx = read_file(dir, "ctx.bin", &nctx);
  void* hsc = read_file(dir, "scales.bin", &nsc);
  if (!hq || !hk || !hv || !hbt || !hctx) {
    fprintf(stderr, "missing input files in %s\n", dir);
    return 2;
  }

  int32_t num_cus = 0;
  int rc = pa_query_device(0, &num_cus);
  if (rc) return die("pa_query_device", rc);
  hipError_t e = hipSetDevice(0);
  if (e != hipSuccess) return hip_die("hipSetDevice", e);

  uint64_t ws_bytes = 0;
  rc = pa_workspace_bytes(&dims, num_cus, &ws_bytes);
  if (rc) return die("pa_workspace_bytes", rc);

  void* q = to_device(hq, nq);
  void* k = to_device(hk, nk);
  void* v = to_device(hv, nv);
  void* bt = to_device(hbt, nbt);
  void* ctx = to_device(hctx, nctx);
  void* sc = hsc ? to_device(hsc, nsc) : NULL;
  void* ws = NULL;
  void* out = NULL;
  if (!q || !k || !v || !bt || !ctx || (hsc && !sc)) return hip_die("inputs to device", hipErrorOutOfMemory);
  if ((e = hipMalloc(&ws, ws_bytes)) != hipSuccess) return hip_die("workspace hipMalloc", e);
  if ((e = hipMalloc(&out, nq)) != hipSuccess) return hip_die("output hipMalloc", e);
  if ((e = hipMemset(out, 0xff, nq)) != hipSuccess) return hip_die("hipMemset", e);

  hipStream_t stream;
  if ((e = hipStreamCreate(&stream)) != hipSuccess) return hip_die("hipStreamCreate", e);

  pa_plan_t plan;
  rc = pa_plan(&dims, (const int32_t*)ctx, ws, ws_bytes, &plan, stream);
  if (rc) return die("pa_plan", rc);
  rc = pa_decode(&plan, q, k, v, (const int32_t*)bt, (const int32_t*)ctx, q_len, scale, mode,
                 (const float*)sc, out, stream);
  if (rc) return die("pa_decode", rc);
  int32_t status = -1;
  rc = pa_plan_status(&plan, &status, stream);
  if (rc) return die("pa_plan_status", rc);

  void* hout = malloc(nq);
  if (!hout) return 2;
  if ((e = hipMemcpy(hout, out, nq, hipMemcpyDeviceToHost)) != hipSuccess) return hip_die("hipMemcpy", e);
  snprintf(path, sizeof(path), "%s/out.bin", dir);
  f = fopen(path, "wb");
  if (!f || fwrite(hout, 1, nq, f) != nq) {
    fprintf(stderr, "cannot write %s\n", path);
    return 2;
  }
  fclose(f);
  printf("status %d grid %d variant %d\n", status, plan.grid, plan.variant);

  hipStreamDestroy(stream);
  hipFree(q);
  hipFree(k);
  hipFree(v);
  hipFree(bt);
  hipFree(ctx);
  if (sc) hipFree(sc);
  hipFree(ws);
  hipFree(out);
  free(hq);
  free(hk);
  free(hv);
  free(hbt);
  free(hctx);
  free(hsc);
  free(hout);
  return status == 0 ? 0 : 1;
}
