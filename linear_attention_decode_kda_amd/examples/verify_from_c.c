/* A plain C caller of the fused verify step: HIP runtime calls and the C ABI of
 * include/kda_verify.h, with no Python or torch anywhere.
 *
 * usage: verify_from_c DIR N T H HV K V DTYPE GATE
 *   DTYPE 0 = fp32, 1 = bf16 (kda_dtype of mixed_qkv, conv_weight, conv_state, gate, beta, o);
 *   GATE 0 = softplus, 1 = safe (kda_gate_mode); every other parameter keeps the value
 *   kda_verify_params_init gives it.
 *
 * Reads the inputs of one call from DIR as raw little-endian arrays in the layouts the
 * header states (mixed_qkv.bin, conv_weight.bin, conv_state.bin, gate.bin, A_log.bin,
 * dt_bias.bin, beta.bin, state.bin), copies them to device memory, runs
 * kda_conv_verify_decode once on a stream of its own with a workspace it allocates and
 * zeroes with kda_workspace_reset, and writes o.bin, inter_ssm.bin, conv_window.bin and the
 * rolled cache conv_state_out.bin back to DIR. Every call is checked: a failed one prints
 * its status and the program exits 1; parameters the library rejects exit 2 before any
 * file is read.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kda_verify.h"

#define HIP_OK(call)                                                              \
  do {                                                                            \
    hipError_t e_ = (call);                                                       \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));           \
      exit(1);                                                                    \
    }                                                                             \
  } while (0)

enum { IN_MIXED, IN_WEIGHT, IN_CSTATE, IN_GATE, IN_ALOG, IN_DTB, IN_BETA, IN_STATE, N_IN };
enum { OUT_O, OUT_SSM, OUT_WIN, N_OUT };
static const char* const in_names[N_IN] = {"mixed_qkv", "conv_weight", "conv_state", "gate",
                                           "A_log",     "dt_bias",     "beta",       "state"};
static const char* const out_names[N_OUT] = {"o", "inter_ssm", "conv_window"};

static void path_of(char* buf, size_t cap, const char* dir, const char* name) {
  if (snprintf(buf, cap, "%s/%s.bin", dir, name) >= (int)cap) {
    fprintf(stderr, "path too long: %s/%s.bin\n", dir, name);
    exit(1);
  }
}

/* the whole file, which must hold exactly `bytes` bytes */
static void* read_exact(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  path_of(path, sizeof path, dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", path);
    exit(1);
  }
  void* buf = malloc(bytes ? bytes : 1);
  if (!buf) {
    fprintf(stderr, "out of host memory\n");
    exit(1);
  }
  const size_t got = fread(buf, 1, bytes, f);
  const int extra = fgetc(f) != EOF;
  fclose(f);
  if (got != bytes || extra) {
    fprintf(stderr, "%s: expected %zu bytes\n", path, bytes);
    exit(1);
  }
  return buf;
}

static void write_all(const char* dir, const char* name, const void* buf, size_t bytes) {
  char path[4096];
  path_of(path, sizeof path, dir, name);
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(buf, 1, bytes, f) != bytes || fclose(f) != 0) {
    fprintf(stderr, "cannot write %s\n", path);
    exit(1);
  }
}

static void check(kda_status st, const char* what) {
  if (st != KDA_OK) {
    fprintf(stderr, "%s: %s\n", what, kda_status_string(st));
    exit(1);
  }
}

int main(int argc, char** argv) {
  if (argc != 10) {
    fprintf(stderr, "usage: %s DIR N T H HV K V DTYPE GATE\n", argv[0]);
    return 2;
  }
  const char* dir = argv[1];
  int v[8];
  for (int i = 0; i < 8; ++i) v[i] = atoi(argv[2 + i]);
  if ((v[6] != 0 && v[6] != 1) || (v[7] != 0 && v[7] != 1)) {
    fprintf(stderr, "DTYPE and GATE must be 0 or 1\n");
    return 2;
  }
  kda_verify_params p;
  kda_verify_params_init(&p, v[0], v[1], v[2], v[3], v[4], v[5]);
  p.in_dtype = v[6] ? KDA_BF16 : KDA_F32;
  p.gate_mode = v[7] ? KDA_GATE_SAFE : KDA_GATE_SOFTPLUS;
  /* the library's own validation (host-only) before any size is formed from the shape */
  const int32_t variant = kda_select_variant(&p);
  if (variant < 0) {
    fprintf(stderr, "invalid parameters: %s\n", kda_status_string(variant));
    return 2;
  }

  const size_t N = (size_t)p.N, T = (size_t)p.T, H = (size_t)p.H, HV = (size_t)p.HV, K = (size_t)p.K,
               V = (size_t)p.V;
  const size_t C = 2 * H * K + HV * V, s = p.in_dtype == KDA_BF16 ? 2 : 4;
  const size_t in_bytes[N_IN] = {N * T * C * s, C * 4 * s,  N * C * 3 * s, N * T * HV * K * s,
                                 HV * 4,        HV * K * 4, N * T * HV * s, N * HV * K * V * 4};
  const size_t out_bytes[N_OUT] = {N * T * HV * V * s, N * T * HV * K * V * 4, N * T * C * 3 * s};

  void* dev_in[N_IN];
  void* dev_out[N_OUT];
  for (int i = 0; i < N_IN; ++i) {
    void* host = read_exact(dir, in_names[i], in_bytes[i]);
    HIP_OK(hipMalloc(&dev_in[i], in_bytes[i] ? in_bytes[i] : 16));
    HIP_OK(hipMemcpy(dev_in[i], host, in_bytes[i], hipMemcpyHostToDevice));
    free(host);
  }
  for (int i = 0; i < N_OUT; ++i) HIP_OK(hipMalloc(&dev_out[i], out_bytes[i] ? out_bytes[i] : 16));

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  const size_t ws_bytes = kda_workspace_bytes(&p);
  void* ws = NULL;
  HIP_OK(hipMalloc(&ws, ws_bytes ? ws_bytes : 16));
  check(kda_workspace_reset(ws, ws_bytes, stream), "kda_workspace_reset");
  check(kda_conv_verify_decode(&p, dev_in[IN_MIXED], dev_in[IN_WEIGHT], dev_in[IN_CSTATE], dev_in[IN_GATE],
                               (const float*)dev_in[IN_ALOG], (const float*)dev_in[IN_DTB], dev_in[IN_BETA],
                               (const float*)dev_in[IN_STATE], dev_out[OUT_O], (float*)dev_out[OUT_SSM],
                               dev_out[OUT_WIN], ws, ws_bytes, stream),
        "kda_conv_verify_decode");
  HIP_OK(hipStreamSynchronize(stream));

  for (int i = 0; i < N_OUT; ++i) {
    void* host = malloc(out_bytes[i] ? out_bytes[i] : 1);
    if (!host) return 1;
    HIP_OK(hipMemcpy(host, dev_out[i], out_bytes[i], hipMemcpyDeviceToHost));
    write_all(dir, out_names[i], host, out_bytes[i]);
    free(host);
  }
  void* host = malloc(in_bytes[IN_CSTATE] ? in_bytes[IN_CSTATE] : 1);
  if (!host) return 1;
  HIP_OK(hipMemcpy(host, dev_in[IN_CSTATE], in_bytes[IN_CSTATE], hipMemcpyDeviceToHost));
  write_all(dir, "conv_state_out", host, in_bytes[IN_CSTATE]);
  free(host);

  for (int i = 0; i < N_IN; ++i) HIP_OK(hipFree(dev_in[i]));
  for (int i = 0; i < N_OUT; ++i) HIP_OK(hipFree(dev_out[i]));
  HIP_OK(hipFree(ws));
  HIP_OK(hipStreamDestroy(stream));
  printf("verify_from_c ok: N=%d T=%d H=%d HV=%d K=%d V=%d\n", p.N, p.T, p.H, p.HV, p.K, p.V);
  return 0;
}
