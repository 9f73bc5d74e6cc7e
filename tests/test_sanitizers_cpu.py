"""AddressSanitizer / UndefinedBehaviorSanitizer runs of host code (no GPU).

* The float64 oracle is compiled with -fsanitize=address,undefined together with a small C
  driver that runs the whole verify step on several shapes (T = 1, T < 3, GVA, K != V).
* The host side of the C ABI (validation, dispatch, status strings; the device code is
  compiled normally) is built with the sanitizers on the host pass only and driven through
  every rejection path with fake pointers, which never reach a HIP call.
"""
import os
import shutil
import subprocess
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

ORACLE_DRIVER = textwrap.dedent(r"""
    #include <stdio.h>
    #include <stdlib.h>
    int oracle_verify(int, int, int, int, int, int, int, double, double, double, double, double,
                      const double*, const double*, const double*, const double*, const double*,
                      const double*, const double*, const double*, double*, double*, double*, double*);
    static double* rnd(size_t n, unsigned* s) {
      double* p = (double*)malloc(sizeof(double) * (n ? n : 1));
      for (size_t i = 0; i < n; ++i) { *s = *s * 1103515245u + 12345u; p[i] = ((*s >> 8) & 0xffff) / 32768.0 - 1.0; }
      return p;
    }
    int main(void) {
      const int shapes[][6] = {{2, 1, 1, 1, 4, 4}, {2, 2, 2, 4, 8, 8}, {1, 5, 1, 3, 4, 6}, {3, 3, 2, 2, 16, 16}};
      unsigned seed = 7;
      for (int s = 0; s < 4; ++s) {
        int N = shapes[s][0], T = shapes[s][1], H = shapes[s][2], HV = shapes[s][3], K = shapes[s][4], V = shapes[s][5];
        size_t C = 2 * (size_t)H * K + (size_t)HV * V;
        double *x = rnd((size_t)N * T * C, &seed), *w = rnd(C * 4, &seed), *cs = rnd((size_t)N * C * 3, &seed);
        double *g = rnd((size_t)N * T * HV * K, &seed), *al = rnd(HV, &seed), *db = rnd((size_t)HV * K, &seed);
        double *b = rnd((size_t)N * T * HV, &seed), *st = rnd((size_t)N * HV * K * V, &seed);
        double *o = rnd((size_t)N * T * HV * V, &seed), *is = rnd((size_t)N * T * HV * K * V, &seed);
        double *cw = rnd((size_t)N * T * C * 3, &seed), *cso = rnd((size_t)N * C * 3, &seed);
        for (int mode = 0; mode < 2; ++mode)
          if (oracle_verify(N, T, H, HV, K, V, mode, -5.0, 1.0, 20.0, 0.25, 1e-6, x, w, cs, g, al, db, b, st, o, is, cw, cso)) return 2;
        if (oracle_verify(N, T, 2, 3, K, V, 0, -5.0, 1.0, 20.0, 0.25, 1e-6, x, w, cs, g, al, db, b, st, o, is, cw, cso) != -1) return 3;
        free(x); free(w); free(cs); free(g); free(al); free(db); free(b); free(st); free(o); free(is); free(cw); free(cso);
      }
      puts("oracle ok");
      return 0;
    }
""")

ABI_DRIVER = textwrap.dedent(r"""
    #include <stdint.h>
    #include <stdio.h>
    #include <string.h>
    #include "kda_verify.h"
    #define CHECK(c) do { if (!(c)) { printf("failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)
    int main(void) {
      void* ptr[14];
      for (int i = 0; i < 14; ++i) ptr[i] = (void*)((uintptr_t)(i + 1) << 40);
      kda_verify_params p;
      kda_verify_params_init(&p, 4, 4, 2, 4, 128, 128);
      size_t ws = kda_workspace_bytes(&p);
      CHECK(ws == 256);
      CHECK(kda_validate(&p, ptr[0], ptr[1], ptr[2], ptr[3], (float*)ptr[4], (float*)ptr[5], ptr[6], (float*)ptr[7],
                         ptr[8], (float*)ptr[9], ptr[10], ptr[11], ws) == KDA_OK);
      for (int k = 0; k < 6; ++k) {
        kda_verify_params q = p;
        if (k == 0) q.T = 0;
        if (k == 1) q.T = KDA_MAX_T + 1;
        if (k == 2) q.HV = 3;
        if (k == 3) q.H = 0;
        if (k == 4) q.K = 32;
        if (k == 5) q.tile_columns = 48;
        CHECK(kda_conv_verify_decode(&q, ptr[0], ptr[1], ptr[2], ptr[3], (float*)ptr[4], (float*)ptr[5], ptr[6],
                                     (float*)ptr[7], ptr[8], (float*)ptr[9], ptr[10], ptr[11], ws, NULL) < 0);
      }
      CHECK(kda_conv_verify_decode(&p, NULL, ptr[1], ptr[2], ptr[3], (float*)ptr[4], (float*)ptr[5], ptr[6],
                                   (float*)ptr[7], ptr[8], (float*)ptr[9], ptr[10], ptr[11], ws, NULL) == KDA_ERR_NULL);
      CHECK(kda_conv_verify_decode(&p, ptr[0], ptr[1], ptr[0], ptr[3], (float*)ptr[4], (float*)ptr[5], ptr[6],
                                   (float*)ptr[7], ptr[8], (float*)ptr[9], ptr[10], ptr[11], ws, NULL) == KDA_ERR_ALIAS);
      kda_pool_desc pd;
      memset(&pd, 0, sizeof(pd));
      pd.conv_state_slots = 4; pd.state_slots = 0; pd.intermediate_slots = 4;
      CHECK(kda_conv_verify_decode_pooled(&p, &pd, ptr[0], ptr[1], ptr[2], ptr[3], (float*)ptr[4], (float*)ptr[5],
                                          ptr[6], (float*)ptr[7], ptr[8], (float*)ptr[9], ptr[10], ptr[11], ws,
                                          NULL) == KDA_ERR_SHAPE);
      CHECK(kda_conv_verify_decode_unfused(&p, NULL, ptr[0], ptr[1], ptr[2], ptr[3], (float*)ptr[4], (float*)ptr[5],
                                           ptr[6], (float*)ptr[7], ptr[8], (float*)ptr[9], ptr[10], ptr[8], ptr[11],
                                           ws, NULL) == KDA_ERR_ALIAS);
      CHECK(kda_verify_commit(&p, NULL, NULL, (float*)ptr[1], ptr[2], (float*)ptr[3], ptr[4], NULL) == KDA_ERR_NULL);
      CHECK(kda_workspace_reset(NULL, 64, NULL) == KDA_ERR_NULL);
      for (int s = -8; s <= 0; ++s) CHECK(kda_status_string(s) != NULL);
      kda_verify_params z;
      kda_verify_params_init(&z, 0, 1, 1, 1, 16, 16);
      CHECK(kda_conv_verify_decode(&z, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0,
                                   NULL) == KDA_OK);
      CHECK(kda_select_variant(&p) == KDA_VARIANT_SMALL || kda_select_variant(&p) == KDA_VARIANT_LARGE);
      puts("abi ok");
      return 0;
    }
""")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc missing")
def test_oracle_under_asan_ubsan(tmp_path):
    drv = tmp_path / "drv.c"
    drv.write_text(ORACLE_DRIVER)
    exe = tmp_path / "oracle_asan"
    rc, log = _run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", str(drv), os.path.join(ROOT, "oracle", "kda_oracle.c"),
                    "-o", str(exe), "-lm"])
    assert rc == 0, log
    rc, log = _run([str(exe)], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"})
    assert rc == 0 and "oracle ok" in log, log


HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc missing")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    lib = tmp_path / "libkda_verify_asan.so"
    rc, log = _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    f"-I{ROOT}/include", os.path.join(ROOT, "linear_attention_decode_kda_amd", "csrc", "kda_verify.hip"),
                    "-o", str(lib)])
    assert rc == 0, log
    drv = tmp_path / "drv.cpp"
    drv.write_text(ABI_DRIVER)
    exe = tmp_path / "abi_asan"
    rc, log = _run([HIPCC, "-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    f"-I{ROOT}/include", str(drv), "-o", str(exe), f"-L{tmp_path}", "-lkda_verify_asan",
                    f"-Wl,-rpath,{tmp_path}"])
    assert rc == 0, log
    env = {**os.environ, "ASAN_OPTIONS": "detect_leaks=0", "UBSAN_OPTIONS": "halt_on_error=1"}
    rc, log = _run([str(exe)], env=env)
    assert rc == 0 and "abi ok" in log, log
