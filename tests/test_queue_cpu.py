"""Host-compiled check of the queue schedule's next-unit computation (csrc/kda_queue.h).

Under the queue schedule a workgroup turns the ticket it drew from the workspace counter
into its next unit. A call that does not run to completion leaves that counter at any
value, so the computation must never form a unit outside [resident, units), whatever the
32-bit ticket holds: the next call then ends every workgroup's loop instead of reading
out of range (pooled index arrays) or walking ~2^31 padding units. The header is compiled
here with g++ under UBSan (signed overflow would trap) and driven over edge values,
2^31 and 2^32 - 1 among them, and exhaustively over small sizes.

Page: "[KDA] Fuse causal conv1d into MTP verify decode #107" (cuLA pull request), code
review: counters left non-zero by an earlier call corrupt the following launches.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_attention_decode_kda_amd", "csrc")

DRIVER = r"""
#include <stdint.h>
#include <stdio.h>
#include <limits.h>
#include "kda_queue.h"

static int fails = 0;

static void check(uint32_t ticket, int units, int resident) {
  const int u = kda_queue_unit(ticket, units, resident);
  const uint64_t rest = units > resident ? (uint64_t)(units - resident) : 0;
  const int want = (uint64_t)ticket < rest ? (int)((int64_t)resident + ticket) : -1;
  if (u != want || (u != -1 && (u < resident || u >= units))) {
    printf("bad: ticket %u units %d resident %d -> %d (want %d)\n", ticket, units, resident, u, want);
    ++fails;
  }
}

int main(void) {
  const uint32_t tickets[] = {0u, 1u, 2u, 3u, 255u, 0x03030303u, 0x7ffffffeu, 0x7fffffffu, 0x80000000u,
                              0x80000001u, 0xfffffffeu, 0xffffffffu};
  const int sizes[] = {1, 2, 3, 255, 256, 257, 2048, 8192, 32768, 65535, 1 << 20, INT_MAX - 1, INT_MAX};
  for (unsigned a = 0; a < sizeof(sizes) / sizeof(sizes[0]); ++a)
    for (unsigned b = 0; b < sizeof(sizes) / sizeof(sizes[0]); ++b) {
      const int units = sizes[a], resident = sizes[b];
      if (resident > units) continue;
      for (unsigned t = 0; t < sizeof(tickets) / sizeof(tickets[0]); ++t) check(tickets[t], units, resident);
      // the tickets right at the end of the queue
      const uint32_t rest = (uint32_t)(units - resident);
      for (uint32_t d = 0; d < 3; ++d) {
        check(rest + d, units, resident);
        if (rest >= d + 1) check(rest - d - 1, units, resident);
      }
    }
  for (int units = 1; units <= 64; ++units)
    for (int resident = 1; resident <= units; ++resident)
      for (uint32_t t = 0; t < 80; ++t) check(t, units, resident);
  // a whole queue drawn in order visits every unit past the first round exactly once
  for (int units = 1; units <= 300; units += 7)
    for (int resident = 1; resident <= units; resident += 5) {
      int seen = 0, next = resident;
      for (uint32_t t = 0;; ++t) {
        const int u = kda_queue_unit(t, units, resident);
        if (u < 0) break;
        if (u != next++) ++fails;
        ++seen;
      }
      if (seen != units - resident) ++fails;
    }
  if (fails) return 1;
  printf("queue ok\n");
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ missing")
def test_queue_next_unit_bounds(tmp_path):
    drv = tmp_path / "queue_drv.cpp"
    drv.write_text(DRIVER)
    exe = tmp_path / "queue_drv"
    r = subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-fsanitize=undefined", "-fno-sanitize-recover=all",
                        f"-I{CSRC}", str(drv), "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0 and "queue ok" in r.stdout, r.stdout + r.stderr


def test_kernel_uses_the_checked_computation():
    """The queue kernel takes its next unit from kda_queue_unit and keeps the ticket
    unsigned (no conversion of a ticket to a signed unit elsewhere)."""
    src = open(os.path.join(CSRC, "kda_verify.hip")).read()
    assert '#include "kda_queue.h"' in src
    assert "lb = kda_queue_unit(s.next[it & 1], units, G);" in src
    assert "uint32_t next[2];" in src
    assert "(int)ticket" not in src
