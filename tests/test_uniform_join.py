"""The 64-bit join behind every wave-uniform address of the matrix-core
kernels (kv_cache_gqa_decode_amd/csrc/uniform_join.h), compiled on the host
with g++ and a broadcast that returns a signed int as the readfirstlane
builtin does.

A join that sign-extends the low half turns any address whose low word has
bit 31 set into 0xffffffff'xxxxxxxx: a device-memory fault the first time
such a pointer reaches a scalar load.  The header's join must round-trip
every such value; the sign-extending form, built from the same mock, must
not (so the check can tell the two apart)."""
import os
import subprocess
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cache_gqa_decode_amd", "csrc")

PROGRAM = textwrap.dedent(r"""
    #include <cstdio>
    #include <cstdint>
    #include "uniform_join.h"

    // the builtin's contract: a 32-bit lane value back as a signed int
    static int mock_readfirstlane(int x) { return x; }

    static uint64_t header_join(uint64_t v) {
      return kvd::join_uniform_halves(v, [](uint32_t x) {
        return mock_readfirstlane(static_cast<int>(x));
      });
    }
    static uint64_t sign_extending_join(uint64_t v) {
      const uint32_t hi = static_cast<uint32_t>(mock_readfirstlane(static_cast<int>(v >> 32)));
      const int lo = mock_readfirstlane(static_cast<int>(static_cast<uint32_t>(v)));
      return (static_cast<uint64_t>(hi) << 32) | static_cast<uint64_t>(static_cast<int64_t>(lo));
    }

    int main() {
      const uint64_t values[] = {
          0x00007f1a80000000ull, 0x00007f1abffffff0ull, 0x0000700000000100ull,
          0x00007fffffffffffull, 0x0000000080000000ull, 0x00007f1a7ffffff0ull,
          0x0ull, 0x00000001ffffffffull, 0x0000155555555000ull};
      int bad_header = 0, caught = 0;
      uint64_t x = 0x2545f4914f6cdd1dull;
      for (int i = 0; i < 200000 + 9; ++i) {
        uint64_t v;
        if (i < 9) {
          v = values[i];
        } else {  // xorshift64: device-like addresses (47 bits), every other with bit 31 set
          x ^= x << 13; x ^= x >> 7; x ^= x << 17;
          v = (x & 0x00007fffffffffffull) | (i % 2 ? 0x80000000ull : 0);
        }
        if (header_join(v) != v) ++bad_header;
        if ((v & 0x80000000ull) && sign_extending_join(v) != v) ++caught;
      }
      std::printf("%d %d\n", bad_header, caught);
      return 0;
    }
""")


def test_join_keeps_bit_31_of_the_low_word(tmp_path):
    src = tmp_path / "join.cpp"
    exe = tmp_path / "join"
    src.write_text(PROGRAM)
    r = subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-Werror", f"-I{CSRC}",
                        str(src), "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()
    bad_header, caught = int(out[0]), int(out[1])
    assert bad_header == 0, f"uniform_join.h corrupted {bad_header} values"
    assert caught > 100000, "the sign-extending join was not told apart"
