"""Code-generation facts the kernels rely on, checked on the CPU (hipcc
cross-compiles for gfx950; nothing here runs on a GPU).

1. While the compiler's wait-count pass tracks a global->LDS copy in flight, it
   treats outstanding LDS reads as completing out of order: before using any
   one it waits for all of them (lgkmcnt(0)). Without the copy it waits only
   for the reads a use needs (lgkmcnt(n), LDS reads return in issue order).
2. The d = 64 backward issues its tile copies from inline assembly, out of the
   pass's sight, so its LDS reads keep those partial waits.
3. The tiled loops of the hot kernels do not copy their running state between
   register sets at every tile (they did while the full and the masked tile
   paths met inside the loop: 16-40 moves per block).
"""

import os
import re
import subprocess

import pytest

from memory_efficient_exact_amd import build

pytestmark = pytest.mark.skipif(not os.path.exists(build.HIPCC), reason="hipcc not available")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# compiled only, never launched: a loop of three 16-byte LDS reads feeding three
# MFMAs, with (DMA = 1) or without a global->LDS copy into another LDS array
TINY = r"""
#include <hip/hip_runtime.h>
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
template <int DMA>
__global__ void probe(const bf16x8* g, float* out, int n) {
  __shared__ bf16x8 s[1024];
  __shared__ bf16x8 s2[512];
  s[threadIdx.x] = g[threadIdx.x];
  __syncthreads();
  f32x16 acc = {};
  const bf16x8 b = g[threadIdx.x + 64];
  for (int i = 0; i < n; ++i) {
    if constexpr (DMA)
      __builtin_amdgcn_global_load_lds(g + i * 64 + threadIdx.x,
                                       (__attribute__((address_space(3))) void*)(s2 + (i & 7) * 64),
                                       16, 0, 0);
    const bf16x8 a0 = s[(threadIdx.x + 3 * i) & 1023];
    const bf16x8 a1 = s[(threadIdx.x + 3 * i + 64) & 1023];
    const bf16x8 a2 = s[(threadIdx.x + 3 * i + 128) & 1023];
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, b, acc, 0, 0, 0);
  }
  for (int r = 0; r < 16; ++r) out[threadIdx.x * 16 + r] = acc[r];
}
template __global__ void probe<0>(const bf16x8*, float*, int);
template __global__ void probe<1>(const bf16x8*, float*, int);
"""


def assemble(src_path, out_path):
    cmd = [build.HIPCC, *build.FLAGS, "-I", os.path.join(ROOT, "include"), "--cuda-device-only",
           "-S", src_path, "-o", out_path]
    subprocess.run(cmd, check=True, capture_output=True, timeout=300)
    return open(out_path).read()


def function_body(asm, symbol_pattern):
    """Instructions of the first function whose label matches the pattern."""
    m = re.search(r"^(" + symbol_pattern + r"):", asm, flags=re.M)
    assert m, symbol_pattern
    body = asm[m.end():]
    return body[:body.index("s_endpgm")]


def lds_waits(body):
    """(full, partial): s_waitcnt instructions with lgkmcnt(0) and with lgkmcnt(n > 0)."""
    counts = [int(c) for c in re.findall(r"s_waitcnt[^\n]*lgkmcnt\((\d+)\)", body)]
    return sum(c == 0 for c in counts), sum(c > 0 for c in counts)


def test_lds_copy_in_flight_makes_every_lds_wait_full(tmp_path):
    src = tmp_path / "probe.hip"
    src.write_text(TINY)
    asm = assemble(str(src), str(tmp_path / "probe.s"))
    _, partial_without = lds_waits(function_body(asm, r"_Z5probeILi0E\w*"))
    full_with, partial_with = lds_waits(function_body(asm, r"_Z5probeILi1E\w*"))
    assert partial_without >= 1   # exact waits without the copy
    assert partial_with == 0 and full_with >= 1   # only full waits with it


def test_d64_backward_keeps_partial_lds_waits(tmp_path):
    src = os.path.join(ROOT, "memory_efficient_exact_amd", "csrc", "bwd_bf16.hip")
    asm = assemble(src, str(tmp_path / "bwd.s"))
    full, partial = lds_waits(function_body(asm, r"_ZN3mea12_GLOBAL__N_115bwd_main_kernelILi64ELi8EEEv\w*"))
    # with the builtin copy all 666 were full; the untracked copies leave ~100+ partial
    assert partial >= 50 and partial > full, (full, partial)


def test_d128_backward_dq_role_keeps_partial_lds_waits(tmp_path):
    # the d = 128 kernel issues only its dQ role's tile copies out of the pass's sight
    src = os.path.join(ROOT, "memory_efficient_exact_amd", "csrc", "bwd_bf16.hip")
    asm = assemble(src, str(tmp_path / "bwd.s"))
    full, partial = lds_waits(function_body(asm, r"_ZN3mea12_GLOBAL__N_118bwd_main128_kernelILi8EEEv\w*"))
    # all 221 were full with the builtin copies in both roles
    assert partial >= 40, (full, partial)


def loop_blocks(body):
    """{label: (loop annotation, number of v_mov instructions)} of the basic blocks."""
    blocks, cur = {}, None
    for line in body.split("\n"):
        t = line.strip()
        m = re.match(r"^(\.LBB\S+|; %bb\.\d+):\s*(.*)$", t)
        if m:
            cur = m.group(1)
            blocks[cur] = [m.group(2), 0]
        elif cur and t.startswith("v_mov"):
            blocks[cur][1] += 1
    return blocks


@pytest.mark.parametrize("src,symbol", [
    ("fwd_bf16.hip", r"_ZN3mea12_GLOBAL__N_115fwd_bf16_kernelILi64ELi2ELi128ELb0ELi8EEEv\w*"),
    ("fwd_bf16.hip", r"_ZN3mea12_GLOBAL__N_115fwd_bf16_kernelILi128ELi1ELi64ELb0ELi8EEEv\w*"),
    ("bwd_bf16.hip", r"_ZN3mea12_GLOBAL__N_115bwd_main_kernelILi64ELi8EEEv\w*"),
    ("bwd_bf16.hip", r"_ZN3mea12_GLOBAL__N_118bwd_main128_kernelILi8EEEv\w*"),
])
def test_tile_loops_do_not_copy_their_running_state(tmp_path, src, symbol):
    # With the ragged last tile handled outside the tiled loops, no block inside a loop
    # moves the accumulators between register sets (a block of 16-80 v_mov per tile
    # when a full and a masked tile path met inside the loop).
    asm = assemble(os.path.join(ROOT, "memory_efficient_exact_amd", "csrc", src),
                   str(tmp_path / "k.s"))
    body = function_body(asm, symbol)
    copies = {b: n for b, (note, n) in loop_blocks(body).items() if "Loop" in note and n >= 12}
    assert not copies, copies
