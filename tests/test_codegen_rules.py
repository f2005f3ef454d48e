"""Rules every kernel's generated code must keep, checked on the CPU from the
gfx950 assembly of each source, built with the library's own flags:

- no write through the scalar data cache (scalar stores, scalar atomics, the
  scalar cache's write-back): every store is a vector store;
- no packed fp32 arithmetic (the build disables the feature; this checks that
  it stays so).
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

from block_wise_int4_amd import build as B

SCALAR_WRITE = re.compile(r"^\s*(s_store|s_buffer_store|s_atomic|s_buffer_atomic|s_dcache_wb|s_scratch_store)")
PACKED_F32 = re.compile(r"^\s*v_pk_(add|mul|fma|mov)_f32")


def _asm(src, tmp):
    out = os.path.join(tmp, os.path.basename(src) + ".s")
    cmd = ([B.HIPCC] + B.COMMON_FLAGS + B.DEVICE_FLAGS + B.EXTRA_FLAGS.get(os.path.basename(src), []) +
           ["-S", "--cuda-device-only", src, "-o", out])
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out


@pytest.mark.skipif(not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None, reason="hipcc missing")
def test_generated_code_keeps_the_rules(tmp_path):
    srcs = [os.path.join(B.CSRC, f) for f in B.SOURCES + [B.YARDSTICK_SRC] if f.endswith(".hip")]
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        outs = list(ex.map(lambda s: _asm(s, str(tmp_path)), srcs))
    bad = []
    for path in outs:
        with open(path) as f:
            for n, line in enumerate(f, 1):
                if SCALAR_WRITE.match(line) or PACKED_F32.match(line):
                    bad.append("%s:%d: %s" % (os.path.basename(path), n, line.strip()))
    assert not bad, "\n".join(bad[:20])


def test_the_patterns_match_what_they_guard():
    for line in ("\ts_store_dword s4, s[0:1], 0x0", "  s_buffer_store_dwordx2 s[4:5], s[8:11], 0x10",
                 "\ts_atomic_add s2, s[0:1], 0x0", "\ts_dcache_wb"):
        assert SCALAR_WRITE.match(line), line
    for line in ("\tv_pk_fma_f32 v[0:1], v[2:3], v[4:5], v[6:7]", "\tv_pk_mul_f32 v[0:1], v[2:3], v[4:5]"):
        assert PACKED_F32.match(line), line
    for line in ("\ts_load_dword s4, s[0:1], 0x0", "\tglobal_store_dword v0, v1, s[0:1]",
                 "\tv_pk_fma_f16 v0, v1, v2, v3", "\ts_waitcnt vmcnt(0)"):
        assert not SCALAR_WRITE.match(line) and not PACKED_F32.match(line), line
