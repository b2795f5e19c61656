"""Source checks for a known miscompile of the HIP toolchain here.

`__builtin_bit_cast(T, v[i])` applied directly to an element of an
ext_vector_type value compiles, for gfx950 with this hipcc, to a read of
element 0 whatever i is (a kernel summing the low halves of the four
elements of a loaded uint32x4 loads one dword and uses it four times).
Casting through a conversion, `__builtin_bit_cast(T, (uint32_t)v[i])`, or
bit-casting the whole vector compiles correctly.  No kernel source may use
the first form."""
import glob
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BAD = re.compile(r"__builtin_bit_cast\(\s*[\w:]+\s*,\s*[A-Za-z_]\w*\s*\[")


def test_no_bit_cast_of_a_bare_vector_element():
    srcs = glob.glob(os.path.join(ROOT, "non_linear_matrix_amd", "csrc", "*.hip")) + \
        glob.glob(os.path.join(ROOT, "non_linear_matrix_amd", "csrc", "*.h"))
    assert srcs
    hits = []
    for path in srcs:
        with open(path) as fh:
            for n, line in enumerate(fh, 1):
                if BAD.search(line):
                    hits.append(f"{os.path.basename(path)}:{n}: {line.strip()}")
    assert not hits, "bit_cast of a bare vector element (miscompiled):\n" + "\n".join(hits)


def test_the_pattern_is_recognised():
    assert BAD.search("x = __builtin_bit_cast(h2, v[i])[0];")
    assert not BAD.search("x = __builtin_bit_cast(float, (uint32_t)r[0]);")
    assert not BAD.search("x = __builtin_bit_cast(h8, (u32x4{a, b, c, d}));")
