"""Source rules for the HIP kernels, checked on the CPU.

The ROCm 7.2 clang lowers __builtin_bit_cast of an element of an
ext_vector_type value (v.y, v[i]) to a read of element 0.  Two kernels'
row scales were wrong that way (their regression tests are in
test_gpu_harp.py and test_gpu_qwha_widths.py).  This check keeps the
pattern out of the sources: elements are copied to a scalar first.
"""
import glob
import os
import re

CSRC = os.path.join(os.path.dirname(__file__), "..", "wht_adapters_amd", "csrc")


def bit_cast_operands(text):
    """The second argument of every __builtin_bit_cast(T, expr) call."""
    out = []
    for m in re.finditer(r"__builtin_bit_cast\(", text):
        i, depth, comma = m.end(), 1, None
        while i < len(text) and depth:
            c = text[i]
            if c in "([{":
                depth += 1
            elif c in ")]}":
                depth -= 1
            elif c == "," and depth == 1 and comma is None:
                comma = i
            i += 1
        if comma is not None:
            out.append((text.count("\n", 0, m.start()) + 1, text[comma + 1:i - 1].strip()))
    return out


# a vector element: name(.member)* [subscripts]* .x/.y/.z/.w, or three or more
# subscripts (an element of a vector held in a 2-D array)
ELEMENT = re.compile(r"^[A-Za-z_]\w*(\[[^\]]+\])*\.(x|y|z|w)$|^[A-Za-z_]\w*(\[[^\]]+\]){3,}$")


def test_no_bit_cast_of_vector_elements():
    bad = []
    for f in sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.hpp"))):
        with open(f) as fh:
            text = fh.read()
        for line, expr in bit_cast_operands(text):
            if ELEMENT.match(expr):
                bad.append(f"{os.path.basename(f)}:{line}: {expr}")
    assert not bad, "bit_cast of a vector element (copy it to a scalar first):\n" + "\n".join(bad)


def test_the_rule_catches_the_pattern():
    text = ("a = __builtin_bit_cast(bf16x2_t, v.y);\nb = __builtin_bit_cast(bf16x2_t, xa[i][k][p]);\n"
            "c = __builtin_bit_cast(uint32_t, w0);\nd = __builtin_bit_cast(f16x4, R[w][k]);\n"
            "e = __builtin_bit_cast(float, f(x, y));\n")
    hits = [e for _, e in bit_cast_operands(text) if ELEMENT.match(e)]
    assert hits == ["v.y", "xa[i][k][p]"]
