"""Host-side check of a contract between kernel sources: the fused selection +
decode kernel has waves with no decode work execute as many workgroup
barriers as the decode statements do (decode_body_barriers in
decode_body.h).  A barrier added to or removed from the decode statements
without updating that count would leave the fused kernel's barriers unmatched,
so the count is checked against the source text here, on the CPU."""
import os
import re

CSRC = os.path.join(os.path.dirname(__file__), os.pardir, "sparse_attention_long_page_amd", "csrc")


def _code(path):
    text = open(os.path.join(CSRC, path)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return "\n".join(line.split("//")[0] for line in text.splitlines())


def test_decode_body_barrier_count_matches_helper():
    body = _code("decode_body.inc")
    n_all = len(re.findall(r"__syncthreads\s*\(\s*\)", body))
    # the one barrier under `if constexpr (STAGED)` and the unconditional one
    staged_block = re.search(r"if constexpr \(STAGED\) \{(.*?)\} else \{", body, flags=re.S)
    assert staged_block is not None
    n_staged_only = len(re.findall(r"__syncthreads\s*\(\s*\)", staged_block.group(1)))
    assert (n_all, n_staged_only) == (2, 1)
    assert "__syncthreads_or" not in body and "s_barrier" not in body and "return;" not in body
    helper = _code("decode_body.h")
    m = re.search(r"decode_body_barriers\(bool staged\)\s*\{\s*return staged \? (\d+) : (\d+);", helper)
    assert m is not None
    assert (int(m.group(1)), int(m.group(2))) == (n_all, n_all - n_staged_only)


def test_fused_kernel_idle_waves_use_the_helper():
    src = _code("select_decode.hip")
    assert "STAGED = true" in src
    assert re.search(r"for \(int i = 0; i < decode_body_barriers\(true\); \+\+i\) __syncthreads\(\);", src)
