"""The header's types and prototypes are the boundary's declared ones.

The three compute calls, the two enums and the RoPE descriptor are checked
twice against the declarations they must have:

* a C11 translation unit that includes include/vx.h binds every entry point to
  a function pointer of exactly the declared type, and checks the enum values
  and the descriptor layout with static assertions; gcc compiles it with
  warnings as errors, so a changed return type, argument type or order fails;
* the prototypes in the header text, comments removed and whitespace
  normalised, equal the declarations below word for word, argument names
  included (the names carry the meaning: n_tokens, head_dim, ...).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vx.h")

# The boundary: status-returning calls with device pointers, int64 sizes,
# a vx_dtype and the caller's stream.
PROTOTYPES = {
    "vx_adaln_modulate":
        "vx_status vx_adaln_modulate(const void* x, const void* shift, const void* scale, "
        "void* y, int64_t n_tokens, int64_t hidden, float eps, vx_dtype dt, void* hip_stream);",
    "vx_rope3d_apply":
        "vx_status vx_rope3d_apply(void* q, void* k, int64_t batch, int64_t n_tokens, "
        "int64_t heads, int64_t head_dim, const vx_rope3d_desc* rope, vx_dtype dt, "
        "void* hip_stream);",
    "vx_flash_attn_fwd":
        "vx_status vx_flash_attn_fwd(const void* q, const void* k, const void* v, void* o, "
        "float* lse, int64_t batch, int64_t n_tokens, int64_t heads, int64_t head_dim, "
        "float softmax_scale, const vx_rope3d_desc* rope_q, vx_dtype dt, void* hip_stream);",
    "vx_last_error": "const char* vx_last_error(void);",
    "vx_version": "int vx_version(void);",
}

C_CHECK = r"""
#include <stddef.h>
#include <stdint.h>
#include "vx.h"

_Static_assert(VX_F32 == 0 && VX_BF16 == 1, "vx_dtype values");
_Static_assert(VX_OK == 0 && VX_ERR_NULL == 1 && VX_ERR_INVALID == 2 &&
               VX_ERR_UNSUPPORTED == 3 && VX_ERR_ALIGN == 4 && VX_ERR_HIP == 5,
               "vx_status values");
_Static_assert(sizeof(vx_dtype) == sizeof(int) && sizeof(vx_status) == sizeof(int),
               "enums are int-sized");
_Static_assert(sizeof(vx_rope3d_desc) == 36, "nine 4-byte fields");
_Static_assert(offsetof(vx_rope3d_desc, T) == 0 && offsetof(vx_rope3d_desc, H) == 4 &&
               offsetof(vx_rope3d_desc, W) == 8 && offsetof(vx_rope3d_desc, n_prefix) == 12 &&
               offsetof(vx_rope3d_desc, d_t) == 16 && offsetof(vx_rope3d_desc, d_h) == 20 &&
               offsetof(vx_rope3d_desc, d_w) == 24 && offsetof(vx_rope3d_desc, theta) == 28 &&
               offsetof(vx_rope3d_desc, pairing) == 32, "descriptor layout");

vx_status (*p_adaln)(const void*, const void*, const void*, void*, int64_t, int64_t, float,
                     vx_dtype, void*) = vx_adaln_modulate;
vx_status (*p_rope)(void*, void*, int64_t, int64_t, int64_t, int64_t, const vx_rope3d_desc*,
                    vx_dtype, void*) = vx_rope3d_apply;
vx_status (*p_attn)(const void*, const void*, const void*, void*, float*, int64_t, int64_t,
                    int64_t, int64_t, float, const vx_rope3d_desc*, vx_dtype,
                    void*) = vx_flash_attn_fwd;
vx_status (*p_adaln_ex)(const void*, const void*, const void*, void*, int64_t, int64_t, int64_t,
                        int64_t, float, vx_dtype, vx_dtype, vx_dtype, void*) = vx_adaln_modulate_ex;
vx_status (*p_attn_kv)(const void*, const void*, const void*, void*, float*, int64_t, int64_t,
                       int64_t, int64_t, int64_t, float, const vx_rope3d_desc*, vx_dtype,
                       void*) = vx_flash_attn_fwd_kv;
vx_status (*p_attn_masked)(const void*, const void*, const void*, void*, float*, int64_t, int64_t,
                           int64_t, int64_t, int64_t, float, const vx_rope3d_desc*,
                           const int32_t*, vx_dtype, void*) = vx_flash_attn_fwd_masked;
vx_status (*p_merge)(const void*, const float*, const void*, const float*, void*, float*,
                     int64_t, int64_t, int64_t, int64_t, vx_dtype, void*) = vx_attn_merge2;
const char* (*p_err)(void) = vx_last_error;
int (*p_ver)(void) = vx_version;
"""


def _prototypes(text):
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    out = {}
    for m in re.finditer(r"((?:const\s+)?\w+\s*\*?\s*(vx_\w+)\s*\([^;{]*\)\s*;)", text):
        proto = re.sub(r"\s+", " ", m.group(1)).replace("( ", "(").replace(" )", ")")
        proto = re.sub(r"\s*\*\s*", "* ", proto).replace("* ,", "*,").replace("* )", "*)")
        out[m.group(2)] = proto.replace(" ;", ";")
    return out


def test_header_prototypes_are_the_declared_ones():
    got = _prototypes(open(HEADER).read())
    for name, want in PROTOTYPES.items():
        assert got.get(name) == want, f"{name}:\n  header: {got.get(name)}\n  wanted: {want}"


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_header_compiles_as_c_with_the_declared_types(tmp_path):
    src = tmp_path / "check.c"
    src.write_text(C_CHECK)
    r = subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic",
                        "-I", os.path.join(ROOT, "include"), "-c", str(src),
                        "-o", str(tmp_path / "check.o")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
