"""The C-ABI library loads, exports every function include/reshard.h declares,
and its structs have the layout the Python binding marshals (checked by
compiling the header with gcc).  No GPU needed."""

import ctypes
import os
import re
import subprocess

import pytest

from rl_weight_refit_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "reshard.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:rs_status|void|const char\*)\s+(reshard_\w+)\s*\(",
                                 text, re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("reshard_plan", "reshard_execute", "reshard_plan_destroy", "reshard_last_error",
              "reshard_plan_info", "reshard_plan_region", "reshard_shard_box"):
        assert n in names


def test_every_declared_symbol_is_exported():
    lib = binding.load()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing


STRUCTS = {
    "rs_view": (binding.View, ["base", "strides"]),
    "rs_tensor_desc": (binding.TensorDesc, ["ndim", "dtype", "global_shape", "mesh_ndim",
                                            "placements", "mesh_shape", "slot_of_coord", "views",
                                            "quant", "scale_views", "split_dim0", "scale_of",
                                            "scale_block"]),
    "rs_plan_opts": (binding.PlanOpts, ["struct_size", "fanout", "unit_bytes", "tiny_bytes",
                                        "thin_bytes", "reserved"]),
    "rs_plan_info": (binding.PlanInfo, [f[0] for f in binding.PlanInfo._fields_]),
    "rs_region": (binding.Region, [f[0] for f in binding.Region._fields_]),
}


def test_struct_layouts_match_header(tmp_path):
    src = ['#include <stdio.h>', '#include <stddef.h>', '#include "reshard.h"', 'int main(void){']
    for s, (_, fields) in STRUCTS.items():
        src.append('printf("%s size %%zu\\n", sizeof(%s));' % (s, s))
        for f in fields:
            src.append('printf("%s.%s %%zu\\n", offsetof(%s, %s));' % (s, f, s, f))
    src.append("return 0;}")
    c = tmp_path / "layout.c"
    c.write_text("\n".join(src))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(c), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    got = dict(l.rsplit(" ", 1) for l in out if l)
    for s, (cls, fields) in STRUCTS.items():
        assert int(got["%s size" % s]) == ctypes.sizeof(cls), s
        for f in fields:
            assert int(got["%s.%s" % (s, f)]) == getattr(cls, f).offset, (s, f)


def test_last_error_is_empty_after_success():
    plan = binding.reshard_plan([{"shape": [4], "dtype": "u8", "mesh": [1], "placements": [-1]}],
                                [{"shape": [4], "dtype": "u8", "mesh": [2], "placements": [0]}])
    plan.info()
    assert binding.reshard_last_error() == ""


C_CLIENT = r"""
#include <stdio.h>
#include "reshard.h"
int main(void) {
  rs_tensor_desc src = {0}, dst = {0};
  src.ndim = 2; src.dtype = RS_BF16;
  src.global_shape[0] = 14336; src.global_shape[1] = 4096;
  src.mesh_ndim = 1; src.mesh_shape[0] = 4; src.placements[0] = 0;
  dst = src;
  dst.mesh_ndim = 2; dst.mesh_shape[0] = 2; dst.mesh_shape[1] = 2;
  dst.placements[0] = 0; dst.placements[1] = RS_REPLICATE;
  rs_plan* plan = NULL;
  if (reshard_plan(&src, &dst, 1, NULL, &plan) != RS_OK) {
    fprintf(stderr, "%s", reshard_last_error());
    return 1;
  }
  rs_plan_info info;
  if (reshard_plan_info(plan, &info) != RS_OK) return 2;
  int64_t off[RS_MAX_DIMS], len[RS_MAX_DIMS];
  if (reshard_shard_box(&dst, 3, off, len) != RS_OK) return 3;
  printf("%llu %llu %llu %lld %lld\n", (unsigned long long)info.n_src_ptrs,
         (unsigned long long)info.n_dst_ptrs, (unsigned long long)info.bytes_written,
         (long long)off[0], (long long)len[0]);
  reshard_plan_destroy(plan);
  dst.placements[1] = 7;   /* not a tensor dim */
  if (reshard_plan(&src, &dst, 1, NULL, &plan) != RS_ERR_INVALID) return 4;
  printf("%s", reshard_last_error());
  return 0;
}
"""


def test_plain_c_client(tmp_path):
    """A C99 program compiled with gcc against the header and the library
    plans a layout, reads its summary and a shard box, and gets a readable
    error for a bad placement (planning needs no GPU)."""
    src = tmp_path / "client.c"
    src.write_text(C_CLIENT)
    exe = tmp_path / "client"
    libdir = os.path.dirname(binding.LIB_PATH)
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                        str(src), "-o", str(exe), "-L", libdir, "-lreshard", "-Wl,-rpath," + libdir],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    first, rest = r.stdout.split("\n", 1)
    # 4 source and 4 destination slots; both DP replicas receive 14336 x 4096 bf16; slot 3 = rows 7168..
    assert first.split() == ["4", "4", str(2 * 14336 * 4096 * 2), "7168", "7168"]
    assert "placements[1] = 7" in rest
