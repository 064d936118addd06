"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point include/dflash.h declares, sizes workspaces and rejects bad
arguments before touching the device."""
import ctypes
import os
import re
import subprocess

import pytest

from block_diffusion_drafter_softmax_amd import _binding as B
from block_diffusion_drafter_softmax_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "dflash.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = header_functions()
    for n in ("dflash_ctx_append", "dflash_draft_block", "dflash_verify", "dflash_create",
              "dflash_destroy", "dflash_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in header_functions():
        assert hasattr(lib, n), n
    assert sorted(B.EXPORTS) == header_functions()


def exported_functions(path):
    """Defined function symbols in the dynamic symbol table (readelf)."""
    out = subprocess.run(["readelf", "--dyn-syms", "-W", path], capture_output=True, text=True, check=True).stdout
    names = set()
    for line in out.splitlines():
        f = line.split()
        # Num: Value Size Type Bind Vis Ndx Name
        if len(f) >= 8 and f[3] == "FUNC" and f[4] in ("GLOBAL", "WEAK") and f[6] != "UND":
            names.add(f[7].split("@")[0])
    return names


def test_library_exports_nothing_but_the_header():
    """The dynamic symbol table holds exactly the header's entry points: the
    kernel launchers and helpers stay internal to the library."""
    assert exported_functions(B.LIB_PATH) == set(header_functions())


def make_cfg(name="qwen3_8b", **kw):
    cfg = synth.config(name)
    c = B.Config()
    for f, _ in B.Config._fields_:
        if f in cfg and f != "fusion":
            setattr(c, f, cfg[f])
    c.fusion = B.FUSION[cfg.get("fusion", "softmax")]
    c.page_size, c.max_seqs, c.max_pages_per_seq, c.n_pages = 16, 4, 260, 1040
    c.max_pos, c.max_batch, c.max_new = 4200, 4, 16
    c.mask_token_id = cfg["mask_token_id"]
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_workspace_sizes_every_config(name):
    c = make_cfg(name)
    n = B.dflash_workspace_bytes(c)
    assert n > 0, B.last_error()
    assert n % 256 == 0
    # more batch needs more workspace
    assert B.dflash_workspace_bytes(make_cfg(name, max_batch=8)) > n


@pytest.mark.parametrize("field,value,msg", [
    ("head_dim", 96, "head_dim"),
    ("page_size", 32, "page_size"),
    ("block_size", 17, "block_size"),
    ("hidden", 100, "hidden"),
    ("vocab", 1000, "vocab"),
    ("n_kv_heads", 5, "multiple"),
    ("mask_token_id", 10 ** 6, "mask_token_id"),
    ("max_batch", 0, "positive"),
    ("fusion", 2, "fusion"),
])
def test_bad_config_is_rejected_with_message(field, value, msg):
    c = make_cfg(**{field: value})
    assert B.dflash_workspace_bytes(c) == 0
    assert msg in B.last_error()


def test_create_rejects_null_pointers_without_device_work():
    c = make_cfg()
    w = B.Weights()
    kv = B.KV()
    rc, h = B.dflash_create(c, w, kv, None, 0)
    assert rc == B.ERR_INVALID_ARG and not h.value
    assert "required" in B.last_error()


def test_calls_reject_null_handle():
    assert B.dflash_ctx_append(None, 1, None, None, None, 1, None) == B.ERR_INVALID_ARG
    assert B.dflash_draft_block(None, 1, None, None, None, None, None, None, None) == B.ERR_INVALID_ARG
    assert B.dflash_verify(None, 1, None, None, None, 0, 0.0, 0, 0, None, None, None, None) == B.ERR_INVALID_ARG
    assert B.dflash_kernel_timer(None, 0, 1) == B.ERR_INVALID_ARG


def test_one_hip_runtime_in_process():
    """The binding's library shares PyTorch's HIP runtime (streams and device
    pointers come from torch)."""
    maps = open("/proc/self/maps").read()
    libs = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(libs) == 1, libs
