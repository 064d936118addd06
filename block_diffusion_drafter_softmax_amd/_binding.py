"""ctypes binding of libdflash.so: the C ABI of include/dflash.h, one Python
function per entry point, same names, argument marshalling only.

The library must have been built (``python -m
block_diffusion_drafter_softmax_amd.build``); importing this module without it
raises, there is no fallback path.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdflash.so")

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_CAPACITY = -3
ERR_HIP = -4

DEV_BAD_SEQ = 1
DEV_BAD_N_NEW = 2
DEV_NO_PAGES = 4
DEV_BAD_PAGE = 8
DEV_BAD_TOKEN = 16

DTYPE_BF16 = 0
DTYPE_F32 = 1

K_FUSE, K_CTX_KV, K_NORM, K_QKV, K_ATTN, K_ATTN_MERGE, K_OPROJ, K_GATE_UP, K_DOWN, \
    K_LM_HEAD, K_ARGMAX, K_VERIFY, K_QKV_FINISH, K_CTX_FINISH, K_D2SD = range(15)
K_COUNT = 15
KERNEL_NAMES = ["fuse", "ctx_kv", "norm", "qkv", "attn", "attn_merge", "o_proj", "gate_up",
                "down", "lm_head", "argmax", "verify", "qkv_finish", "ctx_finish", "d2sd"]

EXPORTS = [
    "dflash_workspace_bytes", "dflash_create", "dflash_destroy", "dflash_ctx_append",
    "dflash_draft_block", "dflash_append_draft", "dflash_verify", "dflash_verify_noalloc", "dflash_d2sd_draft", "dflash_verify_multi",
    "dflash_draft_sample", "dflash_verify_sample",
    "dflash_last_error", "dflash_read_error", "dflash_kernel_timer", "dflash_kernel_timer_read",
]


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "hidden", "n_layers", "n_q_heads", "n_kv_heads", "head_dim", "intermediate", "vocab",
        "n_target_layers", "block_size", "page_size", "max_seqs", "max_pages_per_seq", "n_pages",
        "max_pos", "mask_token_id", "tied_kv", "use_rope", "max_batch", "max_new")] + [
        ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float), ("fusion", ctypes.c_int32)]

FUSION = {"softmax": 0, "fc": 1}


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_fuse", "g_fuse", "g_attn", "g_mlp", "g_final", "wq", "wk_d", "wv_d", "wk_t", "wv_t",
        "wo", "wg", "wu", "wd", "embed", "lm_head", "w_fc", "g_fc")]


class KV(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("kv_pages", "page_table", "ctx_len", "error_word")]


class DFlashError(RuntimeError):
    pass


def _load():
    # Device memory and streams come from PyTorch, so the library must run on
    # PyTorch's HIP runtime: load torch first; libdflash.so's libamdhip64
    # dependency then resolves to that same, already loaded runtime.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python -m block_diffusion_drafter_softmax_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64
    sig = {
        "dflash_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(Config)]),
        "dflash_create": (ctypes.c_int, [ctypes.POINTER(Config), ctypes.POINTER(Weights), ctypes.POINTER(KV),
                                         vp, ctypes.c_size_t, ctypes.POINTER(vp)]),
        "dflash_destroy": (None, [vp]),
        "dflash_ctx_append": (ctypes.c_int, [vp, i32, vp, vp, vp, i32, vp]),
        "dflash_draft_block": (ctypes.c_int, [vp, i32, vp, vp, vp, vp, vp, vp, vp]),
        "dflash_append_draft": (ctypes.c_int, [vp, i32, vp, vp, vp, i32, vp, vp, vp, vp]),
        "dflash_verify": (ctypes.c_int, [vp, i32, vp, vp, vp, i32, ctypes.c_float, u64, u64, vp, vp, vp, vp]),
        "dflash_verify_noalloc": (ctypes.c_int, [vp, i32, vp, vp, vp, i32, ctypes.c_float, u64, u64, vp, vp, vp,
                                                 vp]),
        "dflash_d2sd_draft": (ctypes.c_int, [vp, i32, vp, vp, i32, vp, vp, vp, vp]),
        "dflash_verify_multi": (ctypes.c_int, [vp, i32, i32, vp, vp, vp, i32, vp, vp, vp, vp, vp]),
        "dflash_draft_sample": (ctypes.c_int, [vp, i32, vp, vp, ctypes.c_float, u64, u64, vp, vp, vp]),
        "dflash_verify_sample": (ctypes.c_int, [vp, i32, vp, vp, vp, ctypes.c_float, vp, i32, u64, u64,
                                                vp, vp, vp, vp]),
        "dflash_last_error": (ctypes.c_char_p, []),
        "dflash_read_error": (ctypes.c_int, [vp, vp, ctypes.POINTER(i32)]),
        "dflash_kernel_timer": (ctypes.c_int, [vp, i32, i32]),
        "dflash_kernel_timer_read": (ctypes.c_int, [vp, i32, ctypes.POINTER(ctypes.c_double),
                                                    ctypes.POINTER(ctypes.c_int64)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


def last_error():
    return lib.dflash_last_error().decode()


def check(rc, what):
    if rc != OK:
        raise DFlashError(f"{what} failed ({rc}): {last_error()}")
    return rc


def dflash_workspace_bytes(cfg):
    return lib.dflash_workspace_bytes(ctypes.byref(cfg))


def dflash_create(cfg, weights, kv, workspace_ptr, ws_bytes):
    h = ctypes.c_void_p()
    rc = lib.dflash_create(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(kv),
                           workspace_ptr, ws_bytes, ctypes.byref(h))
    return rc, h


def dflash_destroy(ctx):
    lib.dflash_destroy(ctx)


def dflash_ctx_append(ctx, B, seq_ids, n_new, target_hidden, max_new, stream):
    return lib.dflash_ctx_append(ctx, B, seq_ids, n_new, target_hidden, max_new, stream)


def dflash_draft_block(ctx, B, seq_ids, anchor, draft, top2_gap, dbg_hidden, dbg_logits, stream):
    return lib.dflash_draft_block(ctx, B, seq_ids, anchor, draft, top2_gap, dbg_hidden, dbg_logits, stream)


def dflash_append_draft(ctx, B, seq_ids, n_new, target_hidden, max_new, anchor, draft, top2_gap, stream):
    return lib.dflash_append_draft(ctx, B, seq_ids, n_new, target_hidden, max_new, anchor, draft, top2_gap, stream)


def dflash_verify(ctx, B, seq_ids, draft, target_logits, logits_dtype, temperature, seed, step,
                  accept_len, next_token, commit_len, stream):
    return lib.dflash_verify(ctx, B, seq_ids, draft, target_logits, logits_dtype, float(temperature),
                             seed, step, accept_len, next_token, commit_len, stream)


def dflash_verify_noalloc(ctx, B, seq_ids, draft, target_logits, logits_dtype, temperature, seed, step,
                          accept_len, next_token, commit_len, stream):
    return lib.dflash_verify_noalloc(ctx, B, seq_ids, draft, target_logits, logits_dtype, float(temperature),
                                     seed, step, accept_len, next_token, commit_len, stream)


VERIFY_SCRATCH_BYTES = 1 << 20  # DFLASH_VERIFY_SCRATCH_BYTES


def dflash_d2sd_draft(ctx, B, seq_ids, anchor, K, drafts, conf, cuts, stream):
    return lib.dflash_d2sd_draft(ctx, B, seq_ids, anchor, K, drafts, conf, cuts, stream)


def dflash_verify_multi(ctx, B, C, seq_ids, drafts, target_logits, logits_dtype, accept_len, next_token,
                        commit_len, chosen, stream):
    return lib.dflash_verify_multi(ctx, B, C, seq_ids, drafts, target_logits, logits_dtype, accept_len,
                                   next_token, commit_len, chosen, stream)


def dflash_draft_sample(ctx, B, seq_ids, anchor, temperature, seed, step, draft, draft_logits, stream):
    return lib.dflash_draft_sample(ctx, B, seq_ids, anchor, float(temperature), seed, step, draft, draft_logits,
                                   stream)


def dflash_verify_sample(ctx, B, seq_ids, draft, draft_logits, draft_temperature, target_logits, logits_dtype,
                         seed, step, accept_len, next_token, commit_len, stream):
    return lib.dflash_verify_sample(ctx, B, seq_ids, draft, draft_logits, float(draft_temperature), target_logits,
                                    logits_dtype, seed, step, accept_len, next_token, commit_len, stream)


def dflash_read_error(ctx, stream):
    out = ctypes.c_int32()
    rc = lib.dflash_read_error(ctx, stream, ctypes.byref(out))
    return rc, out.value


def dflash_kernel_timer(ctx, kind, enable):
    return lib.dflash_kernel_timer(ctx, kind, int(enable))


def dflash_kernel_timer_read(ctx, kind):
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    rc = lib.dflash_kernel_timer_read(ctx, kind, ctypes.byref(ms), ctypes.byref(n))
    return rc, ms.value, n.value
