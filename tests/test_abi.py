"""CPU checks of the C ABI: the library loads, exports every function that
include/attn.h declares, validates arguments on the host (no GPU call is
reached on any error path), and plans decode as the pages' formulas say."""

import ctypes
import os
import re

import pytest

import oracle
from softmax_attention_paged_amd import _ffi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20          # a 16-byte aligned non-null address; never dereferenced on the host


def _lib():
    if not os.path.exists(_ffi.LIB_PATH):
        pytest.fail("library not built: run `python -m softmax_attention_paged_amd.build`")
    return _ffi.load()


def _header_functions():
    text = open(os.path.join(ROOT, "include", "attn.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attn_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    lib = _lib()
    names = _header_functions()
    assert {"attn_prefill", "attn_decode_paged", "attn_merge_lse"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_ffi.EXPORTS), "binding and header disagree"


def test_ceiling_kernels_library_loads_and_rejects_bad_arguments():
    # the benchmark's measured ceilings: a separate object, checked on the
    # host only (every call below fails validation before any launch)
    path = os.path.join(ROOT, "softmax_attention_paged_amd", "libattn_ceilings.so")
    assert os.path.exists(path), "ceiling kernels not built"
    lib = ctypes.CDLL(path)
    lib.ceil_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.ceil_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    assert lib.ceil_stream_read(FAKE, 1000, FAKE, 64, None) == -1        # not a multiple of 16 KiB
    assert lib.ceil_stream_read(FAKE + 8, 16384, FAKE, 64, None) == -1   # misaligned
    assert lib.ceil_stream_read(None, 16384, FAKE, 64, None) == -1
    assert lib.ceil_mfma_bf16(FAKE, 0, 8, None) == -1
    assert lib.ceil_mfma_bf16(None, 8, 8, None) == -1
    lib.ceil_mfma_bf16_varied.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    assert lib.ceil_mfma_bf16_varied(FAKE, 12, 8, None) == -1       # not a multiple of 8
    assert lib.ceil_mfma_bf16_varied(FAKE, 0, 8, None) == -1
    assert lib.ceil_mfma_bf16_varied(None, 8, 8, None) == -1
    assert lib.ceil_mfma_bf16_varied(FAKE, 8, 0, None) == -1
    lib.ceil_mfma_fma_overlap.argtypes = [ctypes.c_void_p] + [ctypes.c_int] * 5 + [ctypes.c_void_p]
    for bad in ((None, 0, 1, 8, 8, 4), (FAKE, 2, 1, 8, 8, 4), (FAKE, 0, 0, 8, 8, 4), (FAKE, 0, 4, 8, 8, 4),
                (FAKE, 0, 3, 0, 8, 4), (FAKE, 0, 3, 8, 0, 4), (FAKE, 1, 3, 8, 8, 0)):
        assert lib.ceil_mfma_fma_overlap(*bad, None) == -1
    lib.ceil_lds_read.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    for bad in ((None, 0, 8, 4), (FAKE, 2, 8, 4), (FAKE, 0, 12, 4), (FAKE, 1, 0, 4), (FAKE, 0, 8, 0)):
        assert lib.ceil_lds_read(*bad, None) == -1


def test_ctypes_mirrors_match_the_c_compiler_layout(tmp_path):
    # gcc compiles a probe against include/attn.h that prints sizeof and the
    # offset of every field the ctypes mirrors declare; the two must agree.
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    structs = {"attn_prefill_params": _ffi.PrefillParams, "attn_decode_params": _ffi.DecodeParams,
               "attn_decode_plan_info": _ffi.DecodePlanInfo, "attn_cache_append_params": _ffi.CacheAppendParams,
               "attn_mla_kv_pack_params": _ffi.MlaKvPackParams}
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{os.path.join(ROOT, "include", "attn.h")}"',
             "int main(void) {"]
    expect = []
    for cname, cls in structs.items():
        lines.append(f'  printf("%zu\\n", sizeof({cname}));')
        expect.append(ctypes.sizeof(cls))
        for fname, _ in cls._fields_:
            lines.append(f'  printf("%zu\\n", offsetof({cname}, {fname}));')
            expect.append(getattr(cls, fname).offset)
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    cc = subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", str(src), "-o", str(exe)],
                        capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got == expect


def test_struct_sizes_match_c_layout():
    # ctypes mirrors must match the C layout (checked against offsets the C
    # compiler would use: pointers and int64 are 8-aligned, int32/float 4).
    assert ctypes.sizeof(_ffi.DecodePlanInfo) == 48
    assert _ffi.DecodeParams.workspace.offset % 8 == 0
    assert _ffi.PrefillParams.lse.offset % 8 == 0


def test_status_strings():
    lib = _lib()
    for code, name in [(0, "ATTN_OK"), (1, "ATTN_ERR_INVALID_ARG"), (2, "ATTN_ERR_UNSUPPORTED"),
                       (3, "ATTN_ERR_WORKSPACE_TOO_SMALL"), (4, "ATTN_ERR_HIP")]:
        assert lib.attn_status_string(code).decode() == name


def decode_params(**kw):
    p = _ffi.DecodeParams()
    d = dict(q=FAKE, k_cache=FAKE, v_cache=FAKE + 4096, k_stride_page=16 * 2 * 128, k_stride_tok=2 * 128,
             k_stride_head=128, v_stride_page=16 * 2 * 128, v_stride_tok=2 * 128, v_stride_head=128,
             kv_dtype=_ffi.ATTN_BF16, k_scale=1.0, v_scale=1.0, seq_lens=FAKE, block_table=FAKE,
             block_table_stride=8, batch=2, q_len=1, num_q_heads=8, num_kv_heads=2, head_dim_qk=128,
             head_dim_v=128, page_size=16, num_pages=16, max_seq_len=100, softmax_scale=0.125, causal=0,
             num_splits=0, workspace=None, workspace_bytes=0, o=FAKE, lse=None)
    d.update(kw)
    for k, v in d.items():
        setattr(p, k, v)
    return p


def plan(p):
    info = _ffi.DecodePlanInfo()
    st = _lib().attn_decode_plan(ctypes.byref(p), ctypes.byref(info))
    return st, info


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(o=None), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(num_q_heads=7), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(head_dim_qk=96, head_dim_v=96), _ffi.ATTN_ERR_UNSUPPORTED),
    (dict(head_dim_v=64), _ffi.ATTN_ERR_UNSUPPORTED),
    (dict(page_size=24), _ffi.ATTN_ERR_UNSUPPORTED),
    (dict(page_size=8), _ffi.ATTN_ERR_UNSUPPORTED),
    (dict(q_len=5), _ffi.ATTN_ERR_UNSUPPORTED),
    (dict(q_len=0), _ffi.ATTN_ERR_UNSUPPORTED),
    (dict(max_seq_len=16 * 16 + 1), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(block_table_stride=6), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(softmax_scale=float("nan")), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(causal=2), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(num_splits=257), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(k_scale=0.5), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(kv_dtype=_ffi.ATTN_FP8_E4M3), _ffi.ATTN_ERR_UNSUPPORTED),
    (dict(q=FAKE + 8), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(k_stride_tok=100), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(num_q_heads=68, num_kv_heads=2), _ffi.ATTN_ERR_UNSUPPORTED),
    (dict(window_enabled=2), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(window_enabled=1, window_left=-3), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(q_dtype=7), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(q_dtype=_ffi.ATTN_FP8_E4M3, q_scale=1.0), _ffi.ATTN_ERR_UNSUPPORTED),    # fp8 q needs an fp8 latent cache
    # the caches and the block table may be empty only when no request has a key
    (dict(k_cache=None), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(block_table=None), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(num_pages=0), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(v_cache=FAKE + 8), _ffi.ATTN_ERR_INVALID_ARG),
])
def test_decode_validation_errors(kw, code):
    lib = _lib()
    p = decode_params(**kw)
    st = lib.attn_decode_paged(ctypes.byref(p), None)
    assert st == code, (st, lib.attn_last_error())
    assert lib.attn_last_error().decode() != ""


def test_workspace_too_small_is_reported_before_launch():
    lib = _lib()
    p = decode_params(num_splits=4)
    need = lib.attn_decode_workspace_size(ctypes.byref(p))
    assert need == 4 * (2 * 1 * 8) * (128 + 1) * 4
    p.workspace, p.workspace_bytes = FAKE, need - 4
    assert lib.attn_decode_paged(ctypes.byref(p), None) == _ffi.ATTN_ERR_WORKSPACE_TOO_SMALL
    p.workspace = None
    assert lib.attn_decode_paged(ctypes.byref(p), None) == _ffi.ATTN_ERR_WORKSPACE_TOO_SMALL


def test_batch_zero_is_a_no_op():
    lib = _lib()
    p = decode_params(batch=0, q=None, o=None)
    assert lib.attn_decode_paged(ctypes.byref(p), None) == _ffi.ATTN_OK


def test_merge_validation():
    lib = _lib()
    assert lib.attn_merge_lse(FAKE, FAKE, 0, 10, 128, FAKE, _ffi.ATTN_BF16, None, None) == _ffi.ATTN_ERR_INVALID_ARG
    assert lib.attn_merge_lse(FAKE, FAKE, 300, 10, 128, FAKE, _ffi.ATTN_BF16, None, None) == _ffi.ATTN_ERR_INVALID_ARG
    assert lib.attn_merge_lse(FAKE, FAKE, 2, 10, 130, FAKE, _ffi.ATTN_BF16, None, None) == _ffi.ATTN_ERR_UNSUPPORTED
    assert lib.attn_merge_lse(FAKE, FAKE, 2, 10, 128, FAKE, _ffi.ATTN_FP8_E4M3, None, None) == _ffi.ATTN_ERR_UNSUPPORTED
    assert lib.attn_merge_lse(None, FAKE, 2, 10, 128, FAKE, _ffi.ATTN_BF16, None, None) == _ffi.ATTN_ERR_INVALID_ARG
    assert lib.attn_merge_lse(None, None, 2, 0, 128, None, _ffi.ATTN_BF16, None, None) == _ffi.ATTN_OK


def prefill_params(**kw):
    p = _ffi.PrefillParams()
    d = dict(q=FAKE, q_stride_tok=32 * 128, q_stride_head=128, k=FAKE, v=FAKE, k_stride_page=0,
             k_stride_tok=32 * 128, k_stride_head=128, v_stride_page=0, v_stride_tok=32 * 128,
             v_stride_head=128, cu_seqlens_q=FAKE, cu_seqlens_kv=FAKE, seq_lens_kv=None, block_table=None,
             block_table_stride=0, page_size=0, num_pages=0, batch=1, num_q_heads=32, num_kv_heads=32,
             head_dim_qk=128, head_dim_v=128, max_seqlen_q=8192, max_seqlen_kv=8192, softmax_scale=0.088,
             causal=1, o=FAKE, o_stride_tok=32 * 128, o_stride_head=128, lse=None)
    d.update(kw)
    for k, v in d.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(cu_seqlens_kv=None), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(num_kv_heads=5), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(head_dim_qk=96, head_dim_v=96), _ffi.ATTN_ERR_UNSUPPORTED),
    (dict(head_dim_v=64), _ffi.ATTN_ERR_UNSUPPORTED),
    (dict(block_table=FAKE, seq_lens_kv=FAKE, page_size=48, num_pages=1000, block_table_stride=1000),
     _ffi.ATTN_ERR_UNSUPPORTED),
    (dict(block_table=FAKE, seq_lens_kv=None, page_size=64, num_pages=1000, block_table_stride=1000),
     _ffi.ATTN_ERR_INVALID_ARG),
    (dict(block_table=FAKE, seq_lens_kv=FAKE, page_size=64, num_pages=10, block_table_stride=1000),
     _ffi.ATTN_ERR_INVALID_ARG),
    (dict(q_stride_head=100), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(causal=3), _ffi.ATTN_ERR_INVALID_ARG),
    # K/V may be empty only when no request has a key (max_seqlen_kv == 0)
    (dict(k=None), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(v_stride_tok=0), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(k_stride_head=100), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(block_table=FAKE, seq_lens_kv=FAKE, page_size=64, num_pages=0, block_table_stride=1000),
     _ffi.ATTN_ERR_INVALID_ARG),
])
def test_prefill_validation_errors(kw, code):
    lib = _lib()
    p = prefill_params(**kw)
    assert lib.attn_prefill(ctypes.byref(p), None) == code, lib.attn_last_error()


def test_forced_prefill_splits_without_workspace_are_errors():
    """A forced kv_splits > 1 never runs unsplit in silence: a missing or too
    small workspace is ATTN_ERR_WORKSPACE_TOO_SMALL, a misaligned one
    ATTN_ERR_INVALID_ARG, FP8 inputs or a non-contiguous o
    ATTN_ERR_UNSUPPORTED, and total_q <= 0 ATTN_ERR_INVALID_ARG. All are
    reported before anything is enqueued (the pointers are fake)."""
    lib = _lib()
    base = dict(max_seqlen_q=512, max_seqlen_kv=81920, total_q=512, kv_splits=4)
    p = prefill_params(**base)
    need = lib.attn_prefill_workspace_size(ctypes.byref(p))
    assert need == 4 * 512 * 32 * 129 * 4
    for ws, nbytes, code in ((None, 0, _ffi.ATTN_ERR_WORKSPACE_TOO_SMALL),
                             (FAKE, need - 16, _ffi.ATTN_ERR_WORKSPACE_TOO_SMALL),
                             (FAKE + 8, need, _ffi.ATTN_ERR_INVALID_ARG)):
        p = prefill_params(workspace=ws, workspace_bytes=nbytes, **base)
        assert lib.attn_prefill(ctypes.byref(p), None) == code, lib.attn_last_error()
        assert lib.attn_last_error()
    p = prefill_params(**dict(base, total_q=0), workspace=FAKE, workspace_bytes=need)
    assert lib.attn_prefill(ctypes.byref(p), None) == _ffi.ATTN_ERR_INVALID_ARG
    p = prefill_params(**base, workspace=FAKE, workspace_bytes=need, o_stride_tok=64 * 128)
    assert lib.attn_prefill(ctypes.byref(p), None) == _ffi.ATTN_ERR_UNSUPPORTED
    p = prefill_params(**base, workspace=FAKE, workspace_bytes=need, qkv_dtype=_ffi.ATTN_FP8_E4M3,
                       head_dim_qk=192, head_dim_v=128, q_scale=1.0, k_scale=1.0, v_scale=1.0,
                       q_stride_tok=32 * 192, q_stride_head=192, k_stride_tok=32 * 192, k_stride_head=192)
    assert lib.attn_prefill(ctypes.byref(p), None) == _ffi.ATTN_ERR_UNSUPPORTED
    # the planner's own choice (kv_splits = 0) still runs unsplit without a workspace:
    # validation passes, and the (fake) launch is the first thing that could fail
    p = prefill_params(**dict(base, kv_splits=0))
    assert lib.attn_prefill_workspace_size(ctypes.byref(p)) > 0


# ------------------------------------------------------------- planner --

def test_fold_matches_tokenspeed_example_for_latent_decode():
    # H64, q_len 4 -> F = 2, H_eff = 128, q_eff = 2 (the pages' worked example)
    p = decode_params(num_q_heads=64, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, q_len=4,
                      v_cache=FAKE, k_stride_page=64 * 576, k_stride_tok=576, k_stride_head=576,
                      v_stride_page=64 * 576, v_stride_tok=576, v_stride_head=576, page_size=64,
                      num_pages=10240, max_seq_len=81920, block_table_stride=1280, batch=8)
    st, info = plan(p)
    assert st == 0
    f = oracle.fold_factor(64, 4)
    assert (info.fold, info.q_groups, info.rows_per_unit) == (f, 4 // f, 64 * f) == (2, 2, 128)


def test_latent_workspace_equals_tokenspeed_formula():
    # Our partial layout is S x R x (Dv + 1) fp32 with R = B * q_len * H;
    # for H * q_len a multiple of 128 it equals B * 128 * ceil(H q / 128) * S * 513 * 4.
    for splits in (1, 2, 5, 16):
        p = decode_params(num_q_heads=64, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, q_len=4,
                          v_cache=FAKE, k_stride_page=64 * 576, k_stride_tok=576, k_stride_head=576,
                          v_stride_page=64 * 576, v_stride_tok=576, v_stride_head=576, page_size=64,
                          num_pages=10240, max_seq_len=81920, block_table_stride=1280, batch=8,
                          num_splits=splits)
        st, info = plan(p)
        assert st == 0 and info.num_splits == splits
        assert info.workspace_bytes == oracle.mla_packed_workspace_bytes(8, 64, 4, splits)


@pytest.mark.parametrize("batch,splits", [(8, 16), (12, 10), (24, 16), (64, 2)])
def test_latent_planner_fills_whole_rounds(batch, splits):
    # one workgroup per CU: units = batch x 2 query groups x S; the planner
    # takes whole rounds of 256 (16 x 16, 48 x 16 = 3 x 256, 128 x 2)
    # or just under one (24 x 10 = 240) rather than a partial last round
    p = decode_params(num_q_heads=64, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, q_len=4,
                      v_cache=FAKE, k_stride_page=64 * 576, k_stride_tok=576, k_stride_head=576,
                      v_stride_page=64 * 576, v_stride_tok=576, v_stride_head=576, page_size=64,
                      num_pages=10240 * 8, max_seq_len=81920, block_table_stride=1280, batch=batch)
    st, info = plan(p)
    assert st == 0 and info.num_splits == splits


@pytest.mark.parametrize("batch,max_len,total,hkv,d", [
    (600, 8192, 2_500_000, 8, 128), (600, 4096, 600 * 4096, 8, 128), (700, 513, 2000 * 4, 2, 64),
    (520, 4096, 400000, 8, 256), (600, 8192, 1000, 8, 128)])
def test_gqa_split_planner_with_total_keys_fits_one_round(batch, max_len, total, hkv, d):
    # above 512 requests the GQA plan splits each request: a request walking
    # n keys has at most n / L + 1 units per KV head, so the plan must keep
    # (total / L + batch) * Hkv within the resident waves (12 per CU at D 128,
    # 16 at D 64, 8 at D 256), unless even one split per request does not fit
    p = decode_params(num_q_heads=hkv * 4, num_kv_heads=hkv, head_dim_qk=d, head_dim_v=d, q_len=1, batch=batch,
                      max_seq_len=max_len, page_size=128, num_pages=(max_len // 128 + 1) * batch,
                      block_table_stride=max_len // 128 + 1, k_stride_page=128 * hkv * d, k_stride_tok=hkv * d,
                      k_stride_head=d, v_stride_page=128 * hkv * d, v_stride_tok=hkv * d, v_stride_head=d)
    p.total_kv_tokens = total
    st, info = plan(p)
    assert st == 0 and info.key_ranges == 0
    L = info.split_tokens
    assert L % 32 == 0 and info.num_splits * L >= max_len and (info.num_splits - 1) * L < max_len
    slots = 256 * {64: 16, 128: 12, 256: 8}[d]
    if slots // hkv > batch:
        assert min(total / L + batch, batch * info.num_splits) * hkv <= slots
        assert L >= 256 or info.num_splits == 1
    p.total_kv_tokens = -1
    assert plan(p)[0] == _ffi.ATTN_ERR_INVALID_ARG


@pytest.mark.parametrize("max_len,batch,d,expect_unsplit", [
    (256, 64, 128, True), (257, 64, 128, False), (1, 1, 64, True), (200, 384, 128, True),
    (200, 385, 128, False), (256, 512, 64, True), (288, 512, 64, False), (224, 256, 256, True),
    (224, 257, 256, False)])
def test_short_decodes_run_unsplit(max_len, batch, d, expect_unsplit):
    # a GQA decode whose max_seq_len bound is at most 8 tiles of 32 keys, with
    # every (request, KV head, q-group) unit resident at once (resident waves:
    # 256 CUs x 16 / 12 / 8 at D 64 / 128 / 256), runs as one unsplit launch
    # without partials; otherwise the planner keeps its key ranges (or splits
    # past 512 requests)
    hkv = 8
    p = decode_params(num_q_heads=5 * hkv, num_kv_heads=hkv, head_dim_qk=d, head_dim_v=d, q_len=1, batch=batch,
                      max_seq_len=max_len, page_size=128, num_pages=(max_len // 128 + 1) * batch,
                      block_table_stride=max_len // 128 + 1, k_stride_page=128 * hkv * d, k_stride_tok=hkv * d,
                      k_stride_head=d, v_stride_page=128 * hkv * d, v_stride_tok=hkv * d, v_stride_head=d)
    st, info = plan(p)
    assert st == 0
    if expect_unsplit:
        assert (info.key_ranges, info.num_splits, info.workspace_bytes) == (0, 1, 0)
        assert info.num_units == batch * hkv
    else:
        assert info.key_ranges > 0 or info.num_splits > 1
    if max_len >= 64:
        p.num_splits = 2             # a caller's split count still wins
        assert plan(p)[1].num_splits == 2


@pytest.mark.parametrize("batch,max_len,total,hkv,d,q_len", [
    (64, 8192, 256194, 8, 128, 1), (64, 8192, 0, 8, 128, 1), (8, 65536, 300000, 8, 128, 1),
    (17, 513, 2000, 2, 64, 1), (200, 4096, 400000, 8, 256, 1), (64, 8192, 1000, 8, 128, 1),
    (512, 100, 0, 1, 64, 1), (3, 64, 0, 2, 128, 4), (1, 1, 0, 8, 128, 1)])
def test_gqa_key_range_plan(batch, max_len, total, hkv, d, q_len):
    # up to 512 requests the GQA plan cuts the batch's 32-key tiles into K
    # equal ranges: K = 8 waves per CU / (Hkv q_groups), at most 512, and
    # at most one per 2 tiles of the batch (bounded by max_seq_len, or by the
    # host total when given); partial slots K + batch per row of a request
    hq = hkv * 4
    p = decode_params(num_q_heads=hq, num_kv_heads=hkv, head_dim_qk=d, head_dim_v=d, q_len=q_len, batch=batch,
                      max_seq_len=max_len, page_size=128, num_pages=(max_len // 128 + 1) * batch,
                      block_table_stride=max_len // 128 + 1, k_stride_page=128 * hkv * d, k_stride_tok=hkv * d,
                      k_stride_head=d, v_stride_page=128 * hkv * d, v_stride_tok=hkv * d, v_stride_head=d)
    p.total_kv_tokens = total
    st, info = plan(p)
    assert st == 0
    if -(-max(max_len, 1) // 32) <= 8 and batch * hkv * info.q_groups <= 256 * {64: 16, 128: 12, 256: 8}[d]:
        # no request walks more than 8 tiles and every unit is resident: unsplit
        assert (info.key_ranges, info.num_splits, info.workspace_bytes) == (0, 1, 0)
        return
    slots = 256 * 8                  # two waves per SIMD stream the key ranges
    upper = batch * (-(-max(max_len, 1) // 32) + 1)
    if total:
        upper = min(upper, -(-total // 32) + batch)
    k = max(1, min(slots // (hkv * info.q_groups), 512, -(-upper // 2)))
    assert info.key_ranges == k
    assert info.num_splits == 0 and info.split_tokens == 0
    assert info.num_units == k * hkv * info.q_groups
    assert info.workspace_bytes == (0 if k == 1 else (k + batch) * q_len * hq * (d + 1) * 4)


def test_gqa_plan_folds_heads_and_tokens_into_16_rows():
    for q_len, hq, hkv, expect_f in [(1, 40, 8, 1), (4, 8, 2, 4), (4, 20, 4, 2), (3, 8, 8, 3), (4, 16, 1, 1)]:
        st, info = plan(decode_params(q_len=q_len, num_q_heads=hq, num_kv_heads=hkv, block_table_stride=8))
        assert st == 0
        assert info.group == hq // hkv
        assert info.fold == expect_f == oracle.fold_factor(hq // hkv, q_len, 16)
        assert info.rows_per_unit == info.group * info.fold <= 16
        assert info.q_groups * info.fold == q_len


def test_split_plan_is_nonempty_and_tile_aligned():
    # per-request splits (above 512 requests): whole tiles, every split non-empty
    for max_len in (1, 31, 100, 1000, 8192, 81920):
        pages = -(-max_len // 16)
        st, info = plan(decode_params(batch=513, max_seq_len=max_len, num_pages=pages, block_table_stride=pages))
        assert st == 0 and info.key_ranges == 0
        assert info.split_tokens % 32 == 0
        assert (info.num_splits - 1) * info.split_tokens < max(max_len, 1) <= info.num_splits * info.split_tokens
        assert info.num_units == 513 * 2 * info.num_splits
        assert info.workspace_bytes == (0 if info.num_splits == 1 else info.num_splits * 513 * 8 * 129 * 4)


def test_qwen3_14b_decode_plan():
    pages = 2200
    p = decode_params(batch=64, num_q_heads=40, num_kv_heads=8, page_size=128, num_pages=pages,
                      max_seq_len=8192, block_table_stride=64, k_stride_page=128 * 8 * 128,
                      k_stride_tok=8 * 128, v_stride_page=128 * 8 * 128, v_stride_tok=8 * 128)
    st, info = plan(p)
    assert st == 0
    assert (info.group, info.fold, info.rows_per_unit) == (5, 1, 5)
    # 2048 streaming waves (256 CUs x 8) over 8 KV heads: 256 key ranges
    assert info.key_ranges == 256 and info.num_units == 2048
    assert info.workspace_bytes == (256 + 64) * 40 * 129 * 4


def test_packed_q_must_be_a_flag():
    lib = _lib()
    p = decode_params(packed_q=2)
    assert lib.attn_decode_paged(ctypes.byref(p), None) == _ffi.ATTN_ERR_INVALID_ARG


def _latent(**kw):
    d = dict(num_kv_heads=1, head_dim_qk=576, head_dim_v=512, v_cache=FAKE, k_stride_page=64 * 576,
             k_stride_tok=576, k_stride_head=576, v_stride_page=64 * 576, v_stride_tok=576,
             v_stride_head=576, page_size=64, num_pages=10240, max_seq_len=81920, block_table_stride=1280,
             batch=8)
    d.update(kw)
    return decode_params(**d)


def test_packed_q_tiles_match_tokenspeed_h96_example():
    # "TokenSpeed-MLA", packed-query paragraph: at 96 heads and 4 query
    # tokens, packed rows fill 3 tiles of 128 across the tokens, while folded
    # rows need 4 (one 96-row group per token)
    st, folded = plan(_latent(num_q_heads=96, q_len=4))
    assert st == 0 and (folded.fold, folded.q_groups, folded.rows_per_unit) == (1, 4, 96)
    st, packed = plan(_latent(num_q_heads=96, q_len=4, packed_q=1))
    assert st == 0
    assert packed.q_groups == oracle.packed_query_tiles(96, 4) == 3 and packed.rows_per_unit == 128
    # H64 q4: packing and folding coincide (two tiles of 128)
    st, p64 = plan(_latent(num_q_heads=64, q_len=4, packed_q=1))
    assert st == 0 and (p64.q_groups, p64.rows_per_unit) == (2, 128)
    # GQA: 5 heads x 4 tokens = 20 rows -> ceil(20 / 16) tiles of 16
    st, g = plan(decode_params(q_len=4, num_q_heads=40, num_kv_heads=8, packed_q=1))
    assert st == 0 and (g.fold, g.q_groups, g.rows_per_unit) == (1, 2, 16)
    # the workspace does not depend on the packing (partials are indexed by row)
    st, a = plan(_latent(num_q_heads=96, q_len=4, num_splits=4))
    st, b = plan(_latent(num_q_heads=96, q_len=4, num_splits=4, packed_q=1))
    assert a.workspace_bytes == b.workspace_bytes == 4 * 8 * 4 * 96 * 513 * 4


def test_window_plans_splits_over_the_window():
    # with a window the walk covers the q_len block plus window_left keys of
    # context (plus tile alignment), so the split plan follows the window
    st, full = plan(_latent(num_q_heads=64, q_len=4))
    st2, win = plan(_latent(num_q_heads=64, q_len=4, window_enabled=1, window_left=100))
    assert st == st2 == 0
    assert full.num_splits > 1
    assert win.num_splits == 1 and win.split_tokens >= 100 + 4 and win.split_tokens % 32 == 0
    st, g = plan(decode_params(batch=513, max_seq_len=256, num_pages=16, block_table_stride=16, window_enabled=1,
                               window_left=1000))
    assert st == 0 and g.num_splits * g.split_tokens >= 256     # a window wider than the history
    # key ranges: the tile bound per request follows the window (300 + 4 + 31
    # keys: 11 tiles + 1 of alignment), so K is capped at one per 2 of them
    st, kr = plan(decode_params(batch=4, max_seq_len=8192, num_pages=512, block_table_stride=512, q_len=4,
                                window_enabled=1, window_left=300))
    assert st == 0 and kr.key_ranges == -(-4 * (-(-(300 + 4 + 31) // 32) + 1) // 2)
    # a window of 100 keys walks at most 5 tiles: one unsplit launch
    st, kr = plan(decode_params(batch=4, max_seq_len=8192, num_pages=512, block_table_stride=512, q_len=4,
                                window_enabled=1, window_left=100))
    assert st == 0 and (kr.key_ranges, kr.num_splits, kr.workspace_bytes) == (0, 1, 0)



def append_params(**kw):
    p = _ffi.CacheAppendParams()
    d = dict(k_new=FAKE, k_new_stride_tok=8 * 128, k_new_stride_head=128, v_new=FAKE, v_new_stride_tok=8 * 128,
             v_new_stride_head=128, k_cache=FAKE, k_stride_page=16 * 8 * 128, k_stride_tok=8 * 128,
             k_stride_head=128, v_cache=FAKE, v_stride_page=16 * 8 * 128, v_stride_tok=8 * 128, v_stride_head=128,
             cache_dtype=_ffi.ATTN_BF16, k_scale=1.0, v_scale=1.0, slot_mapping=FAKE, layer_base_rows=0,
             num_cache_rows=1024, num_tokens=4, num_kv_heads=8, head_dim_k=128, head_dim_v=128, page_size=16)
    d.update(kw)
    for k, v in d.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("kw,code", [
    (dict(num_tokens=-1), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(head_dim_k=100), _ffi.ATTN_ERR_UNSUPPORTED),
    (dict(head_dim_v=2048), _ffi.ATTN_ERR_UNSUPPORTED),
    (dict(cache_dtype=_ffi.ATTN_FP32), _ffi.ATTN_ERR_UNSUPPORTED),
    (dict(k_scale=2.0), _ffi.ATTN_ERR_INVALID_ARG),                    # bf16 takes scale 1
    (dict(cache_dtype=_ffi.ATTN_FP8_E4M3, k_scale=0.0), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(cache_dtype=_ffi.ATTN_FP8_E4M3, v_scale=float("nan")), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(page_size=24), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(layer_base_rows=-16), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(slot_mapping=None), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(slot_mapping=FAKE + 4), _ffi.ATTN_ERR_INVALID_ARG),          # int64 alignment
    (dict(k_new=FAKE + 8), _ffi.ATTN_ERR_INVALID_ARG),                 # 16-byte chunks
    (dict(k_stride_tok=8 * 128 + 4), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(v_cache=None), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(k_new_stride_head=-128), _ffi.ATTN_ERR_INVALID_ARG),
])
def test_cache_append_validation_errors(kw, code):
    lib = _lib()
    assert lib.attn_cache_append(ctypes.byref(append_params(**kw)), None) == code
    assert lib.attn_last_error().decode() != ""


def test_cache_append_accepts_a_latent_fp8_cache_without_v_and_zero_tokens():
    lib = _lib()
    # FP8 latent cache: 8-byte aligned rows suffice, no V; zero tokens enqueue nothing
    p = append_params(v_new=None, v_cache=None, head_dim_v=0, cache_dtype=_ffi.ATTN_FP8_E4M3, k_scale=0.5,
                      head_dim_k=576, k_new_stride_tok=576, k_new_stride_head=576, k_cache=FAKE + 8,
                      k_stride_page=64 * 576, k_stride_tok=576, k_stride_head=576, num_kv_heads=1, num_tokens=0)
    assert lib.attn_cache_append(ctypes.byref(p), None) == _ffi.ATTN_OK


def pack_params(**kw):
    p = _ffi.MlaKvPackParams()
    d = dict(k_nope=FAKE, k_nope_stride_tok=16 * 128, k_nope_stride_head=128, k_rope=FAKE, k_rope_stride_tok=64,
             v=FAKE, v_stride_tok=16 * 128, v_stride_head=128, k_out=FAKE, k_out_stride_tok=16 * 192,
             k_out_stride_head=192, v_out=FAKE, v_out_stride_tok=16 * 128, v_out_stride_head=128,
             k_scale=0.01, v_scale=0.01, num_tokens=0, num_heads=16, d_nope=128, d_rope=64, d_v=128)
    d.update(kw)
    for k, v in d.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("kw,code", [
    (dict(num_heads=0), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(d_nope=100), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(d_rope=-8), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(k_scale=0.0), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(v_scale=float("inf")), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(num_tokens=4, k_rope=None), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(num_tokens=4, v=FAKE + 8), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(num_tokens=4, k_out=FAKE + 4), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(num_tokens=4, k_out_stride_head=196), _ffi.ATTN_ERR_INVALID_ARG),
])
def test_mla_pack_validation_errors(kw, code):
    lib = _lib()
    assert lib.attn_mla_kv_pack_fp8(ctypes.byref(pack_params(**kw)), None) == code


def test_mla_pack_zero_tokens_and_no_rope_are_accepted():
    lib = _lib()
    assert lib.attn_mla_kv_pack_fp8(ctypes.byref(pack_params()), None) == _ffi.ATTN_OK
    assert lib.attn_mla_kv_pack_fp8(ctypes.byref(pack_params(d_rope=0, k_rope=None)), None) == _ffi.ATTN_OK


@pytest.mark.parametrize("kw,code", [
    (dict(), _ffi.ATTN_OK),
    (dict(q_scale=0.0), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(q_scale=float("inf")), _ffi.ATTN_ERR_INVALID_ARG),
    (dict(kv_dtype=_ffi.ATTN_BF16, k_scale=1.0, v_scale=1.0), _ffi.ATTN_ERR_UNSUPPORTED),
])
def test_fp8_query_needs_an_fp8_latent_cache_and_a_scale(kw, code):
    # host-side plan only (no pointers read): the FP8 query path is the MLA
    # shape with an FP8 cache and a finite positive q_scale
    d = dict(num_q_heads=64, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, q_len=4, v_cache=FAKE,
             k_stride_page=64 * 576, k_stride_tok=576, k_stride_head=576, v_stride_page=64 * 576, v_stride_tok=576,
             v_stride_head=576, page_size=64, num_pages=64, max_seq_len=4096, block_table_stride=64,
             kv_dtype=_ffi.ATTN_FP8_E4M3, k_scale=0.5, v_scale=0.5, q_dtype=_ffi.ATTN_FP8_E4M3, q_scale=0.25)
    d.update(kw)
    st, _ = plan(decode_params(**d))
    assert st == code, (st, _lib().attn_last_error())
