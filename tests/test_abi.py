"""C ABI checks that need no GPU: the library loads, exports every function that
include/fp4kv.h declares, and rejects bad arguments on the host (nothing launched)."""
import os
import re

import pytest

from fp4_kv_cache_amd import lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4kv.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from fp4_kv_cache_amd import build
        build.build()
    return L.load()


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("kv_quant_append", "fp4_decode_attention", "fp4_decode_partials", "fp4_decode_merge",
              "fp4_decode_workspace_bytes", "fp4kv_cache_layout", "fp4kv_status_string",
              "fp4kv_stream_read", "fp4kv_cache_read", "fp4kv_cache_read_sink_words"):
        assert n in names, n


def test_every_declared_symbol_is_exported(lib):
    for n in _declared():
        assert hasattr(lib, n), "libfp4kv.so does not export %s" % n
        assert n in L._SIGS, "binding lacks %s" % n


def _desc(**kw):
    d = dict(format=0, attn=0, num_pages=8, page_size=64, num_kv_heads=2, head_dim=128, rope_dim=0,
             max_seqs=4)
    d.update(kw)
    return L.FP4KVCache(d["format"], d["attn"], d["num_pages"], d["page_size"], d["num_kv_heads"],
                        d["head_dim"], d["rope_dim"], d["max_seqs"])


def test_layout_sizes(lib):
    st, b = L.fp4kv_cache_layout(_desc())
    assert st == L.OK
    assert b == [8 * 2 * 64 * 64, 8 * 2 * 64 * 8, 8 * 2 * 128 * 32, 8 * 2 * 128 * 4, 4 * 2 * 16 * 128 * 4, 0]
    st, b = L.fp4kv_cache_layout(_desc(format=1, attn=1, num_kv_heads=1, head_dim=512, rope_dim=64))
    assert st == L.OK
    assert b == [8 * 64 * 256, 8 * 2 * 16, 0, 0, 4 * 32 * 512 * 4, 8 * 64 * 64 * 2]


@pytest.mark.parametrize("kw,code", [
    (dict(format=2), L.ERR_INVALID_ARG),
    (dict(page_size=24), L.ERR_INVALID_ARG),
    (dict(page_size=48), L.ERR_UNSUPPORTED),
    (dict(format=1, page_size=16), L.ERR_INVALID_ARG),
    (dict(head_dim=64), L.ERR_UNSUPPORTED),
    (dict(num_pages=0), L.ERR_INVALID_ARG),
    (dict(attn=1, head_dim=512, rope_dim=64), L.ERR_INVALID_ARG),     # MLA needs one KV head
])
def test_bad_descriptors_rejected(lib, kw, code):
    st, _ = L.fp4kv_cache_layout(_desc(**kw))
    assert st == code


def test_null_pointers_rejected_before_launch(lib):
    c = _desc()                     # scalars valid, all buffers NULL
    assert L.kv_quant_append(c, 1, 1, 0, 4, 1, 1, 1, None, None) == L.ERR_INVALID_ARG
    assert L.fp4_decode_attention(c, 1, 0, 1, 4, 1, 4, 1, 0.1, 1, 1, 1 << 20, None, None) == L.ERR_INVALID_ARG
    assert L.kv_quant_append(None, 1, 1, 0, 4, 1, 1, 1, None, None) == L.ERR_INVALID_ARG


def test_workspace_and_group_checks(lib):
    c = _desc()
    # fake non-null device pointers: validation fails before anything dereferences them
    for f in ("k_codes", "k_scales", "v_codes", "v_scales", "stage", "k_tensor_scale", "v_tensor_scale",
              "k_smooth_inv", "q_smooth"):
        setattr(c, f, 0x1000)
    need = L.fp4_decode_workspace_bytes(c, 3, 8, 1000)
    assert need > 0
    assert L.fp4_decode_attention(c, 1, 0, 3, 8, 1, 16, 1, 0.1, 1, 1, need - 1, None, None) == L.ERR_WORKSPACE
    assert L.fp4_decode_attention(c, 1, 0, 3, 7, 1, 16, 1, 0.1, 1, 1, need, None, None) == L.ERR_INVALID_ARG
    # 32 query heads on 2 KV heads: group 16, beyond the supported 1, 2, 4, 8
    assert L.fp4_decode_attention(c, 1, 0, 3, 32, 1, 16, 1, 0.1, 1, 1, 1 << 30, None, None) == L.ERR_UNSUPPORTED
    assert L.fp4_decode_attention(c, 1, 7, 3, 8, 1, 16, 1, 0.1, 1, 1, need, None, None) == L.ERR_INVALID_ARG
    assert L.kv_quant_append(c, 1, 1, 5, 4, 1, 1, 1, None, None) == L.ERR_INVALID_ARG
    assert L.kv_quant_append(c, 1, None, 0, 4, 1, 1, 1, None, None) == L.ERR_INVALID_ARG
    assert L.kv_quant_append(c, 1, 1, 0, 0, 1, 1, 1, None, None) == L.OK        # empty batch: no-op
    assert L.fp4kv_stream_read(1, 1000, 1, None) == L.ERR_INVALID_ARG
    # same-pattern read helper: sink size from the plan, validation like a decode call
    words = L.fp4kv_cache_read_sink_words(c, 3, 8, 1000)
    assert words > 0 and words % 64 == 0
    assert L.fp4kv_cache_read(c, 3, 8, 1, 16, 1, 1, words - 1, None) == L.ERR_INVALID_ARG
    assert L.fp4kv_cache_read(c, 3, 7, 1, 16, 1, 1, words, None) == L.ERR_INVALID_ARG
    # multi-token decode: q_len 1 is the ordinary workspace; limits on q_len and group * q_len
    assert L.fp4_decode_multi_workspace_bytes(c, 3, 1, 8, 1000) == need
    assert L.fp4_decode_multi_workspace_bytes(c, 3, 2, 8, 1000) > need
    big = 1 << 30
    assert L.fp4_decode_attention_multi(c, 1, 0, 3, 0, 8, 1, 16, 1, 0.1, 1, 1, big, None, None) == L.ERR_INVALID_ARG
    assert L.fp4_decode_attention_multi(c, 1, 0, 3, 9, 2, 1, 16, 1, 0.1, 1, 1, big, None, None) == L.ERR_UNSUPPORTED
    # group 4 x q_len 8 = 32 stacked query rows per KV head: beyond two row sets of 8
    assert L.fp4_decode_attention_multi(c, 1, 0, 3, 8, 8, 1, 16, 1, 0.1, 1, 1, big, None, None) == L.ERR_UNSUPPORTED
    need2 = L.fp4_decode_multi_workspace_bytes(c, 3, 2, 8, 1000)
    assert L.fp4_decode_attention_multi(c, 1, 0, 3, 2, 8, 1, 16, 1, 0.1, 1, 1, need2 - 1, None, None) == L.ERR_WORKSPACE
    assert L.fp4kv_status_string(3) == "workspace too small"


def test_split_plan_sizes(lib):
    c = _desc(num_kv_heads=8)
    # Qwen3-4B shape: 16 x 8 (sequence, KV head) units; at most 2048 waves share the tiles, so
    # the workspace holds 2048 + 128 slots of 4 partial rows (128 + 2 floats) and 128 slot ranges
    assert L.fp4_decode_workspace_bytes(c, 16, 32, 32768) == (2048 + 128) * 4 * 130 * 4 + 128 * 8
    c2 = _desc(num_kv_heads=2)
    assert L.fp4_decode_workspace_bytes(c2, 1, 8, 4096) == (2048 + 2) * 4 * 130 * 4 + 2 * 8
    # MLA: at most 128 shares (256 workgroups of 64 query heads for 128 heads) + 32 sequences,
    # 128 partial rows of 512 + 2 floats each, and 32 slot ranges; then, from the next multiple
    # of 256 bytes, one 768-byte prepared query per (sequence, query head)
    cm = _desc(attn=1, num_kv_heads=1, head_dim=512, rope_dim=64, page_size=64)
    part = (128 + 32) * 128 * 514 * 4 + 32 * 8
    assert part % 256 == 0
    assert L.fp4_decode_workspace_bytes(cm, 32, 128, 16384) == part + 32 * 128 * 768
    part3 = (128 + 3) * 128 * 514 * 4 + 3 * 8
    assert part3 % 256 != 0
    assert L.fp4_decode_workspace_bytes(cm, 3, 128, 16384) == (part3 + 255) // 256 * 256 + 3 * 128 * 768


@pytest.mark.parametrize("attn", [0, 1])
def test_workspace_does_not_depend_on_max_seq_len(lib, attn):
    """The size query covers every block table: a caller passing any bound on the sequence
    lengths -- also one below max_pages_per_seq * page_size, which the decode call plans from
    -- gets a workspace the decode call accepts (its need never exceeds this size)."""
    if attn:
        c = _desc(attn=1, num_kv_heads=1, head_dim=512, rope_dim=64, page_size=64)
        hq = 128
    else:
        c = _desc(num_kv_heads=2, page_size=64)
        hq = 8
    sizes = {L.fp4_decode_workspace_bytes(c, 1, hq, m) for m in (0, 1, 4096, 65 * 64, 1 << 24)}
    assert len(sizes) == 1 and sizes.pop() > 0
    if not attn:
        multi = {L.fp4_decode_multi_workspace_bytes(c, 1, 2, hq, m) for m in (1, 4096, 65 * 64)}
        assert len(multi) == 1
        words = {L.fp4kv_cache_read_sink_words(c, 1, hq, m) for m in (1, 4096, 65 * 64)}
        assert len(words) == 1


@pytest.mark.parametrize("name", ["fp4kv.h", "fp4kv_ablation.h"])
def test_header_is_plain_c(name):
    """The public headers compile as C99 (no C++ or torch types at the boundary)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    hdr = os.path.join(ROOT, "include", name)
    r = subprocess.run([cc, "-fsyntax-only", "-x", "c", "-std=c99", "-Wall", "-Werror", "-I",
                        os.path.join(ROOT, "include"), hdr], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_ablation_switches_agree_and_stay_out_of_the_product(lib):
    """include/fp4kv_ablation.h's switch bits equal the kernels' constants and the binding's; the
    study build exports fp4kv_ablation_set, the product library does not."""
    hdr = open(os.path.join(ROOT, "include", "fp4kv_ablation.h")).read()
    bits = {k: int(v) for k, v in re.findall(r"#define FP4KV_ABL_([A-Z_0-9]+) (\d+)", hdr)}
    internal = open(os.path.join(ROOT, "fp4_kv_cache_amd", "csrc", "fp4kv_internal.h")).read()
    kern = {k: int(v) for k, v in re.findall(r"constexpr int kAbl([A-Za-z]+) = (\d+);", internal)}
    assert bits == {"SINGLE_Q": kern["SingleQ"], "NO_ROTATION": kern["NoRotation"],
                    "NO_SEARCH": kern["NoSearch"], "NORMALIZED_P": kern["VanillaP"]}, (bits, kern)
    assert (L.ABL_SINGLE_Q, L.ABL_NO_ROTATION, L.ABL_NO_SEARCH, L.ABL_NORMALIZED_P) == \
        (bits["SINGLE_Q"], bits["NO_ROTATION"], bits["NO_SEARCH"], bits["NORMALIZED_P"])
    assert not hasattr(lib, "fp4kv_ablation_set")
    if not os.path.exists(L.LIB_ABLATION_PATH):
        pytest.skip("study build not built")
    abl = L.load_ablation()
    assert abl.fp4kv_ablation_set(1 << 8) == L.ERR_INVALID_ARG   # an unknown bit
    assert abl.fp4kv_ablation_set(0) == 0


def test_host_entry_points_from_c(lib, tmp_path):
    """A plain C program (tests/c/abi_host.c) links libfp4kv.so and calls the size queries and
    the host-side validation: the boundary is usable without Python."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    libdir = os.path.dirname(L.LIB_PATH)
    exe = str(tmp_path / "abi_host")
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(root, "include"),
                        os.path.join(root, "tests", "c", "abi_host.c"), "-L", libdir, "-lfp4kv",
                        "-Wl,-rpath," + libdir, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "FAIL" not in r.stdout


def test_noalloc_limit_checked_on_the_host(lib):
    """fp4_decode_attention_noalloc refuses, before touching the device, a batch whose workspace
    would not fit its 64 MiB scratch; the stated limits (GQA ~30,000 units at group 4, MLA 92
    sequences at 128 heads) follow from fp4_decode_workspace_bytes."""
    limit = 64 << 20
    c = _desc(num_kv_heads=8)
    assert L.fp4_decode_workspace_bytes(c, 3700, 32, 4096) <= limit        # 29,600 units
    assert L.fp4_decode_workspace_bytes(c, 3800, 32, 4096) > limit         # 30,400 units
    cm = _desc(attn=1, num_kv_heads=1, head_dim=512, rope_dim=64, page_size=64)
    assert L.fp4_decode_workspace_bytes(cm, 92, 128, 4096) <= limit
    assert L.fp4_decode_workspace_bytes(cm, 93, 128, 4096) > limit
    for f in ("k_codes", "k_scales", "v_codes", "v_scales", "stage", "k_tensor_scale", "v_tensor_scale",
              "k_smooth_inv", "q_smooth"):
        setattr(c, f, 0x1000)
    assert L.fp4_decode_attention_noalloc(c, 1, 0, 3800, 32, 1, 16, 1, 0.1, 1, None, None) == L.ERR_WORKSPACE
    assert L.fp4_decode_attention_noalloc(c, 1, 0, -1, 32, 1, 16, 1, 0.1, 1, None, None) == L.ERR_INVALID_ARG


def test_normalized_p_only_through_the_full_decode(lib):
    """In the study build, normalized P (FP4KV_ABL_NORMALIZED_P) needs both passes of one
    fp4_decode_attention call: the partial-only, merge-only and multi-token entry points refuse
    it on the host, before anything is launched (fake non-null pointers, ample workspace)."""
    if not os.path.exists(L.LIB_ABLATION_PATH):
        pytest.skip("study build not built")
    c = _desc()
    for f in ("k_codes", "k_scales", "v_codes", "v_scales", "stage", "k_tensor_scale", "v_tensor_scale",
              "k_smooth_inv", "q_smooth"):
        setattr(c, f, 0x1000)
    ws = 1 << 30
    with L.ablation(L.ABL_NORMALIZED_P):
        assert L.fp4_decode_partials(c, 1, 0, 3, 8, 1, 16, 1, 0.1, 1, ws, None, None) == L.ERR_UNSUPPORTED
        assert L.fp4_decode_merge(c, 3, 8, 16, 1, 1, 1, ws, None) == L.ERR_UNSUPPORTED
        assert L.fp4_decode_attention_multi(c, 1, 0, 3, 2, 8, 1, 16, 1, 0.1, 1, 1, ws, None, None) == \
            L.ERR_UNSUPPORTED
