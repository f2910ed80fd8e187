"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/rkl.h, sizes its workspace, and rejects bad arguments
with a status and a message before anything is launched."""
import ctypes
import os
import re
import shutil
import subprocess
import threading

import pytest

import lm_head_reverse_amd as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rkl.h")

# A non-null, 16-byte aligned address that is never dereferenced: every call
# below fails its host-side checks before any launch.
FAKE = ctypes.c_void_p(0x10000)
MISALIGNED = ctypes.c_void_p(0x10002)


def declared_functions():
    inc = os.path.dirname(HEADER)
    src = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rkl_[a-z_]+)\s*\(", src)))


def test_header_declares_the_path():
    names = declared_functions()
    for want in ("rkl_compact_rows", "rkl_gather_rows", "rkl_scatter_rows", "rkl_workspace_bytes",
                 "rkl_workspace_bytes_teachers",
                 "rkl_forward_hidden", "rkl_forward_logits", "rkl_backward_hidden", "rkl_backward_logits",
                 "rkl_forward_logprob_entropy", "rkl_backward_logprob_entropy",
                 "rkl_forward_hidden_teachers", "rkl_backward_hidden_teachers",
                 "rkl_forward_hidden_shard", "rkl_forward_logits_shard", "rkl_combine_shards",
                 "rkl_forward_logprob_entropy_shard", "rkl_combine_shards_logprob_entropy",
                 "rkl_last_error", "rkl_version"):
        assert want in names


def test_library_exports_every_declared_symbol():
    L = R.lib()
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing
    assert "gfx950" in R.version()


def test_library_exports_nothing_else():
    """Only the C ABI is visible: the library is built with hidden visibility."""
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", R.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = sorted(line.split()[-1] for line in out.splitlines() if line.split()[1:2] == ["T"])
    assert exported == declared_functions()


def test_workspace_sizes():
    # both sides as logits: row kernels need no workspace
    assert R.workspace_bytes(64, 1024, 0, 0) == 0
    a = R.workspace_bytes(2048, 151936, 2048, 2048)
    b = R.workspace_bytes(4096, 151936, 2048, 2048)
    assert 0 < a < b
    # no fp32 [N, V] logits (4096 x 151936 x 4 B = 2.49 GB) are ever held; the
    # backward keeps an fp16 dz chunk of whole 65536-column segments within
    # 2 GiB (the whole vocabulary at N = 4096), an fp16 copy of that chunk of
    # W_s and the scaled fp16 copy of h_s
    assert b < 4096 * 151936 * 4
    assert b <= 4096 * 151936 * 2 + 152064 * 2048 * 2 + 2048 * 4096 * 2 + (1 << 20)
    # N = 8192: two segments (2 GiB of dz); N = 32768: one segment
    assert R.workspace_bytes(8192, 151936, 2048, 2048) <= 8192 * 131072 * 2 + 131072 * 2048 * 2 + 2048 * 8192 * 2 + (1 << 20)
    assert R.workspace_bytes(32768, 151936, 2048, 2048) <= 32768 * 65536 * 2 + 65536 * 2048 * 2 + 2048 * 32768 * 2 + (1 << 20)
    assert R.workspace_bytes(4096, 151936, 2048, 2048) == R.workspace_bytes(4096, 151936, 2048, 4096)
    assert R.workspace_bytes(-1, 10, 64, 64) == 0
    # per-row teachers: the regular workspace plus the rows regrouped by
    # teacher (h_s and h_t bf16, dh fp32, ids, mask and per-row scalars)
    for N, Hs, Ht in ((4096, 2048, 2048), (300, 128, 192), (0, 64, 64)):
        extra = R.workspace_bytes_teachers(N, 151936, Hs, Ht) - R.workspace_bytes(N, 151936, Hs, Ht)
        assert N * (6 * Hs + 2 * Ht + 29) <= extra <= N * (6 * Hs + 2 * Ht + 29) + 8 * 256
    assert R.workspace_bytes_teachers(-1, 10, 64, 64) == 0


def _fwd_hidden(N=4, V=100, Hs=64, Ht=64, p=FAKE, ws=FAKE, nbytes=1 << 30):
    return R.lib().rkl_forward_hidden(N, V, Hs, Ht, p, p, p, p, None, p, p, ws, nbytes, None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(N=-1), 1, "N="),
    (dict(V=0), 1, "V="),
    (dict(Hs=100), 2, "multiple of 64"),
    (dict(Ht=96), 2, "multiple of 64"),
    (dict(Hs=0), 1, "Hs="),
    (dict(p=None), 1, "NULL"),
    (dict(p=MISALIGNED), 1, "aligned"),
    (dict(nbytes=0), 3, "workspace"),
])
def test_forward_hidden_rejects(kw, code, msg):
    assert _fwd_hidden(**kw) == code
    assert msg in R.lib().rkl_last_error().decode()


def test_forward_logits_rejects():
    L = R.lib()
    # student given both ways
    assert L.rkl_forward_logits(4, 100, 64, FAKE, FAKE, FAKE, FAKE, None, 0, None, FAKE, FAKE, FAKE, 1 << 20, None) == 1
    # student as logits but Hs != 0
    assert L.rkl_forward_logits(4, 100, 64, None, None, FAKE, FAKE, None, 0, None, FAKE, FAKE, None, 0, None) == 1
    # teacher logits missing
    assert L.rkl_forward_logits(4, 100, 0, None, None, FAKE, None, None, 0, None, FAKE, FAKE, None, 0, None) == 1
    assert "z_t" in L.rkl_last_error().decode()
    # a row index with no row count, or a misaligned one
    assert L.rkl_forward_logits(4, 100, 0, None, None, FAKE, FAKE, FAKE, 0, None, FAKE, FAKE, None, 0, None) == 1
    assert "T=" in L.rkl_last_error().decode()
    assert L.rkl_forward_logits(4, 100, 0, None, None, FAKE, FAKE, MISALIGNED, 8, None, FAKE, FAKE, None, 0,
                                None) == 1
    assert "z_rows" in L.rkl_last_error().decode()


def test_backward_rejects():
    L = R.lib()
    # student as logits: dh/dW must be NULL
    assert L.rkl_backward_logits(4, 100, 0, None, None, FAKE, FAKE, None, 0, None, None, FAKE, FAKE, FAKE, 0, FAKE,
                                 None, 0, None) == 1
    # student hidden: dz must be NULL
    assert L.rkl_backward_logits(4, 100, 64, FAKE, FAKE, None, FAKE, None, 0, None, None, FAKE, FAKE, FAKE, 0, FAKE,
                                 FAKE, 1 << 30, None) == 1
    # workspace too small
    assert L.rkl_backward_hidden(4, 100, 64, 64, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, 0,
                                 FAKE, 16, None) == 3
    # dW missing
    assert L.rkl_backward_hidden(4, 100, 64, 64, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, None, 0,
                                 FAKE, 1 << 30, None) == 1
    # more rows than the backward's per-call limit (2^22): unsupported, nothing launched
    assert L.rkl_backward_hidden((1 << 22) + 1, 100, 64, 64, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE,
                                 0, FAKE, 1 << 62, None) == 2
    assert "2^22" in L.rkl_last_error().decode()


def test_logprob_entropy_rejects():
    L = R.lib()
    fwd = L.rkl_forward_logprob_entropy
    # sampled tokens missing
    assert fwd(4, 100, 64, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert "y" in L.rkl_last_error().decode()
    # entropy output missing
    assert fwd(4, 100, 64, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, 1 << 30, None) == 1
    # width not a multiple of 64
    assert fwd(4, 100, 96, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == 2
    # workspace too small
    assert fwd(4, 100, 64, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 16, None) == 3
    bwd = L.rkl_backward_logprob_entropy
    # dW missing
    assert bwd(4, 100, 64, FAKE, FAKE, FAKE, None, None, None, FAKE, FAKE, None, 0, FAKE, 1 << 30, None) == 1
    # misaligned upstream gradient
    assert bwd(4, 100, 64, FAKE, FAKE, FAKE, None, MISALIGNED, None, FAKE, FAKE, FAKE, 0, FAKE, 1 << 30, None) == 1
    assert "grad_logp" in L.rkl_last_error().decode()
    # more rows than the backward's per-call limit
    assert bwd((1 << 22) + 1, 100, 64, FAKE, FAKE, FAKE, None, None, None, FAKE, FAKE, FAKE, 0, FAKE, 1 << 62,
               None) == 2


def test_hidden_teachers_rejects():
    L = R.lib()
    fwd = L.rkl_forward_hidden_teachers
    # K out of range
    assert fwd(4, 100, 64, 64, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert fwd(4, 100, 64, 64, 32, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert "K=" in L.rkl_last_error().decode()
    # teacher ids missing
    assert fwd(4, 100, 64, 64, 2, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert "teacher" in L.rkl_last_error().decode()
    # workspace too small: the regular size lacks the regrouped rows
    assert fwd(4, 100, 64, 64, 2, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 16, None) == 3
    assert fwd(4, 100, 64, 64, 2, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE,
               R.workspace_bytes(4, 100, 64, 64), None) == 3
    assert "workspace" in L.rkl_last_error().decode()
    bwd = L.rkl_backward_hidden_teachers
    assert bwd(4, 100, 64, 64, 2, FAKE, FAKE, FAKE, FAKE, MISALIGNED, None, None, FAKE, FAKE, FAKE, 0, FAKE,
               1 << 30, None) == 1
    assert bwd((1 << 22) + 1, 100, 64, 64, 2, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, 0, FAKE,
               1 << 62, None) == 2
    assert bwd(4, 100, 64, 64, 2, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, 0, FAKE,
               R.workspace_bytes(4, 100, 64, 64), None) == 3


def test_vocab_shard_rejects():
    L = R.lib()
    fwd = L.rkl_forward_hidden_shard
    assert fwd(4, 100, 100, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == 2      # Hs % 64
    assert fwd(4, 100, 64, 64, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None) == 1        # partial NULL
    assert "partial" in L.rkl_last_error().decode()
    assert fwd(4, 100, 64, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None) == 3             # workspace
    lg = L.rkl_forward_logits_shard
    assert lg(4, 100, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == 1          # both student forms
    assert lg(4, 100, 0, None, None, FAKE, None, FAKE, None, 0, None) == 1                 # z_t NULL
    assert lg(4, 100, 0, None, None, FAKE, FAKE, None, None, 0, None) == 1                 # partial NULL
    comb = L.rkl_combine_shards
    assert comb(0, 4, FAKE, None, FAKE, FAKE, None) == 1
    assert "G=" in L.rkl_last_error().decode()
    assert comb(2, -1, FAKE, None, FAKE, FAKE, None) == 1
    assert comb(2, 4, None, None, FAKE, FAKE, None) == 1
    assert comb(2, 4, MISALIGNED, None, FAKE, FAKE, None) == 1
    assert comb(2, 0, None, None, None, None, None) == 0                                     # nothing to do
    lf = L.rkl_forward_logprob_entropy_shard
    assert lf(4, 100, 64, FAKE, FAKE, None, FAKE, FAKE, 1 << 30, None) == 1                  # y NULL
    assert lf(4, 100, 64, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None) == 1                  # partial NULL
    assert lf(4, 100, 96, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == 2                  # H % 64
    lc = L.rkl_combine_shards_logprob_entropy
    assert lc(0, 4, FAKE, None, FAKE, FAKE, FAKE, None) == 1
    assert lc(2, 4, FAKE, None, FAKE, None, FAKE, None) == 1                                 # entropy NULL
    assert "entropy" in L.rkl_last_error().decode()


def test_compaction_and_copies_reject():
    L = R.lib()
    assert L.rkl_compact_rows(FAKE, -1, FAKE, FAKE, None, None) == 1
    assert L.rkl_compact_rows(None, 10, FAKE, FAKE, None, None) == 1
    assert L.rkl_compact_rows(FAKE, 10, FAKE, None, None, None) == 1
    assert L.rkl_gather_rows(FAKE, 5, 16, FAKE, 6, FAKE, None) == 1       # N > T
    assert L.rkl_gather_rows(FAKE, 5, 6, FAKE, 2, FAKE, None) == 1        # row_bytes % 4
    assert L.rkl_gather_rows(MISALIGNED, 5, 16, FAKE, 2, FAKE, None) == 1
    assert L.rkl_scatter_rows(FAKE, 3, 8, FAKE, 2, FAKE, None) == 1       # N > T
    assert L.rkl_scatter_rows(FAKE, 1, 8, None, 2, FAKE, None) == 1       # row_idx NULL


def test_last_error_is_per_thread():
    _fwd_hidden(N=-1)
    main_msg = R.lib().rkl_last_error().decode()
    seen = {}

    def other():
        _fwd_hidden(Hs=100)
        seen["msg"] = R.lib().rkl_last_error().decode()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert "multiple of 64" in seen["msg"]
    assert R.lib().rkl_last_error().decode() == main_msg


def test_kernel_times_without_launches():
    # timing on, nothing launched (rejected calls launch nothing): no entries,
    # and nothing that needs a device is touched
    L = R.lib()
    assert L.rkl_kernel_timing(1) == 0
    try:
        assert L.rkl_scatter_rows(FAKE, 3, 8, FAKE, 2, FAKE, None) == 1
        assert R.kernel_times() == {}
        count = ctypes.c_int(-1)
        assert L.rkl_kernel_times(0, None, None, None, ctypes.byref(count)) == 0 and count.value == 0
        assert L.rkl_kernel_times(-1, None, None, None, ctypes.byref(count)) == 1
    finally:
        assert L.rkl_kernel_timing(0) == 0
