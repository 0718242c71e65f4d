"""Host-only checks of the C ABI: the library loads, exports every function
include/lightning_attn.h declares, and rejects bad arguments with the
documented status codes before launching anything (no GPU needed: every
call here returns during validation)."""
import ctypes
import os
import re

import pytest

import linear_attention_lightning_amd as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lightning_attn.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FP32, BF16 = 0, 1
DUMMY = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lightning_attn_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return la.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert "lightning_attn_fwd" in names and "lightning_attn_decode" in names
    for n in names:
        assert hasattr(lib, n), n


def test_exports_only_declared_symbols():
    """The library's dynamic symbol table holds the declared entry points and
    nothing else of its own (internal helpers keep internal linkage)."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    res = subprocess.run([nm, "-D", "--defined-only", la.LIB_PATH], capture_output=True,
                         text=True, check=True)
    syms = {ln.split()[-1] for ln in res.stdout.splitlines() if ln.strip()}
    ours = {n for n in syms if not n.startswith("_Z") and not n.startswith("__hip_cuid")}
    assert ours == set(declared_functions()), sorted(ours ^ set(declared_functions()))


def test_noalloc_scratch_size(lib):
    """The allocation-free prefill's per-GPU scratch array: 256 MiB, enough
    for the plans of the 64-head 32768-token, packed 65536-token and
    1M-token 8-head workloads."""
    assert lib.lightning_attn_noalloc_scratch_bytes() == 256 << 20
    for B, H, N in ((1, 64, 32768), (1, 8, 1 << 20)):
        assert (lib.lightning_attn_fwd_workspace_size(B, H, N, 128, 128, BF16, 0)
                <= lib.lightning_attn_noalloc_scratch_bytes())
    assert (lib.lightning_attn_fwd_varlen_workspace_size(25, 64, 65536, 128, 128, BF16, 0)
            <= lib.lightning_attn_noalloc_scratch_bytes())


def test_status_strings_and_version(lib):
    for s in range(5):
        assert lib.lightning_attn_status_string(s)
    assert lib.lightning_attn_status_string(99) == b"unknown status"
    assert lib.lightning_attn_version() >= 100


def fwd(lib, **kw):
    a = dict(q=DUMMY, k=DUMMY, v=DUMMY, decay=DUMMY, B=1, H=2, N=256, d=128, block=128, dt=BF16,
             init=None, out=DUMMY, fin=DUMMY, seg=0, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.lightning_attn_fwd(a["q"], a["k"], a["v"], a["decay"], a["B"], a["H"], a["N"],
                                  a["d"], a["block"], a["dt"], a["init"], a["out"], a["fin"],
                                  a["seg"], a["ws"], a["wsb"], a["stream"])


def test_fwd_rejects_bad_arguments(lib):
    assert fwd(lib, d=96) == UNSUPPORTED
    assert fwd(lib, d=256) == UNSUPPORTED
    assert fwd(lib, block=48) == UNSUPPORTED
    assert fwd(lib, block=-1) == UNSUPPORTED
    assert fwd(lib, block=512) == UNSUPPORTED
    assert fwd(lib, dt=7) == UNSUPPORTED
    assert fwd(lib, B=-1) == INVALID
    assert fwd(lib, N=-5) == INVALID
    assert fwd(lib, H=-2) == INVALID
    assert fwd(lib, seg=-2) == INVALID  # -1 is LA_SEGMENT_PER_SEQUENCE
    assert fwd(lib, q=None) == INVALID
    assert fwd(lib, out=None) == INVALID
    assert fwd(lib, decay=None) == INVALID
    # B*H == 0 and N == 0 without a state to write are no-ops
    assert fwd(lib, B=0) == OK
    assert fwd(lib, H=0, decay=None) == OK
    assert fwd(lib, N=0, q=None, k=None, v=None, out=None, fin=None) == OK


def test_fwd_workspace_checks(lib):
    # a long single sequence on few heads is cut into segments: needs workspace
    need = lib.lightning_attn_fwd_workspace_size(1, 8, 1 << 20, 128, 256, BF16, 0)
    assert need > 0 and need % (128 * 128 * 4) == 0
    assert fwd(lib, H=8, N=1 << 20, block=256, ws=None, wsb=0) == WORKSPACE
    assert fwd(lib, H=8, N=1 << 20, block=256, ws=DUMMY, wsb=need - 1) == WORKSPACE
    # one segment per sequence needs none
    assert lib.lightning_attn_fwd_workspace_size(1, 8, 1 << 20, 128, 256, BF16, -1) == 0
    assert lib.lightning_attn_fwd_varlen_workspace_size(9, 64, 65536, 128, 128, BF16, -1) == 0
    assert lib.lightning_attn_fwd_varlen_workspace_size(9, 64, 65536, 128, 128, BF16, -2) == 0
    assert lib.lightning_attn_fwd_workspace_size(4, 64, 4096, 128, 128, BF16, 4096) == 0
    # explicit segment lengths
    n = lib.lightning_attn_fwd_workspace_size(1, 2, 1000, 64, 64, FP32, 256)
    assert n == 4 * 2 * 64 * 64 * 4
    assert lib.lightning_attn_fwd_workspace_size(1, 2, 1000, 96, 64, FP32, 256) == 0


def test_block_auto_resolves_by_mean_length(lib):
    """LA_BLOCK_AUTO (0) takes the level the mean input length falls in
    (MiniMax-01 report, section 3.3.3, multi-level padding to 32/64/128/256):
    the workspace size query, which runs the same plan as the call, must give
    the chosen level's figure, and the levels must differ here for that to
    say anything."""
    fs, vs = lib.lightning_attn_fwd_workspace_size, lib.lightning_attn_fwd_varlen_workspace_size
    # fixed length: B=1, H=4, N = mean
    for N, level in ((20, 32), (32, 32), (33, 64), (64, 64), (65, 128), (3000, 128)):
        assert fs(1, 4, N, 128, 0, BF16, 0) == fs(1, 4, N, 128, level, BF16, 0), N
    assert fs(1, 4, 3000, 128, 32, BF16, 0) != fs(1, 4, 3000, 128, 128, BF16, 0)
    # packed: mean = ceil(total / num_seqs)
    for S, total, level in ((20, 118, 32), (20, 640, 32), (20, 641, 64), (20, 1280, 64),
                            (20, 1281, 128), (20, 2000, 128), (20, 4114, 128)):
        assert vs(S, 64, total, 128, 0, BF16, 0) == vs(S, 64, total, 128, level, BF16, 0), total
    assert vs(20, 64, 2000, 128, 32, BF16, 0) != vs(20, 64, 2000, 128, 128, BF16, 0)
    # float32 has one kernel for every level: auto is accepted there too
    assert fs(1, 2, 1000, 64, 0, FP32, 256) == fs(1, 2, 1000, 64, 64, FP32, 256)
    # entry points whose chunk does not follow the block (backward, training pair,
    # channel-wise) accept the automatic level and plan as at block 128
    for q in (lib.lightning_attn_bwd_workspace_size, lib.lightning_attn_saved_states_size,
              lib.lightning_attn_fwd_chdecay_workspace_size):
        assert q(1, 64, 32768, 128, 0, BF16, 0) == q(1, 64, 32768, 128, 128, BF16, 0) > 0
    assert fwd(lib, block=0, ws=None, wsb=0) in (OK, WORKSPACE)


def test_launch_size_limits(lib):
    # A plan with more (segment, head) pairs than one launch can hold
    # (2^23 - 1 workgroups of 512 threads) is refused before anything runs;
    # one segment per token of a 2^20-token sequence on 8 or 64 heads is over.
    assert fwd(lib, H=8, N=1 << 20, seg=1, ws=DUMMY, wsb=1 << 62) == UNSUPPORTED
    assert fwd(lib, H=64, N=1 << 17, seg=1, ws=DUMMY, wsb=1 << 62) == UNSUPPORTED
    # just below the limit the plan passes (and then wants its workspace)
    assert fwd(lib, H=8, N=(1 << 20) - 8, seg=1, ws=None, wsb=0) == WORKSPACE
    assert fwd(lib, B=1 << 21, N=1 << 20) == UNSUPPORTED  # 2^41 tokens
    # the packed form: one segment per sequence, 2^17 sequences x 64 heads
    cu = DUMMY
    assert lib.lightning_attn_fwd_varlen(DUMMY, DUMMY, DUMMY, DUMMY, cu, 1 << 17, 64, 1 << 17,
                                         128, 128, BF16, None, DUMMY, DUMMY, -1, None, 0,
                                         None) == UNSUPPORTED
    # the backward shares the plan check
    assert lib.lightning_attn_bwd(DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, None, None, DUMMY, DUMMY,
                                  DUMMY, DUMMY, 1, 64, 1 << 17, 128, 128, BF16, 0, 1, DUMMY,
                                  1 << 62, None) == UNSUPPORTED
    # decode: one 256-thread workgroup per (sequence, head), at most 2^24 - 1
    assert lib.lightning_attn_decode(DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, 1 << 18, 64, 128,
                                     BF16, None) == UNSUPPORTED


def test_varlen_rejects_bad_arguments(lib):
    f = lib.lightning_attn_fwd_varlen
    args = [DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, 3, 4, 1000, 128, 128, BF16, None, DUMMY, DUMMY, 0,
            None, 0, None]

    def call(**kw):
        a = list(args)
        names = ["q", "k", "v", "decay", "cu", "S", "H", "total", "d", "block", "dt", "init",
                 "out", "fin", "seg", "ws", "wsb", "stream"]
        for key, val in kw.items():
            a[names.index(key)] = val
        return f(*a)

    assert call(cu=None) == INVALID
    assert call(S=-1) == INVALID
    assert call(total=-1) == INVALID
    assert call(d=32) == UNSUPPORTED
    assert call(block=100) == UNSUPPORTED
    assert call() == WORKSPACE
    assert call(S=0) == INVALID  # tokens but no sequences
    assert call(S=0, total=0) == OK
    need = lib.lightning_attn_fwd_varlen_workspace_size(3, 4, 1000, 128, 128, BF16, 0)
    assert need > 0


def test_varlen_snapshots_rejects_bad_arguments(lib):
    f = lib.lightning_attn_fwd_varlen_snapshots
    names = ["q", "k", "v", "decay", "cu", "S", "H", "total", "d", "block", "dt", "layout",
             "init", "out", "fin", "iv", "offs", "snaps", "seg", "ws", "wsb", "stream"]
    args = [DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, 3, 4, 1000, 128, 128, BF16, 0, None, DUMMY, DUMMY,
            128, DUMMY, DUMMY, 0, None, 0, None]

    def call(**kw):
        a = list(args)
        for key, val in kw.items():
            a[names.index(key)] = val
        return f(*a)

    assert call(iv=0) == INVALID
    assert call(iv=-5) == INVALID
    assert call(snaps=None) == INVALID
    assert call(offs=None) == INVALID
    # an interval beyond every sequence stores nothing: buffers may be NULL
    # (then only the workspace is missing here)
    assert call(iv=1001, snaps=None, offs=None) == WORKSPACE
    assert call(layout=2) == UNSUPPORTED
    assert call(d=32) == UNSUPPORTED
    assert call() == WORKSPACE
    assert call(S=0, total=0) == OK


def test_mixed_step_rejects_bad_arguments(lib):
    """Either part's invalid argument fails the call before anything is
    launched (the stream handles here are never used)."""
    f = lib.lightning_attn_mixed_step
    names = ["pq", "pk", "pv", "cu", "S", "total", "layout", "init", "pout", "fin", "seg", "ws",
             "wsb", "pstream", "dq", "dk", "dv", "dstate", "dout", "B", "dstream", "decay", "H",
             "d", "block", "dt"]
    args = [DUMMY, DUMMY, DUMMY, DUMMY, 2, 100, 0, None, DUMMY, DUMMY, 0, DUMMY, 1 << 30, None,
            DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, 18, None, DUMMY, 8, 128, 128, BF16]

    def call(**kw):
        a = list(args)
        for key, val in kw.items():
            a[names.index(key)] = val
        return f(*a)

    assert call(B=-1) == INVALID          # decode part invalid: prefill not launched
    assert call(dstate=None) == INVALID
    assert call(S=-1) == INVALID          # prefill part invalid: decode not launched
    assert call(cu=None) == INVALID
    assert call(ws=None, wsb=0) == WORKSPACE
    assert call(d=96) == UNSUPPORTED
    assert call(layout=5) == UNSUPPORTED
    assert call(decay=None) == INVALID
    assert call(S=0, total=0, B=0) == OK  # both parts empty


def test_bwd_rejects_bad_arguments(lib):
    f = lib.lightning_attn_bwd
    names = ["q", "k", "v", "decay", "dout", "dfin", "init", "dq", "dk", "dv", "dinit", "B", "H",
             "N", "d", "block", "dt", "layout", "seg", "ws", "wsb", "stream"]
    args = [DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, None, None, DUMMY, DUMMY, DUMMY, DUMMY, 1, 2, 256,
            128, 128, BF16, 0, 0, None, 0, None]

    def call(**kw):
        a = list(args)
        for key, val in kw.items():
            a[names.index(key)] = val
        return f(*a)

    assert call(d=96) == UNSUPPORTED
    assert call(layout=3) == UNSUPPORTED
    assert call(B=-1) == INVALID
    assert call(seg=-3) == INVALID
    assert call(dout=None) == INVALID
    assert call(dk=None) == INVALID
    assert call(decay=None) == INVALID
    assert call() == WORKSPACE
    need = lib.lightning_attn_bwd_workspace_size(1, 2, 256, 128, 128, BF16, 0)
    assert need >= 4 * 2 * 128 * 128 * 4
    assert call(ws=DUMMY, wsb=need - 1) == WORKSPACE
    assert call(B=0) == OK
    assert call(H=0, decay=None) == OK


def test_training_pair_sizes_and_rejections(lib):
    """Saved-state sizes follow the backward's segment plan; a missing or
    short `saved` is rejected before anything launches."""
    size = lib.lightning_attn_saved_states_size
    assert size(1, 2, 128, 128, 128, BF16, 0) == 0            # one chunk: nothing kept
    assert size(1, 2, 256, 128, 128, BF16, 0) == 2 * 2 * 128 * 128 * 4  # automatic: 2 segments
    assert size(1, 2, 256, 128, 128, BF16, -1) == 0           # one segment per sequence
    assert size(1, 2, 1024, 128, 128, BF16, 256) == 4 * 2 * 128 * 128 * 4
    assert size(1, 64, 32768, 128, 128, BF16, 0) == 4 * 64 * 128 * 128 * 4  # 4 segments
    assert size(1, 2, 256, 96, 128, BF16, 0) == 0             # unsupported d
    need = size(1, 2, 1024, 128, 128, BF16, 256)
    ws = lib.lightning_attn_bwd_workspace_size(1, 2, 1024, 128, 128, BF16, 256)
    fwd = lib.lightning_attn_fwd_save
    base = [DUMMY, DUMMY, DUMMY, DUMMY, 1, 2, 1024, 128, 128, BF16, 0, None, DUMMY, DUMMY, 256,
            DUMMY, need, DUMMY, ws, None]
    a = list(base); a[15] = None
    assert fwd(*a) == INVALID
    a = list(base); a[16] = need - 1
    assert fwd(*a) == INVALID
    a = list(base); a[17] = None
    assert fwd(*a) == WORKSPACE
    a = list(base); a[7] = 96
    assert fwd(*a) == UNSUPPORTED
    bwd = lib.lightning_attn_bwd_saved
    bbase = [DUMMY] * 5 + [None, None] + [DUMMY] * 4 + [1, 2, 1024, 128, 128, BF16, 0, 256,
                                                         DUMMY, need, DUMMY, ws, None]
    a = list(bbase); a[19] = None
    assert bwd(*a) == INVALID
    a = list(bbase); a[20] = need - 1
    assert bwd(*a) == INVALID
    a = list(bbase); a[21] = None
    assert bwd(*a) == WORKSPACE


def test_misaligned_pointers_are_rejected(lib):
    """Every tensor pointer must be 16-byte aligned; a misaligned one fails
    validation (nothing is launched: the pointers are never dereferenced)."""
    odd = ctypes.c_void_p(0x1002)
    assert fwd(lib, q=odd) == INVALID
    assert fwd(lib, out=odd) == INVALID
    assert fwd(lib, fin=odd) == INVALID
    need = lib.lightning_attn_fwd_workspace_size(1, 2, 256, 128, 128, BF16, 0)
    assert fwd(lib, ws=odd, wsb=need) == INVALID
    base = [DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, 2, 4, 128, BF16, None]
    a = list(base); a[4] = odd                      # decode state
    assert lib.lightning_attn_decode(*a) == INVALID
    bwd = lib.lightning_attn_bwd
    args = [DUMMY, DUMMY, DUMMY, DUMMY, odd, None, None, DUMMY, DUMMY, DUMMY, DUMMY, 1, 2, 256,
            128, 128, BF16, 0, 0, DUMMY, 1 << 30, None]
    assert bwd(*args) == INVALID                    # dout


def test_decode_rejects_bad_arguments(lib):
    f = lib.lightning_attn_decode
    base = [DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, 2, 4, 128, BF16, None]
    for idx in range(6):
        a = list(base)
        a[idx] = None
        assert f(*a) == INVALID
    a = list(base); a[8] = 80
    assert f(*a) == UNSUPPORTED
    a = list(base); a[9] = 3
    assert f(*a) == UNSUPPORTED
    a = list(base); a[6] = -1
    assert f(*a) == INVALID
    a = list(base); a[6] = 0
    assert f(*a) == OK


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        la.load_library(str(tmp_path / "missing.so"))


def test_header_is_c99_and_a_c_caller_links(tmp_path):
    """The public header compiles as strict C99, and a plain C program
    (tests/c_abi_check.c) links against the library and gets the documented
    results from the calls that need no GPU."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    subprocess.run([gcc, "-x", "c", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-fsyntax-only", HEADER], check=True)
    exe = str(tmp_path / "c_abi_check")
    libdir = os.path.dirname(la.LIB_PATH)
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I",
                    os.path.join(ROOT, "include"), "-o", exe,
                    os.path.join(ROOT, "tests", "c_abi_check.c"), "-L", libdir,
                    "-l:" + os.path.basename(la.LIB_PATH), "-Wl,-rpath," + libdir], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failure(s)" in r.stdout
