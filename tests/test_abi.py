"""The C-ABI library: it loads, exports every entry point include/*.h
declares, and validates arguments on the host (no GPU needed: an invalid call
returns its status before anything is enqueued)."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))
SEG_WAVES = 4  # segments per chunk (each shared by two of the select pass's waves)


def stream_tiles(d):
    """16-row tiles per wave iteration of the streaming select plan."""
    return 1


def declared_functions():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(saga_\w+)\s*\(", src))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    from sparse_asymmetric_head_amd import saga

    if not os.path.exists(saga.LIB_PATH):
        from sparse_asymmetric_head_amd import build

        build.build()
    return saga.lib()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("saga_decode_step", "saga_refresh_threshold", "saga_dense_gqa_baseline",
              "saga_workspace_bytes", "saga_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    from sparse_asymmetric_head_amd import saga

    names = declared_functions()
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/*.h but not exported"
    assert set(names) == set(saga.EXPORTS)


def test_status_strings(L):
    from sparse_asymmetric_head_amd import saga

    assert saga.status_string(0) == "SAGA_OK"
    assert saga.status_string(-1) == "SAGA_ERR_INVALID_ARG"
    assert saga.status_string(-3) == "SAGA_ERR_WORKSPACE"
    assert saga.status_string(12345) == "SAGA_ERR_UNKNOWN"
    assert L.saga_version() >= 100


SHAPES = [
    (1, 4, 1, 2, 64, 1024, 64),
    (1, 32, 4, 16, 64, 32768, 256),
    (1, 32, 4, 16, 64, 131072, 512),
    (4, 12, 1, 4, 128, 131072, 512),
    (16, 32, 2, 32, 128, 65536, 1024),
    (2, 6, 4, 5, 64, 1000, 7),      # non-integer group ratio, ragged length
    (1, 64, 1, 8, 128, 333, 333),   # 64 query heads per key head, N = l_kv
]


@pytest.mark.parametrize("shape", SHAPES)
def test_cache_workspace_covers_every_length(L, shape):
    """One cache workspace serves every length up to the capacity: no
    length's own layout needs more (checked on a grid of lengths)."""
    B, h_q, h_k, h_v, d, l_kv, N = shape
    cap = l_kv
    have = L.saga_cache_workspace_bytes(B, h_q, h_k, h_v, d, cap, N)
    assert have > 0
    for ln in sorted(set([N, cap] + [max(N, cap * i // 37) for i in range(1, 37)])):
        assert L.saga_workspace_bytes(B, h_q, h_k, h_v, d, ln, N) <= have, ln


@pytest.mark.parametrize("shape", SHAPES)
def test_workspace_layout_consistent(L, shape):
    from sparse_asymmetric_head_amd import saga

    B, h_q, h_k, h_v, d, l_kv, N = shape
    nbytes = saga.saga_workspace_bytes(*shape)
    assert nbytes > 0 and nbytes % 256 == 0
    lay = saga.saga_workspace_layout(*shape)
    assert lay.bytes == nbytes
    assert lay.n_chunk * lay.chunk_len >= l_kv > (lay.n_chunk - 1) * lay.chunk_len
    assert lay.n_seg == SEG_WAVES * lay.n_chunk and lay.seg_cap * SEG_WAVES == lay.chunk_len
    # record groups of 16-row tiles: one tile on the short plan (at most 128 rows per block),
    # else the streaming tile count (also one)
    per = -(-(B * h_k * l_kv) // 256)
    u = 1 if per <= 128 else stream_tiles(d)
    assert lay.seg_group == 16 * u
    assert lay.chunk_len % (SEG_WAVES * lay.seg_group) == 0
    assert lay.n_seg <= 1024
    assert lay.scores_ld >= l_kv and lay.scores_ld % 4 == 0
    assert lay.seg_words % 16 == 0 and lay.seg_words >= 2 + 2 * lay.seg_cap
    rows = B * h_q
    regions = sorted([
        (lay.seg_off, rows * lay.n_seg * lay.seg_words * 4),
        (lay.scores_off, rows * lay.scores_ld * 4),
    ])
    for (o1, n1), (o2, _) in zip(regions, regions[1:]):
        assert o1 % 256 == 0 and o1 + n1 <= o2
    assert regions[-1][0] + regions[-1][1] <= nbytes
    # h_v does not change the layout (the refresh call uses h_v = h_k)
    assert saga.saga_workspace_bytes(B, h_q, h_k, h_k, d, l_kv, N) == nbytes


def test_invalid_shapes_rejected(L):
    f = L.saga_workspace_bytes
    assert f(1, 4, 1, 2, 64, 1024, 64) > 0
    assert f(0, 4, 1, 2, 64, 1024, 64) == 0       # B < 1
    assert f(1, 4, 3, 2, 64, 1024, 64) == 0       # h_k > h_v
    assert f(1, 4, 1, 8, 64, 1024, 64) == 0       # h_v > h_q
    assert f(1, 4, 1, 2, 96, 1024, 64) == 0       # d unsupported
    assert f(1, 4, 1, 2, 64, 1024, 0) == 0        # N < 1
    assert f(1, 4, 1, 2, 64, 1024, 1025) == 0     # N > l_kv
    assert f(1, 130, 2, 2, 64, 1024, 64) == 0     # group of 65 query heads
    assert f(1, 4, 1, 2, 128, 1 << 23, 64) == 0   # cache rows beyond 2^31 bytes
    assert f(1, 32768, 512, 512, 64, 1024, 64) > 0       # the largest head count
    assert f(1, 32769, 513, 513, 64, 1024, 64) == 0      # head products past 32-bit range
    assert L.saga_dense_workspace_bytes(1, 32769, 4096, 64, 1024) == 0
    assert L.saga_dense_workspace_bytes(1, 32, 8, 64, 4096) > 0
    assert L.saga_dense_workspace_bytes(1, 32, 1, 64, 4096) == 0  # group of 32 > 16
    fw = L.saga_full_attention_workspace_bytes
    assert fw(1, 32, 4, 16, 64, 4096) > 0
    assert fw(1, 32, 2, 32, 128, 4096) > 0       # sixteen value heads per key head
    assert fw(1, 32, 8, 4, 64, 4096) == 0        # h_k > h_v
    assert fw(1, 64, 1, 1, 64, 4096) == 0        # 64 query heads in one block
    assert fw(1, 32, 4, 16, 96, 4096) == 0       # d unsupported


def test_entry_points_validate_before_launch(L):
    """All of these are rejected on the host, so they run without a GPU."""
    from sparse_asymmetric_head_amd import saga

    B, h_q, h_k, h_v, d, l_kv, N = 1, 4, 1, 2, 64, 1024, 64
    need = saga.saga_workspace_bytes(B, h_q, h_k, h_v, d, l_kv, N)
    fake = ctypes.c_void_p(0x10000)        # aligned, never dereferenced
    mis = ctypes.c_void_p(0x10008)         # misaligned
    ds = L.saga_decode_step
    args = [fake, fake, fake, B, h_q, h_k, h_v, d, l_kv, N, fake, 0, fake, None, fake, need, None]
    bad = list(args); bad[0] = None
    assert ds(*bad) == saga.SAGA_ERR_INVALID_ARG
    bad = list(args); bad[1] = mis
    assert ds(*bad) == saga.SAGA_ERR_INVALID_ARG
    bad = list(args); bad[15] = need - 256
    assert ds(*bad) == saga.SAGA_ERR_WORKSPACE
    bad = list(args); bad[14] = mis
    assert ds(*bad) == saga.SAGA_ERR_INVALID_ARG
    bad = list(args); bad[7] = 80
    assert ds(*bad) == saga.SAGA_ERR_UNSUPPORTED
    bad = list(args); bad[9] = l_kv + 1
    assert ds(*bad) == saga.SAGA_ERR_INVALID_ARG
    rt = L.saga_refresh_threshold
    assert rt(fake, None, B, h_q, h_k, d, l_kv, N, fake, fake, need, None) == \
        saga.SAGA_ERR_INVALID_ARG
    assert rt(fake, fake, B, h_q, h_k, d, l_kv, N, fake, fake, 0, None) == saga.SAGA_ERR_WORKSPACE
    dn = L.saga_dense_gqa_baseline
    dneed = L.saga_dense_workspace_bytes(1, 32, 8, 64, 4096)
    assert dn(fake, fake, fake, 1, 32, 8, 64, 4096, None, fake, dneed, None) == \
        saga.SAGA_ERR_INVALID_ARG
    assert dn(fake, fake, fake, 1, 32, 8, 64, 4096, fake, fake, dneed - 256, None) == \
        saga.SAGA_ERR_WORKSPACE
    assert L.saga_workspace_init(None, 1024, None) == saga.SAGA_ERR_INVALID_ARG
    assert L.saga_workspace_layout(B, h_q, h_k, h_v, d, l_kv, N, None) == \
        saga.SAGA_ERR_INVALID_ARG
    assert L.saga_selection_mask(fake, need, B, h_q, h_k, h_v, d, l_kv, N, None, None) == \
        saga.SAGA_ERR_INVALID_ARG
    dp = L.saga_decode_step_pivot
    pargs = [fake, fake, fake, B, h_q, h_k, h_v, d, l_kv, N, fake, fake, 2, fake, None, fake, need,
             None]
    bad = list(pargs); bad[11] = None          # refresh without a pivot array
    assert dp(*bad) == saga.SAGA_ERR_INVALID_ARG
    bad = list(pargs); bad[12] = 3             # unknown refresh mode
    assert dp(*bad) == saga.SAGA_ERR_INVALID_ARG
    bad = list(pargs); bad[16] = need - 256
    assert dp(*bad) == saga.SAGA_ERR_WORKSPACE
    fa = L.saga_full_attention
    fneed = L.saga_full_attention_workspace_bytes(1, 32, 4, 16, 64, 4096)
    assert fa(fake, fake, None, 1, 32, 4, 16, 64, 4096, fake, fake, fneed, None) == \
        saga.SAGA_ERR_INVALID_ARG
    assert fa(fake, fake, fake, 1, 32, 4, 16, 64, 4096, fake, fake, fneed - 256, None) == \
        saga.SAGA_ERR_WORKSPACE
    cw = L.saga_cache_workspace_bytes
    assert cw(1, 32, 4, 16, 64, 8192, 256) >= L.saga_workspace_bytes(1, 32, 4, 16, 64, 8192, 256)
    cneed = cw(1, 32, 4, 16, 64, 8192, 256)
    dc = L.saga_decode_step_cache
    cargs = [fake, fake, fake, 1, 32, 4, 16, 64, 8192, 4000, 256, fake, fake, 0, fake, None, fake,
             cneed, None]
    bad = list(cargs); bad[9] = 8193              # len > cap
    assert dc(*bad) == saga.SAGA_ERR_INVALID_ARG
    bad = list(cargs); bad[10] = 4001             # N > len
    assert dc(*bad) == saga.SAGA_ERR_INVALID_ARG
    bad = list(cargs); bad[17] = cneed - 256
    assert dc(*bad) == saga.SAGA_ERR_WORKSPACE
    ap = L.saga_append_kv
    assert ap(fake, fake, fake, fake, 1, 4, 16, 64, 8192, 8192, None) == saga.SAGA_ERR_INVALID_ARG
    assert ap(fake, fake, fake, mis, 1, 4, 16, 64, 8192, 10, None) == saga.SAGA_ERR_INVALID_ARG
    assert ap(fake, fake, fake, fake, 1, 4, 16, 80, 8192, 10, None) == saga.SAGA_ERR_UNSUPPORTED
    rp = L.saga_read_probe
    assert rp(None, 1024, fake, None) == saga.SAGA_ERR_INVALID_ARG
    assert rp(fake, 1024, None, None) == saga.SAGA_ERR_INVALID_ARG
    assert rp(mis, 1024, fake, None) == saga.SAGA_ERR_INVALID_ARG
    assert rp(fake, 1000, fake, None) == saga.SAGA_ERR_INVALID_ARG   # not a multiple of 16
    assert rp(fake, 0, fake, None) == saga.SAGA_ERR_INVALID_ARG


def test_binding_refuses_without_library(tmp_path):
    from sparse_asymmetric_head_amd import saga

    with pytest.raises(FileNotFoundError):
        saga.lib(str(tmp_path / "missing.so"))


def test_product_path_does_not_import_oracle():
    """The HIP path and its binding never reach the CPU oracle."""
    pkg = os.path.join(ROOT, "sparse_asymmetric_head_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in src and "from oracle" not in src, f
                assert "saga_oracle" not in src and "sao_" not in src, f


def test_merge_validates_before_launch(L):
    """The key-merge entry point rejects bad arguments on the host (no GPU needed)."""
    from sparse_asymmetric_head_amd import saga

    mw = L.saga_merge_workspace_bytes
    assert mw(4096, 32, 8, 64, 2048) > 0
    assert mw(4096, 12, 2, 128, 1536) > 0
    assert mw(8192, 32, 8, 64, 2048) > mw(4096, 32, 8, 64, 2048)
    assert mw(0, 32, 8, 64, 2048) == 0            # no tokens
    assert mw(4096, 32, 7, 64, 2048) == 0         # odd number of teacher key heads
    assert mw(4096, 32, 18, 64, 2048) == 0        # more than 16 teacher key heads
    assert mw(4096, 4, 8, 64, 2048) == 0          # fewer query heads than key heads
    assert mw(4096, 32, 8, 96, 2048) == 0         # d unsupported
    assert mw(4096, 32, 8, 64, 2000) == 0         # d_model not a multiple of 64
    n, h_q, h_kt, d, dm = 1000, 32, 8, 64, 256
    need = mw(n, h_q, h_kt, d, dm)
    fake = ctypes.c_void_p(0x10000)
    mis = ctypes.c_void_p(0x10008)
    f = L.saga_merge_key_heads
    args = [fake, fake, fake, n, h_q, h_kt, d, dm, None, fake, fake, fake, fake, fake, need, None]
    bad = list(args); bad[0] = None
    assert f(*bad) == saga.SAGA_ERR_INVALID_ARG
    bad = list(args); bad[9] = mis
    assert f(*bad) == saga.SAGA_ERR_INVALID_ARG
    bad = list(args); bad[10] = None
    assert f(*bad) == saga.SAGA_ERR_INVALID_ARG
    bad = list(args); bad[14] = need - 256
    assert f(*bad) == saga.SAGA_ERR_WORKSPACE
    bad = list(args); bad[6] = 80
    assert f(*bad) == saga.SAGA_ERR_UNSUPPORTED
    bad = list(args); bad[3] = 0
    assert f(*bad) == saga.SAGA_ERR_INVALID_ARG
    pin = ctypes.c_int32 * 8
    bad = list(args); bad[8] = pin(0, 1, 2, 3, 4, 5, 6, 6)       # head 6 twice
    assert f(*bad) == saga.SAGA_ERR_INVALID_ARG
    bad = list(args); bad[8] = pin(0, 1, 2, 3, 4, 5, 6, 8)       # head 8 does not exist
    assert f(*bad) == saga.SAGA_ERR_INVALID_ARG


@pytest.mark.parametrize("d", [64, 128])
def test_chunking_monotone_over_lengths(L, d):
    """The select plan switches its chunk unit (64 rows on short caches, 128 rows
    otherwise). A workspace sized for a cache's capacity serves every
    shorter length only if the chunk length never decreases as the cache grows, and every
    length must keep the record layout's invariants."""
    from sparse_asymmetric_head_amd import saga

    for B, h_k in [(1, 1), (1, 4), (4, 1), (2, 8), (16, 2), (1, 64)]:
        h_q = h_v = 2 * h_k
        prev = 0
        for l_kv in sorted({int(1.19 ** i) for i in range(1, 90)} | {16384, 16385, 32768, 65536}):
            if l_kv * d * 2 >= 1 << 31:
                break
            lay = saga.saga_workspace_layout(B, h_q, h_k, h_v, d, l_kv, 1)
            assert lay.chunk_len >= prev, (B, h_k, l_kv)
            prev = lay.chunk_len
            assert lay.n_chunk * lay.chunk_len >= l_kv > (lay.n_chunk - 1) * lay.chunk_len
            assert lay.n_seg == SEG_WAVES * lay.n_chunk <= 1024
            assert lay.seg_group == 16 * stream_tiles(d)
            assert lay.chunk_len % (SEG_WAVES * lay.seg_group) == 0
            assert lay.seg_cap * SEG_WAVES == lay.chunk_len
