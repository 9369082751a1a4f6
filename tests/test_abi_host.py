"""Host-only checks of the C ABI (no GPU needed).

libkda validates every argument before its first HIP call, so each error path
below is exercised with made-up device addresses that are never dereferenced.
"""
import ctypes

import pytest

import chunked_gated_delta_12_amd as kda

OK, NULL, SHAPE, DTYPE, ALIGN, WORKSPACE, ALIAS = 0, 1, 2, 3, 4, 5, 6
MB = 1 << 20


@pytest.fixture(scope="module")
def lib():
    try:
        return kda.load_library()
    except RuntimeError as e:   # not built in this checkout
        pytest.skip(str(e))


def test_exports_every_declared_function(lib):
    names = kda.header_functions()
    assert {"kda_chunk_fwd", "kda_decode_step", "kda_gate"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"libkda.so does not export {n}"


def test_peaks_library_exports_its_header():
    """libkda_peaks.so (the benchmark's reference copy and matrix-core loops) exports
    every function include/kda_peaks.h declares, and rejects bad arguments on the host."""
    from chunked_gated_delta_12_amd import peaks
    try:
        plib = peaks.load_library()
    except RuntimeError as e:
        pytest.skip(str(e))
    names = kda.header_functions(peaks.HEADER_PATH)
    assert set(names) == {"kda_peaks_copy", "kda_peaks_mfma_bf16", "kda_peaks_device"}
    for n in names:
        assert hasattr(plib, n), n
    vp = ctypes.c_void_p
    assert plib.kda_peaks_copy(vp(1 << 40), vp(1 << 41), 100, None) == 1          # not a multiple of 16
    assert plib.kda_peaks_copy(vp(1 << 40), vp((1 << 40) + 64), 1 << 20, None) == 1   # overlap
    assert plib.kda_peaks_copy(None, vp(1 << 41), 16, None) == 1
    assert plib.kda_peaks_mfma_bf16(None, 8, 10, None) == 1
    assert plib.kda_peaks_mfma_bf16(vp(1 << 40), 0, 10, None) == 1


def test_abi_version_and_strings(lib):
    assert lib.kda_abi_version() == 1
    for s in range(8):
        assert lib.kda_status_string(s).decode()
    assert lib.kda_status_string(99).decode() == "unknown status"


class Bufs:
    """Disjoint, 16-byte aligned fake device addresses for a chunk_fwd call."""
    def __init__(self, B=1, T=64, H=2, d=64, es=2):
        tok = B * T * H
        sizes = dict(q=tok * d * es, k=tok * d * es, v=tok * d * es, theta=tok * d * 4, beta=tok * 4,
                     S0=B * H * d * d * 4, o=tok * d * es, S_T=B * H * d * d * 4, ws=64 * MB)
        base = 1 << 40
        self.addr = {}
        for name, n in sizes.items():
            self.addr[name] = base
            base += (n + 4095) // 4096 * 4096 + 4096
        self.B, self.T, self.H, self.d = B, T, H, d

    def call(self, lib, dtype=0, segments=1, ws_bytes=64 * MB, **over):
        a = dict(self.addr)
        a.update(over)
        p = lambda n: ctypes.c_void_p(a[n]) if a[n] is not None else None
        return lib.kda_chunk_fwd(dtype, self.B, self.T, self.H, a.get("dk", self.d), a.get("dv", self.d),
                                 segments, p("q"), p("k"), p("v"), p("theta"), p("beta"), p("S0"),
                                 p("o"), p("S_T"), p("ws"), ws_bytes, None)


def test_chunk_fwd_rejects_bad_dtype_and_sizes(lib):
    b = Bufs()
    assert b.call(lib, dtype=2) == DTYPE
    assert b.call(lib, dk=48, dv=48) == SHAPE
    assert b.call(lib, dk=64, dv=32) == SHAPE
    T0 = Bufs(T=64)
    T0.T = 0
    assert T0.call(lib) == SHAPE
    assert b.call(lib, segments=-1) == SHAPE
    assert b.call(lib, segments=5) == SHAPE          # only 4 chunks in T = 64
    assert "segments" in lib.kda_last_error().decode()


def test_chunk_fwd_rejects_null_misaligned_alias(lib):
    b = Bufs()
    for name in ("q", "k", "v", "theta", "beta", "o"):
        assert b.call(lib, **{name: None}) == NULL, name
    assert b.call(lib, q=b.addr["q"] + 8) == ALIGN
    assert b.call(lib, S_T=b.addr["S_T"] + 4) == ALIGN
    assert b.call(lib, o=b.addr["q"]) == ALIAS                    # o over an input
    assert b.call(lib, o=b.addr["S_T"]) == ALIAS                  # o over the state
    assert b.call(lib, S_T=b.addr["theta"]) == ALIAS
    assert b.call(lib, S_T=b.addr["S0"] + 16) == ALIAS            # partial overlap with S0
    assert b.call(lib, ws=b.addr["v"], segments=2) == ALIAS


def test_chunk_fwd_gated_validation(lib):
    b = Bufs()
    z = (1 << 43)
    vp = ctypes.c_void_p

    def call(zaddr, **over):
        a = dict(b.addr)
        a.update(over)
        p = lambda n: vp(a[n]) if a[n] is not None else None
        return lib.kda_chunk_fwd_gated(0, b.B, b.T, b.H, b.d, b.d, 1, p("q"), p("k"), p("v"), p("theta"),
                                       p("beta"), p("S0"), vp(zaddr) if zaddr is not None else None,
                                       p("o"), p("S_T"), p("ws"), 64 * MB, None)

    assert call(None) == NULL
    assert "z" in lib.kda_last_error().decode()
    assert call(z + 8) == ALIGN
    assert call(b.addr["o"]) == ALIAS                 # o may not be written over z
    assert call(z, q=None) == NULL                    # the ungated checks still apply
    assert call(z, o=b.addr["q"]) == ALIAS


def test_chunk_fwd_noalloc_validation(lib):
    """The no-allocation entry point runs kda_chunk_fwd's host checks and refuses a
    segment count whose workspace exceeds its static scratch, before any HIP call."""
    vp = ctypes.c_void_p

    def call(b, segments=1, dtype=0, **over):
        a = dict(b.addr)
        a.update(over)
        p = lambda n: vp(a[n]) if a[n] is not None else None
        return lib.kda_chunk_fwd_noalloc(dtype, b.B, b.T, b.H, b.d, b.d, segments, p("q"), p("k"), p("v"),
                                         p("theta"), p("beta"), p("S0"), p("o"), p("S_T"), None)

    b = Bufs()
    assert call(b, dtype=2) == DTYPE
    for name in ("q", "k", "v", "theta", "beta", "o"):
        assert call(b, **{name: None}) == NULL, name
    assert call(b, q=b.addr["q"] + 8) == ALIGN
    assert call(b, o=b.addr["k"]) == ALIAS
    assert call(b, segments=5) == SHAPE
    limit = 128 * MB
    # 2^17 tokens of 16 heads at d = 128: the automatic 16 segments need 182 MB
    big = Bufs(T=1 << 17, H=16, d=128)
    need = kda.kda_chunk_fwd_workspace_size(1, 1 << 17, 16, 128, 128, 0)
    assert need > limit
    assert call(big, segments=0) == WORKSPACE
    msg = lib.kda_last_error().decode()
    assert "scratch" in msg and str(limit) in msg
    assert call(big, segments=64) == WORKSPACE
    # the 64K prefill at its automatic segment count fits the scratch
    assert 0 < kda.kda_chunk_fwd_workspace_size(1, 65536, 16, 128, 128, 0) <= limit


def test_chunk_fwd_unbounded_validation(lib):
    """The ablation entry point runs the same host checks as kda_chunk_fwd (before any
    HIP call) and takes no workspace."""
    b = Bufs()
    vp = ctypes.c_void_p

    def call(dtype=0, dk=None, **over):
        a = dict(b.addr)
        a.update(over)
        p = lambda n: vp(a[n]) if a[n] is not None else None
        d = dk or b.d
        return lib.kda_chunk_fwd_unbounded(dtype, b.B, b.T, b.H, d, d, p("q"), p("k"), p("v"),
                                           p("theta"), p("beta"), p("S0"), p("o"), p("S_T"), None)

    assert call(dtype=2) == DTYPE
    assert call(dk=48) == SHAPE
    for name in ("q", "k", "v", "theta", "beta", "o"):
        assert call(**{name: None}) == NULL, name
    assert call(theta=b.addr["theta"] + 4) == ALIGN
    assert call(o=b.addr["v"]) == ALIAS
    assert call(S_T=b.addr["beta"]) == ALIAS


def test_chunk_bwd_validation(lib):
    """The backward entry point checks sizes, NULLs, alignment, overlaps and the
    workspace on the host before any HIP call."""
    b = Bufs()
    tok = b.B * b.T * b.H
    base = 1 << 44
    grads = {}
    for name, n in (("dq", tok * b.d * 4), ("dk", tok * b.d * 4), ("dv", tok * b.d * 4),
                    ("dtheta", tok * b.d * 4), ("dbeta", tok * 4), ("dS0", b.H * b.d * b.d * 4),
                    ("do", tok * b.d * 2), ("dS_T", b.H * b.d * b.d * 4)):
        grads[name] = base
        base += (n + 4095) // 4096 * 4096 + 4096
    need = ctypes.c_size_t(0)
    assert lib.kda_chunk_bwd_workspace_size(b.B, b.T, b.H, b.d, b.d, ctypes.byref(need)) == OK
    # per chunk: its start state and its 16-token U and V - K+ S tiles, fp32
    assert need.value == (b.T // 16) * b.B * b.H * (b.d * b.d + 32 * b.d) * 4
    vp = ctypes.c_void_p

    def call(dtype=0, ws_bytes=None, **over):
        a = dict(b.addr)
        a.update(grads)
        a.update(over)
        p = lambda n: vp(a[n]) if a[n] is not None else None
        return lib.kda_chunk_bwd(dtype, b.B, b.T, b.H, b.d, b.d, p("q"), p("k"), p("v"), p("theta"), p("beta"),
                                 p("S0"), p("do"), p("dS_T"), p("dq"), p("dk"), p("dv"), p("dtheta"),
                                 p("dbeta"), p("dS0"), p("ws"), need.value if ws_bytes is None else ws_bytes,
                                 None)

    assert call(dtype=3) == DTYPE
    for name in ("q", "do", "dq", "dtheta", "dbeta"):
        assert call(**{name: None}) == NULL, name
    assert call(dq=grads["dq"] + 4) == ALIGN
    assert call(ws_bytes=need.value - 1) == WORKSPACE
    assert call(ws=None) == WORKSPACE
    assert call(dq=b.addr["q"]) == ALIAS               # a gradient over an input
    assert call(dk=grads["dq"]) == ALIAS               # two gradients over each other
    assert call(dv=b.addr["ws"]) == ALIAS              # a gradient over the workspace


def test_chunk_fwd_workspace_checks(lib):
    b = Bufs(T=1024, H=2, d=64)
    need = kda.kda_chunk_fwd_workspace_size(1, 1024, 2, 64, 64, 4)
    assert need > 0
    assert b.call(lib, segments=4, ws_bytes=need - 1) == WORKSPACE
    assert b.call(lib, segments=4, ws=None, ws_bytes=0) == WORKSPACE
    assert kda.kda_chunk_fwd_workspace_size(1, 1024, 2, 64, 64, 1) == 0


def test_workspace_formula_and_auto_segments(lib):
    # [N | M] per segment but the last, a start state per segment, and the 16x16
    # T = (I + A)^-1 of every chunk, all sized in fp32
    B, T, H, d, P = 1, 65536, 16, 128, 32
    want = ((P - 1) * B * H * d * 2 * d + P * B * H * d * d + (T // 16) * B * H * 256) * 4
    assert kda.kda_chunk_fwd_workspace_size(B, T, H, d, d, P) == want
    assert kda.kda_chunk_fwd_auto_segments(1, 65536, 16, 128, 128) == 16
    assert kda.kda_chunk_fwd_auto_segments(2, 65536, 128, 128, 128) == 2
    assert kda.kda_chunk_fwd_auto_segments(64, 4096, 16, 128, 128) == 1
    assert kda.kda_chunk_fwd_auto_segments(1, 64, 1, 16, 16) == 1       # too short to split
    assert kda.kda_chunk_fwd_auto_segments(1, 64, 1, 24, 24) <= 0       # unsupported size
    with pytest.raises(kda.KdaError):
        kda.kda_chunk_fwd_workspace_size(1, 0, 1, 16, 16)


def test_decode_step_validation(lib):
    base = 1 << 41
    B, H, d = 4, 2, 64
    addr = {}
    for name, n in dict(q=B * H * d * 2, k=B * H * d * 2, v=B * H * d * 2, theta=B * H * d * 4,
                        beta=B * H * 4, S=B * H * d * d * 4, o=B * H * d * 2).items():
        addr[name] = base
        base += (n + 4095) // 4096 * 4096 + 4096

    def call(dtype=0, dk=d, dv=d, **over):
        a = dict(addr)
        a.update(over)
        p = lambda n: ctypes.c_void_p(a[n]) if a[n] is not None else None
        return lib.kda_decode_step(dtype, B, H, dk, dv, p("q"), p("k"), p("v"), p("theta"), p("beta"),
                                   p("S"), p("o"), None)

    assert call(dtype=7) == DTYPE
    assert call(dk=16, dv=32) == SHAPE
    assert call(S=None) == NULL
    assert call(o=addr["o"] + 2) == ALIGN
    assert call(o=addr["S"]) == ALIAS
    assert call(S=addr["q"]) == ALIAS

    z = base

    def gated(zaddr, **over):
        a = dict(addr)
        a.update(over)
        p = lambda n: ctypes.c_void_p(a[n]) if a[n] is not None else None
        return lib.kda_decode_step_gated(0, B, H, d, d, p("q"), p("k"), p("v"), p("theta"), p("beta"),
                                         p("S"), ctypes.c_void_p(zaddr) if zaddr is not None else None,
                                         p("o"), None)

    assert gated(None) == NULL
    assert gated(z + 4) == ALIGN
    assert gated(addr["o"]) == ALIAS                  # o over z
    assert gated(addr["S"]) == ALIAS                  # the state over z
    assert gated(z, S=None) == NULL                   # the ungated checks still apply


def test_gate_validation(lib):
    th, g, gc = 1 << 42, (1 << 42) + (64 << 20), (1 << 42) + (128 << 20)
    vp = ctypes.c_void_p
    assert lib.kda_gate(1, 64, 2, 16, None, vp(g), vp(gc), None) == NULL
    assert lib.kda_gate(1, 64, 2, 16, vp(th), None, None, None) == NULL
    assert lib.kda_gate(1, 0, 2, 16, vp(th), vp(g), vp(gc), None) == SHAPE
    assert lib.kda_gate(1, 64, 2, 20, vp(th), vp(g), vp(gc), None) == SHAPE
    assert lib.kda_gate(1, 64, 2, 16, vp(th), vp(th), vp(gc), None) == ALIAS
    assert lib.kda_gate(1, 64, 2, 16, vp(th), vp(g), vp(g), None) == ALIAS
    assert lib.kda_gate(1, 64, 2, 16, vp(th + 4), vp(g), None, None) == ALIGN


def test_chunk_bwd_workspace_segmented(lib):
    """Few heads over a long sequence: the backward splits each sequence into
    segments and its workspace adds, per segment and head, both segment maps
    (d x 2d each) and the state and carried gradient at the segment's ends."""
    need = ctypes.c_size_t(0)
    B, T, H, d = 1, 65536, 16, 128
    assert lib.kda_chunk_bwd_workspace_size(B, T, H, d, d, ctypes.byref(need)) == OK
    nchunks, nseg = T // 16, 16                 # 256 chunks per segment, 16 x 16 workgroups
    per_chunk = d * d + 32 * d
    assert need.value == 4 * (nchunks * B * H * per_chunk + nseg * B * H * 6 * d * d)
    # many heads: one segment, no extra workspace
    assert lib.kda_chunk_bwd_workspace_size(32, 4096, 16, d, d, ctypes.byref(need)) == OK
    assert need.value == 4 * (4096 // 16) * 32 * 16 * per_chunk
