"""Host-side checks of the C ABI: the library loads, exports what the header
declares, and rejects bad arguments before launching anything.  No GPU is
needed: every call here fails validation (or is the T = 0 no-op), so no
kernel is enqueued and the fake pointers are never touched."""
import ctypes

import pytest

from gated_deltanet_linear_pre_amd import binding as B

P = 0x10000  # 64 KiB-aligned fake device address, never dereferenced


@pytest.fixture(scope="module")
def L():
    return B.lib()


def shape(**kw):
    d = dict(hk=16, hv=48, n_seq=1, total_T=512, max_T=512, io="f16", out="f16")
    d.update(kw)
    return B.make_shape(**d)


def test_exports_every_declared_symbol(L):
    names = B.declared_symbols()
    assert set(names) == {"gdn_abi_version", "gdn_status_str", "gdn_pre", "gdn_scan",
                          "gdn_scan_workspace_bytes", "gdn_post", "gdn_prefill_workspace_bytes",
                          "gdn_prefill_layer", "gdn_prefill_layer_noalloc", "gdn_step"}
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings(L):
    assert B.gdn_abi_version() == 5
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert B.gdn_status_str(code) and B.gdn_status_str(code) != "unknown status"
    assert B.gdn_status_str(-99) == "unknown status"


def test_shape_struct_layout_matches_header():
    assert ctypes.sizeof(B.gdn_shape) == 8 * 4 + 2 * 8 + 2 * 4
    assert B.gdn_shape.total_T.offset == 32 and B.gdn_shape.eps_l2.offset == 48


def test_workspace_bytes():
    s = shape(total_T=2048, max_T=2048)
    T = 2048
    r = lambda x: (x + 255) // 256 * 256
    per_slot = 16 * 32768 + 48 * 6656   # per 32-token chunk: key-head and value-head parts
    scan = (T // 32 + 1 + 1) * per_slot
    assert B.gdn_scan_workspace_bytes(s) == scan
    # fused fp16 path (3 value heads per key head): o, the scan scratch, and a
    # counter per (chunk, value head) and a status word, 256 bytes each, for
    # post run in the chunk kernel's launch
    sync = r((T // 32 * 48 + 1) * 256)
    assert B.gdn_prefill_workspace_bytes(s) == r(T * 48 * 128 * 4) + r(scan) + sync
    # fused fp32 path: the fp32 v as well
    s32 = shape(total_T=2048, max_T=2048, io="f32")
    assert B.gdn_prefill_workspace_bytes(s32) == 2 * r(T * 48 * 128 * 4) + r(scan)
    # staged path (more than 8 value heads per key head): every intermediate
    st = shape(hk=1, hv=10, total_T=2048, max_T=2048)
    scan10 = (T // 32 + 2) * (32768 + 10 * 6656)
    want = 2 * r(T * 128 * 4) + r(T * 10 * 128 * 4) * 2 + 2 * r(T * 10 * 4) + r(scan10)
    assert B.gdn_prefill_workspace_bytes(st) == want
    assert B.gdn_prefill_workspace_bytes(shape(hv=47)) == 0
    assert B.gdn_scan_workspace_bytes(shape(hv=47)) == 0
    # varlen: at most total_T / 32 + n_seq slots per value head
    v = shape(n_seq=4, total_T=27135, max_T=16384)
    assert B.gdn_scan_workspace_bytes(v) == (27135 // 32 + 4 + 1) * per_slot


def _pre(s, **over):
    args = dict(cu=P, qkv=P, conv_w=P, a=P, b=P, A_log=P, dt_bias=P, hist=P, qn=P, kn=P, vc=P,
                g=P, beta=P)
    args.update(over)
    return B.gdn_pre(s, args["cu"], args["qkv"], args["conv_w"], args["a"], args["b"],
                     args["A_log"], args["dt_bias"], args["hist"], args["qn"], args["kn"],
                     args["vc"], args["g"], args["beta"], stream=0, check=False)


def _scan(s, ws_bytes=1 << 40, **over):
    args = dict(cu=P, qn=P, kn=P, vc=P, g=P, beta=P, state=P, o=P, ws=P)
    args.update(over)
    return B.gdn_scan(s, *args.values(), workspace_bytes=ws_bytes, stream=0, check=False)


def _post(s, **over):
    args = dict(o=P, z=P, gamma=P, y=P)
    args.update(over)
    return B.gdn_post(s, *args.values(), stream=0, check=False)


def _layer(s, ws_bytes=1 << 40, **over):
    args = dict(cu=P, qkv=P, conv_w=P, a=P, b=P, A_log=P, dt_bias=P, z=P, gamma=P, hist=P,
                state=P, y=P, ws=P)
    args.update(over)
    return B.gdn_prefill_layer(s, *args.values(), workspace_bytes=ws_bytes, stream=0, check=False)


BAD_SHAPES = [
    (dict(dk=64), -2), (dict(dv=256), -2), (dict(hk=0), -2), (dict(hv=47), -2),
    (dict(n_seq=0), -2), (dict(total_T=-1), -2), (dict(max_T=513), -2),
    (dict(max_T=0), -2), (dict(n_seq=2, max_T=200), -2), (dict(total_T=1 << 31, max_T=1), -2),
    (dict(io=7), -5), (dict(out=2), -5), (dict(eps_l2=-1.0), -2),
    (dict(eps_rms=float("nan")), -2),
]


@pytest.mark.parametrize("over,code", BAD_SHAPES)
def test_bad_shapes_rejected_by_every_entry_point(over, code):
    s = shape(**over)
    assert _pre(s) == code
    assert _scan(s) == code
    assert _post(s) == code
    assert _layer(s) == code
    s2 = shape()
    s2.reserved = 1
    assert _scan(s2) == -2


def test_null_shape_pointer(L):
    assert L.gdn_scan(None, *([P] * 9), 1 << 30, None) == -1
    assert L.gdn_prefill_workspace_bytes(None) == 0


@pytest.mark.parametrize("name", ["cu", "qkv", "conv_w", "a", "b", "A_log", "dt_bias", "hist",
                                  "qn", "kn", "vc", "g", "beta"])
def test_pre_null_pointers(name):
    assert _pre(shape(), **{name: None}) == -1


@pytest.mark.parametrize("name,off,code", [("qkv", 8, -3), ("conv_w", 4, -3), ("hist", 2, -3),
                                            ("qn", 4, -3), ("a", 2, -3), ("g", 1, -3),
                                            ("cu", 2, -3)])
def test_pre_alignment(name, off, code):
    assert _pre(shape(), **{name: P + off}) == code


@pytest.mark.parametrize("name", ["cu", "qn", "kn", "vc", "g", "beta", "state", "o", "ws"])
def test_scan_null_and_alignment(name):
    assert _scan(shape(), **{name: None}) == -1
    assert _scan(shape(), **{name: P + 2}) == -3


def test_scan_workspace_size_and_alignment():
    s = shape()
    need = B.gdn_scan_workspace_bytes(s)
    assert _scan(s, ws_bytes=need - 1) == -4
    assert _scan(s, ws=P + 128) == -3     # scratch needs 256-byte alignment


@pytest.mark.parametrize("name", ["o", "z", "gamma", "y"])
def test_post_null_and_alignment(name):
    assert _post(shape(), **{name: None}) == -1
    assert _post(shape(), **{name: P + 8}) == -3


def test_layer_workspace_checks():
    s = shape()
    need = B.gdn_prefill_workspace_bytes(s)
    assert _layer(s, ws_bytes=need - 1) == -4
    assert _layer(s, ws=None) == -1
    assert _layer(s, ws=P + 16) == -3       # workspace needs 256-byte alignment
    assert _layer(s, z=None) == -1
    assert _layer(s, state=P + 4) == -3


def test_zero_tokens_is_a_noop_that_succeeds():
    s = shape(total_T=0, max_T=0, n_seq=3)
    # nothing is validated beyond the shape and nothing is launched
    assert _pre(s, qkv=None) == 0
    assert _scan(s, o=None, ws=None, ws_bytes=0) == 0
    assert _post(s, y=None) == 0
    assert _layer(s, ws=None, ws_bytes=0) == 0


def _step(s, **over):
    args = dict(qkv=P, conv_w=P, a=P, b=P, A_log=P, dt_bias=P, z=P, gamma=P, hist=P, state=P, y=P)
    args.update(over)
    return B.gdn_step(s, *args.values(), stream=0, check=False)


def step_shape(**kw):
    d = dict(n_seq=4, total_T=4, max_T=1)
    d.update(kw)
    return shape(**d)


def test_step_shape_rules():
    # one token per sequence: total_T == n_seq and max_T == 1
    assert _step(step_shape(total_T=5, max_T=2)) == -2
    assert _step(step_shape(total_T=4, max_T=2)) == -2
    assert _step(step_shape(total_T=3)) == -2
    assert _step(step_shape(total_T=0, max_T=0)) == -2
    for over, code in BAD_SHAPES:
        if "n_seq" in over or "total_T" in over or "max_T" in over:
            continue
        assert _step(step_shape(**over)) == code


@pytest.mark.parametrize("name", ["qkv", "conv_w", "a", "b", "A_log", "dt_bias", "z", "gamma",
                                  "hist", "state", "y"])
def test_step_null_and_alignment(name):
    assert _step(step_shape(), **{name: None}) == -1
    assert _step(step_shape(), **{name: P + 2}) == -3


def test_step_hist_out_alignment():
    # a separate history output is optional, but aligned like hist when given
    s = step_shape()
    args = dict(qkv=P, conv_w=P, a=P, b=P, A_log=P, dt_bias=P, z=P, gamma=P, hist=P, state=P, y=P)
    assert B.gdn_step(s, *args.values(), stream=0, check=False, hist_out=P + 8) == -3



def _noalloc(s, **over):
    args = dict(cu=P, qkv=P, conv_w=P, a=P, b=P, A_log=P, dt_bias=P, z=P, gamma=P, hist=P,
                state=P, y=P)
    args.update(over)
    return B.gdn_prefill_layer_noalloc(s, *args.values(), stream=0, check=False)


def test_noalloc_rejects_before_touching_the_device():
    # every outcome here is decided on the host: no kernel, no runtime call
    assert _noalloc(shape(hv=47)) == -2
    assert _noalloc(shape(total_T=0, max_T=0)) == 0
    assert _noalloc(shape(), y=None) == -1
    assert _noalloc(shape(), state=P + 4) == -3
    # more workspace than the library's static array holds
    big = shape(total_T=100000, max_T=100000)
    assert B.gdn_prefill_workspace_bytes(big) > 128 << 20
    assert _noalloc(big) == -7
    assert B.gdn_status_str(-7) != "unknown status"
