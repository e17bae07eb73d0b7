"""Host-side checks of the C ABI: the library loads, exports everything the
header declares, and rejects bad arguments with a status before touching the
GPU (every call here returns before any HIP call, so it runs without a GPU)."""
import os
import re

import pytest

import gated_delta_rule_83_amd as g

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "gdn2.h")

FAKE = 1 << 40  # a 16-byte aligned address that is never dereferenced by argument checks


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn2_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = g.load()
    names = declared_functions()
    assert set(names) == set(g.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert g.gdn2_version() == 10000
    for s in range(9):
        assert g.gdn2_status_string(s) != "unknown status", s
    assert g.gdn2_status_string(99) == "unknown status"


def _ptrs(n_bytes_each=1 << 30):
    # nine distinct, non-overlapping fake buffers (q, k, v, a, b, w, S0, o, S_T)
    return [FAKE + i * n_bytes_each for i in range(9)]


def fwd(desc, ptrs=None, **kw):
    p = ptrs or _ptrs()
    return g.gdn2_chunk_forward(desc, *p, kw.get("ws", 0), kw.get("ws_bytes", 0), 0)


def test_chunk_forward_argument_errors():
    d = g.make_desc(2, 64, 2, 4, 128, 128, 64, g.GDN2_BF16)
    assert fwd(None) == g.GDN2_ERR_NULL_POINTER
    assert fwd(g.make_desc(2, 64, 2, 4, 128, 128, 64, 7)) == g.GDN2_ERR_BAD_DTYPE
    assert fwd(g.make_desc(-1, 64, 2, 4, 128, 128, 64, 1)) == g.GDN2_ERR_BAD_SHAPE
    assert fwd(g.make_desc(2, -3, 2, 4, 128, 128, 64, 1)) == g.GDN2_ERR_BAD_SHAPE
    assert fwd(g.make_desc(2, 64, 3, 4, 128, 128, 64, 1)) == g.GDN2_ERR_BAD_SHAPE  # H_v % H_qk
    assert fwd(g.make_desc(2, 64, 0, 4, 128, 128, 64, 1)) == g.GDN2_ERR_BAD_SHAPE
    assert fwd(g.make_desc(2, 64, 2, 4, 96, 128, 64, 1)) == g.GDN2_ERR_UNSUPPORTED
    assert fwd(g.make_desc(2, 64, 2, 4, 128, 256, 64, 1)) == g.GDN2_ERR_UNSUPPORTED
    assert fwd(g.make_desc(2, 64, 2, 4, 128, 128, 48, 1)) == g.GDN2_ERR_UNSUPPORTED
    assert fwd(g.make_desc(2, 64, 2, 4, 128, 128, 128, 1)) == g.GDN2_ERR_UNSUPPORTED
    # required pointers
    for i in range(6):
        p = _ptrs()
        p[i] = 0
        assert fwd(d, p) == g.GDN2_ERR_NULL_POINTER, i
    p = _ptrs()
    p[7] = 0  # o
    assert fwd(d, p) == g.GDN2_ERR_NULL_POINTER
    # misaligned
    p = _ptrs()
    p[3] += 4
    assert fwd(d, p) == g.GDN2_ERR_BAD_SHAPE
    # o overlapping an input, or the state
    for i in (0, 1, 2, 3, 4, 5, 6, 8):
        p = _ptrs()
        p[7] = p[i] + 16
        assert fwd(d, p) == g.GDN2_ERR_ALIAS, i
    # S_T partially overlapping S0
    p = _ptrs()
    p[8] = p[6] + 64
    assert fwd(d, p) == g.GDN2_ERR_ALIAS


def test_chunk_forward_empty_batch_is_ok_without_gpu():
    # B == 0: nothing to do, returns before any launch
    assert fwd(g.make_desc(0, 64, 2, 4, 128, 128, 64, 1), [0] * 9) == g.GDN2_OK


def test_workspace_query():
    assert g.gdn2_chunk_forward_workspace_bytes(g.make_desc(8, 4096, 16, 16, 128, 128, 64, 1)) == 0
    assert g.gdn2_chunk_forward_workspace_bytes(None) == 0
    assert g.gdn2_chunk_forward_workspace_bytes(g.make_desc(1, 64, 2, 2, 96, 16, 16, 0)) == 0


def test_split_workspace_query_and_errors(monkeypatch):
    """Few heads over a long sequence: the prefill splits the sequence and asks
    for workspace (segments x (d_k x d_v state + d_k x d_k transition) fp32 per
    head, 256-byte aligned, then the identity columns' query reads, one row of
    d_k per token and value head in the input dtype); too little or an
    overlapping workspace is rejected before any launch."""
    d2 = g.make_desc(1, 65536, 16, 16, 128, 128, 64, g.GDN2_BF16)
    per_seg = 16 * 128 * (128 + 128) * 4
    rows = 65536 * 16 * 128 * 2
    monkeypatch.delenv("GDN2_PREFILL_SPLIT", raising=False)
    need = g.gdn2_chunk_forward_workspace_bytes(d2)
    # the largest power of two of segments whose first pass fits one round of
    # the 256 compute units: 32 value + 32 identity blocks per later segment
    assert need == 4 * per_seg + rows
    assert g.gdn2_chunk_forward_plan(d2)[2] == 4
    monkeypatch.setenv("GDN2_PREFILL_SPLIT", "1")
    assert g.gdn2_chunk_forward_workspace_bytes(d2) == 0
    monkeypatch.setenv("GDN2_PREFILL_SPLIT", "8")
    assert g.gdn2_chunk_forward_workspace_bytes(d2) == 8 * per_seg + rows
    monkeypatch.delenv("GDN2_PREFILL_SPLIT")
    ws = FAKE + 20 * (1 << 30)
    assert fwd(d2) == g.GDN2_ERR_WORKSPACE
    assert fwd(d2, ws=ws, ws_bytes=need - 1) == g.GDN2_ERR_WORKSPACE
    assert fwd(d2, ws=ws + 4, ws_bytes=need) == g.GDN2_ERR_BAD_SHAPE  # misaligned
    for i in (0, 3, 6, 7, 8):
        p = _ptrs()
        assert fwd(d2, p, ws=p[i] + 256, ws_bytes=need) == g.GDN2_ERR_ALIAS, i


def test_split_plan_fills_one_round(monkeypatch):
    """The prefill's own split plan: the largest power of two of segments whose
    first pass (every segment's value column blocks, all but the first
    segment's identity blocks; 64-column blocks at d = 128) stays within one
    round of the 256 compute units, at most one segment per 16 chunks; shapes
    with enough workgroups unsplit run whole."""
    monkeypatch.delenv("GDN2_PREFILL_SPLIT", raising=False)

    def nseg(B, T, Hqk, Hv):
        st, crun, n = g.gdn2_chunk_forward_plan(g.make_desc(B, T, Hqk, Hv, 128, 128, 64, g.GDN2_BF16))
        assert st == g.GDN2_OK and crun == 32
        return n

    # B1 H16: 32 value + 32 identity blocks per segment: 4 segments = 224 workgroups (8 would be 480)
    assert nseg(1, 65536, 16, 16) == 4
    assert nseg(2, 65536, 16, 16) == 2      # 64 + 64 per segment: 2 segments = 192
    assert nseg(1, 65536, 8, 8) == 8        # 16 + 16: 8 segments = 240
    assert nseg(1, 65536, 1, 1) == 64       # 2 + 2: 64 segments = 254 (one per 16 chunks: 128 allowed)
    assert nseg(1, 16 * 32 * 3, 1, 1) == 3  # capped at one segment per 16 chunks (48 chunks)
    assert nseg(1, 65536, 64, 64) == 1      # 128 value blocks: enough workgroups unsplit
    assert nseg(8, 4096, 16, 16) == 1       # the layer shape


def test_coupled_argument_errors():
    def fc(desc, p=None, ws=0, ws_bytes=0):
        p = p or _ptrs()[:8]  # q, k, v, a, beta, S0, o, S_T
        return g.gdn2_chunk_forward_coupled(desc, *p, ws, ws_bytes, 0)

    d = g.make_desc(2, 64, 2, 4, 128, 128, 64, g.GDN2_BF16)
    assert fc(None) == g.GDN2_ERR_NULL_POINTER
    assert fc(g.make_desc(2, 64, 2, 4, 128, 128, 64, 3)) == g.GDN2_ERR_BAD_DTYPE
    assert fc(g.make_desc(2, 64, 2, 4, 128, 128, 48, 1)) == g.GDN2_ERR_UNSUPPORTED
    for i in range(5):
        p = _ptrs()[:8]
        p[i] = 0
        assert fc(d, p) == g.GDN2_ERR_NULL_POINTER, i
    p = _ptrs()[:8]
    p[4] += 2
    assert fc(d, p) == g.GDN2_ERR_BAD_SHAPE
    p[4] += 2  # beta needs 4-byte alignment only: the call gets to the overlap check
    p[6] = p[4] + 12  # o (16-byte aligned) inside beta
    assert fc(d, p) == g.GDN2_ERR_ALIAS
    p = _ptrs()[:8]
    p[3] += 4  # the per-channel decay keeps 16
    assert fc(d, p) == g.GDN2_ERR_BAD_SHAPE
    for i in (0, 3, 4, 5, 7):
        p = _ptrs()[:8]
        p[6] = p[i] + 16
        assert fc(d, p) == g.GDN2_ERR_ALIAS, i
    # the long-context shape needs the split workspace, as for gdn2_chunk_forward
    d2 = g.make_desc(1, 65536, 16, 16, 128, 128, 64, g.GDN2_BF16)
    assert fc(d2) == g.GDN2_ERR_WORKSPACE


def test_scalar_argument_errors():
    d = g.make_desc(2, 64, 2, 4, 128, 128, 64, g.GDN2_BF16)
    p = _ptrs()[:8]
    assert g.gdn2_chunk_forward_scalar(None, *p, 0, 0, 0) == g.GDN2_ERR_NULL_POINTER
    p[3] = 0
    assert g.gdn2_chunk_forward_scalar(d, *p, 0, 0, 0) == g.GDN2_ERR_NULL_POINTER
    p = _ptrs()[:8]
    p[6] = p[3] + 16
    assert g.gdn2_chunk_forward_scalar(d, *p, 0, 0, 0) == g.GDN2_ERR_ALIAS


def test_varlen_argument_errors():
    def fv(desc, cu=FAKE + 30 * (1 << 30), p=None):
        p = p or _ptrs()
        return g.gdn2_chunk_forward_varlen(desc, cu, *p, 0)

    d = g.make_desc(4, 640, 2, 4, 128, 128, 64, g.GDN2_BF16)
    assert fv(None) == g.GDN2_ERR_NULL_POINTER
    assert fv(g.make_desc(4, 640, 2, 4, 128, 128, 64, 9)) == g.GDN2_ERR_BAD_DTYPE
    assert fv(g.make_desc(4, 640, 3, 4, 128, 128, 64, 1)) == g.GDN2_ERR_BAD_SHAPE
    assert fv(g.make_desc(0, 640, 2, 4, 128, 128, 64, 1), cu=0) == g.GDN2_OK  # no sequences: nothing to do
    assert fv(d, cu=0) == g.GDN2_ERR_NULL_POINTER
    p = _ptrs()
    p[1] = 0
    assert fv(d, p=p) == g.GDN2_ERR_NULL_POINTER
    p = _ptrs()
    p[0] += 8
    assert fv(d, p=p) == g.GDN2_ERR_BAD_SHAPE
    for i in (0, 2, 3, 6, 8):
        p = _ptrs()
        p[7] = p[i] + 16
        assert fv(d, p=p) == g.GDN2_ERR_ALIAS, i
    p = _ptrs()
    assert fv(d, cu=p[7] + 64, p=p) == g.GDN2_ERR_ALIAS  # o over the offsets
    assert fv(d, cu=p[8] + 64, p=p) == g.GDN2_ERR_ALIAS  # S_T over the offsets


def test_decode_argument_errors():
    def dec(desc, p=None):
        p = p or _ptrs()[:8]
        return g.gdn2_decode_step(desc, *p, 0)

    d = g.make_desc(256, 1, 16, 16, 128, 128, 64, g.GDN2_BF16)
    assert dec(None) == g.GDN2_ERR_NULL_POINTER
    assert dec(g.make_desc(256, 2, 16, 16, 128, 128, 64, 1)) == g.GDN2_ERR_BAD_SHAPE  # T != 1
    assert dec(g.make_desc(256, 1, 16, 16, 128, 128, 64, 5)) == g.GDN2_ERR_BAD_DTYPE
    assert dec(g.make_desc(256, 1, 16, 16, 80, 128, 64, 1)) == g.GDN2_ERR_UNSUPPORTED
    assert dec(g.make_desc(0, 1, 16, 16, 128, 128, 64, 1), [0] * 8) == g.GDN2_OK
    for i in range(8):
        p = _ptrs()[:8]
        p[i] = 0
        assert dec(d, p) == g.GDN2_ERR_NULL_POINTER, i
    p = _ptrs()[:8]
    p[6] += 8
    assert dec(d, p) == g.GDN2_ERR_BAD_SHAPE
    for i in range(7):
        p = _ptrs()[:8]
        p[7] = p[i]
        assert dec(d, p) == g.GDN2_ERR_ALIAS, i


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="not found"):
        g.load(str(tmp_path / "nope.so"))


def bwd(desc, ptrs=None, ws=0, ws_bytes=0):
    # q, k, v, a, b, w, S0, dO, dS_T, dq, dk, dv, da, db, dw, dS0
    p = ptrs or [FAKE + i * (1 << 30) for i in range(16)]
    return g.gdn2_chunk_backward(desc, *p, ws, ws_bytes, 0)


def test_backward_workspace_query_and_argument_errors():
    """Workspace: fp32 checkpoints every 4 tokens (d_k x d_v per head), four
    d_k-vectors per token, head and 64-column block, one d_v-vector of
    k-reads per token and head, and one value per token, head and column
    block (the coupled gate's value-side sums); errors before any launch."""
    d = g.make_desc(2, 20, 1, 2, 64, 64, 64, g.GDN2_BF16)
    nslot, ncb = 2 * 20 // 4 + 2, 1  # checkpoint slots: B*T/4 + B; one 64-column block
    ck = 2 * nslot * 64 * 64 * 4
    part = ncb * 2 * 20 * 2 * 4 * 64 * 4
    rk = 2 * 2 * 20 * 64 * 4
    wsum = ncb * 2 * 20 * 2 * 4
    up = lambda x: (x + 255) // 256 * 256
    need = g.gdn2_chunk_backward_workspace_bytes(d)
    assert need == up(ck) + up(part) + up(rk) + up(wsum)
    assert g.gdn2_chunk_backward_workspace_bytes(None) == 0
    assert g.gdn2_chunk_backward_workspace_bytes(g.make_desc(1, 0, 1, 1, 16, 16, 16, 0)) == 0
    ws = FAKE + 40 * (1 << 30)
    assert bwd(None) == g.GDN2_ERR_NULL_POINTER
    assert bwd(g.make_desc(2, 20, 1, 2, 96, 64, 64, 1), ws=ws, ws_bytes=need) == g.GDN2_ERR_UNSUPPORTED
    assert bwd(d) == g.GDN2_ERR_WORKSPACE
    assert bwd(d, ws=ws, ws_bytes=need - 1) == g.GDN2_ERR_WORKSPACE
    assert bwd(d, ws=ws + 16, ws_bytes=need) == g.GDN2_ERR_BAD_SHAPE  # workspace needs 256-byte alignment
    assert bwd(g.make_desc(0, 20, 1, 2, 64, 64, 64, 1), [0] * 16) == g.GDN2_OK  # empty batch
    base = [FAKE + i * (1 << 30) for i in range(16)]
    for i in (0, 1, 2, 3, 4, 5, 7, 9, 10, 11, 12, 13, 14):  # required pointers
        p = list(base)
        p[i] = 0
        assert bwd(d, p, ws, need) == g.GDN2_ERR_NULL_POINTER, i
    for i in (6, 8, 15):  # S0, dS_T, dS0 are optional
        p = list(base)
        p[i] = 0
        # the call would launch; only check that the pointer checks pass by
        # making a later check fail (misaligned dq)
        p[9] += 4
        assert bwd(d, p, ws, need) == g.GDN2_ERR_BAD_SHAPE, i
    p = list(base)
    p[12] += 8
    assert bwd(d, p, ws, need) == g.GDN2_ERR_BAD_SHAPE
    for i in range(9):  # an output over an input
        for o in (9, 11, 12, 15):
            p = list(base)
            p[o] = p[i] + 16
            assert bwd(d, p, ws, need) == g.GDN2_ERR_ALIAS, (i, o)
    p = list(base)
    p[10] = p[9] + 256  # two outputs overlapping
    assert bwd(d, p, ws, need) == g.GDN2_ERR_ALIAS
    assert bwd(d, base, base[3] + 256, need) == g.GDN2_ERR_ALIAS  # workspace over an input
    assert bwd(d, base, base[13] + 256, need) == g.GDN2_ERR_ALIAS  # ... over an output
    p = list(base)
    p[15] = p[8] + 64  # dS0 partially over dS_T
    assert bwd(d, p, ws, need) == g.GDN2_ERR_ALIAS


def test_backward_split_workspace(monkeypatch):
    """The per-token backward (GDN2_BACKWARD_CHUNKED=0). Few long sequences:
    it runs as segments and its workspace query accounts for the split's
    buffers (more than the unsplit layout); a workspace of the unsplit size
    is then rejected before any launch."""
    monkeypatch.setenv("GDN2_BACKWARD_CHUNKED", "0")
    d = g.make_desc(1, 8192, 2, 4, 128, 128, 64, g.GDN2_BF16)
    monkeypatch.setenv("GDN2_BACKWARD_SPLIT", "1")
    plain = g.gdn2_chunk_backward_workspace_bytes(d)
    monkeypatch.setenv("GDN2_BACKWARD_SPLIT", "4")
    split = g.gdn2_chunk_backward_workspace_bytes(d)
    assert split > plain > 0
    ws = FAKE + 40 * (1 << 30)
    assert bwd(d, ws=ws, ws_bytes=plain) == g.GDN2_ERR_WORKSPACE
    monkeypatch.delenv("GDN2_BACKWARD_SPLIT")
    # the default plan splits this shape (8 workgroups, 8192 tokens) and not the layer shape
    assert g.gdn2_chunk_backward_workspace_bytes(d) > plain
    # the prefill cannot split d_k = 16 with 32-column workgroups: no split, the plain layout
    small = g.make_desc(1, 8192, 1, 2, 16, 32, 64, g.GDN2_BF16)
    monkeypatch.setenv("GDN2_BACKWARD_SPLIT", "4")
    forced = g.gdn2_chunk_backward_workspace_bytes(small)
    monkeypatch.setenv("GDN2_BACKWARD_SPLIT", "1")
    assert forced == g.gdn2_chunk_backward_workspace_bytes(small)
    c1 = g.make_desc(8, 4096, 16, 16, 128, 128, 64, g.GDN2_BF16)
    monkeypatch.setenv("GDN2_BACKWARD_SPLIT", "1")
    c1_plain = g.gdn2_chunk_backward_workspace_bytes(c1)
    monkeypatch.delenv("GDN2_BACKWARD_SPLIT")
    assert g.gdn2_chunk_backward_workspace_bytes(c1) == c1_plain


def test_backward_chunk_form_workspace(monkeypatch):
    """bf16, d_k = d_v = 128: the query returns the chunk form's workspace
    (with room for the per-token backward in rounds), about 1.5 GB at the
    layer shape B8 T4096 H16 against 11 GB for the per-token backward at
    once; a smaller workspace is rejected before any launch. Other shapes
    keep the per-token backward's size."""
    monkeypatch.delenv("GDN2_BACKWARD_CHUNKED", raising=False)
    c1 = g.make_desc(8, 4096, 16, 16, 128, 128, 64, g.GDN2_BF16)
    chunk = g.gdn2_chunk_backward_workspace_bytes(c1)
    monkeypatch.setenv("GDN2_BACKWARD_CHUNKED", "0")
    per_token = g.gdn2_chunk_backward_workspace_bytes(c1)
    monkeypatch.delenv("GDN2_BACKWARD_CHUNKED")
    assert chunk < 2 * 10**9 < per_token
    assert 1.3e9 < chunk < 1.6e9
    ws = FAKE + 40 * (1 << 30)
    assert bwd(c1, ws=ws, ws_bytes=chunk - 256) == g.GDN2_ERR_WORKSPACE
    for desc in (g.make_desc(2, 300, 1, 2, 64, 64, 64, g.GDN2_BF16), g.make_desc(2, 300, 1, 2, 128, 128, 64,
                                                                                g.GDN2_F32)):
        a = g.gdn2_chunk_backward_workspace_bytes(desc)
        monkeypatch.setenv("GDN2_BACKWARD_CHUNKED", "0")
        assert g.gdn2_chunk_backward_workspace_bytes(desc) == a
        monkeypatch.delenv("GDN2_BACKWARD_CHUNKED")


def test_backward_chunk_form_workspace_long_context(monkeypatch):
    """The long-context shape B1 T65536 H16 (bf16, d128): the chunk form's
    workspace (about 3 GB) adds, to what one launch over the whole sequence
    would need (GDN2_PREFILL_SPLIT=1), the prefill split's 8 segments: their
    transitions, exiting and entering states (3 x 8 x 16 fp32 128 x 128)."""
    monkeypatch.delenv("GDN2_BACKWARD_CHUNKED", raising=False)
    monkeypatch.delenv("GDN2_PREFILL_SPLIT", raising=False)
    c2 = g.make_desc(1, 65536, 16, 16, 128, 128, 64, g.GDN2_BF16)
    seg = g.gdn2_chunk_backward_workspace_bytes(c2)
    monkeypatch.setenv("GDN2_PREFILL_SPLIT", "1")
    whole = g.gdn2_chunk_backward_workspace_bytes(c2)
    monkeypatch.delenv("GDN2_PREFILL_SPLIT")
    assert seg - whole == 3 * 8 * 16 * 128 * 128 * 4
    assert 2.9e9 < seg < 3.1e9


def test_backward_varlen_workspace_and_errors():
    """Packed sequences: the workspace counts desc.T tokens in all; a null
    cu_seqlens and overlaps with it are rejected before any launch."""
    d = g.make_desc(3, 50, 1, 2, 64, 64, 64, g.GDN2_BF16)
    up = lambda x: (x + 255) // 256 * 256
    need = g.gdn2_chunk_backward_varlen_workspace_bytes(d)
    assert need == (up((50 // 4 + 3) * 2 * 64 * 64 * 4) + up(1 * 50 * 2 * 4 * 64 * 4) + up(50 * 2 * 64 * 4)
                    + up(1 * 50 * 2 * 4))
    ws = FAKE + 40 * (1 << 30)
    base = [FAKE + i * (1 << 30) for i in range(16)]
    cu = FAKE + 50 * (1 << 30)
    call = lambda cu_, p, w=ws, nb=need: g.gdn2_chunk_backward_varlen(d, cu_, *p, w, nb, 0)
    assert call(0, base) == g.GDN2_ERR_NULL_POINTER
    assert call(cu, base, 0, 0) == g.GDN2_ERR_WORKSPACE
    p = list(base)
    p[9] = cu  # dq over cu_seqlens
    assert call(cu, p) == g.GDN2_ERR_ALIAS
    assert g.gdn2_chunk_backward_varlen(g.make_desc(0, 50, 1, 2, 64, 64, 64, 1), 0, *([0] * 16), 0, 0, 0) == g.GDN2_OK


def test_backward_coupled_scalar_errors():
    """Coupled and scalar gate forms: beta (and alpha) one fp32 per token and
    value head, no write gate; required pointers, alignment and overlaps at
    those sizes are checked before any launch."""
    d = g.make_desc(2, 20, 1, 2, 64, 64, 64, g.GDN2_BF16)
    need = g.gdn2_chunk_backward_workspace_bytes(d)
    ws = FAKE + 40 * (1 << 30)
    # q, k, v, a, beta, S0, dO, dS_T, dq, dk, dv, da, dbeta, dS0
    base = [FAKE + i * (1 << 30) for i in range(14)]
    for entry in (g.gdn2_chunk_backward_coupled, g.gdn2_chunk_backward_scalar):
        call = lambda p, w=ws, nb=need: entry(d, *p, w, nb, 0)
        assert call(base, 0, 0) == g.GDN2_ERR_WORKSPACE
        for i in (0, 1, 2, 3, 4, 6, 8, 9, 10, 11, 12):  # required pointers
            p = list(base)
            p[i] = 0
            assert call(p) == g.GDN2_ERR_NULL_POINTER, i
        p = list(base)
        p[12] += 2  # dbeta needs 4-byte alignment
        assert call(p) == g.GDN2_ERR_BAD_SHAPE
        p[12] += 2
        p[11] = p[12] + 12  # ... and passes with it: the overlap of da with it is found next
        assert call(p) == g.GDN2_ERR_ALIAS
        p = list(base)
        p[12] = p[4] + 16  # dbeta over beta
        assert call(p) == g.GDN2_ERR_ALIAS
        assert entry(g.make_desc(0, 20, 1, 2, 64, 64, 64, 1), *([0] * 14), 0, 0, 0) == g.GDN2_OK
    # beta holds B*T*H_v floats: dbeta just past it is no overlap (so the
    # call gets as far as the alignment check of a misaligned dq)
    p = list(base)
    p[12] = p[4] + 2 * 20 * 2 * 4
    p[8] += 4
    assert g.gdn2_chunk_backward_scalar(d, *p, ws, need, 0) == g.GDN2_ERR_BAD_SHAPE
    p[12] -= 16  # ... and 16 bytes earlier it is
    p[8] -= 4
    assert g.gdn2_chunk_backward_scalar(d, *p, ws, need, 0) == g.GDN2_ERR_ALIAS


def test_varlen_gate_forms_errors():
    """Packed sequences in the other gate forms: an unknown form is
    unsupported, w may be null for the coupled forms (and is required
    otherwise), a null cu_seqlens is rejected, and the gates are checked for
    overlap at their own sizes; all before any launch."""
    d = g.make_desc(3, 50, 1, 2, 64, 64, 64, g.GDN2_BF16)
    cu = FAKE + 50 * (1 << 30)
    base = [FAKE + i * (1 << 30) for i in range(8)]  # q, k, v, a, b, w, S0, o (S_T last, none)
    fwd = lambda form, p, cu_=cu: g.gdn2_chunk_forward_varlen_gates(d, cu_, form, *p, 0, 0)
    for form in (4, -1, 100):
        assert fwd(form, base) == g.GDN2_ERR_UNSUPPORTED, form
    assert fwd(2, base, 0) == g.GDN2_ERR_NULL_POINTER
    for form in (0, 1):
        p = list(base)
        p[5] = 0
        assert fwd(form, p) == g.GDN2_ERR_NULL_POINTER, form
    for form in (2, 3):
        p = list(base)
        p[5] = 0
        p[7] = p[4] + 16  # o over beta
        assert fwd(form, p) == g.GDN2_ERR_ALIAS, form
        p[7] = p[4] + 50 * 2 * 4  # o just past beta (T * H_v floats): no overlap, fails later on alignment
        p[0] += 4
        assert fwd(form, p) == g.GDN2_ERR_BAD_SHAPE, form
    # scalar alpha holds T * H_v floats; the coupled per-channel decay T * H_v * d_k
    p = list(base)
    p[7] = p[3] + 50 * 2 * 4
    p[0] += 4
    assert fwd(3, p) == g.GDN2_ERR_BAD_SHAPE
    p[0] -= 4
    assert fwd(2, p) == g.GDN2_ERR_ALIAS
    # backward: unknown form, null dw allowed for the coupled forms
    need = g.gdn2_chunk_backward_varlen_workspace_bytes(d)
    ws = FAKE + 40 * (1 << 30)
    bb = [FAKE + i * (1 << 30) for i in range(16)]
    bwd = lambda form, p: g.gdn2_chunk_backward_varlen_gates(d, cu, form, *p, ws, need, 0)
    assert bwd(7, bb) == g.GDN2_ERR_UNSUPPORTED
    assert g.gdn2_chunk_backward_varlen_gates(None, cu, 7, *bb, ws, need, 0) == g.GDN2_ERR_NULL_POINTER
    for form in (0, 1):
        p = list(bb)
        p[14] = 0  # dw
        assert bwd(form, p) == g.GDN2_ERR_NULL_POINTER, form
    for form in (2, 3):
        p = list(bb)
        p[5] = p[14] = 0
        p[9] += 4  # misaligned dq: the pointer checks passed
        assert bwd(form, p) == g.GDN2_ERR_BAD_SHAPE, form


def test_decode_gate_forms_errors():
    """Decode in the other gate forms: unknown form, w optional only for the
    coupled forms, 4-byte alignment for beta and alpha, overlaps at the gate
    sizes; all before any launch."""
    d = g.make_desc(4, 1, 2, 2, 64, 64, 64, g.GDN2_BF16)
    base = [FAKE + i * (1 << 30) for i in range(9)]  # q, k, v, a, b, w, S, o (stream last)
    dec = lambda form, p: g.gdn2_decode_step_gates(d, form, *p[:8], 0)
    assert dec(9, base) == g.GDN2_ERR_UNSUPPORTED
    for form in range(4):  # an empty batch returns before the pointers are looked at
        assert g.gdn2_decode_step_gates(g.make_desc(0, 1, 2, 2, 64, 64, 64, 1), form, *[0] * 8, 0) == g.GDN2_OK
    assert g.gdn2_decode_step_gates(g.make_desc(4, 2, 2, 2, 64, 64, 64, 1), 2, *base[:8], 0) == g.GDN2_ERR_BAD_SHAPE
    for form in (0, 1):
        p = list(base)
        p[5] = 0
        assert dec(form, p) == g.GDN2_ERR_NULL_POINTER, form
    for form in (2, 3):
        p = list(base)
        p[5] = 0
        p[4] += 2
        assert dec(form, p) == g.GDN2_ERR_BAD_SHAPE, form  # beta not 4-byte aligned
        p[4] += 2
        p[7] = p[4] + 12  # o over beta: found after the alignment checks pass
        assert dec(form, p) == g.GDN2_ERR_ALIAS, form
        p[7] = p[4] + 4 * 2 * 4 + 12  # o just past beta's B * H_v floats
        p[0] += 4
        assert dec(form, p) == g.GDN2_ERR_BAD_SHAPE, form


def test_binding_exposes_every_entry_point_wrapper():
    """The torch-level wrappers of every entry point exist (import-time check;
    the GPU tests exercise them)."""
    for name in ("chunk_forward", "chunk_forward_preact", "chunk_forward_coupled", "chunk_forward_scalar",
                 "chunk_forward_varlen", "decode_step", "chunk_backward", "chunk_backward_preact",
                 "chunk_backward_varlen", "chunk_backward_coupled", "chunk_backward_scalar", "gated_delta_rule",
                 "gated_delta_rule_preact", "gated_delta_rule_coupled", "gated_delta_rule_scalar",
                 "gated_delta_rule_varlen", "decode_step"):
        assert callable(getattr(g, name, None)), name


def test_noalloc_argument_errors_and_scratch_limit(monkeypatch):
    """gdn2_chunk_forward_noalloc reports the forward's argument errors, and
    refuses a problem whose split scratch exceeds its static buffer, before
    any HIP call (no GPU needed)."""
    p = _ptrs()
    noalloc = lambda desc, ptrs=p: g.gdn2_chunk_forward_noalloc(desc, *ptrs[:9], 0)
    assert noalloc(None) == g.GDN2_ERR_NULL_POINTER
    assert noalloc(g.make_desc(2, 64, 2, 4, 128, 128, 64, 7)) == g.GDN2_ERR_BAD_DTYPE
    assert noalloc(g.make_desc(2, 64, 2, 4, 96, 128, 64, 1)) == g.GDN2_ERR_UNSUPPORTED
    monkeypatch.setenv("GDN2_PREFILL_SPLIT", "64")
    big = g.make_desc(1, 64 * 64, 32, 32, 128, 128, 64, g.GDN2_BF16)
    assert g.gdn2_chunk_forward_workspace_bytes(big) > g.GDN2_NOALLOC_SCRATCH_BYTES
    assert noalloc(big) == g.GDN2_ERR_SCRATCH
