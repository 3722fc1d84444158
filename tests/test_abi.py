"""The C ABI library loads, exports what include/msr.h declares, and rejects
bad arguments with status codes before launching anything (CPU only: every
call here fails validation, so no GPU is touched)."""
import ctypes
import os
import re

import numpy as np
import pytest

import linear_recurrence_sequence_amd as msr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msr.h")

pytestmark = pytest.mark.skipif(not os.path.exists(msr.library_path()),
                                reason="libmsr.so not built (python -m linear_recurrence_sequence_amd.build)")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msr_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(msr.EXPORTS)


def test_every_declared_symbol_is_exported():
    L = ctypes.CDLL(msr.library_path())
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings():
    names = [msr.msr_status_str(i) for i in range(7)]
    assert names == ["MSR_OK", "MSR_ERR_NULL", "MSR_ERR_SHAPE", "MSR_ERR_DTYPE", "MSR_ERR_UNSUPPORTED",
                     "MSR_ERR_WORKSPACE", "MSR_ERR_HIP"]
    # any int32 is a value of the enum: out-of-range codes are named, not undefined
    assert msr.msr_status_str(99) == msr.msr_status_str(-2 ** 31) == "MSR_ERR_UNKNOWN"


def _gamma(n):
    g = np.full(n, 0.9)
    return g, g.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _chunkwise(dtype=0, dims=(1, 64, 2, 64, 64), chunk=32, gamma=True, ws=(FAKE, 1 << 40), Q=FAKE,
               S_in=None, S_out=None, gam=None):
    L = msr.lib()
    g, gp = _gamma(dims[2]) if gam is None else gam
    return L.msr_chunkwise_fwd(dtype, msr.MsrDims(*dims), chunk, gp if gamma else None, 10000.0, 0, 1.0, Q, FAKE,
                               FAKE, S_in, S_out, FAKE, ws[0], ws[1], None)


def test_chunkwise_validation():
    assert _chunkwise(dtype=7) == 3                               # dtype
    assert _chunkwise(dtype=-1) == 3
    assert _chunkwise(dtype=2 ** 31 - 1) == 3
    assert _chunkwise(dims=(1, 64, 2, 64, 96)) == 4               # unsupported head dims
    assert _chunkwise(dims=(1, 64, 2, 48, 48)) == 4
    assert _chunkwise(dims=(-1, 64, 2, 64, 64)) == 2              # negative size
    assert _chunkwise(dims=(1, 64, 0, 64, 64)) == 2               # no heads
    assert _chunkwise(dims=(1, 64, 129, 64, 64)) == 4             # too many heads
    assert _chunkwise(chunk=0) == 2
    assert _chunkwise(chunk=48) == 4                              # not a multiple of 32
    assert _chunkwise(chunk=8192) == 4                            # above 4096
    assert _chunkwise(gamma=False) == 1                           # gamma NULL
    assert _chunkwise(Q=None) == 1
    assert _chunkwise(ws=(None, 0)) == 5                          # workspace missing
    assert _chunkwise(ws=(FAKE, 16)) == 5                         # workspace too small
    assert _chunkwise(S_in=FAKE, S_out=FAKE) == 2                 # S_out aliases S_in
    g = np.array([0.5, 1.5])
    assert _chunkwise(gam=(g, g.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))) == 2   # gamma > 1
    g = np.array([0.5, np.nan])
    assert _chunkwise(gam=(g, g.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))) == 2
    assert "multiple of 32" in _last(lambda: _chunkwise(chunk=40))


def _last(fn):
    fn()
    return msr.msr_last_error()


def test_other_entry_points_validation():
    L = msr.lib()
    g, gp = _gamma(4)
    d = msr.MsrDims(1, 16, 4, 64, 64)
    assert L.msr_parallel_fwd(0, d, gp, 0.0, -1, 1.0, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 2      # pos0 < 0
    assert L.msr_parallel_fwd(0, d, gp, 0.0, 0, 1.0, None, FAKE, FAKE, FAKE, None, 0, None) == 1
    assert L.msr_parallel_fwd(0, d, gp, 100.0, 0, 1.0, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 5     # rotation needs ws
    assert L.msr_recurrent_step(0, 2, 4, 64, 64, gp, 0.0, 0, 1.0, FAKE, FAKE, FAKE, None, FAKE, None) == 1
    assert L.msr_recurrent_step(0, 2, 4, 32, 32, gp, 0.0, 0, 1.0, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 4
    assert L.msr_recurrent_step(0, 2, 4, 64, 64, gp, 0.0, -3, 1.0, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 2
    lay = lambda dm, chunk=64, ws=1 << 40, eps=1e-5: L.msr_layer_fwd(
        1, 1, 128, dm, 4, 64, 64, chunk, gp, 10000.0, eps, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None)
    assert lay(100) == 4                    # d_model not a multiple of 64
    assert lay(256, chunk=-32) == 2
    assert lay(256, ws=10) == 5
    assert lay(256, eps=-1.0) == 2
    dec = lambda dm=256, dk=64, pos=5, S=FAKE, ws=1 << 40, eps=1e-5, dtype=1: L.msr_layer_decode_step(
        dtype, 2, dm, 4, dk, dk, gp, 10000.0, eps, pos, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, S, FAKE, FAKE, ws, None)
    assert dec(dm=100) == 4                 # d_model not a multiple of 64
    assert dec(dk=96) == 4                  # unsupported head dims
    assert dec(pos=-1) == 2
    assert dec(S=None) == 1
    assert dec(ws=10) == 5
    assert dec(eps=-1.0) == 2
    assert dec(dtype=5) == 3
    assert "multiple of 64" in _last(lambda: dec(dm=96))
    blk = lambda dm=256, F=512, W1=FAKE, ws=1 << 40, ln=1e-5: L.msr_retnet_block_fwd(
        1, 1, 128, dm, 4, 64, 64, 64, F, gp, 10000.0, 1e-5, ln, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, W1, FAKE, FAKE,
        FAKE, ws, None)
    assert blk(F=100) == 4                  # d_ffn not a multiple of 64
    assert blk(dm=16384) == 4               # d_model above 8192
    assert blk(W1=None) == 1
    assert blk(ln=-1.0) == 2
    assert blk(ws=10) == 5
    assert blk(F=0) == 2


def test_backward_validation():
    L = msr.lib()
    g, gp = _gamma(2)
    bwd = lambda dims=(1, 64, 2, 64, 64), chunk=32, gam=gp, scale=1.0, dQ=FAKE, S_in=None, dS_out=None, dS_in=None, \
        ws=1 << 40, dtype=1: L.msr_chunkwise_bwd(dtype, msr.MsrDims(*dims), chunk, gam, 0.0, 0, scale, FAKE, FAKE,
                                                FAKE, FAKE, S_in, dS_out, dQ, FAKE, FAKE, dS_in, FAKE, ws, None)
    assert bwd(dims=(1, 64, 2, 256, 512)) == 4                   # d_k != d_v
    assert "d_k == d_v" in msr.msr_last_error()
    assert bwd(dims=(1, 64, 2, 48, 48)) == 4
    assert bwd(chunk=40) == 4
    assert bwd(dtype=3) == 3
    assert bwd(dQ=None) == 1
    assert bwd(ws=16) == 5
    assert bwd(S_in=FAKE, dS_in=FAKE) == 2                      # dS_in aliases S_in
    z = np.array([0.9, 0.0])
    zp = z.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    assert bwd(gam=zp, dS_out=FAKE) == 4                         # dS_out seeds divide by gamma
    assert bwd(scale=0.0, dS_out=FAKE) == 4
    assert bwd(dims=(0, 64, 2, 64, 64), gam=zp, dS_out=FAKE) == 0   # nothing to do
    assert bwd(dims=(2, 64, 2, 64, 64), gam=zp, ws=16) == 5     # gamma = 0 is fine without dS_out


def test_saved_state_entry_points_validation():
    """The forward that keeps its per-chunk states and the backward that
    reads them need R_chunks when there are tokens, and otherwise validate
    like msr_chunkwise_fwd / msr_chunkwise_bwd."""
    L = msr.lib()
    g, gp = _gamma(2)
    fwd = lambda dims=(1, 64, 2, 64, 64), R=FAKE, dtype=1, ws=1 << 40: L.msr_chunkwise_fwd_save(
        dtype, msr.MsrDims(*dims), 32, gp, 0.0, 0, 1.0, FAKE, FAKE, FAKE, None, None, R, FAKE, FAKE, ws, None)
    assert fwd(R=None) == 1 and "R_chunks" in msr.msr_last_error()
    assert fwd(dims=(0, 64, 2, 64, 64), R=None) == 0              # no tokens: nothing to keep
    assert fwd(dtype=3) == 3
    assert fwd(ws=16) == 5
    bwd = lambda dims=(1, 64, 2, 64, 64), R=FAKE, dtype=1, ws=1 << 40: L.msr_chunkwise_bwd_saved(
        dtype, msr.MsrDims(*dims), 32, gp, 0.0, 0, 1.0, FAKE, FAKE, FAKE, FAKE, None, None, R, FAKE, FAKE, FAKE,
        None, FAKE, ws, None)
    assert bwd(R=None) == 1 and "R_chunks" in msr.msr_last_error()
    assert bwd(dims=(1, 64, 2, 256, 512)) == 4                   # d_k != d_v
    assert bwd(ws=16) == 5


def test_rglru_validation():
    L = msr.lib()
    rg = lambda B=2, T=16, D=128, c=8.0, X=FAKE, lam=FAKE, h0=None, hT=None, ws=1 << 40, dtype=1: L.msr_rglru_fwd(
        dtype, B, T, D, c, X, FAKE, FAKE, FAKE, FAKE, lam, h0, hT, FAKE, FAKE, ws, None)
    assert rg(D=100) == 4                   # width not a multiple of 64
    assert rg(D=0) == 2
    assert rg(T=-1) == 2
    assert rg(c=0.0) == 2
    assert rg(c=float("inf")) == 2
    assert rg(X=None) == 1
    assert rg(lam=None) == 1
    assert rg(ws=10) == 5
    assert rg(h0=FAKE, hT=FAKE) == 2        # h_last aliases h0
    assert rg(dtype=9) == 3
    assert rg(B=0) == 0
    assert msr.msr_rglru_workspace_bytes(1, 2, 16, 128) == 2 * 16 * 256 * 2
    assert msr.msr_rglru_workspace_bytes(0, 3, 5, 64) == -(-3 * 5 * 128 * 4 // 256) * 256


def test_empty_inputs_are_no_ops():
    """batch = 0 or seqlen = 0 (parallel / layer) returns OK without touching memory."""
    L = msr.lib()
    g, gp = _gamma(2)
    assert L.msr_parallel_fwd(0, msr.MsrDims(0, 16, 2, 64, 64), gp, 0.0, 0, 1.0, None, None, None, None, None, 0,
                              None) == 0
    assert L.msr_parallel_fwd(1, msr.MsrDims(3, 0, 2, 64, 64), gp, 0.0, 0, 1.0, None, None, None, None, None, 0,
                              None) == 0
    assert L.msr_chunkwise_fwd(0, msr.MsrDims(0, 16, 2, 64, 64), 32, gp, 0.0, 0, 1.0, None, None, None, None, None,
                               None, None, 0, None) == 0
    assert L.msr_recurrent_step(0, 0, 2, 64, 64, gp, 0.0, 0, 1.0, None, None, None, None, None, None) == 0
    assert L.msr_layer_fwd(1, 2, 0, 256, 2, 64, 64, 32, gp, 1.0, 1e-5, None, None, None, None, None, None, None, None,
                           0, None) == 0
    assert msr.msr_last_error() == ""


def test_workspace_sizes():
    # chunkwise: one [B, H, NC, dk, dv] buffer of the element type (each chunk's state
    # contribution, overwritten in place by R_{i-1}); rotation adds Q, K copies and a table
    B, N, H, dk, dv, C = 2, 1000, 3, 128, 128, 256
    nc = -(-N // C)
    st = B * H * nc * dk * dv
    up = lambda x: -(-x // 256) * 256
    assert msr.msr_chunkwise_workspace_bytes(1, B, N, H, dk, dv, C, 0.0) == up(st * 2)
    assert msr.msr_chunkwise_workspace_bytes(0, B, N, H, dk, dv, C, 0.0) == up(st * 4)
    rot = 2 * up(B * N * H * dk * 2) + up(N * dk // 2 * 8)
    assert msr.msr_chunkwise_workspace_bytes(1, B, N, H, dk, dv, C, 1e4) == rot + up(st * 2)
    assert msr.msr_parallel_workspace_bytes(1, B, N, H, dk, dv, 0.0) == 0
    assert msr.msr_layer_workspace_bytes(1, 2, 64, 256, 2, 64, 64, 32) > 0
    assert msr.msr_layer_workspace_bytes(1, 2, 64, 256, 2, 64, 64, 0) == 0
    # layer decode step: [q|k|v|g] rows (element type), float32 outputs, Z (element type), and
    # float32 split-K partials of the projections (at most 8 slices of the larger product)
    Bd, Hd, kd, vd, dm = 5, 3, 256, 512, 256
    base = up(Bd * Hd * (2 * kd + 2 * vd) * 2) + up(Bd * Hd * vd * 4) + up(Bd * Hd * vd * 2)
    got = msr.msr_layer_decode_workspace_bytes(1, Bd, dm, Hd, kd, vd)
    assert base <= got <= base + up(8 * Bd * max(Hd * (2 * kd + 2 * vd), dm) * 4)
    assert msr.msr_layer_decode_workspace_bytes(1, 0, dm, Hd, kd, vd) == 0
    assert msr.msr_layer_decode_workspace_bytes(1, Bd, 100, Hd, kd, vd) == 0
    # backward: the chunk workspace (with the rotated copies) and two state seeds (its reversed
    # passes read their inputs backwards in place)
    cw = msr.msr_chunkwise_workspace_bytes(1, B, N, H, dk, dv, C, 1e4)
    assert msr.msr_chunkwise_bwd_workspace_bytes(1, B, N, H, dk, dv, C, 1e4) == (
        up(cw) + 2 * up(B * H * dk * dv * 4))
    # RetNet block: the layer's workspace, then LN(X) / LN(Y), Y and the hidden rows
    Bb, Nb, dmb, Hb, db, Cb, Fb = 2, 64, 256, 2, 64, 32, 512
    lay = msr.msr_layer_workspace_bytes(1, Bb, Nb, dmb, Hb, db, db, Cb)
    assert msr.msr_retnet_block_workspace_bytes(1, Bb, Nb, dmb, Hb, db, db, Cb, Fb) == (
        up(lay) + 2 * up(Bb * Nb * dmb * 2) + up(Bb * Nb * Fb * 2))


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(msr, "_lib", None)
    monkeypatch.setattr(msr, "library_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(msr.MsrLibraryMissing):
        msr.lib()


def test_binding_rejects_wrong_tensors_before_the_call():
    """The binding checks dtype, shape and device of every tensor it is
    given before any pointer reaches the library (CPU tensors here: the
    checks run first, so no GPU is touched, and a correct set of shapes
    gets as far as the device check)."""
    import torch
    B, N, H, d, C = 1, 64, 2, 64, 32
    bf = torch.bfloat16
    Q, K, V = (torch.zeros((B, N, H, d), dtype=bf) for _ in range(3))
    g = np.full(H, 0.9)
    bad = [
        (dict(S_in=torch.zeros((B, H, d, d), dtype=bf)), "S_in must be torch.float32"),
        (dict(S_out=torch.zeros((B, H, d, d + 1))), "S_out must have shape"),
        (dict(O=torch.zeros((B, N, H, d), dtype=torch.float32)), "O must be torch.bfloat16"),
    ]
    for kw, msg in bad:
        with pytest.raises(ValueError, match=msg):
            msr.msr_chunkwise_fwd(Q, K, V, g, C, **kw)
    with pytest.raises(ValueError, match="K must have shape"):
        msr.msr_chunkwise_fwd(Q, K[:, :32], V, g, C)
    with pytest.raises(ValueError, match="V must be torch.bfloat16"):
        msr.msr_parallel_fwd(Q, K, V.float(), g)
    with pytest.raises(ValueError, match="R_chunks must have shape"):
        msr.msr_chunkwise_fwd_save(Q, K, V, g, C, torch.zeros((B, H, 3, d, d), dtype=bf))
    with pytest.raises(ValueError, match="R_chunks must be torch.bfloat16"):
        msr.msr_chunkwise_fwd_save(Q, K, V, g, C, torch.zeros(msr.msr_chunkwise_states_shape(B, N, H, d, d, C)))
    with pytest.raises(ValueError, match="dS_out must be torch.float32"):
        msr.msr_chunkwise_bwd(Q, K, V, Q, g, C, dS_out=torch.zeros((B, H, d, d), dtype=bf))
    with pytest.raises(ValueError, match="dV must have shape"):
        msr.msr_chunkwise_bwd(Q, K, V, Q, g, C, dV=torch.zeros((B, N, H, 2 * d), dtype=bf))
    q1 = torch.zeros((B, H, d), dtype=bf)
    with pytest.raises(ValueError, match="S must be torch.float32"):
        msr.msr_recurrent_step(q1, q1, q1, torch.zeros((B, H, d, d), dtype=bf), g, pos=0)
    with pytest.raises(ValueError, match="S must have shape"):
        msr.msr_recurrent_step(q1, q1, q1, torch.zeros((B, H, d, 2 * d)), g, pos=0)
    dm = 192
    X = torch.zeros((B, N, dm), dtype=bf)
    W = [torch.zeros(s, dtype=bf) for s in ((dm, H * d),) * 4 + ((H * d, dm),)]
    with pytest.raises(ValueError, match="W_O must have shape"):
        msr.msr_layer_fwd(X, *W[:4], W[0], g, H, d, d, C)
    with pytest.raises(ValueError, match="W_G must be torch.bfloat16"):
        msr.msr_layer_fwd(X, *W[:3], W[3].float(), W[4], g, H, d, d, C)
    with pytest.raises(ValueError, match="S must have shape"):
        msr.msr_layer_decode_step(X[:, 0], *W, torch.zeros((B, H, d, d + 2)), g, H, d, d, 0)
    with pytest.raises(ValueError, match="Lambda must be torch.float32"):
        Wsq = torch.zeros((dm, dm), dtype=bf)
        msr.msr_rglru_fwd(X, Wsq, torch.zeros(dm), Wsq, torch.zeros(dm), torch.zeros(dm, dtype=bf))
    # shapes and dtypes right: the next check is the device
    with pytest.raises(ValueError, match="on the GPU"):
        msr.msr_chunkwise_fwd(Q, K, V, g, C, S_out=torch.zeros((B, H, d, d)))


def test_noalloc_decode_step_limits():
    """The allocation-free decode step rejects, before anything reaches the
    GPU, a step whose workspace exceeds its static scratch, and validates
    like msr_layer_decode_step."""
    L = msr.lib()
    cap = msr.msr_layer_decode_noalloc_max_bytes()
    assert cap == 64 << 20
    g, gp = _gamma(16)
    big = (1, 256, 4096, 16, 256, 256)            # batch 256 at d_model 4096: 78 MiB
    assert msr.msr_layer_decode_workspace_bytes(*big) > cap
    assert msr.msr_layer_decode_workspace_bytes(1, 128, 4096, 16, 256, 256) <= cap
    call = lambda dtype, B, dm, H, dk, dv, pos=0: L.msr_layer_decode_step_noalloc(
        dtype, B, dm, H, dk, dv, gp, 1e4, 1e-5, pos, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert call(*big) == 5                                        # MSR_ERR_WORKSPACE
    assert "static scratch" in msr.msr_last_error()
    assert call(7, 2, 256, 16, 256, 256) == 3                     # dtype
    assert call(1, 2, 100, 16, 256, 256) == 4                     # d_model not a multiple of 64
    assert call(1, 2, 256, 16, 256, 96) == 4                      # head dims
    assert call(1, 2, 256, 16, 256, 256, pos=-1) == 2             # position
    assert call(1, 0, 256, 16, 256, 256) == 0                     # empty batch: nothing to do
    assert L.msr_layer_decode_step_noalloc(1, 2, 256, 16, 256, 256, gp, 1e4, 1e-5, 0, None, FAKE, FAKE, FAKE,
                                           FAKE, FAKE, FAKE, FAKE, None) == 1
