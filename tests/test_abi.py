"""CPU tests of the C ABI: the library loads, exports every declared symbol, and the
host-only argument checks and tuner selection rule behave as documented."""
import ctypes
import os
import re

import pytest

from gemm_qmm_nbits_amd import qmm as Q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "qmm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert "qmm_nbits" in names and "qmoe_decode_fused" in names and "qmm_codebook4" in names
    L = Q.lib()
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, f"declared in include/qmm.h but not exported: {missing}"


def test_status_strings():
    L = Q.lib()
    for code in range(-10, 1):
        assert L.qmm_status_string(code)


FAKE = 0x1000  # an aligned non-null address, never dereferenced by the validators


def _v_nbits(**kw):
    a = dict(A=FAKE, a_type=Q.QMM_F32, M=1, K=256, N=128, W=FAKE, bits=4, block=64, scales=FAKE,
             zp=FAKE, zp_kind=Q.QMM_ZP_PACKED, bias=None, C=FAKE, c_type=Q.QMM_F32, ws=None, wsb=0)
    a.update(kw)
    return Q.lib().qmm_validate_nbits(a["A"], a["a_type"], a["M"], a["K"], a["N"], a["W"], a["bits"],
                                      a["block"], a["scales"], a["zp"], a["zp_kind"], a["bias"],
                                      a["C"], a["c_type"], a["ws"], a["wsb"])


def test_validate_nbits_codes():
    assert _v_nbits() == 0
    assert _v_nbits(bits=3) == 0                # 3-bit codes, blocks of at least 32
    assert _v_nbits(bits=3, block=16) == -4
    assert _v_nbits(bits=8) == 0                # signed 8-bit codes
    assert _v_nbits(bits=8, block=16) == 0
    for b in (1, 5, 6, 16):
        assert _v_nbits(bits=b) == -3, b
    for b in (8, 48, 96, 512, 0, -64):
        assert _v_nbits(block=b) == -4, b
    for b in (16, 32, 64, 128, 256):
        assert _v_nbits(block=b) == 0
    assert _v_nbits(a_type=7) == -2
    assert _v_nbits(c_type=-1) == -2
    assert _v_nbits(M=-1) == -5
    assert _v_nbits(zp_kind=9) == -8
    assert _v_nbits(zp=None) == -1
    assert _v_nbits(zp=None, zp_kind=Q.QMM_ZP_UNIFORM) == 0
    assert _v_nbits(zp=None, zp_kind=Q.QMM_ZP_NONE) == 0
    assert _v_nbits(W=None) == -1
    assert _v_nbits(C=None) == -1
    assert _v_nbits(A=FAKE + 2) == -6           # fp32 A must be 4-byte aligned
    assert _v_nbits(A=FAKE + 2, a_type=Q.QMM_F16) == 0
    assert _v_nbits(M=0, A=None, W=None, C=None) == 0   # empty problem: nothing to do
    # the prefill path needs its workspace
    need = Q.lib().qmm_nbits_workspace_bytes(2048, 5120, 128, Q.QMM_F32)
    assert need > 0
    assert _v_nbits(M=2048, K=5120) == -7
    assert _v_nbits(M=2048, K=5120, ws=FAKE, wsb=need - 1) == -7
    assert _v_nbits(M=2048, K=5120, ws=FAKE, wsb=need) == 0


def _splits(M, N, kp):
    """The reduction-split rule of the prefill path, restated: least (rounds of 256
    slots x stages per split + partial-sum traffic + 1 launch), smallest count on ties."""
    tiles = -(-M // 256) * -(-N // 256)
    nsteps = kp // 64
    if tiles >= 256:
        return 1
    best, best_cost = 1, float(-(-tiles // 256) * nsteps)
    for s in range(2, min(64, nsteps) + 1):
        cost = -(-tiles * s // 256) * -(-nsteps // s) + s * M * N * 8.0 / 1e7 + 1.0
        if cost < best_cost:
            best, best_cost = s, cost
    return best


@pytest.mark.parametrize("M,K,N", [(16, 4096, 14336), (64, 4096, 1024), (2048, 17920, 5120),
                                   (2048, 5120, 7680), (2048, 5120, 100352), (9, 70, 33),
                                   (8, 4096, 4096), (4, 4096, 14336), (3, 4096, 1024), (4, 4096, 4096),
                                   (4, 4096, 4097), (5, 4096, 1024)])
def test_workspace_sizes(M, K, N):
    """Padded fp16 A, the fp32 row scales of its cast and the fp32 partial sums of a split
    reduction (each from a 256-byte boundary): qmm_nbits from M = 9 on, qmm_codebook4 from
    M = 4 on (its 16-bit outputs take the skinny kernel), except M = 4 on at most 2^24
    codes, which the GEMV keeps."""
    need = Q.lib().qmm_nbits_workspace_bytes(M, K, N, Q.QMM_BF16)
    need_cb = Q.lib().qmm_codebook4_workspace_bytes(M, K, N, Q.QMM_BF16)
    kp = -(-K // 64) * 64
    a16 = -(-M * kp * 2 // 256) * 256
    rs = -(-M * 4 // 256) * 256
    s = _splits(M, N, kp)
    full = a16 + rs + (s * M * N * 4 if s > 1 else 0)
    assert need == (0 if M <= 8 else full)
    assert need_cb == (0 if M < 4 or (M == 4 and N * K <= 1 << 24) else full)


def _v_cb(**kw):
    a = dict(A=FAKE, a_type=Q.QMM_BF16, M=1, K=4096, N=1024, W=FAKE, block=64, absmax=FAKE,
             cb=FAKE, bias=None, C=FAKE, c_type=Q.QMM_BF16, ws=None, wsb=0)
    a.update(kw)
    return Q.lib().qmm_validate_codebook4(a["A"], a["a_type"], a["M"], a["K"], a["N"], a["W"],
                                          a["block"], a["absmax"], a["cb"], a["bias"], a["C"],
                                          a["c_type"], a["ws"], a["wsb"])


def test_validate_codebook_codes():
    assert _v_cb() == 0
    assert _v_cb(block=24) == -4
    assert _v_cb(cb=None) == -1
    assert _v_cb(absmax=FAKE + 2) == -6
    assert _v_cb(a_type=5) == -2
    assert _v_cb(N=-3) == -5
    # 4 <= M <= 8: the workspace is needed for a 16-bit output only, and at M = 4 only
    # above 2^24 codes (the GEMV keeps the smaller shapes)
    assert _v_cb(M=5) == -7
    assert _v_cb(M=4, N=14336) == -7
    assert _v_cb(M=4) == 0
    assert _v_cb(M=4, c_type=Q.QMM_F32, N=14336) == 0
    assert _v_cb(M=4, block=16, N=14336) == 0
    assert _v_cb(M=3) == 0
    need = Q.lib().qmm_codebook4_workspace_bytes(5, 4096, 1024, Q.QMM_BF16)
    assert _v_cb(M=5, ws=FAKE, wsb=need) == 0
    assert _v_cb(M=5, ws=FAKE, wsb=need - 1) == -7
    assert _v_cb(M=5, ws=FAKE + 8, wsb=need) == -6    # the workspace must be 16-byte aligned
    assert _v_cb(M=16, ws=FAKE + 4, wsb=need * 4) == -6


def _v_moe(**kw):
    a = dict(X=FAKE, T=1, H=2880, I=2880, E=32, k=4, ids=FAKE, w=FAKE, bits=4, block=64,
             mode=Q.QMOE_FP, Y=FAKE, scratch=FAKE, sb=None)
    a.update(kw)
    if a["sb"] is None:
        a["sb"] = Q.lib().qmoe_decode_scratch_bytes(a["T"], a["H"], a["I"], a["k"], a["mode"])
    fc = Q.qmoe_weights(FAKE, FAKE, None, None)
    fc1 = kw.get("fc1", fc)
    return Q.lib().qmm_validate_qmoe(a["X"], a["T"], a["H"], a["I"], a["E"], a["k"], a["ids"],
                                     a["w"], fc1, fc, a["bits"], a["block"], a["mode"], a["Y"],
                                     a["scratch"], a["sb"])


def test_validate_qmoe_codes():
    assert _v_moe() == 0
    assert _v_moe(bits=2) == -3
    assert _v_moe(block=16) == -4              # the decode needs block >= 32
    assert _v_moe(block=48) == -4
    assert _v_moe(mode=3) == -8
    assert _v_moe(k=0) == -5
    assert _v_moe(k=33) == -5                  # k <= num_experts
    assert _v_moe(E=0) == -5
    assert _v_moe(T=-1) == -5
    assert _v_moe(ids=None) == -1
    assert _v_moe(fc1=Q.qmoe_weights(None, FAKE, None, None)) == -1
    assert _v_moe(sb=16) == -7
    assert _v_moe(mode=Q.QMOE_INT8_ACT, H=2880, I=2880, block=32) == 0
    assert _v_moe(mode=Q.QMOE_INT8_ACT, H=2890, I=2880, block=32) == -5   # H % 32 != 0
    assert _v_moe(scratch=None) == -7


def test_tuner_selection_rule():
    # 3 rounds x 3 candidates; round 0 is discarded (cold start outlier for candidate 0)
    t = [100.0, 5.0, 6.0,
         1.0, 5.0, 6.0,
         1.0, 5.0, 6.0]
    assert Q.tuner_pick(t, 3, 3) == 0
    # ties go to the lower index
    t = [9.0, 9.0, 9.0,
         4.0, 3.0, 3.0,
         4.0, 3.0, 3.0]
    assert Q.tuner_pick(t, 3, 3) == 1
    # the total decides, not one fast round
    t = [0, 0, 0,
         1.0, 0.1, 2.0,
         1.0, 5.0, 2.0]
    assert Q.tuner_pick(t, 3, 3) == 0
    assert Q.tuner_pick([1.0], 1, 1) == -1


def test_single_launch_preference_rule():
    """MoE decode: candidates 0..n-2 are single-launch forms, n-1 the two-kernel pair;
    the fastest single launch stays unless the pair is more than 5% faster."""
    # 3 rounds (round 0 discarded) x (2 single-launch forms + the pair)
    def times(s0, s1, pair):
        return [50.0, 50.0, 50.0, s0, s1, pair, s0, s1, pair]
    assert Q.tuner_pick_single_launch(times(21.0, 22.0, 20.0), 3, 3) == 0   # 5% slower: single
    assert Q.tuner_pick_single_launch(times(22.0, 21.5, 20.0), 3, 3) == 2   # 7.5% slower: pair
    assert Q.tuner_pick_single_launch(times(19.0, 18.0, 20.0), 3, 3) == 1   # faster: the faster single
    assert Q.tuner_pick_single_launch(times(1e30, 1e30, 20.0), 3, 3) == 2   # no single-launch plan
    assert Q.tuner_pick_single_launch(times(20.0, 20.0, 20.0), 3, 3) == 0   # ties: lower index
    assert Q.tuner_pick_single_launch([1.0, 2.0], 1, 2) == -1
    assert Q.tuner_pick_single_launch([1.0, 2.0], 2, 1) == -1


def test_scratch_queries():
    L = Q.lib()
    assert L.qmm_uniform_scratch_bytes() >= 8
    fp = L.qmoe_decode_scratch_bytes(1, 2880, 2880, 4, Q.QMOE_FP)
    i8 = L.qmoe_decode_scratch_bytes(1, 2880, 2880, 4, Q.QMOE_INT8_ACT)
    a256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    sync = 33 * 256  # the single-launch form's sync slots: top count / flag, 32 sub-counter + phase
    # fp: the sync slots, then h fp16 [T][k][I]
    assert fp == sync + a256(4 * 2880 * 2)
    # int8: sync slots, h, then x codes, x scales, h codes, h scales
    assert i8 == sync + a256(4 * 2880 * 2) + a256(2880) + a256(90 * 4) + a256(4 * 2880) + a256(4 * 90 * 4)
    assert L.qmoe_decode_scratch_bytes(8, 2048, 768, 8, Q.QMOE_FP) == sync + a256(64 * 768 * 2)


def test_decode_status_refusals():
    """Host-side refusals of qmoe_decode_status (no GPU work is reached)."""
    L = Q.lib()
    flag = ctypes.c_int(7)
    assert L.qmoe_decode_status(FAKE, 1 << 20, 1, 2880, 2880, 4, Q.QMOE_FP, None, None) == -1
    assert L.qmoe_decode_status(FAKE, 1 << 20, 1, 2880, 2880, 4, 5, ctypes.byref(flag), None) == -8
    assert L.qmoe_decode_status(None, 1 << 20, 1, 2880, 2880, 4, Q.QMOE_FP, ctypes.byref(flag), None) == -1
    assert L.qmoe_decode_status(FAKE, 16, 1, 2880, 2880, 4, Q.QMOE_FP, ctypes.byref(flag), None) == -7
    assert L.qmoe_decode_status(FAKE + 16, 1 << 20, 1, 2880, 2880, 4, Q.QMOE_FP, ctypes.byref(flag), None) == -6
    # int8 mode has a single-launch form too: the same checks
    assert L.qmoe_decode_status(None, 1 << 20, 1, 2880, 2880, 4, Q.QMOE_INT8_ACT, ctypes.byref(flag), None) == -1
    assert L.qmoe_decode_status(FAKE, 16, 1, 2880, 2880, 4, Q.QMOE_INT8_ACT, ctypes.byref(flag), None) == -7
    # T = 0: nothing ran, 0 without touching the buffer
    assert L.qmoe_decode_status(None, 0, 0, 2880, 2880, 4, Q.QMOE_INT8_ACT, ctypes.byref(flag), None) == 0
    assert flag.value == 0


def test_hbm_read_probe_refusals():
    """Host-side refusals of the streaming-read measurement helper."""
    L = Q.lib()
    assert L.qmm_hbm_read_probe(FAKE, 100, FAKE, 16, None) == -5      # not a multiple of 16
    assert L.qmm_hbm_read_probe(FAKE, 1 << 20, FAKE, 0, None) == -5
    assert L.qmm_hbm_read_probe(FAKE, 1 << 20, FAKE, (1 << 20) + 1, None) == -5
    assert L.qmm_hbm_read_probe(None, 1 << 20, FAKE, 16, None) == -1
    assert L.qmm_hbm_read_probe(FAKE + 8, 1 << 20, FAKE, 16, None) == -6
    assert L.qmm_hbm_read_probe(None, 0, None, 16, None) == 0


def test_launch_timing_host_paths():
    """Launch timing: refusals and the switched-off end (no GPU work)."""
    L = Q.lib()
    count = ctypes.c_int(5)
    assert L.qmm_launch_timing_end(None, 0, ctypes.byref(count)) == 0 and count.value == 0
    assert L.qmm_launch_timing_end(None, 0, None) == -1
    assert L.qmm_launch_timing_begin(0) == -5
    assert L.qmm_launch_timing_begin(65537) == -5


def test_matrix_core_form_rule():
    """Shapes the form serves and shapes it leaves to the v_dot8 kernel."""
    assert Q.nbits_gemv_matrix_core_form(1, 5120, 100352, 2, 64)
    assert Q.nbits_gemv_matrix_core_form(1, 5120, 35840, 2, 64)
    assert not Q.nbits_gemv_matrix_core_form(2, 5120, 100352, 2, 64)    # M = 2
    assert not Q.nbits_gemv_matrix_core_form(1, 5120, 100352, 4, 64)    # 4-bit
    assert not Q.nbits_gemv_matrix_core_form(1, 5120, 100352, 2, 32)    # two groups per chunk
    assert not Q.nbits_gemv_matrix_core_form(1, 5120, 7680, 2, 64)      # 32 lanes, 20 pairs
    assert not Q.nbits_gemv_matrix_core_form(1, 5120, 100352, 2, 128)   # block 128
    assert not Q.nbits_gemv_matrix_core_form(1, 5056, 100352, 2, 64)    # 79 blocks per row
    assert not Q.nbits_gemv_matrix_core_form(1, 17920, 5120, 2, 64)     # operand past LDS
    assert not Q.nbits_gemv_matrix_core_form(1, 4096, 100352, 2, 64)    # 64 lanes per row
    for args in ((1, 0, 100352, 2, 64), (1, 5120, 0, 2, 64), (1, -5120, 100352, 2, 64),
                 (1, 5120, 100352, 2, 48), (1, 5120, 100352, 2, 0), (0, 5120, 100352, 2, 64)):
        assert not Q.nbits_gemv_matrix_core_form(*args), args
