"""C-ABI checks that need no GPU: the library loads, exports every function
include/sconv.h declares, and rejects bad host arguments with the documented
status codes before touching the GPU (so nothing here launches a kernel)."""
import ctypes
import os
import re
import subprocess

import pytest

import causal_depthwise_short_conv1d_amd as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sconv.h")

OK, ENULL, ESHAPE, ESTRIDE, EWIDTH, EALIAS, EALIGN, EARG, ELAUNCH = 0, -1, -2, -3, -4, -5, -6, -7, -8

# fake, well-aligned, non-overlapping "device" addresses: validation only
# compares them, it never dereferences them.
BASE = 0x7F0000000000
GB = 1 << 30


def addr(i):
    return ctypes.c_void_p(BASE + i * GB)


def no_gpu():
    """The validation calls below pass fake addresses.  Where a GPU is
    visible, a check that wrongly let one through would launch a kernel on
    them, so those tests only run where no GPU is."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("fake-address validation runs only where no GPU is visible")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(S.library_path()):
        pytest.fail("libsconv.so is not built (run python -m causal_depthwise_short_conv1d_amd.build)")
    return S.load_library()


def test_header_declares_the_entry_points():
    fns = declared_functions()
    for name in ("conv1d_fwd_varlen", "conv1d_update_decode", "conv1d_update",
                 "sconv_paged_fused", "sconv_paged_fused_multi", "sconv_seq_metadata",
                 "sconv_status_string",
                 "sconv_version"):
        assert name in fns
    assert sorted(S.exported_symbols()) == fns


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", S.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(declared_functions()) <= exported


def test_version_and_strings(lib):
    assert S.version() == (1, 4)
    for code in range(-8, 1):
        assert S.status_string(code) != "unknown status"
    assert S.status_string(-99) == "unknown status"


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(FileNotFoundError):
        S.load_library(str(tmp_path / "nope.so"))


# ------------------------------------------------------------------ fwd --

def fwd(lib, **kw):
    no_gpu()
    a = dict(x=addr(1), xsd=1, xst=64, w=addr(2), wsd=4, b=addr(3), cs=addr(4), csl=192,
             csd=3, cst=1, lines=4, ci=addr(5), hi=addr(6), qsl=addr(7), batch=2, T=10,
             dim=64, width=4, act=1, pad=-1, out=addr(8), osd=1, ost=64)
    a.update(kw)
    return lib.conv1d_fwd_varlen(a["x"], a["xsd"], a["xst"], a["w"], a["wsd"], a["b"], a["cs"],
                                 a["csl"], a["csd"], a["cst"], a["lines"], a["ci"], a["hi"],
                                 a["qsl"], a["batch"], a["T"], a["dim"], a["width"], a["act"],
                                 a["pad"], a["out"], a["osd"], a["ost"], None)


@pytest.mark.parametrize("width", [0, 1, 6, 9])
def test_fwd_width(lib, width):
    assert fwd(lib, width=width) == EWIDTH


def test_fwd_bad_enums_and_sizes(lib):
    assert fwd(lib, act=2) == EARG
    assert fwd(lib, batch=-1) == ESHAPE
    assert fwd(lib, T=-3) == ESHAPE
    assert fwd(lib, T=1 << 31) == ESHAPE
    assert fwd(lib, dim=-1) == ESHAPE


def test_fwd_empty_is_a_noop(lib):
    # returns before any pointer is looked at or any kernel launched
    assert fwd(lib, T=0, x=None, out=None) == OK
    assert fwd(lib, batch=0, x=None) == OK
    assert fwd(lib, dim=0, x=None) == OK


def test_fwd_nulls(lib):
    for k in ("x", "w", "qsl", "out"):
        assert fwd(lib, **{k: None}) == ENULL, k
    assert fwd(lib, cs=None) == ENULL          # has_initial_state needs conv_states


def test_fwd_strides_and_layouts(lib):
    # Any non-negative strides are accepted; layouts outside the vector
    # kernels' storage classes take the general-stride kernel.  Here no GPU
    # is visible, so an accepted call reaches the launch and fails there.
    assert fwd(lib, wsd=3) == ELAUNCH          # overlapping weight rows: read-only, fine
    assert fwd(lib, wsd=0) == ELAUNCH          # one set of taps broadcast to every channel
    assert fwd(lib, xst=2, xsd=2) == ELAUNCH   # x elements shared between (c, t): read-only
    assert fwd(lib, xst=60) == ELAUNCH         # overlapping input rows
    assert fwd(lib, xst=68) == ELAUNCH         # row pitch not a multiple of 8
    assert fwd(lib, osd=10, ost=1) == ELAUNCH  # out token-contiguous, x channel-contiguous
    assert fwd(lib, xsd=-1) == ESTRIDE
    assert fwd(lib, wsd=-4) == ESTRIDE
    assert fwd(lib, osd=1, ost=5) == ESTRIDE   # out rows overlap: two outputs, one address
    assert fwd(lib, osd=0) == ESTRIDE          # every channel's output at one address
    assert fwd(lib, csl=0) == ESTRIDE          # four state lines at one address
    assert fwd(lib, csd=1, cst=1) == ESTRIDE   # state columns overlap the next channel's


def test_fwd_state_shape(lib):
    assert fwd(lib, ci=None, lines=1) == ESHAPE   # line = sequence id needs >= batch lines
    assert fwd(lib, lines=0) == ESHAPE


def test_fwd_alignment(lib):
    # bf16 tensors need 2-byte, index arrays 4-byte alignment; nothing more
    assert fwd(lib, x=ctypes.c_void_p(BASE + GB + 8)) == ELAUNCH
    assert fwd(lib, out=ctypes.c_void_p(BASE + 8 * GB + 2)) == ELAUNCH
    assert fwd(lib, x=ctypes.c_void_p(BASE + GB + 1)) == EALIGN
    assert fwd(lib, out=ctypes.c_void_p(BASE + 8 * GB + 3)) == EALIGN
    assert fwd(lib, w=ctypes.c_void_p(BASE + 2 * GB + 1)) == EALIGN
    assert fwd(lib, cs=ctypes.c_void_p(BASE + 4 * GB + 1)) == EALIGN
    assert fwd(lib, qsl=ctypes.c_void_p(BASE + 7 * GB + 2)) == EALIGN
    assert fwd(lib, ci=ctypes.c_void_p(BASE + 5 * GB + 2)) == EALIGN


def test_fwd_aliasing(lib):
    assert fwd(lib, out=addr(1)) == EALIAS                               # out is x
    assert fwd(lib, out=ctypes.c_void_p(BASE + GB + 512)) == EALIAS      # partial overlap
    assert fwd(lib, cs=ctypes.c_void_p(BASE + 8 * GB + 16)) == EALIAS   # state inside out
    assert fwd(lib, cs=ctypes.c_void_p(BASE + GB)) == EALIAS             # state inside x


# --------------------------------------------------------------- decode --

def upd(lib, **kw):
    no_gpu()
    a = dict(x=addr(1), xsb=64, xsd=1, xst=64, w=addr(2), wsd=4, b=addr(3), cs=addr(4),
             csl=192, csd=3, cst=1, lines=4, ci=addr(5), batch=2, dim=64, seqlen=1,
             width=4, act=1, pad=-1, out=addr(8), osb=64, osd=1, ost=64)
    a.update(kw)
    return lib.conv1d_update_decode(a["x"], a["xsb"], a["xsd"], a["xst"], a["w"], a["wsd"],
                                    a["b"], a["cs"], a["csl"], a["csd"], a["cst"], a["lines"],
                                    a["ci"], a["batch"], a["dim"], a["seqlen"], a["width"],
                                    a["act"], a["pad"], a["out"], a["osb"], a["osd"], a["ost"],
                                    None)


def test_decode_validation(lib):
    assert upd(lib, width=1) == EWIDTH
    assert upd(lib, act=-1) == EARG
    assert upd(lib, seqlen=0, x=None) == OK
    assert upd(lib, batch=0, x=None) == OK
    assert upd(lib, cs=None) == ENULL
    assert upd(lib, ci=None, lines=1) == ESHAPE
    assert upd(lib, wsd=2) == ELAUNCH                                    # any weight stride
    assert upd(lib, wsd=-1) == ESTRIDE
    assert upd(lib, osd=0) == ESTRIDE                                    # outputs coincide
    assert upd(lib, csl=2) == ESTRIDE                                    # state lines overlap
    assert upd(lib, out=ctypes.c_void_p(BASE + GB + 2)) == EALIAS        # partial overlap
    assert upd(lib, out=addr(1), osd=2, osb=128) == EALIAS               # same base, other strides
    assert upd(lib, cs=ctypes.c_void_p(BASE + GB + 4)) == EALIAS
    assert upd(lib, x=ctypes.c_void_p(BASE + GB + 1)) == EALIGN


def updx(lib, **kw):
    no_gpu()
    a = dict(x=addr(1), xsb=64 * 4, xsd=1, xst=64, w=addr(2), wsd=4, b=addr(3), cs=addr(4),
             csl=64 * 6, csd=1, cst=64, lines=16, L=6, ci=addr(5), ring=None, nacc=addr(6),
             it=None, isb=0, ist=0, isd=0, isk=0, osi=None, osb_=0, ost_=0, batch=2, dim=64,
             seqlen=4, width=4, act=1, pad=-1, out=addr(8), osb=64 * 4, osd=1, ost=64)
    a.update(kw)
    return lib.conv1d_update(a["x"], a["xsb"], a["xsd"], a["xst"], a["w"], a["wsd"], a["b"],
                             a["cs"], a["csl"], a["csd"], a["cst"], a["lines"], a["L"], a["ci"],
                             a["ring"], a["nacc"], a["it"], a["isb"], a["ist"], a["isd"],
                             a["isk"], a["osi"], a["osb_"], a["ost_"], a["batch"], a["dim"],
                             a["seqlen"], a["width"], a["act"], a["pad"], a["out"], a["osb"],
                             a["osd"], a["ost"], None)


def test_update_options_validation(lib):
    inter = dict(it=addr(9), isb=4 * 64 * 3, ist=64 * 3, isd=3, isk=1)
    assert updx(lib, width=6) == EWIDTH
    assert updx(lib, ring=addr(7)) == EARG                 # ring with speculative options
    assert updx(lib, ring=addr(7), nacc=None, osi=addr(10)) == EARG
    assert updx(lib, ring=addr(7), nacc=None, **inter) == EARG
    # accepted combinations, checked with batch 0 so that nothing is launched
    assert updx(lib, ring=addr(7), nacc=None, L=3, batch=0) == OK
    assert updx(lib, L=2) == ESHAPE                        # shorter than width-1
    assert updx(lib, L=5) == ESHAPE                        # roll needs width-2+seqlen
    assert updx(lib, L=3, osi=addr(10), osb_=4, ost_=1, batch=0) == OK   # saved windows: no roll
    assert updx(lib, L=3, batch=0, **inter) == OK
    assert updx(lib, L=5, batch=0) == ESHAPE
    assert updx(lib, seqlen=0, x=None) == OK
    assert updx(lib, cs=None) == ENULL
    assert updx(lib, isd=-1, **{k: v for k, v in inter.items() if k != "isd"}) == ESTRIDE
    assert updx(lib, nacc=ctypes.c_void_p(BASE + 6 * GB + 2)) == EALIGN
    assert updx(lib, osi=ctypes.c_void_p(BASE + 10 * GB + 2)) == EALIGN
    assert updx(lib, it=ctypes.c_void_p(BASE + 1 * GB + 64), isb=768, ist=192, isd=3,
                isk=1) == EALIAS                          # windows inside x
    assert updx(lib, it=ctypes.c_void_p(BASE + 4 * GB), isb=768, ist=192, isd=3,
                isk=1) == EALIAS                          # windows inside the state


# ---------------------------------------------------------------- paged --

def paged(lib, **kw):
    no_gpu()
    a = dict(x=addr(1), xst=4096, w=addr(2), wsd=4, b=None, c=addr(3), csb=32 * 16 * 512,
             csh=16 * 512, csn=512, nb=64, H=32, N=16, D=512, off=128, ws=128, pos=addr(4),
             slot=addr(5), qsl=addr(6), R=3, bt=addr(7), btsr=64, mb=64, T=100, width=4,
             act=1, res=1, out=addr(8), ost=4096)
    a.update(kw)
    return lib.sconv_paged_fused(a["x"], a["xst"], a["w"], a["wsd"], a["b"], a["c"], a["csb"],
                                 a["csh"], a["csn"], a["nb"], a["H"], a["N"], a["D"], a["off"],
                                 a["ws"], a["pos"], a["slot"], a["qsl"], a["R"], a["bt"],
                                 a["btsr"], a["mb"], a["T"], a["width"], a["act"], a["res"],
                                 a["out"], a["ost"], None)


def test_paged_validation(lib):
    assert paged(lib, width=6) == EWIDTH
    assert paged(lib, res=2) == EARG
    assert paged(lib, T=0, x=None) == OK
    assert paged(lib, off=400) == ESHAPE          # stream past head_dim
    assert paged(lib, H=0) == ESHAPE
    assert paged(lib, bt=None) == ENULL
    assert paged(lib, slot=None) == ENULL
    assert paged(lib, ost=4000) == ESTRIDE        # output rows overlap
    assert paged(lib, csn=500) == ESTRIDE         # slots overlap inside a head
    assert paged(lib, csb=-1) == ESTRIDE
    assert paged(lib, x=ctypes.c_void_p(BASE + GB + 1)) == EALIGN
    assert paged(lib, pos=ctypes.c_void_p(BASE + 4 * GB + 4)) == EALIGN
    assert paged(lib, bt=ctypes.c_void_p(BASE + 7 * GB + 2)) == EALIGN
    # accepted (the general-stride kernel where the vector one does not fit):
    # here no GPU is visible, so they fail at the launch
    assert paged(lib, xst=4000) == ELAUNCH        # overlapping input rows: read-only
    assert paged(lib, ws=100, xst=3200, ost=3200) == ELAUNCH   # ws not a multiple of 8
    assert paged(lib, off=4) == ELAUNCH
    assert paged(lib, csn=520, csh=16 * 520, csb=32 * 16 * 520) == ELAUNCH
    assert paged(lib, x=ctypes.c_void_p(BASE + GB + 8)) == ELAUNCH
    assert paged(lib, nb=1 << 27, c=addr(64)) == ELAUNCH       # 2^31 slots: 64-bit slots
    assert paged(lib, mb=1 << 27, btsr=1 << 27) == ELAUNCH
    assert paged(lib, out=addr(1)) == EALIAS
    assert paged(lib, out=ctypes.c_void_p(BASE + 3 * GB + 1024)) == EALIAS   # out inside cache


# ------------------------------------------------------------- metadata --

def meta(lib, **kw):
    no_gpu()
    a = dict(qsl=addr(1), R=4, act=100, pad=-1, si=addr(2), sicap=128, qs=addr(3), qscap=128)
    a.update(kw)
    return lib.sconv_seq_metadata(a["qsl"], a["R"], a["act"], a["pad"], a["si"], a["sicap"],
                                  a["qs"], a["qscap"], None)


def test_seq_metadata_validation(lib):
    assert meta(lib, pad=99) == ESHAPE            # padding must cover the actual rows
    assert meta(lib, sicap=99) == ESHAPE          # seq_idx_out too small
    assert meta(lib, qscap=50) == ESHAPE          # query_start_out too small
    assert meta(lib, R=0) == ESHAPE               # actual rows need a request
    assert meta(lib, act=-1) == ESHAPE
    assert meta(lib, act=0, pad=0, si=None) == OK
    assert meta(lib, si=None) == ENULL
    assert meta(lib, qsl=None) == ENULL
    assert meta(lib, qs=ctypes.c_void_p(BASE + 3 * GB + 2)) == EALIGN
    assert meta(lib, qs=ctypes.c_void_p(BASE + 2 * GB + 64)) == EALIAS
    assert meta(lib, qs=addr(1)) == EALIAS        # output over query_start_loc


# ---------------------------------------------------------- paged, multi --

def pmulti(lib, n=2, offs=(0, 128), wss=(128, 128), xs=None, outs=None, **kw):
    no_gpu()
    VP, I64A, I32A = ctypes.c_void_p * n, ctypes.c_int64 * n, ctypes.c_int32 * n
    xs = xs or [addr(10 + i) for i in range(n)]
    outs = outs or [addr(20 + i) for i in range(n)]
    a = dict(c=addr(3), csb=32 * 16 * 512, csh=16 * 512, csn=512, nb=64, H=32, N=16, D=512,
             pos=addr(4), slot=addr(5), qsl=addr(6), R=3, bt=addr(7), btsr=64, mb=64, T=100,
             width=4, act=1, res=1)
    a.update(kw)
    return lib.sconv_paged_fused_multi(
        n, VP(*xs), I64A(*[32 * w for w in wss]), VP(*[addr(30 + i) for i in range(n)]),
        I64A(*[4] * n), None, I32A(*offs), I32A(*wss), VP(*outs), I64A(*[32 * w for w in wss]),
        a["c"], a["csb"], a["csh"], a["csn"], a["nb"], a["H"], a["N"], a["D"], a["pos"],
        a["slot"], a["qsl"], a["R"], a["bt"], a["btsr"], a["mb"], a["T"], a["width"], a["act"],
        a["res"], None)


def test_paged_multi_validation(lib):
    assert pmulti(lib, T=0) == OK
    assert pmulti(lib, offs=(0, 64), T=0) == EALIAS              # D ranges overlap
    assert pmulti(lib, n=1, offs=(400,), wss=(128,), T=0) == ESHAPE   # past head_dim
    assert pmulti(lib, n=9, offs=tuple(range(0, 512, 64))[:8] + (0,), wss=(8,) * 9,
                  T=0) == ESHAPE                                 # too many streams
    assert pmulti(lib, xs=[addr(10), None]) == ENULL
    assert pmulti(lib, outs=[addr(20), addr(10)]) == EALIAS      # out over another x
    assert pmulti(lib, outs=[addr(20), addr(20)]) == EALIAS      # two outs coincide
    assert pmulti(lib, outs=[addr(20), addr(3)]) == EALIAS       # out over the cache
    assert pmulti(lib, offs=(0, 132), wss=(128, 120)) == ELAUNCH  # general kernel (no GPU here)
