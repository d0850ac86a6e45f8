"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, and rejects invalid calls with the documented status codes before
launching anything (no GPU needed: every call here fails validation)."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "palimpsa.h")


@pytest.fixture(scope="module")
def lib():
    import bayesian_metaplastic_memory_amd as pm
    if not os.path.exists(pm.LIB_PATH):
        from bayesian_metaplastic_memory_amd import build
        build.build()
    return pm.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(palimpsa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("palimpsa_fwd_chunked", "palimpsa_fwd_workspace_size", "palimpsa_fwd_frozen",
              "palimpsa_step", "palimpsa_bwd", "palimpsa_bwd_workspace_size", "palimpsa_bwd_frozen",
              "palimpsa_fwd_blockdiag", "palimpsa_step_blockdiag", "palimpsa_bwd_blockdiag",
              "palimpsa_bwd_blockdiag_workspace_size",
              "palimpsa_status_string", "palimpsa_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    import bayesian_metaplastic_memory_amd as pm
    out = subprocess.run(["nm", "-D", "--defined-only", pm.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(lib, n)


def test_status_strings(lib):
    import bayesian_metaplastic_memory_amd as pm
    for s in range(6):
        assert pm.status_string(s)
    assert pm.status_string(99) == "unknown status"
    assert pm.version() >= 100


FAKE = 0x10000       # 16-byte aligned host address, never dereferenced


def _no_gpu_here():
    import torch
    return torch.cuda.device_count() == 0


# The invalid-call tables pass fake pointers: a case that validation let
# through would launch a kernel on them.  They run on a host without a GPU
# (there any such launch fails with PALIMPSA_ERR_HIP and the test catches it).
invalid_calls = pytest.mark.skipif(not _no_gpu_here(), reason="invalid-call tables run on a host without a GPU")


def _fwd_args(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, dt=FAKE, A=FAKE, Ip=FAKE, mu0=None, I0=None,
             y=FAKE, muT=FAKE, IT=FAKE, B=2, T=8, H=3, dk=64, dv=64, chunk=0, segments=0,
             ind=1, outd=1, flags=0, ws=None, wsb=0, stream=None)
    a.update(over)
    return [a[n] for n in ("q", "k", "v", "beta", "dt", "A", "Ip", "mu0", "I0", "y", "muT", "IT",
                           "B", "T", "H", "dk", "dv", "chunk", "segments", "ind", "outd", "flags",
                           "ws", "wsb", "stream")]


FWD_CASES = [
    (dict(q=None), 1), (dict(k=None), 1), (dict(dt=None), 1), (dict(A=None), 1),
    (dict(A=None, T=0), 1), (dict(Ip=None, T=0, q=None), 1),
    (dict(Ip=None), 1), (dict(y=None), 1), (dict(mu0=FAKE), 1), (dict(I0=FAKE), 1),
    (dict(muT=None), 1), (dict(IT=None), 1), (dict(B=0), 1), (dict(H=0), 1), (dict(T=-1), 1),
    (dict(dk=0), 1), (dict(ind=2), 1), (dict(outd=-1), 1), (dict(chunk=12), 1),
    (dict(chunk=256), 1), (dict(chunk=96), 1), (dict(dk=48), 2), (dict(dv=4104), 2), (dict(dv=24), 2), (dict(dk=16), 2),
    (dict(flags=16), 1), (dict(flags=-1), 1), (dict(flags=2, Ip=FAKE + 4), 3),
    # the training forward: a backward workspace, one pass at chunk 16, dk <= 128
    (dict(flags=8), 1), (dict(flags=4), 1), (dict(flags=4, ws=FAKE, wsb=64), 1),
    (dict(flags=4, ws=FAKE, wsb=1 << 40, segments=2), 2), (dict(flags=4, ws=FAKE, wsb=1 << 40, chunk=32), 2),
    (dict(flags=4, ws=FAKE, wsb=1 << 40, dv=2048), 2), (dict(flags=4, ws=FAKE, wsb=1 << 40, dk=256), 2),
    (dict(flags=4, ws=FAKE + 8, wsb=1 << 40), 3), (dict(flags=6, ws=FAKE, wsb=1 << 40, Ip=FAKE + 4), 3),
    (dict(dk=4096), 2), (dict(dk=384), 2), (dict(dk=512, flags=1), 2), (dict(dk=2048, flags=2), 2),
    (dict(dk=512, segments=2), 2), (dict(dv=4112), 2), (dict(dk=256, dv=2048), 2), (dict(dk=1024, dv=24), 2),
    (dict(q=FAKE + 4), 3), (dict(v=FAKE + 8), 3),
    (dict(mu0=FAKE + 4, I0=FAKE), 3), (dict(IT=FAKE + 12), 3), (dict(dt=FAKE + 1), 3),
    (dict(y=FAKE + 1), 3), (dict(A=FAKE + 2), 3), (dict(beta=FAKE + 2), 3),
    (dict(segments=-1), 1), (dict(segments=65), 1), (dict(wsb=64), 1),
    (dict(ws=FAKE + 8, wsb=64), 3),
]


def test_workspace_size_host_logic(lib):
    """Segment planning is host logic: auto splits only under-filled grids."""
    import bayesian_metaplastic_memory_amd as pm
    # 760M layer (768 workgroups): no split
    assert pm.workspace_size(8, 4096, 12, 128, 128, 0) == 0
    # long context, 32 heads (256 workgroups; 3 segments fill 256 CUs at three
    # workgroups each): 4 rounds = 12 segments -> 11 summaries (M_loc,
    # Ibar_loc, decay product) plus one copy of the start state (mu0, I0)
    def split_bytes(nseg, bh, dv, dk):
        return ((nseg - 1) * (2 * bh * dv * dk + bh) + 2 * bh * dv * dk) * 4
    assert pm.workspace_size(1, 32768, 32, 128, 128, 0) == split_bytes(12, 32, 128, 128)
    # MQAR layer (128 workgroups, 6 per round -> 12): at least 256 tokens per segment -> 8
    assert pm.workspace_size(4, 2048, 8, 64, 64, 0) == split_bytes(8, 32, 64, 64)
    # 96 workgroups: one round of 8 segments
    assert pm.workspace_size(1, 4096, 12, 128, 128, 0) == split_bytes(8, 12, 128, 128)
    # 32 workgroups: one round of 24 segments
    assert pm.workspace_size(1, 65536, 8, 64, 64, 0) == split_bytes(24, 8, 64, 64)
    # the choice is capped to the no-allocation scratch (64 MiB): 8 MiB per
    # segment here, so 7 segments rather than 12
    assert pm.workspace_size(1, 32768, 4, 256, 1024, 0) == split_bytes(7, 4, 1024, 256)
    assert split_bytes(7, 4, 1024, 256) <= pm.noalloc_scratch_bytes() < split_bytes(8, 4, 1024, 256)
    # explicit requests; rounding to 64-token segments caps the count
    assert pm.workspace_size(1, 1000, 2, 64, 64, 4) == split_bytes(4, 2, 64, 64)
    assert pm.workspace_size(1, 100, 2, 64, 64, 8) == split_bytes(2, 2, 64, 64)
    assert pm.workspace_size(1, 64, 2, 64, 64, 8) == 0
    assert pm.workspace_size(1, 4096, 2, 64, 64, 1) == 0
    assert pm.workspace_size(1, 0, 2, 64, 64, 4) == 0
    assert pm.workspace_size(1, 64, 2, 48, 64, 0) == 0


def test_wide_rows_workspace_size_host_logic(lib):
    """Heads of 512 keys and wider: the row-parallel form's workspace is the
    column-group records (14 bytes per token and key column, padded to 256
    bytes) plus 4 bytes per output element and column slice (2 slices at
    d_k = 512 and 1024, 4 at 2048); it is offered only when d_v is a multiple
    of 64, T >= 1 and the 64-row x slice grid has a workgroup for each of the
    device's CUs (256 without a device).  The split request is not used."""
    import bayesian_metaplastic_memory_amd as pm

    def expect(B, T, H, dk, dv):
        nq = 2 if dk <= 1024 else 4
        ntok = B * T * H
        return (ntok * dk * 14 + 255) // 256 * 256 + nq * ntok * dv * 4
    for shape in [(16, 2048, 1, 2048, 2048), (16, 2048, 1, 512, 512), (2, 9, 2, 1024, 2048), (1, 3, 1, 2048, 4096),
                  (4, 21, 1, 512, 2048)]:
        assert pm.workspace_size(*shape) == expect(*shape), shape
        assert pm.workspace_size(*shape, 3) == expect(*shape), shape
    assert pm.workspace_size(1, 9, 1, 2048, 2048) == 0      # 128 workgroups
    assert pm.workspace_size(16, 9, 1, 2048, 2016) == 0     # d_v not a multiple of 64
    assert pm.workspace_size(16, 0, 1, 2048, 2048) == 0     # empty sequence
    assert pm.workspace_size(16, 9, 1, 256, 256) == 0       # d_k = 256: the column-parallel kernel


@invalid_calls
@pytest.mark.parametrize("over,status", FWD_CASES)
def test_fwd_rejects_invalid_calls(lib, over, status):
    assert lib.palimpsa_fwd_chunked(*_fwd_args(**over)) == status


def _noalloc_args(**over):
    a = _fwd_args(**over)
    return a[:22] + [a[24]]      # no workspace, no workspace bytes


NOALLOC_CASES = [
    (dict(q=None), 1), (dict(flags=4), 1), (dict(flags=8), 1), (dict(chunk=12), 1), (dict(B=0), 1),
    (dict(dk=48), 2), (dict(q=FAKE + 4), 3), (dict(segments=65), 1),
]


@invalid_calls
@pytest.mark.parametrize("over,status", NOALLOC_CASES)
def test_noalloc_fwd_rejects_invalid_calls(lib, over, status):
    assert lib.palimpsa_fwd_chunked_noalloc(*_noalloc_args(**over)) == status


def _step_args(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, dt=FAKE, A=FAKE, Ip=FAKE, mu=FAKE, I=FAKE, y=FAKE,
             B=2, H=3, dk=128, dv=128, ind=1, outd=1, flags=0, stream=None)
    a.update(over)
    return [a[n] for n in ("q", "k", "v", "beta", "dt", "A", "Ip", "mu", "I", "y",
                           "B", "H", "dk", "dv", "ind", "outd", "flags", "stream")]


STEP_CASES = [
    (dict(q=None), 1), (dict(mu=None), 1), (dict(I=None), 1), (dict(y=None), 1),
    (dict(B=0), 1), (dict(H=-2), 1), (dict(ind=5), 1), (dict(dk=100), 2), (dict(dv=8), 2),
    (dict(mu=FAKE + 4), 3), (dict(I=FAKE + 8), 3), (dict(k=FAKE + 1), 3), (dict(dt=FAKE + 1), 3),
    (dict(y=FAKE + 3), 3), (dict(Ip=FAKE + 2), 3), (dict(flags=4), 1), (dict(flags=8), 1), (dict(dv=40), 2),
    (dict(flags=2, Ip=FAKE + 8), 3), (dict(dk=4096), 2), (dict(dk=768), 2),
]


@invalid_calls
@pytest.mark.parametrize("over,status", STEP_CASES)
def test_step_rejects_invalid_calls(lib, over, status):
    assert lib.palimpsa_step(*_step_args(**over)) == status


def test_product_path_does_not_touch_the_oracle():
    """The package and its library never import, load or link the oracle."""
    pkg = os.path.join(ROOT, "bayesian_metaplastic_memory_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, flags=re.M), f
                assert "palimpsa_oracle" not in text, f
    import bayesian_metaplastic_memory_amd as pm
    if os.path.exists(pm.LIB_PATH):
        needed = subprocess.run(["readelf", "-d", pm.LIB_PATH], capture_output=True,
                                text=True).stdout
        assert "oracle" not in needed


def test_binding_fails_loudly_without_a_gpu_tensor():
    import torch
    import bayesian_metaplastic_memory_amd as pm
    x = torch.zeros(1, 4, 1, 32)
    with pytest.raises(ValueError):
        pm.fwd_chunked(x, x, x, x, torch.zeros(1, 4, 1), torch.ones(1), torch.ones(1))


def _frozen_args(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, dt=FAKE, A=FAKE, Ip=FAKE, mu0=None, y=FAKE,
             muT=FAKE, B=2, T=8, H=3, dk=128, dv=64, ind=1, outd=1, stream=None)
    a.update(over)
    return [a[n] for n in ("q", "k", "v", "beta", "dt", "A", "Ip", "mu0", "y", "muT",
                           "B", "T", "H", "dk", "dv", "ind", "outd", "stream")]


FROZEN_CASES = [
    (dict(q=None), 1), (dict(dt=None), 1), (dict(y=None), 1), (dict(A=None), 1), (dict(B=0), 1),
    (dict(T=-2), 1), (dict(ind=3), 1), (dict(ind=0), 2), (dict(dk=32), 2), (dict(dv=32), 2),
    (dict(dk=48), 2), (dict(q=FAKE + 8), 3), (dict(y=FAKE + 8), 3), (dict(beta=FAKE + 4), 3),
    (dict(mu0=FAKE + 4), 3), (dict(dt=FAKE + 1), 3), (dict(dv=96), 2), (dict(dv=1088), 2),
]


@invalid_calls
@pytest.mark.parametrize("over,status", FROZEN_CASES)
def test_frozen_rejects_invalid_calls(lib, over, status):
    assert lib.palimpsa_fwd_frozen(*_frozen_args(**over)) == status


def _bwd_args(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, dt=FAKE, A=FAKE, Ip=FAKE, mu0=None, I0=None,
             gy=FAKE, gmuT=None, gIT=None, gq=FAKE, gk=FAKE, gv=FAKE, gbeta=FAKE, gdt=FAKE,
             gA=FAKE, gIp=FAKE, gmu0=None, gI0=None, B=2, T=8, H=3, dk=64, dv=64, ind=1, gyd=1,
             flags=0, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(over)
    return [a[n] for n in ("q", "k", "v", "beta", "dt", "A", "Ip", "mu0", "I0", "gy", "gmuT", "gIT",
                           "gq", "gk", "gv", "gbeta", "gdt", "gA", "gIp", "gmu0", "gI0",
                           "B", "T", "H", "dk", "dv", "ind", "gyd", "flags", "ws", "wsb", "stream")]


BWD_CASES = [
    (dict(q=None), 1), (dict(gy=None), 1), (dict(gq=None), 1), (dict(gdt=None), 1),
    (dict(gA=None), 1), (dict(gIp=None), 1), (dict(A=None), 1), (dict(ws=None), 1),
    (dict(mu0=FAKE), 1), (dict(I0=FAKE), 1), (dict(B=0), 1), (dict(T=-1), 1), (dict(H=0), 1),
    (dict(ind=2), 1), (dict(gyd=5), 1), (dict(wsb=64), 1), (dict(q=None, T=0, A=None), 1),
    (dict(dk=48), 2), (dict(dv=1040), 2), (dict(dv=8), 2), (dict(dk=16), 2),
    (dict(flags=4), 1), (dict(flags=16), 1), (dict(flags=12), 1),
    (dict(flags=8, ws=None), 1), (dict(flags=8, wsb=64), 1),
    (dict(flags=2, Ip=FAKE + 4), 3), (dict(flags=2, gIp=FAKE + 4), 3),
    (dict(q=FAKE + 4), 3), (dict(gy=FAKE + 8), 3), (dict(gq=FAKE + 4), 3), (dict(gk=FAKE + 8), 3),
    (dict(gdt=FAKE + 2), 3), (dict(dt=FAKE + 1), 3), (dict(ws=FAKE + 8), 3),
    (dict(gmuT=FAKE + 4), 3), (dict(gmu0=FAKE + 12), 3), (dict(gA=FAKE + 1), 3),
    (dict(mu0=FAKE + 4, I0=FAKE), 3),
]


@invalid_calls
@pytest.mark.parametrize("over,status", BWD_CASES)
def test_bwd_rejects_invalid_calls(lib, over, status):
    assert lib.palimpsa_bwd(*_bwd_args(**over)) == status


def _bwd_fz_args(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, dt=FAKE, A=FAKE, Ip=FAKE, mu0=None, gy=FAKE, gmuT=None,
             gq=FAKE, gk=FAKE, gv=FAKE, gbeta=FAKE, gdt=FAKE, gA=FAKE, gIp=FAKE, gmu0=None,
             B=2, T=8, H=3, dk=64, dv=64, ind=1, gyd=1, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(over)
    return [a[n] for n in ("q", "k", "v", "beta", "dt", "A", "Ip", "mu0", "gy", "gmuT",
                           "gq", "gk", "gv", "gbeta", "gdt", "gA", "gIp", "gmu0",
                           "B", "T", "H", "dk", "dv", "ind", "gyd", "ws", "wsb", "stream")]


# every case fails validation (a NULL beta alone would be a valid call)
BWD_FZ_CASES = [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(dt=None), 1), (dict(gy=None), 1),
    (dict(gq=None), 1), (dict(gk=None), 1), (dict(gv=None), 1), (dict(gdt=None), 1),
    (dict(gbeta=None), 1), (dict(beta=None, gq=None), 1),
    (dict(gA=None), 1), (dict(gIp=None), 1), (dict(A=None), 1), (dict(Ip=None), 1), (dict(ws=None), 1),
    (dict(B=0), 1), (dict(T=-1), 1), (dict(H=0), 1), (dict(dk=0), 1), (dict(ind=2), 1), (dict(gyd=5), 1),
    (dict(wsb=64), 1), (dict(beta=None, gbeta=None, wsb=64), 1), (dict(q=None, T=0, A=None), 1),
    (dict(dk=48), 2), (dict(dk=16), 2), (dict(dv=1040), 2), (dict(dv=8), 2),
    (dict(q=FAKE + 4), 3), (dict(beta=FAKE + 8), 3), (dict(gy=FAKE + 8), 3), (dict(gq=FAKE + 4), 3),
    (dict(gk=FAKE + 8), 3), (dict(mu0=FAKE + 4), 3), (dict(gmuT=FAKE + 4), 3), (dict(gmu0=FAKE + 12), 3),
    (dict(gdt=FAKE + 2), 3), (dict(dt=FAKE + 1), 3), (dict(gA=FAKE + 1), 3), (dict(gIp=FAKE + 2), 3),
    (dict(ws=FAKE + 8), 3),
]


@invalid_calls
@pytest.mark.parametrize("over,status", BWD_FZ_CASES)
def test_bwd_frozen_rejects_invalid_calls(lib, over, status):
    assert lib.palimpsa_bwd_frozen(*_bwd_fz_args(**over)) == status


def test_bwd_workspace_size_host_logic(lib):
    """Checkpoints every 16 tokens plus the row-block partials, each section
    padded to 256 bytes."""
    import bayesian_metaplastic_memory_amd as pm
    pad = lambda n: (4 * n + 255) // 256 * 256

    def expect(B, T, H, dk, dv, per_entry=False):
        nck, nrb, bh = (T + 15) // 16, dv // 16, B * H
        return (pad(bh * nck * 2 * dv * dk) + pad(nrb * bh * T * 2 * dk) + pad(nrb * bh * T * 2)
                + 2 * pad(bh) + pad(bh * nrb) + (pad(bh * dv * dk) if per_entry else 0))
    for shape in [(1, 10, 2, 32, 32), (8, 4096, 12, 128, 128), (1, 0, 3, 64, 128), (2, 9, 1, 128, 64),
                  (1, 33, 2, 128, 256), (2, 5, 3, 64, 48)]:
        assert pm.bwd_workspace_size(*shape) == expect(*shape), shape
        assert pm.bwd_workspace_size(*shape, flags=2) == expect(*shape, per_entry=True), shape
        assert pm.bwd_workspace_size(*shape, flags=1) == expect(*shape), shape
        # either checkpoint bit leaves the size as it is
        assert pm.bwd_workspace_size(*shape, flags=4) == expect(*shape), shape
        assert pm.bwd_workspace_size(*shape, flags=10) == expect(*shape, per_entry=True), shape
    assert pm.bwd_workspace_size(1, 8, 2, 48, 64) == 0
    assert pm.bwd_workspace_size(0, 8, 2, 64, 64) == 0
    assert pm.bwd_workspace_size(1, 8, 2, 64, 24) == 0
    assert pm.bwd_workspace_size(1, 8, 2, 64, 64, flags=16) == 0


def _bd_args(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, dt=FAKE, A=FAKE, Ip=FAKE, mu0=None, P0=None, y=FAKE,
             muT=FAKE, PT=FAKE, B=2, T=8, H=3, dk=64, dv=64, block=2, ind=1, outd=1, flags=0, ws=None, wsb=0,
             stream=None)
    a.update(over)
    return [a[n] for n in ("q", "k", "v", "beta", "dt", "A", "Ip", "mu0", "P0", "y", "muT", "PT",
                           "B", "T", "H", "dk", "dv", "block", "ind", "outd", "flags", "ws", "wsb", "stream")]


BD_CASES = [
    (dict(q=None), 1), (dict(y=None), 1), (dict(A=None), 1), (dict(mu0=FAKE), 1), (dict(PT=None), 1),
    (dict(B=0), 1), (dict(T=-1), 1), (dict(block=0), 1), (dict(ind=4), 1),
    (dict(block=1), 2), (dict(block=3), 2), (dict(block=8), 2), (dict(block=4, dk=32), 2), (dict(dk=48), 2),
    (dict(dv=24), 2),
    (dict(q=FAKE + 4), 3), (dict(PT=FAKE + 8), 3), (dict(mu0=FAKE + 2, P0=FAKE), 3), (dict(dt=FAKE + 1), 3),
    # the training forward: a backward workspace of the right size
    (dict(flags=4), 1), (dict(flags=8, ws=FAKE, wsb=1 << 40), 1), (dict(flags=1), 1),
    (dict(flags=4, ws=FAKE, wsb=64), 1), (dict(flags=4, ws=FAKE + 8, wsb=1 << 40), 3),
    (dict(flags=4, ws=FAKE, wsb=1 << 40, block=3), 2),
]


@invalid_calls
@pytest.mark.parametrize("over,status", BD_CASES)
def test_blockdiag_rejects_invalid_calls(lib, over, status):
    assert lib.palimpsa_fwd_blockdiag(*_bd_args(**over)) == status


def _bd_step_args(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, dt=FAKE, A=FAKE, Ip=FAKE, mu=FAKE, P=FAKE, y=FAKE,
             B=2, H=3, dk=64, dv=64, block=2, ind=1, outd=1, stream=None)
    a.update(over)
    return [a[n] for n in ("q", "k", "v", "beta", "dt", "A", "Ip", "mu", "P", "y",
                           "B", "H", "dk", "dv", "block", "ind", "outd", "stream")]


BD_STEP_CASES = [
    (dict(q=None), 1), (dict(mu=None), 1), (dict(P=None), 1), (dict(y=None), 1), (dict(beta=None), 1),
    (dict(A=None), 1), (dict(B=0), 1), (dict(H=-1), 1), (dict(block=0), 1), (dict(ind=3), 1), (dict(outd=7), 1),
    (dict(block=1), 2), (dict(block=8), 2), (dict(block=4, dk=32), 2), (dict(dk=48), 2), (dict(dk=256), 2),
    (dict(dv=24), 2),
    (dict(mu=FAKE + 4), 3), (dict(P=FAKE + 8), 3), (dict(dt=FAKE + 1), 3), (dict(y=FAKE + 1), 3),
    (dict(ind=0, q=FAKE + 2), 3), (dict(A=FAKE + 2), 3),
]


@invalid_calls
@pytest.mark.parametrize("over,status", BD_STEP_CASES)
def test_blockdiag_step_rejects_invalid_calls(lib, over, status):
    assert lib.palimpsa_step_blockdiag(*_bd_step_args(**over)) == status


def _bd_bwd_args(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, dt=FAKE, A=FAKE, Ip=FAKE, mu0=None, P0=None, gy=FAKE,
             gmuT=None, gPT=None, gq=FAKE, gk=FAKE, gv=FAKE, gbeta=FAKE, gdt=FAKE, gA=FAKE, gIp=FAKE,
             gmu0=None, gP0=None, B=2, T=8, H=3, dk=64, dv=64, block=2, ind=1, gyd=1, flags=0, ws=FAKE,
             wsb=1 << 40, stream=None)
    a.update(over)
    return [a[n] for n in ("q", "k", "v", "beta", "dt", "A", "Ip", "mu0", "P0", "gy", "gmuT", "gPT",
                           "gq", "gk", "gv", "gbeta", "gdt", "gA", "gIp", "gmu0", "gP0",
                           "B", "T", "H", "dk", "dv", "block", "ind", "gyd", "flags", "ws", "wsb", "stream")]


# every case fails validation
BD_BWD_CASES = [
    (dict(q=None), 1), (dict(k=None), 1), (dict(beta=None), 1), (dict(dt=None), 1), (dict(gy=None), 1),
    (dict(gq=None), 1), (dict(gk=None), 1), (dict(gv=None), 1), (dict(gbeta=None), 1), (dict(gdt=None), 1),
    (dict(gA=None), 1), (dict(gIp=None), 1), (dict(A=None), 1), (dict(Ip=None), 1), (dict(ws=None), 1),
    (dict(mu0=FAKE), 1), (dict(P0=FAKE), 1), (dict(B=0), 1), (dict(T=-1), 1), (dict(H=0), 1), (dict(dk=0), 1),
    (dict(block=0), 1), (dict(ind=2), 1), (dict(gyd=5), 1), (dict(wsb=64), 1),
    (dict(q=None, T=0, A=None), 1),
    (dict(block=1), 2), (dict(block=3), 2), (dict(block=8), 2), (dict(block=4, dk=32), 2), (dict(dk=48), 2),
    (dict(dv=1040), 2), (dict(dv=8), 2),
    (dict(q=FAKE + 4), 3), (dict(gy=FAKE + 8), 3), (dict(P0=FAKE + 8, mu0=FAKE), 3),
    (dict(mu0=FAKE + 2, P0=FAKE), 3), (dict(gPT=FAKE + 4), 3), (dict(gP0=FAKE + 8), 3), (dict(gq=FAKE + 4), 3),
    (dict(gmuT=FAKE + 1), 3), (dict(gmu0=FAKE + 2), 3), (dict(gdt=FAKE + 2), 3), (dict(dt=FAKE + 1), 3),
    (dict(ws=FAKE + 8), 3), (dict(flags=4), 1), (dict(flags=9), 1), (dict(flags=8, wsb=64), 1),
]


@invalid_calls
@pytest.mark.parametrize("over,status", BD_BWD_CASES)
def test_blockdiag_bwd_rejects_invalid_calls(lib, over, status):
    assert lib.palimpsa_bwd_blockdiag(*_bd_bwd_args(**over)) == status


def test_bwd_blockdiag_workspace_size_host_logic(lib):
    """Checkpoints of the lane states (h, then the upper triangle of each
    block: 3 entries per 2x2 block, 10 per 4x4, padded to float4s) every 8
    tokens, then the exact backward's partials, then one workgroup block for
    the training forward's stores past the sequence."""
    import bayesian_metaplastic_memory_amd as pm
    pad = lambda n: (4 * n + 255) // 256 * 256

    def expect(B, T, H, dk, dv, block=2):
        nsb, nrb, bh = (T + 7) // 8, dv // 16, B * H
        kc = dk // 16
        lane = (kc + (3 * (kc // 2) if block == 2 else 10 * (kc // 4)) + 3) // 4 * 4
        return (pad(bh * nsb * nrb * 256 * lane) + pad(nrb * bh * T * 2 * dk) + pad(nrb * bh * T * 2)
                + 2 * pad(bh) + pad(bh * nrb)
                + pad(256 * lane))    # the training forward's discard block
    for shape in [(1, 10, 2, 32, 32), (8, 4096, 12, 128, 128), (1, 0, 3, 64, 128), (2, 9, 1, 128, 64)]:
        assert pm.bwd_blockdiag_workspace_size(*shape) == expect(*shape), shape
        if shape[3] > 32:
            assert pm.bwd_blockdiag_workspace_size(*shape, block=4) == expect(*shape, block=4), shape
    assert pm.bwd_blockdiag_workspace_size(1, 8, 2, 32, 64, block=4) == 0
    assert pm.bwd_blockdiag_workspace_size(1, 8, 2, 64, 64, block=8) == 0
    assert pm.bwd_blockdiag_workspace_size(1, 8, 2, 48, 64) == 0
    assert pm.bwd_blockdiag_workspace_size(0, 8, 2, 64, 64) == 0


def test_check_params_host_logic():
    """The opt-in value check of the data preconditions (CPU tensors here)."""
    import torch
    import bayesian_metaplastic_memory_amd as pm
    A, Ip = torch.tensor([0.0, 1.0, 16.0]), torch.tensor([1.0, 0.5, 2.0])
    pm.check_params(A, Ip, dt=torch.zeros(2, 3), beta=torch.rand(2, 3), I0=torch.ones(4))
    bad = [dict(A=torch.tensor([-1.0, 1.0, 1.0])), dict(I_prior=torch.tensor([1.0, 0.0, 1.0])),
           dict(A=torch.tensor([float("nan"), 1.0, 1.0])), dict(I_prior=torch.tensor([1.0, float("inf"), 1.0])),
           dict(dt=torch.tensor([-1e-3])), dict(beta=torch.tensor([-0.5])), dict(I0=torch.tensor([0.0])),
           dict(dt=torch.tensor([1.0, float("nan")], dtype=torch.bfloat16))]
    for over in bad:
        kw = dict(A=A, I_prior=Ip)
        kw.update(over)
        name = next(iter(over))
        with pytest.raises(ValueError, match=name):
            pm.check_params(**kw)
