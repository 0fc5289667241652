"""The C ABI on the host (no GPU): the library loads, exports every function
include/hsa.h declares, and rejects invalid arguments with the documented
status before anything is enqueued."""
import ctypes as ct
import os
import re

import pytest

from token_sparse_attention_compact_amd import hsa as H

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "hsa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:hsa_status|const char \*|int32_t)\s*(hsa_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported():
    L = H.load()
    names = declared_functions()
    assert len(names) >= 18
    for n in names:
        assert hasattr(L, n), f"libhsa.so does not export {n}"
    assert set(names) <= set(H.EXPORTED) | set(names)
    assert set(H.EXPORTED) == set(names), "binding list and header disagree"


def test_abi_version_matches_header_and_binding():
    text = open(HEADER).read()
    v = int(re.search(r"#define HSA_ABI_VERSION (\d+)", text).group(1))
    assert H.load().hsa_abi_version() == v == H.ABI_VERSION
    # struct sizes the binding marshals agree with the header's field lists
    assert [f for f, _ in H.Dims._fields_][-4:] == ["features", "grid_f", "grid_h", "grid_w"]
    assert len(H.Block._fields_) == 17 and H.Model._fields_[-1][0] == "cfg_scale"
    # gather flag of the QKV projection is validated
    assert H.load().hsa_qkv_scatter(None, None, 2, None, None, None, None, 4, 8, 64, 1, None) == -1


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8, 99):
        assert H.status_str(code)


def test_noalloc_attention_validates_on_the_host():
    """The allocation-free attention entry point checks its arguments and its
    scratch limit before any HIP call: a problem whose KV-split partials
    exceed HSA_NOALLOC_SCRATCH_BYTES returns HSA_ERR_TOO_LARGE (-8)."""
    text = open(HEADER).read()
    assert int(eval(re.search(r"#define HSA_NOALLOC_SCRATCH_BYTES (.+)", text).group(1)
                    .replace("(size_t)", ""))) == H.NOALLOC_SCRATCH_BYTES
    L = H.load()
    fake = 4096                                  # aligned, never dereferenced on these paths
    nA, nkv, Hh, Dh = 256, 75600, 200, 128       # 180 MiB of partials (14 KV splits per item)
    assert H.hsa_attn_workspace_size(nA, nkv, Hh, Dh) > H.NOALLOC_SCRATCH_BYTES
    assert L.hsa_attn_active_noalloc(fake, fake, fake, fake, nA, nkv, Hh, Dh, 0.088, 1, None) == -8
    assert L.hsa_attn_active_noalloc(None, fake, fake, fake, 8, 64, 2, 128, 0.088, 1, None) == -1
    assert L.hsa_attn_active_noalloc(fake + 2, fake, fake, fake, 8, 64, 2, 128, 0.088, 1, None) == -4
    assert L.hsa_attn_active_noalloc(fake, fake, fake, fake, 8, 64, 2, 96, 0.088, 1, None) == -2
    assert L.hsa_attn_active_noalloc(fake, fake, fake, fake, 8, 64, 2, 128, -1.0, 1, None) == -1
    assert L.hsa_attn_active_noalloc(fake, fake, fake, fake, 0, 64, 2, 128, 0.088, 1, None) == 0
    assert "HSA_NOALLOC_SCRATCH_BYTES" in H.status_str(-8)


def test_workspace_size_validation():
    d = H.make_dims(32760, 16, 1536, 12, 128, 8960, 30)
    assert H.hsa_workspace_size(d) > 32760 * 1536 * 4
    bad = H.make_dims(32760, 16, 1536, 12, 96, 8960, 30)   # D != H*Dh and Dh unsupported
    with pytest.raises(H.HsaError) as e:
        H.hsa_workspace_size(bad)
    assert e.value.status == -2
    bad = H.make_dims(100, 16, 1536, 12, 128, 8900, 1)     # bf16 needs F % 64 == 0
    with pytest.raises(H.HsaError):
        H.hsa_workspace_size(bad)


def test_schedule_validation_and_closed_form():
    s = H.make_schedule(40, [40, 20, 10], [8190, 8190, 16380])
    assert [H.hsa_n_active(s, i) for i in range(4)] == [32760, 8190, 16380, 8190]
    s3 = H.make_schedule(40, [40, 20, 10], [8190, 8190, 16380], m=3)
    assert H.hsa_n_active(s3, 1) == 32760 and H.hsa_n_active(s3, 37) == 32760
    assert H.hsa_n_active(s3, 5) == 8190
    for budgets in ([40, 15, 10], [20, 20, 10]):                 # 15 does not divide 40; budget[0] != T
        with pytest.raises(H.HsaError) as e:
            H.hsa_n_active(H.make_schedule(40, budgets, [1, 1, 1]), 0)
        assert e.value.status == -7
    with pytest.raises(H.HsaError):
        H.hsa_n_active(s, 40)                                       # iteration out of range


def test_entry_points_reject_bad_arguments_without_a_device():
    L = H.load()
    null = None
    # null pointers / bad shapes come back as errors before any launch
    assert L.hsa_euler(null, null, null, null, null, 10, 16, 0.1, 1e-6, 1, null) == -1
    assert L.hsa_euler(null, null, null, null, null, 10, 15, 0.1, 1e-6, 1, null) == -2
    assert L.hsa_attn_active(null, null, null, null, 4, 8, 2, 96, 0.1, 1, null, 0, null) == -2
    assert L.hsa_attn_active(null, null, null, null, 4, 8, 2, 128, 0.1, 7, null, 0, null) == -3
    assert L.hsa_attn_active(null, null, null, null, 4, 8, 2, 128, 0.1, 1, null, 0, null) == -1
    assert L.hsa_linear(null, null, null, 4, 64, 100, 0, 1, null) == -2   # bf16 K % 64
    assert L.hsa_linear(null, null, null, 4, 64, 128, 2, 1, null) == -1   # bad activation flag
    counts = (ct.c_int32 * 3)(1, 2, 3)
    assert L.hsa_select(null, 7, counts, 3, null, null, 0, null) == -1
    # batched selection: empty batch or rows, null pointers, counts not summing to N
    assert L.hsa_select_batch(null, 0, 6, counts, 3, null, null) == -2
    assert L.hsa_select_batch(null, 4, 0, counts, 3, null, null) == -2
    assert L.hsa_select_batch(null, 4, 6, counts, 3, null, null) == -1
    assert L.hsa_select_batch(ct.c_void_p(0x1000), 4, 7, counts, 3, ct.c_void_p(0x2000), null) == -7
    assert L.hsa_select_batch(ct.c_void_p(0x1000), 4, 6, counts, 9, ct.c_void_p(0x2000), null) == -2
    big = (ct.c_int32 * 1)(1 << 30)
    assert L.hsa_select_batch(ct.c_void_p(0x1000), 1 << 9, 1 << 30, big, 1, ct.c_void_p(0x2000), null) == -2
    assert L.hsa_step(null, null, null, 0, 1.0, 0.9, 0, null, null) == -1
    # misaligned device pointer
    assert L.hsa_layernorm(ct.c_void_p(0x1004), ct.c_void_p(0x2000), 4, 64, null, null, 1, null) == -4
    # modulation needs both shift and scale
    assert L.hsa_layernorm(ct.c_void_p(0x1000), ct.c_void_p(0x2000), 4, 64, ct.c_void_p(0x3000), null, 1,
                           null) == -1


def test_step_rejects_bad_schedule_before_launch():
    d = H.make_dims(256, 16, 128, 2, 64, 512, 1, 0, dtype=None)
    d.dtype = H.HSA_F32
    blocks = (H.Block * 1)()
    for n in ("w_qkv", "w_o", "w_1", "w_2", "k_cache", "v_cache"):
        setattr(blocks[0], n, 0x1000)
    m = H.Model(d, 0x1000, 0x1000, blocks)
    st = H.State(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 1 << 40)
    bad = H.make_schedule(8, [8, 4], [100, 100])      # counts do not sum to N
    assert H.load().hsa_step(ct.byref(m), ct.byref(bad), ct.byref(st), 0, 1.0, 0.875, 0, None, None) == -7
    ok = H.make_schedule(8, [8, 4], [128, 128])
    st.workspace_bytes = 16                            # too small
    assert H.load().hsa_step(ct.byref(m), ct.byref(ok), ct.byref(st), 0, 1.0, 0.875, 0, None, None) == -5


def test_bf16_operands_past_4gib_are_rejected():
    """bf16 operands go through 32-bit buffer descriptors: shapes whose
    operands reach 4 GiB come back as HSA_ERR_SHAPE before any launch."""
    L = H.load()
    big = H.make_dims(1 << 20, 16, 2048, 16, 128, 8192, 1)          # N x F x 2 = 16 GiB
    with pytest.raises(H.HsaError) as e:
        H.hsa_workspace_size(big)
    assert e.value.status == -2
    ok = H.make_dims(75600, 16, 5120, 40, 128, 13824, 40)          # the 14B-shaped stack fits
    assert H.hsa_workspace_size(ok) > 0
    null = None
    # M * K * 2 = 4 GiB exactly
    assert L.hsa_linear(null, null, null, 1 << 21, 64, 1024, 0, 1, null) == -2
    assert L.hsa_linear(null, null, null, 0, 1 << 21, 1024, 0, 1, null) == -2     # W too large
    # n_kv * H * Dh * 2 = 8 GiB
    assert L.hsa_attn_active(null, null, null, null, 4, 1 << 21, 16, 128, 0.1, 1, null, 0, null) == -2
    # float32 has no such limit on these entry points (it fails later on the null pointers)
    assert L.hsa_linear(null, null, null, 1 << 21, 64, 1024, 0, 0, null) == -1


def test_binding_rejects_mismatched_shapes():
    """The C ABI sees raw pointers only; the binding checks tensor shapes against
    the sizes it passes, so a short buffer is an error, not an out-of-bounds
    access.  These raise before any pointer is taken (host tensors suffice)."""
    import torch
    bf = torch.bfloat16
    q = torch.zeros(10, 256, dtype=bf)
    kv = torch.zeros(50, 256, dtype=bf)
    with pytest.raises(ValueError, match="o: expected shape"):
        H.hsa_attn_active(q, kv, kv, torch.zeros(9, 256, dtype=bf), 2, 128)
    with pytest.raises(ValueError, match="q: expected shape"):
        H.hsa_attn_active(q, kv, kv, q, 2, 64)                       # H * Dh != width
    with pytest.raises(ValueError, match="v: expected shape"):
        H.hsa_attn_active(q, kv, torch.zeros(49, 256, dtype=bf), q, 2, 128)
    with pytest.raises(ValueError, match="out: expected shape"):
        H.hsa_linear(q, torch.zeros(128, 256, dtype=bf), torch.zeros(10, 64, dtype=bf))
    with pytest.raises(ValueError, match="a: expected shape"):
        H.hsa_linear(q, torch.zeros(128, 192, dtype=bf), torch.zeros(10, 128, dtype=bf))
    with pytest.raises(ValueError, match="out: expected shape"):
        H.hsa_layernorm(torch.zeros(4, 256), torch.zeros(4, 128, dtype=bf))
    with pytest.raises(ValueError, match="pos: expected shape"):
        x = torch.zeros(8, 16)
        H.hsa_euler(x, x.clone(), torch.zeros(8), None, torch.zeros(7, dtype=torch.int32), 0.1, False)
    d = H.make_dims(64, 16, 256, 2, 128, 512, 1)
    blk = {"w_qkv": torch.zeros(768, 256, dtype=bf), "w_o": torch.zeros(256, 256, dtype=bf),
           "w_1": torch.zeros(512, 256, dtype=bf), "w_2": torch.zeros(256, 512, dtype=bf),
           "k_cache": torch.zeros(64, 256, dtype=bf), "v_cache": torch.zeros(63, 256, dtype=bf)}
    with pytest.raises(ValueError, match="v_cache: expected shape"):
        H.DeviceModel(d, torch.zeros(256, 16, dtype=bf), torch.zeros(16, 256, dtype=bf), [blk])
    blk["v_cache"] = torch.zeros(64, 256, dtype=torch.float32)
    with pytest.raises(ValueError, match="v_cache: expected"):
        H.DeviceModel(d, torch.zeros(256, 16, dtype=bf), torch.zeros(16, 256, dtype=bf), [blk])


def test_probe_library_exports():
    """The benchmark's attainable-peak probes are built beside the library."""
    from token_sparse_attention_compact_amd import build as B
    lib = ct.CDLL(B.PROBE_LIB)
    for name in ("hsa_probe_mfma_peak", "hsa_probe_copy"):
        assert hasattr(lib, name)
    lib.hsa_probe_copy.argtypes = [ct.c_void_p, ct.c_void_p, ct.c_int64, ct.c_int32, ct.c_int32,
                                   ct.c_void_p]
    assert lib.hsa_probe_copy(None, None, 1024, 4, 0, None) == -1    # rejected before any launch
    assert lib.hsa_probe_copy(4096, 8192, 1024, 5, 0, None) == -1     # unsupported loads per thread
    assert lib.hsa_probe_mfma_peak(0, 10, None, None) == -1


def test_feature_flags_are_validated_on_the_host():
    L = H.load()
    n = ct.c_size_t()
    ok = H.make_dims(32760, 16, 1536, 12, 128, 8960, 30, features=("qk_norm", "rope3d", "adaln"),
                     grid=(21, 30, 52))
    assert L.hsa_workspace_size(ct.byref(ok), ct.byref(n)) == 0
    plain = H.make_dims(32760, 16, 1536, 12, 128, 8960, 30)
    m = ct.c_size_t()
    assert L.hsa_workspace_size(ct.byref(plain), ct.byref(m)) == 0
    assert n.value > m.value                               # timestep vectors
    bad = H.make_dims(32760, 16, 1536, 12, 128, 8960, 30, features=16)
    assert L.hsa_workspace_size(ct.byref(bad), ct.byref(n)) == -1   # unknown feature bit
    bad = H.make_dims(32760, 16, 1536, 12, 128, 8960, 30, features=("rope3d",), grid=(21, 30, 51))
    assert L.hsa_workspace_size(ct.byref(bad), ct.byref(n)) == -2   # grid does not cover N
    bad = H.make_dims(32760, 16, 1536, 12, 128, 8960, 30, features=("cfg",))
    assert L.hsa_workspace_size(ct.byref(bad), ct.byref(n)) == -1   # guidance needs text
    cfg = H.make_dims(32760, 16, 1536, 12, 128, 8960, 30, n_text=512, features=("cfg",))
    assert L.hsa_workspace_size(ct.byref(cfg), ct.byref(n)) == 0
    null = None
    assert L.hsa_guidance(null, null, 4, 6, 1.0, null) == -2        # C % 4
    assert L.hsa_guidance(null, null, 4, 8, float("nan"), null) == -1
    assert L.hsa_qk_norm_rope(null, null, null, 4, ct.byref(ok), null, null, null) == -1


def test_feature_parameters_are_required_by_the_model():
    L = H.load()
    d = H.make_dims(256, 16, 128, 2, 64, 512, 1, dtype=None, features=("qk_norm",))
    d.dtype = H.HSA_F32
    blocks = (H.Block * 1)()
    for n in ("w_qkv", "w_o", "w_1", "w_2", "k_cache", "v_cache"):
        setattr(blocks[0], n, 0x1000)
    m = H.Model(d, 0x1000, 0x1000, blocks)
    st = H.State(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 1 << 40)
    sched = H.make_schedule(8, [8, 4], [128, 128])
    assert L.hsa_step(ct.byref(m), ct.byref(sched), ct.byref(st), 0, 1.0, 0.875, 0, None, None) == -1
    blocks[0].q_gain = blocks[0].k_gain = 0x1000
    d.features = H.FEAT_QK_NORM | H.FEAT_ADALN                 # timestep MLP and mod missing
    m = H.Model(d, 0x1000, 0x1000, blocks)
    assert L.hsa_step(ct.byref(m), ct.byref(sched), ct.byref(st), 0, 1.0, 0.875, 0, None, None) == -1
    assert L.hsa_time_embed(ct.byref(m), 0.5, ct.c_void_p(0x1000), ct.c_void_p(0x1000), None) == -1
    # time embedding needs the adaLN feature
    d.features = 0
    m = H.Model(d, 0x1000, 0x1000, blocks)
    assert L.hsa_time_embed(ct.byref(m), 0.5, ct.c_void_p(0x1000), ct.c_void_p(0x1000), None) == -1


def test_binding_checks_feature_tensors():
    import torch
    bf = torch.bfloat16
    d = H.make_dims(64, 16, 256, 2, 128, 512, 1, features=("qk_norm", "adaln"))
    blk = {"w_qkv": torch.zeros(768, 256, dtype=bf), "w_o": torch.zeros(256, 256, dtype=bf),
           "w_1": torch.zeros(512, 256, dtype=bf), "w_2": torch.zeros(256, 512, dtype=bf),
           "k_cache": torch.zeros(64, 256, dtype=bf), "v_cache": torch.zeros(64, 256, dtype=bf),
           "q_gain": torch.ones(256), "k_gain": torch.ones(256)}
    with pytest.raises(ValueError, match="mod missing"):
        H.DeviceModel(d, torch.zeros(256, 16, dtype=bf), torch.zeros(16, 256, dtype=bf), [blk])
    blk["mod"] = torch.zeros(6, 256, dtype=bf)
    with pytest.raises(ValueError, match="mod"):
        H.DeviceModel(d, torch.zeros(256, 16, dtype=bf), torch.zeros(16, 256, dtype=bf), [blk])
    blk["mod"] = torch.zeros(6, 256)
    with pytest.raises(ValueError, match="timestep weights missing"):
        H.DeviceModel(d, torch.zeros(256, 16, dtype=bf), torch.zeros(16, 256, dtype=bf), [blk])


def test_header_and_library_from_plain_c(tmp_path):
    """include/hsa.h compiles as C99 with warnings as errors, and a C program
    linked against libhsa.so gets the same host-side answers (ABI version,
    closed-form |A_i|, workspace size, shape errors) as the binding."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    libdir = os.path.dirname(H.lib_path())
    exe = str(tmp_path / "c_abi_check")
    cmd = [cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(root, "include"),
           os.path.join(root, "tests", "c_abi_check.c"), "-L", libdir, "-lhsa",
           f"-Wl,-rpath,{libdir}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "c abi ok" in r.stdout, (r.returncode, r.stdout, r.stderr)


# Sanitizers for the host side only: each flag sits directly after -Xarch_host,
# so the device code is compiled as usual and no GPU sanitizer is involved.
HOST_SANITIZERS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fno-sanitize-recover=all"]


def test_host_validation_under_sanitizers(tmp_path):
    """The library's host code (argument validation, workspace layout, launch
    sequencing) built with AddressSanitizer and UndefinedBehaviorSanitizer,
    and tests/c_abi_check.c (every entry point family called with invalid
    arguments, plus the host-only calls) built with both and run against it:
    no sanitizer report, every call returns its documented status."""
    import concurrent.futures as cf
    import shutil
    import subprocess
    from token_sparse_attention_compact_amd import build as B
    clang = "/opt/rocm/llvm/bin/clang"
    if not os.path.exists(clang):
        pytest.skip("ROCm clang not found")
    cc = B.hipcc()
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    flags = [f for f in B.FLAGS if f != "-O3"] + ["-O1", "-g"]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = [cc, *flags, *HOST_SANITIZERS, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stdout + r.stderr
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
        objs = list(ex.map(compile_one, B.sources()))
    lib = str(tmp_path / "libhsa_san.so")
    r = subprocess.run([cc, "-shared", "-fPIC", f"--offload-arch={B.ARCH}", *objs, "-o", lib],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    exe = str(tmp_path / "c_abi_san")
    san_c = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    r = subprocess.run([clang, "-std=c99", "-g", *san_c, "-I", os.path.join(root, "include"),
                        os.path.join(root, "tests", "c_abi_check.c"), lib,
                        f"-Wl,-rpath,{tmp_path}", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and "c abi ok" in r.stdout, (r.returncode, r.stdout, r.stderr[-3000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
