"""Build and call the test-only probe library (tests/gather_probe.hip): the
kernels' own K/V tile gathers, with each gathered tile copied out densely so
a test can compare it bit for bit with a host gather; the transposing LDS
read's lane map; the kernels' fp8 conversion of every e4m3 code."""
import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "gather_probe.hip")
LIB = os.path.join(HERE, "libua_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

RING, REGISTERS, LOADER16 = 0, 1, 2
TO_16BIT, FP8_TO_BF16, FP8_TO_F16 = 0, 1, 2


def build() -> str:
    """Compile libua_probe.so in-tree for gfx950 (always rebuilds)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           f"-I{ROOT}/include", f"-I{ROOT}/varlen_attention_serving_amd/csrc", SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("gather probe build failed:\n" + r.stderr[-4000:])
    os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built (run __graft_entry__.build())")
        import torch  # noqa: F401  (bind to torch's HIP runtime first)
        _lib = ctypes.CDLL(LIB)
        _lib.uap_gather.restype = ctypes.c_int
        _lib.uap_gather.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
            ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p]
        _lib.uap_read_tr.restype = ctypes.c_int
        _lib.uap_read_tr.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        _lib.uap_fp8_codes.restype = ctypes.c_int
        _lib.uap_fp8_codes.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    return _lib


def gather(batch, tiles, path, waves=4, fp8_to=TO_16BIT):
    """Gather the (sequence, kv-head, tile) triples in `tiles` (int32 [n, 3]
    device tensor) with the chosen device gather; returns int16 tensors
    [n, 32, d] for K and V."""
    import torch
    w = batch.w
    n = int(tiles.shape[0])
    out_k = torch.zeros((n, 32, w.head_dim), dtype=torch.int16, device=tiles.device)
    out_v = torch.zeros_like(out_k)
    rc = lib().uap_gather(path, waves, fp8_to, w.head_dim, batch.k.data_ptr(), batch.v.data_ptr(),
                          batch.block_table.data_ptr(), batch.seq_lens.data_ptr(),
                          int(w.block_table.shape[1]), int(w.block_size).bit_length() - 1,
                          w.num_kv_heads * w.head_dim, tiles.data_ptr(), n, out_k.data_ptr(),
                          out_v.data_ptr(), torch.cuda.current_stream().cuda_stream)
    if rc != 0:
        raise RuntimeError(f"uap_gather returned {rc}")
    torch.cuda.synchronize()
    return out_k, out_v


def read_tr(addr):
    """One wave's ds_read_b64_tr_b16 over an LDS image whose element x holds x:
    lane l reads at element offset addr[l] (int32 [64] device tensor,
    multiples of 4 below 4093); returns uint16 numpy [64, 4] of what each lane
    received."""
    import torch
    out = torch.zeros((64, 4), dtype=torch.int16, device=addr.device)
    rc = lib().uap_read_tr(addr.data_ptr(), out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    if rc != 0:
        raise RuntimeError(f"uap_read_tr returned {rc}")
    torch.cuda.synchronize()
    return out.cpu().numpy().view("uint16")


def fp8_codes():
    """The 256 e4m3 codes through the kernels' conversion: uint16 numpy [256]
    bf16 bits and [256] f16 bits, in code order."""
    import torch
    ob = torch.zeros(256, dtype=torch.int16, device="cuda")
    oh = torch.zeros_like(ob)
    rc = lib().uap_fp8_codes(ob.data_ptr(), oh.data_ptr(), torch.cuda.current_stream().cuda_stream)
    if rc != 0:
        raise RuntimeError(f"uap_fp8_codes returned {rc}")
    torch.cuda.synchronize()
    return ob.cpu().numpy().view("uint16"), oh.cpu().numpy().view("uint16")
