"""Build and run the ceiling probes (tests/ceiling_probe.hip) and the library
GEMM rate: what the MI355X delivers to a read-only stream and to the decode
kernel's paged reads without its math (plain and non-temporal loads), to a
bf16 hipBLASLt GEMM, and the issue cost of v_exp_f32 against v_fma_f32.

    python tests/ceilings.py        one JSON line of the figures (needs a GPU)
"""
import ctypes
import json
import os
import subprocess
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "ceiling_probe.hip")
LIB = os.path.join(HERE, "libua_ceiling.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HBM_PEAK_GBS = 8000.0
KINDS = {"fma": 0, "exp": 1, "fma+exp": 2}


def build() -> str:
    """Compile libua_ceiling.so in-tree for gfx950 (always rebuilds)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("ceiling probe build failed:\n" + r.stderr[-4000:])
    os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built (run __graft_entry__.build())")
        import torch  # noqa: F401  (bind to torch's HIP runtime first)
        L = ctypes.CDLL(LIB)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.uac_stream_read.restype = i32
        L.uac_stream_read.argtypes = [vp, i64, i32, i32, vp, vp]
        L.uac_paged_read.restype = i32
        L.uac_paged_read.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, i32, vp, vp]
        L.uac_issue_rate.restype = i32
        L.uac_issue_rate.argtypes = [i32, i32, i32, vp, vp, vp, vp]
        _lib = L
    return _lib


def _time(fn, reps, warmup=3):
    """Median ms of fn() over `reps` launches, HIP events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    st = torch.cuda.current_stream()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        fn()
        b.record(st)
        b.synchronize()
        ts.append(a.elapsed_time(b))
    return float(np.median(ts))


def stream_read(nbytes=4 << 30, blocks_per_cu=8, reps=20, nt=False):
    """Read-only streaming bandwidth (GB/s) over an `nbytes` buffer (nt:
    non-temporal loads)."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = cus * blocks_per_cu
    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").random_()
    out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    L = lib()

    def run():
        rc = L.uac_stream_read(src.data_ptr(), nbytes, blocks, int(nt), out.data_ptr(), s)
        assert rc == 0, rc
    ms = _time(run, reps)
    return {"GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes": nbytes, "ms": round(ms, 4),
            "workgroups": blocks}


def paged_read(seed=2, reps=20, block_size=16, num_kv_heads=8, workers_per_cu=1, nt=False):
    """The decode batch's K/V traffic alone: 64 sequences of S_k ~ U{512..8192}
    (the decode batch's lengths), 16-key blocks in random order, 8 kv heads,
    d = 128, 16-bit; GB/s of K+V bytes visited (nt: non-temporal loads)."""
    import torch
    from varlen_attention_serving_amd import workloads as W
    sp = W.named_spec("decode_batch")
    seq_lens = np.asarray(sp["seq_lens"], dtype=np.int64)
    n = seq_lens.size
    blocks_per = (seq_lens + block_size - 1) // block_size
    num_blocks = int(blocks_per.sum())
    g = torch.Generator(device="cuda").manual_seed(seed)
    perm = torch.randperm(num_blocks, device="cuda", generator=g).to(torch.int32)
    bt_stride = int(blocks_per.max())
    table = torch.full((n, bt_stride), -1, dtype=torch.int32, device="cuda")
    first = np.concatenate([[0], np.cumsum(blocks_per)])
    for s in range(n):
        table[s, :blocks_per[s]] = perm[first[s]:first[s + 1]]
    slot_elems = num_kv_heads * 128
    k = torch.empty(num_blocks * block_size * slot_elems, dtype=torch.int16, device="cuda").random_()
    v = torch.empty_like(k).random_()
    tiles = (seq_lens + 31) // 32
    tile_seq = torch.from_numpy(np.repeat(np.arange(n), tiles).astype(np.int32)).cuda()
    tile_idx = torch.from_numpy(np.concatenate([np.arange(t) for t in tiles]).astype(np.int32)).cuda()
    n_tiles = int(tiles.sum())
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    workers = cus * workers_per_cu
    out = torch.empty(workers * 64 * num_kv_heads, dtype=torch.int32, device="cuda")
    sl = torch.from_numpy(seq_lens.astype(np.int32)).cuda()
    s = torch.cuda.current_stream().cuda_stream
    L = lib()
    lb = int(np.log2(block_size))

    def run():
        rc = L.uac_paged_read(k.data_ptr(), v.data_ptr(), table.data_ptr(), sl.data_ptr(),
                              tile_seq.data_ptr(), tile_idx.data_ptr(), n_tiles, bt_stride, lb,
                              num_kv_heads, workers, int(nt), out.data_ptr(), s)
        assert rc == 0, rc
    ms = _time(run, reps)
    kv_bytes = int(seq_lens.sum()) * num_kv_heads * 128 * 2 * 2
    return {"GB/s": round(kv_bytes / (ms * 1e-3) / 1e9, 1), "kv_bytes": kv_bytes,
            "ms": round(ms, 4), "workgroups": workers}


def issue_rate(iters=4096, reps=3):
    """Shader-clock cycles per wave64 instruction (one wave per workgroup,
    one workgroup per CU) of each kind, and the clock they ran at (MHz)."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    cyc = torch.zeros(cus, dtype=torch.int64, device="cuda")
    tick = torch.zeros(cus, dtype=torch.int64, device="cuda")
    sink = torch.empty(cus * 64, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    L = lib()
    res = {}
    for name, kind in KINDS.items():
        best = None
        for _ in range(reps):
            rc = L.uac_issue_rate(kind, iters, cus, cyc.data_ptr(), tick.data_ptr(),
                                  sink.data_ptr(), s)
            assert rc == 0, rc
            torch.cuda.synchronize()
            c = float(np.median(cyc.cpu().numpy()))
            t = float(np.median(tick.cpu().numpy()))
            per = c / (iters * 128)
            if best is None or per < best[0]:
                best = (per, c / (t / 100.0))  # ticks are 100 MHz
        res[name] = {"cycles_per_instruction": round(best[0], 3), "clock_mhz": round(best[1], 1)}
    return res


def gemm(n=8192, reps=10):
    """bf16 torch.matmul (hipBLASLt) of n x n by n x n: TFLOP/s."""
    import torch
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    ms = _time(lambda: torch.matmul(a, b, out=c), reps)
    return {"TFLOP/s": round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1), "n": n, "ms": round(ms, 4)}


def main():
    import torch
    if not torch.cuda.is_available():
        print("ceilings.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    sys.path.insert(0, ROOT)
    out = {"stream_read": stream_read(), "stream_read_nt": stream_read(nt=True),
           "paged_read": paged_read(), "paged_read_nt": paged_read(nt=True),
           "issue_rate": issue_rate(), "gemm_bf16": gemm()}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
