"""The C ABI from a native client: tests/native/chunk_loop.cpp runs a bf16
chunk loop (first chunk finished by attn_rope_qkv, then
attn_prefill_chunk_deferred per chunk with two workspaces, then
attn_prefill_finish) on hipMalloc'd buffers without PyTorch, and checks the
key cache bit for bit and every output row against the C oracle."""
import ctypes
import os

import pytest

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "libchunk_loop_check.so")


@pytest.mark.gpu
def test_native_chunk_loop():
    assert os.path.exists(LIB), "native client not built: run __graft_entry__.build() first"
    import torch

    assert torch.cuda.is_available()
    torch.cuda.set_device(0)
    lib = ctypes.CDLL(LIB)
    lib.chunk_loop_check.argtypes = [ctypes.c_char_p, ctypes.c_int]
    lib.chunk_loop_check.restype = ctypes.c_int
    buf = ctypes.create_string_buffer(512)
    print("native chunk loop: T=700 chunk=128 heads 32/8 hd 128", flush=True)
    rc = lib.chunk_loop_check(buf, len(buf))
    report = buf.value.decode()
    print(report, flush=True)
    assert rc == 0, f"native chunk loop failed (status {rc}): {report}"
