"""The streaming-read probe (dwkv_stream_probe, a measurement aid) through
the C ABI (needs an MI355X): every 16-byte piece of the buffer is read and
folded as its header states.  Each thread's fold is recomputed on the host
from the buffer's words: with `magic` set to one thread's fold the kernel
stores it to sink[0]; with a value no thread folds to, the sink is left as
it was."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _folds(words: np.ndarray, workgroups: int, threads: int) -> np.ndarray:
    """Every thread's fold: pieces lo + tid, lo + tid + nt, ... of its
    workgroup's share, four at a time as (x_a + x_b + x_c + x_d) into an
    xor, then one at a time (x = xor of a piece's four words)."""
    x = np.bitwise_xor.reduce(words.reshape(-1, 4), axis=1).astype(np.uint64)
    n16 = x.size
    per = (n16 + workgroups - 1) // workgroups
    out = np.zeros((workgroups, threads), np.uint64)
    m = np.uint64(0xFFFFFFFF)
    for wg in range(workgroups):
        lo, hi = wg * per, min(wg * per + per, n16)
        for t in range(threads):
            acc, i = np.uint64(0), lo + t
            while i + 3 * threads < hi:
                acc ^= (x[i] + x[i + threads] + x[i + 2 * threads] + x[i + 3 * threads]) & m
                i += 4 * threads
            while i < hi:
                acc ^= x[i]
                i += threads
            out[wg, t] = acc
    return out


@pytest.mark.parametrize("nbytes,workgroups,threads", [(1 << 16, 4, 256), (40000, 3, 64), (16, 2, 64)])
def test_stream_probe_reads_every_piece(nbytes, workgroups, threads):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from compressed_kv_cache_dwkv_amd import dwkv_stream_probe
    rng = np.random.default_rng(nbytes + workgroups)
    words = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    print(f"stream probe test: {nbytes} bytes, {workgroups} x {threads}", flush=True)
    src = torch.from_numpy(words.view(np.int32).copy()).cuda()
    folds = _folds(words, workgroups, threads)
    # a thread that read at least one piece, and its fold
    per = (nbytes // 16 + workgroups - 1) // workgroups
    wg, t = (1 if workgroups > 1 and nbytes > 16 else 0), (5 if per > 5 else 0)
    magic = int(folds[wg, t])
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    dwkv_stream_probe(src, nbytes, workgroups, threads, magic, sink)
    torch.cuda.synchronize()
    assert int(sink[0].item()) & 0xFFFFFFFF == magic
    # a value no thread folds to: nothing is stored
    taken = set(int(v) for v in folds.reshape(-1))
    other = next(v for v in range(1, 1 << 20) if v not in taken)
    sink.fill_(-7)
    dwkv_stream_probe(src, nbytes, workgroups, threads, other, sink)
    torch.cuda.synchronize()
    assert sink.cpu().tolist() == [-7, -7, -7, -7]
