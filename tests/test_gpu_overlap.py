"""Two exchanges on one GPU at once: the key exchange (keys_exchange) on a
second stream of default priority while other work runs on the main stream,
the arrangement the page "Different nccl stream within EmbeddingKey alltoall
and EmbeddingValue..." (TorchRec, description) gives the key alltoall. The
neighbours are the a2av (one call and three calls) and a bf16 GEMM the size of
one expert's. Every repetition's results are compared with the oracle byte
for byte, with guard bands around every buffer."""
import numpy as np
import pytest
import torch

from embeddings_a2av_virtual_amd import _binding as B
from embeddings_a2av_virtual_amd import inputs as I
from embeddings_a2av_virtual_amd.vranks import A2av
from gpu_util import GuardedBuffer, SENT, assert_same, ref_a2av, upload_rows

pytestmark = pytest.mark.gpu

REPS = 4


def _say(*a):
    print(*a, flush=True)


class KeyJob:
    """The fused key exchange of one batch, with its buffers on the device."""

    def __init__(self, ref, W, NT, batch, seed, lam=20.0, cap=100):
        g = I.rng(seed)
        ranks = [I.emb_keys_rank(g, tables=NT, batch=batch, lam=lam, cap=cap) for _ in range(W)]
        self.W, self.NT, self.batch = W, NT, batch
        self.lengths = [r.lengths for r in ranks]
        self.keys = [r.keys for r in ranks]
        self.want = ref.keys_exchange(W, NT, batch, self.lengths, self.keys)
        assert self.want[0] == 0
        self.lcap = [x.size for x in self.want[1]]
        self.kcap = [x.size for x in self.want[2]]
        self.lin = [upload_rows(l.reshape(-1).view(np.uint8)) for l in self.lengths]
        self.kin = [upload_rows(k.view(np.uint8)) for k in self.keys]
        self.lout = [GuardedBuffer(c * 4) for c in self.lcap]
        self.kout = [GuardedBuffer(c * 8) for c in self.kcap]
        z = dict(dtype=torch.int64, device="cuda")
        self.sk = torch.empty((W, W), **z)
        self.sl = torch.empty((W, W), **z)
        self.ro = torch.empty((W, W + 1), **z)
        self.ws = torch.empty(B.keys_exchange_workspace_bytes(W, NT), dtype=torch.uint8,
                              device="cuda")
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def reset(self):
        """Sentinels back in every output, on the current stream."""
        for b in self.lout + self.kout:
            b.view.fill_(SENT)
        for t in (self.sk, self.sl, self.ro):
            t.fill_(-7)
        self.status.zero_()

    def launch(self, stream):
        B.keys_exchange(self.W, self.NT, self.batch, [b.view for b in self.lin],
                        [b.view for b in self.kin], [k.size for k in self.keys],
                        [b.view for b in self.lout], self.lcap, [b.view for b in self.kout],
                        self.kcap, self.sk, self.sl, self.ro, self.ws, self.status, stream)

    def check(self, what):
        rst, rlo, rko, rsk, rsl, rro = self.want
        assert int(self.status.item()) == rst, what
        assert all(b.guards_intact() for b in self.lin + self.kin + self.lout + self.kout), what
        assert np.array_equal(self.sk.cpu().numpy(), rsk), what
        assert np.array_equal(self.sl.cpu().numpy(), rsl), what
        assert np.array_equal(self.ro.cpu().numpy(), rro), what
        for d in range(self.W):
            assert np.array_equal(self.lout[d].host().view(np.int32), rlo[d]), f"{what}: lengths {d}"
            assert np.array_equal(self.kout[d].host().view(np.int64), rko[d]), f"{what}: keys {d}"


class A2avJob:
    """One a2av of W ranks x n rows of R bytes, uniform multinomial splits."""

    def __init__(self, ref, W, n, R, seed, fused):
        g = I.rng(seed)
        self.W, self.R, self.n, self.fused = W, R, n, fused
        self.S = I.uniform_splits(g, W, n)
        self.X = [I.payload_bytes(n, R, seed * 100 + s, device="cuda").cpu().numpy()
                  for s in range(W)]
        self.want = ref_a2av(ref, R, self.X, self.S)
        self.cap = [int(c) for c in self.S.sum(axis=0)]
        self.ins = [upload_rows(x) for x in self.X]
        self.outs = [GuardedBuffer(c * R) for c in self.cap]
        self.st = A2av(W)
        self.st.set_splits(self.S)

    def reset(self):
        for b in self.outs:
            b.view.fill_(SENT)
        for t in (self.st.O, self.st.send_off, self.st.recv_off):
            t.zero_()
        self.st.status.zero_()

    def launch(self, stream):
        self.st(self.R, [b.view for b in self.ins], [self.n] * self.W, [b.view for b in self.outs],
                self.cap, stream=stream, fused=self.fused)

    def check(self, what):
        got = (int(self.st.status.item()), self.st.O.cpu().numpy(),
               self.st.send_off.cpu().numpy(), self.st.recv_off.cpu().numpy(),
               [b.host().reshape(-1, self.R) for b in self.outs],
               all(b.guards_intact() for b in self.outs + self.ins))
        assert_same(got, self.want, what)


def _side_by_side(main_job, key_job, reps=REPS, what=""):
    """Each repetition: sentinels in, then the main job on the current stream
    and the key exchange on a second stream of default priority, both released
    by one event; the main stream waits for the second before the checks."""
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()  # default priority
    for rep in range(reps):
        _say(what, "repetition", rep)
        main_job.reset()
        key_job.reset()
        go = torch.cuda.Event()
        go.record(main)
        side.wait_event(go)
        with torch.cuda.stream(side):
            key_job.launch(side)
        main_job.launch(main)
        done = torch.cuda.Event()
        done.record(side)
        main.wait_event(done)
        torch.cuda.synchronize()
        key_job.check(f"{what} rep {rep}: key exchange")
        main_job.check(f"{what} rep {rep}: neighbour")


@pytest.fixture(scope="module")
def keys_full(ref):
    """W=8, 26 tables, batch 8192, lengths min(Poisson(20), 100)."""
    return KeyJob(ref, 8, 26, 8192, seed=91)


@pytest.mark.parametrize("W,mib,fused", [(4, 32, True), (4, 32, False), (8, 32, True)],
                         ids=["w4_32mib_one_call", "w4_32mib_three_calls", "w8_32mib_one_call"])
def test_keys_exchange_beside_a2av(ref, keys_full, W, mib, fused):
    R = 8192
    job = A2avJob(ref, W, I.rows_for_mib(mib, R), R, seed=300 + W + mib, fused=fused)
    _side_by_side(job, keys_full, what=f"a2av W={W} x {mib} MiB fused={fused}")


class GemmJob:
    """A bf16 GEMM the size of one expert's (2048 rows x 7168 -> 4096); its
    result is compared with the first run's, since only the key exchange is
    under test here."""

    def __init__(self):
        g = torch.Generator().manual_seed(5)
        self.a = torch.randn(2048, 7168, generator=g).to(torch.bfloat16).cuda()
        self.b = torch.randn(7168, 4096, generator=g).to(torch.bfloat16).cuda().contiguous()
        self.c = torch.empty(2048, 4096, dtype=torch.bfloat16, device="cuda")
        self.first = None

    def reset(self):
        self.c.fill_(0)

    def launch(self, stream):
        with torch.cuda.stream(stream):
            torch.matmul(self.a, self.b, out=self.c)

    def check(self, what):
        if self.first is None:
            self.first = self.c.clone()
        assert torch.equal(self.c, self.first), what


def test_keys_exchange_beside_gemm(keys_full):
    _side_by_side(GemmJob(), keys_full, what="expert-sized GEMM")


def test_two_key_exchanges_side_by_side(ref):
    """Two batches' key exchanges, each on its own stream, with disjoint buffers."""
    a = KeyJob(ref, 8, 26, 2048, seed=92)
    b = KeyJob(ref, 8, 26, 2048, seed=93, lam=7.0, cap=30)
    _side_by_side(a, b, what="two key exchanges")
