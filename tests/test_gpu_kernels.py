"""Kernel-level parity on the GPU through the C ABI's single-kernel entry
points: the bf16 MFMA GEMM in every operand layout (against a CPU fp64
product of the same bf16 inputs) and causal GQA attention (against the
oracle)."""
import math

import pytest
import torch

import synth
from oracle import stage as O
from _helpers import ensure_built, max_rel, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    return ensure_built()


def _ctx(B, **kw):
    base = dict(name="k", hidden=256, n_q=4, n_kv=2, head_dim=128, ffn=512, batch=1, seq=64, dtype="bf16")
    base.update(kw)
    return B.Context(synth.StageConfig(**base))


def _operand(rows, cols, kmajor, seed, name):
    """Logical [rows, K=cols] operand stored K-major ([rows, cols]) or
    transposed ([cols, rows]); returns (storage, logical fp64)."""
    t = synth.normal((rows, cols), seed, name, dtype=torch.bfloat16)
    store = t if kmajor else t.t().contiguous()
    return store, t.double()


GEMM_CASES = [
    # M, N, K  (ragged tiles, K tail, both tile configurations)
    (200, 136, 264),
    (64, 8, 8),
    (1000, 520, 72),
    (4096, 4096, 128),   # 256x256 tiles
    (4104, 4232, 200),   # 256x256 tiles with ragged edges
    # 256x256 tiles, a tile count divisible by 8 (tiles dealt to the XCDs in
    # contiguous ranges) and a last group of tile rows shorter than the others
    (1272, 12288, 72),   # 5 x 48 tiles
    (1496, 10240, 136),  # 6 x 40 tiles
]


@pytest.mark.parametrize("M,N,K", GEMM_CASES)
@pytest.mark.parametrize("ak,bk", [(True, True), (True, False), (False, False), (False, True)])
def test_gemm_bf16_layouts(B, M, N, K, ak, bk):
    say("gemm", M, N, K, ak, bk)
    ctx = _ctx(B)
    a_s, a = _operand(M, K, ak, 11, f"A{M}{K}")
    b_s, b = _operand(N, K, bk, 12, f"B{N}{K}")
    ref = a @ b.T
    dev = torch.device("cuda")
    A, Bm = a_s.to(dev), b_s.to(dev)
    lda = K if ak else M
    ldb = K if bk else N
    C32 = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    ctx.op_gemm_bf16(M, N, K, A, lda, ak, Bm, ldb, bk, C32, N, out_f32=True)
    C16 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ctx.op_gemm_bf16(M, N, K, A, lda, ak, Bm, ldb, bk, C16, N, out_f32=False)
    ctx.sync()
    err32 = max_rel(C32, ref)
    err16 = max_rel(C16, ref)
    assert err32 < 1e-5, err32
    assert err16 < 2 ** -8, err16
    # bf16 output = fp32 output rounded once
    assert torch.equal(C16.cpu(), C32.cpu().to(torch.bfloat16))


@pytest.mark.parametrize("rows,cols,pad", [
    (8, 8, 0), (128, 64, 0), (136, 24, 8), (200, 4104, 0), (1000, 200, 16), (8, 1000, 8), (2056, 72, 0),
])
def test_transpose_bf16(B, rows, cols, pad):
    """The weight-gradient activation transpose: bit-exact against torch on
    single, ragged and several tiles (128 source rows x 64 columns), with
    padded leading dimensions whose padding must stay untouched."""
    say("transpose", rows, cols, pad)
    ctx = _ctx(B)
    dev = torch.device("cuda")
    src_full = synth.normal((rows, cols + pad), 21, f"tr{rows}{cols}", dtype=torch.bfloat16).to(dev)
    src = src_full[:, :cols]
    dst = torch.full((cols, rows + pad), -7.0, dtype=torch.bfloat16, device=dev)
    ctx.op_transpose_bf16(src, dst)
    ctx.sync()
    got = dst.cpu()
    assert torch.equal(got[:, :rows], src.cpu().t())
    assert torch.all(got[:, rows:] == -7.0)


@pytest.mark.parametrize("rows,cols", [(8192, 4096), (8192, 32064), (8192, 28672)])
def test_transpose_bf16_full_size(B, rows, cols):
    """Transposes at the step's sizes (8192 tokens x the hidden width 4096,
    and x the larger widths 28672, 32064), every element bit-exact,
    compared on the device."""
    say("transpose full size", rows, cols)
    ctx = _ctx(B)
    dev = torch.device("cuda")
    g = torch.Generator(device=dev).manual_seed(rows + cols)
    src = torch.randn(rows, cols, generator=g, device=dev).to(torch.bfloat16)
    dst = torch.empty(cols, rows, dtype=torch.bfloat16, device=dev)
    ctx.op_transpose_bf16(src, dst)
    ctx.sync()
    assert torch.equal(dst, src.t())


def test_gemm_accumulate_and_strided_output(B):
    say("gemm accumulate")
    ctx = _ctx(B)
    M, N, K = 300, 96, 128
    a_s, a = _operand(M, K, True, 1, "a")
    b_s, b = _operand(N, K, False, 2, "b")
    dev = torch.device("cuda")
    base = synth.normal((M, N + 8), 3, "c")
    C = base.clone().to(dev)
    ctx.op_gemm_bf16(M, N, K, a_s.to(dev), K, True, b_s.to(dev), N, False, C, N + 8, out_f32=True, accumulate=True)
    ctx.sync()
    ref = base.double().clone()
    ref[:, :N] += a @ b.T
    assert max_rel(C, ref) < 1e-5
    assert torch.equal(C[:, N:].cpu(), base[:, N:])  # columns past N untouched


@pytest.mark.parametrize("dtype,d,nq,nkv,batch,seq,qk_scale", [
    ("f32", 64, 4, 4, 2, 50, 1.0),
    ("bf16", 128, 4, 2, 2, 200, 1.0),
    ("bf16", 128, 8, 2, 1, 333, 1.0),
    ("bf16", 128, 2, 1, 1, 1, 1.0),
    ("bf16", 128, 2, 1, 1, 64, 1.0),
    ("bf16", 128, 4, 4, 3, 130, 1.0),
    ("bf16", 128, 8, 2, 1, 1000, 1.0),
    ("bf16", 128, 4, 1, 1, 2049, 1.0),
    # scores with a spread of ~16 (in natural-log units): the running max of
    # a query keeps jumping well past the rescale threshold of the forward
    ("bf16", 128, 4, 2, 1, 700, 4.0),
])
def test_attention_fwd_bwd(B, dtype, d, nq, nkv, batch, seq, qk_scale):
    say("attention", dtype, d, nq, nkv, batch, seq, qk_scale)
    ctx = _ctx(B, n_q=nq, n_kv=nkv, head_dim=d, hidden=max(256, nq * d), dtype=dtype)
    T = batch * seq
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    W = (nq + 2 * nkv) * d
    qkv = synth.normal((T, W), 5, f"qkv{T}{W}")
    qkv[:, :(nq + nkv) * d] *= qk_scale
    qkv = qkv.to(dt)
    dout = synth.normal((T, nq * d), 5, f"do{T}", dtype=dt)
    dev = torch.device("cuda")
    o = torch.empty(T, nq * d, dtype=dt, device=dev)
    lse = torch.empty(nq, T, dtype=torch.float32, device=dev)
    dqkv = torch.empty(T, W, dtype=dt, device=dev)
    ws = torch.empty(nq * T * 4 + 256, dtype=torch.uint8, device=dev)
    qkv_d = qkv.to(dev)
    ctx.op_attn_fwd(batch, seq, qkv_d, o, lse)
    ctx.op_attn_bwd(batch, seq, qkv_d, o, dout.to(dev), lse, dqkv, ws)
    ctx.sync()
    # oracle on the same inputs
    x = qkv.double().requires_grad_(True)
    q = x[:, :nq * d].reshape(T, nq, d)
    k = x[:, nq * d:(nq + nkv) * d].reshape(T, nkv, d)
    v = x[:, (nq + nkv) * d:].reshape(T, nkv, d)
    ref = O.causal_attention(q, k, v, batch, seq).reshape(T, nq * d)
    (gref,) = torch.autograd.grad((ref * dout.double()).sum(), [x])
    tol = 1e-4 if dtype == "f32" else 2e-2
    assert max_rel(o, ref.detach()) < tol
    assert max_rel(dqkv, gref) < tol
    # lse is log sum exp of the scaled causal scores
    s = torch.einsum("thd,uhd->htu", q.detach(), k.detach().repeat_interleave(nq // nkv, dim=1)) / math.sqrt(d)
    pos = torch.arange(seq).repeat(batch)
    row = torch.arange(T) // seq
    mask = (pos[None, :] <= pos[:, None]) & (row[None, :] == row[:, None])
    lref = torch.logsumexp(s.masked_fill(~mask[None], float("-inf")), dim=-1)
    assert (lse.cpu().double() - lref).abs().max().item() < (1e-4 if dtype == "f32" else 2e-2)


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (3 << 20) + 48])
def test_copy_is_bit_exact(B, nbytes):
    ctx = _ctx(B)
    g = torch.Generator().manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g)
    dst = torch.zeros(nbytes + 32, dtype=torch.uint8, device="cuda")
    s = src.to("cuda")
    say(f"copy {nbytes} bytes")
    ctx.op_copy(dst, s)
    ctx.sync()
    out = dst.cpu()
    assert torch.equal(out[:nbytes], src)
    assert not out[nbytes:].any()  # nothing written past the end
    with pytest.raises(B.RPError):
        ctx.op_copy(dst[1:17], s[:16])  # misaligned destination


def test_bf16_output_rounding_is_nearest_even(B):
    """bf16 outputs round fp32 to nearest even exactly like torch: C = A B^T
    with selector rows in A (ones at k = m and k = m + 8) makes every output an
    fp32 sum of two bf16 values, many of them exact ties between two bf16
    neighbours; the bf16 result must equal torch's rounding of that sum bit
    for bit (finite values, including subnormal and huge magnitudes)."""
    ctx = _ctx(B)
    M, N, K = 64, 96, 80
    g = torch.Generator().manual_seed(11)
    A = torch.zeros(M, K, dtype=torch.bfloat16)
    for m in range(M):
        A[m, m] = 1.0
        A[m, m + 8] = 1.0
    # B entries: random magnitudes over a wide exponent range, pairs chosen so
    # that sums need rounding (ties included: b2 = b1 * 2^-8 lands on a tie)
    base = torch.randn(N, K, generator=g) * torch.exp2(torch.randint(-100, 100, (N, K), generator=g).float())
    Bm = base.to(torch.bfloat16)
    Bm[:, 8:16] = (Bm[:, 0:8].float() * 2.0 ** -8).to(torch.bfloat16)
    ref = (Bm.float()[:, :M] + Bm.float()[:, 8:M + 8]).t().contiguous().to(torch.bfloat16)
    C = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    say("bf16 rounding")
    ctx.op_gemm_bf16(M, N, K, A.cuda(), K, True, Bm.cuda(), K, True, C, N, False)
    ctx.sync()
    got = C.cpu()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_embed_out_of_range_ids_give_zero_rows(B):
    """Token embedding with ids outside [0, vocab) (a padding id of -100, vocab
    itself, a large id): those rows of x0 are zero and the backward ignores
    them; the valid rows gather and scatter-add as the oracle does."""
    say("embedding with out-of-range ids")
    cfg = synth.config("tiny")
    ctx = B.Context(cfg)
    V, H = cfg.vocab, cfg.hidden
    table = synth.normal((V, H), 5, "embed_table", 0.02)
    ids = synth.uniform_int((300,), V, 5, "embed_ids")
    ids[[0, 7, 150, 299]] = torch.tensor([-100, V, 1 << 30, -1], dtype=torch.int32)
    ids[10:20] = 3  # repeated id: its gradient row sums ten token rows
    dx0 = synth.normal((300, H), 5, "embed_dx0")
    dev = torch.device("cuda")
    x0 = torch.full((300, H), float("nan"), device=dev)
    dtable = torch.full((V, H), float("nan"), device=dev)
    ids_d, table_d, dx0_d = ids.to(dev), table.to(dev), dx0.to(dev)
    torch.cuda.synchronize()
    ctx.embed_fwd(ids_d, table_d, x0)
    ctx.embed_bwd(ids_d, dx0_d, dtable)
    ctx.sync()
    ok = (ids >= 0) & (ids < V)
    x0 = x0.cpu()
    assert torch.equal(x0[~ok], torch.zeros(int((~ok).sum()), H))
    assert torch.equal(x0[ok], O.embed(ids[ok], table))
    ref = O.embed_backward(ids[ok], dx0[ok].double(), V)
    assert max_rel(dtable, ref) < 1e-6


@pytest.mark.parametrize("M,N,K,ldc,out_f32,accumulate", [
    (70, 131, 80, 131, True, False),    # row stride not a multiple of 4: element-wise epilogue
    (70, 131, 80, 131, False, False),
    (300, 1002, 136, 1002, False, False),  # N = 2 mod 4: a partial last group of four columns
    (300, 94, 128, 100, True, True),    # aligned stride, partial last group, accumulation
    (257, 520, 64, 520, False, False),  # ragged rows, whole groups
])
def test_gemm_epilogue_edges(B, M, N, K, ldc, out_f32, accumulate):
    """The epilogue's four-column accesses: vector accesses only where the row
    stride and base allow, element-wise otherwise, columns past N untouched."""
    say("gemm epilogue", M, N, K, ldc, out_f32, accumulate)
    ctx = _ctx(B)
    a_s, a = _operand(M, K, True, 31, f"ea{M}{K}")
    b_s, b = _operand(N, K, True, 32, f"eb{N}{K}")
    dev = torch.device("cuda")
    dt = torch.float32 if out_f32 else torch.bfloat16
    base = synth.normal((M, ldc), 33, f"ec{M}{ldc}").to(dt)
    C = base.clone().to(dev)
    ctx.op_gemm_bf16(M, N, K, a_s.to(dev), K, True, b_s.to(dev), K, True, C, ldc, out_f32=out_f32,
                     accumulate=accumulate)
    ctx.sync()
    ref = a @ b.T
    if accumulate:
        ref = ref + base[:, :N].double()
    tol = 1e-5 if out_f32 else 2 ** -8
    assert max_rel(C[:, :N], ref) < tol
    assert torch.equal(C[:, N:].cpu(), base[:, N:])  # columns past N untouched


@pytest.mark.parametrize("ak,bk,ldc,out_f32,accumulate", [
    (False, True, 4233, True, True),     # M-major A: the 64 x 128 wave tiles; element-wise epilogue
    (False, True, 4232, False, False),   # the same tiles, bf16 four-column stores
    (False, False, 4236, True, True),    # both operands M-major, aligned stride, accumulation
    (True, False, 4233, True, False),    # M-major B
])
def test_gemm_mmajor_epilogue_edges(B, ak, bk, ldc, out_f32, accumulate):
    """The layouts with an M-major operand (the weight- and input-gradient
    products) at a size that takes the 256 x 256 tiles, with ragged edges, a
    K tail, padded row strides and fp32 accumulation; columns past N are left
    untouched."""
    M, N, K = 4104, 4232, 136
    say("gemm m-major epilogue", ak, bk, ldc, out_f32, accumulate)
    ctx = _ctx(B)
    dev = torch.device("cuda")
    a_s, a = _operand(M, K, ak, 34, f"ma{M}{K}")
    b_s, b = _operand(N, K, bk, 35, f"mb{N}{K}")
    dt = torch.float32 if out_f32 else torch.bfloat16
    base = synth.normal((M, ldc), 36, f"mc{M}{ldc}").to(dt)
    C = base.clone().to(dev)
    ctx.op_gemm_bf16(M, N, K, a_s.to(dev), K if ak else M, ak, b_s.to(dev), K if bk else N, bk, C, ldc,
                     out_f32=out_f32, accumulate=accumulate)
    ctx.sync()
    ref = a @ b.T
    if accumulate:
        ref = ref + base[:, :N].double()
    tol = 1e-5 if out_f32 else 2 ** -8
    assert max_rel(C[:, :N], ref) < tol
    assert torch.equal(C[:, N:].cpu(), base[:, N:])
