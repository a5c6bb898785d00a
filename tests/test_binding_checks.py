"""The torch conveniences of the binding (repack, linear, accept,
tree_attention) check every tensor before its address reaches the C ABI:
shape, element size and contiguity, then that it lives on the GPU.  A wrong
tensor raises ValueError and launches nothing.  CPU tensors exercise each
rejection here (no GPU needed): the shape, size and layout checks come
before the device check."""
import pytest

torch = pytest.importorskip("torch")
w4 = pytest.importorskip("speculative_decoding_verification_w4a16_amd")


def _pk(N=256, K=512):
    qb, sb, zb = w4.w4_repacked_sizes(N, K)
    return w4.PackedLinear(torch.zeros(qb // 4, dtype=torch.int32), torch.zeros(sb // 2, dtype=torch.int16),
                           torch.zeros(zb // 2, dtype=torch.int16), N, K)


def _raises(match, fn, *args, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*args, **kw)


def test_linear_rejects_bad_activations_and_outputs():
    pk = _pk()
    _raises("shape", w4.linear, torch.zeros(4, 256, dtype=torch.int16), pk)            # K mismatch
    _raises("expected \\[M, K\\]", w4.linear, torch.zeros(512, dtype=torch.int16), pk)  # 1-D
    _raises("element", w4.linear, torch.zeros(4, 512, dtype=torch.float32), pk)         # 4-byte x
    _raises("contiguous", w4.linear, torch.zeros(512, 4, dtype=torch.int16).t(), pk)    # strided x
    _raises("GPU", w4.linear, torch.zeros(4, 512, dtype=torch.int16), pk)               # host memory
    x = torch.zeros(4, 512, dtype=torch.int16)
    _raises("shape", w4.linear, x, pk, y=torch.zeros(4, 255))                           # y too small
    _raises("element", w4.linear, x, pk, y=torch.zeros(4, 256, dtype=torch.int16))      # fp32 y of 2 bytes
    _raises("element", w4.linear, x, pk, y=torch.zeros(4, 256), out_bf16=True)          # bf16 y of 4 bytes


def test_linear_rejects_packed_arrays_of_the_wrong_size():
    pk = _pk()
    bad = w4.PackedLinear(pk.qweight_t[:-4], pk.scales_t, pk.zeros_t, pk.N, pk.K)
    _raises("qweight_t: shape", w4.linear, torch.zeros(4, 512, dtype=torch.int16), bad)


def test_repack_rejects_bad_canonical_arrays():
    N, K = 256, 512
    q = torch.zeros(K // 8, N, dtype=torch.int32)
    s = torch.zeros(K // 128, N, dtype=torch.int16)
    z = torch.zeros(K // 128, N // 8, dtype=torch.int32)
    _raises("shape", w4.repack, q[:, :128], s, z, N, K)
    _raises("element", w4.repack, q, s.to(torch.int32), z, N, K)
    _raises("shape", w4.repack, q, s, z[:, :8], N, K)
    _raises("GPU", w4.repack, q, s, z, N, K)


def test_accept_rejects_mismatched_inputs():
    K, V = 4, 1000
    L = torch.zeros(K + 1, V)
    d = torch.zeros(K, dtype=torch.int32)
    _raises("shape", w4.accept, L, torch.zeros(K + 1, dtype=torch.int32))      # one draft token too many
    _raises("element", w4.accept, L, torch.zeros(K, dtype=torch.int64))        # 8-byte tokens
    _raises("shape", w4.accept, L, d, torch.zeros(K + 1, V), torch.zeros(K + 1))  # draft rows
    _raises("shape", w4.accept, L, d, torch.zeros(K, V), torch.zeros(K))       # uniforms
    _raises("both", w4.accept, L, d, torch.zeros(K, V))                         # u missing
    _raises("contiguous", w4.accept, torch.zeros(V, K + 1).t(), d)
    _raises("GPU", w4.accept, L, d)


def test_tree_attention_rejects_mismatched_inputs():
    M, Hq, Hkv, D, L = 3, 8, 2, 128, 16
    q = torch.zeros(M, Hq, D, dtype=torch.int16)
    kc = torch.zeros(L, Hkv, D, dtype=torch.int16)
    kd = torch.zeros(M, Hkv, D, dtype=torch.int16)
    masks = torch.zeros(M, dtype=torch.int64)
    _raises("shape", w4.tree_attention, q, kc, kc[:, :1], kd, kd, masks)         # v_cache heads
    _raises("shape", w4.tree_attention, q, kc, kc, kd, kd[:2], masks)            # v_draft rows
    _raises("shape", w4.tree_attention, q, kc, kc, kd, kd, masks[:2])            # one mask short
    _raises("element", w4.tree_attention, q, kc, kc, kd, kd, masks.to(torch.int32))
    _raises("element", w4.tree_attention, q.float(), kc, kc, kd, kd, masks)
    _raises("3-D", w4.tree_attention, q[0], kc, kc, kd, kd, masks)
    _raises("GPU", w4.tree_attention, q, kc, kc, kd, kd, masks)
