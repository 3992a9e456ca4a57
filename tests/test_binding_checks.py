"""The binding rejects mismatched dtypes, shapes and workspaces before
anything reaches the library (CPU tensors: a call that got past the checks
would stop at the device check, which names GPU memory)."""
import pytest
import torch

import compressed_sparse_kv_overlapping_amd as cskv

bf, f32, i32, i64, u8 = torch.bfloat16, torch.float32, torch.int32, torch.int64, torch.uint8
B, H, N, W, K = 2, 16, 600, 8, 512   # enough rows for split partials (a workspace)


def t(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def raises(match, fn, *args, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*args, **kw)


def attn_args(**over):
    a = dict(q=t(B, H, 576), entries=t(N, 576), window=t(W, 576), idx=t(B, K, dtype=i32))
    a.update(over)
    return a


def test_sparse_attend_checks():
    raises("GPU memory", cskv.sparse_attend, **attn_args())          # the checks pass
    raises("entries: dtype", cskv.sparse_attend, **attn_args(q=t(B, H, 576, dtype=f32)))
    raises("window: dtype", cskv.sparse_attend, **attn_args(window=t(W, 576, dtype=f32)))
    raises("q: shape", cskv.sparse_attend, **attn_args(q=t(B, H, 512)))
    raises("entries: shape", cskv.sparse_attend, **attn_args(entries=t(N, 512)))
    raises("idx: dtype", cskv.sparse_attend, **attn_args(idx=t(B, K, dtype=i64)))
    raises("idx: shape", cskv.sparse_attend, **attn_args(idx=t(B + 1, K, dtype=i32)))
    raises("q_pos: dtype", cskv.sparse_attend, **attn_args(), q_pos=t(B, dtype=i32))
    raises("q_pos: shape", cskv.sparse_attend, **attn_args(), q_pos=t(B + 1, dtype=i64))
    raises("out: dtype", cskv.sparse_attend, **attn_args(), out=t(B, H, 512, dtype=f32))
    raises("out: shape", cskv.sparse_attend, **attn_args(), out=t(B, H, 576))
    raises("lse: dtype", cskv.sparse_attend, **attn_args(), lse=t(B, H))
    raises("entries: shape", cskv.sparse_attend, **attn_args(), per_seq=True)
    need = cskv.attend_workspace_size(B, H, K + W)
    raises("workspace: ", cskv.sparse_attend, **attn_args(), workspace=t(1, dtype=u8))
    raises("workspace: ", cskv.sparse_attend, **attn_args(), workspace=t(max(need, 1), dtype=f32))


def test_csa_and_hca_attend_checks():
    qI, kI = t(B, 64), t(N, 64)
    a = attn_args()
    del a["idx"]
    raises("GPU memory", cskv.csa_attend, q_idx=qI, idx_keys=kI, k=K, **a)
    raises("idx_keys: dtype", cskv.csa_attend, q_idx=qI, idx_keys=t(N, 64, dtype=torch.float8_e4m3fn),
           k=K, **a)
    raises("q_idx: shape", cskv.csa_attend, q_idx=t(B, 32), idx_keys=kI, k=K, **a)
    raises("idx_keys: ", cskv.csa_attend, q_idx=qI, idx_keys=t(N - 1, 64), k=K, **a)
    raises("idx_out: shape", cskv.csa_attend, q_idx=qI, idx_keys=kI, k=K,
           idx_out=t(B, K + 1, dtype=i32), **a)
    raises("workspace: ", cskv.csa_attend, q_idx=qI, idx_keys=kI, k=K, workspace=t(8, dtype=u8), **a)
    raises("GPU memory", cskv.hca_attend, t(B, H, 576), t(N, 576))
    raises("entries: dtype", cskv.hca_attend, t(B, H, 576, dtype=f32), t(N, 576))
    raises("entries: shape", cskv.hca_attend, t(B, H, 576), t(N, 576), per_seq=True)
    raises("q_pos: dtype", cskv.hca_attend, t(B, H, 576), t(N, 576), q_pos=t(B, dtype=i32), m=128)
    raises("needs the block size", cskv.hca_attend, t(B, H, 576), t(N, 576), q_pos=t(B, dtype=i64))


def test_compress_and_topk_checks():
    x, z = t(64, 512), t(64, 512)
    raises("GPU memory", cskv.compress, x, z, t(8, 512, dtype=f32), 4)
    raises("bias: shape", cskv.compress, x, z, t(4, 512, dtype=f32), 4)
    raises("bias: dtype", cskv.compress, x, z, t(8, 512), 4)
    raises("z: dtype", cskv.compress, x, t(64, 512, dtype=f32), t(8, 512, dtype=f32), 4)
    raises("out: ", cskv.compress, x, z, t(8, 512, dtype=f32), 4, out=t(15, 576))
    raises("out: dtype", cskv.compress, x, z, t(8, 512, dtype=f32), 4, out=t(16, 576, dtype=f32))
    raises("workspace: ", cskv.compress2, x, z, t(8, 512, dtype=f32), 4, t(64, 512, dtype=f32), 32,
           workspace=t(16, dtype=u8))
    raises("out_large: ", cskv.compress2, x, z, t(8, 512, dtype=f32), 4, t(64, 512, dtype=f32), 32,
           out_large=t(1, 576))
    qI, kI = t(B, 64), t(N, 64)
    raises("GPU memory", cskv.index_topk, qI, kI, K)
    raises("idx_keys: dtype", cskv.index_topk, qI, t(N, 64, dtype=f32), K)
    raises("q_idx: dtype", cskv.index_topk, t(B, 64, dtype=i32), kI, K)
    raises("q_pos: dtype", cskv.index_topk, qI, kI, K, q_pos=t(B, dtype=i32))
    raises("idx_keys: shape", cskv.index_topk, qI, kI, K, per_seq=True)
    raises("workspace: ", cskv.index_topk, qI, kI, K, workspace=t(8, dtype=u8))
    raises("GPU memory", cskv.index_topk_mxfp4, t(B, 32, dtype=u8), t(B, 2, dtype=u8),
           t(N, 32, dtype=u8), t(N, 2, dtype=u8), K)
    raises("key_scales: shape", cskv.index_topk_mxfp4, t(B, 32, dtype=u8), t(B, 2, dtype=u8),
           t(N, 32, dtype=u8), t(N, 1, dtype=u8), K)
    raises("q_codes: dtype", cskv.index_topk_mxfp4, t(B, 32), t(B, 2, dtype=u8),
           t(N, 32, dtype=u8), t(N, 2, dtype=u8), K)


def test_mxfp4_attend_and_merge_checks():
    q, codes, scales = t(B, H, 576), t(N, 288, dtype=u8), t(N, 18, dtype=u8)
    idx = t(B, K, dtype=i32)
    raises("GPU memory", cskv.sparse_attend_mxfp4, q, codes, scales, t(W, 576), idx)
    raises("ent_codes: shape", cskv.sparse_attend_mxfp4, q, t(N, 576, dtype=u8), scales, t(W, 576), idx)
    raises("ent_scales: shape", cskv.sparse_attend_mxfp4, q, codes, t(N + 1, 18, dtype=u8), t(W, 576), idx)
    raises("q: dtype", cskv.sparse_attend_mxfp4, t(B, H, 576, dtype=f32), codes, scales, t(W, 576), idx)
    raises("window: dtype", cskv.sparse_attend_mxfp4, q, codes, scales, t(W, 576, dtype=f32), idx)
    raises("GPU memory", cskv.hca_attend_mxfp4, q, codes, scales)
    raises("ent_codes: shape", cskv.hca_attend_mxfp4, q, codes, scales, per_seq=True)
    S = 3
    raises("GPU memory", cskv.merge, t(B, H, S, 512, dtype=f32), t(B, H, S, dtype=f32))
    raises("o_part: shape", cskv.merge, t(B, H, S + 1, 512, dtype=f32), t(B, H, S, dtype=f32))
    raises("o_part: dtype", cskv.merge, t(B, H, S, 512), t(B, H, S, dtype=f32))
    raises("out: dtype", cskv.merge, t(B, H, S, 512, dtype=f32), t(B, H, S, dtype=f32),
           out=t(B, H, 512, dtype=f32))
