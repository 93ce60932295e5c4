"""Shared helpers for the GPU parity tests: move seeded inputs to the device,
run the library, run the oracle on the same values, compare."""

import numpy as np
import torch

import chunkwise_gated_delta_chunk_amd as la
from oracle import recurrence

# max relative error gates: bf16 inputs (fp16 MFMA operands, fp32 accumulation)
# and fp32 inputs (fp32 MFMA); fp16 inputs take the bf16 path's operands and
# its gate
TOL = {"bf16": 2e-3, "f16": 2e-3, "f32": 1e-4}
TORCH_DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def rel_err(x, ref, mask=None):
    """max |x - ref| / max |ref| over the valid elements (mask over leading dims)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if mask is not None:
        x, ref = x[mask], ref[mask]
    if ref.size == 0:
        return 0.0
    return float(np.abs(x - ref).max() / max(np.abs(ref).max(), 1e-30))


def bf16_ulp(x):
    """Spacing of bf16 values at |x| (normal range): 2^(floor(log2|x|) - 7)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(e - 7)


def rel_err_bf16_out(x, ref):
    """rel_err of a bf16 output against the fp64 reference, allowing half a
    bf16 ulp of the reference per element for the final rounding."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    over = np.maximum(np.abs(x - ref) - 0.5 * bf16_ulp(ref), 0.0)
    return float(over.max() / max(np.abs(ref).max(), 1e-30))


def gva(inp, H_qk):
    """The inputs with H_qk q/k heads (every G-th head of the drawn ones,
    G = H / H_qk) and, for the oracle, q/k expanded back to the value heads."""
    H = inp["H"]
    G = H // H_qk
    small = dict(inp)
    small["q"] = np.ascontiguousarray(inp["q"][:, ::G])
    small["k"] = np.ascontiguousarray(inp["k"][:, ::G])
    full = dict(inp)
    full["q"] = np.repeat(small["q"], G, axis=1)
    full["k"] = np.repeat(small["k"], G, axis=1)
    return small, full


def to_dev(inp, device="cuda", cu_dtype=torch.int32):
    tdt = TORCH_DT[inp["dtype"]]
    d = {}
    for key in ("q", "k", "v"):
        d[key] = torch.from_numpy(inp[key]).to(device=device, dtype=tdt).contiguous()
    for key in ("g", "beta"):
        d[key] = torch.from_numpy(inp[key]).to(device=device).contiguous()
    d["cu_seqlens"] = torch.from_numpy(inp["cu_seqlens"].astype(np.int64)).to(device, cu_dtype)
    d["h0"] = None if inp["h0"] is None else torch.from_numpy(inp["h0"]).to(device).contiguous()
    return d


def run_gpu(inp, *, dv_split=0, scale=1.0, device="cuda", with_state=True, o=None, ht=None,
            h0=None, stream=None, seg_len=0, o_dtype=None, cu_dtype=torch.int32):
    d = to_dev(inp, device, cu_dtype)
    T = inp["q"].shape[0]
    ci, co, st = la.build_chunk_meta(d["cu_seqlens"], T, stream=stream)
    fwd = la.kda_chunk_fwd if inp["kda"] else la.gdn_chunk_fwd
    o, ht = fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], ci, co,
                h0=d["h0"] if h0 is None else h0, o=o, ht=ht, output_final_state=with_state,
                scale=scale, dv_split=dv_split, seg_len=seg_len, o_dtype=o_dtype, stream=stream)
    torch.cuda.synchronize()
    return o, ht, (ci, co, st)


def run_oracle(inp, *, scale=1.0, heads=None):
    """Oracle on the same input values; ``heads`` restricts to a head subset."""
    sel = slice(None) if heads is None else list(heads)
    q, k, v, g, b = (inp[x][:, sel] for x in ("q", "k", "v", "g", "beta"))
    h0 = None if inp["h0"] is None else inp["h0"][:, sel]
    return recurrence.gated_delta_fwd(q, k, v, g, b, inp["cu_seqlens"], h0, scale,
                                      kda=inp["kda"])


def compare(inp, o, ht, o_ref, ht_ref, heads=None, tol=None):
    """rel errors of o over covered rows and of ht over non-empty sequences."""
    tol = TOL[inp["dtype"]] if tol is None else tol
    sel = slice(None) if heads is None else list(heads)
    cu = inp["cu_seqlens"]
    rows = slice(0, int(cu[-1]))
    o_np = o.float().cpu().numpy()[rows][:, sel]
    eo = rel_err(o_np, o_ref[rows])
    eh = 0.0
    if ht is not None and ht_ref is not None:
        nonempty = np.diff(cu.astype(np.int64)) > 0
        h_np = ht.cpu().numpy()[:, sel]
        eh = rel_err(h_np[nonempty], ht_ref[nonempty])
    return eo, eh, tol


# ------------------------------------------------------ workspace images ---
# Layout of the per-(chunk slot, head) map-stage image, as include/linattn.h
# documents it: regions K, Q, [KT], TN, MM, VEC; matrices stored as rows of
# 16-byte pieces, piece index XOR-swizzled per row, fp16 columns in the
# chained MFMA order.

def kpos(k):
    """Stored position of logical column k in the chained fp16 order."""
    return (k & ~31) + 8 * ((k & 15) >> 2) + (k & 3) + 4 * ((k & 31) >> 4)


def swz(row, P):
    if P == 16:
        return ((row & 3) << 2) | ((row >> 2) & 3)
    if P == 8:
        return (((row >> 1) & 1) << 2) | ((row >> 2) & 3)
    return 0


def image_layout(kda, esz, d, raw=False):
    has_kt = kda or esz == 4
    L = {"K": 0, "Q": 64 * d * esz}
    L["KT"] = L["Q"] + 64 * d * esz
    L["TN"] = L["KT"] + (d * 64 * esz if has_kt else 0)
    L["MM"] = L["TN"] + 64 * 64 * esz
    L["VEC"] = L["MM"] + 64 * 64 * esz
    L["BYTES"] = L["VEC"] + -(-(192 + d) * 4 // 1024) * 1024
    L["has_kt"] = has_kt
    # what the workspace stores per cell: with raw (GDN, 16-bit inputs,
    # 32-column slices) from TN on, since that reduce stages K and Q from the
    # raw rows; otherwise the whole image
    L["SKIP"] = L["TN"] if raw else 0
    L["HBM"] = L["BYTES"] - L["SKIP"]
    return L


def untile(cell, off, rows, cols, esz):
    """Logical [rows][cols] matrix from an image tile at byte offset ``off`` of
    one cell (uint8 numpy array)."""
    P = cols * esz // 16
    ch = 16 // esz
    r = np.arange(rows)[:, None]
    c = np.arange(cols)[None, :]
    pos = np.vectorize(kpos)(c) if esz == 2 else c
    sw = np.vectorize(lambda x: swz(int(x), P))(r)
    byte = off + r * P * 16 + (((pos // ch) ^ sw) * 16) + (pos % ch) * esz
    dt = np.float16 if esz == 2 else np.float32
    flat = cell.view(dt)
    return flat[byte // esz].astype(np.float64)


def decode_images(ws, NT, H, d, kda, esz, raw=False):
    """Every cell of a workspace (torch uint8 tensor) as dict of logical arrays."""
    L = image_layout(kda, esz, d, raw)
    raw = ws[:NT * H * L["HBM"]].cpu().numpy().reshape(NT, H, L["HBM"])
    sk = L["SKIP"]
    out = {}
    for slot in range(NT):
        for h in range(H):
            cell = np.ascontiguousarray(raw[slot, h])
            rec = {"TN": untile(cell, L["TN"] - sk, 64, 64, esz),
                   "MM": untile(cell, L["MM"] - sk, 64, 64, esz),
                   "VEC": cell[L["VEC"] - sk:L["VEC"] - sk + (192 + d) * 4].view(np.float32)
                   .astype(np.float64)}
            if sk == 0:
                rec["K"] = untile(cell, L["K"], 64, d, esz)
                rec["Q"] = untile(cell, L["Q"], 64, d, esz)
            if L["has_kt"]:
                rec["KT"] = untile(cell, L["KT"], d, 64, esz)
            out[(slot, h)] = rec
    return out
