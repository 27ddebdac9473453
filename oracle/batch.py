"""Draft-batch construction, written out row by row.

[PD] "Step 2: parallel drafting": every position of the draft batch pairs a
token embedding with a hidden state; the next-token slot pairs the newly
sampled token with h_context; slots 2..K carry the MASK token and the shared
hidden placeholder h_shared.  [PD] "fused Triton kernel": one pass copies the
previous ids and positions, inserts the new (bonus) token, fills the parallel
slots with the MASK id and emits the rejected-token mask, the masked-token
mask and the hidden-state mapping.  [PD] "hidden-state management": h_shared
is broadcast into the MASK slots and target hidden rows are mapped to their
new positions.  [PD] "KV cache": rejected tokens map to PADDING_SLOT_ID = -1
so that they write nothing to the cache; the batch grows by K rows per
request.

Reading of the row layout: request r contributes its W_r window rows (the
previous verify pass; the trailing n_rej[r] are rejected), then one
next-token row, then K-1 MASK rows.  The next-token row sits at position
kv_len[r] + (W_r - n_rej[r]); MASK row k sits k positions after it.  Every
non-rejected row writes KV slot kv_base[r] + position.
"""
import numpy as np

PADDING_SLOT_ID = -1


def build_draft_batch(K, mask_token_id, cu_window, n_rej, kv_len, kv_base,
                      window_ids, window_pos, window_hrow, new_token, ctx_hrow,
                      target_hidden, h_shared):
    """Returns a dict of the batch arrays (numpy), hidden rows copied bit for bit.

    ``target_hidden`` is [rows, 3, d] and ``h_shared`` is [3, d], in any
    dtype (the copy does not look at the values).
    """
    R = len(n_rej)
    T = int(cu_window[R]) + R * K
    d3 = target_hidden.shape[1:]
    ids = np.zeros(T, np.int32)
    pos = np.zeros(T, np.int32)
    slot = np.zeros(T, np.int32)
    hsrc = np.zeros(T, np.int32)
    req = np.zeros(T, np.int32)
    rejected = np.zeros(T, np.uint8)
    masked = np.zeros(T, np.uint8)
    query_rows = np.zeros(R * K, np.int32)
    cu_draft = np.zeros(R + 1, np.int32)
    hidden = np.zeros((T,) + d3, target_hidden.dtype)

    row = 0
    for r in range(R):
        cu_draft[r] = row
        w0, w1 = int(cu_window[r]), int(cu_window[r + 1])
        W = w1 - w0
        n_acc = W - int(n_rej[r])
        for j in range(W):
            src = w0 + j
            ids[row] = window_ids[src]
            pos[row] = window_pos[src]
            hsrc[row] = window_hrow[src]
            hidden[row] = target_hidden[window_hrow[src]]
            req[row] = r
            if j >= n_acc:
                rejected[row] = 1
                slot[row] = PADDING_SLOT_ID
            else:
                slot[row] = int(kv_base[r]) + int(pos[row])
            row += 1
        p_ntp = int(kv_len[r]) + n_acc
        for k in range(K):
            query_rows[r * K + k] = row
            req[row] = r
            pos[row] = p_ntp + k
            slot[row] = int(kv_base[r]) + p_ntp + k
            if k == 0:
                ids[row] = new_token[r]
                hsrc[row] = ctx_hrow[r]
                hidden[row] = target_hidden[ctx_hrow[r]]
            else:
                ids[row] = mask_token_id
                hsrc[row] = -1
                hidden[row] = h_shared
                masked[row] = 1
            row += 1
    cu_draft[R] = row
    assert row == T
    return dict(draft_ids=ids, draft_pos=pos, slot_mapping=slot, hidden_src=hsrc,
                req_of_row=req, rejected=rejected, masked=masked,
                query_rows=query_rows, cu_draft=cu_draft, draft_hidden=hidden, T=T)
