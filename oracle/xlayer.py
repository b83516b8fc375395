"""Cross-layer prediction residual (test infrastructure only).

Coral-KV news article (Russian page, section on predicting across layers
instead of clustering inside a layer; the Portuguese copy says the same):
the cache state of one layer predicts the keys and values of the next layer
and only the prediction residual is quantized; the predictor is
"block-DPLR", a block-diagonal matrix (channel relations inside each
attention head) plus a global low-rank term (dependencies between heads).

Readings:

* closed loop on the decoder's data: the prediction for layer l+1 is made
  from the *reconstruction* of layer l, rounded to bf16 (nearest even);
  K predicts K and V predicts V.
* for token t with the H*d vector y = bf16(xhat_l[t]) (heads concatenated):
  p = v^T y  (r values), w = bf16(p), pred = blockdiag(B_1..B_H) y + U w,
  where B_h is d x d acting on head h's d channels and U, V are (H*d) x r.
  B, U, V hold bf16 values.
* arithmetic: every product and partial sum in fp64, accumulated in a fixed
  order: p_i = sum over m = 0..H*d-1 of V[m, i] * y[m];
  pred[h, i] = (sum over j = 0..d-1 of B_h[i, j] * y_h[j]) then
  + U[h*d+i, k] * w[k] for k = 0..r-1; pred is rounded once to fp32.
* r0 = fl32(x_{l+1} - pred); the residual then goes through the same PRQ
  stages as the smoothed residual, and decode adds the stages to pred.
"""
import numpy as np

from .numerics import round_to_bf16


def predict(xhat_prev, B, U, V):
    """xhat_prev [H, T, d] fp32; B [H, d, d]; U, V [H*d, r].  Returns pred [H, T, d] fp32."""
    H, T, d = xhat_prev.shape
    y = round_to_bf16(xhat_prev).astype(np.float64)          # [H, T, d]
    yt = np.transpose(y, (1, 0, 2)).reshape(T, H * d)        # token-major [T, H*d]
    V64 = np.asarray(V, dtype=np.float64)
    U64 = np.asarray(U, dtype=np.float64)
    B64 = np.asarray(B, dtype=np.float64)
    r = V64.shape[1]
    p = np.zeros((T, r), dtype=np.float64)
    for m in range(H * d):                                   # fixed order over the H*d inputs
        p = p + yt[:, m:m + 1] * V64[m][None, :]
    w = round_to_bf16(p).astype(np.float64)                  # [T, r]
    pred = np.zeros((H, T, d), dtype=np.float64)
    for j in range(d):                                       # block-diagonal term, channel order
        pred = pred + y[:, :, j][:, :, None] * B64[:, :, j][:, None, :]
    Uh = U64.reshape(H, d, r)
    for k in range(r):                                       # then the low-rank term, rank order
        pred = pred + w[:, k][None, :, None] * Uh[:, :, k][:, None, :]
    return pred.astype(np.float32)


def residual(x_next, pred):
    """r0 = fl32(x_{l+1} - pred)."""
    return np.asarray(x_next, dtype=np.float32) - np.asarray(pred, dtype=np.float32)
