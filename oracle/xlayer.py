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

Adapted configuration (the same page, on its two modes: the reusable one
applies predictors calibrated in advance; the adapted one recomputes the
light block-diagonal predictors for the video at hand).  Readings: the block
B_h of each head is re-fitted once per video, on the tokens of the stream's
first encode call, by least squares with the low-rank term held fixed:
B_h = argmin over B of sum_t |B y_h[t] + (U w[t])_h - x_{l+1,h}[t]|^2,
regularised by lam * I with lam = 2^-20 * trace(G_h) / d (G_h = sum_t y y^T)
so the normal equations stay definite; solved in fp64, rounded to bf16
(nearest even) like the given weights; later calls and the decoder use it.
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


REFIT_RIDGE = 2.0 ** -20


def refit_block(xhat_prev, x_next, U, V):
    """Adapted block-diagonal predictor: B [H, d, d] fp64 (before rounding)
    and its bf16 rounding, from xhat_prev, x_next [H, T, d] and the fixed
    low-rank factors U, V [H*d, r]."""
    H, T, d = xhat_prev.shape
    zeros = np.zeros((H, d, d), dtype=np.float32)
    low_rank = predict(xhat_prev, zeros, U, V).astype(np.float64)      # U w, rounded to fp32
    y = round_to_bf16(xhat_prev).astype(np.float64)
    target = np.asarray(x_next, dtype=np.float64) - low_rank
    B = np.empty((H, d, d), dtype=np.float64)
    for h in range(H):
        G = y[h].T @ y[h]
        R = y[h].T @ target[h]
        A = G + (REFIT_RIDGE * np.trace(G) / d) * np.eye(d)
        B[h] = np.linalg.solve(A, R).T
    return B, round_to_bf16(B)
