// Full back-propagation through time of the current-policy replay, fp32 arithmetic.
//
// What is differentiated: the replay of jiphyeonjeon.kr "Recurrent Looped Transformer"
// §6.2 (eq 5.5) -- fresh H_0, the causal encoder over the history, the memory, the T
// sequential transitions, log p(x_{t+1} | x_<=t) -- under the loss
// L = sum_{b,t} w[b,t] * logprob[b,t]. The same review's appendix B (eq B.4) and §6.4 make
// full BPTT the reference training computation: the gradient reaches s_t through every
// merge, every decoder key/value including the entries the window later drops, and the
// encoder through the memory and the merge inputs e_t. Block forms: greeksharifa.github.io
// "Recurrent Looped Transformer 요약 설명" §2.1-§2.5 (pre-norm RMSNorm, SwiGLU, rotary
// positions, the sigmoid merge over [e_t ; r]).
//
// Schedule (one stream):
//   forward  : embedding, L_E token-parallel encoder blocks, memory projection, then the T
//              transitions one position at a time, every intermediate kept in the workspace
//              (rows are position-major: row = t*B + b), then the readout of all rows;
//   loss     : float64 log-sum-exp per row, logprob and dL/dlogits;
//   backward : readout; the decoder in reverse time -- at position t each layer's FFN,
//              cross-attention (its key/value gradient goes straight into the memory
//              gradient rows 1..t) and window attention (into the key/value gradient rows
//              of the window; the row of t is complete once t itself is done, because only
//              queries t..t+W-1 read it), then the merge, whose state-input gradient is
//              carried to position t-1 (RLT-1) or collected for the chunk register's source
//              position (RLT-2); the weight gradients of every decoder matrix are then one
//              GEMM over all T*B rows each; memory projection; encoder blocks in reverse.
//
// Kernels: a 64x64-tiled fp32 GEMM with both operand orientations (and split-K with
// atomic accumulation for the weight gradients, whose reduction runs over T*B rows);
// wave-per-row RMSNorm forward/backward; column reductions for gains and biases; rotary
// rotation by +/- angle (float64 angles, as in the forward path); one-wave-per-(query,
// head) attention forward (online softmax, log-sum-exp kept) and backward (probabilities
// recomputed from the log-sum-exp; query-side kernel that can also update the key/value
// gradient rows when each launch holds one query per (sequence, head), key-side kernel
// for the causal encoder); SwiGLU, merge and readout elementwise kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <vector>

#include "common.hpp"
#include "grad.hpp"

namespace rlt {
namespace {

constexpr int GT = 64;  // GEMM tile rows / columns
constexpr int GK = 16;  // GEMM k step
constexpr int NOWIN = INT_MAX / 4;

// ----------------------------------------------------------------------------- GEMM
// C[m, n] = (R ? R[m, n] : 0) + sum_k A(m, k) B(k, n), or, when atomic, C[m, n] += sum.
// A(m, k) = AK ? A[m*lda + k] : A[k*lda + m];  B(k, n) = BK ? B[n*ldb + k] : B[k*ldb + n].
// R, when given, has C's layout (it may be C itself). blockIdx.z takes k in
// [z*kchunk, (z+1)*kchunk). With `part`, the k-slice z writes its partial sums to
// part[z][M][N] instead (summed by g_splitk_reduce in a fixed order).
template <bool AK, bool BK>
__global__ __launch_bounds__(256) void g_gemm(int M, int N, int K, const float* __restrict__ A, int64_t lda,
                                              const float* __restrict__ Bm, int64_t ldb, float* C, int64_t ldc,
                                              const float* R, int atomic, int kchunk, float* __restrict__ part) {
  __shared__ float As[GK][GT + 4];
  __shared__ float Bs[GK][GT + 4];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.y * GT, n0 = blockIdx.x * GT;
  const int kb = blockIdx.z * kchunk;
  const int ke = min(K, kb + kchunk);
  float ra[4], rb[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i;
      {
        const int m = AK ? (e >> 4) : (e & 63), k = AK ? (e & 15) : (e >> 6);
        const int gm = m0 + m, gk = k0 + k;
        ra[i] = (gm < M && gk < ke) ? (AK ? A[(int64_t)gm * lda + gk] : A[(int64_t)gk * lda + gm]) : 0.f;
      }
      {
        const int n = BK ? (e >> 4) : (e & 63), k = BK ? (e & 15) : (e >> 6);
        const int gn = n0 + n, gk = k0 + k;
        rb[i] = (gn < N && gk < ke) ? (BK ? Bm[(int64_t)gn * ldb + gk] : Bm[(int64_t)gk * ldb + gn]) : 0.f;
      }
    }
  };
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  const int ty = tid >> 4, tx = tid & 15;
  if (kb < ke) load(kb);
  for (int k0 = kb; k0 < ke; k0 += GK) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i;
      if (AK) As[e & 15][e >> 4] = ra[i]; else As[e >> 6][e & 63] = ra[i];
      if (BK) Bs[e & 15][e >> 4] = rb[i]; else Bs[e >> 6][e & 63] = rb[i];
    }
    __syncthreads();
    if (k0 + GK < ke) load(k0 + GK);
#pragma unroll
    for (int kk = 0; kk < GK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gm = m0 + ty + 16 * i;
    if (gm >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn = n0 + tx + 16 * j;
      if (gn >= N) continue;
      if (part) {
        part[((int64_t)blockIdx.z * M + gm) * N + gn] = acc[i][j];
        continue;
      }
      float* c = C + (int64_t)gm * ldc + gn;
      if (atomic) atomicAdd(c, acc[i][j]);
      else *c = (R ? R[(int64_t)gm * ldc + gn] : 0.f) + acc[i][j];
    }
  }
}

// C[m, n] = (R ? R[m, n] : 0) + sum_{z < splits} part[z][m][n], z ascending
__global__ void g_splitk_reduce(int M, int N, int splits, const float* __restrict__ part, const float* R, float* C,
                                int64_t ldc) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)M * N) return;
  const int64_t m = i / N, n = i % N;
  float v = 0.f;
  for (int z = 0; z < splits; ++z) v += part[(int64_t)z * M * N + i];
  C[m * ldc + n] = (R ? R[m * ldc + n] : 0.f) + v;
}

// ------------------------------------------------------------------------ RMSNorm
// y = x / sqrt(mean(x^2) + eps) * g per row of d; rstd keeps 1/sqrt(mean + eps).
__global__ __launch_bounds__(256) void g_rms_fwd(int M, int d, const float* __restrict__ x,
                                                 const float* __restrict__ g, float eps, float* __restrict__ y,
                                                 float* __restrict__ rstd) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= M) return;
  const float* xr = x + (int64_t)row * d;
  float ss = 0.f;
  for (int j = lane; j < d; j += 64) ss = fmaf(xr[j], xr[j], ss);
  ss = wave_sum(ss);
  const float r = 1.f / sqrtf(ss / (float)d + eps);
  float* yr = y + (int64_t)row * d;
  for (int j = lane; j < d; j += 64) yr[j] = xr[j] * r * g[j];
  if (lane == 0) rstd[row] = r;
}

// out = (res ? res : 0) + dx, dx = r*g*dy - x * r^3 / d * sum_j(g_j dy_j x_j): the input
// gradient of y = x*r*g with r = (mean(x^2) + eps)^(-1/2). res may alias out.
__global__ __launch_bounds__(256) void g_rms_bwd(int M, int d, const float* __restrict__ dy,
                                                 const float* __restrict__ x, const float* __restrict__ rstd,
                                                 const float* __restrict__ g, const float* res, float* out) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= M) return;
  const int64_t o = (int64_t)row * d;
  float dot = 0.f;
  for (int j = lane; j < d; j += 64) dot = fmaf(g[j] * dy[o + j], x[o + j], dot);
  dot = wave_sum(dot);
  const float r = rstd[row];
  const float c = r * r * r * dot / (float)d;
  for (int j = lane; j < d; j += 64) {
    const float v = r * g[j] * dy[o + j] - c * x[o + j];
    out[o + j] = (res ? res[o + j] : 0.f) + v;
  }
}

// dg[j] += sum_rows dy[row, j] * (x ? x[row, j] * rstd[row] : 1)  (gain or bias gradient)
constexpr int kColRows = 64;
__global__ __launch_bounds__(256) void g_colsum(int M, int d, const float* __restrict__ dy,
                                                const float* __restrict__ x, const float* __restrict__ rstd,
                                                float* __restrict__ dg) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= d) return;
  const int r0 = blockIdx.y * kColRows, r1 = min(M, r0 + kColRows);
  float acc = 0.f;
  for (int r = r0; r < r1; ++r) {
    const float v = dy[(int64_t)r * d + j];
    acc += x ? v * x[(int64_t)r * d + j] * rstd[r] : v;
  }
  atomicAdd(dg + j, acc);
}

// ------------------------------------------------------------------ small kernels
// Rotary rotation of the pairs (i, i + dh/2) of every head by sgn * pos * base^(-2i/dh),
// pos = pos0 + row / rpp; angles and their cosine/sine in float64, rounded to fp32.
__global__ void g_rope(int M, int H, int dh, float* x, int pos0, int rpp, double base, float sgn) {
  const int half = dh / 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)M * H * half) return;
  const int i = (int)(idx % half);
  const int h = (int)((idx / half) % H);
  const int64_t row = idx / ((int64_t)half * H);
  const double pos = (double)(pos0 + row / rpp);
  const double a = pos * pow(base, -2.0 * i / dh);
  const float c = (float)cos(a), s = sgn * (float)sin(a);
  float* p = x + row * (int64_t)H * dh + (int64_t)h * dh;
  const float x1 = p[i], x2 = p[i + half];
  p[i] = x1 * c - x2 * s;
  p[i + half] = x1 * s + x2 * c;
}

// h[t*B + b, :] = emb[tok[b, t], :]
__global__ void g_embed(int B, int T, int d, const int32_t* __restrict__ tok, const float* __restrict__ emb,
                        float* __restrict__ h) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)B * T * d) return;
  const int j = (int)(idx % d);
  const int64_t row = idx / d;
  const int b = (int)(row % B), t = (int)(row / B);
  h[idx] = emb[(int64_t)tok[(int64_t)b * T + t] * d + j];
}

__global__ void g_embed_bwd(int B, int T, int d, const int32_t* __restrict__ tok, const float* __restrict__ gh,
                            float* __restrict__ gemb) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)B * T * d) return;
  const int j = (int)(idx % d);
  const int64_t row = idx / d;
  const int b = (int)(row % B), t = (int)(row / B);
  atomicAdd(gemb + (int64_t)tok[(int64_t)b * T + t] * d + j, gh[idx]);
}

__global__ void g_fill(int64_t n, float* p, float v) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

// out = a + (b ? b : 0); out may alias a or b
__global__ void g_add(int64_t n, const float* a, const float* b, float* out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = a[i] + (b ? b[i] : 0.f);
}

// out[r, :] = v for r < rows
__global__ void g_bcast(int rows, int d, const float* __restrict__ v, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < (int64_t)rows * d) out[i] = v[i % d];
}

__device__ __forceinline__ float sigm(float x) { return 1.f / (1.f + expf(-x)); }

// g = silu(f1) * f3
__global__ void g_swiglu_fwd(int64_t n, const float* __restrict__ f1, const float* __restrict__ f3,
                             float* __restrict__ g) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float a = f1[i];
  g[i] = a * sigm(a) * f3[i];
}

// g1 = gg * f3 * silu'(f1), g3 = gg * silu(f1); silu'(a) = s(a) (1 + a (1 - s(a))). g1 may alias gg.
__global__ void g_swiglu_bwd(int64_t n, const float* gg, const float* __restrict__ f1,
                             const float* __restrict__ f3, float* g1, float* __restrict__ g3) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float a = f1[i], s = sigm(a), gv = gg[i];
  g3[i] = gv * a * s;
  g1[i] = gv * f3[i] * s * (1.f + a * (1.f - s));
}

// u = e + alpha * gate * sr, gate = sigmoid(gp + bg)
__global__ void g_merge_fwd(int M, int d, const float* __restrict__ e, const float* __restrict__ gp,
                            const float* __restrict__ bg, const float* __restrict__ sr, float alpha,
                            float* __restrict__ gate, float* __restrict__ u) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)M * d) return;
  const float gt = sigm(gp[i] + bg[i % d]);
  gate[i] = gt;
  u[i] = e[i] + alpha * gt * sr[i];
}

// ggp = alpha * gu * sr * gate (1 - gate), gsr = alpha * gu * gate
__global__ void g_merge_bwd(int64_t n, const float* __restrict__ gu, const float* __restrict__ gate,
                            const float* __restrict__ sr, float alpha, float* __restrict__ ggp,
                            float* __restrict__ gsr) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float gt = gate[i], g = alpha * gu[i];
  ggp[i] = g * sr[i] * gt * (1.f - gt);
  gsr[i] = g * gt;
}

// Row r = t*B + b of the logits: for t < T-1, logprob[b, t] = logit[x_{t+1}] - lse and
// glog = w[b, t] (onehot(x_{t+1}) - softmax), the log-sum-exp in float64; row t = T-1 has
// no target and glog = 0.
__global__ __launch_bounds__(256) void g_readout(int B, int T, int V, const float* __restrict__ logits,
                                                 const int32_t* __restrict__ tok, const float* __restrict__ w,
                                                 float* __restrict__ lp, float* __restrict__ glog) {
  __shared__ double red[256];
  const int64_t r = blockIdx.x;
  const int b = (int)(r % B), t = (int)(r / B), tid = threadIdx.x;
  const float* x = logits + r * V;
  float* gl = glog + r * V;
  if (t == T - 1) {
    for (int v = tid; v < V; v += 256) gl[v] = 0.f;
    return;
  }
  float mx = -INFINITY;
  for (int v = tid; v < V; v += 256) mx = fmaxf(mx, x[v]);
  red[tid] = mx;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] = fmax(red[tid], red[tid + s]);
    __syncthreads();
  }
  const double m = red[0];
  __syncthreads();
  double acc = 0.0;
  for (int v = tid; v < V; v += 256) acc += exp((double)x[v] - m);
  red[tid] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const double lse = m + log(red[0]);
  const int tgt = tok[(int64_t)b * T + t + 1];
  const double wt = w[(int64_t)b * (T - 1) + t];
  if (tid == 0) lp[(int64_t)b * (T - 1) + t] = (float)((double)x[tgt] - lse);
  for (int v = tid; v < V; v += 256)
    gl[v] = (float)(wt * ((v == tgt ? 1.0 : 0.0) - exp((double)x[v] - lse)));
}

// ---------------------------------------------------------------------- attention
// One wave per (query row r, head h). Query r belongs to sequence b = r % B at time
// tq = tq0 + r / B (0-based); it reads keys j in [max(0, tq - win + 1), tq] at rows j*B + b
// of K and V. Q, O rows are local (r); lse is [nq, H].
template <int NV>
__global__ __launch_bounds__(64) void g_attn_fwd(int nq, int B, int tq0, int win, int H, int dh, float scale,
                                                 const float* __restrict__ Q, const float* __restrict__ K,
                                                 const float* __restrict__ Vv, float* __restrict__ O,
                                                 float* __restrict__ lse) {
  __shared__ float qs[64 * NV];
  const int r = blockIdx.x / H, h = blockIdx.x % H, lane = threadIdx.x;
  const int hd = H * dh, b = r % B, tq = tq0 + r / B;
  const int lo = max(0, tq - win + 1);
  for (int i = lane; i < dh; i += 64) qs[i] = Q[(int64_t)r * hd + h * dh + i] * scale;
  __syncthreads();
  float m = -INFINITY, l = 0.f, o[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) o[v] = 0.f;
  for (int j0 = lo; j0 <= tq; j0 += 64) {
    const int j = j0 + lane;
    const bool ok = j <= tq;
    float s = -INFINITY;
    if (ok) {
      const float* kp = K + ((int64_t)j * B + b) * hd + h * dh;
      float a = 0.f;
      for (int i = 0; i < dh; ++i) a = fmaf(qs[i], kp[i], a);
      s = a;
    }
    const float mn = fmaxf(m, wave_max(s));
    const float sc = expf(m - mn);
    const float p = ok ? expf(s - mn) : 0.f;
    l = l * sc + wave_sum(p);
#pragma unroll
    for (int v = 0; v < NV; ++v) o[v] *= sc;
    const int cnt = min(64, tq - j0 + 1);
    for (int k = 0; k < cnt; ++k) {
      const float pk = __shfl(p, k, 64);
      const float* vp = Vv + ((int64_t)(j0 + k) * B + b) * hd + h * dh;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int dd = lane + 64 * v;
        if (dd < dh) o[v] = fmaf(pk, vp[dd], o[v]);
      }
    }
    m = mn;
  }
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int dd = lane + 64 * v;
    if (dd < dh) O[(int64_t)r * hd + h * dh + dd] = o[v] / l;
  }
  if (lane == 0) lse[(int64_t)r * H + h] = m + logf(l);
}

// Query side of the attention backward, same indexing as g_attn_fwd. With probabilities
// p_j = exp(s_j - lse) recomputed, D = dO.O, dS_j = p_j (dO.v_j - D):
//   dQ = scale * sum_j dS_j k_j; Dout (optional) = D;
//   KV: dK[row_j] += scale * dS_j q, dV[row_j] += p_j dO (plain read-modify-write: the
//   launch must hold at most one query per (sequence, head)).
template <int NV, bool KV>
__global__ __launch_bounds__(64) void g_attn_bwd_q(int nq, int B, int tq0, int win, int H, int dh, float scale,
                                                   const float* __restrict__ Q, const float* __restrict__ K,
                                                   const float* __restrict__ Vv, const float* __restrict__ O,
                                                   const float* __restrict__ lse, const float* __restrict__ dO,
                                                   float* __restrict__ dQ, float* __restrict__ Dout, float* dK,
                                                   float* dV) {
  __shared__ float qs[64 * NV], gs[64 * NV];
  const int r = blockIdx.x / H, h = blockIdx.x % H, lane = threadIdx.x;
  const int hd = H * dh, b = r % B, tq = tq0 + r / B;
  const int lo = max(0, tq - win + 1);
  const int64_t qo = (int64_t)r * hd + h * dh;
  float dpart = 0.f;
  for (int i = lane; i < dh; i += 64) {
    qs[i] = Q[qo + i] * scale;
    gs[i] = dO[qo + i];
    dpart = fmaf(dO[qo + i], O[qo + i], dpart);
  }
  const float D = wave_sum(dpart);
  __syncthreads();
  const float L = lse[(int64_t)r * H + h];
  float dq[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) dq[v] = 0.f;
  for (int j0 = lo; j0 <= tq; j0 += 64) {
    const int j = j0 + lane;
    float p = 0.f, ds = 0.f;
    if (j <= tq) {
      const int64_t ro = ((int64_t)j * B + b) * hd + h * dh;
      float s = 0.f, dp = 0.f;
      for (int i = 0; i < dh; ++i) {
        s = fmaf(qs[i], K[ro + i], s);
        dp = fmaf(gs[i], Vv[ro + i], dp);
      }
      p = expf(s - L);
      ds = p * (dp - D);
    }
    const int cnt = min(64, tq - j0 + 1);
    for (int k = 0; k < cnt; ++k) {
      const float dsk = __shfl(ds, k, 64);
      const float pk = __shfl(p, k, 64);
      const int64_t ro = ((int64_t)(j0 + k) * B + b) * hd + h * dh;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int dd = lane + 64 * v;
        if (dd < dh) {
          dq[v] = fmaf(dsk, K[ro + dd], dq[v]);
          if (KV) {
            dK[ro + dd] += dsk * qs[dd];
            dV[ro + dd] += pk * gs[dd];
          }
        }
      }
    }
  }
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int dd = lane + 64 * v;
    if (dd < dh) dQ[qo + dd] = dq[v] * scale;
  }
  if (Dout && lane == 0) Dout[(int64_t)r * H + h] = D;
}

// Key side of the attention backward for token-parallel causal attention over T
// positions: one wave per (key row kr = tk*B + b, head); queries i in [tk, min(T-1,
// tk + win - 1)] at rows i*B + b. dK = scale * sum_i dS_i q_i, dV = sum_i p_i dO_i (written).
template <int NV>
__global__ __launch_bounds__(64) void g_attn_bwd_kv(int B, int T, int win, int H, int dh, float scale,
                                                    const float* __restrict__ Q, const float* __restrict__ K,
                                                    const float* __restrict__ Vv, const float* __restrict__ lse,
                                                    const float* __restrict__ Dq, const float* __restrict__ dO,
                                                    float* __restrict__ dK, float* __restrict__ dV) {
  __shared__ float ks[64 * NV], vs[64 * NV];
  const int kr = blockIdx.x / H, h = blockIdx.x % H, lane = threadIdx.x;
  const int hd = H * dh, b = kr % B, tk = kr / B;
  const int hi = (int)std::min<int64_t>(T - 1, (int64_t)tk + win - 1);
  const int64_t ko = (int64_t)kr * hd + h * dh;
  for (int i = lane; i < dh; i += 64) {
    ks[i] = K[ko + i] * scale;
    vs[i] = Vv[ko + i];
  }
  __syncthreads();
  float dk[NV], dv[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) dk[v] = dv[v] = 0.f;
  for (int i0 = tk; i0 <= hi; i0 += 64) {
    const int i = i0 + lane;
    float p = 0.f, ds = 0.f;
    if (i <= hi) {
      const int64_t qr = (int64_t)i * B + b;
      const int64_t ro = qr * hd + h * dh;
      float s = 0.f, dp = 0.f;
      for (int c = 0; c < dh; ++c) {
        s = fmaf(Q[ro + c], ks[c], s);
        dp = fmaf(dO[ro + c], vs[c], dp);
      }
      p = expf(s - lse[qr * H + h]);
      ds = p * (dp - Dq[qr * H + h]);
    }
    const int cnt = min(64, hi - i0 + 1);
    for (int k = 0; k < cnt; ++k) {
      const float dsk = __shfl(ds, k, 64);
      const float pk = __shfl(p, k, 64);
      const int64_t ro = ((int64_t)(i0 + k) * B + b) * hd + h * dh;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int dd = lane + 64 * v;
        if (dd < dh) {
          dk[v] = fmaf(dsk, Q[ro + dd], dk[v]);
          dv[v] = fmaf(pk, dO[ro + dd], dv[v]);
        }
      }
    }
  }
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int dd = lane + 64 * v;
    if (dd < dh) {
      dK[ko + dd] = dk[v] * scale;
      dV[ko + dd] = dv[v];
    }
  }
}

// ----------------------------------------------------------------- host helpers
struct Ctx {
  hipStream_t st;
  float* part = nullptr;   // split-K partial sums of the small-M products
  int64_t part_cap = 0;    // floats
  hipError_t err = hipSuccess;
  void check() {
    if (err == hipSuccess) err = hipGetLastError();
  }
};

inline unsigned blocks(int64_t n) { return (unsigned)((n + 255) / 256); }

// C = R + A.B (see g_gemm), or C += A.B split over k with atomics. Products with few
// output tiles (the per-position products have B rows) split k over up to 16 slices whose
// partial sums a second kernel adds in a fixed order (deterministic).
constexpr int kMaxSplits = 16;
void gemm(Ctx& c, int M, int N, int K, const float* A, int64_t lda, bool ak, const float* Bm, int64_t ldb, bool bk,
          float* C, int64_t ldc, const float* R, bool atomic) {
  // atomic: C += A.B; otherwise C = R + A.B
  if (M <= 0 || N <= 0) return;
  const int tm = (M + GT - 1) / GT, tn = (N + GT - 1) / GT;
  int splits = 1;
  float* part = nullptr;
  if (atomic) {
    const int want = std::max(1, 1024 / (tm * tn));
    splits = std::max(1, std::min(want, (K + 255) / 256));
    if (splits == 1) {   // one slice: a plain read-add-write is exact and deterministic
      atomic = false;
      R = C;
    }
  } else if (tm * tn < 128 && K >= 128 && c.part) {
    splits = std::min({kMaxSplits, (256 + tm * tn - 1) / (tm * tn), K / 64});
    while (splits > 1 && (int64_t)splits * M * N > c.part_cap) --splits;
    if (splits > 1) part = c.part;
  }
  int kchunk = (K + splits - 1) / splits;
  kchunk = (kchunk + GK - 1) / GK * GK;
  if (kchunk <= 0) kchunk = GK;
  splits = std::max(1, (K + kchunk - 1) / kchunk);
  if (splits == 1) part = nullptr;
  dim3 grid(tn, tm, splits);
  const int at = atomic ? 1 : 0;
  if (ak && bk) g_gemm<true, true><<<grid, 256, 0, c.st>>>(M, N, K, A, lda, Bm, ldb, C, ldc, R, at, kchunk, part);
  else if (ak) g_gemm<true, false><<<grid, 256, 0, c.st>>>(M, N, K, A, lda, Bm, ldb, C, ldc, R, at, kchunk, part);
  else if (bk) g_gemm<false, true><<<grid, 256, 0, c.st>>>(M, N, K, A, lda, Bm, ldb, C, ldc, R, at, kchunk, part);
  else g_gemm<false, false><<<grid, 256, 0, c.st>>>(M, N, K, A, lda, Bm, ldb, C, ldc, R, at, kchunk, part);
  c.check();
  if (part) {
    g_splitk_reduce<<<blocks((int64_t)M * N), 256, 0, c.st>>>(M, N, splits, part, R, C, ldc);
    c.check();
  }
}
// Y[M, out] = R + X[M, in] . W^T, W row-major [out, ldw] (ldw = in unless a column slice)
void lin(Ctx& c, int M, const float* X, int in, const float* W, int64_t ldw, int out, float* Y, const float* R) {
  gemm(c, M, out, in, X, in, true, W, ldw, true, Y, out, R, false);
}
// dX[M, in] = R + dY[M, out] . W, W row-major [out, ldw]
void lin_t(Ctx& c, int M, const float* dY, int out, const float* W, int64_t ldw, int in, float* dX, const float* R) {
  gemm(c, M, in, out, dY, out, true, W, ldw, false, dX, in, R, false);
}
// dW[out, in] (row stride ldc) += dY[M, out]^T . X[M, in]
void wgrad(Ctx& c, int M, const float* dY, int out, const float* X, int in, float* dW, int64_t ldc) {
  gemm(c, out, in, M, dY, out, false, X, in, false, dW, ldc, nullptr, true);
}
void rms_fwd(Ctx& c, int M, int d, const float* x, const float* g, float eps, float* y, float* rstd) {
  if (M <= 0) return;
  g_rms_fwd<<<(M + 3) / 4, 256, 0, c.st>>>(M, d, x, g, eps, y, rstd);
  c.check();
}
void rms_bwd(Ctx& c, int M, int d, const float* dy, const float* x, const float* rstd, const float* g,
             const float* res, float* out) {
  if (M <= 0) return;
  g_rms_bwd<<<(M + 3) / 4, 256, 0, c.st>>>(M, d, dy, x, rstd, g, res, out);
  c.check();
}
void colsum(Ctx& c, int M, int d, const float* dy, const float* x, const float* rstd, float* dg) {
  if (M <= 0) return;
  dim3 grid((d + 255) / 256, (M + kColRows - 1) / kColRows);
  g_colsum<<<grid, 256, 0, c.st>>>(M, d, dy, x, rstd, dg);
  c.check();
}
void rope(Ctx& c, int M, int H, int dh, float* x, int pos0, int rpp, double base, float sgn) {
  const int64_t n = (int64_t)M * H * (dh / 2);
  if (n <= 0) return;
  g_rope<<<blocks(n), 256, 0, c.st>>>(M, H, dh, x, pos0, rpp, base, sgn);
  c.check();
}
void fill(Ctx& c, float* p, int64_t n, float v) {
  if (n <= 0) return;
  g_fill<<<blocks(n), 256, 0, c.st>>>(n, p, v);
  c.check();
}
void add(Ctx& c, int64_t n, const float* a, const float* b, float* out) {
  if (n <= 0) return;
  g_add<<<blocks(n), 256, 0, c.st>>>(n, a, b, out);
  c.check();
}

template <int NV>
void attn_fwd_n(Ctx& c, int nq, int B, int tq0, int win, int H, int dh, const float* Q, const float* K,
                const float* V, float* O, float* lse) {
  g_attn_fwd<NV><<<nq * H, 64, 0, c.st>>>(nq, B, tq0, win, H, dh, 1.f / sqrtf((float)dh), Q, K, V, O, lse);
}
void attn_fwd(Ctx& c, int nq, int B, int tq0, int win, int H, int dh, const float* Q, const float* K,
              const float* V, float* O, float* lse) {
  if (nq <= 0) return;
  if (dh <= 64) attn_fwd_n<1>(c, nq, B, tq0, win, H, dh, Q, K, V, O, lse);
  else if (dh <= 128) attn_fwd_n<2>(c, nq, B, tq0, win, H, dh, Q, K, V, O, lse);
  else attn_fwd_n<4>(c, nq, B, tq0, win, H, dh, Q, K, V, O, lse);
  c.check();
}
template <int NV, bool KV>
void attn_bwd_q_n(Ctx& c, int nq, int B, int tq0, int win, int H, int dh, const float* Q, const float* K,
                  const float* V, const float* O, const float* lse, const float* dO, float* dQ, float* Dout,
                  float* dK, float* dV) {
  g_attn_bwd_q<NV, KV><<<nq * H, 64, 0, c.st>>>(nq, B, tq0, win, H, dh, 1.f / sqrtf((float)dh), Q, K, V, O, lse,
                                                dO, dQ, Dout, dK, dV);
}
void attn_bwd_q(Ctx& c, int nq, int B, int tq0, int win, int H, int dh, const float* Q, const float* K,
                const float* V, const float* O, const float* lse, const float* dO, float* dQ, float* Dout,
                float* dK, float* dV) {
  if (nq <= 0) return;
  const bool kv = dK != nullptr;
  if (dh <= 64) {
    if (kv) attn_bwd_q_n<1, true>(c, nq, B, tq0, win, H, dh, Q, K, V, O, lse, dO, dQ, Dout, dK, dV);
    else attn_bwd_q_n<1, false>(c, nq, B, tq0, win, H, dh, Q, K, V, O, lse, dO, dQ, Dout, dK, dV);
  } else if (dh <= 128) {
    if (kv) attn_bwd_q_n<2, true>(c, nq, B, tq0, win, H, dh, Q, K, V, O, lse, dO, dQ, Dout, dK, dV);
    else attn_bwd_q_n<2, false>(c, nq, B, tq0, win, H, dh, Q, K, V, O, lse, dO, dQ, Dout, dK, dV);
  } else {
    if (kv) attn_bwd_q_n<4, true>(c, nq, B, tq0, win, H, dh, Q, K, V, O, lse, dO, dQ, Dout, dK, dV);
    else attn_bwd_q_n<4, false>(c, nq, B, tq0, win, H, dh, Q, K, V, O, lse, dO, dQ, Dout, dK, dV);
  }
  c.check();
}
void attn_bwd_kv(Ctx& c, int B, int T, int win, int H, int dh, const float* Q, const float* K, const float* V,
                 const float* lse, const float* Dq, const float* dO, float* dK, float* dV) {
  const int nk = B * T;
  if (nk <= 0) return;
  const float sc = 1.f / sqrtf((float)dh);
  if (dh <= 64) g_attn_bwd_kv<1><<<nk * H, 64, 0, c.st>>>(B, T, win, H, dh, sc, Q, K, V, lse, Dq, dO, dK, dV);
  else if (dh <= 128) g_attn_bwd_kv<2><<<nk * H, 64, 0, c.st>>>(B, T, win, H, dh, sc, Q, K, V, lse, Dq, dO, dK, dV);
  else g_attn_bwd_kv<4><<<nk * H, 64, 0, c.st>>>(B, T, win, H, dh, sc, Q, K, V, lse, Dq, dO, dK, dV);
  c.check();
}

// --------------------------------------------------------------------- workspace
struct Arena {
  char* base = nullptr;
  size_t off = 0;
  float* f(int64_t n) {
    float* p = base ? reinterpret_cast<float*>(base + off) : nullptr;
    off += ((size_t)std::max<int64_t>(n, 1) * sizeof(float) + 255) & ~size_t(255);
    return p;
  }
};

struct EncBuf {  // one encoder layer, M = T*B rows
  float *a, *rs1, *q, *k, *v, *o, *lse, *mid, *c, *rs2, *f1, *f3, *g;
};
// One decoder layer. zin, k, v and the key / value gradients hold every position (M rows);
// the others hold every position too, or, with checkpointing, the B rows of the position
// being differentiated (recomputed from zin just before its backward).
struct DecBuf {
  float *zin, *a, *rs1, *q, *k, *v, *o, *lse1, *z1, *b, *rs2, *qx, *ox, *lse2, *z2, *c, *rs3, *f1, *f3, *g;
  float *gq, *gk, *gv, *gz1, *gqx, *gz2, *gz3, *gda, *gdb, *gdc, *gf1, *gf3;
};
struct Bufs {
  bool ck = false;
  std::vector<float*> eh;   // L_E + 1 residual streams
  std::vector<EncBuf> enc;  // every layer, or one (checkpointing: each layer recomputed from eh)
  float *en, *ens;
  std::vector<float*> mk, mv, gmk, gmv;
  std::vector<DecBuf> dec;
  float* msrc;                                   // merge source rows (every position)
  float *mr, *mrs, *gate, *sr, *ggp, *gsr, *gmr;  // every position, or one (checkpointing)
  float *S, *nS, *nrs, *logits, *glog, *gS, *ge, *tMd;
  float *tBd, *tBf, *tBhd, *gu, *carry, *greg;
  // encoder backward
  float *gh, *gmid, *gec, *gf1, *gf3, *geo, *geq, *gek, *gev, *Dq;
  float* part;     // split-K partials of the per-position products
  int64_t part_n;  // its floats
};

void plan(const rlt_config& c, int B, int T, bool ck, Arena& A, Bufs& u) {
  const int64_t M = (int64_t)B * T, d = c.d, hd = (int64_t)c.n_heads * c.d_head, f = c.ffn, H = c.n_heads;
  const int64_t Ms = ck ? B : M;   // rows of a per-position buffer
  u.ck = ck;
  u.eh.resize(c.L_E + 1);
  for (auto& p : u.eh) p = A.f(M * d);
  u.enc.resize(ck ? 1 : c.L_E);
  for (auto& e : u.enc) {
    e.a = A.f(M * d); e.rs1 = A.f(M); e.q = A.f(M * hd); e.k = A.f(M * hd); e.v = A.f(M * hd);
    e.o = A.f(M * hd); e.lse = A.f(M * H); e.mid = A.f(M * d); e.c = A.f(M * d); e.rs2 = A.f(M);
    e.f1 = A.f(M * f); e.f3 = A.f(M * f); e.g = A.f(M * f);
  }
  const int G = c.L_D > 0 ? c.groups : 0;
  u.en = A.f(M * d); u.ens = A.f(M);
  u.mk.resize(G); u.mv.resize(G); u.gmk.resize(G); u.gmv.resize(G);
  for (int g = 0; g < G; ++g) {
    u.mk[g] = A.f(M * hd); u.mv[g] = A.f(M * hd); u.gmk[g] = A.f(M * hd); u.gmv[g] = A.f(M * hd);
  }
  u.dec.resize(c.L_D);
  for (auto& D : u.dec) {
    D.zin = A.f(M * d); D.k = A.f(M * hd); D.v = A.f(M * hd); D.gk = A.f(M * hd); D.gv = A.f(M * hd);
    D.a = A.f(Ms * d); D.rs1 = A.f(Ms); D.q = A.f(Ms * hd);
    D.o = A.f(Ms * hd); D.lse1 = A.f(Ms * H); D.z1 = A.f(Ms * d); D.b = A.f(Ms * d); D.rs2 = A.f(Ms);
    D.qx = A.f(Ms * hd); D.ox = A.f(Ms * hd); D.lse2 = A.f(Ms * H); D.z2 = A.f(Ms * d); D.c = A.f(Ms * d);
    D.rs3 = A.f(Ms); D.f1 = A.f(Ms * f); D.f3 = A.f(Ms * f); D.g = A.f(Ms * f);
    D.gq = A.f(Ms * hd); D.gz1 = A.f(Ms * d); D.gqx = A.f(Ms * hd);
    D.gz2 = A.f(Ms * d); D.gz3 = A.f(Ms * d); D.gda = A.f(Ms * d); D.gdb = A.f(Ms * d); D.gdc = A.f(Ms * d);
    D.gf1 = A.f(Ms * f); D.gf3 = A.f(Ms * f);
  }
  const bool mg = c.variant != RLT_V0;
  const int64_t Mm = mg ? M : 0, Mms = mg ? Ms : 0;
  u.msrc = A.f(Mm * d);
  u.mr = A.f(Mms * d); u.mrs = A.f(Mms); u.gate = A.f(Mms * d); u.sr = A.f(Mms * d);
  u.ggp = A.f(Mms * d); u.gsr = A.f(Mms * d); u.gmr = A.f(Mms * d);
  u.S = A.f(M * d); u.nS = A.f(M * d); u.nrs = A.f(M); u.logits = A.f(M * c.vocab); u.glog = A.f(M * c.vocab);
  u.gS = A.f(M * d); u.ge = A.f(M * d); u.tMd = A.f(M * d);
  u.tBd = A.f((int64_t)B * d); u.tBf = A.f((int64_t)B * f); u.tBhd = A.f((int64_t)B * hd);
  u.gu = A.f((int64_t)B * d); u.carry = A.f((int64_t)B * d); u.greg = A.f((int64_t)B * d);
  u.gh = A.f(M * d); u.gmid = A.f(M * d); u.gec = A.f(M * d); u.gf1 = A.f(M * f); u.gf3 = A.f(M * f);
  u.geo = A.f(M * hd); u.geq = A.f(M * hd); u.gek = A.f(M * hd); u.gev = A.f(M * hd); u.Dq = A.f(M * H);
  u.part_n = (int64_t)kMaxSplits * B * std::max({d, hd, f, 2 * d, (int64_t)c.vocab});
  u.part = A.f(u.part_n);
}

// Pointers of position t (B rows) of decoder layer l.
struct Step {
  float *zin, *a, *rs1, *q, *k, *v, *o, *lse1, *z1, *b, *rs2, *qx, *ox, *lse2, *z2, *c, *rs3, *f1, *f3, *g;
  float *gq, *gk, *gv, *gz1, *gqx, *gz2, *gz3, *gda, *gdb, *gdc, *gf1, *gf3;
};

}  // namespace

size_t grad_workspace_bytes(const rlt_config& c, int B, int T, bool checkpoint) {
  Arena A;
  Bufs u;
  plan(c, B, T, checkpoint, A, u);
  return A.off;
}

hipError_t replay_grad(const rlt_config& cf, const std::map<std::string, const float*>& Wm,
                       const std::map<std::string, std::pair<float*, int64_t>>& Gm, const int32_t* tokens, int B, int T,
                       const float* dlogprob, float* logprob, void* workspace, bool checkpoint, hipStream_t stream) {
  Ctx c{stream};
  Arena A;
  A.base = static_cast<char*>(workspace);
  Bufs u;
  plan(cf, B, T, checkpoint, A, u);
  c.part = u.part;
  c.part_cap = u.part_n;
  const bool ck = checkpoint;
  const int M = B * T, d = cf.d, H = cf.n_heads, dh = cf.d_head, hd = H * dh, f = cf.ffn, V = cf.vocab;
  const double base = cf.rope_base;
  const float eps = cf.rms_eps, alpha = cf.alpha;
  const bool mg = cf.variant != RLT_V0, v2 = cf.variant == RLT_V2;
  auto w = [&](const std::string& n) { return Wm.at(n); };
  auto g = [&](const std::string& n) { return Gm.at(n).first; };
  auto E = [](int l, const char* s) { return "enc." + std::to_string(l) + "." + s; };
  // decoder SWA / FFN matrices alias the encoder layer's under sharing
  auto Ds = [&](int l, const char* s) {
    return (cf.share_enc_dec ? "enc." : "dec.") + std::to_string(l) + "." + s;
  };
  auto Dn = [](int l, const char* s) { return "dec." + std::to_string(l) + "." + s; };
  auto grp = [&](int l) { return cf.groups == 1 ? 0 : l; };
  auto Mg = [](int gi, const char* s) { return "mem." + std::to_string(gi) + "." + s; };

  for (auto& kv : Gm) fill(c, kv.second.first, kv.second.second, 0.f);
  if (T <= 0 || B <= 0) return c.err;

  // position t's rows: R0 in every-position buffers, Rs in per-position ones
  auto step = [&](int l, int t) {
    const DecBuf& D = u.dec[l];
    const int64_t R0 = (int64_t)t * B, Rs = ck ? 0 : R0;
    Step s;
    s.zin = D.zin + R0 * d; s.k = D.k + R0 * hd; s.v = D.v + R0 * hd; s.gk = D.gk + R0 * hd; s.gv = D.gv + R0 * hd;
    s.a = D.a + Rs * d; s.rs1 = D.rs1 + Rs; s.q = D.q + Rs * hd; s.o = D.o + Rs * hd; s.lse1 = D.lse1 + Rs * H;
    s.z1 = D.z1 + Rs * d; s.b = D.b + Rs * d; s.rs2 = D.rs2 + Rs; s.qx = D.qx + Rs * hd; s.ox = D.ox + Rs * hd;
    s.lse2 = D.lse2 + Rs * H; s.z2 = D.z2 + Rs * d; s.c = D.c + Rs * d; s.rs3 = D.rs3 + Rs;
    s.f1 = D.f1 + Rs * f; s.f3 = D.f3 + Rs * f; s.g = D.g + Rs * f;
    s.gq = D.gq + Rs * hd; s.gz1 = D.gz1 + Rs * d; s.gqx = D.gqx + Rs * hd; s.gz2 = D.gz2 + Rs * d;
    s.gz3 = D.gz3 + Rs * d; s.gda = D.gda + Rs * d; s.gdb = D.gdb + Rs * d; s.gdc = D.gdc + Rs * d;
    s.gf1 = D.gf1 + Rs * f; s.gf3 = D.gf3 + Rs * f;
    return s;
  };
  auto mrow = [&](float* p, int t, int64_t width) { return p + (ck ? 0 : (int64_t)t * B * width); };

  // ------------------------------------------------------------ forward: encoder
  auto enc_fwd = [&](int l) {
    EncBuf& e = u.enc[ck ? 0 : l];
    rms_fwd(c, M, d, u.eh[l], w(E(l, "n1")), eps, e.a, e.rs1);
    lin(c, M, e.a, d, w(E(l, "wq")), d, hd, e.q, nullptr);
    lin(c, M, e.a, d, w(E(l, "wk")), d, hd, e.k, nullptr);
    lin(c, M, e.a, d, w(E(l, "wv")), d, hd, e.v, nullptr);
    rope(c, M, H, dh, e.q, 1, B, base, 1.f);
    rope(c, M, H, dh, e.k, 1, B, base, 1.f);
    attn_fwd(c, M, B, 0, NOWIN, H, dh, e.q, e.k, e.v, e.o, e.lse);
    lin(c, M, e.o, hd, w(E(l, "wo")), hd, d, e.mid, u.eh[l]);
    rms_fwd(c, M, d, e.mid, w(E(l, "n2")), eps, e.c, e.rs2);
    lin(c, M, e.c, d, w(E(l, "w1")), d, f, e.f1, nullptr);
    lin(c, M, e.c, d, w(E(l, "w3")), d, f, e.f3, nullptr);
    g_swiglu_fwd<<<blocks((int64_t)M * f), 256, 0, c.st>>>((int64_t)M * f, e.f1, e.f3, e.g);
    c.check();
    lin(c, M, e.g, f, w(E(l, "w2")), f, d, u.eh[l + 1], e.mid);
  };
  {
    const int64_t n = (int64_t)M * d;
    g_embed<<<blocks(n), 256, 0, c.st>>>(B, T, d, tokens, w("emb"), u.eh[0]);
    c.check();
  }
  for (int l = 0; l < cf.L_E; ++l) enc_fwd(l);
  const float* e_all = u.eh[cf.L_E];
  // ------------------------------------------------------------- forward: memory
  if (cf.L_D > 0) {
    rms_fwd(c, M, d, e_all, w("mem.nE"), eps, u.en, u.ens);
    for (int gi = 0; gi < cf.groups; ++gi) {
      lin(c, M, u.en, d, w(Mg(gi, "wk")), d, hd, u.mk[gi], nullptr);
      rope(c, M, H, dh, u.mk[gi], 1, B, base, 1.f);
      lin(c, M, u.en, d, w(Mg(gi, "wv")), d, hd, u.mv[gi], nullptr);
    }
  }
  // --------------------------------------------------------- forward: transitions
  const int64_t Bd = (int64_t)B * d;
  // merge at position t from the source rows already in msrc; writes u (the first block's
  // input, or s_t when there are no blocks)
  auto merge_fwd = [&](int t) {
    const int64_t R0 = (int64_t)t * B;
    const float* et = e_all + R0 * d;
    float* uu = cf.L_D > 0 ? u.dec[0].zin + R0 * d : u.S + R0 * d;
    float* r = mrow(u.mr, t, d);
    rms_fwd(c, B, d, u.msrc + R0 * d, w("merge.ns"), eps, r, mrow(u.mrs, t, 1));
    lin(c, B, et, d, w("merge.wg"), 2 * d, d, u.tBd, nullptr);
    lin(c, B, r, d, w("merge.wg") + d, 2 * d, d, u.tBd, u.tBd);
    lin(c, B, r, d, w("merge.ws"), d, d, mrow(u.sr, t, d), nullptr);
    g_merge_fwd<<<blocks(Bd), 256, 0, c.st>>>(B, d, et, u.tBd, w("merge.bg"), mrow(u.sr, t, d), alpha,
                                               mrow(u.gate, t, d), uu);
    c.check();
  };
  // block l at position t up to its FFN hidden state (the block output is the caller's);
  // with_kv: also this position's key and value rows
  auto layer_fwd = [&](int l, int t, bool with_kv) {
    const DecBuf& D = u.dec[l];
    const Step s = step(l, t);
    rms_fwd(c, B, d, s.zin, w(Dn(l, "m1")), eps, s.a, s.rs1);
    lin(c, B, s.a, d, w(Ds(l, "wq")), d, hd, s.q, nullptr);
    rope(c, B, H, dh, s.q, t + 1, B, base, 1.f);
    if (with_kv) {
      lin(c, B, s.a, d, w(Ds(l, "wk")), d, hd, s.k, nullptr);
      lin(c, B, s.a, d, w(Ds(l, "wv")), d, hd, s.v, nullptr);
      rope(c, B, H, dh, s.k, t + 1, B, base, 1.f);
    }
    attn_fwd(c, B, B, t, cf.window, H, dh, s.q, D.k, D.v, s.o, s.lse1);
    lin(c, B, s.o, hd, w(Ds(l, "wo")), hd, d, s.z1, s.zin);
    rms_fwd(c, B, d, s.z1, w(Dn(l, "m2")), eps, s.b, s.rs2);
    lin(c, B, s.b, d, w(Dn(l, "xq")), d, hd, s.qx, nullptr);
    rope(c, B, H, dh, s.qx, t + 1, B, base, 1.f);
    attn_fwd(c, B, B, t, NOWIN, H, dh, s.qx, u.mk[grp(l)], u.mv[grp(l)], s.ox, s.lse2);
    lin(c, B, s.ox, hd, w(Dn(l, "xo")), hd, d, s.z2, s.z1);
    rms_fwd(c, B, d, s.z2, w(Dn(l, "m3")), eps, s.c, s.rs3);
    lin(c, B, s.c, d, w(Ds(l, "w1")), d, f, s.f1, nullptr);
    lin(c, B, s.c, d, w(Ds(l, "w3")), d, f, s.f3, nullptr);
    g_swiglu_fwd<<<blocks((int64_t)B * f), 256, 0, c.st>>>((int64_t)B * f, s.f1, s.f3, s.g);
    c.check();
    return s;
  };
  int rho_t = -1;  // RLT-2: position whose state the register holds (-1: s*)
  for (int t = 0; t < T; ++t) {
    const int64_t R0 = (int64_t)t * B;
    if (mg) {
      float* src = u.msrc + R0 * d;
      const int st = cf.variant == RLT_V1 ? t - 1 : rho_t;
      if (st < 0) {
        g_bcast<<<blocks(Bd), 256, 0, c.st>>>(B, d, w("merge.s0"), src);
        c.check();
      } else {
        add(c, Bd, u.S + (int64_t)st * B * d, nullptr, src);
      }
      merge_fwd(t);
    } else {
      add(c, Bd, e_all + R0 * d, nullptr, cf.L_D > 0 ? u.dec[0].zin + R0 * d : u.S + R0 * d);
    }
    for (int l = 0; l < cf.L_D; ++l) {
      const Step s = layer_fwd(l, t, true);
      float* out = (l + 1 < cf.L_D ? u.dec[l + 1].zin : u.S) + R0 * d;
      lin(c, B, s.g, f, w(Ds(l, "w2")), f, d, out, s.z2);
    }
    if (v2 && (t + 1) % cf.chunk == 0) rho_t = t;
  }
  // ------------------------------------------------------------- readout + loss
  rms_fwd(c, M, d, u.S, w("out.nO"), eps, u.nS, u.nrs);
  lin(c, M, u.nS, d, w("out.w"), d, V, u.logits, nullptr);
  g_readout<<<M, 256, 0, c.st>>>(B, T, V, u.logits, tokens, dlogprob, logprob, u.glog);
  c.check();
  // ------------------------------------------------------------ backward: readout
  wgrad(c, M, u.glog, V, u.nS, d, g("out.w"), d);
  lin_t(c, M, u.glog, V, w("out.w"), d, d, u.tMd, nullptr);
  colsum(c, M, d, u.tMd, u.S, u.nrs, g("out.nO"));
  rms_bwd(c, M, d, u.tMd, u.S, u.nrs, w("out.nO"), nullptr, u.gS);
  // ------------------------------------------------ backward: transitions, reversed
  // weight and gain gradients of block l over `rows` rows starting at s (every position at
  // once, or one position with checkpointing)
  auto layer_wgrad = [&](int l, const Step& s, int rows) {
    wgrad(c, rows, s.gq, hd, s.a, d, g(Ds(l, "wq")), d);
    wgrad(c, rows, s.gk, hd, s.a, d, g(Ds(l, "wk")), d);
    wgrad(c, rows, s.gv, hd, s.a, d, g(Ds(l, "wv")), d);
    wgrad(c, rows, s.gz1, d, s.o, hd, g(Ds(l, "wo")), hd);
    wgrad(c, rows, s.gqx, hd, s.b, d, g(Dn(l, "xq")), d);
    wgrad(c, rows, s.gz2, d, s.ox, hd, g(Dn(l, "xo")), hd);
    wgrad(c, rows, s.gf1, f, s.c, d, g(Ds(l, "w1")), d);
    wgrad(c, rows, s.gf3, f, s.c, d, g(Ds(l, "w3")), d);
    wgrad(c, rows, s.gz3, d, s.g, f, g(Ds(l, "w2")), f);
    colsum(c, rows, d, s.gda, s.zin, s.rs1, g(Dn(l, "m1")));
    colsum(c, rows, d, s.gdb, s.z1, s.rs2, g(Dn(l, "m2")));
    colsum(c, rows, d, s.gdc, s.z2, s.rs3, g(Dn(l, "m3")));
  };
  auto merge_wgrad = [&](int t, int rows) {   // t: first position of the rows
    const int64_t R0 = (int64_t)t * B;
    float* ggp = mrow(u.ggp, t, d);
    float* mr = mrow(u.mr, t, d);
    wgrad(c, rows, ggp, d, e_all + R0 * d, d, g("merge.wg"), 2 * d);
    wgrad(c, rows, ggp, d, mr, d, g("merge.wg") + d, 2 * d);
    colsum(c, rows, d, ggp, nullptr, nullptr, g("merge.bg"));
    wgrad(c, rows, mrow(u.gsr, t, d), d, mr, d, g("merge.ws"), d);
    colsum(c, rows, d, mrow(u.gmr, t, d), u.msrc + R0 * d, mrow(u.mrs, t, 1), g("merge.ns"));
  };
  fill(c, u.carry, Bd, 0.f);
  fill(c, u.greg, Bd, 0.f);
  for (auto& D : u.dec) {
    fill(c, D.gk, (int64_t)M * hd, 0.f);
    fill(c, D.gv, (int64_t)M * hd, 0.f);
  }
  for (int gi = 0; gi < (int)u.gmk.size(); ++gi) {
    fill(c, u.gmk[gi], (int64_t)M * hd, 0.f);
    fill(c, u.gmv[gi], (int64_t)M * hd, 0.f);
  }
  for (int t = T - 1; t >= 0; --t) {
    const int64_t R0 = (int64_t)t * B, o = R0 * d;
    if (ck) {   // recompute this position's intermediates from the kept block inputs
      if (mg) merge_fwd(t);
      for (int l = 0; l < cf.L_D; ++l) layer_fwd(l, t, false);
    }
    float* gzo = cf.L_D > 0 ? step(cf.L_D - 1, t).gz3 : u.gu;
    add(c, Bd, u.gS + o, cf.variant == RLT_V1 ? u.carry : nullptr, gzo);
    if (v2 && (t + 1) % cf.chunk == 0) {
      add(c, Bd, gzo, u.greg, gzo);
      fill(c, u.greg, Bd, 0.f);
    }
    for (int l = cf.L_D - 1; l >= 0; --l) {
      DecBuf& D = u.dec[l];
      const Step s = step(l, t);
      // FFN
      lin_t(c, B, s.gz3, d, w(Ds(l, "w2")), f, f, u.tBf, nullptr);
      g_swiglu_bwd<<<blocks((int64_t)B * f), 256, 0, c.st>>>((int64_t)B * f, u.tBf, s.f1, s.f3, s.gf1, s.gf3);
      c.check();
      lin_t(c, B, s.gf1, f, w(Ds(l, "w1")), d, d, s.gdc, nullptr);
      lin_t(c, B, s.gf3, f, w(Ds(l, "w3")), d, d, s.gdc, s.gdc);
      rms_bwd(c, B, d, s.gdc, s.z2, s.rs3, w(Dn(l, "m3")), s.gz3, s.gz2);
      // cross-attention over memory rows 1..t
      const int gi = grp(l);
      lin_t(c, B, s.gz2, d, w(Dn(l, "xo")), hd, hd, u.tBhd, nullptr);
      attn_bwd_q(c, B, B, t, NOWIN, H, dh, s.qx, u.mk[gi], u.mv[gi], s.ox, s.lse2, u.tBhd, s.gqx, nullptr,
                 u.gmk[gi], u.gmv[gi]);
      rope(c, B, H, dh, s.gqx, t + 1, B, base, -1.f);
      lin_t(c, B, s.gqx, hd, w(Dn(l, "xq")), d, d, s.gdb, nullptr);
      rms_bwd(c, B, d, s.gdb, s.z1, s.rs2, w(Dn(l, "m2")), s.gz2, s.gz1);
      // window attention; the key/value gradient rows of t are complete afterwards
      lin_t(c, B, s.gz1, d, w(Ds(l, "wo")), hd, hd, u.tBhd, nullptr);
      attn_bwd_q(c, B, B, t, cf.window, H, dh, s.q, D.k, D.v, s.o, s.lse1, u.tBhd, s.gq, nullptr, D.gk, D.gv);
      rope(c, B, H, dh, s.gq, t + 1, B, base, -1.f);
      rope(c, B, H, dh, s.gk, t + 1, B, base, -1.f);
      lin_t(c, B, s.gq, hd, w(Ds(l, "wq")), d, d, s.gda, nullptr);
      lin_t(c, B, s.gk, hd, w(Ds(l, "wk")), d, d, s.gda, s.gda);
      lin_t(c, B, s.gv, hd, w(Ds(l, "wv")), d, d, s.gda, s.gda);
      float* gin = l > 0 ? step(l - 1, t).gz3 : u.gu;
      rms_bwd(c, B, d, s.gda, s.zin, s.rs1, w(Dn(l, "m1")), s.gz1, gin);
      if (ck) layer_wgrad(l, s, B);
    }
    float* get = u.ge + o;
    if (mg) {
      float* ggp = mrow(u.ggp, t, d);
      float* gsr = mrow(u.gsr, t, d);
      float* gmr = mrow(u.gmr, t, d);
      g_merge_bwd<<<blocks(Bd), 256, 0, c.st>>>(Bd, u.gu, mrow(u.gate, t, d), mrow(u.sr, t, d), alpha, ggp, gsr);
      c.check();
      lin_t(c, B, ggp, d, w("merge.wg"), 2 * d, d, get, u.gu);
      lin_t(c, B, ggp, d, w("merge.wg") + d, 2 * d, d, gmr, nullptr);
      lin_t(c, B, gsr, d, w("merge.ws"), d, d, gmr, gmr);
      if (cf.variant == RLT_V1)
        rms_bwd(c, B, d, gmr, u.msrc + o, mrow(u.mrs, t, 1), w("merge.ns"), nullptr, u.carry);
      else
        rms_bwd(c, B, d, gmr, u.msrc + o, mrow(u.mrs, t, 1), w("merge.ns"), u.greg, u.greg);
      if (ck) merge_wgrad(t, B);
    } else {
      add(c, Bd, u.gu, nullptr, get);
    }
  }
  if (mg) colsum(c, B, d, cf.variant == RLT_V1 ? u.carry : u.greg, nullptr, nullptr, g("merge.s0"));
  // --------------------------------------------- decoder and merge weight gradients
  if (!ck) {
    for (int l = 0; l < cf.L_D; ++l) layer_wgrad(l, step(l, 0), M);
    if (mg) merge_wgrad(0, M);
  }
  // ------------------------------------------------------------ backward: memory
  if (cf.L_D > 0) {
    for (int gi = 0; gi < cf.groups; ++gi) {
      rope(c, M, H, dh, u.gmk[gi], 1, B, base, -1.f);
      lin_t(c, M, u.gmk[gi], hd, w(Mg(gi, "wk")), d, d, u.tMd, gi == 0 ? nullptr : u.tMd);
      lin_t(c, M, u.gmv[gi], hd, w(Mg(gi, "wv")), d, d, u.tMd, u.tMd);
      wgrad(c, M, u.gmk[gi], hd, u.en, d, g(Mg(gi, "wk")), d);
      wgrad(c, M, u.gmv[gi], hd, u.en, d, g(Mg(gi, "wv")), d);
    }
    colsum(c, M, d, u.tMd, e_all, u.ens, g("mem.nE"));
    rms_bwd(c, M, d, u.tMd, e_all, u.ens, w("mem.nE"), u.ge, u.ge);
  }
  // ----------------------------------------------------------- backward: encoder
  float* gh = u.ge;
  for (int l = cf.L_E - 1; l >= 0; --l) {
    if (ck) enc_fwd(l);   // recompute the layer's intermediates (its output row is rewritten unchanged)
    EncBuf& e = u.enc[ck ? 0 : l];
    lin_t(c, M, gh, d, w(E(l, "w2")), f, f, u.gf1, nullptr);
    g_swiglu_bwd<<<blocks((int64_t)M * f), 256, 0, c.st>>>((int64_t)M * f, u.gf1, e.f1, e.f3, u.gf1, u.gf3);
    c.check();
    wgrad(c, M, gh, d, e.g, f, g(E(l, "w2")), f);
    lin_t(c, M, u.gf1, f, w(E(l, "w1")), d, d, u.gec, nullptr);
    lin_t(c, M, u.gf3, f, w(E(l, "w3")), d, d, u.gec, u.gec);
    wgrad(c, M, u.gf1, f, e.c, d, g(E(l, "w1")), d);
    wgrad(c, M, u.gf3, f, e.c, d, g(E(l, "w3")), d);
    colsum(c, M, d, u.gec, e.mid, e.rs2, g(E(l, "n2")));
    rms_bwd(c, M, d, u.gec, e.mid, e.rs2, w(E(l, "n2")), gh, u.gmid);
    lin_t(c, M, u.gmid, d, w(E(l, "wo")), hd, hd, u.geo, nullptr);
    wgrad(c, M, u.gmid, d, e.o, hd, g(E(l, "wo")), hd);
    attn_bwd_q(c, M, B, 0, NOWIN, H, dh, e.q, e.k, e.v, e.o, e.lse, u.geo, u.geq, u.Dq, nullptr, nullptr);
    attn_bwd_kv(c, B, T, NOWIN, H, dh, e.q, e.k, e.v, e.lse, u.Dq, u.geo, u.gek, u.gev);
    rope(c, M, H, dh, u.geq, 1, B, base, -1.f);
    rope(c, M, H, dh, u.gek, 1, B, base, -1.f);
    lin_t(c, M, u.geq, hd, w(E(l, "wq")), d, d, u.gec, nullptr);
    lin_t(c, M, u.gek, hd, w(E(l, "wk")), d, d, u.gec, u.gec);
    lin_t(c, M, u.gev, hd, w(E(l, "wv")), d, d, u.gec, u.gec);
    wgrad(c, M, u.geq, hd, e.a, d, g(E(l, "wq")), d);
    wgrad(c, M, u.gek, hd, e.a, d, g(E(l, "wk")), d);
    wgrad(c, M, u.gev, hd, e.a, d, g(E(l, "wv")), d);
    colsum(c, M, d, u.gec, u.eh[l], e.rs1, g(E(l, "n1")));
    rms_bwd(c, M, d, u.gec, u.eh[l], e.rs1, w(E(l, "n1")), u.gmid, u.gh);
    gh = u.gh;
  }
  {
    const int64_t n = (int64_t)M * d;
    g_embed_bwd<<<blocks(n), 256, 0, c.st>>>(B, T, d, tokens, gh, g("emb"));
    c.check();
  }
  return c.err;
}

}  // namespace rlt
