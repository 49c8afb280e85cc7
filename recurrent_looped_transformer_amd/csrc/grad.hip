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
//              cross-attention (its key/value gradient goes into the memory gradient rows
//              1..t at once, or, with every intermediate kept, from a key-side pass per
//              layer after the scan, from the stored dO and D of every row) and window
//              attention (into the key/value gradient rows of the window; the row of t is
//              complete once t itself is done, because only queries t..t+W-1 read it), then
//              the merge, whose state-input gradient is carried to position t-1 (RLT-1) or
//              collected for the chunk register's source position (RLT-2); the weight
//              gradients of every decoder matrix are then one product over all T*B rows
//              each; memory projection; encoder blocks in reverse.
//
// Kernels: fp32 products on v_mfma_f32_16x16x4f32 -- operands straight from memory into
// fragments for k-contiguous A, LDS-staged for the weight gradients (m-contiguous A, with
// atomic split-K accumulation over the T*B rows) -- and a 64x64 FMA tile for the other
// orientations; products of B rows split k into slices whose partial sums are added in a
// fixed order by a reduction fused with the consumer of the rows (RMSNorm forward or
// backward, rotary, SwiGLU, or the attention backward reading its dO); wave-per-row
// RMSNorm forward/backward; column reductions for gains and biases; rotary rotation by +/-
// angle from a per-call table (float64 angles rounded to fp32, as in the forward path);
// attention with a block per (query, head) and dh/4 lanes per key (forward with per-group
// online softmax and the log-sum-exp kept; backward with probabilities recomputed from the
// log-sum-exp: a query-side kernel that can also update the key/value gradient rows when
// each launch holds one query per (sequence, head), and a key-side kernel for the causal
// encoder and the memory); SwiGLU, merge and readout elementwise kernels.
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
constexpr int GK = 16;  // GEMM k step: a 64x16 operand tile is one float4 per thread
constexpr int NOWIN = INT_MAX / 4;

// ----------------------------------------------------------------------------- GEMM
// Optional segments of one product. A along k (A(m, k) with k-contiguous rows only): for
// kseg > 0, k in [p*kseg, (p+1)*kseg) reads a[p][m*lda + k - p*kseg] (a sum of up to three
// products with equal m and n). C and R along n: for nseg > 0, column n in
// [p*nseg, (p+1)*nseg) is c[p][m*ldc + n - p*nseg] (up to three outputs of one input).
struct Seg {
  const float* a[3] = {nullptr, nullptr, nullptr};
  int kseg = 0;
  float* c[3] = {nullptr, nullptr, nullptr};
  const float* r[3] = {nullptr, nullptr, nullptr};
  int nseg = 0;
};
__device__ __forceinline__ int seg_of(int x, int len) { return (x >= len) + (x >= 2 * len); }
// p[i] for i in 0..2 by selects (a runtime index into the kernel-argument array would place
// it in per-lane scratch memory)
template <typename P>
__device__ __forceinline__ P seg_pick(const P (&p)[3], int i) {
  return i == 0 ? p[0] : (i == 1 ? p[1] : p[2]);
}
// C[m, n] = (R ? R[m, n] : 0) + sum_k A(m, k) B(k, n), or, when atomic, C[m, n] += sum.
// A(m, k) = AK ? A[m*lda + k] : A[k*lda + m];  B(k, n) = BK ? B[n*ldb + k] : B[k*ldb + n].
// R, when given, has C's layout (it may be C itself). blockIdx.z takes k in
// [z*kchunk, (z+1)*kchunk). With `part`, the k-slice z writes its partial sums to
// part[z][M][N] instead (summed by g_splitk_reduce in a fixed order). PF k-steps of operand
// loads are in flight at once (a register ring; the launcher takes PF 1: the products with
// short k slices, where deeper rings paid, now run on g_gemm_mfma).
template <bool AK, bool BK, int PF>
__global__ __launch_bounds__(256) void g_gemm(int M, int N, int K, const float* __restrict__ A, int64_t lda,
                                              const float* __restrict__ Bm, int64_t ldb, float* C, int64_t ldc,
                                              const float* R, int atomic, int kchunk, float* __restrict__ part,
                                              Seg sg) {
  __shared__ float As[GK][GT + 4];
  __shared__ float Bs[GK][GT + 4];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.y * GT, n0 = blockIdx.x * GT;
  const int kb = blockIdx.z * kchunk;
  const int ke = min(K, kb + kchunk);
  // Each thread loads one float4 of each operand tile: along k when k is the contiguous index
  // (row = tid / 4, k = 4 * (tid % 4)), else along m / n (k = tid / 16, 4 * (tid % 16)). Every
  // contiguous extent (k for k-contiguous operands, m / n otherwise) is a multiple of 4.
  float4 ra_[PF], rb_[PF];
  auto load = [&](int k0, float4& ra, float4& rb) {
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    if (AK) {
      const int gm = m0 + (tid >> 2), gk = k0 + 4 * (tid & 3);
      if (gm < M && gk < ke) {
        if (sg.kseg) {
          const int sp = seg_of(gk, sg.kseg);
          ra = *reinterpret_cast<const float4*>(seg_pick(sg.a, sp) + (int64_t)gm * lda + gk - sp * sg.kseg);
        } else {
          ra = *reinterpret_cast<const float4*>(A + (int64_t)gm * lda + gk);
        }
      } else {
        ra = z;
      }
    } else {
      const int gk = k0 + (tid >> 4), gm = m0 + 4 * (tid & 15);
      ra = z;
      if (gk < ke && gm < M) ra = *reinterpret_cast<const float4*>(A + (int64_t)gk * lda + gm);
    }
    if (BK) {
      const int gn = n0 + (tid >> 2), gk = k0 + 4 * (tid & 3);
      rb = z;
      if (gn < N && gk < ke) rb = *reinterpret_cast<const float4*>(Bm + (int64_t)gn * ldb + gk);
    } else {
      const int gk = k0 + (tid >> 4), gn = n0 + 4 * (tid & 15);
      rb = z;
      if (gk < ke && gn < N) rb = *reinterpret_cast<const float4*>(Bm + (int64_t)gk * ldb + gn);
    }
  };
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  const int ty = tid >> 4, tx = tid & 15;
  const int nst = kb < ke ? (ke - kb + GK - 1) / GK : 0;   // k-steps of this slice
#pragma unroll
  for (int j = 0; j < PF; ++j)
    if (j < nst) load(kb + j * GK, ra_[j], rb_[j]);
  for (int s0 = 0; s0 < nst; s0 += PF) {
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int st = s0 + j;   // uniform across the block
      if (st < nst) {
        __syncthreads();
        const float4 ra = ra_[j], rb = rb_[j];
        if (AK) {
          const int r = tid >> 2, k = 4 * (tid & 3);
          As[k][r] = ra.x; As[k + 1][r] = ra.y; As[k + 2][r] = ra.z; As[k + 3][r] = ra.w;
        } else {
          const int k = tid >> 4, r = 4 * (tid & 15);
          *reinterpret_cast<float4*>(&As[k][r]) = ra;
        }
        if (BK) {
          const int r = tid >> 2, k = 4 * (tid & 3);
          Bs[k][r] = rb.x; Bs[k + 1][r] = rb.y; Bs[k + 2][r] = rb.z; Bs[k + 3][r] = rb.w;
        } else {
          const int k = tid >> 4, r = 4 * (tid & 15);
          *reinterpret_cast<float4*>(&Bs[k][r]) = rb;
        }
        __syncthreads();
        if (st + PF < nst) load(kb + (st + PF) * GK, ra_[j], rb_[j]);
#pragma unroll
        for (int kk = 0; kk < GK; ++kk) {
          float a[4], b[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) b[jj] = Bs[kk][tx + 16 * jj];
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) acc[i][jj] = fmaf(a[i], b[jj], acc[i][jj]);
        }
      }
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
      float* Cp = C;
      const float* Rp = R;
      int nn = gn;
      if (sg.nseg) {
        const int sp = seg_of(gn, sg.nseg);
        Cp = seg_pick(sg.c, sp); Rp = seg_pick(sg.r, sp); nn = gn - sp * sg.nseg;
      }
      float* cc = Cp + (int64_t)gm * ldc + nn;
      if (atomic) atomicAdd(cc, acc[i][j]);
      else *cc = (Rp ? Rp[(int64_t)gm * ldc + nn] : 0.f) + acc[i][j];
    }
  }
}

// MFMA form of g_gemm (non-atomic) for k-contiguous A (A(m, k) = A[m*lda + k], segments
// along k as g_gemm) and either orientation of B: a workgroup of 4 waves per 64x64 output
// tile and k slice, wave w owning rows 16w..16w+15 and the tile's 4 column blocks of 16.
// Operands go from memory straight into v_mfma_f32_16x16x4f32 fragments, no LDS: in each
// 16-wide k block, lane l holds row (or column) l % 16 at the k quad 4 (l / 16) .. + 3 (one
// float4 for k-contiguous operands, four loads for B(k, n) = B[k*ldb + n]), and the quad's
// four elements feed four MFMAs; KB k blocks of loads are in flight (2 measured best). The MFMA result of
// lane l, element t, is row 4 (l / 16) + t, column l % 16 of the 16x16 block. Every k
// extent is a multiple of 4 (as for g_gemm).
template <bool BK, int KB>
__global__ __launch_bounds__(256) void g_gemm_mfma(int M, int N, int K, const float* __restrict__ A, int64_t lda,
                                                   const float* __restrict__ Bm, int64_t ldb, float* C, int64_t ldc,
                                                   const float* R, int kchunk, float* __restrict__ part, Seg sg) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int m0 = blockIdx.y * GT, n0 = blockIdx.x * GT;
  const int kb = blockIdx.z * kchunk;
  const int ke = min(K, kb + kchunk);
  const int nbl = kb < ke ? (ke - kb + 15) / 16 : 0;   // k blocks of this slice
  const int am = m0 + 16 * w + r;
  float4 fa[KB], fb[KB][4];
  auto load = [&](int blk, float4& a, float4 (&b)[4]) {
    const int k = kb + blk * 16 + 4 * q;
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    a = z;
    if (am < M && k < ke) {
      if (sg.kseg) {
        const int sp = seg_of(k, sg.kseg);
        a = *reinterpret_cast<const float4*>(seg_pick(sg.a, sp) + (int64_t)am * lda + k - sp * sg.kseg);
      } else {
        a = *reinterpret_cast<const float4*>(A + (int64_t)am * lda + k);
      }
    }
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      const int n = n0 + 16 * sb + r;
      b[sb] = z;
      if (n < N && k < ke) {
        if (BK) {
          b[sb] = *reinterpret_cast<const float4*>(Bm + (int64_t)n * ldb + k);
        } else {
          const float* bp = Bm + (int64_t)k * ldb + n;
          b[sb].x = bp[0];
          b[sb].y = bp[ldb];
          b[sb].z = bp[2 * ldb];
          b[sb].w = bp[3 * ldb];
        }
      }
    }
  };
  f32x4 acc[4];
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) acc[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < KB; ++j)
    if (j < nbl) load(j, fa[j], fb[j]);
  for (int b0 = 0; b0 < nbl; b0 += KB) {
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int blk = b0 + j;
      if (blk < nbl) {
        const float4 a = fa[j];
        float4 bb[4];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) bb[sb] = fb[j][sb];
        if (blk + KB < nbl) load(blk + KB, fa[j], fb[j]);
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
          acc[sb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, bb[sb].x, acc[sb], 0, 0, 0);
          acc[sb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, bb[sb].y, acc[sb], 0, 0, 0);
          acc[sb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, bb[sb].z, acc[sb], 0, 0, 0);
          acc[sb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, bb[sb].w, acc[sb], 0, 0, 0);
        }
      }
    }
  }
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) {
    const int gn = n0 + 16 * sb + r;
    if (gn >= N) continue;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int gm = m0 + 16 * w + 4 * q + t;
      if (gm >= M) continue;
      const float v = acc[sb][t];
      if (part) {
        part[((int64_t)blockIdx.z * M + gm) * N + gn] = v;
        continue;
      }
      float* Cp = C;
      const float* Rp = R;
      int nn = gn;
      if (sg.nseg) {
        const int sp = seg_of(gn, sg.nseg);
        Cp = seg_pick(sg.c, sp); Rp = seg_pick(sg.r, sp); nn = gn - sp * sg.nseg;
      }
      float r0 = 0.f;
      if (Rp) r0 = Rp[(int64_t)gm * ldc + nn];
      Cp[(int64_t)gm * ldc + nn] = r0 + v;
    }
  }
}

// MFMA form of g_gemm<false, false> (the weight-gradient products dY^T X: A(m, k) =
// A[k*lda + m], B(k, n) = B[k*ldb + n], both contiguous along m / n): 64x64 tiles, k steps
// of 16 staged through LDS (one float4 per thread and operand, the next step's in
// registers), wave w owning rows 16w..16w+15 and the tile's 4 column blocks of 16; lane l
// reads its fragments at row / column l % 16 and k 4 (l / 16) + j for the j-th of four
// v_mfma_f32_16x16x4f32 per k quad. C = R + A.B, C += A.B (atomic) or the k-slice partials.
__global__ __launch_bounds__(256) void g_gemm_mfma_mn(int M, int N, int K, const float* __restrict__ A, int64_t lda,
                                                      const float* __restrict__ Bm, int64_t ldb, float* C, int64_t ldc,
                                                      const float* R, int atomic, int kchunk,
                                                      float* __restrict__ part) {
  __shared__ float As[GK][GT + 4];
  __shared__ float Bs[GK][GT + 4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int m0 = blockIdx.y * GT, n0 = blockIdx.x * GT;
  const int kb = blockIdx.z * kchunk;
  const int ke = min(K, kb + kchunk);
  const int lk = tid >> 4, lc = 4 * (tid & 15);   // the thread's float4 of each operand tile
  float4 ra, rb;
  auto load = [&](int k0) {
    const int gk = k0 + lk;
    ra = make_float4(0.f, 0.f, 0.f, 0.f);
    rb = ra;
    if (gk < ke && m0 + lc < M) ra = *reinterpret_cast<const float4*>(A + (int64_t)gk * lda + m0 + lc);
    if (gk < ke && n0 + lc < N) rb = *reinterpret_cast<const float4*>(Bm + (int64_t)gk * ldb + n0 + lc);
  };
  f32x4 acc[4];
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) acc[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (kb < ke) load(kb);
  for (int k0 = kb; k0 < ke; k0 += GK) {
    __syncthreads();
    *reinterpret_cast<float4*>(&As[lk][lc]) = ra;
    *reinterpret_cast<float4*>(&Bs[lk][lc]) = rb;
    __syncthreads();
    if (k0 + GK < ke) load(k0 + GK);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = As[4 * q + j][16 * w + r];
#pragma unroll
      for (int sb = 0; sb < 4; ++sb)
        acc[sb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, Bs[4 * q + j][16 * sb + r], acc[sb], 0, 0, 0);
    }
  }
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) {
    const int gn = n0 + 16 * sb + r;
    if (gn >= N) continue;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int gm = m0 + 16 * w + 4 * q + t;
      if (gm >= M) continue;
      const float v = acc[sb][t];
      if (part) {
        part[((int64_t)blockIdx.z * M + gm) * N + gn] = v;
      } else if (atomic) {
        atomicAdd(C + (int64_t)gm * ldc + gn, v);
      } else {
        float r0 = 0.f;
        if (R) r0 = R[(int64_t)gm * ldc + gn];
        C[(int64_t)gm * ldc + gn] = r0 + v;
      }
    }
  }
}

// C[m, n] = (R ? R[m, n] : 0) + sum_{z < splits} part[z][m][n], z ascending
__global__ void g_splitk_reduce(int M, int N, int splits, const float* __restrict__ part, const float* R, float* C,
                                int64_t ldc, Seg sg) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)M * N) return;
  const int64_t m = i / N;
  int n = (int)(i % N);
  float v = 0.f;
  for (int z = 0; z < splits; ++z) v += part[(int64_t)z * M * N + i];
  if (sg.nseg) {
    const int sp = seg_of(n, sg.nseg);
    C = seg_pick(sg.c, sp); R = seg_pick(sg.r, sp); n -= sp * sg.nseg;
  }
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

// dg[j] += sum_rows dy[row, j] * (x ? x[row, j] * rstd[row] : 1)  (gain or bias gradient):
// each chunk of kColRows rows writes its column sums to part[chunk], then g_colsum_reduce adds
// the chunks in ascending order (a fixed summation order: two calls give the same bits)
constexpr int kColRows = 64;
__global__ __launch_bounds__(256) void g_colsum(int M, int d, const float* __restrict__ dy,
                                                const float* __restrict__ x, const float* __restrict__ rstd,
                                                float* __restrict__ part) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= d) return;
  const int r0 = blockIdx.y * kColRows, r1 = min(M, r0 + kColRows);
  float acc = 0.f;
  for (int r = r0; r < r1; ++r) {
    const float v = dy[(int64_t)r * d + j];
    acc += x ? v * x[(int64_t)r * d + j] * rstd[r] : v;
  }
  part[(int64_t)blockIdx.y * d + j] = acc;
}
__global__ void g_colsum_reduce(int d, int chunks, const float* __restrict__ part, float* __restrict__ dg) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= d) return;
  float acc = 0.f;
  for (int y = 0; y < chunks; ++y) acc += part[(int64_t)y * d + j];
  dg[j] += acc;
}

// ------------------------------------------------------------------ small kernels
// cos and sin of pos * base^(-2i/dh) for positions 0..P-1 and i < dh/2: angles and their
// cosine / sine in float64, rounded to fp32 (the rotary factors every kernel below reads).
__global__ void g_rope_table(int P, int dh, double base, float2* __restrict__ tab) {
  const int half = dh / 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)P * half) return;
  const int i = (int)(idx % half);
  const double a = (double)(idx / half) * pow(base, -2.0 * i / dh);
  tab[idx] = make_float2((float)cos(a), (float)sin(a));
}

// Rotary rotation of the pairs (i, i + dh/2) of every head by sgn * angle(pos, i),
// pos = pos0 + row / rpp, with the table's factors.
__global__ void g_rope(int M, int H, int dh, float* x, int pos0, int rpp, const float2* __restrict__ tab,
                       float sgn) {
  const int half = dh / 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)M * H * half) return;
  const int i = (int)(idx % half);
  const int h = (int)((idx / half) % H);
  const int64_t row = idx / ((int64_t)half * H);
  const float2 cs = tab[(pos0 + row / rpp) * half + i];
  const float c = cs.x, s = sgn * cs.y;
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

// Embedding gradient gemb[v] += sum of gh[row] over the rows (row = t * B + b) whose token is v,
// in ascending row order: rows counted per token (integer counts), token starts by a scan,
// rows placed stably into per-token runs, then each (token, column) sums its run in order.
__device__ __forceinline__ int tok_of(const int32_t* tok, int B, int T, int r) {
  return tok[(int64_t)(r % B) * T + r / B];
}
__global__ void g_tok_hist(int M, int B, int T, const int32_t* __restrict__ tok, int* __restrict__ cnt) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r < M) atomicAdd(cnt + tok_of(tok, B, T, r), 1);
}
// start[v] = sum_{u < v} cnt[u] (one workgroup of 1024 threads, each owning a run of ids)
__global__ __launch_bounds__(1024) void g_tok_scan(int V, const int* __restrict__ cnt, int* __restrict__ start) {
  __shared__ int sums[1024];
  const int per = (V + 1023) / 1024, i0 = threadIdx.x * per, i1 = min(V, i0 + per);
  int s = 0;
  for (int i = i0; i < i1; ++i) s += cnt[i];
  sums[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int k = 0; k < 1024; ++k) {
      const int v = sums[k];
      sums[k] = run;
      run += v;
    }
  }
  __syncthreads();
  int run = sums[threadIdx.x];
  for (int i = i0; i < i1; ++i) {
    start[i] = run;
    run += cnt[i];
  }
}
// Stable placement (one workgroup): rows in chunks of 1024, in order; a row's place in its
// token's run is the run's fill so far plus the rows of the same token earlier in the chunk.
__global__ __launch_bounds__(1024) void g_tok_place(int M, int B, int T, const int32_t* __restrict__ tok,
                                                     int* __restrict__ fill, int* __restrict__ order) {
  __shared__ int ct[1024];
  for (int r0 = 0; r0 < M; r0 += 1024) {
    const int r = r0 + threadIdx.x;
    const int v = r < M ? tok_of(tok, B, T, r) : -1;
    ct[threadIdx.x] = v;
    __syncthreads();
    int before = 0, after = 0;
    for (int k = 0; k < 1024; ++k) {
      const int u = ct[k];
      before += (k < (int)threadIdx.x && u == v) ? 1 : 0;
      after += (k > (int)threadIdx.x && u == v) ? 1 : 0;
    }
    int base = 0;
    if (v >= 0) base = fill[v];
    __syncthreads();            // every thread has read fill for this chunk
    if (v >= 0) {
      order[base + before] = r;
      if (after == 0) fill[v] = base + before + 1;   // the chunk's last row of token v
    }
    __syncthreads();
  }
}
__global__ void g_embed_sum(int V, int d, const int* __restrict__ start, const int* __restrict__ cnt,
                            const int* __restrict__ order, const float* __restrict__ gh, float* __restrict__ gemb) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)V * d) return;
  const int v = (int)(idx / d), j = (int)(idx % d);
  const int s0 = start[v], n = cnt[v];
  // eight interleaved partial sums (row i of the run into sum i % 8), added in index order:
  // a fixed order, with eight independent loads in flight
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int i = 0;
  for (; i + 8 <= n; i += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] += gh[(int64_t)order[s0 + i + u] * d + j];
  }
  for (int u = 0; i + u < n; ++u) acc[u] += gh[(int64_t)order[s0 + i + u] * d + j];
  float sum = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) sum += acc[u];
  gemb[idx] += sum;
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

// ------------------------------------------- split-K reduction fused with its consumer
// Each kernel below adds the k-slices of a split product (z ascending, then R, as
// g_splitk_reduce) and applies the operation that consumes the product's rows: the same
// arithmetic as the separate kernel named with it. The rotary and SwiGLU forms give the
// separate forms' bits; the RMSNorm forms run a row on a workgroup (columns spread over 256
// threads), so their row sums are added in another order.
__device__ __forceinline__ float part_sum(const float* __restrict__ part, int64_t MN, int splits, int64_t i) {
  float v = 0.f;
#pragma unroll 8
  for (int z = 0; z < splits; ++z) v += part[(int64_t)z * MN + i];
  return v;
}

constexpr int kRowCols = 4;   // columns per thread of the row kernels: rows of up to 1024

// sum over the 256 threads of a workgroup: wave sums, then the 4 waves in order
__device__ __forceinline__ float block_sum256(float v, float* lds4) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) lds4[threadIdx.x >> 6] = v;
  __syncthreads();
  return ((lds4[0] + lds4[1]) + lds4[2]) + lds4[3];
}

// C = R + sum part (N <= 1024 columns, row stride N), then y = RMSNorm(C) * g and rstd
// (g_rms_fwd). One workgroup per row.
__global__ __launch_bounds__(256) void g_reduce_rms_fwd(int M, int N, int splits, const float* __restrict__ part,
                                                        const float* R, float* C, const float* __restrict__ g,
                                                        float eps, float* __restrict__ y, float* __restrict__ rstd) {
  __shared__ float lds4[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int64_t o = (int64_t)row * N, MN = (int64_t)M * N;
  float xv[kRowCols];
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < kRowCols; ++q) {
    const int j = tid + 256 * q;
    xv[q] = 0.f;
    if (j < N) {
      const float v = part_sum(part, MN, splits, o + j);
      xv[q] = (R ? R[o + j] : 0.f) + v;
      C[o + j] = xv[q];
      ss = fmaf(xv[q], xv[q], ss);
    }
  }
  ss = block_sum256(ss, lds4);
  const float r = 1.f / sqrtf(ss / (float)N + eps);
#pragma unroll
  for (int q = 0; q < kRowCols; ++q) {
    const int j = tid + 256 * q;
    if (j < N) y[o + j] = xv[q] * r * g[j];
  }
  if (tid == 0) rstd[row] = r;
}

// C = R + sum part (the output gradient dy of an RMSNorm, N <= 1024, row stride N), then
// out = res + dx as g_rms_bwd (res may alias out). One workgroup per row.
__global__ __launch_bounds__(256) void g_reduce_rms_bwd(int M, int N, int splits, const float* __restrict__ part,
                                                        const float* R, float* C, const float* __restrict__ x,
                                                        const float* __restrict__ rstd, const float* __restrict__ g,
                                                        const float* res, float* out) {
  __shared__ float lds4[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int64_t o = (int64_t)row * N, MN = (int64_t)M * N;
  float dv[kRowCols], xv[kRowCols], gv[kRowCols];
  float dot = 0.f;
#pragma unroll
  for (int q = 0; q < kRowCols; ++q) {
    const int j = tid + 256 * q;
    dv[q] = xv[q] = gv[q] = 0.f;
    if (j < N) {
      const float v = part_sum(part, MN, splits, o + j);
      dv[q] = (R ? R[o + j] : 0.f) + v;
      xv[q] = x[o + j];
      gv[q] = g[j];
      C[o + j] = dv[q];
      dot = fmaf(gv[q] * dv[q], xv[q], dot);
    }
  }
  dot = block_sum256(dot, lds4);
  const float r = rstd[row];
  const float c = r * r * r * dot / (float)N;
#pragma unroll
  for (int q = 0; q < kRowCols; ++q) {
    const int j = tid + 256 * q;
    if (j < N) {
      const float v = r * gv[q] * dv[q] - c * xv[q];
      out[o + j] = (res ? res[o + j] : 0.f) + v;
    }
  }
}

// C = sum part over heads of dh columns (outputs by Seg when nseg > 0, else row stride N);
// the pairs (i, i + dh/2) of the first nrot columns rotated by +angle as g_rope with
// pos = pos0 + row / rpp. One thread per pair.
__global__ void g_reduce_rope(int M, int N, int splits, const float* __restrict__ part, float* C, Seg sg, int dh,
                              int nrot, int pos0, int rpp, const float2* __restrict__ tab) {
  const int half = dh / 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)M * (N / 2)) return;
  const int npr = N / 2;
  const int64_t row = idx / npr;
  const int pi = (int)(idx % npr);
  const int n1 = (pi / half) * dh + pi % half, n2 = n1 + half;
  const int64_t MN = (int64_t)M * N;
  const float x1 = 0.f + part_sum(part, MN, splits, row * N + n1);   // 0 + v: the reduction's R-less sum
  const float x2 = 0.f + part_sum(part, MN, splits, row * N + n2);
  float y1 = x1, y2 = x2;
  if (n1 < nrot) {
    const float2 cs = tab[(pos0 + row / rpp) * half + pi % half];
    const float c = cs.x, s = 1.f * cs.y;
    y1 = x1 * c - x2 * s;
    y2 = x1 * s + x2 * c;
  }
  float* dst = C + row * N;
  int c1 = n1;
  if (sg.nseg) {
    const int sp = seg_of(n1, sg.nseg);
    dst = seg_pick(sg.c, sp) + row * sg.nseg;
    c1 = n1 - sp * sg.nseg;
  }
  dst[c1] = y1;
  dst[c1 + half] = y2;
}

// f1, f3 = the two f-column outputs of a split product (Seg, nseg = f); g = silu(f1) f3
// (g_swiglu_fwd)
__global__ void g_reduce_swiglu(int M, int f, int splits, const float* __restrict__ part, Seg sg,
                                float* __restrict__ g) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)M * f) return;
  const int64_t row = i / f;
  const int j = (int)(i % f);
  const int64_t MN = (int64_t)M * 2 * f;
  const float a = 0.f + part_sum(part, MN, splits, row * 2 * f + j);
  const float b = 0.f + part_sum(part, MN, splits, row * 2 * f + f + j);
  sg.c[0][i] = a;
  sg.c[1][i] = b;
  g[i] = a * sigm(a) * b;
}

// gg = R + sum part (C, row stride N = f); g1, g3 as g_swiglu_bwd
__global__ void g_reduce_swiglu_bwd(int M, int N, int splits, const float* __restrict__ part, const float* R,
                                    float* C, const float* __restrict__ f1, const float* __restrict__ f3,
                                    float* g1, float* __restrict__ g3) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)M * N) return;
  const float gv = (R ? R[i] : 0.f) + part_sum(part, (int64_t)M * N, splits, i);
  C[i] = gv;
  const float a = f1[i], s = sigm(a);
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
// A block of 256 threads per (row, head); a key (or, key side, a query) is handled by a group
// of G = DH/4 lanes, each with four of its dimensions in a float4, so NG = 256/G of them are in
// flight per round; dot products are group sums over shuffles. Query r of a query-side kernel
// belongs to sequence b = r % B at time tq = tq0 + r / B (0-based) and reads keys j in
// [max(0, tq - win + 1), tq] at rows j*B + b of K and V; Q, O rows are local (r), lse [nq, H].
template <int G>
__device__ __forceinline__ float gsum(float v) {
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float dot4(float4 a, float4 b) { return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w; }
__device__ __forceinline__ float4 fma4(float s, float4 a, float4 c) {
  return make_float4(fmaf(s, a.x, c.x), fmaf(s, a.y, c.y), fmaf(s, a.z, c.z), fmaf(s, a.w, c.w));
}
__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void st4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }

// The float4 x holds elements 4 gl .. 4 gl + 3 of a head row of DH values spread over the
// DH/4 lanes gl of a lane group; returns them rotated by sgn * angle of position pos, as
// g_rope (the pair partner of an element sits in lane gl ^ DH/8 of the same group).
// Every lane of the group must take part.
template <int DH>
__device__ __forceinline__ float4 rope4(float4 x, int gl, int pos, const float2* __restrict__ tab, float sgn) {
  constexpr int HG = DH / 8;
  const float xs[4] = {x.x, x.y, x.z, x.w};
  const float ps[4] = {__shfl_xor(x.x, HG, WAVE), __shfl_xor(x.y, HG, WAVE), __shfl_xor(x.z, HG, WAVE),
                       __shfl_xor(x.w, HG, WAVE)};
  const bool first = gl < HG;
  const int i0 = 4 * (gl & (HG - 1));
  float y[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float2 cs = tab[pos * (DH / 2) + i0 + e];
    const float c = cs.x, sn = sgn * cs.y;
    y[e] = first ? xs[e] * c - ps[e] * sn : ps[e] * sn + xs[e] * c;
  }
  return make_float4(y[0], y[1], y[2], y[3]);
}
template <int DH>
__device__ __forceinline__ float4 rope_inv4(float4 x, int gl, int pos, const float2* __restrict__ tab) {
  return rope4<DH>(x, gl, pos, tab, -1.f);
}

// Online softmax per group, the groups merged at the end: O and lse. With q_part, q is the
// sum of q_splits partial products [z][nq rows][part_ld]; with tab, q is first rotated by
// +angle of its position (the projection's rotary map) and, with q_save, stored rotated.
// With kv_k / kv_v (= K / V), this launch also produces the key / value row of each query's
// own position (from the slices at columns hd / 2 hd, or from K / V unrotated), rotates the
// key, attends to it from registers and stores both.
template <int DH>
__global__ __launch_bounds__(256) void g_attn_fwd(int nq, int B, int tq0, int win, int H, float scale,
                                                  const float* __restrict__ Q, const float* __restrict__ K,
                                                  const float* __restrict__ Vv, float* __restrict__ O,
                                                  float* __restrict__ lse, const float* __restrict__ q_part,
                                                  int q_splits, int part_ld, const float2* __restrict__ tab,
                                                  float* q_save, float* kv_k, float* kv_v) {
  constexpr int G = DH / 4, NG = 256 / G;
  __shared__ float4 pacc[256];
  __shared__ float pm[NG], pl[NG];
  const int r = blockIdx.x / H, h = blockIdx.x % H, tid = threadIdx.x, gi = tid / G, gl = tid % G;
  const int hd = H * DH, b = r % B, tq = tq0 + r / B;
  const int lo = max(0, tq - win + 1);
  const int64_t qo = (int64_t)r * hd + h * DH + gl * 4;
  // q (and, with kv_k, the key / value row of position tq) still as the k-slice partial sums of
  // their product (rows of part_ld columns: q, then k and v at hd and 2 hd): added here, z
  // ascending
  auto psum = [&](int col) {
    const int64_t MN = (int64_t)nq * part_ld;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
    for (int z = 0; z < q_splits; ++z) {
      const float4 v = ld4(q_part + (int64_t)z * MN + (int64_t)r * part_ld + col);
      a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
    }
    return make_float4(0.f + a.x, 0.f + a.y, 0.f + a.z, 0.f + a.w);
  };
  float4 q = q_part ? psum(h * DH + gl * 4) : ld4(Q + qo);
  const int64_t kto = ((int64_t)tq * B + b) * hd + h * DH + gl * 4;   // key / value row of tq
  float4 kt = make_float4(0.f, 0.f, 0.f, 0.f), vt = kt;
  if (kv_k) {
    kt = q_part ? psum(hd + h * DH + gl * 4) : ld4(K + kto);
    vt = q_part ? psum(2 * hd + h * DH + gl * 4) : ld4(Vv + kto);
    kt = rope4<DH>(kt, gl, tq + 1, tab, 1.f);
  }
  if (tab) q = rope4<DH>(q, gl, tq + 1, tab, 1.f);   // the projection's rotary map, applied here
  const float4 q_rot = q;
  q.x *= scale; q.y *= scale; q.z *= scale; q.w *= scale;
  float m = -INFINITY, l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // a group's keys lo + gi, lo + gi + NG, ... in that order, kU of them loaded before any is
  // used (the loads of a chunk in flight together; the arithmetic order is unchanged)
  constexpr int kU = 4;
  for (int j0 = lo + gi; j0 <= tq; j0 += kU * NG) {
    float4 kk[kU], vv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = j0 + u * NG;
      kk[u] = vv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j > tq) continue;
      if (kv_k && j == tq) {   // the row this launch produces (group-uniform branch)
        kk[u] = kt;
        vv[u] = vt;
      } else {
        const int64_t ro = ((int64_t)j * B + b) * hd + h * DH + gl * 4;
        kk[u] = ld4(K + ro);
        vv[u] = ld4(Vv + ro);
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (j0 + u * NG > tq) continue;   // group-uniform
      const float sc = gsum<G>(dot4(q, kk[u]));
      const float mn = fmaxf(m, sc);
      const float c = __expf(m - mn), p = __expf(sc - mn);
      l = l * c + p;
      acc = fma4(p, vv[u], make_float4(acc.x * c, acc.y * c, acc.z * c, acc.w * c));
      m = mn;
    }
  }
  pacc[tid] = acc;
  if (gl == 0) { pm[gi] = m; pl[gi] = l; }
  __syncthreads();
  if (tid < G) {
    float M = -INFINITY;
    for (int k = 0; k < NG; ++k) M = fmaxf(M, pm[k]);
    float den = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < NG; ++k) {
      if (pm[k] == -INFINITY) continue;
      const float e = __expf(pm[k] - M);
      den += e * pl[k];
      o = fma4(e, pacc[k * G + tid], o);
    }
    const float inv = 1.f / den;
    st4(O + (int64_t)r * hd + h * DH + tid * 4, make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv));
    if (tid == 0) lse[(int64_t)r * H + h] = M + logf(den);
    if (q_save) st4(q_save + qo, q_rot);   // after every group has read Q (q_save may be Q)
    if (kv_k) {                            // after every group has read the row (or its slices)
      st4(kv_k + kto, kt);
      st4(kv_v + kto, vt);
    }
  }
}


// Query side of the attention backward. With p_j = exp(s_j - lse) recomputed, D = dO.O,
// dS_j = p_j (dO.v_j - D): dQ = scale * sum_j dS_j k_j; Dout (optional) = D;
// KV: dK[row_j] += scale * dS_j q, dV[row_j] += p_j dO (plain read-modify-write: the launch
// must hold at most one query per (sequence, head)). rot 1: dQ leaves rotated back by the
// query's position (the gradient before the rotary map); rot 2: also the key row of the
// query's own position, whose last contribution this is. With dO_part, dO is read as the
// sum of dO_splits partial products [z][nq rows][H*DH] (the reduction its product skipped).
// dO_save (optional) receives dO, Dout (optional) D, for a later key-side pass.
template <int DH, bool KV>
__global__ __launch_bounds__(256) void g_attn_bwd_q(int nq, int B, int tq0, int win, int H, float scale,
                                                    const float* __restrict__ Q, const float* __restrict__ K,
                                                    const float* __restrict__ Vv, const float* __restrict__ O,
                                                    const float* __restrict__ lse, const float* __restrict__ dO,
                                                    float* __restrict__ dQ, float* __restrict__ Dout, float* dK,
                                                    float* dV, int rot, const float2* __restrict__ tab,
                                                    const float* __restrict__ dO_part, int dO_splits,
                                                    float* __restrict__ dO_save) {
  constexpr int G = DH / 4, NG = 256 / G;
  __shared__ float4 pdq[256];
  const int r = blockIdx.x / H, h = blockIdx.x % H, tid = threadIdx.x, gi = tid / G, gl = tid % G;
  const int hd = H * DH, b = r % B, tq = tq0 + r / B;
  const int lo = max(0, tq - win + 1);
  const int64_t qo = (int64_t)r * hd + h * DH + gl * 4;
  float4 q = ld4(Q + qo);
  q.x *= scale; q.y *= scale; q.z *= scale; q.w *= scale;
  float4 go;
  if (dO_part) {   // dO still as the k-slice partial sums of its product: added here, z ascending
    const int64_t MN = (int64_t)nq * hd;
    go = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
    for (int z = 0; z < dO_splits; ++z) {
      const float4 v = ld4(dO_part + (int64_t)z * MN + qo);
      go.x += v.x; go.y += v.y; go.z += v.z; go.w += v.w;
    }
    go.x = 0.f + go.x; go.y = 0.f + go.y; go.z = 0.f + go.z; go.w = 0.f + go.w;
  } else {
    go = ld4(dO + qo);
  }
  if (dO_save && gi == 0) st4(dO_save + qo, go);
  const float D = gsum<G>(dot4(go, ld4(O + qo)));
  const float L = lse[(int64_t)r * H + h];
  float4 dq = make_float4(0.f, 0.f, 0.f, 0.f);
  // a group's keys in order, kU of them (and their gradient rows) loaded before any is used
  constexpr int kU = 4;
  for (int j0 = lo + gi; j0 <= tq; j0 += kU * NG) {
    float4 kk[kU], vv[kU], gk[kU], gv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = j0 + u * NG;
      kk[u] = vv[u] = gk[u] = gv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j > tq) continue;
      const int64_t ro = ((int64_t)j * B + b) * hd + h * DH + gl * 4;
      kk[u] = ld4(K + ro);
      vv[u] = ld4(Vv + ro);
      if (KV) {   // rows of other keys: no other query of this launch touches them
        gk[u] = ld4(dK + ro);
        gv[u] = ld4(dV + ro);
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = j0 + u * NG;
      if (j > tq) continue;   // group-uniform
      const float p = __expf(gsum<G>(dot4(q, kk[u])) - L);
      const float ds = p * (gsum<G>(dot4(go, vv[u])) - D);
      dq = fma4(ds, kk[u], dq);
      if (KV) {
        const int64_t ro = ((int64_t)j * B + b) * hd + h * DH + gl * 4;
        float4 nk = fma4(ds, q, gk[u]);
        if (rot == 2 && j == tq) nk = rope_inv4<DH>(nk, gl, tq + 1, tab);   // the whole group takes j == tq
        st4(dK + ro, nk);
        st4(dV + ro, fma4(p, go, gv[u]));
      }
    }
  }
  pdq[tid] = dq;
  __syncthreads();
  if (tid < G) {
    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < NG; ++k) {
      const float4 x = pdq[k * G + tid];
      t.x += x.x; t.y += x.y; t.z += x.z; t.w += x.w;
    }
    float4 dqs = make_float4(t.x * scale, t.y * scale, t.z * scale, t.w * scale);
    if (rot) dqs = rope_inv4<DH>(dqs, tid, tq + 1, tab);
    st4(dQ + (int64_t)r * hd + h * DH + tid * 4, dqs);
    if (Dout && tid == 0) Dout[(int64_t)r * H + h] = D;
  }
}

// Key side of the attention backward for token-parallel causal attention over T positions:
// a block per (key row kr = tk*B + b, head); queries i in [tk, min(T-1, tk + win - 1)] at
// rows i*B + b. dK = scale * sum_i dS_i q_i, dV = sum_i p_i dO_i (written, or added when acc).
template <int DH>
__global__ __launch_bounds__(256) void g_attn_bwd_kv(int B, int T, int win, int H, float scale,
                                                     const float* __restrict__ Q, const float* __restrict__ K,
                                                     const float* __restrict__ Vv, const float* __restrict__ lse,
                                                     const float* __restrict__ Dq, const float* __restrict__ dO,
                                                     float* __restrict__ dK, float* __restrict__ dV, int acc) {
  constexpr int G = DH / 4, NG = 256 / G;
  __shared__ float4 pk[256], pv[256];
  const int kr = blockIdx.x / H, h = blockIdx.x % H, tid = threadIdx.x, gi = tid / G, gl = tid % G;
  const int hd = H * DH, b = kr % B, tk = kr / B;
  const int hi = (int)std::min<int64_t>(T - 1, (int64_t)tk + win - 1);
  const int64_t ko = (int64_t)kr * hd + h * DH + gl * 4;
  float4 k = ld4(K + ko);
  k.x *= scale; k.y *= scale; k.z *= scale; k.w *= scale;
  const float4 v = ld4(Vv + ko);
  float4 dk = make_float4(0.f, 0.f, 0.f, 0.f), dv = dk;
  for (int i = tk + gi; i <= hi; i += NG) {
    const int64_t qr = (int64_t)i * B + b;
    const int64_t ro = qr * hd + h * DH + gl * 4;
    const float4 q = ld4(Q + ro), go = ld4(dO + ro);
    const float p = __expf(gsum<G>(dot4(q, k)) - lse[qr * H + h]);
    const float ds = p * (gsum<G>(dot4(go, v)) - Dq[qr * H + h]);
    dk = fma4(ds, q, dk);
    dv = fma4(p, go, dv);
  }
  pk[tid] = dk;
  pv[tid] = dv;
  __syncthreads();
  if (tid < G) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), c = a;
    for (int j = 0; j < NG; ++j) {
      const float4 x = pk[j * G + tid], y = pv[j * G + tid];
      a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
      c.x += y.x; c.y += y.y; c.z += y.z; c.w += y.w;
    }
    const int64_t o = (int64_t)kr * hd + h * DH + tid * 4;
    float4 nk = make_float4(a.x * scale, a.y * scale, a.z * scale, a.w * scale), nv = c;
    if (acc) {
      const float4 pk = ld4(dK + o), pv = ld4(dV + o);
      nk = make_float4(pk.x + nk.x, pk.y + nk.y, pk.z + nk.z, pk.w + nk.w);
      nv = make_float4(pv.x + nv.x, pv.y + nv.y, pv.z + nv.z, pv.w + nv.w);
    }
    st4(dK + o, nk);
    st4(dV + o, nv);
  }
}

// ----------------------------------------------------------------- host helpers
struct Ctx {
  hipStream_t st;
  float* part = nullptr;   // split-K partial sums of the small-M products
  int64_t part_cap = 0;    // floats
  float* wpart = nullptr;  // split-K partial sums of the weight gradients (k = every row)
  int64_t wpart_cap = 0;   // floats
  float* cpart = nullptr;  // column-sum partials (one row per chunk of rows)
  int64_t cpart_cap = 0;   // floats
  const float2* rope_tab = nullptr;   // rotary factors [position][d_head / 2]
  hipError_t err = hipSuccess;
  void check() {
    if (err == hipSuccess) err = hipGetLastError();
  }
};

inline unsigned blocks(int64_t n) { return (unsigned)((n + 255) / 256); }

// The operation that consumes a product's rows, run by the split-K reduction when the product
// splits, else by its own kernel after the product.
// Partial sums of a split product whose reduction its consumer performs (Post::Defer).
struct Deferred {
  const float* part = nullptr;
  int splits = 0;
};
struct Post {
  enum Kind { None, RmsFwd, RmsBwd, Rope, SwiGlu, SwiGluBwd, Defer } kind = None;
  Deferred* defer = nullptr;      // Defer: receives the partials (part null: C was written)
  const float* g = nullptr;       // RmsFwd / RmsBwd: gain
  float eps = 0.f;                // RmsFwd
  float* y = nullptr;             // RmsFwd: normalised rows; SwiGlu: silu(f1) f3
  float* rstd = nullptr;          // RmsFwd: 1 / rms per row
  const float* x = nullptr;       // RmsBwd: the norm's input rows
  const float* rs = nullptr;      // RmsBwd: their 1 / rms
  const float* res = nullptr;     // RmsBwd: added to the input gradient (may alias out)
  float* out = nullptr;           // RmsBwd: input gradient
  int H = 0, dh = 0, nrot = 0, pos0 = 0, rpp = 1;   // Rope: columns [0, nrot) rotated, heads of dh
  const float* f1 = nullptr;      // SwiGluBwd: FFN pre-activations
  const float* f3 = nullptr;
  float* g1 = nullptr;            // SwiGluBwd: their gradients
  float* g3 = nullptr;
};
void post_separate(Ctx& c, int M, int N, float* C, const Seg& sg, const Post& p);

// C = R + A.B (see g_gemm), or C += A.B split over k with atomics. Products with few
// output tiles (the per-position products have B rows) split k over up to 32 slices whose
// partial sums a second kernel adds in a fixed order (deterministic).
constexpr int kMaxSplits = 32;
void gemm(Ctx& c, int M, int N, int K, const float* A, int64_t lda, bool ak, const float* Bm, int64_t ldb, bool bk,
          float* C, int64_t ldc, const float* R, bool atomic, const Seg& sg = Seg(), const Post& post = Post()) {
  // atomic: C += A.B; otherwise C = R + A.B
  if (M <= 0 || N <= 0) return;
  {   // the consumers read rows of N contiguous columns; rotary and SwiGLU products have no R
    const bool rows = post.kind == Post::RmsFwd || post.kind == Post::RmsBwd || post.kind == Post::SwiGluBwd;
    const bool nor = post.kind == Post::Rope || post.kind == Post::SwiGlu;
    if ((rows && (sg.nseg || ldc != N)) || (nor && R) || (post.kind == Post::SwiGlu && sg.nseg * 2 != N) ||
        (post.kind == Post::Rope && (sg.nseg ? sg.nseg : N) % (post.H * post.dh) != 0) ||
        (post.kind == Post::Defer && (R || ldc != (sg.nseg ? sg.nseg : N) || !post.defer)) ||
        (post.kind != Post::None && atomic)) {
      if (c.err == hipSuccess) c.err = hipErrorInvalidValue;
      return;
    }
  }
  const int tm = (M + GT - 1) / GT, tn = (N + GT - 1) / GT;
  int splits = 1;
  float* part = nullptr;
  bool accumulate = false;
  if (atomic) {
    // C += A.B: k slices write partial sums that a second kernel adds to C in slice order
    // (deterministic); one slice adds in place
    const int want = std::max(1, 1024 / (tm * tn));
    splits = std::max(1, std::min(want, (K + 255) / 256));
    while (splits > 1 && (int64_t)splits * M * N > c.wpart_cap) --splits;
    atomic = false;
    R = C;
    accumulate = true;
    if (splits > 1) part = c.wpart;
  } else if (tm * tn < 128 && K >= 128 && c.part) {
    splits = std::min({kMaxSplits, (512 + tm * tn - 1) / (tm * tn), K / 32});
    while (splits > 1 && (int64_t)splits * M * N > c.part_cap) --splits;
    if (splits > 1) part = c.part;
  }
  int kchunk = (K + splits - 1) / splits;
  kchunk = (kchunk + GK - 1) / GK * GK;
  if (kchunk <= 0) kchunk = GK;
  splits = std::max(1, (K + kchunk - 1) / kchunk);
  if (splits == 1) part = nullptr;
  (void)accumulate;
  dim3 grid(tn, tm, splits);
  const int at = atomic ? 1 : 0;
  if (ak && !atomic) {   // k-contiguous A (every product but the weight gradients): the MFMA form
    if (bk)
      g_gemm_mfma<true, 2><<<grid, 256, 0, c.st>>>(M, N, K, A, lda, Bm, ldb, C, ldc, R, kchunk, part, sg);
    else
      g_gemm_mfma<false, 2><<<grid, 256, 0, c.st>>>(M, N, K, A, lda, Bm, ldb, C, ldc, R, kchunk, part, sg);
  } else if (ak) {
    if (bk) g_gemm<true, true, 1><<<grid, 256, 0, c.st>>>(M, N, K, A, lda, Bm, ldb, C, ldc, R, at, kchunk, part, sg);
    else g_gemm<true, false, 1><<<grid, 256, 0, c.st>>>(M, N, K, A, lda, Bm, ldb, C, ldc, R, at, kchunk, part, sg);
  } else if (bk) {
    g_gemm<false, true, 1><<<grid, 256, 0, c.st>>>(M, N, K, A, lda, Bm, ldb, C, ldc, R, at, kchunk, part, sg);
  } else if (sg.kseg == 0 && sg.nseg == 0) {   // the weight gradients: MFMA with LDS-staged operands
    g_gemm_mfma_mn<<<grid, 256, 0, c.st>>>(M, N, K, A, lda, Bm, ldb, C, ldc, R, at, kchunk, part);
  } else {
    g_gemm<false, false, 1><<<grid, 256, 0, c.st>>>(M, N, K, A, lda, Bm, ldb, C, ldc, R, at, kchunk, part, sg);
  }
  c.check();
  const bool row_kernel = post.kind == Post::RmsFwd || post.kind == Post::RmsBwd;
  if (part && row_kernel && N > 256 * kRowCols) {   // rows too long for the fused form
    g_splitk_reduce<<<blocks((int64_t)M * N), 256, 0, c.st>>>(M, N, splits, part, R, C, ldc, sg);
    c.check();
    part = nullptr;
  }
  if (!part) {
    post_separate(c, M, N, C, sg, post);
    return;
  }
  switch (post.kind) {
    case Post::None:
      g_splitk_reduce<<<blocks((int64_t)M * N), 256, 0, c.st>>>(M, N, splits, part, R, C, ldc, sg);
      break;
    case Post::Defer:   // the consumer adds the slices; nothing is written to C
      post.defer->part = part;
      post.defer->splits = splits;
      break;
    case Post::RmsFwd:
      g_reduce_rms_fwd<<<M, 256, 0, c.st>>>(M, N, splits, part, R, C, post.g, post.eps, post.y, post.rstd);
      break;
    case Post::RmsBwd:
      g_reduce_rms_bwd<<<M, 256, 0, c.st>>>(M, N, splits, part, R, C, post.x, post.rs, post.g, post.res, post.out);
      break;
    case Post::Rope:
      g_reduce_rope<<<blocks((int64_t)M * (N / 2)), 256, 0, c.st>>>(M, N, splits, part, C, sg, post.dh, post.nrot,
                                                                   post.pos0, post.rpp, c.rope_tab);
      break;
    case Post::SwiGlu:
      g_reduce_swiglu<<<blocks((int64_t)M * (N / 2)), 256, 0, c.st>>>(M, N / 2, splits, part, sg, post.y);
      break;
    case Post::SwiGluBwd:
      g_reduce_swiglu_bwd<<<blocks((int64_t)M * N), 256, 0, c.st>>>(M, N, splits, part, R, C, post.f1, post.f3,
                                                                     post.g1, post.g3);
      break;
  }
  c.check();
}
// Y_p[M, out] = X[M, in] . W_p^T for the np row blocks W_p of Wcat [np*out, in] (one launch)
void lin_n(Ctx& c, int M, const float* X, int in, const float* Wcat, int out, int np, float* const* Y,
           const Post& post = Post()) {
  Seg sg;
  for (int p = 0; p < np; ++p) sg.c[p] = Y[p];
  sg.nseg = out;
  gemm(c, M, np * out, in, X, in, true, Wcat, in, true, Y[0], out, nullptr, false, sg, post);
}
// dX[M, in] = R + sum_p dY_p[M, out] . W_p for the np row blocks W_p of Wcat [np*out, in]
void lin_tk(Ctx& c, int M, const float* const* dY, int out, int np, const float* Wcat, int in, float* dX,
            const float* R, const Post& post = Post()) {
  Seg sg;
  for (int p = 0; p < np; ++p) sg.a[p] = dY[p];
  sg.kseg = out;
  gemm(c, M, in, np * out, dY[0], out, true, Wcat, in, false, dX, in, R, false, sg, post);
}
// Y[M, out] = R + X[M, in] . W^T, W row-major [out, ldw] (ldw = in unless a column slice)
void lin(Ctx& c, int M, const float* X, int in, const float* W, int64_t ldw, int out, float* Y, const float* R,
         const Post& post = Post()) {
  gemm(c, M, out, in, X, in, true, W, ldw, true, Y, out, R, false, Seg(), post);
}
// dX[M, in] = R + dY[M, out] . W, W row-major [out, ldw]
void lin_t(Ctx& c, int M, const float* dY, int out, const float* W, int64_t ldw, int in, float* dX, const float* R,
           const Post& post = Post()) {
  gemm(c, M, in, out, dY, out, true, W, ldw, false, dX, in, R, false, Seg(), post);
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
  const int chunks = (M + kColRows - 1) / kColRows;
  if ((int64_t)chunks * d > c.cpart_cap) {
    if (c.err == hipSuccess) c.err = hipErrorInvalidValue;
    return;
  }
  dim3 grid((d + 255) / 256, chunks);
  g_colsum<<<grid, 256, 0, c.st>>>(M, d, dy, x, rstd, c.cpart);
  g_colsum_reduce<<<(d + 255) / 256, 256, 0, c.st>>>(d, chunks, c.cpart, dg);
  c.check();
}
void rope(Ctx& c, int M, int H, int dh, float* x, int pos0, int rpp, float sgn) {
  const int64_t n = (int64_t)M * H * (dh / 2);
  if (n <= 0) return;
  g_rope<<<blocks(n), 256, 0, c.st>>>(M, H, dh, x, pos0, rpp, c.rope_tab, sgn);
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

// The consumer of a product that did not split: its own kernel after the product.
void post_separate(Ctx& c, int M, int N, float* C, const Seg& sg, const Post& p) {
  switch (p.kind) {
    case Post::None: break;
    case Post::Defer: *p.defer = Deferred(); break;
    case Post::RmsFwd: rms_fwd(c, M, N, C, p.g, p.eps, p.y, p.rstd); break;
    case Post::RmsBwd: rms_bwd(c, M, N, C, p.x, p.rs, p.g, p.res, p.out); break;
    case Post::Rope:
      if (sg.nseg) {
        for (int q = 0; q < 3 && q * sg.nseg < p.nrot; ++q) rope(c, M, p.H, p.dh, sg.c[q], p.pos0, p.rpp, 1.f);
      } else {
        rope(c, M, p.H, p.dh, C, p.pos0, p.rpp, 1.f);
      }
      break;
    case Post::SwiGlu:
      g_swiglu_fwd<<<blocks((int64_t)M * (N / 2)), 256, 0, c.st>>>((int64_t)M * (N / 2), sg.c[0], sg.c[1], p.y);
      c.check();
      break;
    case Post::SwiGluBwd:
      g_swiglu_bwd<<<blocks((int64_t)M * N), 256, 0, c.st>>>((int64_t)M * N, C, p.f1, p.f3, p.g1, p.g3);
      c.check();
      break;
  }
}

template <int DH>
void attn_fwd_n(Ctx& c, int nq, int B, int tq0, int win, int H, const float* Q, const float* K, const float* V,
                float* O, float* lse, const Deferred& dq, int part_ld, const float2* tab, float* q_save,
                float* kv_k, float* kv_v) {
  g_attn_fwd<DH><<<nq * H, 256, 0, c.st>>>(nq, B, tq0, win, H, 1.f / sqrtf((float)DH), Q, K, V, O, lse, dq.part,
                                           dq.splits, part_ld, tab, q_save, kv_k, kv_v);
}
// rot: Q (or the slices dq of its product) is the unrotated query; it is rotated by the
// query's position here and stored rotated to Q. kv_row (with rot, one query position per
// launch): the key / value rows of that position are the product's too (slices at columns
// hd, 2 hd of rows of 3 hd, or unrotated in K / V), produced and stored here.
void attn_fwd(Ctx& c, int nq, int B, int tq0, int win, int H, int dh, const float* Q, const float* K,
              const float* V, float* O, float* lse, const Deferred& dq = Deferred(), bool rot = false,
              bool kv_row = false) {
  if (nq <= 0) return;
  if (kv_row && (!rot || nq != B)) {
    if (c.err == hipSuccess) c.err = hipErrorInvalidValue;
    return;
  }
  const float2* tab = rot ? c.rope_tab : nullptr;
  float* qs = rot ? const_cast<float*>(Q) : nullptr;
  float* kk = kv_row ? const_cast<float*>(K) : nullptr;
  float* vv = kv_row ? const_cast<float*>(V) : nullptr;
  const int part_ld = (kv_row ? 3 : 1) * H * dh;
  switch (dh) {
    case 16: attn_fwd_n<16>(c, nq, B, tq0, win, H, Q, K, V, O, lse, dq, part_ld, tab, qs, kk, vv); break;
    case 32: attn_fwd_n<32>(c, nq, B, tq0, win, H, Q, K, V, O, lse, dq, part_ld, tab, qs, kk, vv); break;
    case 64: attn_fwd_n<64>(c, nq, B, tq0, win, H, Q, K, V, O, lse, dq, part_ld, tab, qs, kk, vv); break;
    case 128: attn_fwd_n<128>(c, nq, B, tq0, win, H, Q, K, V, O, lse, dq, part_ld, tab, qs, kk, vv); break;
    default: attn_fwd_n<256>(c, nq, B, tq0, win, H, Q, K, V, O, lse, dq, part_ld, tab, qs, kk, vv); break;
  }
  c.check();
}
template <int DH>
void attn_bwd_q_n(Ctx& c, int nq, int B, int tq0, int win, int H, const float* Q, const float* K, const float* V,
                  const float* O, const float* lse, const float* dO, float* dQ, float* Dout, float* dK, float* dV,
                  int rot, const float* dO_part, int dO_splits, float* dO_save) {
  const float sc = 1.f / sqrtf((float)DH);
  if (dK)
    g_attn_bwd_q<DH, true><<<nq * H, 256, 0, c.st>>>(nq, B, tq0, win, H, sc, Q, K, V, O, lse, dO, dQ, Dout, dK, dV,
                                                     rot, c.rope_tab, dO_part, dO_splits, dO_save);
  else
    g_attn_bwd_q<DH, false><<<nq * H, 256, 0, c.st>>>(nq, B, tq0, win, H, sc, Q, K, V, O, lse, dO, dQ, Dout, dK,
                                                      dV, rot, c.rope_tab, dO_part, dO_splits, dO_save);
}
// rot (see g_attn_bwd_q): 0 none, 1 dQ rotated back, 2 dQ and the key row of the query's
// position (needs dK and one query position per launch)
void attn_bwd_q(Ctx& c, int nq, int B, int tq0, int win, int H, int dh, const float* Q, const float* K,
                const float* V, const float* O, const float* lse, const float* dO, float* dQ, float* Dout,
                float* dK, float* dV, int rot = 0, const Deferred& dd = Deferred(), float* dO_save = nullptr) {
  if (nq <= 0) return;
  if (rot == 2 && (!dK || nq != B)) {
    if (c.err == hipSuccess) c.err = hipErrorInvalidValue;
    return;
  }
  switch (dh) {
    case 16: attn_bwd_q_n<16>(c, nq, B, tq0, win, H, Q, K, V, O, lse, dO, dQ, Dout, dK, dV, rot, dd.part, dd.splits, dO_save); break;
    case 32: attn_bwd_q_n<32>(c, nq, B, tq0, win, H, Q, K, V, O, lse, dO, dQ, Dout, dK, dV, rot, dd.part, dd.splits, dO_save); break;
    case 64: attn_bwd_q_n<64>(c, nq, B, tq0, win, H, Q, K, V, O, lse, dO, dQ, Dout, dK, dV, rot, dd.part, dd.splits, dO_save); break;
    case 128: attn_bwd_q_n<128>(c, nq, B, tq0, win, H, Q, K, V, O, lse, dO, dQ, Dout, dK, dV, rot, dd.part, dd.splits, dO_save); break;
    default: attn_bwd_q_n<256>(c, nq, B, tq0, win, H, Q, K, V, O, lse, dO, dQ, Dout, dK, dV, rot, dd.part, dd.splits, dO_save); break;
  }
  c.check();
}
template <int DH>
void attn_bwd_kv_n(Ctx& c, int B, int T, int win, int H, const float* Q, const float* K, const float* V, int acc,
                   const float* lse, const float* Dq, const float* dO, float* dK, float* dV) {
  g_attn_bwd_kv<DH><<<B * T * H, 256, 0, c.st>>>(B, T, win, H, 1.f / sqrtf((float)DH), Q, K, V, lse, Dq, dO, dK, dV,
                                                  acc);
}
// acc: add to dK / dV instead of writing them
void attn_bwd_kv(Ctx& c, int B, int T, int win, int H, int dh, const float* Q, const float* K, const float* V,
                 const float* lse, const float* Dq, const float* dO, float* dK, float* dV, int acc = 0) {
  if (B * T <= 0) return;
  switch (dh) {
    case 16: attn_bwd_kv_n<16>(c, B, T, win, H, Q, K, V, acc, lse, Dq, dO, dK, dV); break;
    case 32: attn_bwd_kv_n<32>(c, B, T, win, H, Q, K, V, acc, lse, Dq, dO, dK, dV); break;
    case 64: attn_bwd_kv_n<64>(c, B, T, win, H, Q, K, V, acc, lse, Dq, dO, dK, dV); break;
    case 128: attn_bwd_kv_n<128>(c, B, T, win, H, Q, K, V, acc, lse, Dq, dO, dK, dV); break;
    default: attn_bwd_kv_n<256>(c, B, T, win, H, Q, K, V, acc, lse, Dq, dO, dK, dV); break;
  }
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
  float *dO2 = nullptr, *D2 = nullptr;   // intermediates kept: cross-attention dO and D of every row
};
struct Bufs {
  bool ck = false;
  float *wpart = nullptr, *cpart = nullptr;
  int64_t wpart_n = 0, cpart_n = 0;
  int *tcnt = nullptr, *tstart = nullptr, *tfill = nullptr, *torder = nullptr;   // embedding gradient order
  float2* rope_tab = nullptr;   // rotary factors of positions 0..T
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
  // row-concatenated copies of each layer's [Wq; Wk; Wv] and [W1; W3] (one launch per group)
  std::vector<float*> qkv_e, w13_e, qkv_d, w13_d;
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
    if (!ck) {
      D.dO2 = A.f(M * hd);
      D.D2 = A.f(M * H);
    }
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
  u.part_n = (int64_t)kMaxSplits * B * std::max({d, hd, f, 2 * d, 3 * hd, 2 * f, (int64_t)c.vocab});
  u.part = A.f(u.part_n);
  // weight-gradient slices: room for 4 slices of the largest weight matrix (fewer slices when a
  // product would need more), at most 256 M floats
  u.wpart_n = std::min<int64_t>((int64_t)4 * std::max({hd * d, f * d, d * d, (int64_t)c.vocab * d}),
                                (int64_t)256 << 20);
  u.wpart = A.f(u.wpart_n);
  u.cpart_n = (M + kColRows - 1) / kColRows * d;
  u.cpart = A.f(u.cpart_n);
  u.tcnt = reinterpret_cast<int*>(A.f(c.vocab));
  u.tstart = reinterpret_cast<int*>(A.f(c.vocab));
  u.tfill = reinterpret_cast<int*>(A.f(c.vocab));
  u.torder = reinterpret_cast<int*>(A.f(M));
  u.rope_tab = reinterpret_cast<float2*>(A.f((int64_t)2 * (T + 1) * (c.d_head / 2)));
  for (int l = 0; l < c.L_E; ++l) {
    u.qkv_e.push_back(A.f(3 * hd * d));
    u.w13_e.push_back(A.f(2 * f * d));
  }
  for (int l = 0; l < c.L_D; ++l) {
    u.qkv_d.push_back(c.share_enc_dec ? u.qkv_e[l] : A.f(3 * hd * d));
    u.w13_d.push_back(c.share_enc_dec ? u.w13_e[l] : A.f(2 * f * d));
  }
}

// Pointers of position t (B rows) of decoder layer l.
struct Step {
  float *zin, *a, *rs1, *q, *k, *v, *o, *lse1, *z1, *b, *rs2, *qx, *ox, *lse2, *z2, *c, *rs3, *f1, *f3, *g;
  float *gq, *gk, *gv, *gz1, *gqx, *gz2, *gz3, *gda, *gdb, *gdc, *gf1, *gf3;
  float *dO2 = nullptr, *D2 = nullptr;
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
  c.wpart = u.wpart;
  c.wpart_cap = u.wpart_n;
  c.cpart = u.cpart;
  c.cpart_cap = u.cpart_n;
  c.rope_tab = u.rope_tab;
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
  {
    const int64_t n = (int64_t)(T + 1) * (dh / 2);
    g_rope_table<<<blocks(n), 256, 0, c.st>>>(T + 1, dh, base, u.rope_tab);
    c.check();
  }
  {
    const int64_t qn = (int64_t)hd * d, fn = (int64_t)f * d;
    auto cat = [&](const std::string& pre, float* qkv, float* w13) {
      add(c, qn, w(pre + "wq"), nullptr, qkv);
      add(c, qn, w(pre + "wk"), nullptr, qkv + qn);
      add(c, qn, w(pre + "wv"), nullptr, qkv + 2 * qn);
      add(c, fn, w(pre + "w1"), nullptr, w13);
      add(c, fn, w(pre + "w3"), nullptr, w13 + fn);
    };
    for (int l = 0; l < cf.L_E; ++l) cat("enc." + std::to_string(l) + ".", u.qkv_e[l], u.w13_e[l]);
    if (!cf.share_enc_dec)
      for (int l = 0; l < cf.L_D; ++l) cat("dec." + std::to_string(l) + ".", u.qkv_d[l], u.w13_d[l]);
  }

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
    if (D.dO2) {
      s.dO2 = D.dO2 + R0 * hd;
      s.D2 = D.D2 + R0 * H;
    }
    return s;
  };
  auto mrow = [&](float* p, int t, int64_t width) { return p + (ck ? 0 : (int64_t)t * B * width); };

  // ------------------------------------------------------------ forward: encoder
  auto enc_fwd = [&](int l) {
    EncBuf& e = u.enc[ck ? 0 : l];
    rms_fwd(c, M, d, u.eh[l], w(E(l, "n1")), eps, e.a, e.rs1);
    {
      float* y[3] = {e.q, e.k, e.v};
      lin_n(c, M, e.a, d, u.qkv_e[l], hd, 3, y);
    }
    rope(c, M, H, dh, e.q, 1, B, 1.f);
    rope(c, M, H, dh, e.k, 1, B, 1.f);
    attn_fwd(c, M, B, 0, NOWIN, H, dh, e.q, e.k, e.v, e.o, e.lse);
    lin(c, M, e.o, hd, w(E(l, "wo")), hd, d, e.mid, u.eh[l]);
    rms_fwd(c, M, d, e.mid, w(E(l, "n2")), eps, e.c, e.rs2);
    {
      float* y[2] = {e.f1, e.f3};
      lin_n(c, M, e.c, d, u.w13_e[l], f, 2, y);
    }
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
      rope(c, M, H, dh, u.mk[gi], 1, B, 1.f);
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
    {
      Seg sg;   // W_g [e_t ; r] in one product (k over the two inputs)
      sg.a[0] = et; sg.a[1] = r; sg.kseg = d;
      gemm(c, B, d, 2 * d, et, d, true, w("merge.wg"), 2 * d, true, u.tBd, d, nullptr, false, sg);
    }
    lin(c, B, r, d, w("merge.ws"), d, d, mrow(u.sr, t, d), nullptr);
    g_merge_fwd<<<blocks(Bd), 256, 0, c.st>>>(B, d, et, u.tBd, w("merge.bg"), mrow(u.sr, t, d), alpha,
                                               mrow(u.gate, t, d), uu);
    c.check();
  };
  // block l at position t up to its FFN hidden state (the block output is the caller's);
  // with_kv: also this position's key and value rows
  // normalised: the block input's RMSNorm (s.a, s.rs1) was written by the producer of s.zin
  auto rope_post = [&](int nrot, int t) {
    Post p;
    p.kind = Post::Rope; p.H = H; p.dh = dh; p.nrot = nrot; p.pos0 = t + 1; p.rpp = B;
    return p;
  };
  auto rms_post = [&](const std::string& gain, float* y, float* rstd) {
    Post p;
    p.kind = Post::RmsFwd; p.g = w(gain); p.eps = eps; p.y = y; p.rstd = rstd;
    return p;
  };
  auto layer_fwd = [&](int l, int t, bool with_kv, bool normalised) {
    const DecBuf& D = u.dec[l];
    const Step s = step(l, t);
    if (!normalised) rms_fwd(c, B, d, s.zin, w(Dn(l, "m1")), eps, s.a, s.rs1);
    {   // q (and the key / value rows of t) from the product's slices (or the product), summed,
        // rotated and stored by the attention kernel
      Deferred dq;
      Post p;
      p.kind = Post::Defer; p.defer = &dq;
      if (with_kv) {
        float* y[3] = {s.q, s.k, s.v};
        lin_n(c, B, s.a, d, u.qkv_d[l], hd, 3, y, p);
      } else {
        lin(c, B, s.a, d, w(Ds(l, "wq")), d, hd, s.q, nullptr, p);
      }
      attn_fwd(c, B, B, t, cf.window, H, dh, s.q, D.k, D.v, s.o, s.lse1, dq, true, with_kv);
    }
    lin(c, B, s.o, hd, w(Ds(l, "wo")), hd, d, s.z1, s.zin, rms_post(Dn(l, "m2"), s.b, s.rs2));
    {   // the cross-attention query: its product's slices (or the product) summed, rotated and
        // stored by the attention kernel
      Deferred dq;
      Post p;
      p.kind = Post::Defer; p.defer = &dq;
      lin(c, B, s.b, d, w(Dn(l, "xq")), d, hd, s.qx, nullptr, p);
      attn_fwd(c, B, B, t, NOWIN, H, dh, s.qx, u.mk[grp(l)], u.mv[grp(l)], s.ox, s.lse2, dq, true);
    }
    lin(c, B, s.ox, hd, w(Dn(l, "xo")), hd, d, s.z2, s.z1, rms_post(Dn(l, "m3"), s.c, s.rs3));
    {
      float* y[2] = {s.f1, s.f3};
      Post p;
      p.kind = Post::SwiGlu; p.y = s.g;
      lin_n(c, B, s.c, d, u.w13_d[l], f, 2, y, p);
    }
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
      const Step s = layer_fwd(l, t, true, l > 0);
      float* out = (l + 1 < cf.L_D ? u.dec[l + 1].zin : u.S) + R0 * d;
      Post p;   // the next block's input norm
      if (l + 1 < cf.L_D) {
        const Step n = step(l + 1, t);
        p = rms_post(Dn(l + 1, "m1"), n.a, n.rs1);
      }
      lin(c, B, s.g, f, w(Ds(l, "w2")), f, d, out, s.z2, p);
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
  auto defer_post = [](Deferred* dd) {
    Post p;
    p.kind = Post::Defer; p.defer = dd;
    return p;
  };
  auto rms_bwd_post = [&](const std::string& gain, const float* x, const float* rs, const float* res, float* out) {
    Post p;
    p.kind = Post::RmsBwd; p.g = w(gain); p.x = x; p.rs = rs; p.res = res; p.out = out;
    return p;
  };
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
      for (int l = 0; l < cf.L_D; ++l) layer_fwd(l, t, false, false);
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
      {
        Post p;
        p.kind = Post::SwiGluBwd; p.f1 = s.f1; p.f3 = s.f3; p.g1 = s.gf1; p.g3 = s.gf3;
        lin_t(c, B, s.gz3, d, w(Ds(l, "w2")), f, f, u.tBf, nullptr, p);
      }
      {
        const float* gy[2] = {s.gf1, s.gf3};
        lin_tk(c, B, gy, f, 2, u.w13_d[l], d, s.gdc, nullptr, rms_bwd_post(Dn(l, "m3"), s.z2, s.rs3, s.gz3, s.gz2));
      }
      // cross-attention over memory rows 1..t
      const int gi = grp(l);
      Deferred dd;   // dO of the attention: the product's slices, added by the attention backward
      lin_t(c, B, s.gz2, d, w(Dn(l, "xo")), hd, hd, u.tBhd, nullptr, defer_post(&dd));
      // the query gradient leaves rotated back; the memory's key / value gradients come from
      // the key-side pass after the scan when every row's dO and D are kept, else here
      if (s.dO2)
        attn_bwd_q(c, B, B, t, NOWIN, H, dh, s.qx, u.mk[gi], u.mv[gi], s.ox, s.lse2, u.tBhd, s.gqx, s.D2, nullptr,
                   nullptr, 1, dd, s.dO2);
      else
        attn_bwd_q(c, B, B, t, NOWIN, H, dh, s.qx, u.mk[gi], u.mv[gi], s.ox, s.lse2, u.tBhd, s.gqx, nullptr,
                   u.gmk[gi], u.gmv[gi], 1, dd);
      lin_t(c, B, s.gqx, hd, w(Dn(l, "xq")), d, d, s.gdb, nullptr, rms_bwd_post(Dn(l, "m2"), s.z1, s.rs2, s.gz2, s.gz1));
      // window attention; the key/value gradient rows of t are complete afterwards
      lin_t(c, B, s.gz1, d, w(Ds(l, "wo")), hd, hd, u.tBhd, nullptr, defer_post(&dd));
      // the query gradient and the (now complete) key gradient row of t leave rotated back
      attn_bwd_q(c, B, B, t, cf.window, H, dh, s.q, D.k, D.v, s.o, s.lse1, u.tBhd, s.gq, nullptr, D.gk, D.gv, 2,
                 dd);
      {
        const float* gy[3] = {s.gq, s.gk, s.gv};
        float* gin = l > 0 ? step(l - 1, t).gz3 : u.gu;
        lin_tk(c, B, gy, hd, 3, u.qkv_d[l], d, s.gda, nullptr, rms_bwd_post(Dn(l, "m1"), s.zin, s.rs1, s.gz1, gin));
      }
      if (ck) layer_wgrad(l, s, B);
    }
    float* get = u.ge + o;
    if (mg) {
      float* ggp = mrow(u.ggp, t, d);
      float* gsr = mrow(u.gsr, t, d);
      float* gmr = mrow(u.gmr, t, d);
      g_merge_bwd<<<blocks(Bd), 256, 0, c.st>>>(Bd, u.gu, mrow(u.gate, t, d), mrow(u.sr, t, d), alpha, ggp, gsr);
      c.check();
      {
        Seg sg;   // [de_t | dr] = ggp . W_g in one product (n over the two outputs); de_t adds du
        sg.c[0] = get; sg.c[1] = gmr; sg.r[0] = u.gu; sg.nseg = d;
        gemm(c, B, 2 * d, d, ggp, d, true, w("merge.wg"), 2 * d, false, get, d, nullptr, false, sg);
      }
      if (cf.variant == RLT_V1)
        lin_t(c, B, gsr, d, w("merge.ws"), d, d, gmr, gmr,
              rms_bwd_post("merge.ns", u.msrc + o, mrow(u.mrs, t, 1), nullptr, u.carry));
      else
        lin_t(c, B, gsr, d, w("merge.ws"), d, d, gmr, gmr,
              rms_bwd_post("merge.ns", u.msrc + o, mrow(u.mrs, t, 1), u.greg, u.greg));
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
  // the memory's key / value gradients, one key-side pass per decoder layer over every
  // (query, key) pair of its cross-attention (keys 1..t for the query at t)
  for (int l = 0; l < cf.L_D; ++l) {
    const DecBuf& D = u.dec[l];
    if (!D.dO2) break;
    attn_bwd_kv(c, B, T, NOWIN, H, dh, D.qx, u.mk[grp(l)], u.mv[grp(l)], D.lse2, D.D2, D.dO2, u.gmk[grp(l)],
                u.gmv[grp(l)], 1);
  }
  // ------------------------------------------------------------ backward: memory
  if (cf.L_D > 0) {
    for (int gi = 0; gi < cf.groups; ++gi) {
      rope(c, M, H, dh, u.gmk[gi], 1, B, -1.f);
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
    {
      const float* gy[2] = {u.gf1, u.gf3};
      lin_tk(c, M, gy, f, 2, u.w13_e[l], d, u.gec, nullptr);
    }
    wgrad(c, M, u.gf1, f, e.c, d, g(E(l, "w1")), d);
    wgrad(c, M, u.gf3, f, e.c, d, g(E(l, "w3")), d);
    colsum(c, M, d, u.gec, e.mid, e.rs2, g(E(l, "n2")));
    rms_bwd(c, M, d, u.gec, e.mid, e.rs2, w(E(l, "n2")), gh, u.gmid);
    lin_t(c, M, u.gmid, d, w(E(l, "wo")), hd, hd, u.geo, nullptr);
    wgrad(c, M, u.gmid, d, e.o, hd, g(E(l, "wo")), hd);
    attn_bwd_q(c, M, B, 0, NOWIN, H, dh, e.q, e.k, e.v, e.o, e.lse, u.geo, u.geq, u.Dq, nullptr, nullptr);
    attn_bwd_kv(c, B, T, NOWIN, H, dh, e.q, e.k, e.v, e.lse, u.Dq, u.geo, u.gek, u.gev);
    rope(c, M, H, dh, u.geq, 1, B, -1.f);
    rope(c, M, H, dh, u.gek, 1, B, -1.f);
    {
      const float* gy[3] = {u.geq, u.gek, u.gev};
      lin_tk(c, M, gy, hd, 3, u.qkv_e[l], d, u.gec, nullptr);
    }
    wgrad(c, M, u.geq, hd, e.a, d, g(E(l, "wq")), d);
    wgrad(c, M, u.gek, hd, e.a, d, g(E(l, "wk")), d);
    wgrad(c, M, u.gev, hd, e.a, d, g(E(l, "wv")), d);
    colsum(c, M, d, u.gec, u.eh[l], e.rs1, g(E(l, "n1")));
    rms_bwd(c, M, d, u.gec, u.eh[l], e.rs1, w(E(l, "n1")), u.gmid, u.gh);
    gh = u.gh;
  }
  {
    fill(c, reinterpret_cast<float*>(u.tcnt), V, 0.f);   // zero bits: integer zeros
    g_tok_hist<<<blocks(M), 256, 0, c.st>>>(M, B, T, tokens, u.tcnt);
    g_tok_scan<<<1, 1024, 0, c.st>>>(V, u.tcnt, u.tstart);
    hipMemcpyAsync(u.tfill, u.tstart, sizeof(int) * V, hipMemcpyDeviceToDevice, c.st);
    g_tok_place<<<1, 1024, 0, c.st>>>(M, B, T, tokens, u.tfill, u.torder);
    g_embed_sum<<<blocks((int64_t)V * d), 256, 0, c.st>>>(V, d, u.tstart, u.tcnt, u.torder, gh, g("emb"));
    c.check();
  }
  return c.err;
}

}  // namespace rlt
