// Behaviour sampling with recorded log-probabilities, and the importance ratio.
//
// The sampler draws each token from mu = softmax(logits / tau) over the whole vocabulary
// and records log mu of the drawn token, the denominator of the trainer's importance ratio
// r = exp(log p_Theta - log mu) (jiphyeonjeon.kr review "Recurrent Looped Transformer",
// §6.2, Figure 4 and eq 5.5). The draw is the Gumbel-max form: argmax_j (logits_j / tau
// + G_j), G_j = -log(-log U_j), with U_j from the counter-based generator Philox4x64-10
// (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011):
// row b, entry j, draw index `step` use key (seed, 0), counter (j / 4, b, step, 0) and
// output word j % 4, U = ((x >> 11) + 0.5) * 2^-53. Every draw is a pure function of
// (seed, step, b, j), so a sequence of draws does not depend on how the calls are split.
// tau = 0 is greedy decoding (lowest index on ties, log mu = 0).
//
// One workgroup of 1024 threads per row; scores and the log-sum-exp in float64. The cost is
// the float64 Gumbel noise (two logarithms per id) and exponentials: a row of 32000 ids is
// about 60 of each per thread. The replay's next-token log-probability (logprob_k) uses the
// same log-sum-exp routine, so both evaluate log softmax identically.
#include <climits>

#include "common.hpp"
#include "ops.hpp"

namespace rlt {
namespace {

constexpr uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ull, kPhiloxM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxW0 = 0x9E3779B97F4A7C15ull, kPhiloxW1 = 0xBB67AE8584CAA73Bull;

// ten rounds of the two multiply-high/low S-boxes, key advanced by the Weyl constants
// between rounds
__device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
    const uint64_t lo0 = kPhiloxM0 * c[0], hi0 = __umul64hi(kPhiloxM0, c[0]);
    const uint64_t lo1 = kPhiloxM1 * c[2], hi1 = __umul64hi(kPhiloxM1, c[2]);
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

constexpr int kSampleThreads = 1024;

// (score, index) with the larger score winning and the lower index breaking ties
__device__ __forceinline__ void best_merge(double& y, int& j, double y2, int j2) {
  if (y2 > y || (y2 == y && j2 < j)) {
    y = y2;
    j = j2;
  }
}

// Row log-sum-exp of z_j = x_j / div in float64, shared by the sampler and the replay's
// log-probability so that both evaluate log softmax with the same operations in the same
// order: thread t visits j = 4 jb .. 4 jb + 3 for jb = t, t + 1024, ...; max, then the sum of
// exp(z - max), each reduced over the block in a fixed tree.
__device__ __forceinline__ double block_max_d(double v, double* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int h = kSampleThreads / 2; h > 0; h >>= 1) {
    if (threadIdx.x < h) red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + h]);
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}
__device__ __forceinline__ double block_sum_d(double v, double* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int h = kSampleThreads / 2; h > 0; h >>= 1) {
    if (threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}
__device__ __forceinline__ double row_sum_exp(const float* x, int V, double div, double mx, double* red) {
  double s = 0.0;
  for (int jb = threadIdx.x; jb < (V + 3) / 4; jb += kSampleThreads)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int j = 4 * jb + w;
      if (j < V) s += exp((double)x[j] / div - mx);
    }
  return block_sum_d(s, red);
}

__global__ __launch_bounds__(kSampleThreads) void sample_k(const float* __restrict__ logits, int64_t ld, int V,
                                                           float tau, uint64_t seed, uint64_t step, int32_t* tok,
                                                           int64_t tok_ld, float* lp, int64_t lp_ld, int32_t* next) {
  __shared__ double red[kSampleThreads];
  __shared__ int redj[kSampleThreads];
  const int b = blockIdx.x;
  const float* x = logits + (int64_t)b * ld;
  const bool greedy = !(tau > 0.f);
  const double div = greedy ? 1.0 : (double)tau;
  double best = -INFINITY, mx = -INFINITY;
  int bj = INT_MAX;
  for (int jb = threadIdx.x; jb < (V + 3) / 4; jb += kSampleThreads) {
    uint64_t c[4] = {(uint64_t)jb, (uint64_t)b, step, 0ull};
    if (!greedy) philox4x64_10(c, seed, 0ull);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int j = 4 * jb + w;
      if (j < V) {
        const double z = (double)x[j] / div;
        mx = fmax(mx, z);
        if (greedy) {
          best_merge(best, bj, z, j);
        } else {
          const double u = ((double)(c[w] >> 11) + 0.5) * 0x1p-53;
          best_merge(best, bj, z - log(-log(u)), j);
        }
      }
    }
  }
  // the draw: block argmax of the scores
  red[threadIdx.x] = best;
  redj[threadIdx.x] = bj;
  __syncthreads();
  for (int h = kSampleThreads / 2; h > 0; h >>= 1) {
    if (threadIdx.x < h) {
      double y = red[threadIdx.x];
      int j = redj[threadIdx.x];
      best_merge(y, j, red[threadIdx.x + h], redj[threadIdx.x + h]);
      red[threadIdx.x] = y;
      redj[threadIdx.x] = j;
    }
    __syncthreads();
  }
  const int j = redj[0];
  __syncthreads();
  if (greedy) {
    if (threadIdx.x == 0) {
      tok[(int64_t)b * tok_ld] = j;
      if (next) next[b] = j;
      if (lp) lp[(int64_t)b * lp_ld] = 0.f;
    }
    return;
  }
  const double M = block_max_d(mx, red);
  const double S = row_sum_exp(x, V, div, M, red);
  if (threadIdx.x == 0) {
    tok[(int64_t)b * tok_ld] = j;
    if (next) next[b] = j;
    if (lp) lp[(int64_t)b * lp_ld] = (float)((double)x[j] / div - (M + log(S)));
  }
}

// log p(tok | logits row) = z_tok - log sum exp(z), z = logits (the sampler's arithmetic at
// temperature 1, so a replay's log-probability of a token drawn at temperature 1 from the
// same logits equals the recorded behaviour log-probability bit for bit)
__global__ __launch_bounds__(kSampleThreads) void logprob_k(const float* __restrict__ logits, RowMap lm,
                                                            const int32_t* __restrict__ tok, RowMap tm,
                                                            float* __restrict__ out, RowMap om, int V) {
  __shared__ double red[kSampleThreads];
  const int r = blockIdx.x;
  const float* x = logits + lm.off(r);
  double mx = -INFINITY;
  for (int jb = threadIdx.x; jb < (V + 3) / 4; jb += kSampleThreads)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int j = 4 * jb + w;
      if (j < V) mx = fmax(mx, (double)x[j] / 1.0);
    }
  const double M = block_max_d(mx, red);
  const double S = row_sum_exp(x, V, 1.0, M, red);
  if (threadIdx.x == 0) {
    const int t = tok[tm.off(r)];
    out[om.off(r)] = t >= 0 ? (float)((double)x[t] / 1.0 - (M + log(S))) : 0.f;
  }
}

__global__ void ratio_k(const float* __restrict__ a, const float* __restrict__ b, int64_t n, float* __restrict__ r) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) r[i] = (float)exp((double)a[i] - (double)b[i]);
}

}  // namespace

void sample_rows(const float* logits, int64_t ld, int rows, int V, float temperature, uint64_t seed, uint64_t step,
                 int32_t* tok, int64_t tok_ld, float* lp, int64_t lp_ld, int32_t* next, hipStream_t st) {
  if (rows <= 0) return;
  hipLaunchKernelGGL(sample_k, dim3(rows), dim3(kSampleThreads), 0, st, logits, ld, V, temperature, seed, step, tok,
                     tok_ld, lp, lp_ld, next);
}

void logprob(const float* logits, RowMap lm, const int32_t* tok, RowMap tm, float* out, RowMap om, int rows, int V,
             hipStream_t st) {
  if (rows <= 0) return;
  hipLaunchKernelGGL(logprob_k, dim3(rows), dim3(kSampleThreads), 0, st, logits, lm, tok, tm, out, om, V);
}

void importance_ratio(const float* lp_cur, const float* lp_beh, int64_t n, float* ratio, hipStream_t st) {
  if (n <= 0) return;
  hipLaunchKernelGGL(ratio_k, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, lp_cur, lp_beh, n, ratio);
}

}  // namespace rlt
