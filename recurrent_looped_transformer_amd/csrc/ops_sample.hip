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
// Scores and the log-sum-exp in float64, in chunks of 4096 ids (one 1024-thread pass each)
// combined in a fixed order: a workgroup per row walks its chunks (rlt_sample), or a
// workgroup per (row, chunk) and a combining pass run them side by side (rlt_generate,
// which has a workspace), with the same values bit for bit. The cost is the float64 Gumbel
// noise (two logarithms per id). The replay's next-token log-probability (logprob_k) uses
// the same chunked log-sum-exp, so both evaluate log softmax identically.
#include <climits>
#include <mutex>

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

// Block-wide float64 max and sum over a fixed tree.
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
// Log-softmax and the draw are defined over chunks of kChunk = 4 * kSampleThreads ids:
// chunk c holds ids [c * kChunk, (c + 1) * kChunk), thread t its group 4 (c * kSampleThreads
// + t) .. + 3. Per chunk (block trees, fixed order): m_c = max z, s_c = sum exp(z - m_c), and
// the best (score, id). Over chunks in ascending order: M = max m_c, S = sum e^(m_c - M) s_c,
// the best (score, id) with ties to the lower id; log softmax(z)_j = z_j - (M + log S).
// Whether one workgroup walks the chunks or a workgroup per chunk computes them, the values
// are the same bit for bit.
constexpr int kChunk = 4 * kSampleThreads;
constexpr int kMaxChunks = 256;   // vocabularies up to 2^20 ids

struct ChunkStat {
  double m, s, best;
  int bj;
};

// Chunk c of the row x (all threads of the block; the result is valid in every thread).
// scores: also the draw's best (score, id): z itself when greedy, else z + Gumbel noise.
__device__ ChunkStat chunk_stat(const float* __restrict__ x, int V, int c, double div, bool scores, bool greedy,
                                uint64_t seed, uint64_t step, int b, double* red, int* redj) {
  const int jb = c * kSampleThreads + threadIdx.x;
  double z[4];
  double mx = -INFINITY, best = -INFINITY;
  int bj = INT_MAX;
  uint64_t cw[4] = {(uint64_t)jb, (uint64_t)b, step, 0ull};
  if (scores && !greedy) philox4x64_10(cw, seed, 0ull);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int j = 4 * jb + w;
    z[w] = -INFINITY;
    if (j < V) {
      z[w] = (double)x[j] / div;
      mx = fmax(mx, z[w]);
      if (scores) {
        if (greedy) {
          best_merge(best, bj, z[w], j);
        } else {
          const double u = ((double)(cw[w] >> 11) + 0.5) * 0x1p-53;
          best_merge(best, bj, z[w] - log(-log(u)), j);
        }
      }
    }
  }
  ChunkStat r;
  r.m = block_max_d(mx, red);
  double sl = 0.0;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    if (4 * jb + w < V) sl += exp(z[w] - r.m);
  r.s = block_sum_d(sl, red);
  r.best = -INFINITY;
  r.bj = INT_MAX;
  if (scores) {
    red[threadIdx.x] = best;
    redj[threadIdx.x] = bj;
    __syncthreads();
    for (int h = kSampleThreads / 2; h > 0; h >>= 1) {
      if (threadIdx.x < h) {
        double y = red[threadIdx.x];
        int jj = redj[threadIdx.x];
        best_merge(y, jj, red[threadIdx.x + h], redj[threadIdx.x + h]);
        red[threadIdx.x] = y;
        redj[threadIdx.x] = jj;
      }
      __syncthreads();
    }
    r.best = red[0];
    r.bj = redj[0];
    __syncthreads();
  }
  return r;
}

// M + log S and the best id over nc chunk statistics (one thread)
__device__ void combine_chunks(const ChunkStat* st, int nc, double& lse, int& bj) {
  double M = -INFINITY, best = -INFINITY;
  bj = INT_MAX;
  for (int c = 0; c < nc; ++c) {
    M = fmax(M, st[c].m);
    best_merge(best, bj, st[c].best, st[c].bj);
  }
  double S = 0.0;
  for (int c = 0; c < nc; ++c) S += exp(st[c].m - M) * st[c].s;
  lse = M + log(S);
}

// One workgroup per row, walking the chunks.
__global__ __launch_bounds__(kSampleThreads) void sample_k(const float* __restrict__ logits, int64_t ld, int V,
                                                           float tau, uint64_t seed, uint64_t step, int32_t* tok,
                                                           int64_t tok_ld, float* lp, int64_t lp_ld, int32_t* next) {
  __shared__ double red[kSampleThreads];
  __shared__ int redj[kSampleThreads];
  __shared__ ChunkStat st[kMaxChunks];
  const int b = blockIdx.x;
  const float* x = logits + (int64_t)b * ld;
  const bool greedy = !(tau > 0.f);
  const double div = greedy ? 1.0 : (double)tau;
  const int nc = (V + kChunk - 1) / kChunk;
  for (int c = 0; c < nc; ++c) {
    const ChunkStat r = chunk_stat(x, V, c, div, true, greedy, seed, step, b, red, redj);
    if (threadIdx.x == 0) st[c] = r;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double lse;
    int j;
    combine_chunks(st, nc, lse, j);
    tok[(int64_t)b * tok_ld] = j;
    if (next) next[b] = j;
    if (lp) lp[(int64_t)b * lp_ld] = greedy ? 0.f : (float)((double)x[j] / div - lse);
  }
}

// A workgroup per (row, chunk) writing its statistics to ws[b][c]; sample_combine_k finishes.
__global__ __launch_bounds__(kSampleThreads) void sample_chunks_k(const float* __restrict__ logits, int64_t ld,
                                                                  int V, float tau, uint64_t seed, uint64_t step,
                                                                  ChunkStat* __restrict__ ws) {
  __shared__ double red[kSampleThreads];
  __shared__ int redj[kSampleThreads];
  const int b = blockIdx.x, c = blockIdx.y;
  const bool greedy = !(tau > 0.f);
  const ChunkStat r = chunk_stat(logits + (int64_t)b * ld, V, c, greedy ? 1.0 : (double)tau, true, greedy, seed,
                                 step, b, red, redj);
  if (threadIdx.x == 0) ws[(int64_t)b * gridDim.y + c] = r;
}

__global__ void sample_combine_k(const float* __restrict__ logits, int64_t ld, int V, int nc, float tau,
                                 const ChunkStat* __restrict__ ws, int rows, int32_t* tok, int64_t tok_ld, float* lp,
                                 int64_t lp_ld, int32_t* next) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= rows) return;
  const bool greedy = !(tau > 0.f);
  const double div = greedy ? 1.0 : (double)tau;
  double lse;
  int j;
  combine_chunks(ws + (int64_t)b * nc, nc, lse, j);
  tok[(int64_t)b * tok_ld] = j;
  if (next) next[b] = j;
  if (lp) lp[(int64_t)b * lp_ld] = greedy ? 0.f : (float)((double)logits[(int64_t)b * ld + j] / div - lse);
}

// log p(tok | logits row) = z_tok - log sum exp(z), z = logits (the sampler's arithmetic at
// temperature 1, so a replay's log-probability of a token drawn at temperature 1 from the
// same logits equals the recorded behaviour log-probability bit for bit)
__global__ __launch_bounds__(kSampleThreads) void logprob_k(const float* __restrict__ logits, RowMap lm,
                                                            const int32_t* __restrict__ tok, RowMap tm,
                                                            float* __restrict__ out, RowMap om, int V) {
  __shared__ double red[kSampleThreads];
  __shared__ int redj[kSampleThreads];
  __shared__ ChunkStat st[kMaxChunks];
  const int r = blockIdx.x;
  const float* x = logits + lm.off(r);
  const int nc = (V + kChunk - 1) / kChunk;
  for (int c = 0; c < nc; ++c) {
    const ChunkStat q = chunk_stat(x, V, c, 1.0, false, false, 0ull, 0ull, 0, red, redj);
    if (threadIdx.x == 0) st[c] = q;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double lse;
    int j;
    combine_chunks(st, nc, lse, j);
    const int t = tok[tm.off(r)];
    out[om.off(r)] = t >= 0 ? (float)((double)x[t] / 1.0 - lse) : 0.f;
  }
}

__global__ void ratio_k(const float* __restrict__ a, const float* __restrict__ b, int64_t n, float* __restrict__ r) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) r[i] = (float)exp((double)a[i] - (double)b[i]);
}

}  // namespace

int64_t sample_workspace_bytes(int rows, int V) {
  return (int64_t)rows * ((V + kChunk - 1) / kChunk) * (int64_t)sizeof(ChunkStat);
}

// Scratch of the allocation-free sampler entry point: the chunk statistics of one call, in a
// device array of fixed size that the library holds on every GPU it runs on until the process
// ends. Host code never passes the array's name to a kernel (in host code it is a stand-in,
// not a device address): the device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[kSampleScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};
bool g_scratch_ok[kMaxDevices] = {};
std::mutex g_scratch_mu;
}  // namespace

hipError_t sample_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ok[dev]) {   // first call on this device (the device is current)
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
    g_scratch_ok[dev] = true;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

void sample_rows(const float* logits, int64_t ld, int rows, int V, float temperature, uint64_t seed, uint64_t step,
                 int32_t* tok, int64_t tok_ld, float* lp, int64_t lp_ld, int32_t* next, hipStream_t st, void* ws) {
  if (rows <= 0) return;
  const int nc = (V + kChunk - 1) / kChunk;
  if (ws && nc > 1) {
    ChunkStat* w = static_cast<ChunkStat*>(ws);
    hipLaunchKernelGGL(sample_chunks_k, dim3(rows, nc), dim3(kSampleThreads), 0, st, logits, ld, V, temperature, seed,
                       step, w);
    hipLaunchKernelGGL(sample_combine_k, dim3((rows + 63) / 64), dim3(64), 0, st, logits, ld, V, nc, temperature, w,
                       rows, tok, tok_ld, lp, lp_ld, next);
  } else {
    hipLaunchKernelGGL(sample_k, dim3(rows), dim3(kSampleThreads), 0, st, logits, ld, V, temperature, seed, step, tok,
                       tok_ld, lp, lp_ld, next);
  }
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
