// A6 - expert co-selection counts W[E][E].
//
// Source: "Expert Coupling in MoE Pretraining" (summary), "Method 1": the
// correlation graph W[e][e'] counts the tokens that select both e and e'; it is
// the input of the placement search.  "Correlation Formation and Stability":
// about 4096 tokens (one micro-batch of one rank) suffice to fit it.
// The diagonal W[e][e] counts the tokens selecting e (a reading; it does not
// change any placement objective).
//
// Design: with S_e the set of tokens that select e, W[a][b] = |S_a & S_b|.
//  1. coselect_bits: one wave per 64-token word.  Lane l takes the word's top-k
//     ids at flat positions l, l + 64, ... (coalesced loads), sets the token's
//     bit in its expert's LDS bitset word (ds_or_b64, order independent) and the
//     wave writes the E words to S[E][words] in the workspace.  Spread over
//     many CUs, so no CU streams all the ids.
//  2. coselect_pairs: one 1024-thread workgroup per 16 x 16 tile of W in the
//     upper triangle.  It stages its 32 experts' bitset rows in LDS (16 KiB per
//     4096 tokens), sums popcount(S_a & S_b) for each cell with four threads per
//     cell, and adds the total to the cell and its mirror.  Each cell belongs to
//     exactly one thread: no atomics touch global memory and the counts are
//     exact integers, so the output is deterministic.
#include "common.hpp"

namespace moe {

constexpr int kCsT = 16;                             // experts per tile side
constexpr int kCsThreads = 1024;
constexpr int kCsCells = kCsT * kCsT;                // 256
constexpr int kCsParts = kCsThreads / kCsCells;      // 4 partial sums per cell
constexpr int kCsWords = 64;                         // bitset words staged per round
constexpr int kCsWordsPerPart = kCsWords / kCsParts; // 16

__host__ __device__ inline int64_t cs_words(int64_t n) { return (n + kWave - 1) / kWave; }

template <int KMAX>
__global__ void __launch_bounds__(kWave)
coselect_bits_kernel(const int32_t* __restrict__ idx, int64_t n, int E, int k, uint32_t kmul,
                     uint64_t* __restrict__ S, int64_t nw) {
  extern __shared__ uint64_t s_word[];  // [E]
  const int lane = lane_id();
  const int64_t wd = blockIdx.x;
  const int64_t f0 = wd * kWave * k;
  const int64_t total = n * k;
  const int nf = int(total - f0 < int64_t(kWave) * k ? total - f0 : int64_t(kWave) * k);
  int raw[KMAX];
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
    const int64_t f = f0 + lane + kWave * r;
    raw[r] = idx[f < total ? f : total - 1];
  }
  for (int e = lane; e < E; e += kWave) s_word[e] = 0ull;
  wave_lds_sync();
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
    const int f = lane + kWave * r;
    if (f < nf) {
      const int t = k == 1 ? f : int(__umulhi(uint32_t(f), kmul));  // token inside the word
      atomicOr(reinterpret_cast<unsigned long long*>(&s_word[clampi(raw[r], 0, E - 1)]),
               1ull << t);
    }
  }
  wave_lds_sync();
  for (int e = lane; e < E; e += kWave) S[int64_t(e) * nw + wd] = s_word[e];
}

__global__ void __launch_bounds__(kCsThreads)
coselect_pairs_kernel(const uint64_t* __restrict__ S, int64_t nw, int E,
                      int32_t* __restrict__ W) {
  __shared__ u32x4 s_rows4[kCsT * kCsWords];  // [32 experts][64 words] as 16-byte pairs, 16 KiB
  __shared__ uint32_t s_red[kCsParts][kCsCells];
  const uint64_t* s_rows = reinterpret_cast<const uint64_t*>(s_rows4);
  const int nt = (E + kCsT - 1) / kCsT;
  int p = blockIdx.x, ta = 0;
  while (p >= nt - ta) {
    p -= nt - ta;
    ++ta;
  }
  const int tb = ta + p;
  const bool diag = ta == tb;
  const int a0 = ta * kCsT, b0 = tb * kCsT;
  const int tid = threadIdx.x;
  const int cell = tid % kCsCells, part = tid / kCsCells;
  const int i = cell / kCsT, j = cell % kCsT;
  // staging: thread tid moves words 2 spair, 2 spair + 1 of staged row srow
  const int srow = tid / (kCsWords / 2), spair = tid % (kCsWords / 2);
  const int sexp = srow < kCsT ? a0 + srow : b0 + (srow - kCsT);
  const bool svalid = sexp < E;
  const int64_t row = int64_t(svalid ? sexp : 0) * nw;
  const uint64_t* ra = s_rows + i * kCsWords;
  const uint64_t* rb = s_rows + (diag ? j : kCsT + j) * kCsWords;
  uint32_t acc = 0;
  for (int64_t w0 = 0; w0 < nw; w0 += kCsWords) {
    const int64_t wa = w0 + 2 * spair;  // words past the end or of experts >= E count as 0
    const uint64_t x0 = S[row + (wa < nw ? wa : nw - 1)];
    const uint64_t x1 = S[row + (wa + 1 < nw ? wa + 1 : nw - 1)];
    u32x4 v;
    v[0] = uint32_t(x0);
    v[1] = uint32_t(x0 >> 32);
    v[2] = uint32_t(x1);
    v[3] = uint32_t(x1 >> 32);
    if (!svalid || wa >= nw) v[0] = v[1] = 0u;
    if (!svalid || wa + 1 >= nw) v[2] = v[3] = 0u;
    __syncthreads();  // the previous round's popcounts are done
    s_rows4[tid] = v;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kCsWordsPerPart; ++q) {
      const int wq = part * kCsWordsPerPart + q;
      acc += __popcll(ra[wq] & rb[wq]);
    }
  }
  s_red[part][cell] = acc;
  __syncthreads();
  if (tid < kCsCells) {
    const int a = a0 + i, b = b0 + j;
    if (a < E && b < E) {
      uint32_t tot = 0;
#pragma unroll
      for (int q = 0; q < kCsParts; ++q) tot += s_red[q][cell];
      W[int64_t(a) * E + b] += int32_t(tot);
      if (!diag) W[int64_t(b) * E + a] += int32_t(tot);
    }
  }
}

size_t coselect_workspace(int64_t n, int E) {
  return align256(size_t(E) * size_t(cs_words(n)) * sizeof(uint64_t));
}

template <int KMAX>
static hipError_t launch_coselect_k(const int32_t* idx, int64_t n, int E, int k, int32_t* W,
                                    void* workspace, hipStream_t stream) {
  const int64_t nw = cs_words(n);
  const uint32_t kmul = k <= 1 ? 0u : uint32_t(((1ull << 32) + uint64_t(k) - 1) / uint64_t(k));
  uint64_t* S = static_cast<uint64_t*>(workspace);
  hipLaunchKernelGGL((coselect_bits_kernel<KMAX>), dim3(unsigned(nw)), dim3(kWave),
                     size_t(E) * sizeof(uint64_t), stream, idx, n, E, k, kmul, S, nw);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int nt = (E + kCsT - 1) / kCsT;
  hipLaunchKernelGGL(coselect_pairs_kernel, dim3(nt * (nt + 1) / 2), dim3(kCsThreads), 0, stream,
                     S, nw, E, W);
  return hipGetLastError();
}

hipError_t launch_coselect(const int32_t* idx, int64_t n, int E, int k, int32_t* W,
                           void* workspace, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  if (k <= 2) return launch_coselect_k<2>(idx, n, E, k, W, workspace, stream);
  if (k <= 4) return launch_coselect_k<4>(idx, n, E, k, W, workspace, stream);
  if (k <= 8) return launch_coselect_k<8>(idx, n, E, k, W, workspace, stream);
  return launch_coselect_k<16>(idx, n, E, k, W, workspace, stream);
}

}  // namespace moe
