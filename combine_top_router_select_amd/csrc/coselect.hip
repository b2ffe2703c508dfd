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
// One kernel.  A workgroup of 1024 threads takes one 16 x 16 tile of W in the
// upper triangle and one slice of the tokens, in rounds of 1024 tokens:
//  1. the round's top-k ids are loaded coalesced (all loads issued before any
//     use) and turned into row codes of the tile's (up to) 32 experts, staged
//     in LDS as bytes;
//  2. one wave per 64-token word, one lane per token: the lane ORs its slots'
//     row bits into a 32-bit mask, and a 5-stage bit-matrix transpose across
//     lanes (ds_swizzle exchanges) turns the 64 masks into the 32 experts'
//     64-bit token bitsets.  No LDS atomics (measured: ds_or_b64 with many
//     lanes is several times slower than this);
//  3. popcount(S_a & S_b) over the round's 16 words for each cell, four
//     threads per cell.
// The cell's owner adds the slice's count to the cell and its mirror with an
// integer atomic add: integer sums are exact in any order, so the result is
// deterministic.  Slicing the tokens puts several workgroups on each tile (the
// E = 64 case has only 10 tiles); there is no intermediate buffer in global
// memory.
#include "common.hpp"
#include "coselect_bm.hpp"

namespace moe {

constexpr int kCsT = 16;                             // experts per tile side
constexpr int kCsThreads = 1024;
constexpr int kCsCells = kCsT * kCsT;                // 256
constexpr int kCsParts = kCsThreads / kCsCells;      // 4 partial sums per cell
constexpr int kCsWords = kCsThreads / kWave;         // 16 words of 64 tokens per round
constexpr int kCsRound = kCsWords * 64;              // 1024 tokens per round
constexpr int kCsStride = kCsWords + 1;              // padded LDS row: rows start in different banks
constexpr int kCsWordsPerPart = kCsWords / kCsParts; // 4
constexpr int kCsTargetBlocks = 256;
constexpr uint8_t kCsNoRow = 0xFF;

// One stage of the lane transpose of a 32 x 32 bit matrix (lane l holds row
// l; afterwards lane c holds column c): lanes l and l ^ J swap the
// off-diagonal J x J blocks of their 2J x 2J block.  ds_swizzle in bit-mask
// mode reads lane l ^ J inside each 32-lane half.
template <int J, uint32_t MASK>
__device__ __forceinline__ uint32_t transpose_stage(uint32_t x, int lane) {
  const uint32_t xp = uint32_t(__builtin_amdgcn_ds_swizzle(int(x), (J << 10) | 0x1F));
  const bool up = (lane & J) != 0;
  const uint32_t t = ((up ? xp : x) ^ ((up ? x : xp) << J)) & MASK;
  return x ^ (up ? (t >> J) : t);
}

template <int KMAX>
__global__ void __launch_bounds__(kCsThreads)
coselect_kernel(const int32_t* __restrict__ idx, int64_t n, int E, int k, int n_slices,
                int64_t slice_tokens, int32_t* __restrict__ W) {
  __shared__ uint8_t s_rows[kCsRound * KMAX];  // row code per id of the round
  __shared__ uint64_t s_bits[2 * kCsT * kCsStride];    // [32 experts][17 words]
  __shared__ uint32_t s_red[kCsParts][kCsCells];
  const int nt = (E + kCsT - 1) / kCsT;
  const int slice = int(blockIdx.x % unsigned(n_slices));
  int p = int(blockIdx.x / unsigned(n_slices)), ta = 0;
  while (p >= nt - ta) {
    p -= nt - ta;
    ++ta;
  }
  const int tb = ta + p;
  const bool diag = ta == tb;
  const int a0 = ta * kCsT, b0 = tb * kCsT;
  const int tid = threadIdx.x;
  const int lane = lane_id(), wv = tid / kWave;
  const int cell = tid % kCsCells, part = tid / kCsCells;
  const int i = cell / kCsT, j = cell % kCsT;
  const int ca = a0 + i, cb = b0 + j;
  const uint64_t* ra = s_bits + i * kCsStride;
  const uint64_t* rb = s_bits + (diag ? j : kCsT + j) * kCsStride;
  const int64_t s0 = int64_t(slice) * slice_tokens;
  const int64_t s1 = s0 + slice_tokens < n ? s0 + slice_tokens : n;
  uint32_t acc = 0;
  for (int64_t t0 = s0; t0 < s1; t0 += kCsRound) {
    const int32_t* ids = idx + t0 * k;  // this round's ids, flat
    const int ntok = int(s1 - t0 < kCsRound ? s1 - t0 : kCsRound);
    const int nf = ntok * k;            // at most 1024 * k: at most KMAX ids per thread
    // 1. loads first (32-bit offsets clamped into the round, no branch)
    int raw[KMAX];
#pragma unroll
    for (int r = 0; r < KMAX; ++r) {
      uint32_t f = uint32_t(tid + kCsThreads * r);
      f = f < uint32_t(nf) ? f : uint32_t(nf - 1);
      raw[r] = ids[f];
    }
    __syncthreads();  // the previous round is done with s_rows and s_bits
#pragma unroll
    for (int r = 0; r < KMAX; ++r) {
      const int f = tid + kCsThreads * r;
      const int e = raw[r];
      uint8_t row = kCsNoRow;
      if (e >= a0 && e < a0 + kCsT) row = uint8_t(e - a0);
      else if (!diag && e >= b0 && e < b0 + kCsT) row = uint8_t(kCsT + (e - b0));
      if (f < nf) s_rows[f] = row;
    }
    __syncthreads();
    // 2. the token of this lane: its experts' row bits, then the transpose
    const int tok = wv * kWave + lane;
    uint32_t m = 0;
    if (tok < ntok) {
      for (int q = 0; q < k; ++q) {
        const uint32_t row = s_rows[tok * k + q];
        m |= row < 32u ? (1u << row) : 0u;
      }
    }
    m = transpose_stage<16, 0xFFFF0000u>(m, lane);
    m = transpose_stage<8, 0xFF00FF00u>(m, lane);
    m = transpose_stage<4, 0xF0F0F0F0u>(m, lane);
    m = transpose_stage<2, 0xCCCCCCCCu>(m, lane);
    m = transpose_stage<1, 0xAAAAAAAAu>(m, lane);
    // lane c < 32: tokens 0..31 of row c; lane 32 + c: tokens 32..63
    const uint32_t hi = uint32_t(__shfl_xor(int(m), 32));
    if (lane < 2 * kCsT) s_bits[lane * kCsStride + wv] = (uint64_t(hi) << 32) | m;
    __syncthreads();
    // 3. popcounts
#pragma unroll
    for (int q = 0; q < kCsWordsPerPart; ++q) {
      const int wq = part * kCsWordsPerPart + q;
      acc += __popcll(ra[wq] & rb[wq]);
    }
  }
  s_red[part][cell] = acc;
  __syncthreads();
  if (part == 0 && ca < E && cb < E) {
    uint32_t tot = 0;
#pragma unroll
    for (int q = 0; q < kCsParts; ++q) tot += s_red[q][cell];
    if (tot != 0) {
      atomicAdd(&W[int64_t(ca) * E + cb], int32_t(tot));
      if (!diag) atomicAdd(&W[int64_t(cb) * E + ca], int32_t(tot));
    }
  }
}

hipError_t launch_coselect(const int32_t* idx, int64_t n, int E, int k, int32_t* W,
                           hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int nt = (E + kCsT - 1) / kCsT;
  const int tiles = nt * (nt + 1) / 2;
  // slices of whole rounds, enough of them to put about kCsTargetBlocks
  // workgroups in flight
  const int64_t rounds = (n + kCsRound - 1) / kCsRound;
  int64_t ns = (kCsTargetBlocks + tiles - 1) / tiles;
  ns = ns < rounds ? ns : rounds;
  const int64_t per = (rounds + ns - 1) / ns;  // rounds per slice
  ns = (rounds + per - 1) / per;               // no empty slice
  const dim3 grid(unsigned(tiles * ns));
  if (k <= 2)
    hipLaunchKernelGGL((coselect_kernel<2>), grid, dim3(kCsThreads), 0, stream, idx, n, E, k,
                       int(ns), per * kCsRound, W);
  else if (k <= 4)
    hipLaunchKernelGGL((coselect_kernel<4>), grid, dim3(kCsThreads), 0, stream, idx, n, E, k,
                       int(ns), per * kCsRound, W);
  else if (k <= 8)
    hipLaunchKernelGGL((coselect_kernel<8>), grid, dim3(kCsThreads), 0, stream, idx, n, E, k,
                       int(ns), per * kCsRound, W);
  else
    hipLaunchKernelGGL((coselect_kernel<16>), grid, dim3(kCsThreads), 0, stream, idx, n, E, k,
                       int(ns), per * kCsRound, W);
  return hipGetLastError();
}

// Co-selection counts from the 64-token expert bitmaps of a plan (see
// coselect_bm.hpp): one workgroup per 16 x 16 block of W and chunk of blocks.
__global__ void __launch_bounds__(kBmThreads) coselect_bm_kernel(CoselectBm a) {
  __shared__ uint64_t s_lds[kBmLdsBytes / sizeof(uint64_t)];
  coselect_bm_block(a, blockIdx.x, s_lds);
}

hipError_t launch_coselect_bm(const uint64_t* bm, int64_t cs_tokens, int E, int32_t* W,
                              hipStream_t stream) {
  if (cs_tokens <= 0) return hipSuccess;
  const CoselectBm a = coselect_bm_args(bm, cs_tokens, E, W);
  hipLaunchKernelGGL(coselect_bm_kernel, dim3(unsigned(a.blocks())), dim3(kBmThreads), 0, stream,
                     a);
  return hipGetLastError();
}

}  // namespace moe
