// Co-selection counts from the plan's 64-token expert bitmaps, as a workgroup
// routine shared by the stand-alone kernel (coselect.hip) and the dispatch
// kernels, which run it in extra workgroups next to the row copies.
//
// W[a][b] += sum over the first `ntiles` 64-token blocks of
// popcount(bm[t][a] & bm[t][b]), the last block masked to the tokens below
// cs_tokens.  A bit-matrix product with a short inner dimension: one
// workgroup per 16 x 16 block of W and chunk of kBmChunk blocks stages the W
// block's 16 + 16 bitmap columns of the chunk in LDS (each bitmap is read by
// E / 16 workgroups instead of E), then thread (a, b) of the W block sums its
// popcounts.  With one chunk (up to 4096 tokens) every W entry has one owner
// and is added with a plain read-modify-write; with several, with an integer
// atomic (exact in any order).
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kBmBlk = 16;    // W block edge
constexpr int kBmChunk = 64;  // 64-token blocks per workgroup
constexpr int kBmThreads = kBmBlk * kBmBlk;
constexpr size_t kBmLdsBytes = size_t(2) * kBmChunk * kBmBlk * sizeof(uint64_t);

struct CoselectBm {
  const uint64_t* bm;   // [ntiles][E] bitmaps
  int64_t ntiles;       // 64-token blocks holding the first cs_tokens tokens
  uint64_t last_mask;   // tokens of the last block that count
  int E;
  int nblk;             // W blocks per side
  int chunks;           // workgroups per W block
  int32_t* W;           // [E][E], accumulated
  __host__ __device__ int64_t blocks() const { return int64_t(nblk) * nblk * chunks; }
};

// The arguments for the first cs_tokens tokens (cs_tokens > 0).
__host__ inline CoselectBm coselect_bm_args(const uint64_t* bm, int64_t cs_tokens, int E,
                                           int32_t* W) {
  CoselectBm a;
  a.bm = bm;
  a.ntiles = (cs_tokens + kWaveTile - 1) / kWaveTile;
  const int rem = int(cs_tokens - (a.ntiles - 1) * kWaveTile);  // tokens of the last block, 1..64
  a.last_mask = rem >= kWaveTile ? ~0ull : ((1ull << rem) - 1ull);
  a.E = E;
  a.nblk = (E + kBmBlk - 1) / kBmBlk;
  int64_t chunks = (a.ntiles + kBmChunk - 1) / kBmChunk;
  a.chunks = int(chunks < 65535 ? chunks : 65535);
  a.W = W;
  return a;
}

// Workgroup q (0 <= q < a.blocks()) of the co-selection counts; every thread
// of a kBmThreads-thread workgroup calls it.  lds: kBmLdsBytes of LDS.
__device__ __forceinline__ void coselect_bm_block(const CoselectBm& a, int64_t q, uint64_t* lds) {
  uint64_t(*s_a)[kBmBlk] = reinterpret_cast<uint64_t(*)[kBmBlk]>(lds);
  uint64_t(*s_b)[kBmBlk] = reinterpret_cast<uint64_t(*)[kBmBlk]>(lds + kBmChunk * kBmBlk);
  const int nb2 = a.nblk * a.nblk;
  const int wb = int(q % nb2);
  const int chunk = int(q / nb2);
  const int tid = threadIdx.x;
  const int E = a.E;
  const int a0 = (wb / a.nblk) * kBmBlk;
  const int b0 = (wb % a.nblk) * kBmBlk;
  const int ai = tid / kBmBlk, bi = tid % kBmBlk;
  const int64_t ntiles = a.ntiles;
  uint32_t acc = 0;
  for (int64_t t0 = int64_t(chunk) * kBmChunk; t0 < ntiles;
       t0 += int64_t(a.chunks) * kBmChunk) {
    // stage: 64 blocks x 16 columns of each side, four 8-byte loads per thread
    // per side (16 consecutive columns of one block are 128 contiguous bytes)
    uint64_t va[kBmChunk * kBmBlk / kBmThreads], vb[kBmChunk * kBmBlk / kBmThreads];
#pragma unroll
    for (int i = 0; i < kBmChunk * kBmBlk / kBmThreads; ++i) {
      const int qq = tid + kBmThreads * i;
      int64_t t = t0 + qq / kBmBlk;
      t = t < ntiles ? t : ntiles - 1;
      const int ca = a0 + qq % kBmBlk, cb = b0 + qq % kBmBlk;
      va[i] = a.bm[t * E + (ca < E ? ca : E - 1)];
      vb[i] = a.bm[t * E + (cb < E ? cb : E - 1)];
    }
    __syncthreads();  // the previous chunk's reads of s_a / s_b are done
#pragma unroll
    for (int i = 0; i < kBmChunk * kBmBlk / kBmThreads; ++i) {
      const int qq = tid + kBmThreads * i;
      const int64_t t = t0 + qq / kBmBlk;
      const uint64_t m = t < ntiles - 1 ? ~0ull : (t == ntiles - 1 ? a.last_mask : 0ull);
      s_a[qq / kBmBlk][qq % kBmBlk] = va[i] & m;
      s_b[qq / kBmBlk][qq % kBmBlk] = vb[i];
    }
    __syncthreads();
    // a short unroll: the dispatch kernels that run this routine must keep
    // their register count (and occupancy) of the copies alone
#pragma unroll 2
    for (int t = 0; t < kBmChunk; ++t) acc += uint32_t(__popcll(s_a[t][ai] & s_b[t][bi]));
  }
  const int ra = a0 + ai, rb = b0 + bi;
  if (ra < E && rb < E && acc != 0) {
    int32_t* w = &a.W[int64_t(ra) * E + rb];
    if (a.chunks == 1) *w += int32_t(acc);  // the only owner of this entry
    else atomicAdd(w, int32_t(acc));
  }
}

}  // namespace moe
