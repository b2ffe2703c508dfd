// A5 + A1/A2 - the combine of one batch and the routing of the next in one
// launch, for a loop over independent batches (microbatches of one layer).
//
// Sources: as combine.hip (the combine) and route_topk.hip (routing and the
// plan's tile counts).  The pages time the dispatch and the combine; the
// routing in front of them is a short, latency-bound step.
//
// Design: the first workgroups of the launch route the next batch, one 32-token
// plan tile each (route_tile_block: ids, gates, tile counts, slot codes and
// expert bitmaps, the plan without its scan), while the rest combine this
// batch (combine_unit, one wave per token and row chunk).  The routing's
// dependent chain of selection rounds then runs beside the combine's row
// reads, which keep HBM busy, instead of as a launch of its own in front of
// the next dispatch, whose workgroups scan the plan themselves
// (moe_dispatch_routed).  Workgroups are 512 threads, the routing tile's
// 32 tokens x 16 lanes; one routing variant (16 logits per lane, scalar
// loads) serves every expert count up to 256, with the gating and the dispatch
// mode as runtime flags, so that the launch has one kernel per combine
// variant.  Larger shapes route in launches of their own (same results).
#include "combine_rows.hpp"
#include "route_tile.hpp"

namespace moe {

constexpr int kCrLanes = 16;                   // lanes per routed token
constexpr int kCrLogits = 16;                  // logits per lane: 256 experts
constexpr int kCrThreads = kTile * kCrLanes;   // one routing tile per workgroup
constexpr int kCrMaxExperts = kCrLanes * kCrLogits;

// This batch's combine.
struct CombineArgs {
  const uint8_t* rows;
  const float* w;
  const int32_t* slot_row;
  int64_t T;
  int row_bytes;
  int k;
  int cpr;
  uint8_t* out;
};

// The next batch's routing (blocks = its plan tiles, 0 for none).
struct RouteArgs {
  const float* logits;
  int64_t T;
  int E, k, R, m;
  const int32_t* place;
  int64_t Bp;
  int32_t* idx;
  float* gate;
  uint8_t* tcnt;
  uint32_t* lslot;
  TilePiece* bm;
  int full, dedup;
  int64_t blocks;
};

// The top-6 combine of bf16 rows in 4-vector chunks takes 126 registers here
// (4 waves per SIMD), as in the combine kernel (125); capping it at 5 waves
// spills, and routing a tile in two passes of 256 threads took as many
// registers (launch_cr_k).
template <int NV, int KMAX, bool IN8>
__global__ void __launch_bounds__(kCrThreads)
combine_route_kernel(CombineArgs c, RouteArgs r) {
  if (int64_t(blockIdx.x) < r.blocks) {
    extern __shared__ TileMask s_cr[];
    route_tile_block<kCrLanes, kCrLogits, 1, false, false>(
        r.logits, r.T, r.E, r.k, r.R, r.place, r.m, r.Bp, r.idx, r.gate, r.tcnt, r.lslot, r.bm,
        blockIdx.x, s_cr, r.full != 0, r.dedup != 0);
    return;
  }
  const int64_t wid = ((int64_t(blockIdx.x) - r.blocks) * blockDim.x + threadIdx.x) / kWave;
  combine_unit<NV, KMAX, IN8, true>(c.rows, c.w, c.slot_row, c.T, c.row_bytes, c.k, c.cpr,
                                    nullptr, c.out, wid);
}

template <int NV, int KMAX, bool IN8>
static hipError_t launch_cr_t(CombineArgs c, const RouteArgs& r, size_t lds,
                              hipStream_t stream) {
  const int chunk = NV * kWave * InVec<IN8>::kBytes;
  c.cpr = (c.row_bytes + chunk - 1) / chunk;
  const int64_t waves = c.T * c.cpr;
  const int64_t cblocks = (waves + kCrThreads / kWave - 1) / (kCrThreads / kWave);
  hipLaunchKernelGGL((combine_route_kernel<NV, KMAX, IN8>), dim3(unsigned(r.blocks + cblocks)),
                     dim3(kCrThreads), lds, stream, c, r);
  return hipGetLastError();
}

// The combine kernel's chunk rule, except that 6 or more rows per token over
// rows longer than one 4-vector chunk take 2-vector chunks: the 4-vector
// variant takes 126 registers (4 waves per SIMD) against 74 (6 waves), and in
// this launch the 2-vector one is faster there (a 16384-token top-6 dedup step
// of 8 KiB rows 308.2-309.1 -> 305.4-305.5 us, top-6 hidden 2688 dedup
// 46.7-47.4 -> 45.4-45.6 us on two streams), while single-chunk rows gain
// from the larger chunk (the 4096-token top-6 step of 4 KiB rows 37.0-37.1
// against 37.4-38.0 us).  The combine kernel alone keeps 4-vector chunks: the
// same rule there slowed the 16384-token top-6 combine (143.5 -> 145.0 us) and
// the reduction (248.8 -> 254.3 us).
template <int KMAX, bool IN8>
static hipError_t launch_cr_k(const CombineArgs& c, const RouteArgs& r, size_t lds,
                              hipStream_t stream) {
  constexpr int NVMAX = combine_nv_max<KMAX>();
  int nv = combine_nv<KMAX, IN8>(c.row_bytes);
  if (nv == 4 && KMAX >= 6 && c.row_bytes > 4 * kWave * InVec<IN8>::kBytes) nv = 2;
  switch (nv) {
    case 4: return launch_cr_t<(NVMAX >= 4 ? 4 : 1), KMAX, IN8>(c, r, lds, stream);
    case 2: return launch_cr_t<(NVMAX >= 2 ? 2 : 1), KMAX, IN8>(c, r, lds, stream);
    default: return launch_cr_t<1, KMAX, IN8>(c, r, lds, stream);
  }
}

template <bool IN8>
static hipError_t launch_cr_f(const CombineArgs& c, const RouteArgs& r, size_t lds,
                              hipStream_t stream) {
  if (c.k <= 1) return launch_cr_k<1, IN8>(c, r, lds, stream);
  if (c.k <= 2) return launch_cr_k<2, IN8>(c, r, lds, stream);
  if (c.k <= 4) return launch_cr_k<4, IN8>(c, r, lds, stream);
  if (c.k <= 6) return launch_cr_k<6, IN8>(c, r, lds, stream);
  if (c.k <= 8) return launch_cr_k<8, IN8>(c, r, lds, stream);
  return launch_cr_k<16, IN8>(c, r, lds, stream);
}

hipError_t launch_combine(const void* rows, const float* w, const int32_t* slot_row, int64_t T,
                          int row_bytes, int k, int in_fp8, const int32_t* n_valid, void* out,
                          hipStream_t stream);
hipError_t launch_route_topk(const float* logits, int64_t tokens, int E, int k, int full_softmax,
                             int32_t* idx, float* gate, hipStream_t stream);
hipError_t launch_tile_counts(const int32_t* idx, int64_t T, int E, int k, int R,
                              const int32_t* place, int dedup, void* workspace,
                              hipStream_t stream);
bool route_tiles_fit(int64_t T, int E);
hipError_t launch_route_tiles(const float* logits, int64_t T, int E, int k, int full_softmax,
                              int R, const int32_t* place, int dedup, int32_t* idx, float* gate,
                              void* workspace, hipStream_t stream);

// The combine of T tokens (as launch_combine, no n_valid) and the routing of
// the next batch of Tn tokens into its plan without the scan (ids, gates,
// tile counts, slot codes, expert bitmaps in `workspace`): one launch, or for
// more than 256 experts (or tokens past the fused routing's limit) the combine,
// the routing kernel and the counting kernel.  With no combine (T = 0) the
// routing takes the fused routing kernel of its own.
hipError_t launch_combine_route(const void* rows, const float* w, const int32_t* slot_row,
                                int64_t T, int row_bytes, int k, int in_fp8, void* out,
                                const float* logits, int64_t Tn, int E, int kn, int full,
                                int R, const int32_t* place, int dedup, int32_t* idx,
                                float* gate, void* workspace, hipStream_t stream) {
  if (Tn > 0 && !(E <= kCrMaxExperts && route_tiles_fit(Tn, E))) {
    hipError_t err = launch_combine(rows, w, slot_row, T, row_bytes, k, in_fp8, nullptr, out,
                                    stream);
    if (err != hipSuccess) return err;
    err = launch_route_topk(logits, Tn, E, kn, full, idx, gate, stream);
    if (err != hipSuccess) return err;
    return launch_tile_counts(idx, Tn, E, kn, R, place, dedup, workspace, stream);
  }
  if (T == 0)
    return Tn == 0 ? hipSuccess
                   : launch_route_tiles(logits, Tn, E, kn, full, R, place, dedup, idx, gate,
                                        workspace, stream);
  CombineArgs c{static_cast<const uint8_t*>(rows), w, slot_row, T, row_bytes, k, 1,
                static_cast<uint8_t*>(out)};
  RouteArgs r{};
  size_t lds = 0;
  if (Tn > 0) {
    const PlanLayout pl = plan_layout(Tn, E, kn, R, dedup);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    r.logits = logits;
    r.T = Tn;
    r.E = E;
    r.k = kn;
    r.R = R;
    r.m = E / R;
    r.place = place;
    r.Bp = pl.tiles_pad;
    r.idx = idx;
    r.gate = gate;
    r.tcnt = ws + pl.tcnt_off;
    r.lslot = reinterpret_cast<uint32_t*>(ws + pl.lslot_off);
    r.bm = reinterpret_cast<TilePiece*>(ws + pl.bm_off);
    r.full = full;
    r.dedup = dedup;
    r.blocks = pl.tiles;
    lds = route_tile_lds(pl.cols, E);
  }
  return in_fp8 ? launch_cr_f<true>(c, r, lds, stream) : launch_cr_f<false>(c, r, lds, stream);
}

}  // namespace moe
