// Bucket relayout by destination rank (the reduce-scatter alternative of the
// DeepSpeed issue "[REQUEST] DeepCompile ZeRO-1: reduce-to-owner instead of
// AllReduce", "Describe alternatives": a reduce-scatter over the bucket needs
// the payload contiguous by destination rank, so the bucket is first
// relaid).  A plan of column pieces (src, dst, len), sorted by dst, moves
// every data-parallel element of a bucket to its segment; these kernels apply
// it to all W rows, either searching the pieces per tile or from a tile plan
// that gives each destination tile inside one piece its source.  Pure data
// movement: HBM bound, W*n*b read + W*n*b written.
#include "device_common.h"
#include "internal.h"

namespace dc {
namespace {

#ifndef DC_RL_TPB
#define DC_RL_TPB 64            // one wave per workgroup (5% faster than 256)
#endif
constexpr int kRT = DC_RL_TPB;          // threads per workgroup
constexpr int kPieceStage = kRT;        // pieces staged per pass (one per thread)
#ifndef DC_RL_U
#define DC_RL_U 1
#endif
constexpr int kRelayoutU = DC_RL_U;
// Stores of whole vectors: through buffer resources with these cache-policy
// bits (gfx950: bit 0 sc0, bit 1 nt, bit 4 sc1), or nontemporal global
// stores when negative; and at most DC_RL_CAP (searched) or DC_RL_PLAN_CAP
// (planned) workgroups per compute unit (0: no cap).  Interleaved sweeps on
// the 402.8M-element W = 8 bucket relayouts: the searched kernel ran at
// 6.00 TB/s with one vector per thread at 10-12 per CU, against 5.80 with
// two vectors at 8 and 5.89 at 14; the planned one at 6.44 at 6 per CU,
// against 6.42 at 4-5, 6.37 at 7, 6.25 at 8, 6.06 uncapped and 5.77 at 16.
// sc0 sc1 nt, nt sc1 and plain nontemporal stores ran within 0.4% of each
// other.
#ifndef DC_RL_SP
#define DC_RL_SP 19
#endif
#ifndef DC_RL_CAP
#define DC_RL_CAP 12
#endif
#ifndef DC_RL_PLAN_CAP
#define DC_RL_PLAN_CAP 6
#endif
static_assert(DC_RL_TPB == kRelayoutTile, "a planned tile is one vector per thread of a wave");

struct RelayoutParams {
  const void* in;
  void* out;
  int64_t ld_in;
  int64_t ld_out;
  int64_t bucket_col;
  int64_t out_numel;
  const dc_piece* pieces;
  int32_t npieces;
  int32_t W;
  int64_t bucket_numel;
  const int64_t* tiles;  // planned launch: one record per tile
};

// Stores of one vector of each row of a tile's run [t0, t1) of destination
// vectors, the run's vector v of every row.
template <int EB, int WT>
__device__ __forceinline__ void store_rows(const RelayoutParams& p, int64_t t0, int64_t t1, int64_t v,
                                           const u32x4* x) {
  constexpr int E = 16 / EB;
  if constexpr (DC_RL_SP >= 0) {
    u32x4* tile = reinterpret_cast<u32x4*>(p.out) + t0;
    const int32_t bytes = (int32_t)(t1 - t0) * 16, off = (int32_t)(v - t0) * 16;
#pragma unroll
    for (int r = 0; r < WT; ++r)
      store_buf<(DC_RL_SP >= 0 ? DC_RL_SP : 0)>(tile + r * (p.ld_out / E), bytes, off, x[r]);
  } else {
    u32x4* dst = reinterpret_cast<u32x4*>(p.out) + v;
#pragma unroll
    for (int r = 0; r < WT; ++r) store16<true>(dst + r * (p.ld_out / E), x[r]);
  }
}

// Destination vectors [t0, t1) by search: the workgroup finds the pieces
// overlapping its run with a k-ary search of the piece table and stages
// them in LDS.  A vector inside one piece whose source is vector aligned
// moves as W 16-byte loads and stores; any other vector moves element by
// element.  Source columns are checked against the bucket, so a bad plan
// never reads or writes outside the bucket of the input or [0, out_numel)
// of the output.  Every thread of the workgroup must call it.
template <int EB, int WT>
__device__ __forceinline__ void relayout_run(const RelayoutParams& p, int64_t t0, int64_t t1) {
  constexpr int E = 16 / EB;
  __shared__ int64_t s_dst[kPieceStage];
  __shared__ int64_t s_src[kPieceStage];
  __shared__ int64_t s_end[kPieceStage];
  const int W = WT > 0 ? WT : p.W;
  const int64_t lo = t0 * E, hi = min(t1 * E, p.out_numel);
  int32_t first, last;
  kary_bounds<kRT>(p.npieces, [&](int32_t i) { return p.pieces[i].dst; }, lo, hi, first, last);
  first = max(first - 1, 0);
  last = last - 1;
  const char* in = reinterpret_cast<const char*>(p.in);
  char* out = reinterpret_cast<char*>(p.out);
  for (int32_t base = first; base <= last; base += kPieceStage) {
    const int32_t cnt = min(kPieceStage, last - base + 1);
    __syncthreads();
    if ((int32_t)threadIdx.x < cnt) {
      const dc_piece pc = p.pieces[base + threadIdx.x];
      const int64_t len = pc.len > 0 ? pc.len : 0;
      s_dst[threadIdx.x] = pc.dst;
      s_src[threadIdx.x] = pc.src;
      s_end[threadIdx.x] = pc.dst + len;
    }
    __syncthreads();
#pragma unroll 1
    for (int64_t v = t0 + threadIdx.x; v < t1; v += kRT) {
      const int64_t d0 = v * E;
      const int64_t d1 = min(d0 + E, p.out_numel);
      const int32_t k = last_le(s_dst, cnt, d0);
      const int64_t src0 = s_src[k] + (d0 - s_dst[k]);
      const bool whole = d1 == d0 + E && s_dst[k] <= d0 && s_end[k] >= d1 &&
                         (p.bucket_col + src0) % E == 0 && src0 >= 0 && src0 + E <= p.bucket_numel;
      if (whole) {
        const u32x4* src = reinterpret_cast<const u32x4*>(in) + (p.bucket_col + src0) / E;
        if constexpr (WT > 0) {
          u32x4 x[WT];
#pragma unroll
          for (int r = 0; r < WT; ++r) x[r] = load16<true>(src + r * (p.ld_in / E));
          store_rows<EB, WT>(p, t0, t1, v, x);
        } else {
          u32x4* dst = reinterpret_cast<u32x4*>(out) + v;
          for (int r = 0; r < W; ++r)
            store16<true>(dst + r * (p.ld_out / E), load16<true>(src + r * (p.ld_in / E)));
        }
      } else {
        for (int64_t d = d0; d < d1; ++d) {
          const int32_t kk = last_le(s_dst, cnt, d);
          if (!(s_dst[kk] <= d && d < s_end[kk])) continue;
          const int64_t sc = s_src[kk] + (d - s_dst[kk]);
          if (sc < 0 || sc >= p.bucket_numel) continue;
          for (int r = 0; r < W; ++r) {
            const int64_t si = (r * p.ld_in + p.bucket_col + sc) * EB;
            const int64_t di = (r * p.ld_out + d) * EB;
            if constexpr (EB == 2)
              *reinterpret_cast<uint16_t*>(out + di) = *reinterpret_cast<const uint16_t*>(in + si);
            else
              *reinterpret_cast<uint32_t*>(out + di) = *reinterpret_cast<const uint32_t*>(in + si);
          }
        }
      }
    }
  }
}

// Searched relayout: one workgroup per run of kRT*U destination vectors
// (16 bytes of every row each).
template <int EB, int WT>
__global__ __launch_bounds__(kRT) void k_relayout(RelayoutParams p) {
  constexpr int E = 16 / EB;
  const int64_t nvec = (p.out_numel + E - 1) / E;
  const int64_t t0 = (int64_t)blockIdx.x * (kRT * kRelayoutU);
  relayout_run<EB, WT>(p, t0, min(t0 + (int64_t)(kRT * kRelayoutU), nvec));
}

// Planned relayout: workgroup b takes tile b, kRelayoutTile destination
// vectors (thread i: vector i).  A tile whose record gives its source run
// copies it straight away, one load and one store per row and thread, with
// no search and no staging; the record is checked against the bucket, so a
// stale plan can misplace data inside the bucket but never reach outside it.
// Any other tile takes the searched path over its run.
template <int EB, int WT>
__global__ __launch_bounds__(kRT) void k_relayout_planned(RelayoutParams p) {
  constexpr int E = 16 / EB;
  const int64_t nvec = (p.out_numel + E - 1) / E;
  const int64_t t0 = (int64_t)blockIdx.x * kRelayoutTile;
  const int64_t t1 = min(t0 + kRelayoutTile, nvec);
  if constexpr (WT > 0) {
    // the record's source run must lie in the bucket: vectors
    // [ceil(bucket_col / E), floor(bucket end / E) - kRelayoutTile], checked
    // without multiplying the record (any int64 is safe)
    const int64_t rec = p.tiles[tile_slot((int64_t)blockIdx.x, (int64_t)gridDim.x)];
    const int64_t rec_lo = (p.bucket_col + E - 1) / E;
    const int64_t rec_hi = (p.bucket_col + p.bucket_numel) / E - kRelayoutTile;
    if (rec >= rec_lo && rec <= rec_hi && t1 * E <= p.out_numel && t1 - t0 == kRelayoutTile) {
      const u32x4* src = reinterpret_cast<const u32x4*>(p.in) + rec + threadIdx.x;
      u32x4 x[WT];
#pragma unroll
      for (int r = 0; r < WT; ++r) x[r] = load16<true>(src + r * (p.ld_in / E));
      store_rows<EB, WT>(p, t0, t1, t0 + threadIdx.x, x);
      return;
    }
  }
  relayout_run<EB, WT>(p, t0, t1);
}

template <int EB>
hipError_t launch_eb(const RelayoutParams& p, hipStream_t stream) {
  constexpr int E = 16 / EB;
  const int64_t nvec = (p.out_numel + E - 1) / E;
  const bool planned = p.tiles != nullptr;
  const dim3 grid((unsigned)(planned ? (nvec + kRelayoutTile - 1) / kRelayoutTile
                                     : (nvec + kRT * kRelayoutU - 1) / (kRT * kRelayoutU)));
#define DC_RL_LAUNCH(kern, cap)                                                                   \
  hipLaunchKernelGGL(kern, grid, dim3(kRT), occupancy_pad(reinterpret_cast<const void*>(kern), cap), \
                     stream, p)
  switch (p.W) {
#define DC_RL_W(w)                                                   \
  case w:                                                            \
    if (planned) DC_RL_LAUNCH((k_relayout_planned<EB, w>), DC_RL_PLAN_CAP); \
    else DC_RL_LAUNCH((k_relayout<EB, w>), DC_RL_CAP);               \
    break;
    DC_RL_W(4)
    DC_RL_W(8)
    DC_RL_W(16)
#undef DC_RL_W
    default:
      if (planned) hipLaunchKernelGGL((k_relayout_planned<EB, 0>), grid, dim3(kRT), 0, stream, p);
      else hipLaunchKernelGGL((k_relayout<EB, 0>), grid, dim3(kRT), 0, stream, p);
  }
#undef DC_RL_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_relayout(int32_t W, int32_t dtype, const void* in, int64_t ld_in, void* out,
                           int64_t ld_out, int64_t bucket_col, int64_t bucket_numel,
                           const dc_piece* pieces, int32_t npieces, int64_t out_numel,
                           const int64_t* tiles, hipStream_t stream) {
  if (out_numel == 0 || npieces == 0) return hipSuccess;
  RelayoutParams p{in, out, ld_in, ld_out, bucket_col, out_numel, pieces, npieces, W, bucket_numel,
                   tiles};
  return dtype == DC_BF16 ? launch_eb<2>(p, stream) : launch_eb<4>(p, stream);
}

}  // namespace dc
