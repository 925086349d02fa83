// Bucket relayout by destination rank (the reduce-scatter alternative of the
// DeepSpeed issue "[REQUEST] DeepCompile ZeRO-1: reduce-to-owner instead of
// AllReduce", "Describe alternatives": a reduce-scatter over the bucket needs
// the payload contiguous by destination rank, so the bucket is first
// relaid).  A plan of column pieces (src, dst, len), sorted by dst, moves
// every data-parallel element of a bucket to its segment; this kernel applies
// it to all W rows.  Pure data movement: HBM bound, W*n*b read + W*n*b written.
#include "device_common.h"
#include "internal.h"

namespace dc {
namespace {

#ifndef DC_RL_TPB
#define DC_RL_TPB 64            // one wave per workgroup (5% faster than 256)
#endif
constexpr int kRT = DC_RL_TPB;          // threads per workgroup
constexpr int kPieceStage = kRT;        // pieces staged per pass (one per thread)
constexpr int kRelayoutU = 2;
// Stores of whole vectors: through buffer resources with these cache-policy
// bits (gfx950: bit 0 sc0, bit 1 nt, bit 4 sc1), or nontemporal global
// stores when negative; and at most DC_RL_CAP workgroups per compute unit
// (0: no cap).  On the 402.8M-element W = 8 bucket relayouts a cap of 8 ran
// 2.6% faster than full occupancy (12: 1.3%); sc0 sc1 nt, nt sc1 and plain
// nontemporal stores ran within 0.2% of each other.
#ifndef DC_RL_SP
#define DC_RL_SP 19
#endif
#ifndef DC_RL_CAP
#define DC_RL_CAP 8
#endif

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
};

// One workgroup per tile of kRT*U destination vectors (16 bytes of every
// row).  A vector inside one piece whose source is vector aligned moves as W
// 16-byte loads and stores; any other vector moves element by element.
// Source columns are checked against the bucket, so a bad plan never reads
// or writes outside the bucket of the input or [0, out_numel) of the output.
template <int EB, int WT>
__global__ __launch_bounds__(kRT) void k_relayout(RelayoutParams p) {
  constexpr int E = 16 / EB;
  __shared__ int64_t s_dst[kPieceStage];
  __shared__ int64_t s_src[kPieceStage];
  __shared__ int64_t s_end[kPieceStage];
  const int W = WT > 0 ? WT : p.W;
  const int64_t nvec = (p.out_numel + E - 1) / E;
  const int64_t t0 = (int64_t)blockIdx.x * (kRT * kRelayoutU);
  const int64_t t1 = min(t0 + (int64_t)(kRT * kRelayoutU), nvec);
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
    for (int u = 0; u < kRelayoutU; ++u) {
      const int64_t v = t0 + threadIdx.x + (int64_t)u * kRT;
      if (v >= t1) break;
      const int64_t d0 = v * E;
      const int64_t d1 = min(d0 + E, p.out_numel);
      const int32_t k = last_le(s_dst, cnt, d0);
      const int64_t src0 = s_src[k] + (d0 - s_dst[k]);
      const bool whole = d1 == d0 + E && s_dst[k] <= d0 && s_end[k] >= d1 &&
                         (p.bucket_col + src0) % E == 0 && src0 >= 0 && src0 + E <= p.bucket_numel;
      if (whole) {
        const u32x4* src = reinterpret_cast<const u32x4*>(in) + (p.bucket_col + src0) / E;
        u32x4* dst = reinterpret_cast<u32x4*>(out) + v;
        u32x4 x[WT > 0 ? WT : 1];
        if constexpr (WT > 0) {
#pragma unroll
          for (int r = 0; r < WT; ++r) x[r] = load16<true>(src + r * (p.ld_in / E));
          if constexpr (DC_RL_SP >= 0) {
            // the tile's run of each row, from its first vector t0
            u32x4* tile = reinterpret_cast<u32x4*>(out) + t0;
            const int32_t bytes = (int32_t)(t1 - t0) * 16, off = (int32_t)(v - t0) * 16;
#pragma unroll
            for (int r = 0; r < WT; ++r)
              store_buf<(DC_RL_SP >= 0 ? DC_RL_SP : 0)>(tile + r * (p.ld_out / E), bytes, off, x[r]);
          } else {
#pragma unroll
            for (int r = 0; r < WT; ++r) store16<true>(dst + r * (p.ld_out / E), x[r]);
          }
        } else {
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

template <int EB>
hipError_t launch_eb(const RelayoutParams& p, hipStream_t stream) {
  constexpr int E = 16 / EB;
  const int64_t nvec = (p.out_numel + E - 1) / E;
  const dim3 grid((unsigned)((nvec + kRT * kRelayoutU - 1) / (kRT * kRelayoutU)));
  switch (p.W) {
#define DC_RL_W(w)                                                                        \
  case w:                                                                                 \
    hipLaunchKernelGGL((k_relayout<EB, w>), grid, dim3(kRT),                              \
                       occupancy_pad(reinterpret_cast<const void*>(k_relayout<EB, w>), DC_RL_CAP), \
                       stream, p);                                                        \
    break;
    DC_RL_W(4)
    DC_RL_W(8)
    DC_RL_W(16)
#undef DC_RL_W
    default:
      hipLaunchKernelGGL((k_relayout<EB, 0>), grid, dim3(kRT), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_relayout(int32_t W, int32_t dtype, const void* in, int64_t ld_in, void* out,
                           int64_t ld_out, int64_t bucket_col, int64_t bucket_numel,
                           const dc_piece* pieces, int32_t npieces, int64_t out_numel,
                           hipStream_t stream) {
  if (out_numel == 0 || npieces == 0) return hipSuccess;
  RelayoutParams p{in, out, ld_in, ld_out, bucket_col, out_numel, pieces, npieces, W, bucket_numel};
  return dtype == DC_BF16 ? launch_eb<2>(p, stream) : launch_eb<4>(p, stream);
}

}  // namespace dc
