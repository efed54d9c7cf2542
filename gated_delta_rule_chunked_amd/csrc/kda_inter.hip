// kda_inter.hip -- inter-chunk state scan of the KDA chunked forward for gfx950.
//
// One workgroup (4 waves) per (sequence, value head, 16-column value tile); the
// chunks of the sequence are processed serially.  Per chunk, following the
// kernel-fun fwd_state module docstring (and FlashKDA's phases 3-6):
//   u   = TmB v                      (TmB = Tm diag(beta), the page's INV with beta)
//   v'  = u - w h                    (h: fp32 [K, 16] state, bf16 as MFMA operand)
//   o   = qg h + Aqk v'              (scale already folded into qg and Aqk)
//   h  <- diag(exp2 G) h + kg^T v'   (fp32; the decay is the MFMA's C input)
//
// State layout: wave w owns key rows [w K/4, (w+1) K/4) of h, in the C layout of
// the kg^T v' MFMA, so the update never leaves registers.  The bf16 copy of h that
// every wave needs as the B operand of w h and qg h goes through LDS once per
// chunk, and so does v' (B operand of Aqk v' and kg^T v').  Two workgroup
// barriers per chunk; everything else is MFMA on register fragments.
//
// Operands are read straight from the workspace records (written by the intra
// kernel in fragment order: one 16-byte load per lane per fragment) into a
// register ring PF chunks deep, so chunk c+PF is in flight while c computes.

#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {

template <int K>
struct InterOps {
  static constexpr int S = K / 32;        // 32-wide steps over the key dim
  static constexpr int MT = K / 64;       // 16-row key blocks per wave
  uint4 qg[S], wn[S];
  uint4 kgt[MT][2];
  uint4 aqk[2], tmb[2];
  float4 alpha[MT];
  uint2 v;                                // 4 columns of one token row of v
};

struct SeqLoc {
  int b;
  int64_t bos;
  int len;
  int64_t cbase;  // chunk index of the sequence's first chunk
};

template <int K>
__device__ __forceinline__ void load_ops(const Params& p, const SeqLoc& sq, int hv, int vt, int c,
                                         int w, int ln, int tid, InterOps<K>& op) {
  using R = Rec<K>;
  using O = InterOps<K>;
  const uint8_t* rec = p.recs + ((sq.cbase + c) * p.HV + hv) * (int64_t)R::BYTES;
#pragma unroll
  for (int s = 0; s < O::S; ++s) {
    op.qg[s] = *reinterpret_cast<const uint4*>(rec + R::QG + ((w * O::S + s) * 64 + ln) * 16);
    op.wn[s] = *reinterpret_cast<const uint4*>(rec + R::WN + ((w * O::S + s) * 64 + ln) * 16);
  }
#pragma unroll
  for (int mt = 0; mt < O::MT; ++mt)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
      op.kgt[mt][s2] = *reinterpret_cast<const uint4*>(
          rec + R::KGT + (((w * O::MT + mt) * 2 + s2) * 64 + ln) * 16);
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    if (s2 < tri_steps(w)) {
      op.aqk[s2] = *reinterpret_cast<const uint4*>(rec + R::AQK + (tri_frag(w, s2) * 64 + ln) * 16);
      op.tmb[s2] = *reinterpret_cast<const uint4*>(rec + R::TMB + (tri_frag(w, s2) * 64 + ln) * 16);
    } else {
      op.aqk[s2] = make_uint4(0, 0, 0, 0);
      op.tmb[s2] = op.aqk[s2];
    }
  }
  const int g = ln >> 4;
#pragma unroll
  for (int mt = 0; mt < O::MT; ++mt)
    op.alpha[mt] = *reinterpret_cast<const float4*>(rec + R::ALPHA + (w * (K / 4) + 16 * mt + 4 * g) * 4);
  // v tile: thread -> token row tid/4, columns 4*(tid%4) .. +3 of the value tile
  const int trow = tid >> 2;
  const int64_t t = (int64_t)c * BT + trow;
  op.v = make_uint2(0, 0);
  if (t < sq.len)
    op.v = *reinterpret_cast<const uint2*>(p.v + (((int64_t)sq.b * p.T + sq.bos + t) * p.HV + hv) * p.V +
                                           vt * BV + 4 * (tid & 3));
}

// LDS: bf16 [16 columns][stride] tiles, key/token index contiguous.
template <int K>
struct InterSmem {
  static constexpr int HS = K + 8;      // h^T row stride
  static constexpr int VS = BT + 8;     // v'^T and v^T row stride
  static constexpr int H = 0;
  static constexpr int VP = H + BV * HS * 2;
  static constexpr int VT = VP + BV * VS * 2;   // two buffers
  static constexpr int BYTES = VT + 2 * BV * VS * 2;
};

__device__ __forceinline__ uint2 pack4(const f32x4& a) {
  return make_uint2(pack2(a[0], a[1]), pack2(a[2], a[3]));
}

template <int K>
__device__ __forceinline__ void store_v_tile(uint16_t* sVT, int tid, const uint2& v) {
  using SM = InterSmem<K>;
  const int trow = tid >> 2, c0 = 4 * (tid & 3);
  sVT[(c0 + 0) * SM::VS + trow] = (uint16_t)(v.x & 0xffff);
  sVT[(c0 + 1) * SM::VS + trow] = (uint16_t)(v.x >> 16);
  sVT[(c0 + 2) * SM::VS + trow] = (uint16_t)(v.y & 0xffff);
  sVT[(c0 + 3) * SM::VS + trow] = (uint16_t)(v.y >> 16);
}

template <int K, int PF>
__global__ __launch_bounds__(NTHREADS, 1) void inter_kernel(Params p, int n_items) {
  using SM = InterSmem<K>;
  using O = InterOps<K>;
  constexpr int S = O::S, MT = O::MT;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SM::BYTES];
  uint16_t* sH = reinterpret_cast<uint16_t*>(smem + SM::H);
  uint16_t* sVP = reinterpret_cast<uint16_t*>(smem + SM::VP);
  uint16_t* sVT = reinterpret_cast<uint16_t*>(smem + SM::VT);

  const int item = xcd_remap(blockIdx.x, gridDim.x);
  if (item >= n_items) return;
  const int NVT = p.V / BV;
  const int vt = item % NVT;
  const int hv = (item / NVT) % p.HV;
  const int n = item / (NVT * p.HV);
  const int tid = threadIdx.x, w = tid >> 6, ln = tid & 63, r = ln & 15, grp = ln >> 4;
  const int dbase = w * (K / 4);

  SeqLoc sq;
  if (p.cu == nullptr) {
    sq.b = n; sq.bos = 0; sq.len = p.T; sq.cbase = (int64_t)n * p.NT;
  } else {
    if (p.table[p.N + 1] != 0) {
      // rejected cu_seqlens: poison this tile's ht and, grid-strided, all of o
      const float qnan = __builtin_nanf("");
      if (p.ht)
        for (int idx = tid; idx < K * BV; idx += NTHREADS)
          p.ht[(((int64_t)n * p.HV + hv) * K + idx / BV) * p.V + vt * BV + idx % BV] = qnan;
      const int64_t total = (int64_t)p.B * p.T * p.HV * p.V;
      for (int64_t idx = (int64_t)item * NTHREADS + tid; idx < total; idx += (int64_t)n_items * NTHREADS)
        p.o[idx] = 0x7fc0;
      return;
    }
    sq.b = 0; sq.bos = p.cu[n]; sq.len = (int)(p.cu[n + 1] - p.cu[n]); sq.cbase = p.table[n];
  }
  const int nc = (sq.len + BT - 1) / BT;

  // initial state: lane holds h[dbase + 16mt + 4grp + rr][vt*16 + r]
  f32x4 h[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int d = dbase + 16 * mt + 4 * grp + rr;
      h[mt][rr] = p.h0 ? p.h0[(((int64_t)n * p.HV + hv) * K + d) * p.V + vt * BV + r] : 0.f;
    }
    *reinterpret_cast<uint2*>(sH + r * SM::HS + dbase + 16 * mt + 4 * grp) = pack4(h[mt]);
  }

  O ring[PF + 1];
#pragma unroll
  for (int j = 0; j < PF; ++j)
    if (j < nc) load_ops<K>(p, sq, hv, vt, j, w, ln, tid, ring[j]);
  if (nc > 0) store_v_tile<K>(sVT, tid, ring[0].v);
  __syncthreads();

  for (int c0 = 0; c0 < nc; c0 += PF + 1) {
#pragma unroll
    for (int j = 0; j <= PF; ++j) {
      const int c = c0 + j;
      if (c >= nc) break;
      O& cur = ring[j];
      if (c + PF < nc) load_ops<K>(p, sq, hv, vt, c + PF, w, ln, tid, ring[(j + PF) % (PF + 1)]);
      const uint16_t* vT = sVT + (c & 1) * BV * SM::VS;

      // u = TmB v  (this wave's 16 rows)
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        if (s2 >= tri_steps(w)) continue;
        const uint4 b = *reinterpret_cast<const uint4*>(vT + r * SM::VS + 32 * s2 + 8 * grp);
        acc = mfma16x32(as_frag(cur.tmb[s2]), as_frag(b), acc);
      }
      // h as B operand: h[32s + 8grp .. +7][r]
      bf16x8 hb[S];
#pragma unroll
      for (int s = 0; s < S; ++s)
        hb[s] = as_frag(*reinterpret_cast<const uint4*>(sH + r * SM::HS + 32 * s + 8 * grp));
      // v' = u + (-w) h ; o = qg h
      f32x4 oacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < S; ++s) {
        acc = mfma16x32(as_frag(cur.wn[s]), hb[s], acc);
        oacc = mfma16x32(as_frag(cur.qg[s]), hb[s], oacc);
      }
      *reinterpret_cast<uint2*>(sVP + r * SM::VS + 16 * w + 4 * grp) = pack4(acc);
      __syncthreads();  // A: v' complete; every read of h and of v^T[c] is done

      const bf16x8 vb0 = as_frag(*reinterpret_cast<const uint4*>(sVP + r * SM::VS + 8 * grp));
      const bf16x8 vb1 = as_frag(*reinterpret_cast<const uint4*>(sVP + r * SM::VS + 32 + 8 * grp));
      // h <- diag(alpha) h + kg^T v'
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 hn;
        hn[0] = cur.alpha[mt].x * h[mt][0];
        hn[1] = cur.alpha[mt].y * h[mt][1];
        hn[2] = cur.alpha[mt].z * h[mt][2];
        hn[3] = cur.alpha[mt].w * h[mt][3];
        hn = mfma16x32(as_frag(cur.kgt[mt][0]), vb0, hn);
        hn = mfma16x32(as_frag(cur.kgt[mt][1]), vb1, hn);
        h[mt] = hn;
        *reinterpret_cast<uint2*>(sH + r * SM::HS + dbase + 16 * mt + 4 * grp) = pack4(hn);
      }
      // o += Aqk v'
      oacc = mfma16x32(as_frag(cur.aqk[0]), vb0, oacc);
      if (tri_steps(w) > 1) oacc = mfma16x32(as_frag(cur.aqk[1]), vb1, oacc);
      // o rows 16w + 4grp + rr, column vt*16 + r
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int t = c * BT + 16 * w + 4 * grp + rr;
        if (t < sq.len)
          p.o[(((int64_t)sq.b * p.T + sq.bos + t) * p.HV + hv) * p.V + vt * BV + r] = f2bf(oacc[rr]);
      }
      // next chunk's v tile into the other buffer
      if (c + 1 < nc) store_v_tile<K>(sVT + ((c + 1) & 1) * BV * SM::VS, tid, ring[(j + 1) % (PF + 1)].v);
      __syncthreads();  // B: h and v^T[c+1] complete; every read of v' is done
    }
  }

  if (p.ht) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d = dbase + 16 * mt + 4 * grp + rr;
        p.ht[(((int64_t)n * p.HV + hv) * K + d) * p.V + vt * BV + r] = h[mt][rr];
      }
  }
}

constexpr int INTER_PF = 1;

hipError_t launch_inter(const Params& p, hipStream_t s) {
  const int64_t items = (int64_t)p.N * p.HV * (p.V / BV);
  if (items == 0) return hipSuccess;
  const int grid = (int)((items + 7) / 8 * 8);
  if (p.K == 128)
    hipLaunchKernelGGL((inter_kernel<128, INTER_PF>), dim3(grid), dim3(NTHREADS), 0, s, p, (int)items);
  else
    hipLaunchKernelGGL((inter_kernel<64, INTER_PF>), dim3(grid), dim3(NTHREADS), 0, s, p, (int)items);
  return hipGetLastError();
}

}  // namespace kda
