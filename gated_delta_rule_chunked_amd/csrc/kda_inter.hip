// kda_inter.hip -- inter-chunk state scan of the KDA chunked forward for gfx950.
//
// One workgroup per (sequence, value head, 16-column value tile); the chunks of
// the sequence are processed serially.  Per chunk, following the kernel-fun
// fwd_state module docstring (and FlashKDA's phases 3-6):
//   u   = TmB v                      (TmB = Tm diag(beta), the page's INV with beta)
//   v'  = u - w h                    (h: fp32 [K, 16] state, bf16 as MFMA operand)
//   o   = qg h + Aqk v'              (scale already folded into qg and Aqk)
//   h  <- diag(exp2 G) h + kg^T v'   (fp32; the decay is the MFMA's C input)
//
// Eight waves in two roles, as the kernel-fun design keeps the o readout off the
// recurrence's critical path:
//   waves 0-3 (state waves): wave w owns key rows [w K/4, (w+1) K/4) of h in the
//     C layout of the kg^T v' MFMA (the update never leaves registers), and rows
//     16w..16w+15 of u, w h and v'.
//   waves 4-7 (output waves): rows 16(w-4).. of qg h + Aqk v', the o stores, and
//     the loads of the v tile.
// The bf16 copy of h (B operand of w h and qg h) and v' (B operand of Aqk v' and
// kg^T v') cross waves through LDS once per chunk; two workgroup barriers per
// chunk.  All B fragments are read in P-order (kda_device.hpp), exactly as the
// owner lanes wrote them.
//
// Operands are read straight from the workspace records (one 16-byte load per
// lane per fragment) into per-role register rings several chunks deep.

#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {

constexpr int INTER_THREADS = 512;

template <int K>
struct StateOps {                          // state-wave operands of one chunk
  static constexpr int S = K / 32;
  static constexpr int MT = K / 64;
  uint4 wn[S];
  uint4 tmb[2];
  uint4 kgt[MT][2];
  float4 alpha[MT];
};
template <int K>
struct OutOps {                            // output-wave operands of one chunk
  static constexpr int S = K / 32;
  uint4 qg[S];
  uint4 aqk[2];
  uint2 v;                                 // 4 columns of one token row of v
};

struct SeqLoc {
  int b;
  int64_t bos;
  int len;
  int64_t cbase;  // chunk index of the sequence's first chunk
};

template <int K>
__device__ __forceinline__ const uint8_t* rec_ptr(const Params& p, const SeqLoc& sq, int hv, int c) {
  return p.recs + rec_index(hv, sq.cbase + c, p.max_chunks) * (int64_t)Rec<K>::BYTES;
}

template <int K>
__device__ __forceinline__ void load_state_ops(const Params& p, const SeqLoc& sq, int hv, int c, int w, int ln,
                                               StateOps<K>& op) {
  using R = Rec<K>;
  using O = StateOps<K>;
  const uint8_t* rec = rec_ptr<K>(p, sq, hv, c);
#pragma unroll
  for (int s = 0; s < O::S; ++s)
    op.wn[s] = *reinterpret_cast<const uint4*>(rec + R::WN + ((w * O::S + s) * 64 + ln) * 16);
#pragma unroll
  for (int mt = 0; mt < O::MT; ++mt)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
      op.kgt[mt][s2] = *reinterpret_cast<const uint4*>(rec + R::KGT + (((w * O::MT + mt) * 2 + s2) * 64 + ln) * 16);
  // row blocks 0, 1 have one nonzero 32-column step; their second load re-reads the
  // first fragment (unused) so that every load is unconditional
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
    op.tmb[s2] = *reinterpret_cast<const uint4*>(rec + R::TMB + (tri_frag(w, min(s2, tri_steps(w) - 1)) * 64 + ln) * 16);
  const int g = ln >> 4;
#pragma unroll
  for (int mt = 0; mt < O::MT; ++mt)
    op.alpha[mt] = *reinterpret_cast<const float4*>(rec + R::ALPHA + (w * (K / 4) + 16 * mt + 4 * g) * 4);
}

template <int K>
__device__ __forceinline__ void load_out_ops(const Params& p, const SeqLoc& sq, int hv, int vt, int c, int w,
                                             int ln, int otid, OutOps<K>& op) {
  using R = Rec<K>;
  using O = OutOps<K>;
  const uint8_t* rec = rec_ptr<K>(p, sq, hv, c);
#pragma unroll
  for (int s = 0; s < O::S; ++s)
    op.qg[s] = *reinterpret_cast<const uint4*>(rec + R::QG + ((w * O::S + s) * 64 + ln) * 16);
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)   // unconditional, as for TMB
    op.aqk[s2] = *reinterpret_cast<const uint4*>(rec + R::AQK + (tri_frag(w, min(s2, tri_steps(w) - 1)) * 64 + ln) * 16);
  // v tile: output thread otid -> token row otid/4, columns 4*(otid%4) .. +3.  The
  // load is unconditional (rows past the sequence end re-read its last row) so the
  // number of loads in flight is the same every chunk; store_v_tile zeroes those rows.
  const int t = min(c * BT + (otid >> 2), sq.len - 1);
  op.v = *reinterpret_cast<const uint2*>(p.v + (((int64_t)sq.b * p.T + sq.bos + t) * p.HV + hv) * p.V +
                                         vt * BV + 4 * (otid & 3));
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
__device__ __forceinline__ void store_v_tile(uint16_t* sVT, int otid, uint2 v, int c, int len) {
  using SM = InterSmem<K>;
  const int trow = otid >> 2, c0 = 4 * (otid & 3);
  if (c * BT + trow >= len) v = make_uint2(0, 0);   // rows past the sequence end
  sVT[(c0 + 0) * SM::VS + trow] = (uint16_t)(v.x & 0xffff);
  sVT[(c0 + 1) * SM::VS + trow] = (uint16_t)(v.x >> 16);
  sVT[(c0 + 2) * SM::VS + trow] = (uint16_t)(v.y & 0xffff);
  sVT[(c0 + 3) * SM::VS + trow] = (uint16_t)(v.y >> 16);
}

template <int K, int PFS, int PFO>
__global__ __launch_bounds__(INTER_THREADS, 1) void inter_kernel(Params p, int n_items) {
  // Both roles run the same number of iterations (whole ring turns), so every
  // workgroup barrier is met by all eight waves.
  static_assert(PFS == PFO, "state and output rings must have the same depth");
  using SM = InterSmem<K>;
  constexpr int S = K / 32, MT = K / 64;
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
  const int tid = threadIdx.x, ln = tid & 63, r = ln & 15, g = ln >> 4;
  // The wave index goes through readfirstlane so that every branch on it is a
  // scalar branch: an MFMA under a lane-predicated branch still writes all lanes.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w = wave & 3;               // row block (and key block for state waves)

  SeqLoc sq;
  if (p.cu == nullptr) {
    sq.b = n; sq.bos = 0; sq.len = p.T; sq.cbase = (int64_t)n * p.NT;
  } else {
    if (p.table[p.N + 1] != 0) {
      // rejected cu_seqlens: poison this tile's ht and, grid-strided, all of o
      const float qnan = __builtin_nanf("");
      if (p.ht)
        for (int idx = tid; idx < K * BV; idx += INTER_THREADS)
          p.ht[(((int64_t)n * p.HV + hv) * K + idx / BV) * p.V + vt * BV + idx % BV] = qnan;
      const int64_t total = (int64_t)p.B * p.T * p.HV * p.V;
      for (int64_t idx = (int64_t)item * INTER_THREADS + tid; idx < total; idx += (int64_t)n_items * INTER_THREADS)
        p.o[idx] = 0x7fc0;
      return;
    }
    sq.b = 0; sq.bos = p.cu[n]; sq.len = (int)(p.cu[n + 1] - p.cu[n]); sq.cbase = p.table[n];
  }
  const int nc = (sq.len + BT - 1) / BT;

  if (wave < 4) {
    // ======================== state waves ========================
    const int dbase = w * (K / 4);
    f32x4 h[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d = dbase + 16 * mt + 4 * g + rr;
        h[mt][rr] = p.h0 ? p.h0[(((int64_t)n * p.HV + hv) * K + d) * p.V + vt * BV + r] : 0.f;
      }
      *reinterpret_cast<uint2*>(sH + r * SM::HS + dbase + 16 * mt + 4 * g) = pack4(h[mt]);
    }
    StateOps<K> ring[PFS + 1];
#pragma unroll
    for (int j = 0; j < PFS; ++j)
      if (nc > 0) load_state_ops<K>(p, sq, hv, min(j, nc - 1), w, ln, ring[j]);
    __syncthreads();  // S0: h and the chunk-0 v tile in LDS

    // u = TmB v for chunk c reads the v tile in buffer c & 1, stored by the output
    // waves before barrier A of chunk c-1 (before S0 for chunk 0); it is computed
    // off the critical path, after barrier A of the previous chunk.
    auto tmb_v = [&](const StateOps<K>& op, int c) {
      const uint16_t* vrow = sVT + (c & 1) * BV * SM::VS + r * SM::VS;
      const bf16x8 v0 = pfrag(vrow, 0, g), v1 = pfrag(vrow, 32, g);
      f32x4 u0 = mfma16x32(as_frag(op.tmb[0]), v0, f32x4{0.f, 0.f, 0.f, 0.f});
      if (tri_steps(w) > 1) u0 = mfma16x32(as_frag(op.tmb[1]), v1, u0);   // scalar branch
      return u0;
    };
    f32x4 u = tmb_v(ring[0], 0);

    // Whole ring turns, no early exit, so every ring slot stays a fixed set of
    // registers; turns past the last chunk are masked (h kept, nothing stored).
    const int nturn = (nc + PFS) / (PFS + 1);
    for (int t0 = 0; t0 < nturn; ++t0) {
#pragma unroll
      for (int j = 0; j <= PFS; ++j) {
        const int c = t0 * (PFS + 1) + j;
        const bool active = c < nc;
        const StateOps<K>& cur = ring[j];
        // unconditional (clamped) so the count of loads in flight is static
        load_state_ops<K>(p, sq, hv, min(c + PFS, nc - 1), w, ln, ring[(j + PFS) % (PFS + 1)]);
        // v' = u + (-w) h  (rows 16w..), two half chains over the key steps
        bf16x8 hb[S];
#pragma unroll
        for (int s = 0; s < S; ++s) hb[s] = pfrag(sH + r * SM::HS, 32 * s, g);
        __builtin_amdgcn_sched_barrier(0);
        f32x4 acc = u, acc2 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < S; s += 2) {
          acc = mfma16x32(as_frag(cur.wn[s]), hb[s], acc);
          acc2 = mfma16x32(as_frag(cur.wn[s + 1]), hb[s + 1], acc2);
        }
        acc += acc2;
        *reinterpret_cast<uint2*>(sVP + r * SM::VS + 16 * w + 4 * g) = pack4(acc);
        f32x4 hn[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          hn[mt][0] = cur.alpha[mt].x * h[mt][0];
          hn[mt][1] = cur.alpha[mt].y * h[mt][1];
          hn[mt][2] = cur.alpha[mt].z * h[mt][2];
          hn[mt][3] = cur.alpha[mt].w * h[mt][3];
        }
        __syncthreads();  // A: v' and v tile c+1 complete; every read of h is done
        const bf16x8 vb0 = pfrag(sVP + r * SM::VS, 0, g);
        const bf16x8 vb1 = pfrag(sVP + r * SM::VS, 32, g);
        __builtin_amdgcn_sched_barrier(0);
        // h <- diag(alpha) h + kg^T v'
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          hn[mt] = mfma16x32(as_frag(cur.kgt[mt][0]), vb0, hn[mt]);
          hn[mt] = mfma16x32(as_frag(cur.kgt[mt][1]), vb1, hn[mt]);
          if (active) h[mt] = hn[mt];
          *reinterpret_cast<uint2*>(sH + r * SM::HS + dbase + 16 * mt + 4 * g) = pack4(h[mt]);
        }
        u = tmb_v(ring[(j + 1) % (PFS + 1)], c + 1);
        __syncthreads();  // B: h complete; every read of v' and of v tile c+1 is done
      }
    }
    if (p.ht) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int d = dbase + 16 * mt + 4 * g + rr;
          p.ht[(((int64_t)n * p.HV + hv) * K + d) * p.V + vt * BV + r] = h[mt][rr];
        }
    }
  } else {
    // ======================== output waves ========================
    const int otid = tid - 256;
    OutOps<K> ring[PFO + 1];
#pragma unroll
    for (int j = 0; j < PFO; ++j)
      if (nc > 0) load_out_ops<K>(p, sq, hv, vt, min(j, nc - 1), w, ln, otid, ring[j]);
    if (nc > 0) store_v_tile<K>(sVT, otid, ring[0].v, 0, sq.len);
    __syncthreads();  // S0

    // Chunk c's o = qg h + Aqk v' is finished after barrier B (with v' kept in
    // registers), so the output waves never hold up the state waves between
    // barriers A and B; its o rows are stored during the next chunk.
    f32x4 oq = f32x4{0.f, 0.f, 0.f, 0.f};   // qg h of the pending chunk
    bf16x8 vbp0 = as_frag(make_uint4(0, 0, 0, 0)), vbp1 = vbp0;
    uint4 aqp0 = make_uint4(0, 0, 0, 0), aqp1 = aqp0;
    auto finish = [&](int c) {   // o rows 16w + 4g + rr of chunk c, column vt*16 + r
      f32x4 o0 = mfma16x32(as_frag(aqp0), vbp0, oq);
      if (tri_steps(w) > 1) o0 = mfma16x32(as_frag(aqp1), vbp1, o0);     // scalar branch
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int t = c * BT + 16 * w + 4 * g + rr;
        if (t < sq.len)
          p.o[(((int64_t)sq.b * p.T + sq.bos + t) * p.HV + hv) * p.V + vt * BV + r] = f2bf(o0[rr]);
      }
    };
    const int nturn = (nc + PFO) / (PFO + 1);   // whole ring turns (see the state waves)
    for (int t0 = 0; t0 < nturn; ++t0) {
#pragma unroll
      for (int j = 0; j <= PFO; ++j) {
        const int c = t0 * (PFO + 1) + j;
        const OutOps<K>& cur = ring[j];
        load_out_ops<K>(p, sq, hv, vt, min(c + PFO, nc - 1), w, ln, otid, ring[(j + PFO) % (PFO + 1)]);
        bf16x8 hb[S];
#pragma unroll
        for (int s = 0; s < S; ++s) hb[s] = pfrag(sH + r * SM::HS, 32 * s, g);
        __builtin_amdgcn_sched_barrier(0);
        if (c > 0) finish(c - 1);
        f32x4 oacc = f32x4{0.f, 0.f, 0.f, 0.f}, oacc2 = oacc;
#pragma unroll
        for (int s = 0; s < S; s += 2) {
          oacc = mfma16x32(as_frag(cur.qg[s]), hb[s], oacc);
          oacc2 = mfma16x32(as_frag(cur.qg[s + 1]), hb[s + 1], oacc2);
        }
        oq = oacc + oacc2;
        aqp0 = cur.aqk[0];
        aqp1 = tri_steps(w) > 1 ? cur.aqk[1] : make_uint4(0, 0, 0, 0);
        // next chunk's v tile (rows past the sequence end, or a whole chunk past it, are zeros)
        store_v_tile<K>(sVT + ((c + 1) & 1) * BV * SM::VS, otid, ring[(j + 1) % (PFO + 1)].v, c + 1, sq.len);
        __syncthreads();  // A
        vbp0 = pfrag(sVP + r * SM::VS, 0, g);
        vbp1 = pfrag(sVP + r * SM::VS, 32, g);
        __syncthreads();  // B
      }
    }
    const int clast = nturn * (PFO + 1) - 1;   // last iteration's chunk
    if (clast < nc) finish(clast);             // else it was finished inside the loop
  }
}

#ifndef KDA_INTER_PF
#define KDA_INTER_PF 3   // chunks in flight ahead of the current one (both roles)
#endif
constexpr int INTER_PFS = KDA_INTER_PF;
constexpr int INTER_PFO = KDA_INTER_PF;

hipError_t launch_inter(const Params& p, hipStream_t s) {
  const int64_t items = (int64_t)p.N * p.HV * (p.V / BV);
  if (items == 0) return hipSuccess;
  const int grid = (int)((items + 7) / 8 * 8);
  if (p.K == 128)
    hipLaunchKernelGGL((inter_kernel<128, INTER_PFS, INTER_PFO>), dim3(grid), dim3(INTER_THREADS), 0, s, p,
                       (int)items);
  else
    hipLaunchKernelGGL((inter_kernel<64, INTER_PFS, INTER_PFO>), dim3(grid), dim3(INTER_THREADS), 0, s, p,
                       (int)items);
  return hipGetLastError();
}

}  // namespace kda
