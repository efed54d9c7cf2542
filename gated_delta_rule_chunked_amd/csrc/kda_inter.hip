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
// Eight waves in three roles, one workgroup barrier per chunk:
//   wave 0 (state wave): holds the whole state h in the C layout of 16x16 MFMA
//     tiles.  A 16x16 C tile is already the B operand of the next product along
//     its rows (P-order, kda_device.hpp), so u, v' = u + (-w) h and
//     h <- diag(alpha) h + kg^T v' run back to back in registers, with no LDS
//     round trip and no barrier inside the recurrence.  It reads its operands
//     (WN, KGT, TMB, ALPHA, v^T) from LDS in two batches ahead of the products
//     and publishes the bf16 h and v' of the chunk for the output waves.
//   waves 1-4 (output waves): o of the previous chunk, o = qg h + Aqk v', from the
//     published h and v' and their own qg / Aqk fragments (a register ring fed
//     from the workspace records five phases ahead); they also stage the v tiles
//     (v^T in LDS).
//   waves 5-7 (loader waves): keep the state operands of three chunks in flight in
//     a register ring (plain 16-byte loads, the record read as 1 KiB steps) and
//     write chunk c+1 into the free slot of a two-slot LDS ring during phase c.
// Phase p (between barriers p-1 and p): the state wave runs chunk p, the output
// waves finish chunk p-1 and store the v tile of chunk p+1, the loaders stage
// chunk p+1 and fetch chunk p+3.  The barrier is a raw s_barrier after the wave's
// own LDS writes, so no wave waits for its outstanding global loads there.

#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {

constexpr int INTER_THREADS = 512;
constexpr int LD_RING = 3;     // chunks of state operands in flight per loader wave
constexpr int OUT_RING = 6;    // output-wave operand ring (phases); a multiple of LD_RING

template <int K>
struct InterSmem {
  using R = Rec<K>;
  static constexpr int NSTEP = (R::STATE_BYTES + 1023) / 1024;  // 1 KiB steps of the state operands
  static constexpr int NLD = (NSTEP + 2) / 3;                    // steps per loader wave
  static constexpr int STAGE = NLD * 3 * 1024;                   // one slot of the LDS ring
  static constexpr int ST = 0;                                   // two slots
  // published bf16 h (K/16 tiles) and v' (4 tiles) of a chunk, 64 lanes x 8 B per tile
  static constexpr int HB_BYTES = (K / 16) * 512 + 4 * 512;
  static constexpr int HB = ST + 2 * STAGE;                      // two buffers
  static constexpr int VS = BT + 8;                              // v^T row stride (bf16)
  static constexpr int VT = HB + 2 * HB_BYTES;                   // two v^T tiles
  static constexpr int BYTES = VT + 2 * BV * VS * 2;
  static_assert(STAGE <= R::BYTES, "padded copy steps stay inside the record");
  static_assert(BYTES <= 160 * 1024, "fits the LDS of one CU");
  static_assert(OUT_RING % LD_RING == 0, "one phase count serves every role");
};

template <int K>
struct OutOps {                            // output-wave operands of one phase
  static constexpr int S = K / 32;
  uint4 qg[S];                             // chunk p-1
  uint4 aqk[2];
  uint2 v;                                 // chunk p+1: 4 columns of one token row of v
};

template <int K>
__device__ __forceinline__ const uint8_t* rec_ptr(const Params& p, const SeqLoc& sq, int hv, int c) {
  return p.recs + rec_index(hv, sq.cbase + c, p.HV) * (int64_t)Rec<K>::BYTES;
}

template <int K>
__global__ __launch_bounds__(INTER_THREADS, 1) void inter_kernel(Params p, int n_items) {
  using SM = InterSmem<K>;
  using R = Rec<K>;
  constexpr int S = K / 32, ND = K / 16, PF = OUT_RING - 1;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SM::BYTES];

  // With the longest-first order (varlen) every workgroup of the grid is mapped to a
  // (sequence rank, head) unit in dispatch order, a unit's tiles following in
  // consecutive rounds of eight on one XCD; otherwise items are XCD-remapped.
  const bool lpt = p.order != nullptr;
  const int item = lpt ? (int)blockIdx.x : xcd_remap(blockIdx.x, gridDim.x);
  if (lpt) n_items = (int)gridDim.x;
  if (item >= n_items) return;
  const int NVT = p.V / BV;
  int vt, hv, n;
  bool unit_ok = true;
  if (lpt) {
    const int rnd = item >> 3;
    const int64_t u = (int64_t)(rnd / NVT) * 8 + (item & 7);
    unit_ok = u < (int64_t)p.N * p.HV;
    vt = rnd % NVT;
    hv = unit_ok ? (int)(u % p.HV) : 0;
    n = unit_ok ? p.order[u / p.HV] : 0;
    if ((unsigned)n >= (unsigned)p.N) unit_ok = false, n = 0;   // never for an order the chunk table wrote
  } else {
    vt = item % NVT;
    hv = (item / NVT) % p.HV;
    n = item / (NVT * p.HV);
  }
  const int tid = threadIdx.x, ln = tid & 63, r = ln & 15, g = ln >> 4;
  // The wave index goes through readfirstlane so that every branch on it is a
  // scalar branch: an MFMA under a lane-predicated branch still writes all lanes.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  SeqLoc sq;
  if (p.cu == nullptr) {
    sq.b = n; sq.bos = 0; sq.len = p.T; sq.cbase = (int64_t)n * p.NT;
  } else {
    if (p.table[p.N + 1] != 0) {
      // rejected cu_seqlens: poison this tile's ht and, grid-strided, all of o
      const float qnan = __builtin_nanf("");
      if (p.ht && unit_ok)
        for (int idx = tid; idx < K * BV; idx += INTER_THREADS)
          store_state(p.flags & FLAG_STATE_BF16, p.ht, (((int64_t)n * p.HV + hv) * K + idx / BV) * p.V + vt * BV + idx % BV, qnan);
      const int64_t total = (int64_t)p.B * p.T * p.HV * p.V;
      for (int64_t idx = (int64_t)item * INTER_THREADS + tid; idx < total; idx += (int64_t)n_items * INTER_THREADS)
        p.o[idx] = 0x7fc0;
      return;
    }
    if (!unit_ok) return;
    sq.b = 0; sq.bos = p.cu[n]; sq.len = (int)(p.cu[n + 1] - p.cu[n]); sq.cbase = p.table[n];
  }
  const int nc = (sq.len + BT - 1) / BT;
  // phases 0..nc (the last only finishes o of chunk nc-1), in whole ring turns;
  // every role runs the same count, one barrier each
  const int nphase = (nc + 1 + OUT_RING - 1) / OUT_RING * OUT_RING;

  if (wave == 0) {
    // ============================ state wave ============================
    // h tile md: lane holds h[16md + 4g + rr][vt*16 + r], rr = 0..3
    f32x4 h[ND];
#pragma unroll
    for (int md = 0; md < ND; ++md)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d = 16 * md + 4 * g + rr;
        h[md][rr] = p.h0 ? load_state(p.flags & FLAG_STATE_BF16, p.h0, (((int64_t)n * p.HV + hv) * K + d) * p.V + vt * BV + r) : 0.f;
      }
    barrier_lds();  // S0
    for (int ph = 0; ph < nphase; ++ph) {
      if (ph < nc) {
        if (p.hc) {   // the state before this chunk; uniform branches, before the operand batches
          // The row stride is re-made opaque every chunk, so the 32 row offsets stay
          // transient scalars instead of being hoisted out of the loop as live
          // 64-bit addresses (which spilled the whole kernel).
          int sv = p.V;
          asm volatile("" : "+s"(sv));
          const int64_t base = (((sq.cbase + ph) * p.HV + hv) * K + 4 * g) * (int64_t)sv + vt * BV + r;
          if (p.flags & FLAG_STATE_BF16) {
            uint16_t* dst = static_cast<uint16_t*>(p.hc) + base;
#pragma unroll
            for (int md = 0; md < ND; ++md)
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) dst[(int64_t)(16 * md + rr) * sv] = f2bf(h[md][rr]);
          } else {
            float* dst = static_cast<float*>(p.hc) + base;
#pragma unroll
            for (int md = 0; md < ND; ++md)
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) dst[(int64_t)(16 * md + rr) * sv] = h[md][rr];
          }
        }
        const uint8_t* st = smem + SM::ST + (ph & 1) * SM::STAGE;
        const uint16_t* vrow = reinterpret_cast<const uint16_t*>(smem + SM::VT) + (ph & 1) * BV * SM::VS + r * SM::VS;
        // batch 1: v^T, TmB, decay, -w (in the order they are consumed)
        const bf16x8 vb0 = pfrag(vrow, 0, g), vb1 = pfrag(vrow, 32, g);
        uint4 tm[6], wn[4 * S];
        float4 al[ND];
#pragma unroll
        for (int f = 0; f < 6; ++f) tm[f] = lds16(st + R::TMB + (f * 64 + ln) * 16);
#pragma unroll
        for (int md = 0; md < ND; ++md) al[md] = *reinterpret_cast<const float4*>(st + R::ALPHA + (16 * md + 4 * g) * 4);
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) wn[s * 4 + mb] = lds16(st + R::WN + ((mb * S + s) * 64 + ln) * 16);
        __builtin_amdgcn_sched_barrier(0);
        // u = TmB v, row blocks mb = 0..3 (lower triangular: 1 or 2 32-steps)
        f32x4 acc[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          acc[mb] = mfma16x32(as_frag(tm[tri_frag(mb, 0)]), vb0, f32x4{0.f, 0.f, 0.f, 0.f});
          if (mb >= 2) acc[mb] = mfma16x32(as_frag(tm[tri_frag(mb, 1)]), vb1, acc[mb]);
        }
        // h as B operand (tiles (2s, 2s+1) form the P-order fragment of 32-step s),
        // published for the output waves; then h <- diag(alpha) h
        uint2 hb[ND];
        uint8_t* hbuf = smem + SM::HB + (ph & 1) * SM::HB_BYTES;
#pragma unroll
        for (int md = 0; md < ND; ++md) {
          hb[md] = pack4(h[md]);
          *reinterpret_cast<uint2*>(hbuf + (md * 64 + ln) * 8) = hb[md];
          h[md][0] *= al[md].x;
          h[md][1] *= al[md].y;
          h[md][2] *= al[md].z;
          h[md][3] *= al[md].w;
        }
        __builtin_amdgcn_sched_barrier(0);
        // batch 2: kg^T
        uint4 kg[2 * ND];
#pragma unroll
        for (int i = 0; i < 2 * ND; ++i) kg[i] = lds16(st + R::KGT + (i * 64 + ln) * 16);
        __builtin_amdgcn_sched_barrier(0);
        // v' = u + (-w) h
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const bf16x8 hbs = cat(hb[2 * s], hb[2 * s + 1]);
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) acc[mb] = mfma16x32(as_frag(wn[s * 4 + mb]), hbs, acc[mb]);
        }
        uint2 vp[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          vp[mb] = pack4(acc[mb]);
          *reinterpret_cast<uint2*>(hbuf + ND * 512 + (mb * 64 + ln) * 8) = vp[mb];
        }
        // h <- diag(alpha) h + kg^T v'   (v' tiles (2s2, 2s2+1) = P-order token step s2)
        const bf16x8 vp0 = cat(vp[0], vp[1]), vp1 = cat(vp[2], vp[3]);
#pragma unroll
        for (int md = 0; md < ND; ++md) {
          h[md] = mfma16x32(as_frag(kg[2 * md]), vp0, h[md]);
          h[md] = mfma16x32(as_frag(kg[2 * md + 1]), vp1, h[md]);
        }
      }
      barrier_lds();
    }
    if (p.ht) {
#pragma unroll
      for (int md = 0; md < ND; ++md)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int d = 16 * md + 4 * g + rr;
          store_state(p.flags & FLAG_STATE_BF16, p.ht, (((int64_t)n * p.HV + hv) * K + d) * p.V + vt * BV + r, h[md][rr]);
        }
    }
  } else if (wave <= 4) {
    // ============================ output waves ============================
    const int w = wave - 1;                 // row block
    const int otid = tid - 64;              // 0..255 across the four output waves
    const int trow = otid >> 2, c4 = 4 * (otid & 3);
    uint16_t* sVT = reinterpret_cast<uint16_t*>(smem + SM::VT);
    auto v_ptr = [&](int c) {               // row trow of chunk c (clamped into the sequence)
      const int t = min(c * BT + trow, sq.len - 1);
      return reinterpret_cast<const uint2*>(p.v + (((int64_t)sq.b * p.T + sq.bos + t) * p.HV + hv) * p.V +
                                            vt * BV + c4);
    };
    auto store_v = [&](int c, uint2 v) {    // v^T tile of chunk c into buffer c & 1; rows past the end are 0
      if (c * BT + trow >= sq.len) v = make_uint2(0, 0);
      uint16_t* dst = sVT + (c & 1) * BV * SM::VS;
      dst[(c4 + 0) * SM::VS + trow] = (uint16_t)(v.x & 0xffff);
      dst[(c4 + 1) * SM::VS + trow] = (uint16_t)(v.x >> 16);
      dst[(c4 + 2) * SM::VS + trow] = (uint16_t)(v.y & 0xffff);
      dst[(c4 + 3) * SM::VS + trow] = (uint16_t)(v.y >> 16);
    };
    // ring slot of phase ph: qg / Aqk of chunk ph-1 and v of chunk ph+1 (clamped loads;
    // unconditional so the number of loads in flight is the same every phase)
    auto load = [&](int ph, OutOps<K>& op) {
      const uint8_t* rec = rec_ptr<K>(p, sq, hv, min(max(ph - 1, 0), nc - 1));
#pragma unroll
      for (int s = 0; s < S; ++s)
        op.qg[s] = *reinterpret_cast<const uint4*>(rec + R::QG + ((w * S + s) * 64 + ln) * 16);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)   // row blocks 0, 1 have one nonzero step; the second load repeats it
        op.aqk[s2] = *reinterpret_cast<const uint4*>(rec + R::AQK + (tri_frag(w, min(s2, tri_steps(w) - 1)) * 64 + ln) * 16);
      op.v = *v_ptr(ph + 1);
    };
    if (nc == 0) {                          // empty sequence: only keep the barrier count
      for (int ph = 0; ph <= nphase; ++ph) barrier_lds();
      return;
    }
    OutOps<K> ring[OUT_RING];
    const uint2 v0 = *v_ptr(0);
#pragma unroll
    for (int j = 0; j < PF; ++j) load(j, ring[j]);
    store_v(0, v0);
    barrier_lds();  // S0
    for (int t0 = 0; t0 < nphase; t0 += OUT_RING) {
#pragma unroll
      for (int j = 0; j < OUT_RING; ++j) {
        const int ph = t0 + j;
        const OutOps<K>& cur = ring[j];
        load(ph + PF, ring[(j + PF) % OUT_RING]);
        if (ph >= 1 && ph <= nc) {
          const int c = ph - 1;
          const uint8_t* hbuf = smem + SM::HB + (c & 1) * SM::HB_BYTES;
          bf16x8 hbs[S];
#pragma unroll
          for (int s = 0; s < S; ++s)
            hbs[s] = cat(lds8(hbuf + ((2 * s) * 64 + ln) * 8), lds8(hbuf + ((2 * s + 1) * 64 + ln) * 8));
          const bf16x8 vp0 = cat(lds8(hbuf + ND * 512 + (0 * 64 + ln) * 8), lds8(hbuf + ND * 512 + (1 * 64 + ln) * 8));
          const bf16x8 vp1 = cat(lds8(hbuf + ND * 512 + (2 * 64 + ln) * 8), lds8(hbuf + ND * 512 + (3 * 64 + ln) * 8));
          // o^T = h^T qg^T + v'^T Aqk^T: the same P-order fragments with A and B
          // swapped, so lane (g, r) ends up with token 16w + r, columns 4g .. 4g+3
          // (one 8-byte store per lane instead of four 2-byte ones)
          f32x4 oacc = f32x4{0.f, 0.f, 0.f, 0.f}, oacc2 = oacc;
#pragma unroll
          for (int s = 0; s < S; s += 2) {
            oacc = mfma16x32(hbs[s], as_frag(cur.qg[s]), oacc);
            oacc2 = mfma16x32(hbs[s + 1], as_frag(cur.qg[s + 1]), oacc2);
          }
          oacc = mfma16x32(vp0, as_frag(cur.aqk[0]), oacc);
          if (tri_steps(w) > 1) oacc2 = mfma16x32(vp1, as_frag(cur.aqk[1]), oacc2);   // scalar branch
          oacc += oacc2;
          const int t = c * BT + 16 * w + r;
          if (t < sq.len)
            *reinterpret_cast<uint2*>(p.o + (((int64_t)sq.b * p.T + sq.bos + t) * p.HV + hv) * p.V + vt * BV + 4 * g) =
                pack4(oacc);
        }
        store_v(ph + 1, cur.v);
        barrier_lds();
      }
    }
  } else {
    // ============================ loader waves ============================
    // Loader wave lw moves 1 KiB steps lw, lw+3, ... of the state operands; chunk c
    // lives in register slot c % 3 and LDS slot c & 1.
    constexpr int NLD = SM::NLD;
    const int lw = wave - 5;
    if (nc == 0) {                          // empty sequence: only keep the barrier count
      for (int ph = 0; ph <= nphase; ++ph) barrier_lds();
      return;
    }
    auto fetch = [&](int c, u32x4* dst) {   // chunk clamped into the sequence: the tail re-reads it
      const uint8_t* src = rec_ptr<K>(p, sq, hv, min(c, nc - 1)) + lw * 1024 + ln * 16;
#pragma unroll
      for (int i = 0; i < NLD; ++i) dst[i] = *reinterpret_cast<const u32x4*>(src + i * 3072);
    };
    auto put = [&](int c, const u32x4* src) {
      uint8_t* dst = smem + SM::ST + (c & 1) * SM::STAGE + lw * 1024 + ln * 16;
#pragma unroll
      for (int i = 0; i < NLD; ++i) *reinterpret_cast<u32x4*>(dst + i * 3072) = src[i];
    };
    // three separately named register slots of native vectors (an array of the
    // uint4 struct, or a 2-D array, is left in scratch by the compiler)
    u32x4 ra[NLD], rb[NLD], rc[NLD];
    fetch(0, ra);
    fetch(1, rb);
    fetch(2, rc);
    put(0, ra);
    barrier_lds();  // S0: chunk 0 in LDS slot 0
    static_assert(LD_RING == 3, "the ring turn below is written out for three slots");
    for (int t0 = 0; t0 < nphase; t0 += LD_RING) {
      // phase ph: refill the slot of chunk ph (staged during phase ph-1) with chunk
      // ph+3, then stage chunk ph+1 while the state wave reads LDS slot ph & 1
      fetch(t0 + 3, ra);
      __builtin_amdgcn_sched_barrier(0);   // loads issue before the LDS writes
      put(t0 + 1, rb);
      barrier_lds();
      fetch(t0 + 4, rb);
      __builtin_amdgcn_sched_barrier(0);   // loads issue before the LDS writes
      put(t0 + 2, rc);
      barrier_lds();
      fetch(t0 + 5, rc);
      __builtin_amdgcn_sched_barrier(0);   // loads issue before the LDS writes
      put(t0 + 3, ra);
      barrier_lds();
    }
  }
}

hipError_t launch_inter(const Params& p, hipStream_t s) {
  if (p.c16) return hipErrorInvalidValue;   // chunk 16 runs on the 64-column scan (kda_plan.hpp choice)
  const int64_t items = (int64_t)p.N * p.HV * (p.V / BV);
  if (items == 0) return hipSuccess;
  // longest-first order: whole rounds of eight units, V / 16 workgroups each
  const int grid = (int)(p.order ? ((int64_t)p.N * p.HV + 7) / 8 * 8 * (p.V / BV) : (items + 7) / 8 * 8);
  if (p.K == 128)
    hipLaunchKernelGGL((inter_kernel<128>), dim3(grid), dim3(INTER_THREADS), 0, s, p, (int)items);
  else
    hipLaunchKernelGGL((inter_kernel<64>), dim3(grid), dim3(INTER_THREADS), 0, s, p, (int)items);
  return hipGetLastError();
}

}  // namespace kda
