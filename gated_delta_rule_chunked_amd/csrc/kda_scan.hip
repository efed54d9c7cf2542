// kda_scan.hip -- segmented inter-chunk state scan of the KDA chunked forward (gfx950).
//
// Per chunk, following the kernel-fun fwd_state module docstring (and FlashKDA's
// phases 3-6), with h the fp32 state [K, V] of one sequence and value head:
//   u   = TmB v                      (TmB = Tm diag(beta))
//   v'  = u - w h
//   o   = qg h + Aqk v'              (scale folded into qg and Aqk)
//   h  <- diag(exp2 G) h + kg^T v'
//
// Work decomposition.  A workgroup covers 64 value columns (four 16-column column
// waves) of one segment of seg_L consecutive chunks, and stages each chunk's record
// once for all four: per useful column, a CU streams a quarter of the record bytes
// of a 16-column workgroup, which is what bounds a scan workgroup (its L1 sits at
// the limit of outstanding misses).  Segments restore the parallelism the wider
// tiles take away.  Over one segment the scan is affine in its start state,
//     h_end = M h_start + b,     M = prod_c (diag(exp2 G_c) - kg_c^T w_c),
// so two passes give the exact result:
//   * the state pass computes, for every segment but a sequence's last, b (the end
//     state from h0 for the first segment, from zero otherwise) and, for every
//     segment but the first and the last, M -- by scanning the columns of the
//     identity with v = 0 (u = 0);
//   * the full pass starts segment s from h_s, with h_1 = b_0 and
//     h_s = M_{s-1} h_{s-1} + b_{s-1} formed in its prologue, and writes o (and the
//     final state after the last segment).
// b is kept in fp32, M in bf16 (it multiplies a bf16 copy of h on MFMA, as w does
// within a chunk); both in the register order the full pass's prologue loads them
// in, so that its s - 1 products wait for one batch of whole-line loads each.
//
// Eight waves per workgroup, one barrier per chunk:
//   waves 0-3 (column waves): wave c holds h for columns 16c..16c+15 of the group
//     in the C layout of 16x16 MFMA tiles and runs the whole chunk in registers:
//     u, v', the update of h and (full pass) o^T = h^T qg^T + v'^T Aqk^T, whose C
//     layout gives each lane four adjacent columns of one token; the four waves
//     stage o in LDS and store it as whole 128-byte rows during the next chunk.
//     Operands come from the staged record; v^T fragments by transpose reads of the
//     row-major v tile.
//   waves 4-7 (loader waves): keep three chunks of records in flight in a register
//     ring (1 KiB steps of the record, steps lw, lw+4, ...) together with 16 rows
//     of the group's v columns, and copy chunk c+1 into the free slot of a
//     two-slot LDS ring during chunk c.  The rest of each record (the o operands in
//     the full pass, half of the state part in the state pass) goes into that slot
//     directly, by LDS-DMA loads issued as chunk c starts.

// Chunk 16 (C16): every 64-row record holds four 16-row chunks (block-diagonal TmB and
// Aqk, one decay row per 16-row chunk, kda_device.hpp).  The column waves then run four
// state updates per staged record: for 16-row chunk I, v'_I = u_I + (-w_I) h,
// o_I = qg_I h + Aqk_II v'_I and h <- diag(alpha_I) h + kg_I^T v'_I, the last two
// contracting over 16 tokens with the 16x16x16 MFMA on one half of a record fragment.

#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {

constexpr int SCAN_THREADS = 512;
constexpr int SCAN_RING = 3;            // chunks in flight per loader wave
enum ScanMode { SCAN_FULL = 0, SCAN_B = 1, SCAN_M = 2 };

template <int K, int MODE>
struct ScanSmem {
  using R = Rec<K>;
  // the full pass copies whole records, the state pass only their state part
  static constexpr int NSTEP = ((MODE == SCAN_FULL ? R::BYTES : R::STATE_BYTES) + 1023) / 1024;
  // The first NREG 1 KiB steps of a chunk go through the loaders' register ring
  // (issued two phases ahead), the others straight into LDS with LDS-DMA loads
  // (issued one phase ahead, into the slot the column waves have just released).
  // Full pass: the state part by the ring, the o part (QG, AQK) by DMA; state pass:
  // about half of the state part each way.  Interleaved A/B timing found these
  // splits best (the whole record by DMA was slower: one phase is too little time
  // for all of it to arrive).
  static constexpr int NREG = MODE == SCAN_FULL ? (R::STATE_BYTES + 1023) / 1024 : (NSTEP + 1) / 2;
  static constexpr int NLD = (NREG + 3) / 4;         // ring steps per loader wave (the last ones repeat)
  static constexpr int NLDD = (NSTEP - NREG + 3) / 4;   // DMA steps per loader wave
  static constexpr int SLOT = NSTEP * 1024;
  static constexpr int VT = 2 * SLOT;                // v tiles: [2 slots][4 column waves][64][16] bf16
  static constexpr int VT_BYTES = BT * BV * 2;
  // full pass: o of a chunk staged as [64 rows][64 columns] bf16 (rows padded to 144
  // bytes), two buffers, so that it leaves in whole 128-byte rows
  static constexpr int OST = VT + (MODE == SCAN_M ? 0 : 2 * 4 * VT_BYTES);
  static constexpr int OSTR = 144;
  static constexpr int OST_BYTES = BT * OSTR;
  static constexpr int BYTES = OST + (MODE == SCAN_FULL ? 2 * OST_BYTES : 0);
  static_assert(BYTES <= 160 * 1024, "fits the LDS of one CU");
};

// The chunks of one segment for one value head and 64-column group (`grp`: value
// columns 64 grp.., or key columns 64 grp.. of M in SCAN_M), with `ntiles` active
// column waves.  Waves from `lwave0` on are the loader waves; column wave cw is wave
// `cwave0` + cw (the state pass runs the b and M column waves of a group in one
// workgroup, each set through its own instantiation, over one set of loaders).
template <int K, int MODE, bool C16>
__device__ __forceinline__ void scan_body(const Params& p, uint8_t* smem, const SegLoc& sl, int hv, int grp,
                                          int ntiles, int64_t sigma, int lwave0 = 4, int cwave0 = 0) {
  using SM = ScanSmem<K, MODE>;
  using R = Rec<K>;
  constexpr int S = K / 32, ND = K / 16;
  const int tid = threadIdx.x, ln = tid & 63, r = ln & 15, g = ln >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool state_bf16 = p.flags & FLAG_STATE_BF16;
  const int ncs = sl.ncs;
  const int nphase = (ncs + SCAN_RING - 1) / SCAN_RING * SCAN_RING;
  const int64_t row0 = (int64_t)sl.b * p.T + sl.bos;        // first token row of the sequence
  auto chunk_of = [&](int ph) { return sl.c0 + min(ph, ncs - 1); };   // tail phases re-read the last chunk

  if (wave >= lwave0) {
    // ============================ loader waves ============================
    constexpr int NLD = SM::NLD;
    const int lw = wave - lwave0;
    if (ncs == 0) {
      barrier_lds();  // S0
      return;
    }
    // v: loader lw moves rows 16 lw .. 16 lw + 15 of the group's 64 columns; lane ln
    // takes row 16 lw + 8 h + (ln >> 3) (h = 0, 1) and the 16 bytes of column wave
    // cw = (ln & 7) >> 1, half ln & 1, so one load instruction covers 8 whole rows of
    // 128 bytes (column tiles past V are clamped to the last one, as the column waves
    // expect).  Row segments of 32 bytes per lane, the earlier layout, measured 4 %
    // slower over the whole scan.
    const int vcw = (ln & 7) >> 1, vhalf = ln & 1;
    const int vcol = min(grp * 64 + BV * vcw, p.V - BV) + 8 * vhalf;
    auto fetch = [&](int ph, u32x4* dst, uint4& v0, uint4& v1) {
      const int c = chunk_of(ph);
      const uint8_t* rec = p.recs + rec_index(hv, sl.cbase + c, p.HV) * (int64_t)R::BYTES + ln * 16;
#pragma unroll
      for (int i = 0; i < NLD; ++i) dst[i] = *reinterpret_cast<const u32x4*>(rec + min(4 * i + lw, SM::NREG - 1) * 1024);
      if (MODE != SCAN_M) {
        const int rbase = c * BT + 16 * lw + (ln >> 3);
        const int64_t t0 = row0 + min(rbase, sl.len - 1), t1 = row0 + min(rbase + 8, sl.len - 1);
        v0 = *reinterpret_cast<const uint4*>(p.v + (t0 * p.HV + hv) * p.V + vcol);
        v1 = *reinterpret_cast<const uint4*>(p.v + (t1 * p.HV + hv) * p.V + vcol);
      }
    };
    auto put = [&](int ph, const u32x4* src, const uint4& v0, const uint4& v1) {
      uint8_t* slot = smem + (ph & 1) * SM::SLOT + ln * 16;
#pragma unroll
      for (int i = 0; i < NLD; ++i) *reinterpret_cast<u32x4*>(slot + min(4 * i + lw, SM::NREG - 1) * 1024) = src[i];
      if (MODE != SCAN_M) {
        const int row = 16 * lw + (ln >> 3);
        const int cb = chunk_of(ph) * BT;                       // rows past the sequence are zero
        uint8_t* vt = smem + SM::VT + ((ph & 1) * 4 + vcw) * SM::VT_BYTES + row * 32 + vhalf * 16;
        *reinterpret_cast<uint4*>(vt) = cb + row < sl.len ? v0 : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(vt + 8 * 32) = cb + row + 8 < sl.len ? v1 : make_uint4(0, 0, 0, 0);
      }
    };
    // steps NREG.. of chunk ph straight into slot ph & 1 (LDS-DMA: lane ln's 16 bytes
    // land at the step's base + 16 ln, the record's own layout)
    auto dma = [&](int ph) {
      if (SM::NLDD == 0) return;
      const int c = chunk_of(ph);
      const uint8_t* rec = p.recs + rec_index(hv, sl.cbase + c, p.HV) * (int64_t)R::BYTES + ln * 16;
      uint8_t* slot = smem + (ph & 1) * SM::SLOT;
#pragma unroll
      for (int i = 0; i < SM::NLDD; ++i) {
        const int st = min(SM::NREG + 4 * i + lw, SM::NSTEP - 1);   // the last steps repeat
        // written as assembly so that the compiler's wait counting does not treat the
        // LDS writes of the copy as aliasing every later LDS store of the wave (it then
        // waits for all loads in flight, the ring's included); its own waits only come
        // out more conservative for not counting these loads
        const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)(slot + st * 1024);
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(rec + st * 1024), "s"(lds) : "memory", "m0");
      }
    };
    // Before a barrier the loader waits until only the ring loads issued after the
    // phase's DMA are outstanding: the DMA data is then in LDS for the column waves.
    constexpr int NAFTER = NLD + (MODE != SCAN_M ? 2 : 0);
    static_assert(NAFTER <= 63, "fits the vmcnt counter");
    auto wait_dma = [&]() {
      if (SM::NLDD > 0) __builtin_amdgcn_s_waitcnt((NAFTER & 15) | ((NAFTER >> 4) << 14) | (7 << 4) | (15 << 8));
    };
    u32x4 ra[NLD], rb[NLD], rc[NLD];
    uint4 va0, va1, vb0, vb1, vc0, vc1;
    dma(0);
    __builtin_amdgcn_sched_barrier(0);
    fetch(0, ra, va0, va1);
    fetch(1, rb, vb0, vb1);
    fetch(2, rc, vc0, vc1);
    put(0, ra, va0, va1);   // waits for chunk 0's ring loads, and so for the older DMA
    barrier_lds();  // S0: chunk 0 of the segment in slot 0
    static_assert(SCAN_RING == 3, "the ring turn below is written out for three slots");
    for (int t0 = 0; t0 < nphase; t0 += SCAN_RING) {
      dma(t0 + 1);
      __builtin_amdgcn_sched_barrier(0);
      fetch(t0 + 3, ra, va0, va1);
      __builtin_amdgcn_sched_barrier(0);   // loads issue before the LDS writes
      put(t0 + 1, rb, vb0, vb1);
      wait_dma();
      barrier_lds();
      dma(t0 + 2);
      __builtin_amdgcn_sched_barrier(0);
      fetch(t0 + 4, rb, vb0, vb1);
      __builtin_amdgcn_sched_barrier(0);
      put(t0 + 2, rc, vc0, vc1);
      wait_dma();
      barrier_lds();
      dma(t0 + 3);
      __builtin_amdgcn_sched_barrier(0);
      fetch(t0 + 5, rc, vc0, vc1);
      __builtin_amdgcn_sched_barrier(0);
      put(t0 + 3, ra, va0, va1);
      wait_dma();
      barrier_lds();
    }
    __builtin_amdgcn_s_waitcnt(0);   // no LDS-DMA write may land after the workgroup ends
    return;
  }

  // ============================ column waves ============================
  const int cw = wave - cwave0;
  if (cw >= ntiles) {                         // columns past V: keep the barrier count only
    for (int ph = 0; ph <= nphase; ++ph) barrier_lds();
    return;
  }
  const int col = grp * 64 + BV * cw + r;     // this lane's column (of V, or of K in SCAN_M)
  // h tile md: lane holds h[16md + 4g + rr][col], rr = 0..3
  f32x4 h[ND];
  if (MODE == SCAN_M) {
#pragma unroll
    for (int md = 0; md < ND; ++md)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) h[md][rr] = (16 * md + 4 * g + rr == col) ? 1.f : 0.f;
  } else if (sl.s == 0 || MODE == SCAN_B) {
    const bool from_h0 = sl.s == 0 && p.h0 != nullptr;
#pragma unroll
    for (int md = 0; md < ND; ++md)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d = 16 * md + 4 * g + rr;
        h[md][rr] = from_h0 ? load_state(state_bf16, p.h0, (((int64_t)sl.n * p.HV + hv) * K + d) * p.V + col) : 0.f;
      }
  } else {
    // full pass, s >= 1: h_1 = b_0, h_{s'+1} = M_{s'} h_{s'} + b_{s'}.  b is stored in
    // this wave's C-layout order and M as P-order A fragments (see the state pass's
    // stores), so both arrive as whole 1 KiB wave loads; a hop's loads are all issued
    // before its products.
    auto load_b = [&](int64_t sig, f32x4* x) {
      const float4* bb = reinterpret_cast<const float4*>(p.bbuf) +
                         ((sig * p.HV + hv) * (p.V / BV) + col / BV) * (int64_t)(ND * 64) + ln;
#pragma unroll
      for (int md = 0; md < ND; ++md) {
        const float4 t = bb[md * 64];
        x[md] = f32x4{t.x, t.y, t.z, t.w};
      }
    };
    load_b(sl.sigma0, h);
    for (int s2 = 1; s2 < sl.s; ++s2) {
      f32x4 hn[ND];
      load_b(sl.sigma0 + s2, hn);
      const uint4* Mf = reinterpret_cast<const uint4*>(p.mbuf + ((sl.sigma0 + s2) * p.HV + hv) * (int64_t)K * K) + ln;
      uint4 mf[ND * S];
#pragma unroll
      for (int f = 0; f < ND * S; ++f) mf[f] = Mf[f * 64];
      uint2 hb[ND];
#pragma unroll
      for (int md = 0; md < ND; ++md) hb[md] = pack4(h[md]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int md = 0; md < ND; ++md)
#pragma unroll
        for (int s3 = 0; s3 < S; ++s3)
          hn[md] = mfma16x32(as_frag(mf[md * S + s3]), cat(hb[2 * s3], hb[2 * s3 + 1]), hn[md]);
#pragma unroll
      for (int md = 0; md < ND; ++md) h[md] = hn[md];
    }
  }
  // per-lane parts of the LDS addresses of the v tile's transpose reads
  const int tr16 = ((4 * (ln >> 4) + ((ln >> 2) & 3)) * BV + 4 * (ln & 3)) * 2;
  // o: this lane's columns in the sequence's first row, and the row stride
  // o of the chunk of phase q, staged in buffer q & 1, leaves in whole rows at the
  // start of the next phase: lane (row 8 h + (ln >> 3), 16-byte column block ln & 7),
  // row blocks h shared out over the active column waves; columns past V are never
  // written.  Each column wave storing its own 32-byte row segments directly was
  // measured 8 % slower over the whole scan.
  auto store_o = [&](int q) {
    const int c = sl.c0 + q;
    const uint8_t* ob = smem + SM::OST + (q & 1) * SM::OST_BYTES;
    const int lc = ln & 7;
    if (lc < 2 * ntiles) {
      for (int h8 = cw; h8 < 8; h8 += ntiles) {
        const int row = 8 * h8 + (ln >> 3);
        if (c * BT + row < sl.len) {
          const uint4 v = *reinterpret_cast<const uint4*>(ob + row * SM::OSTR + 16 * lc);
          *reinterpret_cast<uint4*>(p.o + ((row0 + c * BT + row) * p.HV + hv) * p.V + grp * 64 + 8 * lc) = v;
        }
      }
    }
  };
  barrier_lds();  // S0
  for (int ph = 0; ph < nphase; ++ph) {
    if (MODE == SCAN_FULL && ph >= 1 && ph <= ncs) store_o(ph - 1);
    if (ph < ncs) {
      const int c = sl.c0 + ph;
      if (MODE == SCAN_FULL && !C16 && p.hc) {   // the state before this chunk
        // the row stride is re-made opaque every chunk, so the 32 row offsets stay
        // transient scalars instead of being hoisted as live 64-bit addresses
        int sv = p.V;
        asm volatile("" : "+s"(sv));
        const int64_t base = (((sl.cbase + c) * p.HV + hv) * K + 4 * g) * (int64_t)sv + col;
        if (state_bf16) {
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
      const uint8_t* st = smem + (ph & 1) * SM::SLOT;
      if constexpr (C16) {
        // ---- four 16-row chunks per record ----
        // u = TmB v with TmB block diagonal: row block mb needs only the fragment that
        // holds its diagonal block, (0,0) (1,0) (2,1) (3,1)
        f32x4 u[4];
        if (MODE != SCAN_M) {
          const uint8_t* vt = smem + SM::VT + ((ph & 1) * 4 + cw) * SM::VT_BYTES + tr16;
          const bf16x8 vb0 = cat(lds_tr8(vt), lds_tr8(vt + 16 * BV * 2));
          const bf16x8 vb1 = cat(lds_tr8(vt + 32 * BV * 2), lds_tr8(vt + 48 * BV * 2));
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
            u[mb] = mfma16x32(as_frag(lds16(st + R::TMB + (tri_frag(mb, mb >> 1) * 64 + ln) * 16)), mb < 2 ? vb0 : vb1,
                              f32x4{0.f, 0.f, 0.f, 0.f});
        } else {
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) u[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        uint2 ov[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          // operands of 16-row chunk I: its decay row, the -w rows, the halves of the kg^T
          // fragments that cover its tokens
          float4 al[ND];
          uint4 wn[S];
          uint2 kgh[ND];
#pragma unroll
          for (int md = 0; md < ND; ++md)
            al[md] = *reinterpret_cast<const float4*>(st + alpha16_off<K>(I) + (16 * md + 4 * g) * 4);
#pragma unroll
          for (int s = 0; s < S; ++s) wn[s] = lds16(st + R::WN + ((I * S + s) * 64 + ln) * 16);
#pragma unroll
          for (int md = 0; md < ND; ++md)
            kgh[md] = lds8(st + R::KGT + ((2 * md + (I >> 1)) * 64 + ln) * 16 + (I & 1) * 8);
          __builtin_amdgcn_sched_barrier(0);
          uint2 hb[ND];
#pragma unroll
          for (int md = 0; md < ND; ++md) {
            hb[md] = pack4(h[md]);
            h[md][0] *= al[md].x;
            h[md][1] *= al[md].y;
            h[md][2] *= al[md].z;
            h[md][3] *= al[md].w;
          }
          // v'_I = u_I + (-w_I) h
          f32x4 acc = u[I];
#pragma unroll
          for (int s = 0; s < S; ++s) acc = mfma16x32(as_frag(wn[s]), cat(hb[2 * s], hb[2 * s + 1]), acc);
          const uint2 vp = pack4(acc);
          // h <- diag(alpha_I) h + kg_I^T v'_I  (16 tokens: one 16x16x16 product per tile)
#pragma unroll
          for (int md = 0; md < ND; ++md) h[md] = mfma16x16(as_half(kgh[md]), as_half(vp), h[md]);
          if (MODE == SCAN_FULL) {
            // o_I^T = h^T qg_I^T + v'_I^T Aqk_II^T: h before this 16-row chunk
            uint4 qg[S];
#pragma unroll
            for (int s = 0; s < S; ++s) qg[s] = lds16(st + R::QG + ((I * S + s) * 64 + ln) * 16);
            const uint2 aqh = lds8(st + R::AQK + (tri_frag(I, I >> 1) * 64 + ln) * 16 + (I & 1) * 8);
            f32x4 oacc = f32x4{0.f, 0.f, 0.f, 0.f}, oacc2 = oacc;
#pragma unroll
            for (int s = 0; s < S; s += 2) {
              oacc = mfma16x32(cat(hb[2 * s], hb[2 * s + 1]), as_frag(qg[s]), oacc);
              oacc2 = mfma16x32(cat(hb[2 * s + 2], hb[2 * s + 3]), as_frag(qg[s + 1]), oacc2);
            }
            oacc = mfma16x16(as_half(vp), as_half(aqh), oacc);
            ov[I] = pack4(oacc + oacc2);
          }
        }
        if (MODE == SCAN_FULL) {
          uint8_t* ob = smem + SM::OST + (ph & 1) * SM::OST_BYTES + (16 * cw + 4 * g) * 2;
#pragma unroll
          for (int w = 0; w < 4; ++w) *reinterpret_cast<uint2*>(ob + (16 * w + r) * SM::OSTR) = ov[w];
        }
      } else {
      // batch 1: v^T fragments, TmB, decay, -w (in the order they are consumed)
      bf16x8 vb0, vb1;
      uint4 tm[6];
      if (MODE != SCAN_M) {
        const uint8_t* vt = smem + SM::VT + ((ph & 1) * 4 + cw) * SM::VT_BYTES + tr16;
        vb0 = cat(lds_tr8(vt), lds_tr8(vt + 16 * BV * 2));
        vb1 = cat(lds_tr8(vt + 32 * BV * 2), lds_tr8(vt + 48 * BV * 2));
#pragma unroll
        for (int f = 0; f < 6; ++f) tm[f] = lds16(st + R::TMB + (f * 64 + ln) * 16);
      }
      float4 al[ND];
      uint4 wn[4 * S];
#pragma unroll
      for (int md = 0; md < ND; ++md) al[md] = *reinterpret_cast<const float4*>(st + R::ALPHA + (16 * md + 4 * g) * 4);
#pragma unroll
      for (int s = 0; s < S; ++s)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) wn[s * 4 + mb] = lds16(st + R::WN + ((mb * S + s) * 64 + ln) * 16);
      __builtin_amdgcn_sched_barrier(0);
      // u = TmB v, row blocks mb = 0..3 (lower triangular: 1 or 2 32-steps); zero in SCAN_M
      f32x4 acc[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        if (MODE != SCAN_M) {
          acc[mb] = mfma16x32(as_frag(tm[tri_frag(mb, 0)]), vb0, f32x4{0.f, 0.f, 0.f, 0.f});
          if (mb >= 2) acc[mb] = mfma16x32(as_frag(tm[tri_frag(mb, 1)]), vb1, acc[mb]);
        } else {
          acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      // h as the bf16 B operand (tiles 2s, 2s+1 form the P-order fragment of step s);
      // then h <- diag(alpha) h
      uint2 hb[ND];
#pragma unroll
      for (int md = 0; md < ND; ++md) {
        hb[md] = pack4(h[md]);
        h[md][0] *= al[md].x;
        h[md][1] *= al[md].y;
        h[md][2] *= al[md].z;
        h[md][3] *= al[md].w;
      }
      __builtin_amdgcn_sched_barrier(0);
      // batch 2: kg^T, ahead of the v' products in the full pass; in the state pass
      // (twelve waves, 168 registers) only after them, when the -w fragments are dead
      uint4 kg[2 * ND];
      auto load_kg = [&]() {
#pragma unroll
        for (int i = 0; i < 2 * ND; ++i) kg[i] = lds16(st + R::KGT + (i * 64 + ln) * 16);
      };
      if (MODE == SCAN_FULL) load_kg();
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
      for (int mb = 0; mb < 4; ++mb) vp[mb] = pack4(acc[mb]);
      if (MODE != SCAN_FULL) {
        __builtin_amdgcn_sched_barrier(0);
        load_kg();
      }
      // h <- diag(alpha) h + kg^T v'   (v' tiles (2s2, 2s2+1) = P-order token step s2)
      const bf16x8 vp0 = cat(vp[0], vp[1]), vp1 = cat(vp[2], vp[3]);
#pragma unroll
      for (int md = 0; md < ND; ++md) {
        h[md] = mfma16x32(as_frag(kg[2 * md]), vp0, h[md]);
        h[md] = mfma16x32(as_frag(kg[2 * md + 1]), vp1, h[md]);
      }
      if (MODE == SCAN_FULL) {
        // o^T = h^T qg^T + v'^T Aqk^T per 16-token row block w: the P-order fragments
        // of h (before the update) and v' as A operands, the record's qg / Aqk
        // fragments as B operands; lane (g, r) gets token 16w + r, columns 4g..4g+3.
        // All four blocks first, the guarded stores after, so that no branch splits
        // the operand reads from the products.
        __builtin_amdgcn_sched_barrier(0);
        uint2 ov[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint4 qg[S], aq[2];
#pragma unroll
          for (int s = 0; s < S; ++s) qg[s] = lds16(st + R::QG + ((w * S + s) * 64 + ln) * 16);
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2)
            aq[s2] = lds16(st + R::AQK + (tri_frag(w, min(s2, tri_steps(w) - 1)) * 64 + ln) * 16);
          f32x4 oacc = f32x4{0.f, 0.f, 0.f, 0.f}, oacc2 = oacc;
#pragma unroll
          for (int s = 0; s < S; s += 2) {
            oacc = mfma16x32(cat(hb[2 * s], hb[2 * s + 1]), as_frag(qg[s]), oacc);
            oacc2 = mfma16x32(cat(hb[2 * s + 2], hb[2 * s + 3]), as_frag(qg[s + 1]), oacc2);
          }
          oacc = mfma16x32(vp0, as_frag(aq[0]), oacc);
          if (tri_steps(w) > 1) oacc2 = mfma16x32(vp1, as_frag(aq[1]), oacc2);
          ov[w] = pack4(oacc + oacc2);
        }
        uint8_t* ob = smem + SM::OST + (ph & 1) * SM::OST_BYTES + (16 * cw + 4 * g) * 2;
#pragma unroll
        for (int w = 0; w < 4; ++w) *reinterpret_cast<uint2*>(ob + (16 * w + r) * SM::OSTR) = ov[w];
      }
      }   // chunk 64
    }
    barrier_lds();
  }
  if (MODE == SCAN_FULL && ncs == nphase && ncs > 0) store_o(ncs - 1);   // no spare phase left for it
  // the segment's end state (row strides made opaque, so that the 32 row offsets are
  // not computed ahead of the chunk loop and kept live through it)
  if (MODE == SCAN_B) {
    // b in the C-layout order of this column tile: [segment][HV][V/16][K/16][64 lanes][4]
    float4* bb = reinterpret_cast<float4*>(p.bbuf) + ((sigma * p.HV + hv) * (p.V / BV) + col / BV) * (int64_t)(ND * 64) + ln;
#pragma unroll
    for (int md = 0; md < ND; ++md) bb[md * 64] = make_float4(h[md][0], h[md][1], h[md][2], h[md][3]);
  } else if (MODE == SCAN_M) {
    // M as P-order A fragments of the full pass's products M h: fragment (md, s3) holds
    // rows 16 md.., columns 32 s3..; this lane's column col lands in lane group gp,
    // element e, and its rows 16 md + 4 g + rr in lanes 16 gp + 4 g + rr
    uint16_t* mm = p.mbuf + (sigma * p.HV + hv) * (int64_t)K * K;
    const int s3 = col >> 5, q = col & 31;
    const int gp = (q & 15) >> 2, e = (q & 3) + 4 * (q >> 4);
#pragma unroll
    for (int md = 0; md < ND; ++md)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) mm[((md * S + s3) * 64 + 16 * gp + 4 * g + rr) * 8 + e] = f2bf(h[md][rr]);
  } else if (p.ht && sl.s == sl.nseg - 1) {
#pragma unroll
    for (int md = 0; md < ND; ++md)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d = 16 * md + 4 * g + rr;
        store_state(state_bf16, p.ht, (((int64_t)sl.n * p.HV + hv) * K + d) * p.V + col, h[md][rr]);
      }
  }
}

// State pass: item = (sigma * HV + hv) * NJ + j, NJ = max(V/64, K/64) rounded up.  One
// workgroup of twelve waves computes, over one staged copy of the segment's records,
// b for value columns 64 j.. (waves 0-3, every segment but a sequence's last) and M
// for key columns 64 j.. (waves 4-7, inner segments only); waves 8-11 load.  With b and
// M in separate workgroups the benchmarked shape needed 320 of them, a second round on
// 256 compute units; paired they are 192.
constexpr int SCAN_STATE_THREADS = 768;
template <int K, bool C16>
__global__ __launch_bounds__(SCAN_STATE_THREADS, 1) void scan_state_kernel(Params p, int n_items) {
  static_assert(ScanSmem<K, SCAN_B>::SLOT == ScanSmem<K, SCAN_M>::SLOT, "b and M waves read one staging layout");
  __shared__ __attribute__((aligned(16))) uint8_t smem[ScanSmem<K, SCAN_B>::BYTES];
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  if (item >= n_items) return;
  if (p.cu != nullptr && p.table[p.N + 1] != 0) return;   // rejected cu_seqlens: the full pass reports it
  const int NCG = (p.V + 63) / 64, NJ = max(NCG, K / 64);
  const int j = item % NJ;
  const int hv = (item / NJ) % p.HV;
  const int64_t sigma = item / (NJ * p.HV);
  SegLoc sl;
  if (!locate_segment(p, sigma, sl)) return;
  const bool inner = sl.s < sl.nseg - 1;                  // the last segment's end state is not needed
  const int nb = (inner && j < NCG) ? min(4, (p.V - 64 * j) / BV) : 0;
  const int nm = (inner && sl.s > 0 && j < K / 64) ? 4 : 0;   // M between inner segments only
  if (nb == 0 && nm == 0) return;                         // uniform over the workgroup
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave >= 4 && wave < 8)
    scan_body<K, SCAN_M, C16>(p, smem, sl, hv, j, nm, sigma, 8, 4);
  else   // b column waves and the loaders (which also stage v for the b waves)
    scan_body<K, SCAN_B, C16>(p, smem, sl, hv, j, nb, sigma, 8, 0);
}

// Full pass: item = (sigma * HV + hv) * NCG + cg.
template <int K, bool C16>
__global__ __launch_bounds__(SCAN_THREADS, 1) void scan_full_kernel(Params p, int n_items) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[ScanSmem<K, SCAN_FULL>::BYTES];
  // with the longest-first order every workgroup of the grid is mapped below; otherwise
  // items are XCD-remapped and the grid's padding returns here
  const int item = p.order ? (int)blockIdx.x : xcd_remap(blockIdx.x, gridDim.x);
  if (p.order) n_items = (int)gridDim.x;
  if (item >= n_items) return;
  const int tid = threadIdx.x;
  if (p.cu != nullptr && p.table[p.N + 1] != 0) {
    // rejected cu_seqlens: poison all of o and ht, grid-strided
    const int64_t total = (int64_t)p.B * p.T * p.HV * p.V;
    for (int64_t idx = (int64_t)item * SCAN_THREADS + tid; idx < total; idx += (int64_t)n_items * SCAN_THREADS)
      p.o[idx] = 0x7fc0;
    if (p.ht) {
      const int64_t nh = (int64_t)p.N * p.HV * K * p.V;
      for (int64_t idx = (int64_t)item * SCAN_THREADS + tid; idx < nh; idx += (int64_t)n_items * SCAN_THREADS)
        store_state(p.flags & FLAG_STATE_BF16, p.ht, idx, __builtin_nanf(""));
    }
    return;
  }
  const int NCG = (p.V + 63) / 64;
  int cg, hv;
  int64_t sigma;
  if (p.order) {
    // varlen, one segment per sequence: (sequence rank, head) units in dispatch order,
    // so the longest sequences start first; a unit's column groups go to one XCD (the
    // unit picks the XCD, its column groups follow in consecutive rounds of eight)
    const int b = blockIdx.x, rnd = b >> 3;
    const int64_t u = (int64_t)(rnd / NCG) * 8 + (b & 7);
    if (u >= (int64_t)p.N * p.HV) return;
    cg = rnd % NCG;
    hv = (int)(u % p.HV);
    sigma = p.order[u / p.HV];
    if ((uint64_t)sigma >= (uint64_t)p.N) return;   // never for an order the chunk table wrote
  } else {
    cg = item % NCG;
    hv = (item / NCG) % p.HV;
    sigma = item / (NCG * p.HV);
  }
  SegLoc sl;
  if (!locate_segment(p, sigma, sl)) return;
  scan_body<K, SCAN_FULL, C16>(p, smem, sl, hv, cg, min(4, (p.V - 64 * cg) / BV), sigma);
}

template <int K, bool C16>
static hipError_t launch_scan_k(const Params& p, hipStream_t s) {
  const int64_t NCG = (p.V + 63) / 64;
  if (p.bbuf != nullptr) {
    const int64_t items = p.max_segs * p.HV * std::max<int64_t>(NCG, K / 64);
    hipLaunchKernelGGL((scan_state_kernel<K, C16>), dim3((int)((items + 7) / 8 * 8)), dim3(SCAN_STATE_THREADS), 0, s, p,
                       (int)items);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t items = p.max_segs * p.HV * NCG;
  // longest-first order: whole rounds of eight units, NCG workgroups each
  const int64_t grid = p.order ? ((int64_t)p.N * p.HV + 7) / 8 * 8 * NCG : (items + 7) / 8 * 8;
  hipLaunchKernelGGL((scan_full_kernel<K, C16>), dim3((int)grid), dim3(SCAN_THREADS), 0, s, p, (int)items);
  return hipGetLastError();
}

hipError_t launch_scan(const Params& p, hipStream_t s) {
  if (p.max_segs * p.HV == 0) return hipSuccess;
  if (p.c16) return p.K == 128 ? launch_scan_k<128, true>(p, s) : launch_scan_k<64, true>(p, s);
  return p.K == 128 ? launch_scan_k<128, false>(p, s) : launch_scan_k<64, false>(p, s);
}

}  // namespace kda
